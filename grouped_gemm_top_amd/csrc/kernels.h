// Launchers for the routing and data-movement kernels of the MoE-LoRA layer.
#pragma once
#include "common.h"

namespace moe {

constexpr int kRouteBlockTokens = 256;  // tokens per block in the histogram/rank pass

// Per token: top-k logits (ties -> lower expert id), routing weights, raw scores.
// Top-k over logits given as nsplit partial arrays (split_stride floats apart, summed in order);
// with nsplit > 1 the summed logits are written to zout (when not null).
hipError_t launch_topk(const float* z, int nsplit, long split_stride, float* zout, int s, int E,
                       int k, int score, int renorm, int* idx, float* w, float* psel, hipStream_t st);
// Per block of 256 tokens: expert histogram and each pair's rank among the block's pairs of the
// same expert (token order).
hipError_t launch_hist_rank(const int* idx, int s, int k, int E, int* blk_hist, int* rank,
                            hipStream_t st);
// Expert offsets, per-block bases and row-tile tables from the block histograms (one workgroup).
hipError_t launch_scan(const int* blk_hist, int nb, int E, int P, int* blk_base, int* off,
                       int* tile_tables, int* tile_maps, hipStream_t st);
// The tables of a single group of `rows` rows (a dense expert applied to every token): off = [0, rows],
// the row-tile tables of launch_scan for G = 1, and zeroed row tile -> group maps.
hipError_t launch_one_group_tables(int rows, int* off, int* tile_tables, int* tile_maps, hipStream_t st);
// perm / inv / row token from the bases and ranks.
hipError_t launch_scatter(const int* idx, const int* rank, const int* blk_base, int s, int k, int E,
                          int* perm, int* inv, int* row_tok, hipStream_t st);

// Y[t] = sum_j w[t,j] o[inv[t k + j]] (fp32 accumulate, slot order).
hipError_t launch_combine(int dtype, const void* o, const int* inv, const float* w, void* Y, int s,
                          int k, int m, hipStream_t st);
// ds[p] = sum of the partials ds_part[q * s k + p] over q < nparts (in order of q), then dz[t, j]
// from ds, w, p_sel (softmax or sigmoid, renormalised or not). k <= 1024.
hipError_t launch_router_bwd(const float* ds_part, int nparts, const float* w, const float* psel, int s, int k,
                             int score, int renorm, float* dz, hipStream_t st);
// WT[b][c, a] = W[b][a, c] for `batch` consecutive rows x cols matrices
hipError_t launch_transpose(int dtype, const void* W, void* WT, int rows, int cols, int batch,
                            hipStream_t st);
// dX[t] = sum_j dXp[inv[t k + j]] (+ sum_j dz[t,j] WrT[idx[t,j]] when dz != nullptr)
hipError_t launch_unpermute(int dtype, const void* dXp, const int* inv, const float* dz,
                            const int* idx, const void* WrT, void* dX, int s, int k, int m,
                            hipStream_t st);
// bf16 [rows, cols] -> [rows, ld] (ld >= cols), zeros in columns [cols, ld)
hipError_t launch_pad_cols(const void* W, void* Wp, int rows, int cols, int ld, hipStream_t st);
// zero-fill n 32-bit words
hipError_t launch_zero(void* p, size_t words, hipStream_t st);
// The row-weighted rows out[i, :] = w[pair[i]] * in[i, :] (rows x cols, rounded to dtype) and, when W is
// given, the transpose of W [trows, tcols] into WT, in one launch.
hipError_t launch_bwd_prep(int dtype, const void* in, const int* pair, const float* w, void* out, long rows,
                           int cols, const void* W, void* WT, int trows, int tcols, hipStream_t st);

// Wo = W + c A B over one projection block of every expert (see merge_kernel): kx selects the
// x.W orientation (off = i * ld + j + col0) over the output-major one ((j + col0) * ld + i).
hipError_t launch_merge(int dtype, bool kx, const void* W, const void* A, const void* B, void* Wo,
                        int E, int K, int N, int r, long ld, long col0, long wstride, float c,
                        hipStream_t st);
}  // namespace moe
