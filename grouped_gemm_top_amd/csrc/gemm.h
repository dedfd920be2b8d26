// Grouped GEMM descriptions shared by the MFMA kernels and the plain SIMT kernels.
//
// Two problem kinds:
//  * row-grouped ("GM"): the rows of the output are split into expert groups
//    [goff[e], goff[e+1]); group e computes C[rows_e, :] = A[rows_e, :] . B_e  (+ a LoRA tail
//    A2[rows_e, :] . B2_e), followed by an epilogue. K is shared by all groups.
//  * K-grouped ("GK"): group e computes C_e = scale * L[rows_e, :]^T . R[rows_e, :]; the group
//    rows are the reduction axis (LoRA-factor gradients).
#pragma once
#include "common.h"

namespace moe {

// Operand storage: element (x, kk) of an operand, x the output-side index, kk the reduction index.
enum OperandLayout : int {
  LAYOUT_XK = 0,  // base[x * ld + kk]   (reduction axis contiguous)
  LAYOUT_KX = 1,  // base[kk * ld + x]   (output axis contiguous)
};

enum Epilogue : int {
  EPI_STORE = 0,       // C = scale * acc (+ bias[col])
  EPI_DUAL = 1,        // two column halves: C[:, j] = scale*acc_gate, C[:, cup + j] = scale*acc_up
  EPI_SWIGLU = 2,      // dual, plus H = silu(gate) * up; C holds [gate | up]
  EPI_SWIGLU_BWD = 3,  // acc = dh; reads GU = [g | u]; C[:, j] = dg, C[:, cup + j] = du
};

enum TailMode : int {
  TAIL_NONE = 0,
  TAIL_SINGLE = 1,     // K2 = r2a from source 0
  TAIL_BLOCKDIAG = 2,  // dual: tail rows [0, r2a) feed gate columns from source 0,
                       //       rows [r2a, 2 r2a) feed up columns from source 1
  TAIL_STACKED = 3,    // tail rows [0, r2a) from source 0, [r2a, 2 r2a) from source 1
  TAIL_SHARED = 4,     // dual: the r2a tail rows feed gate columns from source 0 and up columns
                       //       from source 1 (one low-rank input shared by both halves)
};

struct GemmArgs {
  // ---- problem
  int M;             // rows of a single ungrouped problem (goff == nullptr); GK: output rows
  int N;             // output columns (per half for dual epilogues)
  int K;             // reduction length (GM)
  int G;             // number of groups
  const int* goff;   // [G+1] group offsets, or nullptr for one group [0, M)
  const int* toff_all;  // GM: kNumTileSizes tables of [G+1] row-tile prefix sums (one per BM)
  const int* tmap_all;  // GM: kNumTileSizes maps row tile -> group, at tile_map_offset(i, ...)
  // ---- A operand (GM: layout XK with optional row gather; GK: layout KX over group rows)
  const void* A;
  long lda;
  const int* arow;   // GM gather: A row of output row i is arow[i] / arow_div
  int arow_div;
  // ---- B operand
  const void* B;
  long ldb;
  long bstride;      // elements between consecutive groups' B
  const void* Bu;    // dual: base of the up half (same layout, ld and group stride as B)
  // ---- LoRA tail (GM only)
  int tail;          // TailMode
  int r2a;           // rows of the reduction tail taken from each source
  const void* TA;    // [rows][lda2] tail A operand (layout XK, same row space as the output)
  long lda2;
  const void* TB0;   // tail B sources (layout of B), per-group stride tbstride
  const void* TB1;
  long ldtb;
  long tbstride;
  // ---- epilogue
  void* C;
  void* C1;          // GK: columns >= nsplit go to C1 (column index minus nsplit); nullptr: none
  int nsplit;
  int ctrans;        // GK: store C[col * ldc + row] instead of C[row * ldc + col]
  long ldc;
  long cup;          // dual epilogues: column offset of the up half in C
  long cstride;      // GK: elements between groups' outputs
  float scale;
  const float* bias; // EPI_STORE: per-column bias (fp32) or nullptr; added by K split 0 only
  int kchunk;        // GM without groups or tail: gridDim.y K splits of kchunk each (0: one split)
  int accum;         // GM, EPI_STORE, deep-prefetch and reference kernels: C += result instead of C =
                     //   (the other kernels reject it)
  // Row weights (deep-prefetch and reference kernels): grouped row i's weight is wval[arow[i]] (the
  // routing weight of the pair the row holds).
  const float* wval;
  void* C2;          // EPI_STORE: also store the row-weighted result here (same layout as C)
  int wscale;        // EPI_SWIGLU_BWD: dh = row weight * scale * acc before the SwiGLU backward
  // EPI_SWIGLU_BWD with row weights: partial dot products of scale * acc (dh before the row
  // weight) with h = silu(g) u, one per 64 output columns: dspart[(col / 64) * dsstride + arow[i]]
  float* dspart;
  long dsstride;
  long csplit;       //   elements between the outputs of consecutive K splits
  void* H;           // EPI_SWIGLU: silu(gate)*up output
  long ldh;
  const void* GU;    // EPI_SWIGLU_BWD: saved [g | u]
  long ldgu;
  long guup;         // column offset of u in GU
  // nbatch == 2 runs a second, independent problem of the same shape and grouping in the same
  // launch (GM deep-prefetch and reference kernels, and GK), with operands bA, bB, output bC and
  // (GK) partials bgkpart
  int nbatch;
  const void* bA;
  const void* bB;
  void* bC;
  float* bgkpart;
  float* gkpart;
  int gkchunk;       // GK with gkpart: rows per chunk, kGkChunk (also 0) or kGkChunkSmall. The small chunk
                     //   table gives a group without rows no chunk: only for groups that all have rows     // GK: fp32 partial products of groups longer than one chunk, [chunk][M][N]
                     // (gk_part_floats); nullptr: one workgroup reduces a whole group
};

// Launchers (hipStream_t passed as void* to keep this header light). Each returns a HIP error.
// dtype: 0 fp32, 1 bf16. For bf16 the MFMA kernels run unless reference is set.
// GM: rows_bound = upper bound on the total number of rows over all groups (sizes the grid).
hipError_t gemm_gm_launch(const GemmArgs& a, int b_layout, int epi, int out_f32, int dtype,
                          int rows_bound, int reference, hipStream_t stream);
// GK: njobs <= kGkMaxJobs problems over the same row grouping (G, goff, chunk tables, and either all
// or none with partials), in one launch. rows_bound bounds the total group rows (sizes the chunk
// grid when gkpart is set).
hipError_t gemm_gk_launch(const GemmArgs* jobs, int njobs, int dtype, int reference, int rows_bound,
                          hipStream_t stream);

// Row-tile tables for the MFMA row tile sizes used by gemm_gm_launch.
constexpr int kNumTileSizes = 5;
constexpr int kTileSizes[kNumTileSizes] = {32, 64, 128, 256, 1024};
// K-grouped launches split a group's rows into chunks of kGkChunk rows (table kGkChunkTable), so
// that one long group does not serialise its whole reduction in a few workgroups.
constexpr int kGkChunkTable = 4;
constexpr int kGkChunk = 1024;
static_assert(kTileSizes[kGkChunkTable] == kGkChunk, "chunk table");
// Smaller chunks for few large groups (a shared expert: one group of every token), whose 1024-row
// chunks would leave most of the chip idle.
constexpr int kGkChunkSmallTable = 3;
constexpr int kGkChunkSmall = 256;
static_assert(kTileSizes[kGkChunkSmallTable] == kGkChunkSmall, "small chunk table");
__host__ __device__ inline int gk_chunk_table(int gkchunk) {
  return gkchunk == kGkChunkSmall ? kGkChunkSmallTable : kGkChunkTable;
}
int tile_table_index(int bm);
// Row-tile -> group maps: map i has room for rows_bound / kTileSizes[i] + G entries (a row tile
// never spans two groups, so there are at most that many tiles); maps are stored back to back.
__host__ __device__ inline long tile_map_capacity(int i, long rows_bound, int G) { return rows_bound / kTileSizes[i] + G; }
__host__ __device__ inline long tile_map_offset(int i, long rows_bound, int G) {
  long o = 0;
  for (int j = 0; j < i; j++) o += tile_map_capacity(j, rows_bound, G);
  return o;
}

// Floats of GemmArgs::gkpart needed by a K-grouped launch with output M x N.
inline long gk_part_floats(long rows_bound, int G, long M, long N) {
  return tile_map_capacity(kGkChunkTable, rows_bound, G) * M * N;
}
inline long gk_part_floats(long rows_bound, int G, long M, long N, int gkchunk) {
  return tile_map_capacity(gk_chunk_table(gkchunk), rows_bound, G) * M * N;
}
// Completes chunked K-grouped launches (made with gkpart): for every job and every group with
// several chunks, C_e = scale * (sum of the group's chunk partials, in chunk order). Up to
// kGkMaxJobs launches of one routing are completed together.
constexpr int kGkMaxJobs = 8;
constexpr int kGkMaxGroups = 1024;
hipError_t gemm_gk_reduce(const GemmArgs* jobs, int njobs, int rows_bound, hipStream_t stream);
}  // namespace moe
