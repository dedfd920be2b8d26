// Routing and data-movement kernels of the MoE-LoRA layer.
//
// Routing follows the routing equation of the ailinkdeeptech cookbook page "Accelerating
// Mixture-of-Experts Fine-Tuning" (section "The Dynamic Dispatch Bottleneck"): top-k over the
// router scores of x_t W_r, weights s_{t,i} on the selected experts. Grouping of the token-expert
// pairs into contiguous per-expert runs is a counting sort: an LDS bitmask histogram per block of
// 256 tokens gives each pair its rank among earlier tokens of the same expert, a single-workgroup
// scan turns block histograms into bases, and a scatter writes perm/inv. The result is the stable
// order (expert ascending, token ascending) and is independent of thread timing.
#include "kernels.h"
#include "gemm.h"
#include <algorithm>

namespace moe {
namespace {

// ---------------------------------------------------------------------------------------- top-k
constexpr int kMaxPerLane = 16;  // E <= 1024

// z holds nsplit partial logit arrays (split_stride floats apart), summed here in split order;
// with nsplit > 1 the sums are also written to zout. One wave per token; lane L holds experts
// L + 64 q for q < NPL (NPL >= ceil(E / 64)).
// A DPP move of a 32-bit value within rows of 16 lanes (CTRL: a gfx9 DPP control, all rows and banks).
template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ z, int nsplit,
                                                   long split_stride, float* __restrict__ zout, int s,
                                                   int E, int k, int score, int renorm,
                                                   int* __restrict__ idx, float* __restrict__ w,
                                                   float* __restrict__ psel) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= s) return;
  const float* zt = z + (long)t * E;
  // Every load of the first eight partials is issued before any of them is used, at clamped
  // expert and split indices (the surplus values are dropped), and the sums are stored only after
  // the last load: a load issued after a store would make its wait include the store.
  constexpr int NP = 8;
  float part[NPL][NP];
#pragma unroll
  for (int q = 0; q < NPL; q++) {
    const int e = min(lane + 64 * q, E - 1);
#pragma unroll
    for (int pp = 0; pp < NP; pp++) part[q][pp] = zt[(long)min(pp, nsplit - 1) * split_stride + e];
  }
  float v[NPL];
  unsigned taken = 0;
#pragma unroll
  for (int q = 0; q < NPL; q++) {
    float acc = part[q][0];  // partials added in split order
#pragma unroll
    for (int pp = 1; pp < NP; pp++)
      if (pp < nsplit) acc += part[q][pp];
    v[q] = acc;
  }
  for (int p0 = NP; p0 < nsplit; p0++) {  // splits past the eighth, if any, one at a time
#pragma unroll
    for (int q = 0; q < NPL; q++) v[q] += zt[(long)p0 * split_stride + min(lane + 64 * q, E - 1)];
  }
#pragma unroll
  for (int q = 0; q < NPL; q++) {
    const int e = lane + 64 * q;
    if (e < E) {
      if (nsplit > 1 && zout) zout[(long)t * E + e] = v[q];
      // a NaN logit ranks as -inf: never selected before a number, score 0 (and every selection
      // round then finds a valid expert id, since (value, id) is a total order)
      if (v[q] != v[q]) v[q] = -INFINITY;
    } else {
      v[q] = -INFINITY;
      taken |= 1u << q;
    }
  }
  // k selection rounds; lane L keeps the values of the slots j with j % 64 == L
  float selv[NPL];
#pragma unroll
  for (int q = 0; q < NPL; q++) selv[q] = 0.0f;
  for (int j = 0; j < k; j++) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NPL; q++) {
      if (taken & (1u << q)) continue;
      const int e = lane + 64 * q;
      if (v[q] > bv || (v[q] == bv && e < bi)) { bv = v[q]; bi = e; }
    }
    // wave argmax (larger value, then lower index): quads and rows of 16 lanes through DPP moves
    // (quad xor 1 and 2, then rotations by 4 and 8 lanes within each row), the four row winners
    // through readlane
    auto take = [&](float ov, int oi) {
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    };
    take(dpp_f<0xB1>(bv), dpp_i<0xB1>(bi));    // quad_perm [1, 0, 3, 2]
    take(dpp_f<0x4E>(bv), dpp_i<0x4E>(bi));    // quad_perm [2, 3, 0, 1]
    take(dpp_f<0x124>(bv), dpp_i<0x124>(bi));  // row_ror 4
    take(dpp_f<0x128>(bv), dpp_i<0x128>(bi));  // row_ror 8
    {
      const float v16 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16));
      const int i16 = __builtin_amdgcn_readlane(bi, 16);
      const float v32 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 32));
      const int i32 = __builtin_amdgcn_readlane(bi, 32);
      const float v48 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 48));
      const int i48 = __builtin_amdgcn_readlane(bi, 48);
      bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
      bi = __builtin_amdgcn_readlane(bi, 0);
      take(v16, i16);
      take(v32, i32);
      take(v48, i48);
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if ((j & 63) == lane) {
      idx[(long)t * k + j] = bi;
#pragma unroll
      for (int q = 0; q < NPL; q++)
        if (q == (j >> 6)) selv[q] = bv;
    }
  }
  // scores of the selected experts
  float p[NPL];
  float ps = 0.0f;
  if (score == 0) {  // softmax over all E, max-subtracted (the max is the first selection)
    const float zmax = __shfl(selv[0], 0, 64);
    float part_sum = 0.0f;
#pragma unroll
    for (int q = 0; q < NPL; q++)
      if (lane + 64 * q < E) part_sum += expf(v[q] - zmax);
    const float denom = wave_sum(part_sum);
#pragma unroll
    for (int q = 0; q < NPL; q++) {
      p[q] = (q << 6) + lane < k ? expf(selv[q] - zmax) / denom : 0.0f;
      ps += p[q];
    }
  } else {  // sigmoid
#pragma unroll
    for (int q = 0; q < NPL; q++) {
      p[q] = (q << 6) + lane < k ? 1.0f / (1.0f + expf(-selv[q])) : 0.0f;
      ps += p[q];
    }
  }
  ps = wave_sum(ps);
#pragma unroll
  for (int q = 0; q < NPL; q++) {
    if ((q << 6) + lane < k) {
      const long o = (long)t * k + (q << 6) + lane;
      psel[o] = p[q];
      w[o] = renorm ? p[q] / ps : p[q];
    }
  }
}

// ------------------------------------------------------------------------- histogram and ranks
__global__ __launch_bounds__(256) void hist_rank_kernel(const int* __restrict__ idx, int s, int k,
                                                        int E, int* __restrict__ blk_hist,
                                                        int* __restrict__ rank) {
  extern __shared__ unsigned long long lds_masks[];      // [4][E] token bitmasks per wave
  int* wpre = reinterpret_cast<int*>(lds_masks + 4 * E);  // [4][E] per-wave prefix counts
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int t = blockIdx.x * kRouteBlockTokens + tid;
  for (int i = tid; i < 4 * E; i += 256) lds_masks[i] = 0ull;
  __syncthreads();
  if (t < s)
    for (int j = 0; j < k; j++) atomicOr(&lds_masks[wv * E + idx[(long)t * k + j]], 1ull << lane);
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int acc = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      wpre[q * E + e] = acc;
      acc += __popcll(lds_masks[q * E + e]);
    }
    blk_hist[(long)blockIdx.x * E + e] = acc;
  }
  __syncthreads();
  if (t < s) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; j++) {
      const int e = idx[(long)t * k + j];
      rank[(long)t * k + j] = wpre[wv * E + e] + __popcll(lds_masks[wv * E + e] & below);
    }
  }
}

// kKeep: per-block counts kept in registers up to this many blocks (past it they are read twice)
template <int kKeep>
__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ blk_hist, int nb, int E,
                                                    int P, int* __restrict__ blk_base,
                                                    int* __restrict__ off,
                                                    int* __restrict__ tile_tables,
                                                    int* __restrict__ tile_maps) {
  constexpr int NV = 1 + kNumTileSizes;  // expert row count, then its row-tile count in every table
  __shared__ int wsum[16][NV];
  const int e = threadIdx.x, lane = e & 63, wv = e >> 6;
  const bool keep = nb <= kKeep;
  // per-block counts of expert e (one pass; all loads in flight together)
  int h[kKeep];
  int cnt = 0;
  if (e < E) {
    if (keep) {
#pragma unroll
      for (int b = 0; b < kKeep; b++) {  // unconditional loads (clamped block index), issued together
        const int v0 = blk_hist[(long)min(b, nb - 1) * E + e];
        h[b] = b < nb ? v0 : 0;
      }
#pragma unroll
      for (int b = 0; b < kKeep; b++) cnt += h[b];
    } else {
      for (int b0 = 0; b0 < nb; b0 += 8) {
        int t[8];
#pragma unroll
        for (int bb = 0; bb < 8; bb++) {
          const int v0 = blk_hist[(long)min(b0 + bb, nb - 1) * E + e];
          t[bb] = b0 + bb < nb ? v0 : 0;
        }
#pragma unroll
        for (int bb = 0; bb < 8; bb++) cnt += t[bb];
      }
    }
  }
  // the values to scan over experts: the row count and the row-tile counts (the K-grouped chunk table
  // gives an empty group one empty chunk, which writes its zeros)
  int v[NV], x[NV];
  v[0] = e < E ? cnt : 0;
#pragma unroll
  for (int i = 0; i < kNumTileSizes; i++) {
    const int bm = kTileSizes[i];
    v[1 + i] = e < E ? (i == kGkChunkTable ? max(1, (cnt + bm - 1) / bm) : (cnt + bm - 1) / bm) : 0;
  }
  // one block-wide exclusive scan of all NV values: wave scans, then the wave totals through LDS
#pragma unroll
  for (int j = 0; j < NV; j++) {
    x[j] = v[j];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x[j], o, 64);
      if (lane >= o) x[j] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < NV; j++) wsum[wv][j] = x[j];
  }
  __syncthreads();
  int base[NV], tot[NV];
#pragma unroll
  for (int j = 0; j < NV; j++) base[j] = tot[j] = 0;
#pragma unroll 2
  for (int w = 0; w < 16; w++) {
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int t = wsum[w][j];
      if (w < wv) base[j] += t;
      tot[j] += t;
    }
  }
  // offsets and per-block bases
  if (e < E) {
    const int start = base[0] + x[0] - v[0];
    off[e] = start;
    int run = start;
    if (keep) {
#pragma unroll
      for (int b = 0; b < kKeep; b++) {
        if (b < nb) blk_base[(long)b * E + e] = run;
        run += h[b];
      }
    } else {
      for (int b0 = 0; b0 < nb; b0 += 8) {
        int t[8];
#pragma unroll
        for (int bb = 0; bb < 8; bb++) {
          const int v0 = blk_hist[(long)min(b0 + bb, nb - 1) * E + e];
          t[bb] = b0 + bb < nb ? v0 : 0;
        }
#pragma unroll
        for (int bb = 0; bb < 8; bb++) {
          if (b0 + bb < nb) {
            blk_base[(long)(b0 + bb) * E + e] = run;
            run += t[bb];
          }
        }
      }
    }
  }
  if (e == 0) off[E] = tot[0];
  // row-tile prefix sums of every table, and their row tile -> group maps: the thread of group e
  // writes the entries of e's own tiles (no search, no second barrier)
#pragma unroll
  for (int i = 0; i < kNumTileSizes; i++) {
    const int ts = base[1 + i] + x[1 + i] - v[1 + i];
    if (e < E) tile_tables[i * (E + 1) + e] = ts;
    if (e == 0) tile_tables[i * (E + 1) + E] = tot[1 + i];
    if (e < E) {
      int* map = tile_maps + tile_map_offset(i, P, E) + ts;
      for (int t = 0; t < v[1 + i]; t++) map[t] = e;
    }
  }
}

__global__ void scatter_kernel(const int* __restrict__ idx, const int* __restrict__ rank,
                               const int* __restrict__ blk_base, int s, int k, int E,
                               int* __restrict__ perm, int* __restrict__ inv,
                               int* __restrict__ row_tok) {
  const long p = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= (long)s * k) return;
  const int t = (int)(p / k);
  const int e = idx[p];
  const int pos = blk_base[(long)(t / kRouteBlockTokens) * E + e] + rank[p];
  perm[pos] = (int)p;
  inv[p] = pos;
  row_tok[pos] = t;
}

// --------------------------------------------------------------------------- data movement
// Rows are moved as 16-byte chunks; row_elems * sizeof(T) is a multiple of 16.
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  static constexpr int N = 8;
  __device__ static void load(const bf16_t* p, float* f) {
    const i32x4_t r = *reinterpret_cast<const i32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f[2 * i] = bf16_to_f32((bf16_t)(r[i] & 0xffff));
      f[2 * i + 1] = bf16_to_f32((bf16_t)((unsigned)r[i] >> 16));
    }
  }
  __device__ static void store(bf16_t* p, const float* f) {
    i32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; i++)
      r[i] = (int)((unsigned)f32_to_bf16(f[2 * i]) | ((unsigned)f32_to_bf16(f[2 * i + 1]) << 16));
    *reinterpret_cast<i32x4_t*>(p) = r;
  }
};
template <> struct Vec8<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* f) {
    const f32x4_t r = *reinterpret_cast<const f32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) f[i] = r[i];
  }
  __device__ static void store(float* p, const float* f) {
    f32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; i++) r[i] = f[i];
    *reinterpret_cast<f32x4_t*>(p) = r;
  }
};

// The expert rows of one token are gathered in groups of up to kRowGroup, all loads of a group in
// flight together (the token's k rows lie anywhere in the grouped order).
constexpr int kRowGroup = 8;

// One block per token; threads walk the row in 16-byte chunks.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ o, const int* __restrict__ inv,
                                                      const float* __restrict__ w, T* __restrict__ Y,
                                                      int k, int m) {
  constexpr int V = Vec8<T>::N;
  const long t = blockIdx.x;
  for (int c = threadIdx.x; c * V < m; c += blockDim.x) {
    float acc[V] = {};
    for (int j0 = 0; j0 < k; j0 += kRowGroup) {
      // unconditional loads (a slot past the token's last reads the last one, with weight 0) so that
      // the group's rows are all in flight together
      float f[kRowGroup][V], wj[kRowGroup];
#pragma unroll
      for (int jj = 0; jj < kRowGroup; jj++) {
        const int j = min(j0 + jj, k - 1);
        const float wv = w[t * k + j];
        wj[jj] = j0 + jj < k ? wv : 0.0f;
        Vec8<T>::load(o + (long)inv[t * k + j] * m + c * V, f[jj]);
      }
#pragma unroll
      for (int jj = 0; jj < kRowGroup; jj++) {
        if (j0 + jj < k) {
#pragma unroll
          for (int i = 0; i < V; i++) acc[i] += wj[jj] * f[jj][i];
        }
      }
    }
    Vec8<T>::store(Y + t * m + c * V, acc);
  }
}
// One block per group of whole tokens (256 / k of them), in three steps through LDS:
// 1. each pair adds up its ds partials (ds[p] = sum over q < nparts of part[q * P + p], in order of q;
//    coalesced over p, sixteen partials in flight at a time) and loads its w and psel;
// 2. one thread per token forms wds = sum_j w_j ds_j and S = sum_j psel_j (slots in order);
// 3. each pair forms its dz.
// Every load of a step is issued before its values are used and no load follows a store.
constexpr int kRouterMaxK = 1024;
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ part, int nparts,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ psel, int s, int k,
                                                         int score, int renorm, float* __restrict__ dz) {
  constexpr int NB = kRouterMaxK > 256 ? kRouterMaxK : 256;
  __shared__ float dsh[NB], wsh[NB], psh[NB];
  __shared__ float twds[256], tS[256];
  const int TB = max(1, 256 / k);
  const long t0 = (long)blockIdx.x * TB;
  const int ntok = (int)min((long)TB, (long)s - t0);
  const long P = (long)s * k, p0 = t0 * k;
  constexpr int NQ = 16;
  for (int i = threadIdx.x; i < ntok * k; i += blockDim.x) {
    const float* pp = part + p0 + i;
    const float wv = w[p0 + i], pv = psel[p0 + i];
    float v = 0.0f;
    for (int q0 = 0; q0 < nparts; q0 += NQ) {
      float f[NQ];
#pragma unroll
      for (int q = 0; q < NQ; q++) f[q] = pp[(long)min(q0 + q, nparts - 1) * P];
#pragma unroll
      for (int q = 0; q < NQ; q++)
        if (q0 + q < nparts) v += f[q];
    }
    dsh[i] = v;
    wsh[i] = wv;
    psh[i] = pv;
  }
  __syncthreads();
  for (int tt = threadIdx.x; tt < ntok; tt += blockDim.x) {
    float wds = 0.0f, S = 0.0f;
    for (int j = 0; j < k; j++) {
      wds += wsh[tt * k + j] * dsh[tt * k + j];
      S += psh[tt * k + j];
    }
    twds[tt] = wds;
    tS[tt] = S;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ntok * k; i += blockDim.x) {
    const int tt = i / k;
    const float d = dsh[i], wj = wsh[i], pj = psh[i], wds = twds[tt];
    float g;
    if (score == 0) g = wj * (d - wds);  // softmax + renormalise
    else if (renorm) g = pj * (1.0f - pj) / tS[tt] * (d - wds);
    else g = pj * (1.0f - pj) * d;
    dz[p0 + i] = g;
  }
}

template <typename T>
__global__ void transpose_kernel(const T* __restrict__ W, T* __restrict__ WT, int rows, int cols) {
  __shared__ T tile[32][33];
  W += (long)blockIdx.z * rows * cols;  // one matrix of a batch per blockIdx.z
  WT += (long)blockIdx.z * rows * cols;
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int yy = ty; yy < 32; yy += 8) {
    const int r = by + yy, c = bx + tx;
    if (r < rows && c < cols) tile[yy][tx] = W[(long)r * cols + c];
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int r = bx + yy, c = by + tx;  // output row = input column
    if (r < cols && c < rows) WT[(long)r * rows + c] = tile[tx][yy];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void unpermute_kernel(const T* __restrict__ dXp, const int* __restrict__ inv,
                                                        const float* __restrict__ dz,
                                                        const int* __restrict__ idx,
                                                        const T* __restrict__ WrT, T* __restrict__ dX,
                                                        int k, int m) {
  constexpr int V = Vec8<T>::N;
  const long t = blockIdx.x;
  for (int c = threadIdx.x; c * V < m; c += blockDim.x) {
    float acc[V] = {};
    for (int j0 = 0; j0 < k; j0 += kRowGroup) {
      // unconditional loads (a slot past the token's last reads the last one and is dropped)
      float f[kRowGroup][V];
#pragma unroll
      for (int jj = 0; jj < kRowGroup; jj++)
        Vec8<T>::load(dXp + (long)inv[t * k + min(j0 + jj, k - 1)] * m + c * V, f[jj]);
#pragma unroll
      for (int jj = 0; jj < kRowGroup; jj++) {
        if (j0 + jj < k) {
#pragma unroll
          for (int i = 0; i < V; i++) acc[i] += f[jj][i];
        }
      }
      if (dz) {
        float g[kRowGroup];
#pragma unroll
        for (int jj = 0; jj < kRowGroup; jj++) {
          const int j = min(j0 + jj, k - 1);
          g[jj] = dz[t * k + j];
          Vec8<T>::load(WrT + (long)idx[t * k + j] * m + c * V, f[jj]);
        }
#pragma unroll
        for (int jj = 0; jj < kRowGroup; jj++) {
          if (j0 + jj < k) {
#pragma unroll
            for (int i = 0; i < V; i++) acc[i] += g[jj] * f[jj][i];
          }
        }
      }
    }
    Vec8<T>::store(dX + t * m + c * V, acc);
  }
}
// W' = W + c A B over one projection block of every expert: element (i, j) of the block
// (i < K over the reduction axis, j < N over the outputs) is Wo[e * wstride + off(i, j)] with
// off = i * ld + j + col0 (x.W orientation, kx) or (j + col0) * ld + i (output-major); A is
// [E, K, r], B is [E, r, N]. Threads run along the contiguous axis of W; in the x.W orientation
// each thread owns V consecutive outputs (one 16-byte chunk; N is a multiple of 8).
template <typename T>
__global__ __launch_bounds__(256) void merge_kx_kernel(const T* __restrict__ W, const T* __restrict__ A,
                                                       const T* __restrict__ B, T* __restrict__ Wo,
                                                       int K, int N, int r, long ld, long col0,
                                                       long wstride, float c) {
  constexpr int V = Vec8<T>::N;
  const long e = blockIdx.y;
  const int cpr = N / V;  // chunks per row
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)K * cpr) return;
  const int i = (int)(idx / cpr), j = (int)(idx % cpr) * V;
  const T* Ai = A + (e * K + i) * r;
  const T* Bj = B + e * r * N + j;
  float acc[V] = {};
  for (int q0 = 0; q0 < r; q0 += V) {  // r is a multiple of V (8 for bf16, 4 for fp32)
    float a[V];
    Vec8<T>::load(Ai + q0, a);
#pragma unroll
    for (int q = 0; q < V; q++) {
      float b[V];
      Vec8<T>::load(Bj + (long)(q0 + q) * N, b);
#pragma unroll
      for (int u = 0; u < V; u++) acc[u] += a[q] * b[u];
    }
  }
  const long off = e * wstride + (long)i * ld + j + col0;
  float w[V];
  Vec8<T>::load(W + off, w);
#pragma unroll
  for (int u = 0; u < V; u++) w[u] += c * acc[u];
  Vec8<T>::store(Wo + off, w);
}
template <typename T>
__global__ __launch_bounds__(256) void merge_xk_kernel(const T* __restrict__ W, const T* __restrict__ A,
                                                       const T* __restrict__ B, T* __restrict__ Wo,
                                                       int K, int N, int r, long ld, long col0,
                                                       long wstride, float c) {
  const long e = blockIdx.z;
  const int i = blockIdx.x * 256 + threadIdx.x, j = blockIdx.y;
  if (i >= K) return;
  const T* Ai = A + (e * K + i) * r;
  const T* Bj = B + e * r * N + j;
  float acc = 0.0f;
  for (int q = 0; q < r; q++) acc += to_f(Ai[q]) * to_f(Bj[(long)q * N]);
  const long off = e * wstride + (long)(j + col0) * ld + i;
  Wo[off] = from_f<T>(to_f(W[off]) + c * acc);
}

__global__ void one_group_tables_kernel(int rows, int* off, int* tiles, int* maps, long nmaps) {
  const int t = threadIdx.x;
  if (blockIdx.x == 0) {
    if (t == 0) {
      off[0] = 0;
      off[1] = rows;
    }
    if (t < kNumTileSizes) {
      const int bm = kTileSizes[t];
      const int n = (rows + bm - 1) / bm;
      tiles[t * 2] = 0;
      tiles[t * 2 + 1] = t == kGkChunkTable ? max(1, n) : n;  // as launch_scan: >= 1 chunk per group
    }
  }
  for (long i = (long)blockIdx.x * blockDim.x + t; i < nmaps; i += (long)gridDim.x * blockDim.x) maps[i] = 0;
}

// Two independent jobs of the routed backward in one launch: blocks [0, rw_blocks) form the row-weighted
// rows out[i, :] = w[pair[i]] * in[i, :]; the blocks after them transpose W [trows, tcols] into
// WT [tcols, trows] in 32 x 32 tiles (as transpose_kernel), when W is given.
template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const T* __restrict__ in, const int* __restrict__ pair,
                                                       const float* __restrict__ w, T* __restrict__ out,
                                                       long rows, int cols, int rw_blocks,
                                                       const T* __restrict__ W, T* __restrict__ WT, int trows,
                                                       int tcols) {
  if ((int)blockIdx.x < rw_blocks) {
    const long n = rows * cols;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)rw_blocks * blockDim.x)
      out[i] = from_f<T>(w[pair[i / cols]] * to_f(in[i]));
    return;
  }
  __shared__ T tile[32][33];
  const int gx = (tcols + 31) / 32;
  const int tb = (int)blockIdx.x - rw_blocks;
  const int bx = (tb % gx) * 32, by = (tb / gx) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int yy = ty; yy < 32; yy += 8) {
    const int r = by + yy, c = bx + tx;
    if (r < trows && c < tcols) tile[yy][tx] = W[(long)r * tcols + c];
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int r = bx + yy, c = by + tx;  // output row = input column
    if (r < tcols && c < trows) WT[(long)r * trows + c] = tile[tx][yy];
  }
}

__global__ void pad_cols_kernel(const bf16_t* __restrict__ W, bf16_t* __restrict__ Wp, int rows, int cols,
                                int ld) {
  const long n = (long)rows * ld;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const long r = i / ld;
    const int c = (int)(i - r * ld);
    Wp[i] = c < cols ? W[r * cols + c] : (bf16_t)0;
  }
}

__global__ void zero_kernel(int* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

hipError_t launch_topk(const float* z, int nsplit, long split_stride, float* zout, int s, int E,
                       int k, int score, int renorm, int* idx, float* w, float* psel, hipStream_t st) {
  if (s <= 0) return hipSuccess;
  const dim3 grid((s + 3) / 4);
  const int npl = (E + 63) / 64;
  if (npl <= 1)
    hipLaunchKernelGGL(topk_kernel<1>, grid, dim3(256), 0, st, z, nsplit, split_stride, zout, s, E, k, score,
                       renorm, idx, w, psel);
  else if (npl <= 2)
    hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(256), 0, st, z, nsplit, split_stride, zout, s, E, k, score,
                       renorm, idx, w, psel);
  else if (npl <= 4)
    hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, st, z, nsplit, split_stride, zout, s, E, k, score,
                       renorm, idx, w, psel);
  else if (npl <= 8)
    hipLaunchKernelGGL(topk_kernel<8>, grid, dim3(256), 0, st, z, nsplit, split_stride, zout, s, E, k, score,
                       renorm, idx, w, psel);
  else if (npl <= kMaxPerLane)
    hipLaunchKernelGGL(topk_kernel<kMaxPerLane>, grid, dim3(256), 0, st, z, nsplit, split_stride, zout, s, E, k,
                       score, renorm, idx, w, psel);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_hist_rank(const int* idx, int s, int k, int E, int* blk_hist, int* rank,
                            hipStream_t st) {
  if (s <= 0) return hipSuccess;
  const int nb = (s + kRouteBlockTokens - 1) / kRouteBlockTokens;
  const size_t lds = (size_t)4 * E * sizeof(unsigned long long) + (size_t)4 * E * sizeof(int);
  hipLaunchKernelGGL(hist_rank_kernel, dim3(nb), dim3(256), lds, st, idx, s, k, E, blk_hist, rank);
  return hipGetLastError();
}

hipError_t launch_scan(const int* blk_hist, int nb, int E, int P, int* blk_base, int* off,
                       int* tile_tables, int* tile_maps, hipStream_t st) {
  if (nb <= 16)
    hipLaunchKernelGGL(scan_kernel<16>, dim3(1), dim3(1024), 0, st, blk_hist, nb, E, P, blk_base, off,
                       tile_tables, tile_maps);
  else
    hipLaunchKernelGGL(scan_kernel<64>, dim3(1), dim3(1024), 0, st, blk_hist, nb, E, P, blk_base, off,
                       tile_tables, tile_maps);
  return hipGetLastError();
}

hipError_t launch_scatter(const int* idx, const int* rank, const int* blk_base, int s, int k, int E,
                          int* perm, int* inv, int* row_tok, hipStream_t st) {
  const long P = (long)s * k;
  if (P <= 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, st, idx, rank,
                     blk_base, s, k, E, perm, inv, row_tok);
  return hipGetLastError();
}


hipError_t launch_combine(int dtype, const void* o, const int* inv, const float* w, void* Y, int s,
                          int k, int m, hipStream_t st) {
  if (s <= 0) return hipSuccess;
  if (dtype)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(s), dim3(256), 0, st, (const bf16_t*)o, inv, w,
                       (bf16_t*)Y, k, m);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(s), dim3(256), 0, st, (const float*)o, inv, w,
                       (float*)Y, k, m);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* ds_part, int nparts, const float* w, const float* psel, int s, int k,
                             int score, int renorm, float* dz, hipStream_t st) {
  if (s <= 0) return hipSuccess;
  if (k > kRouterMaxK) return hipErrorInvalidValue;
  const int TB = std::max(1, 256 / k);
  hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)((s + TB - 1) / TB)), dim3(256), 0, st, ds_part, nparts, w,
                     psel, s, k, score, renorm, dz);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, const void* W, void* WT, int rows, int cols, int batch,
                            hipStream_t st) {
  if (rows <= 0 || cols <= 0 || batch <= 0) return hipSuccess;
  dim3 grid((cols + 31) / 32, (rows + 31) / 32, batch);
  if (dtype)
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)W, (bf16_t*)WT,
                       rows, cols);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, st, (const float*)W, (float*)WT,
                       rows, cols);
  return hipGetLastError();
}

hipError_t launch_unpermute(int dtype, const void* dXp, const int* inv, const float* dz,
                            const int* idx, const void* WrT, void* dX, int s, int k, int m,
                            hipStream_t st) {
  if (s <= 0) return hipSuccess;
  if (dtype)
    hipLaunchKernelGGL(unpermute_kernel<bf16_t>, dim3(s), dim3(256), 0, st, (const bf16_t*)dXp, inv,
                       dz, idx, (const bf16_t*)WrT, (bf16_t*)dX, k, m);
  else
    hipLaunchKernelGGL(unpermute_kernel<float>, dim3(s), dim3(256), 0, st, (const float*)dXp, inv, dz,
                       idx, (const float*)WrT, (float*)dX, k, m);
  return hipGetLastError();
}

hipError_t launch_one_group_tables(int rows, int* off, int* tile_tables, int* tile_maps, hipStream_t st) {
  const long nmaps = tile_map_offset(kNumTileSizes, rows, 1);
  const long blocks = std::min<long>((nmaps + 255) / 256, 1024);
  hipLaunchKernelGGL(one_group_tables_kernel, dim3((unsigned)std::max<long>(blocks, 1)), dim3(256), 0, st, rows,
                     off, tile_tables, tile_maps, nmaps);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(int dtype, const void* in, const int* pair, const float* w, void* out, long rows,
                           int cols, const void* W, void* WT, int trows, int tcols, hipStream_t st) {
  const long n = rows * cols;
  const int rw_blocks = (int)std::min<long>((n + 255) / 256, 2048);
  const int tr_blocks = W ? ((tcols + 31) / 32) * ((trows + 31) / 32) : 0;
  if (rw_blocks + tr_blocks <= 0) return hipSuccess;
  if (dtype)
    hipLaunchKernelGGL(bwd_prep_kernel<bf16_t>, dim3((unsigned)(rw_blocks + tr_blocks)), dim3(256), 0, st,
                       (const bf16_t*)in, pair, w, (bf16_t*)out, rows, cols, rw_blocks, (const bf16_t*)W,
                       (bf16_t*)WT, trows, tcols);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<float>, dim3((unsigned)(rw_blocks + tr_blocks)), dim3(256), 0, st,
                       (const float*)in, pair, w, (float*)out, rows, cols, rw_blocks, (const float*)W,
                       (float*)WT, trows, tcols);
  return hipGetLastError();
}

hipError_t launch_pad_cols(const void* W, void* Wp, int rows, int cols, int ld, hipStream_t st) {
  const long n = (long)rows * ld;
  if (n <= 0) return hipSuccess;
  const long blocks = std::min<long>((n + 255) / 256, 2048);
  hipLaunchKernelGGL(pad_cols_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const bf16_t*)W, (bf16_t*)Wp, rows,
                     cols, ld);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t words, hipStream_t st) {
  if (words == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((words + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (int*)p, words);
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, bool kx, const void* W, const void* A, const void* B, void* Wo,
                        int E, int K, int N, int r, long ld, long col0, long wstride, float c,
                        hipStream_t st) {
  if (E <= 0 || K <= 0 || N <= 0) return hipSuccess;
  if (kx) {
    const int V = dtype ? 8 : 4;
    if (N % 8 || r % V) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(((long)K * (N / V) + 255) / 256), (unsigned)E);
    if (dtype)
      hipLaunchKernelGGL(merge_kx_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)W,
                         (const bf16_t*)A, (const bf16_t*)B, (bf16_t*)Wo, K, N, r, ld, col0, wstride, c);
    else
      hipLaunchKernelGGL(merge_kx_kernel<float>, grid, dim3(256), 0, st, (const float*)W,
                         (const float*)A, (const float*)B, (float*)Wo, K, N, r, ld, col0, wstride, c);
  } else {
    const dim3 grid((unsigned)((K + 255) / 256), (unsigned)N, (unsigned)E);
    if (dtype)
      hipLaunchKernelGGL(merge_xk_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)W,
                         (const bf16_t*)A, (const bf16_t*)B, (bf16_t*)Wo, K, N, r, ld, col0, wstride, c);
    else
      hipLaunchKernelGGL(merge_xk_kernel<float>, grid, dim3(256), 0, st, (const float*)W,
                         (const float*)A, (const float*)B, (float*)Wo, K, N, r, ld, col0, wstride, c);
  }
  return hipGetLastError();
}

}  // namespace moe
