// Grouped GEMM kernels for the expert projections and the LoRA-factor gradients.
//
// MFMA path (bf16 in, fp32 accumulate): v_mfma_f32_32x32x16_bf16 tiles, 256-thread workgroups,
// global -> register -> LDS double buffering over K tiles of 64, one extra K tile for the Split-LoRA
// tail (alpha/r * (X A) B added as K-extension [X | cXA] . [W ; B]), and fused epilogues.
// Operands stored with the reduction axis contiguous are read from LDS with ds_read_b128; operands
// stored with the output axis contiguous (the x.W weight orientation) are read with gfx950's
// transposing LDS read ds_read_b64_tr_b16, so neither orientation needs a transposed copy.
// Work is split into (group, row tile, column tile) units; consecutive units go to the same XCD
// so the workgroups sharing an expert's weight tile share that XCD's L2.
//
// SIMT path: one thread per output element with the same GemmArgs semantics, used for fp32 layers
// and as a reference for the MFMA kernels.
#include "gemm.h"
#include <algorithm>

namespace moe {

int tile_table_index(int bm) {
  for (int i = 0; i < kNumTileSizes; i++)
    if (kTileSizes[i] == bm) return i;
  return -1;
}

namespace {

constexpr int BK = 64;    // K tile
constexpr int PADE = 8;   // LDS row padding (elements)

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;

__device__ inline bf16x4_t lds_read_tr(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)((lds_bf16_t*)p));
}

// Fragment of a 32x32x16 MFMA operand from an LDS tile whose reduction axis is contiguous
// (element (x, kk) at tile[x*LD + kk]): lane l holds x0 + l%32, kk = k0 + 8*(l/32) .. +7.
__device__ inline bf16x8_t frag_xk(const bf16_t* tile, int LD, int x0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8_t*>(tile + (x0 + (lane & 31)) * LD + k0 + 8 * (lane >> 5));
}

// Same fragment from a tile whose output axis is contiguous (element (x, kk) at tile[kk*LD + x]).
// Within each 16-lane group, ds_read_b64_tr_b16 gathers a 4 (kk) x 16 (x) block: lane (b, c) names
// row b, columns 4c..4c+3, and lane L receives column L of the 4 rows. Two reads give 8 kk values.
__device__ inline bf16x8_t frag_kx(const bf16_t* tile, int LD, int x0, int k0, int lane) {
  const int g = lane >> 4, b = (lane >> 2) & 3, c = lane & 3;
  const bf16_t* p = tile + (k0 + 8 * (g >> 1) + b) * LD + x0 + 16 * (g & 1) + 4 * c;
  bf16x4_t lo = lds_read_tr(p);
  bf16x4_t hi = lds_read_tr(p + 4 * LD);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline i32x4_t ld16(const bf16_t* p) { return *reinterpret_cast<const i32x4_t*>(p); }

__device__ inline float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// Maps blockIdx to a logical work unit so that each XCD (blockIdx % 8) receives a contiguous range
// of units. Returns -1 for surplus blocks.
__device__ inline int xcd_unit(int total) {
  const int per = (total + 7) >> 3;
  const int b = blockIdx.x;
  const int pos = b >> 3;
  if (pos >= per) return -1;
  const int T = (b & 7) * per + pos;
  return T < total ? T : -1;
}

// ------------------------------------------------------------------------------------------------
// Row-grouped MFMA GEMM.
template <int WM, int WN, int TM, int TN, int BL, int EPI, typename OutT>
__global__ __launch_bounds__(WM * WN * 64) void gm_mfma(GemmArgs a, int tidx) {
  constexpr bool DUAL = (EPI == EPI_DUAL || EPI == EPI_SWIGLU);
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32, NT = WM * WN * 64;
  constexpr int BNH = DUAL ? BN / 2 : BN;
  constexpr int LDA = BK + PADE;
  constexpr int LDB = (BL == LAYOUT_XK) ? BK + PADE : BN + PADE;
  constexpr int A_ELEMS = BM * LDA;
  constexpr int B_ELEMS = (BL == LAYOUT_XK) ? BN * LDB : BK * LDB;
  constexpr int STAGE = A_ELEMS + B_ELEMS;
  constexpr int A_PT = BM * BK / 8 / NT;
  constexpr int B_PT = BN * BK / 8 / NT;
  constexpr int CPR_B = BN / 8;  // chunks per KX B row
  static_assert((BM * BK / 8) % NT == 0 && (BN * BK / 8) % NT == 0, "tile/thread mismatch");
  static_assert(!DUAL || (TN % 2 == 0), "dual epilogue needs an even TN");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- which (group, row tile, column tile)
  const int tilesN = (a.N + BNH - 1) / BNH;
  const int* toff = a.goff ? a.toff_all + tidx * (a.G + 1) : nullptr;
  const int mtiles = a.goff ? toff[a.G] : (a.M + BM - 1) / BM;
  const int T = xcd_unit(mtiles * tilesN);
  if (T < 0) return;
  int e = 0, row0, row_end, nt;
  if (a.goff) {
    int lo = 0, hi = a.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (toff[mid] * tilesN <= T) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int nte = toff[e + 1] - toff[e];
    const int local = T - toff[e] * tilesN;
    nt = local / nte;
    row0 = a.goff[e] + (local - nt * nte) * BM;
    row_end = a.goff[e + 1];
  } else {
    const int mt = (a.M + BM - 1) / BM;
    nt = T / mt;
    row0 = (T - nt * mt) * BM;
    row_end = a.M;
  }
  const int j0 = nt * BNH;

  // ---- per-thread global chunk pointers
  const bf16_t* aptr[A_PT];
  int arowc[A_PT];
#pragma unroll
  for (int u = 0; u < A_PT; u++) {
    const int c = tid + u * NT;
    const int row = min(row0 + (c >> 3), row_end - 1);
    arowc[u] = row;
    const long src = a.arow ? (long)(a.arow[row] / a.arow_div) : (long)row;
    aptr[u] = (const bf16_t*)a.A + src * a.lda + (c & 7) * 8;
  }
  const bf16_t* Bg = (const bf16_t*)a.B + (long)e * a.bstride;
  const bf16_t* Bug = DUAL ? (const bf16_t*)a.Bu + (long)e * a.bstride : nullptr;
  const bf16_t* bptr[B_PT];
#pragma unroll
  for (int u = 0; u < B_PT; u++) {
    const int c = tid + u * NT;
    if (BL == LAYOUT_KX) {
      const int kk = c / CPR_B, x = (c % CPR_B) * 8;
      const int half = DUAL ? (x >= BNH) : 0;
      const int jj = min(j0 + x - half * BNH, a.N - 8);
      bptr[u] = (half ? Bug : Bg) + (long)kk * a.ldb + jj;
    } else {
      const int x = c >> 3, q = c & 7;
      const int half = DUAL ? (x >= BNH) : 0;
      const int jj = min(j0 + x - half * BNH, a.N - 1);
      bptr[u] = (half ? Bug : Bg) + (long)jj * a.ldb + q * 8;
    }
  }

  i32x4_t ra[A_PT], rb[B_PT];
  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < A_PT; u++) ra[u] = ld16(aptr[u] + k0);
#pragma unroll
    for (int u = 0; u < B_PT; u++)
      rb[u] = ld16(bptr[u] + (BL == LAYOUT_KX ? (long)k0 * a.ldb : (long)k0));
  };
  auto sstore = [&](int buf) {
    bf16_t* sA = smem + buf * STAGE;
    bf16_t* sB = sA + A_ELEMS;
#pragma unroll
    for (int u = 0; u < A_PT; u++) {
      const int c = tid + u * NT;
      *reinterpret_cast<i32x4_t*>(sA + (c >> 3) * LDA + (c & 7) * 8) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < B_PT; u++) {
      const int c = tid + u * NT;
      if (BL == LAYOUT_KX)
        *reinterpret_cast<i32x4_t*>(sB + (c / CPR_B) * LDB + (c % CPR_B) * 8) = rb[u];
      else
        *reinterpret_cast<i32x4_t*>(sB + (c >> 3) * LDB + (c & 7) * 8) = rb[u];
    }
  };
  auto wcol = [&](int tn) {
    if constexpr (DUAL) {
      constexpr int TH = TN / 2;
      return (tn >= TH ? BNH : 0) + wn * TH * 32 + (tn % TH) * 32;
    } else {
      return wn * TN * 32 + tn * 32;
    }
  };
  auto compute = [&](int buf) {
    const bf16_t* sA = smem + buf * STAGE;
    const bf16_t* sB = sA + A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks++) {
      bf16x8_t fa[TM], fb[TN];
#pragma unroll
      for (int tm = 0; tm < TM; tm++) fa[tm] = frag_xk(sA, LDA, wm * TM * 32 + tm * 32, ks * 16, lane);
#pragma unroll
      for (int tn = 0; tn < TN; tn++)
        fb[tn] = (BL == LAYOUT_XK) ? frag_xk(sB, LDB, wcol(tn), ks * 16, lane)
                                   : frag_kx(sB, LDB, wcol(tn), ks * 16, lane);
#pragma unroll
      for (int tm = 0; tm < TM; tm++)
#pragma unroll
        for (int tn = 0; tn < TN; tn++)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
    }
  };

  const int nk = a.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    if (kt + 1 < nk) gload((kt + 1) * BK);
    compute(kt & 1);
    if (kt + 1 < nk) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- Split-LoRA tail: one more K tile [TA | 0] . [TB ; 0]
  if (a.tail != TAIL_NONE) {
    const int r2 = a.r2a;
    const int K2 = (a.tail == TAIL_SINGLE) ? r2 : 2 * r2;
    const i32x4_t zero = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < A_PT; u++) {
      const int q = (tid + u * NT) & 7;
      ra[u] = (q * 8 < K2) ? ld16((const bf16_t*)a.TA + (long)arowc[u] * a.lda2 + q * 8) : zero;
    }
    const bf16_t* T0 = (const bf16_t*)a.TB0 + (long)e * a.tbstride;
    const bf16_t* T1 = a.TB1 ? (const bf16_t*)a.TB1 + (long)e * a.tbstride : nullptr;
#pragma unroll
    for (int u = 0; u < B_PT; u++) {
      const int c = tid + u * NT;
      const bf16_t* src = nullptr;
      if (BL == LAYOUT_KX) {
        const int kk = c / CPR_B, x = (c % CPR_B) * 8;
        const int half = DUAL ? (x >= BNH) : 0;
        const int jj = min(j0 + x - half * BNH, a.N - 8);
        if (a.tail == TAIL_SINGLE) {
          if (kk < r2) src = T0 + (long)kk * a.ldtb + jj;
        } else if (a.tail == TAIL_BLOCKDIAG) {
          if (half == 0 && kk < r2) src = T0 + (long)kk * a.ldtb + jj;
          else if (half == 1 && kk >= r2 && kk < 2 * r2) src = T1 + (long)(kk - r2) * a.ldtb + jj;
        } else {
          if (kk < r2) src = T0 + (long)kk * a.ldtb + jj;
          else if (kk < 2 * r2) src = T1 + (long)(kk - r2) * a.ldtb + jj;
        }
      } else {
        const int x = c >> 3, k8 = (c & 7) * 8;
        const int half = DUAL ? (x >= BNH) : 0;
        const int jj = min(j0 + x - half * BNH, a.N - 1);
        if (a.tail == TAIL_SINGLE) {
          if (k8 < r2) src = T0 + (long)jj * a.ldtb + k8;
        } else if (a.tail == TAIL_BLOCKDIAG) {
          if (half == 0 && k8 < r2) src = T0 + (long)jj * a.ldtb + k8;
          else if (half == 1 && k8 >= r2 && k8 < 2 * r2) src = T1 + (long)jj * a.ldtb + (k8 - r2);
        } else {
          if (k8 < r2) src = T0 + (long)jj * a.ldtb + k8;
          else if (k8 < 2 * r2) src = T1 + (long)jj * a.ldtb + (k8 - r2);
        }
      }
      rb[u] = src ? ld16(src) : zero;
    }
    sstore(nk & 1);
    __syncthreads();
    compute(nk & 1);
  }

  // ---- epilogue
  OutT* C = (OutT*)a.C;
#pragma unroll
  for (int tm = 0; tm < TM; tm++) {
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int row = row0 + wm * TM * 32 + tm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row >= row_end) continue;
      if constexpr (DUAL) {
#pragma unroll
        for (int t2 = 0; t2 < TN / 2; t2++) {
          const int jj = j0 + wn * (TN / 2) * 32 + t2 * 32 + (lane & 31);
          if (jj >= a.N) continue;
          const float g = acc[tm][t2][v], uu = acc[tm][t2 + TN / 2][v];
          if (EPI == EPI_DUAL) {
            C[(long)row * a.ldc + jj] = from_f<OutT>(a.scale * g);
            C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(a.scale * uu);
          } else {
            C[(long)row * a.ldc + jj] = from_f<OutT>(g);
            C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(uu);
            ((OutT*)a.H)[(long)row * a.ldh + jj] = from_f<OutT>(silu_f(g) * uu);
          }
        }
      } else {
#pragma unroll
        for (int tn = 0; tn < TN; tn++) {
          const int jj = j0 + wn * TN * 32 + tn * 32 + (lane & 31);
          if (jj >= a.N) continue;
          const float val = a.scale * acc[tm][tn][v];
          if (EPI == EPI_STORE) {
            C[(long)row * a.ldc + jj] = from_f<OutT>(val + (a.bias ? a.bias[jj] : 0.0f));
          } else {  // EPI_SWIGLU_BWD
            const OutT* GU = (const OutT*)a.GU;
            const float g = to_f(GU[(long)row * a.ldgu + jj]);
            const float uu = to_f(GU[(long)row * a.ldgu + a.guup + jj]);
            const float sg = 1.0f / (1.0f + __expf(-g));
            C[(long)row * a.ldc + jj] = from_f<OutT>(val * uu * sg * (1.0f + g * (1.0f - sg)));
            C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(val * g * sg);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// K-grouped MFMA GEMM: C_e = scale * L[rows_e]^T . R[rows_e]; both operands stored with the output
// axis contiguous, so both fragments come from transposing LDS reads.
template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(WM * WN * 64) void gk_mfma(GemmArgs a) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32, NT = WM * WN * 64;
  constexpr int LDA = BM + PADE, LDB = BN + PADE;
  constexpr int A_ELEMS = BK * LDA, B_ELEMS = BK * LDB, STAGE = A_ELEMS + B_ELEMS;
  constexpr int CPR_A = BM / 8, CPR_B = BN / 8;
  constexpr int A_PT = BM * BK / 8 / NT, B_PT = BN * BK / 8 / NT;
  static_assert((BM * BK / 8) % NT == 0 && (BN * BK / 8) % NT == 0, "tile/thread mismatch");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tilesM = (a.M + BM - 1) / BM, tilesN = (a.N + BN - 1) / BN;
  const int T = xcd_unit(a.G * tilesM * tilesN);
  if (T < 0) return;
  const int e = T / (tilesM * tilesN);
  const int rem = T - e * tilesM * tilesN;
  const int nt = rem / tilesM, mt = rem - nt * tilesM;
  const int kb = a.goff[e], ke = a.goff[e + 1];

  int acol[A_PT], bcol[B_PT];
#pragma unroll
  for (int u = 0; u < A_PT; u++) acol[u] = min(mt * BM + ((tid + u * NT) % CPR_A) * 8, a.M - 8);
#pragma unroll
  for (int u = 0; u < B_PT; u++) bcol[u] = min(nt * BN + ((tid + u * NT) % CPR_B) * 8, a.N - 8);

  i32x4_t ra[A_PT], rb[B_PT];
  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;
  const i32x4_t zero = {0, 0, 0, 0};

  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < A_PT; u++) {
      const int row = k0 + (tid + u * NT) / CPR_A;
      if (row < ke) {
        const long src = a.arow ? (long)(a.arow[row] / a.arow_div) : (long)row;
        ra[u] = ld16((const bf16_t*)a.A + src * a.lda + acol[u]);
      } else {
        ra[u] = zero;
      }
    }
#pragma unroll
    for (int u = 0; u < B_PT; u++) {
      const int row = k0 + (tid + u * NT) / CPR_B;
      rb[u] = row < ke ? ld16((const bf16_t*)a.B + (long)row * a.ldb + bcol[u]) : zero;
    }
  };
  auto sstore = [&](int buf) {
    bf16_t* sA = smem + buf * STAGE;
    bf16_t* sB = sA + A_ELEMS;
#pragma unroll
    for (int u = 0; u < A_PT; u++) {
      const int c = tid + u * NT;
      *reinterpret_cast<i32x4_t*>(sA + (c / CPR_A) * LDA + (c % CPR_A) * 8) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < B_PT; u++) {
      const int c = tid + u * NT;
      *reinterpret_cast<i32x4_t*>(sB + (c / CPR_B) * LDB + (c % CPR_B) * 8) = rb[u];
    }
  };
  auto compute = [&](int buf) {
    const bf16_t* sA = smem + buf * STAGE;
    const bf16_t* sB = sA + A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks++) {
      bf16x8_t fa[TM], fb[TN];
#pragma unroll
      for (int tm = 0; tm < TM; tm++) fa[tm] = frag_kx(sA, LDA, wm * TM * 32 + tm * 32, ks * 16, lane);
#pragma unroll
      for (int tn = 0; tn < TN; tn++) fb[tn] = frag_kx(sB, LDB, wn * TN * 32 + tn * 32, ks * 16, lane);
#pragma unroll
      for (int tm = 0; tm < TM; tm++)
#pragma unroll
        for (int tn = 0; tn < TN; tn++)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
    }
  };

  const int nk = (ke - kb + BK - 1) / BK;
  if (nk > 0) {
    gload(kb);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
      if (kt + 1 < nk) gload(kb + (kt + 1) * BK);
      compute(kt & 1);
      if (kt + 1 < nk) sstore((kt + 1) & 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int tm = 0; tm < TM; tm++)
#pragma unroll
    for (int tn = 0; tn < TN; tn++)
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int row = mt * BM + wm * TM * 32 + tm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        int col = nt * BN + wn * TN * 32 + tn * 32 + (lane & 31);
        if (row >= a.M || col >= a.N) continue;
        float* C = (float*)a.C;
        if (a.C1 && col >= a.nsplit) { C = (float*)a.C1; col -= a.nsplit; }
        C += (long)e * a.cstride;
        C[a.ctrans ? (long)col * a.ldc + row : (long)row * a.ldc + col] = a.scale * acc[tm][tn][v];
      }
}

// ------------------------------------------------------------------------------------------------
// SIMT reference kernels (same semantics, one output element per thread).
template <typename T>
__device__ inline float opv(const T* base, int layout, long ld, int x, int kk) {
  return to_f(layout == LAYOUT_KX ? base[(long)kk * ld + x] : base[(long)x * ld + kk]);
}

template <typename T, typename OutT, int EPI>
__global__ void gm_simt(GemmArgs a, int b_layout, int total_rows_bound) {
  constexpr bool DUAL = (EPI == EPI_DUAL || EPI == EPI_SWIGLU);
  const int row = blockIdx.x;
  const int jj = blockIdx.y * blockDim.x + threadIdx.x;
  if (jj >= a.N) return;
  int e = 0;
  if (a.goff) {
    if (row >= a.goff[a.G]) return;
    int lo = 0, hi = a.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.goff[mid] <= row) lo = mid; else hi = mid - 1;
    }
    e = lo;
  } else if (row >= a.M) {
    return;
  }
  const long src = a.arow ? (long)(a.arow[row] / a.arow_div) : (long)row;
  const T* Ar = (const T*)a.A + src * a.lda;
  const T* Bg = (const T*)a.B + (long)e * a.bstride;
  const T* Bug = DUAL ? (const T*)a.Bu + (long)e * a.bstride : nullptr;
  float acc0 = 0.0f, acc1 = 0.0f;
  for (int k = 0; k < a.K; k++) {
    const float x = to_f(Ar[k]);
    acc0 += x * opv(Bg, b_layout, a.ldb, jj, k);
    if (DUAL) acc1 += x * opv(Bug, b_layout, a.ldb, jj, k);
  }
  if (a.tail != TAIL_NONE) {
    const int r2 = a.r2a;
    const T* TAr = (const T*)a.TA + (long)row * a.lda2;
    const T* T0 = (const T*)a.TB0 + (long)e * a.tbstride;
    const T* T1 = a.TB1 ? (const T*)a.TB1 + (long)e * a.tbstride : nullptr;
    if (a.tail == TAIL_SINGLE) {
      for (int q = 0; q < r2; q++) acc0 += to_f(TAr[q]) * opv(T0, b_layout, a.ldtb, jj, q);
    } else if (a.tail == TAIL_BLOCKDIAG) {
      for (int q = 0; q < r2; q++) acc0 += to_f(TAr[q]) * opv(T0, b_layout, a.ldtb, jj, q);
      for (int q = 0; q < r2; q++) acc1 += to_f(TAr[r2 + q]) * opv(T1, b_layout, a.ldtb, jj, q);
    } else {
      for (int q = 0; q < r2; q++) acc0 += to_f(TAr[q]) * opv(T0, b_layout, a.ldtb, jj, q);
      for (int q = 0; q < r2; q++) acc0 += to_f(TAr[r2 + q]) * opv(T1, b_layout, a.ldtb, jj, q);
    }
  }
  OutT* C = (OutT*)a.C;
  if (EPI == EPI_STORE) {
    C[(long)row * a.ldc + jj] = from_f<OutT>(a.scale * acc0 + (a.bias ? a.bias[jj] : 0.0f));
  } else if (EPI == EPI_DUAL) {
    C[(long)row * a.ldc + jj] = from_f<OutT>(a.scale * acc0);
    C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(a.scale * acc1);
  } else if (EPI == EPI_SWIGLU) {
    C[(long)row * a.ldc + jj] = from_f<OutT>(acc0);
    C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(acc1);
    ((OutT*)a.H)[(long)row * a.ldh + jj] = from_f<OutT>(acc0 / (1.0f + expf(-acc0)) * acc1);
  } else {
    const OutT* GU = (const OutT*)a.GU;
    const float dh = a.scale * acc0;
    const float g = to_f(GU[(long)row * a.ldgu + jj]);
    const float uu = to_f(GU[(long)row * a.ldgu + a.guup + jj]);
    const float sg = 1.0f / (1.0f + expf(-g));
    C[(long)row * a.ldc + jj] = from_f<OutT>(dh * uu * sg * (1.0f + g * (1.0f - sg)));
    C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(dh * g * sg);
  }
}

template <typename T>
__global__ void gk_simt(GemmArgs a) {
  const int e = blockIdx.z, row = blockIdx.y;
  int col = blockIdx.x * blockDim.x + threadIdx.x;
  if (col >= a.N) return;
  const int kb = a.goff[e], ke = a.goff[e + 1];
  float acc = 0.0f;
  for (int i = kb; i < ke; i++) {
    const long src = a.arow ? (long)(a.arow[i] / a.arow_div) : (long)i;
    acc += to_f(((const T*)a.A)[src * a.lda + row]) * to_f(((const T*)a.B)[(long)i * a.ldb + col]);
  }
  float* C = (float*)a.C;
  if (a.C1 && col >= a.nsplit) { C = (float*)a.C1; col -= a.nsplit; }
  C += (long)e * a.cstride;
  C[a.ctrans ? (long)col * a.ldc + row : (long)row * a.ldc + col] = a.scale * acc;
}

// ------------------------------------------------------------------------------------------------
template <int WM, int WN, int TM, int TN, int BL, int EPI, typename OutT>
hipError_t launch_gm_mfma(const GemmArgs& a, int rows_bound, hipStream_t stream) {
  constexpr bool DUAL = (EPI == EPI_DUAL || EPI == EPI_SWIGLU);
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int BNH = DUAL ? BN / 2 : BN;
  const int tilesN = (a.N + BNH - 1) / BNH;
  const long mtiles = a.goff ? (long)rows_bound / BM + a.G : ((long)a.M + BM - 1) / BM;
  const long units = mtiles * tilesN;
  if (units <= 0) return hipSuccess;
  const long blocks = (units + 7) / 8 * 8;
  const int tidx = tile_table_index(BM);
  if (a.goff && tidx < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gm_mfma<WM, WN, TM, TN, BL, EPI, OutT>), dim3((unsigned)blocks),
                     dim3(WM * WN * 64), 0, stream, a, tidx);
  return hipGetLastError();
}

template <int BL, int EPI, typename OutT>
hipError_t dispatch_gm_mfma(const GemmArgs& a, int rows_bound, hipStream_t stream) {
  constexpr bool DUAL = (EPI == EPI_DUAL || EPI == EPI_SWIGLU);
  if constexpr (DUAL) {
    if (a.N <= 32) return launch_gm_mfma<4, 1, 1, 2, BL, EPI, OutT>(a, rows_bound, stream);
    return launch_gm_mfma<2, 2, 2, 2, BL, EPI, OutT>(a, rows_bound, stream);
  } else {
    if (a.N <= 32) return launch_gm_mfma<4, 1, 1, 1, BL, EPI, OutT>(a, rows_bound, stream);
    return launch_gm_mfma<2, 2, 2, 2, BL, EPI, OutT>(a, rows_bound, stream);
  }
}

template <typename T, typename OutT, int EPI>
hipError_t launch_gm_simt(const GemmArgs& a, int b_layout, int rows_bound, hipStream_t stream) {
  const int rows = a.goff ? rows_bound : a.M;
  if (rows <= 0 || a.N <= 0) return hipSuccess;
  hipLaunchKernelGGL((gm_simt<T, OutT, EPI>), dim3(rows, (a.N + 63) / 64), dim3(64), 0, stream, a,
                     b_layout, rows_bound);
  return hipGetLastError();
}

template <typename T, typename OutT>
hipError_t dispatch_gm_simt(const GemmArgs& a, int b_layout, int epi, int rows_bound,
                            hipStream_t stream) {
  switch (epi) {
    case EPI_STORE: return launch_gm_simt<T, OutT, EPI_STORE>(a, b_layout, rows_bound, stream);
    case EPI_DUAL: return launch_gm_simt<T, OutT, EPI_DUAL>(a, b_layout, rows_bound, stream);
    case EPI_SWIGLU: return launch_gm_simt<T, OutT, EPI_SWIGLU>(a, b_layout, rows_bound, stream);
    case EPI_SWIGLU_BWD: return launch_gm_simt<T, OutT, EPI_SWIGLU_BWD>(a, b_layout, rows_bound, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t gemm_gm_launch(const GemmArgs& a, int b_layout, int epi, int out_f32, int dtype,
                          int rows_bound, int reference, hipStream_t stream) {
  if (dtype == 0) return dispatch_gm_simt<float, float>(a, b_layout, epi, rows_bound, stream);
  if (reference) {
    return out_f32 ? dispatch_gm_simt<bf16_t, float>(a, b_layout, epi, rows_bound, stream)
                   : dispatch_gm_simt<bf16_t, bf16_t>(a, b_layout, epi, rows_bound, stream);
  }
  if (out_f32) {
    if (epi != EPI_STORE) return hipErrorInvalidValue;
    return b_layout == LAYOUT_KX ? dispatch_gm_mfma<LAYOUT_KX, EPI_STORE, float>(a, rows_bound, stream)
                                 : dispatch_gm_mfma<LAYOUT_XK, EPI_STORE, float>(a, rows_bound, stream);
  }
  if (b_layout == LAYOUT_KX) {
    switch (epi) {
      case EPI_STORE: return dispatch_gm_mfma<LAYOUT_KX, EPI_STORE, bf16_t>(a, rows_bound, stream);
      case EPI_DUAL: return dispatch_gm_mfma<LAYOUT_KX, EPI_DUAL, bf16_t>(a, rows_bound, stream);
      case EPI_SWIGLU: return dispatch_gm_mfma<LAYOUT_KX, EPI_SWIGLU, bf16_t>(a, rows_bound, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case EPI_STORE: return dispatch_gm_mfma<LAYOUT_XK, EPI_STORE, bf16_t>(a, rows_bound, stream);
    case EPI_SWIGLU_BWD: return dispatch_gm_mfma<LAYOUT_XK, EPI_SWIGLU_BWD, bf16_t>(a, rows_bound, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_gk_launch(const GemmArgs& a, int dtype, int reference, hipStream_t stream) {
  if (a.G <= 0 || a.M <= 0 || a.N <= 0) return hipSuccess;
  if (dtype == 0 || reference) {
    dim3 grid((a.N + 63) / 64, a.M, a.G);
    if (dtype == 0) hipLaunchKernelGGL(gk_simt<float>, grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL(gk_simt<bf16_t>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  // output rows = the wide dimension (m or n), output columns = the LoRA rank side
  constexpr int WM = 4, WN = 1, TM = 1, TN = 1;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const long units = (long)a.G * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const long blocks = (units + 7) / 8 * 8;
  hipLaunchKernelGGL((gk_mfma<WM, WN, TM, TN>), dim3((unsigned)blocks), dim3(WM * WN * 64), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace moe
