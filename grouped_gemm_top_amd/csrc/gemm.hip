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
#include <climits>
#include <type_traits>

namespace moe {

int tile_table_index(int bm) {
  for (int i = 0; i < kNumTileSizes; i++)
    if (kTileSizes[i] == bm) return i;
  return -1;
}

namespace {

constexpr int BK = 64;    // K tile

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;

__device__ inline bf16x4_t lds_read_tr(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)((lds_bf16_t*)p));
}


// Compile-time loop: f(std::integral_constant<int, I>) for I in [0, N).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
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
//
// LDS tiles are unpadded and XOR-swizzled at 16-byte-chunk granularity: lane L of a copy instruction
// writes the L-th 16-byte chunk of a contiguous 1 KB LDS span and fetches whichever global chunk
// belongs at that position (the layout gfx950's direct-to-LDS loads would write; every kernel here
// copies through registers with plain loads and ds_write). Tiles whose reduction axis is contiguous
// hold 8 chunks per row (BK = 64) with chunk q of row x at q ^ swz_xk(x); tiles whose output axis
// is contiguous hold BN/8 chunks per row with chunk q of row k at q ^ swz_kx(k).
// XOR swizzles (measured conflict-free on gfx950, whose LDS serves 256 bytes per clock: 16 lanes per
// cycle for ds_read_b128, 32 lanes per cycle for ds_read_b64_tr_b16).
// XK tiles (CPR chunks per row): the 16 rows read together by one MFMA fragment must land on
// distinct 16-byte bank groups of each 256-byte window.
template <int CPR>
__host__ __device__ constexpr int swz_xk(int x) { return CPR >= 8 ? ((x >> 1) & 7) : ((x >> 2) & 3); }
// KX tiles: one transposing read covers 4 rows x 4 chunks per 32 lanes; those 16 chunks must be
// distinct modulo 16.
template <int CPR>
__host__ __device__ constexpr int swz_kx(int k) {
  return CPR >= 16 ? 4 * (k & 3) : (CPR == 8 ? 4 * ((k >> 1) & 1) : 0);
}

// Fragment from an XK tile with BKT elements per row (chunk q of row x at q ^ swz_xk(x)).
template <int BKT>
__device__ inline bf16x8_t frag_xk_s(const bf16_t* tile, int x0, int k0, int lane) {
  const int x = x0 + (lane & 31);
  const int q = (k0 >> 3) + (lane >> 5);
  return *reinterpret_cast<const bf16x8_t*>(tile + x * BKT + ((q ^ swz_xk<BKT / 8>(x)) << 3));
}

// Fragment from a KX tile with X elements per row (chunk q of row k at q ^ swz_kx(k)). Within each
// 16-lane group, ds_read_b64_tr_b16 gathers a 4 (k) x 16 (x) block: lane (b, c) names row b,
// columns 4c..4c+3, and lane L receives column L of the 4 rows; two reads give 8 k values.
template <int X>
__device__ inline bf16x8_t frag_kx_s(const bf16_t* tile, int x0, int k0, int lane) {
  constexpr int CPR = X / 8;
  const int g = lane >> 4, b = (lane >> 2) & 3, c = lane & 3;
  const int k = k0 + 8 * (g >> 1) + b;
  const int x = x0 + 16 * (g & 1) + 4 * c;
  const int off = (((x >> 3) ^ swz_kx<CPR>(k)) << 3) + (x & 7);  // same swizzle for rows k, k + 4
  bf16x4_t lo = lds_read_tr(tile + k * X + off);
  bf16x4_t hi = lds_read_tr(tile + (k + 4) * X + off);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row-grouped MFMA GEMM (the router logits and the shapes no other kernel takes).
//
// K tiles of BKT stream through two LDS stages: the 16-byte-per-lane register loads of tile kt+1
// are in flight while tile kt is multiplied, then go to the other stage, and one barrier per tile
// hands the stages over. Lane L of wave instruction i moves the L-th 16-byte chunk of a contiguous
// 1 KB LDS span, so each lane fetches whichever global chunk belongs at that position. LDS tiles are
// unpadded and XOR-swizzled at 16-byte chunk granularity against bank conflicts of the fragment
// reads.
template <int WM, int WN, int TM, int TN, int BKT, int S, int BL, int EPI, typename OutT, bool TAIL>
__global__ __launch_bounds__(WM * WN * 64) void gm_mfma(GemmArgs a, int tidx, const int* tmap) {
  constexpr bool DUAL = (EPI == EPI_DUAL || EPI == EPI_SWIGLU);
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32, NW = WM * WN;
  constexpr int BNH = DUAL ? BN / 2 : BN;
  constexpr int CPR_A = BKT / 8;                                 // chunks per XK row
  constexpr int CPR_B = BN / 8;                                  // chunks per KX B row
  constexpr int A_ELEMS = BM * BKT, B_ELEMS = BN * BKT, STAGE = A_ELEMS + B_ELEMS;
  constexpr int A_IPW = BM * BKT / 8 / 64 / NW;                  // load instructions per wave
  constexpr int B_IPW = BN * BKT / 8 / 64 / NW;
  constexpr int TAIL_STEPS = 64 / BKT;                           // LoRA tail: up to 64 reduction rows
  static_assert(A_IPW * 64 * NW * 8 == BM * BKT && B_IPW * 64 * NW * 8 == BN * BKT, "tile/wave mismatch");
  static_assert(!DUAL || (TN % 2 == 0), "dual epilogue needs an even TN");
  static_assert(BL == LAYOUT_XK || CPR_B >= 4, "KX tiles need >= 4 chunks per row");
  static_assert(S == 2, "two LDS stages");
  static_assert(!TAIL || TAIL_STEPS <= S, "tail tiles reuse the ring stages");
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];  // S * STAGE elements

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- which (group, row tile, column tile)
  const int tilesN = (a.N + BNH - 1) / BNH;
  const int* toff = a.goff ? a.toff_all + tidx * (a.G + 1) : nullptr;
  const int mtiles = a.goff ? toff[a.G] : (a.M + BM - 1) / BM;
  const int T = xcd_unit(mtiles * tilesN);
  if (T < 0) return;
  int e = 0, row0, row_end, nt;
  if (a.goff) {
    e = tmap[T / tilesN];  // row tiles of group e are [toff[e], toff[e+1])
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

  // ---- per-lane source offsets of the chunks this lane moves (32-bit; the shape limits keep them
  //      below 2^31)
  const bf16_t* Ab = (const bf16_t*)a.A;
  long aoff[A_IPW];  // element offsets: an activation matrix may hold more than 2^31 elements
#pragma unroll
  for (int i = 0; i < A_IPW; i++) {
    const int P = (wave * A_IPW + i) * 64 + lane;
    const int x = P / CPR_A, q = (P % CPR_A) ^ swz_xk<CPR_A>(x);
    const int row = min(row0 + x, row_end - 1);
    const int src = a.arow ? a.arow[row] / a.arow_div : row;
    aoff[i] = (long)src * a.lda + q * 8;
  }
  const bf16_t* Bg = (const bf16_t*)a.B + (long)e * a.bstride;
  const bf16_t* Bug = DUAL ? (const bf16_t*)a.Bu + (long)e * a.bstride : nullptr;
  long boff[B_IPW];
  bool bup[B_IPW];
#pragma unroll
  for (int i = 0; i < B_IPW; i++) {
    const int P = (wave * B_IPW + i) * 64 + lane;
    if (BL == LAYOUT_KX) {
      const int k = P / CPR_B, x = ((P % CPR_B) ^ swz_kx<CPR_B>(k)) * 8;
      const int half = DUAL ? (x >= BNH) : 0;
      // (a chunk past the last column re-reads the last whole chunk of the row: the operand rows
      // are padded to a multiple of 8 columns, so that chunk stays aligned)
      const int jj = min(j0 + x - half * BNH, ((a.N + 7) & ~7) - 8);
      bup[i] = half;
      boff[i] = (long)k * a.ldb + jj;
    } else {
      const int x = P / CPR_A, q = (P % CPR_A) ^ swz_xk<CPR_A>(x);
      const int half = DUAL ? (x >= BNH) : 0;
      const int jj = min(j0 + x - half * BNH, a.N - 1);
      bup[i] = half;
      boff[i] = (long)jj * a.ldb + q * 8;
    }
  }

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

  // K split of this workgroup (ungrouped launches only): reduction rows [kbase, kbase + Keff)
  const int kbase = a.kchunk ? (int)blockIdx.y * a.kchunk : 0;
  const int Keff = a.kchunk ? a.kchunk : a.K;
  // Register loads of one K tile, and their copy into the stage at sA (A tile) / sA + A_ELEMS (B tile)
  i32x4_t ra[A_IPW], rb[B_IPW];
  auto gload = [&](int k0) {
    k0 += kbase;
#pragma unroll
    for (int i = 0; i < A_IPW; i++) ra[i] = ld16(Ab + aoff[i] + k0);
    const long kb = (BL == LAYOUT_KX) ? (long)k0 * a.ldb : (long)k0;
#pragma unroll
    for (int i = 0; i < B_IPW; i++) rb[i] = ld16((bup[i] ? Bug : Bg) + boff[i] + kb);
  };
  auto sstore = [&](bf16_t* sA) {
    bf16_t* sB = sA + A_ELEMS;
#pragma unroll
    for (int i = 0; i < A_IPW; i++) *reinterpret_cast<i32x4_t*>(sA + (wave * A_IPW + i) * 512 + lane * 8) = ra[i];
#pragma unroll
    for (int i = 0; i < B_IPW; i++) *reinterpret_cast<i32x4_t*>(sB + (wave * B_IPW + i) * 512 + lane * 8) = rb[i];
  };
  auto wcol = [&](int tn) {
    if constexpr (DUAL) {
      constexpr int TH = TN / 2;
      return (tn >= TH ? BNH : 0) + wn * TH * 32 + (tn % TH) * 32;
    } else {
      return wn * TN * 32 + tn * 32;
    }
  };
  auto frags = [&](const bf16_t* sA, const bf16_t* sB, int ks, bf16x8_t* fa, bf16x8_t* fb) {
#pragma unroll
    for (int tm = 0; tm < TM; tm++) fa[tm] = frag_xk_s<BKT>(sA, wm * TM * 32 + tm * 32, ks * 16, lane);
#pragma unroll
    for (int tn = 0; tn < TN; tn++)
      fb[tn] = (BL == LAYOUT_XK) ? frag_xk_s<BKT>(sB, wcol(tn), ks * 16, lane)
                                 : frag_kx_s<BN>(sB, wcol(tn), ks * 16, lane);
  };
  auto mma = [&](const bf16x8_t* fa, const bf16x8_t* fb) {
    static_for<TM>([&](auto tmc) {
      constexpr int tm = decltype(tmc)::value;
      static_for<TN>([&](auto tnc) {
        constexpr int tn = decltype(tnc)::value;
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
      });
    });
  };
  // fragments of k16 step ks+1 are read while the MFMAs of step ks run
  auto compute = [&](const bf16_t* sA) {
    const bf16_t* sB = sA + A_ELEMS;
    bf16x8_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    frags(sA, sB, 0, fa0, fb0);
    static_for<BKT / 32>([&](auto kc) {
      constexpr int ks = 2 * decltype(kc)::value;
      frags(sA, sB, ks + 1, fa1, fb1);
      mma(fa0, fb0);
      if constexpr (ks + 2 < BKT / 16) frags(sA, sB, ks + 2, fa0, fb0);
      mma(fa1, fb1);
    });
  };
  // ---- main K loop: the loads of tile kt+1 are in flight while tile kt is multiplied; they are
  //      copied into the other stage afterwards (its readers finished before the last barrier)
  const int nk = Keff / BKT;
  bf16_t* const stage0 = smem;
  bf16_t* const stage1 = smem + STAGE;
  gload(0);
  sstore(stage0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    const bool more = kt + 1 < nk;
    if (more) gload((kt + 1) * BKT);
    compute((kt & 1) ? stage1 : stage0);
    if (more) sstore((kt & 1) ? stage0 : stage1);
    __syncthreads();
  }

  // ---- Split-LoRA tail: TAIL_STEPS more K tiles [TA | 0] . [TB ; 0], zero-filled via registers
  if constexpr (TAIL) {
    const int r2 = a.r2a;
    const int K2 = (a.tail == TAIL_SINGLE || a.tail == TAIL_SHARED) ? r2 : 2 * r2;
    const i32x4_t zero = {0, 0, 0, 0};
    const bf16_t* T0 = (const bf16_t*)a.TB0 + (long)e * a.tbstride;
    const bf16_t* T1 = a.TB1 ? (const bf16_t*)a.TB1 + (long)e * a.tbstride : T0;
    static_for<TAIL_STEPS>([&](auto tc) {
      constexpr int ts = decltype(tc)::value;
      bf16_t* sA = smem + ts * STAGE;
      bf16_t* sB = sA + A_ELEMS;
#pragma unroll
      for (int i = 0; i < A_IPW; i++) {
        const int P = (wave * A_IPW + i) * 64 + lane;
        const int x = P / CPR_A, q = ((P % CPR_A) ^ swz_xk<CPR_A>(x)) + ts * CPR_A;
        const int row = min(row0 + x, row_end - 1);
        *reinterpret_cast<i32x4_t*>(sA + P * 8) =
            (q * 8 < K2) ? ld16((const bf16_t*)a.TA + (long)row * a.lda2 + q * 8) : zero;
      }
#pragma unroll
      for (int i = 0; i < B_IPW; i++) {
        const int P = (wave * B_IPW + i) * 64 + lane;
        const bf16_t* src = nullptr;
        if (BL == LAYOUT_KX) {
          const int kk = P / CPR_B + ts * BKT, x = ((P % CPR_B) ^ swz_kx<CPR_B>(P / CPR_B)) * 8;
          const int half = DUAL ? (x >= BNH) : 0;
          const int jj = min(j0 + x - half * BNH, a.N - 8);
          if (a.tail == TAIL_SINGLE) {
            if (kk < r2) src = T0 + (long)kk * a.ldtb + jj;
          } else if (a.tail == TAIL_SHARED) {
            if (kk < r2) src = (half ? T1 : T0) + (long)kk * a.ldtb + jj;
          } else if (a.tail == TAIL_BLOCKDIAG) {
            if (half == 0 && kk < r2) src = T0 + (long)kk * a.ldtb + jj;
            else if (half == 1 && kk >= r2 && kk < 2 * r2) src = T1 + (long)(kk - r2) * a.ldtb + jj;
          } else {
            if (kk < r2) src = T0 + (long)kk * a.ldtb + jj;
            else if (kk < 2 * r2) src = T1 + (long)(kk - r2) * a.ldtb + jj;
          }
        } else {
          const int x = P / CPR_A;
          const int k8 = (((P % CPR_A) ^ swz_xk<CPR_A>(x)) + ts * CPR_A) * 8;
          const int half = DUAL ? (x >= BNH) : 0;
          const int jj = min(j0 + x - half * BNH, a.N - 1);
          if (a.tail == TAIL_SINGLE) {
            if (k8 < r2) src = T0 + (long)jj * a.ldtb + k8;
          } else if (a.tail == TAIL_SHARED) {
            if (k8 < r2) src = (half ? T1 : T0) + (long)jj * a.ldtb + k8;
          } else if (a.tail == TAIL_BLOCKDIAG) {
            if (half == 0 && k8 < r2) src = T0 + (long)jj * a.ldtb + k8;
            else if (half == 1 && k8 >= r2 && k8 < 2 * r2) src = T1 + (long)jj * a.ldtb + (k8 - r2);
          } else {
            if (k8 < r2) src = T0 + (long)jj * a.ldtb + k8;
            else if (k8 < 2 * r2) src = T1 + (long)jj * a.ldtb + (k8 - r2);
          }
        }
        *reinterpret_cast<i32x4_t*>(sB + P * 8) = src ? ld16(src) : zero;
      }
    });
    __syncthreads();
    static_for<TAIL_STEPS>([&](auto tc) { compute(smem + decltype(tc)::value * STAGE); });
  }

  // ---- epilogue (compile-time accumulator indices; one 32-row MFMA tile row at a time)
  OutT* C = (OutT*)a.C + (a.kchunk ? (long)blockIdx.y * a.csplit : 0L);
  // plain store: scale and bias (of the lane's columns, loaded once at clamped columns) are applied
  // to the accumulators here, in straight-line code, so that the store loop issues no loads: a load
  // inside it would make every store wait for the ones before it
  if constexpr (EPI == EPI_STORE) {
    float bcol[TN] = {};
    if (a.bias && (!a.kchunk || blockIdx.y == 0)) {
#pragma unroll
      for (int tn = 0; tn < TN; tn++) bcol[tn] = a.bias[min(j0 + wn * TN * 32 + tn * 32 + (lane & 31), a.N - 1)];
      // wait for them here (s_waitcnt vmcnt(0), other counters untouched): the compiler moves their
      // use into the store loop's branches, where its own waits would include the stores before
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
#pragma unroll
    for (int tm = 0; tm < TM; tm++)
#pragma unroll
      for (int tn = 0; tn < TN; tn++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[tm][tn][v] = a.scale * acc[tm][tn][v] + bcol[tn];
  }
  static_for<TM>([&](auto tmc) {
    constexpr int tm = decltype(tmc)::value;
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto vc) {
      constexpr int v = decltype(vc)::value;
      const int row = row0 + wm * TM * 32 + tm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row < row_end) {
        if constexpr (DUAL) {
          static_for<TN / 2>([&](auto tc) {
            constexpr int t2 = decltype(tc)::value;
            const int jj = j0 + wn * (TN / 2) * 32 + t2 * 32 + (lane & 31);
            if (jj < a.N) {
              const float g = acc[tm][t2][v], uu = acc[tm][t2 + TN / 2][v];
              if constexpr (EPI == EPI_DUAL) {
                C[(long)row * a.ldc + jj] = from_f<OutT>(a.scale * g);
                C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(a.scale * uu);
              } else {
                C[(long)row * a.ldc + jj] = from_f<OutT>(g);
                C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(uu);
                ((OutT*)a.H)[(long)row * a.ldh + jj] = from_f<OutT>(silu_f(g) * uu);
              }
            }
          });
        } else {
          static_for<TN>([&](auto tc) {
            constexpr int tn = decltype(tc)::value;
            const int jj = j0 + wn * TN * 32 + tn * 32 + (lane & 31);
            if (jj < a.N) {
              if constexpr (EPI == EPI_STORE) {
                C[(long)row * a.ldc + jj] = from_f<OutT>(acc[tm][tn][v]);  // scaled, with bias
              } else {  // EPI_SWIGLU_BWD
                const float val = a.scale * acc[tm][tn][v];
                const OutT* GU = (const OutT*)a.GU;
                const float g = to_f(GU[(long)row * a.ldgu + jj]);
                const float uu = to_f(GU[(long)row * a.ldgu + a.guup + jj]);
                const float sg = 1.0f / (1.0f + __expf(-g));
                C[(long)row * a.ldc + jj] = from_f<OutT>(val * uu * sg * (1.0f + g * (1.0f - sg)));
                C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(val * g * sg);
              }
            }
          });
        }
      }
    });
  });
}

// ------------------------------------------------------------------------------------------------
// Row-grouped GEMM with a register prefetch ring, for the expert projections (the launches that carry
// a Split-LoRA tail) and the grouped low-rank products.
//
// Every weight byte of an expert meets only the few hundred rows routed to that expert, so these
// GEMMs stream the expert weights from HBM at about the chip's MFMA/HBM balance point; what limits
// them is the rate at which each CU draws operand bytes from L2. Both operand tiles are fetched with
// fully coalesced 16-byte-per-lane loads (each wave instruction covers whole 128-byte lines) into an
// RS-slot register ring, RS - 1 K tiles ahead of the MFMAs, and copied into a two-stage LDS buffer
// one tile ahead. All loads are plain register loads, so the compiler's waits are exact and leave the later
// tiles in flight; one barrier per tile (without a vector-memory drain) hands the LDS stages over.
// Loads past the last tile repeat the last tile, so every step issues the same loads.
//
// The Split-LoRA tail (up to 128 reduction rows) follows as one or two more tiles through LDS,
// filled with zeros beyond its length.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N_>
using IC = std::integral_constant<int, N_>;

// Whether a gm_ring configuration runs persistent workgroups (one per CU, each taking units in turn):
// the 8-wave tiles on the two-slot ring, except the SwiGLU backward, whose saved gate/up inputs leave
// too few registers for the unit loop (made to fit, it was no faster).
template <int NW, int RS, int EPI>
constexpr bool ring_persist() { return RS == 2 && NW == 8 && EPI != EPI_SWIGLU_BWD; }

template <int WM, int WN, int TM, int TN, int BL, int EPI, int RS>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(RS == 4 || WM * WN >= 8 ? 2 : 3, RS == 4 || WM * WN >= 8 ? 2 : 3)))
void gm_ring(GemmArgs a, int tidx, const int* tmap) {
  constexpr int BKT = 64, NW = WM * WN, NT = NW * 64;
  // RS register-ring slots: each tile is loaded RS - 1 tiles ahead of its copy into LDS
  static_assert(RS == 2 || RS == 4, "ring of two or four slots");
  constexpr bool DUAL = (EPI == EPI_DUAL || EPI == EPI_SWIGLU);
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int BNH = DUAL ? BN / 2 : BN;
  constexpr int A_ELEMS = BM * BKT, STAGE = (BM + BN) * BKT;
  constexpr int A_CPT = A_ELEMS / 8 / NT;           // 16-byte chunks per thread per tile
  constexpr int B_CPT = BN * BKT / 8 / NT;
  constexpr int CPR_A = BKT / 8;
  constexpr int CPR_B = (BL == LAYOUT_KX) ? BN / 8 : BKT / 8;
  // LDS: two K-tile stages, reused afterwards for the fp32 staging of every wave's accumulators
  constexpr int SMEM_ELEMS = std::max(2 * STAGE, NW * TM * TN * 32 * 32 * 2);
  constexpr int LDS_BYTES = SMEM_ELEMS * (int)sizeof(bf16_t);
  static_assert(A_CPT * NT * 8 == A_ELEMS && B_CPT * NT * 8 == BN * BKT, "tile/thread mismatch");
  static_assert(!DUAL || TN % 2 == 0, "dual epilogue needs an even TN");
  static_assert(BL == LAYOUT_XK || CPR_B >= 4, "KX tiles need >= 4 chunks per row");
  __shared__ __attribute__((aligned(16))) bf16_t smem[SMEM_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  if (blockIdx.y) {  // the second problem of a batched launch
    a.A = a.bA;
    a.B = a.bB;
    a.C = a.bC;
  }

  // ---- work units (group, row tile, column tile). Unit p of XCD x's contiguous range of units goes to
  //      the workgroups of that XCD (blockIdx % 8 == x), so the units in flight on an XCD are
  //      consecutive: an expert's row and column tiles share its L2. Persistent configurations run a
  //      grid of one workgroup per CU, each taking its XCD's units in turn; the others run one unit
  //      per workgroup.
  constexpr bool PERSIST = ring_persist<NW, RS, EPI>();
  const int tilesN = (a.N + BNH - 1) / BNH;
  const int* toff = a.toff_all + tidx * (a.G + 1);
  const int total = toff[a.G] * tilesN;
  const int per = (total + 7) >> 3;    // units of each XCD
  const int xbase = (blockIdx.x & 7) * per;
  const int wstride = gridDim.x >> 3;  // workgroups of each XCD (the grid is a multiple of 8)
  int pos = blockIdx.x >> 3;
  auto unit_at = [&](int p) { return (p < per && xbase + p < total) ? xbase + p : -1; };
  const int T0 = unit_at(pos);
  if (T0 < 0) return;

  // a unit: its group, rows and column tile, and the source row of each A chunk this thread moves
  struct Unit {
    int e, row0, row_end, j0;
    int asrow[A_CPT];
  };
  auto meta = [&](int t, Unit& U) {
    const int e = tmap[t / tilesN];  // row tiles of group e are [toff[e], toff[e+1])
    const int nte = toff[e + 1] - toff[e];
    const int local = t - toff[e] * tilesN;
    const int nt = local / nte;
    U.e = e;
    U.row0 = a.goff[e] + (local - nt * nte) * BM;
    U.row_end = a.goff[e + 1];
    U.j0 = nt * BNH;
#pragma unroll
    for (int u = 0; u < A_CPT; u++) {
      const int row = min(U.row0 + (tid + u * NT) / CPR_A, U.row_end - 1);
      U.asrow[u] = a.arow ? a.arow[row] : row;  // (divided by arow_div where used)
    }
  };
  // ---- source of every 16-byte chunk this thread moves; LDS chunk position P of a tile holds
  //      global chunk (P mod CPR) ^ swizzle(row)
  const bf16_t* asrc[A_CPT];
  const bf16_t* bsrc[B_CPT];
  auto point = [&](const Unit& U) {
#pragma unroll
    for (int u = 0; u < A_CPT; u++) {
      const int P = tid + u * NT;
      const int x = P / CPR_A, q = (P % CPR_A) ^ swz_xk<CPR_A>(x);
      const int src = a.arow ? U.asrow[u] / a.arow_div : U.asrow[u];
      asrc[u] = (const bf16_t*)a.A + (long)src * a.lda + q * 8;
    }
    const bf16_t* Bg = (const bf16_t*)a.B + (long)U.e * a.bstride;
    const bf16_t* Bug = DUAL ? (const bf16_t*)a.Bu + (long)U.e * a.bstride : Bg;
#pragma unroll
    for (int u = 0; u < B_CPT; u++) {
      const int P = tid + u * NT;
      if constexpr (BL == LAYOUT_KX) {
        const int k = P / CPR_B, x = ((P % CPR_B) ^ swz_kx<CPR_B>(k)) * 8;
        const int half = DUAL ? (x >= BNH) : 0;
        const int jj = min(U.j0 + x - half * BNH, a.N - 8);
        bsrc[u] = (half ? Bug : Bg) + (long)k * a.ldb + jj;
      } else {
        const int x = P / CPR_B, q = (P % CPR_B) ^ swz_xk<CPR_B>(x);
        const int half = DUAL ? (x >= BNH) : 0;
        const int jj = min(U.j0 + x - half * BNH, a.N - 1);
        bsrc[u] = (half ? Bug : Bg) + (long)jj * a.ldb + q * 8;
      }
    }
  };
  const long bstep = (BL == LAYOUT_KX) ? (long)BKT * a.ldb : (long)BKT;  // source advance per tile
  Unit cur;
  meta(T0, cur);
  point(cur);

  f32x16_t acc[TM][TN];
  i32x4_t ra[RS][A_CPT], rb[RS][B_CPT];  // register ring: slot = tile % RS
  auto load = [&](i32x4_t(&da)[A_CPT], i32x4_t(&db)[B_CPT], int t) {
#pragma unroll
    for (int u = 0; u < A_CPT; u++) da[u] = ld16(asrc[u] + t * BKT);
    const long adv = t * bstep;
#pragma unroll
    for (int u = 0; u < B_CPT; u++) db[u] = ld16(bsrc[u] + adv);
  };
  auto store = [&](bf16_t* st, const i32x4_t(&da)[A_CPT], const i32x4_t(&db)[B_CPT]) {
#pragma unroll
    for (int u = 0; u < A_CPT; u++) *reinterpret_cast<i32x4_t*>(st + (tid + u * NT) * 8) = da[u];
#pragma unroll
    for (int u = 0; u < B_CPT; u++)
      *reinterpret_cast<i32x4_t*>(st + A_ELEMS + (tid + u * NT) * 8) = db[u];
  };
  auto wcol = [&](int tn) {
    if constexpr (DUAL) {
      constexpr int TH = TN / 2;
      return (tn >= TH ? BNH : 0) + wn * TH * 32 + (tn % TH) * 32;
    } else {
      return wn * TN * 32 + tn * 32;
    }
  };
  auto frags = [&](const bf16_t* sA, int ks, bf16x8_t* fa, bf16x8_t* fb) {
    const bf16_t* sB = sA + A_ELEMS;
#pragma unroll
    for (int tm = 0; tm < TM; tm++) fa[tm] = frag_xk_s<BKT>(sA, wm * TM * 32 + tm * 32, ks * 16, lane);
#pragma unroll
    for (int tn = 0; tn < TN; tn++)
      fb[tn] = (BL == LAYOUT_XK) ? frag_xk_s<BKT>(sB, wcol(tn), ks * 16, lane)
                                 : frag_kx_s<BN>(sB, wcol(tn), ks * 16, lane);
  };
  auto mma = [&](const bf16x8_t* fa, const bf16x8_t* fb) {
    static_for<TM>([&](auto tmc) {
      constexpr int tm = decltype(tmc)::value;
      static_for<TN>([&](auto tnc) {
        constexpr int tn = decltype(tnc)::value;
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
      });
    });
  };
  // fragments of k16 step ks+1 are read while the MFMAs of step ks run; side(IC<ks>) runs after
  // the MFMAs of k16 step ks (the main loop hands it the next tile's LDS copy and ring refill, so
  // that each wave's memory work is spread over its MFMAs)
  auto compute = [&](const bf16_t* sA, auto&& side) {
    bf16x8_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    frags(sA, 0, fa0, fb0);
    static_for<BKT / 32>([&](auto kc) {
      constexpr int ks = 2 * decltype(kc)::value;
      frags(sA, ks + 1, fa1, fb1);
      mma(fa0, fb0);
      side(IC<ks>{});
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (ks + 2 < BKT / 16) frags(sA, ks + 2, fa0, fb0);
      mma(fa1, fb1);
      side(IC<ks + 1>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto no_side = [](auto) {};
  // one 16-byte chunk c of a ring slot (c < A_CPT: A chunk c, else B chunk c - A_CPT)
  auto load1 = [&](auto cc, i32x4_t(&da)[A_CPT], i32x4_t(&db)[B_CPT], int t) {
    constexpr int c = decltype(cc)::value;
    if constexpr (c < A_CPT) da[c] = ld16(asrc[c] + t * BKT);
    else db[c - A_CPT] = ld16(bsrc[c - A_CPT] + t * bstep);
  };
  auto store1 = [&](auto cc, bf16_t* st, const i32x4_t(&da)[A_CPT], const i32x4_t(&db)[B_CPT]) {
    constexpr int c = decltype(cc)::value;
    if constexpr (c < A_CPT)
      *reinterpret_cast<i32x4_t*>(st + (tid + c * NT) * 8) = da[c];
    else
      *reinterpret_cast<i32x4_t*>(st + A_ELEMS + (tid + (c - A_CPT) * NT) * 8) = db[c - A_CPT];
  };
  constexpr int CPT = A_CPT + B_CPT, NSIDE = BKT / 16, CPJ = (CPT + NSIDE - 1) / NSIDE;

  // ---- main loop. Step kt: (barrier) multiply tile kt from stage kt&1; spread over its MFMAs, copy
  //      tile kt+1 from registers into LDS stage (kt+1)&1 and load tile kt+RS into the ring slot tile
  //      kt left.
  const int nk = a.K / BKT;
  const int last = nk - 1;
  bf16_t* const s0 = smem;
  bf16_t* const s1 = smem + STAGE;
  static_for<RS>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    load(ra[i], rb[i], min(i, last));
  });
  auto step = [&](auto slot_c, int kt) {
    constexpr int sl = decltype(slot_c)::value;       // kt % RS
    constexpr int nx = (sl + 1) % RS;                 // (kt + 1) % RS
    lds_barrier();
    bf16_t* const st = (sl & 1) ? s0 : s1;
    const int tl = min(kt + RS, last);
    compute((sl & 1) ? s1 : s0, [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      static_for<CPJ>([&](auto qc) {
        constexpr int c = j * CPJ + decltype(qc)::value;
        if constexpr (c < CPT) {
          store1(IC<c>{}, st, ra[nx], rb[nx]);
          load1(IC<c>{}, ra[sl], rb[sl], tl);
        }
      });
    });
  };
  for (;;) {  // the units of this workgroup
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;
  const int e = cur.e, row0 = cur.row0, row_end = cur.row_end, j0 = cur.j0;
  store(s0, ra[0], rb[0]);
  // whole groups of RS steps run unguarded (the same loads in flight on every path into the loop
  // head), the last nk % RS steps after the loop
  int kt = 0;
  for (; kt + RS <= nk; kt += RS) {
    static_for<RS>([&](auto ic) { step(ic, kt + decltype(ic)::value); });
  }
  static_for<RS - 1>([&](auto ic) {
    if (kt + decltype(ic)::value < nk) step(ic, kt + decltype(ic)::value);
  });
  // the workgroup's next unit: its group offsets and gathered row indices load while this unit's tail
  // is fetched (or right away, without a tail); its first RS tiles after this unit's stores (loading
  // them before the stores, with the ring live through the epilogue, made these kernels spill)
  int Tn = -1;
  Unit nxt;
  if constexpr (PERSIST) {
    pos += wstride;
    Tn = unit_at(pos);
    if (a.tail == TAIL_NONE && Tn >= 0) meta(Tn, nxt);
  }

  // ---- epilogue (after the tail): each wave stages its fp32 accumulators in its own LDS region, then writes whole
  //      16-byte row chunks (8 columns). Staged row r keeps its 4-float groups XOR-permuted by one
  //      bit of r, which makes both the MFMA-layout writes and the row-chunk reads conflict-free.
  constexpr int WR = TM * 32, WC = TN * 32;   // rows and columns of a wave's tile
  constexpr int CH = WC / 8;                  // 8-column chunks per staged row
  constexpr int PER = WR * CH / 64;           // chunks per lane
  static_assert(NW * WR * WC * (int)sizeof(float) <= LDS_BYTES, "staging fits the LDS buffer");
  static_assert((WR * CH) % 64 == 0, "whole chunks per lane");
  auto sidx = [](int r, int c) { return r * WC + (c ^ (((r >> (WC >= 64 ? 0 : 1)) & 1) << 2)); };
  const int wrow0 = row0 + wm * WR;
  bf16_t* C = (bf16_t*)a.C;
  auto pack8 = [](const float* f) {
    i32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; i++)
      o[i] = (int)((unsigned)f32_to_bf16(f[2 * i]) | ((unsigned)f32_to_bf16(f[2 * i + 1]) << 16));
    return o;
  };
  auto unpack8 = [](const i32x4_t& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f[2 * i] = bf16_to_f32((bf16_t)(v[i] & 0xffff));
      f[2 * i + 1] = bf16_to_f32((bf16_t)((unsigned)v[i] >> 16));
    }
  };
  // SwiGLU backward reads the saved [g | u] chunks of the lane's outputs; issue those loads first
  i32x4_t gch[EPI == EPI_SWIGLU_BWD ? PER : 1], uch[EPI == EPI_SWIGLU_BWD ? PER : 1];
  if constexpr (EPI == EPI_SWIGLU_BWD) {
    const bf16_t* GU = (const bf16_t*)a.GU;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const int q = lane + 64 * i, r = q / CH, c8 = q % CH;
      const int grow = min(wrow0 + r, row_end - 1);
      const int gcol = min(j0 + wn * WC + 8 * c8, a.N - 8);
      gch[i] = ld16(GU + (long)grow * a.ldgu + gcol);
      uch[i] = ld16(GU + (long)grow * a.ldgu + a.guup + gcol);
    }
  }
  // ---- Split-LoRA tail: [TA | 0] . [TB ; 0] over K2 <= 128 more reduction rows
  if (a.tail != TAIL_NONE) {
    lds_barrier();  // every wave is done with both stages
    const int r2 = a.r2a;
    const int K2 = (a.tail == TAIL_SINGLE || a.tail == TAIL_SHARED) ? r2 : 2 * r2;
    const int tsteps = (K2 + BKT - 1) / BKT;
    const i32x4_t zero = {0, 0, 0, 0};
    const bf16_t* T0 = (const bf16_t*)a.TB0 + (long)e * a.tbstride;
    const bf16_t* T1 = a.TB1 ? (const bf16_t*)a.TB1 + (long)e * a.tbstride : T0;
    // Every chunk of a stage is loaded unconditionally, all loads in flight together: a chunk past
    // the tail's length (or outside its half's block) reads a valid address of the same operand, and
    // the zero is selected when it is copied to LDS.
    for (int ts = 0; ts < tsteps; ts++) {
      bf16_t* sA = smem + ts * STAGE;
      bf16_t* sB = sA + A_ELEMS;
      i32x4_t va[A_CPT], vb[B_CPT];
      bool oka[A_CPT], okb[B_CPT];
#pragma unroll
      for (int u = 0; u < A_CPT; u++) {
        const int P = tid + u * NT;
        const int x = P / CPR_A, q = ((P % CPR_A) ^ swz_xk<CPR_A>(x)) + ts * CPR_A;
        const int row = min(row0 + x, row_end - 1);
        oka[u] = q * 8 < K2;
        va[u] = ld16((const bf16_t*)a.TA + (long)row * a.lda2 + (oka[u] ? q * 8 : 0));
      }
#pragma unroll
      for (int u = 0; u < B_CPT; u++) {
        const int P = tid + u * NT;
        const bf16_t* src = nullptr;
        if constexpr (BL == LAYOUT_KX) {
          const int k = P / CPR_B, x = ((P % CPR_B) ^ swz_kx<CPR_B>(k)) * 8;
          const int kk = k + ts * BKT;
          const int half = DUAL ? (x >= BNH) : 0;
          const int jj = min(j0 + x - half * BNH, a.N - 8);
          if (a.tail == TAIL_SINGLE) {
            if (kk < r2) src = T0 + (long)kk * a.ldtb + jj;
          } else if (a.tail == TAIL_SHARED) {
            if (kk < r2) src = (half ? T1 : T0) + (long)kk * a.ldtb + jj;
          } else if (a.tail == TAIL_BLOCKDIAG) {
            if (half == 0 && kk < r2) src = T0 + (long)kk * a.ldtb + jj;
            else if (half == 1 && kk >= r2 && kk < 2 * r2) src = T1 + (long)(kk - r2) * a.ldtb + jj;
          } else {
            if (kk < r2) src = T0 + (long)kk * a.ldtb + jj;
            else if (kk < 2 * r2) src = T1 + (long)(kk - r2) * a.ldtb + jj;
          }
        } else {
          const int x = P / CPR_B;
          const int k8 = (((P % CPR_B) ^ swz_xk<CPR_B>(x)) + ts * CPR_B) * 8;
          const int half = DUAL ? (x >= BNH) : 0;
          const int jj = min(j0 + x - half * BNH, a.N - 1);
          if (a.tail == TAIL_SINGLE) {
            if (k8 < r2) src = T0 + (long)jj * a.ldtb + k8;
          } else if (a.tail == TAIL_SHARED) {
            if (k8 < r2) src = (half ? T1 : T0) + (long)jj * a.ldtb + k8;
          } else if (a.tail == TAIL_BLOCKDIAG) {
            if (half == 0 && k8 < r2) src = T0 + (long)jj * a.ldtb + k8;
            else if (half == 1 && k8 >= r2 && k8 < 2 * r2) src = T1 + (long)jj * a.ldtb + (k8 - r2);
          } else {
            if (k8 < r2) src = T0 + (long)jj * a.ldtb + k8;
            else if (k8 < 2 * r2) src = T1 + (long)jj * a.ldtb + (k8 - r2);
          }
        }
        okb[u] = src != nullptr;
        vb[u] = ld16(okb[u] ? src : T0);  // T0: the first chunk of this expert's factor
      }
      if constexpr (PERSIST) {
        if (ts == 0 && Tn >= 0) meta(Tn, nxt);
      }
#pragma unroll
      for (int u = 0; u < A_CPT; u++)
        *reinterpret_cast<i32x4_t*>(sA + (tid + u * NT) * 8) = oka[u] ? va[u] : zero;
#pragma unroll
      for (int u = 0; u < B_CPT; u++)
        *reinterpret_cast<i32x4_t*>(sB + (tid + u * NT) * 8) = okb[u] ? vb[u] : zero;
    }
    __syncthreads();
    compute(s0, no_side);
    if (tsteps > 1) compute(s1, no_side);
  }

  // The per-chunk side inputs (the previous output under accum; the routing weight of a row, for a
  // row-weighted copy or the SwiGLU backward's dh; the pair id of a row, for the ds partials) are
  // loaded before the staging, all in flight together at clamped rows, so that the store loop issues
  // no loads: a load there would make every store wait for the ones before it.
  i32x4_t prev[EPI == EPI_STORE ? PER : 1] = {};
  float cw[EPI == EPI_STORE || EPI == EPI_SWIGLU_BWD ? PER : 1] = {};
  int prow[EPI == EPI_SWIGLU_BWD ? PER : 1] = {};
  if constexpr (EPI == EPI_SWIGLU_BWD) {
    if (a.arow && (a.wscale || a.dspart)) {
#pragma unroll
      for (int i = 0; i < PER; i++) prow[i] = a.arow[min(wrow0 + (lane + 64 * i) / CH, row_end - 1)];
      if (a.wscale) {
#pragma unroll
        for (int i = 0; i < PER; i++) cw[i] = a.wval[prow[i]];
      }
    }
  }
  if constexpr (EPI == EPI_STORE) {
    if (a.accum) {
#pragma unroll
      for (int i = 0; i < PER; i++) {
        const int q = lane + 64 * i;
        const int grow = min(wrow0 + q / CH, row_end - 1);
        const int gcol = min(j0 + wn * WC + 8 * (q % CH), a.N - 8);
        prev[i] = ld16(C + (long)grow * a.ldc + gcol);
      }
    }
    if (a.C2) {
      int pr[PER];
#pragma unroll
      for (int i = 0; i < PER; i++) pr[i] = a.arow[min(wrow0 + (lane + 64 * i) / CH, row_end - 1)];
#pragma unroll
      for (int i = 0; i < PER; i++) cw[i] = a.wval[pr[i]];
    }
  }

  lds_barrier();  // every wave is done reading the K-tile stages
  float* stg = reinterpret_cast<float*>(smem) + wave * WR * WC;
  static_for<TM>([&](auto tmc) {
    constexpr int tm = decltype(tmc)::value;
    static_for<TN>([&](auto tnc) {
      constexpr int tn = decltype(tnc)::value;
      static_for<16>([&](auto vc) {
        constexpr int v = decltype(vc)::value;
        const int r = tm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        stg[sidx(r, tn * 32 + (lane & 31))] = acc[tm][tn][v];
      });
    });
  });
  // (a wave reads back only its own region: its LDS operations complete in issue order)
  auto rd8 = [&](int r, int c8, float* f) {
    const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(stg + sidx(r, 8 * c8));
    const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(stg + sidx(r, 8 * c8 + 4));
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f[i] = lo[i];
      f[4 + i] = hi[i];
    }
  };
  if constexpr (DUAL) {
    constexpr int HC = CH / 2;  // gate chunks per row; the up chunk of the same columns is HC later
#pragma unroll
    for (int i = 0; i < WR * HC / 64; i++) {
      const int q = lane + 64 * i, r = q / HC, c8 = q % HC;
      const int grow = wrow0 + r;
      const int gcol = j0 + wn * (WC / 2) + 8 * c8;
      if (grow < row_end && gcol < a.N) {
        float g[8], uu[8];
        rd8(r, c8, g);
        rd8(r, c8 + HC, uu);
        if constexpr (EPI == EPI_DUAL) {
#pragma unroll
          for (int j = 0; j < 8; j++) {
            g[j] *= a.scale;
            uu[j] *= a.scale;
          }
        } else {
          float hh[8];
#pragma unroll
          for (int j = 0; j < 8; j++) hh[j] = silu_f(g[j]) * uu[j];
          *reinterpret_cast<i32x4_t*>((bf16_t*)a.H + (long)grow * a.ldh + gcol) = pack8(hh);
        }
        *reinterpret_cast<i32x4_t*>(C + (long)grow * a.ldc + gcol) = pack8(g);
        *reinterpret_cast<i32x4_t*>(C + (long)grow * a.ldc + a.cup + gcol) = pack8(uu);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const int q = lane + 64 * i, r = q / CH, c8 = q % CH;
      const int grow = wrow0 + r;
      const int gcol = j0 + wn * WC + 8 * c8;
      float hdot = 0.0f;  // SwiGLU backward with dspart: this chunk's share of dh . h
      if (grow < row_end && gcol < a.N) {
        float f[8];
        rd8(r, c8, f);
        if constexpr (EPI == EPI_STORE) {
          float pv[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
          if (a.accum) unpack8(prev[i], pv);
#pragma unroll
          for (int j = 0; j < 8; j++) f[j] = a.scale * f[j] + pv[j];
          *reinterpret_cast<i32x4_t*>(C + (long)grow * a.ldc + gcol) = pack8(f);
          if (a.C2) {  // the row-weighted copy
#pragma unroll
            for (int j = 0; j < 8; j++) f[j] *= cw[i];
            *reinterpret_cast<i32x4_t*>((bf16_t*)a.C2 + (long)grow * a.ldc + gcol) = pack8(f);
          }
        } else {  // EPI_SWIGLU_BWD: f = dh; dg = dh u s (1 + g (1 - s)), du = dh silu(g)
          float g[8], uu[8], dg[8], du[8];
          unpack8(gch[i], g);
          unpack8(uch[i], uu);
          const float sc = a.wscale ? a.scale * cw[i] : a.scale;
#pragma unroll
          for (int j = 0; j < 8; j++) {
            const float dh = sc * f[j];
            const float sg = 1.0f / (1.0f + __expf(-g[j]));
            dg[j] = dh * uu[j] * sg * (1.0f + g[j] * (1.0f - sg));
            du[j] = dh * g[j] * sg;
            hdot += a.scale * f[j] * (g[j] * sg * uu[j]);
          }
          *reinterpret_cast<i32x4_t*>(C + (long)grow * a.ldc + gcol) = pack8(dg);
          *reinterpret_cast<i32x4_t*>(C + (long)grow * a.ldc + a.cup + gcol) = pack8(du);
        }
      }
      if constexpr (EPI == EPI_SWIGLU_BWD && CH == 8) {
        if (a.dspart) {  // the 8 chunks of staged row r sit in 8 consecutive lanes
          hdot += __shfl_xor(hdot, 1, 64);
          hdot += __shfl_xor(hdot, 2, 64);
          hdot += __shfl_xor(hdot, 4, 64);
          const int col0 = j0 + wn * WC;
          if (c8 == 0 && grow < row_end && col0 < a.N)
            a.dspart[(long)(col0 / 64) * a.dsstride + prow[i]] = hdot;
        }
      }
    }
  }
  if constexpr (!PERSIST) break;
  if (Tn < 0) break;
  point(nxt);
  static_for<RS>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    load(ra[i], rb[i], min(i, last));
  });
  lds_barrier();  // every wave has read its staged results back before stage 0 is refilled
  cur = nxt;
  }  // units of this workgroup
}

// Stores element (row, col) of group e's K-grouped output.
template <typename Job>
__device__ inline void gk_store(const Job& a, int e, int row, int col, float v) {
  float* C = (float*)a.C;
  if (a.C1 && col >= a.nsplit) {
    C = (float*)a.C1;
    col -= a.nsplit;
  }
  C += (long)e * a.cstride;
  C[a.ctrans ? (long)col * a.ldc + row : (long)row * a.ldc + col] = v;
}

struct GkJobs {
  GemmArgs job[kGkMaxJobs];
};
// The fields of one K-grouped job that its units read, picked out of a GkJobs with constant indices:
// indexing the kernel-argument array with a run-time job number would copy it to the stack.
struct GkJob {
  const void* A;
  const void* B;
  void* C;
  void* C1;
  float* gkpart;
  const int* arow;
  long lda, ldb, ldc, cstride;
  int M, N, nsplit, ctrans, arow_div;
  float scale;
};
__device__ inline GkJob gk_job(const GkJobs& J, int j) {
  GkJob o;
  switch (j) {
#define MOE_GK_PICK(i)                                                                              \
  case i: {                                                                                         \
    const GemmArgs& a = J.job[i];                                                                   \
    o = GkJob{a.A, a.B, a.C, a.C1, a.gkpart, a.arow, a.lda, a.ldb, a.ldc, a.cstride, a.M, a.N,    \
              a.nsplit, a.ctrans, a.arow_div, a.scale};                                             \
    break;                                                                                          \
  }
    MOE_GK_PICK(0) MOE_GK_PICK(1) MOE_GK_PICK(2) MOE_GK_PICK(3)
    MOE_GK_PICK(4) MOE_GK_PICK(5) MOE_GK_PICK(6) default: MOE_GK_PICK(7)
#undef MOE_GK_PICK
  }
  return o;
}
static_assert(kGkMaxJobs == 8, "gk_job picks one of eight jobs");
// Several K-grouped problems over the same row grouping in one launch: each chunk (or group) of the
// grouping has tiles_pre[njobs] work units, job j's output tiles being [tiles_pre[j], tiles_pre[j + 1]).
struct GkLaunch {
  GkJobs jobs;
  int tiles_pre[kGkMaxJobs + 1];
  int tiles_all;  // tiles_pre[njobs]
  int njobs;
};
static_assert(sizeof(GkLaunch) + 2 * sizeof(void*) <= 4096, "kernel arguments within 4 KB");

// K-grouped MFMA GEMM: C_e = scale * L[rows_e]^T . R[rows_e]; both operands stored with the output
// axis contiguous, so both fragments come from transposing LDS reads. One launch runs every job of a
// GkLaunch (all of them share the row grouping), so that the short reductions fill the chip together.
// Without a.gkpart, one workgroup per output tile reduces all rows of its group. With it, work
// units are (chunk of kGkChunk, or kGkChunkSmall, group rows, output tile), listed by the chunk table (toffc: chunk
// prefix sums per group, tmapc: chunk -> group; an empty group has one empty chunk). A group of
// one chunk stores its result directly; the chunks of a longer group store fp32 partials, which
// gk_reduce adds up in chunk order after the launch.
template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void gk_mfma(const GkLaunch L, const int* toffc, const int* tmapc) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32, NT = WM * WN * 64;
  // both operands have the output axis contiguous: unpadded rows of BM (BN) elements, 16-byte chunks
  // XOR-swizzled by row (swz_kx) so that the transposing fragment reads are free of bank conflicts
  constexpr int A_ELEMS = BK * BM, B_ELEMS = BK * BN, STAGE = A_ELEMS + B_ELEMS;
  constexpr int CPR_A = BM / 8, CPR_B = BN / 8;
  constexpr int A_PT = BM * BK / 8 / NT, B_PT = BN * BK / 8 / NT;
  static_assert((BM * BK / 8) % NT == 0 && (BN * BK / 8) % NT == 0, "tile/thread mismatch");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // unit order: chunk (or group) outermost, then job, then output tile, so that each XCD takes a
  // contiguous range of groups with all of their jobs and reuses their rows in its L2
  const int units = L.jobs.job[0].gkpart ? toffc[L.jobs.job[0].G] : L.jobs.job[0].G;
  const int T = xcd_unit(units * L.tiles_all);
  if (T < 0) return;
  const int u0 = T / L.tiles_all;  // group (whole-group mode) or chunk
  int rem = T - u0 * L.tiles_all;
  int j = 0, jbase = 0;
#pragma unroll
  for (int i = 1; i < kGkMaxJobs; i++) {  // (constant indices: see gk_job)
    if (i < L.njobs && rem >= L.tiles_pre[i]) {
      j = i;
      jbase = L.tiles_pre[i];
    }
  }
  rem -= jbase;
  const GkJob a = gk_job(L.jobs, j);
  const GemmArgs& g0 = L.jobs.job[0];  // the grouping, shared by every job
  const int tilesM = (a.M + BM - 1) / BM;
  const int nt = rem / tilesM, mt = rem - nt * tilesM;
  int e, kb, ke, nch = 1;
  int c0 = 0;
  if (a.gkpart) {
    e = tmapc[u0];
    c0 = toffc[e];
    nch = toffc[e + 1] - c0;
    const int chunk = g0.gkchunk == kGkChunkSmall ? kGkChunkSmall : kGkChunk;
    kb = g0.goff[e] + (u0 - c0) * chunk;
    ke = min(kb + chunk, g0.goff[e + 1]);
  } else {
    e = u0;
    kb = g0.goff[e];
    ke = g0.goff[e + 1];
  }

  int acol[A_PT], bcol[B_PT];
#pragma unroll
  for (int u = 0; u < A_PT; u++) acol[u] = min(mt * BM + ((tid + u * NT) % CPR_A) * 8, a.M - 8);
#pragma unroll
  for (int u = 0; u < B_PT; u++) bcol[u] = min(nt * BN + ((tid + u * NT) % CPR_B) * 8, a.N - 8);

  i32x4_t ra[2][A_PT], rb[2][B_PT];  // two register slots: loads run two K tiles ahead
  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;
  const i32x4_t zero = {0, 0, 0, 0};

  // Every load is issued unconditionally (rows past the group's end read its last row, so the
  // compiler's load counting is the same on every path); those rows are zeroed when copied to LDS.
  // Left-operand source rows of a K tile: with a row gather they come from a.arow, so they are
  // fetched one tile ahead of the data that uses them.
  // (the gathered index is divided only when used, so the index load is not waited for here)
  auto gidx = [&](int k0, int* src) {
#pragma unroll
    for (int u = 0; u < A_PT; u++) {
      const int row = min(k0 + (tid + u * NT) / CPR_A, ke - 1);
      src[u] = a.arow ? a.arow[row] : row;
    }
  };
  auto gload = [&](int k0, const int* src, i32x4_t* ra_, i32x4_t* rb_) {
#pragma unroll
    for (int u = 0; u < A_PT; u++) {
      const long srow = a.arow ? (long)(src[u] / a.arow_div) : (long)src[u];
      ra_[u] = ld16((const bf16_t*)a.A + srow * a.lda + acol[u]);
    }
#pragma unroll
    for (int u = 0; u < B_PT; u++) {
      const int row = min(k0 + (tid + u * NT) / CPR_B, ke - 1);
      rb_[u] = ld16((const bf16_t*)a.B + (long)row * a.ldb + bcol[u]);
    }
  };
  auto sstore = [&](int k0, int buf, const i32x4_t* ra, const i32x4_t* rb) {
    bf16_t* sA = smem + buf * STAGE;
    bf16_t* sB = sA + A_ELEMS;
#pragma unroll
    for (int u = 0; u < A_PT; u++) {
      const int c = tid + u * NT, row = c / CPR_A;
      *reinterpret_cast<i32x4_t*>(sA + row * BM + (((c % CPR_A) ^ swz_kx<CPR_A>(row)) << 3)) =
          k0 + row < ke ? ra[u] : zero;
    }
#pragma unroll
    for (int u = 0; u < B_PT; u++) {
      const int c = tid + u * NT, row = c / CPR_B;
      *reinterpret_cast<i32x4_t*>(sB + row * BN + (((c % CPR_B) ^ swz_kx<CPR_B>(row)) << 3)) =
          k0 + row < ke ? rb[u] : zero;
    }
  };
  // A job whose output is stored transposed (ctrans) multiplies with the operands swapped, so that
  // its accumulators hold the transposed tile: lane l then holds output column l of the stored
  // layout, and each store instruction writes whole rows of it.
  const bool ct = a.ctrans != 0;
  auto compute = [&](const bf16_t* sA) {
    const bf16_t* sB = sA + A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks++) {
      bf16x8_t fa[TM], fb[TN];
#pragma unroll
      for (int tm = 0; tm < TM; tm++) fa[tm] = frag_kx_s<BM>(sA, wm * TM * 32 + tm * 32, ks * 16, lane);
#pragma unroll
      for (int tn = 0; tn < TN; tn++) fb[tn] = frag_kx_s<BN>(sB, wn * TN * 32 + tn * 32, ks * 16, lane);
#pragma unroll
      for (int tm = 0; tm < TM; tm++)
#pragma unroll
        for (int tn = 0; tn < TN; tn++)
          acc[tm][tn] = ct ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[tn], fa[tm], acc[tm][tn], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
    }
  };

  // Tile kt lives in LDS buffer kt & 1 and arrives through register slot kt & 1; its loads are issued
  // two tiles ahead (while tile kt - 2 is multiplied), its row indices three tiles ahead.
  const int nk = (ke - kb + BK - 1) / BK;
  if (nk > 0) {
    // src[j]: rows of the next tile of parity j. Each step issues its index loads before its data
    // loads, so waiting for the indices never waits for the data still in flight.
    int src[2][A_PT];
    gidx(kb, src[0]);
    gidx(kb + BK, src[1]);
    gload(kb, src[0], ra[0], rb[0]);
    gidx(kb + 2 * BK, src[0]);
    gload(kb + BK, src[1], ra[1], rb[1]);
    sstore(kb, 0, ra[0], rb[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      // tile kt (buffer 0); slot 0 is free, slot 1 holds tile kt + 1 (all rows past ke once kt + 1 >= nk)
      gidx(kb + (kt + 3) * BK, src[1]);
      gload(kb + (kt + 2) * BK, src[0], ra[0], rb[0]);
      compute(smem);
      sstore(kb + (kt + 1) * BK, 1, ra[1], rb[1]);
      __syncthreads();
      if (kt + 1 >= nk) break;
      // tile kt + 1 (buffer 1); slot 1 is free, slot 0 holds tile kt + 2
      gidx(kb + (kt + 4) * BK, src[0]);
      gload(kb + (kt + 3) * BK, src[1], ra[1], rb[1]);
      compute(smem + STAGE);
      sstore(kb + (kt + 2) * BK, 0, ra[0], rb[0]);
      __syncthreads();
    }
  }

#pragma unroll
  for (int tm = 0; tm < TM; tm++)
#pragma unroll
    for (int tn = 0; tn < TN; tn++)
#pragma unroll
      for (int v = 0; v < 16; v++) {
        // accumulator element v of this lane: (row, col) of C, or (col, row) with the swapped operands
        const int vr = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), vl = lane & 31;
        const int row = mt * BM + wm * TM * 32 + tm * 32 + (ct ? vl : vr);
        const int col = nt * BN + wn * TN * 32 + tn * 32 + (ct ? vr : vl);
        if (row >= a.M || col >= a.N) continue;
        if (nch == 1) gk_store(a, e, row, col, a.scale * acc[tm][tn][v]);
        else if (ct) a.gkpart[(long)u0 * a.M * a.N + (long)col * a.M + row] = acc[tm][tn][v];  // [N][M]
        else a.gkpart[((long)u0 * a.M + row) * a.N + col] = acc[tm][tn][v];                     // [M][N]
      }
}


// Completion of chunked K-grouped launches: block (x, j) walks the groups of job j and, for each
// group of several chunks, strides over its output with the gridDim.x blocks of the job (groups of
// one chunk are already stored).
__global__ __launch_bounds__(256) void gk_reduce(GkJobs jobs, const int* toffc) {
  __shared__ int off[kGkMaxGroups + 1];
  const GkJob a = gk_job(jobs, blockIdx.y);
  const GemmArgs& g0 = jobs.job[0];  // the grouping, shared by every job
  if (toffc[g0.G] == g0.G) return;  // every group has one chunk (none has fewer): nothing to add up
  for (int e = threadIdx.x; e <= g0.G; e += 256) off[e] = toffc[e];
  __syncthreads();
  const long MN = (long)a.M * a.N;
  for (int e = 0; e < g0.G; e++) {
    const int c0 = off[e], nch = off[e + 1] - c0;
    if (nch <= 1) continue;
    for (long idx = (long)blockIdx.x * 256 + threadIdx.x; idx < MN; idx += (long)gridDim.x * 256) {
      float v = 0.0f;
      for (int c = 0; c < nch; c++) v += a.gkpart[(long)(c0 + c) * MN + idx];
      // partials of a transposed-store job are laid out [N][M], so consecutive threads store
      // consecutive addresses in either case
      if (a.ctrans) gk_store(a, e, (int)(idx % a.M), (int)(idx / a.M), a.scale * v);
      else gk_store(a, e, (int)(idx / a.N), (int)(idx % a.N), a.scale * v);
    }
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
  if (blockIdx.z) {  // the second problem of a batched launch
    a.A = a.bA;
    a.B = a.bB;
    a.C = a.bC;
  }
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
  // four running sums over blocks of four K steps (the steps past the last whole block go to the first),
  // added together at the end in that order, so that the loads of four steps are in flight together
  float p0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, p1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int k = 0;
  for (; k + 4 <= a.K; k += 4) {
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const float x = to_f(Ar[k + u]);
      p0[u] += x * opv(Bg, b_layout, a.ldb, jj, k + u);
      if (DUAL) p1[u] += x * opv(Bug, b_layout, a.ldb, jj, k + u);
    }
  }
  for (; k < a.K; k++) {
    const float x = to_f(Ar[k]);
    p0[0] += x * opv(Bg, b_layout, a.ldb, jj, k);
    if (DUAL) p1[0] += x * opv(Bug, b_layout, a.ldb, jj, k);
  }
  float acc0 = ((p0[0] + p0[1]) + p0[2]) + p0[3];
  float acc1 = ((p1[0] + p1[1]) + p1[2]) + p1[3];
  if (a.tail != TAIL_NONE) {
    const int r2 = a.r2a;
    const T* TAr = (const T*)a.TA + (long)row * a.lda2;
    const T* T0 = (const T*)a.TB0 + (long)e * a.tbstride;
    const T* T1 = a.TB1 ? (const T*)a.TB1 + (long)e * a.tbstride : nullptr;
    if (a.tail == TAIL_SINGLE) {
      for (int q = 0; q < r2; q++) acc0 += to_f(TAr[q]) * opv(T0, b_layout, a.ldtb, jj, q);
    } else if (a.tail == TAIL_SHARED) {
      for (int q = 0; q < r2; q++) acc0 += to_f(TAr[q]) * opv(T0, b_layout, a.ldtb, jj, q);
      for (int q = 0; q < r2; q++) acc1 += to_f(TAr[q]) * opv(T1, b_layout, a.ldtb, jj, q);
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
    const float prev = a.accum ? to_f(C[(long)row * a.ldc + jj]) : 0.0f;
    const float v = a.scale * acc0 + (a.bias ? a.bias[jj] : 0.0f) + prev;
    C[(long)row * a.ldc + jj] = from_f<OutT>(v);
    if (a.C2) ((OutT*)a.C2)[(long)row * a.ldc + jj] = from_f<OutT>(a.wval[a.arow[row]] * v);
  } else if (EPI == EPI_DUAL) {
    C[(long)row * a.ldc + jj] = from_f<OutT>(a.scale * acc0);
    C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(a.scale * acc1);
  } else if (EPI == EPI_SWIGLU) {
    C[(long)row * a.ldc + jj] = from_f<OutT>(acc0);
    C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(acc1);
    ((OutT*)a.H)[(long)row * a.ldh + jj] = from_f<OutT>(acc0 / (1.0f + expf(-acc0)) * acc1);
  } else {
    const OutT* GU = (const OutT*)a.GU;
    const float dh = (a.wscale ? a.scale * a.wval[a.arow[row]] : a.scale) * acc0;
    const float g = to_f(GU[(long)row * a.ldgu + jj]);
    const float uu = to_f(GU[(long)row * a.ldgu + a.guup + jj]);
    const float sg = 1.0f / (1.0f + expf(-g));
    C[(long)row * a.ldc + jj] = from_f<OutT>(dh * uu * sg * (1.0f + g * (1.0f - sg)));
    C[(long)row * a.ldc + a.cup + jj] = from_f<OutT>(dh * g * sg);
    if (a.dspart) {  // one wave per 64 columns (N is a multiple of 64 here)
      const float hd = wave_sum(a.scale * acc0 * (g * sg * uu));
      if (threadIdx.x == 0) a.dspart[(long)blockIdx.y * a.dsstride + a.arow[row]] = hd;
    }
  }
}

// K-grouped products on plain SIMT threads (fp32 layers and the reference mode): every job of a launch in
// one grid. Block b belongs to job j when L.tiles_pre[j] <= b < L.tiles_pre[j + 1]; within the job, blocks
// run over (group, output row, 64-column block), one thread per output element. Each thread reduces its
// group's rows with four running sums over blocks of four rows (the last rows, past the last whole block,
// go to the first sum), added together at the end in that order.
template <typename T>
__global__ __launch_bounds__(64) void gk_simt(const GkLaunch L) {
  const int b = blockIdx.x;
  int j = 0, jbase = 0;
#pragma unroll
  for (int i = 1; i < kGkMaxJobs; i++) {  // (constant indices: see gk_job)
    if (i < L.njobs && b >= L.tiles_pre[i]) {
      j = i;
      jbase = L.tiles_pre[i];
    }
  }
  const GkJob a = gk_job(L.jobs, j);
  const GemmArgs& g0 = L.jobs.job[0];  // the grouping, shared by every job
  const int nb = (a.N + 63) / 64;
  int local = b - jbase;
  const int cb = local % nb;
  local /= nb;
  const int row = local % a.M, e = local / a.M;
  int col = cb * 64 + (int)threadIdx.x;
  if (col >= a.N) return;
  const int kb = g0.goff[e], ke = g0.goff[e + 1];
  const T* A = (const T*)a.A;
  const T* B = (const T*)a.B;
  auto term = [&](int i) {
    const long src = a.arow ? (long)(a.arow[i] / a.arow_div) : (long)i;
    return to_f(A[src * a.lda + row]) * to_f(B[(long)i * a.ldb + col]);
  };
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int i = kb;
  for (; i + 4 <= ke; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; u++) acc[u] += term(i + u);
  }
  for (; i < ke; i++) acc[0] += term(i);
  const float v = ((acc[0] + acc[1]) + acc[2]) + acc[3];
  float* C = (float*)a.C;
  if (a.C1 && col >= a.nsplit) {
    C = (float*)a.C1;
    col -= a.nsplit;
  }
  C += (long)e * a.cstride;
  C[a.ctrans ? (long)col * a.ldc + row : (long)row * a.ldc + col] = a.scale * v;
}

// ------------------------------------------------------------------------------------------------
// Tile configuration of the row-grouped MFMA kernel: WM x WN waves, each TM x TN 32x32 MFMA tiles,
// K tile BKT, S (= 2) LDS stages.
template <int WM_, int WN_, int TM_, int TN_, int BKT_, int S_>
struct TileCfg {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_, BKT = BKT_, S = S_;
  static constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  static constexpr size_t lds_bytes = (size_t)S * (BM + BN) * BKT * sizeof(bf16_t);
};

template <typename Cfg, int BL, int EPI, typename OutT, bool TAIL>
hipError_t launch_gm_mfma_t(const GemmArgs& a, int rows_bound, hipStream_t stream) {
  if (a.accum || a.C2 || a.wscale || a.nbatch > 1) return hipErrorInvalidValue;
  constexpr bool DUAL = (EPI == EPI_DUAL || EPI == EPI_SWIGLU);
  constexpr int BNH = DUAL ? Cfg::BN / 2 : Cfg::BN;
  auto kern = gm_mfma<Cfg::WM, Cfg::WN, Cfg::TM, Cfg::TN, Cfg::BKT, Cfg::S, BL, EPI, OutT, TAIL>;
  // every configuration stays within the 64 KB of dynamic LDS a launch gets without raising the
  // kernel's limit, so no per-process attribute call (and no host state) is needed
  static_assert(Cfg::lds_bytes <= 65536, "dynamic LDS above the default launch limit");
  const int tilesN = (a.N + BNH - 1) / BNH;
  const long mtiles = a.goff ? (long)rows_bound / Cfg::BM + a.G : ((long)a.M + Cfg::BM - 1) / Cfg::BM;
  const long units = mtiles * tilesN;
  if (units <= 0) return hipSuccess;
  const long blocks = (units + 7) / 8 * 8;
  const int tidx = tile_table_index(Cfg::BM);
  if (a.goff && (tidx < 0 || !a.toff_all || !a.tmap_all)) return hipErrorInvalidValue;
  const int* tmap = a.goff ? a.tmap_all + tile_map_offset(tidx, rows_bound, a.G) : nullptr;
  int splits = 1;
  if (a.kchunk) {
    if (a.goff || TAIL || a.kchunk % 64 || a.K % a.kchunk) return hipErrorInvalidValue;
    splits = a.K / a.kchunk;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks, (unsigned)splits), dim3(Cfg::WM * Cfg::WN * 64),
                     Cfg::lds_bytes, stream, a, tidx, tmap);
  return hipGetLastError();
}

template <typename Cfg, int BL, int EPI, typename OutT>
hipError_t launch_gm_mfma(const GemmArgs& a, int rows_bound, hipStream_t stream) {
  if (a.tail != TAIL_NONE) return launch_gm_mfma_t<Cfg, BL, EPI, OutT, true>(a, rows_bound, stream);
  return launch_gm_mfma_t<Cfg, BL, EPI, OutT, false>(a, rows_bound, stream);
}

using CfgSkinny = TileCfg<4, 1, 1, 1, 64, 2>;      // 128 x 32
using CfgSkinnyDual = TileCfg<4, 1, 1, 2, 64, 2>;  // 128 x (32 + 32)
using CfgMid = TileCfg<2, 2, 2, 2, 64, 2>;         // 128 x 128
using CfgRouter = TileCfg<2, 2, 1, 2, 64, 2>;      // 64 x 128: the router logits (fp32 out, split over K)

template <int WM, int WN, int TM, int TN, int BL, int EPI, int RS = 4>
hipError_t launch_gm_ring(const GemmArgs& a, int rows_bound, hipStream_t stream);

template <int BL, int EPI, typename OutT>
hipError_t dispatch_gm_mfma(const GemmArgs& a, int rows_bound, hipStream_t stream) {
  constexpr bool DUAL = (EPI == EPI_DUAL || EPI == EPI_SWIGLU);
  // grouped low-rank products (N <= 32, bf16 out): 64-row tiles of two waves, ~P/64 workgroups (the
  // 128-row skinny tiles leave most of the chip idle on these short launches; 32-row tiles of one wave
  // were 1-2 us slower on each launch)
  if constexpr (std::is_same<OutT, bf16_t>::value && EPI != EPI_SWIGLU && EPI != EPI_SWIGLU_BWD) {
    if (a.goff && a.N <= 32 && a.tail == TAIL_NONE) {
      // (a two-slot ring: fewer registers, three waves per SIMD instead of two; these short launches
      // are latency-bound, and the extra waves took 1.5 us off each of the four)
      if constexpr (DUAL) return launch_gm_ring<2, 1, 1, 2, BL, EPI, 2>(a, rows_bound, stream);
      else return launch_gm_ring<2, 1, 1, 1, BL, EPI, 2>(a, rows_bound, stream);
    }
  }
  // grouped products without a LoRA tail and with wide outputs (merged-weight expert projections)
  if constexpr (std::is_same<OutT, bf16_t>::value && EPI != EPI_DUAL) {
    if (a.goff && a.N > 32 && a.K % 64 == 0 && a.tail == TAIL_NONE && !a.kchunk)
      return launch_gm_ring<2, 2, 2, 2, BL, EPI>(a, rows_bound, stream);
  }
  if constexpr (DUAL) {
    if (a.N <= 32) return launch_gm_mfma<CfgSkinnyDual, BL, EPI, OutT>(a, rows_bound, stream);
    return launch_gm_mfma<CfgMid, BL, EPI, OutT>(a, rows_bound, stream);
  } else {
    if (a.N <= 32) return launch_gm_mfma<CfgSkinny, BL, EPI, OutT>(a, rows_bound, stream);
    if constexpr (std::is_same<OutT, float>::value && EPI == EPI_STORE) {
      if (!a.goff) return launch_gm_mfma<CfgRouter, BL, EPI, OutT>(a, rows_bound, stream);
    }
    return launch_gm_mfma<CfgMid, BL, EPI, OutT>(a, rows_bound, stream);
  }
}

// The expert projections (GEMMs with a Split-LoRA tail) with WN wave columns per workgroup
// (2: 128 x 128 tiles, two workgroups per CU; 4: 128 x 256 tiles, one workgroup of eight waves per CU).
// The 128 x 256 tiles use a two-slot ring: with one workgroup per CU each CU draws operands at the
// same rate either way, and the shorter ring starts a tile sooner and issues fewer loads past the
// last K tile (2-5% faster on each of the four launches than four slots).
template <int WN>
hipError_t launch_expert_projection(const GemmArgs& a, int b_layout, int epi, int rows_bound, hipStream_t stream) {
  constexpr int RS = WN == 4 ? 2 : 4;
  if (b_layout == LAYOUT_KX) {
    if (epi == EPI_SWIGLU) return launch_gm_ring<2, WN, 2, 2, LAYOUT_KX, EPI_SWIGLU, RS>(a, rows_bound, stream);
    if (epi == EPI_STORE) return launch_gm_ring<2, WN, 2, 2, LAYOUT_KX, EPI_STORE, RS>(a, rows_bound, stream);
    if (epi == EPI_SWIGLU_BWD)  // output-major weights
      return launch_gm_ring<2, WN, 2, 2, LAYOUT_KX, EPI_SWIGLU_BWD, RS>(a, rows_bound, stream);
  } else {
    if (epi == EPI_STORE) return launch_gm_ring<2, WN, 2, 2, LAYOUT_XK, EPI_STORE, RS>(a, rows_bound, stream);
    if (epi == EPI_SWIGLU_BWD)
      return launch_gm_ring<2, WN, 2, 2, LAYOUT_XK, EPI_SWIGLU_BWD, RS>(a, rows_bound, stream);
    if (epi == EPI_SWIGLU)  // output-major weights
      return launch_gm_ring<2, WN, 2, 2, LAYOUT_XK, EPI_SWIGLU, RS>(a, rows_bound, stream);
  }
  return hipErrorInvalidValue;
}

// Deep-prefetch kernel (grouped launches).
template <int WM, int WN, int TM, int TN, int BL, int EPI, int RS>
hipError_t launch_gm_ring(const GemmArgs& a, int rows_bound, hipStream_t stream) {
  constexpr bool DUAL = (EPI == EPI_DUAL || EPI == EPI_SWIGLU);
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32, BNH = DUAL ? BN / 2 : BN;
  if (!a.goff || !a.toff_all || !a.tmap_all || a.K % 64 || a.kchunk || a.bias) return hipErrorInvalidValue;
  if (a.C2 && (!a.arow || !a.wval)) return hipErrorInvalidValue;
  if (a.tail != TAIL_NONE) {
    const int K2 = (a.tail == TAIL_SINGLE || a.tail == TAIL_SHARED) ? a.r2a : 2 * a.r2a;
    if (K2 <= 0 || K2 > 128 || K2 % 8) return hipErrorInvalidValue;
  }
  const int tidx = tile_table_index(BM);
  if (tidx < 0) return hipErrorInvalidValue;
  const long tilesN = (a.N + BNH - 1) / BNH;
  const long units = ((long)rows_bound / BM + a.G) * tilesN;
  if (units <= 0) return hipSuccess;
  long blocks = (units + 7) / 8 * 8;
  if (ring_persist<WM * WN, RS, EPI>()) {  // workgroups that take their units in turn: one per CU
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    blocks = std::min(blocks, std::max(8L, (long)cus / 8 * 8));
  }
  const int* tmap = a.tmap_all + tile_map_offset(tidx, rows_bound, a.G);
  if (a.nbatch > 2 || (a.nbatch == 2 && (!a.bA || !a.bB || !a.bC))) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gm_ring<WM, WN, TM, TN, BL, EPI, RS>), dim3((unsigned)blocks, a.nbatch == 2 ? 2u : 1u),
                     dim3(WM * WN * 64), 0, stream, a, tidx, tmap);
  return hipGetLastError();
}

template <typename T, typename OutT, int EPI>
hipError_t launch_gm_simt(const GemmArgs& a, int b_layout, int rows_bound, hipStream_t stream) {
  const int rows = a.goff ? rows_bound : a.M;
  if (rows <= 0 || a.N <= 0) return hipSuccess;
  if (a.nbatch > 2 || (a.nbatch == 2 && (!a.bA || !a.bB || !a.bC))) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gm_simt<T, OutT, EPI>), dim3(rows, (a.N + 63) / 64, a.nbatch == 2 ? 2 : 1), dim3(64), 0,
                     stream, a, b_layout, rows_bound);
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
  if (a.tail != TAIL_NONE) {  // the expert projections
    if (out_f32) return hipErrorInvalidValue;
    // 128 x 256 tiles, one eight-wave workgroup per CU. (128 x 128 tiles, two workgroups per CU, were
    // measured too: slower on the routed layers, and on a shared expert's few large launches no faster
    // in sum.)
    return launch_expert_projection<4>(a, b_layout, epi, rows_bound, stream);
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
    case EPI_SWIGLU: return dispatch_gm_mfma<LAYOUT_XK, EPI_SWIGLU, bf16_t>(a, rows_bound, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_gk_launch(const GemmArgs* jobs, int njobs, int dtype, int reference, int rows_bound,
                          hipStream_t stream) {
  if (njobs <= 0) return hipSuccess;
  if (njobs > kGkMaxJobs) return hipErrorInvalidValue;
  const GemmArgs& a0 = jobs[0];
  for (int i = 0; i < njobs; i++) {
    const GemmArgs& a = jobs[i];
    if (a.nbatch > 1 || a.G != a0.G || a.goff != a0.goff || (a.gkpart != nullptr) != (a0.gkpart != nullptr) ||
        a.gkchunk != a0.gkchunk || a.toff_all != a0.toff_all || a.tmap_all != a0.tmap_all)
      return hipErrorInvalidValue;
  }
  if (a0.G <= 0) return hipSuccess;
  if (dtype == 0 || reference) {  // every job in one launch of the SIMT kernel
    GkLaunch L;
    L.njobs = njobs;
    L.tiles_pre[0] = 0;
    long pre = 0;
    for (int i = 0; i < kGkMaxJobs; i++) {
      const GemmArgs& a = jobs[i < njobs ? i : 0];
      L.jobs.job[i] = a;
      if (i < njobs && a.M > 0 && a.N > 0) pre += (long)((a.N + 63) / 64) * a.M * a.G;
      if (pre > INT_MAX) return hipErrorInvalidValue;
      L.tiles_pre[i + 1] = (int)pre;
    }
    L.tiles_all = L.tiles_pre[njobs];
    if (L.tiles_all <= 0) return hipSuccess;
    if (dtype == 0) hipLaunchKernelGGL(gk_simt<float>, dim3((unsigned)L.tiles_all), dim3(64), 0, stream, L);
    else hipLaunchKernelGGL(gk_simt<bf16_t>, dim3((unsigned)L.tiles_all), dim3(64), 0, stream, L);
    return hipGetLastError();
  }
  // output rows = the wide dimension (m or n), output columns = the LoRA rank side
  constexpr int WM = 4, WN = 1, TM = 1, TN = 1;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  GkLaunch L;
  L.njobs = njobs;
  L.tiles_pre[0] = 0;
  for (int i = 0; i < kGkMaxJobs; i++) {
    L.jobs.job[i] = jobs[i < njobs ? i : 0];
    const GemmArgs& a = jobs[i < njobs ? i : 0];
    const int tiles = (a.M > 0 && a.N > 0) ? ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) : 0;
    L.tiles_pre[i + 1] = L.tiles_pre[i] + (i < njobs ? tiles : 0);
  }
  const int* toffc = nullptr;
  const int* tmapc = nullptr;
  long cap = a0.G;  // units: groups, or (with partials) at most this many chunks
  if (a0.gkpart) {
    if (!a0.toff_all || !a0.tmap_all || rows_bound < 0) return hipErrorInvalidValue;
    if (a0.gkchunk != 0 && a0.gkchunk != kGkChunk && a0.gkchunk != kGkChunkSmall) return hipErrorInvalidValue;
    const int tab = gk_chunk_table(a0.gkchunk);
    toffc = a0.toff_all + tab * (a0.G + 1);
    tmapc = a0.tmap_all + tile_map_offset(tab, rows_bound, a0.G);
    cap = tile_map_capacity(tab, rows_bound, a0.G);
  } else {
    for (int i = 0; i < njobs; i++)
      if (jobs[i].gkpart) return hipErrorInvalidValue;
  }
  L.tiles_all = L.tiles_pre[njobs];
  const long blocks = (cap * L.tiles_all + 7) / 8 * 8;
  if (blocks > 0)
    hipLaunchKernelGGL((gk_mfma<WM, WN, TM, TN>), dim3((unsigned)blocks), dim3(WM * WN * 64), 0, stream, L,
                       toffc, tmapc);
  return hipGetLastError();
}

hipError_t gemm_gk_reduce(const GemmArgs* jobs, int njobs, int rows_bound, hipStream_t stream) {
  if (njobs <= 0) return hipSuccess;
  if (njobs > kGkMaxJobs) return hipErrorInvalidValue;
  GkJobs j;
  long mn = 0;
  for (int i = 0; i < kGkMaxJobs; i++) j.job[i] = jobs[i < njobs ? i : 0];
  for (int i = 0; i < njobs; i++) {
    if (!jobs[i].gkpart || !jobs[i].toff_all || jobs[i].G != jobs[0].G ||
        gk_chunk_table(jobs[i].gkchunk) != gk_chunk_table(jobs[0].gkchunk))
      return hipErrorInvalidValue;
    mn = std::max(mn, (long)jobs[i].M * jobs[i].N);
  }
  if (jobs[0].G <= 0 || mn <= 0) return hipSuccess;
  if (jobs[0].G > kGkMaxGroups) return hipErrorInvalidValue;
  const unsigned bx = (unsigned)std::min<long>((mn + 255) / 256, 256);
  hipLaunchKernelGGL(gk_reduce, dim3(bx, (unsigned)njobs), dim3(256), 0, stream, j,
                     (const int*)(jobs[0].toff_all + gk_chunk_table(jobs[0].gkchunk) * (jobs[0].G + 1)));
  (void)rows_bound;
  return hipGetLastError();
}

}  // namespace moe
