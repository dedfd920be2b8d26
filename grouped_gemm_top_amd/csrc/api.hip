// C ABI of libmoelora: argument checks, buffer layout and the launch sequence of the MoE-LoRA
// layer (routing, forward, backward). See include/moelora.h for the contract of each call.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/moelora.h"
#include "gemm.h"
#include "kernels.h"

using namespace moe;

namespace {

// Bump allocator over a caller buffer; with base == nullptr it only measures.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((char*)b) {}
  template <typename T> T* take(size_t count) {
    off = align_up(off, 256);
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  void* bytes(size_t n) { return take<char>(n); }
};

struct RouteState {
  float* logits;
  float* psel;
  int* row_tok;
  int* rank;
  int* blk_hist;
  int* blk_base;
  int* tiles;
  int* tmaps;
  float* zpart;  // K-split partial router logits
  void* wr_pad;  // bf16 with E % 8 != 0: W_r with rows padded to E8 columns (zeros past E)
};

// K splits of the router-logit GEMM (64 x 128 tiles): the most splits that divide its K tiles into
// chunks of at least 256 with at most 512 workgroups (two per CU), so that each workgroup's chain of
// K tiles is short; every split adds s x E fp32 partials that top-k reads back.
// W_r's rows padded to a multiple of 8 columns (16 bytes of bf16) for the router GEMM's chunk loads
inline int router_cols(const moe_shape& s) { return (s.E + 7) & ~7; }
inline bool router_padded(const moe_shape& s) { return s.dtype == MOE_DTYPE_BF16 && s.E % 8 != 0; }

inline int route_ksplit(const moe_shape& s) {
  const long tiles = ((long)s.s + 63) / 64 * (((long)s.E + 127) / 128);
  const int kt = s.m / 64;  // K tiles (m is a multiple of 64)
  int best = 1;
  for (int n = 2; n <= 16; n++)
    if (kt % n == 0 && s.m / n >= 256 && tiles * n <= 512) best = n;
  return best;
}

struct FwdBufs {
  void *gu, *h, *Tgu, *Td, *o;
};

struct BwdBufs {
  float* ds;
  float* dz;
  void* WrT;
  void *Ud, *dgu, *Ugu, *dXp;
  void *Udw, *Tdw;  // routed rows: w * Uc_d and w * Tc_d (the routing weight of each row's pair)
  float* gkpart;  // partial LoRA-factor gradients of experts longer than one row chunk, one region
                  // per gradient launch (outputs n x r, m x r, m x 2r, n x r, n x r)
  void *At_d, *At_g, *At_u;  // output-major base weights only: A_d, A_g, A_u per expert transposed
};

inline size_t esize(const moe_shape& s) { return s.dtype == MOE_DTYPE_BF16 ? 2 : 4; }
// LoRA scale c: alpha / r, or alpha / sqrt(r) for rank-stabilised LoRA.
inline float lora_scale(const moe_shape& s) {
  return (s.flags & MOE_FLAG_RSLORA) ? s.alpha / std::sqrt((float)s.r) : s.alpha / (float)s.r;
}
inline bool out_in(const moe_shape& s) { return (s.flags & MOE_FLAG_WEIGHTS_OUT_IN) != 0; }
inline bool merged(const moe_shape& s) { return (s.flags & MOE_FLAG_MERGED) != 0; }
inline bool recompute(const moe_shape& s) { return (s.flags & MOE_FLAG_RECOMPUTE) != 0; }
// one LoRA pair on the fused gate/up projection: A [E, m, r] in A_g, B [E, r, 2n] in B_g
inline bool fused_gu(const moe_shape& s) { return (s.flags & MOE_FLAG_FUSED_GU_LORA) != 0; }
inline long pairs(const moe_shape& s) { return (long)s.s * s.k; }
// Rows per chunk of the LoRA-gradient reductions: a shared expert's single group (E == 1 internally,
// and never empty when reduced) takes small chunks so that its reductions fill the chip.
inline int gk_chunk_rows(const moe_shape& s) { return s.E == 1 ? kGkChunkSmall : kGkChunk; }
// ds of a pair arrives as one partial per 64 columns of the expert intermediate (n % 64 == 0)
inline int ds_parts(const moe_shape& s) { return s.n / 64; }
inline int nblocks(const moe_shape& s) { return (s.s + kRouteBlockTokens - 1) / kRouteBlockTokens; }

size_t route_layout(const moe_shape& s, void* base, RouteState* rs) {
  Carve c(base);
  const long P = pairs(s);
  const int nb = nblocks(s);
  RouteState r;
  r.logits = c.take<float>((size_t)s.s * s.E);
  r.psel = c.take<float>((size_t)P);
  r.row_tok = c.take<int>((size_t)P);
  r.rank = c.take<int>((size_t)P);
  r.blk_hist = c.take<int>((size_t)nb * s.E);
  r.blk_base = c.take<int>((size_t)nb * s.E);
  r.tiles = c.take<int>((size_t)kNumTileSizes * (s.E + 1));
  r.tmaps = c.take<int>((size_t)tile_map_offset(kNumTileSizes, P, s.E));
  r.zpart = c.take<float>((size_t)route_ksplit(s) * s.s * s.E);
  r.wr_pad = c.bytes(router_padded(s) ? (size_t)s.m * router_cols(s) * 2 : 0);
  if (rs) *rs = r;
  return align_up(c.off, 256);
}

// with_o: room for the expert outputs o (the routed layer's combine input; a shared expert adds its
// output straight into Y and keeps none)
size_t fwd_layout(const moe_shape& s, void* base, FwdBufs* fb, bool with_o = true) {
  Carve c(base);
  const size_t P = (size_t)pairs(s), es = esize(s);
  FwdBufs f;
  f.gu = c.bytes(P * 2 * s.n * es);
  f.h = c.bytes(P * s.n * es);
  f.Tgu = c.bytes(P * 2 * s.r * es);
  f.Td = c.bytes(P * s.r * es);
  f.o = with_o ? c.bytes(P * s.m * es) : nullptr;
  if (fb) *fb = f;
  return align_up(c.off, 256);
}

// Forward scratch for output-major base weights: B_g, B_u, B_d per expert transposed, so that the
// Split-LoRA tails read them in the layout of the weights they extend.
struct FwdFactors {
  void *Bt_g, *Bt_u, *Bt_d;
};
size_t fwd_factor_layout(const moe_shape& s, void* base, FwdFactors* ff) {
  Carve c(base);
  const size_t es = esize(s), fac = (out_in(s) && !merged(s)) ? 1 : 0;
  FwdFactors f;
  const size_t gu_halves = fused_gu(s) ? 2 : 1;  // fused: B^T [2n, r] per expert, all in Bt_g
  f.Bt_g = c.bytes(fac * gu_halves * s.E * s.r * s.n * es);
  f.Bt_u = c.bytes(fac * (2 - gu_halves) * s.E * s.r * s.n * es);
  f.Bt_d = c.bytes(fac * s.E * s.r * s.m * es);
  if (ff) *ff = f;
  return align_up(c.off, 256);
}

// Backward workspace tail for recomputing the forward's intermediates (MOE_FLAG_RECOMPUTE).
size_t recompute_bytes(const moe_shape& s, bool with_o = true) {
  return recompute(s) ? fwd_layout(s, nullptr, nullptr, with_o) + fwd_factor_layout(s, nullptr, nullptr) : 0;
}

// routed: the router/unpermute buffers (ds, dz, W_r^T, dXp) and the row-weighted low-rank
// products; a shared expert adds its dX straight into the caller's. Both read dY itself as the
// gradient at the expert outputs (the routed rows gather it and apply their routing weight), so no
// dO = w dY rows are written.
size_t bwd_layout(const moe_shape& s, void* base, BwdBufs* bb, bool routed = true) {
  Carve c(base);
  const size_t P = (size_t)pairs(s), es = esize(s), rt = routed ? 1 : 0;
  BwdBufs b;
  b.ds = c.take<float>(rt * P * ds_parts(s));  // [ds_parts][P] partials
  b.dz = c.take<float>(rt * P);
  b.WrT = c.bytes(rt * s.E * s.m * es);
  b.Ud = c.bytes(P * s.r * es);
  b.dgu = c.bytes(P * 2 * s.n * es);
  b.Ugu = c.bytes(P * 2 * s.r * es);
  b.dXp = c.bytes(rt * P * s.m * es);
  b.Udw = c.bytes(rt * P * s.r * es);
  b.Tdw = c.bytes(rt * P * s.r * es);
  b.gkpart = c.take<float>((size_t)gk_part_floats((long)P, s.E, 1, 3L * (s.n + s.m) * s.r, gk_chunk_rows(s)));
  const size_t fac = out_in(s) ? 1 : 0;  // the tails then read the factors in the weights' layout
  b.At_d = c.bytes(fac * s.E * s.r * s.n * es);
  b.At_g = c.bytes(fac * s.E * s.r * s.m * es);
  b.At_u = c.bytes(fac * s.E * s.r * s.m * es);
  if (bb) *bb = b;
  return align_up(c.off, 256);
}

moe_status check_shape(const moe_shape* sp) {
  if (!sp) return MOE_ERR_INVALID_ARG;
  const moe_shape& s = *sp;
  if (s.s < 0 || s.m <= 0 || s.n <= 0 || s.E <= 0 || s.k <= 0 || s.r <= 0) return MOE_ERR_INVALID_ARG;
  if (s.k > s.E) return MOE_ERR_INVALID_ARG;
  if (s.dtype != MOE_DTYPE_F32 && s.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (s.score != MOE_SCORE_SOFTMAX && s.score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if ((s.renormalize != 0 && s.renormalize != 1) || (s.router_grad != 0 && s.router_grad != 1))
    return MOE_ERR_INVALID_ARG;
  if (s.flags & ~(MOE_FLAG_REFERENCE_GEMM | MOE_FLAG_RSLORA | MOE_FLAG_WEIGHTS_OUT_IN | MOE_FLAG_MERGED |
                  MOE_FLAG_RECOMPUTE | MOE_FLAG_FUSED_GU_LORA))
    return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(s.alpha)) return MOE_ERR_INVALID_ARG;
  if (s.m % 64 || s.n % 64) return MOE_ERR_UNSUPPORTED;
  if (s.E > 1024 || s.r > 64) return MOE_ERR_UNSUPPORTED;
  if (s.dtype == MOE_DTYPE_BF16 && s.r % 8) return MOE_ERR_UNSUPPORTED;
  // pair and row indices are 32-bit (element offsets are 64-bit everywhere)
  if ((long)s.s * s.k >= (1L << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// A device pointer argument holding `count` elements: required and 16-byte aligned when count > 0.
inline bool ptr_ok(const void* p, size_t count) {
  if (count == 0) return true;
  return p != nullptr && ((uintptr_t)p & 15u) == 0;
}

// The LoRA factors (or, with a fused gate/up pair, A in A_g and B [E, r, 2n] in B_g; A_u, B_u unused).
inline bool lora_ptrs_ok(const moe_shape& s, const void* A_g, const void* B_g, const void* A_u,
                         const void* B_u, const void* A_d, const void* B_d) {
  const size_t E = s.E, m = s.m, n = s.n, r = s.r;
  const bool fz = fused_gu(s);
  return ptr_ok(A_g, E * m * r) && ptr_ok(B_g, E * r * n * (fz ? 2 : 1)) &&
         (fz || (ptr_ok(A_u, E * m * r) && ptr_ok(B_u, E * r * n))) && ptr_ok(A_d, E * n * r) &&
         ptr_ok(B_d, E * r * m);
}

#define HIP_TRY_STATUS(x)           \
  do {                              \
    const moe_status st_ = (x);     \
    if (st_ != MOE_OK) return st_;  \
  } while (0)

#define HIP_TRY(x)                           \
  do {                                       \
    if ((x) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)


// ------------------------------------------------------------------------------------------------
// Optional per-stage timing (diagnostics): hipEvent pairs recorded on the call's stream around each
// stage while enabled, resolved and summed by moe_timing_read.
enum Stage {
  ST_ROUTE_LOGITS, ST_ROUTE_TOPK, ST_ROUTE_HIST, ST_ROUTE_SCAN, ST_ROUTE_SCATTER,
  ST_FWD_T_GU, ST_FWD_GATE_UP, ST_FWD_T_D, ST_FWD_DOWN, ST_FWD_COMBINE,
  ST_BWD_ROUTER, ST_BWD_U_D, ST_BWD_DOWN, ST_BWD_U_GU,
  ST_BWD_GATE_UP, ST_BWD_UNPERMUTE, ST_BWD_GRADS, ST_COUNT
};
const char* const kStageNames[ST_COUNT] = {
  "route_logits", "route_topk", "route_hist_rank", "route_scan", "route_scatter",
  "fwd_lora_t_gate_up", "fwd_gate_up", "fwd_lora_t_down", "fwd_down", "fwd_combine",
  "bwd_router", "bwd_lora_u_down", "bwd_down",
  "bwd_lora_u_gate_up", "bwd_gate_up", "bwd_unpermute", "bwd_lora_grads"};

struct Timing {
  std::mutex mu;
  bool on = false;
  struct Pending { int stage; hipEvent_t b, e; };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[ST_COUNT] = {};
  long long count[ST_COUNT] = {};
};
Timing g_timing;

hipEvent_t timing_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t ev = g_timing.pool.back();
    g_timing.pool.pop_back();
    return ev;
  }
  hipEvent_t ev = nullptr;
  if (hipEventCreate(&ev) != hipSuccess) return nullptr;
  return ev;
}

struct StageScope {
  int stage;
  hipStream_t st;
  hipEvent_t b = nullptr;
  StageScope(int s_, hipStream_t st_) : stage(s_), st(st_) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!g_timing.on) return;
    b = timing_event();
    if (b && hipEventRecord(b, st) != hipSuccess) {
      g_timing.pool.push_back(b);
      b = nullptr;
    }
  }
  ~StageScope() {
    if (!b) return;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    hipEvent_t e = timing_event();
    if (e && hipEventRecord(e, st) == hipSuccess) {
      g_timing.pending.push_back({stage, b, e});
    } else {
      g_timing.pool.push_back(b);
      if (e) g_timing.pool.push_back(e);
    }
  }
};

#define STAGE(id, x)                  \
  do {                                \
    StageScope stage_scope_((id), hs); \
    HIP_TRY(x);                       \
  } while (0)

// ------------------------------------------------------------------------------------------------
// Device scratch of moe_lora_forward_noalloc: one fixed array per GPU, resident from the library's
// load on that GPU until the process ends. Host code never uses the array's name as an address (on
// the host it is only a stand-in for the symbol): its device address comes from hipGetSymbolAddress,
// looked up once per device with that device current, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on that device).
moe_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

GemmArgs gemm_args() {
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.scale = 1.0f;
  return a;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int32_t moe_abi_version(void) { return 1; }

moe_status moe_check_shape(const moe_shape* shape) { return check_shape(shape); }

size_t moe_route_state_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return route_layout(*shape, nullptr, nullptr);
}

size_t moe_fwd_saved_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return fwd_layout(*shape, nullptr, nullptr, false);
}

// The expert outputs o are scratch: only the forward's combine reads them (the backward takes ds from
// the down projection's backward), so they live in the workspace, not in `saved`.
inline size_t o_bytes(const moe_shape& s) { return align_up((size_t)pairs(s) * s.m * esize(s), 256); }

size_t moe_fwd_ws_bytes(const moe_shape* shape, int32_t with_saved) {
  if (check_shape(shape) != MOE_OK) return 0;
  const moe_shape& s = *shape;
  return (with_saved ? o_bytes(s) : fwd_layout(s, nullptr, nullptr, true)) + fwd_factor_layout(s, nullptr, nullptr);
}

size_t moe_bwd_ws_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return bwd_layout(*shape, nullptr, nullptr) + recompute_bytes(*shape, false);
}

moe_status moe_route(const moe_shape* shape, const void* X, const void* W_r,
                     const float* router_bias, float* logits, int32_t* topk_idx, float* topk_w,
                     int32_t* expert_off, int32_t* perm, int32_t* inv_perm, void* route_state,
                     size_t route_state_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  const long P = pairs(s);
  if (!ptr_ok(X, (size_t)s.s * s.m) || !ptr_ok(W_r, (size_t)s.m * s.E) ||
      !ptr_ok(topk_idx, P) || !ptr_ok(topk_w, P) || !ptr_ok(expert_off, s.E + 1) ||
      !ptr_ok(perm, P) || !ptr_ok(inv_perm, P))
    return MOE_ERR_INVALID_ARG;
  if ((router_bias && ((uintptr_t)router_bias & 15u)) || (logits && ((uintptr_t)logits & 15u)))
    return MOE_ERR_INVALID_ARG;
  const size_t need = route_layout(s, nullptr, nullptr);
  if (!route_state || ((uintptr_t)route_state & 255u)) return MOE_ERR_INVALID_ARG;
  if (route_state_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t hs = (hipStream_t)stream;
  RouteState rs;
  route_layout(s, route_state, &rs);
  if (s.s == 0) {
    HIP_TRY(launch_zero(expert_off, s.E + 1, hs));
    HIP_TRY(launch_zero(rs.tiles, (size_t)kNumTileSizes * (s.E + 1), hs));
    return MOE_OK;
  }
  float* z = logits ? logits : rs.logits;
  const int ref = (s.flags & MOE_FLAG_REFERENCE_GEMM) ? 1 : 0;
  const int nsplit = (ref || s.dtype != MOE_DTYPE_BF16) ? 1 : route_ksplit(s);
  GemmArgs a = gemm_args();
  a.M = s.s;
  a.N = s.E;
  a.K = s.m;
  a.G = 1;
  a.A = X;
  a.lda = s.m;
  a.B = W_r;
  a.ldb = s.E;
  if (router_padded(s)) {  // bf16 rows of E columns are not 16-byte aligned: a padded copy
    STAGE(ST_ROUTE_LOGITS, launch_pad_cols(W_r, rs.wr_pad, s.m, s.E, router_cols(s), hs));
    a.B = rs.wr_pad;
    a.ldb = router_cols(s);
  }
  a.C = nsplit > 1 ? rs.zpart : z;
  a.ldc = s.E;
  a.bias = router_bias;
  if (nsplit > 1) {
    a.kchunk = s.m / nsplit;
    a.csplit = (long)s.s * s.E;
  }
  STAGE(ST_ROUTE_LOGITS, gemm_gm_launch(a, LAYOUT_KX, EPI_STORE, 1, s.dtype, s.s, ref, hs));
  STAGE(ST_ROUTE_TOPK, launch_topk(nsplit > 1 ? rs.zpart : z, nsplit, (long)s.s * s.E, z, s.s, s.E, s.k,
                                   s.score, s.renormalize, topk_idx, topk_w, rs.psel, hs));
  STAGE(ST_ROUTE_HIST, launch_hist_rank(topk_idx, s.s, s.k, s.E, rs.blk_hist, rs.rank, hs));
  STAGE(ST_ROUTE_SCAN, launch_scan(rs.blk_hist, nblocks(s), s.E, (int)P, rs.blk_base, expert_off, rs.tiles, rs.tmaps, hs));
  STAGE(ST_ROUTE_SCATTER, launch_scatter(topk_idx, rs.rank, rs.blk_base, s.s, s.k, s.E, perm, inv_perm, rs.row_tok, hs));
  return MOE_OK;
}

// The forward's expert stages, everything but the combine: the low-rank products Tc, the gate/up
// GEMM with its SwiGLU epilogue and the down GEMM, writing gu, h, Tc_gu, Tc_d and o into f (ff:
// transposed tail factors for output-major weights). Shared by the forward and by a backward that
// recomputes them.
// Routed rows' view of dY: grouped row i holds pair p = pair[i] of token p / k, with weight w[p]; the
// gradient at its expert output is w[p] dY[p / k].
struct RowWeights {
  const int32_t* pair;
  int k;
  const float* w;
  float* ds;  // when set: ds partials of every pair, [ds_parts(s)][P] (see moe_lora_backward)
  // The routed layer's last steps, run inside the expert backward as soon as their inputs exist: the
  // router backward (dz, when ds is set) after the down projection's backward, and the unpermute into dX
  // right after the dXp GEMM (while dXp is still cache-resident).
  float* dz;
  const float* psel;
  const int32_t* inv;
  const int32_t* idx;
  const void* WrT;
  void* dX;
};

// Row grouping of the expert GEMMs: G groups of rows (off[G + 1]); grouped row i reads activation
// row arow[i] / arow_div of X (arow == nullptr: row i), with the row-tile tables of launch_scan.
struct Grouping {
  int G;
  const int32_t* off;
  const int32_t* arow;
  int arow_div;
  const int* tiles;
  const int* tmaps;
};

// The expert MLPs with Split LoRA over the grouped rows. The down projection's output goes to o_dst
// (overwritten, or added to with accum; not computed when o_dst is null).
static moe_status forward_experts(const moe_shape& s, const void* X, const Grouping& gr, const void* W_gu,
                           const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                           const void* B_u, const void* A_d, const void* B_d, const FwdBufs& f,
                           const FwdFactors& ff, void* o_dst, int accum, hipStream_t hs) {
  const long P = pairs(s);
  const size_t m = s.m, n = s.n, r = s.r;
  const int ref = (s.flags & MOE_FLAG_REFERENCE_GEMM) ? 1 : 0;
  const float c = lora_scale(s);
  const int Pi = (int)P;
  const bool fz = fused_gu(s);
  if (out_in(s) && !merged(s)) {  // [E, r, n] -> [E, n, r] and [E, r, m] -> [E, m, r]
    if (fz) {                     // [E, r, 2n] -> [E, 2n, r]
      STAGE(ST_FWD_GATE_UP, launch_transpose(s.dtype, B_g, ff.Bt_g, s.r, 2 * s.n, s.E, hs));
    } else {
      STAGE(ST_FWD_GATE_UP, launch_transpose(s.dtype, B_g, ff.Bt_g, s.r, s.n, s.E, hs));
      STAGE(ST_FWD_GATE_UP, launch_transpose(s.dtype, B_u, ff.Bt_u, s.r, s.n, s.E, hs));
    }
    STAGE(ST_FWD_DOWN, launch_transpose(s.dtype, B_d, ff.Bt_d, s.r, s.m, s.E, hs));
  }


  GemmArgs base = gemm_args();
  base.G = gr.G;
  base.goff = gr.off;
  base.toff_all = gr.tiles;
  base.tmap_all = gr.tmaps;

  // The grouped row i of every expert GEMM is pair perm[i]; its activation row is X[perm[i] / k],
  // gathered by the GEMM kernels (no permuted copy of X is written).
  // Tc_gu = c * Xp [A_g | A_u]  (fused pair: Tc = c * Xp A, P x r)
  if (!merged(s) && fz) {
    GemmArgs a = base;
    a.N = s.r; a.K = s.m;
    a.A = X; a.lda = s.m; a.arow = gr.arow; a.arow_div = gr.arow_div;
    a.B = A_g; a.ldb = s.r; a.bstride = (long)m * r;
    a.C = f.Tgu; a.ldc = s.r; a.scale = c;
    STAGE(ST_FWD_T_GU, gemm_gm_launch(a, LAYOUT_KX, EPI_STORE, 0, s.dtype, Pi, ref, hs));
  } else if (!merged(s)) {
    GemmArgs a = base;
    a.N = s.r; a.K = s.m;
    a.A = X; a.lda = s.m; a.arow = gr.arow; a.arow_div = gr.arow_div;
    a.B = A_g; a.Bu = A_u; a.ldb = s.r; a.bstride = (long)m * r;
    a.C = f.Tgu; a.ldc = 2 * s.r; a.cup = s.r; a.scale = c;
    STAGE(ST_FWD_T_GU, gemm_gm_launch(a, LAYOUT_KX, EPI_DUAL, 0, s.dtype, Pi, ref, hs));
  }
  // [g | u] = Xp W_gu + [Tc_g B_g | Tc_u B_u];  h = silu(g) * u
  {
    GemmArgs a = base;
    a.N = s.n; a.K = s.m;
    a.A = X; a.lda = s.m; a.arow = gr.arow; a.arow_div = gr.arow_div;
    a.B = W_gu; a.bstride = (long)m * 2 * n;
    if (out_in(s)) {  // W_gu [E, 2n, m]: the up half starts n rows in
      a.Bu = (const char*)W_gu + n * m * esize(s); a.ldb = s.m;
    } else {          // W_gu [E, m, 2n]: the up half starts n columns in
      a.Bu = (const char*)W_gu + n * esize(s); a.ldb = 2 * s.n;
    }
    a.tail = merged(s) ? TAIL_NONE : TAIL_BLOCKDIAG; a.r2a = s.r;
    a.TA = f.Tgu; a.lda2 = 2 * s.r;
    if (out_in(s)) {
      a.TB0 = ff.Bt_g; a.TB1 = ff.Bt_u; a.ldtb = s.r;
    } else {
      a.TB0 = B_g; a.TB1 = B_u; a.ldtb = s.n;
    }
    a.tbstride = (long)r * n;
    if (fz && !merged(s)) {  // [g | u] tails Tc [B_g-part | B_u-part] with one shared Tc
      a.tail = TAIL_SHARED;
      a.lda2 = s.r;
      a.tbstride = (long)r * 2 * n;
      if (out_in(s)) {  // B^T [E, 2n, r]: the up rows start n rows in
        a.TB0 = ff.Bt_g; a.TB1 = (const char*)ff.Bt_g + n * r * esize(s); a.ldtb = s.r;
      } else {          // B [E, r, 2n]: the up columns start n columns in
        a.TB0 = B_g; a.TB1 = (const char*)B_g + n * esize(s); a.ldtb = 2 * s.n;
      }
    }
    a.C = f.gu; a.ldc = 2 * s.n; a.cup = s.n;
    a.H = f.h; a.ldh = s.n;
    STAGE(ST_FWD_GATE_UP, gemm_gm_launch(a, out_in(s) ? LAYOUT_XK : LAYOUT_KX, EPI_SWIGLU, 0, s.dtype, Pi,
                                         ref, hs));
  }
  // Tc_d = c * h A_d
  if (!merged(s)) {
    GemmArgs a = base;
    a.N = s.r; a.K = s.n;
    a.A = f.h; a.lda = s.n;
    a.B = A_d; a.ldb = s.r; a.bstride = (long)n * r;
    a.C = f.Td; a.ldc = s.r; a.scale = c;
    STAGE(ST_FWD_T_D, gemm_gm_launch(a, LAYOUT_KX, EPI_STORE, 0, s.dtype, Pi, ref, hs));
  }
  // o = h W_d + Tc_d B_d  (skipped when no destination is given: a recompute that needs only the
  // intermediates before it)
  if (o_dst) {
    GemmArgs a = base;
    a.N = s.m; a.K = s.n;
    a.A = f.h; a.lda = s.n;
    a.B = W_d; a.ldb = out_in(s) ? s.n : s.m; a.bstride = (long)n * m;
    a.tail = merged(s) ? TAIL_NONE : TAIL_SINGLE; a.r2a = s.r;
    a.TA = f.Td; a.lda2 = s.r;
    a.TB0 = out_in(s) ? ff.Bt_d : B_d; a.ldtb = out_in(s) ? s.r : s.m; a.tbstride = (long)r * m;
    a.C = o_dst; a.ldc = s.m; a.accum = accum;
    STAGE(ST_FWD_DOWN, gemm_gm_launch(a, out_in(s) ? LAYOUT_XK : LAYOUT_KX, EPI_STORE, 0, s.dtype, Pi, ref,
                                      hs));
  }
  return MOE_OK;
}

// The routed forward's shape and every buffer but its workspaces (shared by both forward entry points).
static moe_status forward_args(const moe_shape* shape, const void* X, const int32_t* topk_idx,
                               const float* topk_w, const int32_t* expert_off, const int32_t* perm,
                               const int32_t* inv_perm, const void* route_state, const void* W_gu,
                               const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                               const void* B_u, const void* A_d, const void* B_d, const void* Y) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  const long P = pairs(s);
  const size_t E = s.E, m = s.m, n = s.n;
  if (!ptr_ok(X, (size_t)s.s * m) || !ptr_ok(topk_idx, P) || !ptr_ok(topk_w, P) ||
      !ptr_ok(expert_off, E + 1) || !ptr_ok(perm, P) || !ptr_ok(inv_perm, P) ||
      !ptr_ok(W_gu, E * m * 2 * n) || !ptr_ok(W_d, E * n * m) || !ptr_ok(Y, (size_t)s.s * m))
    return MOE_ERR_INVALID_ARG;
  if (!merged(s) && !lora_ptrs_ok(s, A_g, B_g, A_u, B_u, A_d, B_d)) return MOE_ERR_INVALID_ARG;
  if (!route_state || ((uintptr_t)route_state & 255u)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status moe_lora_forward(const moe_shape* shape, const void* X, const int32_t* topk_idx,
                            const float* topk_w, const int32_t* expert_off, const int32_t* perm,
                            const int32_t* inv_perm, const void* route_state, const void* W_gu,
                            const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                            const void* B_u, const void* A_d, const void* B_d, void* Y, void* saved,
                            size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = forward_args(shape, X, topk_idx, topk_w, expert_off, perm, inv_perm, route_state, W_gu, W_d,
                               A_g, B_g, A_u, B_u, A_d, B_d, Y);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  // saved: gu, h and the low-rank products; ws: the expert outputs o (and, for inference, the rest)
  const size_t need_saved = fwd_layout(s, nullptr, nullptr, false);
  const size_t need_inter = saved ? o_bytes(s) : fwd_layout(s, nullptr, nullptr, true);
  const size_t need_fac = fwd_factor_layout(s, nullptr, nullptr);
  const size_t need_ws = need_inter + need_fac;
  if (saved) {
    if ((uintptr_t)saved & 255u) return MOE_ERR_INVALID_ARG;
    if (saved_bytes < need_saved) return MOE_ERR_WORKSPACE;
  }
  if (ws_bytes < need_ws) return MOE_ERR_WORKSPACE;
  if (need_ws && (!ws || ((uintptr_t)ws & 255u))) return MOE_ERR_INVALID_ARG;
  if (s.s == 0) return MOE_OK;
  hipStream_t hs = (hipStream_t)stream;
  RouteState rs;
  route_layout(s, const_cast<void*>(route_state), &rs);
  FwdBufs f;
  if (saved) {
    fwd_layout(s, saved, &f, false);
    f.o = ws;
  } else {
    fwd_layout(s, ws, &f, true);
  }
  FwdFactors ff;
  fwd_factor_layout(s, (char*)ws + need_inter, &ff);
  const Grouping gr{s.E, expert_off, perm, s.k, rs.tiles, rs.tmaps};
  HIP_TRY_STATUS(forward_experts(s, X, gr, W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, f, ff, f.o, 0, hs));
  // combine
  STAGE(ST_FWD_COMBINE, launch_combine(s.dtype, f.o, inv_perm, topk_w, Y, s.s, s.k, s.m, hs));
  return MOE_OK;
}

moe_status moe_lora_forward_noalloc(const moe_shape* shape, const void* X, const int32_t* topk_idx,
                                    const float* topk_w, const int32_t* expert_off, const int32_t* perm,
                                    const int32_t* inv_perm, const void* route_state, const void* W_gu,
                                    const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                                    const void* B_u, const void* A_d, const void* B_d, void* Y,
                                    void* stream) {
  // arguments first: a call that is refused makes no runtime call at all
  moe_status st = forward_args(shape, X, topk_idx, topk_w, expert_off, perm, inv_perm, route_state, W_gu, W_d,
                               A_g, B_g, A_u, B_u, A_d, B_d, Y);
  if (st != MOE_OK) return st;
  const size_t need = moe_fwd_ws_bytes(shape, 0);
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need) HIP_TRY_STATUS(scratch_address(&ws));
  // the inference forward of moe_lora_forward with the scratch as its workspace: every byte of it
  // that a kernel reads is written earlier in the same call, so nothing needs clearing
  return moe_lora_forward(shape, X, topk_idx, topk_w, expert_off, perm, inv_perm, route_state, W_gu, W_d,
                          A_g, B_g, A_u, B_u, A_d, B_d, Y, nullptr, 0, ws, need, stream);
}

moe_status moe_peft_merge(const moe_shape* shape, const void* W_gu, const void* W_d, const void* A_g,
                          const void* B_g, const void* A_u, const void* B_u, const void* A_d,
                          const void* B_d, void* W_gu_merged, void* W_d_merged, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  const size_t E = s.E, m = s.m, n = s.n, r = s.r;
  if (!ptr_ok(W_gu, E * m * 2 * n) || !ptr_ok(W_d, E * n * m) ||
      !lora_ptrs_ok(s, A_g, B_g, A_u, B_u, A_d, B_d) || !ptr_ok(W_gu_merged, E * m * 2 * n) ||
      !ptr_ok(W_d_merged, E * n * m) || W_gu_merged == W_gu || W_d_merged == W_d)
    return MOE_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  const float c = lora_scale(s);
  const bool kx = !out_in(s);
  const long ld_gu = kx ? 2L * n : (long)m, ld_d = kx ? (long)m : (long)n;
  // gate columns [0, n) and up columns [n, 2n) of W_gu (K = m), then W_d (K = n, N = m)
  if (fused_gu(s)) {  // one pair over all 2n columns
    HIP_TRY(launch_merge(s.dtype, kx, W_gu, A_g, B_g, W_gu_merged, s.E, s.m, 2 * s.n, s.r, ld_gu, 0,
                         (long)m * 2 * n, c, hs));
  } else {
    HIP_TRY(launch_merge(s.dtype, kx, W_gu, A_g, B_g, W_gu_merged, s.E, s.m, s.n, s.r, ld_gu, 0,
                         (long)m * 2 * n, c, hs));
    HIP_TRY(launch_merge(s.dtype, kx, W_gu, A_u, B_u, W_gu_merged, s.E, s.m, s.n, s.r, ld_gu, (long)n,
                         (long)m * 2 * n, c, hs));
  }
  HIP_TRY(launch_merge(s.dtype, kx, W_d, A_d, B_d, W_d_merged, s.E, s.n, s.m, s.r, ld_d, 0,
                       (long)n * m, c, hs));
  return MOE_OK;
}

static moe_status backward_experts(const moe_shape& s, const Grouping& gr, const void* X, const void* dO,
                                   const RowWeights* rw, const void* W_gu, const void* W_d, const void* A_g,
                                   const void* B_g,
                                   const void* A_u, const void* B_u, const void* A_d, const void* B_d,
                                   const FwdBufs& f, const BwdBufs& b, void* dXp_dst, int accum,
                                   float* dA_g, float* dB_g, float* dA_u, float* dB_u, float* dA_d,
                                   float* dB_d, hipStream_t hs);

moe_status moe_lora_backward(const moe_shape* shape, const void* dY, const void* X,
                             const void* W_r, const int32_t* topk_idx, const float* topk_w,
                             const int32_t* expert_off, const int32_t* perm,
                             const int32_t* inv_perm, const void* route_state, const void* W_gu,
                             const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                             const void* B_u, const void* A_d, const void* B_d, const void* saved,
                             size_t saved_bytes, void* dX, float* dA_g, float* dB_g, float* dA_u,
                             float* dB_u, float* dA_d, float* dB_d, void* ws, size_t ws_bytes,
                             void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (s.router_grad && s.score == MOE_SCORE_SOFTMAX && !s.renormalize) return MOE_ERR_UNSUPPORTED;
  if (merged(s)) return MOE_ERR_UNSUPPORTED;
  const long P = pairs(s);
  const size_t E = s.E, m = s.m, n = s.n, r = s.r;
  if (!ptr_ok(dY, (size_t)s.s * m) || !ptr_ok(X, (size_t)s.s * m) || !ptr_ok(W_r, m * E) ||
      !ptr_ok(topk_idx, P) || !ptr_ok(topk_w, P) || !ptr_ok(expert_off, E + 1) ||
      !ptr_ok(perm, P) || !ptr_ok(inv_perm, P) || !ptr_ok(W_gu, E * m * 2 * n) ||
      !ptr_ok(W_d, E * n * m) || !lora_ptrs_ok(s, A_g, B_g, A_u, B_u, A_d, B_d) ||
      !ptr_ok(dX, (size_t)s.s * m) || !ptr_ok(dA_g, E * m * r) ||
      !ptr_ok(dB_g, E * r * n * (fused_gu(s) ? 2 : 1)) ||
      (!fused_gu(s) && (!ptr_ok(dA_u, E * m * r) || !ptr_ok(dB_u, E * r * n))) ||
      !ptr_ok(dA_d, E * n * r) || !ptr_ok(dB_d, E * r * m))
    return MOE_ERR_INVALID_ARG;
  if (!route_state || ((uintptr_t)route_state & 255u)) return MOE_ERR_INVALID_ARG;
  const bool redo = !saved;  // recompute the forward's intermediates
  if (redo && !recompute(s)) return MOE_ERR_INVALID_ARG;
  if (saved && ((uintptr_t)saved & 255u)) return MOE_ERR_INVALID_ARG;
  if (saved && saved_bytes < fwd_layout(s, nullptr, nullptr, false)) return MOE_ERR_WORKSPACE;
  const size_t bwd_bytes = bwd_layout(s, nullptr, nullptr);
  const size_t need_ws = bwd_bytes + (redo ? recompute_bytes(s, false) : 0);
  if (ws_bytes < need_ws) return MOE_ERR_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255u)) return MOE_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  if (s.s == 0) {
    HIP_TRY(launch_zero(dA_g, E * m * r, hs));
    HIP_TRY(launch_zero(dB_g, E * r * n * (fused_gu(s) ? 2 : 1), hs));
    if (!fused_gu(s)) {
      HIP_TRY(launch_zero(dA_u, E * m * r, hs));
      HIP_TRY(launch_zero(dB_u, E * r * n, hs));
    }
    HIP_TRY(launch_zero(dA_d, E * n * r, hs));
    HIP_TRY(launch_zero(dB_d, E * r * m, hs));
    return MOE_OK;
  }
  RouteState rs;
  route_layout(s, const_cast<void*>(route_state), &rs);
  const Grouping gr{s.E, expert_off, perm, s.k, rs.tiles, rs.tmaps};
  FwdBufs f;
  BwdBufs b;
  bwd_layout(s, ws, &b);
  if (redo) {
    char* rbase = (char*)ws + bwd_bytes;
    FwdFactors ff;
    fwd_layout(s, rbase, &f, false);
    fwd_factor_layout(s, rbase + fwd_layout(s, nullptr, nullptr, false), &ff);
    // the intermediates only: the backward needs no expert outputs o
    HIP_TRY_STATUS(forward_experts(s, X, gr, W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, f, ff, nullptr, 0, hs));
  } else {
    fwd_layout(s, const_cast<void*>(saved), &f, false);
  }
  // The gradient at the expert outputs, dO = s_{t,j} dY_t, is never written: the expert GEMMs gather
  // dY rows and apply s_{t,j}. The combine's gradient in the routing weights, ds_{t,j} = dY_t . o_{t,j},
  // equals h . (dY_t W_d^T + Uc A_d^T) for the row's h (o = h W_d + c (h A_d) B_d), so the down
  // projection's backward leaves it as partials over 64-column blocks (with the router gradient).
  // Two small independent jobs in one launch: w * Tc_d rows for dB_d, and the W_r^T rows the unpermute
  // reads for the router's term of dX.
  STAGE(ST_BWD_ROUTER, launch_bwd_prep(s.dtype, f.Td, perm, topk_w, b.Tdw, P, s.r, s.router_grad ? W_r : nullptr,
                                       b.WrT, s.m, s.E, hs));
  // (the router backward and the unpermute run inside, as soon as their inputs exist)
  const RowWeights rw{perm, s.k, topk_w, s.router_grad ? b.ds : nullptr, b.dz, rs.psel, inv_perm, topk_idx, b.WrT,
                      dX};
  HIP_TRY_STATUS(backward_experts(s, gr, X, dY, &rw, W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, f, b, b.dXp, 0,
                                  dA_g, dB_g, dA_u, dB_u, dA_d, dB_d, hs));
  return MOE_OK;
}

// Backward of the expert MLPs over the grouped rows, from dO, the gradient at the down projection's
// output: one row per grouped row, or with rw the rows of dY that rw maps each grouped row to, times
// the row's weight. Computes the LoRA-factor gradients, and the gradient at the grouped activation
// rows written to dXp_dst (overwritten, or added to with accum).
static moe_status backward_experts(const moe_shape& s, const Grouping& gr, const void* X, const void* dO,
                                   const RowWeights* rw, const void* W_gu, const void* W_d, const void* A_g,
                                   const void* B_g,
                                   const void* A_u, const void* B_u, const void* A_d, const void* B_d,
                                   const FwdBufs& f, const BwdBufs& b, void* dXp_dst, int accum,
                                   float* dA_g, float* dB_g, float* dA_u, float* dB_u, float* dA_d,
                                   float* dB_d, hipStream_t hs) {
  const long P = pairs(s);
  const size_t m = s.m, n = s.n, r = s.r;
  const int ref = (s.flags & MOE_FLAG_REFERENCE_GEMM) ? 1 : 0;
  const float c = lora_scale(s);
  const int Pi = (int)P;
  const size_t es = esize(s);

  // LoRA-factor gradients (K-grouped jobs over the same row grouping, run together in one launch
  // after the dXp GEMM): an expert longer than one row chunk leaves fp32 partials in its job's region
  // of b.gkpart, and one reduce after the launch completes all of them
  const bool chunked = s.dtype == MOE_DTYPE_BF16 && !ref;
  GemmArgs gk_jobs[kGkMaxJobs];
  int n_gk = 0;
  float* gk_next = b.gkpart;
  auto gk_prep = [&](GemmArgs& a) {
    a.gkpart = nullptr;
    if (chunked) {
      a.gkpart = gk_next;
      a.gkchunk = gk_chunk_rows(s);
      gk_next += gk_part_floats((long)P, s.E, a.M, a.N, a.gkchunk);
    }
    gk_jobs[n_gk++] = a;
  };

  GemmArgs base = gemm_args();
  base.G = gr.G;
  base.goff = gr.off;
  base.toff_all = gr.tiles;
  base.tmap_all = gr.tmaps;

  // Uc_d = c * dO B_d^T. Routed rows: the product of the gathered dY rows without the weight (for the
  // down projection's tail, whose output is weighted as a whole), and w * that in b.Udw (for dA_d).
  {
    GemmArgs a = base;
    a.N = s.r; a.K = s.m;
    a.A = dO; a.lda = s.m;
    if (rw) { a.arow = rw->pair; a.arow_div = rw->k; a.wval = rw->w; a.C2 = b.Udw; }
    a.B = B_d; a.ldb = s.m; a.bstride = (long)r * m;
    a.C = b.Ud; a.ldc = s.r; a.scale = c;
    STAGE(ST_BWD_U_D, gemm_gm_launch(a, LAYOUT_XK, EPI_STORE, 0, s.dtype, Pi, ref, hs));
  }
  // dh = dO W_d^T + Uc_d A_d^T, then SwiGLU backward -> dgu = [dg | du]. Routed rows:
  // dh = w (dY W_d^T + Uc A_d^T) from the gathered dY rows.
  {
    GemmArgs a = base;
    a.N = s.n; a.K = s.m;
    a.A = dO; a.lda = s.m;
    if (rw) {
      a.arow = rw->pair; a.arow_div = rw->k; a.wval = rw->w; a.wscale = 1;
      a.dspart = rw->ds; a.dsstride = P;
    }
    a.B = W_d; a.ldb = out_in(s) ? s.n : s.m; a.bstride = (long)n * m;
    a.tail = TAIL_SINGLE; a.r2a = s.r;
    a.TA = b.Ud; a.lda2 = s.r;
    if (out_in(s)) {  // A_d [E, n, r] -> [E, r, n]
      STAGE(ST_BWD_DOWN, launch_transpose(s.dtype, A_d, b.At_d, s.n, s.r, s.E, hs));
      a.TB0 = b.At_d; a.ldtb = s.n;
    } else {
      a.TB0 = A_d; a.ldtb = s.r;
    }
    a.tbstride = (long)n * r;
    a.GU = f.gu; a.ldgu = 2 * s.n; a.guup = s.n;
    a.C = b.dgu; a.ldc = 2 * s.n; a.cup = s.n;
    STAGE(ST_BWD_DOWN, gemm_gm_launch(a, out_in(s) ? LAYOUT_KX : LAYOUT_XK, EPI_SWIGLU_BWD, 0, s.dtype, Pi,
                                      ref, hs));
  }
  // router backward (its ds partials are complete): dz on the selected logits
  if (rw && rw->ds)
    STAGE(ST_BWD_ROUTER, launch_router_bwd(rw->ds, ds_parts(s), rw->w, rw->psel, s.s, s.k, s.score,
                                           s.renormalize, rw->dz, hs));
  const bool fz = fused_gu(s);
  // Uc_gu = c * [dg B_g^T | du B_u^T]  (fused pair: Uc = c * [dg | du] B^T, one product over 2n)
  if (fz) {
    GemmArgs a = base;
    a.N = s.r; a.K = 2 * s.n;
    a.A = b.dgu; a.lda = 2 * s.n;
    a.B = B_g; a.ldb = 2 * s.n; a.bstride = (long)r * 2 * n;
    a.C = b.Ugu; a.ldc = s.r; a.scale = c;
    STAGE(ST_BWD_U_GU, gemm_gm_launch(a, LAYOUT_XK, EPI_STORE, 0, s.dtype, Pi, ref, hs));
  } else {  // the gate and up products are independent: one launch runs both
    GemmArgs a = base;
    a.N = s.r; a.K = s.n;
    a.A = b.dgu; a.lda = 2 * s.n;
    a.B = B_g; a.ldb = s.n; a.bstride = (long)r * n;
    a.C = b.Ugu; a.ldc = 2 * s.r; a.scale = c;
    a.nbatch = 2;
    a.bA = (const char*)b.dgu + n * es;
    a.bB = B_u;
    a.bC = (char*)b.Ugu + r * es;
    STAGE(ST_BWD_U_GU, gemm_gm_launch(a, LAYOUT_XK, EPI_STORE, 0, s.dtype, Pi, ref, hs));
  }
  // dXp = dgu W_gu^T + Uc_g A_g^T + Uc_u A_u^T
  {
    GemmArgs a = base;
    a.N = s.m; a.K = 2 * s.n;
    a.A = b.dgu; a.lda = 2 * s.n;
    a.B = W_gu; a.ldb = out_in(s) ? s.m : 2 * s.n; a.bstride = (long)m * 2 * n;
    a.tail = fz ? TAIL_SINGLE : TAIL_STACKED; a.r2a = s.r;
    a.TA = b.Ugu; a.lda2 = fz ? s.r : 2 * s.r;
    if (out_in(s)) {  // A_g, A_u [E, m, r] -> [E, r, m]
      STAGE(ST_BWD_GATE_UP, launch_transpose(s.dtype, A_g, b.At_g, s.m, s.r, s.E, hs));
      if (!fz) STAGE(ST_BWD_GATE_UP, launch_transpose(s.dtype, A_u, b.At_u, s.m, s.r, s.E, hs));
      a.TB0 = b.At_g; a.TB1 = fz ? nullptr : b.At_u; a.ldtb = s.m;
    } else {
      a.TB0 = A_g; a.TB1 = fz ? nullptr : A_u; a.ldtb = s.r;
    }
    a.tbstride = (long)m * r;
    a.C = dXp_dst; a.ldc = s.m; a.accum = accum;
    STAGE(ST_BWD_GATE_UP, gemm_gm_launch(a, out_in(s) ? LAYOUT_KX : LAYOUT_XK, EPI_STORE, 0, s.dtype, Pi, ref,
                                         hs));
  }
  // unpermute: dX[t] = sum_j dXp[inv[t k + j]] (+ sum_j dz[t,j] W_r[:, idx[t,j]])
  if (rw && rw->dX)
    STAGE(ST_BWD_UNPERMUTE, launch_unpermute(s.dtype, dXp_dst, rw->inv, rw->ds ? rw->dz : nullptr, rw->idx, rw->WrT,
                                             rw->dX, s.s, s.k, s.m, hs));
  // LoRA-factor gradients, all in one launch (last: the dgu rows are read by the two GEMMs above while
  // they are still cache-resident)
  // dA_d = h^T Uc_d ;  dB_d = Tc_d^T dO  (computed as (dO^T Tc_d)^T; routed rows: as
  // (dY_rows^T (w Tc_d))^T)
  {
    GemmArgs a = base;
    a.M = s.n; a.N = s.r;
    a.A = f.h; a.lda = s.n;
    a.B = rw ? b.Udw : b.Ud; a.ldb = s.r;
    a.C = dA_d; a.ldc = s.r; a.cstride = (long)n * r;
    gk_prep(a);
    a.M = s.m; a.N = s.r;
    a.A = dO; a.lda = s.m;
    a.B = f.Td; a.ldb = s.r;
    if (rw) {  // w * Tc_d rows: formed by the caller (launch_bwd_prep) before the expert backward
      a.arow = rw->pair; a.arow_div = rw->k;
      a.B = b.Tdw;
    }
    a.C = dB_d; a.ldc = s.m; a.cstride = (long)r * m; a.ctrans = 1;
    gk_prep(a);
  }
  // dA_g | dA_u = Xp^T [Uc_g | Uc_u] ;  dB_g = Tc_g^T dg, dB_u = Tc_u^T du
  if (fz) {  // dA = Xp^T Uc ;  dB = Tc^T [dg | du]
    GemmArgs a = base;
    a.M = s.m; a.N = s.r;
    a.A = X; a.lda = s.m; a.arow = gr.arow; a.arow_div = gr.arow_div;
    a.B = b.Ugu; a.ldb = s.r;
    a.C = dA_g; a.ldc = s.r; a.cstride = (long)m * r;
    gk_prep(a);
    GemmArgs bg = base;
    bg.M = 2 * s.n; bg.N = s.r;
    bg.A = b.dgu; bg.lda = 2 * s.n;
    bg.B = f.Tgu; bg.ldb = s.r;
    bg.C = dB_g; bg.ldc = 2 * s.n; bg.cstride = (long)r * 2 * n; bg.ctrans = 1;
    gk_prep(bg);
  } else {
    GemmArgs a = base;
    a.M = s.m; a.N = 2 * s.r;
    a.A = X; a.lda = s.m; a.arow = gr.arow; a.arow_div = gr.arow_div;
    a.B = b.Ugu; a.ldb = 2 * s.r;
    a.C = dA_g; a.C1 = dA_u; a.nsplit = s.r; a.ldc = s.r; a.cstride = (long)m * r;
    gk_prep(a);
    GemmArgs bg = base;
    bg.M = s.n; bg.N = s.r;
    bg.A = b.dgu; bg.lda = 2 * s.n;
    bg.B = f.Tgu; bg.ldb = 2 * s.r;
    bg.C = dB_g; bg.ldc = s.n; bg.cstride = (long)r * n; bg.ctrans = 1;
    gk_prep(bg);
    bg.A = (const char*)b.dgu + n * es;  // dB_u: the up half of dgu against the up half of Tc_gu
    bg.B = (const char*)f.Tgu + r * es;
    bg.C = dB_u;
    gk_prep(bg);
  }
  STAGE(ST_BWD_GRADS, gemm_gk_launch(gk_jobs, n_gk, s.dtype, ref, Pi, hs));
  if (chunked) STAGE(ST_BWD_GRADS, gemm_gk_reduce(gk_jobs, n_gk, Pi, hs));
  return MOE_OK;
}


moe_status moe_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  return MOE_OK;
}

int32_t moe_timing_stage_count(void) { return ST_COUNT; }

const char* moe_timing_stage_name(int32_t stage) {
  return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : nullptr;
}

moe_status moe_timing_read(double* total_ms, int64_t* counts, int32_t nstages) {
  if (!total_ms || !counts || nstages < ST_COUNT) return MOE_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  moe_status st = MOE_OK;
  for (auto& p : g_timing.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.e) != hipSuccess || hipEventElapsedTime(&ms, p.b, p.e) != hipSuccess) {
      st = MOE_ERR_HIP;
    } else {
      g_timing.total_ms[p.stage] += ms;
      g_timing.count[p.stage] += 1;
    }
    g_timing.pool.push_back(p.b);
    g_timing.pool.push_back(p.e);
  }
  g_timing.pending.clear();
  for (int i = 0; i < ST_COUNT; i++) {
    total_ms[i] = g_timing.total_ms[i];
    counts[i] = g_timing.count[i];
    g_timing.total_ms[i] = 0.0;
    g_timing.count[i] = 0;
  }
  return st;
}


// ---------------------------------------------------------------- shared expert
// A dense SwiGLU expert with its own Split-LoRA pairs, applied to every token and added to the
// routed layer's output. Internally one group of s rows (E = 1, k = 1, no gather, no combine).

static moe_status shared_shape(const moe_shape* sp, moe_shape* out) {
  if (!sp) return MOE_ERR_INVALID_ARG;
  moe_shape c = *sp;
  // E, k and the router fields do not apply; check the rest under a valid routed stand-in
  c.E = 8;
  c.k = 1;
  c.score = MOE_SCORE_SOFTMAX;
  c.renormalize = 1;
  c.router_grad = 0;
  const moe_status st = check_shape(&c);
  if (st != MOE_OK) return st;
  if (merged(c)) return MOE_ERR_UNSUPPORTED;
  c.E = 1;
  *out = c;
  return MOE_OK;
}

// off [2], the tile tables [kNumTileSizes][2] and the row tile -> group maps of the single group
static size_t one_group_layout(const moe_shape& sh, void* base, Grouping* gr) {
  Carve c(base);
  int* off = c.take<int>(2);
  int* tiles = c.take<int>((size_t)kNumTileSizes * 2);
  int* tmaps = c.take<int>((size_t)tile_map_offset(kNumTileSizes, sh.s, 1));
  if (gr) *gr = Grouping{1, off, nullptr, 1, tiles, tmaps};
  return align_up(c.off, 256);
}

size_t moe_shared_saved_bytes(const moe_shape* shape) {
  moe_shape sh;
  if (shared_shape(shape, &sh) != MOE_OK) return 0;
  return fwd_layout(sh, nullptr, nullptr, false);
}

size_t moe_shared_fwd_ws_bytes(const moe_shape* shape, int32_t with_saved) {
  moe_shape sh;
  if (shared_shape(shape, &sh) != MOE_OK) return 0;
  return one_group_layout(sh, nullptr, nullptr) + fwd_factor_layout(sh, nullptr, nullptr) +
         (with_saved ? 0 : fwd_layout(sh, nullptr, nullptr, false));
}

size_t moe_shared_bwd_ws_bytes(const moe_shape* shape) {
  moe_shape sh;
  if (shared_shape(shape, &sh) != MOE_OK) return 0;
  return one_group_layout(sh, nullptr, nullptr) + bwd_layout(sh, nullptr, nullptr, false) +
         recompute_bytes(sh, false);
}

moe_status moe_shared_forward(const moe_shape* shape, const void* X, const void* W_gu, const void* W_d,
                              const void* A_g, const void* B_g, const void* A_u, const void* B_u,
                              const void* A_d, const void* B_d, void* Y, void* saved, size_t saved_bytes,
                              void* ws, size_t ws_bytes, void* stream) {
  moe_shape s;
  moe_status st = shared_shape(shape, &s);
  if (st != MOE_OK) return st;
  const size_t m = s.m, n = s.n;
  if (!ptr_ok(X, (size_t)s.s * m) || !ptr_ok(W_gu, m * 2 * n) || !ptr_ok(W_d, n * m) ||
      !lora_ptrs_ok(s, A_g, B_g, A_u, B_u, A_d, B_d) || !ptr_ok(Y, (size_t)s.s * m))
    return MOE_ERR_INVALID_ARG;
  const size_t need_tab = one_group_layout(s, nullptr, nullptr);
  const size_t need_saved = fwd_layout(s, nullptr, nullptr, false);
  const size_t need_fac = fwd_factor_layout(s, nullptr, nullptr);
  const size_t need_ws = need_tab + need_fac + (saved ? 0 : need_saved);
  if (saved) {
    if ((uintptr_t)saved & 255u) return MOE_ERR_INVALID_ARG;
    if (saved_bytes < need_saved) return MOE_ERR_WORKSPACE;
  }
  if (ws_bytes < need_ws) return MOE_ERR_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255u)) return MOE_ERR_INVALID_ARG;
  if (s.s == 0) return MOE_OK;
  hipStream_t hs = (hipStream_t)stream;
  Grouping gr;
  one_group_layout(s, ws, &gr);
  HIP_TRY(launch_one_group_tables(s.s, const_cast<int*>(gr.off), const_cast<int*>(gr.tiles),
                                  const_cast<int*>(gr.tmaps), hs));
  FwdFactors ff;
  fwd_factor_layout(s, (char*)ws + need_tab, &ff);
  FwdBufs f;
  fwd_layout(s, saved ? saved : (char*)ws + need_tab + need_fac, &f, false);
  return forward_experts(s, X, gr, W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, f, ff, Y, 1, hs);
}

moe_status moe_shared_backward(const moe_shape* shape, const void* dY, const void* X, const void* W_gu,
                               const void* W_d, const void* A_g, const void* B_g, const void* A_u,
                               const void* B_u, const void* A_d, const void* B_d, const void* saved,
                               size_t saved_bytes, void* dX, float* dA_g, float* dB_g, float* dA_u,
                               float* dB_u, float* dA_d, float* dB_d, void* ws, size_t ws_bytes,
                               void* stream) {
  moe_shape s;
  moe_status st = shared_shape(shape, &s);
  if (st != MOE_OK) return st;
  const size_t m = s.m, n = s.n, r = s.r;
  const bool fz = fused_gu(s);
  if (!ptr_ok(dY, (size_t)s.s * m) || !ptr_ok(X, (size_t)s.s * m) || !ptr_ok(W_gu, m * 2 * n) ||
      !ptr_ok(W_d, n * m) || !lora_ptrs_ok(s, A_g, B_g, A_u, B_u, A_d, B_d) ||
      !ptr_ok(dX, (size_t)s.s * m) || !ptr_ok(dA_g, m * r) || !ptr_ok(dB_g, r * n * (fz ? 2 : 1)) ||
      (!fz && (!ptr_ok(dA_u, m * r) || !ptr_ok(dB_u, r * n))) || !ptr_ok(dA_d, n * r) ||
      !ptr_ok(dB_d, r * m))
    return MOE_ERR_INVALID_ARG;
  const bool redo = !saved;
  if (redo && !recompute(s)) return MOE_ERR_INVALID_ARG;
  if (saved && ((uintptr_t)saved & 255u)) return MOE_ERR_INVALID_ARG;
  if (saved && saved_bytes < fwd_layout(s, nullptr, nullptr, false)) return MOE_ERR_WORKSPACE;
  const size_t need_tab = one_group_layout(s, nullptr, nullptr);
  const size_t bwd_bytes = bwd_layout(s, nullptr, nullptr, false);
  const size_t need_ws = need_tab + bwd_bytes + (redo ? recompute_bytes(s, false) : 0);
  if (ws_bytes < need_ws) return MOE_ERR_WORKSPACE;
  if (!ws || ((uintptr_t)ws & 255u)) return MOE_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  if (s.s == 0) {  // no rows: zero gradients, dX unchanged
    HIP_TRY(launch_zero(dA_g, m * r, hs));
    HIP_TRY(launch_zero(dB_g, r * n * (fz ? 2 : 1), hs));
    if (!fz) {
      HIP_TRY(launch_zero(dA_u, m * r, hs));
      HIP_TRY(launch_zero(dB_u, r * n, hs));
    }
    HIP_TRY(launch_zero(dA_d, n * r, hs));
    HIP_TRY(launch_zero(dB_d, r * m, hs));
    return MOE_OK;
  }
  Grouping gr;
  one_group_layout(s, ws, &gr);
  HIP_TRY(launch_one_group_tables(s.s, const_cast<int*>(gr.off), const_cast<int*>(gr.tiles),
                                  const_cast<int*>(gr.tmaps), hs));
  BwdBufs b;
  bwd_layout(s, (char*)ws + need_tab, &b, false);
  FwdBufs f;
  if (redo) {
    char* rbase = (char*)ws + need_tab + bwd_bytes;
    FwdFactors ff;
    fwd_layout(s, rbase, &f, false);
    fwd_factor_layout(s, rbase + fwd_layout(s, nullptr, nullptr, false), &ff);
    // the recomputed down projection output is not needed: it goes to the scratch gradient rows
    HIP_TRY_STATUS(forward_experts(s, X, gr, W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, f, ff, nullptr, 0, hs));
  } else {
    fwd_layout(s, const_cast<void*>(saved), &f, false);
  }
  // dO = dY (weight 1, no permutation); dX += the expert's input gradient
  return backward_experts(s, gr, X, dY, nullptr, W_gu, W_d, A_g, B_g, A_u, B_u, A_d, B_d, f, b, dX, 1, dA_g,
                          dB_g, dA_u, dB_u, dA_d, dB_d, hs);
}

}  // extern "C"
