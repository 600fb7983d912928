// libmoe C ABI: argument validation, sizing and kernel launches.
// The contract of every entry point is documented in include/moe.h.
#include <math.h>
#include <string.h>

#include "../../include/moe.h"
#include "common.h"
#include "gemm.h"
#include "gemm_common.h"
#include "kernels.h"

#include <initializer_list>
#include <mutex>
#include <type_traits>

// Scratch of moe_dispatch_noalloc: the dispatch kernels' per-block expert
// counts, per-block bases (inputs of more than 128 blocks) and the experts'
// first rows, for at most 2^20 tokens and 64 experts (2 MiB + 512 bytes).
// Every GPU the library runs on holds its own copy until the process ends.
// Host code never passes `scratch` itself to a kernel (in host code the name
// is only a stand-in): it uses the device address hipGetSymbolAddress returns
// for the current device (scratch_base below).
constexpr int64_t kNoAllocMaxTokens = (int64_t)1 << 20;
constexpr size_t kNoAllocCntBytes = (size_t)(kNoAllocMaxTokens / moe::kDispatchBlock) * 64 * 4;
constexpr size_t kNoAllocBytes = 2 * kNoAllocCntBytes + 64 * 8;
static __device__ __align__(256) char scratch[kNoAllocBytes];

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = (int)e;
  return MOE_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID;
  if (c->T <= 0 || c->d <= 0 || c->ffn <= 0 || c->E <= 0 || c->k <= 0) return MOE_ERR_INVALID;
  if (c->k > c->E) return MOE_ERR_INVALID;
  if (c->gating < MOE_GATE_SOFTMAX_TOPK || c->gating > MOE_GATE_TOPK_SOFTMAX) return MOE_ERR_INVALID;
  if (c->act != MOE_ACT_GELU && c->act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (c->ep_ranks < 1 || c->E % c->ep_ranks != 0) return MOE_ERR_INVALID;
  if (c->placement != MOE_PLACE_CONTIGUOUS && c->placement != MOE_PLACE_ROUND_ROBIN) return MOE_ERR_INVALID;
  if (c->n_shared < 0 || (c->n_shared > 0 && c->ffn_shared <= 0)) return MOE_ERR_INVALID;
  if (!(c->capacity_factor == c->capacity_factor)) return MOE_ERR_INVALID;  // NaN
  if (c->E > 64 || c->k > 8) return MOE_ERR_UNSUPPORTED;
  if (c->d % 8 != 0 || c->ffn % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 0 && (c->n_shared * c->ffn_shared) % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (c->T * c->k >= (int64_t)1 << 31 || c->T >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (c->d >= (int64_t)1 << 24 || c->ffn >= (int64_t)1 << 24) return MOE_ERR_UNSUPPORTED;
  // every buffer resource of the expert GEMMs spans at most 256 rows of one
  // operand, so one row (x: d elements; the saved SwiGLU factors: 2 ffn; the shared experts:
  // 2 n_shared ffn_shared) must stay within kMaxRowBytes for its extent to fit
  const int64_t s = c->dtype == MOE_BF16 ? 2 : 4;
  const int64_t m = c->act == MOE_ACT_SWIGLU ? 2 : 1;
  const int64_t lim = moe::gemm_common::kMaxRowBytes;
  if (c->d * s > lim || m * c->ffn * s > lim) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 0 && (c->n_shared >= (int64_t)1 << 24 || c->ffn_shared >= (int64_t)1 << 24 ||
                          m * c->n_shared * c->ffn_shared * s > lim))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t capacity_of(const moe_config* c) {
  const double cf = (double)c->capacity_factor;
  if (cf <= 0.0) return c->T;
  const double v = ceil(cf * (double)c->k * (double)c->T / (double)c->E);
  return v >= (double)c->T ? c->T : (int64_t)v;
}

int64_t plan_n_max(const moe_config* c) {
  const int64_t tk = c->T * c->k, ec = c->E * capacity_of(c);
  return tk < ec ? tk : ec;
}

size_t elem_bytes(const moe_config* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

struct WsLayout {
  size_t dispatch, route, route_bwd, aux, ffn_routed, ffn_shared, total;
};

// Workspace of one moe_expert_ffn_bwd call over `groups` groups of hidden
// width F and at most rows_max rows: d_act [rows, m F] in the dtype, then
// (bf16) the fp32 partials of the split weight-gradient launches.
size_t ffn_d_act_bytes(const moe_config* c, int64_t F, int64_t rows_max) {
  const int64_t m = c->act == MOE_ACT_SWIGLU ? 2 : 1;
  return round_up((size_t)rows_max * m * F * elem_bytes(c), 256);
}
size_t ffn_split_bytes(const moe_config* c, int64_t groups, int64_t F, int64_t rows_max) {
  if (c->dtype != MOE_BF16) return 0;
  const int64_t m = c->act == MOE_ACT_SWIGLU ? 2 : 1;
  const int64_t s3 = moe::gemm3::wgrad_ksplit(groups, F, c->d, rows_max);
  const int64_t s4 = moe::gemm3::wgrad_ksplit(groups, c->d, m * F, rows_max);
  const size_t b3 = s3 > 1 ? (size_t)s3 * groups * F * c->d * 4 : 0;
  const size_t b4 = s4 > 1 ? (size_t)s4 * groups * c->d * m * F * 4 : 0;
  return round_up(b3 > b4 ? b3 : b4, 256);
}
// bf16 backward on weights transposed once per call: both dgrads become
// forward-kind launches, which read the weights as whole rows (a K-contiguous
// weight panel costs two 64-byte requests per 128-byte line and a 32-K
// stage).  The transposes move 2 (1 + m) E' d F elements; the dgrads' saving
// grows with the rows per weight set.  On the Mixtral shape (4096 rows per
// expert, SwiGLU) the forward-kind dgrads take 1.8 ms less and the whole
// backward 0.45 ms less net of the transposes, while with ~1500 rows
// (DeepSeek-V2-Lite's routed experts) or GELU at 2048 the transposes cost
// more than they save.  Used when rows_max / groups * m / (1 + m) >= 2000
// and the plan's workspace holds the copy.
bool ffn_bwd_transposed(const moe_config* c, int64_t groups, int64_t rows_max) {
  if (c->dtype != MOE_BF16 || groups <= 0) return false;
  const int64_t m = c->act == MOE_ACT_SWIGLU ? 2 : 1;
  return rows_max * m >= 2000 * groups * (1 + m);
}
// the transposed weights: W_out^T [E'][d][F], then per weight set
// [W_in^T | W_up^T] [E'][m F][d]
size_t ffn_wt_bytes(const moe_config* c, int64_t groups, int64_t F) {
  const int64_t m = c->act == MOE_ACT_SWIGLU ? 2 : 1;
  return round_up((size_t)groups * (1 + m) * c->d * F * elem_bytes(c), 256);
}
// what a moe_expert_ffn_bwd call needs (dL/d act and split partials), and
// what the plan reserves for it (plus the transposed weights where they pay)
size_t ffn_bwd_ws(const moe_config* c, int64_t groups, int64_t F, int64_t rows_max) {
  return ffn_d_act_bytes(c, F, rows_max) + ffn_split_bytes(c, groups, F, rows_max);
}
size_t ffn_bwd_ws_planned(const moe_config* c, int64_t groups, int64_t F, int64_t rows_max) {
  return ffn_bwd_ws(c, groups, F, rows_max) +
         (ffn_bwd_transposed(c, groups, rows_max) ? ffn_wt_bytes(c, groups, F) : 0);
}

WsLayout ws_layout(const moe_config* c, int64_t n_max) {
  WsLayout w;
  const int64_t nb = (c->T + moe::kDispatchBlock - 1) / moe::kDispatchBlock;
  w.dispatch = round_up((size_t)nb * c->E * 4, 256) * 2 + round_up((size_t)c->E * 8, 256);
  w.route_bwd = round_up((size_t)moe::router_wgrad_blocks(c->T) * c->d * c->E * 4, 256);
  w.ffn_routed = ffn_bwd_ws_planned(c, c->E, c->ffn, n_max);
  w.ffn_shared = c->n_shared > 0 ? ffn_bwd_ws_planned(c, 1, c->n_shared * c->ffn_shared, c->T) : 0;
  w.route = c->dtype == MOE_BF16 ? round_up(moe::route_ws_bytes(c->d, c->E), 256) : 0;
  w.aux = round_up(moe::aux_ws_bytes(c->E), 256);
  w.total = w.dispatch;
  if (w.route > w.total) w.total = w.route;
  if (w.route_bwd > w.total) w.total = w.route_bwd;
  if (w.aux > w.total) w.total = w.aux;
  if (w.ffn_routed > w.total) w.total = w.ffn_routed;
  if (w.ffn_shared > w.total) w.total = w.ffn_shared;
  return w;
}

int check_groups(const moe_config* c, const moe_groups* g) {
  if (!g || !g->offsets) return MOE_ERR_INVALID;
  if (g->groups < 1 || g->ffn <= 0 || g->rows_max < 0) return MOE_ERR_INVALID;
  if (g->use_placement && g->groups != c->E) return MOE_ERR_INVALID;
  if (g->groups > 65) return MOE_ERR_UNSUPPORTED;
  if (g->ffn % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (g->rows_max >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  const int64_t m = c->act == MOE_ACT_SWIGLU ? 2 : 1;
  if (g->ffn >= (int64_t)1 << 24 || m * g->ffn * (int64_t)elem_bytes(c) > moe::gemm_common::kMaxRowBytes)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

void fill_placement(const moe_config* c, const moe_groups* g, moe::gemm::Args& a) {
  a.groups = (int)g->groups;
  a.offsets = g->offsets;
  a.ends = g->ends;
  if (g->use_placement && c->placement == MOE_PLACE_ROUND_ROBIN && c->ep_ranks > 1) {
    a.rr_R = c->ep_ranks;
    a.rr_L = (int)(c->E / c->ep_ranks);
  } else {
    a.rr_R = 0;
    a.rr_L = 1;
  }
}

template <typename T>
hipError_t ffn_fwd(const moe_config* c, const moe_groups* g, const void* x, const void* w_in, const void* w_up,
                   const void* w_out, void* act_saved, void* h, void* y, hipStream_t st) {
  using namespace moe::gemm;
  const int64_t d = c->d, F = g->ffn;
  const bool swiglu = c->act == MOE_ACT_SWIGLU;
  Args a1;
  fill_placement(c, g, a1);
  a1.A = x; a1.lda = d;
  a1.B = w_in; a1.B2 = swiglu ? w_up : nullptr; a1.ldb = F; a1.b_gstride = d * F;
  a1.N = F; a1.K = d;
  a1.C = act_saved; a1.C2 = h; a1.ldc2 = F;
  if (swiglu) { a1.ldc = 2 * F; a1.c_split = F; } else { a1.ldc = F; }
  hipError_t e = run_rows<T>(KIND_FWD, swiglu ? EPI_SWIGLU_FWD : EPI_GELU_FWD, a1, g->rows_max, st);
  if (e != hipSuccess) return e;
  Args a2;
  fill_placement(c, g, a2);
  a2.A = h; a2.lda = F;
  a2.B = w_out; a2.ldb = d; a2.b_gstride = F * d;
  a2.N = d; a2.K = F;
  a2.C = y; a2.ldc = d;
  return run_rows<T>(KIND_FWD, EPI_STORE, a2, g->rows_max, st);
}

// Data gradients: dL/d act into ws (rows as in the row buffers), then dx.
// The fused forward (bf16): GEMM-1 reads its rows from the token rows
// through assign_of_row, writes only h; GEMM-2 writes row r to row
// assign_of_row[r] of y_tok scaled by topk_w there.
hipError_t ffn_fwd_fused(const moe_config* c, const moe_groups* g, const void* x, const int32_t* assign_of_row,
                         const float* topk_w, const void* w_in, const void* w_up, const void* w_out, void* h,
                         void* y_tok, hipStream_t st) {
  using namespace moe::gemm;
  const int64_t d = c->d, F = g->ffn;
  const bool swiglu = c->act == MOE_ACT_SWIGLU;
  Args a1;
  fill_placement(c, g, a1);
  a1.A = x; a1.lda = d;
  a1.gather = assign_of_row; a1.gather_k = (int)c->k; a1.gather_rows = c->T;
  a1.B = w_in; a1.B2 = swiglu ? w_up : nullptr; a1.ldb = F; a1.b_gstride = d * F;
  a1.N = F; a1.K = d;
  a1.C2 = h; a1.ldc2 = F;
  hipError_t e = run_rows<moe::bf16>(KIND_FWD, swiglu ? EPI_SWIGLU_FWD_H : EPI_GELU_FWD_H, a1, g->rows_max, st);
  if (e != hipSuccess) return e;
  Args a2;
  fill_placement(c, g, a2);
  a2.A = h; a2.lda = F;
  a2.B = w_out; a2.ldb = d; a2.b_gstride = F * d;
  a2.N = d; a2.K = F;
  a2.C = y_tok; a2.ldc = d;
  a2.scatter = assign_of_row; a2.row_scale = topk_w;
  return run_rows<moe::bf16>(KIND_FWD, EPI_STORE_SCATTER, a2, g->rows_max, st);
}

// wt: NULL, or the transposed weights (ffn_wt_bytes layout), which turn both
// dgrads into forward-kind launches over the same products.
template <typename T>
hipError_t ffn_bwd_data(const moe_config* c, const moe_groups* g, const void* w_in, const void* w_up,
                        const void* w_out, const void* act_saved, const void* dy, void* dx, void* ws, hipStream_t st,
                        const void* wt = nullptr) {
  using namespace moe::gemm;
  const int64_t d = c->d, F = g->ffn;
  const bool swiglu = c->act == MOE_ACT_SWIGLU;
  const int64_t m = swiglu ? 2 : 1;
  // 1. dgrad through W_out and the activation backward: d_act in ws.  GELU'
  //    and SwiGLU' are fused into the GEMM's epilogue.
  Args a1;
  fill_placement(c, g, a1);
  a1.A = dy; a1.lda = d;
  if (wt) {  // W_out^T [d][F]: N-contiguous
    a1.B = wt; a1.ldb = F; a1.b_gstride = d * F;
  } else {
    a1.B = w_out; a1.ldb = d; a1.b_gstride = F * d;
  }
  a1.N = F; a1.K = d;
  a1.X1 = act_saved; a1.ldx = m * F;
  a1.C = ws; a1.ldc = m * F; a1.c_split = F;
  const int epi1 = swiglu ? EPI_SWIGLU_BWD : EPI_GELU_BWD;
  hipError_t e = run_rows<T>(wt ? KIND_FWD : KIND_DGRAD, epi1, a1, g->rows_max, st);
  if (e != hipSuccess) return e;
  // 2. dgrad through W_in (and W_up): dx = d_act . [W_in | W_up]^T
  Args a2;
  fill_placement(c, g, a2);
  a2.A = ws; a2.lda = m * F;
  if (wt) {  // [W_in^T | W_up^T] [m F][d] per weight set: N-contiguous, one K range
    a2.B = (const char*)wt + (size_t)g->groups * d * F * sizeof(T); a2.ldb = d; a2.b_gstride = m * F * d;
  } else {
    a2.B = w_in; a2.B2 = swiglu ? w_up : nullptr; a2.ldb = F; a2.b_gstride = d * F;
    a2.b_split = swiglu ? F : 0;
  }
  a2.N = d; a2.K = m * F;
  a2.C = dx; a2.ldc = d;
  return run_rows<T>(wt ? KIND_FWD : KIND_DGRAD, EPI_STORE, a2, g->rows_max, st);
}

// Weight gradients over whole groups, from dL/d act in ws.
template <typename T>
hipError_t ffn_bwd_weights(const moe_config* c, const moe_groups* g, const void* x, const void* h, const void* dy,
                           void* dw_in, void* dw_up, void* dw_out, void* ws, hipStream_t st) {
  using namespace moe::gemm;
  const int64_t d = c->d, F = g->ffn;
  const bool swiglu = c->act == MOE_ACT_SWIGLU;
  const int64_t m = swiglu ? 2 : 1;
  hipError_t e;
  // Launches with few tiles split their reduction (bf16), with fp32 partials
  // placed after d_act in ws, as long as the workspace moe_plan sized holds
  // them (it does for the routed call over all experts and the shared call).
  const bool split_ok = std::is_same<T, moe::bf16>::value &&
                        ffn_bwd_ws(c, g->groups, F, g->rows_max) <= ws_layout(c, plan_n_max(c)).total;
  float* partial = (float*)((char*)ws + ffn_d_act_bytes(c, F, g->rows_max));
  // 3. dW_out = h^T dy
  Args a3;
  fill_placement(c, g, a3);
  a3.A = h; a3.lda = F; a3.M = F;
  a3.B = dy; a3.ldb = d; a3.N = d;
  a3.C = dw_out; a3.ldc = d; a3.c_gstride = F * d;
  if (split_ok) {
    a3.ksplit = moe::gemm3::wgrad_ksplit(g->groups, F, d, g->rows_max);
    a3.partial = partial;
  }
  e = run_wgrad<T>(EPI_STORE, a3, st);
  if (e != hipSuccess) return e;
  // 4. dW_in (| dW_up) = x^T d_act
  Args a4;
  fill_placement(c, g, a4);
  a4.A = x; a4.lda = d; a4.M = d;
  a4.B = ws; a4.ldb = m * F; a4.N = m * F;
  a4.C = dw_in; a4.C2 = swiglu ? dw_up : nullptr; a4.ldc = F; a4.c_gstride = d * F;
  a4.c_split = F;
  if (split_ok) {
    a4.ksplit = moe::gemm3::wgrad_ksplit(g->groups, d, m * F, g->rows_max);
    a4.partial = partial;
  }
  return run_wgrad<T>(swiglu ? EPI_STORE_SPLITN : EPI_STORE, a4, st);
}

template <typename T>
hipError_t ffn_bwd(const moe_config* c, const moe_groups* g, const void* x, const void* w_in, const void* w_up,
                   const void* w_out, const void* act_saved, const void* h, const void* dy, void* dx, void* dw_in,
                   void* dw_up, void* dw_out, void* ws, hipStream_t st) {
  const void* wt = nullptr;
  if (sizeof(T) == 2 && ffn_bwd_transposed(c, g->groups, g->rows_max) &&
      ffn_bwd_ws_planned(c, g->groups, g->ffn, g->rows_max) <= ws_layout(c, plan_n_max(c)).total) {
    // after dL/d act and the split partials: W_out^T, then [W_in^T | W_up^T]
    char* w = (char*)ws + ffn_d_act_bytes(c, g->ffn, g->rows_max) +
              ffn_split_bytes(c, g->groups, g->ffn, g->rows_max);
    const int64_t d = c->d, F = g->ffn, E = g->groups, m = c->act == MOE_ACT_SWIGLU ? 2 : 1;
    char* wio = w + (size_t)E * d * F * 2;
    hipError_t e = moe::gemm3::transpose_bf16(w_out, w, E, F, d, F * d, d * F, st);  // [F][d] -> [d][F]
    if (e == hipSuccess) e = moe::gemm3::transpose_bf16(w_in, wio, E, d, F, d * F, m * F * d, st);  // -> [F][d]
    if (e == hipSuccess && m == 2)
      e = moe::gemm3::transpose_bf16(w_up, wio + (size_t)F * d * 2, E, d, F, d * F, m * F * d, st);
    if (e != hipSuccess) return e;
    wt = w;
  }
  hipError_t e = ffn_bwd_data<T>(c, g, w_in, w_up, w_out, act_saved, dy, dx, ws, st, wt);
  if (e != hipSuccess) return e;
  return ffn_bwd_weights<T>(c, g, x, h, dy, dw_in, dw_up, dw_out, ws, st);
}

// Pointer checks shared by the FFN backward entry points: every pointer of
// `req` present and 16-byte aligned, ws 256-byte aligned and large enough
// for the group table's dL/d act and split partials.
int check_ffn_bwd_ptrs(const moe_config* cfg, const moe_groups* grp, std::initializer_list<const void*> req,
                       void* ws) {
  for (const void* p : req)
    if (!p) return MOE_ERR_INVALID;
  for (const void* p : req)
    if (!aligned16(p)) return MOE_ERR_INVALID;
  if (!ws || ((uintptr_t)ws & 255u)) return MOE_ERR_INVALID;
  // the group table's workspace (dL/d act, then split partials) must fit in
  // moe_plan's workspace_bytes: the routed and shared tables always do
  if (ffn_bwd_ws(cfg, grp->groups, grp->ffn, grp->rows_max) > ws_layout(cfg, plan_n_max(cfg)).total)
    return MOE_ERR_INVALID;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_plan(const moe_config* cfg, moe_sizes* out) {
  const int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!out) return MOE_ERR_INVALID;
  out->C = capacity_of(cfg);
  const int64_t tk = cfg->T * cfg->k, ec = cfg->E * out->C;
  out->n_max = tk < ec ? tk : ec;
  out->workspace_bytes = ws_layout(cfg, out->n_max).total;
  return MOE_OK;
}

int moe_route(const moe_config* cfg, const void* x, const void* w_router, const float* bias, float* logits,
              int32_t* topk_idx, float* topk_w, void* ws, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!x || !w_router || !logits || !topk_idx || !topk_w) return MOE_ERR_INVALID;
  if (cfg->dtype == MOE_BF16 && !ws) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(ws)) return MOE_ERR_INVALID;
  moe::RouteArgs a{x, w_router, (uint32_t*)ws, bias, logits, topk_idx, topk_w, cfg->T, (int)cfg->d, (int)cfg->E,
                   (int)cfg->k, cfg->gating};
  return hip_status(moe::launch_route(a, cfg->dtype == MOE_BF16, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Per-device address of `scratch`, looked up once per device (with that
// device current) on the first moe_dispatch_noalloc call there.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_base(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = (char*)g_scratch_ptr[dev];
  return MOE_OK;
}

// moe_dispatch with its scratch at `w`: block counts [nb, E] int32 at w, block
// bases [nb, E] at w + cnt_bytes, expert starts [E] int64 at w + 2 cnt_bytes.
int dispatch_into(const moe_config* cfg, const void* x, const int32_t* topk_idx, void* x_perm, int32_t* row_of,
                  int32_t* assign_of_row, int32_t* raw_counts, int32_t* expert_counts, int64_t* expert_offsets,
                  int32_t* send_counts, int64_t* send_offsets, char* w, size_t cnt_bytes, void* stream) {
  moe::DispatchArgs a;
  a.x = x; a.topk_idx = topk_idx; a.x_perm = x_perm; a.row_of = row_of; a.assign_of_row = assign_of_row;
  a.raw_counts = raw_counts; a.expert_counts = expert_counts; a.expert_offsets = expert_offsets;
  a.send_counts = send_counts; a.send_offsets = send_offsets;
  a.block_counts = (int32_t*)w;
  a.block_base = (int32_t*)(w + cnt_bytes);
  a.expert_start = (int64_t*)(w + 2 * cnt_bytes);
  a.T = cfg->T; a.d = cfg->d; a.E = (int)cfg->E; a.k = (int)cfg->k; a.C = capacity_of(cfg);
  a.R = cfg->ep_ranks; a.placement = cfg->placement;
  return hip_status(moe::launch_dispatch(a, cfg->dtype == MOE_BF16, (hipStream_t)stream));
}

int check_dispatch_args(const moe_config* cfg, const void* x, const int32_t* topk_idx, void* x_perm,
                        int32_t* row_of, int32_t* assign_of_row, int32_t* raw_counts, int32_t* expert_counts,
                        int64_t* expert_offsets, int32_t* send_counts, int64_t* send_offsets) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!topk_idx || !row_of || !assign_of_row || !raw_counts || !expert_counts || !expert_offsets || !send_counts ||
      !send_offsets)
    return MOE_ERR_INVALID;
  // x_perm NULL: layout only (x unused); else x is copied into it
  if (x_perm && (!x || !aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_dispatch(const moe_config* cfg, const void* x, const int32_t* topk_idx, void* x_perm, int32_t* row_of,
                 int32_t* assign_of_row, int32_t* raw_counts, int32_t* expert_counts, int64_t* expert_offsets,
                 int32_t* send_counts, int64_t* send_offsets, void* ws, void* stream) {
  int s = check_dispatch_args(cfg, x, topk_idx, x_perm, row_of, assign_of_row, raw_counts, expert_counts,
                              expert_offsets, send_counts, send_offsets);
  if (s != MOE_OK) return s;
  if (!ws || ((uintptr_t)ws & 255u)) return MOE_ERR_INVALID;
  const int64_t nb = (cfg->T + moe::kDispatchBlock - 1) / moe::kDispatchBlock;
  return dispatch_into(cfg, x, topk_idx, x_perm, row_of, assign_of_row, raw_counts, expert_counts, expert_offsets,
                       send_counts, send_offsets, (char*)ws, round_up((size_t)nb * cfg->E * 4, 256), stream);
}

int moe_dispatch_noalloc(const moe_config* cfg, const void* x, const int32_t* topk_idx, void* x_perm,
                         int32_t* row_of, int32_t* assign_of_row, int32_t* raw_counts, int32_t* expert_counts,
                         int64_t* expert_offsets, int32_t* send_counts, int64_t* send_offsets, void* stream) {
  int s = check_dispatch_args(cfg, x, topk_idx, x_perm, row_of, assign_of_row, raw_counts, expert_counts,
                              expert_offsets, send_counts, send_offsets);
  if (s != MOE_OK) return s;
  if (cfg->T > kNoAllocMaxTokens) return MOE_ERR_UNSUPPORTED;
  char* w = nullptr;
  s = scratch_base(&w);
  if (s != MOE_OK) return s;
  // every scratch word a call reads it first writes itself (block counts for
  // every block and expert, then the bases and starts), so nothing is cleared
  return dispatch_into(cfg, x, topk_idx, x_perm, row_of, assign_of_row, raw_counts, expert_counts, expert_offsets,
                       send_counts, send_offsets, w, kNoAllocCntBytes, stream);
}

int moe_permute(const moe_config* cfg, const void* x, const int32_t* row_of, void* x_perm, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!x || !row_of || !x_perm) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID;
  moe::DispatchArgs a{};
  a.x = x; a.row_of = const_cast<int32_t*>(row_of); a.x_perm = x_perm;  // read only by the copy
  a.T = cfg->T; a.d = cfg->d; a.E = (int)cfg->E; a.k = (int)cfg->k;
  return hip_status(moe::launch_permute(a, cfg->dtype == MOE_BF16, (hipStream_t)stream));
}

int moe_chunk_rows(const moe_config* cfg, const int32_t* topk_idx, const int32_t* row_of,
                   const int64_t* expert_offsets, int64_t chunks, const int64_t* token_bounds, int64_t* chunk_rows,
                   void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!topk_idx || !row_of || !expert_offsets || !token_bounds || !chunk_rows) return MOE_ERR_INVALID;
  if (chunks < 1) return MOE_ERR_INVALID;
  if (chunks > moe::kMaxChunks) return MOE_ERR_UNSUPPORTED;
  moe::ChunkRowsArgs a{};
  if (token_bounds[0] != 0 || token_bounds[chunks] != cfg->T) return MOE_ERR_INVALID;
  for (int64_t r = 0; r <= chunks; ++r) {
    if (r > 0 && token_bounds[r] < token_bounds[r - 1]) return MOE_ERR_INVALID;
    a.cb.t[r] = token_bounds[r];
  }
  a.cb.chunks = (int)chunks;
  a.topk_idx = topk_idx; a.row_of = row_of; a.expert_offsets = expert_offsets; a.rows = chunk_rows;
  a.T = cfg->T; a.E = (int)cfg->E; a.k = (int)cfg->k; a.R = cfg->ep_ranks; a.placement = cfg->placement;
  return hip_status(moe::launch_chunk_rows(a, (hipStream_t)stream));
}

int moe_expert_ffn_fwd(const moe_config* cfg, const moe_groups* grp, const void* x_rows, const void* w_in,
                       const void* w_up, const void* w_out, void* act_saved, void* h, void* y_rows, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  s = check_groups(cfg, grp);
  if (s != MOE_OK) return s;
  const bool swiglu = cfg->act == MOE_ACT_SWIGLU;
  if (!x_rows || !w_in || !w_out || !act_saved || !h || !y_rows || (swiglu && !w_up)) return MOE_ERR_INVALID;
  if (!aligned16(x_rows) || !aligned16(w_in) || !aligned16(w_out) || !aligned16(act_saved) || !aligned16(h) ||
      !aligned16(y_rows) || (swiglu && !aligned16(w_up)))
    return MOE_ERR_INVALID;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = cfg->dtype == MOE_BF16 ? ffn_fwd<moe::bf16>(cfg, grp, x_rows, w_in, w_up, w_out, act_saved, h, y_rows, st)
                                        : ffn_fwd<float>(cfg, grp, x_rows, w_in, w_up, w_out, act_saved, h, y_rows, st);
  return hip_status(e);
}

int moe_expert_ffn_bwd(const moe_config* cfg, const moe_groups* grp, const void* x_rows, const void* w_in,
                       const void* w_up, const void* w_out, const void* act_saved, const void* h, const void* dy_rows,
                       void* dx_rows, void* dw_in, void* dw_up, void* dw_out, void* ws, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  s = check_groups(cfg, grp);
  if (s != MOE_OK) return s;
  if (grp->ends) return MOE_ERR_INVALID;  // weight gradients need whole groups
  const bool swiglu = cfg->act == MOE_ACT_SWIGLU;
  s = check_ffn_bwd_ptrs(cfg, grp,
                         {x_rows, w_in, w_out, act_saved, h, dy_rows, dx_rows, dw_in, dw_out, swiglu ? w_up : w_in,
                          swiglu ? dw_up : dw_in},
                         ws);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = cfg->dtype == MOE_BF16
                     ? ffn_bwd<moe::bf16>(cfg, grp, x_rows, w_in, w_up, w_out, act_saved, h, dy_rows, dx_rows, dw_in,
                                          dw_up, dw_out, ws, st)
                     : ffn_bwd<float>(cfg, grp, x_rows, w_in, w_up, w_out, act_saved, h, dy_rows, dx_rows, dw_in,
                                      dw_up, dw_out, ws, st);
  return hip_status(e);
}

int moe_expert_ffn_fwd_fused(const moe_config* cfg, const moe_groups* grp, const void* x, const int32_t* assign_of_row,
                             const float* topk_w, const void* w_in, const void* w_up, const void* w_out, void* h,
                             void* y_tok, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  s = check_groups(cfg, grp);
  if (s != MOE_OK) return s;
  const bool swiglu = cfg->act == MOE_ACT_SWIGLU;
  if (!x || !assign_of_row || !topk_w || !w_in || !w_out || !h || !y_tok || (swiglu && !w_up))
    return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(w_in) || !aligned16(w_out) || !aligned16(h) || !aligned16(y_tok) ||
      (swiglu && !aligned16(w_up)))
    return MOE_ERR_INVALID;
  if (grp->ends || grp->groups != cfg->E || !grp->use_placement) return MOE_ERR_INVALID;  // the routed table
  // bf16 direct-load kernels only; x is read through one buffer resource
  if (cfg->dtype != MOE_BF16 || cfg->T * cfg->d * 2 > moe::gemm_common::kMaxExtent) return MOE_ERR_UNSUPPORTED;
  return hip_status(ffn_fwd_fused(cfg, grp, x, assign_of_row, topk_w, w_in, w_up, w_out, h, y_tok,
                                  (hipStream_t)stream));
}

int moe_combine_fused(const moe_config* cfg, const void* y_tok, const int32_t* row_of, const void* y_shared, void* y,
                      void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!y_tok || !row_of || !y) return MOE_ERR_INVALID;
  if (!aligned16(y_tok) || !aligned16(y) || (y_shared && !aligned16(y_shared))) return MOE_ERR_INVALID;
  moe::CombineArgs a{};
  a.y_perm = y_tok; a.row_of = row_of; a.topk_w = nullptr; a.y_shared = y_shared; a.y = y;
  a.T = cfg->T; a.d = cfg->d; a.k = (int)cfg->k;
  return hip_status(moe::launch_combine(a, cfg->dtype == MOE_BF16, (hipStream_t)stream));
}

int moe_expert_ffn_bwd_data(const moe_config* cfg, const moe_groups* grp, const void* w_in, const void* w_up,
                            const void* w_out, const void* act_saved, const void* dy_rows, void* dx_rows, void* ws,
                            void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  s = check_groups(cfg, grp);
  if (s != MOE_OK) return s;
  const bool swiglu = cfg->act == MOE_ACT_SWIGLU;
  s = check_ffn_bwd_ptrs(cfg, grp, {w_in, w_out, act_saved, dy_rows, dx_rows, swiglu ? w_up : w_in}, ws);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = cfg->dtype == MOE_BF16
                     ? ffn_bwd_data<moe::bf16>(cfg, grp, w_in, w_up, w_out, act_saved, dy_rows, dx_rows, ws, st)
                     : ffn_bwd_data<float>(cfg, grp, w_in, w_up, w_out, act_saved, dy_rows, dx_rows, ws, st);
  return hip_status(e);
}

int moe_expert_ffn_bwd_weights(const moe_config* cfg, const moe_groups* grp, const void* x_rows, const void* h,
                               const void* dy_rows, void* dw_in, void* dw_up, void* dw_out, void* ws, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  s = check_groups(cfg, grp);
  if (s != MOE_OK) return s;
  if (grp->ends) return MOE_ERR_INVALID;  // weight gradients need whole groups
  const bool swiglu = cfg->act == MOE_ACT_SWIGLU;
  s = check_ffn_bwd_ptrs(cfg, grp, {x_rows, h, dy_rows, dw_in, dw_out, swiglu ? dw_up : dw_in}, ws);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = cfg->dtype == MOE_BF16
                     ? ffn_bwd_weights<moe::bf16>(cfg, grp, x_rows, h, dy_rows, dw_in, dw_up, dw_out, ws, st)
                     : ffn_bwd_weights<float>(cfg, grp, x_rows, h, dy_rows, dw_in, dw_up, dw_out, ws, st);
  return hip_status(e);
}

int moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* row_of, const float* topk_w,
                const void* y_shared, void* y, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!y_perm || !row_of || !topk_w || !y) return MOE_ERR_INVALID;
  if (!aligned16(y_perm) || !aligned16(y) || (y_shared && !aligned16(y_shared))) return MOE_ERR_INVALID;
  moe::CombineArgs a{};
  a.y_perm = y_perm; a.row_of = row_of; a.topk_w = topk_w; a.y_shared = y_shared; a.y = y;
  a.T = cfg->T; a.d = cfg->d; a.k = (int)cfg->k;
  return hip_status(moe::launch_combine(a, cfg->dtype == MOE_BF16, (hipStream_t)stream));
}

int moe_combine_bwd(const moe_config* cfg, const void* dy, const void* y_perm, const int32_t* row_of,
                    const float* topk_w, void* dy_perm, float* d_topk_w, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!dy || !y_perm || !row_of || !topk_w || !dy_perm || !d_topk_w) return MOE_ERR_INVALID;
  if (!aligned16(dy) || !aligned16(y_perm) || !aligned16(dy_perm)) return MOE_ERR_INVALID;
  moe::CombineArgs a{};
  a.dy = dy; a.y_perm = y_perm; a.row_of = row_of; a.topk_w = topk_w; a.dy_perm = dy_perm; a.d_topk_w = d_topk_w;
  a.T = cfg->T; a.d = cfg->d; a.k = (int)cfg->k;
  return hip_status(moe::launch_combine_bwd(a, cfg->dtype == MOE_BF16, (hipStream_t)stream));
}

int moe_route_bwd(const moe_config* cfg, const void* x, const float* logits, const int32_t* topk_idx,
                  const float* d_topk_w, const float* dlogits_add, float* dlogits, void* dw_router, void* ws,
                  void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!x || !logits || !topk_idx || !d_topk_w || !dlogits || !dw_router || !ws) return MOE_ERR_INVALID;
  if ((uintptr_t)ws & 255u) return MOE_ERR_INVALID;
  moe::RouteBwdArgs a{};
  a.x = x; a.logits = logits; a.topk_idx = topk_idx; a.d_topk_w = d_topk_w; a.dlogits_add = dlogits_add;
  a.dlogits = dlogits;
  a.dw_router = dw_router; a.partial = (float*)ws;
  a.T = cfg->T; a.d = cfg->d; a.E = (int)cfg->E; a.k = (int)cfg->k; a.gating = cfg->gating;
  return hip_status(moe::launch_route_bwd(a, cfg->dtype == MOE_BF16, (hipStream_t)stream));
}

int moe_aux_loss(const moe_config* cfg, const float* logits, const int32_t* raw_counts, float coef, float* loss,
                 void* ws, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!logits || !raw_counts || !loss || !ws) return MOE_ERR_INVALID;
  if (!(coef == coef) || ((uintptr_t)ws & 255u)) return MOE_ERR_INVALID;
  moe::AuxArgs a{};
  a.logits = logits; a.raw_counts = raw_counts; a.coef = coef; a.loss = loss; a.partial = (float*)ws;
  a.T = cfg->T; a.E = (int)cfg->E; a.k = (int)cfg->k;
  return hip_status(moe::launch_aux_loss(a, (hipStream_t)stream));
}

int moe_aux_loss_bwd(const moe_config* cfg, const float* logits, const int32_t* raw_counts, float coef,
                     float* dlogits_aux, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!logits || !raw_counts || !dlogits_aux || !(coef == coef)) return MOE_ERR_INVALID;
  moe::AuxArgs a{};
  a.logits = logits; a.raw_counts = raw_counts; a.coef = coef; a.dlogits = dlogits_aux;
  a.T = cfg->T; a.E = (int)cfg->E; a.k = (int)cfg->k;
  return hip_status(moe::launch_aux_loss_bwd(a, (hipStream_t)stream));
}

int moe_dispatch_bwd(const moe_config* cfg, const void* dx_perm, const int32_t* row_of, const float* dlogits,
                     const void* w_router, const void* dx_add, void* dx, void* stream) {
  int s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!dx_perm || !row_of || !dlogits || !w_router || !dx) return MOE_ERR_INVALID;
  if (!aligned16(dx_perm) || !aligned16(dx) || (dx_add && !aligned16(dx_add))) return MOE_ERR_INVALID;
  moe::DispatchBwdArgs a{};
  a.dx_perm = dx_perm; a.row_of = row_of; a.dlogits = dlogits; a.w_router = w_router; a.dx_add = dx_add; a.dx = dx;
  a.T = cfg->T; a.d = cfg->d; a.E = (int)cfg->E; a.k = (int)cfg->k;
  return hip_status(moe::launch_dispatch_bwd(a, cfg->dtype == MOE_BF16, (hipStream_t)stream));
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
