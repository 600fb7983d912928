// Router backward: gating Jacobian and router weight gradient (tutorial
// ch.4, 专家并行与数据并行的结合 三.4: the replicated gate network has
// gradients that are aggregated across replicas; here they are computed for
// one GPU's tokens).
//
// gating_bwd: lane e of a token's lane group holds expert e (E <= 64).
//   SOFTMAX_TOPK:          dl = p * (dp - <p, dp>),  p = softmax(l), dp[e_j] = dg_j
//   RENORM / TOPK_SOFTMAX: the weights are a softmax over the chosen logits:
//                          dl[e_j] = g_j * (dg_j - sum_m g_m dg_m), 0 elsewhere
// router wgrad: dW_r = x^T dl as a deterministic two-stage reduction over
//   tokens: each block of tokens writes an fp32 partial [d, E], then the
//   partials are summed in block order (at most 64 blocks).
#include "common.h"
#include "kernels.h"

namespace moe {

// G lanes per token (G = E rounded up to a power of two, at least 8), 64 / G
// tokens per wave; the softmax statistics and the weighted sums are
// reductions over the token's G lanes.
template <int G>
__global__ __launch_bounds__(256) void gating_bwd_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ dg, float* __restrict__ dl,
                                                         int64_t Tn, int E, int k, int gating) {
  const int lane = threadIdx.x & 63;
  const int64_t t = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  const int e = lane % G;
  const bool tok = t < Tn;  // every lane stays for the group reductions
  const bool valid = tok && e < E;
  const float l = valid ? logits[t * E + e] : -INFINITY;
  int sel = -1;
  for (int j = 0; j < k; ++j)
    if (tok && idx[t * k + j] == e) sel = j;
  const float dgl = sel >= 0 ? dg[t * k + sel] : 0.0f;
  float out;
  if (gating == 0) {
    const float mx = group_max<G>(l);
    float p = valid ? __expf(l - mx) : 0.0f;
    const float z = group_sum<G>(p);
    p = z > 0.0f ? p / z : 0.0f;
    const float s = group_sum<G>(p * dgl);
    out = p * (dgl - s);
  } else {
    const float lsel = sel >= 0 ? l : -INFINITY;
    const float mx = group_max<G>(lsel);
    float q = sel >= 0 ? __expf(l - mx) : 0.0f;
    const float z = group_sum<G>(q);
    const float g = z > 0.0f ? q / z : 0.0f;
    const float s = group_sum<G>(g * dgl);
    out = sel >= 0 ? g * (dgl - s) : 0.0f;
  }
  if (valid) dl[t * E + e] = out;
}

template <int G>
static hipError_t launch_gating_bwd(const RouteBwdArgs& a, hipStream_t st) {
  constexpr int TPB = 4 * (64 / G);  // tokens per workgroup
  const int64_t blocks = (a.T + TPB - 1) / TPB;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gating_bwd_kernel<G>), dim3((unsigned)blocks), dim3(256), 0, st, a.logits, a.topk_idx,
                     a.d_topk_w, a.dlogits, a.T, a.E, a.k, a.gating);
  return hipGetLastError();
}

// CPT consecutive elements of a row as floats (16, 8, 4 or 2 bytes).
template <typename T, int CPT>
__device__ __forceinline__ void load_row_cols(const T* p, float (&v)[CPT]) {
  if constexpr (CPT * sizeof(T) == 16) {
    unpack16<T>(ld16(p), v);
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) v[c] = to_f32(p[c]);
  }
}

// partial[b][i][e] = sum over tokens t of token block b of x[t, i] * dl[t, e].
// A lane owns CPT = 64 / EP consecutive columns (all EP experts: 64 fp32
// accumulators); the 4 waves of a workgroup take consecutive quarters of the
// block's tokens, 8 tokens per round with their x loads issued first, the
// tokens' dlogits coming in through wave-uniform scalar loads.  The waves'
// sums are added in wave order through LDS, so the partials are deterministic.
constexpr int kRwgWaves = 4;

template <typename T, int EP, int CPT, bool FULL>
__global__ __launch_bounds__(64 * kRwgWaves) void router_wgrad_partial_kernel(const T* __restrict__ x,
                                                                              const float* __restrict__ dl,
                                                                              float* __restrict__ partial,
                                                                              int64_t Tn, int d, int E, int tw) {
  static_assert(CPT * EP == 64, "64 accumulators per lane");
  constexpr int TU = 8;
  __shared__ float red[kRwgWaves - 1][64][64];  // [wave - 1][accumulator][lane]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i0 = (blockIdx.x * 64 + lane) * CPT;
  const bool col_ok = i0 < d;  // d is a multiple of 8: a lane's columns are all in or all out
  const int64_t tbeg = ((int64_t)blockIdx.y * kRwgWaves + wave) * tw;
  const int64_t tend = tbeg + tw < Tn ? tbeg + tw : Tn;
  const int Es = FULL ? EP : E;
  float acc[CPT][EP];
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[c][e] = 0.0f;
  // one token: x[t, i0..] (unconditional load, zeros by select for lanes
  // past the last column) times the token's dlogits
  auto token = [&](int64_t t, const float (&xr)[CPT]) {
    const float* dlt = dl + t * Es;
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      const float lv = (FULL || e < E) ? dlt[e] : 0.0f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c][e] = fmaf(xr[c], lv, acc[c][e]);
    }
    // one token's dlogits at a time in scalar registers (up to 64)
    if constexpr (EP >= 32) __builtin_amdgcn_sched_barrier(0);
  };
  auto load_x = [&](int64_t t, float (&xr)[CPT]) {
    load_row_cols<T, CPT>(col_ok ? x + t * d + i0 : x, xr);
#pragma unroll
    for (int c = 0; c < CPT; ++c) xr[c] = col_ok ? xr[c] : 0.0f;
  };
  int64_t t = tbeg;
  // full rounds of TU tokens: all TU loads issued before the FMAs
  for (; t + TU <= tend; t += TU) {
    float xv[TU][CPT];
#pragma unroll
    for (int u = 0; u < TU; ++u) load_x(t + u, xv[u]);
#pragma unroll
    for (int u = 0; u < TU; ++u) token(t + u, xv[u]);
  }
  for (; t < tend; ++t) {
    float xr[CPT];
    load_x(t, xr);
    token(t, xr);
  }
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < EP; ++e) red[wave - 1][c * EP + e][lane] = acc[c][e];
  }
  __syncthreads();
  if (wave == 0 && col_ok) {
#pragma unroll
    for (int w = 0; w < kRwgWaves - 1; ++w)
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < EP; ++e) acc[c][e] += red[w][c * EP + e][lane];
    float* p = partial + ((int64_t)blockIdx.y * d + i0) * E;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < EP; ++e)
        if (FULL || e < E) p[c * E + e] = acc[c][e];
  }
}

// partial[b][i][e] on the fp32 matrix cores: v_mfma_f32_16x16x4_f32 takes
// A[m][kk] from lane kk * 16 + m and B[kk][n] from lane kk * 16 + n, so 4
// tokens x 16 columns of x and 4 tokens x 16 experts of dlogits enter as one
// value per lane, with no transposition.  A lane loads 16 bytes of x (V
// consecutive columns c0 + V m + j of token t = 4-group base + lane / 16) and
// feeds value j to the MFMA of column block j: block j's row m is column
// c0 + V m + j, so one workgroup covers CW = 16 V columns.  The products are
// exact in fp32 and summed in fp32 in a fixed order, as before; the 4 waves
// take consecutive quarters of the block's tokens (4 token groups per round,
// loads first) and their accumulators are summed in a fixed tree through LDS.
template <typename T, int EP>
__global__ __launch_bounds__(64 * kRwgWaves) void router_wgrad_mfma_kernel(const T* __restrict__ x,
                                                                           const float* __restrict__ dl,
                                                                           float* __restrict__ partial, int64_t Tn,
                                                                           int d, int E, int tw) {
  constexpr int V = Vec16<T>::N, NB = EP / 16, CW = 16 * V, U = 4;
  constexpr int NACC = V * NB;  // f32x4 accumulators per lane
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kk = lane >> 4, m = lane & 15;
  const int c0 = blockIdx.x * CW + V * m;  // this lane's first x column
  const bool col_ok = c0 < d;              // d is a multiple of 8: all V columns in or out
  const int64_t tbeg = ((int64_t)blockIdx.y * kRwgWaves + wave) * tw;
  const int64_t tend = tbeg + tw < Tn ? tbeg + tw : Tn;
  f32x4 acc[V][NB];
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // token group at t4: lane's token t4 + kk; unconditional loads from valid
  // addresses, zeros by select past the range, the last column or E
  auto load = [&](int64_t t4, u32x4& xv, float (&dv)[NB]) {
    const int64_t t = t4 + kk;
    const bool tok = t < tend;
    const int64_t tc = tok ? t : tbeg;
    const u32x4 v = ld16(x + tc * d + (col_ok ? c0 : 0));
    xv = (tok && col_ok) ? v : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = 16 * nb + m;
      const float w = dl[tc * E + (e < E ? e : E - 1)];
      dv[nb] = (tok && e < E) ? w : 0.0f;
    }
  };
  for (int64_t t = tbeg; t < tend; t += 4 * U) {
    u32x4 xv[U];
    float dv[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) load(t + 4 * u, xv[u], dv[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xf[V];
      unpack16<T>(xv[u], xf);
#pragma unroll
      for (int j = 0; j < V; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[j][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[j], dv[u][nb], acc[j][nb], 0, 0, 0);
    }
  }
  // fixed-order tree sum of the 4 waves' accumulators: (w2 + w3) into w0, w1; then w1 into w0
  float* red = reinterpret_cast<float*>(lds);  // [2][NACC * 4][64]
  if (wave >= 2) {
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[(((wave - 2) * NACC + j * NB + nb) * 4 + q) * 64 + lane] = acc[j][nb][q];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j][nb][q] += red[((wave * NACC + j * NB + nb) * 4 + q) * 64 + lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[((j * NB + nb) * 4 + q) * 64 + lane] = acc[j][nb][q];
  }
  __syncthreads();
  if (wave != 0) return;
  // accumulator (j, nb)[q] of lane l: column blockIdx.x CW + V (4 (l / 16) + q) + j, expert 16 nb + l % 16
  float* pb = partial + (int64_t)blockIdx.y * d * E;
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v = acc[j][nb][q] + red[((j * NB + nb) * 4 + q) * 64 + lane];
        const int col = blockIdx.x * CW + V * (4 * kk + q) + j, e = 16 * nb + m;
        if (col < d && e < E) pb[(int64_t)col * E + e] = v;
      }
}

// dw[i] = sum over b in order of partial[b][i].  A thread owns 4 consecutive
// outputs and loads all its partials (nb <= 64, 16-byte loads) before the
// in-order sums, so the loads overlap instead of following one another.
template <typename T>
__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(const float* __restrict__ partial, int nb,
                                                                  int64_t dE, T* __restrict__ dw) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= dE) return;
  if (i0 + 4 <= dE && (dE & 3) == 0) {
    f32x4 v[64];
#pragma unroll
    for (int b = 0; b < 64; ++b)
      if (b < nb) v[b] = *reinterpret_cast<const f32x4*>(partial + (int64_t)b * dE + i0);
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int b = 0; b < 64; ++b)
      if (b < nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) s[q] += v[b][q];
#pragma unroll
    for (int q = 0; q < 4; ++q) dw[i0 + q] = from_f32<T>(s[q]);
  } else {
    for (int64_t i = i0; i < i0 + 4 && i < dE; ++i) {
      float s = 0.0f;
      for (int b = 0; b < nb; ++b) s += partial[(int64_t)b * dE + i];
      dw[i] = from_f32<T>(s);
    }
  }
}

template <typename T, int EP>
static hipError_t launch_rwg(const RouteBwdArgs& a, hipStream_t st) {
  constexpr int CPT = 64 / EP;
  const int nb = router_wgrad_blocks(a.T);
  const int tw = (int)((a.T + (int64_t)nb * kRwgWaves - 1) / ((int64_t)nb * kRwgWaves));  // tokens per wave
  const dim3 grid((unsigned)((a.d + 64 * CPT - 1) / (64 * CPT)), nb);
  if (a.E == EP)
    hipLaunchKernelGGL((router_wgrad_partial_kernel<T, EP, CPT, true>), grid, dim3(64 * kRwgWaves), 0, st,
                       (const T*)a.x, a.dlogits, a.partial, a.T, (int)a.d, a.E, tw);
  else
    hipLaunchKernelGGL((router_wgrad_partial_kernel<T, EP, CPT, false>), grid, dim3(64 * kRwgWaves), 0, st,
                       (const T*)a.x, a.dlogits, a.partial, a.T, (int)a.d, a.E, tw);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t dE = a.d * a.E;
  hipLaunchKernelGGL((router_wgrad_reduce_kernel<T>), dim3((unsigned)((dE + 1023) / 1024)), dim3(256), 0, st,
                     a.partial, nb, dE, (T*)a.dw_router);
  return hipGetLastError();
}

template <typename T, int EP>
static hipError_t launch_rwg_mfma(const RouteBwdArgs& a, hipStream_t st) {
  constexpr int V = Vec16<T>::N, CW = 16 * V;
  constexpr size_t lds = (size_t)2 * V * (EP / 16) * 4 * 64 * 4;
  const int nb = router_wgrad_blocks(a.T);
  const int tw = (int)((a.T + (int64_t)nb * kRwgWaves - 1) / ((int64_t)nb * kRwgWaves));  // tokens per wave
  const dim3 grid((unsigned)((a.d + CW - 1) / CW), nb);
  auto kern = router_wgrad_mfma_kernel<T, EP>;
  if constexpr (lds > 65536) {
    static const hipError_t prep = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (prep != hipSuccess) return prep;
  }
  hipLaunchKernelGGL(kern, grid, dim3(64 * kRwgWaves), lds, st, (const T*)a.x, a.dlogits, a.partial, a.T, (int)a.d,
                     a.E, tw);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t dE = a.d * a.E;
  hipLaunchKernelGGL((router_wgrad_reduce_kernel<T>), dim3((unsigned)((dE + 1023) / 1024)), dim3(256), 0, st,
                     a.partial, nb, dE, (T*)a.dw_router);
  return hipGetLastError();
}

// bf16 x with up to 16 experts: the vector kernel, bound by reading x (the
// fp32 MFMA pads E to 16 and measured slower on the Mixtral shape, 0.059
// against 0.049 ms for the whole router backward).  More experts, or fp32 x:
// the fp32 MFMA kernel (DeepSeek-V2-Lite shape 0.187 -> 0.137 ms).
template <typename T>
static hipError_t launch_rwg_dt(const RouteBwdArgs& a, hipStream_t st) {
  if (sizeof(T) == 2 && a.E <= 8) return launch_rwg<T, 8>(a, st);
  if (sizeof(T) == 2 && a.E <= 16) return launch_rwg<T, 16>(a, st);
  if (a.E <= 16) return launch_rwg_mfma<T, 16>(a, st);
  if (a.E <= 32) return launch_rwg_mfma<T, 32>(a, st);
  return launch_rwg_mfma<T, 64>(a, st);
}

int router_wgrad_blocks(int64_t T) {
  int64_t nb = (T + 255) / 256;
  if (nb > 64) nb = 64;
  if (nb < 1) nb = 1;
  return (int)nb;
}

hipError_t launch_route_bwd(const RouteBwdArgs& a, bool bf16_dtype, hipStream_t st) {
  hipError_t err = a.E <= 8 ? launch_gating_bwd<8>(a, st)
                   : a.E <= 16 ? launch_gating_bwd<16>(a, st)
                   : a.E <= 32 ? launch_gating_bwd<32>(a, st)
                   : launch_gating_bwd<64>(a, st);
  if (err != hipSuccess) return err;
  return bf16_dtype ? launch_rwg_dt<bf16>(a, st) : launch_rwg_dt<float>(a, st);
}

}  // namespace moe
