// Router backward: gating Jacobian and router weight gradient (tutorial
// ch.4, 专家并行与数据并行的结合 三.4: the replicated gate network has
// gradients that are aggregated across replicas; here they are computed for
// one GPU's tokens).
//
// gating_bwd: one wave per token, lane e holds expert e (E <= 64).
//   SOFTMAX_TOPK:          dl = p * (dp - <p, dp>),  p = softmax(l), dp[e_j] = dg_j
//   RENORM / TOPK_SOFTMAX: the weights are a softmax over the chosen logits:
//                          dl[e_j] = g_j * (dg_j - sum_m g_m dg_m), 0 elsewhere
// router wgrad: dW_r = x^T dl as a deterministic two-stage reduction over
//   tokens: each block of tokens writes an fp32 partial [d, E], then the
//   partials are summed in block order.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void gating_bwd_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ dg, float* __restrict__ dl,
                                                         int64_t Tn, int E, int k, int gating) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const bool valid = lane < E;
  const float l = valid ? logits[t * E + lane] : -INFINITY;
  int sel = -1;
  for (int j = 0; j < k; ++j)
    if (idx[t * k + j] == lane) sel = j;
  const float dgl = sel >= 0 ? dg[t * k + sel] : 0.0f;
  float out;
  if (gating == 0) {
    const float mx = group_max<64>(l);
    float p = valid ? __expf(l - mx) : 0.0f;
    const float z = group_sum<64>(p);
    p = p / z;
    const float s = group_sum<64>(p * dgl);
    out = p * (dgl - s);
  } else {
    const float lsel = sel >= 0 ? l : -INFINITY;
    const float mx = group_max<64>(lsel);
    float q = sel >= 0 ? __expf(l - mx) : 0.0f;
    const float z = group_sum<64>(q);
    const float g = q / z;
    const float s = group_sum<64>(g * dgl);
    out = sel >= 0 ? g * (dgl - s) : 0.0f;
  }
  if (valid) dl[t * E + lane] = out;
}

// partial[b][i][e] = sum over tokens t of block b of x[t, i] * dl[t, e]
template <typename T, int EP>
__global__ __launch_bounds__(256) void router_wgrad_partial_kernel(const T* __restrict__ x,
                                                                   const float* __restrict__ dl,
                                                                   float* __restrict__ partial, int64_t Tn, int d,
                                                                   int E, int tb) {
  constexpr int TS = 64;  // tokens staged per step
  __shared__ __attribute__((aligned(16))) float dls[TS * EP];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  const int64_t tbeg = (int64_t)b * tb;
  const int64_t tend = tbeg + tb < Tn ? tbeg + tb : Tn;
  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.0f;
  for (int64_t t0 = tbeg; t0 < tend; t0 += TS) {
    __syncthreads();
    for (int q = threadIdx.x; q < TS * EP; q += 256) {
      const int tl = q / EP, e = q % EP;
      const int64_t t = t0 + tl;
      dls[q] = (t < tend && e < E) ? dl[t * E + e] : 0.0f;
    }
    __syncthreads();
    const int nt = (int)(tend - t0 < TS ? tend - t0 : TS);
    if (i < d) {
      for (int tl = 0; tl < nt; ++tl) {
        const float xv = to_f32(x[(t0 + tl) * d + i]);
        const float* dlt = dls + tl * EP;
#pragma unroll
        for (int e = 0; e < EP; e += 4) {
          const f32x4 lv = *reinterpret_cast<const f32x4*>(dlt + e);
          acc[e] += xv * lv[0];
          acc[e + 1] += xv * lv[1];
          acc[e + 2] += xv * lv[2];
          acc[e + 3] += xv * lv[3];
        }
      }
    }
  }
  if (i < d) {
    float* p = partial + ((int64_t)b * d + i) * E;
#pragma unroll
    for (int e = 0; e < EP; ++e)
      if (e < E) p[e] = acc[e];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(const float* __restrict__ partial, int nb,
                                                                  int64_t dE, T* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= dE) return;
  float s = 0.0f;
  for (int b = 0; b < nb; ++b) s += partial[(int64_t)b * dE + i];
  dw[i] = from_f32<T>(s);
}

template <typename T, int EP>
static hipError_t launch_rwg(const RouteBwdArgs& a, hipStream_t st) {
  const int nb = router_wgrad_blocks(a.T);
  const int tb = (int)((a.T + nb - 1) / nb);
  hipLaunchKernelGGL((router_wgrad_partial_kernel<T, EP>), dim3((unsigned)((a.d + 255) / 256), nb), dim3(256), 0, st,
                     (const T*)a.x, a.dlogits, a.partial, a.T, (int)a.d, a.E, tb);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t dE = a.d * a.E;
  hipLaunchKernelGGL((router_wgrad_reduce_kernel<T>), dim3((unsigned)((dE + 255) / 256)), dim3(256), 0, st,
                     a.partial, nb, dE, (T*)a.dw_router);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_rwg_dt(const RouteBwdArgs& a, hipStream_t st) {
  if (a.E <= 8) return launch_rwg<T, 8>(a, st);
  if (a.E <= 16) return launch_rwg<T, 16>(a, st);
  if (a.E <= 32) return launch_rwg<T, 32>(a, st);
  return launch_rwg<T, 64>(a, st);
}

int router_wgrad_blocks(int64_t T) {
  int64_t nb = (T + 255) / 256;
  if (nb > 64) nb = 64;
  if (nb < 1) nb = 1;
  return (int)nb;
}

hipError_t launch_route_bwd(const RouteBwdArgs& a, bool bf16_dtype, hipStream_t st) {
  const int64_t blocks = (a.T + 3) / 4;
  hipLaunchKernelGGL(gating_bwd_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.logits, a.topk_idx, a.d_topk_w,
                     a.dlogits, a.T, a.E, a.k, a.gating);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return bf16_dtype ? launch_rwg_dt<bf16>(a, st) : launch_rwg_dt<float>(a, st);
}

}  // namespace moe
