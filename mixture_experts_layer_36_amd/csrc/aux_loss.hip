// Auxiliary load-balancing loss (tutorial ch.4, 用于分布式 MoE 的主流框架与库
// 一: DeepSpeed's moe block takes a load-balancing loss coefficient,
// loss_coef; 实践: the logged auxiliary loss should be near 0 with the
// experts chosen about equally often).  The pages give no formula; the
// reading taken is
//   L = coef * E * sum_e f_e P_e,
// f_e = raw_counts[e] / (T k), the share of the routing choices on expert e
// (before capacity), P_e = mean over tokens of softmax(l_t)[e].  Its logits
// gradient, with f constant (it moves only where the top-k changes), is
//   dL/dl[t, j] = coef * E / T * p[t, j] * (f_j - sum_e f_e p[t, e]).
//
// Both are bandwidth kernels over the fp32 logits (T x E x 4 bytes).  The
// loss is a deterministic two-stage reduction: each workgroup sums the
// probabilities of a fixed set of tokens per expert (lane trees, then the
// waves in order), and one wave adds the workgroups' partials in order.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kAuxBlocks = 256;  // partials of the loss reduction (at most)

// G lanes per token (E rounded up to a power of two, at least 8); a pass of
// the workgroup covers 4 * 64 / G tokens; workgroup b takes passes b, b + nb, ...
template <int G>
__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits, int64_t Tn, int E,
                                                          int nb, float* __restrict__ partial) {
  constexpr int TPW = 64 / G, TPP = 4 * TPW;  // tokens per wave / per pass
  __shared__ float wsum[4][G];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = lane % G;
  float acc = 0.0f;
  for (int64_t pass = blockIdx.x; pass * TPP < Tn; pass += nb) {
    const int64_t t = pass * TPP + w * TPW + lane / G;
    const bool tok = t < Tn;
    const bool valid = tok && e < E;
    const float l = valid ? logits[t * E + e] : -INFINITY;
    const float mx = group_max<G>(l);
    float p = valid ? __expf(l - mx) : 0.0f;
    const float z = group_sum<G>(p);
    acc += (valid && z > 0.0f) ? p / z : 0.0f;
  }
  // sum over the wave's token groups (lanes e, e + G, ...), fixed tree
#pragma unroll
  for (int m = G; m < 64; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (lane < G) wsum[w][lane] = acc;
  __syncthreads();
  if (threadIdx.x < E) {
    const int ex = threadIdx.x;
    partial[(int64_t)blockIdx.x * E + ex] = ((wsum[0][ex] + wsum[1][ex]) + wsum[2][ex]) + wsum[3][ex];
  }
}

// One wave: lane e adds expert e's partials in block order, then
// L = coef * E * sum_e (raw_e / (T k)) * (S_e / T).
__global__ __launch_bounds__(64) void aux_finish_kernel(const float* __restrict__ partial, int nb,
                                                        const int32_t* __restrict__ raw, int64_t Tn, int E, int k,
                                                        float coef, float* __restrict__ loss) {
  const int lane = threadIdx.x;
  float s = 0.0f;
  if (lane < E)
    for (int b = 0; b < nb; ++b) s += partial[(int64_t)b * E + lane];
  const float tf = (float)Tn;
  const float term = lane < E ? ((float)raw[lane] / (tf * (float)k)) * (s / tf) : 0.0f;
  const float tot = group_sum<64>(term);
  if (lane == 0) loss[0] = coef * (float)E * tot;
}

// dlogits_aux[t, e] = scale * p[t, e] * (raw_e - sum_m raw_m p[t, m]),
// scale = coef * E / (T * T * k); G lanes per token as in aux_partial_kernel.
template <int G>
__global__ __launch_bounds__(256) void aux_grad_kernel(const float* __restrict__ logits,
                                                       const int32_t* __restrict__ raw, int64_t Tn, int E,
                                                       float scale, float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  const int e = lane % G;
  const bool valid = t < Tn && e < E;
  const float l = valid ? logits[t * E + e] : -INFINITY;
  const float c = valid ? (float)raw[e] : 0.0f;
  const float mx = group_max<G>(l);
  float p = valid ? __expf(l - mx) : 0.0f;
  const float z = group_sum<G>(p);
  p = z > 0.0f ? p / z : 0.0f;
  const float s = group_sum<G>(c * p);
  if (valid) dl[t * E + e] = scale * p * (c - s);
}

size_t aux_ws_bytes(int64_t E) { return (size_t)kAuxBlocks * E * 4; }

template <int G>
static hipError_t launch_aux_loss_g(const AuxArgs& a, hipStream_t st) {
  constexpr int TPP = 4 * (64 / G);
  const int64_t passes = (a.T + TPP - 1) / TPP;
  const int nb = (int)(passes < kAuxBlocks ? passes : kAuxBlocks);
  if (nb <= 0) return hipSuccess;
  hipLaunchKernelGGL((aux_partial_kernel<G>), dim3(nb), dim3(256), 0, st, a.logits, a.T, a.E, nb, a.partial);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(aux_finish_kernel, dim3(1), dim3(64), 0, st, a.partial, nb, a.raw_counts, a.T, a.E, a.k,
                     a.coef, a.loss);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_aux_grad_g(const AuxArgs& a, hipStream_t st) {
  constexpr int TPB = 4 * (64 / G);
  const int64_t blocks = (a.T + TPB - 1) / TPB;
  if (blocks <= 0) return hipSuccess;
  const double scale = (double)a.coef * (double)a.E / ((double)a.T * (double)a.T * (double)a.k);
  hipLaunchKernelGGL((aux_grad_kernel<G>), dim3((unsigned)blocks), dim3(256), 0, st, a.logits, a.raw_counts, a.T,
                     a.E, (float)scale, a.dlogits);
  return hipGetLastError();
}

hipError_t launch_aux_loss(const AuxArgs& a, hipStream_t st) {
  return a.E <= 8 ? launch_aux_loss_g<8>(a, st)
         : a.E <= 16 ? launch_aux_loss_g<16>(a, st)
         : a.E <= 32 ? launch_aux_loss_g<32>(a, st)
         : launch_aux_loss_g<64>(a, st);
}

hipError_t launch_aux_loss_bwd(const AuxArgs& a, hipStream_t st) {
  return a.E <= 8 ? launch_aux_grad_g<8>(a, st)
         : a.E <= 16 ? launch_aux_grad_g<16>(a, st)
         : a.E <= 32 ? launch_aux_grad_g<32>(a, st)
         : launch_aux_grad_g<64>(a, st);
}

}  // namespace moe
