// Gate GEMM + softmax + top-k routing (tutorial ch.4, 专家并行 二 step 1:
// every device scores its local tokens with the replicated router g(x);
// 用于分布式 MoE 的主流框架与库: a top-k gate with k chosen experts).
//
// One token is handled by a group of S lanes of a wave (S = 8 or 16).  Lane s
// streams 16-byte pieces of the token's row (coalesced: the S lanes cover
// S*16 contiguous bytes) and accumulates partial logits for all EP (padded)
// experts against a K-chunk of the router weight staged in LDS as fp32.
// A butterfly reduce-scatter over the S lanes then leaves lane s with the
// complete logits of experts [s*EP/S, (s+1)*EP/S); softmax statistics and the
// k rounds of arg-max are wave shuffles over the group.  Comparisons order by
// (logit descending, expert index ascending), so equal logits go to the lower
// index.  fp32 accumulation throughout; the summation order is fixed, so the
// logits are deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

template <typename T, int S, int EP>
__global__ __launch_bounds__(256) void route_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                   const float* __restrict__ bias, float* __restrict__ logits,
                                                   int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                   int64_t Tn, int d, int E, int k, int gating) {
  constexpr int V = Vec16<T>::N;
  constexpr int KC = S * V;       // K rows per LDS chunk
  constexpr int TPB = 256 / S;    // tokens per block
  constexpr int EPL = EP / S;     // experts per lane after the reduce-scatter
  constexpr int WP = EP + 4;      // LDS row pitch in floats (breaks bank aliasing)
  __shared__ __attribute__((aligned(16))) float wl[KC * WP];

  const int tid = threadIdx.x;
  const int s = tid % S;
  const int64_t t = (int64_t)blockIdx.x * TPB + tid / S;
  const bool tok_ok = t < Tn;

  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.0f;

  for (int k0 = 0; k0 < d; k0 += KC) {
    const int kx = k0 + s * V;
    float xv[V];
    if (tok_ok && kx < d) {
      unpack16<T>(ld16(x + t * d + kx), xv);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) xv[i] = 0.0f;
    }
    __syncthreads();
    for (int i = tid; i < KC * EP; i += 256) {
      const int r = i / EP, e = i % EP;
      float v = 0.0f;
      if (k0 + r < d && e < E) v = to_f32(w[(int64_t)(k0 + r) * E + e]);
      wl[r * WP + e] = v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float* wr = wl + (s * V + i) * WP;
#pragma unroll
      for (int e = 0; e < EP; e += 4) {
        const f32x4 wv = *reinterpret_cast<const f32x4*>(wr + e);
        acc[e] += xv[i] * wv[0];
        acc[e + 1] += xv[i] * wv[1];
        acc[e + 2] += xv[i] * wv[2];
        acc[e + 3] += xv[i] * wv[3];
      }
    }
  }

  // Reduce-scatter over the S lanes: after the step with mask m the lane
  // keeps the half of its experts selected by bit m of s.
#pragma unroll
  for (int m = S / 2; m >= 1; m >>= 1) {
    const int half = EP * m / S;
    const bool upper = (s & m) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = upper ? acc[i] : acc[i + half];
      const float keep = upper ? acc[i + half] : acc[i];
      acc[i] = keep + __shfl_xor(send, m, kWave);
    }
  }
  const int e0 = s * EPL;
  float lv[EPL];
  bool valid[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = e0 + i;
    valid[i] = e < E;
    lv[i] = valid[i] ? acc[i] + (bias ? bias[e] : 0.0f) : -INFINITY;
    if (tok_ok && valid[i]) logits[t * E + e] = lv[i];
  }

  // softmax statistics over all experts of the token
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) mx = fmaxf(mx, lv[i]);
  mx = group_max<S>(mx);
  float z = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) z += valid[i] ? __expf(lv[i] - mx) : 0.0f;
  z = group_sum<S>(z);

  // k rounds of arg-max by (value desc, index asc)
  unsigned taken = 0u;
  float sel_v[8];
  int sel_e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel_v[j] = -INFINITY;
    sel_e[j] = 0;
    if (j < k) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (valid[i] && !((taken >> i) & 1u) && (lv[i] > bv || be == 0x7fffffff)) {
          bv = lv[i];
          be = e0 + i;
        }
      }
#pragma unroll
      for (int m = 1; m < S; m <<= 1) {
        const float ov = __shfl_xor(bv, m, kWave);
        const int oe = __shfl_xor(be, m, kWave);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
      if (be >= e0 && be < e0 + EPL) taken |= 1u << (be - e0);
      sel_v[j] = bv;
      sel_e[j] = be;
    }
  }

  if (tok_ok && s == 0) {
    float den = 0.0f;
    if (gating != 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < k) den += __expf(sel_v[j] - sel_v[0]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        const float g = gating == 0 ? __expf(sel_v[j] - mx) / z : __expf(sel_v[j] - sel_v[0]) / den;
        topk_idx[t * k + j] = sel_e[j];
        topk_w[t * k + j] = g;
      }
    }
  }
}

template <typename T, int S, int EP>
static hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  constexpr int TPB = 256 / S;
  const int64_t blocks = (a.T + TPB - 1) / TPB;
  hipLaunchKernelGGL((route_kernel<T, S, EP>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const T*)a.x, (const T*)a.w, a.bias, a.logits, a.topk_idx, a.topk_w, a.T, a.d, a.E, a.k,
                     a.gating);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_route_dt(const RouteArgs& a, hipStream_t st) {
  if (a.E <= 8) return launch_route_t<T, 8, 8>(a, st);
  if (a.E <= 16) return launch_route_t<T, 16, 16>(a, st);
  if (a.E <= 32) return launch_route_t<T, 16, 32>(a, st);
  return launch_route_t<T, 16, 64>(a, st);
}

hipError_t launch_route(const RouteArgs& a, bool bf16_dtype, hipStream_t st) {
  return bf16_dtype ? launch_route_dt<bf16>(a, st) : launch_route_dt<float>(a, st);
}

}  // namespace moe
