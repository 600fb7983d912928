// Weighted combine, its backward, and the un-permute sum of the backward.
//
// Tutorial ch.4, 专家并行 二 step 4 (results return to the token's device and
// the sequence order is restored), 流水线并行 三 (expert outputs are merged),
// and 专家并行与数据并行的结合 三.3 (gradients routed back to the experts).
// All three are bandwidth kernels: every row is moved with 16-byte accesses
// that are contiguous along the row, and sums are accumulated in fp32 in a
// fixed order (no atomics, deterministic).
#include "common.h"
#include "kernels.h"

namespace moe {

// y[t] = sum_j g[t,j] * y_perm[row_of[t,j]] (+ y_shared[t])
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y_perm, const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ topk_w,
                                                      const T* __restrict__ y_shared, T* __restrict__ y, int64_t Tn,
                                                      int d, int k, int tpb) {
  constexpr int V = Vec16<T>::N;
  const int nch = d / V;
  const int total = tpb * nch;
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  for (int i = threadIdx.x; i < total; i += 256) {
    const int tl = i / nch, c = i - tl * nch;
    const int64_t t = t0 + tl;
    if (t >= Tn) break;
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = row_of[t * k + j];
      if (r < 0) continue;
      const float g = topk_w[t * k + j];
      float v[V];
      unpack16<T>(ld16(y_perm + (int64_t)r * d + (int64_t)c * V), v);
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] += g * v[q];
    }
    if (y_shared) {
      float v[V];
      unpack16<T>(ld16(y_shared + t * d + (int64_t)c * V), v);
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] += v[q];
    }
    st16(y + t * d + (int64_t)c * V, pack16<T>(acc));
  }
}

// One wave per token: dy_perm[row] = g * dy[t]; d_topk_w[t,j] = <dy[t], y_perm[row]>.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ y_perm,
                                                          const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ topk_w, T* __restrict__ dy_perm,
                                                          float* __restrict__ d_topk_w, int64_t Tn, int d, int k) {
  constexpr int V = Vec16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int nch = d / V;
  int rows[8];
  float g[8], dot[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < k ? row_of[t * k + j] : -1;
    g[j] = rows[j] >= 0 ? topk_w[t * k + j] : 0.0f;
    dot[j] = 0.0f;
  }
  for (int c = lane; c < nch; c += 64) {
    float dv[V];
    unpack16<T>(ld16(dy + t * d + (int64_t)c * V), dv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] < 0) continue;
      float ov[V], sv[V];
      unpack16<T>(ld16(y_perm + (int64_t)rows[j] * d + (int64_t)c * V), ov);
      float p = 0.0f;
#pragma unroll
      for (int q = 0; q < V; ++q) {
        p += dv[q] * ov[q];
        sv[q] = g[j] * dv[q];
      }
      dot[j] += p;
      st16(dy_perm + (int64_t)rows[j] * d + (int64_t)c * V, pack16<T>(sv));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const float s = group_sum<64>(dot[j]);
    if (lane == 0) d_topk_w[t * k + j] = rows[j] >= 0 ? s : 0.0f;
  }
}

// dx[t, i] = sum_j dx_perm[row_of[t,j], i] + sum_e dl[t,e] * W_r[i,e] (+ dx_add[t, i]).
// A thread owns CPT consecutive columns and keeps their router-weight rows in
// registers while it walks the block's tokens; the tokens' dlogits are staged
// in LDS.
template <typename T, int EP, int CPT>
__global__ __launch_bounds__(256) void dispatch_bwd_kernel(const T* __restrict__ dx_perm,
                                                           const int32_t* __restrict__ row_of,
                                                           const float* __restrict__ dl, const T* __restrict__ w_r,
                                                           const T* __restrict__ dx_add, T* __restrict__ dx,
                                                           int64_t Tn, int d, int E, int k, int tpw) {
  extern __shared__ __attribute__((aligned(16))) float dls[];  // [tpw][EP]
  const int64_t t0 = (int64_t)blockIdx.x * tpw;
  const int i0 = (blockIdx.y * 256 + threadIdx.x) * CPT;
  for (int q = threadIdx.x; q < tpw * EP; q += 256) {
    const int tl = q / EP, e = q % EP;
    const int64_t t = t0 + tl;
    dls[q] = (t < Tn && e < E) ? dl[t * E + e] : 0.0f;
  }
  __syncthreads();
  if (i0 >= d) return;
  float wr[CPT][EP];
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < EP; ++e) wr[c][e] = e < E ? to_f32(w_r[(int64_t)(i0 + c) * E + e]) : 0.0f;

  for (int tl = 0; tl < tpw; ++tl) {
    const int64_t t = t0 + tl;
    if (t >= Tn) break;
    float acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = row_of[t * k + j];
      if (r < 0) continue;
      const T* p = dx_perm + (int64_t)r * d + i0;
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c] += to_f32(p[c]);
    }
    const float* dlt = dls + tl * EP;
#pragma unroll
    for (int e = 0; e < EP; e += 4) {
      const f32x4 lv = *reinterpret_cast<const f32x4*>(dlt + e);
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        acc[c] += lv[0] * wr[c][e] + lv[1] * wr[c][e + 1] + lv[2] * wr[c][e + 2] + lv[3] * wr[c][e + 3];
    }
    if (dx_add) {
      const T* p = dx_add + t * d + i0;
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c] += to_f32(p[c]);
    }
    T* o = dx + t * d + i0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) o[c] = from_f32<T>(acc[c]);
  }
}

hipError_t launch_combine(const CombineArgs& a, bool bf16_dtype, hipStream_t st) {
  const int tpb = tokens_per_copy_block(a.d, bf16_dtype ? 2 : 4);
  const int64_t blocks = (a.T + tpb - 1) / tpb;
  if (bf16_dtype)
    hipLaunchKernelGGL((combine_kernel<bf16>), dim3((unsigned)blocks), dim3(256), 0, st, (const bf16*)a.y_perm,
                       a.row_of, a.topk_w, (const bf16*)a.y_shared, (bf16*)a.y, a.T, (int)a.d, a.k, tpb);
  else
    hipLaunchKernelGGL((combine_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, st, (const float*)a.y_perm,
                       a.row_of, a.topk_w, (const float*)a.y_shared, (float*)a.y, a.T, (int)a.d, a.k, tpb);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const CombineArgs& a, bool bf16_dtype, hipStream_t st) {
  const int64_t blocks = (a.T + 3) / 4;
  if (bf16_dtype)
    hipLaunchKernelGGL((combine_bwd_kernel<bf16>), dim3((unsigned)blocks), dim3(256), 0, st, (const bf16*)a.dy,
                       (const bf16*)a.y_perm, a.row_of, a.topk_w, (bf16*)a.dy_perm, a.d_topk_w, a.T, (int)a.d, a.k);
  else
    hipLaunchKernelGGL((combine_bwd_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, st, (const float*)a.dy,
                       (const float*)a.y_perm, a.row_of, a.topk_w, (float*)a.dy_perm, a.d_topk_w, a.T, (int)a.d,
                       a.k);
  return hipGetLastError();
}

template <typename T, int EP, int CPT>
static hipError_t launch_dbwd_t(const DispatchBwdArgs& a, hipStream_t st) {
  constexpr int TPW = 32;
  const int64_t bx = (a.T + TPW - 1) / TPW;
  const int by = (int)((a.d + 256 * CPT - 1) / (256 * CPT));
  hipLaunchKernelGGL((dispatch_bwd_kernel<T, EP, CPT>), dim3((unsigned)bx, by), dim3(256),
                     TPW * EP * sizeof(float), st, (const T*)a.dx_perm, a.row_of, a.dlogits, (const T*)a.w_router,
                     (const T*)a.dx_add, (T*)a.dx, a.T, (int)a.d, a.E, a.k, TPW);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_dbwd_dt(const DispatchBwdArgs& a, hipStream_t st) {
  if (a.E <= 8) return launch_dbwd_t<T, 8, 8>(a, st);
  if (a.E <= 16) return launch_dbwd_t<T, 16, 8>(a, st);
  if (a.E <= 32) return launch_dbwd_t<T, 32, 4>(a, st);
  return launch_dbwd_t<T, 64, 2>(a, st);
}

hipError_t launch_dispatch_bwd(const DispatchBwdArgs& a, bool bf16_dtype, hipStream_t st) {
  return bf16_dtype ? launch_dbwd_dt<bf16>(a, st) : launch_dbwd_dt<float>(a, st);
}

}  // namespace moe
