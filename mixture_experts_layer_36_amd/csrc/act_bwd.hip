// Backward of the SwiGLU activation as a bandwidth kernel (tutorial ch.4,
// 专家并行与数据并行的结合 三.3: gradients flow back through the experts).
//
// With H = silu(A) * B and dH given:
//   dA = dH * B * s * (1 + A (1 - s)),  s = sigmoid(A)
//   dB = dH * silu(A)
// d_act [rows, 2F] holds dH in its first F columns on entry and [dA | dB] on
// exit (in place: every element is read and then written by one thread);
// act [rows, 2F] is the saved [A | B].  Only rows below the kept-row count
// offsets[groups] (read on the device) are touched.  Each thread moves 8
// consecutive columns of one row with 16-byte accesses.
#include "common.h"
#include "kernels.h"

namespace moe {

template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(T* __restrict__ d_act, const T* __restrict__ act,
                                                         const int64_t* __restrict__ offsets, int groups,
                                                         int64_t F) {
  constexpr int V = Vec16<T>::N;
  const int64_t rows = offsets[groups];
  const int64_t cpr = F / V;  // chunks per row (F is a multiple of 8)
  const int64_t total = rows * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cpr, c = (i - r * cpr) * V;
    T* dr = d_act + r * 2 * F;
    const T* ar = act + r * 2 * F;
    float dh[V], av[V], bv[V], da[V], db[V];
    unpack16<T>(ld16(dr + c), dh);
    unpack16<T>(ld16(ar + c), av);
    unpack16<T>(ld16(ar + F + c), bv);
#pragma unroll
    for (int q = 0; q < V; ++q) {
      const float s = 1.0f / (1.0f + __expf(-av[q]));
      da[q] = dh[q] * bv[q] * s * (1.0f + av[q] * (1.0f - s));
      db[q] = dh[q] * av[q] * s;
    }
    st16(dr + c, pack16<T>(da));
    st16(dr + F + c, pack16<T>(db));
  }
}

hipError_t launch_swiglu_bwd(void* d_act, const void* act, const int64_t* offsets, int groups, int64_t rows_max,
                             int64_t F, bool bf16_dtype, hipStream_t st) {
  const int64_t chunks = rows_max * (F / (bf16_dtype ? 8 : 4));
  if (chunks <= 0) return hipSuccess;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond
  if (bf16_dtype)
    hipLaunchKernelGGL((swiglu_bwd_kernel<bf16>), dim3((unsigned)blocks), dim3(256), 0, st, (bf16*)d_act,
                       (const bf16*)act, offsets, groups, F);
  else
    hipLaunchKernelGGL((swiglu_bwd_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, st, (float*)d_act,
                       (const float*)act, offsets, groups, F);
  return hipGetLastError();
}

}  // namespace moe
