// Backward of the SwiGLU activation as a bandwidth kernel (tutorial ch.4,
// 专家并行与数据并行的结合 三.3: gradients flow back through the experts).
//
// With H = silu(A) * B and dH given:
//   dA = dH * B * s * (1 + A (1 - s)),  s = sigmoid(A)
//   dB = dH * silu(A)
// d_act [rows, 2F] holds dH in its first F columns on entry and [dA | dB] on
// exit (in place: every element is read and then written by one thread);
// act [rows, 2F] is the saved [A | B].  Only rows below the kept-row count
// offsets[groups] (read on the device) are touched.  Each access moves 16
// bytes (8 bf16 or 4 fp32 columns).
#include "common.h"
#include "kernels.h"

namespace moe {

// A workgroup walks blocks of RB consecutive rows (grid-stride over row
// blocks), RB chosen on the host so that a block holds at least 256 U chunks
// when rows are short.  Per round a thread takes U chunks f = tid + 256 k of
// the block (row f / cpr, chunk f % cpr) and issues all their loads before any
// arithmetic or store.
template <typename T, int U>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(T* __restrict__ d_act, const T* __restrict__ act,
                                                         const int64_t* __restrict__ offsets, int groups,
                                                         int64_t F, int RB) {
  constexpr int V = Vec16<T>::N;
  const int64_t rows = offsets[groups];
  const uint32_t cpr = (uint32_t)(F / V);  // chunks per row (F is a multiple of 8)
  for (int64_t r0 = (int64_t)blockIdx.x * RB; r0 < rows; r0 += (int64_t)gridDim.x * RB) {
    T* dr = d_act + r0 * 2 * F;
    const T* ar = act + r0 * 2 * F;
    const uint32_t n = (uint32_t)min((int64_t)RB, rows - r0) * cpr;
    for (uint32_t f0 = threadIdx.x; f0 < n; f0 += 256 * U) {
      int64_t off[U];
      u32x4 h[U], a[U], b[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        // chunks past the block load its first chunk and store nothing
        const uint32_t f = f0 + 256 * k < n ? f0 + 256 * k : 0;
        const uint32_t row = f / cpr, col = f - row * cpr;
        off[k] = (int64_t)row * 2 * F + col * V;
        h[k] = ld16(dr + off[k]);
        a[k] = ld16(ar + off[k]);
        b[k] = ld16(ar + off[k] + F);
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        float dh[V], av[V], bv[V], da[V], db[V];
        unpack16<T>(h[k], dh);
        unpack16<T>(a[k], av);
        unpack16<T>(b[k], bv);
#pragma unroll
        for (int q = 0; q < V; ++q) {
          const float s = 1.0f / (1.0f + __expf(-av[q]));
          da[q] = dh[q] * bv[q] * s * (1.0f + av[q] * (1.0f - s));
          db[q] = dh[q] * av[q] * s;
        }
        if (f0 + 256 * k < n) {
          st16(dr + off[k], pack16<T>(da));
          st16(dr + off[k] + F, pack16<T>(db));
        }
      }
    }
  }
}

template <typename T>
static void launch_swiglu_bwd_t(T* d_act, const T* act, const int64_t* offsets, int groups, int64_t rows_max,
                                int64_t F, hipStream_t st) {
  const int64_t cpr = F / Vec16<T>::N;
  const int U = cpr > 512 ? 4 : 2;
  const int64_t RB = cpr >= 256 * U ? 1 : (256 * U) / cpr;  // rows per block
  int64_t blocks = (rows_max + RB - 1) / RB;
  if (blocks > 8192) blocks = 8192;  // row blocks beyond: grid-stride
  if (U == 4)
    hipLaunchKernelGGL((swiglu_bwd_kernel<T, 4>), dim3((unsigned)blocks), dim3(256), 0, st, d_act, act, offsets,
                       groups, F, (int)RB);
  else
    hipLaunchKernelGGL((swiglu_bwd_kernel<T, 2>), dim3((unsigned)blocks), dim3(256), 0, st, d_act, act, offsets,
                       groups, F, (int)RB);
}

hipError_t launch_swiglu_bwd(void* d_act, const void* act, const int64_t* offsets, int groups, int64_t rows_max,
                             int64_t F, bool bf16_dtype, hipStream_t st) {
  if (rows_max <= 0 || F <= 0) return hipSuccess;
  if (F / (bf16_dtype ? 8 : 4) > (1 << 20)) return hipErrorInvalidValue;  // chunk indices stay 32-bit
  if (bf16_dtype)
    launch_swiglu_bwd_t<bf16>((bf16*)d_act, (const bf16*)act, offsets, groups, rows_max, F, st);
  else
    launch_swiglu_bwd_t<float>((float*)d_act, (const float*)act, offsets, groups, rows_max, F, st);
  return hipGetLastError();
}

}  // namespace moe
