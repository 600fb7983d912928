// Grouped expert GEMM launch interface (internal to libmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace gemm {

enum { KIND_FWD = 0, KIND_DGRAD = 1 };
enum {
  EPI_STORE = 0,         // C = acc
  EPI_GELU_FWD = 1,      // Z = acc: C = GELU'(Z), C2 = GELU(Z)
  EPI_SWIGLU_FWD = 2,    // tile pairs gate|up columns A|B: C[:, f] = dH/dA, C[:, c_split+f] = dH/dB, C2 = H = silu(A)*B
  EPI_GELU_BWD = 3,      // X1 = GELU'(Z): C = acc * X1
  EPI_SWIGLU_BWD = 4,    // X1 = [dH/dA | dH/dB]; C[:, f] = dA, C[:, c_split+f] = dB with dH = acc
  EPI_STORE_SPLITN = 5,  // wgrad: columns >= c_split go to C2
  // fused forward (no saved activations; weighted, un-permuted output rows)
  EPI_STORE_SCATTER = 6, // C row scatter[r] = row_scale[scatter[r]] * acc of row r
  EPI_SWIGLU_FWD_H = 7,  // as EPI_SWIGLU_FWD, writing only C2 = silu(A)*B
  EPI_GELU_FWD_H = 8     // as EPI_GELU_FWD, writing only C2 = GELU(Z)
};

struct Args {
  const void* A = nullptr;  int64_t lda = 0;
  const void* B = nullptr;  const void* B2 = nullptr;
  int64_t ldb = 0;          // row stride of B (and B2)
  int64_t b_gstride = 0;    // elements between consecutive weight sets
  int64_t b_split = 0;      // DGRAD: K >= b_split reads B2 at K - b_split
  void* C = nullptr;        void* C2 = nullptr;
  int64_t ldc = 0, ldc2 = 0;
  int64_t c_gstride = 0;    // WGRAD: elements between consecutive weight sets
  int64_t c_split = 0;
  const void* X1 = nullptr; int64_t ldx = 0;
  int64_t M = 0, N = 0, K = 0;
  const int64_t* offsets = nullptr;  // device [groups+1]
  const int64_t* ends = nullptr;     // device [groups] or null: row-split groups own [offsets[g], ends[g])
  int groups = 0;
  int rr_R = 0, rr_L = 1;   // round-robin slot -> expert map (rr_R = 0: identity)
  int tiles_m = 0, tiles_n = 0;
  int gm = 8;               // row tiles per ordering group (L2 reuse of column panels)
  // Row-split A gathered (bf16 direct-load kernels): row r of the group is
  // row gather[r] / gather_k of A, which has gather_rows rows
  const int32_t* gather = nullptr;
  int gather_k = 1;
  int64_t gather_rows = 0;
  // EPI_STORE_SCATTER: output row of row r and its scale index
  const int32_t* scatter = nullptr;
  const float* row_scale = nullptr;
  // WGRAD split over the reduction (bf16 only): ksplit > 1 launches write
  // fp32 partials [ksplit][weight sets][M][N] to `partial`, then summed
  float* partial = nullptr;
  int ksplit = 1;
};

template <typename T>
hipError_t run_rows(int kind, int epi, const Args& a, int64_t rows_max, hipStream_t st);
template <typename T>
hipError_t run_wgrad(int epi, const Args& a, hipStream_t st);

}  // namespace gemm

// bf16 kernels with direct global -> LDS loads (gemm3.hip)
namespace gemm3 {
bool supports(const gemm::Args& a);
// Reduction splits of a bf16 WGRAD launch over `groups` groups of at most
// rows_max rows in total (a function of host-known sizes only, so that the
// workspace can be sized for it): 1 unless the launch has too few tiles.
int wgrad_ksplit(int64_t groups, int64_t M, int64_t N, int64_t rows_max);
hipError_t run_rows_bf16(int kind, int epi, const gemm::Args& a, int64_t rows_max, hipStream_t st);
hipError_t run_wgrad_bf16(int epi, const gemm::Args& a, hipStream_t st);
// bf16 batched transpose: dst[b * dst_bstride + c * rows + r] =
// src[b * src_bstride + r * cols + c] for b < batches, r < rows, c < cols;
// rows and cols multiples of 8, both pointers 16-byte aligned.
hipError_t transpose_bf16(const void* src, void* dst, int64_t batches, int64_t rows, int64_t cols,
                          int64_t src_bstride, int64_t dst_bstride, hipStream_t st);
}  // namespace gemm3
}  // namespace moe
