// Device helpers shared by the grouped-GEMM kernels (internal to libmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "gemm.h"

namespace moe {
namespace gemm_common {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int GM = 8;                      // row-tiles per ordering group
constexpr uint32_t kOOB = 0x7FFFFFF0u;     // an offset beyond every extent
constexpr int64_t kMaxExtent = 0x7FFF0000; // extents stay below kOOB
constexpr int kRsrcWord3 = 0x00020000;     // raw (untyped) buffer, gfx9 family

// A buffer resource over [base, base + bytes): loads at offsets at or past
// the extent return zeros (hardware range check).
struct BufRes {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ void init(const void* base, int64_t bytes) {
    const int64_t n = bytes <= 0 ? 0 : (bytes > kMaxExtent ? kMaxExtent : bytes);
    r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
  }
  __device__ __forceinline__ u32x4 ld(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  }
};

// Workgroup id -> linear tile id such that each XCD's workgroups (dispatched
// round-robin over the 8 XCDs) get consecutive tile ids (bijection).
__device__ __forceinline__ int xcd_remap(int hw, int num) {
  const int q = num >> 3, r = num & 7;
  const int xcd = hw & 7, local = hw >> 3;
  const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  return base + local;
}

// Workgroup id -> linear item id, spreading runs of C consecutive items over
// the XCDs: item run j (items jC .. jC + C - 1) goes whole to XCD j % 8, and
// each XCD takes its runs in order, so the items of a run keep sharing that
// XCD's L2 while consecutive runs (the parts of one group) go to different
// XCDs.  Items past the last whole round of 8 runs fall back to xcd_remap.
// A bijection on [0, n).
__device__ __forceinline__ int run_remap(int hw, int n, int C) {
  const int span = 8 * C;
  const int n0 = n / span * span;
  if (hw >= n0) return n0 + xcd_remap(hw - n0, n - n0);
  const int x = hw & 7, l = hw >> 3;
  const int rho = l / C, off = l - rho * C;
  return (rho * 8 + x) * C + off;
}

// Linear tile id -> (row tile, column tile), walking GM row tiles per column
// so that concurrently running tiles share panels in L2.
__device__ __forceinline__ void grouped_order(int lin, int tiles_m, int tiles_n, int& mt, int& nt, int gm = GM) {
  const int span = gm * tiles_n;
  const int gid = lin / span;
  const int first = gid * gm;
  const int gsz = min(tiles_m - first, gm);
  const int rem = lin - gid * span;
  mt = first + rem % gsz;
  nt = rem / gsz;
}

// Row-split launches size the grid for the largest possible row count, since
// the per-group row counts live on the device.  Each workgroup first counts the
// row tiles the groups really hold; surplus workgroups exit, and the XCD remap
// and the grouped order run over the real tiles only, so the work spreads over
// every XCD whatever the row count.  Returns false for a surplus workgroup.
template <int BM>
__device__ __forceinline__ bool row_tile_of(const gemm::Args& a, int& g, int64_t& row_begin, int64_t& row_end,
                                            int& nt) {
  int real_m = 0;
  for (int gg = 0; gg < a.groups; ++gg) real_m += (int)((a.offsets[gg + 1] - a.offsets[gg] + BM - 1) / BM);
  const int real = real_m * a.tiles_n;
  if ((int)blockIdx.x >= real) return false;
  int mt;
  grouped_order(xcd_remap(blockIdx.x, real), real_m, a.tiles_n, mt, nt, a.gm);
  int acc_t = 0;
  for (int gg = 0; gg < a.groups; ++gg) {
    const int64_t o0 = a.offsets[gg], o1 = a.offsets[gg + 1];
    const int nt_g = (int)((o1 - o0 + BM - 1) / BM);
    if (mt < acc_t + nt_g) {
      g = gg;
      row_begin = o0 + (int64_t)(mt - acc_t) * BM;
      row_end = o1;
      return true;
    }
    acc_t += nt_g;
  }
  return false;
}

__device__ __forceinline__ int weight_index(int g, int rr_R, int rr_L) {
  // send slot g = q * L + l holds expert q + R * l under round-robin placement
  return rr_R > 0 ? (g % rr_L) * rr_R + g / rr_L : g;
}

__device__ __forceinline__ float gelu_f(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_grad_f(float z) {
  return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) +
         z * __expf(-0.5f * z * z) * 0.39894228040143268f;
}
__device__ __forceinline__ float sigmoid_f(float a) { return 1.0f / (1.0f + __expf(-a)); }

// Row of accumulator element e (0..15) of a 32x32 MFMA block for this lane
// (the lane holds column lane % 32).
__device__ __forceinline__ int acc_row(int e, int lane) {
  return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
}

// Tile column of a wave's N-block j.  With SwiGLU pairing the tile's first
// half holds gate columns and the second half the matching up columns; each
// wave takes a gate block and the up block of the same columns, so one lane
// holds both values of a hidden unit.
template <int BN, int WN, int FN, bool PAIR>
__device__ __forceinline__ void block_cols(int wn, int (&bcol)[FN]) {
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if (PAIR)
      bcol[j] = j < FN / 2 ? wn * (FN / 2) * 32 + j * 32 : BN / 2 + wn * (FN / 2) * 32 + (j - FN / 2) * 32;
    else
      bcol[j] = wn * FN * 32 + j * 32;
  }
}

template <typename Kern>
static hipError_t prepare_lds(Kern k, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

// Epilogue of the row-split kernels: rows [row_begin, row_end) of the group,
// output columns n0 + tile column.
template <typename T, int FM, int FN, bool PAIR, int EPI>
__device__ __forceinline__ void rows_epilogue(const gemm::Args& a, f32x16 (&acc)[FM][FN], const int (&bcol)[FN],
                                              int wm0, int lane, int64_t row_begin, int64_t row_end, int64_t n0,
                                              int64_t N) {
  T* C = reinterpret_cast<T*>(a.C);
  T* C2 = reinterpret_cast<T*>(a.C2);
  const T* X1 = reinterpret_cast<const T*>(a.X1);
  const int col = lane & 31;
  if constexpr (PAIR) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const int64_t f = n0 + bcol[j] + col;
        if (f >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t rr = row_begin + wm0 + i * 32 + acc_row(e, lane);
          if (rr >= row_end) continue;
          const float av = acc[i][j][e], bv = acc[i][j + FN / 2][e];
          C[rr * a.ldc + f] = from_f32<T>(av);
          C[rr * a.ldc + a.c_split + f] = from_f32<T>(bv);
          C2[rr * a.ldc2 + f] = from_f32<T>(av * sigmoid_f(av) * bv);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + bcol[j] + col;
        if (n >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t rr = row_begin + wm0 + i * 32 + acc_row(e, lane);
          if (rr >= row_end) continue;
          const float v = acc[i][j][e];
          if constexpr (EPI == gemm::EPI_STORE) {
            C[rr * a.ldc + n] = from_f32<T>(v);
          } else if constexpr (EPI == gemm::EPI_GELU_FWD) {
            C[rr * a.ldc + n] = from_f32<T>(v);
            C2[rr * a.ldc2 + n] = from_f32<T>(gelu_f(v));
          } else if constexpr (EPI == gemm::EPI_GELU_BWD) {
            const float z = to_f32(X1[rr * a.ldx + n]);
            C[rr * a.ldc + n] = from_f32<T>(v * gelu_grad_f(z));
          } else if constexpr (EPI == gemm::EPI_SWIGLU_BWD) {
            const float av = to_f32(X1[rr * a.ldx + n]);
            const float bv = to_f32(X1[rr * a.ldx + a.c_split + n]);
            const float s = sigmoid_f(av);
            C[rr * a.ldc + n] = from_f32<T>(v * bv * s * (1.0f + av * (1.0f - s)));
            C[rr * a.ldc + a.c_split + n] = from_f32<T>(v * av * s);
          }
        }
      }
  }
}

// Epilogue of the wgrad kernels: weight set wi, rows m0 + ..., columns
// n0 + ...; EPI_STORE_SPLITN sends columns >= c_split to C2.
template <typename T, int FM, int FN, int EPI>
__device__ __forceinline__ void wgrad_epilogue(const gemm::Args& a, f32x16 (&acc)[FM][FN], const int (&bcol)[FN],
                                               int wm0, int lane, int wi, int64_t m0, int64_t n0, int64_t M,
                                               int64_t N) {
  T* C = reinterpret_cast<T*>(a.C) + (int64_t)wi * a.c_gstride;
  T* C2 = a.C2 ? reinterpret_cast<T*>(a.C2) + (int64_t)wi * a.c_gstride : nullptr;
  const int col = lane & 31;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + bcol[j] + col;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm0 + i * 32 + acc_row(e, lane);
        if (m >= M) continue;
        const T v = from_f32<T>(acc[i][j][e]);
        if (EPI == gemm::EPI_STORE_SPLITN && n >= a.c_split)
          C2[m * a.ldc + (n - a.c_split)] = v;
        else
          C[m * a.ldc + n] = v;
      }
    }
}

// ---------------------------------------------------------------------------
// Epilogues for accumulators holding C^T blocks (the MFMA called with the
// B fragment first): lane l holds row (l % 32) of a 32x32 block of C and,
// for e = 4g + q, column 8g + 4(l / 32) + q.  So every lane owns four runs of
// 4 consecutive columns of one row, stored (and, for the backward
// activation, loaded) 8 bytes at a time.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tacc_col(int g, int lane) { return 8 * g + 4 * (lane >> 5); }

template <typename T> struct Run4;
template <> struct Run4<bf16> {
  typedef u32x2 Raw;  // the 4 elements as stored
  static __device__ __forceinline__ Raw load_raw(const bf16* p) { return *reinterpret_cast<const u32x2*>(p); }
  static __device__ __forceinline__ void unpack(const Raw& w, float (&v)[4]) {
    v[0] = __uint_as_float(w[0] << 16); v[1] = __uint_as_float(w[0] & 0xffff0000u);
    v[2] = __uint_as_float(w[1] << 16); v[3] = __uint_as_float(w[1] & 0xffff0000u);
  }
  static __device__ __forceinline__ void load(const bf16* p, float (&v)[4]) { unpack(load_raw(p), v); }
  static __device__ __forceinline__ void store(bf16* p, const float (&v)[4]) {
    *reinterpret_cast<u32x2*>(p) = u32x2{bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                                         bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
  }
};
template <> struct Run4<float> {
  typedef f32x4 Raw;
  static __device__ __forceinline__ Raw load_raw(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ void unpack(const Raw& w, float (&v)[4]) {
    v[0] = w[0]; v[1] = w[1]; v[2] = w[2]; v[3] = w[3];
  }
  static __device__ __forceinline__ void load(const float* p, float (&v)[4]) { unpack(load_raw(p), v); }
  static __device__ __forceinline__ void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
};

// Row-split kernels; N and every leading dimension are multiples of 8, so a
// run of 4 columns starting at a multiple of 4 is all in range or all out.
template <typename T, int FM, int FN, int EPI>
__device__ __forceinline__ void rows_epilogue_t_bwd(const gemm::Args& a, f32x16 (&acc)[FM][FN],
                                                    const int (&bcol)[FN], int wm0, int lane, int64_t row_begin,
                                                    int64_t row_end, int64_t n0, int64_t N);

template <typename T, int FM, int FN, bool PAIR, int EPI>
__device__ __forceinline__ void rows_epilogue_t(const gemm::Args& a, f32x16 (&acc)[FM][FN], const int (&bcol)[FN],
                                                int wm0, int lane, int64_t row_begin, int64_t row_end, int64_t n0,
                                                int64_t N) {
  if constexpr (EPI == gemm::EPI_GELU_BWD || EPI == gemm::EPI_SWIGLU_BWD) {
    rows_epilogue_t_bwd<T, FM, FN, EPI>(a, acc, bcol, wm0, lane, row_begin, row_end, n0, N);
    return;
  }
  T* C = reinterpret_cast<T*>(a.C);
  T* C2 = reinterpret_cast<T*>(a.C2);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t rr = row_begin + wm0 + i * 32 + (lane & 31);
    if (rr >= row_end) continue;
    if constexpr (PAIR) {
#pragma unroll
      for (int j = 0; j < FN / 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t f = n0 + bcol[j] + tacc_col(g, lane);
          if (f >= N) continue;
          float av[4], bv[4], hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            av[q] = acc[i][j][4 * g + q];
            bv[q] = acc[i][j + FN / 2][4 * g + q];
            hv[q] = av[q] * sigmoid_f(av[q]) * bv[q];
          }
          Run4<T>::store(C + rr * a.ldc + f, av);
          Run4<T>::store(C + rr * a.ldc + a.c_split + f, bv);
          Run4<T>::store(C2 + rr * a.ldc2 + f, hv);
        }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + bcol[j] + tacc_col(g, lane);
          if (n >= N) continue;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q];
          if constexpr (EPI == gemm::EPI_STORE) {
            Run4<T>::store(C + rr * a.ldc + n, v);
          } else if constexpr (EPI == gemm::EPI_GELU_FWD) {
            float h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = gelu_f(v[q]);
            Run4<T>::store(C + rr * a.ldc + n, v);
            Run4<T>::store(C2 + rr * a.ldc2 + n, h);
          }
        }
    }
  }
}

// The backward activations read X1 (Z, or A | B).  Each lane's loads of one
// 32-row block (FN x 4 runs, two per run for SwiGLU) are issued together and
// one block ahead of the arithmetic; they are unconditional, from the tile's
// first row / column when the run is out of range, and only the stores are
// predicated, so no branch forces a wait on a single load.
template <typename T, int FM, int FN, int EPI>
__device__ __forceinline__ void rows_epilogue_t_bwd(const gemm::Args& a, f32x16 (&acc)[FM][FN],
                                                    const int (&bcol)[FN], int wm0, int lane, int64_t row_begin,
                                                    int64_t row_end, int64_t n0, int64_t N) {
  constexpr bool SW = EPI == gemm::EPI_SWIGLU_BWD;
  constexpr int NL = SW ? 2 : 1;
  T* C = reinterpret_cast<T*>(a.C);
  const T* X1 = reinterpret_cast<const T*>(a.X1);
  typedef typename Run4<T>::Raw Raw;
  Raw xin[2][FN][4][NL];  // two 32-row blocks of raw inputs
  auto load_block = [&](int i, Raw (&dst)[FN][4][NL]) {
    const int64_t rr = row_begin + wm0 + i * 32 + (lane & 31);
    const int64_t r = rr < row_end ? rr : row_begin;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t nn = n0 + bcol[j] + tacc_col(g, lane);
        const int64_t n = nn < N ? nn : n0;
#pragma unroll
        for (int h = 0; h < NL; ++h) dst[j][g][h] = Run4<T>::load_raw(X1 + r * a.ldx + h * a.c_split + n);
      }
  };
  load_block(0, xin[0]);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (i + 1 < FM) load_block(i + 1, xin[(i + 1) & 1]);
    const int64_t rr = row_begin + wm0 + i * 32 + (lane & 31);
    const bool row_ok = rr < row_end;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + bcol[j] + tacc_col(g, lane);
        float x0[4];
        Run4<T>::unpack(xin[i & 1][j][g][0], x0);
        if constexpr (SW) {
          float x1[4];
          Run4<T>::unpack(xin[i & 1][j][g][NL - 1], x1);
          float da[4], db[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float v = acc[i][j][4 * g + q], av = x0[q], bv = x1[q];
            const float sg = sigmoid_f(av);
            da[q] = v * bv * sg * (1.0f + av * (1.0f - sg));
            db[q] = v * av * sg;
          }
          if (row_ok && n < N) {
            Run4<T>::store(C + rr * a.ldc + n, da);
            Run4<T>::store(C + rr * a.ldc + a.c_split + n, db);
          }
        } else {
          float dz[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) dz[q] = acc[i][j][4 * g + q] * gelu_grad_f(x0[q]);
          if (row_ok && n < N) Run4<T>::store(C + rr * a.ldc + n, dz);
        }
      }
  }
}

template <typename T, int FM, int FN, int EPI>
__device__ __forceinline__ void wgrad_epilogue_t(const gemm::Args& a, f32x16 (&acc)[FM][FN], const int (&bcol)[FN],
                                                 int wm0, int lane, int wi, int64_t m0, int64_t n0, int64_t M,
                                                 int64_t N) {
  T* C = reinterpret_cast<T*>(a.C) + (int64_t)wi * a.c_gstride;
  T* C2 = a.C2 ? reinterpret_cast<T*>(a.C2) + (int64_t)wi * a.c_gstride : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm0 + i * 32 + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + bcol[j] + tacc_col(g, lane);
        if (n >= N) continue;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q];
        // c_split is a multiple of 8: a run never straddles it
        if (EPI == gemm::EPI_STORE_SPLITN && n >= a.c_split)
          Run4<T>::store(C2 + m * a.ldc + (n - a.c_split), v);
        else
          Run4<T>::store(C + m * a.ldc + n, v);
      }
  }
}

}  // namespace gemm_common
}  // namespace moe
