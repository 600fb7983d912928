// Device helpers shared by the grouped-GEMM kernels (internal to libmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "gemm.h"
#include "gemm_addr.h"

namespace moe {
namespace gemm_common {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int GM = 8;                      // row-tiles per ordering group
constexpr int kRsrcWord3 = 0x00020000;     // raw (untyped) buffer, gfx9 family

// Tile order, load offsets and resource spans: gemm_addr.h (shared with the
// host-side address checker).
using gemm_addr::grouped_order;
using gemm_addr::kMaxExtent;
using gemm_addr::kMaxRowBytes;
using gemm_addr::kOOB;
using gemm_addr::run_remap;
using gemm_addr::Span;
using gemm_addr::weight_index;
using gemm_addr::xcd_remap;

// A buffer resource over [base, base + bytes): loads at offsets at or past
// the extent return zeros (hardware range check).  Every resource the GEMM
// kernels build spans at most 256 rows of one operand (a row tile, a tile of
// K-contiguous weights) or one K stage of an M/N-contiguous operand (rebased
// at every stage, stage_res below), so its extent is bounded by the row width
// alone; the host rejects rows wider than kMaxRowBytes, which keeps every
// extent below kMaxExtent whatever the number of rows.  The clamp is a last
// guard only.
struct BufRes {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ void init(const void* base, int64_t bytes) {
    const int64_t n = bytes <= 0 ? 0 : (bytes > kMaxExtent ? kMaxExtent : bytes);
    r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
  }
  // the span's bytes of the operand at ptr
  __device__ __forceinline__ void init(const void* ptr, const Span& s) {
    init(reinterpret_cast<const char*>(ptr) + s.base, s.bytes);
  }
  __device__ __forceinline__ u32x4 ld(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  }
};

// Resource over K rows [k0, min(k0 + rows, K)) of an operand whose K row k
// starts k * ld_bytes after `first` (which already points at the tile's first
// column, col0_bytes into each row): loads at byte (k - k0) * ld_bytes + c
// read row k, and rows at or past K (or past the stage) read zeros.  Built at
// every K stage (register-staged kernels of gemm.hip), so offsets stay within
// one stage however many rows the operand holds.
__device__ __forceinline__ BufRes stage_res(const char* first, int64_t k0, int64_t rows, int64_t K, int64_t ld_bytes,
                                            int64_t col0_bytes) {
  BufRes b;
  b.init(first + k0 * ld_bytes, (K - k0 < rows ? K - k0 : rows) * ld_bytes - col0_bytes);
  return b;
}

// The stages of an M/N-contiguous operand of the direct-to-LDS kernels,
// walked in order: each call of next() gives the resource of the next stage
// (gemm_addr::stage_span of stage 0, 1, ...), advancing the base by one
// stride, with the extent clamped once.
struct StageRes {
  const char* base;
  int64_t stride;
  int bytes;
  __device__ __forceinline__ void init(const void* ptr, const gemm_addr::StageWalk& w) {
    base = reinterpret_cast<const char*>(ptr) + w.first;
    stride = w.stride;
    bytes = (int)(w.bytes <= 0 ? 0 : (w.bytes > kMaxExtent ? kMaxExtent : w.bytes));
  }
  __device__ __forceinline__ BufRes next() {
    BufRes b;
    b.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, kRsrcWord3);
    base += stride;
    return b;
  }
};

// Device side of gemm_addr::row_tile_of over the launch's group table: the
// same walk (the same tile for every workgroup), with the table read 64
// groups per wave-wide load, the per-group tile counts summed by an inclusive
// scan over the lanes and the group found by a ballot.  The host form's loops
// take two dependent loads per group; on the device that cost every
// workgroup 2.4-3.3 us for 8 groups before its first K stage was issued.
__device__ __forceinline__ int wave_incl_scan_i32(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}
__device__ __forceinline__ int64_t lane_i64(int64_t v, int pos) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, pos);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), pos);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <int BM>
__device__ __forceinline__ bool row_tile_of(const gemm::Args& a, int& g, int64_t& row_begin, int64_t& row_end,
                                            int& nt) {
  const int lane = (int)(threadIdx.x & 63);
  const int hw = (int)blockIdx.x;
  auto load = [&](int gg, int64_t& o0, int64_t& o1) {
    o0 = 0;
    o1 = 0;
    if (gg < a.groups) {
      o0 = a.offsets[gg];
      o1 = gemm_addr::group_end(a.offsets, a.ends, gg);
    }
  };
  // tiles of group c + lane (0 past the last group) and the inclusive sum
  // over the chunk's lanes up to it; one group needs no scan
  auto chunk = [&](int c, int64_t& o0, int64_t& o1, int& nt_g, int& cnt, int& incl) {
    load(c + lane, o0, o1);
    nt_g = (int)((o1 - o0 + BM - 1) / BM);
    cnt = nt_g * a.tiles_n;
    incl = a.groups == 1 ? cnt : wave_incl_scan_i32(cnt, lane);
  };
  // the group holding linear tile lin, found among the chunk's lanes: the
  // first group gg with lin < (tiles before gg) + cnt, as the walk in order
  // finds it
  auto take = [&](int c, int acc_t, int lin, int64_t o0, int64_t o1, int nt_g, int cnt, int incl) -> bool {
    const uint64_t hit = __ballot(c + lane < a.groups && lin < acc_t + incl);
    if (!hit) return false;
    const int pos = __ffsll((unsigned long long)hit) - 1;
    const int ntg = __builtin_amdgcn_readlane(nt_g, pos);
    const int before = acc_t + __builtin_amdgcn_readlane(incl, pos) - __builtin_amdgcn_readlane(cnt, pos);
    const int bands = (ntg + a.gm - 1) / a.gm;
    const int band_m = (ntg + bands - 1) / bands;
    int mt;
    gemm_addr::grouped_order(lin - before, ntg, a.tiles_n, mt, nt, band_m);
    g = c + pos;
    row_begin = lane_i64(o0, pos) + (int64_t)mt * BM;
    row_end = lane_i64(o1, pos);
    return true;
  };
  int64_t o0, o1;
  int nt_g, cnt, incl;
  chunk(0, o0, o1, nt_g, cnt, incl);
  if (a.groups <= 64) {  // one chunk: the last group's sum is the total
    const int real = __builtin_amdgcn_readlane(incl, a.groups - 1);
    if (hw >= real) return false;
    return take(0, 0, gemm_addr::xcd_remap(hw, real), o0, o1, nt_g, cnt, incl);
  }
  int real = __builtin_amdgcn_readlane(incl, 63);
  for (int c = 64; c < a.groups; c += 64) {
    int64_t p0, p1;
    int a1, a2, a3;
    chunk(c, p0, p1, a1, a2, a3);
    real += __builtin_amdgcn_readlane(a3, 63);
  }
  if (hw >= real) return false;
  const int lin = gemm_addr::xcd_remap(hw, real);
  int acc_t = 0;
  for (int c = 0; c < a.groups; c += 64) {
    if (c > 0) chunk(c, o0, o1, nt_g, cnt, incl);
    if (take(c, acc_t, lin, o0, o1, nt_g, cnt, incl)) return true;
    acc_t += __builtin_amdgcn_readlane(incl, 63);
  }
  return false;
}

// Phi(z) = (1 + erf(z / sqrt 2)) / 2, the normal distribution function, from
// erfc of u = |z| / sqrt 2: erfc(u) = t exp(-u^2 + P(t)) with t = 1 / (1 +
// u / 2) and P the degree-9 Chebyshev fit published with this form in
// Numerical Recipes (Press, Teukolsky, Vetterling and Flannery, 2nd ed.,
// section 6.2), whose fractional error stays below 1.2e-7 for every u >= 0.
// Written in z for the hardware 2^x: the exponent is log2(e) (P(t) - u^2) - 1
// (the -1 takes the halving), with log2(e) folded into P's coefficients, and
// w = log2(e) z^2 / 2 is returned for GELU', whose Gaussian term is 2^-w.
// For z < 0 the result is erfc itself, free of the cancellation in 1 + erf.
// One reciprocal, one exponential and eleven multiply-adds, without the range
// branches of a general erff: the GELU epilogues run it once per element.
__device__ __forceinline__ float phi_f(float z, float& w) {
  constexpr float kL2e = 1.4426950408889634f;
  const float a = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.35355339059327373f, a, 1.0f));  // 1 / (1 + u / 2)
  float p = 0.17087277f * kL2e;
  p = fmaf(p, t, -0.82215223f * kL2e);
  p = fmaf(p, t, 1.48851587f * kL2e);
  p = fmaf(p, t, -1.13520398f * kL2e);
  p = fmaf(p, t, 0.27886807f * kL2e);
  p = fmaf(p, t, -0.18628806f * kL2e);
  p = fmaf(p, t, 0.09678418f * kL2e);
  p = fmaf(p, t, 0.37409196f * kL2e);
  p = fmaf(p, t, 1.00002368f * kL2e);
  p = fmaf(p, t, -1.26551223f * kL2e - 1.0f);
  w = (0.5f * kL2e * z) * z;
  const float h = t * __builtin_amdgcn_exp2f(p - w);  // erfc(u) / 2
  return z >= 0.0f ? 1.0f - h : h;
}
__device__ __forceinline__ float gelu_f(float z) {
  float w;
  return z * phi_f(z, w);
}
// the hardware reciprocal (1 ulp) in place of a correctly rounded division,
// whose scale / fix-up sequence the SwiGLU epilogues would run per element
__device__ __forceinline__ float sigmoid_f(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// Forward activations together with the factor that their backward
// multiplies dL/dh by, which the forward saves in place of the
// pre-activations: the backward epilogue is then one product per element
// instead of a second evaluation of Phi or the sigmoid.
//   GELU:   h = z Phi(z),   d = dh/dz = Phi(z) + z exp(-z^2 / 2) / sqrt(2 pi)
//   SwiGLU: h = silu(a) b,  d1 = dh/da = b s (1 + a (1 - s)),  d2 = dh/db = silu(a)
// with s = sigmoid(a); h is formed exactly as without the factors.
__device__ __forceinline__ float gelu_fwd_save(float z, float& d) {
  float w;
  const float ph = phi_f(z, w);
  d = fmaf(z * 0.3989422804014327f, __builtin_amdgcn_exp2f(-w), ph);
  return z * ph;
}
__device__ __forceinline__ float swiglu_fwd_save(float a, float b, float& d1, float& d2) {
  const float s = sigmoid_f(a);
  d2 = a * s;
  d1 = b * s * fmaf(a, 1.0f - s, 1.0f);
  return d2 * b;
}

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
          float d1, d2;
          const float hv = swiglu_fwd_save(acc[i][j][e], acc[i][j + FN / 2][e], d1, d2);
          C[rr * a.ldc + f] = from_f32<T>(d1);
          C[rr * a.ldc + a.c_split + f] = from_f32<T>(d2);
          C2[rr * a.ldc2 + f] = from_f32<T>(hv);
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
            float dv;
            const float hv = gelu_fwd_save(v, dv);
            C[rr * a.ldc + n] = from_f32<T>(dv);
            C2[rr * a.ldc2 + n] = from_f32<T>(hv);
          } else if constexpr (EPI == gemm::EPI_GELU_BWD) {
            C[rr * a.ldc + n] = from_f32<T>(v * to_f32(X1[rr * a.ldx + n]));
          } else if constexpr (EPI == gemm::EPI_SWIGLU_BWD) {
            C[rr * a.ldc + n] = from_f32<T>(v * to_f32(X1[rr * a.ldx + n]));
            C[rr * a.ldc + a.c_split + n] = from_f32<T>(v * to_f32(X1[rr * a.ldx + a.c_split + n]));
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
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]),
                                         pack_bf16x2(v[2], v[3])};
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
          float d1[4], d2[4], hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            hv[q] = swiglu_fwd_save(acc[i][j][4 * g + q], acc[i][j + FN / 2][4 * g + q], d1[q], d2[q]);
          Run4<T>::store(C + rr * a.ldc + f, d1);
          Run4<T>::store(C + rr * a.ldc + a.c_split + f, d2);
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
            float dv[4], h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = gelu_fwd_save(v[q], dv[q]);
            Run4<T>::store(C + rr * a.ldc + n, dv);
            Run4<T>::store(C2 + rr * a.ldc2 + n, h);
          }
        }
    }
  }
}

// The backward activations read X1 (the saved factor dh/dz, or dh/da | dh/db)
// and multiply the accumulators by it.  Each lane's loads of one
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
            da[q] = acc[i][j][4 * g + q] * x0[q];
            db[q] = acc[i][j][4 * g + q] * x1[q];
          }
          if (row_ok && n < N) {
            Run4<T>::store(C + rr * a.ldc + n, da);
            Run4<T>::store(C + rr * a.ldc + a.c_split + n, db);
          }
        } else {
          float dz[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) dz[q] = acc[i][j][4 * g + q] * x0[q];
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
