// Grouped expert GEMMs on the MFMA matrix cores (gfx950).
//
// The expert FFN is the dense contraction of the MoE layer (tutorial ch.4,
// 专家并行 二 step 3: each device runs its local experts on the tokens it
// received; 专家并行与数据并行的结合 三.3: expert parameter gradients are
// computed locally).  Every expert is a GEMM over its own row segment, so
// one launch covers all experts ("groups") and reads the segment bounds from
// a device array: no host synchronisation is needed after the dispatch.
//
// Three kinds of launch:
//   FWD   C[rows, N]  = A[rows, K] . W_g[K, N]      (W row-major, N contiguous)
//   DGRAD C[rows, N]  = A[rows, K] . W_g[N, K]^T    (W row-major, K contiguous)
//   WGRAD C_g[M, N]   = X[rows_g, M]^T . D[rows_g, N]  (reduction over the
//                       group's rows: ragged K; no rows -> exact zeros)
// FWD and DGRAD split M (rows) by group; WGRAD splits K.
//
// Tiling.  A workgroup of 256 threads (4 waves, 2 x 2) computes a BM x BN
// tile with v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2f32 (fp32),
// fp32 accumulation.  Each K stage moves 128 bytes of K per tile row (64 bf16
// or 32 fp32) through LDS, double buffered with one barrier per stage; the
// next stage's global loads are in flight while the current one is
// multiplied.  LDS rows are K-contiguous (what an MFMA lane consumes: 16 bytes
// of consecutive K) with an XOR swizzle of the 16-byte chunk index so that
// both the fragment reads and the transposing writes spread over the banks.
// Operands whose global layout is M- or N-contiguous (forward weights,
// wgrad activations) are loaded as 4(K) x 16-byte blocks and transposed in
// registers on their way into LDS.
//
// Tile order: hardware dispatches consecutive workgroups round-robin over
// the 8 XCDs, each with its own L2; the linear tile id is remapped so that
// the tiles one XCD runs are consecutive, then tiles are walked in groups of
// GM row-tiles so that concurrently running tiles share weight and
// activation panels in that XCD's L2.
#include "common.h"
#include "gemm.h"

namespace moe {
namespace gemm {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NT = 256;
constexpr int ROWB = 128;     // bytes of K per LDS row per stage
constexpr int GM = 8;         // row-tiles per ordering group

__device__ __forceinline__ int swz(int row, int ch) {
  return ch ^ ((row ^ (row >> 3)) & 7);
}

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static __device__ __forceinline__ void run(f32x16& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x16& c, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
  }
};

// Workgroup id -> linear tile id such that each XCD's workgroups get
// consecutive tile ids (bijection on [0, num)).
__device__ __forceinline__ int xcd_remap(int hw, int num) {
  const int q = num >> 3, r = num & 7;
  const int xcd = hw & 7, local = hw >> 3;
  const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  return base + local;
}

__device__ __forceinline__ void grouped_order(int lin, int tiles_m, int tiles_n, int& mt, int& nt) {
  const int span = GM * tiles_n;
  const int gid = lin / span;
  const int first = gid * GM;
  const int gsz = min(tiles_m - first, GM);
  const int rem = lin - gid * span;
  mt = first + rem % gsz;
  nt = rem / gsz;
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

// Transpose a 4(K) x V(MN) register block (4 x 16 bytes) into V rows of 4 K
// elements and write them to LDS.
template <typename T>
__device__ __forceinline__ void write_transposed(char* lds, int row0, int kq, const u32x4 (&v)[4]);

template <>
__device__ __forceinline__ void write_transposed<bf16>(char* lds, int row0, int kq, const u32x4 (&v)[4]) {
  // kq: index of the 4-element K group (0..15); chunk = kq/2, half = kq&1
  const int ch = kq >> 1, half = kq & 1;
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
    const int dw = mm >> 1;
    u32x2 o;
    if (mm & 1) {
      o[0] = (v[0][dw] >> 16) | (v[1][dw] & 0xffff0000u);
      o[1] = (v[2][dw] >> 16) | (v[3][dw] & 0xffff0000u);
    } else {
      o[0] = (v[0][dw] & 0xffffu) | (v[1][dw] << 16);
      o[1] = (v[2][dw] & 0xffffu) | (v[3][dw] << 16);
    }
    const int row = row0 + mm;
    *reinterpret_cast<u32x2*>(lds + row * ROWB + (swz(row, ch) << 4) + half * 8) = o;
  }
}

template <>
__device__ __forceinline__ void write_transposed<float>(char* lds, int row0, int kq, const u32x4 (&v)[4]) {
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
    u32x4 o;
    o[0] = v[0][mm]; o[1] = v[1][mm]; o[2] = v[2][mm]; o[3] = v[3][mm];
    const int row = row0 + mm;
    *reinterpret_cast<u32x4*>(lds + row * ROWB + (swz(row, kq) << 4)) = o;
  }
}

// ---------------------------------------------------------------------------
// Operand tile loaders.  A tile operand covers R rows (M or N) x 128 bytes of K.
// K-contiguous source: R*8 16-byte chunks, R/32 per thread.
// MN-contiguous source: 2R blocks of 4 K-rows x 16 bytes, R/128 per thread.
// ---------------------------------------------------------------------------
template <typename T, int R>
struct KLoader {
  static constexpr int PER = R / 32;
  u32x4 r[PER];
  // src(row, k) returns a pointer or nullptr (-> zeros); k is an element index
  template <typename Src>
  __device__ __forceinline__ void load(const Src& src, int k0) {
    constexpr int V = Vec16<T>::N;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = threadIdx.x + NT * i;
      const int row = q >> 3, ch = q & 7;
      const T* p = src(row, k0 + ch * V);
      r[i] = p ? ld16(p) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = threadIdx.x + NT * i;
      const int row = q >> 3, ch = q & 7;
      *reinterpret_cast<u32x4*>(lds + row * ROWB + (swz(row, ch) << 4)) = r[i];
    }
  }
};

template <typename T, int R>
struct MNLoader {
  static constexpr int V = Vec16<T>::N;
  static constexpr int PER = R / 128;
  static constexpr int NB = R / V;        // 16-byte blocks along MN per K row
  u32x4 r[PER][4];
  // src(k, mn) returns a pointer to 16 bytes (V elements along MN) or nullptr
  template <typename Src>
  __device__ __forceinline__ void load(const Src& src, int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = threadIdx.x + NT * i;
      const int kq = q / NB, nb = q % NB;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const T* p = src(k0 + kq * 4 + kk, nb * V);
        r[i][kk] = p ? ld16(p) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = threadIdx.x + NT * i;
      const int kq = q / NB, nb = q % NB;
      write_transposed<T>(lds, nb * V, kq, r[i]);
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA over one LDS stage for a wave's (BM/2) x (BN/2) sub-tile.
// ---------------------------------------------------------------------------
template <typename T, int FM, int FN>
__device__ __forceinline__ void mma_stage(const char* la, const char* lb, int wm0, const int (&bcol)[FN],
                                          f32x16 (&acc)[FM][FN]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, g = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int ch = 2 * s + g;
    u32x4 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm0 + i * 32 + r;
      af[i] = *reinterpret_cast<const u32x4*>(la + row * ROWB + (swz(row, ch) << 4));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = bcol[j] + r;
      bfr[j] = *reinterpret_cast<const u32x4*>(lb + row * ROWB + (swz(row, ch) << 4));
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) Mma<T>::run(acc[i][j], af[i], bfr[j]);
  }
}

// Row of accumulator element e (0..15) of a 32x32 block for this lane.
__device__ __forceinline__ int acc_row(int e, int lane) {
  return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
}

// ---------------------------------------------------------------------------
// FWD / DGRAD: rows split by group.
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int KIND, int EPI>
__global__ __launch_bounds__(NT) void gemm_rows_kernel(Args a) {
  constexpr int FM = BM / 64, FN = BN / 64;
  constexpr int V = Vec16<T>::N;
  constexpr int BKE = ROWB / sizeof(T);
  constexpr bool SWIGLU_PAIR = (EPI == EPI_SWIGLU_FWD);
  __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * ROWB];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  int mt, nt;
  grouped_order(lin, a.tiles_m, a.tiles_n, mt, nt);
  if (mt >= a.tiles_m) return;
  // m-tile -> group
  int g = -1;
  int64_t row_begin = 0, row_end = 0;
  {
    int acc_t = 0;
    for (int gg = 0; gg < a.groups; ++gg) {
      const int64_t o0 = a.offsets[gg], o1 = a.offsets[gg + 1];
      const int nt_g = (int)((o1 - o0 + BM - 1) / BM);
      if (mt < acc_t + nt_g) {
        g = gg;
        row_begin = o0 + (int64_t)(mt - acc_t) * BM;
        row_end = o1;
        break;
      }
      acc_t += nt_g;
    }
  }
  if (g < 0) return;
  const int wi = weight_index(g, a.rr_R, a.rr_L);
  const int64_t K = a.K;
  const int64_t N = a.N;

  const T* Ab = reinterpret_cast<const T*>(a.A);
  const T* Bg = reinterpret_cast<const T*>(a.B) + (int64_t)wi * a.b_gstride;
  const T* B2g = a.B2 ? reinterpret_cast<const T*>(a.B2) + (int64_t)wi * a.b_gstride : nullptr;

  // tile column c -> weight column (and which weight for the SwiGLU pairing)
  const int64_t n0 = SWIGLU_PAIR ? (int64_t)nt * (BN / 2) : (int64_t)nt * BN;

  auto a_src = [&](int row, int k) -> const T* {
    const int64_t rr = row_begin + row;
    if (rr >= row_end || k >= K) return nullptr;
    return Ab + rr * a.lda + k;
  };

  KLoader<T, BM> la_ld;
  KLoader<T, BN> lbk_ld;   // DGRAD: weights K-contiguous
  MNLoader<T, BN> lbn_ld;  // FWD: weights N-contiguous

  auto b_src_n = [&](int k, int c) -> const T* {   // FWD: element (k, tile col c..c+V)
    if (k >= K) return nullptr;
    if (SWIGLU_PAIR) {
      const int half = c >= BN / 2;
      const int64_t f = n0 + (half ? c - BN / 2 : c);
      if (f >= N) return nullptr;
      return (half ? B2g : Bg) + (int64_t)k * a.ldb + f;
    }
    const int64_t n = n0 + c;
    if (n >= N) return nullptr;
    return Bg + (int64_t)k * a.ldb + n;
  };
  auto b_src_k = [&](int c, int k) -> const T* {   // DGRAD: element (tile col c, k..k+V)
    const int64_t n = n0 + c;
    if (n >= N || k >= K) return nullptr;
    if (a.b_split > 0 && k >= a.b_split) return B2g + n * a.ldb + (k - a.b_split);
    return Bg + n * a.ldb + k;
  };

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm0 = (wave >> 1) * (BM / 2);
  const int wn = wave & 1;
  int bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if (SWIGLU_PAIR)
      bcol[j] = j < FN / 2 ? wn * (BN / 4) + j * 32 : BN / 2 + wn * (BN / 4) + (j - FN / 2) * 32;
    else
      bcol[j] = wn * (BN / 2) + j * 32;
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (int)((K + BKE - 1) / BKE);
  la_ld.load(a_src, 0);
  if (KIND == KIND_FWD) lbn_ld.load(b_src_n, 0); else lbk_ld.load(b_src_k, 0);
  for (int kt = 0; kt < nk; ++kt) {
    char* sa = smem + (kt & 1) * (BM + BN) * ROWB;
    char* sb = sa + BM * ROWB;
    la_ld.store(sa);
    if (KIND == KIND_FWD) lbn_ld.store(sb); else lbk_ld.store(sb);
    __syncthreads();
    if (kt + 1 < nk) {
      const int k0 = (kt + 1) * BKE;
      la_ld.load(a_src, k0);
      if (KIND == KIND_FWD) lbn_ld.load(b_src_n, k0); else lbk_ld.load(b_src_k, k0);
    }
    mma_stage<T, FM, FN>(sa, sb, wm0, bcol, acc);
  }

  // ---------------------------------------------------------------- epilogue
  T* C = reinterpret_cast<T*>(a.C);
  T* C2 = reinterpret_cast<T*>(a.C2);
  const T* X1 = reinterpret_cast<const T*>(a.X1);
  const int col = lane & 31;
  if constexpr (SWIGLU_PAIR) {
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
          if constexpr (EPI == EPI_STORE) {
            C[rr * a.ldc + n] = from_f32<T>(v);
          } else if constexpr (EPI == EPI_GELU_FWD) {
            C[rr * a.ldc + n] = from_f32<T>(v);
            C2[rr * a.ldc2 + n] = from_f32<T>(gelu_f(v));
          } else if constexpr (EPI == EPI_GELU_BWD) {
            const float z = to_f32(X1[rr * a.ldx + n]);
            C[rr * a.ldc + n] = from_f32<T>(v * gelu_grad_f(z));
          } else if constexpr (EPI == EPI_SWIGLU_BWD) {
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

// ---------------------------------------------------------------------------
// WGRAD: C_g[M, N] = X[rows_g, M]^T . D[rows_g, N]; both operands are
// MN-contiguous in memory.  EPI_STORE or EPI_STORE_SPLITN (columns >= c_split
// go to C2 at column - c_split).
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int EPI>
__global__ __launch_bounds__(NT) void gemm_wgrad_kernel(Args a) {
  constexpr int FM = BM / 64, FN = BN / 64;
  constexpr int BKE = ROWB / sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * ROWB];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = a.tiles_m * a.tiles_n;
  const int g = lin / per_g;
  if (g >= a.groups) return;
  int mt, nt;
  grouped_order(lin - g * per_g, a.tiles_m, a.tiles_n, mt, nt);
  const int wi = weight_index(g, a.rr_R, a.rr_L);
  const int64_t r0 = a.offsets[g], r1 = a.offsets[g + 1];
  const int64_t Kr = r1 - r0;
  const int64_t M = a.M, N = a.N;
  const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;

  const T* X = reinterpret_cast<const T*>(a.A);
  const T* D = reinterpret_cast<const T*>(a.B);
  auto a_src = [&](int k, int m) -> const T* {
    if (k >= Kr || m0 + m >= M) return nullptr;
    return X + (r0 + k) * a.lda + m0 + m;
  };
  auto b_src = [&](int k, int n) -> const T* {
    if (k >= Kr || n0 + n >= N) return nullptr;
    return D + (r0 + k) * a.ldb + n0 + n;
  };
  MNLoader<T, BM> la_ld;
  MNLoader<T, BN> lb_ld;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm0 = (wave >> 1) * (BM / 2);
  const int wn = wave & 1;
  int bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) bcol[j] = wn * (BN / 2) + j * 32;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (int)((Kr + BKE - 1) / BKE);
  if (nk > 0) {
    la_ld.load(a_src, 0);
    lb_ld.load(b_src, 0);
  }
  for (int kt = 0; kt < nk; ++kt) {
    char* sa = smem + (kt & 1) * (BM + BN) * ROWB;
    char* sb = sa + BM * ROWB;
    la_ld.store(sa);
    lb_ld.store(sb);
    __syncthreads();
    if (kt + 1 < nk) {
      la_ld.load(a_src, (kt + 1) * BKE);
      lb_ld.load(b_src, (kt + 1) * BKE);
    }
    mma_stage<T, FM, FN>(sa, sb, wm0, bcol, acc);
  }

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
        if (EPI == EPI_STORE_SPLITN && n >= a.c_split)
          C2[m * a.ldc + (n - a.c_split)] = v;
        else
          C[m * a.ldc + n] = v;
      }
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int KIND, int EPI>
static hipError_t launch_rows(Args a, int64_t rows_max, hipStream_t st) {
  const int tiles_n_cols = EPI == EPI_SWIGLU_FWD ? BN / 2 : BN;
  a.tiles_n = (int)((a.N + tiles_n_cols - 1) / tiles_n_cols);
  a.tiles_m = (int)((rows_max + BM - 1) / BM) + a.groups;
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_rows_kernel<T, BM, BN, KIND, EPI>), dim3((unsigned)grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <typename T, int BM, int BN, int EPI>
static hipError_t launch_wgrad(Args a, hipStream_t st) {
  a.tiles_m = (int)((a.M + BM - 1) / BM);
  a.tiles_n = (int)((a.N + BN - 1) / BN);
  const int64_t grid = (int64_t)a.groups * a.tiles_m * a.tiles_n;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_wgrad_kernel<T, BM, BN, EPI>), dim3((unsigned)grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <typename T>
hipError_t run_rows(int kind, int epi, const Args& a, int64_t rows_max, hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  if (kind == KIND_FWD) {
    switch (epi) {
      case EPI_STORE: return launch_rows<T, BM, BN, KIND_FWD, EPI_STORE>(a, rows_max, st);
      case EPI_GELU_FWD: return launch_rows<T, BM, BN, KIND_FWD, EPI_GELU_FWD>(a, rows_max, st);
      case EPI_SWIGLU_FWD: return launch_rows<T, BM, BN, KIND_FWD, EPI_SWIGLU_FWD>(a, rows_max, st);
    }
  } else {
    switch (epi) {
      case EPI_STORE: return launch_rows<T, BM, BN, KIND_DGRAD, EPI_STORE>(a, rows_max, st);
      case EPI_GELU_BWD: return launch_rows<T, BM, BN, KIND_DGRAD, EPI_GELU_BWD>(a, rows_max, st);
      case EPI_SWIGLU_BWD: return launch_rows<T, BM, BN, KIND_DGRAD, EPI_SWIGLU_BWD>(a, rows_max, st);
    }
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t run_wgrad(int epi, const Args& a, hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  if (epi == EPI_STORE) return launch_wgrad<T, BM, BN, EPI_STORE>(a, st);
  if (epi == EPI_STORE_SPLITN) return launch_wgrad<T, BM, BN, EPI_STORE_SPLITN>(a, st);
  return hipErrorInvalidValue;
}

template hipError_t run_rows<float>(int, int, const Args&, int64_t, hipStream_t);
template hipError_t run_rows<bf16>(int, int, const Args&, int64_t, hipStream_t);
template hipError_t run_wgrad<float>(int, const Args&, hipStream_t);
template hipError_t run_wgrad<bf16>(int, const Args&, hipStream_t);

}  // namespace gemm
}  // namespace moe
