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
// Tiling.  A workgroup of WM x WN waves computes a BM x BN tile with
// v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2f32 (fp32), fp32
// accumulation.  Each K stage moves 128 bytes of K per tile row (64 bf16 or
// 32 fp32) through LDS, double buffered with one barrier per stage; the next
// stage's global loads are in flight while the current one is multiplied,
// and inside a stage the MFMA fragments of step s+1 are read from LDS while
// step s multiplies.  LDS rows are K-contiguous (what an MFMA lane consumes:
// 16 bytes of consecutive K) with an XOR swizzle of the 16-byte chunk index
// so that fragment reads and transposing writes spread over the banks.
// Operands whose global layout is M- or N-contiguous (forward weights,
// wgrad activations) are loaded as 4(K) x 16-byte blocks and transposed in
// registers on their way into LDS.
//
// Global loads are buffer loads: each operand gets a buffer resource based
// at its tile (so offsets fit 32 bits) whose extent ends where the valid data
// ends; a masked-off element is given an offset past the extent, which the
// hardware range check turns into zeros.  No branches guard the loads.
//
// Tile order: hardware dispatches consecutive workgroups round-robin over
// the 8 XCDs, each with its own L2; the linear tile id is remapped so that
// the tiles one XCD runs are consecutive, then tiles are walked in groups of
// GM row-tiles so that concurrently running tiles share weight and
// activation panels in that XCD's L2.
#include "common.h"
#include "gemm.h"
#include "gemm_common.h"

namespace moe {
namespace gemm {

using namespace gemm_common;

constexpr int ROWB = 128;                 // bytes of K per LDS row per stage
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
// Operand tile loaders.  A tile operand covers R rows (M or N) x 128 bytes of
// K per stage.  Per-thread byte offsets are computed once (voffset); the
// stage's position along K travels in the scalar offset, and elements outside
// the valid K range or columns get an offset past the resource extent.
// ---------------------------------------------------------------------------
// K-contiguous source (row r of the operand at r * ld elements from the
// resource base): R*8 chunks of 16 bytes, chunk q -> (row q/8, chunk q%8).
template <typename T, int R, int NTH>
struct KLoad {
  static constexpr int V = Vec16<T>::N;
  static constexpr int PER = R * 8 / NTH;
  static_assert(PER >= 1 && R * 8 % NTH == 0, "tile / thread mismatch");
  u32x4 r[PER];
  uint32_t voff[PER];
  int kc;  // K offset of this thread's chunk within a stage

  __device__ __forceinline__ void init(int64_t ld) {
    kc = (threadIdx.x & 7) * V;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int row = (i * NTH + (int)threadIdx.x) >> 3;
      voff[i] = (uint32_t)(((int64_t)row * ld + kc) * (int64_t)sizeof(T));
    }
  }
  __device__ __forceinline__ void load(const BufRes& b, int k0, int64_t K) {
    const bool ok = k0 + kc < K;
    const int soff = k0 * (int)sizeof(T);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      r[i] = __builtin_amdgcn_raw_buffer_load_b128(b.r, ok ? voff[i] : kOOB, soff, 0);
  }
  // K split between two sources: k < split from b0 (at k), k >= split from
  // b1 (at k - split).
  __device__ __forceinline__ void load_split(const BufRes& b0, const BufRes& b1, int64_t ld, int k0, int64_t K,
                                             int64_t split) {
    constexpr int BKE = ROWB / sizeof(T);
    if (k0 + BKE <= split) {
      load(b0, k0, K);
    } else if (k0 >= split) {
      load(b1, k0 - (int)split, K - split);
    } else {
      const int64_t k = k0 + kc;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int row = (i * NTH + (int)threadIdx.x) >> 3;
        const uint32_t o0 = (uint32_t)(((int64_t)row * ld + k) * (int64_t)sizeof(T));
        const uint32_t o1 = (uint32_t)(((int64_t)row * ld + (k - split)) * (int64_t)sizeof(T));
        const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(b0.r, k < split ? o0 : kOOB, 0, 0);
        const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(b1.r, k >= split && k < K ? o1 : kOOB, 0, 0);
        r[i] = v0 | v1;
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = i * NTH + threadIdx.x;
      const int row = q >> 3, ch = q & 7;
      *reinterpret_cast<u32x4*>(lds + row * ROWB + (swz(row, ch) << 4)) = r[i];
    }
  }
};

// MN-contiguous source (element (k, c) at k * ld + c elements from the base
// of the half holding column c).  2R blocks of 4 K-rows x 16 bytes, numbered
// half-major so that every wave's load reads one half: the two halves of the
// tile's columns may come from different tensors (the paired gate / up
// weights of SwiGLU).  Each stage reads through resources rebased at its
// first K row (stage_res), so offsets stay within one stage whatever the
// operand's row count.
template <typename T, int R, int NTH>
struct MNLoad {
  static constexpr int V = Vec16<T>::N;
  static constexpr int PER = 2 * R / NTH;
  static constexpr int RH = R / 2;
  static constexpr int NBH = RH / V;       // 16-byte blocks along MN per K row and half
  static_assert(PER >= 1 && 2 * R % NTH == 0 && R % 128 == 0, "tile / thread mismatch");
  u32x4 r[PER][4];
  uint32_t voff[PER];
  int kq4[PER];     // first K row of the block within a stage
  bool colok[PER];
  int half[PER];    // wave-uniform

  // col_base1: column of half 1 relative to its resource base; valid_cols:
  // columns (relative to each resource base) that hold data.
  __device__ __forceinline__ void init(int64_t ld, int col_base1, int64_t valid_cols) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = i * NTH + threadIdx.x;
      half[i] = __builtin_amdgcn_readfirstlane(b / R);
      const int rr = b % R;
      kq4[i] = (rr / NBH) * 4;
      const int c = (half[i] ? col_base1 : 0) + (rr % NBH) * V;
      colok[i] = c < valid_cols;
      voff[i] = (uint32_t)(((int64_t)kq4[i] * ld + c) * (int64_t)sizeof(T));
    }
  }
  // base0 / base1: element (0, 0) of each half's columns (the tile's first
  // column, col0_bytes into every row); K rows [k0, k0 + BKE) of the stage.
  __device__ __forceinline__ void load(const char* base0, const char* base1, int64_t ld, int k0, int64_t Kvalid,
                                       int64_t col0_bytes) {
    constexpr int BKE = ROWB / sizeof(T);
    const int row_bytes = (int)(ld * (int64_t)sizeof(T));
    const BufRes b0 = stage_res(base0, k0, BKE, Kvalid, row_bytes, col0_bytes);
    const BufRes b1 = stage_res(base1, k0, BKE, Kvalid, row_bytes, col0_bytes);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const BufRes& br = half[i] ? b1 : b0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bool ok = colok[i] && (k0 + kq4[i] + kk < Kvalid);
        r[i][kk] = __builtin_amdgcn_raw_buffer_load_b128(br.r, ok ? voff[i] + kk * row_bytes : kOOB, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = i * NTH + threadIdx.x;
      const int h = b / R, rr = b % R;
      write_transposed<T>(lds, h * RH + (rr % NBH) * V, rr / NBH, r[i]);
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA over one LDS stage for a wave's FM x FN blocks of 32 x 32; fragments of
// k-step s+1 are read while k-step s multiplies.
// ---------------------------------------------------------------------------
template <typename T, int FM, int FN>
__device__ __forceinline__ void mma_stage(const char* la, const char* lb, int wm0, const int (&bcol)[FN],
                                          f32x16 (&acc)[FM][FN]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, g = lane >> 5;
  u32x4 af[2][FM], bfr[2][FN];
  auto fetch = [&](int s, int buf) {
    const int ch = 2 * s + g;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm0 + i * 32 + r;
      af[buf][i] = *reinterpret_cast<const u32x4*>(la + row * ROWB + (swz(row, ch) << 4));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = bcol[j] + r;
      bfr[buf][j] = *reinterpret_cast<const u32x4*>(lb + row * ROWB + (swz(row, ch) << 4));
    }
  };
  fetch(0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    // keep the reads of step s+1 ahead of the MFMAs of step s
    if (s < 3) fetch(s + 1, (s + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) Mma<T>::run(acc[i][j], af[s & 1][i], bfr[s & 1][j]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// FWD / DGRAD: rows split by group.
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WM, int WN, int PIPE, int KIND, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_rows_kernel(Args a) {
  constexpr int NTH = 64 * WM * WN;
  constexpr int FM = BM / (32 * WM), FN = BN / (32 * WN);
  constexpr int BKE = ROWB / sizeof(T);
  constexpr int S = sizeof(T);
  constexpr bool PAIR = (EPI == EPI_SWIGLU_FWD);
  static_assert(!PAIR || FN % 2 == 0, "SwiGLU pairing needs an even number of N-blocks per wave");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  int g = -1, nt = 0;
  int64_t row_begin = 0, row_end = 0;
  if (!row_tile_of<BM>(a, g, row_begin, row_end, nt)) return;
  const int wi = weight_index(g, a.rr_R, a.rr_L);
  const int64_t K = a.K, N = a.N;
  const int64_t rows_valid = min((int64_t)BM, row_end - row_begin);
  const int64_t n0 = PAIR ? (int64_t)nt * (BN / 2) : (int64_t)nt * BN;

  const char* Ab = reinterpret_cast<const char*>(a.A);
  const char* Bg = reinterpret_cast<const char*>(a.B) + (int64_t)wi * a.b_gstride * S;
  const char* B2g = a.B2 ? reinterpret_cast<const char*>(a.B2) + (int64_t)wi * a.b_gstride * S : Bg;

  // A: the tile's rows (at most BM); DGRAD B: the tile's BN weight rows
  // (K-contiguous); FWD B (N-contiguous) is read stage by stage from
  // resources rebased at each stage's first K row.
  BufRes ra, rb0, rb1;
  ra.init(Ab + row_begin * a.lda * S, rows_valid * a.lda * S);
  if (KIND == KIND_DGRAD) {
    const int64_t nrows = min((int64_t)BN, N - n0);
    rb0.init(Bg + n0 * a.ldb * S, nrows * a.ldb * S);
    rb1.init(B2g + n0 * a.ldb * S, nrows * a.ldb * S);
  }
  const int col_base1 = PAIR ? 0 : BN / 2;
  const int64_t valid_cols = N - n0;

  // PIPE register sets of staged global loads: the loads of stage kt+PIPE
  // are issued as soon as stage kt has been written to LDS, so every load has
  // PIPE stages of MFMA work to arrive.
  KLoad<T, BM, NTH> la0, la1;
  KLoad<T, BN, NTH> lbk0, lbk1;   // DGRAD: weights K-contiguous
  MNLoad<T, BN, NTH> lbn0, lbn1;  // FWD: weights N-contiguous
  la0.init(a.lda);
  la1.init(a.lda);
  if (KIND == KIND_FWD) {
    lbn0.init(a.ldb, col_base1, valid_cols);
    lbn1.init(a.ldb, col_base1, valid_cols);
  } else {
    lbk0.init(a.ldb);
    lbk1.init(a.ldb);
  }
  auto load_stage = [&](auto& la, auto& lbk, auto& lbn, int k0) {
    la.load(ra, k0, K);
    if (KIND == KIND_FWD)
      lbn.load(Bg + n0 * S, B2g + n0 * S, a.ldb, k0, K, n0 * S);
    else if (a.b_split > 0)
      lbk.load_split(rb0, rb1, a.ldb, k0, K, a.b_split);
    else
      lbk.load(rb0, k0, K);
  };

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm0 = (wave / WN) * (BM / WM);
  int bcol[FN];
  block_cols<BN, WN, FN, PAIR>(wave % WN, bcol);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (int)((K + BKE - 1) / BKE);
  auto step = [&](auto& la, auto& lbk, auto& lbn, int kt) {
    char* sa = smem + (kt & 1) * (BM + BN) * ROWB;
    char* sb = sa + BM * ROWB;
    la.store(sa);
    if (KIND == KIND_FWD) lbn.store(sb); else lbk.store(sb);
    __syncthreads();
    if (kt + PIPE < nk) load_stage(la, lbk, lbn, (kt + PIPE) * BKE);
    mma_stage<T, FM, FN>(sa, sb, wm0, bcol, acc);
  };
  if (nk > 0) load_stage(la0, lbk0, lbn0, 0);
  if constexpr (PIPE == 1) {
    for (int kt = 0; kt < nk; ++kt) step(la0, lbk0, lbn0, kt);
  } else {
    if (nk > 1) load_stage(la1, lbk1, lbn1, BKE);
    for (int kt = 0; kt < nk; kt += 2) {
      step(la0, lbk0, lbn0, kt);
      if (kt + 1 < nk) step(la1, lbk1, lbn1, kt + 1);
    }
  }

  rows_epilogue<T, FM, FN, PAIR, EPI>(a, acc, bcol, wm0, lane, row_begin, row_end, n0, N);
}

// ---------------------------------------------------------------------------
// WGRAD: C_g[M, N] = X[rows_g, M]^T . D[rows_g, N]; both operands are
// MN-contiguous in memory.  EPI_STORE or EPI_STORE_SPLITN (columns >= c_split
// go to C2 at column - c_split).
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WM, int WN, int PIPE, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_wgrad_kernel(Args a) {
  constexpr int NTH = 64 * WM * WN;
  constexpr int FM = BM / (32 * WM), FN = BN / (32 * WN);
  constexpr int BKE = ROWB / sizeof(T);
  constexpr int S = sizeof(T);
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = a.tiles_m * a.tiles_n;
  const int g = lin / per_g;
  if (g >= a.groups) return;
  int mt, nt;
  grouped_order(lin - g * per_g, a.tiles_m, a.tiles_n, mt, nt, GM);
  const int wi = weight_index(g, a.rr_R, a.rr_L);
  const int64_t r0 = a.offsets[g], r1 = a.offsets[g + 1];
  const int64_t Kr = r1 - r0;
  const int64_t M = a.M, N = a.N;
  const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;

  const char* X = reinterpret_cast<const char*>(a.A);
  const char* D = reinterpret_cast<const char*>(a.B);
  const char* Xs = X + (r0 * a.lda + m0) * S;
  const char* Ds = D + (r0 * a.ldb + n0) * S;
  MNLoad<T, BM, NTH> la0, la1;
  MNLoad<T, BN, NTH> lb0, lb1;
  la0.init(a.lda, BM / 2, M - m0);
  la1.init(a.lda, BM / 2, M - m0);
  lb0.init(a.ldb, BN / 2, N - n0);
  lb1.init(a.ldb, BN / 2, N - n0);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm0 = (wave / WN) * (BM / WM);
  int bcol[FN];
  block_cols<BN, WN, FN, false>(wave % WN, bcol);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (int)((Kr + BKE - 1) / BKE);
  auto load_stage = [&](auto& la, auto& lb, int k0) {
    la.load(Xs, Xs, a.lda, k0, Kr, m0 * S);
    lb.load(Ds, Ds, a.ldb, k0, Kr, n0 * S);
  };
  auto step = [&](auto& la, auto& lb, int kt) {
    char* sa = smem + (kt & 1) * (BM + BN) * ROWB;
    char* sb = sa + BM * ROWB;
    la.store(sa);
    lb.store(sb);
    __syncthreads();
    if (kt + PIPE < nk) load_stage(la, lb, (kt + PIPE) * BKE);
    mma_stage<T, FM, FN>(sa, sb, wm0, bcol, acc);
  };
  if (nk > 0) load_stage(la0, lb0, 0);
  if constexpr (PIPE == 1) {
    for (int kt = 0; kt < nk; ++kt) step(la0, lb0, kt);
  } else {
    if (nk > 1) load_stage(la1, lb1, BKE);
    for (int kt = 0; kt < nk; kt += 2) {
      step(la0, lb0, kt);
      if (kt + 1 < nk) step(la1, lb1, kt + 1);
    }
  }

  wgrad_epilogue<T, FM, FN, EPI>(a, acc, bcol, wm0, lane, wi, m0, n0, M, N);
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WM, int WN, int PIPE, int KIND, int EPI>
static hipError_t launch_rows(Args a, int64_t rows_max, hipStream_t st) {
  const int tiles_n_cols = EPI == EPI_SWIGLU_FWD ? BN / 2 : BN;
  a.tiles_n = (int)((a.N + tiles_n_cols - 1) / tiles_n_cols);
  a.tiles_m = (int)((rows_max + BM - 1) / BM) + a.groups;
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = 2 * (BM + BN) * ROWB;
  auto kern = gemm_rows_kernel<T, BM, BN, WM, WN, PIPE, KIND, EPI>;
  static hipError_t prep = prepare_lds(kern, lds);
  if (prep != hipSuccess) return prep;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WM * WN), lds, st, a);
  return hipGetLastError();
}

template <typename T, int BM, int BN, int WM, int WN, int PIPE, int EPI>
static hipError_t launch_wgrad(Args a, hipStream_t st) {
  a.tiles_m = (int)((a.M + BM - 1) / BM);
  a.tiles_n = (int)((a.N + BN - 1) / BN);
  const int64_t grid = (int64_t)a.groups * a.tiles_m * a.tiles_n;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = 2 * (BM + BN) * ROWB;
  auto kern = gemm_wgrad_kernel<T, BM, BN, WM, WN, PIPE, EPI>;
  static hipError_t prep = prepare_lds(kern, lds);
  if (prep != hipSuccess) return prep;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WM * WN), lds, st, a);
  return hipGetLastError();
}

#ifndef MOE_GEMM_CFG
#define MOE_GEMM_CFG 128, 128, 2, 2, 1
#endif

template <typename T>
hipError_t run_rows(int kind, int epi, const Args& a, int64_t rows_max, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (gemm3::supports(a)) return gemm3::run_rows_bf16(kind, epi, a, rows_max, st);
  }
  if (kind == KIND_FWD) {
    switch (epi) {
      case EPI_STORE: return launch_rows<T, MOE_GEMM_CFG, KIND_FWD, EPI_STORE>(a, rows_max, st);
      case EPI_GELU_FWD: return launch_rows<T, MOE_GEMM_CFG, KIND_FWD, EPI_GELU_FWD>(a, rows_max, st);
      case EPI_SWIGLU_FWD: return launch_rows<T, MOE_GEMM_CFG, KIND_FWD, EPI_SWIGLU_FWD>(a, rows_max, st);
    }
  } else {
    switch (epi) {
      case EPI_STORE: return launch_rows<T, MOE_GEMM_CFG, KIND_DGRAD, EPI_STORE>(a, rows_max, st);
      case EPI_GELU_BWD: return launch_rows<T, MOE_GEMM_CFG, KIND_DGRAD, EPI_GELU_BWD>(a, rows_max, st);
      case EPI_SWIGLU_BWD: return launch_rows<T, MOE_GEMM_CFG, KIND_DGRAD, EPI_SWIGLU_BWD>(a, rows_max, st);
    }
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t run_wgrad(int epi, const Args& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (gemm3::supports(a)) return gemm3::run_wgrad_bf16(epi, a, st);
  }
  if (epi == EPI_STORE) return launch_wgrad<T, MOE_GEMM_CFG, EPI_STORE>(a, st);
  if (epi == EPI_STORE_SPLITN) return launch_wgrad<T, MOE_GEMM_CFG, EPI_STORE_SPLITN>(a, st);
  return hipErrorInvalidValue;
}

template hipError_t run_rows<float>(int, int, const Args&, int64_t, hipStream_t);
template hipError_t run_rows<bf16>(int, int, const Args&, int64_t, hipStream_t);
template hipError_t run_wgrad<float>(int, const Args&, hipStream_t);
template hipError_t run_wgrad<bf16>(int, const Args&, hipStream_t);

}  // namespace gemm
}  // namespace moe
