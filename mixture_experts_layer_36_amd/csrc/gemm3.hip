// bf16 grouped expert GEMMs with direct global -> LDS loads (gfx950).
//
// Same three launch kinds and epilogues as the register-staged kernels of
// gemm.hip (FWD, DGRAD split rows by group; WGRAD splits the reduction by
// group), built around two gfx950 features:
//
//  * buffer_load_dwordx4 ... lds: every lane's 16 bytes go straight from
//    global memory into LDS at M0 + 16 * lane, without passing through
//    registers.  The loads of a K stage therefore cost no VGPRs, and the
//    tile ring holds NS stages in flight (NS - 1 stages of loads overlap the
//    MFMA work of the current one).  A lane's global address is chosen so
//    that its 16 bytes land in the XOR-swizzled slot the fragment reads
//    expect; masked-off lanes get an offset past the buffer extent and the
//    hardware range check writes zeros.
//  * ds_read_b64_tr_b16: operands whose global layout is M- or N-contiguous
//    (forward weights, both wgrad operands) are kept in LDS in that layout,
//    as panels of [K][128 columns]; within each 16-lane group the transposing
//    read hands lane i the 4 consecutive K values of column i of a 4 x 16
//    block, so two reads build the 8-element K run an MFMA lane consumes.
//    K-contiguous operands (the activation rows of FWD / DGRAD, the weights
//    of DGRAD) are stored [rows][BK] and read with ds_read_b128.
//
// Schedule: the 8 waves form two ping-pong groups (k_loop_pingpong), one wave
// of each on every SIMD; per stage a wave runs a memory phase (its share of
// the loads NS - 1 stages ahead, then all fragment reads of the stage) and an
// MFMA-only phase, group 1 one phase behind group 0.  Outputs leave through
// LDS as whole rows (the staged epilogues).
//
// Workgroup: WM x WN waves, tile BM x BN, MFMA v_mfma_f32_32x32x16_bf16 with
// fp32 accumulation.  Tile order as in gemm.hip (XCD-aware, grouped rows).
// The B fragment is the MFMA's first operand, so the accumulators hold C^T
// blocks: a lane owns one row of C and runs of 4 consecutive columns, which
// the epilogues store (and the backward activations load) 8 bytes at a time.
#include <type_traits>

#include "common.h"
#include "gemm.h"
#include "gemm_common.h"

namespace moe {
namespace gemm3 {

using gemm::Args;
using namespace gemm_common;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  // n is wave-uniform; dispatch to immediates (values above the table wait
  // for everything, which is correct, only slower)
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break;
    case 19: wait_vmcnt<19>(); break;
    case 20: wait_vmcnt<20>(); break;
    case 21: wait_vmcnt<21>(); break;
    case 22: wait_vmcnt<22>(); break;
    case 23: wait_vmcnt<23>(); break;
    case 24: wait_vmcnt<24>(); break;
    case 25: wait_vmcnt<25>(); break;
    case 26: wait_vmcnt<26>(); break;
    case 27: wait_vmcnt<27>(); break;
    case 28: wait_vmcnt<28>(); break;
    case 29: wait_vmcnt<29>(); break;
    case 30: wait_vmcnt<30>(); break;
    case 31: wait_vmcnt<31>(); break;
    case 32: wait_vmcnt<32>(); break;
    case 33: wait_vmcnt<33>(); break;
    case 34: wait_vmcnt<34>(); break;
    case 35: wait_vmcnt<35>(); break;
    case 36: wait_vmcnt<36>(); break;
    case 37: wait_vmcnt<37>(); break;
    case 38: wait_vmcnt<38>(); break;
    case 39: wait_vmcnt<39>(); break;
    case 40: wait_vmcnt<40>(); break;
    case 41: wait_vmcnt<41>(); break;
    case 42: wait_vmcnt<42>(); break;
    case 43: wait_vmcnt<43>(); break;
    case 44: wait_vmcnt<44>(); break;
    case 45: wait_vmcnt<45>(); break;
    case 46: wait_vmcnt<46>(); break;
    case 47: wait_vmcnt<47>(); break;
    case 48: wait_vmcnt<48>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void lds_load16(const BufRes& b, char* lds_unit, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (lds_void*)lds_unit, 16, voff, soff, 0, 0);
}

// Layout of one stage of an operand in LDS and the lanes' loads into it:
// gemm_addr.h (kc_swz, mn_swz, kc_lane, mn_lane, shared with the host-side
// address checker).
using gemm_addr::kc_lane;
using gemm_addr::kc_swz;
using gemm_addr::mn_lane;
using gemm_addr::mn_swz;

// One operand's direct loads.  The stage is split into 1 KiB units; unit u of
// the stage is issued by wave u % NW as its (u / NW)-th load.
template <int R, int BK, bool KC, int NW, int W0 = 0>
struct Loader {
  static constexpr int BYTES = gemm_addr::Units<R, BK, NW>::BYTES;
  static constexpr int UNITS = gemm_addr::Units<R, BK, NW>::UNITS;
  static constexpr int PER = gemm_addr::Units<R, BK, NW>::PER;
  uint32_t voff[PER];
  int krow[PER];      // MN: K row (within the stage) this lane loads
  bool colok[PER];    // MN: column in range
  int kcol[PER];      // KC: K element offset (within the stage) of this lane's chunk

  // KC: source row r of the operand is at r * ld elements from the base.
  __device__ __forceinline__ void init_kc(int64_t ld) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) - W0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int row, col;
      kc_lane<BK, NW>(i, wave, lane, row, col);
      kcol[i] = col;
      voff[i] = (uint32_t)(((int64_t)row * ld + col) * 2);
      krow[i] = 0;
      colok[i] = true;
    }
  }
  // KC gathered: tile row r of the group (r < rows_valid) is row
  // gather[row_begin + r] / gather_k of the operand; lanes of rows past the
  // group are masked through their K column (gemm_addr::kc_gather_col).
  __device__ __forceinline__ void init_kc_gather(int64_t ld, const int32_t* gather, int gather_k, int64_t row_begin,
                                                 int64_t rows_valid) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) - W0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int row, col;
      kc_lane<BK, NW>(i, wave, lane, row, col);
      const int32_t a = row < rows_valid ? gather[row_begin + row] : 0;
      kcol[i] = gemm_addr::kc_gather_col(row, col, rows_valid);
      voff[i] = (uint32_t)((gemm_addr::gather_token(a, gather_k) * ld + col) * 2);
      krow[i] = 0;
      colok[i] = true;
    }
  }
  // MN: element (k0 + k, col) of a stage at k * ld + col elements from the
  // base of the stage's resource of the column's panel (col relative to that
  // base, k within the stage).
  __device__ __forceinline__ void init_mn(int64_t ld, bool pair, int64_t valid_cols) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) - W0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int panel, k, col;
      mn_lane<BK, NW>(i, wave, lane, pair, panel, k, col);
      krow[i] = k;
      colok[i] = col < valid_cols;
      voff[i] = (uint32_t)(((int64_t)k * ld + col) * 2);
    }
  }
  // Issue load i (0 <= i < PER) of a stage.  KC: K range [k0, Klim), the
  // stage's K position in the scalar offset; MN: K rows [k0, Klim), from a
  // resource rebased at this stage's first K row (stage_res), so the scalar
  // offset is 0 and every offset stays within one stage.
  template <typename ResOf>
  __device__ __forceinline__ void issue_one(int i, char* stage, const ResOf& res_of_panel, int k0, int64_t Klim,
                                            int64_t ld) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) - W0;
    const int u = i * NW + wave;
    char* dst = stage + u * 1024;
    if constexpr (KC) {
      const bool ok = k0 + kcol[i] < Klim;
      lds_load16(res_of_panel(0), dst, ok ? voff[i] : kOOB, (uint32_t)(k0 * 2));
    } else {
      constexpr int KB = BK / 4;
      const int panel = u / KB;
      const bool ok = colok[i] && (k0 + krow[i] < Klim);
      lds_load16(res_of_panel(panel), dst, ok ? voff[i] : kOOB, 0u);
    }
  }
};

// Fragment reads are issued as inline asm: the compiler cannot tell that they
// never touch an LDS slot with loads in flight and would otherwise wait for
// every outstanding global->LDS load before each read.  Their completion is
// tracked by hand with lgkmcnt (LDS reads complete in order; the loop issues
// no scalar memory loads).
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  // vmcnt = 63 (bits [3:0] = 15, [15:14] = 3), expcnt = 7
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
}

// K-contiguous fragment: 8 consecutive K of row `row` at k-step s.
template <int BK>
__device__ __forceinline__ u32x4 frag_kc(uint32_t tile, int row, int s, int g) {
  const int ch = 2 * s + g;
  return ds_read_b128(tile + row * (BK * 2) + ((ch ^ kc_swz<BK>(row)) << 4));
}

// MN-contiguous fragment of the 32-column block starting at tile column n0:
// lane l gets K = 16 s + 8 (l / 32) + 0..7 of column n0 + (l % 32).
template <int BK>
__device__ __forceinline__ u32x4 frag_mn(uint32_t tile, int n0, int s, int lane) {
  const int G = lane >> 4, j = lane & 15;
  const int n = n0 + (G & 1) * 16 + 4 * (j & 3);
  const int panel = n >> 7, nc = n & 127;
  const uint32_t pbase = tile + panel * (BK * 256);
  u32x4 out;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int k = 16 * s + (G >> 1) * 8 + 4 * r + (j >> 2);
    const u32x2 w = ds_read_tr16(pbase + k * 256 + (((nc >> 3) ^ mn_swz(k)) << 4) + (nc & 7) * 2);
    out[2 * r] = w[0];
    out[2 * r + 1] = w[1];
  }
  return out;
}

template <bool KC, int BK>
__device__ __forceinline__ u32x4 frag(uint32_t tile, int row, int s, int lane) {
  if constexpr (KC) return frag_kc<BK>(tile, row + (lane & 31), s, lane >> 5);
  else return frag_mn<BK>(tile, row, s, lane);
}

// Fragments of one whole stage, read ahead of the MFMAs that use them.
template <int FM, int FN, int BK>
struct StageFrags {
  u32x4 a[BK / 16][FM];
  u32x4 b[BK / 16][FN];
};

template <int FM, int FN, int BK, bool AKC, bool BKC>
__device__ __forceinline__ void read_stage(const char* ta_p, const char* tb_p, int wm0, const int (&bcol)[FN],
                                           StageFrags<FM, FN, BK>& f) {
  const uint32_t ta = lds_addr(ta_p), tb = lds_addr(tb_p);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
#pragma unroll
    for (int i = 0; i < FM; ++i) f.a[s][i] = frag<AKC, BK>(ta, wm0 + i * 32, s, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) f.b[s][j] = frag<BKC, BK>(tb, bcol[j], s, lane);
  }
}

template <int FM, int FN, int BK>
__device__ __forceinline__ void mma_frags(const StageFrags<FM, FN, BK>& f, f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int s = 0; s < BK / 16; ++s)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.b[s][j]),
                                                            __builtin_bit_cast(bf16x8, f.a[s][i]), acc[i][j], 0,
                                                            0, 0);
}

// Ping-pong K loop.  The workgroup's waves form two groups with one wave of
// each on every SIMD (waves w and w + NC/2).  Per stage a wave runs a memory
// phase (issue its share of the loads of the stage NS-1 ahead, read all of
// this stage's fragments into registers) and then a compute phase (only
// MFMAs); group 1 runs one phase behind group 0, so in every phase one wave
// per SIMD issues MFMAs while the other feeds the load path.  Phases are
// separated by workgroup barriers (2 per stage, the same count for both
// groups).  Loads of stage s are issued in the memory phases of stage
// s - (NS-1); each wave waits for its own loads of stage t+1 at the end of
// its memory phase of stage t, so stage t+1 is complete and visible when
// group 0 starts reading it, and the slot reloaded in a phase was last read
// two phases earlier.
template <int NS, int STAGE_BYTES, int Q, typename Issue, typename Read, typename Mma>
__device__ __forceinline__ void k_loop_pingpong(char* smem, int nk, int group, const Issue& issue, const Read& read,
                                                const Mma& mma) {
  constexpr int D = NS - 1;
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < nk) issue(smem + s * STAGE_BYTES, s, 0, Q);
  wait_vmcnt_dyn((min(D, nk) - 1) * Q);
  if (group == 1) barrier();
  for (int kt = 0; kt < nk; ++kt) {
    barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int next = kt + D;
    if (next < nk) issue(smem + (next % NS) * STAGE_BYTES, next, 0, Q);
    read(smem + (kt % NS) * STAGE_BYTES);
    wait_vmcnt_dyn(max(0, min(D - 1, nk - 2 - kt)) * Q);
    wait_lgkmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    barrier();
    __builtin_amdgcn_sched_barrier(0);
    mma();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (group == 0) barrier();
}

// ---------------------------------------------------------------------------
// Staged epilogues (ping-pong kernels, 256 x 256 tiles of 8 waves in 2 x 4).
// Stored straight from the accumulators, a store instruction writes 8 bytes
// into each of 32 rows: partial L2 lines, which the output of every tile of a
// round competes for at once, and which measured as the whole per-tile cost
// beyond the K loop (up to a quarter of a short-K launch).  Instead, once the
// K loop is done and its ring idle, each 32-row pass of the accumulators
// (rows wm0 + 32 i + 0..31 of every wave) is written into an LDS table of 64
// staged rows (wave row band wm: staged rows 32 wm + 0..31) and SC columns,
// and the workgroup then stores the table in 16-byte chunks, consecutive
// threads on consecutive chunks of one row, so every row goes out as whole
// lines.  16-byte chunk c of staged row r sits at chunk c ^ (r & 15): the
// 8-byte writes (32 rows, one column) are at most 2-way bank conflicted and
// the 16-byte reads (16 consecutive chunks of a row) are conflict-free.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char;

template <typename T, int SC>
struct StagedTile {
  static constexpr int ROWB = SC * (int)sizeof(T), CH = ROWB / 16, ROWS = 64;
  static_assert(ROWB % 256 == 0, "rows of whole 256-byte bank windows");
  lds_char* base;
  // 4 consecutive values at element column col (a multiple of 4) of staged row r
  __device__ __forceinline__ void put4(int r, int col, const float (&v)[4]) const {
    const int byte = col * (int)sizeof(T);
    lds_char* p = base + r * ROWB + (((byte >> 4) ^ (r & 15)) << 4) + (byte & 15);
    if constexpr (sizeof(T) == 2)
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(p) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    else
      *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
  __device__ __forceinline__ u32x4 get(int r, int c) const {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + r * ROWB + ((c ^ (r & 15)) << 4));
  }
  // every thread of the workgroup: chunk q = tid + NT k of the table, handed
  // to dst(staged row, element column of the chunk, data)
  template <int NT, typename Dst>
  __device__ __forceinline__ void store_all(const Dst& dst) const {
    static_assert(ROWS * CH % NT == 0, "every thread takes the same number of chunks");
#pragma unroll
    for (int j = 0; j < ROWS * CH / NT; ++j) {
      const int q = (int)threadIdx.x + NT * j, r = q / CH, c = q - r * CH;
      dst(r, c * (16 / (int)sizeof(T)), get(r, c));
    }
  }
  // the chunks of column part P of PARTS equal parts of the table, handed to
  // dst(staged row, element column within the part, data): one destination
  // per call, so no thread selects between outputs
  template <int NT, int PARTS, int P, typename Dst>
  __device__ __forceinline__ void store_part(const Dst& dst) const {
    constexpr int CP = CH / PARTS;
    static_assert(CH % PARTS == 0 && ROWS * CP % NT == 0, "every thread takes the same number of chunks");
#pragma unroll
    for (int j = 0; j < ROWS * CP / NT; ++j) {
      const int q = (int)threadIdx.x + NT * j, r = q / CP, c = q - r * CP;
      dst(r, c * (16 / (int)sizeof(T)), get(r, P * CP + c));
    }
  }
};

// Stores of a tile go to a uniform base (the tile's first row and column)
// plus a 32-bit element offset.  Tile rows are below 256 and every leading
// dimension below 2^22 elements (the entry points reject rows wider than
// 8 MiB), so row * ld + column stays below 2^31 and both factors fit the
// 24-bit multiplier, which issues at the full rate, where the 32-bit and
// 64-bit products of a 64-bit row * ld per 16-byte store take four slots
// each.
__device__ __forceinline__ uint32_t tile_off(int tr, uint32_t ld, int c) {
  return __umul24((uint32_t)tr, ld) + (uint32_t)c;
}
// f(I) for I = 0 .. N-1 with I a compile-time constant: straight-line code
// that no loop pass has to unroll.  (The forward epilogue's pass loop, whose
// store branches depend only on the thread, was unswitched on them and then
// left rolled, with the accumulators indexed at run time from scratch memory.)
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(const F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// rows (or columns) of a tile that exist: min(end - begin, 256), at least 0
__device__ __forceinline__ int tile_extent(int64_t end, int64_t begin) {
  const int64_t n = end - begin;
  return n <= 0 ? 0 : n >= 256 ? 256 : (int)n;
}

// Row-split kernels: EPI_STORE (C), EPI_GELU_FWD (C = GELU'(Z) | C2 = GELU(Z))
// and the SwiGLU gate|up pair (C = dH/dA | dH/dB at column f and c_split + f,
// C2 = silu(A) B): the saved factors are those of gelu_fwd_save and
// swiglu_fwd_save.  Variants of the fused forward: EPI_SWIGLU_FWD_H and EPI_GELU_FWD_H write
// only the hidden activation (C2), EPI_STORE_SCATTER writes output row r to
// row scatter[r] of C, scaled by row_scale[scatter[r]] before rounding.
template <int FM, int FN, bool PAIR, int EPI>
__device__ __forceinline__ void rows_epilogue_staged(const Args& a, f32x16 (&acc)[FM][FN], const int (&bcol)[FN],
                                                     int wave, int lane, int64_t row_begin, int64_t row_end,
                                                     int64_t n0, int64_t N, char* smem) {
  static_assert(FM == 4 && FN == 2, "256 x 256 tile of 8 waves in 2 x 4");
  constexpr bool GELU = EPI == gemm::EPI_GELU_FWD || EPI == gemm::EPI_GELU_FWD_H;
  constexpr bool SAVE = EPI == gemm::EPI_GELU_FWD || EPI == gemm::EPI_SWIGLU_FWD;  // also the factors
  constexpr bool SCAT = EPI == gemm::EPI_STORE_SCATTER;
  // staged columns: PAIR D1 | D2 | H or H; GELU D | GELU(Z) or GELU(Z); else the output
  constexpr int SC = PAIR ? (SAVE ? 384 : 128) : (GELU && SAVE ? 512 : 256);
  constexpr int HOFF = PAIR ? (SAVE ? 256 : 0) : (SAVE ? 256 : 0);  // column of the hidden activation
  const StagedTile<bf16, SC> st{(lds_char*)smem};
  bf16* C = reinterpret_cast<bf16*>(a.C);
  const int wm = wave / 4;
  const int sr = 32 * wm + (lane & 31);  // this lane's staged row
  const int rl = tile_extent(row_end, row_begin), nl = tile_extent(N, n0);
  const uint32_t ldc = (uint32_t)a.ldc, ldc2 = (uint32_t)a.ldc2;
  bf16* const Cp = C + row_begin * a.ldc + n0;
  bf16* const Cup = PAIR ? Cp + a.c_split : Cp;
  bf16* const C2p = (GELU || PAIR) ? reinterpret_cast<bf16*>(a.C2) + row_begin * a.ldc2 + n0 : Cp;
  static_for<0, FM>([&](auto pass) {
    constexpr int i = decltype(pass)::value;
    float scale = 1.0f;
    if constexpr (SCAT) {  // this lane's row's weight
      const int64_t rr = row_begin + wm * 128 + 32 * i + (lane & 31);
      scale = rr < row_end ? a.row_scale[a.scatter[rr]] : 0.0f;
    }
    __syncthreads();  // the table's previous pass has been stored (and the K ring is idle)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int tc = tacc_col(g, lane);
      if constexpr (PAIR) {
        float hv[4];
        if constexpr (SAVE) {
          float d1[4], d2[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hv[q] = swiglu_fwd_save(acc[i][0][4 * g + q], acc[i][1][4 * g + q], d1[q], d2[q]);
          st.put4(sr, bcol[0] + tc, d1);
          st.put4(sr, bcol[1] + tc, d2);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float av = acc[i][0][4 * g + q];
            hv[q] = av * sigmoid_f(av) * acc[i][1][4 * g + q];
          }
        }
        st.put4(sr, HOFF + bcol[0] + tc, hv);
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q] * scale;
          if constexpr (GELU && SAVE) {
            float d[4], h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = gelu_fwd_save(v[q], d[q]);
            st.put4(sr, bcol[j] + tc, d);
            st.put4(sr, HOFF + bcol[j] + tc, h);
          } else if constexpr (GELU) {
            float h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = gelu_f(v[q]);
            st.put4(sr, HOFF + bcol[j] + tc, h);
          } else {
            st.put4(sr, bcol[j] + tc, v);
          }
        }
      }
    }
    __syncthreads();
    // staged row r is tile row (r / 32) 128 + 32 i + r % 32
    auto to = [&](bf16* const base, const uint32_t ld) {
      return [&, base, ld](int r, int c, const u32x4& v) {
        const int tr = (r >> 5) * 128 + 32 * i + (r & 31);
        if (tr < rl && c < nl) st16(base + tile_off(tr, ld, c), v);
      };
    };
    if constexpr (PAIR && SAVE) {  // dH/dA | dH/dB | H
      st.template store_part<512, 3, 0>(to(Cp, ldc));
      st.template store_part<512, 3, 1>(to(Cup, ldc));
      st.template store_part<512, 3, 2>(to(C2p, ldc2));
    } else if constexpr (GELU && SAVE) {  // GELU'(Z) | GELU(Z)
      st.template store_part<512, 2, 0>(to(Cp, ldc));
      st.template store_part<512, 2, 1>(to(C2p, ldc2));
    } else if constexpr (PAIR || GELU) {  // H only
      st.template store_part<512, 1, 0>(to(C2p, ldc2));
    } else if constexpr (SCAT) {
      st.template store_part<512, 1, 0>([&](int r, int c, const u32x4& v) {
        const int tr = (r >> 5) * 128 + 32 * i + (r & 31);
        if (tr < rl && c < nl) st16(C + (int64_t)a.scatter[row_begin + tr] * a.ldc + n0 + c, v);
      });
    } else {
      st.template store_part<512, 1, 0>(to(Cp, ldc));
    }
  });
}

// Activation backward of the row-split DGRAD kernels, staged the same way:
// X1 holds the factors the forward saved, dZ = acc * GELU'(Z), or for SwiGLU
// dA = acc * dH/dA and dB = acc * dH/dB from X1's columns n and c_split + n,
// stored at the same columns of C.  The accumulators are staged in
// fp32; a thread then takes 8 consecutive columns of a staged row, with all
// its 16-byte loads of the saved activations for the pass issued before any
// arithmetic, and stores 16 bytes per output.
template <int FM, int FN, int EPI>
__device__ __forceinline__ void rows_epilogue_staged_bwd(const Args& a, f32x16 (&acc)[FM][FN], const int (&bcol)[FN],
                                                         int wave, int lane, int64_t row_begin, int64_t row_end,
                                                         int64_t n0, int64_t N, char* smem) {
  static_assert(FM == 4 && FN == 2, "256 x 256 tile of 8 waves in 2 x 4");
  constexpr bool SW = EPI == gemm::EPI_SWIGLU_BWD;
  constexpr int PER = 64 * 32 / 512;  // 8-column groups per thread per pass
  const StagedTile<float, 256> st{(lds_char*)smem};
  const int rl = tile_extent(row_end, row_begin), nl = tile_extent(N, n0);
  const uint32_t ldc = (uint32_t)a.ldc, ldx = (uint32_t)a.ldx;
  bf16* const Cp = reinterpret_cast<bf16*>(a.C) + row_begin * a.ldc + n0;
  bf16* const Cup = Cp + a.c_split;
  const bf16* const Xp = reinterpret_cast<const bf16*>(a.X1) + row_begin * a.ldx + n0;
  const int sr = 32 * (wave / 4) + (lane & 31);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q];
        st.put4(sr, bcol[j] + tacc_col(g, lane), v);
      }
    __syncthreads();
    // group u of this thread: staged row r = q / 32, columns 8 (q % 32) .. +7
    uint32_t co[PER];  // element offset of the group in the tile, for C (X1 has its own)
    bool ok[PER];
    u32x4 x0[PER], x1[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = (int)threadIdx.x + 512 * u, r = q >> 5, c8 = (q & 31) * 8;
      const int tr = (r >> 5) * 128 + 32 * i + (r & 31);  // row of the tile
      ok[u] = tr < rl && c8 < nl;
      co[u] = tile_off(tr, ldc, c8);
      // unconditional loads from a valid place (the tile's first row and column) when out of range
      const bf16* xp = Xp + (ok[u] ? tile_off(tr, ldx, c8) : 0u);
      x0[u] = ld16(xp);
      if constexpr (SW) x1[u] = ld16(xp + a.c_split);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = (int)threadIdx.x + 512 * u, r = q >> 5, c = (q & 31) * 2;  // two fp32 chunks
      float g8[8], d0[8];
      {
        const u32x4 lo = st.get(r, c), hi = st.get(r, c + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g8[e] = __uint_as_float(lo[e]);
          g8[4 + e] = __uint_as_float(hi[e]);
        }
      }
      unpack16<bf16>(x0[u], d0);
      if constexpr (SW) {
        float d1[8], da[8], db[8];
        unpack16<bf16>(x1[u], d1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          da[e] = g8[e] * d0[e];
          db[e] = g8[e] * d1[e];
        }
        if (ok[u]) {
          st16(Cp + co[u], pack16<bf16>(da));
          st16(Cup + co[u], pack16<bf16>(db));
        }
      } else {
        float dz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) dz[e] = g8[e] * d0[e];
        if (ok[u]) st16(Cp + co[u], pack16<bf16>(dz));
      }
    }
  }
}

// WGRAD kernels: weight set wi, rows m0 + ..., columns n0 + ... (EPI_STORE_SPLITN
// sends columns >= c_split to C2); T = float for the split partials.
template <typename T, int FM, int FN, int EPI>
__device__ __forceinline__ void wgrad_epilogue_staged(const Args& a, f32x16 (&acc)[FM][FN], const int (&bcol)[FN],
                                                      int wave, int lane, int wi, int64_t m0, int64_t n0, int64_t M,
                                                      int64_t N, char* smem) {
  static_assert(FM == 4 && FN == 2, "256 x 256 tile of 8 waves in 2 x 4");
  const StagedTile<T, 256> st{(lds_char*)smem};
  constexpr bool SPLIT = EPI == gemm::EPI_STORE_SPLITN;
  const int ml = tile_extent(M, m0), nl = tile_extent(N, n0);
  const uint32_t ldc = (uint32_t)a.ldc;
  T* const Cp = reinterpret_cast<T*>(a.C) + (int64_t)wi * a.c_gstride + m0 * a.ldc + n0;
  // columns n >= c_split go to C2 at column n - c_split: tile columns from cs on
  const int cs = SPLIT ? tile_extent(a.c_split, n0) : 256;
  T* const C2p = SPLIT ? reinterpret_cast<T*>(a.C2) + (int64_t)wi * a.c_gstride + m0 * a.ldc +
                             (n0 > a.c_split ? n0 - a.c_split : 0)
                       : Cp;
  const int wm = wave / 4;
  const int sr = 32 * wm + (lane & 31);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q];
        st.put4(sr, bcol[j] + tacc_col(g, lane), v);
      }
    __syncthreads();
    st.template store_all<512>([&](int r, int col, const u32x4& v) {
      const int tr = (r >> 5) * 128 + 32 * i + (r & 31);  // row of the tile
      if (tr >= ml || col >= nl) return;
      // c_split is a multiple of 8: a chunk never straddles it
      if (SPLIT && col >= cs)
        st16(C2p + tile_off(tr, ldc, col - cs), v);
      else
        st16(Cp + tile_off(tr, ldc, col), v);
    });
  }
}

constexpr int kPingPong = -1;  // NP value selecting the ping-pong loop
// WGRAD epilogue selector (internal) of a launch split over the reduction:
// each split writes an fp32 partial [split][weight set][M][N], summed after
constexpr int kEpiPartial = 100;

// ---------------------------------------------------------------------------
// FWD / DGRAD: rows split by group.  A = activation rows (K-contiguous).
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int BK, int NS, int NP, int KIND, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm3_rows_kernel(Args a) {
  static_assert(NP == kPingPong, "the ping-pong schedule is the one built");
  constexpr int NC = WM * WN;                 // waves: every wave loads and multiplies
  constexpr int NW = NC, W0 = 0;
  constexpr int FM = BM / (32 * WM), FN = BN / (32 * WN);
  constexpr bool PAIR = (EPI == gemm::EPI_SWIGLU_FWD || EPI == gemm::EPI_SWIGLU_FWD_H);
  constexpr bool BKC = (KIND == gemm::KIND_DGRAD);
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  static_assert(!PAIR || BN == 256, "gate/up pairing puts one 128-column panel per half");
  static_assert(BM % 128 == 0 && BN % 128 == 0 && (BK == 32 || BK == 64), "tile shape");
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  int g = -1, nt = 0;
  int64_t row_begin = 0, row_end = 0;
  if (!row_tile_of<BM>(a, g, row_begin, row_end, nt)) return;
  const int wi = weight_index(g, a.rr_R, a.rr_L);
  const int64_t K = a.K, N = a.N;
  const int64_t rows_valid = min((int64_t)BM, row_end - row_begin);
  const int64_t n0 = PAIR ? (int64_t)nt * (BN / 2) : (int64_t)nt * BN;

  const char* Ab = reinterpret_cast<const char*>(a.A);
  const char* Bg = reinterpret_cast<const char*>(a.B) + (int64_t)wi * a.b_gstride * 2;
  const char* B2g = a.B2 ? reinterpret_cast<const char*>(a.B2) + (int64_t)wi * a.b_gstride * 2 : Bg;

  // A: the tile's rows (at most BM); DGRAD B: the tile's BN weight rows
  // (K-contiguous); FWD B (N-contiguous): rebased at every K stage in issue.
  BufRes ra, rb0, rb1;
  if (a.gather) ra.init(Ab, gemm_addr::gather_a_span(a.gather_rows, a.lda));
  else ra.init(Ab, gemm_addr::rows_a_span(row_begin, rows_valid, a.lda));
  if (KIND == gemm::KIND_DGRAD) {
    rb0.init(Bg, gemm_addr::dgrad_b_span(0, n0, BN, N, a.ldb));
    rb1.init(B2g, gemm_addr::dgrad_b_span(0, n0, BN, N, a.ldb));
  }

  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Loader<BM, BK, true, NW, W0> la;
  Loader<BN, BK, BKC, NW, W0> lb;
  if (a.gather) la.init_kc_gather(a.lda, a.gather, a.gather_k, row_begin, rows_valid);
  else la.init_kc(a.lda);
  if constexpr (BKC) lb.init_kc(a.ldb);
  else lb.init_mn(a.ldb, PAIR, N - n0);
  const bool split = BKC && a.b_split > 0;

  constexpr int QA = Loader<BM, BK, true, NW, W0>::PER, QB = Loader<BN, BK, BKC, NW, W0>::PER;
  // FWD: the weights' K stages (gate and up for the pair), walked in order:
  // every wave issues its share of each stage once, for kt = 0, 1, ...
  StageRes w0, w1;
  if constexpr (!BKC) {
    w0.init(Bg, gemm_addr::fwd_b_walk(n0, BK, a.ldb));
    w1.init(B2g, gemm_addr::fwd_b_walk(n0, BK, a.ldb));
  }
  auto issue = [&](char* stage, int kt, int q0, int q1) {
    const int k0 = kt * BK;
    BufRes s0, s1;  // FWD: this stage's K rows of the weights (gate / up for the pair)
    if constexpr (!BKC) {
      s0 = w0.next();
      if (PAIR) s1 = w1.next();
      else s1 = s0;
    }
#pragma unroll
    for (int q = 0; q < QA; ++q)
      if (q >= q0 && q < q1) la.issue_one(q, stage, [&](int) -> const BufRes& { return ra; }, k0, K, a.lda);
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (QA + q < q0 || QA + q >= q1) continue;
      if constexpr (BKC) {
        if (split && k0 >= a.b_split)
          lb.issue_one(q, stage + A_BYTES, [&](int) -> const BufRes& { return rb1; }, k0 - (int)a.b_split,
                       K - a.b_split, a.ldb);
        else
          lb.issue_one(q, stage + A_BYTES, [&](int) -> const BufRes& { return rb0; }, k0, split ? a.b_split : K,
                       a.ldb);
      } else {
        lb.issue_one(q, stage + A_BYTES, [&](int p) -> const BufRes& { return (PAIR && p) ? s1 : s0; }, k0, K,
                     a.ldb);
      }
    }
  };

  const int wave = wave_u % NC, lane = threadIdx.x & 63;
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

  const int nk = (int)((K + BK - 1) / BK);
  StageFrags<FM, FN, BK> fr;
  k_loop_pingpong<NS, STAGE, QA + QB>(
      smem, nk, wave_u / (NC / 2), issue,
      [&](const char* st) { read_stage<FM, FN, BK, true, BKC>(st, st + A_BYTES, wm0, bcol, fr); },
      [&]() { mma_frags<FM, FN, BK>(fr, acc); });

  if constexpr (NP == kPingPong && BM == 256 && BN == 256 && WM == 2 && WN == 4 &&
                (EPI == gemm::EPI_STORE || EPI == gemm::EPI_GELU_FWD || EPI == gemm::EPI_SWIGLU_FWD ||
                 EPI == gemm::EPI_STORE_SCATTER || EPI == gemm::EPI_GELU_FWD_H || EPI == gemm::EPI_SWIGLU_FWD_H))
    rows_epilogue_staged<FM, FN, PAIR, EPI>(a, acc, bcol, wave, lane, row_begin, row_end, n0, N, smem);
  else if constexpr (NP == kPingPong && BM == 256 && BN == 256 && WM == 2 && WN == 4 &&
                     (EPI == gemm::EPI_GELU_BWD || EPI == gemm::EPI_SWIGLU_BWD))
    rows_epilogue_staged_bwd<FM, FN, EPI>(a, acc, bcol, wave, lane, row_begin, row_end, n0, N, smem);
  else
    rows_epilogue_t<bf16, FM, FN, PAIR, EPI>(a, acc, bcol, wm0, lane, row_begin, row_end, n0, N);
}

// WGRAD work items (split, group, tile).  The items of groups that have rows
// come first: they take workgroup ids 0 .. nreal-1, remapped over the XCDs,
// so the real work covers every XCD however many groups are empty (remapping
// all items put a skewed routing's few busy groups on two or three XCDs).
// With groups of similar length, each XCD takes consecutive items, whole
// groups, which then share its L2.  When the longest group has more than
// twice the mean rows, whole groups would leave the XCDs that hold the long
// ones working long after the rest, so each group's tiles go instead to the
// 8 XCDs in 8 runs of consecutive tiles (a run still shares one XCD's L2).
// Items of empty groups, which only write zeros, take the ids after the real
// ones.  Returns false for a workgroup past the last item.
__device__ __forceinline__ bool wgrad_item_of(const Args& a, int per_g, int ksplit, int& split, int& g, int& tile,
                                              int64_t& r0, int64_t& r1) {
  // the wave reads the offsets 64 groups at a time; ballots count the groups
  // with rows and find the kth of a kind
  const int lane = (int)(threadIdx.x & 63);
  auto load = [&](int gg, int64_t& lo, int64_t& hi) {
    lo = 0;
    hi = 0;
    if (gg < a.groups) {
      lo = a.offsets[gg];
      hi = a.offsets[gg + 1];
    }
  };
  // (all of it ballots and scalar values: a launch runs many short workgroups
  // one after another on each CU, so this prologue must stay a few cycles)
  int64_t lo0, hi0;  // the first 64 groups, kept for the search below
  load(lane, lo0, hi0);
  const int64_t total = a.offsets[a.groups] - a.offsets[0];  // rows of all groups
  int nz = __popcll(__ballot(hi0 > lo0));
  for (int c = 64; c < a.groups; c += 64) {
    int64_t lo, hi;
    load(c + lane, lo, hi);
    nz += __popcll(__ballot(hi > lo));
  }
  // skewed: some group holds more than twice the mean rows of the groups with rows
  bool skewed = __ballot((hi0 - lo0) * nz > 2 * total) != 0;
  for (int c = 64; c < a.groups; c += 64) {
    int64_t lo, hi;
    load(c + lane, lo, hi);
    skewed = skewed || __ballot((hi - lo) * nz > 2 * total) != 0;
  }
  const int nreal = ksplit * nz * per_g;
  const int hw = (int)blockIdx.x;
  const bool real = hw < nreal;
  const int ng = real ? nz : a.groups - nz;
  const int run = skewed && per_g >= 8 ? per_g / 8 : 0;
  const int lin = !real ? hw - nreal : run > 0 ? run_remap(hw, nreal, run) : xcd_remap(hw, nreal);
  if (ng <= 0 || lin >= ksplit * ng * per_g) return false;
  split = lin / (ng * per_g);
  const int rem = lin - split * ng * per_g;
  int kth = rem / per_g;  // the kth group with (or without) rows
  tile = rem - kth * per_g;
  for (int c = 0; c < a.groups; c += 64) {
    const int gg = c + lane;
    int64_t lo = lo0, hi = hi0;
    if (c > 0) load(gg, lo, hi);
    const uint64_t mask = __ballot(gg < a.groups && (hi > lo) == real);
    const int n = __popcll(mask);
    if (kth < n) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
      const int pos = __ffsll((unsigned long long)__ballot(((mask >> lane) & 1) && below == kth)) - 1;
      g = c + pos;
      auto lane_value = [pos](int64_t v) {  // v of lane pos, wave-uniform
        const uint32_t l = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, pos);
        const uint32_t h = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), pos);
        return (int64_t)(((uint64_t)h << 32) | l);
      };
      r0 = lane_value(lo);
      r1 = lane_value(hi);
      return true;
    }
    kth -= n;
  }
  return false;
}

// ---------------------------------------------------------------------------
// WGRAD: C_g[M, N] = X[rows_g, M]^T . D[rows_g, N], both MN-contiguous.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int BK, int NS, int NP, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm3_wgrad_kernel(Args a) {
  static_assert(NP == kPingPong, "the ping-pong schedule is the one built");
  constexpr int NC = WM * WN;
  constexpr int NW = NC, W0 = 0;
  constexpr int FM = BM / (32 * WM), FN = BN / (32 * WN);
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // EPI_PARTIAL launches split the reduction: an item (split, group, tile)
  // writes the fp32 partial of its split
  constexpr bool SPLIT = EPI == kEpiPartial;
  const int per_g = a.tiles_m * a.tiles_n;
  int split = 0, g = 0, tile = 0;
  int64_t r0 = 0, r1 = 0;
  if (!wgrad_item_of(a, per_g, SPLIT ? a.ksplit : 1, split, g, tile, r0, r1)) return;
  int mt, nt;
  grouped_order(tile, a.tiles_m, a.tiles_n, mt, nt, a.gm);
  const int wi = weight_index(g, a.rr_R, a.rr_L);
  if constexpr (SPLIT) {
    // split s takes rows [r0 + s*chunk, r0 + (s+1)*chunk) of the group, chunk
    // a multiple of BK; a split past the group's rows keeps an empty range
    // and writes zeros
    const int64_t g0 = r0, g1 = r1;
    gemm_addr::split_rows(g0, g1, a.ksplit, split, BK, r0, r1);
  }
  const int64_t Kr = r1 - r0;
  const int64_t M = a.M, N = a.N;
  const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;

  const char* X = reinterpret_cast<const char*>(a.A);
  const char* D = reinterpret_cast<const char*>(a.B);
  // both operands are M/N-contiguous: their resources are rebased at every
  // K stage (rows r0 + k0 ..), so a group of any length keeps 32-bit offsets

  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Loader<BM, BK, false, NW, W0> la;
  Loader<BN, BK, false, NW, W0> lb;
  la.init_mn(a.lda, false, M - m0);
  lb.init_mn(a.ldb, false, N - n0);
  constexpr int QA = Loader<BM, BK, false, NW, W0>::PER, QB = Loader<BN, BK, false, NW, W0>::PER;
  // both operands' K stages, walked in order: every wave issues its share of
  // each stage once, for kt = 0, 1, ...
  StageRes wa, wb;
  wa.init(X, gemm_addr::wgrad_walk(r0, m0, BK, a.lda));
  wb.init(D, gemm_addr::wgrad_walk(r0, n0, BK, a.ldb));
  auto issue = [&](char* stage, int kt, int q0, int q1) {
    const int k0 = kt * BK;
    const BufRes ra = wa.next(), rb = wb.next();
#pragma unroll
    for (int q = 0; q < QA; ++q)
      if (q >= q0 && q < q1) la.issue_one(q, stage, [&](int) -> const BufRes& { return ra; }, k0, Kr, a.lda);
#pragma unroll
    for (int q = 0; q < QB; ++q)
      if (QA + q >= q0 && QA + q < q1)
        lb.issue_one(q, stage + A_BYTES, [&](int) -> const BufRes& { return rb; }, k0, Kr, a.ldb);
  };

  const int wave = wave_u % NC, lane = threadIdx.x & 63;
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

  const int nk = (int)((Kr + BK - 1) / BK);
  StageFrags<FM, FN, BK> fr;
  k_loop_pingpong<NS, STAGE, QA + QB>(
      smem, nk, wave_u / (NC / 2), issue,
      [&](const char* st) { read_stage<FM, FN, BK, false, false>(st, st + A_BYTES, wm0, bcol, fr); },
      [&]() { mma_frags<FM, FN, BK>(fr, acc); });

  if constexpr (SPLIT) {
    // fp32 partial of this split: [split][weight set][M][N]
    Args ap = a;
    ap.C = a.partial + (int64_t)split * a.groups * M * N;
    ap.C2 = nullptr;
    ap.ldc = N;
    ap.c_gstride = M * N;
    if constexpr (NP == kPingPong && BM == 256 && BN == 256 && WM == 2 && WN == 4)
      wgrad_epilogue_staged<float, FM, FN, gemm::EPI_STORE>(ap, acc, bcol, wave, lane, wi, m0, n0, M, N, smem);
    else
      wgrad_epilogue_t<float, FM, FN, gemm::EPI_STORE>(ap, acc, bcol, wm0, lane, wi, m0, n0, M, N);
  } else {
    if constexpr (NP == kPingPong && BM == 256 && BN == 256 && WM == 2 && WN == 4)
      wgrad_epilogue_staged<bf16, FM, FN, EPI>(a, acc, bcol, wave, lane, wi, m0, n0, M, N, smem);
    else
      wgrad_epilogue_t<bf16, FM, FN, EPI>(a, acc, bcol, wm0, lane, wi, m0, n0, M, N);
  }
}

// Sum of the ksplit fp32 partials of a split WGRAD launch, in split order,
// into the weight gradient (columns >= c_split to C2 for EPI_STORE_SPLITN);
// 4 consecutive columns per thread.
__global__ __launch_bounds__(256) void wgrad_split_reduce_kernel(Args a, int epi) {
  const int64_t M = a.M, N = a.N, per = M * N;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;  // over groups x M x N
  if (i >= (int64_t)a.groups * per) return;
  const int64_t wi = i / per, r = i - wi * per, m = r / N, n = r - m * N;
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < a.ksplit; ++s) {
    float p[4];
    Run4<float>::load(a.partial + (int64_t)s * a.groups * per + i, p);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += p[q];
  }
  bf16* C = reinterpret_cast<bf16*>(a.C) + wi * a.c_gstride;
  if (epi == gemm::EPI_STORE_SPLITN && n >= a.c_split) {
    bf16* C2 = reinterpret_cast<bf16*>(a.C2) + wi * a.c_gstride;
    Run4<bf16>::store(C2 + m * a.ldc + (n - a.c_split), v);
  } else {
    Run4<bf16>::store(C + m * a.ldc + n, v);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int BK, int NS, int NP, int KIND, int EPI>
hipError_t launch_rows(Args a, int64_t rows_max, hipStream_t st) {
  constexpr bool PAIR = EPI == gemm::EPI_SWIGLU_FWD || EPI == gemm::EPI_SWIGLU_FWD_H;
  gemm_addr::rows_tiles(a.N, PAIR ? BN / 2 : BN, rows_max, a.groups, BM, a.tiles_m, a.tiles_n);
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = (size_t)NS * (BM + BN) * BK * 2;
  auto kern = gemm3_rows_kernel<BM, BN, WM, WN, BK, NS, NP, KIND, EPI>;
  static hipError_t prep = prepare_lds(kern, lds);
  if (prep != hipSuccess) return prep;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WM * WN), lds, st, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int BK, int NS, int NP, int EPI>
hipError_t launch_wgrad(Args a, hipStream_t st) {
  gemm_addr::wgrad_tiles(a.M, a.N, BM, BN, a.tiles_m, a.tiles_n);
  const int64_t grid = (int64_t)a.groups * a.tiles_m * a.tiles_n * (EPI == kEpiPartial ? a.ksplit : 1);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = (size_t)NS * (BM + BN) * BK * 2;
  auto kern = gemm3_wgrad_kernel<BM, BN, WM, WN, BK, NS, NP, EPI>;
  static hipError_t prep = prepare_lds(kern, lds);
  if (prep != hipSuccess) return prep;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WM * WN), lds, st, a);
  return hipGetLastError();
}

// Tile configuration (BM, BN, WM, WN, BK, NS, NP), from measurements of the
// Mixtral-sized expert GEMMs (d 4096, F 14336): a 256 x 256 tile, 8 waves in
// two ping-pong groups, K-step 32, 4-stage ring, for every kind.  (All 8
// waves in lockstep, 4 MFMA waves fed by 4 load-only waves on 256 x 128
// tiles, and 4-wave 256 x 256 tiles measured slower.)
#define MOE_GEMM3_CFG_PP 256, 256, 2, 4, 32, 4, -1

// Whether the direct-load kernels take this launch: the K split of the SwiGLU
// dgrad (gate | up weights) must fall on a stage boundary.
bool supports(const Args& a) { return a.b_split == 0 || a.b_split % 32 == 0; }

hipError_t run_rows_bf16(int kind, int epi, const Args& a, int64_t rows_max, hipStream_t st) {
  using namespace gemm;
  if (kind == KIND_FWD) {
    switch (epi) {
      case EPI_STORE: return launch_rows<MOE_GEMM3_CFG_PP, KIND_FWD, EPI_STORE>(a, rows_max, st);
      case EPI_GELU_FWD: return launch_rows<MOE_GEMM3_CFG_PP, KIND_FWD, EPI_GELU_FWD>(a, rows_max, st);
      case EPI_SWIGLU_FWD: return launch_rows<MOE_GEMM3_CFG_PP, KIND_FWD, EPI_SWIGLU_FWD>(a, rows_max, st);
      case EPI_STORE_SCATTER: return launch_rows<MOE_GEMM3_CFG_PP, KIND_FWD, EPI_STORE_SCATTER>(a, rows_max, st);
      case EPI_GELU_FWD_H: return launch_rows<MOE_GEMM3_CFG_PP, KIND_FWD, EPI_GELU_FWD_H>(a, rows_max, st);
      case EPI_SWIGLU_FWD_H: return launch_rows<MOE_GEMM3_CFG_PP, KIND_FWD, EPI_SWIGLU_FWD_H>(a, rows_max, st);
      // dgrads over transposed weights (N-contiguous, the forward's loads)
      case EPI_GELU_BWD: return launch_rows<MOE_GEMM3_CFG_PP, KIND_FWD, EPI_GELU_BWD>(a, rows_max, st);
      case EPI_SWIGLU_BWD: return launch_rows<MOE_GEMM3_CFG_PP, KIND_FWD, EPI_SWIGLU_BWD>(a, rows_max, st);
    }
  } else {
    switch (epi) {
      case EPI_STORE: return launch_rows<MOE_GEMM3_CFG_PP, KIND_DGRAD, EPI_STORE>(a, rows_max, st);
      case EPI_GELU_BWD: return launch_rows<MOE_GEMM3_CFG_PP, KIND_DGRAD, EPI_GELU_BWD>(a, rows_max, st);
      case EPI_SWIGLU_BWD: return launch_rows<MOE_GEMM3_CFG_PP, KIND_DGRAD, EPI_SWIGLU_BWD>(a, rows_max, st);
    }
  }
  return hipErrorInvalidValue;
}

// Weights transposed for the backward (forward-kind dgrads): a workgroup
// moves a 64 x 64 tile through LDS, reading 64 rows x 128 bytes and writing
// 64 rows x 128 bytes of the transpose, 16 bytes per thread access.  In LDS
// the tile's rows are unpadded and the 8 16-byte chunks of row r sit in the
// order chunk ^ (r / 8): the 8 lanes of a row write its 128 bytes, and the
// 64 lanes of a column read (8 columns of one chunk x 8 row groups) fall on
// 8 different chunks, 32 different banks.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst, int64_t rows, int64_t cols,
                                                             int64_t sbs, int64_t dbs) {
  using namespace gemm_addr;
  __shared__ __attribute__((aligned(16))) uint16_t t[64 * 64];
  const int tid = (int)threadIdx.x;
  // consecutive workgroups walk 8 row tiles per column tile, so that the
  // ones in flight write 1 KB runs of each transposed row as well as read
  // runs of each source row
  int64_t r0, c0;
  transpose_tile((int)blockIdx.x, rows, cols, r0, c0);
  const uint16_t* s = src + (int64_t)blockIdx.z * sbs;
  uint16_t* d = dst + (int64_t)blockIdx.z * dbs;
  u32x4 v[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // 8-element chunk: tile row tr, columns tc ..
    int tr, tc;
    transpose_load_lane(tid, j, tr, tc);
    const int64_t r = r0 + tr, c = c0 + tc;
    v[j] = u32x4{0u, 0u, 0u, 0u};
    if (r < rows && c < cols) v[j] = ld16(s + r * cols + c);  // rows and cols are multiples of 8
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int tr, tc;
    transpose_load_lane(tid, j, tr, tc);
    *reinterpret_cast<u32x4*>(&t[transpose_lds(tr, tc >> 3)]) = v[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // output chunk: tile column tc, tile rows tr .. tr + 7
    int tc, tr;
    transpose_store_lane(tid, j, tc, tr);
    const uint16_t* col = t + transpose_lds(tr, tc >> 3) + (tc & 7);  // rows tr .. tr + 7 share the chunk order
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)col[(2 * i) * 64] | ((uint32_t)col[(2 * i + 1) * 64] << 16);
    const int64_t c = c0 + tc, r = r0 + tr;
    if (c < cols && r < rows) st16(d + c * rows + r, u32x4{w[0], w[1], w[2], w[3]});
  }
}

hipError_t transpose_bf16(const void* src, void* dst, int64_t batches, int64_t rows, int64_t cols,
                          int64_t src_bstride, int64_t dst_bstride, hipStream_t st) {
  if (batches <= 0 || rows <= 0 || cols <= 0) return hipSuccess;
  if (rows % 8 || cols % 8 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return hipErrorInvalidValue;
  const int64_t gx = (cols + 63) / 64, gy = (rows + 63) / 64;
  if (gx * gy > 0x7fffffff / 8 || batches > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(gx * gy), 1, (unsigned)batches), dim3(256), 0, st,
                     (const uint16_t*)src, (uint16_t*)dst, rows, cols, src_bstride, dst_bstride);
  return hipGetLastError();
}

int wgrad_ksplit(int64_t groups, int64_t M, int64_t N, int64_t rows_max) {
  return gemm_addr::wgrad_ksplit(groups, M, N, rows_max);
}

hipError_t run_wgrad_bf16(int epi, const Args& a, hipStream_t st) {
  using namespace gemm;
  if (a.ksplit > 1) {
    if (!a.partial || (epi != EPI_STORE && epi != EPI_STORE_SPLITN)) return hipErrorInvalidValue;
    hipError_t e = launch_wgrad<MOE_GEMM3_CFG_PP, kEpiPartial>(a, st);
    if (e != hipSuccess) return e;
    const int64_t n4 = (int64_t)a.groups * a.M * a.N / 4;  // N is a multiple of 8
    hipLaunchKernelGGL(wgrad_split_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a, epi);
    return hipGetLastError();
  }
  if (epi == EPI_STORE) return launch_wgrad<MOE_GEMM3_CFG_PP, EPI_STORE>(a, st);
  if (epi == EPI_STORE_SPLITN) return launch_wgrad<MOE_GEMM3_CFG_PP, EPI_STORE_SPLITN>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace gemm3
}  // namespace moe
