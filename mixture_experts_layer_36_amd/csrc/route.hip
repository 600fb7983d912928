// Gate GEMM + softmax + top-k routing (tutorial ch.4, 专家并行 二 step 1:
// every device scores its local tokens with the replicated router g(x);
// 用于分布式 MoE 的主流框架与库: a top-k gate with k chosen experts).
//
// A workgroup owns 64 tokens, one per lane, and its W waves (16, or 8 for more
// than 16 experts) split the model width: wave w takes the 128-byte column
// chunks w, w+W, w+2W, ... of the tokens' rows.  Per chunk the wave loads the
// 64 rows coalesced (8 lanes per 128-byte row piece), transposes them through its own slice of LDS (XOR
// swizzled, so both the writes and the per-lane row reads are free of bank
// conflicts) and then each lane holds 64 consecutive bf16 (or 32 fp32) values
// of its own token.  The router weight rows of the chunk are the same for
// every lane, so they come in through wave-uniform scalar loads and feed the
// dot products straight from scalar registers: bf16 uses the two-term
// fp32-accumulating dot instruction on (x[k], x[k+1]) . (W[k][e], W[k+1][e]),
// with the weight pairs packed once per call into a workspace copy so that
// each pair is one scalar dword; fp32 uses plain FMAs on W itself.  The W per-wave partial logits are then summed in a fixed
// binary tree through LDS, so the logits are deterministic.  Lane t of wave 0
// finally holds all logits of its token and does the softmax statistics and
// the k rounds of arg-max sequentially, ordering by (logit descending, expert
// index ascending): equal logits go to the lower index.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRouteTokens = 64;

// Waves per workgroup: more waves hide more load latency; wide rows (E > 16)
// need more registers per wave, so fewer of them fit.
template <int EP> constexpr int route_waves() { return EP <= 16 ? 16 : 8; }
template <int EP> constexpr size_t route_lds() {
  constexpr size_t stage = (size_t)route_waves<EP>() * kRouteTokens * 128;
  constexpr size_t red = (size_t)(route_waves<EP>() / 2) * EP * kRouteTokens * 4;
  return stage > red ? stage : red;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Router weight pair (W[k][e], W[k+1][e]) for even k, from the packed copy
// wp[k/2][e] (one dword of two bf16) that pack_router_pairs_kernel writes.
template <int EP, bool FULL>
__device__ __forceinline__ uint32_t w_pair(const uint32_t* __restrict__ wp, int k, int e, int E) {
  if constexpr (FULL) {
    return wp[(k >> 1) * EP + e];
  } else {
    const uint32_t v = wp[(k >> 1) * E + (e < E ? e : E - 1)];
    return e < E ? v : 0u;
  }
}

template <int EP, bool FULL>
__device__ __forceinline__ float w_f32(const float* __restrict__ w, int k, int e, int E) {
  const int En = FULL ? EP : E;
  const int ee = FULL ? e : (e < E ? e : E - 1);
  const float v = w[k * En + ee];
  return (FULL || e < E) ? v : 0.0f;
}

// Software-pipelined bf16 path for E equal to its padded width.  The packed
// weight pairs of one 16-byte piece of x (4 pairs x EP experts) are fetched in
// 32-dword units (an even number per piece, pairs-major) into two alternating
// scalar-register buffers.  Scalar loads return out of order, so a step first
// waits for everything outstanding, then issues the next unit's loads and,
// at a piece's first unit, the LDS read of the next piece, and only then
// computes from the unit that has already arrived.
template <int EP>
struct PairUnit {
  static constexpr int DW = 32;                       // dwords per unit
  static constexpr int EPU = EP < DW ? EP : DW;       // experts per unit
  static constexpr int PPU = DW / EPU;                // pairs per unit
  static constexpr int UPP = 4 / PPU * (EP / EPU);    // units per piece
};

__device__ __forceinline__ void wait_lgkm_all() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

template <int EP>
__device__ __forceinline__ void load_unit(const uint32_t* __restrict__ wp, int k0, int v,
                                          uint32_t (&b)[PairUnit<EP>::DW]) {
  using U = PairUnit<EP>;
  constexpr int EG = EP / U::EPU;
  const int pq = v / EG, eg = v % EG;
#pragma unroll
  for (int p = 0; p < U::PPU; ++p) {
    const uint32_t* row = wp + ((k0 >> 1) + pq * U::PPU + p) * EP + eg * U::EPU;
#pragma unroll
    for (int i = 0; i < U::EPU; ++i) b[p * U::EPU + i] = row[i];
  }
}

template <int EP>
__device__ __forceinline__ void compute_unit(const u32x4& xj, int v, const uint32_t (&b)[PairUnit<EP>::DW],
                                             float (&acc)[EP]) {
  using U = PairUnit<EP>;
  constexpr int EG = EP / U::EPU;
  const int pq = v / EG, eg = v % EG;
#pragma unroll
  for (int p = 0; p < U::PPU; ++p) {
    // through a scalar: this compiler's bit_cast of a vector element
    // expression reads element 0 whatever the index
    const uint32_t xu = xj[pq * U::PPU + p];
    const bf16x2_t xp = __builtin_bit_cast(bf16x2_t, xu);
#pragma unroll
    for (int i = 0; i < U::EPU; ++i) {
      const int e = eg * U::EPU + i;
      acc[e] = __builtin_amdgcn_fdot2_f32_bf16(xp, __builtin_bit_cast(bf16x2_t, b[p * U::EPU + i]), acc[e], false);
    }
  }
}

// All pieces of one chunk; piece j of the lane's row is at slot j ^ (lane % 8)
// of its 128-byte LDS row.  Past the last piece the prefetches repeat the last
// one (in range, unused), which keeps them unconditional.
template <int EP>
__device__ __forceinline__ void chunk_pipelined(const uint32_t* __restrict__ wp, const char* lrow, int lane, int kb,
                                                int npiece, float (&acc)[EP]) {
  using U = PairUnit<EP>;
  static_assert(U::UPP % 2 == 0, "buffers alternate within a piece");
  uint32_t wa[U::DW], wb[U::DW];
  u32x4 xcur = ld16(lrow + ((0 ^ (lane & 7)) << 4)), xnext = xcur;
  load_unit<EP>(wp, kb, 0, wa);
  for (int j = 0; j < npiece; ++j) {
    const int k0 = kb + 8 * j;
    const int jn = min(j + 1, npiece - 1);
#pragma unroll
    for (int v = 0; v < U::UPP; ++v) {
      wait_lgkm_all();
      __builtin_amdgcn_sched_barrier(0);
      // next unit: (j, v + 1), or (jn, 0) after the piece's last unit
      if (v + 1 < U::UPP) load_unit<EP>(wp, k0, v + 1, (v & 1) ? wa : wb);
      else load_unit<EP>(wp, kb + 8 * jn, 0, (v & 1) ? wa : wb);
      if (v == 0) xnext = ld16(lrow + ((jn ^ (lane & 7)) << 4));
      __builtin_amdgcn_sched_barrier(0);
      compute_unit<EP>(xcur, v, (v & 1) ? wb : wa, acc);
    }
    xcur = xnext;
  }
}

}  // namespace

// wp[k/2][e] = W[k][e] | W[k+1][e] << 16 for even k (d is even).
__global__ __launch_bounds__(256) void pack_router_pairs_kernel(const uint16_t* __restrict__ w,
                                                                uint32_t* __restrict__ wp, int d, int E) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)(d / 2) * E;
  if (i >= n) return;
  const int64_t kp = i / E, e = i - kp * E;
  wp[i] = (uint32_t)w[2 * kp * E + e] | ((uint32_t)w[(2 * kp + 1) * E + e] << 16);
}

template <typename T, int EP, bool FULL>
__global__ __launch_bounds__(route_waves<EP>() * 64) void route_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                                       const uint32_t* __restrict__ wpack,
                                                                const float* __restrict__ bias,
                                                                float* __restrict__ logits,
                                                                int32_t* __restrict__ topk_idx,
                                                                float* __restrict__ topk_w, int64_t Tn, int d, int E,
                                                                int k, int gating) {
  constexpr int KC = 128 / sizeof(T);  // elements of a 128-byte row piece
  constexpr int kRouteWaves = route_waves<EP>();
  constexpr int STAGE = kRouteTokens * 128;
  extern __shared__ __attribute__((aligned(16))) char lds[];  // route_lds<EP>() bytes

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * kRouteTokens;
  char* stage = lds + wave * STAGE;
  const int nchunks = (d + KC - 1) / KC;

  // load r of a chunk: lanes 8r'..8r'+7 cover the 128-byte piece of token
  // 8r + r', lane l taking its 16-byte part l % 8.
  const int sub = lane & 7, trow = lane >> 3;
  auto load_chunk = [&](int c, u32x4 (&v)[8]) {
    const int col = c * KC + sub * (16 / (int)sizeof(T));
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t t = t0 + r * 8 + trow;
      v[r] = (t < Tn && col < d) ? ld16(x + t * d + col) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.0f;

  u32x4 nx[8];
  int c = wave;
  if (c < nchunks) load_chunk(c, nx);
  for (; c < nchunks; c += kRouteWaves) {
    u32x4 cur[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) cur[r] = nx[r];
    if (c + kRouteWaves < nchunks) load_chunk(c + kRouteWaves, nx);
    // transpose through LDS: row = token, 16-byte slot swizzled by row % 8
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = r * 8 + trow;
      st16(stage + row * 128 + ((sub ^ (row & 7)) << 4), cur[r]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // piece j of the lane's own row: 16 bytes = 4 dwords of x, each a pair
    // (bf16) or a single value (fp32); the pieces are read one at a time so
    // that every register index is static.
    const int kb = c * KC;
    const int npiece = min(KC, d - kb) / (16 / (int)sizeof(T));  // d is a multiple of 8
    // pipelined weight units for E >= 16; with 8 experts a piece's weights
    // are only 32 dwords and the plain loop measured faster
    if constexpr (FULL && sizeof(T) == 2 && EP >= 16) {
      chunk_pipelined<EP>(wpack, stage + lane * 128, lane, kb, npiece, acc);
    } else {
#pragma unroll 2
    for (int j = 0; j < npiece; ++j) {
      const u32x4 xj = ld16(stage + lane * 128 + ((j ^ (lane & 7)) << 4));
      if constexpr (sizeof(T) == 2) {
        const uint32_t* wd = wpack;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kk = kb + 8 * j + 2 * q;
          // through a scalar: this compiler's bit_cast of a vector element
          // expression reads element 0 whatever the index
          const uint32_t xu = xj[q];
          const bf16x2_t xp = __builtin_bit_cast(bf16x2_t, xu);
#pragma unroll
          for (int e = 0; e < EP; ++e) {
            const bf16x2_t wp = __builtin_bit_cast(bf16x2_t, w_pair<EP, FULL>(wd, kk, e, E));
            acc[e] = __builtin_amdgcn_fdot2_f32_bf16(xp, wp, acc[e], false);
          }
          // wide rows: keep one pair's weight rows live in scalar registers
          if constexpr (EP >= 32) __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        const float* wf = reinterpret_cast<const float*>(w);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kk = kb + 4 * j + q;
          const float xv = __uint_as_float(xj[q]);
#pragma unroll
          for (int e = 0; e < EP; ++e) acc[e] = fmaf(xv, w_f32<EP, FULL>(wf, kk, e, E), acc[e]);
          if constexpr (EP >= 32) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    }
    // the next chunk's LDS writes stay behind this chunk's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // fixed-order tree sum of the per-wave partial logits
  float* red = reinterpret_cast<float*>(lds);
  __syncthreads();
#pragma unroll
  for (int h = kRouteWaves / 2; h >= 1; h >>= 1) {
    if (wave >= h && wave < 2 * h) {
#pragma unroll
      for (int e = 0; e < EP; ++e) red[((wave - h) * EP + e) * kRouteTokens + lane] = acc[e];
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[e] += red[(wave * EP + e) * kRouteTokens + lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;
  const int64_t t = t0 + lane;
  if (t >= Tn) return;

  float lv[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    const bool ok = FULL || e < E;
    lv[e] = ok ? acc[e] + (bias ? bias[e] : 0.0f) : -INFINITY;
  }
  float* lrow = logits + t * E;
  if constexpr (FULL) {
#pragma unroll
    for (int e = 0; e < EP; e += 4) st16(lrow + e, u32x4{__float_as_uint(lv[e]), __float_as_uint(lv[e + 1]),
                                                          __float_as_uint(lv[e + 2]), __float_as_uint(lv[e + 3])});
  } else {
#pragma unroll
    for (int e = 0; e < EP; ++e)
      if (e < E) lrow[e] = lv[e];
  }

  // softmax statistics over all experts of the token
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < EP; ++e) mx = fmaxf(mx, lv[e]);
  float z = 0.0f;
#pragma unroll
  for (int e = 0; e < EP; ++e)
    if (FULL || e < E) z += __expf(lv[e] - mx);

  // k rounds of arg-max by (value desc, index asc): a strictly greater value
  // replaces the running best while scanning upwards in the index
  uint64_t taken = 0;
  float sel_v[8];
  int sel_e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel_v[j] = -INFINITY;
    sel_e[j] = 0;
    if (j < k) {
      float bv = -INFINITY;
      int be = -1;
#pragma unroll
      for (int e = 0; e < EP; ++e) {
        const bool ok = (FULL || e < E) && !((taken >> e) & 1u);
        if (ok && (be < 0 || lv[e] > bv)) {
          bv = lv[e];
          be = e;
        }
      }
      if (be >= 0) taken |= (uint64_t)1 << be;
      sel_v[j] = bv;
      sel_e[j] = be;
    }
  }

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

template <typename T, int EP>
static hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  const int64_t blocks = (a.T + kRouteTokens - 1) / kRouteTokens;
  if (blocks <= 0) return hipSuccess;
  constexpr size_t lds = route_lds<EP>();
  auto kern = a.E == EP ? route_kernel<T, EP, true> : route_kernel<T, EP, false>;
  static const hipError_t prep_full = hipFuncSetAttribute(
      reinterpret_cast<const void*>(route_kernel<T, EP, true>), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  static const hipError_t prep_part = hipFuncSetAttribute(
      reinterpret_cast<const void*>(route_kernel<T, EP, false>), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (prep_full != hipSuccess) return prep_full;
  if (prep_part != hipSuccess) return prep_part;
  if constexpr (sizeof(T) == 2) {
    const int64_t n = (int64_t)(a.d / 2) * a.E;
    hipLaunchKernelGGL(pack_router_pairs_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const uint16_t*)a.w, a.wpack, a.d, a.E);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(route_waves<EP>() * 64), lds, st, (const T*)a.x,
                     (const T*)a.w, a.wpack, a.bias, a.logits, a.topk_idx, a.topk_w, a.T, a.d, a.E, a.k,
                     a.gating);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_route_dt(const RouteArgs& a, hipStream_t st) {
  if (a.E <= 8) return launch_route_t<T, 8>(a, st);
  if (a.E <= 16) return launch_route_t<T, 16>(a, st);
  if (a.E <= 32) return launch_route_t<T, 32>(a, st);
  return launch_route_t<T, 64>(a, st);
}

hipError_t launch_route(const RouteArgs& a, bool bf16_dtype, hipStream_t st) {
  return bf16_dtype ? launch_route_dt<bf16>(a, st) : launch_route_dt<float>(a, st);
}

}  // namespace moe
