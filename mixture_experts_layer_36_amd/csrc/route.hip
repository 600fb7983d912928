// Gate GEMM + softmax + top-k routing (tutorial ch.4, 专家并行 二 step 1:
// every device scores its local tokens with the replicated router g(x);
// 用于分布式 MoE 的主流框架与库: a top-k gate with k chosen experts).
//
// bf16: the gate GEMM runs on MFMA (route_mfma_kernel, below).
//
// fp32: a workgroup owns 64 tokens, one per lane, and its W waves (16, or 8
// for more than 16 experts) split the model width: wave w takes the 128-byte
// column chunks w, w+W, w+2W, ... of the tokens' rows.  Per chunk the wave
// loads the 64 rows coalesced (8 lanes per 128-byte row piece) and transposes
// them through its own slice of LDS (XOR swizzled, so both the writes and the
// per-lane row reads are free of bank conflicts); each lane then holds 32
// consecutive values of its own token.  The router weight rows of the chunk
// are the same for every lane, so they come in through wave-uniform scalar
// loads and feed FMAs straight from scalar registers.
//
// Both kernels sum their per-wave partial logits in a fixed binary tree
// through LDS, so the logits are deterministic.  One lane per token then does
// the softmax statistics and the k rounds of arg-max sequentially, ordering by
// (logit descending, expert index ascending): equal logits go to the lower
// index.
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

template <int EP, bool FULL>
__device__ __forceinline__ float w_f32(const float* __restrict__ w, int k, int e, int E) {
  const int En = FULL ? EP : E;
  const int ee = FULL ? e : (e < E ? e : E - 1);
  const float v = w[k * En + ee];
  return (FULL || e < E) ? v : 0.0f;
}

}  // namespace

// Per-token end of routing, for the lane that holds the EP summed products
// acc[e] = x[t] . W[:, e] of token t: bias, logits row, softmax statistics
// and the k rounds of arg-max by (value desc, index asc), then the gate
// weights.
template <int EP, bool FULL>
__device__ __forceinline__ void finish_token(const float (&acc)[EP], int64_t t, int E, int k, int gating,
                                             const float* __restrict__ bias, float* __restrict__ logits,
                                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
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

template <typename T, int EP, bool FULL>
__global__ __launch_bounds__(route_waves<EP>() * 64) void route_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                                       const float* __restrict__ bias,
                                                                       float* __restrict__ logits,
                                                                       int32_t* __restrict__ topk_idx,
                                                                       float* __restrict__ topk_w, int64_t Tn, int d,
                                                                       int E, int k, int gating) {
  static_assert(sizeof(T) == 4, "the bf16 gate GEMM runs on MFMA (route_mfma_kernel)");
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

    // piece j of the lane's own row: 16 bytes = 4 fp32 values of x; the
    // pieces are read one at a time so that every register index is static.
    const int kb = c * KC;
    const int npiece = min(KC, d - kb) / 4;  // d is a multiple of 8
    const float* wf = reinterpret_cast<const float*>(w);
#pragma unroll 2
    for (int j = 0; j < npiece; ++j) {
      const u32x4 xj = ld16(stage + lane * 128 + ((j ^ (lane & 7)) << 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = kb + 4 * j + q;
        const float xv = __uint_as_float(xj[q]);
#pragma unroll
        for (int e = 0; e < EP; ++e) acc[e] = fmaf(xv, w_f32<EP, FULL>(wf, kk, e, E), acc[e]);
        if constexpr (EP >= 32) __builtin_amdgcn_sched_barrier(0);
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

  finish_token<EP, FULL>(acc, t, E, k, gating, bias, logits, topk_idx, topk_w);
}


// ---------------------------------------------------------------------------
// bf16: the gate GEMM on MFMA.  logits = x W_r is a [T x d] . [d x EP]
// product with EP = E rounded up to 16; v_mfma_f32_16x16x32_bf16 (fp32
// accumulation) multiplies a 16-token x 32-K block of x by a 32-K x 16-expert
// block of W_r.  Its A operand is x itself: lane l holds 8 consecutive K
// (16 bytes) of token row l % 16 at K offset 8 (l / 16), loaded straight from
// global memory.  W_r is re-packed once per call into the B operand's lane
// order, so each B block is one 16-byte load per lane:
//   wf[(kb * NB + nb) * 64 + l] = W[32 kb + 8 (l / 16) + 0..7][16 nb + l % 16]
// (zero past d and past E).  The accumulator block holds expert 16 nb + l % 16
// of tokens 4 (l / 16) + 0..3.
// ---------------------------------------------------------------------------
constexpr int kMfmaWaves = 8;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void pack_router_frags_kernel(const uint16_t* __restrict__ w,
                                                                u32x4* __restrict__ wf, int d, int E, int NB) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (kb, nb, lane)
  const int nkb = (d + 31) / 32;
  if (i >= (int64_t)nkb * NB * 64) return;
  const int l = (int)(i & 63), nb = (int)((i >> 6) % NB), kb = (int)((i >> 6) / NB);
  const int e = 16 * nb + (l & 15), k0 = 32 * kb + 8 * (l >> 4);
  uint32_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ka = k0 + 2 * q, kb2 = ka + 1;
    const uint32_t lo = (e < E && ka < d) ? w[(int64_t)ka * E + e] : 0u;
    const uint32_t hi = (e < E && kb2 < d) ? w[(int64_t)kb2 * E + e] : 0u;
    v[q] = lo | (hi << 16);
  }
  wf[i] = u32x4{v[0], v[1], v[2], v[3]};
}

// A workgroup owns 16 TG tokens; its 8 waves take every 8th 32-K block, each
// keeping the x and W blocks of the next P K blocks in flight.  The waves' accumulators are summed in a
// fixed binary tree through LDS (deterministic logits), wave 0 spreads them
// to a [16 TG][EP] table and lane t finishes token t.
template <int EP, int TG, int PER, int P>
__global__ __launch_bounds__(kMfmaWaves * 64) void route_mfma_kernel(
    const bf16* __restrict__ x, const u32x4* __restrict__ wf, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int64_t Tn, int d,
    int E, int k, int gating) {
  constexpr int NB = EP / 16, TOK = 16 * TG, NACC = TG * NB * 4;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * TOK;
  const int nkb = (d + 31) / 32;
  // wave w takes the 32-K blocks w, w + 8, w + 16, ...: at any time the 8
  // waves read neighbouring 64-byte pieces of the same rows
  const int nw = wave < nkb ? (nkb - wave + kMfmaWaves - 1) / kMfmaWaves : 0;  // blocks of this wave

  // this lane's x rows: token t0 + 16 tg + lane % 16 (row t0 when past T),
  // K offset 8 (lane / 16) within each 32-K block
  const int g = lane >> 4;
  const bf16* xr[TG];
  bool tok_ok[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int64_t t = t0 + 16 * tg + (lane & 15);
    tok_ok[tg] = t < Tn;
    xr[tg] = x + (tok_ok[tg] ? t : t0) * d;
  }
  // K block kb of this wave's range, clamped: blocks past the range load the
  // last one again with a zero x operand (no branch around the loads)
  auto load = [&](int i, u32x4 (&a)[TG], u32x4 (&b)[NB]) {
    const bool kin = i < nw;
    const int kc = wave + kMfmaWaves * (kin ? i : nw - 1);
    const int kx = 32 * kc + 8 * g;
    const bool kok = kin && kx < d;  // d is a multiple of 8: a piece is all in or all out
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const u32x4 v = ld16(xr[tg] + (kx < d ? kx : 0));  // masked pieces load the row start
      a[tg] = (kok && tok_ok[tg]) ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[nb] = wf[((int64_t)kc * NB + nb) * 64 + lane];
  };

  f32x4 acc[TG][NB];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[tg][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // the wave's K blocks in fully unrolled chunks of PER: straight-line code,
  // loads P blocks ahead of their MFMAs, no loop-carried load registers (a
  // rotating register buffer across loop iterations makes the compiler copy
  // it and wait for every load)
  for (int c0 = 0; c0 < nw; c0 += PER) {
    u32x4 a[PER][TG], b[PER][NB];
#pragma unroll
    for (int i = 0; i < P && i < PER; ++i) load(c0 + i, a[i], b[i]);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[tg][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i][tg]),
                                                                __builtin_bit_cast(bf16x8, b[i][nb]), acc[tg][nb], 0,
                                                                0, 0);
      if (i + P < PER) load(c0 + i + P, a[i + P], b[i + P]);
    }
  }

  // fixed-order tree sum of the waves' accumulators
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int h = kMfmaWaves / 2; h >= 1; h >>= 1) {
    if (wave >= h && wave < 2 * h) {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) red[((wave - h) * NACC + (tg * NB + nb) * 4 + q) * 64 + lane] = acc[tg][nb][q];
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[tg][nb][q] += red[(wave * NACC + (tg * NB + nb) * 4 + q) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;
  // accumulator (tg, nb)[q] of lane l: token 16 tg + 4 (l / 16) + q, expert 16 nb + l % 16
  float* tab = red;  // [TOK][EP], reused: only wave 0 is left
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) tab[(16 * tg + 4 * g + q) * EP + 16 * nb + (lane & 15)] = acc[tg][nb][q];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int64_t t = t0 + lane;
  if (lane >= TOK || t >= Tn) return;
  float lv[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) lv[e] = tab[lane * EP + e];
  if (E == EP) finish_token<EP, true>(lv, t, E, k, gating, bias, logits, topk_idx, topk_w);
  else finish_token<EP, false>(lv, t, E, k, gating, bias, logits, topk_idx, topk_w);
}

template <int EP, int TG>
static hipError_t launch_route_mfma(const RouteArgs& a, hipStream_t st) {
  const int64_t blocks = (a.T + 16 * TG - 1) / (16 * TG);
  if (blocks <= 0) return hipSuccess;
  constexpr int NB = EP / 16;
  const int64_t nfrag = (int64_t)((a.d + 31) / 32) * NB * 64;
  hipLaunchKernelGGL(pack_router_frags_kernel, dim3((unsigned)((nfrag + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)a.w, (u32x4*)a.wpack, a.d, a.E, NB);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  constexpr size_t red = (size_t)(kMfmaWaves / 2) * TG * NB * 4 * 64 * 4;
  constexpr size_t tab = (size_t)16 * TG * EP * 4;
  constexpr size_t lds = red > tab ? red : tab;
  constexpr int P = EP == 16 ? 4 : 2;  // K blocks in flight per wave
  const int per = ((a.d + 31) / 32 + kMfmaWaves - 1) / kMfmaWaves;  // most K blocks of a wave
#define MOE_ROUTE_MFMA(PER)                                                                                     \
  hipLaunchKernelGGL((route_mfma_kernel<EP, TG, PER, P>), dim3((unsigned)blocks), dim3(kMfmaWaves * 64), lds, st, \
                     (const bf16*)a.x, (const u32x4*)a.wpack, a.bias, a.logits, a.topk_idx, a.topk_w, a.T, a.d,   \
                     a.E, a.k, a.gating)
  if (per <= 4) MOE_ROUTE_MFMA(4);
  else if (per <= 8) MOE_ROUTE_MFMA(8);
  else if (per <= 16) MOE_ROUTE_MFMA(16);
  else MOE_ROUTE_MFMA(32);  // wider models loop over chunks of 32
#undef MOE_ROUTE_MFMA
  return hipGetLastError();
}

// expert width the bf16 route pads E to (its launch instantiations)
static int route_mfma_ep(int64_t E) { return E <= 16 ? 16 : E <= 32 ? 32 : 64; }

// bytes of the re-packed router weights that the bf16 route writes to ws
size_t route_ws_bytes(int64_t d, int64_t E) { return (size_t)((d + 31) / 32) * (route_mfma_ep(E) / 16) * 64 * 16; }

template <int EP>
static hipError_t launch_route_f32(const RouteArgs& a, hipStream_t st) {
  const int64_t blocks = (a.T + kRouteTokens - 1) / kRouteTokens;
  if (blocks <= 0) return hipSuccess;
  constexpr size_t lds = route_lds<EP>();
  auto kern = a.E == EP ? route_kernel<float, EP, true> : route_kernel<float, EP, false>;
  static const hipError_t prep_full = hipFuncSetAttribute(
      reinterpret_cast<const void*>(route_kernel<float, EP, true>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)lds);
  static const hipError_t prep_part = hipFuncSetAttribute(
      reinterpret_cast<const void*>(route_kernel<float, EP, false>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)lds);
  if (prep_full != hipSuccess) return prep_full;
  if (prep_part != hipSuccess) return prep_part;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(route_waves<EP>() * 64), lds, st, (const float*)a.x,
                     (const float*)a.w, a.bias, a.logits, a.topk_idx, a.topk_w, a.T, a.d, a.E, a.k, a.gating);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, bool bf16_dtype, hipStream_t st) {
  if (!bf16_dtype) {
    if (a.E <= 8) return launch_route_f32<8>(a, st);
    if (a.E <= 16) return launch_route_f32<16>(a, st);
    if (a.E <= 32) return launch_route_f32<32>(a, st);
    return launch_route_f32<64>(a, st);
  }
  switch (route_mfma_ep(a.E)) {
    case 16: return launch_route_mfma<16, 2>(a, st);
    case 32: return launch_route_mfma<32, 4>(a, st);
    default: return launch_route_mfma<64, 4>(a, st);
  }
}

}  // namespace moe
