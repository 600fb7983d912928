// Gate GEMM + softmax + top-k routing (tutorial ch.4, 专家并行 二 step 1:
// every device scores its local tokens with the replicated router g(x);
// 用于分布式 MoE 的主流框架与库: a top-k gate with k chosen experts).
//
// bf16: the gate GEMM runs on MFMA: route_stream_kernel for up to 16
// experts and d up to 4096, route_mfma_kernel otherwise (both below).
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
// Every kernel sums its per-wave partial logits in a fixed order through
// LDS, so the logits are deterministic.  The softmax statistics and the k
// rounds of arg-max order by (logit descending, expert index ascending):
// equal logits go to the lower index.  route_stream_kernel spreads a token
// over four lanes and combines them with quad shuffles; the other kernels
// give each token one lane.
#include "common.h"
#include "kernels.h"
#include "stream.h"

#include <algorithm>
#include <atomic>

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

// The value of the partner lane of step S of an all-reduce over groups of L
// lanes (L = 4, 8 or 16), by DPP within each row of 16 lanes: step 0 takes
// lane l ^ 1, step 1 lane l ^ 2 (quad permutations [1, 0, 3, 2] and
// [2, 3, 0, 1]), step 2 the mirror within 8 lanes (quad 0 with quad 1) and
// step 3 the mirror within 16 (the two groups of 8).  After steps 0 .. log2 L
// - 1, combining with a commutative operation, every lane of a group holds
// the same result.
template <int S>
__device__ __forceinline__ int group_step(int v) {
  constexpr int ctrl = S == 0 ? 0xB1 : S == 1 ? 0x4E : S == 2 ? 0x141 : 0x140;
  return __builtin_amdgcn_update_dpp(0, v, ctrl, 0xF, 0xF, false);
}
template <int S>
__device__ __forceinline__ float group_step(float v) {
  return __int_as_float(group_step<S>(__float_as_int(v)));
}
template <int L> constexpr int group_steps() { return L == 4 ? 2 : L == 8 ? 3 : 4; }

// (value, expert) of the better of two candidates: the larger value, then
// the lower expert index
__device__ __forceinline__ void better_of(float& v, int& e, float ov, int oe) {
  if (ov > v || (ov == v && oe < e)) {
    v = ov;
    e = oe;
  }
}

// End of routing for a token spread over a group of L lanes (L = 4, 8 or 16),
// four experts per lane: lane part p = lane % L holds the summed products of
// token t for experts e0 .. e0 + 3, e0 = 4 p, and the same bias entries in
// bq.  The same results as finish_token: bias, logits row, softmax
// statistics, k rounds of arg-max by (value desc, index asc), gate weights;
// the statistics and each round's pick are combined over the group's lanes
// with DPP (group_step).  Round j's pick is stored by part j % L.
template <int L>
__device__ __forceinline__ void finish_group(const f32x4& acc, const float (&bq)[4], int64_t t, int64_t Tn, int e0,
                                             int E, int k, int gating, float* __restrict__ logits,
                                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int NS = group_steps<L>(), SLOTS = (8 + L - 1) / L;
  float v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = e0 + c < E ? acc[c] + bq[c] : -INFINITY;
  const bool live = t < Tn;
  if (live) {
    float* lrow = logits + t * E + e0;
    if ((E & 3) == 0) {
      if (e0 < E) st16(lrow, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                   __float_as_uint(v[3])});
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (e0 + c < E) lrow[c] = v[c];
    }
  }
  // softmax statistics over the token's experts
  float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
  mx = fmaxf(mx, group_step<0>(mx));
  mx = fmaxf(mx, group_step<1>(mx));
  if constexpr (NS > 2) mx = fmaxf(mx, group_step<2>(mx));
  if constexpr (NS > 3) mx = fmaxf(mx, group_step<3>(mx));
  float z = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (e0 + c < E) z += __expf(v[c] - mx);
  z += group_step<0>(z);
  z += group_step<1>(z);
  if constexpr (NS > 2) z += group_step<2>(z);
  if constexpr (NS > 3) z += group_step<3>(z);

  // k rounds of arg-max; every lane of the token sees each round's pick
  const int part = e0 >> 2;
  unsigned taken = 0;
  int my_e[SLOTS];
  float my_v[SLOTS];
#pragma unroll
  for (int r = 0; r < SLOTS; ++r) {
    my_e[r] = 0;
    my_v[r] = 0.0f;
  }
  float v0 = 0.0f, den = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      float bv = -INFINITY;
      int be = 1 << 30;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (e0 + c < E && !((taken >> c) & 1u) && (be == (1 << 30) || v[c] > bv)) {
          bv = v[c];
          be = e0 + c;
        }
      better_of(bv, be, group_step<0>(bv), group_step<0>(be));
      better_of(bv, be, group_step<1>(bv), group_step<1>(be));
      if constexpr (NS > 2) better_of(bv, be, group_step<2>(bv), group_step<2>(be));
      if constexpr (NS > 3) better_of(bv, be, group_step<3>(bv), group_step<3>(be));
      if (be >= e0 && be < e0 + 4) taken |= 1u << (be - e0);
      if (j == 0) v0 = bv;
      den += __expf(bv - v0);
      if (j % L == part) {
        my_e[j / L] = be;
        my_v[j / L] = bv;
      }
    }
  }
  if (!live) return;
#pragma unroll
  for (int r = 0; r < SLOTS; ++r) {
    const int j = L * r + part;
    if (j < k) {
      const float gw = gating == 0 ? __expf(my_v[r] - mx) / z : __expf(my_v[r] - v0) / den;
      topk_idx[t * k + j] = my_e[r];
      topk_w[t * k + j] = gw;
    }
  }
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
  // accumulator (tg, nb)[q] of wave 0's lane l: token 16 tg + 4 (l / 16) + q,
  // expert 16 nb + l % 16, spread into a [16 TG][EP] table
  float* tab = red;  // reused: the tree's reads are done
  if (wave == 0) {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) tab[(16 * tg + 4 * g + q) * EP + 16 * nb + (lane & 15)] = acc[tg][nb][q];
  }
  __syncthreads();
  // every wave finishes tokens, L = EP / 4 lanes per token (four experts a
  // lane), 64 / L tokens per pass
  constexpr int L = EP / 4, TPP = 64 / L, PASSES = TOK / TPP;
  const int e0 = 4 * (lane % L);
  float bq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bq[c] = (bias && e0 + c < E) ? bias[e0 + c] : 0.0f;
  for (int p = wave; p < PASSES; p += kMfmaWaves) {
    const int tt = p * TPP + lane / L;
    const f32x4 v4 = *reinterpret_cast<const f32x4*>(tab + tt * EP + e0);
    finish_group<L>(v4, bq, t0 + tt, Tn, e0, E, k, gating, logits, topk_idx, topk_w);
  }
}

static hipError_t pack_router_frags(const RouteArgs& a, int NB, hipStream_t st) {
  const int64_t nfrag = (int64_t)((a.d + 31) / 32) * NB * 64;
  hipLaunchKernelGGL(pack_router_frags_kernel, dim3((unsigned)((nfrag + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)a.w, (u32x4*)a.wpack, a.d, a.E, NB);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16, up to 16 experts, d up to 4096: the streaming gate GEMM.  Workgroups
// of 8 waves stay resident and walk "steps" of 16 SG tokens (SG = 8 / WPG
// groups of 16 tokens): the WPG waves of a group split its K range into
// contiguous slices of KB 32-K blocks, so every row of a step is read in WPG
// runs of 64 KB bytes at once, and the workgroup reads its rows whole within
// one step (DRAM page locality).  Two steps' x operands are in flight per
// wave: the loads of step i + 2 go out after step i's MFMAs and stay
// outstanding across the step's barrier, which waits for LDS traffic only.
// The waves' partial logits meet in LDS; wave i % WPG of a group sums them in
// the fixed order of the K slices (deterministic logits) and finishes the
// group's tokens, four lanes per token.
//
// Router fragments: the workgroup copies W_r [d][E] into LDS once (rows of
// `wpitch` bytes) and each wave takes the B operands of its slice from there
// with transposing reads (ds_read_b64_tr_b16: within 16 lanes, lane j
// addresses 4 consecutive columns of row j / 4 of a 4 x 16 block and lane i
// receives column i's 4 rows), keeping them in registers for the kernel.
// The LDS then holds the partials.
//
// With at most 8 experts (PAIRS) a load instruction reads whole 128-byte
// lines: 8 tokens x 128 bytes.  The MFMA's rows 0..7 then carry the even
// 16-byte pieces of tokens 0..7 and rows 8..15 their odd pieces; B columns
// 0..7 hold experts 0..7 at the even pieces' K and columns 8..15 the same
// experts at the odd pieces' K, so a token's logit is C[t][e] + C[t+8][e+8]
// (the other two quadrants are unused).  One MFMA still covers 1 KB of x,
// and the fragments of a 64-K line fill all 16 columns (half the registers).
// ---------------------------------------------------------------------------
template <bool PAIRS> constexpr int stream_nh() { return PAIRS ? 2 : 1; }  // accumulators per lane
template <bool PAIRS> constexpr int stream_red_bytes() { return 2 * kMfmaWaves * stream_nh<PAIRS>() * 64 * 16; }
template <bool PAIRS> constexpr int stream_tab_bytes() { return kMfmaWaves * stream_nh<PAIRS>() * 256 * 4; }
constexpr int kStreamMaxLds = 4096 * 32;  // W_r rows of up to 16 experts for d = 4096


// compute units of the current device (asked once per device)
hipError_t device_cus(int* cus) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> count[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  int n = count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    count[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return hipSuccess;
}

// bytes per row of W_r in LDS: E bf16, rounded up to 8 bytes (transposing
// reads take 8-byte aligned addresses)
static int stream_wpitch(int E) { return (2 * E + 7) / 8 * 8; }

template <int WPG, int KB, bool FULLK, bool PAIRS>
__global__ __launch_bounds__(kMfmaWaves * 64) void route_stream_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int64_t Tn, int d,
    int E, int k, int gating, int64_t nsteps, int wpitch) {
  constexpr int TOKS = 16 * (kMfmaWaves / WPG);
  constexpr int NH = stream_nh<PAIRS>();
  constexpr int NW = PAIRS ? KB / 2 : KB;  // router fragments per wave
  static_assert(KB % 2 == 0, "slices hold an even number of K blocks");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave / WPG, kpart = wave % WPG, g = lane >> 4, r16 = lane & 15;
  const int64_t s0 = blockIdx.x, ds = gridDim.x;

  // (1) W_r: 16-byte chunks of [d][E] in flight before the x loads
  const int nch = d * E / 8;  // d is a multiple of 8
  const bool w16 = (reinterpret_cast<uintptr_t>(w) & 15) == 0;  // else 2-byte loads
  u32x4 wc[16];              // d E <= 65536
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    wc[c] = u32x4{0u, 0u, 0u, 0u};
    const int ci = tid + 512 * c;
    if (ci < nch) {
      if (w16) {
        wc[c] = ld16(w + 8 * ci);
      } else {
        const uint16_t* w2 = reinterpret_cast<const uint16_t*>(w) + 8 * ci;
#pragma unroll
        for (int q = 0; q < 4; ++q) wc[c][q] = (uint32_t)w2[2 * q] | ((uint32_t)w2[2 * q + 1] << 16);
      }
    }
  }

  // finishing layout: lane l takes token l / 4 of a group, experts e0 .. e0 + 3
  // (the bias is loaded before the x operands: the waits for W_r cover it)
  const int e0 = 4 * (lane & 3);
  float bq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bq[c] = (bias && e0 + c < E) ? bias[e0 + c] : 0.0f;

  // (2) the x operands of the first two steps.  Plain: lane (r, g) reads
  // token r of its group at K 32 (kb0 + j) + 8 g.  PAIRS: token 8 h + r % 8
  // at byte 16 (2 g + r / 8) of 128-byte line (line0 + jl), a[2 jl + h].
  const int kb0 = kpart * KB;
  const int xoff = PAIRS ? 64 * (kb0 / 2) + 8 * (2 * g + (r16 >> 3)) : 32 * kb0 + 8 * g;  // elements
  auto load = [&](int64_t s, u32x4 (&a)[KB]) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int64_t t = s * TOKS + 16 * slot + (PAIRS ? 8 * h + (r16 & 7) : r16);
      const int64_t row = s >= nsteps ? 0 : (t < Tn ? t : Tn - 1);
      const bf16* xr = x + row * d + xoff;
#pragma unroll
      for (int jl = 0; jl < KB / NH; ++jl) {
        const int step = PAIRS ? 64 : 32;  // elements per load of a lane's row
        u32x4& dst = a[NH * jl + h];
        if constexpr (FULLK) {
          dst = ld16(xr + step * jl);
        } else if constexpr (PAIRS || KB < 16) {
          // a piece is all in or all out of d; pieces past it load the row's
          // first piece (no branch around the load) and are zeroed
          const bool ok = xoff + step * jl < d;
          const u32x4 v = ld16(ok ? xr + step * jl : xr - xoff);
          dst = ok ? v : u32x4{0u, 0u, 0u, 0u};
        } else {
          // (16 blocks of 16 experts: a masked load keeps the registers in bounds)
          u32x4 v = {0u, 0u, 0u, 0u};
          if (xoff + step * jl < d) v = ld16(xr + step * jl);
          dst = v;
        }
      }
    }
  };
  const int64_t iters = s0 < nsteps ? (nsteps - 1 - s0) / ds + 1 : 0;
  u32x4 xa[KB], xb[KB];
  load(s0, xa);
  load(s0 + ds, xb);
  // (a mask other than the loop's: the loop header must not absorb these
  // loads as common code of its two predecessors)
  __builtin_amdgcn_sched_barrier(1);

  // (3) W_r into LDS: element k E + e at byte k wpitch + 2 e
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const int ci = tid + 512 * c;
    if (ci < nch) {
      if (wpitch == 2 * E) {
        st16(lds + 16 * ci, wc[c]);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int el = 8 * ci + q, kk = el / E, e = el - kk * E;
          *reinterpret_cast<uint16_t*>(lds + kk * wpitch + 2 * e) = (uint16_t)(wc[c][q >> 1] >> (16 * (q & 1)));
        }
      }
    }
  }
  lds_only_barrier();

  // (4) this wave's fragments.  Plain, block kb: lane (n, g) gets K
  // 32 kb + 8 g .. + 7 of expert n.  PAIRS, line L: lane (n, g) gets K 64 L
  // + 16 g + 8 (n / 8) .. + 7 of expert n % 8.  Zero past d and past E.
  u32x4 wb[NW];
  {
    const int jr = r16 >> 2, jc = r16 & 3;  // this lane's row and column quad in the 4 x 16 block
    const int en = PAIRS ? (r16 & 7) : r16;  // expert of the column this lane receives
#pragma unroll
    for (int f = 0; f < NW; ++f) {
      int row, col, kr;  // kr: first K of the piece this lane receives
      if constexpr (PAIRS) {
        const int L = kb0 / 2 + f;
        row = 64 * L + 16 * g + 8 * (jc >> 1) + jr;
        col = 4 * (jc & 1);
        kr = 64 * L + 16 * g + 8 * (r16 >> 3);
      } else {
        const int kb = kb0 + f;
        row = 32 * kb + 8 * g + jr;
        col = 4 * jc;
        kr = 32 * kb + 8 * g;
      }
      const char* pa = lds + (row < d ? row : 0) * wpitch + 2 * col;
      const u32x2 r0 = lds_read_tr16(pa), r1 = lds_read_tr16(pa + 4 * wpitch);
      const bool ok = kr < d && en < E;
      wb[f] = ok ? u32x4{r0[0], r0[1], r1[0], r1[1]} : u32x4{0u, 0u, 0u, 0u};
    }
  }
  lds_only_barrier();  // the W_r copy is dead: the LDS now holds partials

  f32x4* red = reinterpret_cast<f32x4*>(lds);  // [2 steps][8 waves][NH][64 lanes]
  float* tab = reinterpret_cast<float*>(lds + stream_red_bytes<PAIRS>()) + wave * 256 * NH;  // [NH][16][16]
  // the loads of step i + 2 into a step's operand registers; the other
  // buffer's loads stay in flight throughout.  The empty asm pins them: their
  // step index passes through it, and it stays after the barriers and stores
  // before it.  The scheduling barrier keeps the next MFMAs from moving up.
  auto reload = [&](int64_t i, u32x4 (&a)[KB]) {
    int64_t next = s0 + (i + 2) * ds;
    asm volatile("" : "+s"(next) : : "memory");
    load(next, a);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](int64_t i, u32x4 (&a)[KB]) {
    f32x4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int j = 0; j < KB; ++j)  // two chains: blocks (plain) or token halves (PAIRS)
      acc[j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                           __builtin_bit_cast(bf16x8, wb[PAIRS ? j / 2 : j]),
                                                           acc[j & 1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sum[NH];
    if constexpr (PAIRS) {
      sum[0] = acc[0];
      sum[NH - 1] = acc[1];
    } else {
      sum[0] = acc[0] + acc[1];
    }
    const int buf = (int)(i & 1);
    bool finisher = true;
    if constexpr (WPG > 1) {
#pragma unroll
      for (int h = 0; h < NH; ++h) red[((buf * kMfmaWaves + wave) * NH + h) * 64 + lane] = sum[h];
      lds_only_barrier();
      finisher = kpart == (int)(i % WPG);
      if (finisher) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          sum[h] = red[((buf * kMfmaWaves + slot * WPG) * NH + h) * 64 + lane];
#pragma unroll
          for (int p = 1; p < WPG; ++p) sum[h] += red[((buf * kMfmaWaves + slot * WPG + p) * NH + h) * 64 + lane];
        }
      }
    }
    if (finisher) {
      // accumulator lane l: MFMA rows 4 (l / 16) + q, column l % 16
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) tab[(h * 16 + 4 * g + q) * 16 + r16] = sum[h][q];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      const int tt = lane >> 2;  // token of the group
      f32x4 v4;
      if constexpr (PAIRS) {
        // C[t][e] + C[t + 8][e + 8] of half tt / 8 (lanes with e0 >= 8 hold no experts)
        const float* th = tab + (tt >> 3) * 256 + (tt & 7) * 16;
        const int e1 = e0 < 8 ? e0 : 0;
        v4 = *reinterpret_cast<const f32x4*>(th + e1) + *reinterpret_cast<const f32x4*>(th + 8 * 16 + 8 + e1);
      } else {
        v4 = *reinterpret_cast<const f32x4*>(tab + tt * 16 + e0);
      }
      finish_group<4>(v4, bq, (s0 + i * ds) * TOKS + 16 * slot + tt, Tn, e0, E, k, gating, logits, topk_idx,
                      topk_w);
    }
    // the loads of step i + 2 go out after the finish, which uses their
    // registers meanwhile (issuing them before the barrier measured slower)
    reload(i, a);
  };
  // both steps in every trip (an odd count gets one more step past the last,
  // which loads row 0, stores nothing and ends at the same barriers), so that
  // the loop's back edge always has the other buffer's loads outstanding
  for (int64_t i = 0; i < iters; i += 2) {
    step(i, xa);
    step(i + 1, xb);
  }
}

template <int WPG, int KB, bool FULLK, bool PAIRS>
static hipError_t launch_route_stream_kb(const RouteArgs& a, hipStream_t st) {
  constexpr int TOKS = 16 * (kMfmaWaves / WPG);
  const int64_t nsteps = (a.T + TOKS - 1) / TOKS;
  auto kern = route_stream_kernel<WPG, KB, FULLK, PAIRS>;
  const int wpitch = stream_wpitch(a.E);
  const int lds = std::max<int>(a.d * wpitch, stream_red_bytes<PAIRS>() + stream_tab_bytes<PAIRS>());
  static const hipError_t prep = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kStreamMaxLds);
  if (prep != hipSuccess) return prep;
  // resident workgroups: as many as fit on every compute unit at once (the
  // register-bound count, asked once, capped by this launch's LDS)
  static int per_cu_regs = 0;
  static const hipError_t occ = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu_regs, reinterpret_cast<const void*>(kern), kMfmaWaves * 64,
      stream_red_bytes<PAIRS>() + stream_tab_bytes<PAIRS>());
  if (occ != hipSuccess) return occ;
  int cus = 0;
  const hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int per_cu = std::max(1, std::min(per_cu_regs, kLdsPerCu / lds));
  const int64_t grid = std::min<int64_t>(nsteps, (int64_t)cus * per_cu);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kMfmaWaves * 64), lds, st, (const bf16*)a.x,
                     (const bf16*)a.w, a.bias, a.logits, a.topk_idx, a.topk_w, a.T, a.d, a.E, a.k, a.gating,
                     nsteps, wpitch);
  return hipGetLastError();
}

// waves per 16-token group (WPG) and 32-K blocks per wave (KB).  Among the
// splits whose slices hold at most 16 blocks, prefer one with a step for
// every compute unit (small T), then one whose slices tile d exactly (no
// masked pieces), then the fewest waves per group.
static hipError_t launch_route_stream(const RouteArgs& a, hipStream_t st) {
  const int nkb = (a.d + 31) / 32;
  int cus = 0;
  const hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  int wpg = 0, kb = 0, score = -1;
  bool full = false;
  for (int w = 1; w <= kMfmaWaves; w *= 2) {
    const int need = (nkb + w - 1) / w;
    if (need > 16) continue;
    const bool f = a.d == 32 * need * w && (need == 4 || need == 6 || need == 8 || need == 12 || need == 16);
    const int64_t toks = 16 * (kMfmaWaves / w);
    const bool wide = (a.T + toks - 1) / toks >= cus;
    const int sc = (wide ? 2 : 0) + (f ? 1 : 0);
    if (sc > score) {
      score = sc;
      wpg = w;
      full = f;
      kb = f ? need : need <= 4 ? 4 : need <= 8 ? 8 : 16;
    }
  }
  const bool pairs = a.E <= 8;
#define MOE_RS(W, K, F)                                                                         \
  return pairs ? launch_route_stream_kb<W, K, F, true>(a, st) : launch_route_stream_kb<W, K, F, false>(a, st);
#define MOE_RS_KB(W)                                  \
  if (full) {                                         \
    switch (kb) {                                     \
      case 4: MOE_RS(W, 4, true)                      \
      case 6: MOE_RS(W, 6, true)                      \
      case 8: MOE_RS(W, 8, true)                      \
      case 12: MOE_RS(W, 12, true)                    \
      default: MOE_RS(W, 16, true)                    \
    }                                                 \
  } else {                                            \
    switch (kb) {                                     \
      case 4: MOE_RS(W, 4, false)                     \
      case 8: MOE_RS(W, 8, false)                     \
      default: MOE_RS(W, 16, false)                   \
    }                                                 \
  }
  switch (wpg) {
    case 1: MOE_RS_KB(1)
    case 2: MOE_RS_KB(2)
    case 4: MOE_RS_KB(4)
    default: MOE_RS_KB(8)
  }
#undef MOE_RS_KB
#undef MOE_RS
}

template <int EP, int TG>
static hipError_t launch_route_mfma(const RouteArgs& a, hipStream_t st) {
  const int64_t blocks = (a.T + 16 * TG - 1) / (16 * TG);
  if (blocks <= 0) return hipSuccess;
  constexpr int NB = EP / 16;
  hipError_t err = pack_router_frags(a, NB, st);
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
    case 16:
      if (a.d <= 4096 && a.T > 0) return launch_route_stream(a, st);
      return launch_route_mfma<16, 2>(a, st);
    // tokens per workgroup (16 TG): with 64 experts, 32 tokens let two
    // workgroups share a compute unit, so one's tree sum and finish overlap
    // the other's loads (DeepSeek-V2-Lite shape, in-step: 44.4 -> 35.6 us;
    // 16 tokens: 39.7 us).  With 32 experts the lighter finish gains nothing
    // (warm caches slower, a written-back cache faster), so 64 tokens stay.
    case 32: return launch_route_mfma<32, 4>(a, st);
    default: return launch_route_mfma<64, 2>(a, st);
  }
}

}  // namespace moe
