// Weighted combine, its backward, and the un-permute sum of the backward.
//
// Tutorial ch.4, 专家并行 二 step 4 (results return to the token's device and
// the sequence order is restored), 流水线并行 三 (expert outputs are merged),
// and 专家并行与数据并行的结合 三.3 (gradients routed back to the experts).
// All three are bandwidth kernels: every row is moved with 16-byte accesses
// that are contiguous along the row, and sums are accumulated in fp32 in a
// fixed order (no atomics, deterministic).
#include "common.h"
#include "kernels.h"

namespace moe {

// One wave per token row.  The row indices and gate weights of the token are
// wave-uniform (scalar loads); each lane takes the 16-byte chunks lane,
// lane + 64, ... of the row, U at a time, and issues all loads of a round
// (U chunks of each of the <= KMAX gathered rows) before it combines them.
constexpr int kRowWaves = 4;  // waves (tokens) per workgroup

// Chunks per lane per round: enough for one round per row on wide rows,
// fewer where most lanes would have nothing to load.
inline int row_unroll(int64_t d, int elem_bytes, int kmax) {
  const int64_t nch = d * elem_bytes / 16;
  if (kmax > 2) return 2;
  return nch > 256 ? 8 : nch > 128 ? 4 : 2;
}

// y[t] = sum_j g[t,j] * y_perm[row_of[t,j]] (+ y_shared[t]).  With topk_w
// NULL the rows are already weighted and token-major (the fused forward's
// GEMM epilogue wrote row t*k + j): y[t] = sum over kept j of y_perm[t*k + j].
template <typename T, int KMAX, int U>
__global__ __launch_bounds__(64 * kRowWaves) void combine_kernel(const T* __restrict__ y_perm,
                                                                 const int32_t* __restrict__ row_of,
                                                                 const float* __restrict__ topk_w,
                                                                 const T* __restrict__ y_shared, T* __restrict__ y,
                                                                 int64_t Tn, int d, int k) {
  constexpr int V = Vec16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kRowWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= Tn) return;
  const int nch = d / V;
  int rows[KMAX];
  float g[KMAX];
  const bool tok_major = topk_w == nullptr;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rows[j] = j < k ? row_of[t * k + j] : -1;
    g[j] = rows[j] >= 0 ? (tok_major ? 1.0f : topk_w[t * k + j]) : 0.0f;
    if (tok_major && rows[j] >= 0) rows[j] = (int)(t * k + j);
  }
  for (int c0 = lane; c0 < nch; c0 += 64 * U) {
    u32x4 v[KMAX][U], sh[U];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 64 * u;
        v[j][u] = (rows[j] >= 0 && c < nch) ? ld16(y_perm + (int64_t)rows[j] * d + (int64_t)c * V)
                                            : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      sh[u] = (y_shared && c < nch) ? ld16(y_shared + t * d + (int64_t)c * V) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c >= nch) break;
      float acc[V], f[V];
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] = 0.0f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (rows[j] < 0) continue;
        unpack16<T>(v[j][u], f);
#pragma unroll
        for (int q = 0; q < V; ++q) acc[q] += g[j] * f[q];
      }
      if (y_shared) {
        unpack16<T>(sh[u], f);
#pragma unroll
        for (int q = 0; q < V; ++q) acc[q] += f[q];
      }
      st16(y + t * d + (int64_t)c * V, pack16<T>(acc));
    }
  }
}

// dy_perm[row] = g * dy[t]; d_topk_w[t,j] = <dy[t], y_perm[row]>, one wave per token.
template <typename T, int KMAX, int U>
__global__ __launch_bounds__(64 * kRowWaves) void combine_bwd_kernel(const T* __restrict__ dy,
                                                                     const T* __restrict__ y_perm,
                                                                     const int32_t* __restrict__ row_of,
                                                                     const float* __restrict__ topk_w,
                                                                     T* __restrict__ dy_perm,
                                                                     float* __restrict__ d_topk_w, int64_t Tn, int d,
                                                                     int k) {
  constexpr int V = Vec16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kRowWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= Tn) return;
  const int nch = d / V;
  int rows[KMAX];
  float g[KMAX], dot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rows[j] = j < k ? row_of[t * k + j] : -1;
    g[j] = rows[j] >= 0 ? topk_w[t * k + j] : 0.0f;
    dot[j] = 0.0f;
  }
  for (int c0 = lane; c0 < nch; c0 += 64 * U) {
    u32x4 dv[U], ov[KMAX][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      dv[u] = c < nch ? ld16(dy + t * d + (int64_t)c * V) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 64 * u;
        ov[j][u] = (rows[j] >= 0 && c < nch) ? ld16(y_perm + (int64_t)rows[j] * d + (int64_t)c * V)
                                             : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c >= nch) break;
      float df[V], of[V], sv[V];
      unpack16<T>(dv[u], df);
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (rows[j] < 0) continue;
        unpack16<T>(ov[j][u], of);
        float p = 0.0f;
#pragma unroll
        for (int q = 0; q < V; ++q) {
          p += df[q] * of[q];
          sv[q] = g[j] * df[q];
        }
        dot[j] += p;
        st16(dy_perm + (int64_t)rows[j] * d + (int64_t)c * V, pack16<T>(sv));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) break;
    const float s = group_sum<64>(dot[j]);
    if (lane == 0) d_topk_w[t * k + j] = rows[j] >= 0 ? s : 0.0f;
  }
}

// CPT consecutive elements (CPT * sizeof(T) bytes, CPT a power of two <= 8).
template <typename T, int CPT>
__device__ __forceinline__ void load_cols(const T* p, float (&v)[CPT]) {
  if constexpr (CPT * sizeof(T) == 16) {
    unpack16<T>(ld16(p), v);
  } else if constexpr (CPT * sizeof(T) == 8) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    if constexpr (sizeof(T) == 2) {
      v[0] = __uint_as_float(w[0] << 16); v[1] = __uint_as_float(w[0] & 0xffff0000u);
      v[2] = __uint_as_float(w[1] << 16); v[3] = __uint_as_float(w[1] & 0xffff0000u);
    } else {
      v[0] = __uint_as_float(w[0]); v[1] = __uint_as_float(w[1]);
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) v[c] = to_f32(p[c]);
  }
}
// load_cols of p when pred, else zeros.  The load is unconditional (from the
// valid address `fallback` when !pred) and the zeros are a select, so no
// branch forces the wait for the load right after it.
template <typename T, int CPT>
__device__ __forceinline__ void load_cols_if(bool pred, const T* p, const T* fallback, float (&v)[CPT]) {
  load_cols<T, CPT>(pred ? p : fallback, v);
#pragma unroll
  for (int c = 0; c < CPT; ++c) v[c] = pred ? v[c] : 0.0f;
}
template <typename T, int CPT>
__device__ __forceinline__ void store_cols(T* p, const float (&v)[CPT]) {
  if constexpr (CPT * sizeof(T) == 16) {
    st16(p, pack16<T>(v));
  } else if constexpr (CPT * sizeof(T) == 8 && sizeof(T) == 2) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]),
                                         pack_bf16x2(v[2], v[3])};
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) p[c] = from_f32<T>(v[c]);
  }
}

// dx[t, i] = sum_j dx_perm[row_of[t,j], i] + sum_e dl[t,e] * W_r[i,e] (+ dx_add[t, i]).
// A lane owns CPT consecutive columns and keeps their router-weight rows in
// registers (fp32; CPT * EP = 64 values, one 128-byte stretch of W_r when
// E == EP, read with 16-byte loads) while its wave walks tpw tokens, two at a
// time.  The tokens' row indices and dlogits are the same for the whole wave
// and come in through scalar loads; the gathered rows of both tokens are
// loaded before they are summed.
template <typename T, int EP, int CPT, bool FULL, int KMAX, int TU, bool ADD>
__global__ __launch_bounds__(256) void dispatch_bwd_kernel(const T* __restrict__ dx_perm,
                                                           const int32_t* __restrict__ row_of,
                                                           const float* __restrict__ dl, const T* __restrict__ w_r,
                                                           const T* __restrict__ dx_add, T* __restrict__ dx,
                                                           int64_t Tn, int d, int E, int k, int tpw) {
  static_assert(CPT * EP == 64, "64 router weights per lane");
  const int64_t t0 = (int64_t)blockIdx.x * tpw;
  const int i0 = (blockIdx.y * 256 + threadIdx.x) * CPT;
  const bool col_ok = i0 < d;  // d is a multiple of 8: a lane's CPT columns are all in or all out
  float wr[CPT][EP];
  if constexpr (FULL) {
    // rows i0 .. i0+CPT-1 of W_r are CPT*EP contiguous elements
    constexpr int NV = CPT * EP / Vec16<T>::N;
    const T* wp = col_ok ? w_r + (int64_t)i0 * EP : w_r;  // unconditional loads, zeros by select
    u32x4 raw[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) raw[v] = ld16(wp + v * Vec16<T>::N);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float f[Vec16<T>::N];
      unpack16<T>(raw[v], f);
#pragma unroll
      for (int q = 0; q < Vec16<T>::N; ++q) {
        const int idx = v * Vec16<T>::N + q;
        wr[idx / EP][idx % EP] = col_ok ? f[q] : 0.0f;
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < EP; ++e) wr[c][e] = (col_ok && e < E) ? to_f32(w_r[(int64_t)(i0 + c) * E + e]) : 0.0f;
  }

  // U tokens at a time: every load of the round issued before any sum; the
  // tail round repeats the last token (in range, result not stored)
  const int64_t tlast = (t0 + tpw < Tn ? t0 + tpw : Tn) - 1;
  for (int64_t tb = t0; tb <= tlast; tb += TU) {
    int64_t tt[TU];
    int rows[TU][KMAX];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      tt[u] = tb + u <= tlast ? tb + u : tlast;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) rows[u][j] = j < k ? row_of[tt[u] * k + j] : -1;
    }
    float g[TU][KMAX][CPT], add[TU][CPT];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const bool ok = col_ok && rows[u][j] >= 0;
        load_cols_if<T, CPT>(ok, dx_perm + (int64_t)(ok ? rows[u][j] : 0) * d + i0, dx_perm, g[u][j]);
      }
      if constexpr (ADD) load_cols_if<T, CPT>(col_ok, dx_add + (col_ok ? tt[u] * d + i0 : 0), dx_add, add[u]);
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      float acc[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c] = 0.0f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] += g[u][j][c];
      const float* dlt = dl + tt[u] * (FULL ? EP : E);
#pragma unroll
      for (int e = 0; e < EP; ++e) {
        const float lv = (FULL || e < E) ? dlt[e] : 0.0f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] = fmaf(lv, wr[c][e], acc[c]);
      }
      // one token's dlogits at a time in scalar registers (up to 64)
      if constexpr (EP >= 32) __builtin_amdgcn_sched_barrier(0);
      if constexpr (ADD) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] += add[u][c];
      }
      if (col_ok && tb + u <= tlast) store_cols<T, CPT>(dx + tt[u] * d + i0, acc);
    }
  }
}

// bf16 dispatch backward with the router term on MFMA, for E a multiple of 8
// (so that every router-weight row starts on a 16-byte boundary).
// v_mfma_f32_16x16x32_bf16 computes C[m][n] = sum_k A[m][k] B[k][n] with
// lane l holding A[l % 16][8 (l / 16) + 0..7], B[8 (l / 16) + 0..7][l % 16]
// and C[4 (l / 16) + 0..3][l % 16].  Here A = dlogits (rows: the wave's 16
// tokens, K: experts) and B = W_r^T; the C column n of block b is column
// i0 + 8 n + b, so over its 8 blocks a lane holds 8 consecutive columns of 4
// tokens, the shape of a 16-byte row access.  dlogits enter as bf16 hi + lo
// (hi = bf16(v), lo = bf16(v - hi), two MFMAs), which keeps about 16
// significant bits; the weights are bf16 already; products and sums are
// fp32.  Then each lane adds, token by token, its 16-byte pieces of the
// token's gathered rows (in j order) and of dx_add, and stores 16 bytes; the
// row indices and the first round of gathers are loaded before the router
// term, whose loads and MFMAs overlap them.
// A wave owns 16 tokens x 128 columns; 4 waves per workgroup take 4
// consecutive token groups of the same columns.
template <int KMAX, int EK>
__global__ __launch_bounds__(256) void dispatch_bwd_mfma_kernel(const bf16* __restrict__ dx_perm,
                                                                const int32_t* __restrict__ row_of,
                                                                const float* __restrict__ dl,
                                                                const bf16* __restrict__ w_r,
                                                                const bf16* __restrict__ dx_add,
                                                                bf16* __restrict__ dx, int64_t Tn, int d, int E,
                                                                int k) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // blockIdx.x: column chunk, so that consecutive workgroups read
  // consecutive pieces of the same rows (DRAM page locality)
  const int64_t t0 = ((int64_t)blockIdx.y * 4 + wave) * 16;
  if (t0 >= Tn) return;
  const int n = lane & 15, kg = lane >> 4;
  const int ic = blockIdx.x * 128 + 8 * n;  // this lane's 8 columns
  const bool col_ok = ic < d;               // d is a multiple of 8

  // the lane's 4 tokens t0 + 4 kg + q and their row indices, loaded first:
  // the gathers depend on them, the router term does not
  constexpr int R = KMAX <= 2 ? 4 : 2;  // tokens per gather round
  int64_t tq[4];
  bool tok_ok[4];
  int rows[4][KMAX];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * kg + q;
    tok_ok[q] = t < Tn;
    tq[q] = tok_ok[q] ? t : t0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) rows[q][j] = j < k ? row_of[tq[q] * k + j] : -1;
  }
  u32x4 g[R][KMAX], ad[R];
  auto gather = [&](int q0) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int q = q0 + u;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const int r = rows[q][j];
        const bool ok = col_ok && tok_ok[q] && r >= 0;
        const u32x4 v = ld16(dx_perm + (ok ? (int64_t)r * d + ic : 0));
        g[u][j] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
      const bool aok = dx_add != nullptr && col_ok && tok_ok[q];
      const u32x4 v = ld16((aok ? dx_add : dx_perm) + (aok ? tq[q] * d + ic : 0));
      ad[u] = aok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // the router term's operands (dlogits of token t0 + n, experts e .. e+7,
  // and W_r[ic + b][e .. e+7] of every 32-expert block) are loaded before
  // the first gathers, so that the MFMAs wait for them alone (the load
  // counter is in order): the gathers stay in flight while they multiply.
  // Loads are unconditional, from valid addresses; zeros are selected at use.
  const int64_t ta = t0 + n < Tn ? t0 + n : Tn - 1;
  u32x4 dlv[EK][2], wv[EK][8];
#pragma unroll
  for (int ek = 0; ek < EK; ++ek) {
    const int e = 32 * ek + 8 * kg;
    const bool e_ok = e < E;  // E is a multiple of 8: a lane's 8 experts are all in or all out
    const float* dp = dl + ta * E + (e_ok ? e : 0);
    dlv[ek][0] = ld16(dp);
    dlv[ek][1] = ld16(dp + 4);
#pragma unroll
    for (int b = 0; b < 8; ++b) wv[ek][b] = ld16(w_r + (int64_t)(col_ok ? ic + b : 0) * E + (e_ok ? e : 0));
  }
  gather(0);  // in flight while the router term multiplies

  f32x4 acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ek = 0; ek < EK; ++ek) {
    const int e = 32 * ek + 8 * kg;
    const bool e_ok = e < E;
    // A: dlogits as hi + lo
    const u32x4 d0 = dlv[ek][0], d1 = dlv[ek][1];
    const bool a_ok = e_ok && t0 + n < Tn;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v2[2];
      v2[0] = a_ok ? __uint_as_float(q < 2 ? d0[2 * q] : d1[2 * q - 4]) : 0.0f;
      v2[1] = a_ok ? __uint_as_float(q < 2 ? d0[2 * q + 1] : d1[2 * q - 3]) : 0.0f;
      const uint32_t h0 = bf16_bits(v2[0]), h1 = bf16_bits(v2[1]);
      hi[q] = h0 | (h1 << 16);
      lo[q] = bf16_bits(v2[0] - __uint_as_float(h0 << 16)) | (bf16_bits(v2[1] - __uint_as_float(h1 << 16)) << 16);
    }
    const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, u32x4{hi[0], hi[1], hi[2], hi[3]});
    const bf16x8_t alo = __builtin_bit_cast(bf16x8_t, u32x4{lo[0], lo[1], lo[2], lo[3]});
    // B: router weights, 16 bytes per block
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bf16x8_t bw =
          __builtin_bit_cast(bf16x8_t, (col_ok && e_ok) ? wv[ek][b] : u32x4{0u, 0u, 0u, 0u});
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bw, acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bw, acc[b], 0, 0, 0);
    }
  }

  // per token: router term, gathered rows in j order, dx_add; 16-byte store
#pragma unroll
  for (int q0 = 0; q0 < 4; q0 += R) {
    if (q0 > 0) gather(q0);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int q = q0 + u;
      float s[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) s[b] = acc[b][q];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        float f[8];
        unpack16<bf16>(g[u][j], f);
#pragma unroll
        for (int b = 0; b < 8; ++b) s[b] += f[b];
      }
      float f[8];
      unpack16<bf16>(ad[u], f);
#pragma unroll
      for (int b = 0; b < 8; ++b) s[b] += f[b];
      if (col_ok && tok_ok[q]) st16(dx + tq[q] * d + ic, pack16<bf16>(s));
    }
  }
}

template <int KMAX, int EK>
static hipError_t launch_dbwd_mfma(const DispatchBwdArgs& a, hipStream_t st) {
  const int64_t by = (a.T + 63) / 64;  // 4 waves x 16 tokens
  const int bx = (int)((a.d + 127) / 128);
  if (by <= 0) return hipSuccess;
  hipLaunchKernelGGL((dispatch_bwd_mfma_kernel<KMAX, EK>), dim3((unsigned)bx, (unsigned)by), dim3(256), 0, st,
                     (const bf16*)a.dx_perm, a.row_of, a.dlogits, (const bf16*)a.w_router, (const bf16*)a.dx_add,
                     (bf16*)a.dx, a.T, (int)a.d, a.E, a.k);
  return hipGetLastError();
}

template <typename T, int KMAX, int U>
static hipError_t launch_combine_u(const CombineArgs& a, bool backward, hipStream_t st) {
  const int64_t blocks = (a.T + kRowWaves - 1) / kRowWaves;
  if (blocks <= 0) return hipSuccess;
  if (!backward)
    hipLaunchKernelGGL((combine_kernel<T, KMAX, U>), dim3((unsigned)blocks), dim3(64 * kRowWaves), 0, st,
                       (const T*)a.y_perm, a.row_of, a.topk_w, (const T*)a.y_shared, (T*)a.y, a.T, (int)a.d, a.k);
  else
    hipLaunchKernelGGL((combine_bwd_kernel<T, KMAX, U>), dim3((unsigned)blocks), dim3(64 * kRowWaves), 0, st,
                       (const T*)a.dy, (const T*)a.y_perm, a.row_of, a.topk_w, (T*)a.dy_perm, a.d_topk_w, a.T,
                       (int)a.d, a.k);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_combine_dt(const CombineArgs& a, bool backward, hipStream_t st) {
  if (a.k > 2) return launch_combine_u<T, 8, 2>(a, backward, st);
  switch (row_unroll(a.d, sizeof(T), a.k)) {
    case 8: return launch_combine_u<T, 2, 8>(a, backward, st);
    case 4: return launch_combine_u<T, 2, 4>(a, backward, st);
    default: return launch_combine_u<T, 2, 2>(a, backward, st);
  }
}

hipError_t launch_combine(const CombineArgs& a, bool bf16_dtype, hipStream_t st) {
  return bf16_dtype ? launch_combine_dt<bf16>(a, false, st) : launch_combine_dt<float>(a, false, st);
}

hipError_t launch_combine_bwd(const CombineArgs& a, bool bf16_dtype, hipStream_t st) {
  return bf16_dtype ? launch_combine_dt<bf16>(a, true, st) : launch_combine_dt<float>(a, true, st);
}

template <typename T, int EP, int CPT, int KMAX>
static hipError_t launch_dbwd_k(const DispatchBwdArgs& a, hipStream_t st) {
  constexpr int TPW = 16;  // tokens per workgroup
  const int64_t bx = (a.T + TPW - 1) / TPW;
  const int by = (int)((a.d + 256 * CPT - 1) / (256 * CPT));
  if (bx <= 0) return hipSuccess;
  // two tokens per round (4 and 8 measured slower: more registers, fewer
  // waves); the shared-expert dx is added only when there is one
#define MOE_DBWD(ADD)                                                                                              \
  hipLaunchKernelGGL((a.E == EP ? dispatch_bwd_kernel<T, EP, CPT, true, KMAX, 2, ADD>                             \
                                : dispatch_bwd_kernel<T, EP, CPT, false, KMAX, 2, ADD>),                          \
                     dim3((unsigned)bx, by), dim3(256), 0, st, (const T*)a.dx_perm, a.row_of, a.dlogits,           \
                     (const T*)a.w_router, (const T*)a.dx_add, (T*)a.dx, a.T, (int)a.d, a.E, a.k, TPW)
  if (a.dx_add != nullptr) MOE_DBWD(true);
  else MOE_DBWD(false);
#undef MOE_DBWD
  return hipGetLastError();
}

template <typename T, int EP, int CPT>
static hipError_t launch_dbwd_t(const DispatchBwdArgs& a, hipStream_t st) {
  return a.k <= 2 ? launch_dbwd_k<T, EP, CPT, 2>(a, st) : launch_dbwd_k<T, EP, CPT, 8>(a, st);
}

// CPT * EP router weights per lane: 64 registers
template <typename T>
static hipError_t launch_dbwd_dt(const DispatchBwdArgs& a, hipStream_t st) {
  if (a.E <= 8) return launch_dbwd_t<T, 8, 8>(a, st);
  if (a.E <= 16) return launch_dbwd_t<T, 16, 4>(a, st);
  if (a.E <= 32) return launch_dbwd_t<T, 32, 2>(a, st);
  return launch_dbwd_t<T, 64, 1>(a, st);
}

hipError_t launch_dispatch_bwd(const DispatchBwdArgs& a, bool bf16_dtype, hipStream_t st) {
  // The MFMA kernel (bf16, E a multiple of 8, 16-byte aligned operands) except
  // for 8 experts on wide rows, where the vector kernel's router term is
  // cheap and a wave reads 1 KiB of a row at once (Mixtral shape: 0.085 ms
  // against 0.090; DeepSeek-V2-Lite 0.321 -> 0.132, GPT-2 0.022 -> 0.015).
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const bool vector_better = a.E <= 8 && a.d >= 2048;
  if (bf16_dtype && a.E % 8 == 0 && !vector_better && (a.T + 63) / 64 <= 65535 && al16(a.dlogits) &&
      al16(a.w_router) && al16(a.dx_perm) && al16(a.dx) && al16(a.dx_add)) {
    if (a.E <= 32) return a.k <= 2 ? launch_dbwd_mfma<2, 1>(a, st) : launch_dbwd_mfma<8, 1>(a, st);
    return a.k <= 2 ? launch_dbwd_mfma<2, 2>(a, st) : launch_dbwd_mfma<8, 2>(a, st);
  }
  return bf16_dtype ? launch_dbwd_dt<bf16>(a, st) : launch_dbwd_dt<float>(a, st);
}

}  // namespace moe
