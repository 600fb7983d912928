// Router backward: gating Jacobian and router weight gradient (tutorial
// ch.4, 专家并行与数据并行的结合 三.4: the replicated gate network has
// gradients that are aggregated across replicas; here they are computed for
// one GPU's tokens).
//
// gating_bwd: lane e of a token's lane group holds expert e (E <= 64).
//   SOFTMAX_TOPK:          dl = p * (dp - <p, dp>),  p = softmax(l), dp[e_j] = dg_j
//   RENORM / TOPK_SOFTMAX: the weights are a softmax over the chosen logits:
//                          dl[e_j] = g_j * (dg_j - sum_m g_m dg_m), 0 elsewhere
// router wgrad: dW_r = x^T dl as a deterministic two-stage reduction over
//   tokens: each block of tokens writes an fp32 partial [d, E] (bf16 MFMA for
//   bf16 x, fp32 MFMA for fp32 x), then the partials (at most 64 blocks) are
//   summed in a fixed order.
#include "common.h"
#include "kernels.h"
#include "stream.h"


namespace moe {

// G lanes per token (G = E rounded up to a power of two, at least 8), 64 / G
// tokens per wave; the softmax statistics and the weighted sums are
// reductions over the token's G lanes.
// dl_add (nullable): another gradient of the logits (the balance loss's),
// added to the Jacobian's.
template <int G>
__global__ __launch_bounds__(256) void gating_bwd_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ dg,
                                                         const float* __restrict__ dl_add, float* __restrict__ dl,
                                                         int64_t Tn, int E, int k, int gating) {
  const int lane = threadIdx.x & 63;
  const int64_t t = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  const int e = lane % G;
  const bool tok = t < Tn;  // every lane stays for the group reductions
  const bool valid = tok && e < E;
  const float l = valid ? logits[t * E + e] : -INFINITY;
  const float add = dl_add && valid ? dl_add[t * E + e] : 0.0f;
  // the token's k choices and their gradients, four at a time, all loads of
  // a group issued together (a gradient is not fetched after its index is
  // known; clamped indices keep every load in the token's row)
  const int64_t tc = tok ? t : 0;
  int sel = -1;
  float dgl = 0.0f;
  for (int j0 = 0; j0 < k; j0 += 4) {
    int ij[4];
    float gj[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u < k ? j0 + u : k - 1;
      ij[u] = idx[tc * k + j];
      gj[u] = dg[tc * k + j];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (tok && j0 + u < k && ij[u] == e) {
        sel = j0 + u;
        dgl = gj[u];
      }
  }
  float out;
  if (gating == 0) {
    const float mx = group_max<G>(l);
    float p = valid ? __expf(l - mx) : 0.0f;
    const float z = group_sum<G>(p);
    p = z > 0.0f ? p / z : 0.0f;
    const float s = group_sum<G>(p * dgl);
    out = p * (dgl - s);
  } else {
    const float lsel = sel >= 0 ? l : -INFINITY;
    const float mx = group_max<G>(lsel);
    float q = sel >= 0 ? __expf(l - mx) : 0.0f;
    const float z = group_sum<G>(q);
    const float g = z > 0.0f ? q / z : 0.0f;
    const float s = group_sum<G>(g * dgl);
    out = sel >= 0 ? g * (dgl - s) : 0.0f;
  }
  if (valid) dl[t * E + e] = dl_add ? out + add : out;
}

template <int G>
static hipError_t launch_gating_bwd(const RouteBwdArgs& a, hipStream_t st) {
  constexpr int TPB = 4 * (64 / G);  // tokens per workgroup
  const int64_t blocks = (a.T + TPB - 1) / TPB;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gating_bwd_kernel<G>), dim3((unsigned)blocks), dim3(256), 0, st, a.logits, a.topk_idx,
                     a.d_topk_w, a.dlogits_add, a.dlogits, a.T, a.E, a.k, a.gating);
  return hipGetLastError();
}

// Waves per workgroup of the fp32 MFMA weight-gradient kernel.
constexpr int kRwgWaves = 4;

// partial[b][i][e] on the fp32 matrix cores: v_mfma_f32_16x16x4_f32 takes
// A[m][kk] from lane kk * 16 + m and B[kk][n] from lane kk * 16 + n, so 4
// tokens x 16 columns of x and 4 tokens x 16 experts of dlogits enter as one
// value per lane, with no transposition.  A lane loads 16 bytes of x (V
// consecutive columns c0 + V m + j of token t = 4-group base + lane / 16) and
// feeds value j to the MFMA of column block j: block j's row m is column
// c0 + V m + j, so one workgroup covers CW = 16 V columns.  Products and
// sums are fp32, in a fixed order: the 4 waves take consecutive quarters of
// the block's tokens (4 token groups per round, loads first) and their
// accumulators are summed in a fixed tree through LDS.
template <typename T, int EP>
__global__ __launch_bounds__(64 * kRwgWaves) void router_wgrad_mfma_kernel(const T* __restrict__ x,
                                                                           const float* __restrict__ dl,
                                                                           float* __restrict__ partial, int64_t Tn,
                                                                           int d, int E, int tw) {
  constexpr int V = Vec16<T>::N, NB = EP / 16, CW = 16 * V, U = 4;
  constexpr int NACC = V * NB;  // f32x4 accumulators per lane
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kk = lane >> 4, m = lane & 15;
  const int c0 = blockIdx.x * CW + V * m;  // this lane's first x column
  const bool col_ok = c0 < d;              // d is a multiple of 8: all V columns in or out
  const int64_t tbeg = ((int64_t)blockIdx.y * kRwgWaves + wave) * tw;
  const int64_t tend = tbeg + tw < Tn ? tbeg + tw : Tn;
  f32x4 acc[V][NB];
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // token group at t4: lane's token t4 + kk; unconditional loads from valid
  // addresses, zeros by select past the range, the last column or E
  auto load = [&](int64_t t4, u32x4& xv, float (&dv)[NB]) {
    const int64_t t = t4 + kk;
    const bool tok = t < tend;
    const int64_t tc = tok ? t : tbeg;
    const u32x4 v = ld16(x + tc * d + (col_ok ? c0 : 0));
    xv = (tok && col_ok) ? v : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = 16 * nb + m;
      const float w = dl[tc * E + (e < E ? e : E - 1)];
      dv[nb] = (tok && e < E) ? w : 0.0f;
    }
  };
  for (int64_t t = tbeg; t < tend; t += 4 * U) {
    u32x4 xv[U];
    float dv[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) load(t + 4 * u, xv[u], dv[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xf[V];
      unpack16<T>(xv[u], xf);
#pragma unroll
      for (int j = 0; j < V; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[j][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[j], dv[u][nb], acc[j][nb], 0, 0, 0);
    }
  }
  // fixed-order tree sum of the 4 waves' accumulators: (w2 + w3) into w0, w1; then w1 into w0
  float* red = reinterpret_cast<float*>(lds);  // [2][NACC * 4][64]
  if (wave >= 2) {
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[(((wave - 2) * NACC + j * NB + nb) * 4 + q) * 64 + lane] = acc[j][nb][q];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j][nb][q] += red[((wave * NACC + j * NB + nb) * 4 + q) * 64 + lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[((j * NB + nb) * 4 + q) * 64 + lane] = acc[j][nb][q];
  }
  __syncthreads();
  if (wave != 0) return;
  // accumulator (j, nb)[q] of lane l: column blockIdx.x CW + V (4 (l / 16) + q) + j, expert 16 nb + l % 16
  float* pb = partial + (int64_t)blockIdx.y * d * E;
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v = acc[j][nb][q] + red[((j * NB + nb) * 4 + q) * 64 + lane];
        const int col = blockIdx.x * CW + V * (4 * kk + q) + j, e = 16 * nb + m;
        if (col < d && e < E) pb[(int64_t)col * E + e] = v;
      }
}

// dw[i] = the sum of partial[b][i] over the nb <= 64 token blocks, in a fixed
// order.  A workgroup owns 64 consecutive outputs (16 quads); its 256 threads
// are 16 slices x 16 quads: slice s adds blocks 4 s .. 4 s + 3 in order (its
// 16-byte loads issued together), the four slices of a wave meet in an xor
// tree (s with s ^ 1, then pairs with pairs) and the four waves' sums are
// added as (w0 + w1) + (w2 + w3).  Floating-point addition commutes exactly,
// so every run gives the same bits.  dE is a multiple of 8: a quad is all in
// or all out.
template <typename T>
__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(const float* __restrict__ partial, int nb,
                                                                  int64_t dE, T* __restrict__ dw) {
  __shared__ f32x4 red[4][16];
  const int tid = threadIdx.x, q = tid & 15, sl = tid >> 4, lane = tid & 63, wave = tid >> 6;
  const int64_t i0 = ((int64_t)blockIdx.x * 16 + q) * 4;
  const bool ok = i0 < dE;
  f32x4 v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int b = 4 * sl + r;
    const f32x4 w = *reinterpret_cast<const f32x4*>(partial + (int64_t)(b < nb ? b : 0) * dE + (ok ? i0 : 0));
    v[r] = (ok && b < nb) ? w : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  f32x4 sum = ((v[0] + v[1]) + v[2]) + v[3];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    sum[c] += __shfl_xor(sum[c], 16);
    sum[c] += __shfl_xor(sum[c], 32);
  }
  if (lane < 16) red[wave][q] = sum;
  __syncthreads();
  if (tid >= 16 || !ok) return;
  const f32x4 r = (red[0][q] + red[1][q]) + (red[2][q] + red[3][q]);
#pragma unroll
  for (int c = 0; c < 4; ++c) dw[i0 + c] = from_f32<T>(r[c]);
}

template <typename T>
static hipError_t launch_rwg_reduce(const RouteBwdArgs& a, int nb, hipStream_t st) {
  const int64_t dE = a.d * a.E;
  hipLaunchKernelGGL((router_wgrad_reduce_kernel<T>), dim3((unsigned)((dE + 63) / 64)), dim3(256), 0, st,
                     a.partial, nb, dE, (T*)a.dw_router);
  return hipGetLastError();
}

template <typename T, int EP>
static hipError_t launch_rwg_mfma(const RouteBwdArgs& a, hipStream_t st) {
  constexpr int V = Vec16<T>::N, CW = 16 * V;
  constexpr size_t lds = (size_t)2 * V * (EP / 16) * 4 * 64 * 4;
  const int nb = router_wgrad_blocks(a.T);
  const int tw = (int)((a.T + (int64_t)nb * kRwgWaves - 1) / ((int64_t)nb * kRwgWaves));  // tokens per wave
  const dim3 grid((unsigned)((a.d + CW - 1) / CW), nb);
  auto kern = router_wgrad_mfma_kernel<T, EP>;
  if constexpr (lds > 65536) {
    static const hipError_t prep = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (prep != hipSuccess) return prep;
  }
  hipLaunchKernelGGL(kern, grid, dim3(64 * kRwgWaves), lds, st, (const T*)a.x, a.dlogits, a.partial, a.T, (int)a.d,
                     a.E, tw);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_rwg_reduce<T>(a, nb, st);
}

// partial[b][i][e] on the bf16 matrix cores (bf16 x; E padded to 16, 32 or 64):
// v_mfma_f32_16x16x32_bf16 with M = 16 columns of x, N = 16 experts and K =
// 32 tokens.  dlogits enter as bf16 hi + lo (hi = bf16(v), lo = bf16(v - hi),
// one MFMA each), which keeps about 16 significant bits; products of bf16
// values are exact in the fp32 accumulators.  Both operands are token-major
// in memory, so each 32-token step stages x[32][64 NW columns] and hi / lo
// [32][EP] in LDS, and the fragments come out transposed by
// ds_read_b64_tr_b16: within a 16-lane group, lane j addresses 4 consecutive
// columns of K row j / 4 of a 4 x 16 block and lane i receives column i's 4 K
// values, so two reads give a lane the 8 consecutive tokens of its MFMA
// operand.  A workgroup of NW waves owns 64 NW columns (64 per wave) for all
// experts and every gridDim.y-th 32-token step, so every token contributes a
// row run of 128 NW bytes.  Two register sets hold the global loads of the next two steps:
// step s + 2 is issued right after step s is in LDS, and the barriers order
// LDS traffic only, so those loads stay in flight across them.  Two LDS
// buffers, one barrier per step: a buffer is rewritten only after every wave
// has passed the barrier that follows its last reads.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int EP, int NW>
struct RwbShape {
  static constexpr int NT = 64 * NW, COLS = 64 * NW;
  static constexpr int CPR = COLS / 8;            // 16-byte chunks per x row
  static constexpr int XP = COLS * 2 + 32;        // x row pitch in bytes: the +32 puts the 4 K rows of a read on other banks
  static constexpr int DP = EP * 2 + 32;          // hi / lo row pitch
  static constexpr int XB = 32 * XP, DB = 32 * DP, BUF = XB + 2 * DB;
  static constexpr int LDS = 2 * BUF;
  // dlogits: 4 experts per thread, DR rows per pass
  static constexpr int DQ = EP / 4, DR = NT / DQ < 32 ? NT / DQ : 32, DPASS = 32 / DR;
};

template <int EP, int NW>
__global__ __launch_bounds__(64 * NW) void router_wgrad_bf16mfma_kernel(const bf16* __restrict__ x,
                                                                       const float* __restrict__ dl,
                                                                       float* __restrict__ partial, int64_t Tn, int d,
                                                                       int E) {
  using S = RwbShape<EP, NW>;
  constexpr int NB = EP / 16, CPR = S::CPR, XP = S::XP, DP = S::DP, XB = S::XB, DB = S::DB, BUF = S::BUF;
  constexpr int DQ = S::DQ, DR = S::DR, DPASS = S::DPASS;
  __shared__ __attribute__((aligned(16))) char lds[S::LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = blockIdx.x * S::COLS;
  const bool dthr = tid / DQ < DR;
  // this workgroup's 32-token steps: global steps blockIdx.y + s gridDim.y,
  // so that the workgroups of a column block read neighbouring tokens at any
  // one time (contiguous blocks of tokens, 2 MB apart on the Mixtral shape,
  // put every workgroup's reads on the same memory channels: 40 against 29
  // us for the route backward, warm)
  const int64_t gsteps = (Tn + 31) / 32;
  const int nbk = (int)gridDim.y;
  const int nsteps = blockIdx.y < gsteps ? (int)((gsteps - blockIdx.y + nbk - 1) / nbk) : 0;
  const int64_t tfirst = 32 * (int64_t)blockIdx.y;  // a valid row for the loads past the end

  // global -> registers for one step: x rows tid / CPR + 8 p, 16-byte chunk
  // tid % CPR; dlogits rows tid / DQ + DR p, experts 4 (tid % DQ) .. + 3.
  // The loads are unconditional, from valid addresses; the zeros past the
  // token range, the last column or E are selected when the registers are
  // written to LDS, so that no select waits for a load in flight.
  const int xcol = c0 + (tid % CPR) * 8;
  const bool xcol_ok = xcol < d;  // d is a multiple of 8: a chunk is all in or all out
  const int de = 4 * (tid % DQ);
  auto gload = [&](int s, u32x4 (&xr)[4], float (&dv)[DPASS][4]) {
    const int64_t t0 = 32 * ((int64_t)blockIdx.y + (int64_t)s * nbk);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int64_t t = t0 + tid / CPR + 8 * p;
      xr[p] = ld16(x + (t < Tn ? t : tfirst) * d + (xcol_ok ? xcol : 0));
    }
#pragma unroll
    for (int p = 0; p < DPASS; ++p) {
      const int64_t t = t0 + tid / DQ + DR * p;
      const int64_t tc = t < Tn ? t : tfirst;
#pragma unroll
      for (int q = 0; q < 4; ++q) dv[p][q] = dl[tc * E + (de + q < E ? de + q : 0)];
    }
  };
  auto lwrite = [&](char* buf, int s, const u32x4 (&xr)[4], const float (&dv)[DPASS][4]) {
    const int64_t t0 = 32 * ((int64_t)blockIdx.y + (int64_t)s * nbk);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool ok = xcol_ok && t0 + tid / CPR + 8 * p < Tn;
      st16(buf + (tid / CPR + 8 * p) * XP + (tid % CPR) * 16, ok ? xr[p] : u32x4{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int p = 0; p < DPASS; ++p) {
      const bool tok = t0 + tid / DQ + DR * p < Tn;
      uint32_t h[4], l[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v = tok && de + q < E ? dv[p][q] : 0.0f;
        h[q] = bf16_bits(v);
        l[q] = bf16_bits(v - __uint_as_float(h[q] << 16));
      }
      const int off = (tid / DQ + DR * p) * DP + de * 2;
      if (dthr) {
        *reinterpret_cast<u32x2*>(buf + XB + off) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        *reinterpret_cast<u32x2*>(buf + XB + DB + off) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
      }
    }
  };

  f32x4 acc[4][NB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // this lane's transposing-read address in a tile: K row 8 G + 4 r + j / 4,
  // column 4 (j % 4) of the 16-column block (G = lane / 16, j = lane % 16)
  const int G = lane >> 4, j = lane & 15;
  const int kr = 8 * G + (j >> 2), cq = 4 * (j & 3);
  auto compute = [&](const char* buf) {
    u32x4 a[4], bh[NB], bl[NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const char* pa = buf + kr * XP + (64 * wave + 16 * mb + cq) * 2;
      const u32x2 r0 = lds_read_tr16(pa), r1 = lds_read_tr16(pa + 4 * XP);
      a[mb] = u32x4{r0[0], r0[1], r1[0], r1[1]};
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const char* ph = buf + XB + kr * DP + (16 * nb + cq) * 2;
      const u32x2 h0 = lds_read_tr16(ph), h1 = lds_read_tr16(ph + 4 * DP);
      const u32x2 l0 = lds_read_tr16(ph + DB), l1 = lds_read_tr16(ph + DB + 4 * DP);
      bh[nb] = u32x4{h0[0], h0[1], h1[0], h1[1]};
      bl[nb] = u32x4{l0[0], l0[1], l1[0], l1[1]};
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[mb]),
                                                              __builtin_bit_cast(bf16x8_t, bh[nb]), acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[mb]),
                                                              __builtin_bit_cast(bf16x8_t, bl[nb]), acc[mb][nb], 0, 0, 0);
      }
  };
  // Register set A carries even steps, B odd ones.  Every load of the first
  // two steps and of the main loop is unconditional (a step past the range
  // reads valid rows that lwrite zeroes), so that the compiler's wait counts
  // see the same loads in flight on every path into the loop: A's loads are
  // then awaited with B's still outstanding.
  if (nsteps == 0) return;
  u32x4 xa[4], xb[4];
  float da[DPASS][4], db[DPASS][4];
  gload(0, xa, da);
  gload(1, xb, db);
  int s = 0;
  for (; s + 3 < nsteps; s += 2) {
    lwrite(lds, s, xa, da);
    lds_only_barrier();
    gload(s + 2, xa, da);
    compute(lds);
    lwrite(lds + BUF, s + 1, xb, db);
    lds_only_barrier();
    gload(s + 3, xb, db);
    compute(lds + BUF);
  }
  // the last one to three steps
  lwrite(lds, s, xa, da);
  lds_only_barrier();
  if (s + 2 < nsteps) gload(s + 2, xa, da);
  compute(lds);
  if (s + 1 < nsteps) {
    lwrite(lds + BUF, s + 1, xb, db);
    lds_only_barrier();
    compute(lds + BUF);
  }
  if (s + 2 < nsteps) {
    lwrite(lds, s + 2, xa, da);
    lds_only_barrier();
    compute(lds);
  }
  // accumulator (mb, nb)[q] of lane l: column 64 wave + 16 mb + 4 (l / 16) + q, expert 16 nb + l % 16
  float* pb = partial + (int64_t)blockIdx.y * d * E;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = c0 + 64 * wave + 16 * mb + 4 * G + q, e = 16 * nb + j;
        if (i < d && e < E) pb[(int64_t)i * E + e] = acc[mb][nb][q];
      }
}

// Workgroups of the bf16 kernel that fit on one compute unit at once (its
// registers and LDS; asked once per instantiation).
template <int EP, int NW>
static hipError_t rwb_per_cu(int* per_cu) {
  static int n = 0;
  static const hipError_t occ = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &n, reinterpret_cast<const void*>(router_wgrad_bf16mfma_kernel<EP, NW>), 64 * NW, 0);
  *per_cu = n > 0 ? n : 1;
  return occ;
}

template <int EP, int NW>
static hipError_t launch_rwg_bf16mfma_nw(const RouteBwdArgs& a, int nb, hipStream_t st) {
  using S = RwbShape<EP, NW>;
  const int64_t gsteps = (a.T + 31) / 32;
  const int nbr = (int)(nb < gsteps ? nb : gsteps);  // token blocks, each with at least one step
  const dim3 grid((unsigned)((a.d + S::COLS - 1) / S::COLS), nbr);
  hipLaunchKernelGGL((router_wgrad_bf16mfma_kernel<EP, NW>), grid, dim3(S::NT), 0, st, (const bf16*)a.x, a.dlogits,
                     a.partial, a.T, (int)a.d, a.E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_rwg_reduce<bf16>(a, nbr, st);
}

// Column width: the widest block (longest row runs) whose workgroups still
// give every compute unit one; token blocks: as many as fill the resident
// slots once, at most router_wgrad_blocks(T) (the planned partials).
template <int EP>
static hipError_t launch_rwg_bf16mfma(const RouteBwdArgs& a, hipStream_t st) {
  int cus = 0;
  hipError_t err = device_cus(&cus);
  if (err != hipSuccess) return err;
  const int nbmax = router_wgrad_blocks(a.T);
  auto blocks = [&](int cols, int per_cu) {
    const int64_t cb = (a.d + cols - 1) / cols;
    int64_t nb = ((int64_t)cus * per_cu + cb - 1) / cb;
    return (int)(nb < 1 ? 1 : nb > nbmax ? nbmax : nb);
  };
  int per_cu = 1;
  if ((a.d + 511) / 512 * nbmax >= cus) {
    if ((err = rwb_per_cu<EP, 8>(&per_cu)) != hipSuccess) return err;
    return launch_rwg_bf16mfma_nw<EP, 8>(a, blocks(512, per_cu), st);
  }
  if ((a.d + 255) / 256 * nbmax >= cus) {
    if ((err = rwb_per_cu<EP, 4>(&per_cu)) != hipSuccess) return err;
    return launch_rwg_bf16mfma_nw<EP, 4>(a, blocks(256, per_cu), st);
  }
  if ((err = rwb_per_cu<EP, 2>(&per_cu)) != hipSuccess) return err;
  return launch_rwg_bf16mfma_nw<EP, 2>(a, blocks(128, per_cu), st);
}

// bf16 x: the bf16 MFMA kernel with dlogits as hi + lo, E padded to 16, 32
// or 64.  Up to 16 experts it replaced the vector kernel (route backward,
// warm / cold caches: GPT-2 24.8 / 30.1 -> 16.9 / 24.9 us, BERT-L 36.3 / 40.7
// -> 22.5 / 28.3 us, Mixtral 39.2 / 45.0 -> 36.0 / 45.4 us); with more
// experts it replaced the fp32 MFMA kernel (DeepSeek-V2-Lite 0.14 -> 0.05 ms).
// Column blocks of up to 512, two steps of loads in flight, a grid sized to
// the resident slots and the 16-way reduce then took the route backward
// inside full steps from 26.5 to 15.9 us (GPT-2), 31.3 to 22.2 (BERT-L), 50.9
// to 45.5 (Mixtral) and 50.2 to 41.0 (DeepSeek-V2-Lite).
// fp32 x: the fp32 MFMA kernel.
template <typename T>
static hipError_t launch_rwg_dt(const RouteBwdArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (a.E <= 16) return launch_rwg_bf16mfma<16>(a, st);
  }
  if (a.E <= 16) return launch_rwg_mfma<T, 16>(a, st);
  if constexpr (sizeof(T) == 2) {
    if (a.E <= 32) return launch_rwg_bf16mfma<32>(a, st);
    return launch_rwg_bf16mfma<64>(a, st);
  }
  if (a.E <= 32) return launch_rwg_mfma<T, 32>(a, st);
  return launch_rwg_mfma<T, 64>(a, st);
}

int router_wgrad_blocks(int64_t T) {
  int64_t nb = (T + 127) / 128;
  if (nb > 64) nb = 64;
  if (nb < 1) nb = 1;
  return (int)nb;
}

hipError_t launch_route_bwd(const RouteBwdArgs& a, bool bf16_dtype, hipStream_t st) {
  hipError_t err = a.E <= 8 ? launch_gating_bwd<8>(a, st)
                   : a.E <= 16 ? launch_gating_bwd<16>(a, st)
                   : a.E <= 32 ? launch_gating_bwd<32>(a, st)
                   : launch_gating_bwd<64>(a, st);
  if (err != hipSuccess) return err;
  return bf16_dtype ? launch_rwg_dt<bf16>(a, st) : launch_rwg_dt<float>(a, st);
}

}  // namespace moe
