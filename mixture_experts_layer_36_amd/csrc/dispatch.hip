// Capacity, counts, EP send layout and token permutation.
//
// Follows the tutorial ch.4 "All-to-All 通信模式" part 二 (device i sends to
// device k the set S_ik of its tokens whose expert lives on k) and part 六
// (those sets have different sizes), and the Piper summary's 方法论 1
// (expert capacity).  Position of assignment (t, j) in its expert's buffer:
// pos = number of tokens t' < t that chose the same expert; it is kept iff
// pos < C, so overflow is dropped in token order.
//
// Stable positions without order-dependent atomics, in three launches (four
// for inputs of more than kFusedScanBlocks blocks, where a one-workgroup
// scan kernel replaces the per-workgroup sums of step 2):
//   1. block_hist: per block of 256 tokens, count the tokens choosing each
//      expert (integer LDS atomics: the count does not depend on order);
//   2. rows: per block, the sums of the block counts before it and in all
//      (each workgroup reduces them itself, so no separate scan launch) give
//      the per-expert bases, raw / kept counts, slot offsets and send
//      segments; each token's rank among the block's earlier tokens (a 64-bit
//      wave ballot per expert and the count of set bits below the lane, then
//      a prefix over the 4 waves) gives pos, the
//      kept flag, the row, row_of and assign_of_row;
//   3. copy: each kept token row is read once and written to its <= k rows
//      (16-byte loads / stores, coalesced along the row).
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(kDispatchBlock) void block_hist_kernel(const int32_t* __restrict__ idx, int64_t Tn,
                                                                    int E, int k, int32_t* __restrict__ block_counts) {
  __shared__ int cnt[64];
  const int tid = threadIdx.x;
  if (tid < 64) cnt[tid] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kDispatchBlock + tid;
  if (t < Tn) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  if (tid < E) block_counts[(int64_t)blockIdx.x * E + tid] = cnt[tid];
}

__device__ __forceinline__ int slot_expert(int s, int E, int R, int placement) {
  const int L = E / R;
  return placement == 0 ? s : (s % L) * R + s / L;
}

// Inclusive prefix sum over the 64 lanes of a wave.
template <typename V>
__device__ __forceinline__ V wave_incl_scan(V v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Many blocks (nb > kFusedScanBlocks): one workgroup of 16 waves scans the
// block counts once for all.  Wave w scans the block-count columns of experts
// w, w + 16, ...: 64 blocks per round, one per lane, by a wave prefix sum plus
// the carry of the earlier rounds (block_base = exclusive prefix down the
// column).  Then wave 0 takes one slot per lane for the prefix over the kept
// counts in slot order, and the send segments.
constexpr int kScanWaves = 16;

__global__ __launch_bounds__(64 * kScanWaves) void scan_kernel(
    const int32_t* __restrict__ block_counts, int nb, int E, int64_t C, int R, int placement,
    int32_t* __restrict__ block_base, int32_t* __restrict__ raw_counts, int32_t* __restrict__ kept_counts,
    int64_t* __restrict__ slot_offsets, int32_t* __restrict__ send_counts, int64_t* __restrict__ send_offsets,
    int64_t* __restrict__ expert_start) {
  __shared__ int64_t kept_s[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = wave; e < E; e += kScanWaves) {
    int carry = 0;  // counts are per-token assignments: T * k < 2^31
    for (int b0 = 0; b0 < nb; b0 += 64) {
      const int b = b0 + lane;
      const int v = b < nb ? block_counts[(int64_t)b * E + e] : 0;
      const int incl = wave_incl_scan(v, lane);
      if (b < nb) block_base[(int64_t)b * E + e] = carry + incl - v;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      raw_counts[e] = carry;
      const int64_t kept = carry < C ? carry : C;
      kept_counts[e] = (int32_t)kept;
      kept_s[e] = kept;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const int ex = lane < E ? slot_expert(lane, E, R, placement) : 0;
  const int64_t v = lane < E ? kept_s[ex] : 0;
  const int64_t incl = wave_incl_scan(v, lane), excl = incl - v;
  const int64_t total = __shfl(incl, 63, 64);
  if (lane < E) {
    slot_offsets[lane] = excl;
    expert_start[ex] = excl;
  }
  // send segment q = lane < R: slots [q L, (q + 1) L)
  const int L = E / R;
  const int s0 = lane < R ? lane * L : 0, s1 = lane < R ? (lane + 1) * L : 0;
  const int64_t o0 = __shfl(excl, s0 & 63, 64);
  const int64_t o1 = s1 < E ? __shfl(excl, s1 & 63, 64) : total;
  if (lane < R) {
    send_offsets[lane] = o0;
    send_counts[lane] = (int32_t)(o1 - o0);
  }
  if (lane == 0) {
    slot_offsets[E] = total;
    send_offsets[R] = total;
  }
}

// Positions and rows, one workgroup per block of kDispatchBlock tokens.
//  a. Each workgroup reduces the block counts itself (nb x E integers that
//     every workgroup reads, from L2): base[e] = tokens of earlier blocks that
//     chose expert e, raw[e] = all of them; kept[e] = min(raw[e], C).  Thread
//     tid adds expert tid % E over the blocks tid / E, tid / E + G, ... and
//     wave 0 sums the G partials of each expert.
//  b. Wave 0 turns the kept counts into slot offsets (a wave prefix sum in
//     slot order), hence each expert's first row; workgroup 0 also writes the
//     counts, the slot offsets and the send segments.
//  c. Each token's rank among the block's earlier tokens choosing the same
//     expert (64-bit wave ballots + popcount, then a prefix over the waves)
//     gives pos = base + rank, the kept flag (pos < C) and the row.
// Every workgroup reading every block count costs nb^2 E reads in all, so
// with more than kFusedScanBlocks blocks (FUSED = false) a and b come from the
// scan kernel's block_base and expert_start instead.
constexpr int kFusedScanBlocks = 128;

template <bool FUSED>
__global__ __launch_bounds__(kDispatchBlock) void dispatch_rows_kernel(
    const int32_t* __restrict__ idx, int64_t Tn, int E, int k, int64_t C, int R, int placement,
    const int32_t* __restrict__ block_counts, int nb, int32_t* __restrict__ raw_counts,
    int32_t* __restrict__ kept_counts, int64_t* __restrict__ slot_offsets, int32_t* __restrict__ send_counts,
    int64_t* __restrict__ send_offsets, const int32_t* __restrict__ block_base,
    const int64_t* __restrict__ expert_start, int32_t* __restrict__ row_of, int32_t* __restrict__ assign_of_row) {
  constexpr int NT = kDispatchBlock, NW = NT / 64;
  __shared__ int pre_s[NT], tot_s[NT];
  __shared__ int base_s[64];
  __shared__ int64_t start_s[64];
  __shared__ int wave_cnt[NW][64];
  __shared__ uint8_t rank_s[NW][64][64];  // [wave][expert][lane]: rank among the wave's earlier lanes
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  const int64_t t = (int64_t)b * NT + tid;
  int my_e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) my_e[j] = (j < k && t < Tn) ? idx[t * k + j] : -1;

  // a. partial sums of the block counts (E <= 64, so G >= 4)
  const int G = NT / E;
  if (FUSED) {
    int pre = 0, tot = 0;
    if (tid < G * E) {
      const int e = tid % E;
      for (int bb = tid / E; bb < nb; bb += G) {
        const int v = block_counts[(int64_t)bb * E + e];
        tot += v;
        pre += bb < b ? v : 0;
      }
    }
    pre_s[tid] = pre;
    tot_s[tid] = tot;
  }

  // c (first half). ranks within the wave, and the wave's count per expert.
  // Bit e of the lane's mask is set when one of its choices is expert e (a
  // token picks an expert at most once); per expert, a ballot of that bit
  // and the count of set bits below the lane (mbcnt) give the rank, which
  // the lane leaves in LDS and reads back for its k choices afterwards.
  uint32_t em[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (my_e[j] >= 0 && my_e[j] < E) em[my_e[j] >> 5] |= 1u << (my_e[j] & 31);
  for (int e = 0; e < E; ++e) {
    const bool c = (em[e >> 5] >> (e & 31)) & 1u;
    const unsigned long long mask = __ballot(c);
    const int before = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    if (c) rank_s[w][e][lane] = (uint8_t)before;
    if (lane == 0) wave_cnt[w][e] = __popcll(mask);
  }
  int rank[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rank[j] = (my_e[j] >= 0 && my_e[j] < E) ? rank_s[w][my_e[j]][lane] : 0;
  __syncthreads();

  // a (end) and b. wave 0: lane e holds expert e's base and raw count; lane s
  // holds slot s for the prefix in slot order
  if (!FUSED) {
    if (tid < E) {
      base_s[tid] = block_base[(int64_t)b * E + tid];
      start_s[tid] = expert_start[tid];
    }
  } else if (w == 0) {
    int base = 0, raw = 0;
    if (lane < E) {
      for (int g = 0; g < G; ++g) {
        base += pre_s[g * E + lane];
        raw += tot_s[g * E + lane];
      }
      base_s[lane] = base;
    }
    const int64_t kept = lane < E ? (raw < C ? raw : C) : 0;
    const int ex = lane < E ? slot_expert(lane, E, R, placement) : 0;
    const int64_t v = __shfl(kept, ex, 64);  // kept count of slot lane's expert
    const int64_t sv = lane < E ? v : 0;
    const int64_t incl = wave_incl_scan(sv, lane), excl = incl - sv;
    const int64_t total = __shfl(incl, 63, 64);
    if (lane < E) start_s[ex] = excl;
    if (b == 0) {
      if (lane < E) {
        raw_counts[lane] = raw;
        kept_counts[lane] = (int32_t)kept;
        slot_offsets[lane] = excl;
      }
      // send segment q = lane < R: slots [q L, (q + 1) L)
      const int L = E / R;
      const int s0 = lane < R ? lane * L : 0, s1 = lane < R ? (lane + 1) * L : 0;
      const int64_t o0 = __shfl(excl, s0 & 63, 64);
      const int64_t o1 = s1 < E ? __shfl(excl, s1 & 63, 64) : total;
      if (lane < R) {
        send_offsets[lane] = o0;
        send_counts[lane] = (int32_t)(o1 - o0);
      }
      if (lane == 0) {
        slot_offsets[E] = total;
        send_offsets[R] = total;
      }
    }
  }
  __syncthreads();

  // c (end). position, kept flag and row of each of the token's choices
  if (t >= Tn) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const int e = my_e[j];
    int32_t row = -1;
    if (e >= 0 && e < E) {
      int prefix = 0;
      for (int ww = 0; ww < w; ++ww) prefix += wave_cnt[ww][e];
      const int64_t pos = (int64_t)base_s[e] + prefix + rank[j];
      if (pos < C) {
        row = (int32_t)(start_s[e] + pos);
        assign_of_row[row] = (int32_t)(t * k + j);
      }
    }
    row_of[t * k + j] = row;
  }
}

// One wave per token: its kept rows (wave-uniform scalar loads) receive the
// token's row; each lane moves the 16-byte chunks lane, lane + 64, ... of it,
// U at a time (2, 4 or 8 by row width), with the U loads issued before the
// stores.
constexpr int kCopyWaves = 4;

template <typename T, int KMAX, int U>
__global__ __launch_bounds__(64 * kCopyWaves) void permute_copy_kernel(const T* __restrict__ x,
                                                                       const int32_t* __restrict__ row_of,
                                                                       T* __restrict__ x_perm, int64_t Tn, int d,
                                                                       int k) {
  constexpr int V = Vec16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kCopyWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= Tn) return;
  int rows[KMAX];
  bool any = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rows[j] = j < k ? row_of[t * k + j] : -1;
    any |= rows[j] >= 0;
  }
  if (!any) return;  // a fully dropped token is not read
  const int nch = d / V;
  for (int c0 = lane; c0 < nch; c0 += 64 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      v[u] = c < nch ? ld16(x + t * d + (int64_t)c * V) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (rows[j] < 0) continue;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 64 * u;
        if (c < nch) st16(x_perm + (int64_t)rows[j] * d + (int64_t)c * V, v[u]);
      }
    }
  }
}

template <typename T, int KMAX>
static void launch_permute_copy_k(const DispatchArgs& a, hipStream_t st) {
  const int64_t blocks = (a.T + kCopyWaves - 1) / kCopyWaves;
  if (blocks <= 0) return;
  // chunks per lane per round: one round per row on wide rows, fewer where
  // most lanes would have nothing to move
  const int64_t nch = a.d * (int64_t)sizeof(T) / 16;
  const dim3 grid((unsigned)blocks), block(64 * kCopyWaves);
  if (nch > 256)
    hipLaunchKernelGGL((permute_copy_kernel<T, KMAX, 8>), grid, block, 0, st, (const T*)a.x, a.row_of,
                       (T*)a.x_perm, a.T, (int)a.d, a.k);
  else if (nch > 128)
    hipLaunchKernelGGL((permute_copy_kernel<T, KMAX, 4>), grid, block, 0, st, (const T*)a.x, a.row_of,
                       (T*)a.x_perm, a.T, (int)a.d, a.k);
  else
    hipLaunchKernelGGL((permute_copy_kernel<T, KMAX, 2>), grid, block, 0, st, (const T*)a.x, a.row_of,
                       (T*)a.x_perm, a.T, (int)a.d, a.k);
}

template <typename T>
static void launch_permute_copy(const DispatchArgs& a, hipStream_t st) {
  if (a.k <= 2) launch_permute_copy_k<T, 2>(a, st);
  else launch_permute_copy_k<T, 8>(a, st);
}

hipError_t launch_permute(const DispatchArgs& a, bool bf16_dtype, hipStream_t st) {
  if (bf16_dtype) launch_permute_copy<bf16>(a, st);
  else launch_permute_copy<float>(a, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rows of token chunks.  With the layout above, the kept rows of expert e
// are its first C choosers in token order, so the tokens of a chunk
// [t_r, t_{r+1}) occupy a contiguous sub-range of each expert's segment:
// rows [b_r, b_{r+1}) with b_r = the first kept row of e chosen by a token
// t >= t_r (the segment's end if none).  chunk_rows[r][s] = b_r of send slot
// s: the group tables of the chunks (offsets = row r, ends = row r + 1).
// Three launches: fill every row with the segment ends (row 0 with the
// starts), an integer atomicMin per kept assignment (order independent, so
// deterministic), then a suffix minimum over the chunks so that a chunk
// without rows of e starts where the next one does.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int slot_of_expert(int e, int E, int R, int placement) {
  const int L = E / R;
  return placement == 0 ? e : (e % R) * L + e / R;
}

__global__ __launch_bounds__(64) void chunk_rows_init_kernel(const int64_t* __restrict__ offsets, int E,
                                                             int chunks, int64_t* __restrict__ rows) {
  for (int i = threadIdx.x; i < (chunks + 1) * E; i += 64) {
    const int r = i / E, s = i - r * E;
    rows[i] = r == 0 ? offsets[s] : offsets[s + 1];
  }
}

__global__ __launch_bounds__(256) void chunk_rows_min_kernel(const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ row_of, int64_t Tn, int E,
                                                             int k, int R, int placement, ChunkBounds cb,
                                                             int64_t* __restrict__ rows) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // assignment t * k + j
  if (i >= Tn * k) return;
  const int32_t row = row_of[i];
  if (row < 0) return;
  const int64_t t = i / k;
  int r = 0;
  while (r + 1 < cb.chunks && t >= cb.t[r + 1]) ++r;
  if (r == 0) return;  // row 0 holds the segment starts already
  const int s = slot_of_expert(idx[i], E, R, placement);
  atomicMin((unsigned long long*)&rows[(int64_t)r * E + s], (unsigned long long)row);
}

__global__ __launch_bounds__(64) void chunk_rows_suffix_kernel(int E, int chunks, int64_t* __restrict__ rows) {
  for (int s = threadIdx.x; s < E; s += 64)
    for (int r = chunks - 1; r >= 1; --r) {
      const int64_t nxt = rows[(int64_t)(r + 1) * E + s];
      if (nxt < rows[(int64_t)r * E + s]) rows[(int64_t)r * E + s] = nxt;
    }
}

hipError_t launch_chunk_rows(const ChunkRowsArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(chunk_rows_init_kernel, dim3(1), dim3(64), 0, st, a.expert_offsets, a.E, a.cb.chunks, a.rows);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n = a.T * a.k;
  if (a.cb.chunks > 1 && n > 0) {
    hipLaunchKernelGGL(chunk_rows_min_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.topk_idx,
                       a.row_of, a.T, a.E, a.k, a.R, a.placement, a.cb, a.rows);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(chunk_rows_suffix_kernel, dim3(1), dim3(64), 0, st, a.E, a.cb.chunks, a.rows);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& a, bool bf16_dtype, hipStream_t st) {
  const int nb = (int)((a.T + kDispatchBlock - 1) / kDispatchBlock);
  hipLaunchKernelGGL(block_hist_kernel, dim3(nb), dim3(kDispatchBlock), 0, st, a.topk_idx, a.T, a.E, a.k,
                     a.block_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (nb <= kFusedScanBlocks) {
    hipLaunchKernelGGL(dispatch_rows_kernel<true>, dim3(nb), dim3(kDispatchBlock), 0, st, a.topk_idx, a.T, a.E,
                       a.k, a.C, a.R, a.placement, a.block_counts, nb, a.raw_counts, a.expert_counts,
                       a.expert_offsets, a.send_counts, a.send_offsets, nullptr, nullptr, a.row_of,
                       a.assign_of_row);
  } else {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(64 * kScanWaves), 0, st, a.block_counts, nb, a.E, a.C, a.R,
                       a.placement, a.block_base, a.raw_counts, a.expert_counts, a.expert_offsets, a.send_counts,
                       a.send_offsets, a.expert_start);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(dispatch_rows_kernel<false>, dim3(nb), dim3(kDispatchBlock), 0, st, a.topk_idx, a.T, a.E,
                       a.k, a.C, a.R, a.placement, a.block_counts, nb, a.raw_counts, a.expert_counts,
                       a.expert_offsets, a.send_counts, a.send_offsets, a.block_base, a.expert_start, a.row_of,
                       a.assign_of_row);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (!a.x_perm) return hipSuccess;  // layout only
  return launch_permute(a, bf16_dtype, st);
}

}  // namespace moe
