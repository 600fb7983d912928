// Host-side check of every direct-to-LDS load of the bf16 grouped-GEMM
// launches of one expert FFN forward + backward (libmoe's gemm3 kernels), for
// a given group table, before any of it runs on a GPU.
//
// The kernels take their tile mapping, per-lane load offsets and buffer
// resource spans from gemm_addr.h; this program calls the same functions for
// every workgroup of each launch, every wave and lane, and a sample of K
// stages (all of them for short reductions; otherwise the first and last
// eight and an even spread), and checks each load against the tensor it
// reads, whose size it derives only from the shapes:
//   * every resource span starts 16-byte aligned, fits below the extent cap,
//     and every offset fits 31 bits;
//   * a load the hardware serves (offset below the extent) reads 16 bytes
//     inside the tensor, exactly at the element the tile needs there;
//   * a load of an element the tile needs (inside the group's rows, the
//     operand's columns and K) is served; a load of anything else is masked
//     or past the extent (reads zeros);
//   * every LDS destination lies inside its stage;
//   * the row-split launches map their real tiles one to one onto workgroups.
//
// Input (stdin), one FFN call:  d F swiglu groups rows_max rr_R rr_L
// followed by groups+1 offsets, and optionally a chunk count followed by
// chunks+1 rows of per-group bounds (token chunks of every group: the
// row-split launches are then also checked once per chunk on the sub-ranges
// [bounds[r][g], bounds[r+1][g])).  Output: "OK <loads checked>" or the first
// violation, exit status 1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "gemm_addr.h"

using namespace moe::gemm_addr;

namespace {

constexpr int BM = 256, BN = 256, BK = 32, NW = 8;  // the tile every gemm3 launch uses

long long g_checked = 0;

[[noreturn]] void fail(const std::string& what) {
  std::printf("FAIL %s\n", what.c_str());
  std::exit(1);
}

struct Tensor {
  const char* name;
  int64_t bytes;  // allocation size
};

// One load: resource span [span.base, span.base + span.bytes) of tensor t,
// offset off + soff (kOOB when masked); the element the tile needs there is at
// byte `want` of t, and `valid` says whether it exists (else zero is needed).
void check_load(const char* launch, const Tensor& t, const Span& span, uint32_t off, uint32_t soff, bool valid,
                int64_t want, int lds_dst, int stage_bytes) {
  ++g_checked;
  char buf[512];
  if (lds_dst < 0 || lds_dst + 16 > stage_bytes) {
    std::snprintf(buf, sizeof buf, "%s %s: LDS destination %d outside the stage of %d bytes", launch, t.name,
                  lds_dst, stage_bytes);
    fail(buf);
  }
  if (span.base % 16 != 0 || span.bytes > kMaxExtent) {
    std::snprintf(buf, sizeof buf, "%s %s: span base %lld bytes %lld (alignment or extent cap)", launch, t.name,
                  (long long)span.base, (long long)span.bytes);
    fail(buf);
  }
  const bool masked = off == kOOB;
  const int64_t rel = (int64_t)off + soff;
  const bool served = !masked && rel + 16 <= span.bytes;
  if (!masked && rel < span.bytes && !served) {
    std::snprintf(buf, sizeof buf, "%s %s: a 16-byte load straddles the extent (offset %lld of %lld)", launch,
                  t.name, (long long)rel, (long long)span.bytes);
    fail(buf);
  }
  if (!masked && (rel >= ((int64_t)1 << 31) || rel % 16 != 0)) {
    std::snprintf(buf, sizeof buf, "%s %s: offset %lld (31-bit range, 16-byte alignment)", launch, t.name,
                  (long long)rel);
    fail(buf);
  }
  if (valid && !served) {
    std::snprintf(buf, sizeof buf, "%s %s: a needed element (byte %lld) is read as zero", launch, t.name,
                  (long long)want);
    fail(buf);
  }
  if (!served) return;
  const int64_t abs = span.base + rel;
  if (!valid) {
    std::snprintf(buf, sizeof buf, "%s %s: byte %lld is loaded where zeros are needed", launch, t.name,
                  (long long)abs);
    fail(buf);
  }
  if (abs < 0 || abs + 16 > t.bytes) {
    std::snprintf(buf, sizeof buf, "%s %s: load of bytes [%lld, %lld) outside the tensor of %lld", launch, t.name,
                  (long long)abs, (long long)(abs + 16), (long long)t.bytes);
    fail(buf);
  }
  if (abs != want) {
    std::snprintf(buf, sizeof buf, "%s %s: load at byte %lld, the tile needs byte %lld", launch, t.name,
                  (long long)abs, (long long)want);
    fail(buf);
  }
}

std::vector<int> sample_stages(int nk) {
  std::vector<int> s;
  if (nk <= 48) {
    for (int i = 0; i < nk; ++i) s.push_back(i);
    return s;
  }
  std::set<int> st;
  for (int i = 0; i < 8; ++i) {
    st.insert(i);
    st.insert(nk - 1 - i);
  }
  for (int i = 0; i < nk; i += nk / 16) st.insert(i);
  return std::vector<int>(st.begin(), st.end());
}

struct RowsLaunch {
  const char* name;
  bool dgrad, pair;
  Tensor A, B, B2;
  int64_t lda, ldb, gstride, N, K, b_split;
  const int32_t* gather = nullptr;  // the fused forward: A rows gathered from the token rows
  int gather_k = 1;
  int64_t gather_rows = 0;
};

// ends: null (group g owns [off[g], off[g + 1])) or [groups] sub-range ends.
void check_rows(const RowsLaunch& L, const std::vector<int64_t>& off, const int64_t* ends, int groups,
                int64_t rows_max, int rr_R, int rr_L, int weight_sets) {
  int tiles_m, tiles_n;
  rows_tiles(L.N, L.pair ? BN / 2 : BN, rows_max, groups, BM, tiles_m, tiles_n);
  const int64_t grid = (int64_t)tiles_m * tiles_n;
  int real_m = 0;
  for (int g = 0; g < groups; ++g) real_m += (int)((group_end(off.data(), ends, g) - off[g] + BM - 1) / BM);
  std::set<std::tuple<int, int64_t, int>> seen;
  const int real = real_m * tiles_n;
  const int every = real > 600 ? real / 600 : 1;
  constexpr int A_BYTES = BM * BK * 2, STAGE = A_BYTES + BN * BK * 2;
  constexpr int QA = Units<BM, BK, NW>::PER, QB = Units<BN, BK, NW>::PER;
  for (int hw = 0; hw < grid; ++hw) {
    int g = -1, nt = 0;
    int64_t rb = 0, re = 0;
    if (!row_tile_of<BM>(off.data(), ends, groups, tiles_n, 8, hw, g, rb, re, nt)) {
      if (hw < real) fail(std::string(L.name) + ": a real tile's workgroup exits");
      continue;
    }
    if (hw >= real) fail(std::string(L.name) + ": a surplus workgroup takes a tile");
    if (!seen.insert({g, rb, nt}).second) fail(std::string(L.name) + ": two workgroups take one tile");
    const int64_t gend = group_end(off.data(), ends, g);
    if (rb < off[g] || rb >= gend || re != gend || (rb - off[g]) % BM != 0)
      fail(std::string(L.name) + ": tile rows outside its group");
    const int wi = weight_index(g, rr_R, rr_L);
    if (wi < 0 || wi >= weight_sets) fail(std::string(L.name) + ": weight set out of range");
    const bool last_row = rb + BM >= re, last_col = nt == tiles_n - 1;
    if (!(hw % every == 0 || last_row || last_col)) continue;
    const int64_t rows_valid = min64(BM, re - rb);
    const int64_t n0 = L.pair ? (int64_t)nt * (BN / 2) : (int64_t)nt * BN;
    const int64_t set0 = (int64_t)wi * L.gstride * 2;
    const Span sa = L.gather ? gather_a_span(L.gather_rows, L.lda) : rows_a_span(rb, rows_valid, L.lda);
    const StageWalk wb = fwd_b_walk(n0, BK, L.ldb);
    const int nk = (int)((L.K + BK - 1) / BK);
    for (int kt : sample_stages(nk)) {
      const int64_t k0 = (int64_t)kt * BK;
      for (int wave = 0; wave < NW; ++wave)
        for (int lane = 0; lane < 64; ++lane) {
          for (int i = 0; i < QA; ++i) {  // A: the tile's rows, K-contiguous
            int row, col;
            kc_lane<BK, NW>(i, wave, lane, row, col);
            const bool valid = row < rows_valid && k0 + col < L.K;
            uint32_t o;
            int64_t want;
            if (L.gather) {  // the lane's token row, masked through its K column past the group
              const int64_t tok = row < rows_valid ? gather_token(L.gather[rb + row], L.gather_k) : 0;
              const int kc = kc_gather_col(row, col, rows_valid);
              o = k0 + kc < L.K ? (uint32_t)((tok * L.lda + col) * 2) : kOOB;
              want = (tok * L.lda + k0 + col) * 2;
            } else {
              o = k0 + col < L.K ? (uint32_t)(((int64_t)row * L.lda + col) * 2) : kOOB;
              want = ((rb + row) * L.lda + k0 + col) * 2;
            }
            check_load(L.name, L.A, sa, o, (uint32_t)(k0 * 2), valid, want, (i * NW + wave) * 1024 + lane * 16,
                       A_BYTES);
          }
          for (int i = 0; i < QB; ++i) {
            const int dst = (i * NW + wave) * 1024 + lane * 16;
            if (L.dgrad) {  // weights K-contiguous: rows n of [N][ldb], K split over two tensors
              int row, col;
              kc_lane<BK, NW>(i, wave, lane, row, col);
              const bool second = L.b_split > 0 && k0 >= L.b_split;
              const int64_t kk0 = second ? k0 - L.b_split : k0;
              const int64_t klim = second ? L.K - L.b_split : (L.b_split > 0 ? L.b_split : L.K);
              const Tensor& t = second ? L.B2 : L.B;
              Span sb = dgrad_b_span(0, n0, BN, L.N, L.ldb);
              sb.base += set0;
              const bool ok = kk0 + col < klim;
              const uint32_t o = ok ? (uint32_t)(((int64_t)row * L.ldb + col) * 2) : kOOB;
              const bool valid = n0 + row < L.N && kk0 + col < klim;
              const int64_t want = set0 + ((n0 + row) * L.ldb + kk0 + col) * 2;
              check_load(L.name, t, sb, o, (uint32_t)(kk0 * 2), valid, want, dst, STAGE - A_BYTES);
            } else {  // weights N-contiguous: K rows of [K][ldb]
              int panel, k, col;
              mn_lane<BK, NW>(i, wave, lane, L.pair, panel, k, col);
              const Tensor& t = (L.pair && panel) ? L.B2 : L.B;
              Span sb = stage_span(wb, kt);
              sb.base += set0;
              const bool colok = col < L.N - n0;
              const bool ok = colok && k0 + k < L.K;
              const uint32_t o = ok ? (uint32_t)(((int64_t)k * L.ldb + col) * 2) : kOOB;
              const bool valid = k0 + k < L.K && n0 + col < L.N;
              const int64_t want = set0 + ((k0 + k) * L.ldb + n0 + col) * 2;
              check_load(L.name, t, sb, o, 0u, valid, want, dst, STAGE - A_BYTES);
            }
          }
        }
    }
  }
  if ((int)seen.size() != real) fail(std::string(L.name) + ": some real tile has no workgroup");
}

struct WgradLaunch {
  const char* name;
  Tensor A, B;
  int64_t lda, ldb, M, N;
  int ksplit;
};

void check_wgrad(const WgradLaunch& L, const std::vector<int64_t>& off, int groups) {
  int tiles_m, tiles_n;
  wgrad_tiles(L.M, L.N, BM, BN, tiles_m, tiles_n);
  const int per_g = tiles_m * tiles_n;
  const int64_t items = (int64_t)L.ksplit * groups * per_g;
  const int every = items > 600 ? (int)(items / 600) : 1;
  constexpr int A_BYTES = BM * BK * 2, STAGE = A_BYTES + BN * BK * 2;
  constexpr int QA = Units<BM, BK, NW>::PER, QB = Units<BN, BK, NW>::PER;
  for (int64_t it = 0; it < items; ++it) {
    const int split = (int)(it / ((int64_t)groups * per_g));
    const int rem = (int)(it - (int64_t)split * groups * per_g);
    const int g = rem / per_g, tile = rem - g * per_g;
    int mt, nt;
    grouped_order(tile, tiles_m, tiles_n, mt, nt, 8);
    if (mt >= tiles_m || nt >= tiles_n) fail(std::string(L.name) + ": tile outside the grid");
    int64_t r0 = off[g], r1 = off[g + 1];
    if (L.ksplit > 1) split_rows(off[g], off[g + 1], L.ksplit, split, BK, r0, r1);
    if (r0 < off[g] || r1 > off[g + 1] || r1 < r0) fail(std::string(L.name) + ": split rows outside the group");
    const bool last = r1 - r0 > 0 && (mt == tiles_m - 1 || nt == tiles_n - 1);
    if (!(it % every == 0 || last)) continue;
    const int64_t Kr = r1 - r0, m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;
    const StageWalk wa = wgrad_walk(r0, m0, BK, L.lda), wb = wgrad_walk(r0, n0, BK, L.ldb);
    const int nk = (int)((Kr + BK - 1) / BK);
    for (int kt : sample_stages(nk)) {
      const int64_t k0 = (int64_t)kt * BK;
      const Span sa = stage_span(wa, kt), sb = stage_span(wb, kt);
      for (int wave = 0; wave < NW; ++wave)
        for (int lane = 0; lane < 64; ++lane) {
          for (int i = 0; i < QA + QB; ++i) {
            const bool isb = i >= QA;
            const int ii = isb ? i - QA : i;
            const int64_t ld = isb ? L.ldb : L.lda, c0 = isb ? n0 : m0, C = isb ? L.N : L.M;
            int panel, k, col;
            mn_lane<BK, NW>(ii, wave, lane, false, panel, k, col);
            const bool ok = col < C - c0 && k0 + k < Kr;
            const uint32_t o = ok ? (uint32_t)(((int64_t)k * ld + col) * 2) : kOOB;
            const bool valid = k0 + k < Kr && c0 + col < C;
            const int64_t want = ((r0 + k0 + k) * ld + c0 + col) * 2;
            check_load(L.name, isb ? L.B : L.A, isb ? sb : sa, o, 0u, valid, want,
                       (ii * NW + wave) * 1024 + lane * 16, isb ? STAGE - A_BYTES : A_BYTES);
          }
        }
    }
  }
}

// The weight transpose over a [rows][cols] source: every workgroup's tile
// inside the grid and each tile once, every source load and output store in
// bounds, each LDS chunk written once per tile, each output chunk's 8 column
// elements read from the LDS slots its source rows were written to, and every
// output element written exactly once with the source element it transposes.
void check_transpose(const char* name, int64_t rows, int64_t cols) {
  const int64_t gx = (cols + 63) / 64, gy = (rows + 63) / 64;
  std::vector<uint8_t> done((size_t)(rows * cols), 0);
  std::vector<int64_t> lds(64 * 64);
  std::set<std::pair<int64_t, int64_t>> tiles;
  for (int L = 0; L < (int)(gx * gy); ++L) {
    int64_t r0, c0;
    transpose_tile(L, rows, cols, r0, c0);
    if (r0 < 0 || c0 < 0 || r0 >= gy * 64 || c0 >= gx * 64 || r0 % 64 || c0 % 64 || !tiles.insert({r0, c0}).second)
      fail(std::string(name) + ": transpose tile outside the grid or repeated");
    std::fill(lds.begin(), lds.end(), -1);
    for (int tid = 0; tid < 256; ++tid)
      for (int j = 0; j < 2; ++j) {
        int tr, tc;
        transpose_load_lane(tid, j, tr, tc);
        const int a = transpose_lds(tr, tc >> 3);
        if (tr < 0 || tr >= 64 || tc < 0 || tc > 56 || tc % 8 || a < 0 || a + 8 > 64 * 64 || a % 8)
          fail(std::string(name) + ": transpose LDS write outside the tile");
        for (int e = 0; e < 8; ++e) {
          if (lds[a + e] != -1) fail(std::string(name) + ": transpose LDS slot written twice");
          const int64_t r = r0 + tr, c = c0 + tc + e;
          lds[a + e] = r < rows && c < cols ? r * cols + c : -2;  // -2: zero filler
        }
      }
    for (int tid = 0; tid < 256; ++tid)
      for (int j = 0; j < 2; ++j) {
        int tc, tr;
        transpose_store_lane(tid, j, tc, tr);
        const int64_t c = c0 + tc, r = r0 + tr;
        if (!(c < cols && r < rows)) continue;
        const int base = transpose_lds(tr, tc >> 3) + (tc & 7);
        for (int e = 0; e < 8; ++e) {
          const int a = base + e * 64;
          if (a < 0 || a >= 64 * 64) fail(std::string(name) + ": transpose LDS read outside the tile");
          const int64_t src = lds[a], o = c * rows + r + e;
          if (o < 0 || o >= rows * cols) fail(std::string(name) + ": transpose store outside the output");
          if (src != (r + e) * cols + c) fail(std::string(name) + ": transpose output element from the wrong source");
          if (done[o]++) fail(std::string(name) + ": transpose output element written twice");
          ++g_checked;
        }
      }
  }
  for (uint8_t v : done)
    if (v != 1) fail(std::string(name) + ": transpose output element never written");
}

}  // namespace

int main() {
  long long d, F, swiglu, groups, rows_max, rr_R, rr_L;
  if (std::scanf("%lld %lld %lld %lld %lld %lld %lld", &d, &F, &swiglu, &groups, &rows_max, &rr_R, &rr_L) != 7)
    fail("input: d F swiglu groups rows_max rr_R rr_L offsets... [chunks, then chunks+1 rows of groups bounds]");
  std::vector<int64_t> off(groups + 1);
  for (auto& o : off)
    if (std::scanf("%lld", (long long*)&o) != 1) fail("input: offsets");
  if (off[0] != 0 || off[groups] > rows_max) fail("input: offsets");
  for (int g = 0; g < groups; ++g)
    if (off[g + 1] < off[g]) fail("input: offsets must ascend");
  // optional token chunks: bounds[r][g] = first row of chunk r in group g
  // (bounds[0] = the group starts, bounds[chunks] = the group ends); the
  // row-split launches then also run once per chunk on [bounds[r], bounds[r+1])
  long long chunks = 0;
  std::vector<std::vector<int64_t>> bounds;
  if (std::scanf("%lld", &chunks) == 1) {
    bounds.assign(chunks + 1, std::vector<int64_t>(groups));
    for (auto& row : bounds)
      for (auto& b : row)
        if (std::scanf("%lld", (long long*)&b) != 1) fail("input: chunk bounds");
    for (int g = 0; g < groups; ++g) {
      if (bounds[0][g] != off[g] || bounds[chunks][g] != off[g + 1]) fail("input: chunk bounds must span the groups");
      for (int r = 0; r < chunks; ++r)
        if (bounds[r + 1][g] < bounds[r][g]) fail("input: chunk bounds must ascend");
    }
  }
  const int64_t m = swiglu ? 2 : 1;
  if (d * 2 > kMaxRowBytes || m * F * 2 > kMaxRowBytes) fail("input: rows wider than the host limit");
  const int W = (int)groups;  // weight sets (one per group)
  const Tensor x{"x_rows", rows_max * d * 2}, h{"h", rows_max * F * 2}, dy{"dy_rows", rows_max * d * 2},
      dact{"d_act", rows_max * m * F * 2}, w_in{"w_in", W * d * F * 2}, w_up{"w_up", W * d * F * 2},
      w_out{"w_out", W * F * d * 2};
  const int64_t b_split = swiglu ? F : 0;
  for (long long r = -1; r < chunks; ++r) {  // r = -1: whole groups; else chunk r's sub-ranges
    std::vector<int64_t> o = off;
    const int64_t* ends = nullptr;
    if (r >= 0) {
      for (int g = 0; g < groups; ++g) o[g] = bounds[r][g];
      ends = bounds[r + 1].data();
    }
    // forward: [x] [W_in | W_up] with the activation, then h W_out
    check_rows({"fwd gate|up", false, swiglu != 0, x, w_in, swiglu ? w_up : w_in, d, F, d * F, F, d, 0}, o, ends,
               (int)groups, rows_max, (int)rr_R, (int)rr_L, W);
    check_rows({"fwd down", false, false, h, w_out, w_out, F, d, F * d, d, F, 0}, o, ends, (int)groups, rows_max,
               (int)rr_R, (int)rr_L, W);
    // backward: dH = dY W_out^T (activation backward in the epilogue), dx = d_act [W_in | W_up]^T
    check_rows({"dgrad W_out", true, false, dy, w_out, w_out, d, d, F * d, F, d, 0}, o, ends, (int)groups, rows_max,
               (int)rr_R, (int)rr_L, W);
    if (b_split % BK == 0)  // otherwise the register-staged kernels take this launch
      check_rows({"dgrad W_in", true, false, dact, w_in, swiglu ? w_up : w_in, m * F, F, d * F, d, m * F, b_split},
                 o, ends, (int)groups, rows_max, (int)rr_R, (int)rr_L, W);
  }
  // backward on transposed weights (bf16 calls with many rows per weight
  // set): both dgrads as forward-kind launches over W_out^T [W][d][F] and
  // [W_in^T | W_up^T] [W][m F][d], whole groups only
  {
    check_transpose("W_out [F][d]", F, d);
    check_transpose("W_in [d][F]", d, F);
    const Tensor wt_out{"W_out^T", W * d * F * 2}, wt_io{"[W_in | W_up]^T", W * m * F * d * 2};
    check_rows({"dgrad W_out^T", false, false, dy, wt_out, wt_out, d, F, d * F, F, d, 0}, off, nullptr, (int)groups,
               rows_max, (int)rr_R, (int)rr_L, W);
    check_rows({"dgrad [W_in | W_up]^T", false, false, dact, wt_io, wt_io, m * F, d, m * F * d, d, m * F, 0}, off,
               nullptr, (int)groups, rows_max, (int)rr_R, (int)rr_L, W);
  }
  // the fused forward's GEMM-1: rows gathered from T = rows_max tokens of x
  // through a synthetic assignment map (t*k + j, k = 2), every row a
  // different token choice
  {
    const int gk = 2;
    std::vector<int32_t> assign(rows_max);
    for (int64_t r = 0; r < rows_max; ++r) assign[r] = (int32_t)((r * 2654435761LL) % (rows_max * gk));
    const Tensor xt{"x (tokens)", rows_max * d * 2};
    RowsLaunch L{"fused gate|up", false, swiglu != 0, xt, w_in, swiglu ? w_up : w_in, d, F, d * F, F, d, 0};
    L.gather = assign.data();
    L.gather_k = gk;
    L.gather_rows = rows_max;
    if (rows_max * d * 2 <= kMaxExtent) check_rows(L, off, nullptr, (int)groups, rows_max, (int)rr_R, (int)rr_L, W);
  }
  // weight gradients: dW_out = h^T dY, [dW_in | dW_up] = x^T d_act
  check_wgrad({"wgrad W_out", h, dy, F, d, F, d, wgrad_ksplit(groups, F, d, rows_max)}, off, (int)groups);
  check_wgrad({"wgrad W_in", x, dact, d, m * F, d, m * F, wgrad_ksplit(groups, d, m * F, rows_max)}, off,
              (int)groups);
  std::printf("OK %lld\n", g_checked);
  return 0;
}
