// Address arithmetic of the bf16 grouped-GEMM kernels (gemm3.hip): which tile
// a workgroup computes, which bytes each lane's direct-to-LDS load reads and
// where it lands, and the span of every buffer resource.  Pure integer code,
// callable from the kernels and from the host, so that a host program can
// enumerate every load of a launch and check it against the tensors' bounds
// before the launch reaches a GPU (tests/gemm_addr_check.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace gemm_addr {

#define MOE_HD __host__ __device__ __forceinline__

constexpr uint32_t kOOB = 0x7FFFFFF0u;      // an offset beyond every extent
constexpr int64_t kMaxExtent = 0x7FFF0000;  // extents stay below kOOB
// Every resource spans at most 256 rows of one operand (or one K stage of an
// M/N-contiguous one), so rows of at most kMaxRowBytes keep every extent
// below kMaxExtent; the host rejects wider rows.
constexpr int64_t kMaxRowBytes = kMaxExtent / 256;

MOE_HD int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// ---------------------------------------------------------------------------
// Tile order
// ---------------------------------------------------------------------------
// Workgroup id -> linear tile id such that each XCD's workgroups (dispatched
// round-robin over the 8 XCDs) get consecutive tile ids (bijection on [0, num)).
MOE_HD int xcd_remap(int hw, int num) {
  const int q = num >> 3, r = num & 7;
  const int xcd = hw & 7, local = hw >> 3;
  const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  return base + local;
}

// Workgroup id -> linear item id, spreading runs of C consecutive items over
// the XCDs: item run j (items jC .. jC + C - 1) goes whole to XCD j % 8, and
// each XCD takes its runs in order, so the items of a run keep sharing that
// XCD's L2 while consecutive runs (the parts of one group) go to different
// XCDs.  Items past the last whole round of 8 runs fall back to xcd_remap.
// A bijection on [0, n).
MOE_HD int run_remap(int hw, int n, int C) {
  const int span = 8 * C;
  const int n0 = n / span * span;
  if (hw >= n0) return n0 + xcd_remap(hw - n0, n - n0);
  const int x = hw & 7, l = hw >> 3;
  const int rho = l / C, off = l - rho * C;
  return (rho * 8 + x) * C + off;
}

// Linear tile id -> (row tile, column tile), walking gm row tiles per column
// so that concurrently running tiles share panels in L2.
MOE_HD void grouped_order(int lin, int tiles_m, int tiles_n, int& mt, int& nt, int gm) {
  const int span = gm * tiles_n;
  const int gid = lin / span;
  const int first = gid * gm;
  const int gsz = (tiles_m - first) < gm ? (tiles_m - first) : gm;
  const int rem = lin - gid * span;
  mt = first + rem % gsz;
  nt = rem / gsz;
}

// Row-split launches (FWD, DGRAD) size the grid for the largest possible row
// count, since the per-group row counts live on the device.  Each workgroup
// counts the BM-row tiles the groups really hold; surplus workgroups exit,
// and the XCD remap and the grouped order run over the real tiles only.
// Group g owns rows [offsets[g], offsets[g + 1]), or [offsets[g], ends[g])
// when ends is given (disjoint sub-ranges, e.g. one token chunk of every
// expert's segment).  Returns false for a surplus workgroup; else group g,
// its rows [row_begin, row_end) from the tile's first row, and the column
// tile nt.
MOE_HD int64_t group_end(const int64_t* offsets, const int64_t* ends, int g) {
  return ends ? ends[g] : offsets[g + 1];
}
// Tiles are walked group by group (a group's tiles are consecutive linear
// ids, so an XCD works on few groups' weight panels at a time), and within a
// group in row bands of at most gm row tiles, balanced (a group of 17 row
// tiles with gm 8 walks bands of 6, 6 and 5), each band column by column.
template <int BM>
MOE_HD bool row_tile_of(const int64_t* offsets, const int64_t* ends, int groups, int tiles_n, int gm, int hw, int& g,
                        int64_t& row_begin, int64_t& row_end, int& nt) {
  int real_m = 0;
  for (int gg = 0; gg < groups; ++gg) real_m += (int)((group_end(offsets, ends, gg) - offsets[gg] + BM - 1) / BM);
  const int real = real_m * tiles_n;
  if (hw >= real) return false;
  const int lin = xcd_remap(hw, real);
  int acc_t = 0;
  for (int gg = 0; gg < groups; ++gg) {
    const int64_t o0 = offsets[gg], o1 = group_end(offsets, ends, gg);
    const int nt_g = (int)((o1 - o0 + BM - 1) / BM);
    const int cnt = nt_g * tiles_n;
    if (lin < acc_t + cnt) {
      const int bands = (nt_g + gm - 1) / gm;
      const int band_m = (nt_g + bands - 1) / bands;
      int mt;
      grouped_order(lin - acc_t, nt_g, tiles_n, mt, nt, band_m);
      g = gg;
      row_begin = o0 + (int64_t)mt * BM;
      row_end = o1;
      return true;
    }
    acc_t += cnt;
  }
  return false;
}

// Launch sizes.  Row-split launches: tiles_n column tiles of `cols` columns
// (BN, or BN / 2 hidden units for the SwiGLU gate|up pair) and tiles_m row
// tiles enough for rows_max rows spread over `groups` groups (each group's
// last tile may be partial); grid = tiles_m * tiles_n.
MOE_HD void rows_tiles(int64_t N, int cols, int64_t rows_max, int groups, int BM, int& tiles_m, int& tiles_n) {
  tiles_n = (int)((N + cols - 1) / cols);
  tiles_m = (int)((rows_max + BM - 1) / BM) + groups;
}
// Weight-gradient launches: every (split, group, tile) item, grid =
// ksplit * groups * tiles_m * tiles_n.
MOE_HD void wgrad_tiles(int64_t M, int64_t N, int BM, int BN, int& tiles_m, int& tiles_n) {
  tiles_m = (int)((M + BM - 1) / BM);
  tiles_n = (int)((N + BN - 1) / BN);
}
// Reduction splits of a bf16 weight-gradient launch over `groups` groups of at
// most rows_max rows in all (a function of host-known sizes only, so that the
// workspace can be sized for it): a launch with fewer than 512 256 x 256 tiles
// (two per CU) splits each group's rows into s chunks, s = min(512 / tiles,
// rows per group / 1024, 8).
MOE_HD int wgrad_ksplit(int64_t groups, int64_t M, int64_t N, int64_t rows_max) {
  const int64_t tiles = groups * ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles <= 0 || tiles >= 512) return 1;
  int64_t s = 512 / tiles;
  const int64_t by_rows = rows_max / (groups > 0 ? groups : 1) / 1024;  // >= 1024 rows per split
  if (s > by_rows) s = by_rows;
  if (s > 8) s = 8;
  return s < 1 ? 1 : (int)s;
}
// Rows [r0, r1) of split `split` of a group's rows [g0, g1): chunks of a
// multiple of BK rows; a split past the group's rows keeps an empty range.
MOE_HD void split_rows(int64_t g0, int64_t g1, int ksplit, int split, int BK, int64_t& r0, int64_t& r1) {
  const int64_t chunk = ((g1 - g0 + ksplit - 1) / ksplit + BK - 1) / BK * BK;
  const int64_t b = g0 + split * chunk;
  r0 = b < g1 ? b : g1;
  r1 = b + chunk < g1 ? b + chunk : g1;
}

MOE_HD int weight_index(int g, int rr_R, int rr_L) {
  // send slot g = q * L + l holds expert q + R * l under round-robin placement
  return rr_R > 0 ? (g % rr_L) * rr_R + g / rr_L : g;
}

// ---------------------------------------------------------------------------
// Operand stages in LDS and the lanes' direct-to-LDS loads
//   K-contiguous (KC): [R rows][BK], row pitch BK*2 bytes, 16-byte chunk c of
//     row r stored at chunk c ^ kc_swz(r).
//   MN-contiguous: panels of 128 columns, each [BK][128], pitch 256 bytes,
//     chunk c of K-row k stored at chunk c ^ (4 * (k & 3)).
// A stage of R x BK bf16 is split into 1 KiB units; unit u is issued by wave
// u % NW as its (u / NW)-th load, lane l writing LDS bytes
// [1024 u + 16 l, 1024 u + 16 l + 16) of the stage.
// ---------------------------------------------------------------------------
template <int BK>
MOE_HD int kc_swz(int row) {
  if constexpr (BK == 32) return (row >> 2) & 3;
  else return (row ^ (row >> 3)) & 7;
}
MOE_HD int mn_swz(int k) { return 4 * (k & 3); }

template <int R, int BK, int NW>
struct Units {
  static constexpr int BYTES = R * BK * 2;
  static constexpr int UNITS = BYTES / 1024;
  static_assert(UNITS % NW == 0, "units must split evenly over the waves");
  static constexpr int PER = UNITS / NW;
};

// KC: load i of wave `wave`, lane `lane` reads element column `col` (a
// multiple of 8, within the stage) of tile row `row`.
template <int BK, int NW>
MOE_HD void kc_lane(int i, int wave, int lane, int& row, int& col) {
  constexpr int CPR = BK * 2 / 16;  // chunks per row
  constexpr int RPU = 64 / CPR;     // rows per unit
  const int u = i * NW + wave;
  row = u * RPU + lane / CPR;
  col = ((lane % CPR) ^ kc_swz<BK>(row)) * 8;
}

// MN: load i of wave `wave`, lane `lane` reads K row `k` (within the stage)
// at column `col` relative to the base of its panel's resource (pair: the
// tile's two 128-column panels come from two tensors, both at column 0);
// `panel` selects that resource.
template <int BK, int NW>
MOE_HD void mn_lane(int i, int wave, int lane, bool pair, int& panel, int& k, int& col) {
  constexpr int KB = BK / 4;  // units per panel (4 K rows each)
  const int u = i * NW + wave;
  panel = u / KB;
  k = (u % KB) * 4 + lane / 16;
  const int c = (lane % 16) ^ mn_swz(k);
  col = (pair ? 0 : panel * 128) + c * 8;
}

// ---------------------------------------------------------------------------
// Buffer resource spans: [base, base + bytes) in bytes from the operand's
// pointer.  Loads at or past `bytes` read zeros.
// ---------------------------------------------------------------------------
struct Span {
  int64_t base, bytes;
};

// Row-split A: the tile's rows [row_begin, row_begin + rows_valid), rows_valid <= BM.
MOE_HD Span rows_a_span(int64_t row_begin, int64_t rows_valid, int64_t lda) {
  return Span{row_begin * lda * 2, rows_valid * lda * 2};
}

// DGRAD B (K-contiguous weights of one set, N rows of ldb): the tile's rows
// [n0, n0 + min(BN, N - n0)), gstride_bytes apart per weight set.
MOE_HD Span dgrad_b_span(int64_t set_base, int64_t n0, int64_t nrows_max, int64_t N, int64_t ldb) {
  return Span{set_base + n0 * ldb * 2, min64(nrows_max, N - n0) * ldb * 2};
}

// Row-split A gathered from the token rows (the fused forward): tile row r
// of the group is token row gather[row_begin + r] / gather_k of x, whose
// resource spans all x_rows rows; a lane whose tile row is past the group's
// rows is masked by a K offset no stage reaches (kc_gather_col).
MOE_HD Span gather_a_span(int64_t x_rows, int64_t lda) { return Span{0, x_rows * lda * 2}; }
constexpr int kMaskedCol = 1 << 30;
MOE_HD int kc_gather_col(int row, int col, int64_t rows_valid) { return row < rows_valid ? col : kMaskedCol; }
MOE_HD int64_t gather_token(int32_t assign, int gather_k) { return (int64_t)assign / gather_k; }

// A stage of an M/N-contiguous operand whose K row k starts at first +
// k * ld_bytes (first points at the tile's first column, col0_bytes into its
// row): stage kt covers K rows [kt BK, kt BK + BK).  Every stage has the same
// extent, BK rows minus the columns before the tile; the loaders mask rows at
// or past the operand's last K row themselves (offset kOOB), so the kernels
// only advance the base by BK * ld_bytes per stage and offsets stay within
// one stage however many rows the operand holds.
struct StageWalk {
  int64_t first, stride, bytes;
};
MOE_HD StageWalk stage_walk(int64_t first, int BK, int64_t ld_bytes, int64_t col0_bytes) {
  return StageWalk{first, BK * ld_bytes, BK * ld_bytes - col0_bytes};
}
MOE_HD Span stage_span(const StageWalk& w, int kt) { return Span{w.first + kt * w.stride, w.bytes}; }

// FWD B (N-contiguous weights of one set, rows of ldb): stages from the
// tile's column n0.
MOE_HD StageWalk fwd_b_walk(int64_t n0, int BK, int64_t ldb) { return stage_walk(n0 * 2, BK, ldb * 2, n0 * 2); }

// WGRAD operand (the group's rows from r0, ld columns): stages from the
// tile's column c0.
MOE_HD StageWalk wgrad_walk(int64_t r0, int64_t c0, int BK, int64_t ld) {
  return stage_walk((r0 * ld + c0) * 2, BK, ld * 2, c0 * 2);
}

// Weight transpose (64 x 64 tiles, 256 threads): workgroup L's tile, with
// consecutive workgroups walking 8 row tiles per column tile.
MOE_HD void transpose_tile(int L, int64_t rows, int64_t cols, int64_t& r0, int64_t& c0) {
  const int gx = (int)((cols + 63) >> 6), gy = (int)((rows + 63) >> 6);
  const int grp = L / (8 * gx), rem = L - grp * 8 * gx;
  const int gsz = gy - grp * 8 < 8 ? gy - grp * 8 : 8;
  r0 = (int64_t)(grp * 8 + rem % gsz) * 64;
  c0 = (int64_t)(rem / gsz) * 64;
}
// LDS element of tile row tr's 16-byte chunk ch (rows unpadded, the chunks of
// row tr in the order ch ^ (tr / 8 % 8)).
MOE_HD int transpose_lds(int tr, int ch) { return tr * 64 + ((ch ^ ((tr >> 3) & 7)) << 3); }
// Thread tid's j-th source chunk (tile row, first column) and j-th output
// chunk (tile column, first of 8 tile rows), j = 0, 1.
MOE_HD void transpose_load_lane(int tid, int j, int& tr, int& tc) {
  const int q = tid + 256 * j;
  tr = q >> 3;
  tc = (q & 7) * 8;
}
MOE_HD void transpose_store_lane(int tid, int j, int& tc, int& tr) {
  const int q = tid + 256 * j;
  tc = q >> 3;
  tr = (q & 7) * 8;
}

}  // namespace gemm_addr
}  // namespace moe
