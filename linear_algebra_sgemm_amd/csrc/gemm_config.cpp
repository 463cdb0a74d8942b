// Shape -> configuration: which tile configuration and how many K chunks a
// call uses.  Host code only.
//
// Two sources, in order:
//  1. an offline-tuned table (gemm_tuned.inc, written by tune.py beside the
//     package from timings of every legal configuration on MI355X), keyed by
//     the size class of M, N and K (log2 rounded to the nearest integer,
//     clamped to 7..14, i.e. 128 .. 16384); it only lists classes where a
//     configuration beat the built-in rule;
//  2. the built-in rule below.
// Either way the result then passes the legality filter: the split count is
// clamped to the K tiles there are and to the workspace.  This follows the
// parameter search of the SGEMM page (kernel k9, section "k7、k8、k9": many
// tile-parameter combinations timed on the target GPU, the best one kept) and
// the DeepGEMM page's offline tuning of block shapes and split-K with a table
// lookup at run time (section 5.3).
#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cstring>

#include "gemm_launch.h"

namespace lasg {

namespace {

struct TunedEntry {
  signed char op, lm, ln, lk, tile, splits;
};

const TunedEntry kTuned[] = {
#include "gemm_tuned.inc"
    {-1, 0, 0, 0, 0, 0},  // end marker
};

std::atomic<bool> g_use_tuned{true};

// log2(x) rounded to the nearest integer, clamped to [7, 14]: floor(log2 x),
// plus one where x exceeds 2^c sqrt(2) (x^2 > 2^(2c+1); never equal for integers).
int size_class(int x) {
  if (x <= 1) return 7;
  int c = 31 - __builtin_clz((unsigned)x);
  if ((uint64_t)x * (uint64_t)x > (uint64_t(1) << (2 * c + 1))) ++c;
  return c < 7 ? 7 : c > 14 ? 14 : c;
}

// The table as a direct index (op, class of M, N, K), the first entry of a
// class winning as in a scan of kTuned; built once.
struct TunedIndex {
  signed char tile[2][8][8][8];
  signed char splits[2][8][8][8];
};

const TunedIndex& tuned_index() {
  static const TunedIndex index = [] {
    TunedIndex t;
    std::memset(t.tile, -1, sizeof(t.tile));
    std::memset(t.splits, -1, sizeof(t.splits));
    for (const TunedEntry* e = kTuned; e->op >= 0; ++e) {
      if (e->op > 1 || e->lm < 7 || e->lm > 14 || e->ln < 7 || e->ln > 14 || e->lk < 7 ||
          e->lk > 14)
        continue;
      signed char& tile = t.tile[e->op][e->lm - 7][e->ln - 7][e->lk - 7];
      if (tile >= 0) continue;
      tile = e->tile;
      t.splits[e->op][e->lm - 7][e->ln - 7][e->lk - 7] = e->splits;
    }
    return t;
  }();
  return index;
}

long ceil_div(long a, long b) { return (a + b - 1) / b; }

// Share of the tiles' rows (or columns) that fall inside a dimension of size x.
double fill(long x, long tile) { return (double)x / (double)(ceil_div(x, tile) * tile); }

// K chunks of the one-per-CU direct-to-LDS tiles when their tiles do not
// cover the CUs: as many as keep every chunk in one round (at most 16), with
// chunks of at least 384 (shorter ones lose to the fixed cost of a workgroup,
// its prologue and epilogue, and to the extra traffic of the reduction).
long direct_splits(long tiles, int K, int cus) {
  if (tiles >= cus) return 1;
  long s = cus / tiles;
  if (s > 16) s = 16;
  while (s > 1 && K / s < 384) --s;
  return s;
}

// Share of the workgroup slots of the last round that the tiles use, in
// percent, for tiles that fill one CU each (`per_cu` 1) or two per CU (2; a
// last round of at most one workgroup per CU runs each at the full CU rate and
// counts as half a round).
long round_use(long tiles, int cus, int per_cu) {
  const long slots = (long)per_cu * cus;
  const long full = tiles / slots, rem = tiles % slots;
  const long halves = 2 * full + (rem == 0 ? 0 : (per_cu == 2 && rem <= cus) ? 1 : 2);
  return 200 * tiles / (halves * slots);
}

// Built-in tile rule, measured on MI355X (the size sweep over powers of two and
// a sweep of ragged shapes):
//  * Outputs of at most one 16x16 tile per CU with K at most 4096, two per CU
//    with K at most 2048, or four per CU with K at most 512: the 16x16 tile
//    whose eight waves split K (tile 13), ragged or not (four per CU, against
//    the 32x32 tile: 300 x 520 x 400: 6.5 vs 9.4 us; 1000 x 200 x 400: 7.6 vs
//    9.5; 130 x 1000 x 400: 6.2 vs 9.0; but 500 x 500 x 100: 5.5 vs 5.0); per call, against the choice before it: 250 x 250 x
//    400: 4.5 vs 20.1 us (64x64 register-staged); 200 x 120 x 2000: 8.3 vs 35.2
//    (32x32); 300 x 520 x 777: 15.6 vs 16.8; 60 x 2000 x 2000: 21.0 vs 34.3;
//    330 x 330 x 777: 12.5 vs 14.2; 128 x 128 x 4096: 11.0 vs 15.4 (64x64
//    direct in 8 chunks); 256 x 256 x 4096: 13.2 vs 16.2.  Past two tiles per CU
//    it loses where K is long (500 x 500 x 777: 20.2 vs 17.0 for 32x32; 700 x
//    700 x 400: 13.2 vs 12.8 for 64x64 direct), and at 4096 already past one
//    (256 x 512 x 4096: 24.0 vs 17.9), as at K = 8192 (128 x 128: 21.2 vs 14.1
//    for 32x32 in 16 chunks).
//  * The direct-to-LDS kernels wherever their copies are legal (rows of B
//    16-byte aligned and readable in whole 4-float chunks, rows of A 4-byte
//    aligned: `operands_ok`, which holds after packing too) and their 256x256
//    tiles cover the CUs:
//    eight waves of 256x256 (4096^3: 146 TFLOP/s, 8192^3: 149; ragged 4000^3:
//    138 vs 111 for the best register-staged tile), or 128x256 at two per CU
//    when that wastes less of the last round (6000^3: 116 vs 104; 7000 x 3000 x
//    2000: 109 vs 89) — weighed by their full-round rates, 89 vs 93 % of peak.
//    On a ragged shape K must reach 384 (5000 x 5000 x 333: 64 vs 74 for 64x64).
//  * Fewer 256x256 tiles than CUs: the 128x128 direct-to-LDS tile, unsplit
//    once its tiles give every CU one and use at least 80 % of the last round
//    of slots, two per CU (3000^3, 576 tiles, 75 %: 100 vs 120 for 64x64;
//    2048^3: 130 vs 114 for the split 256x256 tile;
//    4096 x 2048 x 2048: 139 vs 125 for register-staged 128x128; 2800^3: 128 vs
//    124; but 1536 x 3072 x 2048, 288 tiles in 512 slots: 80 vs 108 for 64x64),
//    else with K split so that one round uses at least 70 % of the CUs, in two
//    or more chunks of at least 384 (1024 x 1024 x 8192: 123 vs 117 for the
//    256x256 tile in 16 chunks; 1024 x 2048 x 4096: 121 vs 116), as long as
//    there are 32 tiles (512 x 512 x 8192 keeps 64x64 in 16 chunks: 82 vs 59);
//    but with K >= 4096 the 256x256 tile in chunks of at least 768 where that
//    fills a tenth of the CUs more (1280 x 1280 x 8192 in 10 chunks: 124 vs
//    103 for 128x128 in 2; 1024 x 1024 x 8192 keeps 128x128 in 4, the 256x256
//    tile's 16 chunks being 512 long).
//    Not where 128-wide tiles leave a much larger part of the last tile row or
//    column empty than 64-wide ones (777 x 7777 x 777: 76 vs 86 for 64x64).
//    Where neither applies and K >= 4096, the eight-wave 256x256 tile with K
//    split the same way when a round then uses 70 % of the CUs (1536 x 1536 x
//    6144 in 7 chunks: 126 vs 102 for 64x64).
//  * Else the register-staged 128x256 tile at two per CU, then 128x128, where
//    their tiles give every CU two (4096^3: 134 vs 130 for 256x256) — on shapes
//    the direct-to-LDS kernel takes, only where they are whole (their
//    bounds-checked form is slow: 3000^3 at 128x128: 77).
//  * Else 64x64 tiles, which spread small outputs over more CUs: direct-to-LDS
//    where the copies are legal (1024 x 3072 x 768: 118 vs 103 for the
//    register-staged 64x64 tile and 94 for 128x128 direct at 192 tiles;
//    1000 x 3000 x 777: 83 vs 69; 1500^3: 89 vs 73 for the best register-staged
//    tile; 256^3: 4.8 vs 3.8), else register-staged.  But where there are at
//    most a quarter as many 64x64 tiles as CUs and K is at most 1024, the
//    32x32 tile of 16x16x4 blocks: its shorter per-wave MFMA chain sets the
//    time there (per call, 512^3: 10.1 us vs 13.9; ragged too, bounds-checked:
//    300 x 520 x 100: 9.5 vs 12.6, 500 x 500 x 777: 17.0 vs 20.6; but 1024 x
//    1024 x 256, 256 tiles of 64x64: 11.8 vs 10.5; and its time grows with K
//    faster than the 64x64 tile's: 500 x 500 x 2000: 34.7 vs 20.0).
int sgemm_rule_tile(int M, int N, int K, int cus, bool operands_ok) {
  // Small outputs first: see the rule's description above.
  const long t16 = ceil_div(M, 16) * ceil_div(N, 16);
  if ((t16 <= cus && K <= 4096) || (t16 <= 2L * cus && K <= 2048) || (t16 <= 4L * cus && K <= 512))
    return 13;
  const long t_large = ceil_div(M, 256) * ceil_div(N, 256);
  const long t_tall = ceil_div(M, 128) * ceil_div(N, 256);
  const long t_med = ceil_div(M, 128) * ceil_div(N, 128);
  const bool direct = operands_ok;
  const bool whole = M % 256 == 0 && N % 256 == 0 && K % 32 == 0;
  if (direct && (whole || K >= 384)) {
    if (t_large >= cus)
      return 89 * round_use(t_tall, cus, 2) > 93 * round_use(t_large, cus, 1) ? 8 : 9;
    if (t_med >= cus) {
      // (not where the 128-row or -column tiles leave much more of the last
      // tile row or column empty than 64-wide ones would)
      const double fill128 = fill(M, 128) * fill(N, 128), fill64 = fill(M, 64) * fill(N, 64);
      if (round_use(t_med, cus, 2) >= 80 && fill128 >= 0.95 * fill64) return 10;
    } else {
      const long s = direct_splits(t_med, K, cus);
      // The 256x256 tile in K chunks instead, where its chunks stay long and it
      // fills clearly more of the CUs.
      const long s9 = direct_splits(t_large, K, cus);
      if (K >= 4096 && s9 >= 2 && K / s9 >= 768 && 10 * t_large * s9 >= 10 * t_med * s + cus &&
          10 * t_large * s9 >= 7L * cus)
        return 9;
      if (t_med >= 32 && s >= 2 && 10 * t_med * s >= 7L * cus) return 10;
    }
    if (K >= 4096) {
      const long s = direct_splits(t_large, K, cus);
      if (s >= 2 && 10 * t_large * s >= 7L * cus) return 9;
    }
  }
  // (on shapes the direct-to-LDS kernel can take, only where these tiles are whole)
  if (t_tall >= 2L * cus && (!direct || (M % 128 == 0 && N % 256 == 0 && K % 16 == 0))) return 4;
  if (t_med >= 2L * cus && (!direct || (M % 128 == 0 && N % 128 == 0 && K % 16 == 0))) return 1;
  const long t_small = ceil_div(M, 64) * ceil_div(N, 64);
  if (direct && 4 * t_small <= cus && K <= 1024) return 12;
  return direct ? 11 : 2;
}

// Built-in split rule: the direct-to-LDS tiles as in direct_splits (the
// 128x128 one counted at one workgroup per CU, as measured best); for the
// register-staged tiles (from the size sweep), when the output has fewer tiles
// than there are CUs and K is at least 512, split K until there are about four
// workgroups per CU (small tiles share a CU), keeping chunks of at least 128.
int sgemm_rule_splits(int M, int N, int K, int tile, int cus) {
  const long tiles = ceil_div(M, sgemm_tile_bm(tile)) * ceil_div(N, sgemm_tile_bn(tile));
  if (tile == 7 || tile == 9 || tile == 10) return (int)direct_splits(tiles, K, cus);
  if (tile == 12) return 1;   // measured unsplit only
  if (tile == 13) return 1;   // splits K inside the workgroup instead
  if (tile == 11) {
    // Up to four workgroups share a CU: split only outputs of at most half as
    // many tiles as CUs, to about two workgroups per CU, in chunks of at least
    // 512 (600 x 600 x 5000, 100 tiles: 39 unsplit, 66 in 2, 72 in 4; 700 x 900
    // x 777, 165 tiles: 35 unsplit, 33 in 2).
    if (2 * tiles > cus) return 1;
    long s = 2L * cus / tiles;
    if (s > K / 512) s = K / 512;
    if (s > 16) s = 16;
    return s < 1 ? 1 : (int)s;
  }
  if (tile == 8) return (int)direct_splits((tiles + 1) / 2, K, cus);
  if (tiles >= cus || K < 512) return 1;
  const long by_cus = ceil_div(4L * cus, tiles);
  const long by_k = ceil_div(K, sgemm_tile_bk(tile)) * sgemm_tile_bk(tile) / 128;
  long s = by_cus < by_k ? by_cus : by_k;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

}  // namespace

void set_use_tuned(bool on) { g_use_tuned.store(on); }
bool use_tuned() { return g_use_tuned.load(); }

namespace {
std::atomic<int> g_force_group{0};      // 0: each launch's own group size
std::atomic<bool> g_xcd_remap{true};
}  // namespace

void set_swizzle(int group_m, bool xcd_remap) {
  g_force_group.store(group_m);
  g_xcd_remap.store(xcd_remap);
}

int swizzle_group(int launch_group_m) {
  const int forced = g_force_group.load();
  const int g = forced > 0 ? forced : launch_group_m;
  return g_xcd_remap.load() ? g : -g;
}

bool tuned_config(int op, int M, int N, int K, int* tile, int* splits) {
  if (!g_use_tuned.load()) return false;
  if (op < 0 || op > 1) return false;
  const int lm = size_class(M) - 7, ln = size_class(N) - 7, lk = size_class(K) - 7;
  const TunedIndex& index = tuned_index();
  if (index.tile[op][lm][ln][lk] < 0) return false;
  *tile = index.tile[op][lm][ln][lk];
  *splits = index.splits[op][lm][ln][lk];
  return true;
}

SgemmPlan plan_sgemm(int M, int N, int K, int cus, int force_tile, int force_splits,
                     size_t ws_floats, bool operands_ok) {
  int tuned_tile = -1, tuned_splits = -1;
  bool tuned = tuned_config(0, M, N, K, &tuned_tile, &tuned_splits) && tuned_tile >= 0 &&
               tuned_tile < kSgemmTileCount && tuned_splits >= 1;
  // Table entries were measured on whole tiles with packed aligned operands;
  // where the entry's tile would run bounds-checked here, the rule chooses
  // instead (it knows the ragged shapes).
  if (tuned && !(operands_ok && M % sgemm_tile_bm(tuned_tile) == 0 &&
                 N % sgemm_tile_bn(tuned_tile) == 0 && K % sgemm_tile_bk(tuned_tile) == 0))
    tuned = false;
  SgemmPlan p;
  p.tile = force_tile >= 0 ? force_tile
           : tuned        ? tuned_tile
                          : sgemm_rule_tile(M, N, K, cus, operands_ok);
  long s = force_splits > 0 ? force_splits
           : (tuned && force_tile < 0) ? tuned_splits
                                       : sgemm_rule_splits(M, N, K, p.tile, cus);
  // Small outputs that would split K across workgroups (a second launch adds the
  // partials): the 16x16 tile, whose waves split K inside the workgroup,
  // where its tiles fit one round (at most one per CU) and K is at most 2048.
  // Kernel time, split choice + reduction -> tile 13: 192 x 192 x 768: 4.7 + 4.5 ->
  // 5.1 us; 256 x 256 x 1024: 5.1 + 4.6 -> 6.5; 256 x 256 x 2048: 6.0 + 4.6 -> 10.1
  // (but 512 x 256 x 1536, two tiles per CU: 7.3 + 4.6 -> 12.6).
  if (force_tile < 0 && force_splits < 0 && s > 1 && K <= 2048 &&
      ceil_div(M, 16) * ceil_div(N, 16) <= cus) {
    p.tile = 13;
    s = 1;
  }
  // Legality: whole K tiles per chunk, no empty chunk, partials fit the workspace.
  const long bk = sgemm_tile_bk(p.tile);
  const long ktiles = ceil_div(K, bk);
  const long mn = (long)M * N;
  if (p.tile == 13) s = 1;   // its waves split K; it never splits across workgroups
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > ktiles) s = ktiles;
  if (mn > 0 && s > (long)(ws_floats / (size_t)mn)) s = (long)(ws_floats / (size_t)mn);
  long chunk = K;
  if (s > 1) {
    chunk = ceil_div(ktiles, s) * bk;
    s = ceil_div(K, chunk);  // no chunk is empty
  }
  if (s <= 1) {
    s = 1;
    chunk = K;
  }
  p.splits = (int)s;
  p.k_chunk = (int)chunk;
  // What runs (the launch resolves again with the actual operands, to the same
  // answer when `operands_ok` describes them).
  p.tile = sgemm_resolve_tile(p.tile, M, N, K, p.splits, operands_ok);
  return p;
}

namespace {

int half_rule_tile(int M, int N, int K, int cus, bool operands_ok) {
  // Built-in rule (from the size sweep).  Small outputs first, whatever the
  // operands: the 16x16 tile whose eight waves split K (tile 9) for at most one
  // such tile per CU with K <= 4096, or four per CU with K <= 2048; per call
  // (FP16, bias + GELU), against the earlier choice: 250 x 250 x 400: 4.4 us vs
  // 37.4 (64x64 register-staged, bounds-checked); 500 x 500 x 400: 9.0 vs 37.0;
  // 128 x 128 x 2048: 5.1 vs 9.5 (64x64 in 8 chunks); 256 x 256 x 4096: 9.1 vs
  // 11.9 (128x128 direct in 8); 1000 x 200 x 777: 16.0 vs 27.3; but 60 x 2000 x
  // 2000: 18.6 vs 13.2 for 128x128 direct, and 700 x 700 x 400 (1936 tiles):
  // 18.8 vs 15.7.  Where the direct-to-LDS copies are
  // legal (`operands_ok`: rows of A and B 16-byte aligned, B readable in whole
  // 8-half chunks, as given or after packing):
  //  * 256x256 tiles with eight waves once they give every CU one, or once the
  //    128x128 tiles would need more than one round at two per CU (K >= 128),
  //    with the head/tail column split (tile 7, which runs as tile 6 where no
  //    split exists) for K >= 2048.  The eight-wave tile leads the four-wave one
  //    at every K measured (4096^2 x 1024: 902 vs 758; x 512: 670 vs 530; 3072^3:
  //    906 vs 758) and the register-staged tiles by far (3072^3: 906 vs 450 for
  //    128x128; 4096^2 x 256: 443 vs 358; 3000^3: 652 vs 92).
  //  * Between a quarter of the CUs and two per CU in 128x128 tiles (one round
  //    at two per CU), the 128x128 direct-to-LDS tile (2048^3: 640 vs 404 for
  //    64x64; 1024 x 4096 x 4096: 776 vs 528 for 128x128 register-staged;
  //    2048 x 2048 x 8192: 823 vs 641; 1000^3: 129 vs 68 for 128x256 direct;
  //    1024^3: 185 vs 155); with K split (below) it also takes smaller outputs
  //    once K reaches 4096 (512 x 512 x 8192 in 8 chunks: 225 vs 188 for 64x64
  //    in 16; 512 x 512 x 4096 in 4: 151 vs 137; 300 x 500 x 4096, 12 tiles:
  //    26 us vs 62 for 64x64 in 22 chunks; 128 x 128 x 8192: 13.6 vs 16.7), and
  //    from 16 tiles already once K reaches 1024 (64 x 4096 x 2049: 17.6 us vs
  //    43.7 for the eight-wave 256x256 tile below; 100 x 4096 x 3000: 20.2 vs
  //    55.5; 200 x 3000 x 2500: 27.8 vs 61.0; 96 x 6000 x 3000: 23.1 vs 56.8).
  //  * Smaller outputs: the register-staged 64x64 tile, which spreads them over
  //    the most CUs with split-K -- unless it would run bounds-checked (ragged
  //    M, N or K) and there are 16 tiles of 128x256: then 128x256 direct-to-LDS
  //    (or the eight-wave 256x256 tile for K >= 2048; 504 x 504 x 8000 stays on
  //    the split 64x64 tile: 33 vs 27).
  // Otherwise (operands the copies cannot take) the register-staged 256x256
  // tile where 256x256 tiles give every CU one and K >= 512, else 128x128 tiles
  // once they give every CU two, else 64x64.
  const long t16 = ceil_div(M, 16) * ceil_div(N, 16);
  if ((t16 <= cus && K <= 4096) || (t16 <= 4L * cus && K <= 2048)) return 9;
  const long t_large = ceil_div(M, 256) * ceil_div(N, 256);
  const long t_med = ceil_div(M, 128) * ceil_div(N, 128);
  const bool direct = operands_ok;
  if (direct && K >= 128 && (t_large >= cus || t_med > 2L * cus)) return K >= 2048 ? 7 : 6;
  if (direct && t_med <= 2L * cus && (4 * t_med >= cus || K >= 4096 || (t_med >= 16 && K >= 1024)))
    return 8;
  if (!direct && t_large >= cus && K >= 512) return 0;
  const int reg = t_med >= 2L * cus ? 1 : 2;
  const int bm = half_tile_bm(reg);
  const bool reg_whole = M % bm == 0 && N % bm == 0 && K % kHalfBK == 0;
  const long t_tall = ceil_div(M, 128) * ceil_div(N, 256);
  if (direct && !reg_whole && t_tall >= 16) return K >= 2048 ? 6 : 4;
  return reg;
}

// Built-in split rule of the half products, as for FP32: split K (the
// register-staged tiles and the 128x128 direct-to-LDS tile) when the tiles do
// not cover the CUs and K is at least 512, aiming at four workgroups per CU
// with chunks of at least 128 on the register-staged tiles.
int half_rule_splits(int M, int N, int K, int tile, int cus) {
  if (tile == 8) {
    // The 128x128 direct-to-LDS tile: split outputs of at most half as many
    // tiles as CUs to about one workgroup per CU, in chunks of at least 1024
    // (1024 x 1024 x 4096, 64 tiles: 209 TFLOP/s unsplit, 301 in 2, 358 in 4,
    // 293 in 8; 2048 x 1024 x 8192, 128 tiles: 453, 620 in 2, 604 in 4; per
    // call, against chunks of 512: 128 x 8192 x 1024 unsplit 10.5 us vs 14.6 in
    // 2, 128 x 4096 x 4096 in 4 18.6 vs 20.0 in 8, 128 x 2048 x 8192 in 8 19.2
    // vs 20.6 in 16).
    const long tiles = ceil_div(M, 128) * ceil_div(N, 128);
    if (2 * tiles > cus) return 1;
    long s = cus / tiles;
    if (s > K / 1024) s = K / 1024;
    if (s > 16) s = 16;
    return s < 1 ? 1 : (int)s;
  }
  if (tile > 2) return 1;
  const long tiles = ceil_div(M, half_tile_bm(tile)) * ceil_div(N, half_tile_bm(tile));
  if (tiles >= cus || K < 512) return 1;
  const long by_cus = ceil_div(4L * cus, tiles);
  const long by_k = ceil_div(K, kHalfBK) * kHalfBK / 128;
  long s = by_cus < by_k ? by_cus : by_k;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

}  // namespace

HalfPlan plan_half(int M, int N, int K, int cus, int force_tile, int force_splits,
                   size_t ws_floats, bool operands_ok) {
  int tuned_tile = -1, tuned_splits = -1;
  bool tuned = tuned_config(1, M, N, K, &tuned_tile, &tuned_splits) && tuned_tile >= 0 &&
               tuned_tile < kHgemmTileCount && tuned_splits >= 1;
  // Table entries were measured on whole tiles with aligned operands; where the
  // entry's tile would run bounds-checked here, the rule chooses instead.
  if (tuned) {
    const int bm = half_tile_rows(tuned_tile);
    const int bn = half_tile_cols(tuned_tile);
    if (!(operands_ok && M % bm == 0 && N % bn == 0 && K % kHalfBK == 0))
      tuned = false;
  }
  HalfPlan p;
  p.tile = force_tile >= 0 ? force_tile
           : tuned         ? tuned_tile
                           : half_rule_tile(M, N, K, cus, operands_ok);
  p.tile = hgemm_resolve_tile(p.tile, M, N, K, operands_ok, cus);
  long s = force_splits > 0 ? force_splits
           : (tuned && force_tile < 0) ? tuned_splits
                                       : half_rule_splits(M, N, K, p.tile, cus);
  // Legality: register-staged tiles and the 128x128 direct-to-LDS tile only,
  // whole K steps per chunk, no empty chunk, partials fit the workspace.
  const long ktiles = ceil_div(K, kHalfBK);
  const long mn = (long)M * N;
  if (p.tile > 2 && p.tile != 8) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > ktiles) s = ktiles;
  if (mn > 0 && s > (long)(ws_floats / (size_t)mn)) s = (long)(ws_floats / (size_t)mn);
  long chunk = K;
  if (s > 1) {
    chunk = ceil_div(ktiles, s) * kHalfBK;
    s = ceil_div(K, chunk);
  }
  if (s <= 1) {
    s = 1;
    chunk = K;
  }
  p.splits = (int)s;
  p.k_chunk = (int)chunk;
  return p;
}

}  // namespace lasg
