// kda_launch.h -- launch-shape decisions shared by the host entry points and
// the gfx950 kernels of the KDA decode library.  Internal header.
#pragma once

#include <stdint.h>

#include "kda_decode.h"

// The one helper the kernels also call is marked for both sides when the
// file is compiled as HIP; the host-only translation unit sees plain C++.
#if defined(__HIP__)
#define KDA_HD __host__ __device__
#else
#define KDA_HD
#endif

namespace kda {

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kNumXcd = 8;     // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kHeadK = KDA_HEAD_K;
constexpr int kHeadV = KDA_HEAD_V;

// Columns one lane holds: a 16-byte vector of the pool's element type.
inline int32_t cols_per_lane(kda_dtype dt) { return dt == KDA_F32 ? 4 : 8; }

// Default launch shape, chosen by measurement on MI355X (graph-replayed
// launches, 1 GiB of rotating pools, nontemporal state traffic):
//  - one row per request, fp32: whole 128-column tile rows, so every wave
//    instruction reads or writes whole 512-byte state rows, K split over 2
//    waves.  At 64 requests x 12 heads: 18.0 us, against 19.8 us over 4 or
//    8 waves and 20.6-22.1 us for 32/64-column tiles.
//  - one row per request, fp16: 64-column tiles (a whole 128-byte line per
//    tile row) held by one wave, so a row's column sums never leave the
//    wave: no LDS exchange and no barrier.  9.6-9.7 us, against 9.9 us for
//    128 columns over 2 waves and 10.0-10.1 us over 4.
//  - one row per request, small launches (units = requests x heads), where
//    latency rather than bandwidth decides: narrower tiles or more waves
//    put more workgroups and waves in flight.  fp32: up to 48 units 32
//    columns over 1 wave (1 request: 3.7 us against 5.3 us; 4 requests: 4.0
//    against 5.4), up to 128 units 64 columns over 8 waves (8 requests: 4.6
//    against 5.8; 16 requests measured even, 32 best at the wide default).
//    fp16: up to 96 units 64 columns over 4 waves (1 request: 4.1 against
//    4.6 us; 8 requests: 4.5 against 4.9; 32 best at one wave).
//  - chained rows: 64-column tiles with K over 8 (fp32) or 4 (fp16) waves:
//    few tiles exist, so K is spread over more waves and each row's partial
//    column sums meet in LDS.
inline int32_t default_bv(kda_dtype dt, int32_t n_rows, int64_t units = 1 << 30) {
  if (n_rows == 1 && dt == KDA_F32) return units <= 48 ? 32 : units <= 128 ? 64 : 128;
  return 64;
}
inline int32_t default_waves_per_tile(kda_dtype dt, int32_t n_rows, int64_t units = 1 << 30) {
  if (n_rows == 1) {
    if (dt == KDA_F32) return units <= 48 ? 1 : units <= 128 ? 8 : 2;
    return units <= 96 ? 4 : 1;
  }
  return dt == KDA_F32 ? 8 : 4;
}

// The single-row default tile width of launches large enough to be bound by
// bandwidth (what kda_tile_bv reports).
inline int32_t tile_bv(kda_dtype dt) { return default_bv(dt, 1); }

// The (bv, waves) shapes the kernels are instantiated for: 8, 16 or 32
// lanes per tile row (bv = lanes x columns per lane, at most 128), 1, 2, 4
// or 8 waves, at least 2 rows per lane (rows per lane = 2 * lanes / waves)
// and at most 128 state elements per lane, which keeps every variant free of
// register spills.
inline bool shape_supported(kda_dtype dt, int32_t bv, int32_t nw) {
  const int32_t cpl = cols_per_lane(dt);
  if (bv <= 0 || bv % cpl != 0 || kHeadV % bv != 0) return false;
  const int32_t lpr = bv / cpl;
  if (lpr != 8 && lpr != 16 && lpr != 32) return false;
  if (nw != 1 && nw != 2 && nw != 4 && nw != 8) return false;
  const int32_t rpl = 2 * lpr / nw;
  return rpl >= 2 && rpl * cpl <= 128;
}

// Whole-K chained-row shapes: bv = waves x lanes x columns per lane, with 2
// or 4 lanes per 16-byte row piece (32 or 16 row groups, 4 or 8 rows per
// lane: 16 or 32 state values per lane for fp32, 32 or 64 for fp16) and 2, 4
// or 8 waves; bv at most 128.  (One lane per piece, or one wave per
// workgroup, measured far slower: 16-byte pieces of a row written by
// different waves cost the stores most of their bandwidth.)
inline bool wave_k_supported(kda_dtype dt, int32_t bv, int32_t nw) {
  const int32_t cpl = cols_per_lane(dt);
  if (nw != 2 && nw != 4 && nw != 8) return false;
  if (bv <= 0 || bv % (nw * cpl) != 0 || kHeadV % bv != 0) return false;
  const int32_t lpr = bv / (nw * cpl);
  return lpr == 2 || lpr == 4;
}

// The chained-row layout of a launch of `units` = requests x heads with
// n_rows rows each.  An explicit rows_layout wins; the block_rows option
// alone means the K-split block form; a bv or waves option asks for a
// row-after-row shape (the whole-K layout for fp16, the K split for fp32).
// Otherwise, chosen by measurement on MI355X (H = 12, graph-replayed
// launches over 1 GiB of rotating pools; microseconds):
//   fp16: the matrix-core block form for 3 rows or more up to 240 units
//     (8 x 8: 8.4 against 12.0 with K split; 20 x 8: 15.0 against 15.6;
//     16 x 4: 8.8 against 9.1), the K split beyond (24 x 8: 19.6 against
//     20.9; 24 x 4: 11.6 against 13.9); for 2 rows the whole-K layout up to
//     48 units (1 x 2, 4 x 2: 4.3, 4.6 against 4.7, 5.0 with K split), the
//     K split beyond (16 x 2: 6.7 against 7.8 as a block, 7.7 whole-K).
//   fp32: the block form for 6 rows or more up to 48 units (1 x 8, 4 x 8:
//     7.5, 9.2 against 9.4, 10.6 with K split), the K split otherwise (8 x 8:
//     11.6 against 12.8; 8 x 6: 9.6 against 10.6; 1 x 2: 4.4 against 5.2).
inline int32_t chained_rows_layout(kda_dtype dt, int32_t n_rows, const kda_launch_opts* opts,
                                   int64_t units) {
  const int32_t asked = opts != nullptr ? opts->rows_layout : KDA_ROWS_DEFAULT;
  if (asked != KDA_ROWS_DEFAULT) return asked;
  if (opts != nullptr && opts->block_rows != 0) return KDA_ROWS_K_SPLIT;
  const bool shaped = opts != nullptr && (opts->bv != 0 || opts->waves_per_tile != 0);
  if (dt == KDA_F16) {
    if (shaped) return KDA_ROWS_WAVE_K;
    if (n_rows >= 3 && units <= 240) return KDA_ROWS_MATRIX;
    return units <= 48 ? KDA_ROWS_WAVE_K : KDA_ROWS_K_SPLIT;
  }
  return !shaped && n_rows >= 6 && units <= 48 ? KDA_ROWS_MATRIX : KDA_ROWS_K_SPLIT;
}
inline int32_t default_wave_k_bv(kda_dtype /*dt*/) { return 64; }
inline int32_t default_wave_k_waves(kda_dtype /*dt*/) { return 4; }

// The chained-rows block form: fp16 pools need at least 2 waves per tile.
inline bool block_supported(kda_dtype dt, int32_t nw) { return dt != KDA_F16 || nw > 1; }

// The matrix-core block form of chained rows: 64 columns per workgroup, K
// over 8 waves by default or over 4 (the first form, kept selectable); with
// the fused convolution, whole heads: two 64-column halves of 8 waves by
// default, or of 4.
constexpr int32_t kMatrixBV = 64;
constexpr int32_t kMatrixWaves = 8;
constexpr int32_t kMatrixWaves4 = 4;
constexpr int32_t kMatrixConvWaves = 2 * kMatrixWaves;
constexpr int32_t kMatrixConvWaves4 = 2 * kMatrixWaves4;
// The kernels take H packed into 16 bits of a kernel argument.
constexpr int32_t kMaxHeads = 0xFFFF;

struct Shape {
  int32_t bv;      // value columns per workgroup
  int32_t nw;      // waves per workgroup
  int32_t layout;  // KDA_ROWS_K_SPLIT (also every single-row launch), _WAVE_K or _MATRIX
};

// The shape a launch of `units` = requests x heads uses: each option field
// that is set overrides the default.  Returns false if the result is not an
// instantiated shape.
inline bool resolve_shape(kda_dtype dt, int32_t n_rows, int64_t units, const kda_launch_opts* opts,
                          Shape* out) {
  const int32_t asked = opts != nullptr ? opts->rows_layout : KDA_ROWS_DEFAULT;
  if (asked < KDA_ROWS_DEFAULT || asked > KDA_ROWS_MATRIX) return false;
  if (opts != nullptr && opts->g_raw != 0) return false;  // the fused front end's option
  const int32_t layout = n_rows > 1 ? chained_rows_layout(dt, n_rows, opts, units) : KDA_ROWS_K_SPLIT;
  if (layout == KDA_ROWS_MATRIX) {
    // 64 columns over 8 waves (default) or 4; a block form whatever
    // block_rows says
    const bool bv_ok = opts == nullptr || opts->bv == 0 || opts->bv == kMatrixBV;
    const int32_t nw = opts == nullptr || opts->waves_per_tile == 0 ? kMatrixWaves : opts->waves_per_tile;
    *out = Shape{kMatrixBV, nw, KDA_ROWS_MATRIX};
    return bv_ok && (nw == kMatrixWaves || nw == kMatrixWaves4);
  }
  // the K-split block form
  if (n_rows > 1 && opts != nullptr && opts->block_rows != 0 && layout == KDA_ROWS_WAVE_K) return false;
  Shape s{default_bv(dt, n_rows, units), default_waves_per_tile(dt, n_rows, units), layout};
  if (layout == KDA_ROWS_WAVE_K) {
    s.bv = default_wave_k_bv(dt);
    s.nw = default_wave_k_waves(dt);
  }
  if (opts != nullptr) {
    if (opts->bv != 0) s.bv = opts->bv;
    if (opts->waves_per_tile != 0) s.nw = opts->waves_per_tile;
  }
  *out = s;
  if (layout == KDA_ROWS_WAVE_K) return wave_k_supported(dt, s.bv, s.nw);
  // The block form keeps, per lane, the fp32 state and 3 x 8 column sums per
  // column; with one wave an fp16 tile (128 state values per lane) would
  // spill registers.
  if (n_rows > 1 && opts != nullptr && opts->block_rows != 0 && !block_supported(dt, s.nw))
    return false;
  return shape_supported(dt, s.bv, s.nw);
}

// Bytes of static LDS per workgroup: the staged per-row vectors (normalised
// q and k and the decay, 128 each; the workgroup's bv columns of v; beta and
// qn.kn) for up to KDA_MAX_ROWS rows (1 for single-row launches), plus, in
// the K-split layout, the cross-wave sums: row after row, double-buffered
// [2][nw][2][bv] (nw > 1); as a block, [nw][2 KDA_MAX_ROWS][bv] (nw > 1)
// and the two coupling matrices [KDA_MAX_ROWS][KDA_MAX_ROWS].
inline int32_t lds_bytes(int32_t bv, int32_t nw, int32_t n_rows, bool rows_block, int32_t layout) {
  if (layout == KDA_ROWS_MATRIX) {
    constexpr int32_t t = KDA_MAX_ROWS;
    // 8 waves: kn, qn, decays [8][132]; v [8][bv]; the waves' partial sums
    // [8][16][bv] and their totals [16][bv]; two 8 x 8 couplings; beta
    if (nw == kMatrixWaves) return 4 * (3 * t * (kHeadK + 4) + t * bv + (nw + 1) * 16 * bv + 2 * t * t + t);
    // 4 waves (and the convolution's two halves of 4): kn, qn, decays,
    // cumulative decays [8][132]; v [8][bv]; partial sums [nw][16][64]
    return 4 * (4 * t * (kHeadK + 4) + t * bv + nw * 16 * kMatrixBV + 2 * t * t + t);
  }
  const int32_t tmax = n_rows == 1 ? 1 : KDA_MAX_ROWS;
  const int32_t staged = tmax * (3 * kHeadK + bv + 2);
  if (layout == KDA_ROWS_WAVE_K) return 4 * staged;
  const bool block = n_rows > 1 && rows_block;
  const int32_t red = (nw > 1 && !block ? 2 * nw : 1) * 2 * bv;
  const int32_t wp = block && nw > 1 ? nw * 2 * tmax * bv : 4;
  const int32_t coupling = block ? 2 * tmax * tmax : 2;
  return 4 * (staged + red + wp + coupling);
}

// Fused-convolution launches take whole heads (bv = 128) so that a head's
// convolution history is read and rewritten inside one workgroup, except
// chained rows in the matrix-core block form with pair counters: those may
// take 64-column halves (bv = 64, 8 waves; the two halves of a head hand the
// initial slot's history over through the request's and head's counter).
// An explicit rows_layout wins (the matrix-core form: halves with counters,
// whole heads without, unless bv says which); bv 64 alone asks for the
// halves; a waves or block_rows option asks for the K split.  Otherwise,
// measured on MI355X (H = 12, graph-replayed launches over 1 GiB of rotating
// pools; microseconds):
//   halves, with counters: fp16 up to 96 units (8 x 8: 10.9 against 13.2
//     whole heads and 17.4 with K split; 8 x 2: 7.5 against 8.1 K split),
//     fp32 up to 48 units, or up to 96 with 6 rows or more (4 x 8: 11.2
//     against 13.2 and 15.8; 8 x 8: 15.7 against 16.0 and 16.3; 8 x 4: 11.2
//     against 10.9 with K split);
//   whole heads over 16 waves, for 3 rows or more: fp16 up to 192 units
//     (12 x 8: 14.3 against 14.9 in halves and 17.8 K split; 16 x 4: 11.7
//     against 11.5 K split), fp32 up to 48 (4 x 4: 10.4 against 10.7);
//   the K split beyond (fp16 24 x 4: 15.1 against 19.3 in halves; 48 x 2:
//     14.0 against 24.0; fp32 12 x 8: 19.4 against 21.1 whole heads).
// The K split takes 2, 4 or 8 waves per tile (default: 2 fp32 / 4 fp16 for
// one row, 8 / 4 for chained rows).  A bv option other than 0, 64 (the
// halves, which need counters) or 128, or the whole-K row layout, is
// refused; rows_layout is ignored for one row.
inline bool resolve_conv_shape(kda_dtype dt, int32_t n_rows, int64_t units, const kda_launch_opts* opts,
                               bool pairs, Shape* out) {
  const int32_t asked = opts != nullptr ? opts->rows_layout : KDA_ROWS_DEFAULT;
  if (asked < KDA_ROWS_DEFAULT || asked > KDA_ROWS_MATRIX || asked == KDA_ROWS_WAVE_K) return false;
  if (opts != nullptr && opts->g_raw != 0 && opts->g_raw != 1) return false;
  const int32_t bv = opts != nullptr ? opts->bv : 0;
  if (bv != 0 && bv != kHeadV && bv != kMatrixBV) return false;
  if (n_rows > 1) {
    const bool shaped = opts != nullptr && (opts->waves_per_tile != 0 || opts->block_rows != 0);
    int32_t bvm = 0;  // columns per workgroup of the matrix-core form; 0: the K split
    if (asked == KDA_ROWS_MATRIX || (asked == KDA_ROWS_DEFAULT && bv == kMatrixBV)) {
      bvm = bv != 0 ? bv : (pairs ? kMatrixBV : kHeadV);
    } else if (asked == KDA_ROWS_DEFAULT && !shaped) {
      const bool f16 = dt == KDA_F16;
      const bool halves = pairs && bv == 0 &&
                          (f16 ? units <= 96 || (units <= 240 && n_rows >= 6)
                               : units <= 48 || (units <= 96 && n_rows >= 4));
      const bool head = n_rows >= 3 && units <= (f16 ? 192 : 48);
      bvm = halves ? kMatrixBV : head ? kHeadV : 0;
    }
    if (bvm != 0) {
      const int32_t nw_default = bvm == kMatrixBV ? kMatrixWaves : kMatrixConvWaves;
      const int32_t nw = opts == nullptr || opts->waves_per_tile == 0 ? nw_default : opts->waves_per_tile;
      *out = Shape{bvm, nw, KDA_ROWS_MATRIX};
      if (bvm == kMatrixBV) return pairs && nw == kMatrixWaves;
      return nw == kMatrixConvWaves || nw == kMatrixConvWaves4;
    }
  }
  if (bv == kMatrixBV) return false;  // halves: the matrix-core form only
  // one row: fp16 over 4 waves; fp32 over 2, or 4 from 384 requests x heads
  // (measured: 64 x 12 units 19.1 -> 18.2 us)
  const int32_t one_row = dt == KDA_F32 ? (units >= 384 ? 4 : 2) : 4;
  Shape s{kHeadV, n_rows == 1 ? one_row : (dt == KDA_F32 ? 8 : 4), KDA_ROWS_K_SPLIT};
  if (opts != nullptr && opts->waves_per_tile != 0) s.nw = opts->waves_per_tile;
  *out = s;
  return s.nw == 2 || s.nw == 4 || s.nw == 8;
}

// XCD-aware block -> tile map.  The dispatcher sends block b to XCD b % 8;
// give XCD x the x-th contiguous range of tiles, so the V-tiles of one
// (request, head) run on one XCD and share its L2.  A bijection of [0, n).
KDA_HD inline int32_t tile_of_block(int32_t b, int32_t n) {
  const int32_t per = n / kNumXcd;
  const int32_t rem = n % kNumXcd;
  const int32_t x = b % kNumXcd;
  const int32_t i = b / kNumXcd;
  const int32_t start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return start + i;
}

}  // namespace kda
