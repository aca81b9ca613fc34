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

// Value columns per tile: one 128-byte line per tile row, i.e. 32 fp32 or
// 64 fp16 columns; a wavefront then spans 8 lanes x 16 bytes per row.
inline int32_t tile_bv(kda_dtype dt) { return dt == KDA_F32 ? 32 : 64; }

// Wavefronts splitting the K rows of one tile.  One wave per tile when each
// request has one row: no LDS, no barrier, 16 rows per lane.  Chained rows
// (speculative verify) have few tiles and write one snapshot per row, so K
// is split over more waves to spread the fp32 work and the stores over the
// chip; the partial column sums then meet in LDS once per row.
inline int32_t default_waves_per_tile(kda_dtype /*dt*/, int32_t n_rows) {
  return n_rows == 1 ? 1 : 4;
}

inline bool waves_allowed(int32_t nw) { return nw == 0 || nw == 1 || nw == 2 || nw == 4 || nw == 8; }

// The wave count a launch uses: the option if set, else the default.
inline int32_t waves_per_tile(kda_dtype dt, int32_t n_rows, const kda_launch_opts* opts) {
  if (opts != nullptr && opts->waves_per_tile != 0) return opts->waves_per_tile;
  return default_waves_per_tile(dt, n_rows);
}

// Bytes of static LDS per workgroup: the staged per-row vectors (normalised
// q and k and the decay, 128 each; the tile's bv columns of v; beta and
// qn.kn) for up to KDA_MAX_ROWS rows (1 for single-row launches), plus, with
// nw > 1, the double-buffered cross-wave sums [2][nw][2][bv].
inline int32_t lds_bytes(int32_t bv, int32_t nw, int32_t n_rows) {
  const int32_t tmax = n_rows == 1 ? 1 : KDA_MAX_ROWS;
  const int32_t staged = tmax * (3 * kHeadK + bv + 2);
  const int32_t red = nw == 1 ? 0 : 2 * nw * 2 * bv;
  return 4 * (staged + red);
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
