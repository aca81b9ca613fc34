// host_abi_check.cpp -- CPU test driver for the host half of the KDA decode
// C ABI (csrc/kda_host.cpp): validation, addressing, sizing, launch
// description, the block-to-tile map and the error strings.  It is built
// with plain g++ and the address and undefined-behaviour sanitizers by
// tests/test_sanitizers_cpu.py, linked with kda_host.cpp alone (no HIP
// runtime, no device code), and exits non-zero on the first failed check.
//
// The refusals follow ROCm/ATOM PR #2945, Changes (bf16 refused rather than
// reinterpreted; a pool of the other dtype refused) and PR #2130, Copilot
// review (a missing table is refused early, never dereferenced).  The random
// slot tables are checked against a brute-force statement of the rules that
// kda_validate and kda_prefill_validate document.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <set>
#include <vector>

#include "kda_decode.h"
#include "kda_launch.h"

static int g_failures = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, \
                   #cond);                                                 \
      ++g_failures;                                                        \
    }                                                                      \
  } while (0)

static kda_pool make_pool(int32_t n_slots, int32_t H = 12, int32_t K = 128, int32_t V = 128,
                          kda_dtype dt = KDA_F32) {
  static char dummy[16];  // never dereferenced: only host checks run here
  kda_pool p;
  p.base = dummy;
  p.n_slots = n_slots;
  p.H = H;
  p.K = K;
  p.V = V;
  p.dtype = dt;
  return p;
}

// splitmix64: a small deterministic generator for the random tables
static uint64_t g_rng = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64() {
  uint64_t z = (g_rng += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
static int32_t rand_in(int32_t lo, int32_t hi) {  // [lo, hi]
  return lo + static_cast<int32_t>(next_u64() % static_cast<uint64_t>(hi - lo + 1));
}

static void validate_refusals() {
  const int32_t ids[4] = {0, 1, 2, 3};
  kda_pool p = make_pool(8);
  CHECK(kda_validate(nullptr, ids, nullptr, 4, 1, KDA_F32) == KDA_ERR_NULL);
  CHECK(kda_validate(&p, nullptr, nullptr, 4, 1, KDA_F32) == KDA_ERR_NULL);
  kda_pool nb = p;
  nb.base = nullptr;
  CHECK(kda_validate(&nb, ids, nullptr, 4, 1, KDA_F32) == KDA_ERR_NULL);
  kda_pool bf = make_pool(8, 12, 128, 128, KDA_BF16);
  CHECK(kda_validate(&bf, ids, nullptr, 4, 1, KDA_BF16) == KDA_ERR_DTYPE_REFUSED);
  CHECK(kda_validate(&p, ids, nullptr, 4, 1, KDA_BF16) == KDA_ERR_DTYPE_REFUSED);
  CHECK(kda_validate(&p, ids, nullptr, 4, 1, static_cast<kda_dtype>(7)) == KDA_ERR_DTYPE_REFUSED);
  CHECK(kda_validate(&p, ids, nullptr, 4, 1, KDA_F16) == KDA_ERR_DTYPE_MISMATCH);
  kda_pool k64 = make_pool(8, 12, 64);
  CHECK(kda_validate(&k64, ids, nullptr, 4, 1, KDA_F32) == KDA_ERR_SHAPE);
  kda_pool v256 = make_pool(8, 12, 128, 256);
  CHECK(kda_validate(&v256, ids, nullptr, 4, 1, KDA_F32) == KDA_ERR_SHAPE);
  kda_pool h0 = make_pool(8, 0);
  CHECK(kda_validate(&h0, ids, nullptr, 4, 1, KDA_F32) == KDA_ERR_SHAPE);
  kda_pool s0 = make_pool(0);
  CHECK(kda_validate(&s0, ids, nullptr, 4, 1, KDA_F32) == KDA_ERR_SHAPE);
  CHECK(kda_validate(&p, ids, nullptr, 4, 0, KDA_F32) == KDA_ERR_ROWS);
  CHECK(kda_validate(&p, ids, nullptr, 4, 9, KDA_F32) == KDA_ERR_ROWS);
  CHECK(kda_validate(&p, ids, nullptr, -1, 1, KDA_F32) == KDA_ERR_ARG);
  CHECK(kda_validate(&p, ids, nullptr, 3, 3, KDA_F32) == KDA_ERR_SLOT);  // 9 rows > 8 slots
  // the workgroup count must fit in int32 at the narrowest tile
  kda_pool huge = make_pool(INT32_MAX, 65535);
  CHECK(kda_validate(&huge, ids, nullptr, 10000, 1, KDA_F32) == KDA_ERR_ARG);
  // H is packed into 16 bits of the kernels' arguments
  kda_pool wide = make_pool(8, 65536);
  CHECK(kda_validate(&wide, ids, nullptr, 4, 1, KDA_F32) == KDA_ERR_SHAPE);
  CHECK(kda_validate(&p, ids, nullptr, 4, 1, KDA_F32) == KDA_OK);
  CHECK(kda_validate(&p, ids, nullptr, 0, 1, KDA_F32) == KDA_OK);
  const int32_t dup[4] = {0, 1, 1, 3};
  CHECK(kda_validate(&p, dup, nullptr, 4, 1, KDA_F32) == KDA_ERR_SLOT);
  const int32_t oob[4] = {0, 1, 8, 3};
  CHECK(kda_validate(&p, oob, nullptr, 4, 1, KDA_F32) == KDA_ERR_SLOT);
  const int32_t neg[4] = {0, -1, 2, 3};
  CHECK(kda_validate(&p, neg, nullptr, 4, 1, KDA_F32) == KDA_ERR_SLOT);
  // initial slots: in range, the request's own snapshot slot or a slot no
  // request writes; never another request's snapshot slot
  const int32_t rows2[4] = {0, 1, 2, 3};  // 2 requests x 2 rows
  const int32_t init_ok[2] = {1, 7};
  CHECK(kda_validate(&p, rows2, init_ok, 2, 2, KDA_F32) == KDA_OK);
  const int32_t init_other[2] = {2, 7};
  CHECK(kda_validate(&p, rows2, init_other, 2, 2, KDA_F32) == KDA_ERR_SLOT);
  const int32_t init_oob[2] = {0, 8};
  CHECK(kda_validate(&p, rows2, init_oob, 2, 2, KDA_F32) == KDA_ERR_SLOT);
}

// kda_validate on random tables against the documented rules, written out
static void validate_random() {
  for (int it = 0; it < 4000; ++it) {
    const int32_t n_slots = rand_in(1, 64);
    const int32_t n_rows = rand_in(1, 8);
    const int32_t n_req = rand_in(0, n_slots / n_rows);
    const int64_t R = static_cast<int64_t>(n_req) * n_rows;
    std::vector<int32_t> ids(static_cast<size_t>(R) + 1);
    std::vector<int32_t> init(static_cast<size_t>(n_req) + 1);
    for (auto& x : ids) x = rand_in(-2, n_slots + 1);
    for (auto& x : init) x = rand_in(-1, n_slots);
    // mostly valid tables: a permutation prefix, sometimes perturbed
    if (next_u64() % 2 == 0) {
      std::vector<int32_t> perm(static_cast<size_t>(n_slots));
      for (int32_t i = 0; i < n_slots; ++i) perm[static_cast<size_t>(i)] = i;
      for (int32_t i = n_slots - 1; i > 0; --i) std::swap(perm[static_cast<size_t>(i)], perm[static_cast<size_t>(rand_in(0, i))]);
      for (int64_t i = 0; i < R; ++i) ids[static_cast<size_t>(i)] = perm[static_cast<size_t>(i)];
      if (R > 0 && next_u64() % 4 == 0) ids[static_cast<size_t>(rand_in(0, static_cast<int32_t>(R - 1)))] = rand_in(-1, n_slots);
    }
    const bool with_init = next_u64() % 2 == 0;
    // the rules
    int expect = KDA_OK;
    std::set<int32_t> seen;
    for (int64_t i = 0; i < R && expect == KDA_OK; ++i) {
      const int32_t s = ids[static_cast<size_t>(i)];
      if (s < 0 || s >= n_slots || !seen.insert(s).second) expect = KDA_ERR_SLOT;
    }
    if (expect == KDA_OK && with_init) {
      for (int32_t r = 0; r < n_req && expect == KDA_OK; ++r) {
        const int32_t s = init[static_cast<size_t>(r)];
        if (s < 0 || s >= n_slots) {
          expect = KDA_ERR_SLOT;
          break;
        }
        for (int64_t i = 0; i < R; ++i)
          if (ids[static_cast<size_t>(i)] == s && i / n_rows != r) expect = KDA_ERR_SLOT;
      }
    }
    kda_pool p = make_pool(n_slots, 2);
    const int got = kda_validate(&p, ids.data(), with_init ? init.data() : nullptr, n_req, n_rows, KDA_F32);
    CHECK(got == expect);
    if (got != expect) {
      std::fprintf(stderr, "  random table %d: got %d, expected %d\n", it, got, expect);
      return;
    }
  }
}

static void prefill_validate() {
  kda_pool p = make_pool(8);
  const int32_t init[3] = {0, 1, 2};
  const int32_t dst[3] = {3, 4, 5};
  const int32_t cu[4] = {0, 5, 5, 9};
  CHECK(kda_prefill_validate(&p, init, dst, cu, 3, 9, KDA_F32) == KDA_OK);
  CHECK(kda_prefill_validate(&p, init, nullptr, cu, 3, 9, KDA_F32) == KDA_OK);
  CHECK(kda_prefill_validate(&p, init, dst, cu, 3, 8, KDA_F32) == KDA_ERR_ARG);   // past n_tokens
  CHECK(kda_prefill_validate(&p, init, dst, cu, 3, -1, KDA_F32) == KDA_ERR_ARG);
  const int32_t dec[4] = {0, 5, 4, 9};
  CHECK(kda_prefill_validate(&p, init, dst, dec, 3, 9, KDA_F32) == KDA_ERR_ARG);
  const int32_t negc[4] = {-1, 5, 5, 9};
  CHECK(kda_prefill_validate(&p, init, dst, negc, 3, 9, KDA_F32) == KDA_ERR_ARG);
  CHECK(kda_prefill_validate(&p, nullptr, dst, cu, 3, 9, KDA_F32) == KDA_ERR_NULL);
  CHECK(kda_prefill_validate(&p, init, dst, nullptr, 3, 9, KDA_F32) == KDA_ERR_NULL);
  CHECK(kda_prefill_validate(&p, nullptr, nullptr, nullptr, 0, 0, KDA_F32) == KDA_OK);
  const int32_t dst_dup[3] = {3, 3, 5};
  CHECK(kda_prefill_validate(&p, init, dst_dup, cu, 3, 9, KDA_F32) == KDA_ERR_SLOT);
  const int32_t dst_other_init[3] = {3, 0, 5};  // sequence 1 stores to sequence 0's initial slot
  CHECK(kda_prefill_validate(&p, init, dst_other_init, cu, 3, 9, KDA_F32) == KDA_ERR_SLOT);
  const int32_t dst_oob[3] = {3, 8, 5};
  CHECK(kda_prefill_validate(&p, init, dst_oob, cu, 3, 9, KDA_F32) == KDA_ERR_SLOT);
  const int32_t init_dup_inplace[3] = {0, 0, 2};  // two sequences storing back to slot 0
  CHECK(kda_prefill_validate(&p, init_dup_inplace, nullptr, cu, 3, 9, KDA_F32) == KDA_ERR_SLOT);
  CHECK(kda_prefill_validate(&p, init, dst, cu, 3, 9, KDA_BF16) == KDA_ERR_DTYPE_REFUSED);
  CHECK(kda_prefill_validate(&p, init, dst, cu, 3, 9, KDA_F16) == KDA_ERR_DTYPE_MISMATCH);
  CHECK(kda_prefill_validate(&p, init, dst, cu, 9, 9, KDA_F32) == KDA_ERR_SLOT);  // n_seq > n_slots
}

static void state_at_and_sizes() {
  kda_pool p = make_pool(96, 12);
  std::vector<int32_t> ids(64);
  for (int i = 0; i < 64; ++i) ids[static_cast<size_t>(i)] = (i * 37 + 5) % 96;
  const int64_t slot = 12ll * 128 * 128;
  for (int r = 0; r < 8; ++r)
    for (int t = 0; t < 8; ++t)
      CHECK(kda_state_at(&p, ids.data(), 8, r, t) == ids[static_cast<size_t>(r * 8 + t)] * slot);
  CHECK(kda_state_at(nullptr, ids.data(), 8, 0, 0) == -KDA_ERR_NULL);
  CHECK(kda_state_at(&p, nullptr, 8, 0, 0) == -KDA_ERR_NULL);
  CHECK(kda_state_at(&p, ids.data(), 9, 0, 0) == -KDA_ERR_ROWS);
  CHECK(kda_state_at(&p, ids.data(), 8, 0, 8) == -KDA_ERR_ARG);
  CHECK(kda_state_at(&p, ids.data(), 8, -1, 0) == -KDA_ERR_ARG);
  const int32_t bad[1] = {96};
  CHECK(kda_state_at(&p, bad, 1, 0, 0) == -KDA_ERR_SLOT);
  kda_pool bf = make_pool(96, 12, 128, 128, KDA_BF16);
  CHECK(kda_state_at(&bf, ids.data(), 1, 0, 0) == -KDA_ERR_DTYPE_REFUSED);
  // offsets past 2^31 elements stay exact (64-bit)
  kda_pool big = make_pool(20000, 12);
  const int32_t high[1] = {19999};
  CHECK(kda_state_at(&big, high, 1, 0, 0) == 19999ll * slot);
  // sizing: 69 layers of one slot, fp32 minus fp16, is the pages' memory
  // table difference (56.17 - 29.04 MB, PR #2130 Memory)
  const size_t f32 = kda_pool_bytes(1, 12, 128, 128, KDA_F32);
  const size_t f16 = kda_pool_bytes(1, 12, 128, 128, KDA_F16);
  CHECK(f32 == 786432u && f16 == 393216u);
  CHECK((f32 - f16) * 69 == 27131904u);
  CHECK(kda_pool_bytes(1, 12, 128, 128, KDA_BF16) == 0);
  CHECK(kda_pool_bytes(-1, 12, 128, 128, KDA_F32) == 0);
  CHECK(kda_pool_bytes(11000, 12, 128, 128, KDA_F16) == 4325376000ull);
  CHECK(kda_tile_bv(KDA_F32) == 128 && kda_tile_bv(KDA_F16) == 64);
  CHECK(kda_tile_bv(KDA_BF16) < 0);
}

static void describe_launch() {
  kda_launch_desc d;
  CHECK(kda_describe_launch(1, 1, 12, KDA_F32, nullptr, nullptr) == KDA_ERR_NULL);
  CHECK(kda_describe_launch(1, 1, 12, KDA_BF16, nullptr, &d) == KDA_ERR_DTYPE_REFUSED);
  CHECK(kda_describe_launch(1, 1, 0, KDA_F32, nullptr, &d) == KDA_ERR_SHAPE);
  CHECK(kda_describe_launch(1, 1, 65536, KDA_F32, nullptr, &d) == KDA_ERR_SHAPE);
  CHECK(kda_describe_launch(1, 0, 12, KDA_F32, nullptr, &d) == KDA_ERR_ROWS);
  CHECK(kda_describe_launch(-1, 1, 12, KDA_F32, nullptr, &d) == KDA_ERR_ARG);
  // every default shape, and every option combination: a described launch
  // is internally consistent, and the workgroup count is the tile count
  const kda_dtype dts[2] = {KDA_F32, KDA_F16};
  for (kda_dtype dt : dts)
    for (int32_t n_rows = 1; n_rows <= 8; ++n_rows)
      for (int32_t n_req : {0, 1, 2, 3, 4, 5, 8, 16, 32, 64, 100, 200})
        for (int32_t nw : {0, 1, 2, 4, 8, 3})
          for (int32_t bv : {0, 32, 64, 128, 48})
            for (int32_t blk : {0, 1})
              for (int32_t layout : {0, 1, 2, 3, 4, -1}) {
                kda_launch_opts o{nw, bv, blk, layout, 0};
                std::memset(&d, 0, sizeof d);
                const int rc = kda_describe_launch(n_req, n_rows, 12, dt, &o, &d);
                CHECK(rc == KDA_OK || rc == KDA_ERR_ARG);
                if (rc != KDA_OK) continue;
                CHECK(d.bv > 0 && 128 % d.bv == 0);
                CHECK(d.waves_per_tile >= 1 && d.waves_per_tile <= 8);
                CHECK(d.threads == 64 * d.waves_per_tile);
                CHECK(d.tiles == n_req * 12 * (128 / d.bv));
                CHECK(d.blocks == d.tiles);
                CHECK(d.lds_bytes > 0 && d.lds_bytes <= 160 * 1024);  // gfx950: 160 KiB per CU
                CHECK(d.kernel != nullptr && std::strlen(d.kernel) > 0);
                CHECK(d.rows_layout >= 1 && d.rows_layout <= 3);
                if (n_rows == 1) CHECK(d.rows_layout == KDA_ROWS_K_SPLIT);
                if (nw == 3 || bv == 48) CHECK(false);  // never an admitted shape
              }
}

// The fused convolution's launch shapes (resolve_conv_shape): the defaults
// the layout header states, and every option combination consistent.
static bool conv_shape(kda_dtype dt, int32_t n_req, int32_t n_rows, bool pairs, kda::Shape* s,
                       int32_t nw = 0, int32_t bv = 0, int32_t blk = 0, int32_t layout = 0) {
  const kda_launch_opts o{nw, bv, blk, layout, 0};
  return kda::resolve_conv_shape(dt, n_rows, static_cast<int64_t>(n_req) * 12, &o, pairs, s);
}

static bool is_shape(const kda::Shape& s, int32_t bv, int32_t nw, int32_t layout) {
  return s.bv == bv && s.nw == nw && s.layout == layout;
}

static void conv_shapes() {
  using kda::Shape;
  Shape s{};
  const int32_t M = KDA_ROWS_MATRIX, KS = KDA_ROWS_K_SPLIT;
  // halves with counters: fp16 up to 96 units (240 from 6 rows), fp32 up to
  // 48 (96 from 4 rows)
  CHECK(conv_shape(KDA_F16, 8, 8, true, &s) && is_shape(s, 64, 8, M));
  CHECK(conv_shape(KDA_F16, 8, 2, true, &s) && is_shape(s, 64, 8, M));
  CHECK(conv_shape(KDA_F16, 9, 8, true, &s) && is_shape(s, 64, 8, M));
  CHECK(conv_shape(KDA_F16, 20, 6, true, &s) && is_shape(s, 64, 8, M));
  CHECK(conv_shape(KDA_F16, 9, 5, true, &s) && is_shape(s, 128, 16, M));   // whole heads
  CHECK(conv_shape(KDA_F16, 21, 8, true, &s) && is_shape(s, 128, 4, KS));  // K split
  CHECK(conv_shape(KDA_F16, 9, 2, true, &s) && is_shape(s, 128, 4, KS));
  CHECK(conv_shape(KDA_F32, 4, 2, true, &s) && is_shape(s, 64, 8, M));
  CHECK(conv_shape(KDA_F32, 8, 8, true, &s) && is_shape(s, 64, 8, M));
  CHECK(conv_shape(KDA_F32, 8, 4, true, &s) && is_shape(s, 64, 8, M));
  CHECK(conv_shape(KDA_F32, 8, 3, true, &s) && is_shape(s, 128, 8, KS));
  CHECK(conv_shape(KDA_F32, 9, 8, true, &s) && is_shape(s, 128, 8, KS));
  // without counters: whole heads from 3 rows, up to 192 (fp16) or 48 units
  CHECK(conv_shape(KDA_F16, 8, 8, false, &s) && is_shape(s, 128, 16, M));
  CHECK(conv_shape(KDA_F16, 16, 3, false, &s) && is_shape(s, 128, 16, M));
  CHECK(conv_shape(KDA_F16, 8, 2, false, &s) && is_shape(s, 128, 4, KS));
  CHECK(conv_shape(KDA_F16, 17, 8, false, &s) && is_shape(s, 128, 4, KS));
  CHECK(conv_shape(KDA_F32, 4, 4, false, &s) && is_shape(s, 128, 16, M));
  CHECK(conv_shape(KDA_F32, 8, 8, false, &s) && is_shape(s, 128, 8, KS));
  // one row: the single-row kernel over whole heads whatever the counters;
  // fp32 over 4 waves from 384 requests x heads
  CHECK(conv_shape(KDA_F16, 8, 1, true, &s) && is_shape(s, 128, 4, KS));
  CHECK(conv_shape(KDA_F16, 64, 1, false, &s) && is_shape(s, 128, 4, KS));
  CHECK(conv_shape(KDA_F32, 8, 1, true, &s) && is_shape(s, 128, 2, KS));
  CHECK(conv_shape(KDA_F32, 31, 1, false, &s) && is_shape(s, 128, 2, KS));
  CHECK(conv_shape(KDA_F32, 32, 1, false, &s) && is_shape(s, 128, 4, KS));
  CHECK(conv_shape(KDA_F32, 64, 1, true, &s) && is_shape(s, 128, 4, KS));
  // explicit choices
  CHECK(conv_shape(KDA_F16, 64, 8, true, &s, 0, 0, 0, M) && is_shape(s, 64, 8, M));
  CHECK(conv_shape(KDA_F16, 64, 8, false, &s, 0, 0, 0, M) && is_shape(s, 128, 16, M));
  CHECK(conv_shape(KDA_F16, 64, 8, true, &s, 0, 64) && is_shape(s, 64, 8, M));
  CHECK(conv_shape(KDA_F16, 8, 8, true, &s, 0, 128) && is_shape(s, 128, 16, M));
  CHECK(conv_shape(KDA_F16, 8, 8, true, &s, 8, 128, 0, M) && is_shape(s, 128, 8, M));
  CHECK(conv_shape(KDA_F16, 8, 8, true, &s, 8) && is_shape(s, 128, 8, KS));
  CHECK(!conv_shape(KDA_F16, 8, 8, false, &s, 0, 64));      // halves need counters
  CHECK(!conv_shape(KDA_F16, 8, 8, true, &s, 16, 64, 0, M));
  CHECK(!conv_shape(KDA_F16, 8, 8, true, &s, 0, 64, 0, KS));
  CHECK(!conv_shape(KDA_F16, 8, 1, true, &s, 0, 64));
  // the raw gate: 0 or 1 on the fused entries, refused on the plain ones
  {
    kda_launch_opts o{0, 0, 0, 0, 1};
    CHECK(kda::resolve_conv_shape(KDA_F16, 8, 96, &o, true, &s) && is_shape(s, 64, 8, M));
    o.g_raw = 2;
    CHECK(!kda::resolve_conv_shape(KDA_F16, 8, 96, &o, true, &s));
    o.g_raw = 1;
    kda_launch_desc d;
    CHECK(kda_describe_launch(8, 8, 12, KDA_F16, &o, &d) == KDA_ERR_ARG);
  }
  // every combination: an admitted shape is one a kernel exists for
  const kda_dtype dts[2] = {KDA_F32, KDA_F16};
  for (kda_dtype dt : dts)
    for (int32_t n_rows = 1; n_rows <= 8; ++n_rows)
      for (int32_t n_req : {1, 2, 4, 8, 9, 16, 17, 64})
        for (bool pairs : {false, true})
          for (int32_t nw : {0, 2, 4, 8, 16, 3})
            for (int32_t bv : {0, 64, 128, 32})
              for (int32_t blk : {0, 1})
                for (int32_t layout : {0, 1, 2, 3, 4}) {
                  if (!conv_shape(dt, n_req, n_rows, pairs, &s, nw, bv, blk, layout)) continue;
                  if (s.layout == M) {
                    CHECK(n_rows > 1);
                    CHECK(is_shape(s, 64, 8, M) || is_shape(s, 128, 16, M) || is_shape(s, 128, 8, M));
                    if (s.bv == 64) CHECK(pairs);
                  } else {
                    CHECK(s.layout == KS && s.bv == 128 && (s.nw == 2 || s.nw == 4 || s.nw == 8));
                  }
                  CHECK(nw != 3 && bv != 32 && layout != 2 && layout != 4);
                }
}

static void tile_map_and_strings() {
  for (int32_t n = 1; n <= 3100; n += (n < 64 ? 1 : 37)) {
    std::vector<char> hit(static_cast<size_t>(n), 0);
    for (int32_t b = 0; b < n; ++b) {
      const int32_t t = kda_tile_of_block(b, n);
      CHECK(t >= 0 && t < n);
      if (t >= 0 && t < n) {
        CHECK(hit[static_cast<size_t>(t)] == 0);
        hit[static_cast<size_t>(t)] = 1;
      }
    }
  }
  CHECK(kda_tile_of_block(-1, 10) == -1);
  CHECK(kda_tile_of_block(10, 10) == -1);
  CHECK(kda_tile_of_block(0, 0) == -1);
  for (int c = -3; c < 16; ++c) {
    const char* s = kda_strerror(c);
    CHECK(s != nullptr && std::strlen(s) > 0);
  }
  CHECK(kda_abi_version() == KDA_ABI_VERSION);
}

int main() {
  validate_refusals();
  validate_random();
  prefill_validate();
  state_at_and_sizes();
  describe_launch();
  conv_shapes();
  tile_map_and_strings();
  if (g_failures != 0) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host ABI checks ok\n");
  return 0;
}
