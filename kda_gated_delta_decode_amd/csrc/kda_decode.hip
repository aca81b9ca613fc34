// kda_decode.hip -- gfx950 (MI355X) kernels and launch entry points of the
// KDA recurrent decode library.
//
// The update (one decode row of one request, per head; the state S is a
// [K=128, V=128] fp32 matrix while it is in registers):
//   S' = diag(exp(g)) S,  u = v - S'^T kn,  S = S' + beta kn u^T,
//   o = scale * S^T qn,   with qn, kn the L2-normalised q, k and
//   beta = sigmoid(b).
// Pool handling follows ROCm/ATOM PR #2945 (Summary, Changes): the pool's
// dtype is a build constant, loads widen to fp32, the recurrence is fp32,
// fp16 stores round to nearest even, and one address function (state_at)
// locates the initial state and every row's snapshot.  ROCm/ATOM PR #2130
// (What) places the normalisation of q and k inside the kernel.
//
// Work decomposition.  A tile is (request, head, V-tile): all 128 key rows
// by BV value columns, BV chosen so a tile row is one 128-byte line (32 fp32
// or 64 fp16 columns).  Value columns are independent, so a tile needs no
// data from any other tile.  Inside a wavefront, 8 lanes cover one tile row
// with 16-byte loads; the 8 row groups of a wave each own a contiguous run
// of rows.  Column sums over K are an in-lane sum over the lane's rows, then
// an exchange across the row groups (lane bits 3..5: DPP row_ror:8, then the
// gfx950 permlane16/permlane32 swaps), which leaves the same bits in every
// lane.  With NW > 1 waves per tile the per-wave sums meet in LDS.
//
// The state is streamed: each tile is read once and written once per launch,
// so its loads and stores carry the nontemporal hint (measured on MI355X: a
// plain-load build of this kernel is about 15% slower).
//
// The read-out uses o_j = scale * (qn . s'_j + beta (qn . kn) u_j), the same
// quantity as scale * qn . s_j after the update (s_j = s'_j + beta kn u_j),
// so one pass over S' gives both column sums and the stores need not wait
// for a second reduction.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "kda_decode.h"
#include "kda_internal.h"
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

struct Args {
  void* pool;
  const int32_t* slot_ids;
  const int32_t* init_slot_ids;  // nullable: per-request initial-state slot
  const float* q;
  const float* k;
  const float* v;
  const float* g;
  const float* b;
  float* out;
  // fused short convolution (CONV kernels only)
  const float* x;          // raw q|k|v inputs [R, 3, H, 128]
  const float* conv_w;     // taps [3, H, 128, 4], tap 3 on the newest input
  uint16_t* conv_pool;     // bf16 history [n_slots, 3, 3 * H * 128], entry 0 oldest
  uint32_t* pair_counts;   // per (request, head) arrival counters (convolution in halves)
  int32_t n_slots;
  int32_t H;
  int32_t n_rows;
  int32_t n_vt;  // V-tiles per head
  int32_t rows_block;  // chained rows: 1 = as one block, 0 = row after row (default)
  float scale;
  int32_t g_raw;  // fused front end: g holds the raw gate x, g = -softplus(x)
};

// Every decode kernel takes the values its first memory requests depend on
// as leading plain arguments, 13 dwords in all, which the dispatcher
// preloads into scalar registers (the build asks for 14): the slot tables,
// the pool, q and k, the block count (the block-to-tile map needs it before
// anything else; the grid size would be one more fetch), the slot count (the
// range check of the ids gates the state loads) and the packed sizes
//   dims = H | n_vt << 16 | n_rows << 20 | init_stride << 24
// (H < 2^16, n_vt <= 4, n_rows <= 8; init_stride is 1 when an initial-slot
// table is given and n_rows when the row-0 ids are the initial slots, so the
// initial slot of request r is init_ids[r * init_stride] either way).  The
// rest of Args is fetched from memory as usual.
#define KDA_HOT_PARAMS                                                                         \
  const int32_t *__restrict__ hot_ids, const int32_t *__restrict__ hot_init, void *hot_pool,     \
      const float *__restrict__ hot_q, const float *__restrict__ hot_k, int32_t hot_blocks,    \
      int32_t hot_slots, int32_t hot_dims
struct Hot {
  const int32_t* ids;
  const int32_t* init;
  void* pool;
  const float* q;
  const float* k;
  int32_t blocks;
  int32_t slots;
  int32_t dims;
};
#define KDA_HOT_ARGS(h) (h).ids, (h).init, (h).pool, (h).q, (h).k, (h).blocks, (h).slots, (h).dims

// The preloaded values back into Args (the kernels read them from there);
// returns the initial-slot stride.
__device__ __forceinline__ int unpack_hot(Args& a, const int32_t* ids, void* pool, const float* q,
                                          const float* k, int32_t slots, int32_t dims) {
  a.slot_ids = ids;
  a.pool = pool;
  a.q = q;
  a.k = k;
  a.n_slots = slots;
  a.H = dims & 0xFFFF;
  a.n_vt = (dims >> 16) & 0xF;
  a.n_rows = (dims >> 20) & 0xF;
  return (dims >> 24) & 0xF;
}

// ---------------------------------------------------------------------------
// 16-byte state vectors: 4 fp32 or 8 fp16 columns of one tile row.
// ---------------------------------------------------------------------------
template <typename T>
struct Lane16;

template <>
struct Lane16<float> {
  using vec = f4;
  static constexpr int kCols = 4;
  __device__ __forceinline__ static void widen(const vec& r, float* s) {
#pragma unroll
    for (int c = 0; c < kCols; ++c) s[c] = r[c];
  }
  __device__ __forceinline__ static vec narrow(const float* s) {
    vec r;
#pragma unroll
    for (int c = 0; c < kCols; ++c) r[c] = s[c];
    return r;
  }
  __device__ __forceinline__ static void settle(float*) {}
};

template <>
struct Lane16<_Float16> {
  using vec = h8;
  static constexpr int kCols = 8;
  // fp16 -> fp32 is exact.
  __device__ __forceinline__ static void widen(const vec& r, float* s) {
#pragma unroll
    for (int c = 0; c < kCols; ++c) s[c] = static_cast<float>(r[c]);
  }
  // fp32 -> fp16 under the default round-to-nearest-even mode
  // (v_cvt_pk_f16_f32).  Its operands must have been settled (below).
  __device__ __forceinline__ static vec narrow(const float* s) {
    vec r;
#pragma unroll
    for (int c = 0; c < kCols; ++c) r[c] = static_cast<_Float16>(s[c]);
    return r;
  }
  // Pins each fp32 value, where it is computed, as a rounded fp32 register:
  // otherwise the backend may fold the fp32 fma that made it and a later
  // narrowing into one mixed-precision fma, which rounds once, straight to
  // fp16, instead of storing the rounded fp32 state's RNE (it does so even
  // where the fp32 value stays live, by computing the fma twice).  Pinned
  // at the definition, the value needs no copy when it stays live.
  __device__ __forceinline__ static void settle(float* s) {
#pragma unroll
    for (int c = 0; c < kCols; ++c) asm("" : "+v"(s[c]));
  }
};

// ---------------------------------------------------------------------------
// bfloat16 history entries of the short convolution: widening is exact (the
// top half of a binary32); narrowing rounds to nearest even (v_cvt_pk_bf16_f32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
// History words are loaded raw and widened only once the state tile's loads
// are issued: widening a word next to its load makes the wave wait for that
// load there, in front of its tile.
__device__ __forceinline__ f2 bf16_x2(uint32_t p) { return f2{bf16_lo(p), bf16_hi(p)}; }
__device__ __forceinline__ f4 bf16_x4(uint2 p) {
  return f4{bf16_lo(p.x), bf16_hi(p.x), bf16_lo(p.y), bf16_hi(p.y)};
}
__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {
  const uint16_t a = __builtin_bit_cast(uint16_t, static_cast<__bf16>(lo));
  const uint16_t b = __builtin_bit_cast(uint16_t, static_cast<__bf16>(hi));
  return static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float silu(float s) { return s / (1.0f + expf(-s)); }

// The decay a = e^g of a log-decay input g, or, when the input is the raw
// gate x of g = -softplus(x) = -log(1 + e^x), the same decay 1 / (1 + e^x)
// without forming the logarithm.
__device__ __forceinline__ float decay_of(float x, bool raw) {
  const float e = expf(x);
  return raw ? 1.0f / (1.0f + e) : e;
}

// ---------------------------------------------------------------------------
// Reads of N consecutive fp32 values from LDS (N a multiple of 2; 16-byte
// reads where N is a multiple of 4).
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void lds_rows(const float* src, float (&dst)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int m = 0; m < N; m += 4) {
      const f4 x = *reinterpret_cast<const f4*>(src + m);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[m + e] = x[e];
    }
  } else {
#pragma unroll
    for (int m = 0; m < N; m += 2) {
      const f2 x = *reinterpret_cast<const f2*>(src + m);
      dst[m] = x[0];
      dst[m + 1] = x[1];
    }
  }
}

// ---------------------------------------------------------------------------
// The decode kernel.  One workgroup = one tile = NW wavefronts splitting the
// 128 key rows.  MULTI selects the chained-rows variant (the fp32 state stays
// in registers across the request's rows); otherwise the request has one row
// and the tile stays packed in its storage type, widened where it is used.
// ---------------------------------------------------------------------------
template <typename T, int LPR, int NW, bool MULTI, bool CONV, bool BLOCK>
__global__ __launch_bounds__(kWave * NW) void kda_decode_tile(KDA_HOT_PARAMS, Args a) {
  const int init_stride = unpack_hot(a, hot_ids, hot_pool, hot_q, hot_k, hot_slots, hot_dims);
  using L = Lane16<T>;
  using vec = typename L::vec;
  constexpr int CPL = L::kCols;         // columns per lane
  constexpr int BV = LPR * CPL;         // columns per tile (LPR lanes per row)
  constexpr int GROUPS = kWave / LPR;   // row groups per wave
  constexpr int RPW = kHeadK / NW;      // rows per wave
  constexpr int RPL = RPW / GROUPS;     // rows per lane
  constexpr int TMAX = MULTI ? KDA_MAX_ROWS : 1;
  constexpr int TPW = (TMAX + NW - 1) / NW;  // prologue rows per wave
  static_assert(RPL % 2 == 0 && RPL >= 2 && RPL * CPL <= 128, "2+ rows, <= 128 elements per lane");
  static_assert(BV <= kHeadV && kHeadV % BV == 0, "tiles must divide V");
  // the fused convolution needs every channel of a head in one workgroup:
  // its history reads and snapshot writes are then ordered by a barrier
  static_assert(!CONV || BV == kHeadV, "the fused convolution takes whole heads");

  // Per-row vectors staged once: normalised q and k, decay a = exp(g), the
  // tile's columns of v, and the scalars beta and qn . kn.
  // (16-byte aligned: they are read and written with 8- and 16-byte ops)
  __shared__ __attribute__((aligned(16))) float s_qn[TMAX][kHeadK];
  __shared__ __attribute__((aligned(16))) float s_kn[TMAX][kHeadK];
  __shared__ __attribute__((aligned(16))) float s_a[TMAX][kHeadK];
  __shared__ __attribute__((aligned(16))) float s_v[TMAX][BV];
  __shared__ float s_beta[TMAX];
  __shared__ float s_qk[TMAX];
  __shared__ __attribute__((aligned(16))) float s_red[NW > 1 && !BLOCK ? 2 : 1][NW > 1 && !BLOCK ? NW : 1][2][BV];
  // rows as a block: each wave's partial column sums of the 2 x TMAX
  // projections of the initial state, and the TMAX x TMAX coupling matrices
  constexpr int BW = BLOCK && NW > 1 ? NW : 1;
  constexpr int BR = BLOCK && NW > 1 ? 2 * TMAX : 1;
  __shared__ __attribute__((aligned(16))) float s_wp[BW][BR][BLOCK && NW > 1 ? BV : 4];
  __shared__ float s_cA[BLOCK ? TMAX : 1][BLOCK ? TMAX : 1];
  __shared__ float s_cP[BLOCK ? TMAX : 1][BLOCK ? TMAX : 1];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int cg = lane % LPR;
  const int rg = lane / LPR;
  const int row0 = wave * RPW + rg * RPL;

  const int tile = tile_of_block(blockIdx.x, hot_blocks);
  const int vt = tile % a.n_vt;
  const int rh = tile / a.n_vt;
  const int h = rh % a.H;
  const int r = rh / a.H;
  const int n_rows = MULTI ? a.n_rows : 1;
  const int col0 = vt * BV + cg * CPL;
  const bool writer = (wave == 0) && (rg == 0);  // lanes that write `out`

  // Slot ids of this request, read once into wave-uniform registers before
  // any store (a re-read after the snapshot stores would be a vector load
  // that waits for every earlier store to retire).  A request with an id out
  // of range is skipped: its out rows become NaN, the pool is not touched.
  // both id loads are issued before either is waited for
  const int32_t init_slot = hot_init[static_cast<int64_t>(r) * init_stride];
  const int32_t* ids = a.slot_ids + static_cast<int64_t>(r) * n_rows;
  int32_t sid[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) sid[t] = t < n_rows ? ids[t] : 0;
  __builtin_amdgcn_sched_barrier(0);
  bool ids_ok = init_slot >= 0 && init_slot < a.n_slots;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) ids_ok = ids_ok && sid[t] >= 0 && sid[t] < a.n_slots;
  if (!ids_ok) {
    if (writer) {
      for (int t = 0; t < n_rows; ++t) {
        const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
        float* op = a.out + (rho * a.H + h) * kHeadV + col0;
#pragma unroll
        for (int c = 0; c < CPL; c += 4) *reinterpret_cast<f4*>(op + c) = f4{NAN, NAN, NAN, NAN};
      }
    }
    return;
  }

  // -- prologue loads: each wave takes rows wave, wave + NW, ... ------------
  // Every load a row's prologue needs is issued here, before the state
  // tile's, and consumed after the tile's loads are issued: a wave that
  // waited for its row inputs before issuing its tile would queue its tile
  // behind every other wave's and finish last.
  f2 q2[TPW], k2[TPW], g2[TPW];
  f4 v4[TPW];
  float braw[TPW];
  // fused convolution: the window win[t + m], m = 0..3 (3-entry history,
  // then this request's rows) of this lane's 2 q, 2 k and 4 v channels
  // (lanes past BV / 4 repeat the v channels of the first ones, so no load
  // sits behind a per-lane branch), and their taps
  constexpr int TC = CONV ? TPW : 1;
  f2 eq[TC][4], ek[TC][4];
  f4 ev[TC][4];
  uint32_t hwq[TC][4], hwk[TC][4];  // history entries as loaded (bf16 pairs)
  uint2 hwv[TC][4];
  f4 wq0, wq1, wk0, wk1, wv[4];
  const int64_t conv_c = static_cast<int64_t>(3) * a.H * kHeadK;  // channels per history entry
  const int64_t chq = static_cast<int64_t>(h) * kHeadK + 2 * lane;
  const int64_t chk = chq + static_cast<int64_t>(a.H) * kHeadK;
  const int64_t chv = static_cast<int64_t>(2 * a.H + h) * kHeadK + 4 * (CONV ? lane % (BV / 4) : lane);
  // unused here; without it the compiler orders the plain single-row kernels differently
  [[maybe_unused]] const bool conv_vl = lane < BV / 4;
  if constexpr (CONV) {
    if (wave < n_rows) {
      wq0 = *reinterpret_cast<const f4*>(a.conv_w + chq * 4);
      wq1 = *reinterpret_cast<const f4*>(a.conv_w + chq * 4 + 4);
      wk0 = *reinterpret_cast<const f4*>(a.conv_w + chk * 4);
      wk1 = *reinterpret_cast<const f4*>(a.conv_w + chk * 4 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) wv[e] = *reinterpret_cast<const f4*>(a.conv_w + (chv + e) * 4);
    }
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = wave + j * NW;
    if (t < n_rows) {
      const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
      const int64_t voff = (rho * a.H + h) * kHeadK;
      if constexpr (CONV) {
        // the history comes from the initial slot
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int pos = t + m;              // window index
          if (pos < 3) {
            const uint16_t* hb = a.conv_pool + (static_cast<int64_t>(init_slot) * 3 + pos) * conv_c;
            hwq[j][m] = *reinterpret_cast<const uint32_t*>(hb + chq);
            hwk[j][m] = *reinterpret_cast<const uint32_t*>(hb + chk);
            hwv[j][m] = *reinterpret_cast<const uint2*>(hb + chv);
          } else {
            const float* xr = a.x + (static_cast<int64_t>(r) * n_rows + (pos - 3)) * conv_c;
            eq[j][m] = *reinterpret_cast<const f2*>(xr + chq);
            ek[j][m] = *reinterpret_cast<const f2*>(xr + chk);
            ev[j][m] = *reinterpret_cast<const f4*>(xr + chv);
          }
        }
      } else {
        q2[j] = reinterpret_cast<const f2*>(a.q + voff)[lane];
        k2[j] = reinterpret_cast<const f2*>(a.k + voff)[lane];
        if (lane < BV / 4)
          v4[j] = *reinterpret_cast<const f4*>(a.v + (rho * a.H + h) * kHeadV + vt * BV + 4 * lane);
      }
      g2[j] = reinterpret_cast<const f2*>(a.g + voff)[lane];
      braw[j] = a.b[rho * a.H + h];
    }
  }

  // -- the state tile: RPL rows x 16 bytes per lane --------------------------
  const int64_t head_elems = static_cast<int64_t>(kHeadK) * kHeadV;
  const int64_t slot_elems = static_cast<int64_t>(a.H) * head_elems;
  const int64_t lane_off = h * head_elems + static_cast<int64_t>(row0) * kHeadV + col0;
  T* const pool = static_cast<T*>(a.pool);
  vec raw[RPL];
  {
    const T* src = pool + static_cast<int64_t>(init_slot) * slot_elems + lane_off;
#pragma unroll
    for (int m = 0; m < RPL; ++m)
      raw[m] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(src + m * kHeadV));
  }

  // -- fused convolution: y_t = silu(sum_m w_m win[t + m]) --------------------
  f2 hq[TC][3], hk[TC][3];  // the history each row's snapshot keeps (entries t+1 .. t+3)
  f4 hv[TC][3];
  if constexpr (CONV) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wave + j * NW;
      if (t < n_rows) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (t + m < 3) {
            eq[j][m] = bf16_x2(hwq[j][m]);
            ek[j][m] = bf16_x2(hwk[j][m]);
            ev[j][m] = bf16_x4(hwv[j][m]);
          }
        }
        float sq0 = 0.0f, sq1 = 0.0f, sk0 = 0.0f, sk1 = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          sq0 = fmaf(wq0[m], eq[j][m][0], sq0);
          sq1 = fmaf(wq1[m], eq[j][m][1], sq1);
          sk0 = fmaf(wk0[m], ek[j][m][0], sk0);
          sk1 = fmaf(wk1[m], ek[j][m][1], sk1);
        }
        q2[j] = f2{silu(sq0), silu(sq1)};
        k2[j] = f2{silu(sk0), silu(sk1)};
        f4 yv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sv = 0.0f;
#pragma unroll
          for (int m = 0; m < 4; ++m) sv = fmaf(wv[e][m], ev[j][m][e], sv);
          yv[e] = silu(sv);
        }
        v4[j] = yv;
#pragma unroll
        for (int e = 0; e < 3; ++e) {
          hq[j][e] = eq[j][e + 1];
          hk[j][e] = ek[j][e + 1];
          hv[j][e] = ev[j][e + 1];
        }
      }
    }
  }

  // -- prologue compute: norms over all 128 entries (lane holds 2), stage ----
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = wave + j * NW;
    if (t < n_rows) {
      const float sq = wave_sum(fmaf(q2[j][1], q2[j][1], q2[j][0] * q2[j][0]));
      const float sk = wave_sum(fmaf(k2[j][1], k2[j][1], k2[j][0] * k2[j][0]));
      const float sqk = wave_sum(fmaf(q2[j][1], k2[j][1], q2[j][0] * k2[j][0]));
      const float rq = 1.0f / sqrtf(sq + 1e-6f);
      const float rk = 1.0f / sqrtf(sk + 1e-6f);
      *reinterpret_cast<f2*>(&s_qn[t][2 * lane]) = f2{q2[j][0] * rq, q2[j][1] * rq};
      *reinterpret_cast<f2*>(&s_kn[t][2 * lane]) = f2{k2[j][0] * rk, k2[j][1] * rk};
      const bool raw = CONV && a.g_raw != 0;
      *reinterpret_cast<f2*>(&s_a[t][2 * lane]) = f2{decay_of(g2[j][0], raw), decay_of(g2[j][1], raw)};
      if (lane < BV / 4) *reinterpret_cast<f4*>(&s_v[t][4 * lane]) = v4[j];
      if (lane == 0) {
        s_beta[t] = 1.0f / (1.0f + expf(-braw[j]));
        s_qk[t] = (sqk * rq) * rk;
      }
    }
  }
  __syncthreads();

  if constexpr (CONV) {
    // every wave has read the history: the rows' snapshots may now overwrite
    // it (row 0's slot is the initial slot of an in-place launch)
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wave + j * NW;
      if (t < n_rows) {
        int32_t st = sid[0];
#pragma unroll
        for (int u = 1; u < TMAX; ++u)
          if (u == t) st = sid[u];
#pragma unroll
        for (int e = 0; e < 3; ++e) {
          uint16_t* hb = a.conv_pool + (static_cast<int64_t>(st) * 3 + e) * conv_c;
          *reinterpret_cast<uint32_t*>(hb + chq) = bf16_pack(hq[j][e][0], hq[j][e][1]);
          *reinterpret_cast<uint32_t*>(hb + chk) = bf16_pack(hk[j][e][0], hk[j][e][1]);
          if (lane < BV / 4)
            *reinterpret_cast<uint2*>(hb + chv) = uint2{bf16_pack(hv[j][e][0], hv[j][e][1]),
                                                         bf16_pack(hv[j][e][2], hv[j][e][3])};
        }
      }
    }
  }

  // fp32 state kept across rows (chained variant only)
  float S[MULTI ? RPL : 1][CPL];
  if constexpr (MULTI) {
#pragma unroll
    for (int m = 0; m < RPL; ++m) L::widen(raw[m], S[m]);
  }

  if constexpr (BLOCK) {
    // ---- the request's rows as one block ------------------------------------
    // With gamma_t = a_0 ... a_t (per key channel), Delta_t = beta_t u_t and
    // E_ts = a_(s+1) ... a_t, the chain unrolls to
    //   Delta_t = beta_t (v_t - w0_t - sum_{s<t} C_ts Delta_s),
    //   w0_t = S0^T (gamma_t kn_t),     C_ts = sum_i kn_ti kn_si E_ts,i,
    //   S_t  = diag(a_t) S_(t-1) + kn_t Delta_t^T,
    //   o_t  = scale (p0_t + sum_{s<=t} P_ts Delta_s),
    //   p0_t = S0^T (gamma_t qn_t),     P_ts = sum_i qn_ti kn_si E_ts,i.
    // All 2 n column sums over K are taken in one pass over S0 and reduced
    // together; the per-row work is then element-wise (no reduction, no
    // barrier between rows).
    // (1) C and P (wave 0): each lane forms the 64 partial sums (36 P_ts,
    // s <= t, then 28 C_ts, s < t) over its two key channels, and one
    // reduce-scatter over the wave leaves each total in one lane
    static_assert(TMAX == 8, "64 coupling values: 36 of P and 28 of C");
    if (wave == 0) {
      const int i0 = 2 * lane;
      float cv[64];
#pragma unroll
      for (int f = 0; f < 64; ++f) cv[f] = 0.0f;
#pragma unroll
      for (int s = 0; s < TMAX; ++s) {
        if (s >= n_rows) break;
        const f2 ks = *reinterpret_cast<const f2*>(&s_kn[s][i0]);
        float e0 = 1.0f, e1 = 1.0f;
#pragma unroll
        for (int t = s; t < TMAX; ++t) {
          if (t >= n_rows) break;
          const f2 qt = *reinterpret_cast<const f2*>(&s_qn[t][i0]);
          if (t > s) {
            const f2 at = *reinterpret_cast<const f2*>(&s_a[t][i0]);
            e0 *= at[0];
            e1 *= at[1];
          }
          const float f0 = ks[0] * e0, f1 = ks[1] * e1;
          cv[t * (t + 1) / 2 + s] = fmaf(qt[1], f1, qt[0] * f0);
          if (t > s) {
            const f2 kt = *reinterpret_cast<const f2*>(&s_kn[t][i0]);
            cv[36 + t * (t - 1) / 2 + s] = fmaf(kt[1], f1, kt[0] * f0);
          }
        }
      }
      const float tot = wave_reduce_scatter64(cv, lane);
      const int f = bitrev6(lane);
      const bool is_p = f < 36;
      const int c = is_p ? f : f - 36;
      int t = is_p ? 0 : 1;
      while ((is_p ? (t + 1) * (t + 2) / 2 : (t + 1) * t / 2) <= c) ++t;
      const int s = c - (is_p ? t * (t + 1) / 2 : t * (t - 1) / 2);
      if (is_p)
        s_cP[t][s] = tot;
      else
        s_cA[t][s] = tot;
    }
    // (2) per projection (w0: gamma kn, then p0: gamma qn): this lane's
    // partial column sums over its rows, summed over the row groups (and,
    // with NW > 1, left per wave in LDS for the sum over the waves)
    constexpr int NP = TMAX * CPL;  // [t][column]
    float w0[NP];                   // w0 totals (all lanes)
    float p0[NW == 1 ? NP : 1];     // p0 totals (NW == 1 only; else read from LDS)
#pragma unroll
    for (int qty = 0; qty < 2; ++qty) {
      float wp[NP];
      float gam[RPL];
#pragma unroll
      for (int m = 0; m < RPL; ++m) gam[m] = 1.0f;
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        float* w = &wp[t * CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) w[c] = 0.0f;
        if (t < n_rows) {
          float x[RPL], am[RPL];
          lds_rows<RPL>(qty == 0 ? &s_kn[t][row0] : &s_qn[t][row0], x);
          lds_rows<RPL>(&s_a[t][row0], am);
#pragma unroll
          for (int m = 0; m < RPL; ++m) {
            gam[m] *= am[m];
            const float gx = gam[m] * x[m];
#pragma unroll
            for (int c = 0; c < CPL; ++c) w[c] = fmaf(gx, S[m][c], w[c]);
          }
        }
      }
      if constexpr (NW == 1) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          if (qty == 0)
            w0[i] = rowgroup_sum<LPR>(wp[i]);
          else
            p0[i] = rowgroup_sum<LPR>(wp[i]);
        }
      } else {
        constexpr int Q = rs_quadrants<LPR>();
        constexpr int M = NP / Q;
        float part[M];
        rowgroup_reduce_scatter<LPR>(wp, part);
        const int quad = Q == 2 ? (lane >> 5) : ((lane >> 4) & 1) * 2 + (lane >> 5);
        if (LPR != 8 || (lane & 8) == 0) {
#pragma unroll
          for (int j = 0; j < M; j += 4) {
            const int f = quad * M + j;  // flat [t][column] index, 4 columns at a time
            *reinterpret_cast<f4*>(&s_wp[wave][qty * TMAX + f / CPL][cg * CPL + f % CPL]) =
                f4{part[j], part[j + 1], part[j + 2], part[j + 3]};
          }
        }
      }
    }
    __syncthreads();
    // totals over the waves: w0 for every lane; p0 is read by the writers below
    auto wave_total = [&](int row, float (&tot)[CPL]) {
      lds_rows<CPL>(&s_wp[0][row][cg * CPL], tot);
#pragma unroll
      for (int x = 1; x < NW; ++x) {
        float xs[CPL];
        lds_rows<CPL>(&s_wp[x][row][cg * CPL], xs);
#pragma unroll
        for (int c = 0; c < CPL; ++c) tot[c] += xs[c];
      }
    };
    if constexpr (NW > 1) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        if (t >= n_rows) break;
        float tot[CPL];
        wave_total(t, tot);
#pragma unroll
        for (int c = 0; c < CPL; ++c) w0[t * CPL + c] = tot[c];
      }
    }
    // (4) Delta for this lane's columns, row after row
    float dl[TMAX][CPL];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t >= n_rows) break;
      const float beta = s_beta[t];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float d = s_v[t][cg * CPL + c] - w0[t * CPL + c];
#pragma unroll
        for (int s2 = 0; s2 < t; ++s2) d = fmaf(-s_cA[t][s2], dl[s2][c], d);
        dl[t][c] = beta * d;
      }
    }
    // (5) each row's snapshot: S_t = diag(a_t) S_(t-1) + kn_t Delta_t^T
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t >= n_rows) break;
      float kn[RPL], am[RPL];
      lds_rows<RPL>(&s_kn[t][row0], kn);
      lds_rows<RPL>(&s_a[t][row0], am);
      T* dst = pool + static_cast<int64_t>(sid[t]) * slot_elems + lane_off;
#pragma unroll
      for (int m = 0; m < RPL; ++m) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) S[m][c] = fmaf(kn[m], dl[t][c], am[m] * S[m][c]);
        L::settle(S[m]);
        __builtin_nontemporal_store(L::narrow(S[m]), reinterpret_cast<vec*>(dst + m * kHeadV));
      }
    }
    // (6) outputs
    if (writer) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        if (t >= n_rows) break;
        const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
        float* op = a.out + (rho * a.H + h) * kHeadV + col0;
        float pt[CPL];
        if constexpr (NW == 1) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) pt[c] = p0[t * CPL + c];
        } else {
          wave_total(TMAX + t, pt);
        }
#pragma unroll
        for (int c = 0; c < CPL; c += 4) {
          f4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = pt[c + e];
#pragma unroll
            for (int s2 = 0; s2 <= t; ++s2) x = fmaf(s_cP[t][s2], dl[s2][c + e], x);
            o[e] = a.scale * x;
          }
          *reinterpret_cast<f4*>(op + c) = o;
        }
      }
    }
    return;
  }

  // Rows unrolled: every LDS index and slot id below is static.
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t >= n_rows) break;
    const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
    float qn[RPL], kn[RPL], am[RPL];
    lds_rows<RPL>(&s_qn[t][row0], qn);
    lds_rows<RPL>(&s_kn[t][row0], kn);
    lds_rows<RPL>(&s_a[t][row0], am);

    // Decay, then both column sums over this lane's rows.
    float w[CPL], p[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      w[c] = 0.0f;
      p[c] = 0.0f;
    }
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      float sp[CPL];
      if constexpr (MULTI) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) sp[c] = S[m][c];
      } else {
        L::widen(raw[m], sp);
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        sp[c] = am[m] * sp[c];
        w[c] = fmaf(kn[m], sp[c], w[c]);
        p[c] = fmaf(qn[m], sp[c], p[c]);
      }
      if constexpr (MULTI) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) S[m][c] = sp[c];
      }
    }
    if constexpr (NW == 1) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        w[c] = rowgroup_sum<LPR>(w[c]);
        p[c] = rowgroup_sum<LPR>(p[c]);
      }
    } else {
      // reduce-scatter inside the wave, then the waves' sums meet in LDS
      constexpr int Q = rs_quadrants<LPR>();
      constexpr int M = 2 * CPL / Q;
      float wp[2 * CPL], part[M];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        wp[c] = w[c];
        wp[CPL + c] = p[c];
      }
      rowgroup_reduce_scatter<LPR>(wp, part);
      const int quad = Q == 2 ? (lane >> 5) : ((lane >> 4) & 1) * 2 + (lane >> 5);
      const int qty = (quad * M) / CPL;        // 0: w, 1: p
      const int off = (quad * M) % CPL;        // first column of the quadrant
      const int par = t & 1;
      if (LPR != 8 || (lane & 8) == 0) {
        float* dstp = &s_red[par][wave][qty][cg * CPL + off];
        if constexpr (M == 4) {
          *reinterpret_cast<f4*>(dstp) = f4{part[0], part[1], part[2], part[3]};
        } else {
#pragma unroll
          for (int m = 0; m < M; m += 2) *reinterpret_cast<f2*>(dstp + m) = f2{part[m], part[m + 1]};
        }
      }
      __syncthreads();
      float tw[CPL], tp[CPL];
      lds_rows<CPL>(&s_red[par][0][0][cg * CPL], tw);
      lds_rows<CPL>(&s_red[par][0][1][cg * CPL], tp);
#pragma unroll
      for (int x = 1; x < NW; ++x) {
        float xw[CPL], xp[CPL];
        lds_rows<CPL>(&s_red[par][x][0][cg * CPL], xw);
        lds_rows<CPL>(&s_red[par][x][1][cg * CPL], xp);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          tw[c] += xw[c];
          tp[c] += xp[c];
        }
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        w[c] = tw[c];
        p[c] = tp[c];
      }
    }

    const float beta = s_beta[t];
    float u[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) u[c] = s_v[t][cg * CPL + c] - w[c];

    // Rank-1 correction and this row's snapshot store.
    T* dst = pool + static_cast<int64_t>(sid[t]) * slot_elems + lane_off;
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      const float bk = beta * kn[m];
      float s1[CPL];
      if constexpr (MULTI) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) s1[c] = fmaf(bk, u[c], S[m][c]);
      } else {
        // S' recomputed from the packed tile: the same product as above
        L::widen(raw[m], s1);
#pragma unroll
        for (int c = 0; c < CPL; ++c) s1[c] = fmaf(bk, u[c], am[m] * s1[c]);
      }
      L::settle(s1);
      if constexpr (MULTI) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) S[m][c] = s1[c];
      }
      __builtin_nontemporal_store(L::narrow(s1), reinterpret_cast<vec*>(dst + m * kHeadV));
    }

    if (writer) {
      const float bqk = beta * s_qk[t];
      float* op = a.out + (rho * a.H + h) * kHeadV + col0;
#pragma unroll
      for (int c = 0; c < CPL; c += 4) {
        f4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = a.scale * fmaf(bqk, u[c + e], p[c + e]);
        *reinterpret_cast<f4*>(op + c) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Chained rows with the whole of K inside each wavefront.  A workgroup takes
// NWB x BVW value columns of one (request, head); each of its waves holds all
// 128 key rows of BVW of them (LPR = 2 or 4 lanes per 16-byte piece of a
// row, 64/LPR row groups, RPL rows per lane), so a row's two column sums over K never
// leave the wave: no LDS round trip and no barrier between rows, and the
// waves of a workgroup run their chains independently.  Per row:
//  - in-lane partial sums w (over kn) and p (over qn) of the decayed state;
//  - reduce-scatter over the top log2(CPL) lane bits (permlane32/16 swaps
//    of register pairs, then DPP with a select) until each lane holds one w
//    and one p, for the column c(lane) its top bits name;
//  - all-reduce of those two over the remaining row-group bits (DPP);
//  - all-gather of w back over the top bits, so every lane has the w of its
//    CPL columns for the rank-1 update; the lanes whose all-reduced bits are
//    zero write o for their column.
// Rows t of the request run in order; row t's post-update state is stored
// to its snapshot slot before row t + 1 starts (ROCm/ATOM PR #2945, Changes:
// one snapshot per token, the state staying fp32 between tokens).
// ---------------------------------------------------------------------------
constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// The value that lane (lane xor 2^B) holds, for B = 0 .. 3 (DPP).
template <int B>
__device__ __forceinline__ float partner(float x) {
  static_assert(B >= 0 && B <= 3, "DPP partners only");
  if constexpr (B == 0) return dpp<kDppQuadXor1>(x);
  if constexpr (B == 1) return dpp<kDppQuadXor2>(x);
  if constexpr (B == 2) return dpp<kDppQuadXor3>(dpp<kDppRowHalfMirror>(x));
  return dpp<kDppRowRor8>(x);
}

// One reduce-scatter stage over lane bit B: pairs (x[2i], x[2i+1]) become
// one value y[i], the sum over the lane pair of x[2i] where bit B is clear
// and of x[2i+1] where it is set.
template <int B, int N>
__device__ __forceinline__ void rs_stage(const float (&x)[N], float (&y)[N / 2], int lane) {
  if constexpr (B == 5 || B == 4) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const auto r = B == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x[2 * i]),
                                                               __float_as_uint(x[2 * i + 1]), false, false)
                            : __builtin_amdgcn_permlane16_swap(__float_as_uint(x[2 * i]),
                                                               __float_as_uint(x[2 * i + 1]), false, false);
      y[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  } else {
    const bool hi = (lane >> B) & 1;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float keep = hi ? x[2 * i + 1] : x[2 * i];
      const float send = hi ? x[2 * i] : x[2 * i + 1];
      y[i] = keep + partner<B>(send);
    }
  }
}

// One all-gather stage over lane bit B: each lane's N values and its
// partner's become 2N, ordered so that out[2j + b] comes from the lane whose
// bit B is b.
template <int B, int N>
__device__ __forceinline__ void ag_stage(const float (&x)[N], float (&y)[2 * N], int lane) {
  if constexpr (B == 5 || B == 4) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const auto r = B == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]),
                                                               __float_as_uint(x[j]), false, false)
                            : __builtin_amdgcn_permlane16_swap(__float_as_uint(x[j]),
                                                               __float_as_uint(x[j]), false, false);
      y[2 * j] = __uint_as_float(r[0]);
      y[2 * j + 1] = __uint_as_float(r[1]);
    }
  } else {
    const bool hi = (lane >> B) & 1;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float other = partner<B>(x[j]);
      y[2 * j] = hi ? other : x[j];
      y[2 * j + 1] = hi ? x[j] : other;
    }
  }
}

// Column sums over the 64/LPR row groups of a wave.  x = [w_0..w_{C-1},
// p_0..p_{C-1}] per lane (C = CPL).  Returns the totals w_c, p_c of the
// column c = sum_s bit(5 - s) << s that the lane's top log2(C) bits name,
// and in wall[] the totals w_0 .. w_{C-1} of all C columns.
template <int C, int LB>
__device__ __forceinline__ void wave_column_sums(const float (&x)[2 * C], int lane, float& w_c,
                                                 float& p_c, float (&wall)[C]) {
  constexpr int TB = ilog2c(C);
  static_assert(C == 4 || C == 8, "4 or 8 columns per lane");
  static_assert(6 - TB >= LB, "the top bits must be row-group bits");
  float y[C], z[C / 2];
  rs_stage<5>(x, y, lane);
  rs_stage<4>(y, z, lane);
  float u[2];
  if constexpr (C == 8) {
    rs_stage<3>(z, u, lane);
  } else {
    u[0] = z[0];
    u[1] = z[1];
  }
  // all-reduce over the row-group bits below the top ones
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float v = u[e];
    if constexpr (5 - TB >= 3 && LB <= 3) v += partner<3>(v);
    if constexpr (5 - TB >= 2 && LB <= 2) v += partner<2>(v);
    if constexpr (5 - TB >= 1 && LB <= 1) v += partner<1>(v);
    if constexpr (LB <= 0) v += partner<0>(v);
    u[e] = v;
  }
  w_c = u[0];
  p_c = u[1];
  // all-gather of w over the top bits, lowest of them first
  float g1[1] = {w_c};
  if constexpr (C == 8) {
    float g2[2], g4[4];
    ag_stage<3>(g1, g2, lane);
    ag_stage<4>(g2, g4, lane);
    ag_stage<5>(g4, wall, lane);
  } else {
    float g2[2];
    ag_stage<4>(g1, g2, lane);
    ag_stage<5>(g2, wall, lane);
  }
}

template <typename T, int LPR, int NWB>
__global__ __launch_bounds__(kWave * NWB) void kda_rows_kernel(KDA_HOT_PARAMS, Args a) {
  const int init_stride = unpack_hot(a, hot_ids, hot_pool, hot_q, hot_k, hot_slots, hot_dims);
  using L = Lane16<T>;
  using vec = typename L::vec;
  constexpr int CPL = L::kCols;           // columns per lane
  constexpr int BVW = LPR * CPL;          // columns per wave
  constexpr int BVB = NWB * BVW;          // columns per workgroup
  constexpr int GROUPS = kWave / LPR;     // row groups per wave
  constexpr int RPL = kHeadK / GROUPS;    // rows per lane
  constexpr int TMAX = KDA_MAX_ROWS;
  constexpr int TPW = (TMAX + NWB - 1) / NWB;
  constexpr int LB = ilog2c(LPR);         // lowest row-group lane bit
  constexpr int TB = ilog2c(CPL);         // top lane bits that name a column
  // lanes that write o: all-reduced bits (LB .. 5 - TB) clear
  constexpr int kArMask = ((1 << (6 - TB)) - 1) & ~((1 << LB) - 1);
  static_assert(RPL % 2 == 0 && RPL * CPL <= 64, "2+ rows and <= 64 state values per lane");
  static_assert(BVB <= kHeadV && kHeadV % BVB == 0, "workgroups must divide V");

  __shared__ __attribute__((aligned(16))) float s_qn[TMAX][kHeadK];
  __shared__ __attribute__((aligned(16))) float s_kn[TMAX][kHeadK];
  __shared__ __attribute__((aligned(16))) float s_a[TMAX][kHeadK];
  __shared__ __attribute__((aligned(16))) float s_v[TMAX][BVB];
  __shared__ float s_beta[TMAX];
  __shared__ float s_qk[TMAX];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int cg = lane % LPR;
  const int row0 = (lane / LPR) * RPL;

  const int tile = tile_of_block(blockIdx.x, hot_blocks);
  const int vt = tile % a.n_vt;
  const int rh = tile / a.n_vt;
  const int h = rh % a.H;
  const int r = rh / a.H;
  const int n_rows = a.n_rows;
  const int wcol = wave * BVW + cg * CPL;  // the lane's first column inside the workgroup's
  const int col0 = vt * BVB + wcol;

  // Slot ids: wave-uniform scalar loads, issued first and read once (a
  // re-read after the snapshot stores would be a vector load that waits for
  // every earlier store).  The initial slot is one load from a selected
  // address: a select between two loaded values would wait for the ids
  // before the row loads below go out.
  // both id loads are issued before either is waited for
  const int32_t init_slot = hot_init[static_cast<int64_t>(r) * init_stride];
  const int32_t* ids = a.slot_ids + static_cast<int64_t>(r) * n_rows;
  int32_t sid[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) sid[t] = t < n_rows ? ids[t] : 0;
  __builtin_amdgcn_sched_barrier(0);

  // Row inputs (wave w stages rows w, w + NWB, ...), issued before anything
  // waits on the ids.  Every address is valid whatever n_rows is (a row past
  // the last re-reads the last one; lanes past the workgroup's v columns
  // re-read its first ones), so no branch join waits for their data.  b goes
  // through a vector register (an opaque zero in its index): a scalar load
  // would share the ids' counter and be waited for with them.
  int zero_v;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero_v));
  f2 q2[TPW], k2[TPW], g2[TPW];
  f4 v4[TPW];
  float braw[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = min(wave + j * NWB, n_rows - 1);
    const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
    const int64_t off = (rho * a.H + h) * kHeadK;
    q2[j] = reinterpret_cast<const f2*>(a.q + off)[lane];
    k2[j] = reinterpret_cast<const f2*>(a.k + off)[lane];
    g2[j] = reinterpret_cast<const f2*>(a.g + off)[lane];
    v4[j] = *reinterpret_cast<const f4*>(a.v + off + vt * BVB + 4 * (lane % (BVB / 4)));
    braw[j] = a.b[rho * a.H + h + zero_v];
  }
  __builtin_amdgcn_sched_barrier(0);

  // A request with an id out of range is skipped: out rows NaN, pool untouched.
  bool ids_ok = init_slot >= 0 && init_slot < a.n_slots;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) ids_ok = ids_ok && sid[t] >= 0 && sid[t] < a.n_slots;

  // The state: RPL rows x 16 bytes per lane (slot 0 for a request that is
  // skipped below, so every address stays valid).
  const int64_t head_elems = static_cast<int64_t>(kHeadK) * kHeadV;
  const int64_t slot_elems = static_cast<int64_t>(a.H) * head_elems;
  const int64_t lane_off = h * head_elems + static_cast<int64_t>(row0) * kHeadV + col0;
  T* const pool = static_cast<T*>(a.pool);
  vec raw[RPL];
  {
    const T* src = pool + static_cast<int64_t>(ids_ok ? init_slot : 0) * slot_elems + lane_off;
#pragma unroll
    for (int m = 0; m < RPL; ++m)
      raw[m] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(src + m * kHeadV));
  }
  __builtin_amdgcn_sched_barrier(0);

  // Per-row vectors: norms over all 128 entries (lane holds 2), staged.
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = wave + j * NWB;
    if (t < n_rows) {
      const float sq = wave_sum(fmaf(q2[j][1], q2[j][1], q2[j][0] * q2[j][0]));
      const float sk = wave_sum(fmaf(k2[j][1], k2[j][1], k2[j][0] * k2[j][0]));
      const float sqk = wave_sum(fmaf(q2[j][1], k2[j][1], q2[j][0] * k2[j][0]));
      const float rq = 1.0f / sqrtf(sq + 1e-6f);
      const float rk = 1.0f / sqrtf(sk + 1e-6f);
      *reinterpret_cast<f2*>(&s_qn[t][2 * lane]) = f2{q2[j][0] * rq, q2[j][1] * rq};
      *reinterpret_cast<f2*>(&s_kn[t][2 * lane]) = f2{k2[j][0] * rk, k2[j][1] * rk};
      *reinterpret_cast<f2*>(&s_a[t][2 * lane]) = f2{expf(g2[j][0]), expf(g2[j][1])};
      if (lane < BVB / 4) *reinterpret_cast<f4*>(&s_v[t][4 * lane]) = v4[j];
      if (lane == 0) {
        s_beta[t] = 1.0f / (1.0f + expf(-braw[j]));
        s_qk[t] = (sqk * rq) * rk;
      }
    }
  }
  if (!ids_ok) {  // uniform over the workgroup: no wave waits at the barrier
    if (wave == 0 && lane < BVB / 4) {
      for (int t = 0; t < n_rows; ++t) {
        const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
        *reinterpret_cast<f4*>(a.out + (rho * a.H + h) * kHeadV + vt * BVB + 4 * lane) =
            f4{NAN, NAN, NAN, NAN};
      }
    }
    return;
  }
  __syncthreads();

  float S[RPL][CPL];
#pragma unroll
  for (int m = 0; m < RPL; ++m) L::widen(raw[m], S[m]);

  const int c_mine = ((lane >> 5) & 1) | (((lane >> 4) & 1) << 1) | (CPL == 8 ? ((lane >> 3) & 1) << 2 : 0);
  const bool writer = (lane & kArMask) == 0;

#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t >= n_rows) break;
    float kn[RPL], qn[RPL], am[RPL], vv[CPL];
    lds_rows<RPL>(&s_kn[t][row0], kn);
    lds_rows<RPL>(&s_qn[t][row0], qn);
    lds_rows<RPL>(&s_a[t][row0], am);
    lds_rows<CPL>(&s_v[t][wcol], vv);

    // decay, then this lane's partial sums over its rows
    float x[2 * CPL];
#pragma unroll
    for (int c = 0; c < 2 * CPL; ++c) x[c] = 0.0f;
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float sp = am[m] * S[m][c];
        S[m][c] = sp;
        x[c] = fmaf(kn[m], sp, x[c]);
        x[CPL + c] = fmaf(qn[m], sp, x[CPL + c]);
      }
    }
    float w_c, p_c, w[CPL];
    wave_column_sums<CPL, LB>(x, lane, w_c, p_c, w);

    const float beta = s_beta[t];
    float u[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) u[c] = vv[c] - w[c];

    // rank-1 correction and this row's snapshot.  A wave writes 32-byte
    // (fp16) or 64-byte (fp32) pieces of each 128-byte line, the rest of the
    // line coming from its sibling waves, so the stores are ordinary
    // write-back stores: the L2 merges the pieces into whole lines.  With
    // nontemporal stores the pieces reach memory as partial writes unless
    // the waves' stores of a line happen to arrive together; measured on
    // MI355X that made the launch 11.0 to 19.4 us depending on instruction
    // timing alone (and 17 us at bv 128 over 8 waves), against a steady
    // 11.9 (and 14.1) us with write-back stores.
    T* dst = pool + static_cast<int64_t>(sid[t]) * slot_elems + lane_off;
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      const float bk = beta * kn[m];
#pragma unroll
      for (int c = 0; c < CPL; ++c) S[m][c] = fmaf(bk, u[c], S[m][c]);
      L::settle(S[m]);
      *reinterpret_cast<vec*>(dst + m * kHeadV) = L::narrow(S[m]);
    }

    if (writer) {
      const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
      const float uc = s_v[t][wcol + c_mine] - w_c;
      a.out[(rho * a.H + h) * kHeadV + col0 + c_mine] = a.scale * fmaf(beta * s_qk[t], uc, p_c);
    }
  }
}

// ---------------------------------------------------------------------------
// Chained rows as one block on the matrix cores (kda_rows_mfma_kernel<T, CONV>).
//
// With gamma_t = a_0 ... a_t and E_ts = a_(s+1) ... a_t (per key channel)
// and Delta_t = beta_t u_t, a request's n rows unroll to
//   w_t  = w0_t + sum_{s<t} C_ts Delta_s,      w0_t = S0^T (gamma_t kn_t),
//   C_ts = sum_i kn_ti kn_si E_ts,i,           Delta_t = beta_t (v_t - w_t),
//   o_t  = scale (p0_t + sum_{s<=t} P_ts Delta_s),   p0_t = S0^T (gamma_t qn_t),
//   P_ts = sum_i qn_ti kn_si E_ts,i,           S_t = diag(a_t) S_(t-1) + kn_t Delta_t^T.
// The 2n column sums are one product of the stacked weights [16 x 128]
// (gamma_t kn_t, then gamma_t qn_t) with the initial state, a dense
// contraction over the key channels that runs on the matrix cores
// (v_mfma_f32_16x16x4_f32, fp32 operands and accumulation) and needs no
// exchange between the lanes of a wave.  The n x n couplings depend only on
// the row vectors.  Each column then needs a triangular solve, Delta_t row
// after row, and each row's snapshot is element-wise, so a wave writes row
// t's snapshot as soon as its Delta_t is known: no reduction and no barrier
// between rows, and the snapshot stores stream.
//
// Workgroup: (request, head, 64-column half), 4 waves (with the fused
// convolution a whole head: two halves of 4 waves).  Wave w of a half holds key
// rows 32 w .. 32 w + 31; lane (gq = lane / 16, li = lane % 16) holds rows
// 32 w + 8 gq + j (j < 8) and columns 4 li .. 4 li + 3 of the half.  Each
// state load or store instruction therefore covers whole rows of the half:
// 4 rows of 128 bytes (fp16) or 256 bytes (fp32).  In matrix-core step j,
// the B operand B[k][n] = S[32 w + 8 k + j][4 n + e] is exactly that
// register of lane (k, n), for each of the 4 column offsets e (4
// accumulators), and the A operand is W[m][32 w + 8 k + j] for row m = li
// of the stacked weights; D[m][n] accumulates the wave's share of the sums
// over K (lane (gq, li), register r: D[4 gq + r][li]).  The four waves'
// shares meet in LDS.
// ---------------------------------------------------------------------------
template <typename T>
struct Piece4;  // 4 consecutive columns of one state row
template <>
struct Piece4<float> {
  using vec = f4;
};
template <>
struct Piece4<_Float16> {
  using vec = h4;
};

constexpr int kMfmaBV = kMatrixBV;  // columns per half (per workgroup without the convolution)
constexpr int kMfmaWaves = kMatrixWaves4;  // waves per half of the 4-wave form
constexpr int kLdRow = kHeadK + 4;  // padded row stride of the [t][channel] LDS arrays

// The couplings P_ts (s <= t) and C_ts (s < t) for the two columns s = W and
// s = 7 - W of the n x n matrices: 16 values in all, for every W.  Lane l
// sums over its key channels 2 l and 2 l + 1; a reduce-scatter over the wave
// leaves each total in 4 lanes, one of which stores it.
template <int W>
__device__ __forceinline__ void coupling_pair(const float (*kn)[kLdRow], const float (*qn)[kLdRow],
                                              const float (*am)[kLdRow], int lane, float (*cP)[8],
                                              float (*cA)[8]) {
  constexpr int S0 = W, S1 = 7 - W;
  constexpr int N0P = 8 - S0, N0C = 7 - S0, N1P = 8 - S1;
  const int i0 = 2 * lane;
  float cv[16];
  int k = 0;
#pragma unroll
  for (int slot = 0; slot < 2; ++slot) {
    const int s = slot == 0 ? S0 : S1;
    const f2 ks = *reinterpret_cast<const f2*>(&kn[s][i0]);
    float P[8], C[8];
    float e0 = 1.0f, e1 = 1.0f;
#pragma unroll
    for (int t = s; t < 8; ++t) {
      if (t > s) {
        const f2 at = *reinterpret_cast<const f2*>(&am[t][i0]);
        e0 *= at[0];
        e1 *= at[1];
      }
      const float f0 = ks[0] * e0, f1 = ks[1] * e1;
      const f2 qt = *reinterpret_cast<const f2*>(&qn[t][i0]);
      P[t] = fmaf(qt[1], f1, qt[0] * f0);
      if (t > s) {
        const f2 kt = *reinterpret_cast<const f2*>(&kn[t][i0]);
        C[t] = fmaf(kt[1], f1, kt[0] * f0);
      }
    }
#pragma unroll
    for (int t = s; t < 8; ++t) cv[k++] = P[t];
#pragma unroll
    for (int t = s + 1; t < 8; ++t) cv[k++] = C[t];
  }
  float y[8], z[4], u[2], p[1];
  rs_stage<5>(cv, y, lane);
  rs_stage<4>(y, z, lane);
  rs_stage<3>(z, u, lane);
  rs_stage<2>(u, p, lane);
  float tot = p[0];
  tot += partner<1>(tot);
  tot += partner<0>(tot);
  // the value this lane holds: index 8 b2 + 4 b3 + 2 b4 + b5 of cv
  const int idx = ((lane >> 2) & 1) * 8 + ((lane >> 3) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 5) & 1);
  if ((lane & 3) == 0) {
    if (idx < N0P)
      cP[S0 + idx][S0] = tot;
    else if (idx < N0P + N0C)
      cA[S0 + 1 + (idx - N0P)][S0] = tot;
    else if (idx < N0P + N0C + N1P)
      cP[S1 + (idx - N0P - N0C)][S1] = tot;
    else
      cA[S1 + 1 + (idx - N0P - N0C - N1P)][S1] = tot;
  }
}

// CONV fuses the short convolution in front (as kda_decode_tile's CONV
// variant does): a workgroup then takes a whole head, two 64-column halves of
// 4 waves each, so that the convolution history it reads at the initial slot
// and rewrites at the rows' slots belongs to no other workgroup.
template <typename T, bool CONV>
__global__ __launch_bounds__(kWave * kMfmaWaves * (CONV ? 2 : 1)) void kda_rows_mfma_kernel(KDA_HOT_PARAMS, Args a) {
  const int init_stride = unpack_hot(a, hot_ids, hot_pool, hot_q, hot_k, hot_slots, hot_dims);
  using vec = typename Piece4<T>::vec;
  constexpr int TMAX = KDA_MAX_ROWS;
  constexpr int HALVES = CONV ? 2 : 1;        // 64-column halves per workgroup
  constexpr int NW = kMfmaWaves * HALVES;
  constexpr int BH = kMfmaBV;                 // columns per half
  constexpr int BV = BH * HALVES;             // columns per workgroup
  static_assert(TMAX == 8, "the stacked weights fill the 16 rows of the matrix-core operand");

  __shared__ __attribute__((aligned(16))) float s_kn[TMAX][kLdRow];
  __shared__ __attribute__((aligned(16))) float s_qn[TMAX][kLdRow];
  __shared__ __attribute__((aligned(16))) float s_a[TMAX][kLdRow];
  __shared__ __attribute__((aligned(16))) float s_gam[TMAX][kLdRow];
  __shared__ __attribute__((aligned(16))) float s_v[TMAX][BV];
  // [half][wave of the half][gq][column of the half] = D[4 gq + r]
  __shared__ __attribute__((aligned(16))) f4 s_part[HALVES][kMfmaWaves][4][BH];
  __shared__ __attribute__((aligned(16))) float s_cP[TMAX][TMAX];
  __shared__ __attribute__((aligned(16))) float s_cA[TMAX][TMAX];
  __shared__ __attribute__((aligned(16))) float s_beta[TMAX];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int half = wave / kMfmaWaves, rw = wave % kMfmaWaves;
  const int gq = lane / 16, li = lane % 16;

  const int tile = tile_of_block(blockIdx.x, hot_blocks);
  const int vt = tile % a.n_vt;
  const int rh = tile / a.n_vt;
  const int h = rh % a.H;
  const int r = rh / a.H;
  const int n_rows = a.n_rows;
  const int hcol = vt * BV + half * BH;  // the first column of this wave's half

  // both id loads are issued before either is waited for
  const int32_t init_slot = hot_init[static_cast<int64_t>(r) * init_stride];
  const int32_t* ids = a.slot_ids + static_cast<int64_t>(r) * n_rows;
  int32_t sid[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) sid[t] = t < n_rows ? ids[t] : 0;
  __builtin_amdgcn_sched_barrier(0);

  // Row inputs: wave w normalises rows w, w + NW, ... (a row past the last
  // re-reads the last one and is staged as zeros).
  int zero_v;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero_v));
  constexpr int TPW = TMAX / NW;
  f2 q2[TPW], k2[TPW];
  f4 v4[TPW];
  float braw[TPW];
  // fused convolution: the window win[t + m], m = 0..3 (3-entry history,
  // then this request's rows) of this lane's 2 q, 2 k and 4 v channels
  // (lanes < 32 hold the 128 v channels, the others repeat theirs), and
  // their taps
  constexpr int TC = CONV ? TPW : 1;
  f2 eq[TC][4], ek[TC][4];
  f4 ev[TC][4];
  uint32_t hwq[TC][4], hwk[TC][4];  // history entries as loaded (bf16 pairs)
  uint2 hwv[TC][4];
  f4 wq0, wq1, wk0, wk1, wv[4];
  const int64_t conv_c = static_cast<int64_t>(3) * a.H * kHeadK;  // channels per history entry
  const int64_t chq = static_cast<int64_t>(h) * kHeadK + 2 * lane;
  const int64_t chk = chq + static_cast<int64_t>(a.H) * kHeadK;
  const int64_t chv = static_cast<int64_t>(2 * a.H + h) * kHeadK + 4 * (CONV ? lane % (BV / 4) : lane);
  const bool conv_vl = lane < BV / 4;
  if constexpr (!CONV) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = min(wave + j * NW, n_rows - 1);
      const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
      const int64_t off = (rho * a.H + h) * kHeadK;
      q2[j] = reinterpret_cast<const f2*>(a.q + off)[lane];
      k2[j] = reinterpret_cast<const f2*>(a.k + off)[lane];
      v4[j] = *reinterpret_cast<const f4*>(a.v + off + vt * BV + 4 * (lane % (BV / 4)));
      braw[j] = a.b[rho * a.H + h + zero_v];
    }
  } else {
    // the history is read at the initial slot (slot 0 for a request with a
    // bad id, which is skipped below, so every address stays valid)
    bool ok0 = init_slot >= 0 && init_slot < a.n_slots;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) ok0 = ok0 && sid[t] >= 0 && sid[t] < a.n_slots;
    const int64_t hslot = ok0 ? init_slot : 0;
#pragma unroll
    for (int j = 0; j < TPW; ++j) braw[j] = 0.0f;
    if (wave < n_rows) {
      wq0 = *reinterpret_cast<const f4*>(a.conv_w + chq * 4);
      wq1 = *reinterpret_cast<const f4*>(a.conv_w + chq * 4 + 4);
      wk0 = *reinterpret_cast<const f4*>(a.conv_w + chk * 4);
      wk1 = *reinterpret_cast<const f4*>(a.conv_w + chk * 4 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) wv[e] = *reinterpret_cast<const f4*>(a.conv_w + (chv + e) * 4);
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wave + j * NW;
      if (t < n_rows) {
        const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int pos = t + m;  // window index
          if (pos < 3) {
            const uint16_t* hb = a.conv_pool + (hslot * 3 + pos) * conv_c;
            hwq[j][m] = *reinterpret_cast<const uint32_t*>(hb + chq);
            hwk[j][m] = *reinterpret_cast<const uint32_t*>(hb + chk);
            hwv[j][m] = *reinterpret_cast<const uint2*>(hb + chv);
          } else {
            const float* xr = a.x + (static_cast<int64_t>(r) * n_rows + (pos - 3)) * conv_c;
            eq[j][m] = *reinterpret_cast<const f2*>(xr + chq);
            ek[j][m] = *reinterpret_cast<const f2*>(xr + chk);
            ev[j][m] = *reinterpret_cast<const f4*>(xr + chv);
          }
        }
        braw[j] = a.b[rho * a.H + h];
      }
    }
  }
  // Decays per key channel: threads 0..127 each take one channel through all
  // rows (the cumulative products need every row).
  float graw[TMAX];
  const int chan = threadIdx.x % kHeadK;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    const int tt = min(t, n_rows - 1);
    const int64_t rho = static_cast<int64_t>(r) * n_rows + tt;
    graw[t] = a.g[(rho * a.H + h) * kHeadK + chan];
  }
  __builtin_amdgcn_sched_barrier(0);

  bool ids_ok = init_slot >= 0 && init_slot < a.n_slots;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) ids_ok = ids_ok && sid[t] >= 0 && sid[t] < a.n_slots;

  // The initial state: rows 32 rw + 8 gq + j, columns 4 li .. 4 li + 3 of
  // the wave's half.
  const int64_t head_elems = static_cast<int64_t>(kHeadK) * kHeadV;
  const int64_t slot_elems = static_cast<int64_t>(a.H) * head_elems;
  const int row0 = 32 * rw + 8 * gq;
  const int64_t lane_off = h * head_elems + static_cast<int64_t>(row0) * kHeadV + hcol + 4 * li;
  T* const pool = static_cast<T*>(a.pool);
  vec raw[8];
  {
    const T* src = pool + static_cast<int64_t>(ids_ok ? init_slot : 0) * slot_elems + lane_off;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      raw[j] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(src + j * kHeadV));
  }
  __builtin_amdgcn_sched_barrier(0);

  // -- fused convolution: y_t = silu(sum_m w_m win[t + m]) --------------------
  f2 hq[TC][3], hk[TC][3];  // the history each row's snapshot keeps (entries t+1 .. t+3)
  f4 hv[TC][3];
  if constexpr (CONV) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wave + j * NW;
      q2[j] = f2{0.0f, 0.0f};
      k2[j] = f2{0.0f, 0.0f};
      v4[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      if (t < n_rows) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (t + m < 3) {
            eq[j][m] = bf16_x2(hwq[j][m]);
            ek[j][m] = bf16_x2(hwk[j][m]);
            ev[j][m] = bf16_x4(hwv[j][m]);
          }
        }
        float sq0 = 0.0f, sq1 = 0.0f, sk0 = 0.0f, sk1 = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          sq0 = fmaf(wq0[m], eq[j][m][0], sq0);
          sq1 = fmaf(wq1[m], eq[j][m][1], sq1);
          sk0 = fmaf(wk0[m], ek[j][m][0], sk0);
          sk1 = fmaf(wk1[m], ek[j][m][1], sk1);
        }
        q2[j] = f2{silu(sq0), silu(sq1)};
        k2[j] = f2{silu(sk0), silu(sk1)};
        f4 yv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sv = 0.0f;
#pragma unroll
          for (int m = 0; m < 4; ++m) sv = fmaf(wv[e][m], ev[j][m][e], sv);
          yv[e] = silu(sv);
        }
        v4[j] = yv;
#pragma unroll
        for (int e = 0; e < 3; ++e) {
          hq[j][e] = eq[j][e + 1];
          hk[j][e] = ek[j][e + 1];
          hv[j][e] = ev[j][e + 1];
        }
      }
    }
  }

#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = wave + j * NW;
    const bool live = t < n_rows;
    const float sq = wave_sum(fmaf(q2[j][1], q2[j][1], q2[j][0] * q2[j][0]));
    const float sk = wave_sum(fmaf(k2[j][1], k2[j][1], k2[j][0] * k2[j][0]));
    const float rq = live ? 1.0f / sqrtf(sq + 1e-6f) : 0.0f;
    const float rk = live ? 1.0f / sqrtf(sk + 1e-6f) : 0.0f;
    *reinterpret_cast<f2*>(&s_qn[t][2 * lane]) = f2{q2[j][0] * rq, q2[j][1] * rq};
    *reinterpret_cast<f2*>(&s_kn[t][2 * lane]) = f2{k2[j][0] * rk, k2[j][1] * rk};
    if (lane < BV / 4) *reinterpret_cast<f4*>(&s_v[t][4 * lane]) = live ? v4[j] : f4{0, 0, 0, 0};
    if (lane == 0) s_beta[t] = live ? 1.0f / (1.0f + expf(-braw[j])) : 0.0f;
  }
  if (threadIdx.x < kHeadK) {
    float gam = 1.0f;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const float at = t < n_rows ? decay_of(graw[t], CONV && a.g_raw != 0) : 0.0f;
      gam *= at;
      s_a[t][chan] = at;
      s_gam[t][chan] = gam;
    }
  }
  if (!ids_ok) {  // uniform over the workgroup: no wave waits at the barrier
    if (wave == 0 && lane < BV / 4) {
      for (int t = 0; t < n_rows; ++t) {
        const int64_t rho = static_cast<int64_t>(r) * n_rows + t;
        *reinterpret_cast<f4*>(a.out + (rho * a.H + h) * kHeadV + vt * BV + 4 * lane) =
            f4{NAN, NAN, NAN, NAN};
      }
    }
    return;
  }
  __syncthreads();

  if constexpr (CONV) {
    // every wave has read the history: the rows' snapshots may now overwrite
    // it (row 0's slot is the initial slot of an in-place launch)
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wave + j * NW;
      if (t < n_rows) {
        int32_t st = sid[0];
#pragma unroll
        for (int u = 1; u < TMAX; ++u)
          if (u == t) st = sid[u];
#pragma unroll
        for (int e = 0; e < 3; ++e) {
          uint16_t* hb = a.conv_pool + (static_cast<int64_t>(st) * 3 + e) * conv_c;
          *reinterpret_cast<uint32_t*>(hb + chq) = bf16_pack(hq[j][e][0], hq[j][e][1]);
          *reinterpret_cast<uint32_t*>(hb + chk) = bf16_pack(hk[j][e][0], hk[j][e][1]);
          if (conv_vl)
            *reinterpret_cast<uint2*>(hb + chv) = uint2{bf16_pack(hv[j][e][0], hv[j][e][1]),
                                                         bf16_pack(hv[j][e][2], hv[j][e][3])};
        }
      }
    }
  }

  // fp32 state
  float S[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) S[j][e] = static_cast<float>(raw[j][e]);

  // (1) the wave's share of w0 and p0 on the matrix cores, then (2) the
  // couplings on the vector units (on MI355X the fp32 products and the
  // vector instructions of one wave did not overlap: interleaving them
  // measured no faster)
  {
    const int tw = li & 7;
    const float* wsrc = li < 8 ? &s_kn[tw][row0] : &s_qn[tw][row0];
    float x[8], gm[8];
    lds_rows<8>(wsrc, x);
    lds_rows<8>(&s_gam[tw][row0], gm);
    f4 acc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wj = gm[j] * x[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(wj, S[j][e], acc[e], 0, 0, 0);
    }
    if (half == 0) {
      switch (rw) {  // wave-uniform: each wave of the first half takes two columns of the couplings
        case 0: coupling_pair<0>(s_kn, s_qn, s_a, lane, s_cP, s_cA); break;
        case 1: coupling_pair<1>(s_kn, s_qn, s_a, lane, s_cP, s_cA); break;
        case 2: coupling_pair<2>(s_kn, s_qn, s_a, lane, s_cP, s_cA); break;
        default: coupling_pair<3>(s_kn, s_qn, s_a, lane, s_cP, s_cA); break;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s_part[half][rw][gq][4 * li + e] = acc[e];
  }
  __syncthreads();

  // (3) and (4): every wave solves the 64 columns of its half (lane l:
  // column l of the half) and
  // writes row t's snapshot as soon as Delta_t is known, so the snapshot
  // stores begin after the first step of the solve.  The couplings and beta
  // are the same for every column: each lane reads one of them and the
  // solve takes them with readlane.  (The empty volatile asm keeps those
  // reads in every lane; a read sunk into a branch that only some lanes take
  // would leave the others' registers unloaded.)
  float cA_l = s_cA[lane >> 3][lane & 7];
  float cP_l = s_cP[lane >> 3][lane & 7];
  float bt_l = s_beta[lane & 7];
  asm volatile("" : "+v"(cA_l), "+v"(cP_l), "+v"(bt_l));
  auto cA = [&](int t, int s2) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cA_l), 8 * t + s2)); };
  auto cP = [&](int t, int s2) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cP_l), 8 * t + s2)); };
  float tot[16], vv[TMAX];
  {
    f4 part[kMfmaWaves][4];
#pragma unroll
    for (int x = 0; x < kMfmaWaves; ++x)
#pragma unroll
      for (int g = 0; g < 4; ++g) part[x][g] = s_part[half][x][g][lane];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) vv[t] = s_v[t][half * BH + lane];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        tot[4 * g + e] = (part[0][g][e] + part[1][g][e]) + (part[2][g][e] + part[3][g][e]);
  }
  float* op = a.out + (static_cast<int64_t>(r) * n_rows * a.H + h) * kHeadV + hcol + lane;
  const int64_t o_row = static_cast<int64_t>(a.H) * kHeadV;
  float dl[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t >= n_rows) break;
    float d = vv[t] - tot[t];
#pragma unroll
    for (int s2 = 0; s2 < t; ++s2) d = fmaf(-cA(t, s2), dl[s2], d);
    dl[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bt_l), t)) * d;
    if ((t & 3) == rw) {  // this wave writes row t's outputs of its half
      float o = tot[8 + t];
#pragma unroll
      for (int s2 = 0; s2 <= t; ++s2) o = fmaf(cP(t, s2), dl[s2], o);
      op[t * o_row] = a.scale * o;
    }
    // Delta_t of the lane's snapshot columns 4 li .. 4 li + 3
    float dc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dc[e] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * li + e), __float_as_int(dl[t])));
    float kn[8], am[8];
    lds_rows<8>(&s_kn[t][row0], kn);
    lds_rows<8>(&s_a[t][row0], am);
    T* dst = pool + static_cast<int64_t>(sid[t]) * slot_elems + lane_off;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      vec o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s1 = fmaf(kn[j], dc[e], am[j] * S[j][e]);
        asm("" : "+v"(s1));  // a rounded fp32 value before any narrowing
        S[j][e] = s1;
        o[e] = static_cast<T>(s1);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<vec*>(dst + j * kHeadV));
    }
  }
}

// ---------------------------------------------------------------------------
// The same block form with K split over 8 waves (kda_rows_mfma8_kernel<T,
// FORM>, the default layout of chained rows on the matrix cores).  Workgroup
// = (request, head, 64-column half), 8 waves: wave w holds key rows 16 w ..
// 16 w + 15, lane (gq, li) rows 16 w + 4 gq + j (j < 4) and columns 4 li ..
// 4 li + 3 of the half, so each state load or store instruction still covers
// whole 128-byte (fp16) or 256-byte (fp32) rows of the half.  Against the
// 4-wave form, each wave runs half the matrix-core steps (16 instead of 32 of
// v_mfma_f32_16x16x4_f32) and half the snapshot work per row, and two waves
// share each SIMD, so one wave's vector work runs while the other's products
// or stores are in flight.  Each wave loads and normalises one row of the
// request (one 8-byte q, k and g vector per lane): the prologue issues 4 row
// loads per wave instead of 22.  The eight waves' partial column sums meet in
// LDS in two steps (each thread sums one 8-byte piece over the waves, then
// every lane reads the 16 totals of its column), which keeps the LDS traffic
// of the 4-wave form.
//
// Three forms:
//  kRowsPlain     the decode step as described.
//  kRowsConvHead  the short convolution fused in front, a whole head per
//                 workgroup: two 64-column halves of 8 waves, 16 waves in
//                 all.  Wave w of each half takes row w: in half 0 its q,
//                 in half 1 its k (2 channels per lane), and in both its
//                 half's 64 v channels (one per lane), so the 16 waves share
//                 the convolution's loads and arithmetic evenly; half 0
//                 stages beta, half 1 the decays.  One workgroup owns all of
//                 a head's history, so the history it reads at the initial
//                 slot may be rewritten at row 0's slot with a barrier
//                 between the two.
//  kRowsConvHalf  the convolution fused in front, 64-column halves as in
//                 the plain form (twice the workgroups: on MI355X a CU's
//                 store throughput, not the HBM, bounds the whole-head
//                 form's snapshots when a launch has fewer heads than CUs).
//                 Both halves of a head form its q and k (wave w: row w, 2
//                 channels of each per lane) and their own v channels.  The
//                 history is written by channel owner: v by its half, q by
//                 half 0, k by half 1, except at a row whose slot is the
//                 initial slot (at most one per request, slots being
//                 distinct): both halves read q and k there, so neither may
//                 overwrite them before the other has read them.  That row's
//                 wave in each half counts its half's arrival on the
//                 request's and head's counter after the third barrier (the
//                 workgroup's history reads were done before the first);
//                 the half that arrives second (odd count before its
//                 increment) writes that row's q and k history at the end.  No wave
//                 waits on another workgroup.  Each launch adds 2 per such
//                 counter, so counters that start even stay even.
// ---------------------------------------------------------------------------
constexpr int kMfma8Waves = 8;  // waves per 64-column half
constexpr int kRowsPlain = 0, kRowsConvHead = 1, kRowsConvHalf = 2;

template <typename T, int FORM>
__global__ __launch_bounds__(kWave * kMfma8Waves * (FORM == kRowsConvHead ? 2 : 1)) void kda_rows_mfma8_kernel(
    KDA_HOT_PARAMS, Args a) {
  const int init_stride = unpack_hot(a, hot_ids, hot_pool, hot_q, hot_k, hot_slots, hot_dims);
  using vec = typename Piece4<T>::vec;
  constexpr bool CONV = FORM != kRowsPlain;
  constexpr bool HEAD = FORM == kRowsConvHead;
  constexpr int TMAX = KDA_MAX_ROWS;
  constexpr int HALVES = HEAD ? 2 : 1;  // 64-column halves per workgroup
  constexpr int NW = kMfma8Waves;       // waves per half
  constexpr int BH = kMfmaBV;           // columns per half
  constexpr int BV = BH * HALVES;       // columns per workgroup
  constexpr int RPW = kHeadK / NW;      // key rows per wave
  constexpr int J = RPW / 4;            // key rows per lane (= matrix-core steps)
  static_assert(TMAX == NW, "one row of the request per wave of a half");

  __shared__ __attribute__((aligned(16))) float s_kn[TMAX][kLdRow];
  __shared__ __attribute__((aligned(16))) float s_qn[TMAX][kLdRow];
  __shared__ __attribute__((aligned(16))) float s_a[TMAX][kLdRow];
  __shared__ __attribute__((aligned(16))) float s_v[TMAX][BV];
  // [half][wave of the half][gq][column of the half] = the wave's D[4 gq + r][column], r = 0..3
  __shared__ __attribute__((aligned(16))) f4 s_part[HALVES][NW][4][BH];
  // [half][gq][column of the half] = the totals over the half's waves
  __shared__ __attribute__((aligned(16))) f4 s_tot[HALVES][4][BH];
  __shared__ __attribute__((aligned(16))) float s_cP[TMAX][TMAX];
  __shared__ __attribute__((aligned(16))) float s_cA[TMAX][TMAX];
  __shared__ __attribute__((aligned(16))) float s_beta[TMAX];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int half = HEAD ? wave / NW : 0;
  const int rw = HEAD ? wave % NW : wave;  // the wave's place in its half, and its row
  const int gq = lane / 16, li = lane % 16;
  const int H = a.H;
  const int n_rows = a.n_rows;

  const int tile = tile_of_block(blockIdx.x, hot_blocks);
  const int vt = tile % (kHeadV / BV);
  const int rh = tile / (kHeadV / BV);
  const int h = rh % H;
  const int r = rh / H;
  const int hcol = vt * BV + half * BH;  // the first column of this wave's half

  // both id loads are issued before either is waited for
  const int32_t init_slot = hot_init[static_cast<int64_t>(r) * init_stride];
  const int32_t* ids = a.slot_ids + static_cast<int64_t>(r) * n_rows;
  int32_t sid[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) sid[t] = t < n_rows ? ids[t] : 0;
  __builtin_amdgcn_sched_barrier(0);

  // This wave's row of the request (a wave past the last row re-reads the
  // last one and stages zeros).
  int zero_v;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero_v));
  const int trow = min(rw, n_rows - 1);
  const int64_t rho = static_cast<int64_t>(r) * n_rows + trow;
  const int64_t roff = (rho * H + h) * kHeadK;
  f2 q2, k2, g2;
  float v1, braw;
  // fused convolution: the window win[trow + m], m = 0..3 (the 3-entry
  // history, then this request's rows) of the lane's 2 q channels (eq; the
  // whole-head form: q or k by half), 2 k channels (ek; halves form only)
  // and its v channel, and their taps
  f2 eq[4], ek[4];
  float ev[4];
  // both candidates of each window entry as loaded: the history's (bf16) and
  // the request row's (fp32)
  uint32_t hwq[4], hwk[4], hwv[4];
  f2 xwq[4], xwk[4];
  float xwv[4];
  f4 wq0, wq1, wk0, wk1, wv;
  const int64_t conv_c = static_cast<int64_t>(3) * H * kHeadK;  // channels per history entry
  const int64_t chq = static_cast<int64_t>(half * H + h) * kHeadK + 2 * lane;
  const int64_t chk = static_cast<int64_t>(H + h) * kHeadK + 2 * lane;
  const int64_t chv = static_cast<int64_t>(2 * H + h) * kHeadK + hcol + lane;
  if constexpr (!CONV) {
    q2 = reinterpret_cast<const f2*>(a.q + roff)[lane];
    k2 = reinterpret_cast<const f2*>(a.k + roff)[lane];
    g2 = reinterpret_cast<const f2*>(a.g + roff)[lane];
    v1 = a.v[roff + hcol + lane];
    braw = a.b[rho * H + h + zero_v];
  } else {
    // the history is read at the initial slot (slot 0 for a request with a
    // bad id, which is skipped below, so every address stays valid)
    bool ok0 = init_slot >= 0 && init_slot < a.n_slots;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) ok0 = ok0 && sid[t] >= 0 && sid[t] < a.n_slots;
    const int64_t hslot = ok0 ? init_slot : 0;
    wq0 = *reinterpret_cast<const f4*>(a.conv_w + chq * 4);
    wq1 = *reinterpret_cast<const f4*>(a.conv_w + chq * 4 + 4);
    if constexpr (!HEAD) {
      wk0 = *reinterpret_cast<const f4*>(a.conv_w + chk * 4);
      wk1 = *reinterpret_cast<const f4*>(a.conv_w + chk * 4 + 4);
    }
    wv = *reinterpret_cast<const f4*>(a.conv_w + chv * 4);
    // Entry m of the window is history entry trow + m while that is below 3,
    // else row trow + m - 3 of the request.  Both are loaded (the one not
    // taken from an in-range place: history entry 2, the request's row 0) and
    // the entry is chosen once the state tile's loads are issued, so no load
    // sits behind a branch whose arms the compiler would join by waiting.
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int pos = trow + m;  // window index (wave-uniform)
      const uint16_t* hb = a.conv_pool + (hslot * 3 + min(pos, 2)) * conv_c;
      const float* xr = a.x + (static_cast<int64_t>(r) * n_rows + max(pos - 3, 0)) * conv_c;
      hwq[m] = *reinterpret_cast<const uint32_t*>(hb + chq);
      xwq[m] = *reinterpret_cast<const f2*>(xr + chq);
      if constexpr (!HEAD) {
        hwk[m] = *reinterpret_cast<const uint32_t*>(hb + chk);
        xwk[m] = *reinterpret_cast<const f2*>(xr + chk);
      }
      hwv[m] = hb[chv];
      xwv[m] = xr[chv];
    }
    if (!HEAD || half == 0) braw = a.b[rho * H + h + zero_v];
    if (!HEAD || half == 1) g2 = reinterpret_cast<const f2*>(a.g + roff)[lane];
  }
  __builtin_amdgcn_sched_barrier(0);

  bool ids_ok = init_slot >= 0 && init_slot < a.n_slots;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) ids_ok = ids_ok && sid[t] >= 0 && sid[t] < a.n_slots;

  // The initial state: rows 16 rw + 4 gq + j, columns 4 li .. 4 li + 3 of the half.
  const int64_t head_elems = static_cast<int64_t>(kHeadK) * kHeadV;
  const int64_t slot_elems = static_cast<int64_t>(H) * head_elems;
  const int row0 = RPW * rw + J * gq;
  const int64_t lane_off = h * head_elems + static_cast<int64_t>(row0) * kHeadV + hcol + 4 * li;
  T* const pool = static_cast<T*>(a.pool);
  vec raw[J];
  {
    const T* src = pool + static_cast<int64_t>(ids_ok ? init_slot : 0) * slot_elems + lane_off;
#pragma unroll
    for (int j = 0; j < J; ++j)
      raw[j] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(src + j * kHeadV));
  }
  __builtin_amdgcn_sched_barrier(0);

  const bool live = rw < n_rows;
  {
    if constexpr (CONV) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bool hist = trow + m < 3;
        eq[m] = hist ? bf16_x2(hwq[m]) : xwq[m];
        if constexpr (!HEAD) ek[m] = hist ? bf16_x2(hwk[m]) : xwk[m];
        ev[m] = hist ? bf16_lo(hwv[m]) : xwv[m];
      }
      // y = silu(sum_m w_m win[trow + m]), the sum taken in window order
      float sq0 = 0.0f, sq1 = 0.0f, sk0 = 0.0f, sk1 = 0.0f, sv = 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        sq0 = fmaf(wq0[m], eq[m][0], sq0);
        sq1 = fmaf(wq1[m], eq[m][1], sq1);
        if constexpr (!HEAD) {
          sk0 = fmaf(wk0[m], ek[m][0], sk0);
          sk1 = fmaf(wk1[m], ek[m][1], sk1);
        }
        sv = fmaf(wv[m], ev[m], sv);
      }
      q2 = f2{silu(sq0), silu(sq1)};
      if constexpr (!HEAD) k2 = f2{silu(sk0), silu(sk1)};
      v1 = silu(sv);
    }
    if constexpr (!HEAD) {
      const float sq = wave_sum(fmaf(q2[1], q2[1], q2[0] * q2[0]));
      const float sk = wave_sum(fmaf(k2[1], k2[1], k2[0] * k2[0]));
      const float rq = live ? 1.0f / sqrtf(sq + 1e-6f) : 0.0f;
      const float rk = live ? 1.0f / sqrtf(sk + 1e-6f) : 0.0f;
      *reinterpret_cast<f2*>(&s_qn[rw][2 * lane]) = f2{q2[0] * rq, q2[1] * rq};
      *reinterpret_cast<f2*>(&s_kn[rw][2 * lane]) = f2{k2[0] * rk, k2[1] * rk};
      const bool raw = CONV && a.g_raw != 0;
      *reinterpret_cast<f2*>(&s_a[rw][2 * lane]) =
          live ? f2{decay_of(g2[0], raw), decay_of(g2[1], raw)} : f2{0.0f, 0.0f};
      s_v[rw][lane] = live ? v1 : 0.0f;
      if (lane == 0) s_beta[rw] = live ? 1.0f / (1.0f + expf(-braw)) : 0.0f;
    } else {
      // half 0 normalises q, half 1 k
      const float ss = wave_sum(fmaf(q2[1], q2[1], q2[0] * q2[0]));
      const float rn = live ? 1.0f / sqrtf(ss + 1e-6f) : 0.0f;
      float* xn = half == 0 ? &s_qn[rw][2 * lane] : &s_kn[rw][2 * lane];
      *reinterpret_cast<f2*>(xn) = f2{q2[0] * rn, q2[1] * rn};
      s_v[rw][half * BH + lane] = live ? v1 : 0.0f;
      if (half == 0) {
        if (lane == 0) s_beta[rw] = live ? 1.0f / (1.0f + expf(-braw)) : 0.0f;
      } else {
        const bool raw = a.g_raw != 0;
        *reinterpret_cast<f2*>(&s_a[rw][2 * lane]) =
            live ? f2{decay_of(g2[0], raw), decay_of(g2[1], raw)} : f2{0.0f, 0.0f};
      }
    }
  }
  if (!ids_ok) {  // uniform over the workgroup: no wave waits at the barrier
    if (live) {
      const int64_t orow = static_cast<int64_t>(r) * n_rows + rw;
      a.out[(orow * H + h) * kHeadV + hcol + lane] = NAN;
    }
    return;
  }
  __syncthreads();

  // -- history snapshots: row t keeps win[t + 1 .. t + 3] ----------------------
  // After the first barrier every wave of the workgroup has read the history
  // it needs (its values are in LDS); the stores are issued after the third
  // barrier: a store issued earlier would hold up the waits for the state
  // loads before the products (loads and stores share one counter).
  int32_t st = sid[0];  // this wave's row's slot
#pragma unroll
  for (int u = 1; u < TMAX; ++u)
    if (u == rw) st = sid[u];
  uint16_t* const hrow = CONV ? a.conv_pool + static_cast<int64_t>(st) * 3 * conv_c : nullptr;
  auto store_pair = [&](int64_t ch, const f2 (&e)[4]) {
#pragma unroll
    for (int m = 0; m < 3; ++m)
      *reinterpret_cast<uint32_t*>(hrow + m * conv_c + ch) = bf16_pack(e[m + 1][0], e[m + 1][1]);
  };
  // the initial slot's row, if any (kRowsConvHalf): its q and k history
  // waits for the pair counter
  const bool handover = !HEAD && CONV && live && st == init_slot;

  // couplings (waves 0..3: two columns of the n x n matrices each), then
  // this wave's share of w0 and p0 on the matrix cores
  switch (wave) {  // wave-uniform
    case 0: coupling_pair<0>(s_kn, s_qn, s_a, lane, s_cP, s_cA); break;
    case 1: coupling_pair<1>(s_kn, s_qn, s_a, lane, s_cP, s_cA); break;
    case 2: coupling_pair<2>(s_kn, s_qn, s_a, lane, s_cP, s_cA); break;
    case 3: coupling_pair<3>(s_kn, s_qn, s_a, lane, s_cP, s_cA); break;
    default: break;
  }
  float S[J][4];
  {
    // weight row li: gamma_t kn_t (li < 8) or gamma_t qn_t, t = li mod 8,
    // with gamma_t = a_0 ... a_t multiplied in row order
    const int tw = li & 7;
    float x[J], gm[J];
    lds_rows<J>(li < 8 ? &s_kn[tw][row0] : &s_qn[tw][row0], x);
#pragma unroll
    for (int j = 0; j < J; ++j) gm[j] = 1.0f;
#pragma unroll
    for (int s2 = 0; s2 < TMAX; ++s2) {
      float as[J];
      lds_rows<J>(&s_a[s2][row0], as);
#pragma unroll
      for (int j = 0; j < J; ++j) gm[j] = s2 <= tw ? gm[j] * as[j] : gm[j];
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[j][e] = static_cast<float>(raw[j][e]);
    f4 acc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float wj = gm[j] * x[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(wj, S[j][e], acc[e], 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s_part[half][rw][gq][4 * li + e] = acc[e];
  }
  __syncthreads();
  // totals over a half's waves: thread i of the half sums the 8-byte piece
  // (i mod 2) of entry i / 2 of the half's [4][64] f4 array, in a fixed tree
  // order
  {
    const int ti = HEAD ? threadIdx.x % (kWave * NW) : threadIdx.x;
    const int ent = ti >> 1, pc = ti & 1;
    const int eg = ent / BH, ec = ent % BH;
    f2 x[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) x[w] = reinterpret_cast<const f2*>(&s_part[half][w][eg][ec])[pc];
    const f2 t01 = x[0] + x[1], t23 = x[2] + x[3], t45 = x[4] + x[5], t67 = x[6] + x[7];
    reinterpret_cast<f2*>(&s_tot[half][eg][ec])[pc] = (t01 + t23) + (t45 + t67);
  }
  __syncthreads();

  // The in-place row's pair-counter increment (its result is used at the
  // end, where the second half writes the q and k history).
  uint32_t arrival = 0;
  if constexpr (CONV && !HEAD) {
    if (handover && lane == 0)
      arrival = __hip_atomic_fetch_add(a.pair_counts + static_cast<int64_t>(r) * H + h, 1u,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if constexpr (CONV) {
    if (live) {
#pragma unroll
      for (int m = 0; m < 3; ++m) hrow[m * conv_c + chv] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(ev[m + 1]));
      if constexpr (HEAD) {
        store_pair(chq, eq);  // q (half 0) or k (half 1)
      } else if (!handover) {
        if (vt == 0)
          store_pair(chq, eq);
        else
          store_pair(chk, ek);
      }
    }
  }

  // Every wave solves the 64 columns of its half (lane l: column l) and
  // writes row t's snapshot as soon as Delta_t is known; wave t of the half
  // writes row t's outputs.  The couplings and beta are the same for every
  // column: each lane reads one and the solve takes them with readlane (the
  // empty volatile asm keeps those reads in every lane).
  float cA_l = s_cA[lane >> 3][lane & 7];
  float cP_l = s_cP[lane >> 3][lane & 7];
  float bt_l = s_beta[lane & 7];
  asm volatile("" : "+v"(cA_l), "+v"(cP_l), "+v"(bt_l));
  auto cA = [&](int t, int s2) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cA_l), 8 * t + s2)); };
  auto cP = [&](int t, int s2) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cP_l), 8 * t + s2)); };
  float tot[16], vv[TMAX];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const f4 x = s_tot[half][gi][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) tot[4 * gi + e] = x[e];
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) vv[t] = s_v[t][half * BH + lane];
  float* op = a.out + (static_cast<int64_t>(r) * n_rows * H + h) * kHeadV + hcol + lane;
  const int64_t o_row = static_cast<int64_t>(H) * kHeadV;
  float dl[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t >= n_rows) break;
    float d = vv[t] - tot[t];
#pragma unroll
    for (int s2 = 0; s2 < t; ++s2) d = fmaf(-cA(t, s2), dl[s2], d);
    dl[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bt_l), t)) * d;
    if (t == rw) {  // this wave writes row t's outputs of the half
      float o = tot[8 + t];
#pragma unroll
      for (int s2 = 0; s2 <= t; ++s2) o = fmaf(cP(t, s2), dl[s2], o);
      op[t * o_row] = a.scale * o;
    }
    // Delta_t of the lane's snapshot columns 4 li .. 4 li + 3
    float dc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dc[e] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * li + e), __float_as_int(dl[t])));
    float kn[J], am[J];
    lds_rows<J>(&s_kn[t][row0], kn);
    lds_rows<J>(&s_a[t][row0], am);
    T* dst = pool + static_cast<int64_t>(sid[t]) * slot_elems + lane_off;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      vec o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s1 = fmaf(kn[j], dc[e], am[j] * S[j][e]);
        asm("" : "+v"(s1));  // a rounded fp32 value before any narrowing
        S[j][e] = s1;
        o[e] = static_cast<T>(s1);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<vec*>(dst + j * kHeadV));
    }
  }

  // The initial slot's row: the half that arrives second on the pair
  // counter writes its q and k history.  What must be ordered is the first
  // half's history reads before the second half's history stores, and
  // nothing else: every read of this workgroup returned its data before the
  // first barrier (the values are in LDS), the increment is issued after the
  // third (and read back only here, so that no wave waits for it earlier)
  // and performed at device scope, and the second half's stores depend on
  // the value its increment returns.  The increment is therefore relaxed:
  // an agent-scope release would also write back this XCD's L2
  // (buffer_wbl2), which measured 14.2 against 10.9 us for 8 requests x 8
  // rows and 58 against 24 us for 48 x 2 (fp16), for stores no other
  // workgroup reads.
  if constexpr (CONV && !HEAD) {
    if (handover && (__builtin_amdgcn_readlane(static_cast<int>(arrival), 0) & 1) != 0) {
      store_pair(chq, eq);
      store_pair(chk, ek);
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming copy used to calibrate bandwidth and byte counters: one 16-byte
// vector per thread, consecutive threads on consecutive vectors (the copy
// form that measured fastest on MI355X, ahead of grid-stride loops).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kda_copy_probe_kernel(const f4* __restrict__ src,
                                                             f4* __restrict__ dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// Whole-slot copies (checkpoint flush / load): grid.y = pair, grid.x covers
// the slot's bytes, one 16-byte vector per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kda_state_copy_kernel(
    char* __restrict__ pool, const int32_t* __restrict__ src_ids, const int32_t* __restrict__ dst_ids,
    int32_t n_slots, int64_t slot_vecs) {
  const int32_t s = src_ids[blockIdx.y];
  const int32_t d = dst_ids[blockIdx.y];
  if (s < 0 || s >= n_slots || d < 0 || d >= n_slots) return;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= slot_vecs) return;
  const f4* src = reinterpret_cast<const f4*>(pool) + s * slot_vecs;
  f4* dst = reinterpret_cast<f4*>(pool) + d * slot_vecs;
  __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// The preloaded leading arguments of a launch (see KDA_HOT_PARAMS).
static Hot hot_of(const Args& a, int32_t blocks) {
  Hot h;
  h.ids = a.slot_ids;
  h.init = a.init_slot_ids != nullptr ? a.init_slot_ids : a.slot_ids;
  h.pool = a.pool;
  h.q = a.q;
  h.k = a.k;
  h.blocks = blocks;
  h.slots = a.n_slots;
  const int32_t stride = a.init_slot_ids != nullptr ? 1 : a.n_rows;
  h.dims = a.H | (a.n_vt << 16) | (a.n_rows << 20) | (stride << 24);
  return h;
}

template <typename T, int LPR, int NW>
static hipError_t launch_tile(const Args& a, int32_t blocks, hipStream_t stream) {
  const Hot h = hot_of(a, blocks);
  if (a.n_rows == 1)
    hipLaunchKernelGGL((kda_decode_tile<T, LPR, NW, false, false, false>), dim3(blocks),
                       dim3(kWave * NW), 0, stream, KDA_HOT_ARGS(h), a);
  else if (a.rows_block) {
    // not instantiated for the shapes resolve_shape refuses (block_supported)
    if constexpr (!std::is_same_v<T, _Float16> || NW > 1)
      hipLaunchKernelGGL((kda_decode_tile<T, LPR, NW, true, false, true>), dim3(blocks),
                         dim3(kWave * NW), 0, stream, KDA_HOT_ARGS(h), a);
    else
      return hipErrorInvalidValue;  // unreachable: shapes are checked first
  } else
    hipLaunchKernelGGL((kda_decode_tile<T, LPR, NW, true, false, false>), dim3(blocks),
                       dim3(kWave * NW), 0, stream, KDA_HOT_ARGS(h), a);
  return hipGetLastError();
}

// Fused-convolution launches: whole-head tiles (32 fp32 / 16 fp16 lanes per
// row), 2, 4 or 8 waves.
template <typename T, int LPR, int NW>
static hipError_t launch_conv(const Args& a, int32_t blocks, hipStream_t stream) {
  const Hot h = hot_of(a, blocks);
  if (a.n_rows == 1)
    hipLaunchKernelGGL((kda_decode_tile<T, LPR, NW, false, true, false>), dim3(blocks),
                       dim3(kWave * NW), 0, stream, KDA_HOT_ARGS(h), a);
  else if (a.rows_block)
    hipLaunchKernelGGL((kda_decode_tile<T, LPR, NW, true, true, true>), dim3(blocks),
                       dim3(kWave * NW), 0, stream, KDA_HOT_ARGS(h), a);
  else
    hipLaunchKernelGGL((kda_decode_tile<T, LPR, NW, true, true, false>), dim3(blocks),
                       dim3(kWave * NW), 0, stream, KDA_HOT_ARGS(h), a);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_conv(const Args& a, int32_t nw, int32_t blocks, hipStream_t s) {
  constexpr int LPR = kHeadV / Lane16<T>::kCols;
  switch (nw) {
    case 2: return launch_conv<T, LPR, 2>(a, blocks, s);
    case 4: return launch_conv<T, LPR, 4>(a, blocks, s);
    case 8: return launch_conv<T, LPR, 8>(a, blocks, s);
    default: return hipErrorInvalidValue;  // unreachable: checked on the host
  }
}

template <typename T, int LPR, int NWB>
static hipError_t launch_rows(const Args& a, int32_t blocks, hipStream_t stream) {
  if constexpr (NWB * LPR * Lane16<T>::kCols > kHeadV) {
    return hipErrorInvalidValue;  // unreachable: wave_k_supported() refuses it
  } else {
    const Hot h = hot_of(a, blocks);
    hipLaunchKernelGGL((kda_rows_kernel<T, LPR, NWB>), dim3(blocks), dim3(kWave * NWB), 0, stream,
                       KDA_HOT_ARGS(h), a);
    return hipGetLastError();
  }
}

// One instantiation per shape that wave_k_supported() admits.
template <typename T>
static hipError_t dispatch_rows(const Args& a, const Shape& sh, int32_t blocks, hipStream_t s) {
  const int lpr = sh.bv / (sh.nw * Lane16<T>::kCols);
  switch (lpr * 16 + sh.nw) {
    case 2 * 16 + 2: return launch_rows<T, 2, 2>(a, blocks, s);
    case 2 * 16 + 4: return launch_rows<T, 2, 4>(a, blocks, s);
    case 2 * 16 + 8: return launch_rows<T, 2, 8>(a, blocks, s);
    case 4 * 16 + 2: return launch_rows<T, 4, 2>(a, blocks, s);
    case 4 * 16 + 4: return launch_rows<T, 4, 4>(a, blocks, s);
    case 4 * 16 + 8: return launch_rows<T, 4, 8>(a, blocks, s);
    default: return hipErrorInvalidValue;  // unreachable: shapes are checked first
  }
}

// One instantiation per shape that shape_supported() admits.
template <typename T>
static hipError_t dispatch(const Args& a, const Shape& sh, int32_t blocks, hipStream_t s) {
  if (sh.layout == KDA_ROWS_WAVE_K) return dispatch_rows<T>(a, sh, blocks, s);
  if (sh.layout == KDA_ROWS_MATRIX) {
    const Hot h = hot_of(a, blocks);
    if (sh.nw == kMatrixWaves)
      hipLaunchKernelGGL((kda_rows_mfma8_kernel<T, kRowsPlain>), dim3(blocks), dim3(kWave * kMatrixWaves), 0, s,
                         KDA_HOT_ARGS(h), a);
    else
      hipLaunchKernelGGL((kda_rows_mfma_kernel<T, false>), dim3(blocks), dim3(kWave * kMfmaWaves), 0, s,
                         KDA_HOT_ARGS(h), a);
    return hipGetLastError();
  }
  const int lpr = sh.bv / Lane16<T>::kCols;
  switch (lpr * 16 + sh.nw) {
    case 8 * 16 + 1: return launch_tile<T, 8, 1>(a, blocks, s);
    case 8 * 16 + 2: return launch_tile<T, 8, 2>(a, blocks, s);
    case 8 * 16 + 4: return launch_tile<T, 8, 4>(a, blocks, s);
    case 8 * 16 + 8: return launch_tile<T, 8, 8>(a, blocks, s);
    case 16 * 16 + 2: return launch_tile<T, 16, 2>(a, blocks, s);
    case 16 * 16 + 4: return launch_tile<T, 16, 4>(a, blocks, s);
    case 16 * 16 + 8: return launch_tile<T, 16, 8>(a, blocks, s);
    default: break;
  }
  if constexpr (Lane16<T>::kCols == 4) {  // fp32 only: 32 rows per lane, bv 128
    switch (lpr * 16 + sh.nw) {
      case 16 * 16 + 1: return launch_tile<T, 16, 1>(a, blocks, s);
      case 32 * 16 + 2: return launch_tile<T, 32, 2>(a, blocks, s);
      case 32 * 16 + 4: return launch_tile<T, 32, 4>(a, blocks, s);
      case 32 * 16 + 8: return launch_tile<T, 32, 8>(a, blocks, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;  // unreachable: shapes are checked first
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace kda

using namespace kda;

extern "C" int kda_decode_step_ex(const kda_pool* pool, const int32_t* slot_ids,
                                  const int32_t* init_slot_ids, const float* q, const float* k,
                                  const float* v, const float* g, const float* b, float* out,
                                  int32_t n_req, int32_t n_rows_per_slot, kda_dtype state_dtype,
                                  float scale, const kda_launch_opts* opts, void* stream) {
  const int rc = check_common(pool, n_req, n_rows_per_slot, state_dtype);
  if (rc != KDA_OK) return rc;
  if (n_req == 0) return KDA_OK;  // empty launch: the row buffers may be NULL
  if (slot_ids == nullptr || q == nullptr || k == nullptr || v == nullptr || g == nullptr ||
      b == nullptr || out == nullptr)
    return KDA_ERR_NULL;
  if (!std::isfinite(scale)) return KDA_ERR_ARG;
  Shape shape;
  if (!resolve_shape(state_dtype, n_rows_per_slot, static_cast<int64_t>(n_req) * pool->H, opts, &shape))
    return KDA_ERR_ARG;
  if (!aligned16(pool->base) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      !aligned16(g) || !aligned16(out) || !aligned4(b) || !aligned4(slot_ids) ||
      !aligned4(init_slot_ids))
    return KDA_ERR_ALIGN;

  Args a;
  a.pool = pool->base;
  a.slot_ids = slot_ids;
  a.init_slot_ids = init_slot_ids;
  a.x = nullptr;
  a.conv_w = nullptr;
  a.conv_pool = nullptr;
  a.pair_counts = nullptr;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.b = b;
  a.out = out;
  a.n_slots = pool->n_slots;
  a.H = pool->H;
  a.n_rows = n_rows_per_slot;
  a.n_vt = kHeadV / shape.bv;
  a.rows_block = opts != nullptr && opts->block_rows != 0 ? 1 : 0;
  a.g_raw = 0;
  a.scale = scale;
  const int32_t blocks = n_req * pool->H * a.n_vt;
  hipStream_t s = static_cast<hipStream_t>(stream);

  const hipError_t err = state_dtype == KDA_F32 ? dispatch<float>(a, shape, blocks, s)
                                                : dispatch<_Float16>(a, shape, blocks, s);
  return err == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

extern "C" int kda_decode_step(const kda_pool* pool, const int32_t* slot_ids, const float* q,
                               const float* k, const float* v, const float* g, const float* b,
                               float* out, int32_t n_req, int32_t n_rows_per_slot,
                               kda_dtype state_dtype, float scale, void* stream) {
  return kda_decode_step_ex(pool, slot_ids, nullptr, q, k, v, g, b, out, n_req, n_rows_per_slot,
                            state_dtype, scale, nullptr, stream);
}

// The fused step's host half: every check, the shape and the kernel
// arguments, before any HIP call.  pairs says whether pair counters will be
// there (n_pairs of them; pair_counts may still be NULL when the caller
// supplies them later), which lets chained rows in the matrix-core form take
// 64-column halves.  *blocks = 0: nothing to launch.
static int conv_prepare(const kda_pool* pool, const kda_conv_pool* conv, const int32_t* slot_ids,
                        const int32_t* init_slot_ids, const float* x, const float* conv_w,
                        const float* g, const float* b, float* out, int32_t n_req,
                        int32_t n_rows_per_slot, kda_dtype state_dtype, float scale, bool pairs,
                        uint32_t* pair_counts, int64_t n_pairs, const kda_launch_opts* opts, Args* a,
                        Shape* shape, int32_t* blocks) {
  *blocks = 0;
  const int rc = check_common(pool, n_req, n_rows_per_slot, state_dtype);
  if (rc != KDA_OK) return rc;
  if (conv == nullptr || conv->base == nullptr) return KDA_ERR_NULL;
  if (conv->n_slots != pool->n_slots || conv->H != pool->H) return KDA_ERR_SHAPE;
  if (n_req == 0) return KDA_OK;
  if (slot_ids == nullptr || x == nullptr || conv_w == nullptr || g == nullptr || b == nullptr ||
      out == nullptr)
    return KDA_ERR_NULL;
  if (!std::isfinite(scale)) return KDA_ERR_ARG;
  const int64_t units = static_cast<int64_t>(n_req) * pool->H;
  if (pairs && n_pairs < units) return KDA_ERR_ARG;
  if (!resolve_conv_shape(state_dtype, n_rows_per_slot, units, opts, pairs, shape)) return KDA_ERR_ARG;
  if (!aligned16(pool->base) || !aligned16(conv->base) || !aligned16(x) || !aligned16(conv_w) ||
      !aligned16(g) || !aligned16(out) || !aligned4(b) || !aligned4(slot_ids) ||
      !aligned4(init_slot_ids) || !aligned4(pair_counts))
    return KDA_ERR_ALIGN;
  const int64_t tiles = units * (kHeadV / shape->bv);
  if (tiles > INT32_MAX) return KDA_ERR_ARG;
  a->pool = pool->base;
  a->slot_ids = slot_ids;
  a->init_slot_ids = init_slot_ids;
  a->q = nullptr;
  a->k = nullptr;
  a->v = nullptr;
  a->g = g;
  a->b = b;
  a->out = out;
  a->x = x;
  a->conv_w = conv_w;
  a->conv_pool = static_cast<uint16_t*>(conv->base);
  a->pair_counts = pair_counts;
  a->n_slots = pool->n_slots;
  a->H = pool->H;
  a->n_rows = n_rows_per_slot;
  a->n_vt = kHeadV / shape->bv;
  a->rows_block = opts != nullptr && opts->block_rows != 0 ? 1 : 0;
  a->g_raw = opts != nullptr ? opts->g_raw : 0;
  a->scale = scale;
  *blocks = static_cast<int32_t>(tiles);
  return KDA_OK;
}

static int conv_launch(const Args& a, const Shape& shape, int32_t blocks, kda_dtype state_dtype,
                       void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (shape.layout == KDA_ROWS_MATRIX) {
    const Hot h = hot_of(a, blocks);
    const dim3 grid(blocks), block(kWave * shape.nw);
    const bool f32 = state_dtype == KDA_F32;
    if (shape.bv == kMatrixBV) {
      if (f32)
        hipLaunchKernelGGL((kda_rows_mfma8_kernel<float, kRowsConvHalf>), grid, block, 0, s, KDA_HOT_ARGS(h), a);
      else
        hipLaunchKernelGGL((kda_rows_mfma8_kernel<_Float16, kRowsConvHalf>), grid, block, 0, s, KDA_HOT_ARGS(h), a);
    } else if (shape.nw == kMatrixConvWaves) {
      if (f32)
        hipLaunchKernelGGL((kda_rows_mfma8_kernel<float, kRowsConvHead>), grid, block, 0, s, KDA_HOT_ARGS(h), a);
      else
        hipLaunchKernelGGL((kda_rows_mfma8_kernel<_Float16, kRowsConvHead>), grid, block, 0, s, KDA_HOT_ARGS(h), a);
    } else {
      if (f32)
        hipLaunchKernelGGL((kda_rows_mfma_kernel<float, true>), grid, block, 0, s, KDA_HOT_ARGS(h), a);
      else
        hipLaunchKernelGGL((kda_rows_mfma_kernel<_Float16, true>), grid, block, 0, s, KDA_HOT_ARGS(h), a);
    }
    err = hipGetLastError();
  } else {
    err = state_dtype == KDA_F32 ? dispatch_conv<float>(a, shape.nw, blocks, s)
                                 : dispatch_conv<_Float16>(a, shape.nw, blocks, s);
  }
  return err == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// The fused step; pair_counts (nullable, n_pairs entries) lets chained rows
// in the matrix-core form take 64-column halves.
static int decode_step_conv(const kda_pool* pool, const kda_conv_pool* conv, const int32_t* slot_ids,
                            const int32_t* init_slot_ids, const float* x, const float* conv_w,
                            const float* g, const float* b, float* out, int32_t n_req,
                            int32_t n_rows_per_slot, kda_dtype state_dtype, float scale,
                            uint32_t* pair_counts, int64_t n_pairs, const kda_launch_opts* opts,
                            void* stream) {
  Args a;
  Shape shape;
  int32_t blocks = 0;
  const int rc = conv_prepare(pool, conv, slot_ids, init_slot_ids, x, conv_w, g, b, out, n_req,
                              n_rows_per_slot, state_dtype, scale, pair_counts != nullptr, pair_counts,
                              n_pairs, opts, &a, &shape, &blocks);
  if (rc != KDA_OK || blocks == 0) return rc;
  return conv_launch(a, shape, blocks, state_dtype, stream);
}

// Pair counters of kda_decode_step_conv_noalloc, for callers that cannot
// allocate: one per (request, head) of a launch, at most
// KDA_NOALLOC_MAX_PAIRS; every GPU the library runs on holds its own copy
// until the process ends.  They need only be even between calls, never
// cleared: zero when the code object loads, and every call adds 0 or 2 to
// each (calls that overlap on one GPU still add 2 each, though they race on
// which half writes the handed-over history).
static __device__ __align__(256) uint32_t scratch[KDA_NOALLOC_MAX_PAIRS];

// The device address of `scratch` on each device, looked up once per device
// with that device current.  In host code the array's name stands for a
// host-side shadow, not a device address: kernels get only these pointers.
constexpr int kMaxDevices = 64;
static std::atomic<uint32_t*> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mutex;

static hipError_t scratch_on_device(int dev, uint32_t** out) {
  uint32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = -1;
      hipError_t e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (cur != dev) {
        const hipError_t back = hipSetDevice(cur);
        if (e == hipSuccess) e = back;
      }
      if (e != hipSuccess) return e;
      if (addr == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<uint32_t*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

extern "C" int kda_decode_step_conv(const kda_pool* pool, const kda_conv_pool* conv,
                                    const int32_t* slot_ids, const int32_t* init_slot_ids,
                                    const float* x, const float* conv_w, const float* g,
                                    const float* b, float* out, int32_t n_req,
                                    int32_t n_rows_per_slot, kda_dtype state_dtype, float scale,
                                    const kda_launch_opts* opts, void* stream) {
  return decode_step_conv(pool, conv, slot_ids, init_slot_ids, x, conv_w, g, b, out, n_req,
                          n_rows_per_slot, state_dtype, scale, nullptr, 0, opts, stream);
}

extern "C" int kda_decode_step_conv_ws(const kda_pool* pool, const kda_conv_pool* conv,
                                       const int32_t* slot_ids, const int32_t* init_slot_ids,
                                       const float* x, const float* conv_w, const float* g,
                                       const float* b, float* out, int32_t n_req,
                                       int32_t n_rows_per_slot, kda_dtype state_dtype, float scale,
                                       uint32_t* pair_counts, int32_t n_pair_counts,
                                       const kda_launch_opts* opts, void* stream) {
  if (pair_counts == nullptr && n_pair_counts != 0) return KDA_ERR_NULL;
  if (n_pair_counts < 0) return KDA_ERR_ARG;
  return decode_step_conv(pool, conv, slot_ids, init_slot_ids, x, conv_w, g, b, out, n_req,
                          n_rows_per_slot, state_dtype, scale, pair_counts, n_pair_counts, opts, stream);
}

extern "C" int kda_decode_step_conv_noalloc(const kda_pool* pool, const kda_conv_pool* conv,
                                            const int32_t* slot_ids, const int32_t* init_slot_ids,
                                            const float* x, const float* conv_w, const float* g,
                                            const float* b, float* out, int32_t n_req,
                                            int32_t n_rows_per_slot, kda_dtype state_dtype,
                                            float scale, const kda_launch_opts* opts, void* stream) {
  Args a;
  Shape shape;
  int32_t blocks = 0;
  const int rc = conv_prepare(pool, conv, slot_ids, init_slot_ids, x, conv_w, g, b, out, n_req,
                              n_rows_per_slot, state_dtype, scale, true, nullptr, KDA_NOALLOC_MAX_PAIRS,
                              opts, &a, &shape, &blocks);
  if (rc != KDA_OK || blocks == 0) return rc;
  // the device the launch runs on: the stream's (the current one for the
  // null stream)
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return KDA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_LAUNCH;
  uint32_t* counters = nullptr;
  if (scratch_on_device(dev, &counters) != hipSuccess) return KDA_ERR_LAUNCH;
  a.pair_counts = counters;
  return conv_launch(a, shape, blocks, state_dtype, stream);
}

extern "C" int kda_state_copy(const kda_pool* pool, const int32_t* src_slot_ids,
                              const int32_t* dst_slot_ids, int32_t n, kda_dtype state_dtype,
                              void* stream) {
  const int rc = check_common(pool, 0, 1, state_dtype);
  if (rc != KDA_OK) return rc;
  if (n < 0) return KDA_ERR_ARG;
  if (n == 0) return KDA_OK;
  if (src_slot_ids == nullptr || dst_slot_ids == nullptr) return KDA_ERR_NULL;
  if (!aligned16(pool->base) || !aligned4(src_slot_ids) || !aligned4(dst_slot_ids))
    return KDA_ERR_ALIGN;
  const int64_t elem = state_dtype == KDA_F32 ? 4 : 2;
  const int64_t slot_vecs = static_cast<int64_t>(pool->H) * kHeadK * kHeadV * elem / 16;
  const int64_t bx = (slot_vecs + 255) / 256;
  if (bx > INT32_MAX || n > 65535) return KDA_ERR_ARG;
  hipLaunchKernelGGL(kda_state_copy_kernel, dim3(static_cast<uint32_t>(bx), static_cast<uint32_t>(n)),
                     dim3(256), 0, static_cast<hipStream_t>(stream), static_cast<char*>(pool->base),
                     src_slot_ids, dst_slot_ids, pool->n_slots, slot_vecs);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

extern "C" int kda_copy_probe(void* dst, const void* src, size_t bytes, void* stream) {
  if (dst == nullptr || src == nullptr) return KDA_ERR_NULL;
  if (!aligned16(dst) || !aligned16(src)) return KDA_ERR_ALIGN;
  if (bytes % 16 != 0) return KDA_ERR_ARG;
  if (bytes == 0) return KDA_OK;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  const int64_t blocks = (n + 255) / 256;
  if (blocks > INT32_MAX) return KDA_ERR_ARG;
  hipLaunchKernelGGL(kda_copy_probe_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const f4*>(src),
                     static_cast<f4*>(dst), n);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}
