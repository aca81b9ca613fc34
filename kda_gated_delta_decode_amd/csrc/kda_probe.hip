// kda_probe.hip -- measurement helpers of the KDA decode library: streaming
// bandwidth probes and the decode tile's own access pattern without its
// arithmetic.  None of them is on the decode path; they exist so that the
// bandwidth a decode launch reaches can be set against what this GPU reaches
// on the same traffic (ROCm/ATOM PR #2130, What: the production kernel is
// quoted as a fraction of achievable bandwidth, a figure the pages do not
// define; these probes define it here).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_decode.h"
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kProbeThreads = 256;

// One workgroup covers kProbeThreads * V consecutive 16-byte vectors; thread
// x takes vectors x, x + 256, ..., so every wave instruction touches 1 KiB of
// consecutive bytes.  All loads of a thread are issued before its first
// store.  MODE: KDA_PROBE_COPY (src -> dst), KDA_PROBE_READ (src only; the
// loaded bits are folded and written to dst[0] only if they equal `tag`,
// which the caller makes impossible, so no byte is written in practice but
// the loads cannot be dropped), KDA_PROBE_WRITE (dst only: the vector index).
template <int MODE, int V, bool NT>
__global__ __launch_bounds__(kProbeThreads) void kda_bw_probe_kernel(const f4* __restrict__ src,
                                                                     f4* __restrict__ dst, int64_t n,
                                                                     uint32_t tag) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kProbeThreads * V + threadIdx.x;
  if constexpr (MODE == KDA_PROBE_WRITE) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = base + static_cast<int64_t>(j) * kProbeThreads;
      if (i < n) {
        const float x = static_cast<float>(i);
        const f4 w = f4{x, x, x, x};
        if constexpr (NT)
          __builtin_nontemporal_store(w, dst + i);
        else
          dst[i] = w;
      }
    }
  } else {
    f4 r[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = base + static_cast<int64_t>(j) * kProbeThreads;
      if (i < n) r[j] = NT ? __builtin_nontemporal_load(src + i) : src[i];
    }
    if constexpr (MODE == KDA_PROBE_COPY) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int64_t i = base + static_cast<int64_t>(j) * kProbeThreads;
        if (i < n) {
          if constexpr (NT)
            __builtin_nontemporal_store(r[j], dst + i);
          else
            dst[i] = r[j];
        }
      }
    } else {
      uint32_t acc = 0;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int64_t i = base + static_cast<int64_t>(j) * kProbeThreads;
        if (i < n)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc ^= __float_as_uint(r[j][e]);
      }
      if (acc == tag) dst[0] = f4{0.0f, 0.0f, 0.0f, 1.0f};
    }
  }
}

template <int MODE, bool NT>
hipError_t launch_bw(int v, const f4* src, f4* dst, int64_t n, hipStream_t s) {
  const int64_t per = static_cast<int64_t>(kProbeThreads) * v;
  const int64_t blocks = (n + per - 1) / per;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(blocks));
  const uint32_t tag = 0x5a5a5a5au;
  switch (v) {
    case 1: hipLaunchKernelGGL((kda_bw_probe_kernel<MODE, 1, NT>), grid, dim3(kProbeThreads), 0, s, src, dst, n, tag); break;
    case 2: hipLaunchKernelGGL((kda_bw_probe_kernel<MODE, 2, NT>), grid, dim3(kProbeThreads), 0, s, src, dst, n, tag); break;
    case 4: hipLaunchKernelGGL((kda_bw_probe_kernel<MODE, 4, NT>), grid, dim3(kProbeThreads), 0, s, src, dst, n, tag); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The single-row decode launch's memory traffic with the arithmetic taken
// out: the same grid, the same XCD-aware block-to-tile map, the same slot id
// load and the same lane-to-row layout and 16-byte nontemporal loads and
// stores of the state tile; each tile is read and written back in place
// (xor with a zero the compiler cannot see, so the store is not elided).
template <typename T, int LPR, int NW>
__global__ __launch_bounds__(kWave * NW) void kda_tile_probe_kernel(T* pool, const int32_t* slot_ids,
                                                                    int32_t n_slots, int32_t H,
                                                                    int32_t n_vt, uint32_t zero) {
  constexpr int CPL = 16 / static_cast<int>(sizeof(T));
  constexpr int BV = LPR * CPL;
  constexpr int GROUPS = kWave / LPR;
  constexpr int RPW = kHeadK / NW;
  constexpr int RPL = RPW / GROUPS;
  using u4 = uint32_t __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int row0 = wave * RPW + (lane / LPR) * RPL;
  const int tile = tile_of_block(blockIdx.x, gridDim.x);
  const int vt = tile % n_vt;
  const int rh = tile / n_vt;
  const int h = rh % H;
  const int r = rh / H;
  const int32_t sid = slot_ids[r];
  if (sid < 0 || sid >= n_slots) return;  // as the decode: a bad id is skipped
  const int64_t head_elems = static_cast<int64_t>(kHeadK) * kHeadV;
  const int64_t off = static_cast<int64_t>(sid) * H * head_elems + h * head_elems +
                      static_cast<int64_t>(row0) * kHeadV + vt * BV + (lane % LPR) * CPL;
  u4* p = reinterpret_cast<u4*>(pool + off);
  u4 raw[RPL];
#pragma unroll
  for (int m = 0; m < RPL; ++m) raw[m] = __builtin_nontemporal_load(p + m * (kHeadV / CPL));
#pragma unroll
  for (int m = 0; m < RPL; ++m) __builtin_nontemporal_store(raw[m] ^ zero, p + m * (kHeadV / CPL));
}

// The chained rows' memory traffic in the matrix-core block form with the
// arithmetic taken out: the grid, block-to-tile map, slot id loads, lane
// layout and nontemporal loads and stores of kda_rows_mfma8_kernel, with the
// initial state written unchanged to every row's slot (xor with a zero the
// compiler cannot see, so the stores stay).  A workgroup takes NH column
// groups of BH columns, 8 waves each; wave w holds key rows 16 w .. 16 w +
// 15, lane (gq, li) 4-column piece li of the group's row 16 w + J gq + j
// (j < J), so one instruction covers 64 / (BH / 4) whole rows of the group.
// BH = 64, NH = 1 is the block form's layout and BH = 64, NH = 2 its
// whole-head form with the convolution fused; BH = 32 and BH = 128 are the
// narrower and wider tiles it was weighed against.
template <typename T, int BH, int NH>
__global__ __launch_bounds__(kWave * kMatrixWaves * NH) void kda_rows_probe_kernel(
    T* pool, const int32_t* slot_ids, const int32_t* init_ids, int32_t n_slots, int32_t H,
    int32_t n_rows, uint32_t zero) {
  constexpr int NW = kMatrixWaves;  // waves per column group
  constexpr int LPR = BH / 4;       // lanes per row
  constexpr int RPI = kWave / LPR;  // rows per instruction
  constexpr int RPW = kHeadK / NW;  // key rows per wave
  constexpr int J = RPW / RPI;      // rows per lane
  constexpr int BW = BH * NH;       // columns per workgroup
  constexpr int TMAX = KDA_MAX_ROWS;
  static_assert(J >= 1 && RPW % RPI == 0 && kHeadV % BW == 0, "a tile the lanes cover exactly");
  // 4 columns of one row: 8 bytes (fp16) or 16 (fp32)
  using piece = uint32_t __attribute__((ext_vector_type(sizeof(T))));
  const int lane = threadIdx.x % kWave;
  const int wave = (threadIdx.x / kWave) % NW;
  const int grp = threadIdx.x / (kWave * NW);
  const int gq = lane / LPR, li = lane % LPR;
  const int tile = tile_of_block(blockIdx.x, gridDim.x);
  const int vt = tile % (kHeadV / BW);
  const int rh = tile / (kHeadV / BW);
  const int h = rh % H;
  const int r = rh / H;
  const int32_t* ids = slot_ids + static_cast<int64_t>(r) * n_rows;
  int32_t sid[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) sid[t] = t < n_rows ? ids[t] : 0;
  const int32_t init = init_ids != nullptr ? init_ids[r] : sid[0];
  bool ok = init >= 0 && init < n_slots;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) ok = ok && (t >= n_rows || (sid[t] >= 0 && sid[t] < n_slots));
  if (!ok) return;  // as the kernel: a request with a bad id is skipped
  const int64_t head_elems = static_cast<int64_t>(kHeadK) * kHeadV;
  const int64_t slot_elems = static_cast<int64_t>(H) * head_elems;
  const int row0 = RPW * wave + J * gq;
  const int64_t lane_off = h * head_elems + static_cast<int64_t>(row0) * kHeadV + vt * BW + grp * BH + 4 * li;
  piece raw[J];
  {
    const piece* src = reinterpret_cast<const piece*>(pool + static_cast<int64_t>(init) * slot_elems + lane_off);
#pragma unroll
    for (int j = 0; j < J; ++j) raw[j] = __builtin_nontemporal_load(src + j * (kHeadV / 4));
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t >= n_rows) break;
    piece* dst = reinterpret_cast<piece*>(pool + static_cast<int64_t>(sid[t]) * slot_elems + lane_off);
#pragma unroll
    for (int j = 0; j < J; ++j) __builtin_nontemporal_store(raw[j] ^ zero, dst + j * (kHeadV / 4));
  }
}

template <typename T, int BH, int NH>
hipError_t launch_rows_probe(const kda_pool* pool, const int32_t* slot_ids, const int32_t* init_slot_ids,
                             int32_t n_req, int32_t n_rows, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(n_req) * pool->H * (kHeadV / (BH * NH));
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kda_rows_probe_kernel<T, BH, NH>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(kWave * kMatrixWaves * NH), 0, s, static_cast<T*>(pool->base), slot_ids, init_slot_ids,
                     pool->n_slots, pool->H, n_rows, 0u);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_rows_probe(int32_t cols, int32_t waves, const kda_pool* pool, const int32_t* slot_ids,
                               const int32_t* init_slot_ids, int32_t n_req, int32_t n_rows, hipStream_t s) {
  if (waves == kMatrixWaves && cols == 32)
    return launch_rows_probe<T, 32, 1>(pool, slot_ids, init_slot_ids, n_req, n_rows, s);
  if (waves == kMatrixWaves && cols == 64)
    return launch_rows_probe<T, 64, 1>(pool, slot_ids, init_slot_ids, n_req, n_rows, s);
  if (waves == kMatrixWaves && cols == 128)
    return launch_rows_probe<T, 128, 1>(pool, slot_ids, init_slot_ids, n_req, n_rows, s);
  return launch_rows_probe<T, 64, 2>(pool, slot_ids, init_slot_ids, n_req, n_rows, s);  // 128 columns, 16 waves
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace kda

using namespace kda;

extern "C" int kda_bw_probe(void* dst, const void* src, size_t bytes, int32_t mode,
                            int32_t vectors_per_thread, int32_t nontemporal, void* stream) {
  if (mode != KDA_PROBE_COPY && mode != KDA_PROBE_READ && mode != KDA_PROBE_WRITE) return KDA_ERR_ARG;
  if (vectors_per_thread != 1 && vectors_per_thread != 2 && vectors_per_thread != 4) return KDA_ERR_ARG;
  if (dst == nullptr || (mode != KDA_PROBE_WRITE && src == nullptr)) return KDA_ERR_NULL;
  if (!aligned16(dst) || !aligned16(src)) return KDA_ERR_ALIGN;
  if (bytes % 16 != 0) return KDA_ERR_ARG;
  if (bytes == 0) return KDA_OK;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  const f4* s = static_cast<const f4*>(src);
  f4* d = static_cast<f4*>(dst);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  const int v = vectors_per_thread;
  if (mode == KDA_PROBE_COPY)
    e = nontemporal ? launch_bw<KDA_PROBE_COPY, true>(v, s, d, n, st) : launch_bw<KDA_PROBE_COPY, false>(v, s, d, n, st);
  else if (mode == KDA_PROBE_READ)
    e = nontemporal ? launch_bw<KDA_PROBE_READ, true>(v, s, d, n, st) : launch_bw<KDA_PROBE_READ, false>(v, s, d, n, st);
  else
    e = nontemporal ? launch_bw<KDA_PROBE_WRITE, true>(v, s, d, n, st) : launch_bw<KDA_PROBE_WRITE, false>(v, s, d, n, st);
  if (e == hipErrorInvalidValue) return KDA_ERR_ARG;
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

extern "C" int kda_tile_probe(const kda_pool* pool, const int32_t* slot_ids, int32_t n_req,
                              kda_dtype state_dtype, void* stream) {
  if (pool == nullptr || pool->base == nullptr) return KDA_ERR_NULL;
  if (state_dtype != KDA_F32 && state_dtype != KDA_F16) return KDA_ERR_DTYPE_REFUSED;
  if (pool->dtype != state_dtype) return KDA_ERR_DTYPE_MISMATCH;
  if (pool->K != kHeadK || pool->V != kHeadV || pool->H < 1 || pool->n_slots < 1) return KDA_ERR_SHAPE;
  if (n_req < 0 || n_req > pool->n_slots) return KDA_ERR_ARG;
  if (n_req == 0) return KDA_OK;
  if (slot_ids == nullptr) return KDA_ERR_NULL;
  if (!aligned16(pool->base) || (reinterpret_cast<uintptr_t>(slot_ids) & 3u) != 0) return KDA_ERR_ALIGN;
  const int32_t bv = tile_bv(state_dtype);
  const int32_t nw = default_waves_per_tile(state_dtype, 1);
  const int64_t blocks = static_cast<int64_t>(n_req) * pool->H * (kHeadV / bv);
  if (blocks > INT32_MAX) return KDA_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the single-row default shapes of launches bound by bandwidth
  if (state_dtype == KDA_F32 && bv == 128 && nw == 2)
    hipLaunchKernelGGL((kda_tile_probe_kernel<float, 32, 2>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kWave * 2), 0, s, static_cast<float*>(pool->base), slot_ids, pool->n_slots, pool->H,
                       kHeadV / bv, 0u);
  else if (state_dtype == KDA_F16 && bv == 64 && nw == 1)
    hipLaunchKernelGGL((kda_tile_probe_kernel<_Float16, 8, 1>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kWave), 0, s, static_cast<_Float16*>(pool->base), slot_ids, pool->n_slots, pool->H,
                       kHeadV / bv, 0u);
  else
    return KDA_ERR_ARG;  // the default shapes changed: this probe follows them
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

extern "C" int kda_rows_probe(const kda_pool* pool, const int32_t* slot_ids, const int32_t* init_slot_ids,
                              int32_t n_req, int32_t n_rows, int32_t tile_cols, int32_t waves,
                              kda_dtype state_dtype, void* stream) {
  if (pool == nullptr || pool->base == nullptr) return KDA_ERR_NULL;
  if (state_dtype != KDA_F32 && state_dtype != KDA_F16) return KDA_ERR_DTYPE_REFUSED;
  if (pool->dtype != state_dtype) return KDA_ERR_DTYPE_MISMATCH;
  if (pool->K != kHeadK || pool->V != kHeadV || pool->H < 1 || pool->n_slots < 1) return KDA_ERR_SHAPE;
  if (n_rows < 1 || n_rows > KDA_MAX_ROWS) return KDA_ERR_ROWS;
  if (n_req < 0 || static_cast<int64_t>(n_req) * n_rows > pool->n_slots) return KDA_ERR_ARG;
  const int32_t cols = tile_cols == 0 ? kMatrixBV : tile_cols;
  const int32_t nw = waves == 0 ? kMatrixWaves : waves;
  const bool shape_ok = (nw == kMatrixWaves && (cols == 32 || cols == 64 || cols == 128)) ||
                        (nw == 2 * kMatrixWaves && cols == 128);
  if (!shape_ok) return KDA_ERR_ARG;
  if (n_req == 0) return KDA_OK;
  if (slot_ids == nullptr) return KDA_ERR_NULL;
  if (!aligned16(pool->base) || (reinterpret_cast<uintptr_t>(slot_ids) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(init_slot_ids) & 3u) != 0)
    return KDA_ERR_ALIGN;
  if (static_cast<int64_t>(n_req) * pool->H * (kHeadV / cols) > INT32_MAX) return KDA_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = state_dtype == KDA_F32
                           ? dispatch_rows_probe<float>(cols, nw, pool, slot_ids, init_slot_ids, n_req, n_rows, s)
                           : dispatch_rows_probe<_Float16>(cols, nw, pool, slot_ids, init_slot_ids, n_req, n_rows, s);
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}
