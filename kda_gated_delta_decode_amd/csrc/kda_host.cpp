// kda_host.cpp -- host half of the KDA decode C ABI: argument validation,
// addressing (state_at), pool sizing, launch description and error strings.
// Makes no HIP call, so every refusal can be exercised without a GPU.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <unordered_map>

#include "kda_decode.h"
#include "kda_internal.h"
#include "kda_launch.h"

namespace kda {

static bool dtype_known(int dt) { return dt == KDA_F32 || dt == KDA_F16; }

// The checks every entry point shares, in the documented order (ROCm/ATOM
// PR #2945, Changes: refuse anything but fp32 or fp16 rather than
// reinterpret it; refuse a pool of the other dtype, which would be read at
// the wrong element size).
int check_common(const kda_pool* pool, int32_t n_req, int32_t n_rows,
                 kda_dtype state_dtype) {
  if (pool == nullptr || pool->base == nullptr) return KDA_ERR_NULL;
  if (!dtype_known(state_dtype) || !dtype_known(pool->dtype)) return KDA_ERR_DTYPE_REFUSED;
  if (state_dtype != pool->dtype) return KDA_ERR_DTYPE_MISMATCH;
  if (pool->K != kHeadK || pool->V != kHeadV || pool->H < 1 || pool->H > kMaxHeads || pool->n_slots < 1)
    return KDA_ERR_SHAPE;
  if (n_rows < 1 || n_rows > KDA_MAX_ROWS) return KDA_ERR_ROWS;
  if (n_req < 0) return KDA_ERR_ARG;
  if (static_cast<int64_t>(n_req) * n_rows > pool->n_slots) return KDA_ERR_SLOT;
  // grid size: n_req * H * (V / bv) workgroups must fit in int32 for the
  // narrowest tile any launch shape uses (bv = 32)
  const int64_t tiles = static_cast<int64_t>(n_req) * pool->H * (kHeadV / 32);
  if (tiles > INT32_MAX) return KDA_ERR_ARG;
  return KDA_OK;
}

}  // namespace kda

using namespace kda;

extern "C" {

int kda_validate(const kda_pool* pool, const int32_t* slot_ids_host,
                 const int32_t* init_slot_ids_host, int32_t n_req, int32_t n_rows,
                 kda_dtype state_dtype) {
  if (slot_ids_host == nullptr) return KDA_ERR_NULL;
  const int rc = check_common(pool, n_req, n_rows, state_dtype);
  if (rc != KDA_OK) return rc;
  const int64_t R = static_cast<int64_t>(n_req) * n_rows;
  std::unordered_map<int32_t, int32_t> owner;  // snapshot slot -> request
  owner.reserve(static_cast<size_t>(R));
  for (int64_t i = 0; i < R; ++i) {
    const int32_t s = slot_ids_host[i];
    if (s < 0 || s >= pool->n_slots) return KDA_ERR_SLOT;
    if (!owner.emplace(s, static_cast<int32_t>(i / n_rows)).second) return KDA_ERR_SLOT;
  }
  if (init_slot_ids_host != nullptr) {
    for (int32_t r = 0; r < n_req; ++r) {
      const int32_t s = init_slot_ids_host[r];
      if (s < 0 || s >= pool->n_slots) return KDA_ERR_SLOT;
      const auto it = owner.find(s);
      if (it != owner.end() && it->second != r) return KDA_ERR_SLOT;  // another request writes it
    }
  }
  return KDA_OK;
}

int kda_prefill_validate(const kda_pool* pool, const int32_t* init_slot_ids_host,
                         const int32_t* dst_slot_ids_host, const int32_t* cu_seqlens_host,
                         int32_t n_seq, int64_t n_tokens, kda_dtype state_dtype) {
  const int rc = check_common(pool, n_seq, 1, state_dtype);
  if (rc != KDA_OK) return rc;
  if (n_tokens < 0) return KDA_ERR_ARG;
  if (n_seq == 0) return KDA_OK;
  if (init_slot_ids_host == nullptr || cu_seqlens_host == nullptr) return KDA_ERR_NULL;
  if (cu_seqlens_host[0] < 0) return KDA_ERR_ARG;
  for (int32_t s = 0; s < n_seq; ++s)
    if (cu_seqlens_host[s + 1] < cu_seqlens_host[s]) return KDA_ERR_ARG;
  if (cu_seqlens_host[n_seq] > n_tokens) return KDA_ERR_ARG;
  std::unordered_map<int32_t, int32_t> writer;  // destination slot -> sequence
  writer.reserve(static_cast<size_t>(n_seq));
  for (int32_t s = 0; s < n_seq; ++s) {
    const int32_t i = init_slot_ids_host[s];
    const int32_t d = dst_slot_ids_host != nullptr ? dst_slot_ids_host[s] : i;
    if (i < 0 || i >= pool->n_slots || d < 0 || d >= pool->n_slots) return KDA_ERR_SLOT;
    if (!writer.emplace(d, s).second) return KDA_ERR_SLOT;
  }
  for (int32_t s = 0; s < n_seq; ++s) {
    const auto it = writer.find(init_slot_ids_host[s]);
    if (it != writer.end() && it->second != s) return KDA_ERR_SLOT;  // another sequence writes it
  }
  return KDA_OK;
}

int64_t kda_state_at(const kda_pool* pool, const int32_t* slot_ids_host, int32_t n_rows,
                     int32_t req, int32_t row) {
  if (pool == nullptr || slot_ids_host == nullptr) return -KDA_ERR_NULL;
  if (!dtype_known(pool->dtype)) return -KDA_ERR_DTYPE_REFUSED;
  if (pool->K < 1 || pool->V < 1 || pool->H < 1 || pool->n_slots < 1) return -KDA_ERR_SHAPE;
  if (n_rows < 1 || n_rows > KDA_MAX_ROWS) return -KDA_ERR_ROWS;
  if (req < 0 || row < 0 || row >= n_rows) return -KDA_ERR_ARG;
  const int32_t s = slot_ids_host[static_cast<int64_t>(req) * n_rows + row];
  if (s < 0 || s >= pool->n_slots) return -KDA_ERR_SLOT;
  return static_cast<int64_t>(s) * pool->H * pool->K * pool->V;
}

size_t kda_pool_bytes(int32_t n_slots, int32_t H, int32_t K, int32_t V, kda_dtype dtype) {
  if (!dtype_known(dtype) || n_slots < 0 || H < 0 || K < 0 || V < 0) return 0;
  const size_t elem = dtype == KDA_F32 ? 4 : 2;
  return static_cast<size_t>(n_slots) * H * K * V * elem;
}

int32_t kda_tile_bv(kda_dtype dtype) {
  if (!dtype_known(dtype)) return -KDA_ERR_DTYPE_REFUSED;
  return tile_bv(dtype);
}

int kda_describe_launch(int32_t n_req, int32_t n_rows, int32_t H, kda_dtype dtype,
                        const kda_launch_opts* opts, kda_launch_desc* desc) {
  if (desc == nullptr) return KDA_ERR_NULL;
  if (!dtype_known(dtype)) return KDA_ERR_DTYPE_REFUSED;
  if (H < 1 || H > kMaxHeads) return KDA_ERR_SHAPE;
  if (n_rows < 1 || n_rows > KDA_MAX_ROWS) return KDA_ERR_ROWS;
  if (n_req < 0) return KDA_ERR_ARG;
  Shape shape;
  if (!resolve_shape(dtype, n_rows, static_cast<int64_t>(n_req) * H, opts, &shape)) return KDA_ERR_ARG;
  const int32_t bv = shape.bv;
  const int32_t nw = shape.nw;
  const int64_t tiles = static_cast<int64_t>(n_req) * H * (kHeadV / bv);
  if (tiles > INT32_MAX) return KDA_ERR_ARG;
  desc->bv = bv;
  desc->waves_per_tile = nw;
  desc->threads = nw * kWave;
  desc->tiles = static_cast<int32_t>(tiles);
  desc->blocks = static_cast<int32_t>(tiles);
  desc->lds_bytes = lds_bytes(bv, nw, n_rows, opts != nullptr && opts->block_rows != 0, shape.layout);
  desc->kernel = shape.layout == KDA_ROWS_WAVE_K   ? "kda_rows_kernel"
                 : shape.layout == KDA_ROWS_MATRIX ? (nw == kMatrixWaves ? "kda_rows_mfma8_kernel"
                                                                         : "kda_rows_mfma_kernel")
                                                   : "kda_decode_tile";
  desc->rows_layout = shape.layout;
  return KDA_OK;
}

int32_t kda_tile_of_block(int32_t block, int32_t n_blocks) {
  if (n_blocks < 1 || block < 0 || block >= n_blocks) return -1;
  return tile_of_block(block, n_blocks);
}

const char* kda_strerror(int code) {
  switch (code) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_DTYPE_REFUSED: return "state dtype refused: only fp32 and fp16 pools are supported (bf16 is refused, not reinterpreted)";
    case KDA_ERR_DTYPE_MISMATCH: return "state dtype does not match the pool's dtype (it would be read at the wrong element size)";
    case KDA_ERR_SHAPE: return "unsupported shape: K and V must be 128, H in [1, 65535], n_slots at least 1";
    case KDA_ERR_ROWS: return "rows per request must be in [1, 8]";
    case KDA_ERR_SLOT: return "slot id out of range or repeated, or more rows than slots";
    case KDA_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case KDA_ERR_ARG: return "bad argument (negative count, index out of range or non-finite scale)";
    case KDA_ERR_LAUNCH: return "the HIP runtime reported a kernel launch error";
    default: return "unknown kda status code";
  }
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
