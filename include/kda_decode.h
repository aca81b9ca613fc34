/*
 * kda_decode.h -- C ABI of the MI355X (gfx950) KDA recurrent decode library.
 *
 * The operation (Kimi Delta Attention decode, one launch):
 *   for each request r, head h, and each of the request's rows t in order,
 *   with the state S of (r, h) held in fp32 between rows:
 *     qn = q / sqrt(|q|^2 + 1e-6),  kn = k / sqrt(|k|^2 + 1e-6)
 *     a  = exp(g)  (per key channel),  beta = 1 / (1 + exp(-b))
 *     S' = diag(a) S;  u = v - S'^T kn;  S = S' + beta kn u^T
 *     o  = scale * S^T qn
 *     state_at(r, t) <- S   (fp32 as is, or fp16 rounded to nearest even)
 *   The first row's initial state is read from state_at(r, 0).
 *
 * Passages this follows (page title, then section):
 *  - ROCm/ATOM PR #2945 (gfx950 mono K1 takes an fp16 KDA state pool),
 *    Summary and Changes: the pool's dtype is a build constant of the
 *    kernel; each loaded state is widened to fp32, the recurrence runs in
 *    fp32, each stored state is rounded to fp16 to nearest even; one address
 *    function, state_at, serves the request's initial state and every
 *    token's snapshot slot; a pool of the other dtype is refused (it would
 *    be read at the wrong element size); bf16 is refused, not reinterpreted.
 *    Limitations: k is unit after normalisation, beta in (0, 1), decay <= 1.
 *  - ROCm/ATOM PR #2130 "perf(kimi-k3): make the KDA temporal state dtype
 *    configurable", What: a [12, 128, 128] state per layer streams through
 *    HBM every decode token (state-bandwidth bound); q and k are
 *    L2-normalised in-kernel; the recurrence accumulates in fp32 whatever
 *    the pool stores.  Copilot review: the initial state must be validated
 *    early instead of being dereferenced when absent.
 *
 * Conventions for every function:
 *  - Return value: KDA_OK (0) or a kda_status code; kda_strerror() names it.
 *    Functions returning a size or offset return a negative kda_status on
 *    error instead.
 *  - Arguments are validated on the host before any HIP call; a refused call
 *    changes nothing and launches nothing.
 *  - The caller owns every buffer.  The library allocates no memory, never
 *    synchronises, and enqueues its work on the caller's stream (a
 *    hipStream_t passed as void*, NULL = the null stream).  A device fault
 *    surfaces at the caller's next synchronisation.
 */
#ifndef KDA_DECODE_H
#define KDA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 11  /* 11: kda_launch_opts.g_raw; 10: kda_rows_probe tile shapes; 9: kda_decode_step_conv_noalloc; 8: kda_decode_step_conv_ws; 7: kda_rows_probe; 6: kda_bw_probe and kda_tile_probe; 5: KDA_ROWS_MATRIX */

/* Head dimensions this build supports (the Kimi-K3 KDA layer shape). */
#define KDA_HEAD_K 128
#define KDA_HEAD_V 128
/* Rows (tokens) one request may chain in one launch: 1 + up to 7 drafts. */
#define KDA_MAX_ROWS 8

/* Element type of a state pool. */
typedef enum kda_dtype {
  KDA_F32 = 0,
  KDA_F16 = 1,
  KDA_BF16 = 2 /* named only to be refused */
} kda_dtype;

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,           /* a required pointer is NULL */
  KDA_ERR_DTYPE_REFUSED = 2,  /* bf16 or an unknown dtype */
  KDA_ERR_DTYPE_MISMATCH = 3, /* state_dtype differs from the pool's dtype */
  KDA_ERR_SHAPE = 4,          /* K or V != 128, H outside [1, 65535], n_slots < 1 */
  KDA_ERR_ROWS = 5,           /* rows per request outside [1, KDA_MAX_ROWS] */
  KDA_ERR_SLOT = 6,           /* slot id out of range or repeated, or more
                                 rows than slots */
  KDA_ERR_ALIGN = 7,          /* a device pointer is not 16-byte aligned */
  KDA_ERR_ARG = 8,            /* other bad argument (negative count, index
                                 out of range, non-finite scale) */
  KDA_ERR_LAUNCH = 9          /* the HIP runtime reported a launch error */
} kda_status;

/*
 * A state pool: device memory holding [n_slots, H, K, V] elements of dtype,
 * row-major with V fastest, i.e. slot s, head h, key row i, value column j
 * lives at element ((s * H + h) * K + i) * V + j.  base must be 16-byte
 * aligned.  The caller allocates, owns and frees it.
 */
typedef struct kda_pool {
  void* base;
  int32_t n_slots;
  int32_t H;
  int32_t K;
  int32_t V;
  kda_dtype dtype;
} kda_pool;

/*
 * kda_decode_step -- one decode launch over n_req requests of
 * n_rows_per_slot rows each (R = n_req * n_rows_per_slot rows in all).
 *
 *  pool        the state pool (dtype F32 or F16), updated in place.
 *  slot_ids    device int32 [R]: row t of request r uses slot
 *              slot_ids[r * n_rows_per_slot + t] (see kda_state_at).  The
 *              ids of one launch must be distinct and in [0, n_slots):
 *              kda_validate checks a host copy.  On the device, a request
 *              with any id out of range is skipped: its out rows are set to
 *              NaN and no state is read or written.  Repeated ids are not
 *              detected on the device and give an unspecified result.
 *  q, k, g     device fp32 [R, H, 128]; v: device fp32 [R, H, 128];
 *  b           device fp32 [R, H]; rows of one request are adjacent.
 *              g is the log-decay (a = exp(g)); callers keep g <= 0.
 *  out         device fp32 [R, H, 128], written.
 *  state_dtype the dtype the caller built for; must equal pool->dtype.
 *  scale       read-out scale, usually 1/sqrt(128).  Must be finite.
 *  stream      hipStream_t as void*, NULL for the null stream.
 *
 * All device pointers must be 16-byte aligned (slot_ids and b: 4-byte).
 * n_req == 0 is a valid no-op, and then only the pool must be non-NULL.
 * Checks run in the order: pool NULL, DTYPE_REFUSED, DTYPE_MISMATCH,
 * SHAPE, ROWS, ARG (counts), SLOT, then the row buffers' NULL, ARG (scale,
 * opts), ALIGN.  Errors: KDA_ERR_NULL, KDA_ERR_DTYPE_REFUSED,
 * KDA_ERR_DTYPE_MISMATCH, KDA_ERR_SHAPE, KDA_ERR_ROWS, KDA_ERR_SLOT (more
 * rows than slots), KDA_ERR_ALIGN, KDA_ERR_ARG, KDA_ERR_LAUNCH.
 */
int kda_decode_step(const kda_pool* pool, const int32_t* slot_ids,
                    const float* q, const float* k, const float* v,
                    const float* g, const float* b, float* out, int32_t n_req,
                    int32_t n_rows_per_slot, kda_dtype state_dtype,
                    float scale, void* stream);

/*
 * Chained-row layouts (kda_launch_opts.rows_layout; chained rows only).
 *  KDA_ROWS_K_SPLIT  each wave of a workgroup holds a slice of the 128 key
 *                    rows for all of the tile's bv columns; every row's
 *                    partial column sums over K meet in LDS behind a barrier.
 *  KDA_ROWS_WAVE_K   each wave holds all 128 key rows of bv / waves_per_tile
 *                    columns (2 or 4 lanes per 16-byte row piece): a
 *                    row's column sums over K stay inside the wave (DPP and
 *                    permlane exchanges), and the waves of a workgroup run
 *                    their chains with no barrier between rows.
 *  KDA_ROWS_MATRIX   the request's rows as one block: all 2 n column sums
 *                    of the initial state (w0_t = S0^T (gamma_t kn_t) and
 *                    p0_t = S0^T (gamma_t qn_t), gamma_t the decays of rows
 *                    0..t multiplied) in one fp32 matrix-core product per
 *                    wave, the n x n couplings of the rows, a triangular
 *                    solve per column, then element-wise snapshots streamed
 *                    as whole rows.  Fixed shape: 64 columns over 4 waves
 *                    (bv and waves_per_tile must be 0 or 64 and 4).
 */
#define KDA_ROWS_DEFAULT 0
#define KDA_ROWS_K_SPLIT 1
#define KDA_ROWS_WAVE_K 2
#define KDA_ROWS_MATRIX 3

/*
 * Launch options of kda_decode_step_ex.  Zero-initialise for the library's
 * defaults; each non-zero field overrides one choice.
 *  waves_per_tile  wavefronts per workgroup: 1, 2, 4, 8.  K-split layout and
 *                  single rows: the waves split one tile's 128 key rows.
 *  bv              value columns per workgroup.  K-split layout and single
 *                  rows: 32, 64 or 128 for fp32 pools (8, 16, 32 lanes per
 *                  tile row), 64 or 128 for fp16.  Whole-K layout: waves x
 *                  lanes x columns per lane (4 fp32, 8 fp16) with 2 or 4
 *                  lanes and 2, 4 or 8 waves, at most 128.
 *  block_rows      chained rows only: 0 (default) runs a request's rows
 *                  one after the other (two column sums over K and a
 *                  cross-lane reduction per row); non-zero takes them as one
 *                  block (all 2 n column sums of the initial state in one
 *                  pass, an n x n triangular solve, then element-wise
 *                  snapshots).  Both compute the same chain and round
 *                  differently; on MI355X the block form measured slower at
 *                  8 rows (its n x n coupling sums cost more than the
 *                  per-row reductions they replace).  The block form uses
 *                  the K-split layout (with KDA_ROWS_WAVE_K it is refused)
 *                  and, for fp16 pools, at least 2 waves (one wave's 128
 *                  state values and 8 x 8 x 3 column sums per lane do not
 *                  fit in the register file: refused).
 *  rows_layout     chained rows only: KDA_ROWS_DEFAULT, KDA_ROWS_K_SPLIT,
 *                  KDA_ROWS_WAVE_K or KDA_ROWS_MATRIX (a block form
 *                  whatever block_rows says); ignored for one row.  The
 *                  default, with units = requests x heads: for fp16 pools
 *                  the matrix-core block form for 3 rows or more up to 240
 *                  units, else the whole-K layout up to 48 units and the K
 *                  split beyond; when bv or waves_per_tile is set, the
 *                  whole-K layout (bv 64 over 4 waves unless set).  For
 *                  fp32 pools the matrix-core block form for 6 rows or
 *                  more up to 48 units with no bv or waves option, else the
 *                  K split (bv 64 over 8 waves).  block_rows alone selects
 *                  the K-split block form.
 * Supported K-split combinations keep 2..32 key rows per lane (rows per
 * lane = 2 * lanes per row / waves).  The shape changes the order of the
 * fp32 column sums over K (so results may differ in the last bits), never
 * the operation; fixing it fixes every result bit for given inputs.
 */
typedef struct kda_launch_opts {
  int32_t waves_per_tile;
  int32_t bv;
  int32_t block_rows;
  int32_t rows_layout;
  int32_t g_raw;  /* fused convolution entries only (0 elsewhere): see kda_decode_step_conv */
} kda_launch_opts;

/*
 * kda_decode_step_ex -- kda_decode_step with a separate initial-state slot
 * per request and launch options.
 *
 *  init_slot_ids  NULL, or device int32 [n_req]: request r reads its initial
 *                 state from slot init_slot_ids[r] instead of its row-0 slot
 *                 slot_ids[r * n_rows_per_slot].  This is how a speculative
 *                 step resumes from the snapshot of its last accepted token,
 *                 and how a checkpointed state is loaded (ROCm/ATOM PR #2945,
 *                 Changes: one address function serves the initial state,
 *                 every token's snapshot slot, and the checkpoint load and
 *                 flush).  An initial slot may be one of its own request's
 *                 snapshot slots (it is read before any store) but must not
 *                 be written by another request of the launch; kda_validate
 *                 checks a host copy.  With one row per request and
 *                 init_slot_ids[r] != slot_ids[r], the update is out of
 *                 place (ping-pong between two slots).
 *  opts           NULL for the defaults (see kda_launch_opts): for tests
 *                 that must hold the summation order fixed across launches
 *                 and for tuning sweeps.
 * Additional errors: KDA_ERR_ARG for a shape that is not supported; a request
 * whose initial slot is out of range is skipped on the device like one with
 * a bad snapshot slot (out rows NaN, nothing stored).
 */
int kda_decode_step_ex(const kda_pool* pool, const int32_t* slot_ids,
                       const int32_t* init_slot_ids,
                       const float* q, const float* k, const float* v,
                       const float* g, const float* b, float* out,
                       int32_t n_req, int32_t n_rows_per_slot,
                       kda_dtype state_dtype, float scale,
                       const kda_launch_opts* opts, void* stream);

/*
 * A short-convolution history pool: device memory holding [n_slots, 3, C]
 * bfloat16 values, C = 3 * H * 128 channels ordered (q | k | v) x H x 128,
 * entry 0 the oldest of the last 3 raw inputs of each channel.  Slot s of
 * the conv pool belongs with slot s of the state pool (one slot id addresses
 * both).  2 bytes x 3 entries x 4608 channels = 27,648 bytes per slot per
 * layer at H = 12: the part of the pages' per-slot memory that does not
 * follow the state dtype (ROCm/ATOM PR #2130, Memory).  base 16-byte aligned.
 */
typedef struct kda_conv_pool {
  void* base;
  int32_t n_slots;
  int32_t H;
} kda_conv_pool;

/*
 * kda_decode_step_conv -- the decode step with the short causal convolution
 * fused in front (q, k and v each pass a 4-tap depthwise causal convolution,
 * then SiLU; ROCm/ATOM PR #2894, the two-node trial: a 3-entry history is
 * read, then the old entries and the step's inputs are written back).
 *
 *  conv        the history pool (n_slots and H equal to the state pool's).
 *  x           device fp32 [R, 3, H, 128]: the raw q, k, v inputs (before
 *              the convolution) of every row.
 *  conv_w      device fp32 [3, H, 128, 4]: per-channel taps, tap 3 on the
 *              newest input.  No bias.
 *  g, b, out, slot_ids, init_slot_ids, n_req, n_rows_per_slot,
 *  state_dtype, scale, opts, stream: as in kda_decode_step_ex.
 * For row t of request r: q, k, v = silu(sum_j w_j win[t + j]) over the
 * window win = (history of the initial slot, raw rows 0..t of the request),
 * then the decode update.  Row t's snapshot slot receives both the state and
 * the history after row t (its last 3 raw inputs, rounded to bfloat16 to
 * nearest even); rows of one launch use their fp32 inputs directly.
 * Launch shapes: whole heads only (opts->bv 0 or 128), since a head's
 * history at the initial slot is read and may be rewritten in place by one
 * workgroup.  Chained rows take the matrix-core block form (KDA_ROWS_MATRIX:
 * 16 waves, two 64-column halves of 8; waves_per_tile 8: two halves of 4)
 * when rows_layout asks for it, or by default for 3 rows or more up to 192
 * (fp16) or 48 (fp32) requests x heads unless waves_per_tile or block_rows
 * is set; otherwise the K-split kernel with 2, 4 or 8 waves.  One row per
 * request: the single-row kernel over whole heads, by default 4 waves for
 * fp16 pools, and for fp32 pools 2 waves below 384 requests x heads and 4
 * from there.
 * KDA_ROWS_WAVE_K is refused; rows_layout is ignored for one row.
 * opts->g_raw: 0 (default), g is the log-decay as in kda_decode_step; 1, g
 * holds the raw gate x of each key channel and the step takes the
 * log-decay g = -softplus(x) = -log(1 + e^x), computing the decay as
 * 1 / (1 + e^x), so the gate is fused into the front end beside the
 * convolution.  Other values are refused, as is g_raw != 0 on the entries
 * without the convolution.
 * Errors: as kda_decode_step_ex, plus KDA_ERR_NULL for a missing conv pool,
 * x or conv_w, KDA_ERR_SHAPE if the pools' n_slots or H differ.
 */
int kda_decode_step_conv(const kda_pool* pool, const kda_conv_pool* conv,
                         const int32_t* slot_ids, const int32_t* init_slot_ids,
                         const float* x, const float* conv_w, const float* g,
                         const float* b, float* out, int32_t n_req,
                         int32_t n_rows_per_slot, kda_dtype state_dtype,
                         float scale, const kda_launch_opts* opts, void* stream);

/*
 * kda_decode_step_conv_ws -- kda_decode_step_conv with pair counters, which
 * let chained rows in the matrix-core block form split each head into two
 * 64-column workgroups of 8 waves (twice the workgroups: with fewer heads
 * than compute units, a unit's store throughput bounds the whole-head form).
 * Both halves read the initial slot's q and k history; the row whose slot
 * is the initial slot may overwrite it only after both have read it, so each
 * half adds 1 to the counter of its (request, head) once its reads are done,
 * and the half that finds an odd count writes that row's q and k history.
 * No workgroup waits for another.
 *
 *  pair_counts    NULL (then exactly kda_decode_step_conv), or device
 *                 uint32 [n_pair_counts], n_pair_counts >= n_req * H,
 *                 4-byte aligned: counter r * H + h serves request r, head
 *                 h.  Owned by the caller.  Every entry must be even
 *                 (zero-fill once) before the first call; each call adds 0
 *                 or 2 to an entry, so entries stay even and one buffer
 *                 serves any number of calls in sequence.  Calls that may run
 *                 at the same time (other streams, concurrent graphs) need
 *                 buffers of their own.
 *  n_pair_counts  entries of pair_counts (0 with NULL).
 *  opts           as kda_decode_step_conv, plus bv 64: the halves, which
 *                 need pair_counts.  With pair_counts, chained rows take
 *                 the halves when rows_layout is KDA_ROWS_MATRIX or by
 *                 default for fp16 up to 96 requests x heads, or 240 with
 *                 6 rows or more, and for fp32 up to 48, or 96 with 4 rows
 *                 or more, unless waves_per_tile or block_rows is set;
 *                 bv 128 keeps whole heads; beyond, the
 *                 defaults of kda_decode_step_conv.
 * Errors: as kda_decode_step_conv, plus KDA_ERR_NULL for NULL pair_counts
 * with n_pair_counts != 0, KDA_ERR_ARG for n_pair_counts < 0 or, with
 * counters given, n_pair_counts < n_req * H, or bv 64 without counters,
 * KDA_ERR_ALIGN for misaligned counters.
 */
int kda_decode_step_conv_ws(const kda_pool* pool, const kda_conv_pool* conv,
                            const int32_t* slot_ids, const int32_t* init_slot_ids,
                            const float* x, const float* conv_w, const float* g,
                            const float* b, float* out, int32_t n_req,
                            int32_t n_rows_per_slot, kda_dtype state_dtype,
                            float scale, uint32_t* pair_counts,
                            int32_t n_pair_counts, const kda_launch_opts* opts,
                            void* stream);

/*
 * kda_decode_step_conv_noalloc -- kda_decode_step_conv_ws for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the pair counters live in a
 * static device array of KDA_NOALLOC_MAX_PAIRS entries inside the library,
 * one per GPU it runs on, held until the process ends.  The call allocates
 * nothing; its first call on a device looks the array's address up on that
 * device (the stream's device, or the current one for the null stream).
 * Arguments and launch shapes as kda_decode_step_conv_ws with counters given.
 * Every call on a GPU shares that GPU's counters: calls that overlap on one
 * GPU race (results of chained rows in halves are then undefined), calls in
 * sequence do not.  Nothing needs clearing between calls: the counters stay
 * even.
 * Errors: as kda_decode_step_conv_ws, plus KDA_ERR_ARG when n_req * H exceeds
 * KDA_NOALLOC_MAX_PAIRS (checked before any device work), KDA_ERR_LAUNCH if
 * the counters' address cannot be found on the device.
 */
#define KDA_NOALLOC_MAX_PAIRS 4096
int kda_decode_step_conv_noalloc(const kda_pool* pool, const kda_conv_pool* conv,
                                 const int32_t* slot_ids, const int32_t* init_slot_ids,
                                 const float* x, const float* conv_w, const float* g,
                                 const float* b, float* out, int32_t n_req,
                                 int32_t n_rows_per_slot, kda_dtype state_dtype,
                                 float scale, const kda_launch_opts* opts, void* stream);

/*
 * kda_validate -- host-side check of a launch's arguments and slot tables
 * (ROCm/ATOM PR #2945, Changes: the step checks the pool's dtype against
 * the build; anything but fp32 or fp16 is refused).  slot_ids_host is a
 * HOST copy of the slot table [n_req * n_rows]; every id must lie in
 * [0, n_slots) and appear once.  init_slot_ids_host is NULL or a host copy
 * of the initial slots [n_req]: each in range and not among another
 * request's snapshot slots.  Touches no device memory.  Returns KDA_OK or
 * the first error found, in the order: NULL, DTYPE_REFUSED, DTYPE_MISMATCH,
 * SHAPE, ROWS, ARG, SLOT.
 */
int kda_validate(const kda_pool* pool, const int32_t* slot_ids_host,
                 const int32_t* init_slot_ids_host, int32_t n_req,
                 int32_t n_rows, kda_dtype state_dtype);

/*
 * kda_state_copy -- copy whole slots of a pool: for i in [0, n), the
 * [H, K, V] block of slot dst_slot_ids[i] becomes that of src_slot_ids[i]
 * (every head).  The ReplaySSM-style checkpoint flush (a chosen snapshot
 * into a checkpoint slot) and load (back into a working slot) through the
 * same slot addressing as the decode (ROCm/ATOM PR #2945, Changes).
 * src_slot_ids, dst_slot_ids: device int32 [n].  dst ids must be distinct
 * and no dst may be another pair's src (caller contract).  A pair with an
 * id out of range is skipped on the device.  Bytes are copied as they are:
 * the pool keeps its dtype.  Errors: KDA_ERR_NULL, KDA_ERR_DTYPE_REFUSED,
 * KDA_ERR_DTYPE_MISMATCH, KDA_ERR_SHAPE, KDA_ERR_ARG (n < 0 or n > 65535),
 * KDA_ERR_ALIGN, KDA_ERR_LAUNCH.  n == 0 is a no-op.
 */
int kda_state_copy(const kda_pool* pool, const int32_t* src_slot_ids,
                   const int32_t* dst_slot_ids, int32_t n, kda_dtype state_dtype,
                   void* stream);

/*
 * kda_state_at -- element offset, from pool->base, of the [H, K, V] block
 * that row `row` of request `req` reads or writes (ROCm/ATOM PR #2945,
 * Changes: one address function for the initial state and every token's
 * snapshot slot).  Head h's [K, V] state follows at + h * K * V.  Row 0's
 * block is also the request's initial state.  slot_ids_host is a host copy
 * of the slot table.  Returns a negative kda_status on error.
 */
int64_t kda_state_at(const kda_pool* pool, const int32_t* slot_ids_host,
                     int32_t n_rows, int32_t req, int32_t row);

/*
 * kda_pool_bytes -- bytes of a pool of n_slots slots of [H, K, V] elements
 * of dtype: every size derives from the one dtype decision (ROCm/ATOM PR
 * #2130, What and Memory).  Returns 0 for a refused dtype or a bad size.
 */
size_t kda_pool_bytes(int32_t n_slots, int32_t H, int32_t K, int32_t V,
                      kda_dtype dtype);

/*
 * kda_tile_bv -- value columns per state tile that single-row launches use
 * by default once they are large enough to be bound by bandwidth (more than
 * 128 requests x heads for fp32, 96 for fp16): 128 for fp32 pools (whole
 * 512-byte state rows per wave instruction, K over 2 waves), 64 for fp16
 * (whole 128-byte lines, one wave per tile).  Smaller single-row launches
 * take narrower tiles or more waves by default (kda_describe_launch reports
 * the shape of any launch).  Other widths (32 fp32 / 64 fp16 columns is the V-block cap of
 * the pages' portable kernel, ROCm/ATOM PR #2130, Copilot review) remain
 * available through kda_launch_opts.  Returns a negative kda_status for a
 * refused dtype.
 */
int32_t kda_tile_bv(kda_dtype dtype);

/*
 * kda_prefill -- chunked prefill: whole prompts through the same recurrence
 * as kda_decode_step (ROCm/ATOM PR #2130, What and Depends on: every path,
 * prefill included, reads and writes the state in the pool's dtype while
 * the recurrence runs in fp32; the prefill kernel takes its initial state
 * from the pool, fp16 included).
 *
 * Sequence s owns tokens cu_seqlens[s] .. cu_seqlens[s + 1] - 1.  Its state
 * starts from slot init_slot_ids[s] (widened exactly), every token t is
 * applied in order, out[t] receives scale * S_t^T qn_t, and only the final
 * state is stored, to slot dst_slot_ids[s] (NULL: back to init_slot_ids[s];
 * fp16 pools round to nearest even).  An empty sequence copies its state.
 *
 *  pool           device pool [n_slots, H, 128, 128] of state_dtype.
 *  init_slot_ids  device int32 [n_seq].
 *  dst_slot_ids   NULL or device int32 [n_seq]: distinct, and none is
 *                 another sequence's initial slot (kda_prefill_validate
 *                 checks host copies).
 *  cu_seqlens     device int32 [n_seq + 1], non-decreasing, cu_seqlens[0]
 *                 >= 0, cu_seqlens[n_seq] <= n_tokens.
 *  q, k, g        device fp32 [n_tokens, H, 128], 16-byte aligned; v, out
 *                 device fp32 [n_tokens, H, 128]; b device fp32 [n_tokens, H].
 *  n_seq          sequences (<= n_slots); n_tokens: rows of the token arrays.
 *  opts           NULL or kda_prefill_opts (chunk: 0 = default 32, or 32/64
 *                 tokens per chunk; the chunk changes the rounding order,
 *                 never the operation).
 * The chunked form (per-channel cumulative decay, a unit lower-triangular
 * solve per chunk, matrix-core products) equals the token-by-token
 * recurrence up to rounding.  Device-side, a sequence whose table entries
 * are out of range is skipped (nothing written for it).
 * Errors: as kda_decode_step (KDA_ERR_SLOT: n_seq > n_slots; KDA_ERR_SHAPE
 * also for H > 16384, which keeps byte offsets within a chunk below 2^31),
 * KDA_ERR_ARG (bad chunk, n_tokens < 0, n_seq * H > INT32_MAX, non-finite
 * scale).  Asynchronous on stream.
 */
typedef struct kda_prefill_opts {
  int32_t chunk;
} kda_prefill_opts;

int kda_prefill(const kda_pool* pool, const int32_t* init_slot_ids,
                const int32_t* dst_slot_ids, const int32_t* cu_seqlens, const float* q,
                const float* k, const float* v, const float* g, const float* b, float* out,
                int32_t n_seq, int64_t n_tokens, kda_dtype state_dtype, float scale,
                const kda_prefill_opts* opts, void* stream);

/*
 * kda_prefill_validate -- host-side check of a prefill's tables (host
 * copies): KDA_ERR_NULL, KDA_ERR_ARG (cu_seqlens not non-decreasing from
 * >= 0 to <= n_tokens), KDA_ERR_SLOT (an id out of range, two sequences
 * storing to one slot, or a destination that is another sequence's initial
 * slot), plus the pool checks of kda_validate.  CPU only.
 */
int kda_prefill_validate(const kda_pool* pool, const int32_t* init_slot_ids_host,
                         const int32_t* dst_slot_ids_host, const int32_t* cu_seqlens_host,
                         int32_t n_seq, int64_t n_tokens, kda_dtype state_dtype);

/* Launch shape kda_decode_step uses for a given problem (host only). */
typedef struct kda_launch_desc {
  int32_t bv;              /* value columns per workgroup */
  int32_t waves_per_tile;  /* wavefronts per workgroup */
  int32_t threads;         /* threads per workgroup */
  int32_t tiles;           /* n_req * H * (V / bv) */
  int32_t blocks;          /* workgroups launched */
  int32_t lds_bytes;       /* static LDS per workgroup */
  const char* kernel;      /* kernel symbol family name */
  int32_t rows_layout;     /* KDA_ROWS_K_SPLIT, _WAVE_K or _MATRIX (one row: K_SPLIT) */
} kda_launch_desc;

/* Fills *desc for (n_req, n_rows, H, dtype) under opts (NULL = defaults).
 * Errors: KDA_ERR_NULL, KDA_ERR_DTYPE_REFUSED, KDA_ERR_SHAPE (H < 1),
 * KDA_ERR_ROWS, KDA_ERR_ARG. */
int kda_describe_launch(int32_t n_req, int32_t n_rows, int32_t H,
                        kda_dtype dtype, const kda_launch_opts* opts,
                        kda_launch_desc* desc);

/*
 * kda_tile_of_block -- the tile a workgroup processes.  Workgroups are
 * handed to the 8 XCDs of the chip round-robin; this maps them so that the
 * workgroups one XCD runs hold consecutive tiles (the tiles of one
 * (request, head) share that XCD's L2 for q, k, g).  A bijection of
 * [0, n_blocks).  Returns -1 for block out of range.
 */
int32_t kda_tile_of_block(int32_t block, int32_t n_blocks);

/*
 * kda_copy_probe -- measurement helper: copies `bytes` (a multiple of 16)
 * from src to dst with a plain streaming kernel of the same load/store
 * width as the decode kernel, on `stream`.  Used to calibrate achievable
 * bandwidth and hardware byte counters.  Both pointers 16-byte aligned.
 */
int kda_copy_probe(void* dst, const void* src, size_t bytes, void* stream);

/*
 * kda_bw_probe -- measurement helper: a streaming kernel over `bytes` (a
 * multiple of 16) on `stream`, to set the decode's bandwidth against what the
 * GPU reaches on plain traffic (ROCm/ATOM PR #2130, What: the production
 * kernel is quoted at 71-90% of "achievable" bandwidth, which the pages leave
 * undefined).
 *  mode                KDA_PROBE_COPY: read src, write dst; KDA_PROBE_READ:
 *                      read src only (dst must be a 16-byte device buffer it
 *                      never writes in practice); KDA_PROBE_WRITE: write dst
 *                      only (src may be NULL).
 *  vectors_per_thread  1, 2 or 4 16-byte vectors per thread, all loads
 *                      issued before the first store; consecutive threads
 *                      on consecutive vectors.
 *  nontemporal         non-zero: loads and stores carry the nontemporal
 *                      hint, as the decode's state traffic does.
 * Both pointers 16-byte aligned; src and dst hold at least `bytes` (dst 16
 * bytes for KDA_PROBE_READ).  Errors: KDA_ERR_NULL, KDA_ERR_ALIGN,
 * KDA_ERR_ARG (mode, vectors_per_thread, bytes), KDA_ERR_LAUNCH.
 */
#define KDA_PROBE_COPY 0
#define KDA_PROBE_READ 1
#define KDA_PROBE_WRITE 2
int kda_bw_probe(void* dst, const void* src, size_t bytes, int32_t mode,
                 int32_t vectors_per_thread, int32_t nontemporal, void* stream);

/*
 * kda_tile_probe -- measurement helper: the memory traffic of a single-row
 * decode launch over n_req requests with the arithmetic taken out.  Same grid
 * and block-to-tile map as kda_decode_step at its default shape for launches
 * bound by bandwidth (kda_tile_bv columns; fp32 2 waves, fp16 1 wave), same
 * slot id load, lane layout and 16-byte nontemporal loads; each tile is
 * written back unchanged, in place, to slot_ids[r].  slot_ids: device int32
 * [n_req]; an id out of range skips its request.  Errors: as kda_state_copy
 * for the pool; KDA_ERR_ARG (n_req outside [0, n_slots]).
 */
int kda_tile_probe(const kda_pool* pool, const int32_t* slot_ids, int32_t n_req,
                   kda_dtype state_dtype, void* stream);

/*
 * kda_rows_probe -- measurement helper: the memory traffic of a chained-row
 * launch in the matrix-core block form (KDA_ROWS_MATRIX at its default 8
 * waves: 64-column halves, K over the waves) with the arithmetic taken out.
 * Same grid, block-to-tile map, slot id loads, lane layout and nontemporal
 * loads and stores as kda_decode_step there; each request's initial state
 * (init_slot_ids[r], or slot_ids[r * n_rows] if init_slot_ids is NULL) is
 * written unchanged to each of its rows' slots slot_ids[r * n_rows + t].
 *  slot_ids       device int32 [n_req * n_rows]; init_slot_ids: NULL or
 *                 device int32 [n_req].  A request with an id out of range
 *                 is skipped.
 *  tile_cols, waves  the workgroup's value columns and waves: 0, 0 or 64, 8
 *                 (the block form), 32 or 128 over 8 waves (narrower and
 *                 wider tiles, each lane still 4 columns of a row), or 128
 *                 over 16 waves (two 64-column halves of 8, the fused
 *                 convolution's whole-head form).
 * Errors: as kda_tile_probe; KDA_ERR_ROWS (n_rows outside [1,
 * KDA_MAX_ROWS]); KDA_ERR_ARG (n_req < 0, n_req * n_rows > n_slots, or
 * another tile shape).
 */
int kda_rows_probe(const kda_pool* pool, const int32_t* slot_ids, const int32_t* init_slot_ids,
                   int32_t n_req, int32_t n_rows, int32_t tile_cols, int32_t waves,
                   kda_dtype state_dtype, void* stream);

/* Message for a kda_status code (static string, never NULL). */
const char* kda_strerror(int code);

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_DECODE_H */
