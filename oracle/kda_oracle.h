/*
 * kda_oracle.h -- CPU oracle for the KDA (Kimi Delta Attention) recurrent
 * decode update.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no source, header, table
 * or helper with the HIP library; both sides meet only through the seeded
 * inputs that the test harness hands to each.
 *
 * What it computes (one decode launch over a host copy of the state pool):
 *
 *   for each request r and head h:
 *     S = widen(pool[slot(r, 0)][h])                  -- exact widening
 *     for each of the request's rows t (tokens, in order):
 *       qn = q / sqrt(sum q^2 + eps), kn likewise      -- in-kernel L2 norm
 *       a_i = exp(g_i), beta = 1 / (1 + exp(-b))      -- decay, sigmoid gate
 *       S'  = diag(a) S
 *       u   = v - S'^T kn
 *       S   = S' + beta kn u^T
 *       o   = scale * S^T qn                           -- post-update state
 *       pool[slot(r, t)][h] = narrow(S)                -- identity or RNE fp16
 *
 * Sources (page title, then section):
 *  - ROCm/ATOM PR #2945 (gfx950 mono K1 on an fp16 KDA state pool),
 *    Summary and Changes: every loaded state is widened to fp32, the
 *    recurrence runs in fp32, every stored state is rounded to fp16 to
 *    nearest even; one address function serves the initial state and each
 *    token's snapshot slot.  Limitations: k is L2-normalised, beta lies in
 *    (0, 1), the decay is at most 1.
 *  - ROCm/ATOM PR #2130 "perf(kimi-k3): make the KDA temporal state dtype
 *    configurable", What: a [12, 128, 128] state per layer per token; q and
 *    k are L2-normalised in-kernel; the recurrence accumulates in fp32
 *    whatever the pool stores.  Copilot review: the fused sigmoid gating
 *    kernel takes the pool as its initial state.
 * The equations themselves (decay, delta correction, read-out after the
 * update) are the standard KDA / gated-delta-rule decode step that these
 * pages build on; the pages corroborate each ingredient but print none.
 *
 * Readings where the pages are silent: eps = 1e-6 added to the sum of
 * squares; the read-out uses the post-update state; beta is one scalar per
 * (row, head); a multi-row request chains its tokens through the fp32 state
 * and rounds only the stores; the initial state comes from the request's
 * row-0 slot.
 *
 * Precision: the pages fix the recurrence at fp32, so kdao_step_f32 is the
 * pages' precision (sequential sums, no fused multiply-add: build with
 * -ffp-contract=off).  kdao_step_f64 is the same loop in fp64, used as the
 * near-exact reference and for drift reports.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Pool element kinds understood by the oracle (its own numbering). */
#define KDAO_POOL_F32 0
#define KDAO_POOL_F16 1
#define KDAO_POOL_BF16 2 /* error studies only: the library refuses bf16 pools */

/* Return codes. */
#define KDAO_OK 0
#define KDAO_EARG 1 /* bad argument (null pointer, bad size, bad slot id) */

/* IEEE 754 binary32 -> binary16, round to nearest, ties to even.  Overflow
 * gives +-inf, NaN stays NaN (quiet, payload truncated), subnormal results
 * are produced, never flushed. */
uint16_t kdao_f32_to_f16_rne(float x);
/* IEEE 754 binary16 -> binary32, exact. */
float kdao_f16_to_f32(uint16_t h);
void kdao_f32_to_f16_rne_array(const float* x, uint16_t* h, int64_t n);
void kdao_f16_to_f32_array(const uint16_t* h, float* x, int64_t n);

/* bfloat16 (the top 16 bits of binary32): RNE narrowing, exact widening.
 * Used only to measure what a bf16 pool would cost in accuracy (ROCm/ATOM
 * PR #2130, What: bf16's 3 fewer mantissa bits cost roughly 8x the error). */
uint16_t kdao_f32_to_bf16_rne(float x);
float kdao_bf16_to_f32(uint16_t h);
void kdao_f32_to_bf16_rne_array(const float* x, uint16_t* h, int64_t n);

/*
 * One decode launch, fp32 recurrence.
 *   pool       host pool [n_slots, H, K, V] (V fastest), element kind
 *              pool_kind (float for F32, uint16_t fp16 bits for F16,
 *              uint16_t bf16 bits for BF16).
 *              Updated in place: row t of request r writes its post-update
 *              state to slot slot_ids[r * n_rows + t]; the initial state is
 *              read from slot init_slot_ids[r] if init_slot_ids is not NULL,
 *              else from slot slot_ids[r * n_rows].  Slots not named are
 *              untouched.
 *   slot_ids   [n_req * n_rows], distinct, each in [0, n_slots).
 *   init_slot_ids  NULL or [n_req], each in [0, n_slots): where each
 *              request's initial state is read (an earlier step's accepted
 *              snapshot, or a checkpoint slot; ROCm/ATOM PR #2945, Changes:
 *              the same address function serves the initial state, the
 *              snapshots, and the checkpoint load).
 *   q, k, g    [n_req * n_rows, H, K]; v [.., H, V]; b [.., H]; fp32.
 *   out        [n_req * n_rows, H, V] fp32.
 * Returns KDAO_OK or KDAO_EARG (no partial writes on KDAO_EARG).
 */
int kdao_step_f32(void* pool, int pool_kind, int32_t n_slots, int32_t H,
                  int32_t K, int32_t V, const int32_t* slot_ids,
                  const int32_t* init_slot_ids, int32_t n_req, int32_t n_rows, const float* q,
                  const float* k, const float* v, const float* g,
                  const float* b, float scale, float* out);

/* The same loop carried out in fp64 on an fp64 pool (inputs widened). */
int kdao_step_f64(double* pool, int32_t n_slots, int32_t H, int32_t K,
                  int32_t V, const int32_t* slot_ids, const int32_t* init_slot_ids, int32_t n_req,
                  int32_t n_rows, const float* q, const float* k,
                  const float* v, const float* g, const float* b,
                  double scale, double* out);

/*
 * Prefill: whole sequences through the same recurrence, token by token
 * (ROCm/ATOM PR #2130, What and Depends on: the prefill kernel reads its
 * initial state from the pool in the pool's dtype and writes the final state
 * back; the recurrence is the decode step's, applied to every token of the
 * prompt in order).
 *   init_slot_ids  [n_seq]: slot of each sequence's initial state (widened).
 *   dst_slot_ids   NULL (= init_slot_ids) or [n_seq]: where the final state is
 *                  stored (narrowed).  Distinct, and none is another
 *                  sequence's initial slot.
 *   cu_seqlens     [n_seq + 1] non-decreasing token offsets: sequence s owns
 *                  tokens cu_seqlens[s] .. cu_seqlens[s + 1] - 1 of q, k, v,
 *                  g [T, H, K|V], b [T, H] and out [T, H, V].  Empty
 *                  sequences copy their state (widened, then narrowed).
 * Only the final state of each sequence is stored; out holds every token's
 * read-out.
 */
int kdao_prefill_f32(void* pool, int pool_kind, int32_t n_slots, int32_t H, int32_t K,
                     int32_t V, const int32_t* init_slot_ids, const int32_t* dst_slot_ids,
                     const int32_t* cu_seqlens, int32_t n_seq, const float* q, const float* k,
                     const float* v, const float* g, const float* b, float scale, float* out);
int kdao_prefill_f64(double* pool, int32_t n_slots, int32_t H, int32_t K, int32_t V,
                     const int32_t* init_slot_ids, const int32_t* dst_slot_ids,
                     const int32_t* cu_seqlens, int32_t n_seq, const float* q, const float* k,
                     const float* v, const float* g, const float* b, double scale,
                     double* out);

/*
 * Short causal convolution in front of the recurrence (q, k and v each pass
 * a depthwise causal convolution of 4 taps, then SiLU).  The conv state of a
 * slot holds the last 3 raw inputs of every channel in bfloat16: ROCm/ATOM
 * PR #2130, Memory: the per-slot remainder that does not follow the state
 * dtype is 1.91 MB over 69 layers = 3 entries x (3 x 12 x 128) channels x 2
 * bytes; ROCm/ATOM PR #2894 (the two-node trial): the conv reads a 3-entry
 * history, then writes back the old entries followed by the step's inputs.
 *
 *   conv_pool  [n_slots, 3, C] uint16 bf16 bits (entry 0 oldest), updated:
 *              row t of request r writes its history after token t -- the
 *              last 3 entries of (history, x_0 .. x_t) -- rounded to bf16
 *              to nearest even, to slot slot_ids[r * n_rows + t].
 *   slot_ids / init_slot_ids as in kdao_step_f32 (init NULL: the history is
 *              read from the row-0 slot).
 *   x          [n_req * n_rows, C] fp32 raw inputs; the rows of one launch use
 *              their fp32 inputs directly, only the stored history rounds.
 *   w          [C, 4] fp32 taps, w[c][3] multiplies the newest input.
 *   y          [n_req * n_rows, C] fp32 outputs:
 *              y_t = silu(sum_j w[j] * win[t + j]),  win = (hist, x_0 .. x_t),
 *              silu(s) = s / (1 + exp(-s)), the sum taken j = 0..3 in order.
 */
int kdao_conv_f32(uint16_t* conv_pool, int32_t n_slots, int32_t C,
                  const int32_t* slot_ids, const int32_t* init_slot_ids,
                  int32_t n_req, int32_t n_rows, const float* x, const float* w,
                  float* y);

/*
 * Planted-mistake switch, for the tests that show the pins catch a wrong
 * oracle.  0 = none (default).  Any other value changes one term of
 * kdao_step_f32 / kdao_step_f64 (see kda_oracle.c).  Never set outside those
 * tests.
 */
void kdao_set_mutation(int which);

#ifdef __cplusplus
}
#endif

#endif /* KDA_ORACLE_H */
