/*
 * kda_oracle.c -- plain, slow CPU oracle of the KDA decode update.
 *
 * TEST INFRASTRUCTURE ONLY (see kda_oracle.h): never linked into, loaded by
 * or called from the product library.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * The loop is written in the order the update is defined, one operation at
 * a time, with sequential sums and no blocking or reordering.
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int g_mutation = 0;

void kdao_set_mutation(int which) { g_mutation = which; }

/* ------------------------------------------------------------------------ */
/* binary16 conversions, from the IEEE 754 encoding definitions             */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return u;
}

static float bits_f32(uint32_t u) {
  float x;
  memcpy(&x, &u, sizeof x);
  return x;
}

/*
 * Round to nearest, ties to even.  binary16: 1 sign bit, 5 exponent bits
 * (bias 15), 10 fraction bits.  Largest finite 65504; smallest normal
 * 2^-14; smallest subnormal 2^-24.
 */
uint16_t kdao_f32_to_f16_rne(float x) {
  const uint32_t u = f32_bits(x);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t mag = u & 0x7fffffffu;

  if (mag > 0x7f800000u) { /* NaN: keep it a NaN, make it quiet */
    return (uint16_t)(sign | 0x7e00u | ((mag & 0x007fffffu) >> 13));
  }
  if (mag == 0x7f800000u) return (uint16_t)(sign | 0x7c00u); /* inf */

  const int32_t e32 = (int32_t)(mag >> 23);     /* biased, 0..254 */
  const int32_t e = e32 - 127;                   /* unbiased exponent */
  uint32_t frac = mag & 0x007fffffu;

  if (e >= -14) {
    /* Normal range of binary16 (before rounding). */
    uint32_t h = ((uint32_t)(e + 15) << 10) | (frac >> 13);
    const uint32_t rest = frac & 0x1fffu; /* 13 dropped bits */
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u;
    /* A carry out of the fraction bumps the exponent, which is the right
     * encoding; reaching exponent 31 means overflow to infinity. */
    if (h >= 0x7c00u) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | h);
  }

  /* Below the normal range: the result is a multiple of 2^-24. */
  if (e32 == 0) return sign; /* binary32 subnormal: < 2^-126, rounds to 0 */
  const uint32_t sig = frac | 0x00800000u;   /* value = sig * 2^(e - 23) */
  const int32_t shift = -e - 1;              /* value / 2^-24 = sig >> shift */
  if (shift > 24) return sign;               /* below half of 2^-24 */
  uint32_t h = sig >> shift;
  const uint32_t rest = sig & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rest > half || (rest == half && (h & 1u))) h += 1u;
  return (uint16_t)(sign | h); /* h == 0x400 is the smallest normal: right */
}

float kdao_f16_to_f32(uint16_t hbits) {
  const uint32_t sign = ((uint32_t)hbits & 0x8000u) << 16;
  const uint32_t e = ((uint32_t)hbits >> 10) & 0x1fu;
  const uint32_t frac = (uint32_t)hbits & 0x3ffu;
  if (e == 0) {
    /* zero or subnormal: frac * 2^-24, exact in binary32 */
    const float m = (float)frac * 0x1p-24f;
    return sign ? -m : m;
  }
  if (e == 31) return bits_f32(sign | 0x7f800000u | (frac << 13));
  return bits_f32(sign | ((e - 15u + 127u) << 23) | (frac << 13));
}

void kdao_f32_to_f16_rne_array(const float* x, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = kdao_f32_to_f16_rne(x[i]);
}

void kdao_f16_to_f32_array(const uint16_t* h, float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = kdao_f16_to_f32(h[i]);
}

/* bfloat16 keeps binary32's sign and 8-bit exponent and the top 7 fraction
 * bits; narrowing rounds the dropped 16 bits to nearest, ties to even (a
 * carry into the exponent is the right encoding, up to infinity). */
uint16_t kdao_f32_to_bf16_rne(float x) {
  const uint32_t u = f32_bits(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  const uint32_t rest = u & 0xffffu;
  uint32_t hi = u >> 16;
  if (rest > 0x8000u || (rest == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

float kdao_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

void kdao_f32_to_bf16_rne_array(const float* x, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = kdao_f32_to_bf16_rne(x[i]);
}

static float widen_any(const void* pool, int kind, int64_t i) {
  if (kind == KDAO_POOL_F32) return ((const float*)pool)[i];
  const uint16_t h = ((const uint16_t*)pool)[i];
  return kind == KDAO_POOL_F16 ? kdao_f16_to_f32(h) : kdao_bf16_to_f32(h);
}

static void narrow_any(void* pool, int kind, int64_t i, float x) {
  if (kind == KDAO_POOL_F32)
    ((float*)pool)[i] = x;
  else if (kind == KDAO_POOL_F16)
    ((uint16_t*)pool)[i] = kdao_f32_to_f16_rne(x);
  else
    ((uint16_t*)pool)[i] = kdao_f32_to_bf16_rne(x);
}

/* ------------------------------------------------------------------------ */
/* argument checks shared by both precisions                                */
/* ------------------------------------------------------------------------ */

static int check_args(const void* pool, int32_t n_slots, int32_t H, int32_t K,
                      int32_t V, const int32_t* slot_ids, const int32_t* init_slot_ids,
                      int32_t n_req, int32_t n_rows, const void* q, const void* k,
                      const void* v, const void* g, const void* b,
                      const void* out) {
  if (!pool || !slot_ids || !q || !k || !v || !g || !b || !out) return 0;
  if (n_slots <= 0 || H <= 0 || K <= 0 || V <= 0 || n_req < 0 || n_rows <= 0)
    return 0;
  const int64_t R = (int64_t)n_req * n_rows;
  for (int64_t i = 0; i < R; ++i)
    if (slot_ids[i] < 0 || slot_ids[i] >= n_slots) return 0;
  if (init_slot_ids)
    for (int32_t r = 0; r < n_req; ++r)
      if (init_slot_ids[r] < 0 || init_slot_ids[r] >= n_slots) return 0;
  return 1;
}

/* Element offset of the [K, V] state of (slot, head) inside the pool. */
static int64_t state_offset(int32_t slot, int32_t h, int32_t H, int32_t K,
                            int32_t V) {
  return ((int64_t)slot * H + h) * (int64_t)K * V;
}

/* ------------------------------------------------------------------------ */
/* fp32 recurrence                                                          */
/* ------------------------------------------------------------------------ */

/* One token of the recurrence on one head, fp32 (the order of the update's
 * definition: normalise, gate, decay, delta correction, rank-1 update, read
 * out the post-update state).  S [K, V] is updated in place; qn, kn, a, w, u
 * are work arrays; ov receives the V outputs. */
static void token_f32(float* S, int32_t K, int32_t V, const float* qv, const float* kv,
                      const float* gv, const float* vv, float bv, float scale, float* qn,
                      float* kn, float* a, float* w, float* u, float* ov) {
  const float eps = 1e-6f;

  /* L2 normalisation of q and k */
  float sq = 0.0f, sk = 0.0f;
  for (int32_t i = 0; i < K; ++i) sq = sq + qv[i] * qv[i];
  for (int32_t i = 0; i < K; ++i) sk = sk + kv[i] * kv[i];
  const float rq = g_mutation == 6 ? 1.0f / (sq + eps) : 1.0f / sqrtf(sq + eps);
  const float rk = 1.0f / sqrtf(sk + eps);
  for (int32_t i = 0; i < K; ++i) qn[i] = qv[i] * rq;
  for (int32_t i = 0; i < K; ++i) kn[i] = kv[i] * rk;

  /* per-key-channel decay and sigmoid gate */
  for (int32_t i = 0; i < K; ++i)
    a[i] = g_mutation == 1 ? 1.0f : (g_mutation == 8 ? expf(-gv[i]) : expf(gv[i]));
  const float beta = g_mutation == 11 ? 1.0f / (1.0f + expf(bv))
                                      : 1.0f / (1.0f + expf(-bv));

  /* S' = diag(a) S */
  for (int32_t i = 0; i < K; ++i)
    for (int32_t j = 0; j < V; ++j) S[(int64_t)i * V + j] = a[i] * S[(int64_t)i * V + j];

  if (g_mutation == 4) { /* planted: read-out before the update */
    for (int32_t j = 0; j < V; ++j) ov[j] = 0.0f;
    for (int32_t i = 0; i < K; ++i)
      for (int32_t j = 0; j < V; ++j) ov[j] = ov[j] + qn[i] * S[(int64_t)i * V + j];
    for (int32_t j = 0; j < V; ++j) ov[j] = scale * ov[j];
  }

  /* w = S'^T kn ; u = v - w.  Each w_j is the sum over i = 0..K-1 in
   * order; the loops run i-outer only so that rows are read
   * contiguously. */
  for (int32_t j = 0; j < V; ++j) w[j] = 0.0f;
  for (int32_t i = 0; i < K; ++i)
    for (int32_t j = 0; j < V; ++j) {
      const float s = g_mutation == 3 ? S[(int64_t)j * V + i] : S[(int64_t)i * V + j];
      w[j] = w[j] + kn[i] * s;
    }
  for (int32_t j = 0; j < V; ++j) u[j] = g_mutation == 2 ? vv[j] + w[j] : vv[j] - w[j];

  /* S = S' + (beta kn) u^T */
  for (int32_t i = 0; i < K; ++i) {
    const float bk = g_mutation == 5 ? kn[i] : beta * kn[i];
    for (int32_t j = 0; j < V; ++j)
      S[(int64_t)i * V + j] = S[(int64_t)i * V + j] + bk * u[j];
  }

  /* o = scale * S^T qn (post-update state), sums in i order */
  if (g_mutation != 4) {
    for (int32_t j = 0; j < V; ++j) w[j] = 0.0f;
    for (int32_t i = 0; i < K; ++i)
      for (int32_t j = 0; j < V; ++j) w[j] = w[j] + qn[i] * S[(int64_t)i * V + j];
    for (int32_t j = 0; j < V; ++j) ov[j] = (g_mutation == 7 ? scale * scale : scale) * w[j];
  }
}

int kdao_step_f32(void* pool, int pool_kind, int32_t n_slots, int32_t H,
                  int32_t K, int32_t V, const int32_t* slot_ids,
                  const int32_t* init_slot_ids, int32_t n_req, int32_t n_rows, const float* q,
                  const float* k, const float* v, const float* g,
                  const float* b, float scale, float* out) {
  if (pool_kind != KDAO_POOL_F32 && pool_kind != KDAO_POOL_F16 && pool_kind != KDAO_POOL_BF16)
    return KDAO_EARG;
  if (!check_args(pool, n_slots, H, K, V, slot_ids, init_slot_ids, n_req, n_rows, q, k, v, g,
                  b, out))
    return KDAO_EARG;

  float* S = (float*)malloc(sizeof(float) * (size_t)K * V);
  float* qn = (float*)malloc(sizeof(float) * (size_t)K);
  float* kn = (float*)malloc(sizeof(float) * (size_t)K);
  float* a = (float*)malloc(sizeof(float) * (size_t)K);
  float* w = (float*)malloc(sizeof(float) * (size_t)V);
  float* u = (float*)malloc(sizeof(float) * (size_t)V);
  if (!S || !qn || !kn || !a || !w || !u) {
    free(S); free(qn); free(kn); free(a); free(w); free(u);
    return KDAO_EARG;
  }

  for (int32_t r = 0; r < n_req; ++r) {
    for (int32_t h = 0; h < H; ++h) {
      /* initial state: the request's initial slot if given, else its row-0
       * slot; widened exactly */
      const int32_t s0 = init_slot_ids ? init_slot_ids[r] : slot_ids[(int64_t)r * n_rows];
      const int64_t off0 = state_offset(s0, h, H, K, V);
      for (int64_t e = 0; e < (int64_t)K * V; ++e)
        S[e] = widen_any(pool, pool_kind, off0 + e);

      for (int32_t t = 0; t < n_rows; ++t) {
        const int64_t rho = (int64_t)r * n_rows + t;
        if (g_mutation == 9 && t > 0) { /* planted: chain not carried */
          for (int64_t e = 0; e < (int64_t)K * V; ++e)
            S[e] = widen_any(pool, pool_kind, off0 + e);
        }
        token_f32(S, K, V, q + (rho * H + h) * K, k + (rho * H + h) * K, g + (rho * H + h) * K,
                  v + (rho * H + h) * V, b[rho * H + h], scale, qn, kn, a, w, u,
                  out + (rho * H + h) * V);

        /* store this token's state to its snapshot slot */
        const int32_t dst_slot = g_mutation == 10 ? slot_ids[(int64_t)r * n_rows] : slot_ids[rho];
        const int64_t offt = state_offset(dst_slot, h, H, K, V);
        for (int64_t e = 0; e < (int64_t)K * V; ++e) narrow_any(pool, pool_kind, offt + e, S[e]);
      }
    }
  }
  free(S); free(qn); free(kn); free(a); free(w); free(u);
  return KDAO_OK;
}

/* ------------------------------------------------------------------------ */
/* fp64 twin of the same loop                                               */
/* ------------------------------------------------------------------------ */

/* The same token in fp64 (inputs widened exactly). */
static void token_f64(double* S, int32_t K, int32_t V, const float* qv, const float* kv,
                      const float* gv, const float* vv, float b32, double scale, double* qn,
                      double* kn, double* a, double* w, double* u, double* ov) {
  const double eps = 1e-6;
  const double bv = (double)b32;

  double sq = 0.0, sk = 0.0;
  for (int32_t i = 0; i < K; ++i) sq = sq + (double)qv[i] * (double)qv[i];
  for (int32_t i = 0; i < K; ++i) sk = sk + (double)kv[i] * (double)kv[i];
  const double rq = g_mutation == 6 ? 1.0 / (sq + eps) : 1.0 / sqrt(sq + eps);
  const double rk = 1.0 / sqrt(sk + eps);
  for (int32_t i = 0; i < K; ++i) qn[i] = (double)qv[i] * rq;
  for (int32_t i = 0; i < K; ++i) kn[i] = (double)kv[i] * rk;

  for (int32_t i = 0; i < K; ++i)
    a[i] = g_mutation == 1 ? 1.0 : (g_mutation == 8 ? exp(-(double)gv[i]) : exp((double)gv[i]));
  const double beta = g_mutation == 11 ? 1.0 / (1.0 + exp(bv)) : 1.0 / (1.0 + exp(-bv));

  for (int32_t i = 0; i < K; ++i)
    for (int32_t j = 0; j < V; ++j) S[(int64_t)i * V + j] = a[i] * S[(int64_t)i * V + j];

  if (g_mutation == 4) {
    for (int32_t j = 0; j < V; ++j) ov[j] = 0.0;
    for (int32_t i = 0; i < K; ++i)
      for (int32_t j = 0; j < V; ++j) ov[j] = ov[j] + qn[i] * S[(int64_t)i * V + j];
    for (int32_t j = 0; j < V; ++j) ov[j] = scale * ov[j];
  }

  for (int32_t j = 0; j < V; ++j) w[j] = 0.0;
  for (int32_t i = 0; i < K; ++i)
    for (int32_t j = 0; j < V; ++j) {
      const double s = g_mutation == 3 ? S[(int64_t)j * V + i] : S[(int64_t)i * V + j];
      w[j] = w[j] + kn[i] * s;
    }
  for (int32_t j = 0; j < V; ++j)
    u[j] = g_mutation == 2 ? (double)vv[j] + w[j] : (double)vv[j] - w[j];

  for (int32_t i = 0; i < K; ++i) {
    const double bk = g_mutation == 5 ? kn[i] : beta * kn[i];
    for (int32_t j = 0; j < V; ++j)
      S[(int64_t)i * V + j] = S[(int64_t)i * V + j] + bk * u[j];
  }

  if (g_mutation != 4) {
    for (int32_t j = 0; j < V; ++j) w[j] = 0.0;
    for (int32_t i = 0; i < K; ++i)
      for (int32_t j = 0; j < V; ++j) w[j] = w[j] + qn[i] * S[(int64_t)i * V + j];
    for (int32_t j = 0; j < V; ++j) ov[j] = (g_mutation == 7 ? scale * scale : scale) * w[j];
  }
}

int kdao_step_f64(double* pool, int32_t n_slots, int32_t H, int32_t K,
                  int32_t V, const int32_t* slot_ids, const int32_t* init_slot_ids, int32_t n_req,
                  int32_t n_rows, const float* q, const float* k,
                  const float* v, const float* g, const float* b,
                  double scale, double* out) {
  if (!check_args(pool, n_slots, H, K, V, slot_ids, init_slot_ids, n_req, n_rows, q, k, v, g,
                  b, out))
    return KDAO_EARG;

  double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
  double* qn = (double*)malloc(sizeof(double) * (size_t)K);
  double* kn = (double*)malloc(sizeof(double) * (size_t)K);
  double* a = (double*)malloc(sizeof(double) * (size_t)K);
  double* w = (double*)malloc(sizeof(double) * (size_t)V);
  double* u = (double*)malloc(sizeof(double) * (size_t)V);
  if (!S || !qn || !kn || !a || !w || !u) {
    free(S); free(qn); free(kn); free(a); free(w); free(u);
    return KDAO_EARG;
  }

  for (int32_t r = 0; r < n_req; ++r) {
    for (int32_t h = 0; h < H; ++h) {
      const int32_t s0 = init_slot_ids ? init_slot_ids[r] : slot_ids[(int64_t)r * n_rows];
      const int64_t off0 = state_offset(s0, h, H, K, V);
      for (int64_t e = 0; e < (int64_t)K * V; ++e) S[e] = pool[off0 + e];

      for (int32_t t = 0; t < n_rows; ++t) {
        const int64_t rho = (int64_t)r * n_rows + t;
        if (g_mutation == 9 && t > 0)
          for (int64_t e = 0; e < (int64_t)K * V; ++e) S[e] = pool[off0 + e];
        token_f64(S, K, V, q + (rho * H + h) * K, k + (rho * H + h) * K, g + (rho * H + h) * K,
                  v + (rho * H + h) * V, b[rho * H + h], scale, qn, kn, a, w, u,
                  out + (rho * H + h) * V);

        const int32_t dst_slot = g_mutation == 10 ? slot_ids[(int64_t)r * n_rows] : slot_ids[rho];
        const int64_t offt = state_offset(dst_slot, h, H, K, V);
        for (int64_t e = 0; e < (int64_t)K * V; ++e) pool[offt + e] = S[e];
      }
    }
  }
  free(S); free(qn); free(kn); free(a); free(w); free(u);
  return KDAO_OK;
}

/* ------------------------------------------------------------------------ */
/* prefill: whole sequences through the same per-token recurrence           */
/* ------------------------------------------------------------------------ */

static int check_prefill(const void* pool, int32_t n_slots, int32_t H, int32_t K, int32_t V,
                         const int32_t* init_slot_ids, const int32_t* dst_slot_ids,
                         const int32_t* cu_seqlens, int32_t n_seq, const void* q,
                         const void* k, const void* v, const void* g, const void* b,
                         const void* out) {
  if (!pool || !init_slot_ids || !cu_seqlens || !q || !k || !v || !g || !b || !out) return 0;
  if (n_slots <= 0 || H <= 0 || K <= 0 || V <= 0 || n_seq < 0) return 0;
  if (n_seq > 0 && cu_seqlens[0] < 0) return 0;
  for (int32_t s = 0; s < n_seq; ++s) {
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return 0;
    if (init_slot_ids[s] < 0 || init_slot_ids[s] >= n_slots) return 0;
    const int32_t d = dst_slot_ids ? dst_slot_ids[s] : init_slot_ids[s];
    if (d < 0 || d >= n_slots) return 0;
  }
  /* a destination slot is written by one sequence only and is no other
   * sequence's initial slot: then every sequence reads the pool as it was
   * before the launch, whatever the order of the sequences */
  for (int32_t s = 0; s < n_seq; ++s) {
    const int32_t d = dst_slot_ids ? dst_slot_ids[s] : init_slot_ids[s];
    for (int32_t u = 0; u < n_seq; ++u) {
      if (u == s) continue;
      const int32_t du = dst_slot_ids ? dst_slot_ids[u] : init_slot_ids[u];
      if (du == d || init_slot_ids[u] == d) return 0;
    }
  }
  return 1;
}

int kdao_prefill_f32(void* pool, int pool_kind, int32_t n_slots, int32_t H, int32_t K,
                     int32_t V, const int32_t* init_slot_ids, const int32_t* dst_slot_ids,
                     const int32_t* cu_seqlens, int32_t n_seq, const float* q, const float* k,
                     const float* v, const float* g, const float* b, float scale, float* out) {
  if (pool_kind != KDAO_POOL_F32 && pool_kind != KDAO_POOL_F16 && pool_kind != KDAO_POOL_BF16)
    return KDAO_EARG;
  if (!check_prefill(pool, n_slots, H, K, V, init_slot_ids, dst_slot_ids, cu_seqlens, n_seq, q,
                     k, v, g, b, out))
    return KDAO_EARG;
  float* S = (float*)malloc(sizeof(float) * (size_t)K * V);
  float* qn = (float*)malloc(sizeof(float) * (size_t)K);
  float* kn = (float*)malloc(sizeof(float) * (size_t)K);
  float* a = (float*)malloc(sizeof(float) * (size_t)K);
  float* w = (float*)malloc(sizeof(float) * (size_t)V);
  float* u = (float*)malloc(sizeof(float) * (size_t)V);
  if (!S || !qn || !kn || !a || !w || !u) {
    free(S); free(qn); free(kn); free(a); free(w); free(u);
    return KDAO_EARG;
  }
  for (int32_t sq = 0; sq < n_seq; ++sq) {
    for (int32_t h = 0; h < H; ++h) {
      const int64_t off0 = state_offset(init_slot_ids[sq], h, H, K, V);
      for (int64_t e = 0; e < (int64_t)K * V; ++e) S[e] = widen_any(pool, pool_kind, off0 + e);
      for (int64_t t = cu_seqlens[sq]; t < cu_seqlens[sq + 1]; ++t)
        token_f32(S, K, V, q + (t * H + h) * K, k + (t * H + h) * K, g + (t * H + h) * K,
                  v + (t * H + h) * V, b[t * H + h], scale, qn, kn, a, w, u,
                  out + (t * H + h) * V);
      const int32_t d = dst_slot_ids ? dst_slot_ids[sq] : init_slot_ids[sq];
      const int64_t offd = state_offset(d, h, H, K, V);
      for (int64_t e = 0; e < (int64_t)K * V; ++e) narrow_any(pool, pool_kind, offd + e, S[e]);
    }
  }
  free(S); free(qn); free(kn); free(a); free(w); free(u);
  return KDAO_OK;
}

int kdao_prefill_f64(double* pool, int32_t n_slots, int32_t H, int32_t K, int32_t V,
                     const int32_t* init_slot_ids, const int32_t* dst_slot_ids,
                     const int32_t* cu_seqlens, int32_t n_seq, const float* q, const float* k,
                     const float* v, const float* g, const float* b, double scale,
                     double* out) {
  if (!check_prefill(pool, n_slots, H, K, V, init_slot_ids, dst_slot_ids, cu_seqlens, n_seq, q,
                     k, v, g, b, out))
    return KDAO_EARG;
  double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
  double* qn = (double*)malloc(sizeof(double) * (size_t)K);
  double* kn = (double*)malloc(sizeof(double) * (size_t)K);
  double* a = (double*)malloc(sizeof(double) * (size_t)K);
  double* w = (double*)malloc(sizeof(double) * (size_t)V);
  double* u = (double*)malloc(sizeof(double) * (size_t)V);
  if (!S || !qn || !kn || !a || !w || !u) {
    free(S); free(qn); free(kn); free(a); free(w); free(u);
    return KDAO_EARG;
  }
  for (int32_t sq = 0; sq < n_seq; ++sq) {
    for (int32_t h = 0; h < H; ++h) {
      const int64_t off0 = state_offset(init_slot_ids[sq], h, H, K, V);
      for (int64_t e = 0; e < (int64_t)K * V; ++e) S[e] = pool[off0 + e];
      for (int64_t t = cu_seqlens[sq]; t < cu_seqlens[sq + 1]; ++t)
        token_f64(S, K, V, q + (t * H + h) * K, k + (t * H + h) * K, g + (t * H + h) * K,
                  v + (t * H + h) * V, b[t * H + h], scale, qn, kn, a, w, u,
                  out + (t * H + h) * V);
      const int32_t d = dst_slot_ids ? dst_slot_ids[sq] : init_slot_ids[sq];
      const int64_t offd = state_offset(d, h, H, K, V);
      for (int64_t e = 0; e < (int64_t)K * V; ++e) pool[offd + e] = S[e];
    }
  }
  free(S); free(qn); free(kn); free(a); free(w); free(u);
  return KDAO_OK;
}

/* ------------------------------------------------------------------------ */
/* short causal convolution (see kda_oracle.h)                              */
/* ------------------------------------------------------------------------ */

int kdao_conv_f32(uint16_t* conv_pool, int32_t n_slots, int32_t C,
                  const int32_t* slot_ids, const int32_t* init_slot_ids,
                  int32_t n_req, int32_t n_rows, const float* x, const float* w,
                  float* y) {
  if (!conv_pool || !slot_ids || !x || !w || !y) return KDAO_EARG;
  if (n_slots <= 0 || C <= 0 || n_req < 0 || n_rows <= 0) return KDAO_EARG;
  const int64_t R = (int64_t)n_req * n_rows;
  for (int64_t i = 0; i < R; ++i)
    if (slot_ids[i] < 0 || slot_ids[i] >= n_slots) return KDAO_EARG;
  if (init_slot_ids)
    for (int32_t r = 0; r < n_req; ++r)
      if (init_slot_ids[r] < 0 || init_slot_ids[r] >= n_slots) return KDAO_EARG;

  const int32_t HIST = 3, TAPS = 4;
  float* win = (float*)malloc(sizeof(float) * (size_t)(HIST + n_rows));
  uint16_t* snap = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)R * HIST * C);
  if (!win || !snap) {
    free(win); free(snap);
    return KDAO_EARG;
  }
  /* all reads of a launch see the pool as it was before the launch: the
   * snapshots are staged and written at the end */
  for (int32_t r = 0; r < n_req; ++r) {
    const int32_t s0 = init_slot_ids ? init_slot_ids[r] : slot_ids[(int64_t)r * n_rows];
    for (int32_t c = 0; c < C; ++c) {
      for (int32_t e = 0; e < HIST; ++e)
        win[e] = kdao_bf16_to_f32(conv_pool[((int64_t)s0 * HIST + e) * C + c]);
      for (int32_t t = 0; t < n_rows; ++t) win[HIST + t] = x[((int64_t)r * n_rows + t) * C + c];
      for (int32_t t = 0; t < n_rows; ++t) {
        const int64_t rho = (int64_t)r * n_rows + t;
        float acc = 0.0f;
        for (int32_t j = 0; j < TAPS; ++j) acc = acc + w[(int64_t)c * TAPS + j] * win[t + j];
        y[rho * C + c] = g_mutation == 12 ? acc : acc / (1.0f + expf(-acc));
        for (int32_t e = 0; e < HIST; ++e)
          snap[(rho * HIST + e) * C + c] = kdao_f32_to_bf16_rne(win[t + 1 + e]);
      }
    }
  }
  for (int64_t rho = 0; rho < R; ++rho)
    for (int32_t e = 0; e < HIST; ++e)
      for (int32_t c = 0; c < C; ++c)
        conv_pool[((int64_t)slot_ids[rho] * HIST + e) * C + c] = snap[(rho * HIST + e) * C + c];
  free(win);
  free(snap);
  return KDAO_OK;
}
