// kda_prefill.hip -- gfx950 (MI355X) chunked prefill of the KDA recurrence.
//
// A prefill runs a whole prompt through the same recurrence as decode,
//   S_t = diag(a_t) S_(t-1) + kn_t Delta_t^T,  Delta_t = beta_t (v_t - (diag(a_t) S_(t-1))^T kn_t),
//   o_t = scale S_t^T qn_t,
// starting from the sequence's slot of the state pool (fp32, or fp16 widened
// exactly) and storing only the final state (fp16: rounded to nearest
// even).  ROCm/ATOM PR #2130 (What, Depends on) is the source: every path,
// prefill included, reads and writes the state in the pool's own dtype while
// the recurrence runs in fp32, and the prefill kernel takes its initial
// state from the pool.
//
// Chunked form.  Inside a chunk of C tokens let G_t be the inclusive
// cumulative log-decay from the chunk start (per key channel).  Unrolling
// the recurrence gives, with S0 the state at the chunk start,
//   (I + A) Delta = beta V - Kb S0,          Kb_t = beta_t kn_t e^(G_t),
//   A_ts = beta_t sum_i kn_ti kn_si e^(G_ti - G_si)           (s < t),
//   o_t  = scale (Qg S0 + P Delta)_t,        Qg_t = qn_t e^(G_t),
//   P_ts = sum_i qn_ti kn_si e^(G_ti - G_si)                   (s <= t),
//   S_C  = e^(G_C) S0 + Kd^T Delta,          Kd_s = kn_s e^(G_C - G_s).
// Every product over the 128 key channels or over the C tokens is a dense
// contraction and runs on the matrix cores (v_mfma_f32_16x16x4_f32: fp32
// operands, fp32 accumulation).
//
// Bounded exponentials.  A and P need e^(G_t - G_s) <= 1 as a product of a
// t-factor and an s-factor.  Tokens are grouped in blocks of 16; for row
// block bt the reference is the cumulative decay just before the block, so
// the t-factor e^(G_t - G_ref) is <= 1 and, for s in an earlier block, the
// s-factor e^(G_ref - G_s) is <= 1 too.  Inside the diagonal block the
// s-factor exceeds 1 by at most the block's own decay; should that exceed
// e^80 for some channel (a decay of more than 80 nats within 16 tokens) the
// block is computed pair by pair instead.  All exponents are formed from
// block-local sums, so the ones that matter (close tokens) are small and
// accurate.
//
// Work decomposition.  One workgroup = one (sequence, head); its 4
// wavefronts split the 128 value columns (32 each) for everything that
// touches the state, and split the chunk's token blocks for the per-chunk
// quantities (norms, decays, A, P, the diagonal inverses), which they share
// through LDS.  The state slice of a wave stays in registers, in the matrix
// cores' accumulator layout, for the whole prompt; that layout is also a
// valid B operand for the next contraction over the key channels (the
// k-order of a 16x16x4 step is permuted to match, and the A operand is read
// from LDS in the same order).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kda_decode.h"
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kPWaves = 4;     // wavefronts per workgroup
constexpr int kPCols = 32;     // value columns per wavefront
constexpr int kLdK = 132;      // row stride (floats) of [C][128] LDS arrays
constexpr float kDiagLimit = 80.0f;  // largest in-block decay (nats) of the factored path
constexpr int32_t kDefaultChunk = 64;

struct PrefillArgs {
  void* pool;
  const int32_t* init_ids;
  const int32_t* dst_ids;  // nullable: store to the initial slot
  const int32_t* cu;
  const float* q;
  const float* k;
  const float* v;
  const float* g;
  const float* b;
  float* out;
  int64_t n_tokens;
  int32_t n_slots;
  int32_t H;
  int32_t n_seq;
  float scale;
};

__device__ __forceinline__ f4 mma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// sum over the 4 lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float group_sum(float x) { return sum_xor32(sum_xor16(x)); }

// inclusive prefix sum over the 16 lanes of a DPP row (row_shr with zero fill)
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x110 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_scan(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  return x;
}

template <typename T>
__device__ __forceinline__ float widen1(const T* p) { return static_cast<float>(*p); }

template <typename T>
__device__ __forceinline__ void narrow1(T* p, float x) {
  if constexpr (sizeof(T) == 2) {
    asm("" : "+v"(x));  // store RNE of the rounded fp32 value (no fused narrowing)
    *p = static_cast<T>(x);
  } else {
    *p = x;
  }
}

// Chunk of NB blocks of 16 tokens (C = 16 NB).  Waves w < NB own token block
// w for the per-chunk quantities; every wave owns value columns
// 32 w .. 32 w + 31 of the state.
template <typename T, int NB>
__global__ __launch_bounds__(64 * kPWaves) void kda_prefill_kernel(PrefillArgs a) {
  constexpr int C = 16 * NB;
  constexpr int LdC = C + 4;  // row stride of [C][C] and [128][C] arrays
  // kn, then -Kb (A operand of R = beta V - Kb S)
  __shared__ __attribute__((aligned(16))) float sX[C * kLdK];
  // block-local cumulative log-decay, then Qg
  __shared__ __attribute__((aligned(16))) float sY[C * kLdK];
  __shared__ __attribute__((aligned(16))) float sKdT[128 * LdC];  // Kd^T
  __shared__ __attribute__((aligned(16))) float sA[C * LdC];      // -A (strictly lower)
  __shared__ __attribute__((aligned(16))) float sP[C * LdC];      // P (lower)
  __shared__ __attribute__((aligned(16))) float sTd[NB][16 * 20]; // (I + A_bb)^-1
  __shared__ float sBtot[NB][128];  // per block: sum of g over its tokens
  __shared__ float sGC[128];        // e^(G_C)
  __shared__ float sBeta[C];

  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int li = lane % 16;  // MFMA row / column index
  const int gq = lane / 16;  // lane group
  const int seq = blockIdx.x / a.H;
  const int h = blockIdx.x % a.H;

  const int64_t t0 = a.cu[seq];
  const int64_t t1 = a.cu[seq + 1];
  const int32_t init = a.init_ids[seq];
  const int32_t dst = a.dst_ids != nullptr ? a.dst_ids[seq] : init;
  if (!(t0 >= 0 && t0 <= t1 && t1 <= a.n_tokens && init >= 0 && init < a.n_slots && dst >= 0 &&
        dst < a.n_slots))
    return;  // refused by the host checks; never touch memory outside the launch's bounds

  const int64_t hk = static_cast<int64_t>(a.H) * 128;  // floats per token of q, k, g, v, out
  const int col_w = kPCols * wave;                       // this wave's first value column

  // -- initial state slice: S[sb][cb] holds rows 16 sb + 4 gq + r, column
  //    col_w + 16 cb + li (the 16x16 accumulator layout)
  const T* pool = static_cast<const T*>(a.pool);
  const int64_t head_off = static_cast<int64_t>(h) * 128 * 128;
  f4 S[8][2];
  {
    const T* src = pool + static_cast<int64_t>(init) * a.H * 128 * 128 + head_off;
#pragma unroll
    for (int sb = 0; sb < 8; ++sb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[sb][cb][r] = widen1(src + (16 * sb + 4 * gq + r) * 128 + col_w + 16 * cb + li);
  }

  for (int64_t c0 = t0; c0 < t1; c0 += C) {
    const int n = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);

    // ---- per-chunk quantities: wave w < NB, token 16 w + li, channels 32 gq .. 32 gq + 31
    float qn[32], kn[32], gl[32];
    float beta = 0.0f;
    const bool tok_wave = wave < NB;
    if (tok_wave) {
      const int tl = 16 * wave + li;
      const bool valid = tl < n;
      float sq = 0.0f, sk = 0.0f;
      if (valid) {
        const int64_t off = (c0 + tl) * hk + static_cast<int64_t>(h) * 128 + 32 * gq;
#pragma unroll
        for (int m = 0; m < 32; m += 4) {
          const f4 x = *reinterpret_cast<const f4*>(a.q + off + m);
          const f4 y = *reinterpret_cast<const f4*>(a.k + off + m);
          const f4 z = *reinterpret_cast<const f4*>(a.g + off + m);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qn[m + e] = x[e];
            kn[m + e] = y[e];
            gl[m + e] = z[e];
          }
        }
        beta = 1.0f / (1.0f + expf(-a.b[(c0 + tl) * a.H + h]));
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) qn[i] = kn[i] = gl[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        sq = fmaf(qn[i], qn[i], sq);
        sk = fmaf(kn[i], kn[i], sk);
      }
      const float rq = 1.0f / sqrtf(group_sum(sq) + 1e-6f);
      const float rk = 1.0f / sqrtf(group_sum(sk) + 1e-6f);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        qn[i] *= rq;
        kn[i] *= rk;
        gl[i] = row_scan(gl[i]);  // block-local inclusive cumulative log-decay
      }
      float* xr = sX + tl * kLdK + 32 * gq;
      float* yr = sY + tl * kLdK + 32 * gq;
#pragma unroll
      for (int m = 0; m < 32; m += 4) {
        *reinterpret_cast<f4*>(xr + m) = f4{kn[m], kn[m + 1], kn[m + 2], kn[m + 3]};
        *reinterpret_cast<f4*>(yr + m) = f4{gl[m], gl[m + 1], gl[m + 2], gl[m + 3]};
      }
      if (li == 15) {
#pragma unroll
        for (int i = 0; i < 32; ++i) sBtot[wave][32 * gq + i] = gl[i];
      }
      if (gq == 0) sBeta[tl] = beta;
    }
    __syncthreads();

    // ---- A and P, row block w: t-factors e^(G_t - G_ref) = e^(gl_t)
    if (tok_wave) {
      const int w = wave;
      float lq[32], lk[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float e = expf(gl[i]);
        lq[i] = qn[i] * e;
        lk[i] = (beta * kn[i]) * e;
      }
      // in-block decay beyond the factored range: this wave's block goes pair by pair
      float span = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) span = fmaxf(span, -gl[i]);
      const bool exact_diag = __builtin_amdgcn_ballot_w64(span > kDiagLimit) != 0;

      // column blocks bs = w, w - 1, .., 0; cum = sum of Btot_u over bs <= u < w
      float cum[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) cum[i] = 0.0f;
      for (int bs = w; bs >= 0; --bs) {
        if (bs < w) {
#pragma unroll
          for (int i = 0; i < 32; ++i) cum[i] += sBtot[bs][32 * gq + i];
        }
        // s-factors for token s = 16 bs + li, channels 32 gq + i:
        // e^(G_ref - G_s) = e^(cum - gl_s)
        const float* kr = sX + (16 * bs + li) * kLdK + 32 * gq;
        const float* gr = sY + (16 * bs + li) * kLdK + 32 * gq;
        f4 accp = {0.f, 0.f, 0.f, 0.f}, acca = {0.f, 0.f, 0.f, 0.f};
        if (bs < w || !exact_diag) {
#pragma unroll
          for (int m = 0; m < 32; m += 4) {
            const f4 kx = *reinterpret_cast<const f4*>(kr + m);
            const f4 gx = *reinterpret_cast<const f4*>(gr + m);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float rf = kx[e] * expf(cum[m + e] - gx[e]);
              accp = mma(lq[m + e], rf, accp);
              acca = mma(lk[m + e], rf, acca);
            }
          }
        }
        // accumulator layout: row 16 w + 4 gq + r, column 16 bs + li
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = 4 * gq + r;
          float p = accp[r], x = acca[r];
          if (bs == w) {
            if (li > tr) p = 0.0f;
            if (li >= tr) x = 0.0f;
          }
          sP[(16 * w + tr) * LdC + 16 * bs + li] = p;
          sA[(16 * w + tr) * LdC + 16 * bs + li] = -x;
        }
      }
      if (exact_diag) {
        // pair by pair: lane (li = t, gq) sums its 32 channels for every s <= t
        const float* grow = sY + 16 * w * kLdK + 32 * gq;
        const float* krow = sX + 16 * w * kLdK + 32 * gq;
        for (int s = 0; s < 16; ++s) {
          float pp = 0.0f, pa = 0.0f;
          if (s <= li) {
#pragma unroll 4
            for (int i = 0; i < 32; ++i) {
              const float f = krow[s * kLdK + i] * expf(gl[i] - grow[s * kLdK + i]);
              pp = fmaf(qn[i], f, pp);
              pa = fmaf(kn[i], f, pa);
            }
          }
          pp = group_sum(pp);
          pa = group_sum(pa);
          if (gq == 0) {
            sP[(16 * w + li) * LdC + 16 * w + s] = s <= li ? pp : 0.0f;
            sA[(16 * w + li) * LdC + 16 * w + s] = s < li ? -(beta * pa) : 0.0f;
          }
        }
      }
    }
    __syncthreads();

    // ---- operands of the state contractions; diagonal inverses
    if (tok_wave) {
      const int w = wave;
      const int tl = 16 * w + li;
      float before[32], after[32];  // sums of Btot over blocks before / after w
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        float sb = 0.0f, sa = 0.0f;
        for (int u = 0; u < w; ++u) sb += sBtot[u][32 * gq + i];
        for (int u = w + 1; u < NB; ++u) sa += sBtot[u][32 * gq + i];
        before[i] = sb;
        after[i] = sa + (sBtot[w][32 * gq + i] - gl[i]);  // G_C - G_t
      }
      float* xr = sX + tl * kLdK + 32 * gq;
      float* yr = sY + tl * kLdK + 32 * gq;
#pragma unroll
      for (int m = 0; m < 32; m += 4) {
        f4 nkb, qg;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float eg = expf(before[m + e] + gl[m + e]);  // e^(G_t)
          nkb[e] = -((beta * kn[m + e]) * eg);
          qg[e] = qn[m + e] * eg;
        }
        *reinterpret_cast<f4*>(xr + m) = nkb;
        *reinterpret_cast<f4*>(yr + m) = qg;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) sKdT[(32 * gq + i) * LdC + tl] = kn[i] * expf(after[i]);
      // (I + A_ww)^-1 by forward substitution, one column per lane of group 0
      if (gq == 0) {
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          float acc = t == li ? 1.0f : 0.0f;
#pragma unroll
          for (int s = 0; s < t; ++s) acc = fmaf(sA[(16 * w + t) * LdC + 16 * w + s], x[s], acc);
          x[t] = acc;  // sA holds -A
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) sTd[w][t * 20 + li] = x[t];
      }
    }
    if (wave == 0) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float gc = 0.0f;
        for (int u = 0; u < NB; ++u) gc += sBtot[u][2 * lane + e];
        sGC[2 * lane + e] = expf(gc);
      }
    }
    __syncthreads();

    // ---- the state contractions, this wave's 32 value columns
    // R = beta V - Kb S  (token block tb: rows 16 tb + 4 gq + r)
    f4 D[NB][2];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tl = 16 * tb + 4 * gq + r;
          D[tb][cb][r] = tl < n ? sBeta[tl] * a.v[(c0 + tl) * hk + static_cast<int64_t>(h) * 128 +
                                                  col_w + 16 * cb + li]
                               : 0.0f;
        }
      }
#pragma unroll
      for (int sb = 0; sb < 8; ++sb) {
        const f4 x = *reinterpret_cast<const f4*>(sX + (16 * tb + li) * kLdK + 16 * sb + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          D[tb][0] = mma(x[r], S[sb][0][r], D[tb][0]);
          D[tb][1] = mma(x[r], S[sb][1][r], D[tb][1]);
        }
      }
    }
    // Delta = (I + A)^-1 R, block by block: Delta_b = T_bb (R_b - sum_{k<b} A_bk Delta_k)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int k = 0; k < b; ++k) {
        const f4 x = *reinterpret_cast<const f4*>(sA + (16 * b + li) * LdC + 16 * k + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          D[b][0] = mma(x[r], D[k][0][r], D[b][0]);
          D[b][1] = mma(x[r], D[k][1][r], D[b][1]);
        }
      }
      const f4 x = *reinterpret_cast<const f4*>(&sTd[b][li * 20 + 4 * gq]);
      f4 y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y0 = mma(x[r], D[b][0][r], y0);
        y1 = mma(x[r], D[b][1][r], y1);
      }
      D[b][0] = y0;
      D[b][1] = y1;
    }
    // o = scale (Qg S + P Delta)
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      f4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sb = 0; sb < 8; ++sb) {
        const f4 x = *reinterpret_cast<const f4*>(sY + (16 * tb + li) * kLdK + 16 * sb + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o0 = mma(x[r], S[sb][0][r], o0);
          o1 = mma(x[r], S[sb][1][r], o1);
        }
      }
#pragma unroll
      for (int kb = 0; kb <= tb; ++kb) {
        const f4 x = *reinterpret_cast<const f4*>(sP + (16 * tb + li) * LdC + 16 * kb + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o0 = mma(x[r], D[kb][0][r], o0);
          o1 = mma(x[r], D[kb][1][r], o1);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tl = 16 * tb + 4 * gq + r;
        if (tl < n) {
          float* op = a.out + (c0 + tl) * hk + static_cast<int64_t>(h) * 128 + col_w + li;
          op[0] = a.scale * o0[r];
          op[16] = a.scale * o1[r];
        }
      }
    }
    // S = e^(G_C) S + Kd^T Delta
#pragma unroll
    for (int sb = 0; sb < 8; ++sb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d = sGC[16 * sb + 4 * gq + r];
        S[sb][0][r] *= d;
        S[sb][1][r] *= d;
      }
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        const f4 x = *reinterpret_cast<const f4*>(sKdT + (16 * sb + li) * LdC + 16 * tb + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          S[sb][0] = mma(x[r], D[tb][0][r], S[sb][0]);
          S[sb][1] = mma(x[r], D[tb][1][r], S[sb][1]);
        }
      }
    }
    __syncthreads();  // the next chunk overwrites the LDS operands
  }

  // -- final state to the destination slot
  T* dstp = static_cast<T*>(a.pool) + static_cast<int64_t>(dst) * a.H * 128 * 128 + head_off;
#pragma unroll
  for (int sb = 0; sb < 8; ++sb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        narrow1(dstp + (16 * sb + 4 * gq + r) * 128 + col_w + 16 * cb + li, S[sb][cb][r]);
}

template <typename T, int NB>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((kda_prefill_kernel<T, NB>), dim3(static_cast<uint32_t>(a.n_seq) * a.H),
                     dim3(64 * kPWaves), 0, s, a);
  return hipGetLastError();
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace
}  // namespace kda

using namespace kda;

extern "C" int kda_prefill(const kda_pool* pool, const int32_t* init_slot_ids,
                           const int32_t* dst_slot_ids, const int32_t* cu_seqlens, const float* q,
                           const float* k, const float* v, const float* g, const float* b,
                           float* out, int32_t n_seq, int64_t n_tokens, kda_dtype state_dtype,
                           float scale, const kda_prefill_opts* opts, void* stream) {
  // dtype, shape, and at most one sequence per slot (destinations are distinct)
  const int rc = check_common(pool, n_seq, 1, state_dtype);
  if (rc != KDA_OK) return rc;
  if (n_tokens < 0) return KDA_ERR_ARG;
  if (static_cast<int64_t>(n_seq) * pool->H > INT32_MAX) return KDA_ERR_ARG;
  const int32_t chunk = opts != nullptr && opts->chunk != 0 ? opts->chunk : kDefaultChunk;
  if (chunk != 32 && chunk != 64) return KDA_ERR_ARG;
  if (n_seq == 0) return KDA_OK;
  if (init_slot_ids == nullptr || cu_seqlens == nullptr) return KDA_ERR_NULL;
  if (n_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || g == nullptr ||
                       b == nullptr || out == nullptr))
    return KDA_ERR_NULL;
  if (!std::isfinite(scale)) return KDA_ERR_ARG;
  if (!al16(pool->base) || !al16(q) || !al16(k) || !al16(g) || !al4(v) || !al4(out) || !al4(b) ||
      !al4(init_slot_ids) || !al4(dst_slot_ids) || !al4(cu_seqlens))
    return KDA_ERR_ALIGN;
  PrefillArgs a;
  a.pool = pool->base;
  a.init_ids = init_slot_ids;
  a.dst_ids = dst_slot_ids;
  a.cu = cu_seqlens;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.b = b;
  a.out = out;
  a.n_tokens = n_tokens;
  a.n_slots = pool->n_slots;
  a.H = pool->H;
  a.n_seq = n_seq;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (state_dtype == KDA_F32)
    err = chunk == 64 ? launch_prefill<float, 4>(a, s) : launch_prefill<float, 2>(a, s);
  else
    err = chunk == 64 ? launch_prefill<_Float16, 4>(a, s) : launch_prefill<_Float16, 2>(a, s);
  return err == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}
