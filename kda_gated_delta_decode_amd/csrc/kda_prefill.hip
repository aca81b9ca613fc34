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
// Bounded exponentials.  A and P need 2^(G_t - G_s) <= 1 (decays are kept
// in log2 units, g log2 e, so each exponential is one v_exp_f32) as a
// product of a t-factor and an s-factor.  Tokens are grouped in blocks of
// 16; for row block bt the reference is the cumulative decay just before the
// block, so the t-factor 2^(G_t - G_ref) is <= 1 and, for s in an earlier
// block, the s-factor 2^(G_ref - G_s) is <= 1 too.  Inside the diagonal
// block the s-factor exceeds 1 by at most the block's own decay; should that
// exceed 2^115 (80 nats) for some channel, the block is computed pair by
// pair instead.  All exponents are formed from block-local sums, so the ones
// that matter (close tokens) are small and accurate.  Kd's exponent G_C - G_s
// is summed from the decays after token s (in its block, then the totals of
// the later blocks), never taken as a difference of cumulative sums: for the
// last tokens of a chunk, whose Kd rows are the largest, it is then exactly 0
// or small, where a difference would leave about one ulp of the chunk's total
// decay (a relative error of 1e-6 in Kd at a total of 25 in log2 units).
// In the 32-token kernel the block-local cumulative decays are summed in fp64
// and kept as fp32 high and low parts (see row_scan2), and A and P take both:
// their in-block factors 2^(G_t - G_s) are products of 2^(+-G) factors whose
// exponents are large where the decay between t and s is small, so one ulp of
// G would be a relative error of 1e-6 in an O(1) factor.  (The 64-token
// kernel keeps plain sums: its LDS has no room for the low parts.)
// P's diagonal, qn_t . kn_t with no decay, is summed without the two
// exponentials: their per-channel rounding (about an ulp each, from
// v_exp_f32) does not cancel in the product, and qn_t . kn_t is often a
// small difference of terms (0.002 from terms summing to 0.6 in magnitude)
// that multiplies the token's own, large, Delta_t in its output.
//
// Work decomposition.  One workgroup = one (sequence, head).  The default
// 32-token chunks use the warp-specialised kernel (kda_prefill_ws_kernel):
// 8 state waves keep 16 value columns of the state each, in registers, in
// the matrix cores' accumulator layout, for the whole prompt, and run the
// contractions of one chunk while 8 preparation waves build the next chunk
// (rows, decays, A, P, operands, diagonal inverses) in the other half of a
// double-buffered LDS.  The accumulator layout is also a valid B operand for
// the next contraction over the key channels (the k-order of a 16x16x4 step
// is permuted to match, and the A operand is read from LDS in the same
// order).  64-token chunks use kda_prefill_kernel, where the same 8 waves do
// both in turn (two buffers of 64 tokens would not fit in LDS).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kda_decode.h"
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kLdK = 132;      // row stride (floats) of [C][128] LDS arrays
// Decays are carried in log2 units (g * log2 e) so every exponential is one
// v_exp_f32 (2^x, about 1 ulp); the factored path admits an in-block decay
// of up to 2^115 (80 nats).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kDiagLimit = 115.0f;
constexpr int32_t kDefaultChunk = 32;
// Word 3 of a raw buffer descriptor on gfx9-family GPUs (gfx950 included):
// 32-bit data format, no swizzle; out-of-range accesses are dropped.
constexpr int kBufferWord3 = 0x00020000;

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

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Which sequence a workgroup takes.  A CU holds one prefill workgroup at a
// time (its LDS), and workgroups are dispatched in block order (dealt over
// the XCDs), so the launch is a list schedule over (sequence, head) pairs:
// with the longest sequences first, the last workgroups to start are short
// ones and the launch ends close to the longest sequence's own time, where
// in index order a long sequence may start only as the others end.  Block b
// takes head b mod H of the sequence of rank b / H, the rank of a sequence
// being the number of sequences longer than it, or as long with a smaller
// index (a permutation of 0 .. n_seq - 1).  Every wave ranks the lengths
// itself: each lane counts, for its sequences, the longer ones, reading all
// lengths through readlane.  Above kRankedSeqs sequences that costs more
// than it saves, and blocks take the sequences in index order.
constexpr int kRankedSeqs = 256;

__device__ __forceinline__ int32_t seq_length(const int32_t* cu, int i) {
  const int64_t d = static_cast<int64_t>(cu[i + 1]) - cu[i];
  return d < 0 ? -1 : (d > INT32_MAX ? INT32_MAX : static_cast<int32_t>(d));
}

__device__ int seq_of_rank(const int32_t* cu, int n_seq, int rank) {
  if (n_seq > kRankedSeqs) return rank;
  const int lane = threadIdx.x % 64;
  for (int ib = 0; ib < n_seq; ib += 64) {
    const int i = ib + lane;
    const int32_t li = i < n_seq ? seq_length(cu, i) : -1;
    int r = 0;
    for (int jb = 0; jb < n_seq; jb += 64) {
      const int32_t lj = jb + lane < n_seq ? seq_length(cu, jb + lane) : -1;
      const int cnt = min(64, n_seq - jb);
      for (int jj = 0; jj < cnt; ++jj) {
        const int32_t l = __builtin_amdgcn_readlane(lj, jj);
        r += (l > li || (l == li && jb + jj < i)) ? 1 : 0;
      }
    }
    const unsigned long long hit = __ballot(i < n_seq && r == rank);
    if (hit != 0) return ib + __ffsll(static_cast<long long>(hit)) - 1;
  }
  return rank;  // not reached: the ranks are a permutation of 0 .. n_seq - 1
}

// Raw buffer stores: a 128-bit descriptor {base, stride 0, range in bytes,
// word 3} in scalar registers and a per-lane byte offset; the hardware drops
// a store whose offset is past the range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_descriptor(const void* base, uint32_t range_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(range_bytes), kBufferWord3);
}
__device__ __forceinline__ void raw_buffer_store_f32(float v, __amdgpu_buffer_rsrc_t rsrc, int voffset) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc, voffset, 0, 0);
}

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
// exclusive suffix sum over the 16 lanes of a DPP row (row_shl with zero
// fill): lane i gets the sum of lanes i + 1 .. 15, and lane 15 exactly 0.
// The decays from a token to the end of its block are summed this way, not
// taken as the block total minus the token's prefix sum: two lanes of the
// prefix scan associate their sums differently, so that difference carries an
// absolute error of about one ulp of the block total (2^-19 at a total of
// 25 in log2 units) even where the true value is 0.
template <int N>
__device__ __forceinline__ float row_shl(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x100 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_suffix(float x) {
  x = row_shl<1>(x);
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  x += row_shl<8>(x);
  return x;
}
// Inclusive prefix sum over a DPP row carried in fp64 (two 32-bit row_shr
// moves and one fp64 add per step): the sums of at most 16 fp32 terms are
// then exact but for a relative 2^-53, the same value whatever the lane's
// association, and come back as an fp32 high part and the fp32 remainder
// lo = sum - hi.  The in-block decays 2^(G_t - G_s) are formed as products of
// 2^(hi + lo) factors whose only errors are the exponentials' and the
// products' roundings, not an ulp of the (large) cumulative sums.
template <int N>
__device__ __forceinline__ double row_shr_f64(double x) {
  const int2 v = __builtin_bit_cast(int2, x);
  int2 r;
  r.x = __builtin_amdgcn_mov_dpp(v.x, 0x110 + N, 0xF, 0xF, true);
  r.y = __builtin_amdgcn_mov_dpp(v.y, 0x110 + N, 0xF, 0xF, true);
  return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ void row_scan2(float& hi, float& lo) {
  double d = static_cast<double>(hi);
  d += row_shr_f64<1>(d);
  d += row_shr_f64<2>(d);
  d += row_shr_f64<4>(d);
  d += row_shr_f64<8>(d);
  hi = static_cast<float>(d);
  lo = static_cast<float>(d - static_cast<double>(hi));
}
constexpr float kLn2 = 0.6931471805599453f;
// 2^(hi + lo) for |lo| <= an ulp of hi: 2^hi (1 + lo ln 2), rounded once
__device__ __forceinline__ float exp2_hilo(float hi, float lo) {
  const float e = exp2_fast(hi);
  return fmaf(e, lo * kLn2, e);
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

// Chunk of NB blocks of 16 tokens (C = 16 NB), NW wavefronts.
//  - per-token rows (norms, decays, operands): wave w takes token block
//    w % NB and channel part w / NB (NW / NB parts of 128 / (NW / NB)
//    channels; a lane holds CPL of them);
//  - A and P: the NB (NB + 1) / 2 block pairs (bt >= bs) go round-robin to
//    the waves;
//  - the state: wave w owns value columns CPW w .. CPW w + CPW - 1.
template <typename T, int NB, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void kda_prefill_kernel(PrefillArgs a) {
  constexpr int C = 16 * NB;
  constexpr int LdC = C + 4;       // row stride of [C][C] arrays
  constexpr int PARTS = NW / NB;   // channel parts of the per-token phases
  constexpr int CPL = 32 / PARTS;  // channels per lane in those phases
  constexpr int CPW = 128 / NW;    // value columns per wave
  constexpr int NCB = CPW / 16;    // 16-column blocks per wave
  constexpr int NPAIR = NB * (NB + 1) / 2;
  static_assert(NW % NB == 0 && CPL % 4 == 0 && CPW % 16 == 0, "launch shape");
  // Per-token rows [C][128]: raw k, block-local cumulative log2-decay and
  // raw q; then, in place, the operands -Kb, Qg and Kd.
  __shared__ __attribute__((aligned(16))) float sX[C * kLdK];
  __shared__ __attribute__((aligned(16))) float sY[C * kLdK];
  __shared__ __attribute__((aligned(16))) float sZ[C * kLdK];
  __shared__ __attribute__((aligned(16))) float sA[C * LdC];      // -A (strictly lower)
  __shared__ __attribute__((aligned(16))) float sP[C * LdC];      // P (lower)
  __shared__ __attribute__((aligned(16))) float sTd[NB][16 * 20]; // (I + A_bb)^-1
  __shared__ __attribute__((aligned(16))) float sBtot[NB][128];   // per block: sum of g log2 e
  __shared__ __attribute__((aligned(16))) float sPre[NB][128];      // sums of Btot over blocks < u
  __shared__ __attribute__((aligned(16))) float sSuf[NB][128];      // sums of Btot over blocks > u
  __shared__ float sGC[128];                                      // 2^(G_C)
  __shared__ float sBeta[C];
  __shared__ float sSq[PARTS][C];  // partial sums of q^2, k^2 per channel part
  __shared__ float sSk[PARTS][C];
  __shared__ float sSqk[PARTS][C];  // partial sums of q k

  // wave-uniform: in scalar registers, and so everything derived from it
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / 64));
  const int seq = seq_of_rank(a.cu, a.n_seq, blockIdx.x / a.H);
  const int h = blockIdx.x % a.H;

  const int64_t t0 = a.cu[seq];
  const int64_t t1 = a.cu[seq + 1];
  const int32_t init = a.init_ids[seq];
  const int32_t dst = a.dst_ids != nullptr ? a.dst_ids[seq] : init;
  if (!(t0 >= 0 && t0 <= t1 && t1 <= a.n_tokens && init >= 0 && init < a.n_slots && dst >= 0 &&
        dst < a.n_slots))
    return;  // refused by the host checks; never touch memory outside the launch's bounds

  const int64_t hk = static_cast<int64_t>(a.H) * 128;  // floats per token of q, k, g, v, out
  const int col_w = CPW * wave;                          // this wave's first value column
  const int64_t head_off = static_cast<int64_t>(h) * 128 * 128;

  // -- initial state slice: S[sb][cb] holds rows 16 sb + 4 gq + r, column
  //    col_w + 16 cb + li (the 16x16 accumulator layout)
  f4 S[8][NCB];
  {
    const int li = threadIdx.x % 16, gq = (threadIdx.x % 64) / 16;
    const T* src = static_cast<const T*>(a.pool) + static_cast<int64_t>(init) * a.H * 128 * 128 +
                   head_off;
#pragma unroll
    for (int sb = 0; sb < 8; ++sb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[sb][cb][r] = widen1(src + (16 * sb + 4 * gq + r) * 128 + col_w + 16 * cb + li);
  }

  // Rows of the next chunk are loaded one chunk ahead (q, k, g of this
  // lane's token and channels, b, and v of the wave's columns), so the loads
  // overlap the current chunk's work instead of opening each chunk.
  f4 nq[CPL / 4], nk[CPL / 4], ng[CPL / 4], nv[NB][NCB];
  float nb = 0.0f;
  // Addresses: a chunk-uniform 64-bit base plus a 32-bit per-lane offset.
  // Rows past the end of the sequence read row 0 of the chunk instead, so no
  // load sits behind a branch; they are zeroed where the data is used (a
  // select right after the load would make the wave wait for it here).
  const uint32_t hk32 = static_cast<uint32_t>(hk);
  auto prefetch = [&](int64_t c, int li_, int gq_) {
    const int m_ = static_cast<int>(t1 - c < C ? t1 - c : C);
    const int tl_ = 16 * (wave % NB) + li_;
    const int ch_ = (wave / NB) * (128 / PARTS) + gq_ * CPL;
    const uint32_t row_ = static_cast<uint32_t>(tl_ < m_ ? tl_ : 0);
    const int64_t base = c * hk + static_cast<int64_t>(h) * 128;
    const float* qb = a.q + base;
    const float* kb = a.k + base;
    const float* gb = a.g + base;
    const uint32_t off = row_ * hk32 + static_cast<uint32_t>(ch_);
#pragma unroll
    for (int m = 0; m < CPL / 4; ++m) {
      nq[m] = *reinterpret_cast<const f4*>(qb + (off + 4 * m));
      nk[m] = *reinterpret_cast<const f4*>(kb + (off + 4 * m));
      ng[m] = *reinterpret_cast<const f4*>(gb + (off + 4 * m));
    }
    nb = (a.b + c * a.H + h)[row_ * static_cast<uint32_t>(a.H)];
    const float* vb = a.v + base + col_w;
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = 16 * tb + 4 * gq_ + r;
          const uint32_t rr = static_cast<uint32_t>(tr < m_ ? tr : 0);
          nv[tb][cb][r] = vb[rr * hk32 + static_cast<uint32_t>(16 * cb + li_)];
        }
  };
  if (t0 < t1) prefetch(t0, threadIdx.x % 16, (threadIdx.x % 64) / 16);

  for (int64_t c0 = t0; c0 < t1; c0 += C) {
    const int n = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);
    // Lane indices re-derived from an opaque copy of the thread id in every
    // chunk: the many lane-dependent LDS addresses and constants of the loop
    // body are then recomputed per chunk (a few integer ops) instead of being
    // hoisted out of the loop and held in registers, which would leave too
    // few for the state and accumulators.
    int tid_v = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(tid_v));
    const int li = tid_v % 16;
    const int gq = (tid_v % 64) / 16;
    // the per-token phases: token block, channel part, this lane's row and channels
    const int pb = wave % NB;
    const int pp = wave / NB;
    const int tl = 16 * pb + li;
    const int ch0 = pp * (128 / PARTS) + gq * CPL;
    const int row = tl * kLdK + ch0;

    // ---- per-token rows from the prefetched registers: raw q and k, partial
    // sums of squares, block-local cumulative decays
    f4 D[NB][NCB];  // v (rows past the sequence zeroed); beta is applied later
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) D[tb][cb][r] = 16 * tb + 4 * gq + r < n ? nv[tb][cb][r] : 0.0f;
    {
      const bool valid = tl < n;
      const f4 zero = {0.f, 0.f, 0.f, 0.f};
      float sq = 0.0f, sk = 0.0f, sqk = 0.0f;
#pragma unroll
      for (int m = 0; m < CPL / 4; ++m) {
        const f4 q4 = valid ? nq[m] : zero;
        const f4 k4 = valid ? nk[m] : zero;
        const f4 g4 = valid ? ng[m] : zero;
        f4 gl4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sq = fmaf(q4[e], q4[e], sq);
          sk = fmaf(k4[e], k4[e], sk);
          sqk = fmaf(q4[e], k4[e], sqk);
          gl4[e] = row_scan(g4[e] * kLog2e);  // block-local inclusive cumulative sum
        }
        *reinterpret_cast<f4*>(sZ + row + 4 * m) = q4;
        *reinterpret_cast<f4*>(sX + row + 4 * m) = k4;
        *reinterpret_cast<f4*>(sY + row + 4 * m) = gl4;
        if (li == 15) *reinterpret_cast<f4*>(&sBtot[pb][ch0 + 4 * m]) = gl4;
      }
      sq = group_sum(sq);
      sk = group_sum(sk);
      sqk = group_sum(sqk);
      if (gq == 0) {
        sSq[pp][tl] = sq;
        sSk[pp][tl] = sk;
        sSqk[pp][tl] = sqk;
        if (pp == 0) sBeta[tl] = valid ? 1.0f / (1.0f + expf(-nb)) : 0.0f;
      }
    }
    __syncthreads();

    // ---- block prefix sums of the decay and 2^(G_C) (wave 0), then A and P
    if (wave == 0) {
      const int lane = tid_v % 64;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int ch = 2 * lane + e;
        float acc = 0.0f;
        sPre[0][ch] = 0.0f;
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          acc += sBtot[u][ch];
          if (u + 1 < NB) sPre[u + 1][ch] = acc;
        }
        sGC[ch] = exp2_fast(acc);
        float later = 0.0f;
#pragma unroll
        for (int u = NB - 1; u >= 0; --u) {
          sSuf[u][ch] = later;
          later += sBtot[u][ch];
        }
      }
    }
    // Chains (block pair (bt, bs), P or A) go round-robin to the waves.  Step
    // (m, e) of the contraction is channel 32 gq + m + e in both operands.
    // t-factors 2^(G_t - G_ref) = 2^(gl_t); s-factors for token s = 16 bs + li:
    // 2^(G_ref - G_s) = 2^(cum - gl_s), cum = sum of Btot over bs <= u < bt.
    for (int ci = wave; ci < 2 * NPAIR; ci += NW) {
      const int pi = ci / 2;
      const bool is_a = (ci & 1) != 0;  // A (with beta kn) or P (with qn)
      int bt = 0;
      while ((bt + 1) * (bt + 2) / 2 <= pi) ++bt;
      const int bs = pi - bt * (bt + 1) / 2;
      const int trow = (16 * bt + li) * kLdK + 32 * gq;
      const int srow = (16 * bs + li) * kLdK + 32 * gq;
      float st = 0.0f, ss = 0.0f;
#pragma unroll
      for (int u = 0; u < PARTS; ++u) {
        st += is_a ? sSk[u][16 * bt + li] : sSq[u][16 * bt + li];
        ss += sSk[u][16 * bs + li];
      }
      const float beta = sBeta[16 * bt + li];
      // t-side scale: beta / |k_t| for A, 1 / |q_t| for P
      const float r_t = (is_a ? beta : 1.0f) / sqrtf(st + 1e-6f);
      const float rk_s = 1.0f / sqrtf(ss + 1e-6f);
      const float* tsrc = is_a ? sX : sZ;
      // in-block decay beyond the factored range: the diagonal block goes pair by pair
      bool exact = false;
      if (bt == bs) {
        float span = 0.0f;
#pragma unroll
        for (int m = 0; m < 32; m += 4) {
          const f4 gl4 = *reinterpret_cast<const f4*>(sY + trow + m);
#pragma unroll
          for (int e = 0; e < 4; ++e) span = fmaxf(span, -gl4[e]);
        }
        exact = __builtin_amdgcn_ballot_w64(span > kDiagLimit) != 0;
      }
      if (!exact) {
        f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 32; m += 4) {
          f4 cum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < NB - 1; ++u)
            if (u >= bs && u < bt) cum += *reinterpret_cast<const f4*>(&sBtot[u][32 * gq + m]);
          const f4 xt = *reinterpret_cast<const f4*>(tsrc + trow + m);
          const f4 gt = *reinterpret_cast<const f4*>(sY + trow + m);
          const f4 ks = *reinterpret_cast<const f4*>(sX + srow + m);
          const f4 gs = *reinterpret_cast<const f4*>(sY + srow + m);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lf = (xt[e] * r_t) * exp2_fast(gt[e]);
            const float rf = (ks[e] * rk_s) * exp2_fast(cum[e] - gs[e]);
            if (e % 2 == 0)
              acc0 = mma(lf, rf, acc0);
            else
              acc1 = mma(lf, rf, acc1);
          }
        }
        // accumulator layout: row 16 bt + 4 gq + r, column 16 bs + li
        float* dstm = is_a ? sA : sP;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = 4 * gq + r;
          float x = acc0[r] + acc1[r];
          if (bs == bt && (is_a ? li >= tr : li > tr)) x = 0.0f;
          dstm[(16 * bt + tr) * LdC + 16 * bs + li] = is_a ? -x : x;
        }
      } else {
        // pair by pair: lane (li = t, gq) sums its 32 channels for every s <= t
        for (int s2 = 0; s2 < 16; ++s2) {
          const int s2row = (16 * bt + s2) * kLdK + 32 * gq;
          float sk2 = 0.0f;
#pragma unroll
          for (int u = 0; u < PARTS; ++u) sk2 += sSk[u][16 * bt + s2];
          const float rk_s2 = 1.0f / sqrtf(sk2 + 1e-6f);
          float acc = 0.0f;
          if (s2 <= li) {
            for (int i = 0; i < 32; ++i) {
              const float f = (sX[s2row + i] * rk_s2) * exp2_fast(sY[trow + i] - sY[s2row + i]);
              acc = fmaf(tsrc[trow + i] * r_t, f, acc);
            }
          }
          acc = group_sum(acc);
          if (gq == 0) {
            if (is_a)
              sA[(16 * bt + li) * LdC + 16 * bt + s2] = s2 < li ? -acc : 0.0f;
            else
              sP[(16 * bt + li) * LdC + 16 * bt + s2] = s2 <= li ? acc : 0.0f;
          }
        }
      }
    }
    __syncthreads();

    // ---- operands of the state contractions (in place of the rows); diagonal inverses
    {
      float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
      for (int u = 0; u < PARTS; ++u) {
        ssq += sSq[u][tl];
        ssk += sSk[u][tl];
      }
      const float rq = 1.0f / sqrtf(ssq + 1e-6f);
      const float rk = 1.0f / sqrtf(ssk + 1e-6f);
      const float beta = sBeta[tl];
      const bool valid = tl < n;
      const f4 zero = {0.f, 0.f, 0.f, 0.f};
      // G_t = (sum of Btot before block pb) + gl_t;
      // G_C - G_t = (sum of Btot after block pb) + (decay from t to the end of
      // block pb), both parts <= 0 and each summed directly
#pragma unroll
      for (int m = 0; m < CPL; m += 4) {
        const int ch = ch0 + m;
        const f4 k4 = *reinterpret_cast<const f4*>(sX + row + m);
        const f4 gl4 = *reinterpret_cast<const f4*>(sY + row + m);
        const f4 q4 = *reinterpret_cast<const f4*>(sZ + row + m);
        const f4 pre = *reinterpret_cast<const f4*>(&sPre[pb][ch]);
        const f4 post = *reinterpret_cast<const f4*>(&sSuf[pb][ch]);
        const f4 g4 = valid ? ng[m / 4] : zero;
        f4 nkb, qg, kd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float kn = k4[e] * rk;
          const float eg = exp2_fast(pre[e] + gl4[e]);
          nkb[e] = -((beta * kn) * eg);
          qg[e] = (q4[e] * rq) * eg;
          kd[e] = kn * exp2_fast(post[e] + row_suffix(g4[e] * kLog2e));
        }
        *reinterpret_cast<f4*>(sX + row + m) = nkb;
        *reinterpret_cast<f4*>(sY + row + m) = qg;
        *reinterpret_cast<f4*>(sZ + row + m) = kd;
      }
      // The next chunk's rows, once this chunk's g has been used for Kd (issued
      // earlier, the prefetched rows would stay live through the chains and
      // this phase, beyond the register budget).  Unconditional (the last
      // chunk reloads its own rows): a conditional prefetch would merge old and
      // new registers with copies that wait for the previous chunk's stores.
      // P_tt = qn_t . kn_t (no decay) in place of the chain's value: summed
      // from the partial sums of q k, without the chain's two exponentials
      if (pp == 0 && gq == 0) {
        float qk = 0.0f;
#pragma unroll
        for (int u = 0; u < PARTS; ++u) qk += sSqk[u][tl];
        sP[tl * LdC + tl] = (qk * rq) * rk;
      }
      prefetch(c0 + C < t1 ? c0 + C : c0, li, gq);
      // (I + A_bb)^-1 by forward substitution, one column per lane of group 0
      if (wave < NB && gq == 0) {
        const int b = wave;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          float acc = t == li ? 1.0f : 0.0f;
#pragma unroll
          for (int s2 = 0; s2 < t; ++s2)
            acc = fmaf(sA[(16 * b + t) * LdC + 16 * b + s2], x[s2], acc);
          x[t] = acc;  // sA holds -A
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) sTd[b][t * 20 + li] = x[t];
      }
    }
    __syncthreads();

    // ---- the state contractions, this wave's CPW value columns.  Loops keep
    // several independent accumulators in flight per step.
    // R = beta V - Kb S  (token block tb: rows 16 tb + 4 gq + r)
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float bt = sBeta[16 * tb + 4 * gq + r];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) D[tb][cb][r] *= bt;
      }
#pragma unroll
    for (int sb = 0; sb < 8; ++sb) {
      f4 x[NB];
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
        x[tb] = *reinterpret_cast<const f4*>(sX + (16 * tb + li) * kLdK + 16 * sb + 4 * gq);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) D[tb][cb] = mma(x[tb][r], S[sb][cb][r], D[tb][cb]);
    }
    // Delta = (I + A)^-1 R, block by block: Delta_b = T_bb (R_b - sum_{k<b} A_bk Delta_k)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int k = 0; k < b; ++k) {
        const f4 x = *reinterpret_cast<const f4*>(sA + (16 * b + li) * LdC + 16 * k + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) D[b][cb] = mma(x[r], D[k][cb][r], D[b][cb]);
      }
      const f4 x = *reinterpret_cast<const f4*>(&sTd[b][li * 20 + 4 * gq]);
      f4 y[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) y[cb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) y[cb] = mma(x[r], D[b][cb][r], y[cb]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) D[b][cb] = y[cb];
    }
    // o = scale (Qg S + P Delta)
    {
      f4 O[NB][NCB];
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) O[tb][cb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sb = 0; sb < 8; ++sb) {
        f4 x[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
          x[tb] = *reinterpret_cast<const f4*>(sY + (16 * tb + li) * kLdK + 16 * sb + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int tb = 0; tb < NB; ++tb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) O[tb][cb] = mma(x[tb][r], S[sb][cb][r], O[tb][cb]);
      }
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        f4 x[NB];
#pragma unroll
        for (int tb = kb; tb < NB; ++tb)
          x[tb] = *reinterpret_cast<const f4*>(sP + (16 * tb + li) * LdC + 16 * kb + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int tb = kb; tb < NB; ++tb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) O[tb][cb] = mma(x[tb][r], D[kb][cb][r], O[tb][cb]);
      }
      // Buffer stores: the descriptor's range ends after the chunk's last
      // token, so the hardware drops the rows past the sequence without a
      // branch (a branch around the stores would make the next chunk's first
      // use of the prefetched rows wait for every store to be acknowledged).
      const __amdgpu_buffer_rsrc_t orsrc =
          buffer_descriptor(a.out + (c0 * hk + static_cast<int64_t>(h) * 128 + col_w),
                            (static_cast<uint32_t>(n - 1) * hk32 + CPW) * 4);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t tr = static_cast<uint32_t>(16 * tb + 4 * gq + r);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            raw_buffer_store_f32(
                a.scale * O[tb][cb][r], orsrc,
                static_cast<int>((tr * hk32 + static_cast<uint32_t>(16 * cb + li)) * 4));
        }
    }
    // S = 2^(G_C) S + Kd^T Delta
#pragma unroll
    for (int sb = 0; sb < 8; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d = sGC[16 * sb + 4 * gq + r];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) S[sb][cb][r] *= d;
      }
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      // A operand Kd^T[channel 16 sb + li][token 16 tb + 4 gq + r], read from the Kd rows
      f4 x[8];
#pragma unroll
      for (int sb = 0; sb < 8; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[sb][r] = sZ[(16 * tb + 4 * gq + r) * kLdK + 16 * sb + li];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int sb = 0; sb < 8; ++sb)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) S[sb][cb] = mma(x[sb][r], D[tb][cb][r], S[sb][cb]);
    }
    __syncthreads();  // the next chunk overwrites the LDS operands
  }

  // -- final state to the destination slot.  The empty asm makes the slot
  // offset opaque, so the compiler cannot compute these addresses before the
  // chunk loop and hold them in registers through it.
  int64_t dst_off = static_cast<int64_t>(dst) * a.H * 128 * 128 + head_off;
  asm volatile("" : "+s"(dst_off));
  T* dstp = static_cast<T*>(a.pool) + dst_off;
  const int li = threadIdx.x % 16, gq = (threadIdx.x % 64) / 16;
#pragma unroll
  for (int sb = 0; sb < 8; ++sb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        narrow1(dstp + (16 * sb + 4 * gq + r) * 128 + col_w + 16 * cb + li, S[sb][cb][r]);
}

// ---------------------------------------------------------------------------
// Warp-specialised form for 32-token chunks (the default).  Eight state
// waves keep the state (16 value columns each) and run the contractions of
// chunk i - 1 while four preparation waves build chunk i (rows, decays, A,
// P, operands, diagonal inverses) in the other half of a double-buffered LDS.
// The two groups meet at three barriers per chunk; between two barriers the
// state waves issue matrix-core work while the preparation waves issue
// vector, transcendental and LDS work, so the two overlap on every SIMD.
// ---------------------------------------------------------------------------
constexpr int kWsNB = 2;                // token blocks per chunk
constexpr int kWsC = 16 * kWsNB;        // tokens per chunk
constexpr int kWsState = 8;             // state waves (16 value columns each)
constexpr int kWsPrep = 8;              // preparation waves
constexpr int kWsParts = kWsPrep / kWsNB;  // channel parts of the per-token phases
constexpr int kWsCpl = 32 / kWsParts;   // channels per lane in those phases
constexpr int kWsLdC = kWsC + 4;

struct __attribute__((aligned(16))) WsBuf {
  float X[kWsC * kLdK];   // raw k, then -Kb
  float Y[kWsC * kLdK];   // block-local cumulative log2 decay, then Qg
  float Z[kWsC * kLdK];   // raw q, then Kd
  float A[kWsC * kWsLdC];  // -A (strictly lower)
  float P[kWsC * kWsLdC];  // P (lower)
  float Td[kWsNB][16 * 20];  // (I + A_bb)^-1
  float Btot[kWsNB][128];
  float Pre[kWsNB][128];   // sums of Btot over earlier blocks
  float Suf[kWsNB][128];   // sums of Btot over later blocks
  float GC[128];
  float Beta[kWsC];
  float Sq[kWsParts][kWsC];
  float Sk[kWsParts][kWsC];
  float Sqk[kWsParts][kWsC];  // partial sums of q k
};

template <typename T>
__global__ __launch_bounds__(64 * (kWsState + kWsPrep)) __attribute__((amdgpu_waves_per_eu((kWsState + kWsPrep) / 4)))
void kda_prefill_ws_kernel(PrefillArgs a) {
  constexpr int NB = kWsNB;
  constexpr int C = kWsC;
  constexpr int LdC = kWsLdC;
  constexpr int PARTS = kWsParts;
  constexpr int CPL = kWsCpl;
  constexpr int NPAIR = NB * (NB + 1) / 2;
  __shared__ WsBuf sb[2];
  // low parts (fp64 sum minus its fp32 rounding) of the block-local
  // cumulative decays (the high parts are the rows of Y) and of the block
  // totals: read only by the preparation waves within the chunk that wrote
  // them, so single-buffered
  __shared__ __attribute__((aligned(16))) float sYlo[kWsC * kLdK];
  __shared__ __attribute__((aligned(16))) float sBlo[kWsNB][128];

  // wave-uniform: in scalar registers, and so everything derived from it
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / 64));
  const bool state_wave = wave < kWsState;
  const int pw = wave - kWsState;  // preparation wave index (prep waves only)
  // The preparation waves issue ahead of the state waves on their SIMDs: the
  // state waves' matrix-core products then fill the gaps in the preparation
  // waves' vector work rather than delaying it (34K-token batch: 761 -> 720
  // us; raising the state waves instead changes nothing).
  if (!state_wave) __builtin_amdgcn_s_setprio(1);
  const int seq = seq_of_rank(a.cu, a.n_seq, blockIdx.x / a.H);
  const int h = blockIdx.x % a.H;

  const int64_t t0 = a.cu[seq];
  const int64_t t1 = a.cu[seq + 1];
  const int32_t init = a.init_ids[seq];
  const int32_t dst = a.dst_ids != nullptr ? a.dst_ids[seq] : init;
  if (!(t0 >= 0 && t0 <= t1 && t1 <= a.n_tokens && init >= 0 && init < a.n_slots && dst >= 0 &&
        dst < a.n_slots))
    return;  // refused by the host checks; never touch memory outside the launch's bounds

  const int64_t hk = static_cast<int64_t>(a.H) * 128;
  const uint32_t hk32 = static_cast<uint32_t>(hk);
  const int64_t head_off = static_cast<int64_t>(h) * 128 * 128;
  const int col_w = 16 * (state_wave ? wave : 0);  // a state wave's value columns
  const int n_chunks = static_cast<int>((t1 - t0 + C - 1) / C);

  // The registers carried from chunk to chunk, shared by the two roles (a
  // wave only ever plays one): state waves keep the state slice (rows
  // 16 sb + 4 gq + r of their 16 columns, accumulator layout) in reg[0..7],
  // the next chunk's v in reg[8..9] and R / Delta in reg[10..11];
  // preparation waves keep the next chunk's q, k, g in reg[0..1], reg[2..3],
  // reg[4..5] and, from the per-token rows to the operands, the decay from
  // each of their tokens to the end of its block in reg[6..7].
  constexpr int kS = 0, kV = 8, kD = 10, kQ = 0, kK = CPL / 4, kG = 2 * (CPL / 4),
                kF = 3 * (CPL / 4);
  static_assert(4 * (CPL / 4) <= 12, "q, k, g, suffix of a preparation lane fit the shared registers");
  f4 reg[12];
  if (state_wave) {
    const int li = threadIdx.x % 16, gq = (threadIdx.x % 64) / 16;
    const T* src = static_cast<const T*>(a.pool) + static_cast<int64_t>(init) * a.H * 128 * 128 +
                   head_off;
#pragma unroll
    for (int sb2 = 0; sb2 < 8; ++sb2)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        reg[kS + sb2][r] = widen1(src + (16 * sb2 + 4 * gq + r) * 128 + col_w + li);
  }

  // prefetched rows: preparation waves hold q, k, g, b of their token and
  // channels for the next chunk to prepare; state waves hold v of their
  // columns for the next chunk to contract.  Rows past the sequence read
  // row 0 of the chunk and are zeroed where used.
  float nb = 0.0f;
  auto prefetch_rows = [&](int64_t c, int li_, int gq_) {
    const int m_ = static_cast<int>(t1 - c < C ? t1 - c : C);
    const int tl_ = 16 * (pw % NB) + li_;
    const int ch_ = (pw / NB) * (128 / PARTS) + gq_ * CPL;
    const uint32_t row_ = static_cast<uint32_t>(tl_ < m_ ? tl_ : 0);
    const int64_t base = c * hk + static_cast<int64_t>(h) * 128;
    const uint32_t off = row_ * hk32 + static_cast<uint32_t>(ch_);
#pragma unroll
    for (int m = 0; m < CPL / 4; ++m) {
      reg[kQ + m] = *reinterpret_cast<const f4*>(a.q + base + (off + 4 * m));
      reg[kK + m] = *reinterpret_cast<const f4*>(a.k + base + (off + 4 * m));
      reg[kG + m] = *reinterpret_cast<const f4*>(a.g + base + (off + 4 * m));
    }
    nb = (a.b + c * a.H + h)[row_ * static_cast<uint32_t>(a.H)];
  };
  auto prefetch_v = [&](int64_t c, int li_, int gq_) {
    const int m_ = static_cast<int>(t1 - c < C ? t1 - c : C);
    const float* vb = a.v + c * hk + static_cast<int64_t>(h) * 128 + col_w;
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 16 * tb + 4 * gq_ + r;
        const uint32_t rr = static_cast<uint32_t>(tr < m_ ? tr : 0);
        reg[kV + tb][r] = vb[rr * hk32 + static_cast<uint32_t>(li_)];
      }
  };
  if (t0 < t1) {
    if (state_wave)
      prefetch_v(t0, threadIdx.x % 16, (threadIdx.x % 64) / 16);
    else
      prefetch_rows(t0, threadIdx.x % 16, (threadIdx.x % 64) / 16);
  }

  for (int it = 0; it <= n_chunks; ++it) {
    int tid_v = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(tid_v));  // see the note in kda_prefill_kernel
    const int li = tid_v % 16;
    const int gq = (tid_v % 64) / 16;
    const bool prep_now = !state_wave && it < n_chunks;   // prepares chunk it
    const bool state_now = state_wave && it >= 1;          // contracts chunk it - 1
    const int64_t cp = t0 + static_cast<int64_t>(it) * C;        // chunk being prepared
    const int64_t cs = t0 + static_cast<int64_t>(it - 1) * C;    // chunk being contracted
    const int np = prep_now ? static_cast<int>(t1 - cp < C ? t1 - cp : C) : 0;
    const int ns = state_now ? static_cast<int>(t1 - cs < C ? t1 - cs : C) : 0;
    WsBuf& bp = sb[it & 1];
    WsBuf& bs = sb[(it + 1) & 1];

    // ================= segment 1 =================
    if (prep_now) {
      // per-token rows of chunk it: raw q and k, partial sums of squares, decays
      const int pb = pw % NB, pp = pw / NB;
      const int tl = 16 * pb + li;
      const int ch0 = pp * (128 / PARTS) + gq * CPL;
      const int row = tl * kLdK + ch0;
      const bool valid = tl < np;
      const f4 zero = {0.f, 0.f, 0.f, 0.f};
      float sq = 0.0f, sk = 0.0f, sqk = 0.0f;
#pragma unroll
      for (int m = 0; m < CPL / 4; ++m) {
        const f4 q4 = valid ? reg[kQ + m] : zero;
        const f4 k4 = valid ? reg[kK + m] : zero;
        const f4 g4 = valid ? reg[kG + m] : zero;
        f4 gl4, lo4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sq = fmaf(q4[e], q4[e], sq);
          sk = fmaf(k4[e], k4[e], sk);
          sqk = fmaf(q4[e], k4[e], sqk);
          float hi = g4[e] * kLog2e, lo = 0.0f;
          row_scan2(hi, lo);
          gl4[e] = hi;
          lo4[e] = lo;
          reg[kF + m][e] = row_suffix(g4[e] * kLog2e);
        }
        *reinterpret_cast<f4*>(bp.Z + row + 4 * m) = q4;
        *reinterpret_cast<f4*>(bp.X + row + 4 * m) = k4;
        *reinterpret_cast<f4*>(bp.Y + row + 4 * m) = gl4;
        *reinterpret_cast<f4*>(sYlo + row + 4 * m) = lo4;
        if (li == 15) {
          *reinterpret_cast<f4*>(&bp.Btot[pb][ch0 + 4 * m]) = gl4;
          *reinterpret_cast<f4*>(&sBlo[pb][ch0 + 4 * m]) = lo4;
        }
      }
      sq = group_sum(sq);
      sk = group_sum(sk);
      sqk = group_sum(sqk);
      if (gq == 0) {
        bp.Sq[pp][tl] = sq;
        bp.Sk[pp][tl] = sk;
        bp.Sqk[pp][tl] = sqk;
        if (pp == 0) bp.Beta[tl] = valid ? 1.0f / (1.0f + expf(-nb)) : 0.0f;
      }
    }
    if (state_now) {
      // R = beta V - Kb S for chunk it - 1
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = 16 * tb + 4 * gq + r;
          reg[kD + tb][r] = tr < ns ? bs.Beta[tr] * reg[kV + tb][r] : 0.0f;
        }
      prefetch_v(cs + C < t1 ? cs + C : cs, li, gq);
#pragma unroll
      for (int sb2 = 0; sb2 < 8; ++sb2) {
        f4 x[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
          x[tb] = *reinterpret_cast<const f4*>(bs.X + (16 * tb + li) * kLdK + 16 * sb2 + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int tb = 0; tb < NB; ++tb) reg[kD + tb] = mma(x[tb][r], reg[kS + sb2][r], reg[kD + tb]);
      }
    }
    __syncthreads();

    // ================= segment 2 =================
    if (prep_now) {
      if (pw == 0) {
        const int lane = tid_v % 64;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ch = 2 * lane + e;
          float acc = 0.0f;
          bp.Pre[0][ch] = 0.0f;
#pragma unroll
          for (int u = 0; u < NB; ++u) {
            acc += bp.Btot[u][ch];
            if (u + 1 < NB) bp.Pre[u + 1][ch] = acc;
          }
          bp.GC[ch] = exp2_fast(acc);
          float later = 0.0f;
#pragma unroll
          for (int u = NB - 1; u >= 0; --u) {
            bp.Suf[u][ch] = later;
            later += bp.Btot[u][ch];
          }
        }
      }
      // chains: one block pair per preparation wave, P and A together (they
      // share the decay factors of both operands)
      for (int pi = pw; pi < NPAIR; pi += kWsPrep) {
        int bt = 0;
        while ((bt + 1) * (bt + 2) / 2 <= pi) ++bt;
        const int bsb = pi - bt * (bt + 1) / 2;
        const int trow = (16 * bt + li) * kLdK + 32 * gq;
        const int srow = (16 * bsb + li) * kLdK + 32 * gq;
        float sq_t = 0.0f, sk_t = 0.0f, ss = 0.0f;
#pragma unroll
        for (int u = 0; u < PARTS; ++u) {
          sq_t += bp.Sq[u][16 * bt + li];
          sk_t += bp.Sk[u][16 * bt + li];
          ss += bp.Sk[u][16 * bsb + li];
        }
        const float beta = bp.Beta[16 * bt + li];
        const float rq_t = 1.0f / sqrtf(sq_t + 1e-6f);
        const float rk_t = beta / sqrtf(sk_t + 1e-6f);
        const float rk_s = 1.0f / sqrtf(ss + 1e-6f);
        bool exact = false;
        if (bt == bsb) {
          float span = 0.0f;
#pragma unroll
          for (int m = 0; m < 32; m += 4) {
            const f4 gl4 = *reinterpret_cast<const f4*>(bp.Y + trow + m);
#pragma unroll
            for (int e = 0; e < 4; ++e) span = fmaxf(span, -gl4[e]);
          }
          exact = __builtin_amdgcn_ballot_w64(span > kDiagLimit) != 0;
        }
        if (!exact) {
          // Step (m, e): channel 32 gq + m + e of both operands.  Diagonal
          // block: t-factor 2^(gl_t), s-factor 2^(-gl_s), each from the high
          // and low parts (their exponents cancel to the small in-block
          // decay).  Block bt > bsb: t-factor 2^(gl_t), whose exponent is the
          // product's own order (no low part needed), s-factor
          // 2^(Btot_bsb - gl_s), the difference taken in high and low parts.
          static_assert(NB == 2, "no blocks between bsb and bt");
          f4 accp = {0.f, 0.f, 0.f, 0.f}, acca = {0.f, 0.f, 0.f, 0.f};
          if (bsb == bt) {
#pragma unroll 2
            for (int m = 0; m < 32; m += 2) {
              const f2 xq = *reinterpret_cast<const f2*>(bp.Z + trow + m);
              const f2 xk = *reinterpret_cast<const f2*>(bp.X + trow + m);
              const f2 gt = *reinterpret_cast<const f2*>(bp.Y + trow + m);
              const f2 gtl = *reinterpret_cast<const f2*>(sYlo + trow + m);
              const f2 ks = *reinterpret_cast<const f2*>(bp.X + srow + m);
              const f2 gs = *reinterpret_cast<const f2*>(bp.Y + srow + m);
              const f2 gsl = *reinterpret_cast<const f2*>(sYlo + srow + m);
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const float et = exp2_hilo(gt[e], gtl[e]);
                const float rf = (ks[e] * rk_s) * exp2_hilo(-gs[e], -gsl[e]);
                accp = mma((xq[e] * rq_t) * et, rf, accp);
                acca = mma((xk[e] * rk_t) * et, rf, acca);
              }
            }
          } else {
#pragma unroll 2
            for (int m = 0; m < 32; m += 2) {
              const f2 bh = *reinterpret_cast<const f2*>(&bp.Btot[bsb][32 * gq + m]);
              const f2 bl = *reinterpret_cast<const f2*>(&sBlo[bsb][32 * gq + m]);
              const f2 xq = *reinterpret_cast<const f2*>(bp.Z + trow + m);
              const f2 xk = *reinterpret_cast<const f2*>(bp.X + trow + m);
              const f2 gt = *reinterpret_cast<const f2*>(bp.Y + trow + m);
              const f2 ks = *reinterpret_cast<const f2*>(bp.X + srow + m);
              const f2 gs = *reinterpret_cast<const f2*>(bp.Y + srow + m);
              const f2 gsl = *reinterpret_cast<const f2*>(sYlo + srow + m);
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const float et = exp2_fast(gt[e]);
                const float rf = (ks[e] * rk_s) * exp2_hilo(bh[e] - gs[e], bl[e] - gsl[e]);
                accp = mma((xq[e] * rq_t) * et, rf, accp);
                acca = mma((xk[e] * rk_t) * et, rf, acca);
              }
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tr = 4 * gq + r;
            float xp = accp[r], xa = acca[r];
            if (bsb == bt && li > tr) xp = 0.0f;
            if (bsb == bt && li >= tr) xa = 0.0f;
            bp.P[(16 * bt + tr) * LdC + 16 * bsb + li] = xp;
            bp.A[(16 * bt + tr) * LdC + 16 * bsb + li] = -xa;
          }
        } else {
          for (int s2 = 0; s2 < 16; ++s2) {
            const int s2row = (16 * bt + s2) * kLdK + 32 * gq;
            float sk2 = 0.0f;
#pragma unroll
            for (int u = 0; u < PARTS; ++u) sk2 += bp.Sk[u][16 * bt + s2];
            const float rk_s2 = 1.0f / sqrtf(sk2 + 1e-6f);
            float ap = 0.0f, aa = 0.0f;
            if (s2 <= li) {
              for (int i = 0; i < 32; ++i) {
                const float f =
                    (bp.X[s2row + i] * rk_s2) *
                    exp2_fast((bp.Y[trow + i] - bp.Y[s2row + i]) + (sYlo[trow + i] - sYlo[s2row + i]));
                ap = fmaf(bp.Z[trow + i] * rq_t, f, ap);
                aa = fmaf(bp.X[trow + i] * rk_t, f, aa);
              }
            }
            ap = group_sum(ap);
            aa = group_sum(aa);
            if (gq == 0) {
              bp.A[(16 * bt + li) * LdC + 16 * bt + s2] = s2 < li ? -aa : 0.0f;
              bp.P[(16 * bt + li) * LdC + 16 * bt + s2] = s2 <= li ? ap : 0.0f;
            }
          }
        }
      }
    }
    if (state_now) {
      // Delta = (I + A)^-1 R by blocks, then o = scale (Qg S + P Delta)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int k = 0; k < b; ++k) {
          const f4 x = *reinterpret_cast<const f4*>(bs.A + (16 * b + li) * LdC + 16 * k + 4 * gq);
#pragma unroll
          for (int r = 0; r < 4; ++r) reg[kD + b] = mma(x[r], reg[kD + k][r], reg[kD + b]);
        }
        const f4 x = *reinterpret_cast<const f4*>(&bs.Td[b][li * 20 + 4 * gq]);
        f4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) y = mma(x[r], reg[kD + b][r], y);
        reg[kD + b] = y;
      }
      f4 O[NB];
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) O[tb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sb2 = 0; sb2 < 8; ++sb2) {
        f4 x[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
          x[tb] = *reinterpret_cast<const f4*>(bs.Y + (16 * tb + li) * kLdK + 16 * sb2 + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int tb = 0; tb < NB; ++tb) O[tb] = mma(x[tb][r], reg[kS + sb2][r], O[tb]);
      }
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        f4 x[NB];
#pragma unroll
        for (int tb = kb; tb < NB; ++tb)
          x[tb] = *reinterpret_cast<const f4*>(bs.P + (16 * tb + li) * LdC + 16 * kb + 4 * gq);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int tb = kb; tb < NB; ++tb) O[tb] = mma(x[tb][r], reg[kD + kb][r], O[tb]);
      }
      const __amdgpu_buffer_rsrc_t orsrc =
          buffer_descriptor(a.out + (cs * hk + static_cast<int64_t>(h) * 128 + col_w),
                            (static_cast<uint32_t>(ns - 1) * hk32 + 16) * 4);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t tr = static_cast<uint32_t>(16 * tb + 4 * gq + r);
          raw_buffer_store_f32(a.scale * O[tb][r], orsrc,
                               static_cast<int>((tr * hk32 + static_cast<uint32_t>(li)) * 4));
        }
    }
    __syncthreads();

    // ================= segment 3 =================
    if (prep_now) {
      // operands -Kb, Qg, Kd of chunk it in place of its rows; diagonal inverses
      prefetch_rows(cp + C < t1 ? cp + C : cp, li, gq);
      const int pb = pw % NB, pp = pw / NB;
      const int tl = 16 * pb + li;
      const int ch0 = pp * (128 / PARTS) + gq * CPL;
      const int row = tl * kLdK + ch0;
      float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
      for (int u = 0; u < PARTS; ++u) {
        ssq += bp.Sq[u][tl];
        ssk += bp.Sk[u][tl];
      }
      const float rq = 1.0f / sqrtf(ssq + 1e-6f);
      const float rk = 1.0f / sqrtf(ssk + 1e-6f);
      const float beta = bp.Beta[tl];
#pragma unroll
      for (int m = 0; m < CPL; m += 4) {
        const int ch = ch0 + m;
        const f4 k4 = *reinterpret_cast<const f4*>(bp.X + row + m);
        const f4 gl4 = *reinterpret_cast<const f4*>(bp.Y + row + m);
        const f4 q4 = *reinterpret_cast<const f4*>(bp.Z + row + m);
        const f4 pre = *reinterpret_cast<const f4*>(&bp.Pre[pb][ch]);
        const f4 post = *reinterpret_cast<const f4*>(&bp.Suf[pb][ch]);
        const f4 sf = reg[kF + m / 4];
        f4 nkb, qg, kd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float kn = k4[e] * rk;
          const float eg = exp2_fast(pre[e] + gl4[e]);
          nkb[e] = -((beta * kn) * eg);
          qg[e] = (q4[e] * rq) * eg;
          kd[e] = kn * exp2_fast(post[e] + sf[e]);
        }
        *reinterpret_cast<f4*>(bp.X + row + m) = nkb;
        *reinterpret_cast<f4*>(bp.Y + row + m) = qg;
        *reinterpret_cast<f4*>(bp.Z + row + m) = kd;
      }
      // P_tt = qn_t . kn_t (no decay) in place of the chain's value
      if (pp == 0 && gq == 0) {
        float qk = 0.0f;
#pragma unroll
        for (int u = 0; u < PARTS; ++u) qk += bp.Sqk[u][tl];
        bp.P[tl * LdC + tl] = (qk * rq) * rk;
      }
      if (pw < NB && gq == 0) {
        const int b = pw;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          float acc = t == li ? 1.0f : 0.0f;
#pragma unroll
          for (int s2 = 0; s2 < t; ++s2)
            acc = fmaf(bp.A[(16 * b + t) * LdC + 16 * b + s2], x[s2], acc);
          x[t] = acc;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) bp.Td[b][t * 20 + li] = x[t];
      }
    }
    if (state_now) {
      // S = 2^(G_C) S + Kd^T Delta
#pragma unroll
      for (int sb2 = 0; sb2 < 8; ++sb2)
#pragma unroll
        for (int r = 0; r < 4; ++r) reg[kS + sb2][r] *= bs.GC[16 * sb2 + 4 * gq + r];
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int hb = 0; hb < 8; hb += 4) {  // four state row blocks at a time
          f4 x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              x[j][r] = bs.Z[(16 * tb + 4 * gq + r) * kLdK + 16 * (hb + j) + li];
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              reg[kS + hb + j] = mma(x[j][r], reg[kD + tb][r], reg[kS + hb + j]);
        }
    }
    __syncthreads();
  }

  // -- final state (state waves) to the destination slot.  The lane indices
  // and the wave's columns are re-derived from an opaque thread id, as in
  // the chunk loop: kept live from the kernel's start, the column offset
  // was spilled to scratch.
  if (state_wave) {
    int64_t dst_off = static_cast<int64_t>(dst) * a.H * 128 * 128 + head_off;
    asm volatile("" : "+s"(dst_off));
    T* dstp = static_cast<T*>(a.pool) + dst_off;
    int tid_f = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(tid_f));
    const int li = tid_f % 16, gq = (tid_f % 64) / 16, cw = 16 * (tid_f / 64);
#pragma unroll
    for (int sb2 = 0; sb2 < 8; ++sb2)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        narrow1(dstp + (16 * sb2 + 4 * gq + r) * 128 + cw + li, reg[kS + sb2][r]);
  }
}

template <typename T>
hipError_t launch_prefill_ws(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((kda_prefill_ws_kernel<T>), dim3(static_cast<uint32_t>(a.n_seq) * a.H),
                     dim3(64 * (kWsState + kWsPrep)), 0, s, a);
  return hipGetLastError();
}

template <typename T, int NB, int NW>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((kda_prefill_kernel<T, NB, NW>), dim3(static_cast<uint32_t>(a.n_seq) * a.H),
                     dim3(64 * NW), 0, s, a);
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
  if (pool->H > 16384) return KDA_ERR_SHAPE;  // byte offsets within a chunk stay below 2^31
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
    err = chunk == 64 ? launch_prefill<float, 4, 8>(a, s) : launch_prefill_ws<float>(a, s);
  else
    err = chunk == 64 ? launch_prefill<_Float16, 4, 8>(a, s) : launch_prefill_ws<_Float16>(a, s);
  return err == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}
