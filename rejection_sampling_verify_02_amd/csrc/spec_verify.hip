// spec_verify.hip -- batched speculative-sampling verification for MI355X (gfx950).
//
// What is computed ("Speculative Decoding 的朴素思想", sections "一次 sampling 怎么执行",
// "Correction 为什么用正残差", "从单个 token 接到一段 draft"; "推测解码：接受规则、状态与
// 收益边界", section "两模型精确采样"; greedy: tannlonggtaoo note, "Greedy Sampling"):
// for each sequence, the drafted tokens are tested in order against min(1, p/q); the
// first rejection draws a correction from norm([p - q]_+), an all-accept round draws a
// bonus from the target's next distribution, both by inverse CDF.
//
// How it is laid out on the GPU.  Every logit row is cut into chunks of
// CHUNK_VECS 16-byte vectors (8192 bf16 / 4096 f32 values); one 256-thread workgroup
// (four wave64s) streams one chunk.  The work is HBM-bound streaming with one exp per
// element, so there is no MFMA: the design goal is coalesced 128-bit loads, few VALU
// operations per element, and no second pass over the bulk of the data.
//
//   k_topk_digit  (only with top-k)  radix select of the k-th largest raw logit per row,
//                 one 8-bit digit per launch (2 launches for bf16, 4 for f32), LDS
//                 histograms per chunk, the last chunk of a row picks the digit.
//   k_norm        per chunk: max and sum of 2^(z*log2(e)/T - offset) (one v_exp_f32 per
//                 element); the last chunk of a row combines the chunk partials into
//                 the row's log-partition; the last row of a sequence runs the
//                 acceptance scan (first rejection, row / token / uniform checks) and
//                 leaves a job (reject at j, or bonus) for the second kernel.
//   k_argmax      greedy (T == 0) counterpart of k_norm over the target rows only.
//   k_sample      per chunk of a rejecting sequence: mass of [p_j - q_j]_+; the last
//                 chunk chooses the chunk / 64-vector segment / lane / element where the
//                 cumulative mass passes u*Z.  Bonus sequences choose the chunk from the
//                 first kernel's partial sums and re-read only that chunk.
//
// "Last chunk / last row" is decided with self-resetting ticket counters (atomicInc
// with wrap-around) kept at the start of the workspace: a call needs those leading
// bytes at zero and leaves them at zero, so no host sync or memset happens between
// kernels or between calls of one shape.  All reductions use fixed trees or fixed orders, so
// results are bitwise reproducible run to run.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spec_verify.h"

#define SVD __device__ __forceinline__

namespace sv {

constexpr int NT = 256;                // threads per workgroup
constexpr int WAVE = 64;               // gfx950 wavefront
constexpr int NW = NT / WAVE;          // waves per workgroup
constexpr int VPT = 4;                 // 16-byte vectors per thread per chunk
constexpr int CHUNK_VECS = NT * VPT;   // vectors per chunk (16 KiB of logits)
constexpr int SEGS = VPT * NW;         // 64-vector segments per chunk
constexpr double LN2 = 0.69314718055994530942;
constexpr double LOG2E = 1.44269504088896340736;

enum : int { JOB_NONE = 0, JOB_REJECT = 1, JOB_BONUS = 2 };

// ---------------------------------------------------------------- element formats

template <typename T>
struct Fmt;

template <>
struct Fmt<uint16_t> {  // bf16 bit patterns: the upper half of an IEEE binary32
  static constexpr int VEC = 8;
  SVD static float at(const uint16_t *p, size_t i) { return __uint_as_float((uint32_t)p[i] << 16); }
  SVD static void vec(const uint16_t *p, size_t v, float (&o)[8]) {
    const uint4 w = reinterpret_cast<const uint4 *>(p)[v];
    o[0] = __uint_as_float(w.x << 16);
    o[1] = __uint_as_float(w.x & 0xffff0000u);
    o[2] = __uint_as_float(w.y << 16);
    o[3] = __uint_as_float(w.y & 0xffff0000u);
    o[4] = __uint_as_float(w.z << 16);
    o[5] = __uint_as_float(w.z & 0xffff0000u);
    o[6] = __uint_as_float(w.w << 16);
    o[7] = __uint_as_float(w.w & 0xffff0000u);
  }
};

template <>
struct Fmt<float> {
  static constexpr int VEC = 4;
  SVD static float at(const float *p, size_t i) { return p[i]; }
  SVD static void vec(const float *p, size_t v, float (&o)[4]) {
    const float4 w = reinterpret_cast<const float4 *>(p)[v];
    o[0] = w.x;
    o[1] = w.y;
    o[2] = w.z;
    o[3] = w.w;
  }
};

// Vector k of this thread in chunk c is vector c*CHUNK_VECS + k*NT + tid of the row, so
// one wave's k-th load covers 64 consecutive vectors (a "segment") and segments are in
// vocabulary order (k-major, then wave).  Vectors past the row end read as -inf.
template <typename T, bool ALIGNED>
SVD void load_chunk(const T *row, int V, int nvec, int c, int tid, float (&x)[VPT][Fmt<T>::VEC]) {
  constexpr int VEC = Fmt<T>::VEC;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = c * CHUNK_VECS + k * NT + tid;
    if (ALIGNED) {
      if (v < nvec) {
        Fmt<T>::vec(row, (size_t)v, x[k]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[k][e] = -INFINITY;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const long idx = (long)v * VEC + e;
        x[k][e] = (v < nvec && idx < V) ? Fmt<T>::at(row, (size_t)idx) : -INFINITY;
      }
    }
  }
}

// Index of element (k, e) of this thread in chunk c.
template <typename T>
SVD long elem_index(int c, int k, int tid, int e) {
  return ((long)c * CHUNK_VECS + (long)k * NT + tid) * Fmt<T>::VEC + e;
}

// ---------------------------------------------------------------- arguments

struct Work {                  // carved from the caller's workspace
  float *part_off;             // [R*C] chunk offset (log2 units) / greedy: chunk best value
  double *part_sum;            // [R*C] chunk sum of 2^(z*k2 - off)
  int *part_idx;               // [R*C] greedy: chunk best index; bit flags in part_flag
  int *part_flag;              // [R*C] greedy: 1 = NaN/+inf seen, 2 = finite seen
  float *row_off;              // [R] row offset
  double *row_l2s;             // [R] log2 of the row sum: log2-partition = off + l2s
  int *row_ok;                 // [R] row usable
  int *row_arg;                // [R] greedy argmax
  float *row_tau;              // [R] top-k threshold (raw logit); rows with no cut: -inf
  uint2 *tk_state;             // [R] radix-select prefix and remaining rank
  unsigned *tk_hist;           // [R*C*256] per-chunk digit histograms
  unsigned *t_row;             // [R] tickets (self-resetting)
  unsigned *t_seq;             // [B]
  unsigned *t_p2;              // [B]
  int2 *job;                   // [B] (j, kind)
  double *p2_chunk;            // [B*C] residual mass per chunk
};

struct Args {
  const void *target, *draft;
  const int32_t *tokens;
  const float *u_accept, *u_sample;
  int B, G, V, C, nvec, rps;   // rps: rows per sequence (2G+1 sampling, G+1 greedy)
  float k2;                    // log2(e) / T, the one rounding of the temperature used everywhere
  int top_k;
  int32_t *accepted_len, *out_tokens;
  float *row_stats;
  Work w;
};

// Row r of the flattened (sequence, row) list: rows 0..G of a sequence are target rows
// 0..G, rows G+1..2G are draft rows 0..G-1.
template <typename T>
SVD const T *seq_row(const Args &a, int b, int j) {
  if (j <= a.G) return static_cast<const T *>(a.target) + ((size_t)b * (a.G + 1) + j) * (size_t)a.V;
  return static_cast<const T *>(a.draft) + ((size_t)b * a.G + (j - a.G - 1)) * (size_t)a.V;
}

// ---------------------------------------------------------------- small helpers

SVD float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32; 0 for x < -126

// (off, s) pairs stand for s * 2^off; combining keeps the larger offset.  Chunks that
// hold only -inf have off = -inf and s = 0 (or NaN when a NaN was seen); the rule never
// forms (-inf) - (-inf).
SVD void lse_combine(float &off, double &s, float off2, double s2) {
  const float mx = fmaxf(off, off2);
  const double w1 = (off == mx) ? 1.0 : (double)fast_exp2(off - mx);
  const double w2 = (off2 == mx) ? 1.0 : (double)fast_exp2(off2 - mx);
  s = s * w1 + s2 * w2;
  off = mx;
}

SVD void wave_lse(float &off, double &s) {
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) {
    const float off2 = __shfl_xor(off, o);
    const double s2 = __shfl_xor(s, o);
    lse_combine(off, s, off2, s2);
  }
}

SVD double wave_sum(double v) {
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Is this workgroup the last of n to arrive at *ctr?  The counter wraps back to zero on
// the last arrival, so it is ready for the next call.  Release / acquire fences at
// device scope make the partial results of the other workgroups (possibly on other
// XCDs) visible to the winner.
SVD bool last_arrival(unsigned *ctr, unsigned n) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicInc(ctr, n - 1) == n - 1);
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __threadfence();
  return last;
}

// Order-preserving 32-bit key of a float (bf16 values are floats with zero low half);
// -0 and +0 share a key.
SVD uint32_t f2key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
SVD float key2f(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }

// ---------------------------------------------------------------- top-k threshold

// One radix-select digit (bits [shift, shift+8) of the key) for every row.  The prefix
// of higher digits and the remaining rank come from the previous pass.  The threshold
// kept in row_tau is the smallest value whose key has the final prefix, so the kept set
// {z >= tau} is exactly the values >= the k-th largest, ties included.
template <typename T, bool ALIGNED>
__global__ __launch_bounds__(NT) void k_topk_digit(const Args a, int pass, int last_pass) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ unsigned hist[256];
  __shared__ unsigned s_ge[256];
  const int tid = threadIdx.x;
  const int r = blockIdx.x / a.C, c = blockIdx.x - r * a.C;
  const int b = r / a.rps, jr = r - b * a.rps;
  const int shift = 24 - 8 * pass;
  const uint2 st = (pass == 0) ? make_uint2(0u, (unsigned)a.top_k) : a.w.tk_state[r];
  const uint32_t hi_mask = (pass == 0) ? 0u : (0xffffffffu << (shift + 8));

  hist[tid] = 0u;
  __syncthreads();
  float x[VPT][VEC];
  load_chunk<T, ALIGNED>(seq_row<T>(a, b, jr), a.V, a.nvec, c, tid, x);
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (elem_index<T>(c, k, tid, e) < a.V) {
        const uint32_t key = f2key(x[k][e]);
        if ((key & hi_mask) == (st.x & hi_mask)) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
  __syncthreads();
  a.w.tk_hist[((size_t)r * a.C + c) * 256 + tid] = hist[tid];
  if (!last_arrival(&a.w.t_row[r], (unsigned)a.C)) return;

  // Row total of digit d = tid, then counts of keys with digit >= d.
  unsigned tot = 0;
  for (int cc = 0; cc < a.C; ++cc) tot += a.w.tk_hist[((size_t)r * a.C + cc) * 256 + tid];
  s_ge[tid] = tot;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {  // suffix sums (Hillis-Steele)
    const unsigned add = (tid + o < 256) ? s_ge[tid + o] : 0u;
    __syncthreads();
    s_ge[tid] += add;
    __syncthreads();
  }
  // The chosen digit is the largest d whose suffix count reaches the remaining rank.
  const unsigned krem = st.y;
  const bool reach = s_ge[tid] >= krem;
  const bool next_reach = (tid < 255) ? (s_ge[tid + 1] >= krem) : false;
  if (reach && !next_reach) {
    const unsigned above = (tid < 255) ? s_ge[tid + 1] : 0u;
    const uint32_t prefix = (st.x & hi_mask) | ((uint32_t)tid << shift);
    if (last_pass) a.w.row_tau[r] = key2f(prefix);
    else a.w.tk_state[r] = make_uint2(prefix, krem - above);
  }
}

// ---------------------------------------------------------------- acceptance scan

// Run by the last-finishing row of sequence b, after every row's statistics are in
// the workspace.  Position i of the chain: token range, row validity, uniform range,
// draft support, then the test U_i <= min(1, p_i(x)/q_i(x)) with p_i(x) > 0 ([WY]
// "一次 sampling 怎么执行" step 4; the ratio is formed from log2-probabilities in double).
template <typename T, bool GREEDY>
SVD void sequence_scan(const Args &a, int b) {
  __shared__ int s_j, s_flags;
  const int tid = threadIdx.x;
  const int G = a.G, rps = a.rps;
  if (tid == 0) {
    s_j = G;
    s_flags = 0;
  }
  __syncthreads();
  int flags = 0;  // 1 bad token, 2 bad row, 4 bad uniform, 8 q(x) = 0
  for (int i = tid; i < G; i += NT) {
    const int x = a.tokens[(size_t)b * G + i];
    const bool tok_ok = (x >= 0) && (x < a.V);
    if (!tok_ok) flags |= 1;
    const int rt = b * rps + i;
    bool accept = false;
    if (GREEDY) {
      if (!a.w.row_ok[rt]) flags |= 2;
      accept = tok_ok && a.w.row_ok[rt] && (x == a.w.row_arg[rt]);
    } else {
      const int rd = b * rps + G + 1 + i;
      if (!a.w.row_ok[rt] || !a.w.row_ok[rd]) flags |= 2;
      const float u = a.u_accept[(size_t)b * G + i];
      if (!(u >= 0.0f && u < 1.0f)) flags |= 4;
      if (tok_ok) {
        const float tau_t = a.w.row_tau[rt], tau_d = a.w.row_tau[rd];
        const float zt = Fmt<T>::at(seq_row<T>(a, b, i), (size_t)x);
        const float zd = Fmt<T>::at(seq_row<T>(a, b, G + 1 + i), (size_t)x);
        const bool supp_t = (zt > -INFINITY) && !(zt < tau_t);
        const bool supp_d = (zd > -INFINITY) && !(zd < tau_d);
        if (!supp_d) flags |= 8;
        if (supp_t && supp_d && a.w.row_ok[rt] && a.w.row_ok[rd]) {
          const double k2 = (double)a.k2;
          const double l2p = (double)zt * k2 - ((double)a.w.row_off[rt] + a.w.row_l2s[rt]);
          const double l2q = (double)zd * k2 - ((double)a.w.row_off[rd] + a.w.row_l2s[rd]);
          const double alpha = exp2(fmin(0.0, l2p - l2q));
          accept = (double)u <= alpha;
        }
      }
    }
    if (!accept) atomicMin(&s_j, i);
  }
  if (tid == 0) {
    const int rg = b * rps + G;  // target row G (the bonus distribution)
    if (!a.w.row_ok[rg]) flags |= 2;
    if (!GREEDY) {
      const float u = a.u_sample[b];
      if (!(u >= 0.0f && u < 1.0f)) flags |= 4;
    }
  }
  if (flags) atomicOr(&s_flags, flags);
  __syncthreads();
  const int fl = s_flags, j = s_j;
  const int err = (fl & 1) ? SV_ROW_BAD_TOKEN
                : (fl & 2) ? SV_ROW_BAD_LOGITS
                : (fl & 4) ? SV_ROW_BAD_UNIFORM
                : (fl & 8) ? SV_ROW_Q_ZERO : 0;
  int32_t *out = a.out_tokens + (size_t)b * (G + 1);
  for (int i = tid; i <= G; i += NT) {
    int32_t v;
    if (err) v = -1;
    else if (i < j) v = a.tokens[(size_t)b * G + i];
    else if (i > j) v = -1;
    else if (GREEDY) v = a.w.row_arg[b * rps + j];  // the target's own choice
    else continue;                                  // drawn by k_sample
    out[i] = v;
  }
  if (tid == 0) {
    a.accepted_len[b] = err ? err : j;
    a.w.job[b] = make_int2(j, (err || GREEDY) ? JOB_NONE : (j < G ? JOB_REJECT : JOB_BONUS));
  }
}

// ---------------------------------------------------------------- pass 1: normaliser

// Per chunk: m = max kept z, off = m*k2 (rounded once), s = sum 2^(fma(z, k2, -off)).
// The log2-partition of the row is off_row + log2(s_row), with off_row the float actually
// subtracted, so every consumer reproduces the same probabilities.
template <typename T, bool ALIGNED, bool TOPK>
__global__ __launch_bounds__(NT) void k_norm(const Args a) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ float s_off[NW];
  __shared__ double s_sum[NW];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;
  const int r = blockIdx.x / a.C, c = blockIdx.x - r * a.C;
  const int b = r / a.rps, jr = r - b * a.rps;

  float x[VPT][VEC];
  load_chunk<T, ALIGNED>(seq_row<T>(a, b, jr), a.V, a.nvec, c, tid, x);
  if (TOPK) {
    const float tau = a.w.row_tau[r];
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[k][e] = (x[k][e] < tau) ? -INFINITY : x[k][e];
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) m = fmaxf(m, x[k][e]);

  float off;
  double s;
  const float k2 = a.k2;
  if (m > -INFINITY) {
    off = m * k2;
    float acc[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float t[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) t[e] = fast_exp2(fmaf(x[k][e], k2, -off));
#pragma unroll
      for (int h = VEC / 2; h > 0; h >>= 1)
#pragma unroll
        for (int e = 0; e < h; ++e) t[e] += t[e + h];
      acc[k] = t[0];
    }
    s = (double)((acc[0] + acc[1]) + (acc[2] + acc[3]));
  } else {  // nothing finite here: keep a NaN visible, otherwise an empty partial
    off = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) nan |= (x[k][e] != x[k][e]);
    s = nan ? (double)NAN : 0.0;
  }
  wave_lse(off, s);
  if (lane == 0) {
    s_off[wid] = off;
    s_sum[wid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float o = s_off[0];
    double t = s_sum[0];
    for (int w = 1; w < NW; ++w) lse_combine(o, t, s_off[w], s_sum[w]);
    a.w.part_off[(size_t)r * a.C + c] = o;
    a.w.part_sum[(size_t)r * a.C + c] = t;
  }
  if (!last_arrival(&a.w.t_row[r], (unsigned)a.C)) return;

  // Row: combine the C chunk partials (strided per thread, then a fixed tree).
  {
    float o = -INFINITY;
    double t = 0.0;
    for (int cc = tid; cc < a.C; cc += NT)
      lse_combine(o, t, a.w.part_off[(size_t)r * a.C + cc], a.w.part_sum[(size_t)r * a.C + cc]);
    wave_lse(o, t);
    __syncthreads();
    if (lane == 0) {
      s_off[wid] = o;
      s_sum[wid] = t;
    }
    __syncthreads();
    if (tid == 0) {
      o = s_off[0];
      t = s_sum[0];
      for (int w = 1; w < NW; ++w) lse_combine(o, t, s_off[w], s_sum[w]);
      const bool ok = isfinite(o) && isfinite(t) && t > 0.0;
      a.w.row_off[r] = o;
      a.w.row_l2s[r] = ok ? log2(t) : 0.0;
      a.w.row_ok[r] = ok ? 1 : 0;
      if (!TOPK) a.w.row_tau[r] = -INFINITY;
      if (a.row_stats) {
        a.row_stats[(size_t)r * 2 + 0] = (float)((double)o * LN2);
        a.row_stats[(size_t)r * 2 + 1] = (float)t;
      }
    }
  }
  if (!last_arrival(&a.w.t_seq[b], (unsigned)a.rps)) return;
  sequence_scan<T, false>(a, b);
}

// ---------------------------------------------------------------- pass 1: greedy argmax

// Largest value wins, ties go to the lower index; NaN and +inf mark the row unusable.
SVD void best_combine(float &v, int &i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

template <typename T, bool ALIGNED>
__global__ __launch_bounds__(NT) void k_argmax(const Args a) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ float s_v[NW];
  __shared__ int s_i[NW], s_f[NW];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;
  const int r = blockIdx.x / a.C, c = blockIdx.x - r * a.C;
  const int b = r / a.rps, jr = r - b * a.rps;

  float x[VPT][VEC];
  load_chunk<T, ALIGNED>(seq_row<T>(a, b, jr), a.V, a.nvec, c, tid, x);
  float best = -INFINITY;
  int bi = 0x7fffffff, fl = 0;
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float z = x[k][e];
      if (z > best) {  // strict: the first (lowest-index) maximum of this thread stays
        best = z;
        bi = (int)elem_index<T>(c, k, tid, e);
      }
      fl |= ((z != z) || (z == INFINITY)) ? 1 : 0;
    }
  if (best > -INFINITY && best < INFINITY) fl |= 2;
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(best, o);
    const int i2 = __shfl_xor(bi, o);
    fl |= __shfl_xor(fl, o);
    best_combine(best, bi, v2, i2);
  }
  if (lane == 0) {
    s_v[wid] = best;
    s_i[wid] = bi;
    s_f[wid] = fl;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < NW; ++w) {
      best_combine(best, bi, s_v[w], s_i[w]);
      fl |= s_f[w];
    }
    a.w.part_off[(size_t)r * a.C + c] = best;
    a.w.part_idx[(size_t)r * a.C + c] = bi;
    a.w.part_flag[(size_t)r * a.C + c] = fl;
  }
  if (!last_arrival(&a.w.t_row[r], (unsigned)a.C)) return;

  {
    best = -INFINITY;
    bi = 0x7fffffff;
    fl = 0;
    for (int cc = tid; cc < a.C; cc += NT) {
      best_combine(best, bi, a.w.part_off[(size_t)r * a.C + cc], a.w.part_idx[(size_t)r * a.C + cc]);
      fl |= a.w.part_flag[(size_t)r * a.C + cc];
    }
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(best, o);
      const int i2 = __shfl_xor(bi, o);
      fl |= __shfl_xor(fl, o);
      best_combine(best, bi, v2, i2);
    }
    __syncthreads();
    if (lane == 0) {
      s_v[wid] = best;
      s_i[wid] = bi;
      s_f[wid] = fl;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NW; ++w) {
        best_combine(best, bi, s_v[w], s_i[w]);
        fl |= s_f[w];
      }
      a.w.row_arg[r] = bi;
      a.w.row_ok[r] = (fl == 2) ? 1 : 0;
    }
  }
  if (!last_arrival(&a.w.t_seq[b], (unsigned)a.rps)) return;
  sequence_scan<T, true>(a, b);
}

// ---------------------------------------------------------------- pass 2: the draw

// Weights of the correction draw: w = max(p - q, 0) with p = 2^(z_t*k2 - Mt) and
// q = 2^(z_d*k2 - Md).  The log2-partitions are split into a float head and tail so the
// per-element arguments carry only their own rounding.
struct ResidualW {
  float k2, mt_hi, mt_lo, md_hi, md_lo, tau_t, tau_d;
  SVD float operator()(float zt, float zd) const {
    zt = (zt < tau_t) ? -INFINITY : zt;
    zd = (zd < tau_d) ? -INFINITY : zd;
    const float p = fast_exp2(fmaf(zt, k2, -mt_hi) - mt_lo);
    const float q = fast_exp2(fmaf(zd, k2, -md_hi) - md_lo);
    return fmaxf(p - q, 0.0f);
  }
};

// Weights of a draw from the target row itself (bonus, or the zero-residual fallback),
// relative to one chunk's offset as in the first kernel.
struct TargetW {
  float k2, off, tau;
  SVD float operator()(float zt, float) const {
    zt = (zt < tau) ? -INFINITY : zt;
    return fast_exp2(fmaf(zt, k2, -off));
  }
};

// Inverse CDF inside one chunk: the element whose cumulative weight (in vocabulary
// order) first exceeds t.  Segment masses and lane masses are summed in fixed orders;
// when rounding leaves t at or past the chunk's total, the last element with positive
// weight is taken.  If `store_total`, also returns the chunk total through *total.
// Returns the element index within the row (block-uniform), or -1 for a zero chunk.
template <typename T, bool ALIGNED, typename WFn>
SVD int chunk_draw(const Args &a, const T *rowA, const T *rowB, int c, const WFn &wf, double t,
                   bool search, double *total) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ double s_seg[SEGS];
  __shared__ double s_t;
  __shared__ int s_seg_pick, s_last_mode, s_result;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;

  float xa[VPT][VEC], xb[VPT][VEC];
  load_chunk<T, ALIGNED>(rowA, a.V, a.nvec, c, tid, xa);
  if (rowB) {
    load_chunk<T, ALIGNED>(rowB, a.V, a.nvec, c, tid, xb);
  } else {
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) xb[k][e] = -INFINITY;
  }
  float wv[VPT][VEC], ls[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      wv[k][e] = wf(xa[k][e], xb[k][e]);
      acc += wv[k][e];
    }
    ls[k] = acc;
    const double seg = wave_sum((double)acc);
    if (lane == 0) s_seg[k * NW + wid] = seg;
  }
  __syncthreads();
  if (tid == 0) {
    double cum = 0.0;
    int pick = -1, lastpos = -1;
    for (int sidx = 0; sidx < SEGS; ++sidx) {
      const double m = s_seg[sidx];
      if (m > 0.0) lastpos = sidx;
      if (pick < 0 && search && cum + m > t) {
        pick = sidx;
        s_t = t - cum;
      }
      cum += m;
    }
    if (total) *total = cum;
    s_last_mode = 0;
    if (pick < 0) {  // rounding (or a zero chunk): take the last positive element
      pick = lastpos;
      s_last_mode = 1;
      s_t = 0.0;
    }
    s_seg_pick = pick;
    s_result = -1;
  }
  __syncthreads();
  if (!search) return -1;
  const int sp = s_seg_pick;
  if (sp >= 0 && wid == sp % NW) {
    const int kp = sp / NW;
    float lsum = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      if (k == kp) lsum = ls[k];
    // inclusive scan of lane masses across the wave (double)
    double cum = (double)lsum;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
      const double up = __shfl_up(cum, o);
      if (lane >= o) cum += up;
    }
    const double before = cum - (double)lsum;
    const double tt = s_t;
    const bool last_mode = s_last_mode != 0;
    const unsigned long long cross = __ballot(!last_mode && cum > tt);
    const unsigned long long posm = __ballot(lsum > 0.0f);
    int pl;
    bool lane_last = last_mode;
    if (cross) {
      pl = __ffsll((long long)cross) - 1;
    } else {
      pl = 63 - __clzll((long long)posm);
      lane_last = true;
    }
    if (lane == pl) {
      float we[VEC];
#pragma unroll
      for (int k = 0; k < VPT; ++k)
        if (k == kp)
#pragma unroll
          for (int e = 0; e < VEC; ++e) we[e] = wv[k][e];
      int pe = -1, lastpe = -1;
      double run = before;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        if (we[e] > 0.0f) lastpe = e;
        run += (double)we[e];
        if (pe < 0 && !lane_last && run > tt) pe = e;
      }
      if (pe < 0) pe = lastpe;
      s_result = (int)elem_index<T>(c, kp, tid, pe);
    }
  }
  __syncthreads();
  return s_result;
}

// Choose the chunk of a target row from the first kernel's partials (masses
// S_c * 2^(off_c - off_row), summed in chunk order) and the in-chunk target.
SVD void pick_chunk_from_partials(const Args &a, int r, float u, int *c_out, double *t_out) {
  const float off_r = a.w.row_off[r];
  double total = 0.0;
  for (int cc = 0; cc < a.C; ++cc) {
    const double s = a.w.part_sum[(size_t)r * a.C + cc];
    if (s > 0.0) total += s * (double)fast_exp2(a.w.part_off[(size_t)r * a.C + cc] - off_r);
  }
  const double t = (double)u * total;
  double cum = 0.0;
  int pick = -1, lastpos = -1;
  double tin = 0.0;
  for (int cc = 0; cc < a.C; ++cc) {
    const double s = a.w.part_sum[(size_t)r * a.C + cc];
    if (!(s > 0.0)) continue;
    const float d = a.w.part_off[(size_t)r * a.C + cc] - off_r;
    const double m = s * (double)fast_exp2(d);
    lastpos = cc;
    if (pick < 0 && cum + m > t) {
      pick = cc;
      tin = (t - cum) * (double)fast_exp2(-d);  // back in the chunk's own scale
    }
    cum += m;
  }
  if (pick < 0) {
    pick = lastpos;
    tin = INFINITY;  // past the end: the chunk search falls back to its last positive element
  }
  *c_out = pick;
  *t_out = tin;
}

template <typename T, bool ALIGNED>
SVD int draw_from_target_row(const Args &a, int b, int jrow, float u) {
  __shared__ int s_c;
  __shared__ double s_tin;
  const int r = b * a.rps + jrow;
  if (threadIdx.x == 0) {
    int c;
    double tin;
    pick_chunk_from_partials(a, r, u, &c, &tin);
    s_c = c;
    s_tin = tin;
  }
  __syncthreads();
  const int c = s_c;
  if (c < 0 || c >= a.C) return -1;  // no chunk with positive mass: nothing to draw
  TargetW wf{a.k2, a.w.part_off[(size_t)r * a.C + c], a.w.row_tau[r]};
  return chunk_draw<T, ALIGNED>(a, seq_row<T>(a, b, jrow), (const T *)nullptr, c, wf, s_tin, true,
                                nullptr);
}

template <typename T, bool ALIGNED>
__global__ __launch_bounds__(NT) void k_sample(const Args a) {
  __shared__ double s_total;
  __shared__ int s_c;
  __shared__ double s_tc;
  __shared__ int s_fallback;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / a.C, c = blockIdx.x - b * a.C;
  const int2 jk = a.w.job[b];
  const int j = jk.x, kind = jk.y, G = a.G;
  int32_t *out = a.out_tokens + (size_t)b * (G + 1);
  const float u = a.u_sample[b];

  // The job comes from the workspace: accept only well-formed ones, so that stale or
  // foreign workspace contents can never become an out-of-range row index.
  if (!((kind == JOB_REJECT && j >= 0 && j < G) || (kind == JOB_BONUS && j == G))) return;
  if (kind == JOB_BONUS) {
    if (tid == 0) {
      int cp;
      double tin;
      pick_chunk_from_partials(a, b * a.rps + G, u, &cp, &tin);
      s_c = cp;
    }
    __syncthreads();
    if (s_c != c) return;  // also covers s_c == -1 (no chunk with positive mass)
    const int tok = draw_from_target_row<T, ALIGNED>(a, b, G, u);
    if (tid == 0) out[G] = tok;
    return;
  }

  // Rejection at position j: mass of [p_j - q_j]_+ over this chunk.
  const int rt = b * a.rps + j, rd = b * a.rps + G + 1 + j;
  const double mt = (double)a.w.row_off[rt] + a.w.row_l2s[rt];
  const double md = (double)a.w.row_off[rd] + a.w.row_l2s[rd];
  ResidualW wf;
  wf.k2 = a.k2;
  wf.mt_hi = (float)mt;
  wf.mt_lo = (float)(mt - (double)wf.mt_hi);
  wf.md_hi = (float)md;
  wf.md_lo = (float)(md - (double)wf.md_hi);
  wf.tau_t = a.w.row_tau[rt];
  wf.tau_d = a.w.row_tau[rd];
  const T *row_t = seq_row<T>(a, b, j), *row_d = seq_row<T>(a, b, G + 1 + j);
  chunk_draw<T, ALIGNED>(a, row_t, row_d, c, wf, 0.0, false, &s_total);
  if (tid == 0) a.w.p2_chunk[(size_t)b * a.C + c] = s_total;
  if (!last_arrival(&a.w.t_p2[b], (unsigned)a.C)) return;

  if (tid == 0) {
    double Z = 0.0;
    for (int cc = 0; cc < a.C; ++cc) Z += a.w.p2_chunk[(size_t)b * a.C + cc];
    s_fallback = !(Z > 0.0);
    const double t = (double)u * Z;
    double cum = 0.0;
    int pick = -1, lastpos = -1;
    double tc = 0.0;
    for (int cc = 0; cc < a.C; ++cc) {
      const double m = a.w.p2_chunk[(size_t)b * a.C + cc];
      if (m > 0.0) lastpos = cc;
      if (pick < 0 && m > 0.0 && cum + m > t) {
        pick = cc;
        tc = t - cum;
      }
      cum += m;
    }
    if (pick < 0) {
      pick = lastpos;
      tc = INFINITY;
    }
    s_c = pick;
    s_tc = tc;
  }
  __syncthreads();
  int tok = -1;
  if (s_fallback) {  // zero residual (only through rounding): draw from p_j itself
    tok = draw_from_target_row<T, ALIGNED>(a, b, j, u);
  } else if (s_c >= 0 && s_c < a.C) {
    tok = chunk_draw<T, ALIGNED>(a, row_t, row_d, s_c, wf, s_tc, true, nullptr);
  }
  if (tid == 0) out[j] = tok;
}

}  // namespace sv

// ======================================================================== host side

namespace {

using namespace sv;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  bool greedy, topk, aligned;
  int esz, vec, nvec, C, rps;
  long long R;
  int digit_passes;
  // workspace offsets
  size_t part_off, part_sum, part_idx, part_flag, row_off, row_l2s, row_ok, row_arg, row_tau,
      tk_state, tk_hist, t_row, t_seq, t_p2, job, p2_chunk, total;
  size_t zero_bytes;  // leading bytes (the tickets) that must be zero when a call starts
};

bool make_plan(int32_t B, int32_t G, int32_t V, sv_dtype dt, float T, int32_t top_k, Plan &p) {
  p.greedy = (T == 0.0f);
  p.esz = (dt == SV_BF16) ? 2 : 4;
  p.vec = 16 / p.esz;
  p.nvec = (int)(((long long)V + p.vec - 1) / p.vec);
  p.C = (p.nvec + CHUNK_VECS - 1) / CHUNK_VECS;
  p.rps = p.greedy ? (G + 1) : (2 * G + 1);
  p.R = (long long)B * p.rps;
  p.topk = !p.greedy && top_k > 0 && top_k < V;
  p.digit_passes = (dt == SV_BF16) ? 2 : 4;
  if (p.R * p.C > 0x7fffffffLL || (long long)B * p.C > 0x7fffffffLL) return false;
  const size_t R = (size_t)p.R, C = (size_t)p.C, Bz = (size_t)B;
  size_t o = 0;
  // tickets first: the part that must start (and stays) at zero
  p.t_row = o; o = align256(o + R * 4);
  p.t_seq = o; o = align256(o + Bz * 4);
  p.t_p2 = o; o = align256(o + Bz * 4);
  p.zero_bytes = o;
  p.part_off = o; o = align256(o + R * C * 4);
  p.part_sum = o; o = align256(o + R * C * 8);
  p.part_idx = o; o = align256(o + (p.greedy ? R * C * 4 : 0));
  p.part_flag = o; o = align256(o + (p.greedy ? R * C * 4 : 0));
  p.row_off = o; o = align256(o + R * 4);
  p.row_l2s = o; o = align256(o + R * 8);
  p.row_ok = o; o = align256(o + R * 4);
  p.row_arg = o; o = align256(o + R * 4);
  p.row_tau = o; o = align256(o + R * 4);
  p.tk_state = o; o = align256(o + (p.topk ? R * 8 : 0));
  p.tk_hist = o; o = align256(o + (p.topk ? R * C * 256 * 4 : 0));
  p.job = o; o = align256(o + Bz * 8);
  p.p2_chunk = o; o = align256(o + (p.greedy ? 0 : Bz * C * 8));
  p.total = o;
  return true;
}

const char *kPlanNames[] = {
    "k_topk_digit;k_topk_digit;k_norm;k_sample",
    "k_topk_digit;k_topk_digit;k_topk_digit;k_topk_digit;k_norm;k_sample",
    "k_norm;k_sample",
    "k_argmax",
};

template <typename T, bool AL>
hipError_t launch_all(const Plan &p, const Args &a, hipStream_t st, void *const *ev, int nev,
                      int *nl) {
  const dim3 blk(NT);
  const unsigned rows_grid = (unsigned)(p.R * p.C);
  const unsigned seq_grid = (unsigned)((long long)a.B * p.C);
  int n = 0;
  hipError_t e = hipSuccess;
  auto rec = [&](int i) {
    if (ev && i < nev) (void)hipEventRecord((hipEvent_t)ev[i], st);
  };
  auto go = [&](const void *fn, unsigned grid, void **args) {
    if (e != hipSuccess) return;
    e = hipLaunchKernel(fn, dim3(grid), blk, args, 0, st);
    if (e == hipSuccess) rec(++n);
  };
  rec(0);
  Args aa = a;
  if (p.greedy) {
    void *args[] = {&aa};
    go((const void *)&k_argmax<T, AL>, rows_grid, args);
  } else {
    if (p.topk) {
      for (int pass = 0; pass < p.digit_passes; ++pass) {
        int ps = pass, lp = (pass == p.digit_passes - 1) ? 1 : 0;
        void *args[] = {&aa, &ps, &lp};
        go((const void *)&k_topk_digit<T, AL>, rows_grid, args);
      }
      void *args[] = {&aa};
      go((const void *)&k_norm<T, AL, true>, rows_grid, args);
    } else {
      void *args[] = {&aa};
      go((const void *)&k_norm<T, AL, false>, rows_grid, args);
    }
    void *args2[] = {&aa};
    go((const void *)&k_sample<T, AL>, seq_grid, args2);
  }
  if (nl) *nl = n;
  return e;
}

sv_status run(const void *target, const void *draft, sv_dtype dt, const int32_t *tokens,
              const float *u_accept, const float *u_sample, int32_t B, int32_t G, int32_t V,
              float T, int32_t top_k, int32_t *acc, int32_t *out, float *row_stats, void *ws,
              size_t ws_bytes, void *stream, void *const *ev, int32_t nev, int32_t *nl) {
  if (nl) *nl = 0;
  if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_DTYPE;
  if (B < 1 || G < 0 || V < 1) return SV_ERR_SHAPE;
  if (!(T >= 0.0f) || !isfinite(T)) return SV_ERR_TEMPERATURE;
  Plan p;
  if (!make_plan(B, G, V, dt, T, top_k, p)) return SV_ERR_SHAPE;
  const bool sampling = !p.greedy;
  if (!target || !acc || !out || !ws) return SV_ERR_NULL;
  if (G > 0 && !tokens) return SV_ERR_NULL;
  if (sampling && (!u_sample || (G > 0 && (!draft || !u_accept)))) return SV_ERR_NULL;
  const uintptr_t ta = (uintptr_t)target, da = (uintptr_t)draft;
  if (ta % p.esz || (sampling && G > 0 && da % p.esz)) return SV_ERR_ALIGN;
  if (ws_bytes < p.total || ((uintptr_t)ws & 255)) return SV_ERR_WORKSPACE;
  const bool aligned = ((size_t)V * p.esz) % 16 == 0 && ta % 16 == 0 &&
                       (!sampling || G == 0 || da % 16 == 0);

  char *base = static_cast<char *>(ws);
  Args a;
  a.target = target;
  a.draft = draft;
  a.tokens = tokens;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.B = B;
  a.G = G;
  a.V = V;
  a.C = p.C;
  a.nvec = p.nvec;
  a.rps = p.rps;
  a.k2 = sampling ? (float)(LOG2E / (double)T) : 0.0f;
  a.top_k = top_k;
  a.accepted_len = acc;
  a.out_tokens = out;
  a.row_stats = sampling ? row_stats : nullptr;
  a.w.part_off = (float *)(base + p.part_off);
  a.w.part_sum = (double *)(base + p.part_sum);
  a.w.part_idx = (int *)(base + p.part_idx);
  a.w.part_flag = (int *)(base + p.part_flag);
  a.w.row_off = (float *)(base + p.row_off);
  a.w.row_l2s = (double *)(base + p.row_l2s);
  a.w.row_ok = (int *)(base + p.row_ok);
  a.w.row_arg = (int *)(base + p.row_arg);
  a.w.row_tau = (float *)(base + p.row_tau);
  a.w.tk_state = (uint2 *)(base + p.tk_state);
  a.w.tk_hist = (unsigned *)(base + p.tk_hist);
  a.w.t_row = (unsigned *)(base + p.t_row);
  a.w.t_seq = (unsigned *)(base + p.t_seq);
  a.w.t_p2 = (unsigned *)(base + p.t_p2);
  a.w.job = (int2 *)(base + p.job);
  a.w.p2_chunk = (double *)(base + p.p2_chunk);

  hipStream_t st = (hipStream_t)stream;
  int n = 0;
  hipError_t e;
  if (dt == SV_BF16) {
    e = aligned ? launch_all<uint16_t, true>(p, a, st, ev, nev, &n)
                : launch_all<uint16_t, false>(p, a, st, ev, nev, &n);
  } else {
    e = aligned ? launch_all<float, true>(p, a, st, ev, nev, &n)
                : launch_all<float, false>(p, a, st, ev, nev, &n);
  }
  if (nl) *nl = n;
  return e == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t sv_workspace_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype, float temperature,
                          int32_t top_k) {
  if (B < 1 || G < 0 || V < 1 || (dtype != SV_F32 && dtype != SV_BF16)) return 256;
  if (!(temperature >= 0.0f) || !isfinite(temperature)) return 256;
  Plan p;
  if (!make_plan(B, G, V, dtype, temperature, top_k, p)) return 256;
  return p.total;
}

size_t sv_workspace_zero_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                               float temperature, int32_t top_k) {
  if (B < 1 || G < 0 || V < 1 || (dtype != SV_F32 && dtype != SV_BF16)) return 0;
  if (!(temperature >= 0.0f) || !isfinite(temperature)) return 0;
  Plan p;
  if (!make_plan(B, G, V, dtype, temperature, top_k, p)) return 0;
  return p.zero_bytes;
}

sv_status spec_verify(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                      const int32_t *draft_tokens, const float *u_accept, const float *u_sample,
                      int32_t B, int32_t G, int32_t V, float temperature, int32_t top_k,
                      int32_t *accepted_len, int32_t *out_tokens, float *row_stats,
                      void *workspace, size_t workspace_bytes, void *stream) {
  return run(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, B, G, V,
             temperature, top_k, accepted_len, out_tokens, row_stats, workspace, workspace_bytes,
             stream, nullptr, 0, nullptr);
}

sv_status spec_verify_timed(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                            const int32_t *draft_tokens, const float *u_accept,
                            const float *u_sample, int32_t B, int32_t G, int32_t V,
                            float temperature, int32_t top_k, int32_t *accepted_len,
                            int32_t *out_tokens, float *row_stats, void *workspace,
                            size_t workspace_bytes, void *stream, void *const *events,
                            int32_t n_events, int32_t *n_launched) {
  return run(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, B, G, V,
             temperature, top_k, accepted_len, out_tokens, row_stats, workspace, workspace_bytes,
             stream, events, n_events, n_launched);
}

const char *sv_launch_plan(int32_t B, int32_t G, int32_t V, sv_dtype dtype, float temperature,
                           int32_t top_k) {
  (void)B;
  (void)G;
  if (temperature == 0.0f) return kPlanNames[3];
  if (top_k > 0 && top_k < V) return dtype == SV_BF16 ? kPlanNames[0] : kPlanNames[1];
  return kPlanNames[2];
}

const char *sv_status_string(sv_status status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "invalid shape (B < 1, G < 0, V < 1, or too large for one launch)";
    case SV_ERR_DTYPE: return "unsupported logit dtype";
    case SV_ERR_TEMPERATURE: return "temperature must be finite and >= 0";
    case SV_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case SV_ERR_ALIGN: return "logit pointer not aligned to its element size";
    case SV_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"
