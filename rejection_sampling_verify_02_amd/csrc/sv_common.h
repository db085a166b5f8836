// sv_common.h -- what the kernels of the library share beyond device helpers: the
// workspace carve-up and kernel arguments, the row numbering, the top-k radix select
// that runs before the sampling kernels, and the host's launch helpers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_device.h"

namespace sv {

// ---------------------------------------------------------------- arguments

struct Work {                  // carved from the caller's workspace
  // tagged words (see tw_put)
  u64 *tw_part;                // [R*C*3] per chunk: sampling offset m_c*k2 and sum of
                               //   2^(z*k2 - off) (head, tail); greedy best value, index, flags
  u64 *tw_job;                 // [B*JW] the acceptance scan's record for the draw
  u64 *tw_seg;                 // [B*C*SEGS*2] residual mass per 64-vector segment (head, tail)
  u64 *tw_gseg;                // [B*C*SEGS*2] the bonus row's mass per segment (head, tail)
  u64 *tw_hist;                // [R*C*128] top-k digit histogram per chunk (16-bit counts)
  u64 *tw_ov;                  // [P*C*4] overlap: per pair and chunk, sum min(p, q) and
                               //   sum (p - min(p, q)) (head, tail each)
  // plain, handed from one kernel to the next
  float *row_tau;              // [R] top-k threshold (raw logit)
  uint2 *tk_state;             // [R] radix-select prefix and remaining rank
};

struct Args {
  const void *target, *draft;
  const int32_t *tokens;
  const float *u_accept, *u_sample;
  int B, G, V, C, nvec, rps;   // rps: rows per sequence (2G+1 sampling, G+1 greedy, 2G overlap)
  int ntr;                     // target rows among a sequence's rows (G+1 verification, G overlap)
  int tgt_rows;                // target rows per sequence in memory (G+1, or G for overlap pairs)
  float k2;                    // log2(e) / T, the one rounding of the temperature used everywhere
  int top_k;
  int32_t *accepted_len, *out_tokens;
  float *row_stats;
  double *beta, *tv;           // overlap outputs [B*G]
  int32_t *pair_status;        // overlap status [B*G]
  int lag;                     // overlap: pairs between a pair's two phases in an XCD lane
  unsigned tag;                // this call's tag (never 0): marks the words it publishes
  unsigned spin_limit;         // polls a waiting wave makes before giving up
  Work w;
};

// Row j of sequence b: rows 0..ntr-1 are target rows 0..ntr-1 (a sequence holds tgt_rows
// of them in memory), rows ntr..ntr+G-1 draft rows 0..G-1.  Verification numbers G+1
// target rows then G draft rows; the overlap G target rows then G draft rows.
template <typename T>
SVD const T *seq_row(const Args &a, int b, int j) {
  if (j < a.ntr) return static_cast<const T *>(a.target) + ((size_t)b * a.tgt_rows + j) * (size_t)a.V;
  return static_cast<const T *>(a.draft) + ((size_t)b * a.G + (j - a.ntr)) * (size_t)a.V;
}

// ---------------------------------------------------------------- top-k threshold

// One radix-select digit (bits [shift, shift+8) of the key) for every row.  The prefix
// of higher digits and the remaining rank come from the previous pass.  The threshold
// kept in row_tau is the smallest value whose key has the final prefix, so the kept set
// {z >= tau} is exactly the values >= the k-th largest, ties included.  Each chunk
// publishes its digit histogram as 128 tagged words (two 16-bit counts each; a chunk
// holds at most 16384 values); the row's last chunk in grid order collects them.
// The first pass counts its histogram in HREP copies, lane l adding into copy l % HREP:
// logits crowd into a few leading digits (the exponent), and one copy would make a whole
// wave's LDS atomics land on the same address one after another.  Later passes count
// only the values that carry the prefix found so far, few per chunk: one copy.
template <typename T, bool ALIGNED, int HREP>
__global__ __launch_bounds__(NT) void k_topk_digit(const Args a, int pass, int last_pass) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ unsigned hist[256 * HREP];
  __shared__ unsigned s_ge[256];
  __shared__ int s_alive;
  const int tid = threadIdx.x;
  int phase, xi;
  if (!lane_item((int)(a.B * a.rps), a.C, 0, phase, xi)) return;  // units: rows
  const int r = xi / a.C, c = xi - r * a.C;
  const int b = r / a.rps, jr = r - b * a.rps;
  const int shift = 24 - 8 * pass;
  const uint2 st = (pass == 0) ? make_uint2(0u, (unsigned)a.top_k) : a.w.tk_state[r];
  const uint32_t hi_mask = (pass == 0) ? 0u : (0xffffffffu << (shift + 8));
  const unsigned tag = a.tag;

  for (int i = tid; i < 256 * HREP; i += NT) hist[i] = 0u;
  __syncthreads();
  float x[VPT][VEC];
  load_chunk<T, ALIGNED, true>(seq_row<T>(a, b, jr), a.V, a.nvec, c, tid, x);
  const unsigned rep = (unsigned)tid & (HREP - 1);
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (elem_index<T>(c, k, tid, e) < a.V) {
        const uint32_t key = f2key(x[k][e]);
        if ((key & hi_mask) == (st.x & hi_mask)) atomicAdd(&hist[((key >> shift) & 255u) * HREP + rep], 1u);
      }
    }
  __syncthreads();
  if (HREP > 1) {  // fold the copies: thread d owns digit d
    unsigned h = 0;
#pragma unroll
    for (int r2 = 0; r2 < HREP; ++r2) h += hist[tid * HREP + ((r2 + tid) & (HREP - 1))];
    __syncthreads();
    hist[tid] = h;
    __syncthreads();
  }
  u64 *hw = a.w.tw_hist + (size_t)r * a.C * 128;
  if (c != a.C - 1) {
    if (tid < 128) tw_put(&hw[(size_t)c * 128 + tid], tag, hist[2 * tid] | (hist[2 * tid + 1] << 16));
    return;
  }

  // The row's last chunk: wait for the other chunks' histograms (every load in flight
  // at once), then the row total of digit d = tid.
  unsigned tot = 0;
  unsigned polls = 0;
  for (;;) {
    tot = hist[tid];
    bool ok = true;
    for (int cc = 0; cc < a.C - 1; ++cc) {
      const u64 w = ld_dev(&hw[(size_t)cc * 128 + (tid >> 1)]);
      ok = ok && tw_ok(w, tag);
      tot += ((unsigned)w >> ((tid & 1) * 16)) & 0xffffu;
    }
    if (__syncthreads_and(ok ? 1 : 0)) break;
    if (++polls >= a.spin_limit) break;
    __builtin_amdgcn_s_sleep(2);
  }
  // A row whose collector gave up (here or in an earlier pass) carries a marker to the
  // end: tk_state (~0, ~0), then a NaN threshold, which the scan reports as an error.
  const bool dead = st.x == 0xffffffffu && st.y == 0xffffffffu;
  if (tid == 0) s_alive = polls < a.spin_limit && !dead;
  s_ge[tid] = tot;
  __syncthreads();
  if (!s_alive) {
    if (tid == 0) {
      if (last_pass) a.w.row_tau[r] = NAN;
      else a.w.tk_state[r] = make_uint2(0xffffffffu, 0xffffffffu);
    }
    return;
  }
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

// ---------------------------------------------------------------- per-chunk normaliser

// The normaliser partial of chunk c of one row (whole workgroup): m = block max of the
// kept z (top-k: z >= tau), off = m*k2 rounded once, and S = the sum of 2^(fma(z, k2,
// -off)) (a vector's elements as a tree, vectors in order, waves as a fixed tree).  A
// chunk with nothing finite gives off = -inf and S = 0, or NaN if it holds a NaN.  The
// results are the same in every thread.
template <typename T, bool ALIGNED, bool TOPK, bool STREAM>
SVD void chunk_norm(const T *row, int V, int nvec, int c, float tau, float k2, float &off,
                    double &S) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ float s_m[NW];
  __shared__ double s_s[NW];
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  float x[VPT][VEC];
  load_chunk<T, ALIGNED, STREAM>(row, V, nvec, c, tid, x);
  if (TOPK) {
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
  m = wave_max(m);
  if (lane == 0) s_m[wid] = m;
  __syncthreads();
  m = s_m[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, s_m[w]);
  double s;
  if (m > -INFINITY) {
    off = m * k2;
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float t[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) t[e] = fast_exp2(fmaf(x[k][e], k2, -off));
#pragma unroll
      for (int h = VEC / 2; h > 0; h >>= 1)
#pragma unroll
        for (int e = 0; e < h; ++e) t[e] += t[e + h];
      acc += t[0];
    }
    s = (double)acc;
  } else {
    off = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) nan |= (x[k][e] != x[k][e]);
    s = nan ? (double)NAN : 0.0;
  }
  s = wave_sum(s);
  if (lane == 0) s_s[wid] = s;
  __syncthreads();
  S = (s_s[0] + s_s[1]) + (s_s[2] + s_s[3]);
}

}  // namespace sv

// ---------------------------------------------------------------- host helpers

namespace sv_host {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Every kernel launch of the library takes its own tag from one process-wide counter
// (never 0: a clean workspace holds zeros), so a word left in a shared workspace by any
// earlier launch of any entry point can never pass for the current one's.
unsigned next_tag();

// Launches kernels in order on one stream.  With events, kernel i is launched with
// (events[2i], events[2i+1]) as its start and stop events, which time the dispatch
// itself without extra packets on the stream.
struct Launcher {
  hipStream_t st;
  void *const *ev;
  int nev;
  int n = 0;
  hipError_t e = hipSuccess;
  int block = sv::NT;  // threads per workgroup of the next launches
  void go(const void *fn, unsigned grid, void **args) {
    if (e != hipSuccess) return;
    const dim3 blk(block);
    if (ev && 2 * n + 1 < nev)
      e = hipExtLaunchKernel(fn, dim3(grid), blk, args, 0, st, (hipEvent_t)ev[2 * n],
                             (hipEvent_t)ev[2 * n + 1], 0);
    else
      e = hipLaunchKernel(fn, dim3(grid), blk, args, 0, st);
    if (e == hipSuccess) ++n;
  }
};

}  // namespace sv_host
