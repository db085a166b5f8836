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
  uint2 *tk_state;             // [R] radix-select prefix and remaining rank, or the one-pass
                               //   select's chunk lists (see k_topk_select)
  uint4 *tk_rowp;              // [R] or null: per row after the one-pass select, the kept
                               //   set's normaliser (offset, sum head, tail) and the length
                               //   of its index-ordered list, or KEEP_NONE (see k_topk_merge)
  uint2 *tk_keep;              // [R*cap] the kept (index, logit bits) of each row, in index order
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
  unsigned long long *stamps;  // timeline stamps (the timeline build of the library), or null
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

// The threshold of a selected key: the smallest value whose key carries it.  With a
// 16-bit (bf16) key that value can be a NaN (the bucket of -inf, whose low half is set):
// then every value of the row passes, which is what -inf says.  A NaN threshold is kept
// for a selection that did not complete.
SVD float tau_of_key(uint32_t key) {
  const float t = key2f(key);
  return (t == t) ? t : -INFINITY;
}

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

  // The row's last chunk: wait for the other chunks' histograms (eight chunks' words in
  // flight at once, not one load waited for at a time), then the row total of digit d = tid.
  unsigned tot = 0;
  unsigned polls = 0;
  for (;;) {
    tot = hist[tid];
    bool ok = true;
    for (int cc0 = 0; cc0 < a.C - 1; cc0 += 8) {
      u64 w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        w[k] = (cc0 + k < a.C - 1) ? ld_dev(&hw[(size_t)(cc0 + k) * 128 + (tid >> 1)]) : ((u64)tag << 32);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ok = ok && tw_ok(w[k], tag);
        tot += ((unsigned)w[k] >> ((tid & 1) * 16)) & 0xffffu;
      }
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
    if (last_pass) a.w.row_tau[r] = tau_of_key(prefix);
    else a.w.tk_state[r] = make_uint2(prefix, krem - above);
  }
}

// One-pass top-k threshold, for 0 < k <= TOPK_SELECT_MAX.  Every chunk publishes a
// multiset of its values that holds its k largest (count word, then the keys), and the
// row's last chunk in grid order takes the k-th largest key of their union, which is the
// row's k-th largest: each chunk contributes at most k values to the row's top k, and
// those are among its own k largest (k_topk_merge takes that k-th largest, one workgroup
// per row, in a launch of its own).  A chunk finds a lower bound on its k-th largest
// from its threads' maxima (wave w's ceil(k/4)-th largest maximum, the smallest over the
// four waves: at least 4*ceil(k/4) >= k values lie at or above it) and publishes every
// value at or above that bound.  Should that be more than `cap` values (heavy ties), it
// takes its exact k-th largest tau_c by radix select over its registers and publishes the
// values above tau_c and enough copies of tau_c to make k.  Keys are f2key of the value;
// elements past the row's end are not part of it.  The lists are plain data in the
// workspace's tk_state region (cap + 1 words per chunk: the count, then the keys).
constexpr int TOPK_SELECT_MAX = 256;    // largest k of the one-pass select
constexpr int TOPK_SELECT_MAX_C = 256;   // most chunks per row of the one-pass select
constexpr int TOPK_LDS_KEYS = 1024;      // a chunk's list (at most cap <= 1024 keys), and the
                                         // collector's keys while they fit (else read again)
constexpr unsigned KEEP_NONE = 0xffffffffu;  // a row whose kept set has no list (see k_topk_merge)

// 32-bit words of one chunk's list: count, flags, cap keys, cap 16-bit indices (cap is a
// multiple of 4, so every list stays 8-byte aligned).
SV_HD size_t topk_list_words(int cap) { return (size_t)cap + 2 + (size_t)cap / 2; }

// Inclusive scan of unsigned values over the wave (DPP).
SVD unsigned scan_add_u(unsigned x) {
#define STEP(C, R) x += dpp_u<C, R>(x, 0u);
  SV_SCAN_STEPS(STEP)
#undef STEP
  return x;
}

// Exclusive prefix of v over the workgroup (thread order), and the total.
SVD unsigned block_excl_scan(unsigned v, unsigned *s_w, unsigned &total) {
  const int lane = lane_id(), wid = (int)threadIdx.x / WAVE;
  const unsigned inc = scan_add_u(v);
  if (lane == WAVE - 1) s_w[wid] = inc;
  __syncthreads();
  unsigned before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += (w < wid) ? s_w[w] : 0u;
    tot += s_w[w];
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// The k-th largest (1-based) of a multiset of keys spread over the workgroup's threads,
// by radix select, 8 bits a pass from the top (npass = 2 for bf16 values, whose keys have
// zero low halves; 4 otherwise).  each(f) calls f(key) for every key this thread holds.
// The multiset must hold at least k keys.  Thread d owns histogram bin d.
template <bool AGG = false, typename Each>
SVD uint32_t block_kth_largest(int k, int npass, const Each &each, unsigned *hist, unsigned *sge,
                               unsigned *s_pick) {
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  uint32_t prefix = 0;
  unsigned krem = (unsigned)k;
  for (int pass = 0; pass < npass; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hm = pass ? (0xffffffffu << (shift + 8)) : 0u;
    hist[tid] = 0u;
    if (tid == 0) {
      s_pick[0] = 0u;
      s_pick[1] = 0u;
    }
    __syncthreads();
    // AGG: keys that are close together share their high digits, so when every counted key
    // of the wave falls in one bin, one atomic adds them all (the first pass of a top-k
    // merge would otherwise send hundreds of atomics to one LDS word).
    each([&](uint32_t key) {
      const bool in = (key & hm) == (prefix & hm);
      const unsigned bin = (key >> shift) & 255u;
      if (!AGG) {
        if (in) atomicAdd(&hist[bin], 1u);
        return;
      }
      const unsigned long long cnt = __ballot(in);
      const unsigned b0 = (unsigned)__builtin_amdgcn_readfirstlane((int)bin);
      if (__ballot(in && bin == b0) == cnt) {
        if (cnt && lane == __ffsll((long long)__ballot(true)) - 1) atomicAdd(&hist[b0], (unsigned)__popcll(cnt));
      } else if (in) {
        atomicAdd(&hist[bin], 1u);
      }
    });
    __syncthreads();
    // suffix counts of bin d = tid: the total minus the prefix before d (prefix by a wave
    // scan, the waves' totals through LDS)
    const unsigned h = hist[tid];
    const unsigned incl = scan_add_u(h);
    if (lane == WAVE - 1) sge[wid] = incl;
    __syncthreads();
    unsigned before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      before += (w < wid) ? sge[w] : 0u;
      total += sge[w];
    }
    const unsigned at = total - (before + incl - h);  // values with digit >= d
    const unsigned above = total - (before + incl);   // values with digit > d
    // the largest digit whose suffix count reaches the remaining rank
    if (at >= krem && above < krem) {
      s_pick[0] = (unsigned)tid;
      s_pick[1] = above;
    }
    __syncthreads();
    prefix |= s_pick[0] << shift;
    krem -= s_pick[1];
    __syncthreads();
  }
  return prefix;
}

// The q-th largest (1-based, q <= 64) of the wave's 64 keys, bit by bit from the top:
// at each bit, if at least the remaining rank of the lanes still in the running have it
// set, the answer has it set and the others drop out; otherwise they stay and the rank
// shrinks by their count.  Bits below `low` are taken as zero (bf16 keys).
SVD uint32_t wave_kth_largest(uint32_t v, int q, int low) {
  uint32_t ans = 0;
  unsigned rank = (unsigned)q;
  bool in = true;
  for (int bit = 31; bit >= low; --bit) {
    const bool one = (v >> bit) & 1u;
    const unsigned c = (unsigned)__popcll(__ballot(in && one));
    if (c >= rank) {
      ans |= 1u << bit;
      in = in && one;
    } else {
      rank -= c;
      in = in && !one;
    }
  }
  return ans;
}

// One chunk's list for k_topk_select (whole workgroup), from its raw vectors w: the
// values at or above the lower bound, or, with heavy ties, the exact top k.  Leaves the
// keys in s_keys[0, n) and returns n.  A value enters the list unless it is below the
// bound, so every NaN of the chunk does, with its own key (above +inf's or below -inf's),
// and k_topk_merge sees it.  Elements past the row's end hold -inf: they can enter a list
// only when the bound is -inf, and a -inf can move a k-th largest only when that is -inf
// already; their terms are 0.  A list is incomplete (*incomplete) when it comes from the
// exact select: it then holds the values above the chunk's k-th largest and copies of it.
// A complete list also leaves each key's element index within the chunk in s_idx.
template <typename T>
SVD unsigned topk_chunk_list(u32x4 (&w)[VPT], int k, int cap, unsigned *s_keys, uint16_t *s_idx,
                             bool *incomplete, unsigned *s_hist, unsigned *s_ge, unsigned *s_wv,
                             unsigned *s_pick) {
  constexpr int VEC = Fmt<T>::VEC;
  constexpr int NPASS = (sizeof(T) == 2) ? 2 : 4;
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  // bf16 keys keep only their upper half: a negative value's key has its low half set,
  // and the radix select resolves 16 bits, so every comparison happens at that width.
  constexpr uint32_t KMASK = (sizeof(T) == 2) ? 0xffff0000u : 0xffffffffu;
  auto key = [&](int kk, int e) -> uint32_t {
    float f[VEC];
    Fmt<T>::unpack(w[kk], f);
    return f2key(f[e]) & KMASK;
  };
  // Between passes over the chunk the raw vectors are marked as changed, so each pass
  // unpacks its values again instead of keeping all of them live in registers.
  auto fresh = [&]() {
#pragma unroll
    for (int kk = 0; kk < VPT; ++kk) asm volatile("" : "+v"(w[kk]));
  };
  // lower bound: per wave the ceil(k/4)-th largest thread maximum, the smallest over the
  // waves.  Comparisons against it
  // are made on values: x >= key2f(lb) exactly when key(x) >= lb, for every value that is
  // not a NaN (a row with a NaN is reported as an error whatever its threshold).
  float tm = -INFINITY;
#pragma unroll
  for (int kk = 0; kk < VPT; ++kk) {
    float f[VEC];
    Fmt<T>::unpack(w[kk], f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) tm = fmaxf(tm, f[e]);
  }
  const uint32_t v = f2key(tm) & KMASK;
  const uint32_t wv = wave_kth_largest(v, (k + NW - 1) / NW, sizeof(T) == 2 ? 16 : 0);
  if (lane == 0) s_wv[wid] = wv;
  if (tid == 0) s_pick[0] = 0u;  // the candidate count
  __syncthreads();
  uint32_t lb = s_wv[0];
#pragma unroll
  for (int w2 = 1; w2 < NW; ++w2) lb = (s_wv[w2] < lb) ? s_wv[w2] : lb;
  float lbf = key2f(lb);
  lbf = (lbf == lbf) ? lbf : -INFINITY;  // the -inf bucket of a bf16 key: every value

  // candidates: every value not below lbf, into LDS in any order (a multiset).  A branch-free
  // count, one LDS atomic per wave to reserve the wave's range, then the writes.
  fresh();
  unsigned cnt = 0;
#pragma unroll
  for (int kk = 0; kk < VPT; ++kk) {
    float f[VEC];
    Fmt<T>::unpack(w[kk], f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) cnt += (f[e] < lbf) ? 0u : 1u;
  }
  const unsigned incl = scan_add_u(cnt);
  unsigned wbase = 0;
  if (lane == WAVE - 1 && incl > 0u) wbase = atomicAdd(&s_pick[0], incl);
  unsigned pos = (unsigned)__builtin_amdgcn_readlane((int)wbase, WAVE - 1) + incl - cnt;
  if (cnt > 0u) {
    fresh();
#pragma unroll
    for (int kk = 0; kk < VPT; ++kk) {
      float f[VEC];
      Fmt<T>::unpack(w[kk], f);
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (!(f[e] < lbf)) {
          if (pos < (unsigned)cap) {
            s_keys[pos] = f2key(f[e]) & KMASK;
            s_idx[pos] = (uint16_t)((kk * NT + tid) * VEC + e);
          }
          ++pos;
        }
    }
  }
  __syncthreads();
  const unsigned n = s_pick[0];
  __syncthreads();  // every thread holds n before s_pick is reused
  unsigned own_n;
  *incomplete = n > (unsigned)cap;
  if (n <= (unsigned)cap) {
    own_n = n;
  } else {  // heavy ties: the exact k-th largest of the chunk, then keys above it
    auto each = [&](auto fn) {
#pragma unroll
      for (int kk = 0; kk < VPT; ++kk)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          fn(key(kk, e));
    };
    fresh();
    const uint32_t tc = block_kth_largest(k, NPASS, each, s_hist, s_ge, s_pick);
    fresh();
    if (tid == 0) s_pick[0] = 0u;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < VPT; ++kk)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const uint32_t kv = key(kk, e);
        if (kv > tc) {
          const unsigned i = atomicAdd(&s_pick[0], 1u);
          if (i < (unsigned)k) s_keys[i] = kv;  // fewer than k lie above the k-th largest
        }
      }
    __syncthreads();
    const unsigned na = s_pick[0] < (unsigned)k ? s_pick[0] : (unsigned)k;
    for (unsigned i = na + tid; i < (unsigned)k; i += NT) s_keys[i] = tc;
    __syncthreads();
    own_n = (unsigned)k;
  }
  return own_n;
}

// Seven resident waves per SIMD (at most 72 registers; the rare exact-select path spills a
// little): the pass streams faster with more workgroups in flight than with fewer and no spill.
template <typename T, bool ALIGNED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(7))) void k_topk_select(const Args a, int cap) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ unsigned s_hist[256], s_ge[256], s_wv[NW], s_pick[2];
  __shared__ unsigned s_keys[TOPK_LDS_KEYS];
  __shared__ uint16_t s_idx[TOPK_LDS_KEYS];
  const int tid = threadIdx.x;
  int phase, xi;
  if (!lane_item((int)(a.B * a.rps), a.C, 0, phase, xi)) return;  // units: rows
  const int r = xi / a.C, c = xi - r * a.C;
  const int b = r / a.rps, jr = r - b * a.rps;
  const int k = a.top_k;

  // The chunk stays in registers as raw 16-byte vectors (8 bf16 or 4 f32 values each);
  // elements past the row's end are -inf.
  u32x4 w[VPT];
  {
    const T *row = seq_row<T>(a, b, jr);
    if (ALIGNED) {
      const u32x4 *rv = reinterpret_cast<const u32x4 *>(row);
#pragma unroll
      for (int kk = 0; kk < VPT; ++kk) {
        const int vi = c * CHUNK_VECS + kk * NT + tid;
        w[kk] = __builtin_nontemporal_load(rv + (vi < a.nvec ? vi : a.nvec - 1));
      }
      if ((c + 1) * CHUNK_VECS > a.nvec) {  // the row's tail: vectors past its end
        constexpr unsigned NEG_INF = (sizeof(T) == 2) ? 0xff80ff80u : 0xff800000u;
#pragma unroll
        for (int kk = 0; kk < VPT; ++kk)
          if (c * CHUNK_VECS + kk * NT + tid >= a.nvec) w[kk] = u32x4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
      }
    } else {  // a row off the 16-byte grid: each vector built from the two blocks that hold it
      const unsigned off = row_off16(row);
      u32x4 lo[VPT], hi[VPT];
#pragma unroll
      for (int kk = 0; kk < VPT; ++kk) {
        const int vi = c * CHUNK_VECS + kk * NT + tid;
        load_pair<T, true>(row, row + a.V, off, vi < a.nvec ? vi : a.nvec - 1, lo[kk], hi[kk]);
      }
#pragma unroll
      for (int kk = 0; kk < VPT; ++kk) w[kk] = funnel16(lo[kk], hi[kk], off);
      if ((long)(c + 1) * CHUNK_VECS * VEC > a.V) {  // the row's tail: elements past its end are -inf
#pragma unroll
        for (int kk = 0; kk < VPT; ++kk) {
          const long i0 = elem_index<T>(c, kk, tid, 0);
          unsigned d[4] = {w[kk].x, w[kk].y, w[kk].z, w[kk].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (VEC == 8) {
              if (i0 + 2 * j >= a.V) d[j] = (d[j] & 0xffff0000u) | 0xff80u;
              if (i0 + 2 * j + 1 >= a.V) d[j] = (d[j] & 0x0000ffffu) | 0xff800000u;
            } else if (i0 + j >= a.V) {
              d[j] = 0xff800000u;
            }
          }
          w[kk] = u32x4{d[0], d[1], d[2], d[3]};
        }
      }
    }
  }
  bool incomplete;
  const unsigned own_n = topk_chunk_list<T>(w, k, cap, s_keys, s_idx, &incomplete, s_hist, s_ge, s_wv, s_pick);
  // The list goes to the workspace as plain data for k_topk_merge: the count, the flags
  // (2: the list is incomplete), the keys, then (complete lists) the 16-bit element
  // indices within the chunk.
  uint32_t *lw = reinterpret_cast<uint32_t *>(a.w.tk_state) + ((size_t)r * a.C + c) * topk_list_words(cap);
  for (unsigned i = tid; i < own_n; i += NT) lw[2 + i] = s_keys[i];
  if (!incomplete) {
    uint16_t *li = reinterpret_cast<uint16_t *>(lw + 2 + cap);
    for (unsigned i = tid; i < own_n; i += NT) li[i] = s_idx[i];
  }
  if (tid == 0) {
    lw[0] = own_n;
    lw[1] = incomplete ? 2u : 0u;
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

// ---------------------------------------------------------------- top-k row merge

// The row threshold of the one-pass select (one workgroup per row, after k_topk_select):
// tau = the k-th largest key of the union of the row's chunk lists, staged in LDS when
// they fit (else read again by each radix pass).  Every value at or above tau lies in
// those lists: a chunk lists every value not below its own bound, and k of its values
// lie at or above that bound, so tau is not below it.
//
// With tk_rowp (the verification after the threshold) the kept set of the row, {z >= tau,
// z > -inf}, is summarised too: the offset off = m*k2 of its largest value m and
// S = sum 2^(z*k2 - off), so the row's log2-partition is off + log2(S) ("推测解码：接受
// 规则、状态与收益边界", section "两模型精确采样": each distribution is renormalised over
// what it keeps).  When every chunk's list is complete and at most cap values are kept,
// the kept (index, logit) pairs go to tk_keep in index order and S is summed in that
// order; otherwise (heavy ties) the row is streamed again, chunk by chunk, and the row
// has no list (KEEP_NONE).  S is NaN when the row holds a NaN or keeps a +inf; with
// nothing finite kept, off = -inf and S = 0.
template <typename T, bool ALIGNED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(7))) void k_topk_merge(const Args a, int cap) {
  constexpr int NPASS = (sizeof(T) == 2) ? 2 : 4;
  constexpr long CE = (long)CHUNK_VECS * Fmt<T>::VEC;  // values per chunk
  __shared__ unsigned s_hist[256], s_ge[256], s_w[NW], s_pick[2];
  __shared__ unsigned s_keys[TOPK_LDS_KEYS], s_gidx[TOPK_LDS_KEYS];
  __shared__ unsigned s_coff[TOPK_SELECT_MAX_C + 1];
  __shared__ unsigned s_incomplete, s_nk;
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  const long long r = blockIdx.x;
  if (r >= (long long)a.B * a.rps) return;
  const int k = a.top_k, C = a.C;
  const size_t W = topk_list_words(cap);
  const uint32_t *rl = reinterpret_cast<const uint32_t *>(a.w.tk_state) + (size_t)r * C * W;
  if (tid == 0) {
    s_incomplete = 0u;
    s_nk = 0u;
  }
  unsigned total = 0;
  for (int c0 = 0; c0 < C; c0 += NT) {
    const int cc = c0 + tid;
    unsigned nc = (cc < C) ? rl[(size_t)cc * W] : 0u;
    nc = (nc <= (unsigned)cap) ? nc : 0u;  // never trust a count beyond the chunk's words
    if (cc < C && (rl[(size_t)cc * W + 1] & 2u)) s_incomplete = 1u;
    unsigned tot;
    const unsigned before = block_excl_scan(nc, s_w, tot);
    if (cc < C) s_coff[cc] = total + before;
    total += tot;
  }
  if (tid == 0) s_coff[C] = total;
  __syncthreads();
  const bool complete = s_incomplete == 0u;
  // candidate g: its chunk is the last one whose first candidate is <= g; its row index
  // (complete lists only) is the chunk's first index plus the listed offset
  auto cand = [&](unsigned g, unsigned &gi) -> uint32_t {
    int lo = 0, hi = C - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_coff[mid] <= g) lo = mid;
      else hi = mid - 1;
    }
    const uint32_t *cl = rl + (size_t)lo * W;
    const unsigned i = g - s_coff[lo];
    gi = complete ? (unsigned)(lo * CE) + reinterpret_cast<const uint16_t *>(cl + 2 + cap)[i] : 0u;
    return cl[2 + i];
  };
  const bool in_lds = total <= (unsigned)TOPK_LDS_KEYS;
  if (in_lds)
    for (unsigned g = tid; g < total; g += NT) s_keys[g] = cand(g, s_gidx[g]);
  __syncthreads();
  uint4 *rowp = a.w.tk_rowp;
  if (total < (unsigned)k) {  // cannot happen with a complete select pass
    if (tid == 0) {
      a.w.row_tau[r] = NAN;
      if (rowp) rowp[r] = make_uint4(__float_as_uint(NAN), __float_as_uint(NAN), 0u, KEEP_NONE);
    }
    return;
  }
  auto each = [&](auto f) {
    unsigned gi;
    for (unsigned g = tid; g < total; g += NT) f(in_lds ? s_keys[g] : cand(g, gi));
  };
  const uint32_t tk = block_kth_largest<true>(k, NPASS, each, s_hist, s_ge, s_pick);
  const float tau = tau_of_key(tk);
  if (tid == 0) a.w.row_tau[r] = tau;
  if (!rowp) return;

  // The kept values among the candidates, compacted (the first cap of them) in any order:
  // one LDS atomic per wave reserves its range.
  auto val = [&](uint32_t key) -> float {  // a bf16 key keeps its upper half only
    if (sizeof(T) == 2 && !(key & 0x80000000u)) key |= 0xffffu;
    return key2f(key);
  };
  // keys above +inf's or below -inf's are NaNs (for bf16 as masked keys)
  constexpr uint32_t KPINF = 0xff800000u;
  constexpr uint32_t KNINF = (sizeof(T) == 2) ? 0x007f0000u : 0x007fffffu;
  __shared__ float s_kz[TOPK_LDS_KEYS];
  __shared__ unsigned s_kidx[TOPK_LDS_KEYS];
  __shared__ float s_rm[NW];
  __shared__ unsigned s_rn[NW];
  unsigned nanl = 0;
  float m = -INFINITY;
  for (unsigned g = tid; g < total; g += NT) {  // lane 0 is active whenever any lane is
    unsigned gi;
    uint32_t key;
    if (in_lds) {
      key = s_keys[g];
      gi = s_gidx[g];
    } else {
      key = cand(g, gi);
    }
    const bool isnan_k = key > KPINF || key < KNINF;
    nanl |= isnan_k ? 1u : 0u;
    const float v = val(key);
    const bool kept = !isnan_k && key >= tk && v > -INFINITY;
    if (kept) m = fmaxf(m, v);
    const unsigned long long bal = __ballot(kept);
    unsigned base = 0;
    if (lane == 0 && bal) base = atomicAdd(&s_nk, (unsigned)__popcll(bal));
    const unsigned pos = (unsigned)__builtin_amdgcn_readlane((int)base, 0) +
                         (unsigned)__popcll(bal & ((1ull << lane) - 1ull));
    if (kept && pos < (unsigned)cap) {
      s_kidx[pos] = gi;
      s_kz[pos] = v;
    }
  }
  m = wave_max(m);
  nanl = wave_or(nanl);
  if (lane == 0) {
    s_rm[wid] = m;
    s_rn[wid] = nanl;
  }
  __syncthreads();
  m = fmaxf(fmaxf(s_rm[0], s_rm[1]), fmaxf(s_rm[2], s_rm[3]));
  const bool has_nan = (s_rn[0] | s_rn[1] | s_rn[2] | s_rn[3]) != 0u;
  const unsigned nkeep = s_nk;

  const float k2 = a.k2;
  float off;
  double S;
  unsigned count;
  if (complete && nkeep <= (unsigned)cap) {
    // Index order: an entry's rank is the number of kept entries with a smaller index
    // (indices are distinct).  The sorted logits reuse s_keys.
    float *s_sz = reinterpret_cast<float *>(s_keys);
    uint2 *kl = a.w.tk_keep + (size_t)r * cap;
    for (unsigned e = tid; e < nkeep; e += NT) {
      const unsigned ie = s_kidx[e];
      unsigned rank = 0;
      for (unsigned f = 0; f < nkeep; ++f) rank += (s_kidx[f] < ie) ? 1u : 0u;
      kl[rank] = make_uint2(ie, __float_as_uint(s_kz[e]));
      s_sz[rank] = s_kz[e];
    }
    __syncthreads();
    if (wid != 0) return;  // one wave sums, lane l taking entries l, l + 64, ... in order
    off = (m > -INFINITY) ? m * k2 : -INFINITY;
    double acc = 0.0;
    if (m > -INFINITY)
      for (unsigned e = lane; e < nkeep; e += WAVE) acc += (double)fast_exp2(fmaf(s_sz[e], k2, -off));
    S = wave_sum(acc);
    if (has_nan || m == INFINITY) S = NAN;
    count = nkeep;
  } else {
    // Heavy ties: the kept set's normaliser from the row itself, in two passes of one
    // vector per thread at a time (the largest kept value, then the sum with its offset;
    // each thread's values in order, the threads by a fixed tree).
    const int b = (int)(r / a.rps), jr = (int)(r - (long long)b * a.rps);
    const T *row = seq_row<T>(a, b, jr);
    constexpr int VEC = Fmt<T>::VEC;
    float mr = -INFINITY;
    unsigned nan = 0;
    for (int c = 0; c < C; ++c)
      for (int kk = 0; kk < VPT; ++kk) {
        float x[1][VEC];
        load_vectors<T, ALIGNED, false, 1>(row, a.V, a.nvec, c, kk, tid, x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          nan |= (x[0][e] != x[0][e]) ? 1u : 0u;
          if (!(x[0][e] < tau)) mr = fmaxf(mr, x[0][e]);
        }
      }
    mr = wave_max(mr);
    nan = wave_or(nan);
    __syncthreads();  // the s_rm, s_rn values above have been read by every wave
    if (lane == 0) {
      s_rm[wid] = mr;
      s_rn[wid] = nan;
    }
    __syncthreads();
    mr = fmaxf(fmaxf(s_rm[0], s_rm[1]), fmaxf(s_rm[2], s_rm[3]));
    const bool row_nan = (s_rn[0] | s_rn[1] | s_rn[2] | s_rn[3]) != 0u;
    off = (mr > -INFINITY) ? mr * k2 : -INFINITY;
    double acc = 0.0;
    if (mr > -INFINITY)
      for (int c = 0; c < C; ++c)
        for (int kk = 0; kk < VPT; ++kk) {
          float x[1][VEC];
          load_vectors<T, ALIGNED, false, 1>(row, a.V, a.nvec, c, kk, tid, x);
          float t = 0.0f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) t += fast_exp2(fmaf((x[0][e] < tau) ? -INFINITY : x[0][e], k2, -off));
          acc += (double)t;
        }
    acc = wave_sum(acc);
    __shared__ double s_rs[NW];
    if (lane == 0) s_rs[wid] = acc;
    __syncthreads();
    S = (s_rs[0] + s_rs[1]) + (s_rs[2] + s_rs[3]);
    if (row_nan || mr == INFINITY) S = NAN;
    else if (!(mr > -INFINITY)) S = 0.0;  // nothing finite kept
    count = KEEP_NONE;
  }
  if (tid == 0) rowp[r] = make_uint4(__float_as_uint(off), __float_as_uint(d_head(S)), __float_as_uint(d_tail(S)), count);
}

}  // namespace sv

// ---------------------------------------------------------------- host helpers

namespace sv_host {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Every kernel launch of the library takes its own tag from one process-wide counter
// (never 0: a clean workspace holds zeros), so a word left in a shared workspace by any
// earlier launch of any entry point can never pass for the current one's.
unsigned next_tag();
// n consecutive tags (none of them 0) for one launch; returns the first.
unsigned next_tag_block(unsigned n);

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

// The top-k threshold: one k_topk_select pass when k and the row's chunk count allow it,
// else the radix digit passes (2 for bf16, 4 for f32).  tw_hist holds topk_words(...)
// tagged words in either case.
inline bool topk_one_pass(int top_k, int C) { return top_k <= sv::TOPK_SELECT_MAX && C <= sv::TOPK_SELECT_MAX_C; }
inline int topk_cap(int top_k) {
  const int c = 4 * top_k;
  return c < 128 ? 128 : (c > 1024 ? 1024 : c);
}
// Tagged words of the digit passes' histograms (none for the one-pass select).
inline size_t topk_words(long long R, int C, int top_k) {
  return topk_one_pass(top_k, C) ? 0 : (size_t)R * (size_t)C * 128;
}
// Bytes of the plain tk_state region: the chunk lists of the one-pass select, or the
// digit passes' (prefix, rank) per row.  With keep (the verification), each row's kept-set
// summary (16 bytes) and its kept list (cap entries of 8 bytes) follow the lists.
inline size_t topk_list_bytes(long long R, int C, int top_k) {
  return (size_t)R * (size_t)C * sv::topk_list_words(topk_cap(top_k)) * 4;
}
// Offsets (from the region's start, 256-byte aligned) of the kept-set summaries and lists.
inline size_t topk_rowp_offset(long long R, int C, int top_k) { return align256(topk_list_bytes(R, C, top_k)); }
inline size_t topk_keep_offset(long long R, int C, int top_k) {
  return topk_rowp_offset(R, C, top_k) + align256((size_t)R * 16);
}
inline size_t topk_state_bytes(long long R, int C, int top_k, bool keep = false) {
  if (!topk_one_pass(top_k, C)) return (size_t)R * 8;
  if (!keep) return topk_list_bytes(R, C, top_k);
  return topk_keep_offset(R, C, top_k) + (size_t)R * (size_t)topk_cap(top_k) * 8;
}
// Chunks per row (as the kernels cut rows) for a row of V values of esz bytes.
inline int row_chunks(int V, int esz) {
  const long long nvec = ((long long)V * esz + 15) / 16;
  return (int)((nvec + sv::CHUNK_VECS - 1) / sv::CHUNK_VECS);
}
template <typename T, bool AL>
void launch_topk(Launcher &L, sv::Args aa, unsigned grid, int C) {
  if (topk_one_pass(aa.top_k, C)) {
    aa.tag = next_tag();
    int cap = topk_cap(aa.top_k);
    void *args[] = {&aa, &cap};
    L.go((const void *)&sv::k_topk_select<T, AL>, grid, args);
    aa.tag = next_tag();
    L.go((const void *)&sv::k_topk_merge<T, AL>, (unsigned)((long long)aa.B * aa.rps), args);
    return;
  }
  const int passes = (sizeof(T) == 2) ? 2 : 4;
  for (int pass = 0; pass < passes; ++pass) {
    int ps = pass, lp = (pass == passes - 1) ? 1 : 0;
    aa.tag = next_tag();
    void *args[] = {&aa, &ps, &lp};
    const void *fn = (pass == 0) ? (const void *)&sv::k_topk_digit<T, AL, 16> : (const void *)&sv::k_topk_digit<T, AL, 1>;
    L.go(fn, grid, args);
  }
}

}  // namespace sv_host
