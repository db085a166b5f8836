// spec_verify.hip -- batched speculative-sampling verification for MI355X (gfx950).
//
// What is computed ("Speculative Decoding 的朴素思想", sections "一次 sampling 怎么执行",
// "Correction 为什么用正残差", "从单个 token 接到一段 draft"; "推测解码：接受规则、状态与
// 收益边界", section "两模型精确采样"; greedy: tannlonggtaoo note, "Greedy Sampling"):
// for each sequence, the drafted tokens are tested in order against min(1, p/q); the
// first rejection draws a correction from norm([p - q]_+), an all-accept round draws a
// bonus from the target's next distribution, both by inverse CDF.
//
// How it is laid out on the GPU.  Every logit row is cut into chunks of CHUNK_VECS
// 16-byte vectors (32 KiB: 16384 bf16 / 8192 f32 values); one 256-thread workgroup
// (four wave64s) streams one chunk with non-temporal 128-bit loads, all issued before
// any is used.  The work is HBM-bound streaming with one exp per element, so there is
// no MFMA: the goals are memory-level parallelism, few VALU operations per element, and
// no second pass over the bulk of the data.
//
//   k_topk_digit  (only with top-k)  radix select of the k-th largest raw logit per row,
//                 one 8-bit digit per launch (2 launches for bf16, 4 for f32), LDS
//                 histograms per chunk, the last chunk of a row picks the digit.
//   k_verify      one grid per call.  First-pass items, per chunk of every row: block
//                 max m_c and sum of 2^(z*log2(e)/T - m_c*log2(e)/T), one v_exp_f32 per
//                 element, published as a partial.  The last item of a sequence combines
//                 its rows' partials, runs the acceptance scan (first rejection; token /
//                 row / uniform / support checks) and leaves the sequence's job.  Draw
//                 items follow: for a rejection at j, the masses of [p_j - q_j]_+ per
//                 64-vector segment of both rows at j; the last draw item picks segment,
//                 lane and element where the cumulative mass passes u*Z.  For a bonus, the
//                 chunk of p_G picked from the partials re-reads itself.  With no drafts
//                 (G = 0: the batched sampler) no draw items are launched: the row's chunks
//                 publish masses per segment and the finisher draws, re-reading one segment.
//   k_argmax      greedy (T == 0): per-chunk argmax, row combine and scan, one launch.
//
// Workgroups hand results to one another as tagged 64-bit words (the call's tag in the
// upper half), written and read with device-scope atomic stores and loads; a reader
// polls until the words it needs carry the tag.  Waits only go to items earlier in the
// same XCD lane (see lane_item), so no grid can stall.  All reductions use fixed trees or
// fixed orders, so results are bitwise reproducible run to run.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "spec_verify.h"
#include "sv_common.h"
#include "sv_draw.h"

namespace sv {

// Timeline stamps, in the library built for timelines (-DSV_TIMELINE) only: the first lane
// of a wave stores the wall clock (wall_clock64) at fixed points of each sequence's path
// into a caller's buffer, word 0 when the grid starts and, for sequence b, words TL_SEQ(b)
// + TL_*: first-pass item (row jr, chunk c) at jr*C + c when that is below 256, the
// finisher's entry, its last partial in and its record out, draw item i (c*4 + sub) at
// TL_DRAW_SEEN + i when it has the record and TL_DRAW_PUB + i when its masses are out (i <
// 96), the combiner with every mass in and the sequence's token written (with no drafts:
// the finisher with the picked chunk's segment masses in, and the token written).  In the
// library's own build the stamps compile to nothing.
#ifdef SV_TIMELINE
#define SV_TL(a, idx) do { if ((a).stamps && lane_id() == 0) st_dev(&(a).stamps[(idx)], (unsigned long long)wall_clock64()); } while (0)
#else
#define SV_TL(a, idx) do { } while (0)
#endif
constexpr size_t TL_STRIDE = 512;  // words a sequence
SVD size_t TL_SEQ(int b) { return 8 + (size_t)b * TL_STRIDE; }
enum : int { TL_FIN_IN = 256, TL_FIN_PARTS = 257, TL_FIN_REC = 258, TL_DRAW_SEEN = 260, TL_DRAW_PUB = 360,
             TL_COMB_IN = 460, TL_DONE = 461, TL_DRAW_MAX = 96 };

constexpr int NSUB = 4;                // second-pass workgroups per chunk of a rejected pair
constexpr int KSUB = VPT / NSUB;       // vectors per thread of each of them
enum : int { JOB_NONE = 0, JOB_REJECT = 1, JOB_BONUS = 2 };  // NONE: nothing to draw (a row error, or G = 0)

// The acceptance scan's record for the draw of one sequence: JW tagged words, field f
// in word f (ints as their bits, floats as theirs; a double as a float head and tail).
enum : int {
  JW_J, JW_KIND, JW_CBONUS, JW_OFFBONUS, JW_TB_HI, JW_TB_LO,  // bonus: chunk, its offset, u*S left in it
  JW_MT_HI, JW_MT_LO, JW_DM,                                 // rejection: log2-partition of p_j; that of q_j minus it
  JW_TAU_T, JW_TAU_D,                                        // top-k thresholds (bonus: row G in TAU_T)
  JW_OFF_J,                                                  // rejection: row offset of p_j
  JW_USED, JW = 16
};

// ---------------------------------------------------------------- acceptance scan

// ---------------------------------------------------------------- draw helpers
// (ResidualW, TargetW, chunk_masses, segment_draw, wave_chunk_draw: sv_draw.h)

// One wave: pick the chunk of target row r from the first pass's partials (mass
// S_c * 2^(off_c - off_r)), and express the remainder in the chunk's own scale.  The
// partials are complete: the scan that published the job read all of them.
SVD int pick_target_chunk(const Args &a, int r, float off_r, float u, double *t_in) {
  const u64 *pw = a.w.tw_part + (size_t)r * a.C * 3;
  auto cm = [&](int cc) {
    const double s = d_join(tw_f(ld_dev(&pw[cc * 3 + 1])), tw_f(ld_dev(&pw[cc * 3 + 2])));
    const float d = tw_f(ld_dev(&pw[cc * 3])) - off_r;
    return (s > 0.0) ? s * (double)fast_exp2(d) : 0.0;
  };
  const double total = wave_total(a.C, cm);
  double trem;
  const int c = wave_pick(a.C, (double)u * total, cm, &trem);
  *t_in = (c >= 0) ? trem * (double)fast_exp2(off_r - tw_f(ld_dev(&pw[c * 3]))) : 0.0;
  return c;
}

constexpr int SEQ_LDS_PARTS = 256;   // (row, chunk) partials of one sequence staged in LDS
constexpr int SEQ_LDS_ROWS = 129;    // rows of one sequence kept in LDS (G <= 64)

// Greedy (T == 0): the sequence's finisher -- its last item in grid order, one wave --
// waits until every chunk partial of the sequence carries this call's tag, combines each
// row (largest value, lowest index; NaN / +inf mark a row unusable), then scans:
// position i is accepted when the drafted token equals the target argmax
// ("tannlonggtaoo" note, "Greedy Sampling"); the first mismatch, or the bonus position,
// takes the target argmax.  Its own partial (index np - 1) comes from its registers.
template <typename T, bool LDS>
SVD void greedy_finish(const Args &a, int b, float own_best, int own_idx, int own_flag) {
  constexpr int UNR = SEQ_LDS_PARTS / WAVE;
  __shared__ float s_po[SEQ_LDS_PARTS];
  __shared__ int s_pi[SEQ_LDS_PARTS], s_pf[SEQ_LDS_PARTS];
  __shared__ int s_rok[SEQ_LDS_ROWS], s_rarg[SEQ_LDS_ROWS];
  const int lane = lane_id();
  const int G = a.G, rps = a.rps, C = a.C;
  const size_t r0 = (size_t)b * rps;
  const int np = rps * C, own = np - 1;
  constexpr bool lds = LDS;  // the sequence fits in LDS (every access below is resolved at compile time)
  const unsigned tag = a.tag;
  const u64 *pw = a.w.tw_part + r0 * C * 3;
  const int x0 = (lane < G) ? a.tokens[(size_t)b * G + lane] : 0;

  bool alive = true;
  unsigned polls = 0;
  for (int blk = 0; blk < np && alive; blk += SEQ_LDS_PARTS) {
    for (;;) {
      u64 w0[UNR], w1[UNR], w2[UNR];
#pragma unroll
      for (int k = 0; k < UNR; ++k) {
        const int i = blk + lane + k * WAVE;
        const int ii = (i < np && i != own) ? i : 0;
        w0[k] = ld_dev(&pw[(size_t)ii * 3 + 0]);
        w1[k] = ld_dev(&pw[(size_t)ii * 3 + 1]);
        w2[k] = ld_dev(&pw[(size_t)ii * 3 + 2]);
      }
      bool ok = true;
#pragma unroll
      for (int k = 0; k < UNR; ++k) {
        const int i = blk + lane + k * WAVE;
        if (i < np && i != own) ok = ok && tw_ok(w0[k], tag) && tw_ok(w1[k], tag) && tw_ok(w2[k], tag);
      }
      if (__ballot(!ok) == 0) {
        if (lds) {
#pragma unroll
          for (int k = 0; k < UNR; ++k) {
            const int i = lane + k * WAVE;
            if (i < np) {
              s_po[i] = (i == own) ? own_best : tw_f(w0[k]);
              s_pi[i] = (i == own) ? own_idx : (int)(unsigned)w1[k];
              s_pf[i] = (i == own) ? own_flag : (int)(unsigned)w2[k];
            }
          }
        }
        break;
      }
      if (++polls >= a.spin_limit) {
        alive = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  int32_t *out = a.out_tokens + (size_t)b * (G + 1);
  if (!alive) {  // gave up waiting: report it
    for (int i = lane; i <= G; i += WAVE) out[i] = -1;
    if (lane == 0) a.accepted_len[b] = SV_ROW_INTERNAL;
    return;
  }
  lds_sync();
  auto part = [&](int jr, int cc, float &v, int &i, int &f) {
    const int k = jr * C + cc;
    if (lds) {
      v = s_po[k];
      i = s_pi[k];
      f = s_pf[k];
    } else if (k == own) {
      v = own_best;
      i = own_idx;
      f = own_flag;
    } else {
      v = tw_f(ld_dev(&pw[(size_t)k * 3]));
      i = (int)(unsigned)ld_dev(&pw[(size_t)k * 3 + 1]);
      f = (int)(unsigned)ld_dev(&pw[(size_t)k * 3 + 2]);
    }
  };
  auto combine_row = [&](int jr, int &arg, int &ok) {
    float best = -INFINITY;
    int bi = 0x7fffffff, fl = 0;
    for (int cc = 0; cc < C; ++cc) {
      float v;
      int i, f;
      part(jr, cc, v, i, f);
      best_combine(best, bi, v, i);
      fl |= f;
    }
    arg = bi;
    ok = (fl == 2) ? 1 : 0;
  };
  if (lds) {
    for (int jr0 = 0; jr0 < rps; jr0 += WAVE) {  // lane jr combines row jr in chunk order
      const int jr = jr0 + lane;
      if (jr < rps) combine_row(jr, s_rarg[jr], s_rok[jr]);
    }
    lds_sync();
  }
  auto r_stat = [&](int jr, int &arg, int &ok) {
    if (lds) {
      arg = s_rarg[jr];
      ok = s_rok[jr];
    } else {
      combine_row(jr, arg, ok);
    }
  };

  int j = G;
  unsigned flags = 0;  // 1 bad token, 2 bad row
  for (int i0 = 0; i0 < G; i0 += WAVE) {
    const int i = i0 + lane;
    const bool act = i < G;
    bool accept = false;
    if (act) {
      const int x = (i0 == 0) ? x0 : a.tokens[(size_t)b * G + i];
      const bool tok_ok = (x >= 0) && (x < a.V);
      if (!tok_ok) flags |= 1;
      int arg, ok;
      r_stat(i, arg, ok);
      if (!ok) flags |= 2;
      accept = tok_ok && ok && (x == arg);
    }
    const unsigned long long rej = __ballot(act && !accept);
    if (j == G && rej) j = i0 + __ffsll((long long)rej) - 1;
  }
  int argj, okj, argG, okG;
  r_stat(j, argj, okj);
  r_stat(G, argG, okG);
  if (!okG) flags |= 2;  // target row G: the bonus distribution
  flags = wave_or(flags);
  const int err = (flags & 1) ? SV_ROW_BAD_TOKEN : (flags & 2) ? SV_ROW_BAD_LOGITS : 0;
  for (int i = lane; i <= G; i += WAVE) {
    int32_t v;
    if (err) v = -1;
    else if (i < j) v = (i < WAVE) ? x0 : a.tokens[(size_t)b * G + i];
    else if (i > j) v = -1;
    else v = argj;  // the target's own choice
    out[i] = v;
  }
  if (lane == 0) a.accepted_len[b] = err ? err : j;
}

// Sampling: the sequence's finisher -- its last first-pass item in grid order, one wave --
// waits until every chunk partial and drafted-token logit of the sequence carries this
// call's tag (they come from workgroups earlier in the grid), combines each row's
// partials into its log2-partition, then runs the acceptance scan.  Position i of the
// chain: token range, row validity, uniform range, draft support, then the test
// U_i <= min(1, p_i(x)/q_i(x)) with p_i(x) > 0 ("Speculative Decoding 的朴素思想",
// "一次 sampling 怎么执行" step 4; the ratio is formed from log2-probabilities in double).
// It writes the accepted prefix and the -1 padding, and publishes the draw's record
// (the drawn token and accepted_len are written by the draw).  The finisher's own
// partial (index np - 1) and token logit come from its registers.
template <typename T, bool ALIGNED, bool TOPK, bool LDS, bool G0>
SVD void sampling_finish(const Args &a, int b, float own_off, float own_hi, float own_lo,
                         int gx, float gzt, float gzd, const double *s_own_gseg) {
  constexpr int UNR = SEQ_LDS_PARTS / WAVE;
  __shared__ float s_po[SEQ_LDS_PARTS];
  __shared__ double s_ps[SEQ_LDS_PARTS];
  __shared__ float s_roff[SEQ_LDS_ROWS], s_rzx[SEQ_LDS_ROWS], s_rtau[SEQ_LDS_ROWS], s_rsum[SEQ_LDS_ROWS];
  __shared__ double s_rl2s[SEQ_LDS_ROWS];
  __shared__ int s_rok[SEQ_LDS_ROWS];
  const int lane = lane_id();
  const int G = a.G, rps = a.rps, C = a.C;
  const size_t r0 = (size_t)b * rps;
  const int np = rps * C, own = np - 1;
  constexpr bool lds = LDS;  // the sequence fits in LDS (every access below is resolved at compile time)
  const unsigned tag = a.tag;
  const u64 *pw = a.w.tw_part + r0 * C * 3;

  // inputs of positions lane, lane+64, ... (first round only kept in registers; the
  // tokens and their logits of the first round were loaded while this item's chunk
  // streamed in)
  const int x0 = gx;
  const float u0 = (lane < G) ? a.u_accept[(size_t)b * G + lane] : 0.0f;
  const float us = a.u_sample[b];
  // The logit of position p's token in target row p and draft row p (NaN for a token
  // outside [0, V)); positions of the first round come from registers.
  auto gather_zx = [&](int p, float &zt, float &zd) {
    if (p < WAVE) {
      zt = gzt;
      zd = gzd;
      return;
    }
    const int x = a.tokens[(size_t)b * G + p];
    const bool in = x >= 0 && x < a.V;
    zt = in ? Fmt<T>::at(seq_row<T>(a, b, p), (size_t)x) : NAN;
    zd = in ? Fmt<T>::at(seq_row<T>(a, b, G + 1 + p), (size_t)x) : NAN;
  };

  SV_TL(a, TL_SEQ(b) + TL_FIN_IN);
  // Wait for the partials (blocks of SEQ_LDS_PARTS, every load of a block in flight at
  // once); stage them in LDS when the sequence fits.
  bool alive = true;
  unsigned polls = 0;
  for (int blk = 0; blk < np && alive; blk += SEQ_LDS_PARTS) {
    for (;;) {
      u64 w0[UNR], w1[UNR], w2[UNR];
#pragma unroll
      for (int k = 0; k < UNR; ++k) {
        const int i = blk + lane + k * WAVE;
        const int ii = (i < np && i != own) ? i : 0;
        w0[k] = ld_dev(&pw[(size_t)ii * 3 + 0]);
        w1[k] = ld_dev(&pw[(size_t)ii * 3 + 1]);
        w2[k] = ld_dev(&pw[(size_t)ii * 3 + 2]);
      }
      bool ok = true;
#pragma unroll
      for (int k = 0; k < UNR; ++k) {
        const int i = blk + lane + k * WAVE;
        if (i < np && i != own) ok = ok && tw_ok(w0[k], tag) && tw_ok(w1[k], tag) && tw_ok(w2[k], tag);
      }
      if (__ballot(!ok) == 0) {
        if (lds) {
#pragma unroll
          for (int k = 0; k < UNR; ++k) {
            const int i = lane + k * WAVE;
            if (i < np) {
              s_po[i] = (i == own) ? own_off : tw_f(w0[k]);
              s_ps[i] = (i == own) ? d_join(own_hi, own_lo) : d_join(tw_f(w1[k]), tw_f(w2[k]));
            }
          }
        }
        break;
      }
      if (++polls >= a.spin_limit) {
        alive = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  SV_TL(a, TL_SEQ(b) + TL_FIN_PARTS);
  if (lds && alive) {
    for (int jr = lane; jr < rps; jr += WAVE) s_rtau[jr] = TOPK ? a.w.row_tau[r0 + jr] : -INFINITY;
    for (int p = lane; p < G; p += WAVE) {
      float zt, zd;
      gather_zx(p, zt, zd);
      s_rzx[p] = zt;
      s_rzx[G + 1 + p] = zd;
    }
    if (lane == 0) s_rzx[G] = NAN;
  }
  lds_sync();
  u64 *jw = a.w.tw_job + (size_t)b * JW;
  int32_t *out = a.out_tokens + (size_t)b * (G + 1);
  if (!alive) {  // gave up waiting: report it, and let the draw items go
    for (int i = lane; i <= G; i += WAVE) out[i] = -1;
    if (lane == 0) a.accepted_len[b] = SV_ROW_INTERNAL;
    if (lane < JW_USED) tw_put(&jw[lane], tag, lane == JW_KIND ? (unsigned)JOB_NONE : 0u);
    return;
  }

  auto p_off = [&](int jr, int cc) -> float {
    const int i = jr * C + cc;
    if (lds) return s_po[i];
    return (i == own) ? own_off : tw_f(ld_dev(&pw[(size_t)i * 3]));
  };
  auto p_sum = [&](int jr, int cc) -> double {
    const int i = jr * C + cc;
    if (lds) return s_ps[i];
    if (i == own) return d_join(own_hi, own_lo);
    return d_join(tw_f(ld_dev(&pw[(size_t)i * 3 + 1])), tw_f(ld_dev(&pw[(size_t)i * 3 + 2])));
  };
  auto zx_of = [&](int jr) -> float {
    if (lds) return s_rzx[jr];
    if (jr == G) return NAN;
    float zt, zd;
    gather_zx(jr < G ? jr : jr - G - 1, zt, zd);
    return jr < G ? zt : zd;
  };
  auto tau_of = [&](int jr) -> float { return lds ? s_rtau[jr] : (TOPK ? a.w.row_tau[r0 + jr] : -INFINITY); };

  // Row statistics: lane jr combines row jr's chunks (rows in parallel): the row offset
  // is the largest chunk offset, the row sum is sum_c S_c * 2^(off_c - off) in chunk
  // order; the chunks' reads are batched so they are in flight together.  A row with no
  // finite value (every offset -inf) or a NaN comes out with a NaN sum.  Rows beyond the
  // LDS capacity are recombined on demand, which gives the same values.
  auto combine_row = [&](int jr, float &o, double &t) {
    constexpr int CB = 4;
    o = -INFINITY;
    for (int c0 = 0; c0 < C; c0 += CB) {
      float v[CB];
#pragma unroll
      for (int k = 0; k < CB; ++k) v[k] = (c0 + k < C) ? p_off(jr, c0 + k) : -INFINITY;
#pragma unroll
      for (int k = 0; k < CB; ++k) o = fmaxf(o, v[k]);
    }
    t = 0.0;
    for (int c0 = 0; c0 < C; c0 += CB) {
      float v[CB];
      double sc[CB];
#pragma unroll
      for (int k = 0; k < CB; ++k) {
        v[k] = (c0 + k < C) ? p_off(jr, c0 + k) : o;
        sc[k] = (c0 + k < C) ? p_sum(jr, c0 + k) : 0.0;
      }
#pragma unroll
      for (int k = 0; k < CB; ++k) t += sc[k] * (double)fast_exp2(v[k] - o);
    }
  };
  // No drafts, one row of at most 64 chunks and no row statistics asked for: the row's
  // offset is a maximum over chunk lanes, and the chunk is picked right here by the same
  // masses the pick below would use (the chunk masses' total stands for the row sum in
  // the validity test: both are sums of the same terms, and a NaN chunk sum, which the
  // masses skip, marks the row unusable as it makes the row sum NaN).
  const bool g0fast = G0 && lds && !a.row_stats && C <= WAVE;
  int c_fast = -1;
  double trem_fast = 0.0;
  if (G0 && g0fast) {
    const float offc = (lane < C) ? s_po[lane] : -INFINITY;
    const double scv = (lane < C) ? s_ps[lane] : 0.0;
    const float o = wave_max(offc);
    const bool nan = __ballot(lane < C && scv != scv) != 0;
    auto cmf = [&](int cc) {
      const double sc = s_ps[cc];
      return (sc > 0.0) ? sc * (double)fast_exp2(s_po[cc] - o) : 0.0;
    };
    double tot;
    c_fast = wave_pick_frac(C, (double)us, cmf, &trem_fast, &tot);
    const bool ok = isfinite(o) && !nan && isfinite(tot) && tot > 0.0;
    if (lane == 0) {
      s_roff[0] = o;
      s_rl2s[0] = 0.0;
      s_rok[0] = ok ? 1 : 0;
      s_rsum[0] = (float)tot;
    }
  }
  for (int jr0 = 0; jr0 < rps && !(G0 && g0fast); jr0 += WAVE) {
    const int jr = jr0 + lane;
    if (jr < rps) {
      float o;
      double t;
      combine_row(jr, o, t);
      const bool ok = isfinite(o) && isfinite(t) && t > 0.0;
      if (lds) {  // the optional row_stats output is written last, from LDS
        s_roff[jr] = o;
        s_rl2s[jr] = (ok && !G0) ? log2(t) : 0.0;  // no acceptance test reads it without drafts
        s_rok[jr] = ok ? 1 : 0;
        s_rsum[jr] = (float)t;
      } else if (a.row_stats) {
        a.row_stats[(r0 + jr) * 2 + 0] = (float)((double)o * LN2);
        a.row_stats[(r0 + jr) * 2 + 1] = (float)t;
      }
    }
  }
  lds_sync();
  auto r_stat = [&](int jr, float &o, double &l2s, int &ok) {
    if (lds) {
      o = s_roff[jr];
      l2s = s_rl2s[jr];
      ok = s_rok[jr];
    } else {
      double t;
      combine_row(jr, o, t);
      ok = (isfinite(o) && isfinite(t) && t > 0.0) ? 1 : 0;
      l2s = ok ? log2(t) : 0.0;
    }
  };

  int j = G;
  unsigned flags = 0;  // 1 bad token, 2 bad row, 4 bad uniform, 8 q(x) = 0
  for (int i0 = 0; i0 < G; i0 += WAVE) {
    const int i = i0 + lane;
    const bool act = i < G;
    bool accept = false;
    if (act) {
      const int x = (i0 == 0) ? x0 : a.tokens[(size_t)b * G + i];
      const bool tok_ok = (x >= 0) && (x < a.V);
      if (!tok_ok) flags |= 1;
      const int id = G + 1 + i;
      float ot, od;
      double lt, ld;
      int okt, okd;
      r_stat(i, ot, lt, okt);
      r_stat(id, od, ld, okd);
      if (!okt || !okd) flags |= 2;
      const float u = (i0 == 0) ? u0 : a.u_accept[(size_t)b * G + i];
      if (!(u >= 0.0f && u < 1.0f)) flags |= 4;
      if (tok_ok) {
        const float zt = zx_of(i), zd = zx_of(id);
        const bool supp_t = (zt > -INFINITY) && !(zt < tau_of(i));
        const bool supp_d = (zd > -INFINITY) && !(zd < tau_of(id));
        if (!supp_d) flags |= 8;
        if (supp_t && supp_d && okt && okd) {
          const double k2 = (double)a.k2;
          const double l2p = (double)zt * k2 - ((double)ot + lt);
          const double l2q = (double)zd * k2 - ((double)od + ld);
          const double alpha = exp2(fmin(0.0, l2p - l2q));
          accept = (double)u <= alpha;
        }
      }
    }
    const unsigned long long rej = __ballot(act && !accept);
    if (j == G && rej) j = i0 + __ffsll((long long)rej) - 1;
  }
  float oG;
  double l2G;
  int okG;
  r_stat(G, oG, l2G, okG);
  if (!okG) flags |= 2;  // target row G: the bonus distribution
  if (!(us >= 0.0f && us < 1.0f)) flags |= 4;
  if (TOPK) {  // a NaN threshold marks a top-k selection that did not complete
    for (int jr = lane; jr < rps; jr += WAVE)
      if (tau_of(jr) != tau_of(jr)) flags |= 16;
  }
  flags = wave_or(flags);
  const int err = (flags & 16) ? SV_ROW_INTERNAL
                : (flags & 1) ? SV_ROW_BAD_TOKEN
                : (flags & 2) ? SV_ROW_BAD_LOGITS
                : (flags & 4) ? SV_ROW_BAD_UNIFORM
                : (flags & 8) ? SV_ROW_Q_ZERO : 0;
  // The draw's record, one tagged word per lane, goes out first; the outputs follow.
  // With no drafts (G = 0) the bonus is drawn right here (below) and no draw items exist.
  const int kind = (err || G0) ? (int)JOB_NONE : (j < G ? (int)JOB_REJECT : (int)JOB_BONUS);

  // The bonus draw's chunk, when every draft is accepted (or there are none): chunk
  // masses of p_G, S_c * 2^(off_c - off_row) in chunk order, and the remainder in that
  // chunk's scale.
  int c_bonus = -1;
  float off_bonus = 0.0f;
  double t_bonus = 0.0;
  if (okG && (kind == JOB_BONUS || (G0 && !err))) {
    auto cm = [&](int cc) {
      const double sc = p_sum(G, cc);
      return (sc > 0.0) ? sc * (double)fast_exp2(p_off(G, cc) - oG) : 0.0;
    };
    double trem, total;
    if (G0 && g0fast) {
      c_bonus = c_fast;
      trem = trem_fast;
    } else {
      c_bonus = wave_pick_frac(C, (double)us, cm, &trem, &total);
    }
    if (c_bonus >= 0) {
      off_bonus = p_off(G, c_bonus);
      t_bonus = trem * (double)fast_exp2(oG - off_bonus);
    }
  }
  float mt_hi = 0.0f, mt_lo = 0.0f, dm = 0.0f, tau_t = -INFINITY, tau_d = -INFINITY;
  float off_j = 0.0f;
  if (kind == JOB_REJECT) {
    float ot, od;
    double lt, ld;
    int okt, okd;
    r_stat(j, ot, lt, okt);
    r_stat(G + 1 + j, od, ld, okd);
    const double mt = (double)ot + lt, md = (double)od + ld;
    mt_hi = d_head(mt);
    mt_lo = d_tail(mt);
    dm = (float)(md - mt);
    tau_t = tau_of(j);
    tau_d = tau_of(G + 1 + j);
    off_j = ot;
  } else if (kind == JOB_BONUS) {
    tau_t = tau_of(G);
  }
  unsigned bits = 0;
  switch (lane) {
    case JW_J: bits = (unsigned)j; break;
    case JW_KIND: bits = (unsigned)kind; break;
    case JW_CBONUS: bits = (unsigned)c_bonus; break;
    case JW_OFFBONUS: bits = __float_as_uint(off_bonus); break;
    case JW_TB_HI: bits = __float_as_uint(d_head(t_bonus)); break;
    case JW_TB_LO: bits = __float_as_uint(d_tail(t_bonus)); break;
    case JW_MT_HI: bits = __float_as_uint(mt_hi); break;
    case JW_MT_LO: bits = __float_as_uint(mt_lo); break;
    case JW_DM: bits = __float_as_uint(dm); break;
    case JW_TAU_T: bits = __float_as_uint(tau_t); break;
    case JW_TAU_D: bits = __float_as_uint(tau_d); break;
    case JW_OFF_J: bits = __float_as_uint(off_j); break;
    default: break;
  }
  if (!G0 && lane < JW_USED) tw_put(&jw[lane], tag, bits);  // no draw items without drafts
  SV_TL(a, TL_SEQ(b) + TL_FIN_REC);
  for (int i = lane; i <= G; i += WAVE) {
    if (!err && i == j) continue;  // written by the draw, with accepted_len
    out[i] = (!err && i < j) ? ((i < WAVE) ? x0 : a.tokens[(size_t)b * G + i]) : -1;
  }
  if (err && lane == 0) a.accepted_len[b] = err;
  if (lds && a.row_stats) {
    for (int jr = lane; jr < rps; jr += WAVE) {
      a.row_stats[(r0 + jr) * 2 + 0] = (float)((double)s_roff[jr] * LN2);
      a.row_stats[(r0 + jr) * 2 + 1] = s_rsum[jr];
    }
  }
  if (!G0 || err) return;

  // No drafts: the draw from p_1 (the row), in the chunk picked above, by the segment
  // masses that chunk's item published (this item's own when it is that chunk), then one
  // re-read segment.
  int tok = -1;
  if (c_bonus >= 0 && c_bonus < C) {
    double segv = (lane < SEGS) ? s_own_gseg[lane] : 0.0;
    const bool own = (c_bonus == C - 1);  // this item is the row's last chunk
    bool ok = true;
    if (!own) {
      const u64 *gw = a.w.tw_gseg + (((size_t)b * C + c_bonus) * SEGS) * 2;
      const int sl = (lane < SEGS) ? lane : 0;
      for (unsigned polls = 0;;) {
        const u64 h = ld_dev(&gw[2 * sl]), l = ld_dev(&gw[2 * sl + 1]);
        segv = (lane < SEGS) ? d_join(tw_f(h), tw_f(l)) : 0.0;
        if (__ballot(lane < SEGS && !(tw_ok(h, tag) && tw_ok(l, tag))) == 0) break;
        if (++polls >= a.spin_limit) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (!ok) {
      for (int i = lane; i <= G; i += WAVE) out[i] = -1;
      if (lane == 0) a.accepted_len[b] = SV_ROW_INTERNAL;
      return;
    }
    SV_TL(a, TL_SEQ(b) + TL_COMB_IN);
    auto segm = [&](int) { return segv; };
    double ts;
    const int sp = wave_pick(SEGS, t_bonus, segm, &ts);
    if (sp >= 0)
      tok = segment_draw<T, ALIGNED>(a, seq_row<T>(a, b, G), (const T *)nullptr, c_bonus, sp,
                                     TargetW{a.k2, off_bonus, tau_of(G)}, ts);
  }
  if (lane == 0) {
    out[G] = tok;
    a.accepted_len[b] = G;
  }
  SV_TL(a, TL_SEQ(b) + TL_DONE);
}

// ---------------------------------------------------------------- pass 1: normaliser

// First-pass item (row r, chunk c).  Per chunk: m_c = block max of the kept z, off = m_c*k2 (rounded once, stored as is),
// s = sum 2^(fma(z, k2, -off)).  The log2-partition of a row is off_row + log2(s_row)
// with off_row the float actually subtracted, so every consumer reproduces the same
// probabilities; the second pass recomputes a chunk's terms bit for bit from the same offset.
template <typename T, bool ALIGNED, bool TOPK, bool G0>
SVD void norm_item(const Args &a, int item) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ float s_m[NW];
  __shared__ double s_s[NW];
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  const int r = item / a.C, c = item - r * a.C;
  const int b = r / a.rps, jr = r - b * a.rps;

  // The sequence's finisher (its last item) gathers the drafted tokens and their logits
  // in every target and draft row (positions = lanes of wave 0) while its own chunk
  // streams in: the token loads go first, the gathers right after the chunk's loads,
  // before any of them is waited for.
  const bool finisher = (jr == a.rps - 1 && c == a.C - 1);
  const bool gath = finisher && !G0 && wid == 0 && lane < a.G;
  const int gx = gath ? a.tokens[(size_t)b * a.G + lane] : 0;
  const T *row = seq_row<T>(a, b, jr);
  float gzt = NAN, gzd = NAN;

  // The partial goes out (or the sequence is finished) from wave 0.
  __shared__ double s_gseg[SEGS];
  auto finish = [&](float off, float s_hi, float s_lo) {
    if (jr == a.rps - 1 && c == a.C - 1) {
      if (a.rps * a.C <= SEQ_LDS_PARTS && a.rps <= SEQ_LDS_ROWS)
        sampling_finish<T, ALIGNED, TOPK, true, G0>(a, b, off, s_hi, s_lo, gx, gzt, gzd, s_gseg);
      else
        sampling_finish<T, ALIGNED, TOPK, false, G0>(a, b, off, s_hi, s_lo, gx, gzt, gzd, s_gseg);
      return;
    }
    u64 *pw = a.w.tw_part + ((size_t)r * a.C + c) * 3;
    if (lane < 3) tw_putf(pw + lane, a.tag, lane == 0 ? off : (lane == 1 ? s_hi : s_lo));
    if (jr * a.C + c < TL_FIN_IN) SV_TL(a, TL_SEQ(b) + jr * a.C + c);
    if (G0 && lane < 2 * SEGS) {
      u64 *gw = a.w.tw_gseg + (((size_t)b * a.C + c) * SEGS) * 2;
      const double v = s_gseg[lane >> 1];
      tw_putf(&gw[lane], a.tag, (lane & 1) ? d_tail(v) : d_head(v));
    }
  };
  float x[VPT][VEC];
  if (ALIGNED) {
    u32x4 w[VPT];
    const u32x4 *rv = reinterpret_cast<const u32x4 *>(row);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = c * CHUNK_VECS + k * NT + tid;
      w[k] = __builtin_nontemporal_load(rv + (v < a.nvec ? v : a.nvec - 1));
    }
    if (finisher && gath && gx >= 0 && gx < a.V) {
      gzt = Fmt<T>::at(seq_row<T>(a, b, lane), (size_t)gx);
      gzd = Fmt<T>::at(seq_row<T>(a, b, a.G + 1 + lane), (size_t)gx);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) Fmt<T>::unpack(w[k], x[k]);
    if ((c + 1) * CHUNK_VECS > a.nvec) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const bool in = c * CHUNK_VECS + k * NT + tid < a.nvec;
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[k][e] = in ? x[k][e] : -INFINITY;
      }
    }
  } else {
    load_chunk<T, ALIGNED, true>(row, a.V, a.nvec, c, tid, x);
    if (gath && gx >= 0 && gx < a.V) {
      gzt = Fmt<T>::at(seq_row<T>(a, b, lane), (size_t)gx);
      gzd = Fmt<T>::at(seq_row<T>(a, b, a.G + 1 + lane), (size_t)gx);
    }
  }
  if (TOPK) {
    const float tau = a.w.row_tau[r];  // written by the previous kernel
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

  const float k2 = a.k2;
  float off;
  double s;
  // With no drafts (G = 0, the batched sampler) the row's chunks give masses per 64-vector
  // segment, a lane's elements summed in index order and the lanes by one DPP tree (the
  // order the draw uses when it re-reads one segment); the chunk sum is the sum of its
  // segments.  The finisher then draws without a second pass over a chunk.
  constexpr bool bonus_row = G0;  // the batched sampler: the finisher draws from segment masses
  if (bonus_row) {
    off = (m > -INFINITY) ? m * k2 : -INFINITY;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float lm = 0.0f;
      if (m > -INFINITY) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) lm += fast_exp2(fmaf(x[k][e], k2, -off));
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) nan |= (x[k][e] != x[k][e]);
      }
      const double sm = wave_sum((double)lm);
      if (lane == 0) s_gseg[k * NW + wid] = sm;
    }
    s = (!(m > -INFINITY) && nan) ? (double)NAN : 0.0;  // an empty chunk still shows a NaN
  } else if (m > -INFINITY) {
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
  } else {  // nothing finite in the chunk: keep a NaN visible, otherwise an empty partial
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
  if (wid != 0) return;  // one wave finishes the workgroup

  double S = (s_s[0] + s_s[1]) + (s_s[2] + s_s[3]);
  if (bonus_row) S = (S != S) ? S : wave_sum((lane < SEGS) ? s_gseg[lane] : 0.0);
  // The sequence's last item in grid order finishes the sequence, from its own values
  // and the other items' published ones.
  finish(off, d_head(S), d_tail(S));
}

// ---------------------------------------------------------------- pass 1: greedy argmax

template <typename T, bool ALIGNED>
__global__ __launch_bounds__(NT) void k_argmax(const Args a) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ float s_v[NW];
  __shared__ int s_i[NW], s_f[NW];
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  int phase, item;
  if (!lane_item(a.B, a.rps * a.C, 0, phase, item)) return;  // units: sequences
  const int r = item / a.C, c = item - r * a.C;
  const int b = r / a.rps, jr = r - b * a.rps;

  float x[VPT][VEC];
  load_chunk<T, ALIGNED, true>(seq_row<T>(a, b, jr), a.V, a.nvec, c, tid, x);
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
  wave_best(best, bi, fl);
  if (lane == 0) {
    s_v[wid] = best;
    s_i[wid] = bi;
    s_f[wid] = fl;
  }
  __syncthreads();
  if (wid != 0) return;  // one wave finishes the workgroup

  best = s_v[0];
  bi = s_i[0];
  fl = s_f[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    best_combine(best, bi, s_v[w], s_i[w]);
    fl |= s_f[w];
  }
  // The sequence's last item in grid order finishes the sequence.
  if (jr == a.rps - 1 && c == a.C - 1) {
    if (a.rps * a.C <= SEQ_LDS_PARTS && a.rps <= SEQ_LDS_ROWS) greedy_finish<T, true>(a, b, best, bi, fl);
    else greedy_finish<T, false>(a, b, best, bi, fl);
    return;
  }
  u64 *pw = a.w.tw_part + ((size_t)r * a.C + c) * 3;
  if (lane < 3) tw_put(pw + lane, a.tag, lane == 0 ? __float_as_uint(best) : (lane == 1 ? (unsigned)bi : (unsigned)fl));
}

// ---------------------------------------------------------------- pass 2: the draw

constexpr int COMB_LDS_SEGS = 1024;  // segment masses of one sequence kept in LDS by the combiner

// The sequence's last draw item (one wave): wait for every other item's segment masses
// (lane l reads segments 4l..4l+3 of each block of 256, every load of a block in flight
// at once), keep them in LDS (FITS: all of them; otherwise the rest are read on demand),
// then one inverse CDF over all segments in index order picks the segment, and the
// segment is re-read to pick lane and element.
template <typename T, bool ALIGNED, bool FITS>
SVD void combine_draw(const Args &a, int b, int j, float u, const T *row_t, const T *row_d,
                      const ResidualW &wf, const double *s_seg, double *s_cs, int own0) {
  constexpr int SB = 4, BLK = SB * WAVE, MINE = KSUB * NW;
  const int lane = lane_id();
  const unsigned tag = a.tag;
  const int G = a.G;
  const int nseg = a.C * SEGS;
  const int cown = own0 / SEGS;
  const u64 *sw = a.w.tw_seg + (size_t)b * a.C * SEGS * 2;
  auto mine = [&](int i) { return i >= own0 && i < own0 + MINE; };
  bool alive = true;
  unsigned polls = 0;
  for (int blk = 0; blk < nseg && alive; blk += BLK) {
    for (;;) {
      u64 wh[SB], wl[SB];
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const int i = blk + lane * SB + k;
        const int ii = (i < nseg && !mine(i)) ? i : 0;
        wh[k] = ld_dev(&sw[(size_t)ii * 2]);
        wl[k] = ld_dev(&sw[(size_t)ii * 2 + 1]);
      }
      bool ok = true;
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const int i = blk + lane * SB + k;
        if (i < nseg && !mine(i)) ok = ok && tw_ok(wh[k], tag) && tw_ok(wl[k], tag);
      }
      if (__ballot(!ok) == 0) {
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          const int i = blk + lane * SB + k;
          if (i < nseg && i < COMB_LDS_SEGS) s_cs[i] = mine(i) ? s_seg[i - cown * SEGS] : d_join(tw_f(wh[k]), tw_f(wl[k]));
        }
        break;
      }
      if (++polls >= a.spin_limit) {
        alive = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  if (!alive) {
    if (lane == 0) a.accepted_len[b] = SV_ROW_INTERNAL;
    return;
  }
  lds_sync();
  SV_TL(a, TL_SEQ(b) + TL_COMB_IN);
  auto seg_of = [&](int i) -> double {
    if (FITS || i < COMB_LDS_SEGS) return s_cs[i];
    if (mine(i)) return s_seg[i - cown * SEGS];
    return d_join(tw_f(ld_dev(&sw[(size_t)i * 2])), tw_f(ld_dev(&sw[(size_t)i * 2 + 1])));
  };
  double Z, ts;
  const int sp = wave_pick4_frac(nseg, (double)u, seg_of, &ts, &Z);
  int tok = -1;
  if (Z > 0.0) {
    if (sp >= 0 && sp < nseg) tok = segment_draw<T, ALIGNED>(a, row_t, row_d, sp / SEGS, sp % SEGS, wf, ts);
  } else {  // zero residual (p and q differ only where p's mass is lost to rounding): draw from p_j
    const int rt = b * a.rps + j;
    double tin;
    const int cp = pick_target_chunk(a, rt, wf.off_j, u, &tin);
    if (cp >= 0 && cp < a.C) {
      const TargetW tw{a.k2, tw_f(ld_dev(&a.w.tw_part[((size_t)rt * a.C + cp) * 3])), wf.tau_t};
      tok = wave_chunk_draw<T, ALIGNED>(a, row_t, (const T *)nullptr, cp, tw, tin);
    }
  }
  if (lane == 0) {
    a.out_tokens[(size_t)b * (G + 1) + j] = tok;
    a.accepted_len[b] = j;
  }
  SV_TL(a, TL_SEQ(b) + TL_DONE);
}

// Draw item (sequence b, chunk c, quarter sub).  All draw items follow every first-pass
// item in the grid.  Each waits until the sequence's record carries this call's tag, then
// for a rejection at j computes the masses of [p_j - q_j]_+ of its quarter of the chunk
// per 64-vector segment and publishes them; the sequence's last draw item in grid order
// (c = C-1, sub = NSUB-1) waits for all of them, picks the segment over all of them, and
// one wave re-reads that segment to pick lane and element.  For a bonus, the chunk picked
// by the scan from the first pass's partials re-reads itself and draws from p_G (one
// item; the others leave).  With a row error the items leave.  The item that writes the
// drawn token also writes accepted_len.
template <typename T, bool ALIGNED>
SVD void draw_item(const Args &a, int item) {
  __shared__ double s_seg[SEGS];
  __shared__ unsigned s_job[JW];
  __shared__ int s_ready;
  const int tid = threadIdx.x, wid = tid / WAVE, lane = lane_id();
  const int b = item / (a.C * NSUB);
  const int rem = item - b * a.C * NSUB;
  const int c = rem / NSUB, sub = rem - c * NSUB;
  const int G = a.G;
  const unsigned tag = a.tag;
  int32_t *out = a.out_tokens + (size_t)b * (G + 1);

  // Wave 0 polls the record (one word per lane); the other waves wait at the barrier.
  if (wid == 0) {
    const u64 *jw = a.w.tw_job + (size_t)b * JW;
    bool ready = false;
    u64 w = 0;
    for (unsigned n = 0; n < a.spin_limit; ++n) {
      w = (lane < JW_USED) ? ld_dev(&jw[lane]) : 0ull;
      if (__ballot(lane < JW_USED && !tw_ok(w, tag)) == 0) {
        ready = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (lane < JW) s_job[lane] = (unsigned)w;
    if (lane == 0) s_ready = ready ? 1 : 0;
  }
  __syncthreads();
  if (c * NSUB + sub < TL_DRAW_MAX && wid == 0) SV_TL(a, TL_SEQ(b) + TL_DRAW_SEEN + c * NSUB + sub);
  if (!s_ready) {  // gave up: report it instead of drawing
    if (tid == 0) a.accepted_len[b] = SV_ROW_INTERNAL;
    return;
  }
  const int kind = (int)s_job[JW_KIND], j = (int)s_job[JW_J];
  // Accept only well-formed jobs, so workspace contents can never become an
  // out-of-range row or chunk index.
  if (!((kind == JOB_REJECT && j >= 0 && j < G) || (kind == JOB_BONUS && j == G))) return;
  const float u = a.u_sample[b];
  auto jf = [&](int f) { return __uint_as_float(s_job[f]); };

  if (kind == JOB_BONUS) {
    // The scan already picked the chunk from p_G's partials; only that chunk works (chunk
    // 0 reports -1 if the record names no chunk).
    const int cb = (int)s_job[JW_CBONUS];
    const bool cb_ok = cb >= 0 && cb < a.C;
    if (sub != 0 || c != (cb_ok ? cb : 0)) return;
    if (!cb_ok) {
      if (tid == 0) {
        out[G] = -1;
        a.accepted_len[b] = G;
      }
      return;
    }
    const TargetW tw{a.k2, jf(JW_OFFBONUS), jf(JW_TAU_T)};
    const double t_bonus = d_join(jf(JW_TB_HI), jf(JW_TB_LO));
    const T *row = seq_row<T>(a, b, G);
    chunk_masses<T, ALIGNED, VPT, VPT, false>(a, row, (const T *)nullptr, c, 0, tw, s_seg);
    if (wid != 0) return;
    auto segm = [&](int i) { return s_seg[i]; };
    double ts;
    const int sp = wave_pick(SEGS, t_bonus, segm, &ts);
    const int tok = (sp >= 0) ? segment_draw<T, ALIGNED>(a, row, (const T *)nullptr, c, sp, tw, ts) : -1;
    if (lane == 0) {
      out[G] = tok;
      a.accepted_len[b] = G;
    }
    SV_TL(a, TL_SEQ(b) + TL_DONE);
    return;
  }

  // Rejection at position j.
  ResidualW wf;
  wf.k2 = a.k2;
  wf.mt_hi = jf(JW_MT_HI);
  wf.mt_lo = jf(JW_MT_LO);
  wf.dm = jf(JW_DM);
  wf.tau_t = jf(JW_TAU_T);
  wf.tau_d = jf(JW_TAU_D);
  wf.off_j = jf(JW_OFF_J);
  const T *row_t = seq_row<T>(a, b, j), *row_d = seq_row<T>(a, b, G + 1 + j);
  chunk_masses<T, ALIGNED, KSUB, KSUB, true>(a, row_t, row_d, c, sub * KSUB, wf, s_seg);
  if (wid != 0) return;  // wave 0 publishes and finishes
  u64 *sw = a.w.tw_seg + (size_t)b * a.C * SEGS * 2;
  const int own0 = c * SEGS + sub * KSUB * NW;
  if (c != a.C - 1 || sub != NSUB - 1) {
    if (lane < 2 * KSUB * NW) {
      const double m = s_seg[sub * KSUB * NW + (lane >> 1)];
      tw_putf(&sw[(size_t)own0 * 2 + lane], tag, (lane & 1) ? d_tail(m) : d_head(m));
    }
    if (c * NSUB + sub < TL_DRAW_MAX) SV_TL(a, TL_SEQ(b) + TL_DRAW_PUB + c * NSUB + sub);
    return;
  }
  // The sequence's last draw item combines (its own masses stay in LDS, unpublished).
  __shared__ double s_cs[COMB_LDS_SEGS];
  if (a.C * SEGS <= COMB_LDS_SEGS)
    combine_draw<T, ALIGNED, true>(a, b, j, u, row_t, row_d, wf, s_seg, s_cs, own0);
  else
    combine_draw<T, ALIGNED, false>(a, b, j, u, row_t, row_d, wf, s_seg, s_cs, own0);
}

// Sampling: the first pass (normalisers, acceptance scan) and the draws in one grid;
// units are sequences: first-pass items (rows in order, chunks in order), then draw items.
// G0: no drafted positions (the batched sampler): first-pass items only.  Four resident
// waves per SIMD (up to 128 registers) measure faster than five, except after the top-k
// passes, where five do.
template <typename T, bool ALIGNED, bool TOPK, bool G0>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(TOPK ? 5 : 4))) void k_verify(const Args a) {
  int phase, item;
  if (blockIdx.x == 0 && threadIdx.x < WAVE) SV_TL(a, 0);
  if (!lane_item(a.B, a.rps * a.C, G0 ? 0 : a.C * NSUB, phase, item)) return;
  if (phase == 1) norm_item<T, ALIGNED, TOPK, G0>(a, item);
  else if (!G0) draw_item<T, ALIGNED>(a, item);
}

// ---------------------------------------------------------------- after the one-pass top-k

// Weights of a draw from target row j alone (the bonus, or the zero-residual fallback):
// p_j(v) = 2^(z*k2 - Mt) for kept z (z >= tau), Mt the row's log2-partition as a float
// head and tail.
struct KeptW {
  float k2, mt_hi, mt_lo, tau;
  SVD float operator()(float zt, float) const {
    zt = (zt < tau) ? -INFINITY : zt;
    return fast_exp2(fmaf(zt, k2, -mt_hi) - mt_lo);
  }
};

// Inverse CDF over whole rows by one workgroup, for a row whose kept set has no list
// (heavy ties): every chunk's mass (its segment masses summed in order), the chunk that
// holds u*Z, that chunk's segment masses again, then one segment re-read for lane and
// element.  Returns the token in every thread (-1 with no positive mass) and the total in
// *Z.
template <typename T, bool ALIGNED, bool PAIR, typename WFn>
SVD int block_row_draw(const Args &a, const T *rowA, const T *rowB, const WFn &wf, float u,
                       double *s_seg, double *s_ctot, double *Z) {
  __shared__ int s_res;
  __shared__ double s_rem, s_tot;
  const int wid = threadIdx.x / WAVE, lane = lane_id();
  const int C = a.C;
  for (int c = 0; c < C; ++c) {
    chunk_masses<T, ALIGNED, VPT, VPT, PAIR>(a, rowA, rowB, c, 0, wf, s_seg);
    if (wid == 0) {
      const double t = wave_sum((lane < SEGS) ? s_seg[lane] : 0.0);
      if (lane == 0) s_ctot[c] = t;
    }
    __syncthreads();
  }
  if (wid == 0) {
    double trem, tot;
    auto cm = [&](int i) { return s_ctot[i]; };
    const int cp = wave_pick4_frac(C, (double)u, cm, &trem, &tot);
    if (lane == 0) {
      s_res = cp;
      s_rem = trem;
      s_tot = tot;
    }
  }
  __syncthreads();
  const int cp = s_res;
  *Z = s_tot;
  if (cp < 0 || cp >= C) return -1;
  const double trem = s_rem;
  __syncthreads();  // every thread holds cp and the remainder before they are reused
  chunk_masses<T, ALIGNED, VPT, VPT, PAIR>(a, rowA, rowB, cp, 0, wf, s_seg);
  if (wid == 0) {
    auto segm = [&](int i) { return s_seg[i]; };
    double ts;
    const int sp = wave_pick(SEGS, trem, segm, &ts);
    const int tok = (sp >= 0) ? segment_draw<T, ALIGNED>(a, rowA, PAIR ? rowB : (const T *)nullptr, cp, sp, wf, ts) : -1;
    if (lane == 0) s_res = tok;
  }
  __syncthreads();
  return s_res;
}

// Verification after the one-pass top-k threshold: one workgroup per sequence, and no
// logit row is read in bulk.  k_topk_merge left each row's kept-set normaliser and (unless
// heavy ties) its kept (index, logit) pairs in index order, so:
//  - the acceptance test of every position (thread i: positions i, i + 256, ...) needs its
//    token's logit in the two rows and the two rows' log2-partitions; every position's row,
//    token, uniform and support checks count, as in the streamed scan, and the first
//    rejection comes from an LDS minimum;
//  - a rejection at j draws from [p_j - q_j]_+ ("Speculative Decoding 的朴素思想", section
//    "Correction 为什么用正残差"), which is zero outside p_j's kept set: the weights of the
//    listed values, with q_j's logit gathered at each index, and one inverse CDF over them
//    in index order; a zero residual draws from p_j over the same list;
//  - all accepted draws the bonus from p_G's list the same way.
// A row with no list is streamed by the workgroup itself (block_row_draw).
template <typename T, bool ALIGNED>
__global__ __launch_bounds__(NT) void k_topk_verify(const Args a, int cap) {
  __shared__ int s_j;
  __shared__ unsigned s_flags;
  __shared__ float s_w[TOPK_LDS_KEYS];  // the kept list's weights (cap <= 1024)
  __shared__ double s_seg[SEGS], s_ctot[TOPK_SELECT_MAX_C];
  const int tid = threadIdx.x, wid = tid / WAVE, lane = lane_id();
  const int b = blockIdx.x;
  if (b >= a.B) return;
  const int G = a.G, rps = a.rps;
  const size_t r0 = (size_t)b * rps;
  const uint4 *rowp = a.w.tk_rowp;  // written by the previous kernel
  const float *rtau = a.w.row_tau;
  int32_t *out = a.out_tokens + (size_t)b * (G + 1);
  if (tid == 0) {
    s_j = G;
    s_flags = 0u;
  }
  __syncthreads();

  // A row's offset and log2 of its sum; false for an unusable row (no finite value kept,
  // a NaN, or a kept +inf).
  auto rstat = [&](size_t r, float &o, double &l2s) -> bool {
    const uint4 v = rowp[r];
    o = __uint_as_float(v.x);
    const double S = d_join(__uint_as_float(v.y), __uint_as_float(v.z));
    const bool ok = isfinite(o) && isfinite(S) && S > 0.0;
    l2s = ok ? log2(S) : 0.0;
    return ok;
  };

  unsigned flags = 0;  // 1 bad token, 2 bad row, 4 bad uniform, 8 q(x) = 0, 16 no threshold
  for (int i = tid; i < G; i += NT) {
    const int x = a.tokens[(size_t)b * G + i];
    const bool tok_ok = x >= 0 && x < a.V;
    if (!tok_ok) flags |= 1;
    float ot, od;
    double lt, ld;
    const bool okt = rstat(r0 + i, ot, lt);
    const bool okd = rstat(r0 + G + 1 + i, od, ld);
    if (!okt || !okd) flags |= 2;
    const float u = a.u_accept[(size_t)b * G + i];
    if (!(u >= 0.0f && u < 1.0f)) flags |= 4;
    bool accept = false;
    if (tok_ok) {
      const float zt = Fmt<T>::at(seq_row<T>(a, b, i), (size_t)x);
      const float zd = Fmt<T>::at(seq_row<T>(a, b, G + 1 + i), (size_t)x);
      const bool supp_t = (zt > -INFINITY) && !(zt < rtau[r0 + i]);
      const bool supp_d = (zd > -INFINITY) && !(zd < rtau[r0 + G + 1 + i]);
      if (!supp_d) flags |= 8;
      if (supp_t && supp_d && okt && okd) {
        const double k2 = (double)a.k2;
        const double l2p = (double)zt * k2 - ((double)ot + lt);
        const double l2q = (double)zd * k2 - ((double)od + ld);
        accept = (double)u <= exp2(fmin(0.0, l2p - l2q));
      }
    }
    if (!accept) atomicMin(&s_j, i);
  }
  for (int jr = tid; jr < rps; jr += NT)
    if (rtau[r0 + jr] != rtau[r0 + jr]) flags |= 16;  // a selection that did not complete
  const float us = a.u_sample[b];
  if (tid == 0) {
    float o;
    double l;
    if (!rstat(r0 + G, o, l)) flags |= 2;  // target row G: the bonus distribution
    if (!(us >= 0.0f && us < 1.0f)) flags |= 4;
  }
  flags = wave_or(flags);
  if (lane == 0 && flags) atomicOr(&s_flags, flags);
  __syncthreads();
  const int j = s_j;
  const unsigned fl = s_flags;
  const int err = (fl & 16) ? SV_ROW_INTERNAL
                : (fl & 1) ? SV_ROW_BAD_TOKEN
                : (fl & 2) ? SV_ROW_BAD_LOGITS
                : (fl & 4) ? SV_ROW_BAD_UNIFORM
                : (fl & 8) ? SV_ROW_Q_ZERO : 0;
  if (a.row_stats) {
    for (int jr = tid; jr < rps; jr += NT) {
      const uint4 v = rowp[r0 + jr];
      a.row_stats[(r0 + jr) * 2 + 0] = (float)((double)__uint_as_float(v.x) * LN2);
      a.row_stats[(r0 + jr) * 2 + 1] = (float)d_join(__uint_as_float(v.y), __uint_as_float(v.z));
    }
  }
  if (err) {
    for (int i = tid; i <= G; i += NT) out[i] = -1;
    if (tid == 0) a.accepted_len[b] = err;
    return;
  }
  for (int i = tid; i <= G; i += NT)
    if (i != j) out[i] = (i < j) ? a.tokens[(size_t)b * G + i] : -1;

  // The draw at j (a rejection) or G (the bonus).
  const bool rej = j < G;
  const size_t rt = r0 + j, rd = r0 + G + 1 + j;
  float ot, od = 0.0f;
  double lt, ld = 0.0;
  rstat(rt, ot, lt);
  if (rej) rstat(rd, od, ld);
  const double mt = (double)ot + lt, md = (double)od + ld;
  ResidualW rw;
  rw.k2 = a.k2;
  rw.mt_hi = d_head(mt);
  rw.mt_lo = d_tail(mt);
  rw.dm = rej ? (float)(md - mt) : 0.0f;
  rw.tau_t = rtau[rt];
  rw.tau_d = rej ? rtau[rd] : -INFINITY;
  rw.off_j = ot;
  const KeptW pw{a.k2, rw.mt_hi, rw.mt_lo, rw.tau_t};
  const T *row_t = seq_row<T>(a, b, j);
  const T *row_d = rej ? seq_row<T>(a, b, G + 1 + j) : (const T *)nullptr;
  const unsigned n = rowp[rt].w;
  if (n != KEEP_NONE && n <= (unsigned)cap) {
    const uint2 *kl = a.w.tk_keep + rt * (size_t)cap;
    for (unsigned e = tid; e < n; e += NT) {
      const uint2 kv = kl[e];
      const float zt = __uint_as_float(kv.y);
      float w;
      if (rej) {
        const bool in = kv.x < (unsigned)a.V;  // the list is workspace data: never index past the row
        const float zd = in ? Fmt<T>::at(row_d, (size_t)kv.x) : -INFINITY;
        w = in ? rw(zt, zd) : 0.0f;
      } else {
        w = (kv.x < (unsigned)a.V) ? pw(zt, 0.0f) : 0.0f;
      }
      s_w[e] = w;
    }
    __syncthreads();
    if (wid != 0) return;
    auto wm = [&](int i) { return (double)s_w[i]; };
    double trem, Z;
    int pk = wave_pick4_frac((int)n, (double)us, wm, &trem, &Z);
    if (rej && !(Z > 0.0)) {  // zero residual: draw from p_j
      for (unsigned e = lane; e < n; e += WAVE) {
        const uint2 kv = kl[e];
        s_w[e] = (kv.x < (unsigned)a.V) ? pw(__uint_as_float(kv.y), 0.0f) : 0.0f;
      }
      lds_sync();
      pk = wave_pick4_frac((int)n, (double)us, wm, &trem, &Z);
    }
    const int tok = (pk >= 0) ? (int)kl[pk].x : -1;
    if (lane == 0) {
      out[j] = tok;
      a.accepted_len[b] = j;
    }
    return;
  }
  // No list: the workgroup streams the rows at j.
  double Z = 0.0;
  int tok;
  if (rej) {
    tok = block_row_draw<T, ALIGNED, true>(a, row_t, row_d, rw, us, s_seg, s_ctot, &Z);
    if (!(Z > 0.0)) tok = block_row_draw<T, ALIGNED, false>(a, row_t, (const T *)nullptr, pw, us, s_seg, s_ctot, &Z);
  } else {
    tok = block_row_draw<T, ALIGNED, false>(a, row_t, (const T *)nullptr, pw, us, s_seg, s_ctot, &Z);
  }
  if (tid == 0) {
    out[j] = tok;
    a.accepted_len[b] = j;
  }
}

}  // namespace sv

// ======================================================================== host side

namespace sv_host {

// Launches counted over the process; a launch's tag is the count's low 32 bits (never 0),
// so a tag value comes back after 2^32 - 1 launches (see sv_tag_epoch).
std::atomic<unsigned long long> g_launches{0};
unsigned long long *g_stamps = nullptr;  // timeline stamps (the timeline build only)
unsigned next_tag() {
  for (;;) {
    const unsigned t = (unsigned)(g_launches.fetch_add(1ull, std::memory_order_relaxed) + 1ull);
    if (t != 0u) return t;
  }
}
unsigned next_tag_block(unsigned n) {
  for (;;) {
    const unsigned long long c = g_launches.fetch_add((unsigned long long)n, std::memory_order_relaxed);
    const unsigned t = (unsigned)(c + 1ull);
    if (t != 0u && (unsigned long long)t + n - 1ull <= 0xffffffffull) return t;  // the block holds no 0
  }
}

}  // namespace sv_host

namespace {

using namespace sv;
using sv_host::align256;
using sv_host::next_tag;

struct Plan {
  bool greedy, topk, aligned;
  int esz, vec, nvec, C, rps;
  long long R;
  // workspace offsets
  size_t tw_part, tw_job, tw_seg, tw_gseg, tw_hist, row_tau, tk_state, total;
  size_t zero_bytes;  // leading bytes (tagged words) that must be clean when a call starts
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
  // grids padded to whole lanes (see lane_item)
  const long long lanes_b = (B + LANES - 1) / LANES * LANES, lanes_r = (p.R + LANES - 1) / LANES * LANES;
  if (lanes_b * ((long long)p.rps * p.C + (long long)p.C * NSUB) > 0x7fffffffLL || lanes_r * p.C > 0x7fffffffLL)
    return false;
  const size_t R = (size_t)p.R, C = (size_t)p.C, Bz = (size_t)B;
  const bool smp = !p.greedy;
  size_t o = 0;
  // The tagged words first: the part that must be clean (zero, or words of completed
  // calls) when a call starts.  Every one of them is an 8-byte aligned word with its tag
  // in the upper half, so whatever layout wrote them, a tag position holds zero or an
  // earlier tag: never the tag of a call to come.
  p.tw_part = o; o = align256(o + R * C * 3 * 8);
  p.tw_job = o; o = align256(o + (smp ? Bz * JW * 8 : 0));
  p.tw_seg = o; o = align256(o + (smp ? Bz * C * SEGS * 2 * 8 : 0));
  p.tw_gseg = o; o = align256(o + (smp ? Bz * C * SEGS * 2 * 8 : 0));
  p.tw_hist = o; o = align256(o + (p.topk ? sv_host::topk_words(p.R, p.C, top_k) * 8 : 0));
  p.zero_bytes = o;
  p.row_tau = o; o = align256(o + (p.topk ? R * 4 : 0));
  p.tk_state = o; o = align256(o + (p.topk ? sv_host::topk_state_bytes(p.R, p.C, top_k, true) : 0));
  p.total = o;
  return true;
}

const char *kPlanNames[] = {
    "k_topk_digit;k_topk_digit;k_verify",
    "k_topk_digit;k_topk_digit;k_topk_digit;k_topk_digit;k_verify",
    "k_verify",
    "k_argmax",
    "k_topk_select;k_topk_merge;k_topk_verify",
};

template <typename T, bool AL>
hipError_t launch_all(const Plan &p, const Args &a, hipStream_t st, void *const *ev, int nev,
                      int *nl) {
  // Grids padded to whole lanes of units (see lane_item): rows for the top-k passes,
  // sequences for k_argmax and k_verify.
  const long long lb = (a.B + LANES - 1) / LANES, lr = (p.R + LANES - 1) / LANES;
  const unsigned topk_grid = (unsigned)(LANES * lr * p.C);
  const unsigned argmax_grid = (unsigned)(LANES * lb * p.rps * p.C);
  const unsigned verify_grid = (unsigned)(LANES * lb * ((long long)p.rps * p.C + (a.G > 0 ? (long long)p.C * NSUB : 0)));
  sv_host::Launcher L{st, ev, nev};
  auto go = [&](const void *fn, unsigned grid, void **args) { L.go(fn, grid, args); };
  Args aa = a;
  if (p.greedy) {
    aa.tag = next_tag();
    void *args[] = {&aa};
    go((const void *)&k_argmax<T, AL>, argmax_grid, args);
  } else {
    if (p.topk) {
      sv_host::launch_topk<T, AL>(L, aa, topk_grid, p.C);
      aa.tag = next_tag();
      if (sv_host::topk_one_pass(a.top_k, p.C)) {
        // the merge left every row's normaliser and kept list: one workgroup per sequence
        int cap = sv_host::topk_cap(a.top_k);
        void *args[] = {&aa, &cap};
        go((const void *)&k_topk_verify<T, AL>, (unsigned)a.B, args);
      } else {
        void *args[] = {&aa};
        go(a.G == 0 ? (const void *)&k_verify<T, AL, true, true> : (const void *)&k_verify<T, AL, true, false>,
           verify_grid, args);
      }
    } else {
      aa.tag = next_tag();
      void *args[] = {&aa};
      go(a.G == 0 ? (const void *)&k_verify<T, AL, false, true> : (const void *)&k_verify<T, AL, false, false>,
         verify_grid, args);
    }
  }
  if (nl) *nl = L.n;
  return L.e;
}

// Every check of the arguments before the workspace's size and alignment, in the
// documented order (ws_null: a workspace pointer is required and NULL).
sv_status check_args(const void *target, const void *draft, sv_dtype dt, const int32_t *tokens,
                     const float *u_accept, const float *u_sample, int32_t B, int32_t G, int32_t V,
                     float T, int32_t top_k, const int32_t *acc, const int32_t *out, bool ws_null,
                     Plan &p) {
  if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_DTYPE;
  if (B < 1 || G < 0 || V < 1) return SV_ERR_SHAPE;
  if (!(T >= 0.0f) || !isfinite(T)) return SV_ERR_TEMPERATURE;
  if (!make_plan(B, G, V, dt, T, top_k, p)) return SV_ERR_SHAPE;
  const bool sampling = !p.greedy;
  if (!target || !acc || !out || ws_null) return SV_ERR_NULL;
  if (G > 0 && !tokens) return SV_ERR_NULL;
  if (sampling && (!u_sample || (G > 0 && (!draft || !u_accept)))) return SV_ERR_NULL;
  const uintptr_t ta = (uintptr_t)target, da = (uintptr_t)draft;
  if (ta % p.esz || (sampling && G > 0 && da % p.esz)) return SV_ERR_ALIGN;
  return SV_OK;
}

sv_status run(const void *target, const void *draft, sv_dtype dt, const int32_t *tokens,
              const float *u_accept, const float *u_sample, int32_t B, int32_t G, int32_t V,
              float T, int32_t top_k, int32_t *acc, int32_t *out, float *row_stats, void *ws,
              size_t ws_bytes, void *stream, void *const *ev, int32_t nev, int32_t *nl) {
  if (nl) *nl = 0;
  Plan p;
  const sv_status cs = check_args(target, draft, dt, tokens, u_accept, u_sample, B, G, V, T, top_k, acc, out,
                                  ws == nullptr, p);
  if (cs != SV_OK) return cs;
  const bool sampling = !p.greedy;
  const uintptr_t ta = (uintptr_t)target, da = (uintptr_t)draft;
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
  a.ntr = G + 1;
  a.tgt_rows = G + 1;
  a.k2 = sampling ? (float)(LOG2E / (double)T) : 0.0f;
  a.top_k = top_k;
  a.accepted_len = acc;
  a.out_tokens = out;
  a.row_stats = sampling ? row_stats : nullptr;
  a.beta = a.tv = nullptr;
  a.pair_status = nullptr;
  a.lag = 0;
  a.tag = 0u;  // each launch takes its own
  a.spin_limit = SPIN_LIMIT;
  a.stamps = sv_host::g_stamps;
  a.w.tw_part = (u64 *)(base + p.tw_part);
  a.w.tw_job = (u64 *)(base + p.tw_job);
  a.w.tw_seg = (u64 *)(base + p.tw_seg);
  a.w.tw_gseg = (u64 *)(base + p.tw_gseg);
  a.w.tw_hist = (u64 *)(base + p.tw_hist);
  a.w.tw_ov = nullptr;
  a.w.row_tau = (float *)(base + p.row_tau);
  a.w.tk_state = (uint2 *)(base + p.tk_state);
  // after the one-pass top-k threshold: each row's kept-set normaliser and kept list
  const bool one_pass = p.topk && sv_host::topk_one_pass(top_k, p.C);
  a.w.tk_rowp = one_pass ? (uint4 *)(base + p.tk_state + sv_host::topk_rowp_offset(p.R, p.C, top_k)) : nullptr;
  a.w.tk_keep = one_pass ? (uint2 *)(base + p.tk_state + sv_host::topk_keep_offset(p.R, p.C, top_k)) : nullptr;

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

// ---------------------------------------------------------------- allocation-free calls

// The scratch memory of spec_verify_noalloc: one array per GPU, a static device variable
// of the library (held by each GPU the library runs on until the process ends).  Host code
// never passes this name to a kernel or a copy: on the host it is only a stand-in, and the
// device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void k_fill_zero(u64 *p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n_words; i += (size_t)gridDim.x * 256) p[i] = 0ull;
}

struct ScratchState {
  void *ptr = nullptr;   // the device address of this GPU's array
  size_t clean = 0;      // leading bytes known to hold zeros or words of completed calls
  size_t used = 0;       // longest prefix any call has marked since the array was last cleared
  uint32_t epoch = 0;    // tag epoch when that clearing happened
};
constexpr int SCRATCH_MAX_DEVICES = 64;
ScratchState g_scratch[SCRATCH_MAX_DEVICES];
std::mutex g_scratch_mu;

}  // namespace

extern "C" {

int32_t sv_timeline_stamps(void *buf, int32_t *clock_khz) {
#ifdef SV_TIMELINE
  if (clock_khz) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      return 7;
    *clock_khz = khz;
  }
  sv_host::g_stamps = static_cast<unsigned long long *>(buf);
  return 0;
#else
  (void)buf;
  (void)clock_khz;
  return 1;
#endif
}

sv_status spec_verify_noalloc(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                              const int32_t *draft_tokens, const float *u_accept,
                              const float *u_sample, int32_t B, int32_t G, int32_t V,
                              float temperature, int32_t top_k, int32_t *accepted_len,
                              int32_t *out_tokens, float *row_stats, void *stream) {
  Plan p;
  const sv_status cs = check_args(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, B, G,
                                  V, temperature, top_k, accepted_len, out_tokens, false, p);
  if (cs != SV_OK) return cs;
  if (p.total > SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return SV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchState &sc = g_scratch[dev];
  if (!sc.ptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SV_ERR_LAUNCH;
    sc.ptr = ptr;
    sc.clean = sc.used = 0;
    sc.epoch = sv_tag_epoch();
  }
  const uint32_t epoch = sv_tag_epoch();
  size_t need = p.zero_bytes;
  if (epoch != sc.epoch) {  // tags of calls before this epoch may come back: clear every marked word
    need = need > sc.used ? need : sc.used;
    sc.clean = 0;
  }
  if (need > sc.clean) {
    const size_t words = (need + 7) / 8;
    const unsigned grid = (unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024);
    hipLaunchKernelGGL(k_fill_zero, dim3(grid), dim3(256), 0, (hipStream_t)stream, (u64 *)sc.ptr, words);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    sc.clean = need;
    if (epoch != sc.epoch) {
      sc.used = 0;
      sc.epoch = epoch;
    }
  }
  const sv_status st = run(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, B, G, V,
                           temperature, top_k, accepted_len, out_tokens, row_stats, sc.ptr,
                           SV_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0, nullptr);
  if (st == SV_OK) {  // a call leaves its own prefix clean and may overwrite what follows it
    sc.clean = p.zero_bytes;
    sc.used = sc.used > p.zero_bytes ? sc.used : p.zero_bytes;
  }
  return st;
}

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
  if (top_k > 0 && top_k < V) {
    if (sv_host::topk_one_pass(top_k, sv_host::row_chunks(V, dtype == SV_BF16 ? 2 : 4))) return kPlanNames[4];
    return dtype == SV_BF16 ? kPlanNames[0] : kPlanNames[1];
  }
  return kPlanNames[2];
}

uint32_t sv_tag_epoch(void) {
  return (uint32_t)(sv_host::g_launches.load(std::memory_order_relaxed) >> 31);
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
    case SV_ERR_PARAM: return "epsilon and delta must be finite and >= 0";
    case SV_ERR_SCRATCH: return "the arguments need more scratch memory than spec_verify_noalloc holds";
  }
  return "unknown status";
}

}  // extern "C"
