// sv_draw.h -- inverse-CDF draws over one or two logit rows, shared by the kernels that
// draw a token: weight functors, per-segment masses of a chunk, and the pick of lane and
// element inside one 64-vector segment or one chunk ("Speculative Decoding 的朴素思想",
// section "一次 sampling 怎么执行", step 1: the token whose cumulative interval holds u).
#pragma once

#include "sv_common.h"

namespace sv {

// max(0, 1 - 2^d): 0 for d >= 0 and for a NaN d.  Near d = 0 the difference 1 - 2^d
// would cancel, so for -1/2 < d < 0 it is the series of -expm1(y), y = d ln 2, to the
// y^7 term (truncation below 2e-8 relative); further out 2^d <= 0.71 and 1 - 2^d keeps
// full relative precision.
SVD float one_minus_exp2(float d) {
  const float y = d * 0.69314718055994531f;
  float h = 1.0f / 5040.0f;
  h = fmaf(h, y, 1.0f / 720.0f);
  h = fmaf(h, y, 1.0f / 120.0f);
  h = fmaf(h, y, 1.0f / 24.0f);
  h = fmaf(h, y, 1.0f / 6.0f);
  h = fmaf(h, y, 0.5f);
  h = fmaf(h, y, 1.0f);
  const float m = (d > -0.5f) ? -y * h : 1.0f - fast_exp2(d);
  return (d < 0.0f) ? m : 0.0f;
}

// Weights of the correction draw, [p - q]_+ ("Speculative Decoding 的朴素思想", section
// "Correction 为什么用正残差"), formed as p * max(0, 1 - q/p) with p = 2^(z_t*k2 - Mt) and
// log2(q/p) = (z_d - z_t)*k2 - (Md - Mt) taken from the two logits' own difference, so a
// draft close to the target (q ~ p) keeps the weight's relative precision instead of
// losing it to the cancellation of p - q.  Mt is split into a float head and tail so the
// argument of p carries only its own rounding; dm = Md - Mt is rounded once.
struct ResidualW {
  float k2, mt_hi, mt_lo, dm, tau_t, tau_d;
  float off_j;  // row offset of p_j (the zero-residual fallback's reference)
  SVD float operator()(float zt, float zd) const {
    zt = (zt < tau_t) ? -INFINITY : zt;
    zd = (zd < tau_d) ? -INFINITY : zd;
    const float p = fast_exp2(fmaf(zt, k2, -mt_hi) - mt_lo);
    return __fmul_rn(p, one_minus_exp2(fmaf(zd - zt, k2, -dm)));  // never fused into a sum
  }
};

// Weights of a draw from a target row itself (bonus, or the zero-residual fallback):
// the first pass's terms of one chunk, recomputed bit for bit from its offset.
struct TargetW {
  float k2, off, tau;
  SVD float operator()(float zt, float) const {
    zt = (zt < tau) ? -INFINITY : zt;
    return fast_exp2(fmaf(zt, k2, -off));
  }
};

// Segment masses of vectors kbeg..kbeg+NK-1 of chunk c (whole workgroup): weights
// wf(zA, zB) per element (zB = -inf without a second row), a lane mass per vector
// (elements summed in order), and the wave sum of each 64-vector segment into
// s_seg[k*NW + wave].  Loads are issued KG vectors per thread at a time (KG = NK: every
// load in flight at once).
template <typename T, bool ALIGNED, int KG, int NK, bool PAIR, typename WFn>
SVD void chunk_masses(const Args &a, const T *rowA, const T *rowB, int c, int kbeg, const WFn &wf,
                      double *s_seg) {
  constexpr int VEC = Fmt<T>::VEC;
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
#pragma unroll
  for (int kg = 0; kg < NK; kg += KG) {
    const int k0 = kbeg + kg;
    float acc[KG];
    if (ALIGNED) {
      // Raw 16-byte vectors stay packed until their own turn: KG*4 registers per row.
      u32x4 wa[KG], wb[PAIR ? KG : 1];
      const u32x4 *ra = reinterpret_cast<const u32x4 *>(rowA);
      const u32x4 *rb = reinterpret_cast<const u32x4 *>(rowB);
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        const int v = c * CHUNK_VECS + (k0 + k) * NT + tid;
        const int vs = v < a.nvec ? v : a.nvec - 1;
        wa[k] = ra[vs];
        if (PAIR) wb[PAIR ? k : 0] = rb[vs];
      }
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        const bool in = c * CHUNK_VECS + (k0 + k) * NT + tid < a.nvec;
        float xa[VEC], xb[VEC];
        Fmt<T>::unpack(wa[k], xa);
        if (PAIR) Fmt<T>::unpack(wb[PAIR ? k : 0], xb);
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) m += wf(in ? xa[e] : -INFINITY, (PAIR && in) ? xb[e] : -INFINITY);
        acc[k] = m;
      }
    } else {
      float xa[KG][VEC], xb[PAIR ? KG : 1][VEC];
      load_vectors<T, ALIGNED, false, KG>(rowA, a.V, a.nvec, c, k0, tid, xa);
      if (PAIR) load_vectors<T, ALIGNED, false, PAIR ? KG : 1>(rowB, a.V, a.nvec, c, k0, tid, xb);
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) m += wf(xa[k][e], PAIR ? xb[PAIR ? k : 0][e] : -INFINITY);
        acc[k] = m;
      }
    }
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const double seg = wave_sum((double)acc[k]);
      if (lane == 0) s_seg[(k0 + k) * NW + wid] = seg;
    }
  }
  __syncthreads();
}

// Inverse CDF inside segment s of chunk c, by one wave: each lane re-reads its vector of
// the segment (rows A and B), recomputes the element weights and its lane mass exactly
// as chunk_masses did, then picks lane and element.  With t = +inf the last positive
// element is taken.  Returns the element index in the row (same in every lane), or -1.
template <typename T, bool ALIGNED, typename WFn>
SVD int segment_draw(const Args &a, const T *rowA, const T *rowB, int c, int s, const WFn &wf,
                     double t) {
  constexpr int VEC = Fmt<T>::VEC;
  const int lane = lane_id();
  const int k = s / NW, w = s % NW;
  const int tid_equiv = w * WAVE + lane;  // the thread that held this vector
  float xa[VEC], xb[VEC];
  if (ALIGNED) {  // one 16-byte vector per row
    const int v = c * CHUNK_VECS + k * NT + tid_equiv;
    const bool in = v < a.nvec;
    const int vs = in ? v : a.nvec - 1;
    Fmt<T>::unpack(reinterpret_cast<const u32x4 *>(rowA)[vs], xa);
    if (rowB) Fmt<T>::unpack(reinterpret_cast<const u32x4 *>(rowB)[vs], xb);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      xa[e] = in ? xa[e] : -INFINITY;
      xb[e] = (in && rowB) ? xb[e] : -INFINITY;
    }
  } else {  // the same vector of a row that is not 16-byte aligned (see load_pair)
    const int v = c * CHUNK_VECS + k * NT + tid_equiv;
    const int vs = v < a.nvec ? v : a.nvec - 1;
    u32x4 la, ha, lb, hb;
    load_pair<T, false>(rowA, rowA + a.V, row_off16(rowA), vs, la, ha);
    if (rowB) load_pair<T, false>(rowB, rowB + a.V, row_off16(rowB), vs, lb, hb);
    Fmt<T>::unpack(funnel16(la, ha, row_off16(rowA)), xa);
    if (rowB) Fmt<T>::unpack(funnel16(lb, hb, row_off16(rowB)), xb);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const bool in = elem_index<T>(c, k, tid_equiv, e) < a.V;
      xa[e] = in ? xa[e] : -INFINITY;
      xb[e] = (in && rowB) ? xb[e] : -INFINITY;
    }
  }
  float we[VEC];
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    we[e] = wf(xa[e], xb[e]);
    acc += we[e];
  }
  auto lanem = [&](int) { return (double)acc; };
  double lrem;
  const int pl = wave_pick(WAVE, t, lanem, &lrem);
  int res = -1;
  if (lane == pl) {
    int pe = -1, lastpe = -1;
    double run = 0.0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (we[e] > 0.0f) lastpe = e;
      run += (double)we[e];
      if (pe < 0 && we[e] > 0.0f && run > lrem) pe = e;
    }
    if (pe < 0) pe = lastpe;
    res = (pe < 0) ? -1 : (int)elem_index<T>(c, k, tid_equiv, pe);
  }
  return __builtin_amdgcn_readlane(res, pl < 0 ? 0 : pl);
}

// Whole-chunk inverse CDF by one wave (rare path: the zero-residual fallback, after
// the other waves of the workgroup have finished): segment masses one segment at a
// time, then segment_draw.
template <typename T, bool ALIGNED, typename WFn>
SVD int wave_chunk_draw(const Args &a, const T *rowA, const T *rowB, int c, const WFn &wf,
                        double t) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ double s_wseg[SEGS];
  const int lane = lane_id();
  for (int sg = 0; sg < SEGS; ++sg) {
    const int k = sg / NW, w = sg % NW;
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const long idx = elem_index<T>(c, k, w * WAVE + lane, e);
      const bool in = idx < a.V;
      const size_t ii = (size_t)(in ? idx : (long)a.V - 1);
      const float za = in ? Fmt<T>::at(rowA, ii) : -INFINITY;
      const float zb = (in && rowB) ? Fmt<T>::at(rowB, ii) : -INFINITY;
      acc += wf(za, zb);
    }
    const double m = wave_sum((double)acc);
    if (lane == 0) s_wseg[sg] = m;
  }
  lds_sync();
  auto segm = [&](int i) { return s_wseg[i]; };
  double srem;
  const int sp = wave_pick(SEGS, t, segm, &srem);
  if (sp < 0) return -1;
  return segment_draw<T, ALIGNED>(a, rowA, rowB, c, sp, wf, srem);
}

}  // namespace sv
