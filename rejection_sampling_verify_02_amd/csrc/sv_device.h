// sv_device.h -- device building blocks shared by the library's HIP kernels (gfx950):
// chunk geometry and loads, wave64 DPP scans and reductions, tagged-word hand-off
// between workgroups, inverse-CDF picks by one wave, and XCD-lane block placement.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_lanes.h"

#define SVD __device__ __forceinline__

namespace sv {

constexpr int NT = 256;                // threads per workgroup
constexpr int WAVE = 64;               // gfx950 wavefront
constexpr int NW = NT / WAVE;          // waves per workgroup
constexpr int VPT = 8;                 // 16-byte vectors per thread per chunk
constexpr int CHUNK_VECS = NT * VPT;   // vectors per chunk (32 KiB of logits)
constexpr int SEGS = VPT * NW;         // 64-vector segments per chunk
constexpr unsigned SPIN_LIMIT = 1u << 20;  // polls before a waiting wave gives up (~a second)
constexpr double LN2 = 0.69314718055994530942;
constexpr double LOG2E = 1.44269504088896340736;


typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- element formats

template <typename T>
struct Fmt;

template <>
struct Fmt<uint16_t> {  // bf16 bit patterns: the upper half of an IEEE binary32
  static constexpr int VEC = 8;
  SVD static float at(const uint16_t *p, size_t i) { return __uint_as_float((uint32_t)p[i] << 16); }
  SVD static void unpack(u32x4 w, float (&o)[8]) {
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
  SVD static void unpack(u32x4 w, float (&o)[4]) {
    o[0] = __uint_as_float(w.x);
    o[1] = __uint_as_float(w.y);
    o[2] = __uint_as_float(w.z);
    o[3] = __uint_as_float(w.w);
  }
};

// Rows that do not start on a 16-byte boundary (a bf16 row of odd length, say) are read
// with the same 16-byte loads: row vector v (row elements v*VEC .. v*VEC + VEC - 1) spans
// at most two aligned 16-byte blocks, and its offset inside the first, off, is the same
// for every vector of the row (the row pointer's own offset).  Both blocks are loaded and
// the vector's 16 bytes taken out of the pair: dword shifts by selects on off's bits, then
// one v_alignbyte per dword.  The second block is loaded only when it holds a byte of the
// row (else the first is loaded twice; its bytes then lie past the row's end and are
// masked by the caller), so every load touches a block that holds row data.
SVD u32x4 funnel16(const u32x4 &lo, const u32x4 &hi, unsigned off) {
  const bool s2 = (off & 8u) != 0, s1 = (off & 4u) != 0;
  const unsigned b = off & 3u;
  const unsigned q0 = s2 ? lo.z : lo.x, q1 = s2 ? lo.w : lo.y, q2 = s2 ? hi.x : lo.z, q3 = s2 ? hi.y : lo.w,
                 q4 = s2 ? hi.z : hi.x, q5 = s2 ? hi.w : hi.y;
  const unsigned r0 = s1 ? q1 : q0, r1 = s1 ? q2 : q1, r2 = s1 ? q3 : q2, r3 = s1 ? q4 : q3, r4 = s1 ? q5 : q4;
  return u32x4{__builtin_amdgcn_alignbyte(r1, r0, b), __builtin_amdgcn_alignbyte(r2, r1, b),
               __builtin_amdgcn_alignbyte(r3, r2, b), __builtin_amdgcn_alignbyte(r4, r3, b)};
}
// The two blocks of row vector v (v < the row's vector count), loads issued, not waited for.
template <typename T, bool STREAM>
SVD void load_pair(const T *row, const T *row_end, unsigned off, int v, u32x4 &lo, u32x4 &hi) {
  const char *a = reinterpret_cast<const char *>(row + (size_t)v * Fmt<T>::VEC);
  const u32x4 *p0 = reinterpret_cast<const u32x4 *>(a - off);
  const u32x4 *p1 = (reinterpret_cast<const char *>(p0 + 1) < reinterpret_cast<const char *>(row_end)) ? p0 + 1 : p0;
  lo = STREAM ? __builtin_nontemporal_load(p0) : *p0;
  hi = STREAM ? __builtin_nontemporal_load(p1) : *p1;
}
template <typename T>
SVD unsigned row_off16(const T *row) { return (unsigned)(reinterpret_cast<uintptr_t>(row) & 15u); }

// Vector k of this thread in chunk c is vector c*CHUNK_VECS + k*NT + tid of the row, so
// one wave's k-th load covers 64 consecutive vectors (a "segment") and segments are in
// vocabulary order (k-major, then wave).  Elements past the row end read as -inf.
// Every load is issued before any is used: past the end a load re-reads the row's last
// vector, and the tail is masked afterwards by a uniform branch.  `mid` runs after the
// loads are issued and before any is waited for, so that loads it issues are in flight
// with the chunk's.
struct NoMid {
  SVD void operator()() const {}
};
template <typename T, bool ALIGNED, bool STREAM, typename Mid = NoMid>
SVD void load_chunk(const T *row, int V, int nvec, int c, int tid, float (&x)[VPT][Fmt<T>::VEC], Mid mid = {}) {
  constexpr int VEC = Fmt<T>::VEC;
  if (ALIGNED) {
    u32x4 w[VPT];
    const u32x4 *rv = reinterpret_cast<const u32x4 *>(row);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = c * CHUNK_VECS + k * NT + tid;
      const u32x4 *p = rv + (v < nvec ? v : nvec - 1);
      w[k] = STREAM ? __builtin_nontemporal_load(p) : *p;
    }
    mid();
#pragma unroll
    for (int k = 0; k < VPT; ++k) Fmt<T>::unpack(w[k], x[k]);
    if ((c + 1) * CHUNK_VECS > nvec) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const bool in = c * CHUNK_VECS + k * NT + tid < nvec;
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[k][e] = in ? x[k][e] : -INFINITY;
      }
    }
  } else {
    const unsigned off = row_off16(row);
    const T *row_end = row + V;
    u32x4 lo[VPT], hi[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = c * CHUNK_VECS + k * NT + tid;
      load_pair<T, STREAM>(row, row_end, off, v < nvec ? v : nvec - 1, lo[k], hi[k]);
    }
    mid();
#pragma unroll
    for (int k = 0; k < VPT; ++k) Fmt<T>::unpack(funnel16(lo[k], hi[k], off), x[k]);
    if ((long)(c + 1) * CHUNK_VECS * VEC > V) {  // the row's end: elements past it read as -inf
#pragma unroll
      for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          x[k][e] = (((long)c * CHUNK_VECS + (long)k * NT + tid) * VEC + e < V) ? x[k][e] : -INFINITY;
    }
  }
}

// Vectors k0..k0+NK-1 of this thread in chunk c, as load_chunk does for all VPT of them.
template <typename T, bool ALIGNED, bool STREAM, int NK>
SVD void load_vectors(const T *row, int V, int nvec, int c, int k0, int tid,
                      float (&x)[NK][Fmt<T>::VEC]) {
  constexpr int VEC = Fmt<T>::VEC;
  if (ALIGNED) {
    u32x4 w[NK];
    const u32x4 *rv = reinterpret_cast<const u32x4 *>(row);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int v = c * CHUNK_VECS + (k0 + k) * NT + tid;
      const u32x4 *p = rv + (v < nvec ? v : nvec - 1);
      w[k] = STREAM ? __builtin_nontemporal_load(p) : *p;
    }
#pragma unroll
    for (int k = 0; k < NK; ++k) Fmt<T>::unpack(w[k], x[k]);
    if ((c + 1) * CHUNK_VECS > nvec) {
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const bool in = c * CHUNK_VECS + (k0 + k) * NT + tid < nvec;
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[k][e] = in ? x[k][e] : -INFINITY;
      }
    }
  } else {
    const unsigned off = row_off16(row);
    const T *row_end = row + V;
    u32x4 lo[NK], hi[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int v = c * CHUNK_VECS + (k0 + k) * NT + tid;
      load_pair<T, STREAM>(row, row_end, off, v < nvec ? v : nvec - 1, lo[k], hi[k]);
    }
#pragma unroll
    for (int k = 0; k < NK; ++k) Fmt<T>::unpack(funnel16(lo[k], hi[k], off), x[k]);
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        x[k][e] = (((long)c * CHUNK_VECS + (long)(k0 + k) * NT + tid) * VEC + e < V) ? x[k][e] : -INFINITY;
  }
}

// Index of element (k, e) of this thread in chunk c.
template <typename T>
SVD long elem_index(int c, int k, int tid, int e) {
  return ((long)c * CHUNK_VECS + (long)k * NT + tid) * Fmt<T>::VEC + e;
}

typedef unsigned long long u64;


// ---------------------------------------------------------------- small helpers

SVD float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32; 0 for x < -126
SVD int lane_id() { return (int)(threadIdx.x & (WAVE - 1)); }

// This wave's LDS writes are complete before any of its lanes reads them.  Only the LDS
// counter is waited for: outstanding global stores (published results) keep going.
SVD void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt left at their maxima
  __builtin_amdgcn_wave_barrier();
}

// (off, s) pairs stand for s * 2^off; combining keeps the larger offset.  Parts that
// hold only -inf have off = -inf and s = 0 (or NaN when a NaN was seen); the rule never
// forms (-inf) - (-inf).  The combine is commutative bit for bit.
SVD void lse_combine(float &off, double &s, float off2, double s2) {
  const float mx = fmaxf(off, off2);
  const double w1 = (off == mx) ? 1.0 : (double)fast_exp2(off - mx);
  const double w2 = (off2 == mx) ? 1.0 : (double)fast_exp2(off2 - mx);
  s = s * w1 + s2 * w2;
  off = mx;
}

// ---- cross-lane primitives (DPP) ----
// Wave-wide scans and reductions use DPP lane moves (row_shr within 16-lane rows, then
// row_bcast:15 / row_bcast:31 across rows) instead of LDS-routed shuffles: each step is
// one VALU move.  A move leaves `id` in lanes that have no source, so every scan below
// is an inclusive scan with identity id; a reduction is the scan's lane 63 read back.
template <int CTRL, int ROWM>
SVD unsigned dpp_u(unsigned v, unsigned id) {
  return (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWM, 0xf, false);
}
template <int CTRL, int ROWM>
SVD float dpp_f(float v, float id) { return __uint_as_float(dpp_u<CTRL, ROWM>(__float_as_uint(v), __float_as_uint(id))); }
template <int CTRL, int ROWM>
SVD double dpp_d(double v, double id) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned long long ib = (unsigned long long)__double_as_longlong(id);
  const unsigned lo = dpp_u<CTRL, ROWM>((unsigned)b, (unsigned)ib);
  const unsigned hi = dpp_u<CTRL, ROWM>((unsigned)(b >> 32), (unsigned)(ib >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
template <int CTRL, int ROWM>
SVD int dpp_i(int v, int id) { return (int)dpp_u<CTRL, ROWM>((unsigned)v, (unsigned)id); }

// The six steps of a 64-lane inclusive scan; STEP(ctrl, rowmask) applies one lane move.
#define SV_SCAN_STEPS(STEP) \
  STEP(0x111, 0xf) /* row_shr:1 */ \
  STEP(0x112, 0xf) /* row_shr:2 */ \
  STEP(0x114, 0xf) /* row_shr:4 */ \
  STEP(0x118, 0xf) /* row_shr:8 */ \
  STEP(0x142, 0xa) /* row_bcast:15 into rows 1 and 3 */ \
  STEP(0x143, 0xc) /* row_bcast:31 into rows 2 and 3 */

SVD double scan_sum(double x) {
#define STEP(C, R) x += dpp_d<C, R>(x, 0.0);
  SV_SCAN_STEPS(STEP)
#undef STEP
  return x;
}
SVD float scan_max(float x) {
#define STEP(C, R) x = fmaxf(x, dpp_f<C, R>(x, -INFINITY));
  SV_SCAN_STEPS(STEP)
#undef STEP
  return x;
}
SVD unsigned scan_or(unsigned x) {
#define STEP(C, R) x |= dpp_u<C, R>(x, 0u);
  SV_SCAN_STEPS(STEP)
#undef STEP
  return x;
}

SVD double readlane_d(double v, int l) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
SVD float readlane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

SVD double wave_sum(double v) { return readlane_d(scan_sum(v), WAVE - 1); }
SVD float wave_max(float v) { return readlane_f(scan_max(v), WAVE - 1); }
SVD unsigned wave_or(unsigned v) { return (unsigned)__builtin_amdgcn_readlane((int)scan_or(v), WAVE - 1); }

// (off, s) pairs over the wave, combined with lse_combine (identity (-inf, 0)).
SVD void wave_lse(float &off, double &s) {
#define STEP(C, R)                                  \
  {                                                 \
    const float o2 = dpp_f<C, R>(off, -INFINITY);   \
    const double s2 = dpp_d<C, R>(s, 0.0);          \
    lse_combine(off, s, o2, s2);                    \
  }
  SV_SCAN_STEPS(STEP)
#undef STEP
  off = readlane_f(off, WAVE - 1);
  s = readlane_d(s, WAVE - 1);
}

// Results that one workgroup hands to another inside a kernel are written and read with
// device-scope (agent) atomic stores and loads: on gfx950 these are ordinary vector
// memory instructions with the device scope bit set, so they are complete device-wide
// (across the XCDs' separate L2s) when the store counter drains, and the loads observe
// them.  This avoids the whole-L2 write-back that a device-scope release fence costs.
template <typename T>
SVD void st_dev(T *p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
SVD T ld_dev(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tagged words.  Inside the sampling kernel every value one workgroup hands to another
// travels as a 64-bit word (call tag << 32 | 32-bit payload) written and read with one
// device-scope 64-bit store / load, which is single-copy atomic.  A reader takes a word
// as present when it carries this call's tag: no fence, store wait or counter is needed,
// and a record is complete once all of its words carry the tag.  A double travels as a
// float head and tail (d ~ head + tail to 2^-48).  The only waits are polls of words
// written by workgroups that come earlier in the grid.
SVD void tw_put(u64 *p, unsigned tag, unsigned bits) { st_dev(p, ((u64)tag << 32) | (u64)bits); }
SVD void tw_putf(u64 *p, unsigned tag, float f) { tw_put(p, tag, __float_as_uint(f)); }
SVD bool tw_ok(u64 w, unsigned tag) { return (unsigned)(w >> 32) == tag; }
SVD float tw_f(u64 w) { return __uint_as_float((unsigned)w); }
SVD float d_head(double d) { return (float)d; }
SVD float d_tail(double d) { return (float)(d - (double)(float)d); }
SVD double d_join(float hi, float lo) { return (double)hi + (double)lo; }

// Order-preserving 32-bit key of a float (bf16 values are floats with zero low half);
// -0 and +0 share a key.
SVD uint32_t f2key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
SVD float key2f(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }

// Inverse CDF over n ordered items, by one whole wave: masses come from mfn(i); the
// prefix runs in index order (groups of 64 lanes, inclusive scan, carried), so the same
// masses always give the same total and prefixes.  wave_total returns the total;
// wave_pick returns the first item whose inclusive prefix exceeds t and, in *t_rem,
// t minus the prefix before it.  When rounding leaves t at or past the total it returns
// the last item with positive mass and *t_rem = +inf (which makes the finer levels take
// their last positive entry too).  -1 if no item has positive mass.
template <typename MFn>
SVD double wave_scan_group(int n, int i0, const MFn &mfn, double carry, double &m, double &cum) {
  const int i = i0 + lane_id();
  m = (i < n) ? mfn(i) : 0.0;
  cum = scan_sum(m) + carry;
  return readlane_d(cum, WAVE - 1);
}

template <typename MFn>
SVD double wave_total(int n, const MFn &mfn) {
  double carry = 0.0, m, cum;
  for (int i0 = 0; i0 < n; i0 += WAVE) carry = wave_scan_group(n, i0, mfn, carry, m, cum);
  return carry;
}

template <typename MFn>
SVD int wave_pick(int n, double t, const MFn &mfn, double *t_rem) {
  double carry = 0.0, m, cum;
  int pick = -1, lastpos = -1;
  double trem = INFINITY;
  for (int i0 = 0; i0 < n; i0 += WAVE) {
    const double carry_in = carry;
    carry = wave_scan_group(n, i0, mfn, carry, m, cum);
    const unsigned long long pos = __ballot(m > 0.0);
    if (pos) lastpos = i0 + 63 - __clzll((long long)pos);
    if (pick < 0) {
      const unsigned long long cr = __ballot(m > 0.0 && cum > t);
      if (cr) {
        const int l = __ffsll((long long)cr) - 1;
        const double prev = (l == 0) ? carry_in : readlane_d(cum, l - 1);
        pick = i0 + l;
        trem = t - prev;
      }
    }
  }
  if (pick < 0) {
    pick = lastpos;
    trem = INFINITY;
  }
  *t_rem = trem;
  return pick;
}

// wave_pick with t = u * (total of the same masses): for n <= 64 one scan gives both.
template <typename MFn>
SVD int wave_pick_frac(int n, double u, const MFn &mfn, double *t_rem, double *total) {
  if (n > WAVE) {
    *total = wave_total(n, mfn);
    return wave_pick(n, u * *total, mfn, t_rem);
  }
  const int i = lane_id();
  const double m = (i < n) ? mfn(i) : 0.0;
  const double cum = scan_sum(m);
  const double tot = readlane_d(cum, WAVE - 1);
  const double t = u * tot;
  *total = tot;
  const unsigned long long pos = __ballot(m > 0.0);
  const unsigned long long cr = __ballot(m > 0.0 && cum > t);
  if (cr) {
    const int l = __ffsll((long long)cr) - 1;
    const double prev = (l == 0) ? 0.0 : readlane_d(cum, l - 1);
    *t_rem = t - prev;
    return l;
  }
  *t_rem = INFINITY;
  return pos ? 63 - __clzll((long long)pos) : -1;
}

// Inverse CDF over n masses in index order, four consecutive ones per lane in blocks of
// 256: lane sums (in order), one scan per block.  t = u * total; returns the first index
// whose prefix exceeds t and, in *t_rem, t minus the prefix before it; when rounding
// leaves t at or past the total, the last positive index and +inf; -1 if nothing is
// positive.  A single block reads its masses once.
template <typename MFn>
SVD int wave_pick4_frac(int n, double u, const MFn &mfn, double *t_rem, double *total) {
  constexpr int SB = 4, BLK = SB * WAVE;
  const int lane = lane_id();
  double m[SB];
  auto lane_masses = [&](int b0) {
    double ls = 0.0;
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      const int i = b0 + lane * SB + k;
      m[k] = (i < n) ? mfn(i) : 0.0;
    }
#pragma unroll
    for (int k = 0; k < SB; ++k) ls += m[k];
    return ls;
  };
  // The lane that holds the crossing picks its element; the result is broadcast.
  auto in_lane = [&](int b0, int l, double rem, double *t_out) {
    int pk = -1, last = -1;
    double run = 0.0, r_out = INFINITY;
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      if (m[k] > 0.0) last = k;
      if (pk < 0 && m[k] > 0.0 && run + m[k] > rem) {
        pk = k;
        r_out = rem - run;
      }
      run += m[k];
    }
    if (pk < 0) pk = last;
    const int idx = (pk < 0) ? -1 : b0 + lane * SB + pk;
    *t_out = readlane_d(r_out, l);
    return __builtin_amdgcn_readlane(idx, l);
  };
  if (n <= BLK) {
    const double ls = lane_masses(0);
    const double cum = scan_sum(ls);
    *total = readlane_d(cum, WAVE - 1);
    const double t = u * *total;
    const unsigned long long cr = __ballot(ls > 0.0 && cum > t);
    const unsigned long long pos = __ballot(ls > 0.0);
    if (cr) {
      const int l = __ffsll((long long)cr) - 1;
      const double prev = (l == 0) ? 0.0 : readlane_d(cum, l - 1);
      return in_lane(0, l, t - prev, t_rem);
    }
    if (!pos) return -1;
    const int l = 63 - __clzll((long long)pos);
    return in_lane(0, l, INFINITY, t_rem);
  }
  double carry = 0.0;
  for (int b0 = 0; b0 < n; b0 += BLK) carry += readlane_d(scan_sum(lane_masses(b0)), WAVE - 1);
  *total = carry;
  const double t = u * carry;
  double c2 = 0.0;
  int lb = -1, ll = -1;
  for (int b0 = 0; b0 < n; b0 += BLK) {
    const double ls = lane_masses(b0);
    const double cum = scan_sum(ls) + c2;
    const unsigned long long pos = __ballot(ls > 0.0);
    if (pos) {
      lb = b0;
      ll = 63 - __clzll((long long)pos);
    }
    const unsigned long long cr = __ballot(ls > 0.0 && cum > t);
    if (cr) {
      const int l = __ffsll((long long)cr) - 1;
      const double prev = (l == 0) ? c2 : readlane_d(cum, l - 1);
      return in_lane(b0, l, t - prev, t_rem);
    }
    c2 = readlane_d(cum, WAVE - 1);
  }
  if (lb < 0) return -1;
  lane_masses(lb);
  return in_lane(lb, ll, INFINITY, t_rem);
}

// ---------------------------------------------------------------- block placement

// Block p's item of the grid (see sv_lanes.h for the placement and why).
SVD bool lane_item(int units, int per1, int per2, int &phase, int &item) {
  return lane_decode((int)blockIdx.x, units, per1, per2, phase, item);
}

SVD bool lane_item_lag(int units, int per1, int per2, int lag, int &phase, int &unit, int &sub) {
  return lane_decode_lag((int)blockIdx.x, units, per1, per2, lag, phase, unit, sub);
}

// Largest value wins, ties go to the lower index; NaN and +inf mark the row unusable.
SVD void best_combine(float &v, int &i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

SVD void wave_best(float &v, int &i, int &fl) {
#define STEP(C, R)                                   \
  {                                                  \
    const float v2 = dpp_f<C, R>(v, -INFINITY);      \
    const int i2 = dpp_i<C, R>(i, 0x7fffffff);       \
    fl |= dpp_i<C, R>(fl, 0);                        \
    best_combine(v, i, v2, i2);                      \
  }
  SV_SCAN_STEPS(STEP)
#undef STEP
  v = readlane_f(v, WAVE - 1);
  i = __builtin_amdgcn_readlane(i, WAVE - 1);
  fl = __builtin_amdgcn_readlane(fl, WAVE - 1);
}


}  // namespace sv
