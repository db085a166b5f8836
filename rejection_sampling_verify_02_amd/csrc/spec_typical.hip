// spec_typical.hip -- Medusa's typical acceptance, for MI355X (gfx950).
//
// What is computed ("Speculative Decoding 的朴素思想", section "Medusa-1 与 typical
// acceptance"): drafted token x_i is accepted when p_i(x_i) > min(eps, delta *
// exp(-H(p_i))), with H the entropy (natural log) of the target's distribution p_i after
// temperature and top-k; the accepted prefix is the longest run of accepted positions,
// and the token after it is the target's greedy choice argmax p_{j+1} (the next
// candidate's first token, taken greedily and accepted directly).  No uniform and no
// draft distribution is read.  The rule is not distribution-preserving.
//
// One kernel (after the top-k radix select, when top-k is on).  Per chunk of every target
// row: block max m and argmax, off = m*k2, S = sum e and M = sum e*t over the chunk with
// t = fma(z, k2, -off) and e = 2^t (one v_exp_f32 per logit), published as tagged words
// (the last row, which only gives the greedy next token, publishes its argmax and validity
// alone).
// The sequence's last item combines each row's chunks: the log2-partition
// L = o + log2(sum_c S_c 2^(off_c - o)) and, from the same sums, the entropy
//   H = ln2 * (log2 t - D),  D = sum_c 2^(off_c - o) (M_c + (off_c - o) S_c) / t,
// which is ln2 * (L - E_p[z*k2]) written around o so that nothing large cancels; then it
// tests the positions in fp64: ln p(x) = ln2 * (z_x*k2 - L) against
// min(ln eps, ln delta - H).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_common.h"

namespace sv {

constexpr int TYP_WORDS = 8;         // per chunk: off, S hi/lo, M hi/lo, best value, index, flags
constexpr int TYP_MAX_ROWS = 257;    // rows of one sequence (G <= 256)
constexpr int TYP_LDS_PARTS = 768;   // (row, chunk) partials of one sequence staged in LDS

// The chunks' (largest value, its lowest index) pairs as one key whose maximum is the
// row's: the value's bits in an order-preserving form (-0 taken as +0, which compares
// equal to it; NaN lowest, which never wins), then the complemented index, so that of
// equal values the lower index wins.  A max over keys has no branch.
SVD u64 best_key(float v, int i) {
  const float c = v + 0.0f;
  const unsigned u = __float_as_uint(c);
  const unsigned ord = (c != c) ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
  return ((u64)ord << 32) | (u64)(0xffffffffu - (unsigned)i);
}

// Lowest value over the wave.
SVD int wave_min_i(int v) {
#define STEP(C, R) v = min(v, dpp_i<C, R>(v, 0x7fffffff));
  SV_SCAN_STEPS(STEP)
#undef STEP
  return __builtin_amdgcn_readlane(v, WAVE - 1);
}

struct TypArgs {
  Args a;           // rps = G + 1 target rows per sequence (ntr = tgt_rows = G + 1)
  double ln_eps;    // log(eps) (-inf for eps = 0)
  double ln_delta;  // log(delta)
};

// The sequence's last item: combine, test, write.  One wave; lane f < TYP_WORDS holds
// word f of this item's own partial in own_v (a value per lane, so the partial never
// needs an addressable array, which would live in scratch memory); lane i < G holds
// position i's token in gx and its logit in gz (NaN for a token outside [0, V)).
template <typename T, bool TOPK>
SVD void typical_finish(const TypArgs &ta, int b, float own_v, int own_c, int gx, float gz) {
  const Args &a = ta.a;
  const int lane = lane_id();
  const int G = a.G, rps = a.rps, C = a.C;
  const size_t r0 = (size_t)b * rps;
  const u64 *pw = a.w.tw_part + r0 * C * TYP_WORDS;
  const int own = (rps - 1) * C + own_c;
  __shared__ double s_l2[TYP_MAX_ROWS], s_h[TYP_MAX_ROWS];
  __shared__ int s_arg[TYP_MAX_ROWS], s_ok[TYP_MAX_ROWS];
  __shared__ __align__(16) float s_w[TYP_LDS_PARTS * TYP_WORDS];
  __shared__ float s_own[TYP_WORDS];
  __shared__ float s_o[TYP_MAX_ROWS];
  const bool lds = rps * C <= TYP_LDS_PARTS;
  if (lane < TYP_WORDS) s_own[lane] = own_v;

  // Wait for every partial of the sequence, all lanes loading at once; they are kept in
  // LDS as they arrive (when they fit), so the combine below reads no global memory.
  bool done = false;
  for (unsigned polls = 0; polls < a.spin_limit && !done; ++polls) {
    bool mine = true;
    for (int i = lane; i < rps * C; i += WAVE) {
      if (i == own) continue;
      u64 w[TYP_WORDS];
#pragma unroll
      for (int f = 0; f < TYP_WORDS; ++f) w[f] = ld_dev(pw + (size_t)i * TYP_WORDS + f);
      bool okw = true;
#pragma unroll
      for (int f = 0; f < TYP_WORDS; ++f) okw = okw && tw_ok(w[f], a.tag);
      mine = mine && okw;
      if (okw && lds) {
#pragma unroll
        for (int f = 0; f < TYP_WORDS; ++f) s_w[i * TYP_WORDS + f] = tw_f(w[f]);
      }
    }
    done = wave_or(mine ? 0u : 1u) == 0u;
    if (!done) __builtin_amdgcn_s_sleep(2);
  }
  if (lds && lane < TYP_WORDS) s_w[own * TYP_WORDS + lane] = own_v;
  lds_sync();
  int32_t *out = a.out_tokens + (size_t)b * (G + 1);
  if (!done) {
    for (int i = lane; i <= G; i += WAVE) out[i] = -1;
    if (lane == 0) a.accepted_len[b] = SV_ROW_INTERNAL;
    return;
  }
  // A chunk's two terms for its row's sums, S 2^(off - o) and (M + (off - o) S) 2^(off - o),
  // as +0.0 for an empty chunk (S = 0, whose offset may be -inf like o).
  auto terms = [&](float off, float o, double S, double M, double &ts, double &td) {
    const bool use = S > 0.0 || S != S;
    const double e = (double)fast_exp2(off - o);
    ts = use ? S * e : 0.0;
    td = use ? (M + ((double)off - (double)o) * S) * e : 0.0;
  };
  if (lds) {
    // The combine in three steps, so that the exponentials of all chunks run in parallel
    // lanes: (1) lanes over rows, each row's largest offset; (2) lanes over chunks, each
    // chunk's two terms, written over its first four words; (3) lanes over rows, the sums
    // in chunk order.
    const float4 *q = reinterpret_cast<const float4 *>(s_w);
    for (int r = lane; r < rps; r += WAVE) {
      float o = -INFINITY;
#pragma unroll 8
      for (int c = 0; c < C; ++c) o = fmaxf(o, q[2 * (r * C + c)].x);
      s_o[r] = o;
    }
    lds_sync();
    for (int i = lane; i < rps * C; i += WAVE) {
      const float4 u = q[2 * i];
      const float m_lo = s_w[i * TYP_WORDS + 4];
      double ts, td;
      terms(u.x, s_o[i / C], d_join(u.y, u.z), d_join(u.w, m_lo), ts, td);
      reinterpret_cast<double2 *>(s_w)[2 * i] = make_double2(ts, td);
    }
    lds_sync();
  }
  // per row (lanes over rows): chunks in order
  for (int r = lane; r < rps; r += WAVE) {
    float o = -INFINITY;
    double t = 0.0, dn = 0.0;
    u64 bkey = best_key(-INFINITY, 0x7fffffff);
    int fl = 0;
    if (lds) {
      o = s_o[r];
      const double2 *qd = reinterpret_cast<const double2 *>(s_w) + (size_t)r * C * 2;
      const float4 *q = reinterpret_cast<const float4 *>(s_w) + (size_t)r * C * 2;
#pragma unroll 4
      for (int c = 0; c < C; ++c) {
        const double2 d = qd[2 * c];
        const float4 v = q[2 * c + 1];
        t += d.x;
        dn += d.y;
        bkey = max(bkey, best_key(v.y, (int)__float_as_uint(v.z)));
        fl |= (int)__float_as_uint(v.w);
      }
    } else {
      auto word = [&](int i, int f) -> float {
        return i == own ? s_own[f] : tw_f(ld_dev(pw + (size_t)i * TYP_WORDS + f));
      };
      for (int c = 0; c < C; ++c) o = fmaxf(o, word(r * C + c, 0));
      for (int c = 0; c < C; ++c) {
        const int i = r * C + c;
        double ts, td;
        terms(word(i, 0), o, d_join(word(i, 1), word(i, 2)), d_join(word(i, 3), word(i, 4)), ts, td);
        t += ts;
        dn += td;
        bkey = max(bkey, best_key(word(i, 5), (int)__float_as_uint(word(i, 6))));
        fl |= (int)__float_as_uint(word(i, 7));
      }
    }
    const bool ok = isfinite(o) && isfinite(t) && t > 0.0 && !(fl & 1) && (fl & 2);
    const double l2t = ok ? log2(t) : 0.0;
    s_l2[r] = (double)o + l2t;
    s_h[r] = ok ? LN2 * (l2t - dn / t) : 0.0;
    s_arg[r] = (int)(0xffffffffu - (unsigned)bkey);
    s_ok[r] = ok ? 1 : 0;
  }
  lds_sync();

  const int32_t *xt = a.tokens + (size_t)b * G;
  const T *rows = static_cast<const T *>(a.target) + r0 * (size_t)a.V;
  unsigned flags = 0;  // 1 token, 2 row, 16 internal
  for (int r = lane; r < rps; r += WAVE) {
    if (!s_ok[r]) flags |= 2;
    if (TOPK) {
      const float tau = a.w.row_tau[r0 + r];
      if (tau != tau) flags |= 16;
    }
  }
  int j = G;
  for (int i0 = 0; i0 < G; i0 += WAVE) {
    const int i = i0 + lane;
    bool accept = false;
    if (i < G) {
      const int x = (i0 == 0) ? gx : xt[i];
      if (x < 0 || x >= a.V) {
        flags |= 1;
      } else if (s_ok[i]) {
        const float zx = (i0 == 0) ? gz : Fmt<T>::at(rows + (size_t)i * a.V, (size_t)x);
        const float tau = TOPK ? a.w.row_tau[r0 + i] : -INFINITY;
        const bool supp = (zx > -INFINITY) && !(zx < tau);
        const double lnp = ((double)zx * (double)a.k2 - s_l2[i]) * LN2;
        const double thr = fmin(ta.ln_eps, ta.ln_delta - s_h[i]);
        accept = supp && lnp > thr;
      }
    }
    const unsigned long long rej = __ballot(i < G && !accept);
    if (j == G && rej) j = i0 + __ffsll((long long)rej) - 1;
  }
  flags = wave_or(flags);
  const int err = (flags & 16) ? SV_ROW_INTERNAL : (flags & 1) ? SV_ROW_BAD_TOKEN : (flags & 2) ? SV_ROW_BAD_LOGITS : 0;
  for (int i = lane; i <= G; i += WAVE) {
    int v = -1;
    if (!err) v = (i < j) ? xt[i] : (i == j ? s_arg[j] : -1);
    out[i] = v;
  }
  if (lane == 0) a.accepted_len[b] = err ? err : j;
}

template <typename T, bool ALIGNED, bool TOPK>
__global__ __launch_bounds__(NT) void k_typical(const TypArgs ta) {
  constexpr int VEC = Fmt<T>::VEC;
  const Args &a = ta.a;
  __shared__ float s_m[NW];
  __shared__ int s_bi[NW], s_fl[NW];
  __shared__ double s_s[NW], s_mm[NW];
  int phase, item;
  if (!lane_item(a.B, a.rps * a.C, 0, phase, item)) return;  // units: sequences
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  const int r = item / a.C, c = item - r * a.C;
  const int b = r / a.rps, jr = r - b * a.rps;
  const T *row = static_cast<const T *>(a.target) + (size_t)r * a.V;

  // The sequence's last item (its finisher) gathers the drafted tokens and their logits
  // (positions = lanes of wave 0, the first 64) while its own chunk streams in: the token
  // loads go first, the logit loads right after the chunk's.
  const bool gath = jr == a.rps - 1 && c == a.C - 1 && wid == 0 && lane < a.G;
  const int gx = gath ? a.tokens[(size_t)b * a.G + lane] : -1;
  float gz = NAN;
  float x[VPT][VEC];
  load_chunk<T, ALIGNED, true>(row, a.V, a.nvec, c, tid, x, [&] {
    if (gath && gx >= 0 && gx < a.V)
      gz = Fmt<T>::at(static_cast<const T *>(a.target) + ((size_t)b * a.rps + lane) * a.V, (size_t)gx);
  });
  if (TOPK) {
    const float tau = a.w.row_tau[r];
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[k][e] = (x[k][e] < tau) ? -INFINITY : x[k][e];
  }
  float mt = -INFINITY;  // this thread's maximum (top-k keeps the maximum and its ties)
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) mt = fmaxf(mt, x[k][e]);
  float m = wave_max(mt);
  if (lane == 0) s_m[wid] = m;
  __syncthreads();
  m = s_m[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, s_m[w]);

  // The argmax: only the threads whose maximum is the chunk's look for its lowest index
  // (elements of a thread are in index order); then the lowest over the waves.
  int bi = 0x7fffffff;
  if (mt == m && m > -INFINITY) {
#pragma unroll
    for (int k = VPT - 1; k >= 0; --k)
#pragma unroll
      for (int e = VEC - 1; e >= 0; --e)
        if (x[k][e] == m) bi = (int)elem_index<T>(c, k, tid, e);
  }
  bi = wave_min_i(bi);

  const float k2 = a.k2;
  float off = -INFINITY;
  // A vector's terms are summed as a pairwise tree in fp32, the vectors in fp64, so each
  // chunk sum carries at most about three fp32 roundings of relative error.
  double acc_s = 0.0, acc_m = 0.0;
  int fl = (m == INFINITY) ? 1 : 0;  // a NaN or +inf also makes the sum NaN below
  if (m > -INFINITY && jr == a.rps - 1) {
    // The row after the last drafted position only ever gives the greedy next token: its
    // argmax and its validity suffice, so its sums are not formed (S = 1 keeps the row's
    // combine defined; a NaN, which would have made the sum NaN, is found by comparison).
    off = m * k2;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) nan |= (x[k][e] != x[k][e]);
    if (__ballot(nan)) fl |= 1;
    acc_s = (tid == 0) ? 1.0 : 0.0;
    fl |= 2;
  } else if (m > -INFINITY) {
    off = m * k2;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float es[VEC], ms[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float t = fmaf(x[k][e], k2, -off);
        const float ev = fast_exp2(t);
        es[e] = ev;
        ms[e] = ev * fmaxf(t, -200.0f);  // e = 0 below 2^-126: -inf terms add 0
      }
#pragma unroll
      for (int h = VEC / 2; h > 0; h >>= 1)
#pragma unroll
        for (int e = 0; e < h; ++e) {
          es[e] += es[e + h];
          ms[e] += ms[e + h];
        }
      acc_s += (double)es[0];
      acc_m += (double)ms[0];
    }
    fl |= 2;
  } else {
    bool nan = false;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) nan |= (x[k][e] != x[k][e]);
    if (__ballot(nan)) fl |= 1;
  }
  const double ws = wave_sum(acc_s), wm = wave_sum(acc_m);
  if (lane == 0) {
    s_s[wid] = ws;
    s_mm[wid] = wm;
    s_bi[wid] = bi;
    s_fl[wid] = fl;
  }
  __syncthreads();
  if (wid != 0) return;
  const double S = (s_s[0] + s_s[1]) + (s_s[2] + s_s[3]);
  const double M = (s_mm[0] + s_mm[1]) + (s_mm[2] + s_mm[3]);
  bi = s_bi[0];
  fl = s_fl[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    bi = min(bi, s_bi[w]);
    fl |= s_fl[w];
  }
  const float best = m;
  const float words[TYP_WORDS] = {off, d_head(S), d_tail(S), d_head(M), d_tail(M), best,
                                   __uint_as_float((unsigned)bi), __uint_as_float((unsigned)fl)};
  float v = words[0];  // lane f's word (constant indices: the array stays in registers)
#pragma unroll
  for (int f = 1; f < TYP_WORDS; ++f) v = (lane == f) ? words[f] : v;
  if (jr == a.rps - 1 && c == a.C - 1) {
    typical_finish<T, TOPK>(ta, b, v, c, gx, gz);
    return;
  }
  u64 *pw = a.w.tw_part + ((size_t)r * a.C + c) * TYP_WORDS;
  if (lane < TYP_WORDS) tw_putf(pw + lane, a.tag, v);
}

}  // namespace sv

// ======================================================================== host side

namespace {

using namespace sv;
using sv_host::align256;
using sv_host::next_tag;

struct TypPlan {
  bool topk;
  int esz, nvec, C, rps;
  long long R;
  size_t tw_part, tw_hist, row_tau, tk_state, total, zero_bytes;
};

bool typ_plan(int32_t B, int32_t G, int32_t V, sv_dtype dt, int32_t top_k, TypPlan &p) {
  p.esz = (dt == SV_BF16) ? 2 : 4;
  const int vec = 16 / p.esz;
  p.nvec = (int)(((long long)V + vec - 1) / vec);
  p.C = (p.nvec + CHUNK_VECS - 1) / CHUNK_VECS;
  p.rps = G + 1;
  p.R = (long long)B * p.rps;
  p.topk = top_k > 0 && top_k < V;
  const long long lb = (B + LANES - 1) / LANES, lr = (p.R + LANES - 1) / LANES;
  if (LANES * lb * (long long)p.rps * p.C > 0x7fffffffLL || LANES * lr * (long long)p.C > 0x7fffffffLL) return false;
  const size_t R = (size_t)p.R, C = (size_t)p.C;
  size_t o = 0;
  p.tw_part = o; o = align256(o + R * C * TYP_WORDS * 8);
  p.tw_hist = o; o = align256(o + (p.topk ? sv_host::topk_words(p.R, p.C, top_k) * 8 : 0));
  p.zero_bytes = o;
  p.row_tau = o; o = align256(o + (p.topk ? R * 4 : 0));
  p.tk_state = o; o = align256(o + (p.topk ? sv_host::topk_state_bytes(p.R, p.C, top_k) : 0));
  p.total = o;
  return true;
}

bool typ_args_ok(int32_t B, int32_t G, int32_t V, sv_dtype dt, float T) {
  return B >= 1 && G >= 0 && G + 1 <= TYP_MAX_ROWS && V >= 1 && (dt == SV_F32 || dt == SV_BF16) && T > 0.0f &&
         isfinite(T);
}

template <typename T, bool AL>
hipError_t typ_launch(const TypPlan &p, const TypArgs &t0, hipStream_t st, void *const *ev, int nev, int *nl) {
  sv_host::Launcher L{st, ev, nev};
  const long long lb = (t0.a.B + LANES - 1) / LANES, lr = (p.R + LANES - 1) / LANES;
  TypArgs t = t0;
  if (p.topk) sv_host::launch_topk<T, AL>(L, t.a, (unsigned)(LANES * lr * p.C), p.C);
  t.a.tag = next_tag();
  void *args[] = {&t};
  L.go(p.topk ? (const void *)&k_typical<T, AL, true> : (const void *)&k_typical<T, AL, false>,
       (unsigned)(LANES * lb * (long long)p.rps * p.C), args);
  if (nl) *nl = L.n;
  return L.e;
}

sv_status typ_run(const void *target, sv_dtype dt, const int32_t *tokens, int32_t B, int32_t G, int32_t V,
                  float T, int32_t top_k, float eps, float delta, int32_t *acc, int32_t *out, void *ws,
                  size_t ws_bytes, void *stream, void *const *ev, int32_t nev, int32_t *nl) {
  if (nl) *nl = 0;
  if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_DTYPE;
  if (B < 1 || G < 0 || G + 1 > TYP_MAX_ROWS || V < 1) return SV_ERR_SHAPE;
  if (!(T > 0.0f) || !isfinite(T)) return SV_ERR_TEMPERATURE;
  if (!(eps >= 0.0f) || !isfinite(eps) || !(delta >= 0.0f) || !isfinite(delta)) return SV_ERR_PARAM;
  TypPlan p;
  if (!typ_plan(B, G, V, dt, top_k, p)) return SV_ERR_SHAPE;
  if (!target || !acc || !out || !ws || (G > 0 && !tokens)) return SV_ERR_NULL;
  const uintptr_t ta = (uintptr_t)target;
  if (ta % p.esz) return SV_ERR_ALIGN;
  if (ws_bytes < p.total || ((uintptr_t)ws & 255)) return SV_ERR_WORKSPACE;
  const bool aligned = ((size_t)V * p.esz) % 16 == 0 && ta % 16 == 0;

  char *base = static_cast<char *>(ws);
  TypArgs t = {};
  Args &a = t.a;
  a.target = target;
  a.tokens = tokens;
  a.B = B;
  a.G = G;
  a.V = V;
  a.C = p.C;
  a.nvec = p.nvec;
  a.rps = p.rps;
  a.ntr = G + 1;
  a.tgt_rows = G + 1;
  a.k2 = (float)(LOG2E / (double)T);
  a.top_k = top_k;
  a.accepted_len = acc;
  a.out_tokens = out;
  a.spin_limit = SPIN_LIMIT;
  a.stamps = nullptr;
  a.w.tw_part = (u64 *)(base + p.tw_part);
  a.w.tw_hist = (u64 *)(base + p.tw_hist);
  a.w.row_tau = (float *)(base + p.row_tau);
  a.w.tk_state = (uint2 *)(base + p.tk_state);
  a.w.tk_rowp = nullptr;
  a.w.tk_keep = nullptr;
  t.ln_eps = log((double)eps);  // -inf for eps = 0: every token of the support passes
  t.ln_delta = log((double)delta);

  hipStream_t st = (hipStream_t)stream;
  int n = 0;
  hipError_t e;
  if (dt == SV_BF16)
    e = aligned ? typ_launch<uint16_t, true>(p, t, st, ev, nev, &n) : typ_launch<uint16_t, false>(p, t, st, ev, nev, &n);
  else
    e = aligned ? typ_launch<float, true>(p, t, st, ev, nev, &n) : typ_launch<float, false>(p, t, st, ev, nev, &n);
  if (nl) *nl = n;
  return e == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t sv_typical_workspace_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype, float temperature,
                                  int32_t top_k) {
  TypPlan p;
  if (!typ_args_ok(B, G, V, dtype, temperature) || !typ_plan(B, G, V, dtype, top_k, p)) return 256;
  return p.total;
}

size_t sv_typical_workspace_zero_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype, float temperature,
                                       int32_t top_k) {
  TypPlan p;
  if (!typ_args_ok(B, G, V, dtype, temperature) || !typ_plan(B, G, V, dtype, top_k, p)) return 0;
  return p.zero_bytes;
}

sv_status spec_typical_verify(const void *target_logits, sv_dtype dtype, const int32_t *draft_tokens,
                              int32_t B, int32_t G, int32_t V, float temperature, int32_t top_k,
                              float epsilon, float delta, int32_t *accepted_len, int32_t *out_tokens,
                              void *workspace, size_t workspace_bytes, void *stream) {
  return typ_run(target_logits, dtype, draft_tokens, B, G, V, temperature, top_k, epsilon, delta, accepted_len,
                 out_tokens, workspace, workspace_bytes, stream, nullptr, 0, nullptr);
}

sv_status spec_typical_verify_timed(const void *target_logits, sv_dtype dtype, const int32_t *draft_tokens,
                                    int32_t B, int32_t G, int32_t V, float temperature, int32_t top_k,
                                    float epsilon, float delta, int32_t *accepted_len, int32_t *out_tokens,
                                    void *workspace, size_t workspace_bytes, void *stream,
                                    void *const *events, int32_t n_events, int32_t *n_launched) {
  return typ_run(target_logits, dtype, draft_tokens, B, G, V, temperature, top_k, epsilon, delta, accepted_len,
                 out_tokens, workspace, workspace_bytes, stream, events, n_events, n_launched);
}

const char *sv_typical_launch_plan(int32_t B, int32_t G, int32_t V, sv_dtype dtype, float temperature,
                                   int32_t top_k) {
  (void)B;
  (void)G;
  (void)temperature;
  if (top_k > 0 && top_k < V) {
    if (sv_host::topk_one_pass(top_k, sv_host::row_chunks(V, dtype == SV_BF16 ? 2 : 4))) return "k_topk_select;k_topk_merge;k_typical";
    return dtype == SV_BF16 ? "k_topk_digit;k_topk_digit;k_typical"
                            : "k_topk_digit;k_topk_digit;k_topk_digit;k_topk_digit;k_typical";
  }
  return "k_typical";
}

}  // extern "C"
