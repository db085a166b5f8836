// spec_overlap.hip -- overlap of the target and draft distributions at every drafted
// position, for MI355X (gfx950).
//
// What is computed.  At position i of sequence b the verification compares p_i (target
// row i) with q_i (draft row i), both after the same temperature and top-k.  The
// probability that the position accepts its drafted token is the overlap mass
//   beta = sum_v min(p_v, q_v)
// ("Speculative Decoding 的朴素思想", section "为什么接受概率恰好是这个比值"; the rejection
// mass Z = sum_v [p_v - q_v]_+ = 1 - beta is worked out in section 手稿中的数值例子), which
// the second page also uses as 1 - TV(p, q) under the LK loss -log beta and as DSpark's
// confidence label c* = 1 - ||p - q||_1 / 2 ("推测解码：接受规则、状态与收益边界").  Both
// beta and tv = sum_v [p_v - q_v]_+ are summed, each from its own terms.
//
// How it is laid out.  A unit is one (b, i) pair: two rows of C chunks.  One kernel:
//   first-phase items, one per chunk of either row: block max m_c and the sum of
//     2^(z*k2 - m_c*k2), published as a tagged partial (the same per-chunk normaliser as
//     the verification kernel);
//   second-phase items, one per chunk c of a pair: issue the loads of both rows' chunk c,
//     then one wave per row combines that row's partials into its log2-partition, and the
//     workgroup sums min(p, q) over the chunk with one exponential per element pair (the
//     smaller of the two arguments); the chunk's tv term is p's chunk mass from the first
//     phase less that sum; the pair's last chunk collects the others' sums and writes
//     beta, tv and the pair's status.
// Every row is read twice, and much of the second read is served from the XCD's L2: in
// each XCD lane (lane_item_lag) a pair's second phase comes OV_LAG pairs after its first,
// a few MB of that lane's traffic later.  The first phase loads with ordinary cached loads
// and the second, the data's last use, with non-temporal ones, so that it does not push
// out rows still waiting for their second read.  With one v_exp_f32 per logit in the
// first phase and one per element pair in the second, the kernel is bound by VALU and
// waits more than by HBM.  A design that keeps the first phase's terms in registers and
// waits for the pair's other workgroups was measured slower: every workgroup then holds
// its slot through a device-scope round trip.
// All reductions have fixed orders: results are bitwise reproducible.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_common.h"

namespace sv {

constexpr int OV_LAG = 5;  // pairs between a pair's first and second phase in a lane (2 to
                           // 12 measured: 5 and 6 are best)

// First phase: the normaliser partial of chunk c of row r (in the pair's numbering),
// formed as the verification kernel forms it (chunk_norm), with cached loads: the second
// phase re-reads the chunk soon after.
template <typename T, bool ALIGNED, bool TOPK>
SVD void ov_first(const Args &a, int r, const T *row, int c) {
  const int lane = lane_id(), wid = threadIdx.x / WAVE;
  float off;
  double S;
  chunk_norm<T, ALIGNED, TOPK, false>(row, a.V, a.nvec, c, TOPK ? a.w.row_tau[r] : 0.0f, a.k2, off, S);
  if (wid != 0) return;
  u64 *pw = a.w.tw_part + ((size_t)r * a.C + c) * 3;
  if (lane < 3) tw_putf(pw + lane, a.tag, lane == 0 ? off : (lane == 1 ? d_head(S) : d_tail(S)));
}

// One wave: the log2-partition of row r from its chunks' partials (lanes over chunks,
// then one fixed tree), waiting until every partial carries the call's tag, and chunk
// c's own partial (its offset and sum) as published.  Returns false if the wait gave up.
SVD bool row_partition(const Args &a, int r, int c, float &o, double &t, float &off_c, double &s_c) {
  const int lane = lane_id();
  unsigned polls = 0;
  float my_off = -INFINITY;
  double my_s = 0.0;
  for (;;) {
    o = -INFINITY;
    t = 0.0;
    bool mine = true;
    for (int cc = lane; cc < a.C; cc += WAVE) {
      const u64 *pw = a.w.tw_part + ((size_t)r * a.C + cc) * 3;
      const u64 w0 = ld_dev(pw), w1 = ld_dev(pw + 1), w2 = ld_dev(pw + 2);
      mine = mine && tw_ok(w0, a.tag) && tw_ok(w1, a.tag) && tw_ok(w2, a.tag);
      const float f0 = tw_f(w0);
      const double sd = d_join(tw_f(w1), tw_f(w2));
      if (cc == c) {
        my_off = f0;
        my_s = sd;
      }
      lse_combine(o, t, f0, sd);
    }
    if (wave_or(mine ? 0u : 1u) == 0u) break;
    if (++polls >= a.spin_limit) return false;
    __builtin_amdgcn_s_sleep(2);
  }
  wave_lse(o, t);
  off_c = readlane_f(my_off, c % WAVE);
  s_c = readlane_d(my_s, c % WAVE);
  return true;
}

// Second phase: chunk c of pair u, with one exponential per element pair.  With
// off_t, off_d the chunk's first-phase offsets and Lp, Lq the rows' log2-partitions,
// p_v = 2^(at_v + dt) and q_v = 2^(ad_v + dd), where at_v = z_t*k2 - off_t is the very
// argument the first phase exponentiated, ad_v = z_d*k2 - off_d, dt = off_t - Lp and
// dd = off_d - Lq.  Then min(p_v, q_v) = 2^dt * 2^min(at_v, z_d*k2 - (off_d - dd + dt)),
// the second argument one fma with the shift off_d - dd + dt rounded to fp32 once per
// chunk (exactly off_d when dd = dt, as for p = q): the chunk's
// beta term is 2^dt * B with B = sum_v 2^min(...), and its tv term sum_v [p_v - q_v]_+ =
// sum_v (p_v - min(p_v, q_v)) is 2^dt * (S - B), S being the first phase's sum of
// 2^at_v over the chunk.  B is summed in the first phase's order (per thread, then the
// waves), so where q_v >= p_v throughout the chunk B equals S bit for bit and the tv term
// is exactly 0 (p = q bitwise gives tv = 0).
template <typename T, bool ALIGNED, bool TOPK>
SVD void ov_second(const Args &a, int u, int c) {
  constexpr int VEC = Fmt<T>::VEC;
  __shared__ float s_off[2];  // the chunk's offsets in p's and q's rows (0 for an empty chunk)
  __shared__ double s_dl[2];  // dt, dd
  __shared__ double s_sc;     // S of p's chunk
  __shared__ int s_flags;     // 1: a row is unusable, 2: a wait gave up, 4 / 8: p's / q's chunk is empty
  __shared__ double s_sum[NW];
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  const int b = u / a.G, i = u - b * a.G;
  const int rt = b * a.rps + i, rd = rt + a.G;
  const T *row_t = seq_row<T>(a, b, i);
  const T *row_d = seq_row<T>(a, b, a.G + i);

  // Both chunks' loads are issued first (L2 hits, mostly); the normalisers are gathered
  // while they fly.
  u32x4 wa[ALIGNED ? VPT : 1], wb[ALIGNED ? VPT : 1];
  // Rows off the 16-byte grid: the first half of both rows' vectors, as the pairs of
  // aligned blocks that hold them (the same registers as all vectors of aligned rows).
  constexpr int UH = VPT / 2;
  u32x4 la[ALIGNED ? 1 : UH], ha[ALIGNED ? 1 : UH], lb[ALIGNED ? 1 : UH], hb[ALIGNED ? 1 : UH];
  if (ALIGNED) {
    const u32x4 *ra = reinterpret_cast<const u32x4 *>(row_t);
    const u32x4 *rb = reinterpret_cast<const u32x4 *>(row_d);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int v = c * CHUNK_VECS + k * NT + tid;
      const int vs = v < a.nvec ? v : a.nvec - 1;
      wa[k] = __builtin_nontemporal_load(ra + vs);
      wb[k] = __builtin_nontemporal_load(rb + vs);
    }
  } else {
#pragma unroll
    for (int k = 0; k < UH; ++k) {
      const int v = c * CHUNK_VECS + k * NT + tid;
      const int vs = v < a.nvec ? v : a.nvec - 1;
      load_pair<T, true>(row_t, row_t + a.V, row_off16(row_t), vs, la[ALIGNED ? 0 : k], ha[ALIGNED ? 0 : k]);
      load_pair<T, true>(row_d, row_d + a.V, row_off16(row_d), vs, lb[ALIGNED ? 0 : k], hb[ALIGNED ? 0 : k]);
    }
  }
  if (tid == 0) s_flags = 0;
  __syncthreads();
  if (wid < 2) {
    float o, offc = -INFINITY;
    double t, sc = 0.0;
    const bool done = row_partition(a, wid == 0 ? rt : rd, c, o, t, offc, sc);
    const bool ok = done && isfinite(o) && isfinite(t) && t > 0.0;
    if (lane == 0) {
      const bool empty = !(offc > -INFINITY);
      s_off[wid] = empty ? 0.0f : offc;
      s_dl[wid] = (ok && !empty) ? (double)offc - ((double)o + log2(t)) : 0.0;
      if (wid == 0) s_sc = sc;
      if (!done) atomicOr(&s_flags, 2);
      else if (!ok) atomicOr(&s_flags, 1);
      if (empty) atomicOr(&s_flags, 4 << wid);
    }
  }
  __syncthreads();
  const int flags = s_flags;
  float acc = 0.0f;
  if (flags == 0) {
    const float k2 = a.k2;
    const float off_t = s_off[0], off_d = s_off[1];
    const float sh_d = (float)((double)off_d - (s_dl[1] - s_dl[0]));
    const float tau_t = TOPK ? a.w.row_tau[rt] : -INFINITY;
    const float tau_d = TOPK ? a.w.row_tau[rd] : -INFINITY;
    if (ALIGNED && (c + 1) * CHUNK_VECS > a.nvec) {  // vectors past the row's end hold -inf
      constexpr unsigned NEG_INF = (sizeof(T) == 2) ? 0xff80ff80u : 0xff800000u;
      const u32x4 ninf = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const bool in = c * CHUNK_VECS + k * NT + tid < a.nvec;
        wa[k] = in ? wa[k] : ninf;
        wb[k] = in ? wb[k] : ninf;
      }
    }
    auto add_vec = [&](const float (&xa)[VEC], const float (&xb)[VEC]) {
      float tb[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float zt = (TOPK && xa[e] < tau_t) ? -INFINITY : xa[e];
        const float zd = (TOPK && xb[e] < tau_d) ? -INFINITY : xb[e];
        tb[e] = fast_exp2(fminf(fmaf(zt, k2, -off_t), fmaf(zd, k2, -sh_d)));
      }
#pragma unroll
      for (int h = VEC / 2; h > 0; h >>= 1)
#pragma unroll
        for (int e = 0; e < h; ++e) tb[e] += tb[e + h];
      acc += tb[0];
    };
    if (ALIGNED) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        float xa[VEC], xb[VEC];
        Fmt<T>::unpack(wa[k], xa);
        Fmt<T>::unpack(wb[k], xb);
        add_vec(xa, xb);
      }
    } else {
      // Rows off the 16-byte grid: the prefetched half, then two vectors of each row at a
      // time (each vector built from the two aligned blocks that hold it), in the same order.
#pragma unroll
      for (int k = 0; k < UH; ++k) {
        float xa[VEC], xb[VEC];
        Fmt<T>::unpack(funnel16(la[ALIGNED ? 0 : k], ha[ALIGNED ? 0 : k], row_off16(row_t)), xa);
        Fmt<T>::unpack(funnel16(lb[ALIGNED ? 0 : k], hb[ALIGNED ? 0 : k], row_off16(row_d)), xb);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const bool in = elem_index<T>(c, k, tid, e) < a.V;
          xa[e] = in ? xa[e] : -INFINITY;
          xb[e] = in ? xb[e] : -INFINITY;
        }
        add_vec(xa, xb);
      }
      constexpr int KG = 2;
#pragma unroll
      for (int k0 = UH; k0 < VPT; k0 += KG) {
        float xa[KG][VEC], xb[KG][VEC];
        load_vectors<T, false, true, KG>(row_t, a.V, a.nvec, c, k0, tid, xa);
        load_vectors<T, false, true, KG>(row_d, a.V, a.nvec, c, k0, tid, xb);
#pragma unroll
        for (int kk = 0; kk < KG; ++kk) add_vec(xa[kk], xb[kk]);
      }
    }
  }
  const double wsum = wave_sum((double)acc);
  if (lane == 0) s_sum[wid] = wsum;
  __syncthreads();
  if (wid != 0) return;
  // beta and tv terms of the chunk; nothing where p's chunk is empty, all of p's mass as
  // tv where q's chunk is empty.
  double cb = 0.0, ct = 0.0;
  if ((flags & 7) == 0) {
    const double scale = exp2(s_dl[0]);
    if (flags & 8) {
      ct = scale * s_sc;
    } else {
      const double B = (s_sum[0] + s_sum[1]) + (s_sum[2] + s_sum[3]);
      const double Bj = d_join(d_head(B), d_tail(B));  // rounded as S was for its partial
      cb = scale * Bj;
      ct = scale * (s_sc - Bj);
    }
  }
  u64 *ow = a.w.tw_ov + (size_t)u * a.C * 4;
  if (c != a.C - 1) {
    if (lane < 4) {
      const double v = (lane < 2) ? cb : ct;
      tw_putf(ow + (size_t)c * 4 + lane, a.tag, (lane & 1) ? d_tail(v) : d_head(v));
    }
    return;
  }

  // The pair's last chunk: the other chunks' sums, lanes over chunks, one fixed tree.
  double sbeta = 0.0, stv = 0.0;
  bool gave_up = false;
  if ((flags & 3) == 0) {
    unsigned polls = 0;
    for (;;) {
      sbeta = 0.0;
      stv = 0.0;
      bool mine = true;
      for (int cc = lane; cc < a.C; cc += WAVE) {
        if (cc == c) {
          sbeta += cb;
          stv += ct;
          continue;
        }
        const u64 *pw = ow + (size_t)cc * 4;
        const u64 w0 = ld_dev(pw), w1 = ld_dev(pw + 1), w2 = ld_dev(pw + 2), w3 = ld_dev(pw + 3);
        mine = mine && tw_ok(w0, a.tag) && tw_ok(w1, a.tag) && tw_ok(w2, a.tag) && tw_ok(w3, a.tag);
        sbeta += d_join(tw_f(w0), tw_f(w1));
        stv += d_join(tw_f(w2), tw_f(w3));
      }
      if (wave_or(mine ? 0u : 1u) == 0u) break;
      if (++polls >= a.spin_limit) {
        gave_up = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    sbeta = wave_sum(sbeta);
    stv = wave_sum(stv);
  }
  if (lane == 0) {
    bool internal = gave_up || (flags & 2);
    if (TOPK && !internal) {  // a top-k collector that gave up leaves a NaN threshold
      const float tt = a.w.row_tau[rt], td = a.w.row_tau[rd];
      internal = (tt != tt) || (td != td);
    }
    const int st_ = internal ? SV_ROW_INTERNAL : ((flags & 1) ? SV_ROW_BAD_LOGITS : 0);
    a.pair_status[u] = st_;
    a.beta[u] = st_ ? (double)NAN : sbeta;
    a.tv[u] = st_ ? (double)NAN : stv;
  }
}

// At least four resident waves per SIMD: on aligned rows the kernel fits in 96 registers
// and runs five, with nothing spilled.  Six (80 registers) spill and take 47.7 us against 35.6 on the
// headline batch.
template <typename T, bool ALIGNED, bool TOPK>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void k_overlap(const Args a) {
  int phase, unit, sub;
  if (!lane_item_lag(a.B * a.G, 2 * a.C, a.C, a.lag, phase, unit, sub)) return;
  if (phase == 1) {
    const int side = sub >= a.C ? 1 : 0, c = sub - side * a.C;
    const int b = unit / a.G, i = unit - b * a.G;
    const int jr = side * a.G + i;
    ov_first<T, ALIGNED, TOPK>(a, b * a.rps + jr, seq_row<T>(a, b, jr), c);
  } else {
    ov_second<T, ALIGNED, TOPK>(a, unit, sub);
  }
}

}  // namespace sv

// ======================================================================== host side

namespace {

using namespace sv;
using sv_host::align256;
using sv_host::next_tag;

struct OvPlan {
  bool topk;
  int esz, nvec, C, rps;
  long long R, U;
  size_t tw_part, tw_ov, tw_hist, row_tau, tk_state, total, zero_bytes;
};

bool ov_plan(int32_t B, int32_t G, int32_t V, sv_dtype dt, int32_t top_k, OvPlan &p) {
  p.esz = (dt == SV_BF16) ? 2 : 4;
  const int vec = 16 / p.esz;
  p.nvec = (int)(((long long)V + vec - 1) / vec);
  p.C = (p.nvec + CHUNK_VECS - 1) / CHUNK_VECS;
  p.rps = 2 * G;
  p.R = (long long)B * p.rps;
  p.U = (long long)B * G;
  p.topk = top_k > 0 && top_k < V;
  const long long lu = (p.U + LANES - 1) / LANES, lr = (p.R + LANES - 1) / LANES;
  if (LANES * lu * 3LL * p.C > 0x7fffffffLL || LANES * lr * (long long)p.C > 0x7fffffffLL) return false;
  const size_t R = (size_t)p.R, C = (size_t)p.C, U = (size_t)p.U;
  size_t o = 0;
  // tagged words first (the part that must be clean when a call starts)
  p.tw_part = o; o = align256(o + R * C * 3 * 8);
  p.tw_ov = o; o = align256(o + U * C * 4 * 8);
  p.tw_hist = o; o = align256(o + (p.topk ? sv_host::topk_words(p.R, p.C, top_k) * 8 : 0));
  p.zero_bytes = o;
  p.row_tau = o; o = align256(o + (p.topk ? R * 4 : 0));
  p.tk_state = o; o = align256(o + (p.topk ? sv_host::topk_state_bytes(p.R, p.C, top_k) : 0));
  p.total = o;
  return true;
}

bool ov_args_ok(int32_t B, int32_t G, int32_t V, sv_dtype dt, float T) {
  return B >= 1 && G >= 0 && V >= 1 && (dt == SV_F32 || dt == SV_BF16) && T > 0.0f && isfinite(T);
}

template <typename T, bool AL>
hipError_t ov_launch(const OvPlan &p, const Args &a, hipStream_t st, void *const *ev, int nev,
                     int *nl) {
  sv_host::Launcher L{st, ev, nev};
  const long long lu = (p.U + LANES - 1) / LANES, lr = (p.R + LANES - 1) / LANES;
  Args aa = a;
  if (p.topk) sv_host::launch_topk<T, AL>(L, aa, (unsigned)(LANES * lr * p.C), p.C);
  aa.tag = next_tag();
  void *args[] = {&aa};
  L.go(p.topk ? (const void *)&k_overlap<T, AL, true> : (const void *)&k_overlap<T, AL, false>,
       (unsigned)(LANES * lu * 3LL * p.C), args);
  if (nl) *nl = L.n;
  return L.e;
}

sv_status ov_run(const void *target, const void *draft, sv_dtype dt, int32_t B, int32_t G,
                 int32_t V, int32_t target_rows, float T, int32_t top_k, double *beta, double *tv,
                 int32_t *pair_status, void *ws, size_t ws_bytes, void *stream, void *const *ev,
                 int32_t nev, int32_t *nl) {
  if (nl) *nl = 0;
  if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_DTYPE;
  if (B < 1 || G < 0 || V < 1 || (target_rows != G && target_rows != G + 1)) return SV_ERR_SHAPE;
  if (!(T > 0.0f) || !isfinite(T)) return SV_ERR_TEMPERATURE;
  OvPlan p;
  if (!ov_plan(B, G, V, dt, top_k, p)) return SV_ERR_SHAPE;
  if (G == 0) return SV_OK;  // no drafted positions: nothing to compute
  if (!target || !draft || !beta || !tv || !pair_status || !ws) return SV_ERR_NULL;
  const uintptr_t ta = (uintptr_t)target, da = (uintptr_t)draft;
  if (ta % p.esz || da % p.esz) return SV_ERR_ALIGN;
  if (ws_bytes < p.total || ((uintptr_t)ws & 255)) return SV_ERR_WORKSPACE;
  const bool aligned = ((size_t)V * p.esz) % 16 == 0 && ta % 16 == 0 && da % 16 == 0;

  char *base = static_cast<char *>(ws);
  Args a = {};
  a.target = target;
  a.draft = draft;
  a.B = B;
  a.G = G;
  a.V = V;
  a.C = p.C;
  a.nvec = p.nvec;
  a.rps = p.rps;
  a.ntr = G;
  a.tgt_rows = target_rows;
  a.k2 = (float)(LOG2E / (double)T);
  a.top_k = top_k;
  a.beta = beta;
  a.tv = tv;
  a.pair_status = pair_status;
  a.lag = OV_LAG;
  a.spin_limit = SPIN_LIMIT;
  a.stamps = nullptr;
  a.w.tw_part = (u64 *)(base + p.tw_part);
  a.w.tw_ov = (u64 *)(base + p.tw_ov);
  a.w.tw_hist = (u64 *)(base + p.tw_hist);
  a.w.row_tau = (float *)(base + p.row_tau);
  a.w.tk_state = (uint2 *)(base + p.tk_state);
  a.w.tk_rowp = nullptr;
  a.w.tk_keep = nullptr;

  hipStream_t st = (hipStream_t)stream;
  int n = 0;
  hipError_t e;
  if (dt == SV_BF16)
    e = aligned ? ov_launch<uint16_t, true>(p, a, st, ev, nev, &n) : ov_launch<uint16_t, false>(p, a, st, ev, nev, &n);
  else
    e = aligned ? ov_launch<float, true>(p, a, st, ev, nev, &n) : ov_launch<float, false>(p, a, st, ev, nev, &n);
  if (nl) *nl = n;
  return e == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t sv_overlap_workspace_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                                  float temperature, int32_t top_k) {
  OvPlan p;
  if (!ov_args_ok(B, G, V, dtype, temperature) || !ov_plan(B, G, V, dtype, top_k, p)) return 256;
  return p.total > 0 ? p.total : 256;
}

size_t sv_overlap_workspace_zero_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                                       float temperature, int32_t top_k) {
  OvPlan p;
  if (!ov_args_ok(B, G, V, dtype, temperature) || !ov_plan(B, G, V, dtype, top_k, p)) return 0;
  return p.zero_bytes;
}

sv_status spec_overlap(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                       int32_t B, int32_t G, int32_t V, int32_t target_rows, float temperature,
                       int32_t top_k, double *beta, double *tv, int32_t *pair_status,
                       void *workspace, size_t workspace_bytes, void *stream) {
  return ov_run(target_logits, draft_logits, dtype, B, G, V, target_rows, temperature, top_k,
                beta, tv, pair_status, workspace, workspace_bytes, stream, nullptr, 0, nullptr);
}

sv_status spec_overlap_timed(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                             int32_t B, int32_t G, int32_t V, int32_t target_rows,
                             float temperature, int32_t top_k, double *beta, double *tv,
                             int32_t *pair_status, void *workspace, size_t workspace_bytes,
                             void *stream, void *const *events, int32_t n_events,
                             int32_t *n_launched) {
  return ov_run(target_logits, draft_logits, dtype, B, G, V, target_rows, temperature, top_k,
                beta, tv, pair_status, workspace, workspace_bytes, stream, events, n_events,
                n_launched);
}

const char *sv_overlap_launch_plan(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                                   float temperature, int32_t top_k) {
  (void)B;
  (void)temperature;
  if (G == 0) return "";
  if (top_k > 0 && top_k < V) {
    if (sv_host::topk_one_pass(top_k, sv_host::row_chunks(V, dtype == SV_BF16 ? 2 : 4))) return "k_topk_select;k_topk_merge;k_overlap";
    return dtype == SV_BF16 ? "k_topk_digit;k_topk_digit;k_overlap"
                            : "k_topk_digit;k_topk_digit;k_topk_digit;k_topk_digit;k_overlap";
  }
  return "k_overlap";
}

}  // extern "C"
