// spec_tree.hip -- verification of a draft tree, for MI355X (gfx950).
//
// What is computed.  A tree of N nodes per sequence: node 0 is the committed context,
// every other node n has a parent parent[n] < n and a token x_n; p_u (target row u) is
// the target's next-token distribution after node u's path and q_u (draft row u) the
// distribution u's children were drawn from, independently.  The walk starts at the
// root and tests u's children in index order against the current distribution: p_u
// first, and after each rejection norm([cur - q_u]_+) ("Speculative Decoding 的朴素思想",
// section "Token Tree Verifier", on SpecInfer's multi-step speculative sampling; the EAGLE
// page, section 6.2, rejection node by node).  An accepted child becomes the new node;
// when every child is rejected the token is drawn from the current distribution, at a
// leaf the bonus is drawn from p_u.  T = 0: the first child whose token is argmax p_u is
// accepted, else argmax p_u is emitted.
//
// The residual family is one-parameter: after k rejections at u the current
// distribution is [p_u - c_k q_u]_+ / Z_k with c_0 = 0, Z_0 = 1 and
// c_{k+1} = c_k + Z_k, Z_k = sum_v [p_u(v) - c_k q_u(v)]_+ (induction on
// [([p - c q]_+)/Z - q]_+ = [p - (c + Z) q]_+ / Z).  The chain Z_1, Z_2, ... depends on
// no uniform, so it is computed for every node in parallel before the walk, and the walk
// itself touches only gathered scalars.
//
// Launches (each data-parallel; results pass through the workspace between launches):
//   k_topk_digit   (top-k only) the radix select of every row's threshold.
//   k_tree_rows    per chunk of every target row and of every internal node's draft row:
//                  the normaliser partial (argmax at T = 0); the row's last chunk combines
//                  them into the row's log2-partition (argmax).
//                  Target row 0's first chunk also lists the tree's nodes with two or
//                  more children.
//   k_tree_resid   (T > 0, the listed nodes) Z_1, Z_2, ...: the node's items read its two
//                  rows once, keep them in registers and run the rounds from them,
//                  exchanging only each round's partial sums.
//   k_tree_draw    (T > 0) per tree and chunk: wave 0 walks the tree (checks, gathered
//                  logits, the walk; chunk 0's item writes the accepted tokens and path),
//                  then the item forms the segment masses of its chunk of the chosen
//                  weights ([p - c q]_+ or p); the last chunk picks the segment and, in
//                  it, the token by inverse CDF with u_sample.
//   k_tree_walk    (T = 0 only) one wave per tree: the walk, with nothing to draw.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_common.h"
#include "sv_draw.h"

namespace sv {

enum : int { TJ_NONE = 0, TJ_TARGET = 1, TJ_RESID = 2 };
constexpr int TREE_MAX_NODES = 1024;   // nodes per tree (the walk keeps them in LDS)
constexpr int TREE_DRAW_LDS_SEGS = 2048;  // segment masses the draw's collector keeps in LDS
constexpr int TREE_MAX_ITEMS = 64;     // k_tree_resid items per node (V up to 64 * 16 KiB of a row)

struct TreeArgs {
  Args a;                  // rows per tree: rps = 2N (N target rows, then N draft rows); a.G = N
  const int32_t *parent;   // [B, N]
  int32_t *path;           // [B, N] out, nullable
  int S;                   // largest number of children a node may have
  // plain, handed from one launch to the next
  float *row_off;          // [R] row offset o (the largest chunk offset)
  double *row_lt;          // [R] log2 of the row sum in o's scale: log2-partition = o + lt
  int32_t *row_arg;        // [R] greedy: lowest-index argmax
  int32_t *row_ok;         // [R] 1 usable, 0 not (NaN, +inf, nothing finite kept), -1 not read,
                           //   -2 a wait gave up
  double *zc;              // [B*N*S] Z_j of node u at [u*S + j], j = 1..S-1
  // tagged words within one launch
  u64 *tw_z;               // [B*N*(S-1)*I*2] per node, round and item: sum [p - c_j q]_+
  u64 *tw_seg;             // [B*C*SEGS*2] per tree, chunk and segment: the draw's masses
  int32_t *act;            // [B*kmax] or null: per tree, its nodes with two or more children
                           //   in index order (node | children << 16), from k_tree_rows
  int32_t *act_n;          // [B] how many
  int kmax;                // most such nodes a tree of N nodes can have: (N - 1) / 2, at least 1
};

// The nodes' children, counted by one wave: nch = children of node u in tree b.
SVD int child_count(const TreeArgs &t, int b, int u) {
  const int N = t.a.G;
  const int32_t *par = t.parent + (size_t)b * N;
  unsigned cnt = 0;
  for (int n = lane_id() + 1; n < N; n += WAVE) cnt += (par[n] == u) ? 1u : 0u;
  return (int)wave_sum((double)cnt);
}

// Sampling: chunk c of row r.  Every chunk publishes its normaliser partial; the row's
// last chunk combines the row -- o = the largest offset, then sum_c S_c 2^(off_c - o) in
// chunk order (the order the verification kernel uses, so both give the same partition)
// -- into row_off / row_lt / row_ok.
template <typename T, bool ALIGNED, bool TOPK>
SVD void tree_row_chunk(const TreeArgs &t, int r, const T *row, int c) {
  const Args &a = t.a;
  const int lane = lane_id(), wid = threadIdx.x / WAVE;
  u64 *pw = a.w.tw_part + (size_t)r * a.C * 3;
  float off;
  double S;
  chunk_norm<T, ALIGNED, TOPK, true>(row, a.V, a.nvec, c, TOPK ? a.w.row_tau[r] : 0.0f, a.k2, off, S);
  if (wid != 0) return;
  if (c != a.C - 1) {
    if (lane < 3) tw_putf(pw + (size_t)c * 3 + lane, a.tag, lane == 0 ? off : (lane == 1 ? d_head(S) : d_tail(S)));
    return;
  }
  bool done = false;
  for (unsigned polls = 0; polls < a.spin_limit && !done; ++polls) {
    bool mine = true;
    for (int cc = lane; cc < a.C - 1; cc += WAVE)
      mine = mine && tw_ok(ld_dev(pw + (size_t)cc * 3), a.tag) && tw_ok(ld_dev(pw + (size_t)cc * 3 + 1), a.tag) &&
             tw_ok(ld_dev(pw + (size_t)cc * 3 + 2), a.tag);
    done = wave_or(mine ? 0u : 1u) == 0u;
    if (!done) __builtin_amdgcn_s_sleep(2);
  }
  if (lane == 0) {
    auto p_off = [&](int cc) { return cc == c ? off : tw_f(ld_dev(pw + (size_t)cc * 3)); };
    auto p_sum = [&](int cc) {
      return cc == c ? S : d_join(tw_f(ld_dev(pw + (size_t)cc * 3 + 1)), tw_f(ld_dev(pw + (size_t)cc * 3 + 2)));
    };
    float o = -INFINITY;
    for (int cc = 0; cc < a.C; ++cc) o = fmaxf(o, p_off(cc));
    double tt = 0.0;
    for (int cc = 0; cc < a.C; ++cc) tt += p_sum(cc) * (double)fast_exp2(p_off(cc) - o);
    const bool ok = done && isfinite(o) && isfinite(tt) && tt > 0.0;
    t.row_off[r] = o;
    t.row_lt[r] = ok ? log2(tt) : 0.0;
    t.row_ok[r] = !done ? -2 : (ok ? 1 : 0);
  }
}

// Tree b's nodes with two or more children, in index order, for k_tree_resid (one wave).
// Parent entries outside [0, n) are not counted (the walk reports such a tree).  Each
// counted entry is one child, so at most (N - 1) / 2 nodes have two or more.
SVD void list_multi_child(const TreeArgs &t, int b) {
  __shared__ int s_cnt[TREE_MAX_NODES];
  const int N = t.a.G, lane = lane_id();
  const int32_t *par = t.parent + (size_t)b * N;
  for (int n = lane; n < N; n += WAVE) s_cnt[n] = 0;
  lds_sync();
  for (int n = lane + 1; n < N; n += WAVE) {
    const int p = par[n];
    if (p >= 0 && p < n) atomicAdd(&s_cnt[p], 1);
  }
  lds_sync();
  int base = 0;
  for (int n0 = 0; n0 < N; n0 += WAVE) {
    const int n = n0 + lane;
    const int c = (n < N) ? s_cnt[n] : 0;
    const unsigned long long bal = __ballot(c >= 2);
    const int pos = base + (int)__popcll(bal & ((1ull << lane) - 1ull));
    if (c >= 2 && pos < t.kmax) t.act[(size_t)b * t.kmax + pos] = n | (c << 16);
    base += (int)__popcll(bal);
  }
  if (lane == 0) t.act_n[b] = base < t.kmax ? base : t.kmax;
}

// ---------------------------------------------------------------- k_tree_rows

template <typename T, bool ALIGNED, bool TOPK, bool GREEDY>
__global__ __launch_bounds__(NT) void k_tree_rows(const TreeArgs t) {
  constexpr int VEC = Fmt<T>::VEC;
  const Args &a = t.a;
  int phase, item;
  if (!lane_item(a.B * a.rps, a.C, 0, phase, item)) return;  // units: rows
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  const int r = item / a.C, c = item - r * a.C;
  const int b = r / a.rps, j = r - b * a.rps;
  const int N = a.G;
  if (j >= N && (GREEDY || child_count(t, b, j - N) == 0)) {  // a draft row nobody reads
    if (c == a.C - 1 && tid == 0) t.row_ok[r] = -1;
    return;
  }
  const T *row = seq_row<T>(a, b, j);
  u64 *pw = a.w.tw_part + (size_t)r * a.C * 3;

  if (GREEDY) {
    __shared__ float s_v[NW];
    __shared__ int s_i[NW], s_f[NW];
    float x[VPT][VEC];
    load_chunk<T, ALIGNED, true>(row, a.V, a.nvec, c, tid, x);
    float best = -INFINITY;
    int bi = 0x7fffffff, fl = 0;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float z = x[k][e];
        if (z > best) {
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
    if (wid != 0) return;
    best = s_v[0];
    bi = s_i[0];
    fl = s_f[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      best_combine(best, bi, s_v[w], s_i[w]);
      fl |= s_f[w];
    }
    if (c != a.C - 1) {
      if (lane < 3)
        tw_put(pw + (size_t)c * 3 + lane, a.tag,
               lane == 0 ? __float_as_uint(best) : (lane == 1 ? (unsigned)bi : (unsigned)fl));
      return;
    }
    // the row's last chunk: the other chunks' bests in chunk order
    bool done = false;
    for (unsigned polls = 0; polls < a.spin_limit && !done; ++polls) {
      bool mine = true;
      for (int cc = lane; cc < a.C - 1; cc += WAVE)
        mine = mine && tw_ok(ld_dev(pw + (size_t)cc * 3), a.tag) && tw_ok(ld_dev(pw + (size_t)cc * 3 + 1), a.tag) &&
               tw_ok(ld_dev(pw + (size_t)cc * 3 + 2), a.tag);
      done = wave_or(mine ? 0u : 1u) == 0u;
      if (!done) __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) {
      float v = -INFINITY;
      int vi = 0x7fffffff, f = 0;
      for (int cc = 0; cc < a.C - 1; ++cc) {
        best_combine(v, vi, __uint_as_float((unsigned)ld_dev(pw + (size_t)cc * 3)),
                     (int)(unsigned)ld_dev(pw + (size_t)cc * 3 + 1));
        f |= (int)(unsigned)ld_dev(pw + (size_t)cc * 3 + 2);
      }
      best_combine(v, vi, best, bi);
      f |= fl;
      t.row_arg[r] = vi;
      t.row_ok[r] = !done ? -2 : (((f & 1) == 0 && (f & 2)) ? 1 : 0);
    }
    return;
  }

  // target row 0's first chunk also lists the tree's nodes that need residual masses
  if (t.act && j == 0 && c == 0 && wid == 0) list_multi_child(t, b);
  tree_row_chunk<T, ALIGNED, TOPK>(t, r, row, c);
}

// ---------------------------------------------------------------- k_tree_resid

// Items of k_tree_resid: RKV 16-byte vectors per thread of each of a node's two rows.
// Aligned rows keep their raw vectors in registers, 8 a thread; otherwise p and q are
// kept as floats, 4 vectors a thread.
template <bool ALIGNED>
constexpr int resid_rkv() { return ALIGNED ? 8 : 4; }
__host__ __device__ inline int resid_items(int nvec, bool aligned) {
  const int iv = NT * (aligned ? resid_rkv<true>() : resid_rkv<false>());
  return (nvec + iv - 1) / iv;
}

// The residual masses Z_1 .. Z_{k-1} of a node with k >= 2 children.  Units are the slots
// of each tree's list of such nodes (k_tree_rows wrote it), so no workgroup is spent on a
// node without rounds.  The node's rows are cut into items; each item loads its part of
// both rows once and keeps it in registers, and for j = 1, 2, ...: sums [p - c_j q]_+ over
// its part (p and q formed from the rows' log2-partitions as the draw forms them),
// publishes the sum, and waits for the node's other items' sums of the same round, whose
// total is Z_j and gives c_{j+1} = c_j + Z_j.  The items of a node sit in consecutive
// blocks of one XCD lane, so they are resident together; every wait is bounded.
template <typename T, bool ALIGNED, bool TOPK>
__global__ __launch_bounds__(NT) void k_tree_resid(const TreeArgs t) {
  constexpr int VEC = Fmt<T>::VEC;
  constexpr int RKV = resid_rkv<ALIGNED>();
  const Args &a = t.a;
  const int R1 = t.S - 1;
  const int I = resid_items(a.nvec, ALIGNED);  // items per node
  int phase, item;
  if (!lane_item(a.B * t.kmax, I, 0, phase, item)) return;  // units: list slots
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  const int slot = item / I, it = item - slot * I;
  // slots are numbered list position first (slot = ks * B + b), so each XCD lane meets the
  // trees' first list entries first and the (mostly empty) later positions last
  const int N = a.G, ks = slot / a.B, b = slot - ks * a.B;
  // Two rounds of loads before the data: the slot's entry (with the count), then the rows'
  // statistics together with the rows' data.
  const int cnt = t.act_n[b], ent = t.act[(size_t)b * t.kmax + ks];
  if (ks >= cnt) return;  // an empty slot
  const int u = ent & 0xffff, nch = ent >> 16;
  if (u < 0 || u >= N || nch < 2) return;
  const int unit = b * N + u;
  const int rt = b * a.rps + u, rd = rt + N;
  const int okt = t.row_ok[rt], okd = t.row_ok[rd];
  const float ot = t.row_off[rt], od = t.row_off[rd];
  const double ltt = t.row_lt[rt], ltd = t.row_lt[rd];
  const float tau_t = TOPK ? a.w.row_tau[rt] : -INFINITY, tau_d = TOPK ? a.w.row_tau[rd] : -INFINITY;
  const int rounds = (nch - 1 < R1) ? nch - 1 : R1;
  const float k2 = a.k2;
  const T *row_t = seq_row<T>(a, b, u), *row_d = seq_row<T>(a, b, N + u);
  // aligned: the raw vectors (past the row's end: -inf), loaded while the statistics
  // arrive; otherwise p and q
  u32x4 wt[ALIGNED ? RKV : 1], wd[ALIGNED ? RKV : 1];
  float p[ALIGNED ? 1 : RKV][VEC], q[ALIGNED ? 1 : RKV][VEC];
  if (ALIGNED) {
    const u32x4 *ra = reinterpret_cast<const u32x4 *>(row_t), *rb = reinterpret_cast<const u32x4 *>(row_d);
#pragma unroll
    for (int k = 0; k < RKV; ++k) {
      const int v = it * NT * RKV + k * NT + tid;
      const int vs = v < a.nvec ? v : a.nvec - 1;
      wt[k] = __builtin_nontemporal_load(ra + vs);
      wd[k] = __builtin_nontemporal_load(rb + vs);
    }
  }
  if (okt != 1 || okd != 1) return;  // no rounds (the walk reports bad rows)
  const double lp = (double)ot + ltt, lq = (double)od + ltd;
  const float mt_hi = d_head(lp), mt_lo = d_tail(lp), md_hi = d_head(lq), md_lo = d_tail(lq);
  auto pq = [&](float za, float zb, float &pv, float &qv) {
    const float zt = (TOPK && za < tau_t) ? -INFINITY : za;
    const float zd = (TOPK && zb < tau_d) ? -INFINITY : zb;
    pv = fast_exp2(fmaf(zt, k2, -mt_hi) - mt_lo);
    qv = fast_exp2(fmaf(zd, k2, -md_hi) - md_lo);
  };
  if (ALIGNED) {
    constexpr unsigned NEG_INF = (sizeof(T) == 2) ? 0xff80ff80u : 0xff800000u;
#pragma unroll
    for (int k = 0; k < RKV; ++k)
      if (it * NT * RKV + k * NT + tid >= a.nvec) {
        wt[k] = u32x4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
        wd[k] = wt[k];
      }
  } else {
#pragma unroll
    for (int k = 0; k < RKV; ++k) {
      const int v = it * NT * RKV + k * NT + tid;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const long idx = (long)v * VEC + e;
        const bool in = idx < a.V;
        pq(in ? Fmt<T>::at(row_t, (size_t)idx) : -INFINITY, in ? Fmt<T>::at(row_d, (size_t)idx) : -INFINITY,
           p[ALIGNED ? 0 : k][e], q[ALIGNED ? 0 : k][e]);
      }
    }
  }

  __shared__ double s_w[NW];
  __shared__ double s_z;
  u64 *zw = t.tw_z + (size_t)unit * R1 * I * 2;
  double cj = 1.0;  // c_1 = c_0 + Z_0 = 1
  for (int j = 1; j <= rounds; ++j) {
    const float cf = (float)cj;
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < RKV; ++k) {
      float w[VEC];
      if (ALIGNED) {
        float za[VEC], zb[VEC];
        Fmt<T>::unpack(wt[ALIGNED ? k : 0], za);
        Fmt<T>::unpack(wd[ALIGNED ? k : 0], zb);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float pe, qe;
          pq(za[e], zb[e], pe, qe);
          w[e] = fmaxf(fmaf(-cf, qe, pe), 0.0f);
        }
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) w[e] = fmaxf(fmaf(-cf, q[ALIGNED ? 0 : k][e], p[ALIGNED ? 0 : k][e]), 0.0f);
      }
#pragma unroll
      for (int h = VEC / 2; h > 0; h >>= 1)
#pragma unroll
        for (int e = 0; e < h; ++e) w[e] += w[e + h];
      acc += w[0];
    }
    const double ws = wave_sum((double)acc);
    if (lane == 0) s_w[wid] = ws;
    __syncthreads();
    if (wid == 0) {
      const double mine = (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
      u64 *rw = zw + (size_t)(j - 1) * I * 2;
      if (lane < 2) tw_putf(rw + (size_t)it * 2 + lane, a.tag, lane ? d_tail(mine) : d_head(mine));
      double zj = (double)NAN;
      for (unsigned polls = 0; polls < a.spin_limit; ++polls) {
        bool ready = true;
        double part = 0.0;
        for (int cc = lane; cc < I; cc += WAVE) {
          const u64 w0 = ld_dev(rw + (size_t)cc * 2), w1 = ld_dev(rw + (size_t)cc * 2 + 1);
          ready = ready && (cc == it || (tw_ok(w0, a.tag) && tw_ok(w1, a.tag)));
          part += (cc == it) ? mine : d_join(tw_f(w0), tw_f(w1));
        }
        if (wave_or(ready ? 0u : 1u) == 0u) {
          zj = wave_sum(part);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0) {
        s_z = zj;
        if (it == I - 1) t.zc[(size_t)unit * t.S + j] = zj;  // a wait that gave up leaves NaN
      }
    }
    __syncthreads();
    // c_{j+1} = c_j + Z_j; a zero mass makes p the current distribution again, whose
    // next residual is [p - q]_+ (c = 1)
    cj = (s_z > 0.0) ? cj + s_z : 1.0;
  }
}

// ---------------------------------------------------------------- k_tree_walk

// The walk of tree b by one wave: checks, gathered logits, then the walk itself.  With
// writer, the accepted tokens and path, the padding and accepted_len (or the row code) are
// written.  Leaves in s_res the node u where the walk ended, the draw's kind and the
// accepted depth, and in *s_c the draw's c (kind TJ_RESID).
template <typename T, bool TOPK, bool GREEDY>
SVD void tree_walk(const TreeArgs &t, int b, bool writer, int *s_res, double *s_c) {
  const Args &a = t.a;
  const int lane = lane_id();
  const int N = a.G, V = a.V;
  constexpr int ZP = 4;  // residual masses per node staged in LDS (zc[1..4]); later ones are read on demand
  __shared__ int s_par[TREE_MAX_NODES], s_tok[TREE_MAX_NODES], s_nch[TREE_MAX_NODES];
  __shared__ float s_zt[TREE_MAX_NODES], s_zd[TREE_MAX_NODES], s_ua[TREE_MAX_NODES], s_tau[TREE_MAX_NODES],
      s_taud[TREE_MAX_NODES];
  __shared__ double s_lp[TREE_MAX_NODES], s_lq[TREE_MAX_NODES], s_zp[TREE_MAX_NODES * ZP];
  __shared__ int s_arg[GREEDY ? TREE_MAX_NODES : 1];  // greedy: each target row's argmax
  const int32_t *par = t.parent + (size_t)b * N;
  const int32_t *tok = a.tokens + (size_t)b * N;
  int32_t *out = a.out_tokens + (size_t)b * N;
  int32_t *path = t.path ? t.path + (size_t)b * N : nullptr;
  const size_t r0 = (size_t)b * a.rps;
  const int zs = min(t.S - 1, ZP);  // staged residual masses per node

  // Two rounds of loads.  First everything indexed by the node alone: parent, token, both
  // rows' status, log2-partition and threshold, the uniform and the first residual masses
  // (whether or not the node turns out to have children).  The node checks count only for
  // a well-formed tree (f1 joins flags after that test).
  unsigned flags = 0, f1 = 0;  // 1 token, 2 row, 4 uniform, 8 q(x) = 0, 16 internal, 32 tree
  int okt_l = 0, okd_l = 0;    // this lane's last node (N <= 64: its only one)
  for (int n = lane; n < N; n += WAVE) {
    const int p = par[n];
    const int x = tok[n];
    const int okt = t.row_ok[r0 + n];
    s_par[n] = p;
    s_tok[n] = x;
    s_nch[n] = 0;
    if (n == 0 ? (p != -1) : (p < 0 || p >= n)) flags |= 32;
    if (n > 0 && (x < 0 || x >= V)) f1 |= 1;
    f1 |= (okt == -2) ? 16 : (okt != 1 ? 2 : 0);
    okt_l = okt;
    if (GREEDY) s_arg[n] = t.row_arg[r0 + n];
    if (!GREEDY) {
      s_lp[n] = (double)t.row_off[r0 + n] + t.row_lt[r0 + n];
      s_lq[n] = (double)t.row_off[r0 + N + n] + t.row_lt[r0 + N + n];  // used only with children
      okd_l = t.row_ok[r0 + N + n];
      const float u = n ? a.u_accept[(size_t)b * N + n] : 0.0f;
      s_ua[n] = u;
      if (n > 0 && !(u >= 0.0f && u < 1.0f)) f1 |= 4;
      const float tt = TOPK ? a.w.row_tau[r0 + n] : -INFINITY;
      s_tau[n] = tt;
      if (tt != tt) f1 |= 16;  // a NaN threshold marks a top-k selection that did not complete
      s_taud[n] = TOPK ? a.w.row_tau[r0 + N + n] : -INFINITY;
      const double *zc = t.zc + ((size_t)b * N + n) * t.S;
      double zv[ZP];
#pragma unroll
      for (int j = 0; j < ZP; ++j) zv[j] = (j < zs) ? zc[j + 1] : 0.0;
#pragma unroll
      for (int j = 0; j < ZP; ++j) s_zp[n * ZP + j] = zv[j];
    }
  }
  if (!GREEDY && lane == 0 && !(a.u_sample[b] >= 0.0f && a.u_sample[b] < 1.0f)) f1 |= 4;
  flags = wave_or(flags);
  lds_sync();
  if (!(flags & 32)) {
    flags |= wave_or(f1);
    for (int n = lane + 1; n < N; n += WAVE) atomicAdd(&s_nch[s_par[n]], 1);
    lds_sync();
    // Then the token logits of every node in its parent's rows (checks passed so far), and
    // the checks that need the children counts.
    const bool gather = !GREEDY && !(flags & 1);
    for (int n = lane; n < N; n += WAVE) {
      float zt = 0.0f, zd = 0.0f;
      const int p = s_par[n], x = s_tok[n];
      if (gather && n > 0) {
        zt = Fmt<T>::at(static_cast<const T *>(seq_row<T>(a, b, p)), (size_t)x);
        zd = Fmt<T>::at(static_cast<const T *>(seq_row<T>(a, b, N + p)), (size_t)x);
      }
      const int nch = s_nch[n];
      if (!GREEDY && nch > t.S) flags |= 32;
      if (!GREEDY && nch > 0) {
        const int okt = (N <= WAVE) ? okt_l : t.row_ok[r0 + n];
        const int okd = (N <= WAVE) ? okd_l : t.row_ok[r0 + N + n];
        flags |= (okd == -2) ? 16 : (okd != 1 ? 2 : 0);
        if (TOPK && s_taud[n] != s_taud[n]) flags |= 16;
        // the residual masses of a node's later children (a NaN marks a wait that gave up)
        if (okt == 1 && okd == 1) {
          const int nz = min(nch, t.S) - 1;
          for (int jj = 1; jj <= nz; ++jj) {
            const double z = (jj <= ZP) ? s_zp[n * ZP + jj - 1] : t.zc[((size_t)b * N + n) * t.S + jj];
            if (!(z >= 0.0) || !isfinite(z)) flags |= 16;
          }
        }
      }
      if (gather && n > 0) {
        s_zt[n] = zt;
        s_zd[n] = zd;
        if (!(zd > -INFINITY) || zd < s_taud[p]) flags |= 8;
      }
    }
    flags = wave_or(flags);
    lds_sync();
  }
  const int err = (flags & 16) ? SV_ROW_INTERNAL
                : (flags & 32) ? SV_ROW_BAD_TREE
                : (flags & 1) ? SV_ROW_BAD_TOKEN
                : (flags & 2) ? SV_ROW_BAD_LOGITS
                : (flags & 4) ? SV_ROW_BAD_UNIFORM
                : (flags & 8) ? SV_ROW_Q_ZERO : 0;
  if (err) {
    if (writer) {
      for (int n = lane; n < N; n += WAVE) {
        out[n] = -1;
        if (path) path[n] = -1;
      }
      if (lane == 0) a.accepted_len[b] = err;
    }
    if (lane == 0) {
      s_res[0] = 0;
      s_res[1] = TJ_NONE;
      s_res[2] = 0;
      *s_c = 0.0;
    }
    lds_sync();
    return;
  }

  // The walk, by the whole wave in step: at each node a ballot over the nodes (64 at a
  // time, in index order) finds its children, whose tests then run in order on values that
  // are the same in every lane (no lane scans the tree alone).
  int u = 0, depth = 0, kind = TJ_NONE;
  double cc = 0.0;
  const double k2 = (double)a.k2;
  for (;;) {
    if (GREEDY) {
      const int am = s_arg[u];
      int next = -1;
      for (int n0 = u + 1; n0 < N && next < 0; n0 += WAVE) {
        const int n = n0 + lane;
        const unsigned long long m = __ballot(n < N && s_par[n] == u && s_tok[n] == am);
        if (m) next = n0 + (int)__ffsll((long long)m) - 1;
      }
      if (writer && lane == 0) out[depth] = am;
      if (next < 0) break;
      if (writer && lane == 0 && path) path[depth] = next;
      ++depth;
      u = next;
      continue;
    }
    const int nch = s_nch[u];
    if (nch == 0) {
      kind = TJ_TARGET;
      break;
    }
    const double lp = s_lp[u], lq = s_lq[u];
    const float tau_t = s_tau[u];
    auto zc_at = [&](int k) {  // Z_k of node u, k = 1 .. min(nch, S) - 1
      return (k <= ZP) ? s_zp[u * ZP + k - 1] : t.zc[((size_t)b * N + u) * t.S + k];
    };
    int k = 0, next = -1;
    // the current distribution is [p - cc q]_+ / cz; (cc, cz) = (0, 1) is p itself
    double cz = 1.0;
    cc = 0.0;
    for (int n0 = u + 1; n0 < N && next < 0 && k < nch; n0 += WAVE) {
      const int n = n0 + lane;
      unsigned long long m = __ballot(n < N && s_par[n] == u);
      while (m && next < 0) {
        const int sn = n0 + (int)__ffsll((long long)m) - 1;
        m &= m - 1ull;
        const float zt = s_zt[sn], zd = s_zd[sn];
        const bool supp_t = (zt > -INFINITY) && !(zt < tau_t);
        const double l2p = (double)zt * k2 - lp, l2q = (double)zd * k2 - lq;
        const double us = (double)s_ua[sn];
        bool accept = false;
        if (cc == 0.0) {
          accept = supp_t && us <= exp2(fmin(0.0, l2p - l2q));
        } else {
          const double ratio = exp2(l2p - l2q);
          accept = supp_t && ratio > cc && us <= fmin(1.0, (ratio - cc) / cz);
        }
        if (accept) {
          next = sn;
          break;
        }
        // rejected: the next distribution is [p - (cc + cz) q]_+ with mass zc[k + 1]
        // (k_tree_resid's round k + 1); a zero mass leaves p itself (as the chain's
        // zero-residual fallback).  After the last child the draw finds the mass.
        cc += cz;
        ++k;
        if (k < nch) {
          const double zk = zc_at(k);
          if (zk > 0.0) {
            cz = zk;
          } else {
            cc = 0.0;
            cz = 1.0;
          }
        }
      }
    }
    if (next < 0) {
      kind = TJ_RESID;
      break;
    }
    if (writer && lane == 0) {
      out[depth] = s_tok[next];
      if (path) path[depth] = next;
    }
    ++depth;
    u = next;
  }
  if (lane == 0) {
    if (writer) a.accepted_len[b] = depth;
    s_res[0] = u;
    s_res[1] = kind;
    s_res[2] = depth;
    *s_c = cc;
  }
  lds_sync();
  if (!writer) return;
  // padding: out[depth] is the final token (the greedy choice, or the draw's), path[depth]
  // onward are not accepted nodes
  for (int n = lane; n < N; n += WAVE) {
    if (n > depth) out[n] = -1;
    if (path && n >= depth) path[n] = -1;
  }
}

// Greedy (T = 0): one wave per tree walks it; nothing is drawn.
template <typename T>
__global__ __launch_bounds__(WAVE) void k_tree_walk(const TreeArgs t) {
  __shared__ int s_res[3];
  __shared__ double s_c;
  tree_walk<T, false, true>(t, (int)blockIdx.x, true, s_res, &s_c);
}

// ---------------------------------------------------------------- k_tree_draw

// Weights of the tree's draw: [p - c q]_+ at a node whose children were all rejected,
// p itself at a leaf (or where the current distribution is p again).  As the chain's
// correction weights: p * max(0, 1 - c q/p), with log2(c q/p) = (z_d - z_t)*k2 - dmc and
// dmc = (Md - Mt) - log2 c, so a draft close to the target keeps relative precision.
struct TreeW {
  float k2, mt_hi, mt_lo, dmc, tau_t, tau_d;
  bool resid;
  SVD float operator()(float zt, float zd) const {
    zt = (zt < tau_t) ? -INFINITY : zt;
    const float p = fast_exp2(fmaf(zt, k2, -mt_hi) - mt_lo);
    if (!resid) return p;
    zd = (zd < tau_d) ? -INFINITY : zd;
    return __fmul_rn(p, one_minus_exp2(fmaf(zd - zt, k2, -dmc)));  // never fused into a sum
  }
};

// Total weight of chunk c by one wave (the rare fallback path), in the segment order of
// wave_chunk_draw.
template <typename T, typename WFn>
SVD double wave_chunk_mass(const Args &a, const T *row, int c, const WFn &wf) {
  constexpr int VEC = Fmt<T>::VEC;
  const int lane = lane_id();
  double tot = 0.0;
  for (int sg = 0; sg < SEGS; ++sg) {
    const int k = sg / NW, w = sg % NW;
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const long idx = elem_index<T>(c, k, w * WAVE + lane, e);
      const bool in = idx < a.V;
      acc += wf(in ? Fmt<T>::at(row, (size_t)(in ? idx : 0)) : -INFINITY, -INFINITY);
    }
    tot += wave_sum((double)acc);
  }
  return tot;
}

template <typename T, bool ALIGNED, bool TOPK>
__global__ __launch_bounds__(NT) void k_tree_draw(const TreeArgs t) {
  const Args &a = t.a;
  int phase, item;
  if (!lane_item(a.B, a.C, 0, phase, item)) return;  // units: trees
  const int lane = lane_id(), wid = threadIdx.x / WAVE;
  const int b = item / a.C, c = item - b * a.C;
  // Every chunk item of the tree walks it (wave 0, the same walk in each); chunk 0's writes
  // the accepted tokens, path and accepted_len.
  __shared__ int s_res[3];
  __shared__ double s_c;
  if (wid == 0) tree_walk<T, TOPK, false>(t, b, c == 0, s_res, &s_c);
  __syncthreads();
  const int kind = s_res[1];
  if (kind == TJ_NONE) return;
  const int u = s_res[0], depth = s_res[2], N = a.G;
  if (u < 0 || u >= N || depth < 0 || depth >= N) return;  // cannot happen: the walk keeps both in range
  const size_t rt = (size_t)b * a.rps + u, rd = rt + N;
  const double cjob = s_c;
  const bool resid = kind == TJ_RESID && cjob > 0.0;  // c = 0: the current distribution is p
  const double lp = (double)t.row_off[rt] + t.row_lt[rt];
  const double lq = resid ? (double)t.row_off[rd] + t.row_lt[rd] : 0.0;
  TreeW wf{a.k2, d_head(lp), d_tail(lp), resid ? (float)((lq - lp) - log2(cjob)) : 0.0f,
           TOPK ? a.w.row_tau[rt] : -INFINITY, (TOPK && resid) ? a.w.row_tau[rd] : -INFINITY, resid};
  const T *row_t = seq_row<T>(a, b, u);
  const T *row_d = resid ? seq_row<T>(a, b, N + u) : nullptr;
  __shared__ double s_seg[SEGS];
  if (resid) chunk_masses<T, ALIGNED, VPT / 2, VPT, true>(a, row_t, row_d, c, 0, wf, s_seg);
  else chunk_masses<T, ALIGNED, VPT, VPT, false>(a, row_t, nullptr, c, 0, wf, s_seg);
  if (wid != 0) return;
  u64 *sw = t.tw_seg + (size_t)b * a.C * SEGS * 2;
  if (c != a.C - 1) {
    for (int i = lane; i < 2 * SEGS; i += WAVE) {
      const double v = s_seg[i >> 1];
      tw_putf(sw + (size_t)c * SEGS * 2 + i, a.tag, (i & 1) ? d_tail(v) : d_head(v));
    }
    return;
  }
  // The tree's last chunk: every segment's mass (earlier chunks' words, its own from LDS),
  // then the segment, lane and element where the cumulative mass passes u * total.
  const int nseg = a.C * SEGS;
  __shared__ double s_all[TREE_DRAW_LDS_SEGS];
  const bool fits = nseg <= TREE_DRAW_LDS_SEGS;
  bool done = false;
  for (unsigned polls = 0; polls < a.spin_limit && !done; ++polls) {
    bool mine = true;
    for (int i = lane; i < (a.C - 1) * SEGS; i += WAVE) {
      const u64 w0 = ld_dev(sw + (size_t)i * 2), w1 = ld_dev(sw + (size_t)i * 2 + 1);
      const bool okw = tw_ok(w0, a.tag) && tw_ok(w1, a.tag);
      mine = mine && okw;
      if (okw && fits) s_all[i] = d_join(tw_f(w0), tw_f(w1));
    }
    done = wave_or(mine ? 0u : 1u) == 0u;
    if (!done) __builtin_amdgcn_s_sleep(2);
  }
  if (!done) {
    if (lane == 0) {
      a.accepted_len[b] = SV_ROW_INTERNAL;
      a.out_tokens[(size_t)b * N + depth] = -1;
    }
    return;
  }
  if (fits)
    for (int i = lane; i < SEGS; i += WAVE) s_all[(a.C - 1) * SEGS + i] = s_seg[i];
  lds_sync();
  auto segm = [&](int i) -> double {
    if (fits) return s_all[i];
    if (i >= (a.C - 1) * SEGS) return s_seg[i - (a.C - 1) * SEGS];
    return d_join(tw_f(ld_dev(sw + (size_t)i * 2)), tw_f(ld_dev(sw + (size_t)i * 2 + 1)));
  };
  const float us = a.u_sample[b];
  double srem = 0.0, total = 0.0;
  int sp = wave_pick_frac(nseg, (double)us, segm, &srem, &total);
  int y = -1;
  if (sp >= 0 && total > 0.0) {
    y = segment_draw<T, ALIGNED>(a, row_t, row_d, sp / SEGS, sp % SEGS, wf, srem);
  } else if (resid) {
    // No residual mass (p and q differ only where p's mass is lost to rounding): draw from
    // p_u, chunk by chunk, as a zero mass before the last child would have.
    TreeW wp = wf;
    wp.resid = false;
    double tot = 0.0;
    for (int cc = 0; cc < a.C; ++cc) tot += wave_chunk_mass<T>(a, row_t, cc, wp);
    double tr = (double)us * tot;
    for (int cc = 0; cc < a.C && y < 0; ++cc) {
      const double m = wave_chunk_mass<T>(a, row_t, cc, wp);
      if (tr < m || cc == a.C - 1) y = wave_chunk_draw<T, ALIGNED>(a, row_t, nullptr, cc, wp, tr);
      else tr -= m;
    }
  }
  if (lane == 0) a.out_tokens[(size_t)b * N + depth] = y;
}

}  // namespace sv

// ======================================================================== host side

namespace {

using namespace sv;
using sv_host::align256;
using sv_host::next_tag;

struct TreePlan {
  bool greedy, topk;
  int esz, nvec, C, I, rps, S;  // I: k_tree_resid items per node
  long long R;
  size_t tw_part, tw_z, tw_seg, tw_hist, row_off, row_lt, row_arg, row_ok, zc, act, act_n,
      row_tau, tk_state, total, zero_bytes;
  bool resid;  // nodes may have two or more children: k_tree_resid runs
  int kmax;    // list slots per tree
};

bool tree_plan(int32_t B, int32_t N, int32_t V, int32_t S, sv_dtype dt, float T, int32_t top_k,
               TreePlan &p) {
  p.greedy = (T == 0.0f);
  p.esz = (dt == SV_BF16) ? 2 : 4;
  const int vec = 16 / p.esz;
  p.nvec = (int)(((long long)V + vec - 1) / vec);
  p.C = (p.nvec + CHUNK_VECS - 1) / CHUNK_VECS;
  p.I = resid_items(p.nvec, false);  // the larger count (unaligned rows)
  p.rps = 2 * N;
  p.R = (long long)B * p.rps;
  p.S = S < 1 ? 1 : S;
  p.resid = p.S > 1 && T != 0.0f;
  p.kmax = N > 2 ? (N - 1) / 2 : 1;
  p.topk = !p.greedy && top_k > 0 && top_k < V;
  const long long lr = (p.R + LANES - 1) / LANES, ln = ((long long)B * N + LANES - 1) / LANES,
                  lb = (B + LANES - 1) / LANES;
  // the items of a node in k_tree_resid wait for one another: at most TREE_MAX_ITEMS of them
  if (!p.greedy && p.S > 1 && p.I > TREE_MAX_ITEMS) return false;
  if (LANES * lr * p.C > 0x7fffffffLL || LANES * ln * (long long)p.I > 0x7fffffffLL ||
      LANES * lb * (long long)p.C > 0x7fffffffLL)
    return false;
  const size_t R = (size_t)p.R, C = (size_t)p.C, Bz = (size_t)B, Nz = (size_t)N, Sz = (size_t)p.S;
  const bool smp = !p.greedy;
  size_t o = 0;
  p.tw_part = o; o = align256(o + R * C * 3 * 8);
  p.tw_z = o; o = align256(o + (smp ? Bz * Nz * (Sz - 1) * (size_t)p.I * 2 * 8 : 0));
  p.tw_seg = o; o = align256(o + (smp ? Bz * C * SEGS * 2 * 8 : 0));
  p.tw_hist = o; o = align256(o + (p.topk ? sv_host::topk_words(p.R, p.C, top_k) * 8 : 0));
  p.zero_bytes = o;
  p.row_off = o; o = align256(o + R * 4);
  p.row_lt = o; o = align256(o + R * 8);
  p.row_arg = o; o = align256(o + R * 4);
  p.row_ok = o; o = align256(o + R * 4);
  p.zc = o; o = align256(o + Bz * Nz * Sz * 8);
  p.act = o; o = align256(o + (p.resid ? Bz * (size_t)p.kmax * 4 : 0));
  p.act_n = o; o = align256(o + (p.resid ? Bz * 4 : 0));
  p.row_tau = o; o = align256(o + (p.topk ? R * 4 : 0));
  p.tk_state = o; o = align256(o + (p.topk ? sv_host::topk_state_bytes(p.R, p.C, top_k) : 0));
  p.total = o;
  return true;
}

bool tree_args_ok(int32_t B, int32_t N, int32_t V, int32_t S, sv_dtype dt, float T) {
  return B >= 1 && N >= 1 && N <= TREE_MAX_NODES && V >= 1 && S >= 0 && S < N + (N == 1) &&
         (dt == SV_F32 || dt == SV_BF16) && T >= 0.0f && isfinite(T);
}

template <typename T, bool AL>
hipError_t tree_launch(const TreePlan &p, const TreeArgs &t0, hipStream_t st, void *const *ev,
                       int nev, int *nl) {
  sv_host::Launcher L{st, ev, nev};
  const long long B = t0.a.B;
  const long long lr = (p.R + LANES - 1) / LANES, lb = (B + LANES - 1) / LANES;
  const long long lk = (B * p.kmax + LANES - 1) / LANES;  // lanes of list slots
  TreeArgs t = t0;
  if (p.topk) sv_host::launch_topk<T, AL>(L, t.a, (unsigned)(LANES * lr * p.C), p.C);
  {
    t.a.tag = next_tag();
    void *args[] = {&t};
    const void *fn = p.greedy ? (const void *)&k_tree_rows<T, AL, false, true>
                   : p.topk ? (const void *)&k_tree_rows<T, AL, true, false>
                            : (const void *)&k_tree_rows<T, AL, false, false>;
    L.go(fn, (unsigned)(LANES * lr * p.C), args);
  }
  if (p.resid) {  // the residual masses of the listed nodes
    t.a.tag = next_tag();
    void *args[] = {&t};
    L.go(p.topk ? (const void *)&k_tree_resid<T, AL, true> : (const void *)&k_tree_resid<T, AL, false>,
         (unsigned)(LANES * lk * resid_items(p.nvec, AL)), args);
  }
  if (p.greedy) {  // the walk alone
    t.a.tag = next_tag();
    void *args[] = {&t};
    L.block = WAVE;
    L.go((const void *)&k_tree_walk<T>, (unsigned)B, args);
    L.block = NT;
  } else {  // the walk, then the draw, in each of the tree's chunk items
    t.a.tag = next_tag();
    void *args[] = {&t};
    L.go(p.topk ? (const void *)&k_tree_draw<T, AL, true> : (const void *)&k_tree_draw<T, AL, false>,
         (unsigned)(LANES * lb * p.C), args);
  }
  if (nl) *nl = L.n;
  return L.e;
}

sv_status tree_run(const void *target, const void *draft, sv_dtype dt, const int32_t *tokens,
                   const int32_t *parent, const float *u_accept, const float *u_sample, int32_t B,
                   int32_t N, int32_t V, int32_t S, float T, int32_t top_k, int32_t *acc,
                   int32_t *out, int32_t *path, void *ws, size_t ws_bytes, void *stream,
                   void *const *ev, int32_t nev, int32_t *nl) {
  if (nl) *nl = 0;
  if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_DTYPE;
  if (B < 1 || N < 1 || N > TREE_MAX_NODES || V < 1 || S < 0 || (N > 1 && S > N - 1)) return SV_ERR_SHAPE;
  if (!(T >= 0.0f) || !isfinite(T)) return SV_ERR_TEMPERATURE;
  TreePlan p;
  if (!tree_plan(B, N, V, S, dt, T, top_k, p)) return SV_ERR_SHAPE;
  const bool smp = !p.greedy;
  if (!target || !tokens || !parent || !acc || !out || !ws) return SV_ERR_NULL;
  if (smp && (!draft || !u_accept || !u_sample)) return SV_ERR_NULL;
  const uintptr_t ta = (uintptr_t)target, da = (uintptr_t)draft;
  if (ta % p.esz || (smp && da % p.esz)) return SV_ERR_ALIGN;
  if (ws_bytes < p.total || ((uintptr_t)ws & 255)) return SV_ERR_WORKSPACE;
  const bool aligned = ((size_t)V * p.esz) % 16 == 0 && ta % 16 == 0 && (!smp || da % 16 == 0);

  char *base = static_cast<char *>(ws);
  TreeArgs t = {};
  Args &a = t.a;
  a.target = target;
  a.draft = draft;
  a.tokens = tokens;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.B = B;
  a.G = N;
  a.V = V;
  a.C = p.C;
  a.nvec = p.nvec;
  a.rps = p.rps;
  a.ntr = N;
  a.tgt_rows = N;
  a.k2 = smp ? (float)(LOG2E / (double)T) : 0.0f;
  a.top_k = top_k;
  a.accepted_len = acc;
  a.out_tokens = out;
  a.spin_limit = SPIN_LIMIT;
  a.w.tw_part = (u64 *)(base + p.tw_part);
  a.w.tw_hist = (u64 *)(base + p.tw_hist);
  a.w.row_tau = (float *)(base + p.row_tau);
  a.w.tk_state = (uint2 *)(base + p.tk_state);
  a.w.tk_rowp = nullptr;
  a.w.tk_keep = nullptr;
  t.parent = parent;
  t.path = path;
  t.S = p.S;
  t.row_off = (float *)(base + p.row_off);
  t.row_lt = (double *)(base + p.row_lt);
  t.row_arg = (int32_t *)(base + p.row_arg);
  t.row_ok = (int32_t *)(base + p.row_ok);
  t.zc = (double *)(base + p.zc);
  t.tw_z = (u64 *)(base + p.tw_z);
  t.tw_seg = (u64 *)(base + p.tw_seg);
  t.act = p.resid ? (int32_t *)(base + p.act) : nullptr;
  t.act_n = p.resid ? (int32_t *)(base + p.act_n) : nullptr;
  t.kmax = p.kmax;

  hipStream_t st = (hipStream_t)stream;
  int n = 0;
  hipError_t e;
  if (dt == SV_BF16)
    e = aligned ? tree_launch<uint16_t, true>(p, t, st, ev, nev, &n) : tree_launch<uint16_t, false>(p, t, st, ev, nev, &n);
  else
    e = aligned ? tree_launch<float, true>(p, t, st, ev, nev, &n) : tree_launch<float, false>(p, t, st, ev, nev, &n);
  if (nl) *nl = n;
  return e == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t sv_tree_workspace_bytes(int32_t B, int32_t N, int32_t V, int32_t max_children, sv_dtype dtype,
                               float temperature, int32_t top_k) {
  TreePlan p;
  if (!tree_args_ok(B, N, V, max_children, dtype, temperature) ||
      !tree_plan(B, N, V, max_children, dtype, temperature, top_k, p))
    return 256;
  return p.total;
}

size_t sv_tree_workspace_zero_bytes(int32_t B, int32_t N, int32_t V, int32_t max_children,
                                    sv_dtype dtype, float temperature, int32_t top_k) {
  TreePlan p;
  if (!tree_args_ok(B, N, V, max_children, dtype, temperature) ||
      !tree_plan(B, N, V, max_children, dtype, temperature, top_k, p))
    return 0;
  return p.zero_bytes;
}

sv_status spec_tree_verify(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                           const int32_t *tokens, const int32_t *parent, const float *u_accept,
                           const float *u_sample, int32_t B, int32_t N, int32_t V,
                           int32_t max_children, float temperature, int32_t top_k,
                           int32_t *accepted_len, int32_t *out_tokens, int32_t *path_nodes,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return tree_run(target_logits, draft_logits, dtype, tokens, parent, u_accept, u_sample, B, N, V,
                  max_children, temperature, top_k, accepted_len, out_tokens, path_nodes, workspace,
                  workspace_bytes, stream, nullptr, 0, nullptr);
}

sv_status spec_tree_verify_timed(const void *target_logits, const void *draft_logits,
                                 sv_dtype dtype, const int32_t *tokens, const int32_t *parent,
                                 const float *u_accept, const float *u_sample, int32_t B,
                                 int32_t N, int32_t V, int32_t max_children, float temperature,
                                 int32_t top_k, int32_t *accepted_len, int32_t *out_tokens,
                                 int32_t *path_nodes, void *workspace, size_t workspace_bytes,
                                 void *stream, void *const *events, int32_t n_events,
                                 int32_t *n_launched) {
  return tree_run(target_logits, draft_logits, dtype, tokens, parent, u_accept, u_sample, B, N, V,
                  max_children, temperature, top_k, accepted_len, out_tokens, path_nodes, workspace,
                  workspace_bytes, stream, events, n_events, n_launched);
}

const char *sv_tree_launch_plan(int32_t B, int32_t N, int32_t V, int32_t max_children,
                                sv_dtype dtype, float temperature, int32_t top_k) {
  (void)B;
  (void)N;
  if (temperature == 0.0f) return "k_tree_rows;k_tree_walk";  // greedy: the walk alone
  const bool topk = top_k > 0 && top_k < V;
  const bool resid = max_children > 1;
  // [threshold: none, one select pass, 2 digit passes (bf16), 4 digit passes (f32)][resid]
  static const char *names[4][2] = {
      {"k_tree_rows;k_tree_draw", "k_tree_rows;k_tree_resid;k_tree_draw"},
      {"k_topk_select;k_topk_merge;k_tree_rows;k_tree_draw",
       "k_topk_select;k_topk_merge;k_tree_rows;k_tree_resid;k_tree_draw"},
      {"k_topk_digit;k_topk_digit;k_tree_rows;k_tree_draw",
       "k_topk_digit;k_topk_digit;k_tree_rows;k_tree_resid;k_tree_draw"},
      {"k_topk_digit;k_topk_digit;k_topk_digit;k_topk_digit;k_tree_rows;k_tree_draw",
       "k_topk_digit;k_topk_digit;k_topk_digit;k_topk_digit;k_tree_rows;k_tree_resid;k_tree_draw"}};
  const int esz = dtype == SV_BF16 ? 2 : 4;
  const int th = !topk ? 0 : sv_host::topk_one_pass(top_k, sv_host::row_chunks(V, esz)) ? 1 : (esz == 2 ? 2 : 3);
  return names[th][resid ? 1 : 0];
}

}  // extern "C"
