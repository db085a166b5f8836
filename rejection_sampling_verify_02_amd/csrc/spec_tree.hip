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
// [([p - c q]_+)/Z - q]_+ = [p - (c + Z) q]_+ / Z).  The walk needs Z_k only after a
// rejection with a later child left, so each tree forms only the masses on its own path,
// when the walk reaches them.
//
// Launches (each data-parallel; results pass through the workspace between launches):
//   k_topk_select, k_topk_merge, or k_topk_digit   (top-k only) every row's threshold.
//   k_tree_rows    per chunk of every target row and of every internal node's draft row:
//                  the normaliser partial (argmax at T = 0); the row's last chunk combines
//                  them into the row's log2-partition (argmax).
//   k_tree_draw    (T > 0) per tree and chunk: every item walks the tree (its first wave
//                  stages checks, gathered logits and row values in LDS; its waves walk in
//                  step; chunk 0's item writes the accepted tokens and path), the tree's
//                  items forming each residual mass the walk needs together, each from
//                  its chunk of the node's two rows; then each item forms the segment
//                  masses of its chunk of the chosen weights ([p - c q]_+ or p), and the
//                  last chunk picks the segment and, in it, the token by inverse CDF with
//                  u_sample.
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
constexpr int TREE_LAZY_MAX_C = 32;    // chunks a row, and draw items a tree, at most when nodes may
                                       // have two or more children

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
  float *node_z;           // [B, N, 2] sampling: node n's token logit in its parent's target and
                           //   draft rows (NaN for a node whose parent or token is out of range)
  // tagged words within one launch
  u64 *tw_seg;             // [B*C*SEGS*2] per tree, chunk and segment: the draw's masses
  u64 *tw_lz;              // [B*2*C*TS*2] residual masses formed by the walk: per tree two
                           //   slots (alternating rounds), per draw item a tagged double
};

// The logits the walk of tree b tests (node n's token in its parent's target and draft
// rows), gathered by one wave into node_z while the rows stream, so that the walk's setup
// loads them with everything else it reads instead of in a second, dependent round.
template <typename T>
SVD void gather_node_logits(const TreeArgs &t, int b) {
  const Args &a = t.a;
  const int N = a.G;
  const int32_t *par = t.parent + (size_t)b * N;
  const int32_t *tok = a.tokens + (size_t)b * N;
  for (int n = lane_id(); n < N; n += WAVE) {
    const int p = (n > 0) ? par[n] : -1;
    const int x = (n > 0) ? tok[n] : -1;
    float zt = NAN, zd = NAN;
    if (p >= 0 && p < n && x >= 0 && x < a.V) {
      zt = Fmt<T>::at(static_cast<const T *>(seq_row<T>(a, b, p)), (size_t)x);
      zd = Fmt<T>::at(static_cast<const T *>(seq_row<T>(a, b, N + p)), (size_t)x);
    }
    t.node_z[((size_t)b * N + n) * 2] = zt;
    t.node_z[((size_t)b * N + n) * 2 + 1] = zd;
  }
}

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
  // The row's last chunk: lanes over chunks, 64 at a time (lane l of block c0 holds chunk
  // c0 + l; this item's own values for chunk c), each block polled until all of its words
  // carry the tag; the largest offset by a wave max, then the sum in chunk order from the
  // lanes' registers (readlane), so no load waits inside the sum.
  const int C = a.C;
  auto block = [&](int c0, float &vo, double &vs) -> bool {
    const int cc = c0 + lane;
    for (unsigned polls = 0; polls < a.spin_limit; ++polls) {
      bool mine = true;
      vo = -INFINITY;
      vs = 0.0;
      if (cc == c) {
        vo = off;
        vs = S;
      } else if (cc < C) {
        const u64 w0 = ld_dev(pw + (size_t)cc * 3), w1 = ld_dev(pw + (size_t)cc * 3 + 1), w2 = ld_dev(pw + (size_t)cc * 3 + 2);
        mine = tw_ok(w0, a.tag) && tw_ok(w1, a.tag) && tw_ok(w2, a.tag);
        vo = tw_f(w0);
        vs = d_join(tw_f(w1), tw_f(w2));
      }
      if (wave_or(mine ? 0u : 1u) == 0u) return true;
      __builtin_amdgcn_s_sleep(2);
    }
    return false;
  };
  bool done = true;
  float o = -INFINITY, vo = -INFINITY;
  double vs = 0.0;
  for (int c0 = 0; c0 < C && done; c0 += WAVE) {
    done = block(c0, vo, vs);
    o = fmaxf(o, wave_max(vo));
  }
  double tt = 0.0;
  for (int c0 = 0; c0 < C && done; c0 += WAVE) {
    if (C > WAVE) block(c0, vo, vs);  // a row of one block keeps its values from the first pass
    const int nb = (C - c0 < WAVE) ? C - c0 : WAVE;
    for (int l = 0; l < nb; ++l) tt += readlane_d(vs, l) * (double)fast_exp2(readlane_f(vo, l) - o);
  }
  if (lane == 0) {
    const bool ok = done && isfinite(o) && isfinite(tt) && tt > 0.0;
    t.row_off[r] = o;
    t.row_lt[r] = ok ? log2(tt) : 0.0;
    t.row_ok[r] = !done ? -2 : (ok ? 1 : 0);
  }
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
    // The last node never has children (a parent precedes its child), so in every
    // well-formed tree this item exists; it gathers the walk's token logits.
    if (!GREEDY && j == 2 * N - 1 && c == 0 && wid == 0) gather_node_logits<T>(t, b);
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
    // the row's last chunk: the other chunks' bests, lanes over chunks 64 at a time (the
    // largest value, lowest index, is the same in any order)
    bool done = true;
    float v = best;
    int vi = bi, f = fl;
    for (int c0 = 0; c0 < a.C - 1 && done; c0 += WAVE) {
      const int cc = c0 + lane;
      done = false;
      for (unsigned polls = 0; polls < a.spin_limit; ++polls) {
        bool mine = true;
        float bv = -INFINITY;
        int bx = 0x7fffffff, bf = 0;
        if (cc < a.C - 1) {
          const u64 w0 = ld_dev(pw + (size_t)cc * 3), w1 = ld_dev(pw + (size_t)cc * 3 + 1), w2 = ld_dev(pw + (size_t)cc * 3 + 2);
          mine = tw_ok(w0, a.tag) && tw_ok(w1, a.tag) && tw_ok(w2, a.tag);
          bv = __uint_as_float((unsigned)w0);
          bx = (int)(unsigned)w1;
          bf = (int)(unsigned)w2;
        }
        if (wave_or(mine ? 0u : 1u) == 0u) {
          wave_best(bv, bx, bf);
          best_combine(v, vi, bv, bx);
          f |= bf;
          done = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (lane == 0) {
      t.row_arg[r] = vi;
      t.row_ok[r] = !done ? -2 : (((f & 1) == 0 && (f & 2)) ? 1 : 0);
    }
    return;
  }

  tree_row_chunk<T, ALIGNED, TOPK>(t, r, row, c);
}

// ---------------------------------------------------------------- k_tree_walk

// What the walk of one tree reads, staged in LDS by its first wave, and the accepted
// nodes it leaves (node[0] = 0, node[d] the node accepted at depth d).
struct WalkLds {
  int par[TREE_MAX_NODES], tok[TREE_MAX_NODES], nch[TREE_MAX_NODES], node[TREE_MAX_NODES];
  float zt[TREE_MAX_NODES], zd[TREE_MAX_NODES], ua[TREE_MAX_NODES], tau[TREE_MAX_NODES], taud[TREE_MAX_NODES];
  double lp[TREE_MAX_NODES], lq[TREE_MAX_NODES];
  int err;
};

// The checks of tree b and everything its walk reads, into W, by one wave in one round of
// loads, everything indexed by the node alone: parent, token, both rows' status,
// log2-partition and threshold, the uniform, and the node's token logits in its parent's
// rows (gathered by the row pass).  The node checks count only for a well-formed tree.
// W.err is the tree's row code, 0 if none.  Greedy: W.lp holds each row's argmax instead.
template <typename T, bool TOPK, bool GREEDY>
SVD void walk_setup(const TreeArgs &t, int b, WalkLds &W) {
  const Args &a = t.a;
  const int lane = lane_id();
  const int N = a.G, V = a.V;
  const int32_t *par = t.parent + (size_t)b * N;
  const int32_t *tok = a.tokens + (size_t)b * N;
  const size_t r0 = (size_t)b * a.rps;
  unsigned flags = 0, f1 = 0;  // 1 token, 2 row, 4 uniform, 8 q(x) = 0, 16 internal, 32 tree
  int okd_l = 0;               // this lane's last node (N <= 64: its only one)
  for (int n = lane; n < N; n += WAVE) {
    const int p = par[n];
    const int x = tok[n];
    const int okt = t.row_ok[r0 + n];
    W.par[n] = p;
    W.tok[n] = x;
    W.nch[n] = 0;
    if (n == 0 ? (p != -1) : (p < 0 || p >= n)) flags |= 32;
    if (n > 0 && (x < 0 || x >= V)) f1 |= 1;
    f1 |= (okt == -2) ? 16 : (okt != 1 ? 2 : 0);
    if (GREEDY) {
      W.lp[n] = (double)t.row_arg[r0 + n];
    } else {
      W.lp[n] = (double)t.row_off[r0 + n] + t.row_lt[r0 + n];
      W.lq[n] = (double)t.row_off[r0 + N + n] + t.row_lt[r0 + N + n];  // used only with children
      okd_l = t.row_ok[r0 + N + n];
      const float u = n ? a.u_accept[(size_t)b * N + n] : 0.0f;
      W.ua[n] = u;
      if (n > 0 && !(u >= 0.0f && u < 1.0f)) f1 |= 4;
      const float tt = TOPK ? a.w.row_tau[r0 + n] : -INFINITY;
      W.tau[n] = tt;
      if (tt != tt) f1 |= 16;  // a NaN threshold marks a top-k selection that did not complete
      W.taud[n] = TOPK ? a.w.row_tau[r0 + N + n] : -INFINITY;
      // the token logits gathered by the row pass (used only for a well-formed tree with
      // every token in range, for which that pass wrote them)
      W.zt[n] = t.node_z[((size_t)b * N + n) * 2];
      W.zd[n] = t.node_z[((size_t)b * N + n) * 2 + 1];
    }
  }
  if (!GREEDY && lane == 0 && !(a.u_sample[b] >= 0.0f && a.u_sample[b] < 1.0f)) f1 |= 4;
  flags = wave_or(flags);
  lds_sync();
  if (!(flags & 32)) {
    flags |= wave_or(f1);
    for (int n = lane + 1; n < N; n += WAVE) atomicAdd(&W.nch[W.par[n]], 1);
    lds_sync();
    const bool gather = !GREEDY && !(flags & 1);
    for (int n = lane; n < N; n += WAVE) {
      const int p = W.par[n];
      const int nch = W.nch[n];
      if (!GREEDY && nch > t.S) flags |= 32;
      if (!GREEDY && nch > 0) {
        const int okd = (N <= WAVE) ? okd_l : t.row_ok[r0 + N + n];
        flags |= (okd == -2) ? 16 : (okd != 1 ? 2 : 0);
        if (TOPK && W.taud[n] != W.taud[n]) flags |= 16;
      }
      if (gather && n > 0) {
        const float zd = W.zd[n];
        if (!(zd > -INFINITY) || zd < W.taud[p]) flags |= 8;
      }
    }
    flags = wave_or(flags);
  }
  if (lane == 0) {
    W.err = (flags & 16) ? SV_ROW_INTERNAL
          : (flags & 32) ? SV_ROW_BAD_TREE
          : (flags & 1) ? SV_ROW_BAD_TOKEN
          : (flags & 2) ? SV_ROW_BAD_LOGITS
          : (flags & 4) ? SV_ROW_BAD_UNIFORM
          : (flags & 8) ? SV_ROW_Q_ZERO : 0;
    W.node[0] = 0;
  }
  lds_sync();
}

struct WalkEnd {
  int u, kind, depth;
  double c;  // the draw's c (kind TJ_RESID)
};

// The walk, by every wave that calls it, in step (every value it uses is the same in
// every lane of every wave): at each node a ballot over the nodes (64 at a time, in index
// order) finds its children, which are tested in order against the current distribution
// [p - cc q]_+ / cz ("Speculative Decoding 的朴素思想", section "Token Tree Verifier").  After
// a rejection with a later child left, zfn(u, cc) gives the next residual's mass
// Z = sum_v [p_u(v) - cc q_u(v)]_+ (NaN if it could not be formed: the walk stops with kind
// TJ_NONE).  Thread 0 records the accepted nodes in W.node.
template <bool GREEDY, typename ZFn>
SVD WalkEnd walk_run(const TreeArgs &t, WalkLds &W, const ZFn &zfn) {
  const int lane = lane_id();
  const int N = t.a.G;
  const double k2 = (double)t.a.k2;
  int u = 0, depth = 0, kind = TJ_NONE;
  double cc = 0.0;
  for (;;) {
    if (GREEDY) {
      const int am = (int)W.lp[u];
      int next = -1;
      for (int n0 = u + 1; n0 < N && next < 0; n0 += WAVE) {
        const int n = n0 + lane;
        const unsigned long long m = __ballot(n < N && W.par[n] == u && W.tok[n] == am);
        if (m) next = n0 + (int)__ffsll((long long)m) - 1;
      }
      if (next < 0) break;
      ++depth;
      if (threadIdx.x == 0) W.node[depth] = next;
      u = next;
      continue;
    }
    const int nch = W.nch[u];
    if (nch == 0) {
      kind = TJ_TARGET;
      break;
    }
    const double lp = W.lp[u], lq = W.lq[u];
    const float tau_t = W.tau[u];
    int k = 0, next = -1;
    bool failed = false;
    // the current distribution is [p - cc q]_+ / cz; (cc, cz) = (0, 1) is p itself
    double cz = 1.0;
    cc = 0.0;
    for (int n0 = u + 1; n0 < N && next < 0 && k < nch && !failed; n0 += WAVE) {
      const int n = n0 + lane;
      unsigned long long m = __ballot(n < N && W.par[n] == u);
      while (m && next < 0 && !failed) {
        const int sn = n0 + (int)__ffsll((long long)m) - 1;
        m &= m - 1ull;
        const float zt = W.zt[sn], zd = W.zd[sn];
        const bool supp_t = (zt > -INFINITY) && !(zt < tau_t);
        const double l2p = (double)zt * k2 - lp, l2q = (double)zd * k2 - lq;
        const double us = (double)W.ua[sn];
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
        // rejected: the next distribution is [p - (cc + cz) q]_+ with mass Z; a zero mass
        // leaves p itself (as the chain's zero-residual fallback).  After the last child
        // the draw finds the mass.
        cc += cz;
        ++k;
        if (k < nch) {
          const double zk = zfn(u, k, cc);
          if (zk != zk) {
            failed = true;
          } else if (zk > 0.0) {
            cz = zk;
          } else {
            cc = 0.0;
            cz = 1.0;
          }
        }
      }
    }
    if (failed) {
      kind = TJ_NONE;
      depth = -1;
      break;
    }
    if (next < 0) {
      kind = TJ_RESID;
      break;
    }
    ++depth;
    if (threadIdx.x == 0) W.node[depth] = next;
    u = next;
  }
  return WalkEnd{u, kind, depth, cc};
}

// The walk's outputs, by one wave: the accepted tokens and path, the padding and
// accepted_len (the greedy final token too; the sampled one is the draw's), or the row
// code err with every output -1.
template <bool GREEDY>
SVD void walk_write(const TreeArgs &t, int b, const WalkLds &W, int depth, int err) {
  const Args &a = t.a;
  const int lane = lane_id(), N = a.G;
  int32_t *out = a.out_tokens + (size_t)b * N;
  int32_t *path = t.path ? t.path + (size_t)b * N : nullptr;
  for (int n = lane; n < N; n += WAVE) {
    if (err) {
      out[n] = -1;
      if (path) path[n] = -1;
      continue;
    }
    if (n < depth) out[n] = GREEDY ? (int)W.lp[W.node[n]] : W.tok[W.node[n + 1]];
    else if (n == depth && GREEDY) out[n] = (int)W.lp[W.node[n]];
    else if (n > depth) out[n] = -1;
    if (path) path[n] = (n < depth) ? W.node[n + 1] : -1;
  }
  if (lane == 0) a.accepted_len[b] = err ? err : depth;
}

// Greedy (T = 0): one wave per tree walks it; nothing is drawn.
template <typename T>
__global__ __launch_bounds__(WAVE) void k_tree_walk(const TreeArgs t) {
  __shared__ WalkLds W;
  const int b = (int)blockIdx.x;
  walk_setup<T, false, true>(t, b, W);
  const int err = W.err;
  int depth = 0;
  if (!err) {
    auto none = [](int, int, double) { return 0.0; };
    depth = walk_run<true>(t, W, none).depth;
    lds_sync();
  }
  walk_write<true>(t, b, W, depth, err);
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

// Sampling (T > 0): the walk and the draw of each tree by its C * TS items, TS = VPT / KS
// to a chunk (item (c, sub) owns vectors sub*KS .. sub*KS + KS - 1 of chunk c of every row
// of the tree, so that small trees still spread over the device).  Every item walks the
// tree (its first wave stages what the walk reads; then all its waves walk in step; the
// first item writes the accepted tokens and path).
// A residual mass is formed when the walk needs it, by all the tree's items together: each
// sums [p_u - c q_u]_+ over its part of node u's two rows (the raw vectors stay in
// registers while the walk stays at u; p and q formed from the rows' log2-partitions as
// the draw forms them), publishes the sum as a tagged double (round r of the call uses tag
// + 1 + r; two slots, alternating by round), and waits for the others' sums of the round;
// every item adds them in item order, so all take the same decisions.  The walk needs
// one mass per rejection before a node's last child, so most nodes never have theirs
// formed.  A tree's items are consecutive blocks of one XCD lane, and they wait for one
// another only when a node has two or more children, which the host allows only for at
// most TREE_LAZY_MAX_C items a tree (every wait is bounded).
// Then the draw: segment masses of the item's part of the chosen weights; the tree's last
// item picks segment, lane and element.
template <typename T, bool ALIGNED, bool TOPK, int KS>
__global__ __launch_bounds__(NT) void k_tree_draw(const TreeArgs t) {
  constexpr int VEC = Fmt<T>::VEC;
  constexpr int TS = VPT / KS;  // items a chunk
  static_assert(KS >= 1 && VPT % KS == 0, "a chunk splits into whole parts");
  const Args &a = t.a;
  int phase, item;
  if (!lane_item(a.B, a.C * TS, 0, phase, item)) return;  // units: trees
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / WAVE;
  const int NI = a.C * TS;  // items a tree
  const int b = item / NI, ii = item - b * NI;  // ii: the item's index in its tree
  const int c = ii / TS, kb = (ii - c * TS) * KS;
  const int N = a.G;
  __shared__ WalkLds W;
  __shared__ double s_w[NW], s_z;
  if (wid == 0) walk_setup<T, TOPK, false>(t, b, W);
  __syncthreads();
  int err = W.err;
  WalkEnd we{0, TJ_NONE, 0, 0.0};
  if (!err) {
    // chunk c of node zu's two rows, loaded at the first mass formed at zu
    int zu = -1, round = 0;
    u32x4 wt[ALIGNED ? KS : 1], wd[ALIGNED ? KS : 1];
    auto zfn = [&](int u, int, double cval) -> double {
      const T *row_t = seq_row<T>(a, b, u), *row_d = seq_row<T>(a, b, N + u);
      if (ALIGNED && zu != u) {
        constexpr unsigned NEG_INF = (sizeof(T) == 2) ? 0xff80ff80u : 0xff800000u;
        const u32x4 *ra = reinterpret_cast<const u32x4 *>(row_t), *rb = reinterpret_cast<const u32x4 *>(row_d);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int v = c * CHUNK_VECS + (kb + kk) * NT + tid;
          const int vs = v < a.nvec ? v : a.nvec - 1;
          wt[ALIGNED ? kk : 0] = ra[vs];
          wd[ALIGNED ? kk : 0] = rb[vs];
        }
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          if (c * CHUNK_VECS + (kb + kk) * NT + tid >= a.nvec) {
            wt[ALIGNED ? kk : 0] = u32x4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
            wd[ALIGNED ? kk : 0] = wt[ALIGNED ? kk : 0];
          }
        zu = u;
      }
      const double lp = W.lp[u], lq = W.lq[u];
      const float mt_hi = d_head(lp), mt_lo = d_tail(lp), md_hi = d_head(lq), md_lo = d_tail(lq);
      const float tau_t = W.tau[u], tau_d = W.taud[u];
      const float k2 = a.k2, cf = (float)cval;
      float acc = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        float za[VEC], zb[VEC], w[VEC];
        if (ALIGNED) {
          Fmt<T>::unpack(wt[ALIGNED ? kk : 0], za);
          Fmt<T>::unpack(wd[ALIGNED ? kk : 0], zb);
        } else {  // a row off the 16-byte grid: the vector built from the two blocks that hold it
          float xa[1][VEC], xb[1][VEC];
          load_vectors<T, false, false, 1>(row_t, a.V, a.nvec, c, kb + kk, tid, xa);
          load_vectors<T, false, false, 1>(row_d, a.V, a.nvec, c, kb + kk, tid, xb);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            za[e] = xa[0][e];
            zb[e] = xb[0][e];
          }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float zt = (TOPK && za[e] < tau_t) ? -INFINITY : za[e];
          const float zd = (TOPK && zb[e] < tau_d) ? -INFINITY : zb[e];
          const float p = fast_exp2(fmaf(zt, k2, -mt_hi) - mt_lo);
          const float q = fast_exp2(fmaf(zd, k2, -md_hi) - md_lo);
          w[e] = fmaxf(fmaf(-cf, q, p), 0.0f);
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
        const unsigned tag = a.tag + 1u + (unsigned)round;
        u64 *zw = t.tw_lz + ((size_t)b * 2 + (round & 1)) * (size_t)NI * 2;
        if (lane < 2) tw_putf(zw + (size_t)ii * 2 + lane, tag, lane ? d_tail(mine) : d_head(mine));
        double z = (double)NAN;
        for (unsigned polls = 0; polls < a.spin_limit; ++polls) {
          bool ready = true;
          double part = 0.0;
          for (int cc = lane; cc < NI; cc += WAVE) {
            const u64 w0 = ld_dev(zw + (size_t)cc * 2), w1 = ld_dev(zw + (size_t)cc * 2 + 1);
            ready = ready && (cc == ii || (tw_ok(w0, tag) && tw_ok(w1, tag)));
            part += (cc == ii) ? mine : d_join(tw_f(w0), tw_f(w1));
          }
          if (wave_or(ready ? 0u : 1u) == 0u) {
            z = wave_sum(part);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) s_z = z;  // NaN: a wait that gave up
      }
      __syncthreads();
      ++round;
      return s_z;
    };
    we = walk_run<false>(t, W, zfn);
    if (we.depth < 0) err = SV_ROW_INTERNAL;  // a mass that could not be formed
    __syncthreads();  // W.node is complete
  }
  if (ii == 0 && wid == 0) walk_write<false>(t, b, W, we.depth, err);
  if (err || we.kind == TJ_NONE) return;
  const int kind = we.kind, u = we.u, depth = we.depth;
  if (u < 0 || u >= N || depth < 0 || depth >= N) return;  // cannot happen: the walk keeps both in range
  const size_t rt = (size_t)b * a.rps + u, rd = rt + N;
  const double cjob = we.c;
  const bool resid = kind == TJ_RESID && cjob > 0.0;  // c = 0: the current distribution is p
  const double lp = W.lp[u];
  const double lq = resid ? W.lq[u] : 0.0;
  TreeW wf{a.k2, d_head(lp), d_tail(lp), resid ? (float)((lq - lp) - log2(cjob)) : 0.0f,
           TOPK ? a.w.row_tau[rt] : -INFINITY, (TOPK && resid) ? a.w.row_tau[rd] : -INFINITY, resid};
  const T *row_t = seq_row<T>(a, b, u);
  const T *row_d = resid ? seq_row<T>(a, b, N + u) : nullptr;
  __shared__ double s_seg[SEGS];
  constexpr int KG = (KS > 4) ? KS / 2 : KS;  // the pair's loads in flight at once
  if (resid) chunk_masses<T, ALIGNED, KG, KS, true>(a, row_t, row_d, c, kb, wf, s_seg);
  else chunk_masses<T, ALIGNED, KS, KS, false>(a, row_t, nullptr, c, kb, wf, s_seg);
  if (wid != 0) return;
  u64 *sw = t.tw_seg + (size_t)b * a.C * SEGS * 2;
  const int own0 = c * SEGS + kb * NW;  // this item's first segment in the tree's order
  if (ii != NI - 1) {
    for (int i = lane; i < 2 * KS * NW; i += WAVE) {
      const double v = s_seg[kb * NW + (i >> 1)];
      tw_putf(sw + (size_t)own0 * 2 + i, a.tag, (i & 1) ? d_tail(v) : d_head(v));
    }
    return;
  }
  // The tree's last item: every segment's mass (the other items' words, its own from
  // LDS), then the segment, lane and element where the cumulative mass passes u * total.
  // The other items' segments precede this item's own: polled in blocks of 256, four
  // consecutive segments a lane, every load of a block issued before any is checked.
  const int nseg = a.C * SEGS;
  __shared__ double s_all[TREE_DRAW_LDS_SEGS];
  const bool fits = nseg <= TREE_DRAW_LDS_SEGS;
  constexpr int SB = 4, BLK = SB * WAVE;
  bool done = true;
  unsigned polls = 0;
  for (int blk = 0; blk < own0 && done; blk += BLK) {
    for (;;) {
      u64 wh[SB], wl[SB];
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const int i = blk + lane * SB + k;
        const int ii = (i < own0) ? i : 0;
        wh[k] = ld_dev(sw + (size_t)ii * 2);
        wl[k] = ld_dev(sw + (size_t)ii * 2 + 1);
      }
      bool ok = true;
#pragma unroll
      for (int k = 0; k < SB; ++k)
        if (blk + lane * SB + k < own0) ok = ok && tw_ok(wh[k], a.tag) && tw_ok(wl[k], a.tag);
      if (__ballot(!ok) == 0) {
        if (fits) {
#pragma unroll
          for (int k = 0; k < SB; ++k) {
            const int i = blk + lane * SB + k;
            if (i < own0) s_all[i] = d_join(tw_f(wh[k]), tw_f(wl[k]));
          }
        }
        break;
      }
      if (++polls >= a.spin_limit) {
        done = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  if (!done) {
    if (lane == 0) {
      a.accepted_len[b] = SV_ROW_INTERNAL;
      a.out_tokens[(size_t)b * N + depth] = -1;
    }
    return;
  }
  if (fits)
    for (int i = lane; i < KS * NW; i += WAVE) s_all[own0 + i] = s_seg[kb * NW + i];
  lds_sync();
  auto segm = [&](int i) -> double {
    if (fits) return s_all[i];
    if (i >= own0) return s_seg[i - (a.C - 1) * SEGS];
    return d_join(tw_f(ld_dev(sw + (size_t)i * 2)), tw_f(ld_dev(sw + (size_t)i * 2 + 1)));
  };
  const float us = a.u_sample[b];
  double srem = 0.0, total = 0.0;
  int sp = wave_pick4_frac(nseg, (double)us, segm, &srem, &total);
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
  int esz, nvec, C, rps, S, ts;  // ts: draw items a chunk
  long long R;
  size_t tw_part, tw_seg, tw_lz, tw_hist, row_off, row_lt, row_arg, row_ok, node_z, row_tau, tk_state, total,
      zero_bytes;
};

bool tree_plan(int32_t B, int32_t N, int32_t V, int32_t S, sv_dtype dt, float T, int32_t top_k,
               TreePlan &p) {
  p.greedy = (T == 0.0f);
  p.esz = (dt == SV_BF16) ? 2 : 4;
  const int vec = 16 / p.esz;
  p.nvec = (int)(((long long)V + vec - 1) / vec);
  p.C = (p.nvec + CHUNK_VECS - 1) / CHUNK_VECS;
  p.rps = 2 * N;
  p.R = (long long)B * p.rps;
  p.S = S < 1 ? 1 : S;
  p.topk = !p.greedy && top_k > 0 && top_k < V;
  const long long lr = (p.R + LANES - 1) / LANES, lb = (B + LANES - 1) / LANES;
  // a tree's draw items wait for one another when a node may have two or more children:
  // then a tree has at most TREE_LAZY_MAX_C of them (4 a chunk where that allows, fewer
  // for longer rows); otherwise 4 a chunk
  if (!p.greedy && p.S > 1 && p.C > TREE_LAZY_MAX_C) return false;
  p.ts = (p.S <= 1 || 4 * p.C <= TREE_LAZY_MAX_C) ? 4 : (2 * p.C <= TREE_LAZY_MAX_C ? 2 : 1);
  if (LANES * lr * p.C > 0x7fffffffLL || LANES * lb * (long long)p.C * p.ts > 0x7fffffffLL) return false;
  const size_t R = (size_t)p.R, C = (size_t)p.C, Bz = (size_t)B;
  const bool smp = !p.greedy;
  size_t o = 0;
  p.tw_part = o; o = align256(o + R * C * 3 * 8);
  p.tw_seg = o; o = align256(o + (smp ? Bz * C * SEGS * 2 * 8 : 0));
  p.tw_lz = o; o = align256(o + (smp ? Bz * 2 * C * (size_t)p.ts * 2 * 8 : 0));
  p.tw_hist = o; o = align256(o + (p.topk ? sv_host::topk_words(p.R, p.C, top_k) * 8 : 0));
  p.zero_bytes = o;
  p.row_off = o; o = align256(o + R * 4);
  p.row_lt = o; o = align256(o + R * 8);
  p.row_arg = o; o = align256(o + R * 4);
  p.row_ok = o; o = align256(o + R * 4);
  p.node_z = o; o = align256(o + (smp ? Bz * (size_t)N * 2 * 4 : 0));
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
  if (p.greedy) {  // the walk alone
    t.a.tag = next_tag();
    void *args[] = {&t};
    L.block = WAVE;
    L.go((const void *)&k_tree_walk<T>, (unsigned)B, args);
    L.block = NT;
  } else {  // the walk (forming the residual masses it needs), then the draw
    t.a.tag = sv_host::next_tag_block((unsigned)t.a.G + 1u);  // the call's tag, then one a round
    void *args[] = {&t};
    const void *fn = p.ts == 4 ? (p.topk ? (const void *)&k_tree_draw<T, AL, true, VPT / 4>
                                         : (const void *)&k_tree_draw<T, AL, false, VPT / 4>)
                   : p.ts == 2 ? (p.topk ? (const void *)&k_tree_draw<T, AL, true, VPT / 2>
                                         : (const void *)&k_tree_draw<T, AL, false, VPT / 2>)
                               : (p.topk ? (const void *)&k_tree_draw<T, AL, true, VPT>
                                         : (const void *)&k_tree_draw<T, AL, false, VPT>);
    L.go(fn, (unsigned)(LANES * lb * p.C * p.ts), args);
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
  a.stamps = nullptr;
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
  t.node_z = smp ? (float *)(base + p.node_z) : nullptr;
  t.tw_seg = (u64 *)(base + p.tw_seg);
  t.tw_lz = smp ? (u64 *)(base + p.tw_lz) : nullptr;

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
  (void)max_children;
  const bool topk = top_k > 0 && top_k < V;
  // [threshold: none, one select pass, 2 digit passes (bf16), 4 digit passes (f32)]
  static const char *names[4] = {"k_tree_rows;k_tree_draw", "k_topk_select;k_topk_merge;k_tree_rows;k_tree_draw",
                                 "k_topk_digit;k_topk_digit;k_tree_rows;k_tree_draw",
                                 "k_topk_digit;k_topk_digit;k_topk_digit;k_topk_digit;k_tree_rows;k_tree_draw"};
  const int esz = dtype == SV_BF16 ? 2 : 4;
  const int th = !topk ? 0 : sv_host::topk_one_pass(top_k, sv_host::row_chunks(V, esz)) ? 1 : (esz == 2 ? 2 : 3);
  return names[th];
}

}  // extern "C"
