"""Seeded synthetic inputs for batched speculative-sampling verification.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no temperature, softmax, top-k cut, acceptance test or
inverse CDF).  Steps of a workload recipe that need that arithmetic -- drawing
the draft tokens from q, or finding the target's top-k set -- are left to the
caller, which passes the result back in (the oracle in tests, the library
itself in the benchmark).

Logits follow the recipe "Zipf prior plus Gaussian noise": for sequence b,
    z_target[b, i, v] = 1.5 * N(0, 1) - 1.1 * ln(rank_b(v) + 1),
where rank_b is one seeded permutation of the vocabulary per sequence (shared by
that sequence's positions), and the draft is the target plus Gaussian noise.
The pages measure on real models and datasets (Vicuna-7B / LLaMA2-Chat on
MT-bench, HumanEval, GSM8K, Alpaca); those are not available, and these
synthetic logits stand in for them.  No benchmark item is reproduced.

bf16 logits are stored as uint16 bit patterns (round-to-nearest-even from f32).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    G: int
    V: int
    dtype: str            # "f32" or "bf16"
    temperature: float
    top_k: int
    draft_noise: float
    seed: int
    notes: str = ""


CONFIGS = {
    1: Config(1, "tiny_chain", 1, 4, 32, "f32", 1.0, 0, 0.5, 1001,
              "target ~ 2*N(0,1), draft = target + 0.5*N(0,1); one worked-example row appended"),
    2: Config(2, "zipf_f32", 8, 5, 32000, "f32", 0.7, 0, 1.0, 1002,
              "Zipf+Gaussian target, draft = target + 1.0*N(0,1)"),
    3: Config(3, "zipf_bf16_b64", 64, 4, 128256, "bf16", 1.0, 0, 0.5, 1003,
              "Zipf+Gaussian target, draft = target + 0.5*N(0,1)"),
    4: Config(4, "greedy_bf16", 256, 7, 152064, "bf16", 0.0, 0, 0.8, 1004,
              "Zipf+Gaussian target, draft = target + 0.8*N(0,1), 1/8 of rows with a planted tie"),
    5: Config(5, "topk_stress", 128, 6, 128256, "bf16", 0.8, 50, 1.5, 1005,
              "three groups: draft == target, draft = target + 1.5*N, disjoint top-k support"),
}

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BF16_NEG_1E4 = int(bf16_bits(np.array([-1e4], np.float32))[0])
# a value above every Zipf+Gaussian logit generated here (|1.5*N(0,1)| stays far below it)
PLANT_BF16 = int(bf16_bits(np.array([24.0], np.float32))[0])


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def zipf_prior(rng: np.random.Generator, V: int) -> np.ndarray:
    """-1.1 * ln(rank + 1) over a seeded random permutation of the vocabulary."""
    rank = rng.permutation(V).astype(np.float32)
    return (-1.1 * np.log(rank + 1.0)).astype(np.float32)


@dataclass
class Raw:
    """Inputs of one call, before the draft tokens are drawn."""
    cfg: Config
    target: np.ndarray            # [B, G+1, V] float32 or uint16 (bf16 bits)
    draft: np.ndarray             # [B, G, V]
    u_draft: np.ndarray           # [B, G] float32 in [0,1): drives the draft's own draw X ~ q
    u_accept: np.ndarray          # [B, G] float32 in [0,1)
    u_sample: np.ndarray          # [B]    float32 in [0,1)
    fixed_tokens: np.ndarray      # [B, G] int32; -1 where the token is still to be drawn
    disjoint_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    tie_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def G(self):
        return self.target.shape[1] - 1

    @property
    def V(self):
        return self.target.shape[2]


def zipf_gauss(B: int, G: int, V: int, dtype: str, draft_noise: float, seed: int,
               *, noise_scale: float = 1.5, block: int = 8) -> tuple[np.ndarray, np.ndarray]:
    """Target [B, G+1, V] and draft [B, G, V] logits, generated a few sequences at a time."""
    rng = np.random.default_rng(seed)
    st = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((B, G + 1, V), st)
    draft = np.empty((B, G, V), st)
    for b0 in range(0, B, block):
        b1 = min(B, b0 + block)
        for b in range(b0, b1):
            prior = zipf_prior(rng, V)
            zt = rng.standard_normal((G + 1, V), dtype=np.float32) * np.float32(noise_scale) + prior
            zd = zt[:G] + rng.standard_normal((G, V), dtype=np.float32) * np.float32(draft_noise)
            target[b] = _store(zt, dtype)
            draft[b] = _store(zd, dtype)
    return target, draft


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.random(shape, dtype=np.float32)


def make_config(cid: int, seed: int | None = None) -> Raw:
    """Raw inputs of one of the five workloads (seed defaults to 1000 + config id)."""
    cfg = CONFIGS[cid]
    seed = cfg.seed if seed is None else seed
    B, G, V = cfg.B, cfg.G, cfg.V
    rng = np.random.default_rng(seed + 7919)
    if cid == 1:
        z = np.random.default_rng(seed)
        zt = (2.0 * z.standard_normal((B, G + 1, V))).astype(np.float32)
        zd = (zt[:, :G] + 0.5 * z.standard_normal((B, G, V))).astype(np.float32)
        # worked two-token row: p = [0.8, 0.2], q = [0.2, 0.8], token 1, U = 0.9
        # ("推测解码：接受规则、状态与收益边界", section "单位置接受 reference")
        ct = np.full((1, G + 1, V), -np.inf, np.float32)
        cd = np.full((1, G, V), -np.inf, np.float32)
        ct[..., 0], ct[..., 1] = np.log(0.8), np.log(0.2)
        cd[..., 0], cd[..., 1] = np.log(0.2), np.log(0.8)
        target = np.concatenate([zt, ct])
        draft = np.concatenate([zd, cd])
        B2 = B + 1
        u_accept = uniforms(rng, (B2, G))
        u_accept[B] = 0.9
        fixed = np.full((B2, G), -1, np.int32)
        fixed[B] = 1
        return Raw(cfg, target, draft, uniforms(rng, (B2, G)), u_accept, uniforms(rng, (B2,)), fixed)

    target, draft = zipf_gauss(B, G, V, cfg.dtype, cfg.draft_noise, seed)
    fixed = np.full((B, G), -1, np.int32)
    raw = Raw(cfg, target, draft, uniforms(rng, (B, G)), uniforms(rng, (B, G)),
              uniforms(rng, (B,)), fixed)
    if cid == 4:
        # In 1/8 of the target rows, write one value above every generated logit at two
        # random indices, so the row's maximum is an exact tie; the draft row of the same
        # position gets the same plant (lowest-index rule decides), and a further 1/16 of
        # draft rows get a plant of their own at other indices.
        nt = B * (G + 1)
        rows = np.sort(rng.choice(nt, size=nt // 8, replace=False))
        raw.tie_rows = rows
        t2, d2 = raw.target.reshape(nt, V), raw.draft.reshape(B * G, V)
        for r in rows:
            i1, i2 = rng.choice(V, size=2, replace=False)
            t2[r, i1] = t2[r, i2] = PLANT_BF16
            b, i = divmod(int(r), G + 1)
            if i < G:
                d2[b * G + i, i1] = d2[b * G + i, i2] = PLANT_BF16
        for r in np.sort(rng.choice(B * G, size=(B * G) // 16, replace=False)):
            i1, i2 = rng.choice(V, size=2, replace=False)
            d2[r, i1] = d2[r, i2] = PLANT_BF16
    if cid == 5:
        # group 1: draft == target bitwise; group 2: noisy draft; group 3: disjoint top-k support
        g1 = B // 3 + (1 if B % 3 else 0)
        g2 = g1 + B // 3 + (1 if B % 3 == 2 else 0)
        raw.draft[:g1] = raw.target[:g1, :G]
        raw.disjoint_rows = np.arange(g2, B)
    return raw


def apply_disjoint_support(raw: Raw, target_keep: np.ndarray) -> None:
    """Set the draft logit to -1e4 wherever the target's kept set is, for the listed rows.

    target_keep [B, G, V] (bool) is the target's top-k set for positions 0..G-1, found
    by the caller.  The draft's own top-k then falls outside it, so its support and the
    target's are disjoint at every position.
    """
    neg = BF16_NEG_1E4 if raw.draft.dtype == np.uint16 else np.float32(-1e4)
    for b in raw.disjoint_rows:
        raw.draft[b][target_keep[b]] = neg


def make_random(B: int, G: int, V: int, dtype: str, seed: int, *, draft_noise: float = 0.7,
                noise_scale: float = 1.5) -> Raw:
    """A Zipf+Gaussian call of any shape (used for ragged and edge-case parity tests)."""
    target, draft = zipf_gauss(B, G, V, dtype, draft_noise, seed, noise_scale=noise_scale)
    rng = np.random.default_rng(seed + 7919)
    cfg = Config(0, f"random_{B}x{G}x{V}_{dtype}", B, G, V, dtype, 1.0, 0, draft_noise, seed)
    return Raw(cfg, target, draft, uniforms(rng, (B, G)), uniforms(rng, (B, G)),
               uniforms(rng, (B,)), np.full((B, G), -1, np.int32))


# ---------------------------------------------------------------- batched sampling

@dataclass(frozen=True)
class SampleConfig:
    name: str
    B: int
    V: int
    dtype: str
    temperature: float
    top_k: int
    seed: int


# One decode step of a batch of 256 sequences over a LLaMA-3-sized vocabulary: the
# draft's X ~ q step, or plain decoding from p.
SAMPLE_CONFIGS = {
    "sample_bf16_b256": SampleConfig("sample_bf16_b256", 256, 128256, "bf16", 1.0, 0, 2001),
}


def make_sample(B: int, V: int, dtype: str, seed: int, *, noise_scale: float = 1.5):
    """Zipf+Gaussian logits [B, V] (one prior per row) and uniforms [B]."""
    target, _ = zipf_gauss(B, 0, V, dtype, 0.0, seed, noise_scale=noise_scale)
    rng = np.random.default_rng(seed + 7919)
    return np.ascontiguousarray(target[:, 0]), uniforms(rng, (B,))


# ---------------------------------------------------------------- draft trees

@dataclass(frozen=True)
class TreeConfig:
    name: str
    B: int
    N: int
    V: int
    dtype: str
    temperature: float
    top_k: int
    max_children: int
    draft_noise: float
    seed: int


# A batch of 16 draft trees of 32 nodes (at most 4 children per node) over a LLaMA-3-sized
# vocabulary: the size of the dynamic trees the EAGLE page describes (tens of nodes per
# round), with the Zipf+Gaussian logits of the chain workloads.
TREE_CONFIGS = {
    "tree_bf16_b16_n32": TreeConfig("tree_bf16_b16_n32", 16, 32, 128256, "bf16", 1.0, 0, 4, 0.5, 3001),
}


@dataclass
class TreeRaw:
    target: np.ndarray   # [B, N, V]: the target's distribution after each node
    draft: np.ndarray    # [B, N, V]: the distribution each node's children are drawn from
    parent: np.ndarray   # [B, N] int32, parent[:, 0] = -1, parent[n] < n
    u_draft: np.ndarray  # [B, N] uniforms for drawing each node's token from its parent's q
    u_accept: np.ndarray  # [B, N]
    u_sample: np.ndarray  # [B]


def random_parents(rng: np.random.Generator, N: int, max_children: int) -> np.ndarray:
    """A random tree in topological order: node n picks its parent among nodes < n that
    still have room, preferring recent (deeper) ones half of the time."""
    parent = np.full(N, -1, np.int32)
    nch = np.zeros(N, np.int64)
    for n in range(1, N):
        room = np.nonzero(nch[:n] < max_children)[0]
        if rng.random() < 0.5:
            p = int(room[-1 - rng.integers(0, min(3, len(room)))])
        else:
            p = int(room[rng.integers(0, len(room))])
        parent[n] = p
        nch[p] += 1
    return parent


def make_tree(B: int, N: int, V: int, dtype: str, seed: int, *, max_children: int = 4,
              draft_noise: float = 0.5, noise_scale: float = 1.5, parents=None) -> TreeRaw:
    """Random trees with Zipf+Gaussian logits at every node (the draft is the target plus
    noise), their uniforms, and the uniforms for drawing node tokens.  Drawing the tokens
    from q is left to the caller."""
    target, draft = zipf_gauss(B, N, V, dtype, draft_noise, seed, noise_scale=noise_scale)
    target = np.ascontiguousarray(target[:, :N])  # N target rows (the generator gives N + 1)
    rng = np.random.default_rng(seed + 7919)
    if parents is None:
        parents = np.stack([random_parents(rng, N, max_children) for _ in range(B)])
    parents = np.ascontiguousarray(np.broadcast_to(np.asarray(parents, np.int32), (B, N)))
    return TreeRaw(target, draft, parents, uniforms(rng, (B, N)), uniforms(rng, (B, N)), uniforms(rng, (B,)))


# ---------------------------------------------------------------- degenerate residuals

# A drafted token whose target logit sits far below the rest of the row (-460, so that
# e^-460 is lost against the row's partition even in double precision) and whose draft
# logit is larger by 1 (f32) or 2 (bf16: -459 is not a bf16 value): p(x) < q(x), and every
# other token has the same logit in both rows.
ZERO_RESIDUAL_LOGITS = {"f32": (-460.0, -459.0), "bf16": (-460.0, -458.0)}


def make_zero_residual(B: int, G: int, V: int, dtype: str, seed: int, *, scale: float = 2.0) -> Raw:
    """Calls whose draft rows equal their target rows except at the drafted token x of each
    position, where the logits are ZERO_RESIDUAL_LOGITS[dtype].  Target rows differ between
    positions (seeded 'scale * N(0, 1)' logits).  Tokens are fixed (fixed_tokens); every
    u_accept is 0.9 and u_sample is U(0, 1)."""
    rng = np.random.default_rng(seed)
    zt = (scale * rng.standard_normal((B, G + 1, V))).astype(np.float32)
    tok = rng.integers(0, V, (B, G)).astype(np.int32)
    zd = zt[:, :G].copy()
    lt, ld = ZERO_RESIDUAL_LOGITS[dtype]
    bi, gi = np.meshgrid(np.arange(B), np.arange(G), indexing="ij")
    zt[bi, gi, tok] = lt
    zd[bi, gi, tok] = ld
    cfg = Config(0, f"zero_residual_{B}x{G}x{V}_{dtype}", B, G, V, dtype, 1.0, 0, 0.0, seed)
    ua = np.full((B, G), 0.9, np.float32)
    return Raw(cfg, _store(zt, dtype), _store(zd, dtype), np.zeros((B, G), np.float32), ua,
               uniforms(rng, (B,)), tok)
