"""Statistical pins of the oracle: the law of the output and the accepted length.

* The output of a round is distributed exactly as the target ("Speculative
  Decoding 的朴素思想", section "Correction 为什么用正残差"; tannlonggtaoo note,
  section "验证方式：reject sampling").  Pinned three ways on V <= 4: exact
  rational enumeration of the method on Markov toy models equals the target's
  autoregressive law; a stratified sweep of the oracle's uniforms reproduces p;
  a Monte Carlo chi-square of the oracle's emitted tokens against that law.
* Expected tokens per round with a constant acceptance rate a is
  (1 - a^(gamma+1)) / (1 - a) ("推测解码：接受规则、状态与收益边界", section
  "接受长度与速度模型"), and with a position profile alpha_i it is
  1 + sum_i prod_{j<=i} alpha_j ("LLM 推测解码精读笔记 · 04 EAGLE", section 8 and
  exercise 2 of section 14; values in tests/golden/eagle_expected_output.json).
"""
import itertools
import json
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle

GOLD = Path(__file__).resolve().parent / "golden"


def logits_of(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, np.float64)).astype(np.float32)


# ------------------------------------------------------------- accepted length

def constant_rate_rows(alphas, n, seed):
    """Positions whose acceptance probability is exactly alpha_i for every drafted token.

    p_i = (a/2, a/2, (1-a)/2, (1-a)/2), q_i = (1/2, 1/2, 0, 0): the draft only
    proposes tokens 0 or 1, and p(x)/q(x) = a for both.
    """
    G = len(alphas)
    rng = np.random.default_rng(seed)
    t = np.empty((n, G + 1, 4), np.float32)
    for i, a in enumerate(list(alphas) + [0.5]):
        t[:, i] = logits_of([a / 2, a / 2, (1 - a) / 2, (1 - a) / 2])
    d = np.broadcast_to(logits_of([0.5, 0.5, 0.0, 0.0]), (n, G, 4)).copy()
    x = rng.integers(0, 2, (n, G)).astype(np.int32)
    ua = rng.random((n, G), dtype=np.float32)
    us = rng.random(n, dtype=np.float32)
    return t, d, x, ua, us


@pytest.mark.parametrize("a,G", [(0.3, 4), (0.6, 4), (0.8, 5), (0.95, 7)])
def test_expected_tokens_constant_rate(a, G):
    """mean(accepted+1) = (1-a^(G+1))/(1-a); mean(accepted) = a(1-a^G)/(1-a); law truncated geometric."""
    n = 200_000
    t, d, x, ua, us = constant_rate_rows([a] * G, n, seed=int(a * 1000) + G)
    acc, out = oracle.spec_verify_ref(t, d, x, ua, us, 1.0)
    k = np.arange(G + 1)
    law = np.where(k < G, a ** k * (1 - a), a ** G)
    mean_k = float(np.sum((k + 1) * law))
    assert abs(mean_k - (1 - a ** (G + 1)) / (1 - a)) < 1e-12
    assert abs(float(np.sum(k * law)) - a * (1 - a ** G) / (1 - a)) < 1e-12
    sd = np.sqrt(np.sum((k + 1 - mean_k) ** 2 * law))
    assert abs(np.mean(acc + 1) - mean_k) < 5 * sd / np.sqrt(n)
    counts = np.bincount(acc, minlength=G + 1)
    assert scipy.stats.chisquare(counts, n * law).pvalue > 1e-3


def test_expected_tokens_position_profiles():
    """E[N] = 1 + sum_i prod_{j<=i} alpha_j on the printed profiles (3.53, 2.176, 3.908, 2.306)."""
    g = json.loads((GOLD / "eagle_expected_output.json").read_text())
    n = 200_000
    for ci, case in enumerate(g["cases"]):
        al = case["alpha"]
        expect = 1 + sum(np.prod(al[: i + 1]) for i in range(len(al)))
        assert round(expect, 3) == case["E_N"]
        t, d, x, ua, us = constant_rate_rows(al, n, seed=100 + ci)
        acc, _ = oracle.spec_verify_ref(t, d, x, ua, us, 1.0)
        G = len(al)
        law = [(1 - al[k]) * np.prod(al[:k]) if k < G else np.prod(al) for k in range(G + 1)]
        sd = np.sqrt(sum((k + 1 - expect) ** 2 * law[k] for k in range(G + 1)))
        assert abs(np.mean(acc + 1) - expect) < 5 * sd / np.sqrt(n)


def test_first_position_acceptance_rate_is_overlap():
    """Pr(accept) = sum_x min(p(x), q(x)) = 1 - TV(p, q) (MC at one position)."""
    rng = np.random.default_rng(31)
    V, n = 4, 200_000
    p = np.array([0.1, 0.4, 0.3, 0.2])
    q = np.array([0.4, 0.1, 0.25, 0.25])
    t = np.broadcast_to(np.stack([logits_of(p)] * 2), (n, 2, V)).copy()
    d = np.broadcast_to(logits_of(q), (n, 1, V)).copy()
    x = oracle.sample_rows(d, rng.random((n, 1), dtype=np.float32), 1.0)
    acc, _ = oracle.spec_verify_ref(t, d, x, rng.random((n, 1), dtype=np.float32),
                                    rng.random(n, dtype=np.float32), 1.0)
    beta = np.sum(np.minimum(p, q))
    assert abs(beta - (1 - 0.5 * np.abs(p - q).sum())) < 1e-15
    assert abs(np.mean(acc == 1) - beta) < 5 * np.sqrt(beta * (1 - beta) / n)


# ------------------------------------------------------------- exact law (Fractions)

P_TAB = [[Fraction(1, 2), Fraction(1, 4), Fraction(1, 8), Fraction(1, 8)],
         [Fraction(1, 10), Fraction(3, 10), Fraction(3, 5), Fraction(0)],
         [Fraction(1, 4), Fraction(1, 4), Fraction(1, 4), Fraction(1, 4)],
         [Fraction(0), Fraction(1, 3), Fraction(1, 3), Fraction(1, 3)]]
Q_TAB = [[Fraction(1, 5), Fraction(1, 5), Fraction(1, 5), Fraction(2, 5)],
         [Fraction(1, 2), Fraction(0), Fraction(1, 4), Fraction(1, 4)],
         [Fraction(7, 10), Fraction(1, 10), Fraction(1, 10), Fraction(1, 10)],
         [Fraction(1, 4), Fraction(1, 4), Fraction(1, 2), Fraction(0)]]


def exact_round_law(p_tab, q_tab, s0, G):
    """Exact law of the tokens one round emits, from the method written in rationals.

    Enumerates every draft chain x_1..x_G with weight prod q(x_i | x_{i-1}), then the
    accept / reject branches: accept x_i with probability min(1, p/q); on the first
    rejection emit a draw from norm([p - q]_+); after G acceptances emit a bonus from
    p(. | x_G).  Returns {emitted tuple: probability}.
    """
    V = len(p_tab)
    law = {}

    def add(key, w):
        law[key] = law.get(key, Fraction(0)) + w

    def walk(prefix_tokens, last, w, depth):
        if depth == G:
            for y in range(V):
                if p_tab[last][y]:
                    add(tuple(prefix_tokens) + (y,), w * p_tab[last][y])
            return
        p, q = p_tab[last], q_tab[last]
        res = [max(p[v] - q[v], Fraction(0)) for v in range(V)]
        Z = sum(res)
        for x in range(V):
            if q[x] == 0:
                continue
            alpha = min(Fraction(1), p[x] / q[x])
            if alpha:
                walk(prefix_tokens + [x], x, w * q[x] * alpha, depth + 1)
            if alpha < 1:
                for y in range(V):
                    if res[y]:
                        add(tuple(prefix_tokens) + (y,), w * q[x] * (1 - alpha) * res[y] / Z)

    walk([], s0, Fraction(1), 0)
    return law


def ar_law(p_tab, s0, L):
    """Target's own autoregressive law of the next L tokens."""
    V = len(p_tab)
    out = {}
    for seq in itertools.product(range(V), repeat=L):
        w, last = Fraction(1), s0
        for y in seq:
            w *= p_tab[last][y]
            last = y
        if w:
            out[seq] = w
    return out


def marginal_first_tokens(round_law, p_tab, L):
    """Law of the first L emitted tokens when rounds continue until L are out."""
    out = {}

    def extend(prefix, w):
        if len(prefix) >= L:
            key = prefix[:L]
            out[key] = out.get(key, Fraction(0)) + w
            return
        for tail, wt in exact_round_law(p_tab, Q_TAB, prefix[-1], 2).items():
            extend(prefix + tail, w * wt)

    for seq, w in round_law.items():
        extend(seq, w)
    return out


@pytest.mark.parametrize("G", [1, 2, 3])
def test_exact_enumeration_equals_target_law(G):
    """Rational enumeration of the method: emitted tokens follow p exactly (first 2 tokens)."""
    for s0 in range(4):
        rl = exact_round_law(P_TAB, Q_TAB, s0, G)
        assert sum(rl.values()) == 1
        first = {}
        for seq, w in rl.items():
            first[seq[0]] = first.get(seq[0], Fraction(0)) + w
        assert first == {y: P_TAB[s0][y] for y in range(4) if P_TAB[s0][y]}
        assert marginal_first_tokens(rl, P_TAB, 2) == ar_law(P_TAB, s0, 2)


def test_exact_enumeration_detects_wrong_correction():
    """Control: correcting from p instead of [p - q]_+ breaks the equality."""
    bad_q = Q_TAB
    rl = exact_round_law(P_TAB, bad_q, 0, 1)
    # rebuild with the wrong correction rule
    p, q = P_TAB[0], bad_q[0]
    wrong = {}
    for x in range(4):
        if q[x] == 0:
            continue
        a = min(Fraction(1), p[x] / q[x])
        wrong[x] = wrong.get(x, Fraction(0)) + q[x] * a
        for y in range(4):
            wrong[y] = wrong.get(y, Fraction(0)) + q[x] * (1 - a) * p[y]
    assert {y: wrong[y] for y in wrong if wrong[y]} != {y: P_TAB[0][y] for y in range(4) if P_TAB[0][y]}
    assert rl  # the right rule was built from the same tables


# ------------------------------------------------------------- the oracle's law

def tables_as_logits(tab):
    return np.array([[float(v) for v in row] for row in tab])


def policy_probs(tab, T, k):
    """Processed distributions of each table row (temperature, top-k) in float64."""
    w = tables_as_logits(tab)
    z = np.full((4, 4), -np.inf)
    z[w > 0] = np.log(w[w > 0])
    out = np.zeros((4, 4))
    for r in range(4):
        keep = np.isfinite(z[r])
        if 0 < k < 4:
            keep &= z[r] >= np.sort(z[r])[::-1][k - 1]
        out[r, keep] = scipy.special.softmax(z[r, keep] / T)
    return out, z.astype(np.float32)


def run_rounds(zp, zq, s0, G, T, k, rng):
    """One round per entry of s0 (prefix token), drafts drawn from q with the oracle's sampler."""
    n = len(s0)
    x = np.empty((n, G), np.int32)
    last = s0.copy()
    drows = np.empty((n, G, 4), np.float32)
    trows = np.empty((n, G + 1, 4), np.float32)
    for i in range(G):
        drows[:, i] = zq[last]
        trows[:, i] = zp[last]
        x[:, i] = oracle.sample_rows(drows[:, i], rng.random(n, dtype=np.float32), T, k)
        last = x[:, i]
    trows[:, G] = zp[last]
    return oracle.spec_verify_ref(trows, drows, x, rng.random((n, G), dtype=np.float32),
                                  rng.random(n, dtype=np.float32), T, k)


@pytest.mark.parametrize("T,k", [(1.0, 0), (0.7, 0), (1.0, 2), (1.3, 3)])
def test_monte_carlo_law_matches_target(T, k):
    """Chi-square of the oracle's first and first-two emitted tokens against p (V=4, G=3)."""
    rng = np.random.default_rng(int(T * 100) + k)
    Pp, zp = policy_probs(P_TAB, T, k)
    _, zq = policy_probs(Q_TAB, T, k)
    n, G = 200_000, 3
    s0 = np.zeros(n, np.int64)
    acc, out = run_rounds(zp, zq, s0, G, T, k, rng)
    assert np.all(acc >= 0)
    y1 = out[:, 0].astype(np.int64)
    y2 = np.where(acc >= 1, out[:, 1], -1).astype(np.int64)
    need = y2 < 0
    acc2, out2 = run_rounds(zp, zq, y1[need], G, T, k, rng)
    y2[need] = out2[:, 0]
    # first token
    sup = Pp[0] > 0
    c1 = np.bincount(y1, minlength=4)
    assert np.all(c1[~sup] == 0)
    assert scipy.stats.chisquare(c1[sup], n * Pp[0][sup]).pvalue > 1e-3
    # first two tokens
    joint = Pp[0][:, None] * Pp
    sup2 = joint.ravel() > 0
    c2 = np.bincount(y1 * 4 + y2, minlength=16)
    assert np.all(c2[~sup2] == 0)
    assert scipy.stats.chisquare(c2[sup2], n * joint.ravel()[sup2]).pvalue > 1e-3


@pytest.mark.parametrize("G", [1, 2])
def test_stratified_sweep_of_uniforms_reproduces_p(G):
    """Every draft chain x weighted by q, uniforms on a midpoint grid: the first emitted
    token's law is p(. | s0) up to the grid's resolution."""
    _, zp = policy_probs(P_TAB, 1.0, 0)
    _, zq = policy_probs(Q_TAB, 1.0, 0)
    n = 60 if G == 2 else 400
    cells = (np.arange(n) + 0.5) / n
    total = np.zeros(4)
    for s0 in [0, 1]:
        total[:] = 0
        for chain in itertools.product(range(4), repeat=G):
            w, last = 1.0, s0
            for xi in chain:
                w *= float(Q_TAB[last][xi])
                last = xi
            if w == 0:
                continue
            grids = np.meshgrid(*([cells] * (G + 1)), indexing="ij")
            us = [g.ravel().astype(np.float32) for g in grids]
            m = us[0].size
            trows = np.empty((m, G + 1, 4), np.float32)
            drows = np.empty((m, G, 4), np.float32)
            last = s0
            for i, xi in enumerate(chain):
                trows[:, i] = zp[last]
                drows[:, i] = zq[last]
                last = xi
            trows[:, G] = zp[last]
            x = np.broadcast_to(np.array(chain, np.int32), (m, G)).copy()
            ua = np.stack(us[:G], axis=1)
            acc, out = oracle.spec_verify_ref(trows, drows, x, ua, us[G], 1.0)
            total += w * np.bincount(out[:, 0], minlength=4) / m
        expect = np.array([float(v) for v in P_TAB[s0]])
        np.testing.assert_allclose(total, expect, atol=4.0 / n)
