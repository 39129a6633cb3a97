"""Pins of the fp64 oracle against things other than itself: library routines,
exact binary boundaries, closed forms, special cases and an exact-rational
second implementation.  Citations: wikillm.com card for arXiv 2302.01318,
Method ("Modified rejection sampling", paper sec. 4.2; "Algorithm: Speculative
Sampling (SpS)", alg. 2; "Decoding transforms") and Pitfalls."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import special

import oracle
from oracle import micro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even) and return the raw uint16 bits."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- softmax row

@pytest.mark.parametrize("T", [0.5, 0.8, 1.0, 2.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_softmax_row_matches_scipy(T, dtype):
    rng = np.random.default_rng(11)
    V = 1000
    z = (3 * rng.standard_normal(V) - 1.1 * np.log(rng.permutation(V) + 1.0)).astype(np.float32)
    if dtype == "bf16":
        row = bf16_bits(z)
        zf = bf16_to_f64(row)
    else:
        row = z
        zf = z.astype(np.float64)
    T = float(np.float32(T))
    prob, M, S = oracle.softmax_row(row, T)
    ref = special.softmax(zf / T)
    np.testing.assert_allclose(prob, ref, rtol=1e-13, atol=0)
    assert M == np.max(zf / T)
    assert abs((M + math.log(S)) - special.logsumexp(zf / T)) < 1e-12


def test_softmax_row_masks_and_invalid_rows():
    z = np.array([0.0, -np.inf, 1.0, -np.inf], np.float32)
    prob, M, S = oracle.softmax_row(z, 1.0)
    assert prob[1] == 0.0 and prob[3] == 0.0
    np.testing.assert_allclose(prob[[0, 2]], special.softmax([0.0, 1.0]), rtol=1e-15)
    assert oracle.softmax_row(np.array([0.0, np.nan], np.float32), 1.0) is None
    assert oracle.softmax_row(np.full(4, -np.inf, np.float32), 1.0) is None
    assert oracle.softmax_row(np.array([0.0, np.inf], np.float32), 1.0) is None


# ---------------------------------------------------------------- accept test

def test_accept_strict_inequality_at_exact_boundary():
    # rho = 0.25/0.5 = 0.5 exactly; u == rho must reject (strict <).
    assert oracle.accept(0.25, 0.5, 0.5) == (False, 0.0)
    acc, d = oracle.accept(0.25, 0.5, 0.5 - 2.0 ** -24)
    assert acc and d == 2.0 ** -24
    # rho >= 1 always accepts for u in [0, 1).
    assert oracle.accept(0.5, 0.25, 1.0 - 2.0 ** -24)[0]
    assert oracle.accept(0.3, 0.3, 1.0 - 2.0 ** -24)[0]
    # q == 0 < p: never accept, not even u == 0.
    assert not oracle.accept(0.0, 0.5, 0.0)[0]
    # p == 0 < q: ratio +inf, always accept; p == q == 0: reject.
    assert oracle.accept(0.1, 0.0, 1.0 - 2.0 ** -24) == (True, math.inf)
    assert not oracle.accept(0.0, 0.0, 0.0)[0]


# ---------------------------------------------------------------- inverse CDF

def test_inverse_cdf_exact_breakpoints():
    w = np.array([0.25, 0.0, 0.5, 0.25])
    assert oracle.inverse_cdf(w, 0.0)[0] == 0
    # u*S exactly at C(0): strict '>' moves on, and skips the zero-weight token.
    assert oracle.inverse_cdf(w, 0.25)[0] == 2
    assert oracle.inverse_cdf(w, 0.75)[0] == 3
    assert oracle.inverse_cdf(w, 1.0 - 2.0 ** -24)[0] == 3
    x, d = oracle.inverse_cdf(w, 0.5)
    assert x == 2 and d == 0.25
    assert oracle.inverse_cdf(np.zeros(3), 0.5)[0] == -1


def test_inverse_cdf_matches_numpy_searchsorted():
    rng = np.random.default_rng(5)
    for trial in range(50):
        V = int(rng.integers(1, 300))
        w = rng.exponential(size=V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[0] = 1.0
        c = np.cumsum(w)  # sequential partial sums, as the oracle adds them
        for u in rng.integers(0, 1 << 24, 40) * 2.0 ** -24:
            x, _ = oracle.inverse_cdf(w, u)
            assert x == int(np.searchsorted(c, u * c[-1], side="right"))
            assert w[x] > 0


# ---------------------------------------------------------------- residual

def test_residual_weights_closed_form():
    rng = np.random.default_rng(2)
    for _ in range(20):
        V = int(rng.integers(2, 500))
        q = special.softmax(rng.standard_normal(V) * 2)
        p = special.softmax(rng.standard_normal(V) * 2)
        w, fell_back = oracle.residual_weights(q, p)
        assert not fell_back
        np.testing.assert_array_equal(w, np.maximum(0.0, q - p))
        # sum (q-p)_+ = 1 - sum min(p, q) = total variation distance
        tv = 0.5 * np.abs(q - p).sum()
        assert abs(w.sum() - (1.0 - np.minimum(p, q).sum())) < 1e-14
        assert abs(w.sum() - tv) < 1e-14


def test_residual_zero_mass_falls_back_to_q():
    q = special.softmax(np.arange(5.0))
    w, fell_back = oracle.residual_weights(q, q.copy())
    assert fell_back
    np.testing.assert_array_equal(w, q)


# ---------------------------------------------------------------- full verify

def _rows(rng, B, K, V, mask_frac=0.0, dtype="f32"):
    tgt = (2.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    dft = (tgt[:, :K] + 0.7 * rng.standard_normal((B, K, V))).astype(np.float32)
    if mask_frac:
        tgt[rng.random(tgt.shape) < mask_frac] = -np.inf
        dft[rng.random(dft.shape) < mask_frac] = -np.inf
        tgt[..., 0] = 0.0
        dft[..., 0] = 0.0
    if dtype == "bf16":
        return bf16_bits(tgt), bf16_bits(dft)
    return tgt, dft


def _sample_tokens(rng, dft_probs):
    B, K, V = dft_probs.shape
    return np.array([[rng.choice(V, p=dft_probs[b, t]) for t in range(K)] for b in range(B)],
                    np.int32)


def _row_probs(rows, T):
    return np.stack([np.stack([oracle.softmax_row(r, T)[0] for r in seq]) for seq in rows])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_equals_rowwise_softmax_plus_verify_dists(dtype):
    """The batched entry point slices rows [b][t] correctly: it must agree with
    softmax of each explicitly sliced row followed by the distribution-level
    verify."""
    rng = np.random.default_rng(3)
    B, K, V, T = 6, 3, 40, float(np.float32(0.8))
    tgt, dft = _rows(rng, B, K, V, mask_frac=0.1, dtype=dtype)
    qp = _row_probs(tgt, T)
    pp = _row_probs(dft, T)
    tokens = _sample_tokens(rng, pp)
    uni = (rng.integers(0, 1 << 24, (B, K + 1)) * 2.0 ** -24).astype(np.float32)
    out = oracle.verify(tgt, dft, tokens, uni, T)
    for b in range(B):
        ref = oracle.verify_dists(qp[b], pp[b], tokens[b:b + 1], uni[b:b + 1])
        assert out["num_accepted"][b] == ref["num_accepted"][0]
        np.testing.assert_array_equal(out["out_tokens"][b], ref["out_tokens"][0])
        assert out["draw_kind"][b] == ref["draw_kind"][0]
        for t in range(K):
            assert out["probs"][b, t, 0] == qp[b, t, tokens[b, t]]
            assert out["probs"][b, t, 1] == pp[b, t, tokens[b, t]]
    assert np.all(out["num_emitted"] == out["num_accepted"] + 1)


def test_invariants_random_tiny_cases():
    """Each loop emits between 1 and K+1 tokens; the emitted prefix is the
    drafted prefix; the final token carries positive mass under the law it was
    drawn from (paper sec. 4.2)."""
    rng = np.random.default_rng(4)
    for trial in range(200):
        K = int(rng.integers(1, 7))
        V = int(rng.integers(2, 65))
        T = float(np.float32(rng.choice([0.5, 0.8, 1.0, 1.7])))
        tgt, dft = _rows(rng, 1, K, V, mask_frac=rng.choice([0.0, 0.3]))
        qp = _row_probs(tgt, T)[0]
        pp = _row_probs(dft, T)[0]
        tokens = _sample_tokens(rng, pp[None])
        uni = (rng.integers(0, 1 << 24, (1, K + 1)) * 2.0 ** -24).astype(np.float32)
        o = oracle.verify(tgt, dft, tokens, uni, T)
        n = int(o["num_accepted"][0])
        assert 0 <= n <= K and o["num_emitted"][0] == n + 1
        out = o["out_tokens"][0]
        assert list(out[:n]) == list(tokens[0, :n])
        assert np.all(out[n + 1:] == -1)
        x = out[n]
        if o["draw_kind"][0] == 0:
            assert qp[n, x] > pp[n, x]
        else:
            assert qp[n, x] > 0
        assert o["draw_kind"][0] == (1 if n == K else 0)


def test_equal_distributions_accept_everything_and_bonus_is_categorical():
    """p == q: every ratio is 1 so every token is accepted, and the bonus token
    is a plain categorical draw from the last target row (numpy searchsorted)."""
    rng = np.random.default_rng(7)
    B, K, V, T = 64, 4, 50, 1.0
    tgt, _ = _rows(rng, B, K, V)
    dft = np.ascontiguousarray(tgt[:, :K])
    pp = _row_probs(dft, T)
    tokens = _sample_tokens(rng, pp)
    uni = (rng.integers(0, 1 << 24, (B, K + 1)) * 2.0 ** -24).astype(np.float32)
    o = oracle.verify(tgt, dft, tokens, uni, T)
    assert np.all(o["num_accepted"] == K)
    assert np.all(o["draw_kind"] == 1)
    for b in range(B):
        c = np.cumsum(oracle.softmax_row(tgt[b, K], T)[0])
        assert o["out_tokens"][b, K] == np.searchsorted(c, float(uni[b, K]) * c[-1], side="right")


def test_disjoint_supports_reject_first_and_resample_from_q():
    """Draft mass only where the target has none: q(x~)=0 so the first test
    rejects, and (q-p)_+ = q, a plain categorical draw from q_0."""
    rng = np.random.default_rng(8)
    B, K, V = 32, 3, 20
    tgt = np.full((B, K + 1, V), -np.inf, np.float32)
    dft = np.full((B, K, V), -np.inf, np.float32)
    tgt[:, :, :10] = rng.standard_normal((B, K + 1, 10))
    dft[:, :, 10:] = rng.standard_normal((B, K, 10))
    pp = _row_probs(dft, 1.0)
    tokens = _sample_tokens(rng, pp)
    uni = (rng.integers(0, 1 << 24, (B, K + 1)) * 2.0 ** -24).astype(np.float32)
    o = oracle.verify(tgt, dft, tokens, uni, 1.0)
    assert np.all(o["num_accepted"] == 0)
    for b in range(B):
        c = np.cumsum(oracle.softmax_row(tgt[b, 0], 1.0)[0])
        assert o["out_tokens"][b, 0] == np.searchsorted(c, float(uni[b, K]) * c[-1], side="right")


def test_one_hot_rows_reduce_to_greedy_rule():
    """One-hot p and q (every other logit -inf): the general accept test then
    becomes a match of the two rows' single supported tokens, and the residual
    at the first mismatch puts all its mass on the target row's token (card's
    Pitfalls, greedy mode)."""
    rng = np.random.default_rng(9)
    K, V = 5, 16
    for trial in range(100):
        a_q = rng.integers(0, V, K + 1)
        a_p = np.where(rng.random(K) < 0.6, a_q[:K], rng.integers(0, V, K))
        tgt = np.full((1, K + 1, V), -np.inf, np.float32)
        dft = np.full((1, K, V), -np.inf, np.float32)
        tgt[0, np.arange(K + 1), a_q] = 1.0
        dft[0, np.arange(K), a_p] = 1.0
        uni = (rng.integers(0, 1 << 24, (1, K + 1)) * 2.0 ** -24).astype(np.float32)
        o = oracle.verify(tgt, dft, a_p[None].astype(np.int32), uni, 1.0)
        mism = np.nonzero(a_p != a_q[:K])[0]
        n = int(mism[0]) if len(mism) else K
        assert o["num_accepted"][0] == n
        assert list(o["out_tokens"][0, :n + 1]) == list(a_q[:n]) + [a_q[n]]


def test_invalid_sequences_get_sentinels():
    rng = np.random.default_rng(10)
    B, K, V = 4, 2, 8
    tgt, dft = _rows(rng, B, K, V)
    tokens = np.zeros((B, K), np.int32)
    uni = np.full((B, K + 1), 0.5, np.float32)
    tgt[1, 2, 3] = np.nan                 # NaN in the bonus row
    dft[2, 0, :] = -np.inf                # a draft row with no mass
    tokens[3, 1] = V                      # token out of range
    o = oracle.verify(tgt, dft, tokens, uni, 1.0)
    assert o["num_accepted"][0] >= 0
    for b in (1, 2, 3):
        assert o["num_accepted"][b] == -1
        assert np.all(o["out_tokens"][b] == -1)
        assert o["num_emitted"][b] == 0
    assert np.isnan(o["target_stats"][1, 2]).all()
    assert np.isnan(o["draft_stats"][2, 0]).all()


def test_final_draw_forced_counts():
    """oracle_final_draw with caller-supplied n reproduces the draw of the full
    verify, and takes the q fallback on identical rows."""
    rng = np.random.default_rng(12)
    B, K, V = 16, 3, 30
    tgt, dft = _rows(rng, B, K, V)
    pp = _row_probs(dft, 1.0)
    tokens = _sample_tokens(rng, pp)
    uni = (rng.integers(0, 1 << 24, (B, K + 1)) * 2.0 ** -24).astype(np.float32)
    o = oracle.verify(tgt, dft, tokens, uni, 1.0)
    f = oracle.final_draw(tgt, dft, uni, o["num_accepted"], 1.0)
    for b in range(B):
        assert f["token"][b] == o["out_tokens"][b, o["num_accepted"][b]]
        assert f["draw_kind"][b] == o["draw_kind"][b]
    same = np.ascontiguousarray(tgt[:, :K])
    f2 = oracle.final_draw(tgt, same, uni, np.zeros(B, np.int32), 1.0)
    assert np.all(f2["draw_kind"] == 2)
    for b in range(B):
        c = np.cumsum(oracle.softmax_row(tgt[b, 0], 1.0)[0])
        assert f2["token"][b] == np.searchsorted(c, float(uni[b, K]) * c[-1], side="right")
    bad = oracle.final_draw(tgt, dft, uni, np.full(B, K + 1, np.int32), 1.0)
    assert np.all(bad["token"] == -1)


# ---------------------------------------------------------------- exact rationals

def _rational_case(rng, K, V, den=16):
    """Random probability vectors whose entries are multiples of 1/den (exact
    in binary64), some entries zero."""
    def vec():
        while True:
            c = rng.multinomial(den, rng.dirichlet(np.ones(V)))
            if c.sum() == den:
                return c
    q = [vec() for _ in range(K + 1)]
    p = [vec() for _ in range(K)]
    return q, p


def test_fp64_oracle_equals_exact_rational_oracle():
    """On probabilities that are multiples of 1/16 (exact in binary64) and
    uniforms that are multiples of 2**-24, every fp64 decision is the exact
    one, so the fp64 oracle must agree token for token with the Fraction
    implementation - including uniforms sitting exactly on a boundary."""
    rng = np.random.default_rng(13)
    den = 16
    checked = 0
    for trial in range(300):
        K = int(rng.integers(1, 5))
        V = int(rng.integers(2, 9))
        qc, pc = _rational_case(rng, K, V, den)
        qf = np.array(qc, np.float64) / den
        pf = np.array(pc, np.float64) / den
        tokens = [int(rng.choice(V, p=pf[t])) for t in range(K)]
        uni = []
        for t in range(K + 1):
            u = Fraction(int(rng.integers(0, 1 << 24)), 1 << 24)
            if t < K and pc[t][tokens[t]] > 0 and rng.random() < 0.3:
                r = Fraction(int(qc[t][tokens[t]]), int(pc[t][tokens[t]]))
                if r < 1 and (r * (1 << 24)).denominator == 1:
                    u = r  # uniform exactly on the accept boundary
            uni.append(u)
        o = oracle.verify_dists(qf, pf, np.array([tokens], np.int32),
                                np.array([[float(u) for u in uni]], np.float32))
        qF = [[Fraction(int(c), den) for c in row] for row in qc]
        pF = [[Fraction(int(c), den) for c in row] for row in pc]
        n, out = micro.verify(qF, pF, tokens, uni)
        assert o["num_accepted"][0] == n
        assert list(o["out_tokens"][0, :n + 1]) == out
        checked += 1
    assert checked == 300


def test_golden_rational_fixture():
    """Hand-derived fixture (tests/golden/rational_v4_k2.json): exact rational
    distributions, the decision at each step worked out by hand in the file."""
    with open(os.path.join(GOLDEN, "rational_v4_k2.json")) as f:
        g = json.load(f)
    den = g["denominator"]
    q = np.array(g["q_counts"], np.float64) / den
    p = np.array(g["p_counts"], np.float64) / den
    T = 1.0
    # logits = log(prob) give back prob under softmax up to rounding; feed the
    # distributions directly to keep the boundaries exact.
    for case in g["cases"]:
        o = oracle.verify_dists(q, p, np.array([case["tokens"]], np.int32),
                                np.array([case["uniforms"]], np.float32))
        assert o["num_accepted"][0] == case["expect_num_accepted"], case["why"]
        n = case["expect_num_accepted"]
        assert list(o["out_tokens"][0, :n + 1]) == case["expect_tokens"], case["why"]
        assert o["draw_kind"][0] == case["expect_kind"], case["why"]
    # the same fixture through the logit path: logits log(prob) with -inf for 0
    with np.errstate(divide="ignore"):
        tgt = np.log(q).astype(np.float32)[None]
        dft = np.log(p).astype(np.float32)[None]
    for case in g["cases"]:
        if not case.get("logit_path_safe", True):
            continue
        o = oracle.verify(tgt, dft, np.array([case["tokens"]], np.int32),
                          np.array([case["uniforms"]], np.float32), T)
        n = case["expect_num_accepted"]
        assert o["num_accepted"][0] == n, case["why"]
        assert list(o["out_tokens"][0, :n + 1]) == case["expect_tokens"], case["why"]
