"""Pins of the oracle's decoding transforms (top-k, nucleus) and of the verify
on transformed rows.

wikillm.com card for arXiv 2302.01318, Method, "Decoding transforms", and
Pitfalls: temperature, top-k and nucleus are applied to both p and q before
the ratio and the residual, and draft tokens are drawn from the transformed
p.  The thresholds are pinned by properties that hold for the exact sets
(numpy sorting, scipy softmax masses): top-k keeps the k largest values and
their ties; the nucleus keeps at least top_p of the mass and loses that
guarantee when its smallest value class is dropped.  The transformed verify
is pinned to Theorem 1 on the transformed target row (chi-square).
"""
import numpy as np
import pytest
from scipy import special

import oracle
from tests.stats_util import chisquare_pvalue
from tests.test_oracle_pins import bf16_bits, bf16_to_f64


def rows(rng, n, V, dtype):
    z = (3 * rng.standard_normal((n, V)) - 1.1 * np.log(rng.permutation(V) + 1.0))
    z = np.round(z.astype(np.float32) * 4) / 4  # a coarse grid: ties occur
    if dtype == "bf16":
        b = bf16_bits(z)
        return b, bf16_to_f64(b)
    return z.astype(np.float32), z.astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_top_k_threshold(dtype):
    rng = np.random.default_rng(1)
    st, zf = rows(rng, 60, 500, dtype)
    for r in range(60):
        k = int(rng.integers(1, 500))
        t = oracle.filter_threshold(st[r], 1.0, top_k=k)
        srt = np.sort(zf[r])[::-1]
        assert t == srt[k - 1] or (t == -np.inf and srt[k - 1] == srt[-1])
        kept = zf[r] >= t
        assert kept.sum() >= k                       # the k largest and their ties
        assert np.all(zf[r][~kept] < srt[k - 1])     # nothing at or above the k-th value dropped
    # k >= V or k <= 0: nothing removed
    assert oracle.filter_threshold(st[0], 1.0, top_k=500) == -np.inf
    assert oracle.filter_threshold(st[0], 1.0, top_k=0) == -np.inf


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.7, 1.0, 1.5])
def test_nucleus_threshold_is_the_smallest_sufficient_set(dtype, T):
    rng = np.random.default_rng(2)
    st, zf = rows(rng, 80, 800, dtype)
    T = float(np.float32(T))
    for r in range(80):
        top_p = float(rng.uniform(0.05, 0.99))
        t = oracle.filter_threshold(st[r], T, top_p=top_p)
        prob = special.softmax(zf[r] / T)
        kept = zf[r] >= t
        assert prob[kept].sum() >= top_p - 1e-12        # enough mass
        smallest = zf[r][kept].min()
        rest = prob[kept & (zf[r] > smallest)].sum()
        assert rest < top_p + 1e-12                      # minimal: its smallest class is needed
    assert oracle.filter_threshold(st[0], T, top_p=1.0) == -np.inf
    # a tiny top_p keeps only the maximal value class
    t = oracle.filter_threshold(st[0], T, top_p=1e-9)
    assert t == zf[0].max()


def test_top_k_then_nucleus_nest():
    rng = np.random.default_rng(3)
    st, zf = rows(rng, 40, 300, "f32")
    for r in range(40):
        k, p = int(rng.integers(2, 300)), float(rng.uniform(0.1, 0.95))
        tk = oracle.filter_threshold(st[r], 1.0, top_k=k)
        tb = oracle.filter_threshold(st[r], 1.0, top_k=k, top_p=p)
        assert tb >= tk                                    # a subset of the top-k set
        kept_k = zf[r] >= tk
        prob = special.softmax(np.where(kept_k, zf[r], -np.inf))  # renormalised over top-k
        assert prob[zf[r] >= tb].sum() >= p - 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
def test_top_k_then_nucleus_is_the_smallest_sufficient_set_of_the_survivors(dtype, T):
    """The nucleus after top-k measures mass over the top-k survivors only:
    renormalised over that set (numpy, no oracle call), the kept classes hold
    at least top_p, and without the smallest kept class they hold less.  A
    normaliser taken over the whole row instead keeps too many classes and
    fails the second check."""
    rng = np.random.default_rng(6)
    st, zf = rows(rng, 120, 400, dtype)
    T = float(np.float32(T))
    narrowed = 0
    for r in range(120):
        k, p = int(rng.integers(2, 200)), float(rng.uniform(0.05, 0.97))
        tk = oracle.filter_threshold(st[r], T, top_k=k)
        tb = oracle.filter_threshold(st[r], T, top_k=k, top_p=p)
        srt = np.sort(zf[r])[::-1]
        survivors = zf[r] >= srt[k - 1]
        e = np.where(survivors, np.exp((zf[r] - srt[0]) / T), 0.0)
        prob_k = e / e.sum()
        kept = zf[r] >= tb
        assert np.all(kept <= survivors)                       # inside the top-k set
        assert prob_k[kept].sum() >= p - 1e-12                  # sufficient
        smallest = zf[r][kept].min()
        assert prob_k[kept & (zf[r] > smallest)].sum() < p + 1e-12   # minimal
        narrowed += int(tb > tk)
    assert narrowed > 30  # the nucleus really cuts inside the top-k set in many rows


# Equal-mass rows: with T = 2^60 every (z - m)/T is below 2^-56 in magnitude,
# so every token's mass exp((z - m)/T) is exactly 1.0 in binary64 and the
# nucleus reduces to counting tokens: the threshold is the largest value v
# with #{x : z[x] >= v} >= top_p * (number of top-k survivors).  The expected
# thresholds below are counted by hand on the row 7,7,6,6,...,0,0 (two
# tokens per value, V = 16), with dyadic top_p placing several cases exactly
# on the boundary, where ">=" keeps the class and ">" would not.
EQUAL_MASS_T = 2.0 ** 60
EQUAL_MASS_ROW = np.repeat(np.arange(7, -1, -1, dtype=np.float32), 2)
EQUAL_MASS_CASES = [
    # (top_k, top_p, threshold)            count needed -> classes kept
    (0, 0.5, 4.0),    # 8 of 16: values 7..4 hold exactly 8
    (0, 0.75, 2.0),   # 12 of 16: values 7..2 hold exactly 12
    (0, 0.3, 5.0),    # 4.8 of 16: values 7..5 hold 6
    (8, 0.5, 6.0),    # survivors 7..4 (8): 4 needed, values 7..6 hold exactly 4
    (8, 0.25, 7.0),   # 2 needed, value 7 holds exactly 2
    (3, 0.5, 7.0),    # 3rd largest is 6, ties kept: 4 survivors, 2 needed, value 7 holds 2
    (3, 0.75, 6.0),   # 3 needed: value 7 holds 2, 7..6 hold 4
    (5, 1.0, 5.0),    # top-k alone: 5th largest is 5
    (0, 1e-9, 7.0),   # a vanishing top_p keeps the top class
    (16, 1.0, -np.inf),  # nothing removed
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("top_k,top_p,want", EQUAL_MASS_CASES)
def test_nucleus_boundary_on_equal_mass_rows(dtype, top_k, top_p, want):
    row = EQUAL_MASS_ROW if dtype == "f32" else bf16_bits(EQUAL_MASS_ROW)
    got = oracle.filter_threshold(row, EQUAL_MASS_T, top_k=top_k, top_p=top_p)
    assert got == want


def test_invalid_rows_and_parameters():
    assert oracle.filter_threshold(np.array([0.0, np.nan], np.float32), 1.0, top_k=1) is None
    assert oracle.filter_threshold(np.full(4, -np.inf, np.float32), 1.0, top_p=0.5) is None
    assert oracle.filter_threshold(np.zeros(4, np.float32), 1.0, top_p=0.0) is None


def test_filtered_verify_reduces_to_verify_and_to_masked_rows():
    rng = np.random.default_rng(4)
    B, K, V = 20, 3, 400
    tgt = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    dft = (tgt[:, :K] + 0.5 * rng.standard_normal((B, K, V))).astype(np.float32)
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = (rng.integers(0, 1 << 24, size=(B, K + 1)) * 2.0 ** -24).astype(np.float32)
    plain = oracle.verify(tgt, dft, tok, u, 1.0)
    off = oracle.verify_filtered(tgt, dft, tok, u, 1.0, top_k=V, top_p=1.0)
    for k in ("num_accepted", "out_tokens", "num_emitted"):
        np.testing.assert_array_equal(off[k], plain[k])
    f = oracle.verify_filtered(tgt, dft, tok, u, 1.0, top_k=50, top_p=0.8)
    mt = np.where(tgt < f["target_thr"][..., None], -np.inf, tgt).astype(np.float32)
    md = np.where(dft < f["draft_thr"][..., None], -np.inf, dft).astype(np.float32)
    ref = oracle.verify(mt, md, tok, u, 1.0)
    for k in ("num_accepted", "out_tokens", "num_emitted"):
        np.testing.assert_array_equal(f[k], ref[k])


def test_theorem_1_on_transformed_rows():
    """K=1, tokens drawn from the transformed p: the emitted token follows the
    transformed q (Theorem 1 applies to the modified distributions)."""
    rng = np.random.default_rng(5)
    V, N, T, k, p = 64, 200_000, 0.9, 20, 0.85
    zq = (2 * rng.standard_normal(V)).astype(np.float32)
    zp = (zq + 0.8 * rng.standard_normal(V)).astype(np.float32)
    T = float(np.float32(T))
    tq = oracle.filter_threshold(zq, T, top_k=k, top_p=p)
    tp = oracle.filter_threshold(zp, T, top_k=k, top_p=p)
    q = special.softmax(np.where(zq >= tq, zq, -np.inf).astype(np.float64) / T)
    pp = special.softmax(np.where(zp >= tp, zp, -np.inf).astype(np.float64) / T)
    tok = rng.choice(V, size=(N, 1), p=pp).astype(np.int32)
    u = (rng.integers(0, 1 << 24, size=(N, 2)) * 2.0 ** -24).astype(np.float32)
    tgt = np.broadcast_to(np.stack([zq, zq]), (N, 2, V)).copy()
    dft = np.broadcast_to(zp, (N, 1, V)).copy()
    out = oracle.verify_filtered(tgt, dft, tok, u, T, top_k=k, top_p=p)
    first = out["out_tokens"][:, 0]
    assert chisquare_pvalue(np.bincount(first, minlength=V), q) > 1e-4
    assert np.all(q[first] > 0)  # nothing outside the transformed support is emitted
