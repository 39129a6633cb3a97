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
