"""Pins of the oracle's greedy verify and draft-side sampler.

Greedy mode: wikillm.com card for arXiv 2302.01318, Pitfalls (greedy mode):
the card infers the rule from the general accept rule on one-hot
distributions.  The pin is that inference itself: the general oracle (pinned
in test_oracle_pins / test_oracle_laws) run on one-hot rows must give what the
greedy oracle gives on the same rows.  Argmax ties follow numpy's argmax.

Draft sampling: "Algorithm: Speculative Sampling (SpS)" (alg. 2) step 1 and
"Decoding transforms": tokens drawn from softmax(z/T).  Pinned to numpy's
searchsorted on the cumulative sum and to the law of the draws (chi-square).
"""
import numpy as np
import pytest
from scipy import special

import oracle
from tests.stats_util import chisquare_pvalue
from tests.test_oracle_pins import bf16_bits, bf16_to_f64


# ---------------------------------------------------------------- argmax

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_argmax_row_matches_numpy_first_occurrence(dtype):
    rng = np.random.default_rng(3)
    for trial in range(200):
        V = int(rng.integers(1, 300))
        z = rng.integers(-4, 5, size=V).astype(np.float32)  # many ties
        if trial % 3 == 0:
            z[rng.random(V) < 0.3] = -np.inf
            z[int(rng.integers(V))] = 1.0
        row = bf16_bits(z) if dtype == "bf16" else z
        ref = int(np.argmax(bf16_to_f64(row) if dtype == "bf16" else z))
        assert oracle.argmax_row(row) == ref


def test_argmax_row_invalid_rows():
    assert oracle.argmax_row(np.array([0.0, np.nan, 1.0], np.float32)) is None
    assert oracle.argmax_row(np.full(5, -np.inf, np.float32)) is None
    assert oracle.argmax_row(np.array([0.0, np.inf], np.float32)) is None
    assert oracle.argmax_row(np.array([-np.inf, -3.0, -np.inf], np.float32)) == 1


# ---------------------------------------------------------------- greedy verify

def one_hot_logits(idx: np.ndarray, V: int) -> np.ndarray:
    """Logit rows whose softmax is one-hot at idx: 0 there, -inf elsewhere."""
    z = np.full(idx.shape + (V,), -np.inf, np.float32)
    np.put_along_axis(z, idx[..., None], 0.0, axis=-1)
    return z


@pytest.mark.parametrize("K", [1, 3, 8])
def test_greedy_is_the_general_rule_on_one_hot_rows(K):
    """Pitfalls (greedy mode): the general verify on one-hot p and q accepts
    while the drafted token is the target argmax and then emits the target
    argmax; the greedy oracle must agree token for token."""
    rng = np.random.default_rng(K)
    B, V = 400, 6
    a = rng.integers(0, V, size=(B, K + 1))
    d = np.where(rng.random((B, K)) < 0.7, a[:, :K], rng.integers(0, V, size=(B, K)))
    target = one_hot_logits(a, V)
    draft = one_hot_logits(d, V)
    tokens = d.astype(np.int32)  # the draft's own argmax, as greedy drafting gives
    u = (rng.integers(0, 1 << 24, size=(B, K + 1)) * 2.0 ** -24).astype(np.float32)
    gen = oracle.verify(target, draft, tokens, u, 1.0)
    gre = oracle.greedy_verify(target, tokens)
    np.testing.assert_array_equal(gre["num_accepted"], gen["num_accepted"])
    np.testing.assert_array_equal(gre["out_tokens"], gen["out_tokens"])
    np.testing.assert_array_equal(gre["num_emitted"], gen["num_emitted"])
    np.testing.assert_array_equal(gre["argmax"], a)
    # both kinds of ending occur
    assert (gre["num_accepted"] == K).any() and (gre["num_accepted"] < K).any()


def test_greedy_on_real_rows_and_invalid_sequences():
    rng = np.random.default_rng(5)
    B, K, V = 50, 4, 300
    z = (3 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    a = np.argmax(z, axis=-1)
    tokens = np.where(rng.random((B, K)) < 0.8, a[:, :K], rng.integers(0, V, size=(B, K)))
    tokens = tokens.astype(np.int32)
    tokens[3, 1] = V        # out of range -> invalid
    z[7, 2, 5] = np.nan     # NaN row -> invalid
    z[9, K, :] = -np.inf    # bonus row with no maximum -> invalid
    g = oracle.greedy_verify(z, tokens)
    for b in range(B):
        if b in (3, 7, 9):
            assert g["num_accepted"][b] == -1 and g["num_emitted"][b] == 0
            assert np.all(g["out_tokens"][b] == -1)
            continue
        n = 0
        while n < K and tokens[b, n] == a[b, n]:
            n += 1
        assert g["num_accepted"][b] == n and g["num_emitted"][b] == n + 1
        assert list(g["out_tokens"][b, :n]) == list(tokens[b, :n])
        assert g["out_tokens"][b, n] == a[b, n]
        assert np.all(g["out_tokens"][b, n + 1:] == -1)


# ---------------------------------------------------------------- draft sampler

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.5, 1.0, 1.7])
def test_sample_rows_matches_searchsorted(dtype, T):
    rng = np.random.default_rng(7)
    R, V = 300, 2000
    z = (3 * rng.standard_normal((R, V)) - 1.1 * np.log(rng.permutation(V) + 1.0)).astype(np.float32)
    rows = bf16_bits(z) if dtype == "bf16" else z
    zf = bf16_to_f64(rows) if dtype == "bf16" else z.astype(np.float64)
    T = float(np.float32(T))
    u = (rng.integers(0, 1 << 24, size=R) * 2.0 ** -24).astype(np.float32)
    got = oracle.sample_rows(rows, u, T)
    for r in range(R):
        p = special.softmax(zf[r] / T)
        c = np.cumsum(p)
        ref = int(np.searchsorted(c, float(u[r]) * c[-1], side="right"))
        if got["tokens"][r] != ref:  # only possible within rounding of a breakpoint
            assert got["dist"][r] < 1e-12, (r, got["tokens"][r], ref)


def test_sample_rows_law_chi_square():
    rng = np.random.default_rng(9)
    V, N, T = 64, 200_000, 0.8
    z = (2 * rng.standard_normal(V)).astype(np.float32)
    rows = np.broadcast_to(z, (N, V)).copy()
    u = (rng.integers(0, 1 << 24, size=N) * 2.0 ** -24).astype(np.float32)
    tok = oracle.sample_rows(rows, u, T)["tokens"]
    counts = np.bincount(tok, minlength=V)
    p = special.softmax(z.astype(np.float64) / float(np.float32(T)))
    assert chisquare_pvalue(counts, p) > 1e-4
    # and the test has power: the untempered distribution is rejected
    assert chisquare_pvalue(counts, special.softmax(z.astype(np.float64))) < 1e-6


def test_sample_rows_invalid_and_masked_rows():
    z = np.array([[0.0, -np.inf, 0.0, -np.inf],
                  [np.nan, 0.0, 0.0, 0.0],
                  [-np.inf, -np.inf, -np.inf, -np.inf],
                  [-np.inf, -np.inf, 5.0, -np.inf]], np.float32)
    u = np.array([0.75, 0.5, 0.5, 0.999], np.float32)
    got = oracle.sample_rows(z, u, 1.0)["tokens"]
    assert list(got) == [2, -1, -1, 2]  # masked tokens are never drawn
