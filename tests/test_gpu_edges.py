"""GPU edge cases of the verify path, each checked against the oracle (or a
rule the pages fix): rows that define no distribution, out-of-range tokens,
-inf masks, p == q, disjoint supports, one-hot rows (the greedy reduction in
the Pitfalls notes), the zero-residual fallback to q, extreme logits and
temperatures, and caller-supplied accepted counts."""
import sys

import numpy as np
import pytest
import torch

import oracle
import parity
from speculative_sampling_verification_softmax_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
    binding.load()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _to_dev(tgt, dft, tok, uni, T, dtype="f32"):
    if dtype == "bf16":
        t = torch.from_numpy(tgt).to(torch.bfloat16)
        d = torch.from_numpy(dft).to(torch.bfloat16)
    else:
        t = torch.from_numpy(tgt)
        d = torch.from_numpy(dft)
    return dict(target=t.cuda(), draft=d.cuda(), tokens=torch.from_numpy(tok).cuda(),
                uniforms=torch.from_numpy(uni).cuda(), T=T)


def _check(inp, label):
    host = synth.to_host_arrays(inp)
    o = parity.oracle_verify(host)
    out = None
    for path in parity.PATHS:
        say(f"[edge] {label} ({path}): shapes {tuple(inp['target'].shape)}")
        g = parity.gpu_verify(inp, path=path)
        rep = parity.compare(g, o, inp["T"])
        say(f"[edge] {label} ({path}): flagged={len(rep['flagged'])} failures={rep['failures'][:3]}")
        parity.assert_parity(rep, f"{label} {path}")
        if out is not None:
            same_as_other_path(g, out, label)
        out = g
    return out, o


def same_as_other_path(g, h, label):
    """Both paths draw the same tokens; their fp32 normalisers may differ in
    the last bits (different summation shapes)."""
    for k in ("num_accepted", "out_tokens", "num_emitted"):
        np.testing.assert_array_equal(g[k], h[k], err_msg=f"{label}: {k} differs by path")
    for k in ("target_stats", "draft_stats", "probs"):
        np.testing.assert_allclose(g[k], h[k], rtol=1e-5, atol=0, equal_nan=True,
                                   err_msg=f"{label}: {k} differs by path")


def _uni(rng, B, K):
    return (rng.integers(0, 1 << 24, (B, K + 1)) * 2.0 ** -24).astype(np.float32)


def _tokens_from(rng, dft, T):
    B, K, V = dft.shape
    out = np.zeros((B, K), np.int32)
    for b in range(B):
        for t in range(K):
            r = oracle.softmax_row(np.ascontiguousarray(dft[b, t]), T)
            out[b, t] = rng.choice(V, p=r[0]) if r is not None else 0
    return out


def test_invalid_rows_and_tokens_get_sentinels():
    rng = np.random.default_rng(1)
    B, K, V = 8, 3, 300
    tgt = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    dft = (tgt[:, :K] + 0.3 * rng.standard_normal((B, K, V))).astype(np.float32)
    tok = _tokens_from(rng, dft, 1.0)
    tgt[1, 3, 17] = np.nan          # NaN in a bonus row
    dft[2, 1, :] = -np.inf          # draft row with no mass
    tgt[3, 0, 5] = np.inf           # +inf logit
    tok[4, 2] = V                   # out of range
    tok[5, 0] = -1
    tgt[6, 2, :] = -np.inf          # target row with no mass
    g, o = _check(_to_dev(tgt, dft, tok, _uni(rng, B, K), 1.0), "invalid")
    for b in range(1, 7):
        assert g["num_accepted"][b] == -1 and np.all(g["out_tokens"][b] == -1)
        assert g["num_emitted"][b] == 0
        assert np.isnan(g["probs"][b]).all()
    assert g["num_accepted"][0] >= 0 and g["num_accepted"][7] >= 0
    assert np.isnan(g["target_stats"][1, 3, 1]) and np.isnan(g["draft_stats"][2, 1, 1])
    assert np.isnan(g["target_stats"][3, 0, 1]) and np.isnan(g["target_stats"][6, 2, 1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_masked_rows(dtype):
    rng = np.random.default_rng(2)
    B, K, V = 32, 5, 5000
    tgt = (3 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    dft = (tgt[:, :K] + 0.8 * rng.standard_normal((B, K, V))).astype(np.float32)
    tgt[rng.random(tgt.shape) < 0.4] = -np.inf
    dft[rng.random(dft.shape) < 0.4] = -np.inf
    tgt[:, :, 0] = 0.0
    dft[:, :, 0] = 0.0
    inp = _to_dev(tgt, dft, np.zeros((B, K), np.int32), _uni(rng, B, K), 0.9, dtype)
    host = synth.to_host_arrays(inp)
    inp["tokens"] = torch.from_numpy(_tokens_from(rng, host["draft"] if dtype == "f32"
                                                  else _bf16_f32(host["draft"]), 0.9)).cuda()
    _check(inp, f"masked-{dtype}")


def _bf16_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_equal_rows_accept_all_and_bonus():
    rng = np.random.default_rng(3)
    B, K, V = 64, 4, 2000
    tgt = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    dft = np.ascontiguousarray(tgt[:, :K])
    tok = _tokens_from(rng, dft, 1.0)
    g, _ = _check(_to_dev(tgt, dft, tok, _uni(rng, B, K), 1.0), "p==q")
    assert np.all(g["num_accepted"] == K)


def test_disjoint_supports_reject_first():
    rng = np.random.default_rng(4)
    B, K, V = 32, 3, 512
    tgt = np.full((B, K + 1, V), -np.inf, np.float32)
    dft = np.full((B, K, V), -np.inf, np.float32)
    tgt[:, :, :256] = rng.standard_normal((B, K + 1, 256))
    dft[:, :, 256:] = rng.standard_normal((B, K, 256))
    tok = _tokens_from(rng, dft, 1.0)
    g, _ = _check(_to_dev(tgt, dft, tok, _uni(rng, B, K), 1.0), "disjoint")
    assert np.all(g["num_accepted"] == 0)
    assert np.all(g["out_tokens"][:, 0] < 256)


def test_one_hot_rows_greedy_rule():
    rng = np.random.default_rng(5)
    B, K, V = 64, 6, 100
    a_q = rng.integers(0, V, (B, K + 1))
    a_p = np.where(rng.random((B, K)) < 0.7, a_q[:, :K], rng.integers(0, V, (B, K)))
    tgt = np.full((B, K + 1, V), -np.inf, np.float32)
    dft = np.full((B, K, V), -np.inf, np.float32)
    for b in range(B):
        tgt[b, np.arange(K + 1), a_q[b]] = 5.0
        dft[b, np.arange(K), a_p[b]] = 5.0
    g, _ = _check(_to_dev(tgt, dft, a_p.astype(np.int32), _uni(rng, B, K), 1.0), "one-hot")
    for b in range(B):
        mism = np.nonzero(a_p[b] != a_q[b, :K])[0]
        n = int(mism[0]) if len(mism) else K
        assert g["num_accepted"][b] == n
        assert list(g["out_tokens"][b, :n + 1]) == list(a_q[b, :n]) + [a_q[b, n]]


@pytest.mark.parametrize("T", [0.05, 0.3, 3.0, 20.0])
def test_temperature_extremes(T):
    inp = synth.make_inputs(synth.workload("small", B=32, T=T, name=f"T{T}"), seed=9,
                            device="cuda")
    _check(inp, f"T={T}")


def test_extreme_logit_magnitudes():
    rng = np.random.default_rng(6)
    B, K, V = 16, 3, 1000
    tgt = (rng.standard_normal((B, K + 1, V)) * 1e4).astype(np.float32)
    tgt[:, :, :10] = 3e37
    tgt[:, :, 10:20] = -3e37
    dft = (tgt[:, :K] + 1e3 * rng.standard_normal((B, K, V))).astype(np.float32)
    tok = _tokens_from(rng, dft, 1.0)
    _check(_to_dev(tgt, dft, tok, _uni(rng, B, K), 1.0), "extreme")


@pytest.mark.parametrize("T", [0.8, 3.0])
def test_extreme_logit_magnitudes_bf16(T):
    """bf16 rows whose maxima lie far beyond the draw's shared exp(z/T)
    table (|m|/T > 300): 3e37 tied tops over a -3e37 floor, maxima whose
    product with log2(e)/T overflows fp32 (2.5e38, and 3.3e38 in some
    drafts only), and rows scaled to 1e30; every path against the oracle."""
    rng = np.random.default_rng(16)
    B, K, V = 16, 3, 1000
    tgt = (rng.standard_normal((B, K + 1, V)) * 1e4).astype(np.float32)
    tgt[:, :, :10] = 3e37
    tgt[:, :, 10:20] = -3e37
    tgt[::4, :, 500] = 2.5e38
    tgt[1::4, :, 20:] *= np.float32(1e26)
    dft = (tgt[:, :K] + 1e3 * rng.standard_normal((B, K, V))).astype(np.float32)
    dft[2::4, :, 700] = 3.3e38
    tok = _tokens_from(rng, dft, T)
    _check(_to_dev(tgt, dft, tok, _uni(rng, B, K), T, "bf16"), f"extreme bf16 T={T}")


def test_forced_counts_and_zero_residual_fallback():
    """Caller-supplied accepted counts: identical rows at the rejected position
    give a residual with no mass, so the draw falls back to q (Pitfalls)."""
    rng = np.random.default_rng(7)
    B, K, V = 24, 4, 3000
    tgt = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    dft = (tgt[:, :K] + 0.5 * rng.standard_normal((B, K, V))).astype(np.float32)
    n_forced = rng.integers(0, K + 1, B).astype(np.int32)
    for b in range(0, B, 2):           # identical rows at the forced position
        if n_forced[b] < K:
            dft[b, n_forced[b]] = tgt[b, n_forced[b]]
    n_forced[3] = -1
    n_forced[5] = K + 1
    uni = _uni(rng, B, K)
    inp = _to_dev(tgt, dft, np.zeros((B, K), np.int32), uni, 1.0)
    ts, ds = binding.softmax_stats(inp["target"], inp["draft"], 1.0)
    out = torch.full((B, K + 1), 77, dtype=torch.int32, device="cuda")
    nacc = torch.from_numpy(n_forced).cuda()
    ne = binding.residual_sample(inp["target"], inp["draft"], inp["uniforms"], ts, ds, nacc, 1.0,
                                 out)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ne = ne.cpu().numpy()
    ref = oracle.final_draw(tgt, dft, uni, n_forced, 1.0)
    for b in range(B):
        n = n_forced[b]
        if n < 0 or n > K:
            assert ne[b] == 0 and np.all(out[b] == 77)
            continue
        assert ne[b] == n + 1
        if out[b, n] != ref["token"][b]:
            assert ref["draw_dist"][b] < parity.BOUNDARY, (b, out[b, n], ref["token"][b])
        others = np.delete(out[b], n)
        assert np.all(others == 77)
    assert np.sum(ref["draw_kind"] == 2) >= 5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_residual_after_a_clean_fast_sweep(dtype):
    """Both rows at the rejected position keep one and the same token (the
    rest -inf) and the drafted token lies outside it, so q = p = 0 there: the
    token is rejected and the residual has no mass, while the one-sweep fast
    path itself succeeds (one uncertain token).  The draw falls back to q_n
    (Pitfalls).  Rows before n are identical, so they are always accepted."""
    rng = np.random.default_rng(11)
    B, K, V = 48, 4, 2000
    tgt = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    dft = (tgt[:, :K] + 0.5 * rng.standard_normal((B, K, V))).astype(np.float32)
    tok = _tokens_from(rng, dft, 1.0)
    n_of = rng.integers(0, K, B)
    for b in range(0, B, 3):           # every third sequence keeps a control
        n = int(n_of[b])
        dft[b, :n] = tgt[b, :n]
        keep = int(rng.integers(0, V))
        tgt[b, n] = -np.inf
        dft[b, n] = -np.inf
        tgt[b, n, keep] = float(rng.uniform(-3, 3))
        dft[b, n, keep] = float(rng.uniform(-3, 3))
        tok[b, n] = (keep + 1 + int(rng.integers(0, V - 1))) % V
    inp = _to_dev(tgt, dft, tok, _uni(rng, B, K), 1.0, dtype=dtype)
    g, o = _check(inp, f"empty residual {dtype}")
    fell_back = [b for b in range(0, B, 3) if g["num_accepted"][b] == n_of[b]]
    assert len(fell_back) == len(range(0, B, 3))
    assert np.all(o["draw_kind"][::3] == 2)


def _distinct_values(rng, V, dtype):
    """V distinct logits, shuffled: evenly spaced fp32 values, or distinct
    bf16 codes (1 + m/128) * 2**e for e in -6..3, both signs."""
    if dtype == "f32":
        vals = np.linspace(-5.0, 5.0, V)
    else:
        mags = np.array([(1 + m / 128) * 2.0 ** e for e in range(-6, 4) for m in range(128)])
        vals = np.concatenate([mags, -mags])
        assert V <= vals.size
        vals = rng.choice(vals, V, replace=False)
    return rng.permutation(vals).astype(np.float32)


def _permutation_fixing(rng, V, fixed):
    """A permutation of range(V) whose only fixed points are `fixed`."""
    fixed = np.asarray(sorted(set(int(f) for f in fixed)), np.int64)
    rest = np.setdiff1d(np.arange(V), fixed)
    img = rng.permutation(rest)
    for i in np.nonzero(img == rest)[0]:  # break accidental fixed points
        j = (i + 1) % rest.size
        img[i], img[j] = img[j], img[i]
    perm = np.arange(V)
    perm[rest] = img
    assert np.array_equal(np.sort(np.nonzero(perm == np.arange(V))[0]), fixed)
    return perm


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_uncertain_tokens_resolved_from_the_records(dtype):
    """Draft rows that permute their target row's distinct values, leaving a
    few tokens in place: p and q are the same distribution over the same
    values, so the fixed tokens have q = p (their residual sign is within
    rounding: uncertain, resolved exactly once the normalisers are known) and
    every other token differs clearly.  One fixed token per sweep item, two in
    the first item (the most the fast path resolves), or three there (the
    exact two-sweep path); some sequences fix the row's top token.  Modified
    rejection sampling, the residual max(0, q - p) normalised ("Algorithm:
    Speculative Sampling (SpS)", alg. 2)."""
    rng = np.random.default_rng(23)
    B, K = 12, 3
    V, item = (3000, 512) if dtype == "f32" else (2560, 1024)
    tgt = np.empty((B, K + 1, V), np.float32)
    dft = np.empty((B, K, V), np.float32)
    for b in range(B):
        for t in range(K + 1):
            tgt[b, t] = _distinct_values(rng, V, dtype)
        for t in range(K):
            fixed = [int(rng.integers(i, min(V, i + item))) for i in range(0, V, item)]
            extra = b % 3  # 0, 1 or 2 more fixed tokens in the first item
            while len(set(fixed)) < (V + item - 1) // item + extra:
                fixed.append(int(rng.integers(0, item)))
            if b % 4 == 0:
                fixed.append(int(np.argmax(tgt[b, t])))
            perm = _permutation_fixing(rng, V, fixed)
            dft[b, t] = tgt[b, t][perm]
    tok = _tokens_from(rng, dft, 1.0)
    g, o = _check(_to_dev(tgt, dft, tok, _uni(rng, B, K), 1.0, dtype), f"uncertain {dtype}")
    assert np.sum((o["num_accepted"] >= 0) & (o["num_accepted"] < K)) >= B // 2


def test_binding_rejects_bad_tensors():
    inp = synth.make_inputs("tiny", seed=0, device="cuda")
    with pytest.raises(ValueError):
        binding.softmax_stats(inp["target"].cpu(), inp["draft"].cpu(), 1.0)
    with pytest.raises(binding.SpecError):
        binding.softmax_stats(inp["target"], inp["draft"], 0.0)
    with pytest.raises(TypeError):
        binding.softmax_stats(inp["target"].double(), inp["draft"].double(), 1.0)


BOUNDARY_BF16 = [0x3C00, 0xBC00,   # +-2^-7: the first codes the residual kernel tabulates
                 0x3BFF, 0xBBFF,   # just below 2^-7 in magnitude: computed
                 0x427F, 0xC27F,   # +-63.75: the last tabulated codes
                 0x4280, 0xC280,   # +-64: computed
                 0x3B80, 0x0000, 0x8000, 0x0001, 0x8001,  # 2^-8, +-0, denormals
                 0x42C8, 0xC2C8,   # +-100
                 0xFF80]           # -inf


@pytest.mark.parametrize("T", [0.01, 0.05, 1.0, 20.0])
def test_bf16_table_boundary_codes(T):
    """bf16 rows made of the codes at and around the edges of the draw
    kernels' exponential table (2^-7 <= |z| < 2^6), -inf, zeros and
    denormals: every verify path (one-workgroup draws with the tables, the
    step's split draw) and the draft sampler against the oracle.  The low temperatures put
    most table entries at or near 0 and the top codes' entries far apart."""
    rng = np.random.default_rng(int(T))
    B, K, V = 64, 3, 700
    codes = np.array(BOUNDARY_BF16, np.uint32)

    def rows(shape):
        pick = codes[rng.integers(0, len(codes), shape)]
        z = (pick << 16).view(np.float32).copy()
        # a random third of the entries plain values, so rows differ
        plain = rng.random(shape) < 0.3
        z[plain] = rng.uniform(-8, 8, plain.sum()).astype(np.float32)
        return z

    tgt = rows((B, K + 1, V))
    dft = rows((B, K, V))
    tgt[:, :, 0] = 1.0  # every row has a finite maximum
    dft[:, :, 0] = 1.0
    tok = _tokens_from(rng, np.ascontiguousarray(
        (np.asarray(torch.from_numpy(dft).to(torch.bfloat16).float()))), float(np.float32(T)))
    inp = _to_dev(tgt, dft, tok, _uni(rng, B, K), T, dtype="bf16")
    _check(inp, f"bf16 table edges T={T}")
    # the sampler on the draft rows
    rows_dev = inp["draft"].reshape(B * K, V)
    u = torch.from_numpy((rng.integers(0, 1 << 24, B * K) * 2.0 ** -24).astype(np.float32)).cuda()
    got = binding.sample(rows_dev, u, T)["tokens"].cpu().numpy()
    lh = rows_dev.cpu().view(torch.int16).numpy().view(np.uint16)
    o = oracle.sample_rows(lh, u.cpu().numpy(), float(np.float32(T)))
    bad = [(r, int(got[r]), int(o["tokens"][r])) for r in range(B * K)
           if got[r] != o["tokens"][r] and not (o["dist"][r] < parity.BOUNDARY)]
    assert bad == [], bad[:5]
