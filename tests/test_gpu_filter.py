"""GPU parity of the decoding transforms (spec_filter, through the C ABI)
against the fp64 oracle on the same seeded bytes.

The card's Method, "Decoding transforms", and Pitfalls: top-k and nucleus
are applied alike to the target and draft rows before the verify.

Thresholds: top-k is a pure order statistic of the stored values, so it must
be bit-identical.  The nucleus threshold compares a sum of masses with top_p
times the total.  The oracle sums fp64 exponentials; the kernel sums fp64
exponentials rounded to 2^-42 fixed point near the maximum and fp32 exp2
terms (each below 2^-16) further down, so a threshold may differ only where
the oracle's mass at the deciding value lies within 1e-7 of the total of
top_p * S (counted, under 1e-3 of rows).  The
filtered rows must be the input with exactly the tokens below the kernel's
threshold set to -inf (bit-exact).  End to end, verify on the filtered rows
follows the parity rule of the plain verify against oracle.verify_filtered.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import parity
from speculative_sampling_verification_softmax_amd import synth

pytestmark = pytest.mark.gpu

MASS_TOL = 1e-7
MAX_NUCLEUS_FLAGGED = 1e-3


@pytest.fixture(scope="module", autouse=True)
def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
    from speculative_sampling_verification_softmax_amd import binding
    binding.load()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_logits(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def as_f64(h: np.ndarray) -> np.ndarray:
    if h.dtype == np.uint16:
        return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return h.astype(np.float64)


def neg_inf_bits(h: np.ndarray):
    return np.uint16(0xFF80) if h.dtype == np.uint16 else np.float32(-np.inf)


def nucleus_margin(z: np.ndarray, T: float, top_k: int, top_p: float, v: float) -> float:
    """|mass(z >= v) - top_p * S| / S over the top-k survivors, in fp64."""
    keep = np.ones_like(z, bool)
    if 0 < top_k < z.size:
        keep = z >= np.sort(z)[::-1][top_k - 1]
    e = np.where(keep, np.exp((z - z.max()) / T), 0.0)
    S = e.sum()
    return abs(e[z >= v].sum() - top_p * S) / S


def check_filter(logits: torch.Tensor, T: float, top_k: int, top_p: float, label: str,
                 rows=None, inplace=False):
    """Thresholds against the oracle (on `rows`, or all) and the filtered rows
    against the input masked at the kernel's own thresholds."""
    from speculative_sampling_verification_softmax_amd import binding
    V = logits.shape[-1]
    R = logits.numel() // V
    T32 = float(np.float32(T))
    p32 = float(np.float32(top_p))
    say(f"[filter] {label}: R={R} V={V} {logits.dtype} T={T32} top_k={top_k} top_p={p32} "
        f"inplace={inplace} -> gpu")
    before = host_logits(logits).reshape(R, V).copy()
    src = logits.clone() if inplace else logits
    out = binding.filter_rows(src, T, top_k, top_p, inplace=inplace, stats=True)
    torch.cuda.synchronize()
    thr = out["thresholds"].reshape(-1).cpu().numpy().astype(np.float64)
    got = host_logits(out["filtered"]).reshape(R, V)
    st = out["stats"].reshape(R, 2).cpu().numpy().astype(np.float64)
    rows = list(range(R)) if rows is None else list(rows)
    flagged, checked, kept = 0, 0, []
    for r in rows:
        o = oracle.filter_threshold(before[r], T32, top_k=top_k, top_p=p32)
        zr = as_f64(before[r])
        kept.append(int((zr >= thr[r]).sum()))
        checked += 1
        if o is None:
            assert np.isnan(thr[r]), f"{label}: row {r} should be invalid, got {thr[r]}"
            assert got[r].tobytes() == before[r].tobytes(), f"{label}: invalid row {r} changed"
            assert np.isnan(st[r, 1]), f"{label}: invalid row {r} has s={st[r, 1]}"
            continue
        if thr[r] != o:
            hi = max(thr[r], o)
            assert p32 < 1.0, f"{label}: row {r} top-k threshold {thr[r]} != {o}"
            m = nucleus_margin(zr, T32, top_k, p32, hi)
            assert m <= MASS_TOL, f"{label}: row {r} threshold {thr[r]} != {o} (margin {m:.3e})"
            flagged += 1
        # the rows: the input with exactly z < thr set to -inf
        exp = before[r].copy()
        if thr[r] > -np.inf:
            exp[zr < thr[r]] = neg_inf_bits(before)
        assert got[r].tobytes() == exp.tobytes(), f"{label}: row {r} filtered row differs"
        # the filtered row's stats against the oracle's own row statistics
        _, M, S = oracle.softmax_row(exp, T32)
        assert st[r, 0] / T32 == M, f"{label}: row {r} stats max {st[r, 0]}"
        assert abs(st[r, 1] - S) <= 1e-5 * S, f"{label}: row {r} stats s {st[r, 1]} vs {S}"
    assert flagged <= MAX_NUCLEUS_FLAGGED * max(checked, 1), f"{label}: {flagged} near-tie rows"
    kept = np.asarray(kept)
    say(f"[filter] {label}: {checked} rows checked, {flagged} near-tie thresholds, "
        f"kept tokens min/median/max {kept.min()}/{int(np.median(kept))}/{kept.max()}")
    return out


def zipf_rows(R, V, dtype, seed, grid=None):
    g = torch.Generator(device="cuda").manual_seed(seed)
    ranks = torch.randperm(V, generator=g, device="cuda").to(torch.float32) + 1.0
    z = 2.0 * torch.randn(R, V, device="cuda", generator=g) - 1.1 * torch.log(ranks)
    if grid:
        z = torch.round(z * grid) / grid  # coarse values: many exact ties
    return z.to(torch.bfloat16) if dtype == "bf16" else z


@pytest.mark.parametrize("top_k,top_p", [(50, 1.0), (0, 0.9), (40, 0.8), (1, 1.0), (0, 1e-6),
                                         (1000, 0.95)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_thresholds_and_rows(dtype, top_k, top_p):
    z = zipf_rows(48, 32000, dtype, seed=top_k + int(top_p * 100))
    check_filter(z, 0.8, top_k, top_p, f"{dtype} k={top_k} p={top_p}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ties_on_a_coarse_grid(dtype):
    z = zipf_rows(40, 5000, dtype, seed=7, grid=2)
    for k, p in [(10, 1.0), (100, 1.0), (0, 0.5), (30, 0.7)]:
        check_filter(z, 1.0, k, p, f"grid {dtype} k={k} p={p}")


@pytest.mark.parametrize("V,dtype", [(1, "f32"), (7, "bf16"), (63, "f32"), (1025, "bf16"),
                                     (100003, "f32")])
def test_ragged_rows_off_alignment(V, dtype):
    R = 13
    z = zipf_rows(R, V, dtype, seed=V)
    big = torch.empty(R * V + 3, dtype=z.dtype, device="cuda")
    view = big[3:].view(R, V)  # rows off 16-byte boundaries
    view.copy_(z)
    for k, p in [(min(5, V), 1.0), (0, 0.9), (3, 0.5)]:
        check_filter(view, 1.3, k, p, f"V={V} {dtype} k={k} p={p}")


def test_headline_rows_in_place_sampled():
    """The full target and draft batch of the bf16 V=128256 workload, filtered
    in place; thresholds checked on a sample of rows (the oracle sorts each)."""
    inp = synth.make_inputs("headline", seed=5, device="cuda")
    rows = inp["target"].reshape(-1, inp["target"].shape[-1])
    sample = list(range(0, rows.shape[0], 97))
    check_filter(rows, inp["T"], 50, 0.9, "headline target", rows=sample, inplace=True)


@pytest.mark.parametrize("case", ["k_below_window", "p_below_window", "window_over_capacity",
                                  "k_and_p_below_window"])
def test_rows_outside_the_window(case):
    """Rows whose threshold lies more than 16 powers of two of probability
    below the maximum, or whose window holds more values than LDS keeps: the
    selects then run over the whole row."""
    if case == "k_below_window":
        z, T, k, p = zipf_rows(24, 32000, "bf16", seed=31), 0.8, 6000, 1.0
    elif case == "p_below_window":
        z, T, k, p = zipf_rows(24, 32000, "f32", seed=32), 0.8, 0, 0.9999
    elif case == "window_over_capacity":
        g = torch.Generator(device="cuda").manual_seed(33)
        z, T, k, p = 0.3 * torch.randn(16, 60000, device="cuda", generator=g), 1.0, 20, 0.5
    else:
        z, T, k, p = zipf_rows(24, 32000, "bf16", seed=34), 0.8, 9000, 0.9999
    check_filter(z, T, k, p, case)


@pytest.mark.parametrize("case", ["late_max", "staging_over_capacity", "window_list_over_capacity",
                                  "tail_below_staged_window", "invalid_and_masked",
                                  "at_the_top_p_bound", "headline_rows"])
def test_nucleus_alone_one_read(case):
    """bf16 nucleus without top-k: one streamed read stages the vectors near the
    block's running maximum, and the cut is settled over them when their
    window holds top_p of the mass.  Rows whose maximum comes last (the running
    maximum rises late, so many vectors are staged), rows that stage more
    vectors than LDS holds, whose window holds more values than its list
    (4000 near-maximal values in 500 consecutive vectors), or whose cut lies
    below the staged window but above the deeper one (all three then take the
    window pass), invalid and masked rows,
    top_p on both sides of the bound above which the two-read path is taken,
    and sampled headline rows."""
    seed = {"late_max": 71, "staging_over_capacity": 72, "tail_below_staged_window": 73,
            "invalid_and_masked": 74, "at_the_top_p_bound": 75, "headline_rows": 76,
            "window_list_over_capacity": 77}[case]
    g = torch.Generator(device="cuda").manual_seed(seed)
    if case == "late_max":
        z = zipf_rows(24, 32000, "f32", seed=61)
        z[:, -1] = z.max(dim=1).values + 2.0
        check_filter(z.to(torch.bfloat16), 0.8, 0, 0.9, case)
    elif case == "staging_over_capacity":
        z = 0.3 * torch.randn(16, 60000, device="cuda", generator=g)
        check_filter(z.to(torch.bfloat16), 1.0, 0, 0.5, case)
    elif case == "window_list_over_capacity":
        z = torch.full((8, 32000), -30.0, device="cuda")
        z[:, 1000:5000] = 0.3 * torch.randn(8, 4000, device="cuda", generator=g)
        check_filter(z.to(torch.bfloat16), 1.0, 0, 0.9, case)
    elif case == "tail_below_staged_window":
        # the maximum (0) carries ~73 % of the mass; 3000 values between 12.3
        # and 13.7 powers of two of probability below it carry the rest
        R, V = 12, 32000
        z = torch.full((R, V), -30.0, device="cuda")
        for r in range(R):
            pos = torch.randperm(V, generator=g, device="cuda")
            z[r, pos[0]] = 0.0
            z[r, pos[1:3001]] = -9.0 + (torch.rand(3000, generator=g, device="cuda") - 0.5)
        check_filter(z.to(torch.bfloat16), 1.0, 0, 0.9, case)
    elif case == "invalid_and_masked":
        z = zipf_rows(8, 4000, "f32", seed=62)
        z[1, 7] = float("nan")
        z[2, :] = float("-inf")
        z[3, ::2] = float("-inf")
        z[4, :] = 0.5
        z[5, 11] = float("inf")
        z[6, 100:3000] = float("-inf")
        check_filter(z.to(torch.bfloat16), 0.8, 0, 0.9, case)
    elif case == "at_the_top_p_bound":
        z = zipf_rows(24, 32000, "bf16", seed=63)
        for p in (0.97, float(np.nextafter(np.float32(0.97), np.float32(1.0)))):
            check_filter(z, 0.8, 0, p, f"{case} p={p!r}")
    else:
        inp = synth.make_inputs("headline", seed=6, device="cuda")
        rows = inp["draft"].reshape(-1, inp["draft"].shape[-1])
        check_filter(rows, inp["T"], 0, 0.9, case, rows=list(range(0, rows.shape[0], 61)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_top_k_at_the_block_size(dtype):
    """top_k up to the filter's block size (512 threads) takes the window from
    the per-thread maxima and re-reads only the vectors whose largest key
    reaches it; top_k one past it re-reads the whole row.  Both around the
    switch, plus constant rows (every vector marked, the window over LDS) and
    rows with -inf runs (already filtered rows), including a ragged head."""
    z = zipf_rows(20, 32000, dtype, seed=51)
    z[3, :] = 1.5
    z[4, 100:20000] = float("-inf")
    z[5, ::3] = float("-inf")
    for k, p in [(512, 1.0), (513, 1.0), (512, 0.6), (2, 0.99)]:
        check_filter(z, 0.9, k, p, f"block-size {dtype} k={k} p={p}")
    big = torch.empty(20 * 32000 + 5, dtype=z.dtype, device="cuda")
    view = big[5:].view(20, 32000)  # rows off 16-byte boundaries
    view.copy_(z)
    check_filter(view, 0.9, 300, 0.95, f"block-size ragged {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_transform(dtype):
    """top_k off and top_p = 1: thresholds -inf (NaN for rows that define no
    distribution), the rows copied bit for bit, their own stats; one streamed
    pass when the output shares the input's offset within 16 bytes (a new
    buffer, or in place with nothing written), the general path otherwise."""
    z = zipf_rows(16, 32000, "f32", seed=81)
    z[3, 77] = float("nan")
    z[4, :] = float("-inf")
    z[5, 9] = float("inf")
    z[6, ::2] = float("-inf")
    z = z.to(torch.bfloat16) if dtype == "bf16" else z
    check_filter(z, 0.8, 0, 1.0, f"no transform {dtype}")
    check_filter(z.clone(), 0.8, 0, 1.0, f"no transform in place {dtype}", inplace=True)
    big = torch.empty(16 * 32000 + 3, dtype=z.dtype, device="cuda")
    view = big[3:].view(16, 32000)  # rows off 16-byte boundaries
    view.copy_(z)
    check_filter(view, 0.8, 0, 1.0, f"no transform unaligned {dtype}")
    check_filter(zipf_rows(9, 7, dtype, seed=82), 1.1, 0, 1.0, f"no transform V=7 {dtype}")


@pytest.mark.parametrize("top_k,top_p", [(0, 1.0), (50, 0.9), (0, 0.9), (0, 0.5), (0, 0.99)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_huge_logits(dtype, top_k, top_p):
    """Logits whose max times log2(e)/T reaches 2^22 and beyond, up to where
    that product overflows fp32: the statistics switch to the wide route
    (difference to the max taken first), and no reference or rescale in the
    passes may overflow; ties at the top, a masked half, and rows far apart in
    scale."""
    z = zipf_rows(10, 4000, "f32", seed=85)
    z[0] *= 1e4              # |m c2| below 2^22
    z[1] *= 1e7              # above 2^22: the wide statistics
    z[2, 100:110] = 3e37     # ten tied maxima far above the rest
    z[3, 3000:3010] = 2.5e38  # m c2 beyond the largest float (T = 0.8)
    z[4, ::2] = -3e38
    z[5, :] = 3e37           # every value tied
    z[6] *= 1e30
    z[7, 17] = 3.3e38
    z[7, 18] = 3.2e38
    z[8] = z[8] * 1e35 + 2e38  # a dense top near the fp32 limit
    z = z.to(torch.bfloat16) if dtype == "bf16" else z
    check_filter(z, 0.8, top_k, top_p, f"huge logits {dtype} k={top_k} p={top_p}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_maximum_vocabulary(dtype):
    """V = 2^20, the largest vocabulary the header admits: rows longer than the
    vector map (no marked re-read, no one-read nucleus) take the plain passes."""
    z = zipf_rows(3, 1 << 20, dtype, seed=91)
    for k, p in [(50, 0.9), (0, 0.9), (700, 1.0)]:
        check_filter(z, 0.8, k, p, f"V=2^20 {dtype} k={k} p={p}")


def test_repeatable():
    from speculative_sampling_verification_softmax_amd import binding
    z = zipf_rows(64, 32000, "f32", seed=41)
    for k, p in [(0, 0.9), (100, 0.95), (0, 0.999)]:
        a = binding.filter_rows(z, 0.7, k, p, write_rows=False)["thresholds"].cpu().numpy()
        for _ in range(3):
            b = binding.filter_rows(z, 0.7, k, p, write_rows=False)["thresholds"].cpu().numpy()
            assert a.tobytes() == b.tobytes()


def test_invalid_rows_and_trivial_parameters():
    from speculative_sampling_verification_softmax_amd import binding
    R, V = 6, 300
    z = torch.randn(R, V, device="cuda")
    z[1, 7] = float("nan")
    z[2, :] = float("-inf")
    z[3, ::2] = float("-inf")   # masked half: a top-k inside the finite half
    z[4, :] = 0.0               # all equal: nothing removed by either transform
    z[5, 11] = float("inf")
    check_filter(z, 1.0, 20, 0.9, "invalid/masked")
    # k >= V and p >= 1: nothing removed anywhere, rows copied
    out = binding.filter_rows(z, 1.0, V, 1.0)
    thr = out["thresholds"].cpu().numpy()
    assert np.all(thr[[0, 3, 4]] == -np.inf) and np.all(np.isnan(thr[[1, 2, 5]]))
    assert torch.equal(out["filtered"].view(torch.int32), z.view(torch.int32))
    # thresholds only: no rows written
    only = binding.filter_rows(z, 1.0, 20, 0.9, write_rows=False, stats=True)
    full = binding.filter_rows(z, 1.0, 20, 0.9, stats=True)
    assert only["filtered"] is None
    np.testing.assert_array_equal(only["thresholds"].cpu().numpy(),
                                  full["thresholds"].cpu().numpy())
    assert only["stats"].cpu().numpy().tobytes() == full["stats"].cpu().numpy().tobytes()


@pytest.mark.parametrize("wl,top_k,top_p", [("small", 40, 0.9), ("batch1", 0, 0.8),
                                            ("tiny", 10, 1.0)])
def test_verify_on_filtered_rows(wl, top_k, top_p):
    """filter -> three-call verify on the filtered rows against the oracle's
    verify_filtered, with the drafted tokens drawn (by the oracle) from the
    filtered draft rows as step 1 of the method does."""
    from speculative_sampling_verification_softmax_amd import binding
    inp = synth.make_inputs(wl, seed=11, device="cuda", B=256 if wl == "tiny" else None)
    host = synth.to_host_arrays(inp)
    T32 = float(np.float32(inp["T"]))
    p32 = float(np.float32(top_p))
    B, K1, V = inp["target"].shape
    K = K1 - 1
    # draft tokens from the oracle's filtered draft rows
    dh = host["draft"].reshape(B * K, V).copy()
    zf = as_f64(dh)
    for r in range(B * K):
        t = oracle.filter_threshold(dh[r], T32, top_k=top_k, top_p=p32)
        if t is not None and t > -np.inf:
            dh[r][zf[r] < t] = neg_inf_bits(dh)
    rng = np.random.default_rng(3)
    u = (rng.integers(0, 1 << 24, size=B * K) * 2.0 ** -24).astype(np.float32)
    tok = oracle.sample_rows(dh, u, T32)["tokens"].reshape(B, K).astype(np.int32)
    tok = np.where(tok < 0, 0, tok).astype(np.int32)
    host["tokens"] = tok
    say(f"[filtered verify] {wl} B={B} K={K} V={V} k={top_k} p={p32} -> gpu filter + verify")
    ftr = binding.filter_rows(inp["target"], inp["T"], top_k, top_p, stats=True)
    fdr = binding.filter_rows(inp["draft"], inp["T"], top_k, top_p, stats=True)
    ft, fd = ftr["filtered"], fdr["filtered"]
    tok_d = torch.as_tensor(tok, device="cuda")
    g = parity.gpu_verify(dict(target=ft, draft=fd, tokens=tok_d, uniforms=inp["uniforms"],
                               T=inp["T"]))
    o = oracle.verify_filtered(host["target"], host["draft"], tok, host["uniforms"], T32,
                               top_k=top_k, top_p=p32)
    rep = parity.compare(g, o, inp["T"])
    say(f"[filtered verify] {wl}: draws={rep['draws']} flagged={len(rep['flagged'])} "
        f"failures={len(rep['failures'])} accept_hist={rep['accept_hist']}")
    parity.assert_parity(rep, f"filtered {wl}")
    # the filter's own stats straight into spec_verify_sample (no stats pass)
    n, out, probs, ne = binding.verify_sample(ft, fd, tok_d, inp["uniforms"], ftr["stats"],
                                              fdr["stats"], inp["T"])
    torch.cuda.synchronize()
    g2 = dict(target_stats=ftr["stats"].cpu().numpy(), draft_stats=fdr["stats"].cpu().numpy(),
              num_accepted=n.cpu().numpy(), out_tokens=out.cpu().numpy(),
              probs=probs.cpu().numpy(), num_emitted=ne.cpu().numpy())
    rep2 = parity.compare(g2, o, inp["T"])
    say(f"[filtered verify, filter stats] {wl}: flagged={len(rep2['flagged'])} "
        f"failures={len(rep2['failures'])}")
    parity.assert_parity(rep2, f"filtered {wl} (filter stats)")
