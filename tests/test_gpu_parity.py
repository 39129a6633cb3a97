"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded input bytes, for every workload shape and for ragged shapes.

Workloads (speculative_sampling_verification_softmax_amd.synth): tiny, batch1,
small, headline (all sequences checked) and large (a sample of sequences
checked; the launch is the full B=1024, K=16, V=256000 fp32 batch)."""
import sys

import numpy as np
import pytest
import torch

import parity
from speculative_sampling_verification_softmax_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
    from speculative_sampling_verification_softmax_amd import binding
    binding.load()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_case(wl, seed, B=None, seqs=None, label="", path="three_call"):
    say(f"[case] {label or wl if isinstance(wl, str) else wl.name} seed={seed} B={B} -> generate")
    inp = synth.make_inputs(wl, seed=seed, device="cuda", B=B)
    w = inp["workload"]
    say(f"[case] {w.name} B={w.B} K={w.K} V={w.V} {w.dtype} T={w.T} -> gpu verify ({path})")
    g = parity.gpu_verify(inp, path=path)
    if seqs is not None:
        idx = torch.as_tensor(seqs, device="cuda")
        sub = dict(target=inp["target"][idx], draft=inp["draft"][idx], tokens=inp["tokens"][idx],
                   uniforms=inp["uniforms"][idx], T=inp["T"])
        host = synth.to_host_arrays(sub)
        o = parity.oracle_verify(host)
    else:
        host = synth.to_host_arrays(inp)
        o = parity.oracle_verify(host)
    rep = parity.compare(g, o, w.T, seqs=None if seqs is None else np.asarray(seqs))
    say(f"[case] {w.name} seed={seed} {path}: seqs={rep['sequences']} draws={rep['draws']} "
        f"flagged={len(rep['flagged'])} failures={len(rep['failures'])} "
        f"stats_rel={rep['stats_max_rel']:.2e} probs_rel={rep['probs_max_rel']:.2e} "
        f"accept_hist={rep['accept_hist']}")
    return rep


@pytest.mark.parametrize("path", parity.PATHS)
@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_many_sequences(seed, path):
    parity.assert_parity(run_case("tiny", seed, B=5000, path=path), "tiny")


@pytest.mark.parametrize("path", parity.PATHS)
def test_batch1_latency_shape(path):
    """1000 independent B=1 launches (each its own seed and vocabulary
    permutation): every decision matches the oracle's, and the boundary draws
    over all of them stay under 1e-4 of all draws."""
    total_draws, flagged, stats_rel, probs_rel = 0, 0, 0.0, 0.0
    for seed in range(1000):
        inp = synth.make_inputs("batch1", seed=seed, device="cuda")
        g = parity.gpu_verify(inp, path=path)
        o = parity.oracle_verify(synth.to_host_arrays(inp))
        rep = parity.compare(g, o, inp["T"])
        assert rep["failures"] == [], (seed, rep["failures"])
        assert rep["stats_validity_mismatch"] == 0 and rep["stats_max_not_exact"] == 0, seed
        total_draws += rep["draws"]
        flagged += len(rep["flagged"])
        stats_rel = max(stats_rel, rep["stats_max_rel"])
        probs_rel = max(probs_rel, rep["probs_max_rel"])
    say(f"[case] batch1 x1000 {path}: draws={total_draws} flagged={flagged} "
        f"stats_rel={stats_rel:.2e} probs_rel={probs_rel:.2e}")
    assert stats_rel <= parity.PROB_RTOL and probs_rel <= parity.PROB_RTOL
    assert flagged <= parity.MAX_FLAGGED_FRACTION * total_draws


@pytest.mark.parametrize("path", parity.PATHS)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_small_batch(seed, path):
    parity.assert_parity(run_case("small", seed, path=path), "small")


@pytest.mark.parametrize("path", parity.PATHS)
@pytest.mark.parametrize("seed", [0, 1])
def test_headline_all_sequences(seed, path):
    rep = run_case("headline", seed, path=path)
    parity.assert_parity(rep, "headline")
    assert rep["sequences"] == 256


@pytest.mark.parametrize("path", parity.PATHS)
def test_large_sampled_sequences(path):
    rng = np.random.default_rng(0)
    seqs = np.sort(rng.choice(1024, size=64, replace=False))
    rep = run_case("large", 0, seqs=seqs, path=path)
    parity.assert_parity(rep, "large")


RAGGED = [
    # (V, K, dtype, B) -- unaligned rows, tiny rows, the maximum K
    (1, 1, "bf16", 3), (2, 2, "f32", 5), (63, 3, "bf16", 7), (65, 4, "f32", 9),
    (777, 5, "bf16", 11), (1001, 2, "f32", 6), (4097, 64, "bf16", 3), (40000, 7, "f32", 5),
    (129, 64, "f32", 2), (32003, 3, "bf16", 17),
    # the draw's fast sweep takes items of two 16-byte-per-lane chunks (1024 bf16 or 512 fp32
    # tokens) across 16 waves: fewer items than waves, exactly 16, one more (with a lone or
    # ragged last chunk)
    (15360, 3, "bf16", 8), (16384, 3, "bf16", 8), (16385, 3, "bf16", 8), (16896, 2, "bf16", 6),
    (8192, 3, "f32", 8), (8449, 2, "f32", 6),
    # the draw's LDS routes at large vocabularies: bf16 without the exponential tables (fast
    # sweep, computed exponentials), bf16 at the largest V (slow two-sweep path, tables on),
    # fp32 past the fast sweep's LDS (slow path, computed)
    (600000, 2, "bf16", 3), (1 << 20, 2, "bf16", 2), (600000, 2, "f32", 2),
]


@pytest.mark.parametrize("path", parity.PATHS)
@pytest.mark.parametrize("V,K,dtype,B", RAGGED)
def test_ragged_shapes(V, K, dtype, B, path):
    wl = synth.workload("batch1", V=V, K=K, dtype=dtype, B=B, T=0.7, name=f"ragged{V}")
    rep = run_case(wl, seed=V + K, path=path)
    parity.assert_parity(rep, f"V={V} K={K} {dtype}")


# Row counts B*(2K+1) around the stats launch's workgroup-size switches (1024 threads up to 512
# rows; 512 threads past 512 rows; fp32 back to 1024 threads past 1024 rows) and batches around
# the split draw's part rule (fewer parts once B*P would reach every CU), K = 1: rows = 3B.
LAUNCH_SHAPES = [(170, "bf16"), (171, "bf16"), (341, "bf16"), (342, "bf16"),
                 (170, "f32"), (171, "f32"), (341, "f32"), (342, "f32")]


@pytest.mark.parametrize("B,dtype", LAUNCH_SHAPES)
def test_stats_launch_shapes(B, dtype):
    wl = synth.workload("batch1", V=3001, K=1, dtype=dtype, B=B, T=0.9, name=f"rows{3 * B}")
    rep = run_case(wl, seed=B, path="two_call")
    parity.assert_parity(rep, f"{3 * B} rows {dtype}")


@pytest.mark.parametrize("B", [2, 8, 9, 16, 17, 33, 64])
def test_split_draw_part_counts(B):
    """spec_verify_step at batches where the number of parts per sequence
    changes (headline-length rows, 126 sweep items), against the oracle and
    bit for bit against the two calls."""
    wl = synth.workload("headline", B=B, K=2, V=128256, name=f"parts{B}")
    inp = synth.make_inputs(wl, seed=100 + B, device="cuda")
    say(f"[parts] B={B}: step vs two calls vs oracle")
    a = parity.gpu_verify(inp, path="two_call")
    b = parity.gpu_verify(inp, path="step")
    for k in a:
        assert a[k].tobytes() == b[k].tobytes(), k
    o = parity.oracle_verify(synth.to_host_arrays(inp))
    parity.assert_parity(parity.compare(b, o, inp["T"]), f"parts B={B}")


def test_repeatable_and_stream_independent():
    inp = synth.make_inputs("small", seed=5, device="cuda")
    torch.cuda.synchronize()
    a = parity.gpu_verify(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = parity.gpu_verify(inp, stream=s)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("wl,B", [("headline", 256), ("small", 64), ("small", 31),
                                   ("batch1", 1), ("headline", 7), ("large", 3)])
def test_step_equals_two_call_and_reuses_workspace(wl, B):
    """spec_verify_step splits each sequence's draw over several workgroups
    for small batches; every output is the same bits as the two-call path's
    (the split draw forms the same sums in the same order), and every call
    leaves the workspace's counters at zero for the next."""
    from speculative_sampling_verification_softmax_amd import binding
    inp = synth.make_inputs(wl, seed=11, device="cuda", B=B)
    torch.cuda.synchronize()
    say(f"[step] {wl} B={B}: two calls, then the step three times on one workspace")
    a = parity.gpu_verify(inp, path="two_call")
    K, V = inp["tokens"].shape[1], inp["target"].shape[2]
    ws = binding.new_workspace(B, K, V, inp["target"].dtype, "cuda")
    counters = (B * 4 + 255) // 256 * 256
    for rep in range(3):
        b = parity.gpu_verify(inp, path="step", workspace=ws)
        for k in a:
            assert a[k].tobytes() == b[k].tobytes(), f"{k} call {rep}"
        if rep == 0:
            first = b
        else:
            for k in first:
                np.testing.assert_array_equal(first[k], b[k], err_msg=f"step repeat {k}")
        dump = ws[:counters].view(torch.int32).cpu().numpy()
        assert np.all(dump == 0), "counters not reset"


def test_step_smaller_batch_after_larger_on_same_workspace():
    """One workspace, sized for the largest of the calls, serves them in turn
    (each call leaves its counters zero)."""
    from speculative_sampling_verification_softmax_amd import binding
    Bs = (64, 31, 5, 1)
    need = max(binding.workspace_size(B, 4, 32000, torch.bfloat16) for B in Bs)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for B in Bs:
        inp = synth.make_inputs("small", seed=B, device="cuda", B=B)
        say(f"[step] small B={B} on a workspace of {need} bytes")
        g = parity.gpu_verify(inp, path="step", workspace=ws)
        o = parity.oracle_verify(synth.to_host_arrays(inp))
        parity.assert_parity(parity.compare(g, o, inp["T"]), f"step B={B}")


@pytest.mark.parametrize("path,B", [("two_call", 16), ("step", 16), ("step", 1)])
def test_phase_stamped_build_matches_the_library(path, B):
    """libspec_phases.so (the kernels with their phase timestamps compiled in,
    which bench.py --mode phases times) gives the library's outputs bit for
    bit, and its stamps are in phase order in every workgroup."""
    import ctypes
    from speculative_sampling_verification_softmax_amd import binding
    from speculative_sampling_verification_softmax_amd import build as hip_build
    wl = "small" if B > 1 else "batch1"
    inp = synth.make_inputs(wl, seed=29, device="cuda", B=B)
    K, V = inp["tokens"].shape[1], inp["target"].shape[2]
    ws = binding.new_workspace(B, K, V, inp["target"].dtype, "cuda")
    say(f"[phases] {wl} B={B} {path}: library, then the stamped build")
    a = parity.gpu_verify(inp, path=path, workspace=ws)
    ph = binding.open_library(hip_build.PHASES_LIB)
    ph.spec_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    main = binding.load()
    binding._lib = ph
    try:
        torch.cuda.synchronize()
        assert ph.spec_phase_clear() == 0
        b = parity.gpu_verify(inp, path=path, workspace=ws)
        torch.cuda.synchronize()
        rows = np.zeros((8192, 2), np.uint64)
        draw = np.zeros((8192, 8), np.uint64)
        assert ph.spec_phase_stamps(rows.ctypes.data, rows.nbytes, 0) == 0
        assert ph.spec_phase_stamps(draw.ctypes.data, draw.nbytes, 1) == 0
    finally:
        binding._lib = main
    for k in a:
        assert a[k].tobytes() == b[k].tobytes(), k
    R = B * (2 * K + 1)
    r = rows[:R].astype(np.int64)
    assert np.all(r[:, 0] > 0) and np.all(r[:, 1] >= r[:, 0]) and not np.any(rows[R:])
    nwg = int(np.count_nonzero(draw[:, 0]))
    d = draw[:nwg].astype(np.int64)
    if path == "step":  # the split draw: parts per sequence, then the finishing part's stamps
        assert nwg % B == 0 and nwg > B
        assert np.all(np.diff(d[:, :4], axis=1) >= 0)
        fin = d[:, 4] > 0
        assert fin.sum() == B and np.all(np.diff(d[fin][:, 3:7], axis=1) >= 0)
    else:  # one workgroup per sequence, every phase stamped in order
        assert nwg == B and np.all(np.diff(d[:, :7], axis=1) >= 0)


@pytest.mark.parametrize("wl", ["small", "headline"])
def test_two_call_equals_three_call_bit_for_bit(wl):
    """spec_verify_sample runs the same accept and draw arithmetic as spec_verify
    plus spec_residual_sample: every output must be identical, floats included."""
    inp = synth.make_inputs(wl, seed=7, device="cuda")
    say(f"[two_call] {wl}: three calls vs two calls")
    a = parity.gpu_verify(inp, path="three_call")
    b = parity.gpu_verify(inp, path="two_call")
    for k in ("num_accepted", "out_tokens", "num_emitted"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    for k in ("target_stats", "draft_stats", "probs"):
        assert a[k].tobytes() == b[k].tobytes(), k


def test_two_call_repeats_bit_for_bit_under_load():
    """The draw's sweep hands its items to waves in the order the hardware
    schedules them, and every sum is formed per item and added in item order:
    repeated calls, with another stream's copies competing for the CUs, give
    identical bits."""
    inp = synth.make_inputs("headline", seed=3, device="cuda")
    torch.cuda.synchronize()
    say("[repeat] headline two_call: reference call")
    first = parity.gpu_verify(inp, path="two_call")
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()
    for rep in range(4):
        with torch.cuda.stream(side):
            for _ in range(4):
                dst.copy_(src)
        say(f"[repeat] call {rep} with copies on a second stream")
        b = parity.gpu_verify(inp, path="two_call")
        torch.cuda.synchronize()
        for k in first:
            np.testing.assert_array_equal(first[k], b[k], err_msg=f"{k} repeat {rep}")
