"""The verify step captured in a HIP graph and replayed (the use the
no-allocation entry point exists for: callers that capture their serving
loop).  Each path is run once eagerly, captured once, then replayed several
times with eager work between the replays (the outputs overwritten with
garbage, other kernels on the stream); every replay must reproduce the eager
outputs bit for bit.  The library records no memset into a graph: the split
draw's counters end every call at zero, and the no-allocation scratch is
cleared by a fill kernel on its first, eager, call."""
import sys

import pytest
import torch

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


def outputs(B, K, dev):
    return dict(ts=torch.empty((B, K + 1, 2), dtype=torch.float32, device=dev),
                ds=torch.empty((B, K, 2), dtype=torch.float32, device=dev),
                n=torch.empty(B, dtype=torch.int32, device=dev),
                out=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                pr=torch.empty((B, K, 2), dtype=torch.float32, device=dev),
                ne=torch.empty(B, dtype=torch.int32, device=dev))


@pytest.mark.parametrize("path", ["two_call", "step", "noalloc"])
@pytest.mark.parametrize("wl,B", [("batch1", None), ("small", None), ("headline", 24)])
def test_graph_replays_match_eager(path, wl, B):
    from speculative_sampling_verification_softmax_amd import binding
    inp = synth.make_inputs(wl, seed=21, device="cuda", B=B)
    tgt, dft, tok, uni, T = inp["target"], inp["draft"], inp["tokens"], inp["uniforms"], inp["T"]
    Bn, K1, V = tgt.shape
    K = K1 - 1
    dev = tgt.device
    ws = binding.new_workspace(Bn, K, V, tgt.dtype, dev) if path == "step" else None
    o = outputs(Bn, K, dev)

    def launch():
        if path == "two_call":
            binding.softmax_stats(tgt, dft, T, o["ts"], o["ds"])
            binding.verify_sample(tgt, dft, tok, uni, o["ts"], o["ds"], T, o["n"], o["out"],
                                  o["pr"], o["ne"])
        elif path == "step":
            binding.verify_step(tgt, dft, tok, uni, T, ws, o["ts"], o["ds"], o["n"], o["out"],
                                o["pr"], o["ne"])
        else:
            binding.verify_step_noalloc(tgt, dft, tok, uni, T, o["ts"], o["ds"], o["n"], o["out"],
                                        o["pr"], o["ne"])

    say(f"[graph] {wl} B={Bn} K={K} V={V} {path}: eager call")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in o.items()}

    say(f"[graph] {wl} {path}: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for v in o.values():  # garbage in every output before each replay
            v.fill_(-7)
        junk.mul_(1.0001).add_(0.5)  # other work on the stream between replays
        g.replay()
        torch.cuda.synchronize()
        for k, v in o.items():
            assert torch.equal(v.view(torch.int32), ref[k].view(torch.int32)), \
                f"{wl} {path}: replay {rep} differs in {k}"
        if rep == 1:  # an eager call between replays leaves them unchanged
            launch()
            torch.cuda.synchronize()
    say(f"[graph] {wl} {path}: 4 replays identical to the eager call")
