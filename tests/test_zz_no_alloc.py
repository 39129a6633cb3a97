"""spec_verify_step_noalloc (the library's static scratch, no workspace)
against spec_verify_step (a caller workspace) through the C ABI: calls in a
row on the same device, each smaller than the one before, every output the
same bits.  The draw of these batches (64 sequences or fewer) is split over
several workgroups, so the scratch's counters and records are in use, and a
call after a larger one finds its counters cleared."""
import sys

import numpy as np
import pytest
import torch

import parity
from speculative_sampling_verification_softmax_amd import binding, synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
    binding.load()


def test_noalloc_equals_step_on_calls_in_a_row():
    for wl, B in (("small", 64), ("small", 24), ("small", 5), ("batch1", 1)):
        inp = synth.make_inputs(wl, seed=B, device="cuda", B=B)
        K, V = inp["tokens"].shape[1], inp["target"].shape[2]
        say(f"[noalloc] {wl} B={B} K={K} V={V}: step with a workspace, then noalloc")
        ws = binding.new_workspace(B, K, V, inp["target"].dtype, "cuda")
        a = binding.verify_step(inp["target"], inp["draft"], inp["tokens"], inp["uniforms"],
                                inp["T"], ws)
        b = binding.verify_step_noalloc(inp["target"], inp["draft"], inp["tokens"],
                                        inp["uniforms"], inp["T"])
        torch.cuda.synchronize()
        for k in a:
            assert a[k].cpu().numpy().tobytes() == b[k].cpu().numpy().tobytes(), f"{wl} B={B} {k}"
        o = parity.oracle_verify(synth.to_host_arrays(inp))
        g = {k: v.cpu().numpy() for k, v in b.items()}
        parity.assert_parity(parity.compare(g, o, inp["T"]), f"noalloc {wl} B={B}")
