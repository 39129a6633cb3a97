"""GPU-vs-oracle comparison with boundary accounting.

Rule (the tolerance stated for this path): accepted counts and emitted tokens
must be identical, except where the oracle's own uniform lies within 1e-6 of
the boundary that separates the two outcomes; such draws are counted and must
stay under 1e-4 of all draws.  After a differing accept decision the two runs
go different ways, so that sequence counts one flagged draw and is not
compared further.  Normalised probabilities (row normalisers s and the
probabilities at the drafted tokens) must agree within 1e-5 relative.
"""
from __future__ import annotations

import numpy as np

import oracle

BOUNDARY = 1e-6
MAX_FLAGGED_FRACTION = 1e-4
PROB_RTOL = 1e-5


PATHS = ("three_call", "two_call", "step")


def gpu_verify(inp: dict, stream=None, path: str = "three_call", workspace=None) -> dict:
    """Run the HIP verify through the C ABI: the three calls, the two calls
    (stats, then spec_verify_sample), or spec_verify_step (with a fresh zeroed
    workspace unless one is given)."""
    import torch
    from speculative_sampling_verification_softmax_amd import binding
    if path == "three_call":
        out = binding.verify_all(inp["target"], inp["draft"], inp["tokens"], inp["uniforms"],
                                 inp["T"], stream=stream)
    elif path == "two_call":
        out = binding.verify_two_call(inp["target"], inp["draft"], inp["tokens"],
                                      inp["uniforms"], inp["T"], stream=stream)
    elif path == "step":
        B, K1, V = inp["target"].shape
        if workspace is None:
            workspace = binding.new_workspace(B, K1 - 1, V, inp["target"].dtype,
                                              inp["target"].device)
        out = binding.verify_step(inp["target"], inp["draft"], inp["tokens"], inp["uniforms"],
                                  inp["T"], workspace, stream=stream)
    else:
        raise ValueError(path)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle_verify(host: dict, seqs=None, nthreads: int = 0) -> dict:
    """Run the oracle on all sequences, or on the listed subset."""
    T = float(np.float32(host["T"]))
    tgt, dft, tok, uni = host["target"], host["draft"], host["tokens"], host["uniforms"]
    if seqs is not None:
        tgt, dft, tok, uni = tgt[seqs], dft[seqs], tok[seqs], uni[seqs]
    return oracle.verify(tgt, dft, tok, uni, T, nthreads=nthreads)


def _sel(a, seqs):
    return a if seqs is None else a[seqs]


def compare(g: dict, o: dict, T: float, seqs=None) -> dict:
    """g: GPU outputs (all sequences); o: oracle outputs (for `seqs` or all)."""
    T = float(np.float32(T))
    gn = _sel(g["num_accepted"], seqs)
    gout = _sel(g["out_tokens"], seqs)
    gne = _sel(g["num_emitted"], seqs)
    on, oout = o["num_accepted"], o["out_tokens"]
    B, K1 = oout.shape
    K = K1 - 1
    failures, flagged = [], []
    draws = 0
    for b in range(B):
        nb_o, nb_g = int(on[b]), int(gn[b])
        if nb_o < 0 or nb_g < 0:
            if nb_o != nb_g or not np.all(gout[b] == -1):
                failures.append((b, "validity", nb_g, nb_o))
            continue
        draws += min(nb_o + 1, K) + 1
        if gne[b] != nb_g + 1:
            failures.append((b, "num_emitted", int(gne[b]), nb_g + 1))
        if nb_g != nb_o:
            t = min(nb_g, nb_o)
            d = float(o["accept_dist"][b, t])
            (flagged if d < BOUNDARY else failures).append((b, f"accept@{t}", nb_g, nb_o, d))
            continue
        if not np.array_equal(gout[b, :nb_o], oout[b, :nb_o]):
            failures.append((b, "prefix", gout[b].tolist(), oout[b].tolist()))
            continue
        if np.any(gout[b, nb_o + 1:] != -1):
            failures.append((b, "padding", gout[b].tolist()))
        if gout[b, nb_o] != oout[b, nb_o]:
            d = float(o["draw_dist"][b])
            (flagged if d < BOUNDARY else failures).append(
                (b, "draw", int(gout[b, nb_o]), int(oout[b, nb_o]), d))

    # normalisers and probabilities
    def stats_err(gs, os_):
        gs = gs.reshape(-1, 2).astype(np.float64)
        os_ = os_.reshape(-1, 2)
        bad_o = np.isnan(os_[:, 1])
        bad_g = np.isnan(gs[:, 1])
        mism = int(np.sum(bad_o != bad_g))
        ok = ~bad_o & ~bad_g
        m_exact = int(np.sum((gs[ok, 0] / T) != os_[ok, 0]))
        rel = np.abs(gs[ok, 1] - os_[ok, 1]) / os_[ok, 1]
        return mism, m_exact, float(rel.max()) if rel.size else 0.0

    tm, tmx, trel = stats_err(_sel(g["target_stats"], seqs), o["target_stats"])
    dm, dmx, drel = stats_err(_sel(g["draft_stats"], seqs), o["draft_stats"])
    gp = _sel(g["probs"], seqs).astype(np.float64)
    op = o["probs"]
    okp = ~np.isnan(op)
    prel = np.abs(gp[okp] - op[okp]) / (op[okp] + 1e-37 / PROB_RTOL)
    return dict(
        sequences=B, draws=draws, flagged=flagged, failures=failures,
        stats_validity_mismatch=tm + dm, stats_max_not_exact=tmx + dmx,
        stats_max_rel=max(trel, drel),
        probs_nan_mismatch=int(np.sum(np.isnan(gp) != np.isnan(op))),
        probs_max_rel=float(prel.max()) if prel.size else 0.0,
        accept_hist=np.bincount(on[on >= 0], minlength=K + 1).tolist(),
    )


def assert_parity(rep: dict, label: str = ""):
    assert rep["failures"] == [], f"{label}: non-boundary mismatches {rep['failures'][:10]}"
    assert rep["stats_validity_mismatch"] == 0, label
    assert rep["stats_max_not_exact"] == 0, f"{label}: row max differs"
    assert rep["stats_max_rel"] <= PROB_RTOL, f"{label}: stats rel err {rep['stats_max_rel']}"
    assert rep["probs_nan_mismatch"] == 0, label
    assert rep["probs_max_rel"] <= PROB_RTOL, f"{label}: probs rel err {rep['probs_max_rel']}"
    assert len(rep["flagged"]) <= MAX_FLAGGED_FRACTION * max(rep["draws"], 1), \
        f"{label}: {len(rep['flagged'])} boundary draws of {rep['draws']}"
