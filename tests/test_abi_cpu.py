"""CPU checks of the C ABI: the library loads, exports every symbol that
include/spec_softmax.h declares, and rejects bad arguments synchronously with
SPEC_ERR_INVALID_ARG (validation runs before any HIP call, so no GPU is needed)."""
import ctypes
import math
import os
import re

import pytest

from speculative_sampling_verification_softmax_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_softmax.h")


def _lib():
    if not os.path.exists(binding.LIB_PATH):
        from speculative_sampling_verification_softmax_amd import build
        build.build()
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(spec_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_phase_stamps_only_in_the_measurement_build():
    """libspec_phases.so (the kernels with their phase timestamps) exports the
    stamp readers as well as every declared entry point; the library itself
    has none of them and rejects nothing differently."""
    from speculative_sampling_verification_softmax_amd import build
    if not os.path.exists(build.PHASES_LIB):
        build.build()
    lib = _lib()
    assert not hasattr(lib, "spec_phase_stamps") and not hasattr(lib, "spec_phase_clear")
    ph = ctypes.CDLL(build.PHASES_LIB)
    for name in declared_functions() + ["spec_phase_stamps", "spec_phase_clear"]:
        assert hasattr(ph, name), name
    ph.spec_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    buf = (ctypes.c_uint64 * 16)()
    assert ph.spec_phase_stamps(None, 8, 0) == 1  # SPEC_ERR_INVALID_ARG
    assert ph.spec_phase_stamps(buf, 8, 2) == 1  # SPEC_ERR_INVALID_ARG
    assert ph.spec_phase_stamps(buf, 8192 * 2 * 8 + 8, 0) == 1  # SPEC_ERR_INVALID_ARG


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(SPEC_\w+)\s+(\S+(?:\s*<<\s*\d+\))?)", text))
    assert int(consts["SPEC_DTYPE_F32"]) == binding.SPEC_DTYPE_F32
    assert int(consts["SPEC_DTYPE_BF16"]) == binding.SPEC_DTYPE_BF16
    assert int(consts["SPEC_MAX_K"]) == binding.SPEC_MAX_K
    assert eval(consts["SPEC_MAX_V"]) == binding.SPEC_MAX_V
    assert int(consts["SPEC_MAX_ROWS"]) == binding.SPEC_MAX_ROWS == (2**32 - 1) // 1024


def test_status_strings():
    L = _lib()
    for rc in range(4):
        assert L.spec_status_string(rc)
    assert b"INVALID_ARG" in L.spec_status_string(1)
    assert L.spec_status_string(99) == b"unknown status"


# fake, never-dereferenced addresses: validation must reject before any launch
P = 4096


@pytest.mark.parametrize("args", [
    dict(tgt=None), dict(dft=None), dict(dtype=2), dict(B=0), dict(K=0),
    dict(K=binding.SPEC_MAX_K + 1), dict(V=0), dict(V=binding.SPEC_MAX_V + 1),
    dict(T=0.0), dict(T=-1.0), dict(T=math.nan), dict(T=math.inf),
    dict(tgt=P + 1), dict(ts=None), dict(ds=None), dict(ts=P + 2),
])
def test_stats_rejects_bad_arguments(args):
    L = _lib()
    a = dict(tgt=P, dft=P, dtype=1, B=2, K=3, V=100, T=1.0, ts=P, ds=P)
    a.update(args)
    rc = L.spec_softmax_stats(a["tgt"], a["dft"], a["dtype"], a["B"], a["K"], a["V"], a["T"],
                              a["ts"], a["ds"], None)
    assert rc == 1


@pytest.mark.parametrize("missing", ["tok", "uni", "ts", "ds", "nacc", "out"])
def test_verify_rejects_null_pointers(missing):
    L = _lib()
    a = dict(tok=P, uni=P, ts=P, ds=P, nacc=P, out=P)
    a[missing] = None
    rc = L.spec_verify(P, P, 0, a["tok"], a["uni"], a["ts"], a["ds"], 2, 3, 100, 1.0,
                       a["nacc"], a["out"], None, None)
    assert rc == 1


@pytest.mark.parametrize("missing", ["uni", "ts", "ds", "nacc", "out"])
def test_residual_rejects_null_pointers(missing):
    L = _lib()
    a = dict(uni=P, ts=P, ds=P, nacc=P, out=P)
    a[missing] = None
    rc = L.spec_residual_sample(P, P, 0, a["uni"], a["ts"], a["ds"], a["nacc"], 2, 3, 100, 1.0,
                                a["out"], None, None)
    assert rc == 1


def test_residual_rejects_misaligned_optional_output():
    L = _lib()
    rc = L.spec_residual_sample(P, P, 0, P, P, P, P, 2, 3, 100, 1.0, P, P + 1, None)
    assert rc == 1


def test_binding_fails_loudly_without_library(tmp_path):
    binding_mod = binding
    saved = binding_mod._lib
    try:
        binding_mod._lib = None
        with pytest.raises(binding.SpecError):
            binding_mod.load(str(tmp_path / "missing.so"))
    finally:
        binding_mod._lib = saved


def test_workspace_size_host_only():
    L = _lib()
    L.spec_verify_step_workspace_size.restype = ctypes.c_size_t
    size = lambda *a: L.spec_verify_step_workspace_size(*a)
    # from 65 sequences on, one workgroup per sequence: the counters only
    assert size(256, 8, 128256, 1) == 1024
    assert size(65, 4, 32000, 1) == 512
    # 64 or fewer split the draw: one record of 160 bytes per sweep item of
    # 1024 bf16 / 512 fp32 tokens and sequence, after the counters
    assert size(1, 4, 32000, 0) == 256 + (63 * 160 + 255) // 256 * 256
    assert size(31, 4, 32000, 1) == 256 + 31 * 32 * 160
    assert size(64, 4, 32000, 1) == 256 + 64 * 32 * 160
    # the no-allocation array's limits as its declaration states them
    cap = binding.SPEC_NOALLOC_SCRATCH_BYTES
    assert size(64, 1, 800000, 1) <= cap < size(64, 1, 900000, 1)
    assert size(64, 1, 400000, 0) <= cap < size(64, 1, 450000, 0)
    assert size(32, 1, 1 << 20, 1) <= cap
    assert size(16, 4, 32000, 0) > size(16, 4, 32000, 1)  # fp32 items hold fewer tokens
    assert size(0, 8, 100, 1) == 0
    assert size(1, 0, 100, 1) == 0
    assert size(1, 1, 100, 7) == 0
    assert size(1, 65, 100, 1) == 0
    assert size(4194303, 1, 100, 1) == 0  # 3 * B rows past one launch


@pytest.mark.parametrize("case", ["null_ws", "small_ws", "misaligned_ws", "null_out", "bad_T"])
def test_step_rejects_bad_arguments(case):
    L = _lib()
    L.spec_verify_step_workspace_size.restype = ctypes.c_size_t
    need = L.spec_verify_step_workspace_size(2, 3, 100, 1)
    ws, nbytes, out, T = P * 256, need, P, 1.0
    if case == "null_ws":
        ws = None
    elif case == "small_ws":
        nbytes = need - 1
    elif case == "misaligned_ws":
        ws = P * 256 + 16
    elif case == "null_out":
        out = None
    elif case == "bad_T":
        T = -1.0
    rc = L.spec_verify_step(P, P, 1, P, P, 2, 3, 100, T, P, P, P, out, None, None, ws,
                            ctypes.c_size_t(nbytes), None)
    assert rc == 1


@pytest.mark.parametrize("case", ["too_big", "null_tok", "bad_K", "misaligned"])
def test_noalloc_rejects_before_touching_the_device(case):
    """spec_verify_step_noalloc checks its arguments, then whether the shape's
    workspace fits its static scratch, before it looks the scratch up or
    launches anything."""
    L = _lib()
    B, K, V, dtype, tok, ne = 2, 3, 100, 1, P, None
    if case == "too_big":  # 31 sequences of 2^20 fp32 tokens: 10 MB of item records
        B, K, V, dtype = 31, 1, 1 << 20, 0
    elif case == "null_tok":
        tok = None
    elif case == "bad_K":
        K = 65
    else:
        ne = P + 2
    rc = L.spec_verify_step_noalloc(P, P, dtype, tok, P, B, K, V, ctypes.c_float(1.0), P, P, P, P,
                                    None, ne, None)
    assert rc == (2 if case == "too_big" else 1)
    L.spec_verify_step_workspace_size.restype = ctypes.c_size_t
    if case == "too_big":
        assert L.spec_verify_step_workspace_size(B, K, V, dtype) > binding.SPEC_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("fn", ["stats", "verify_sample", "sample", "filter"])
def test_launch_size_limit(fn):
    """Shapes whose launch would exceed 2^32 - 1 threads are argument errors,
    reported before anything is enqueued."""
    L = _lib()
    if fn == "stats":  # 2K+1 = 3 rows per sequence
        assert L.spec_softmax_stats(P, P, 1, 1398102, 1, 4, ctypes.c_float(1.0), P, P, None) == 1
        assert L.spec_softmax_stats(P, P, 1, 4194304, 1, 4, ctypes.c_float(1.0), P, P, None) == 1
    elif fn == "verify_sample":
        assert L.spec_verify_sample(P, P, 1, P, P, P, P, 1398102, 1, 4, ctypes.c_float(1.0), P, P,
                                    None, None, None) == 1
    elif fn == "sample":
        assert L.spec_sample(P, 1, 4194304, 4, ctypes.c_float(1.0), P, P, P, None) == 1
    else:
        assert L.spec_filter(P, 1, 4194304, 4, ctypes.c_float(1.0), 2, ctypes.c_float(1.0), P,
                             None, None, None) == 1


@pytest.mark.parametrize("case", ["tgt", "tok", "am", "nacc", "out", "dtype", "K", "misaligned"])
def test_greedy_rejects_bad_arguments(case):
    L = _lib()
    a = dict(tgt=P, dtype=1, tok=P, K=3, am=P, nacc=P, out=P, ne=None)
    if case == "dtype":
        a["dtype"] = 5
    elif case == "K":
        a["K"] = 0
    elif case == "misaligned":
        a["ne"] = P + 2
    else:
        a[case] = None
    rc = L.spec_greedy_verify(a["tgt"], a["dtype"], a["tok"], 2, a["K"], 100, a["am"], a["nacc"],
                              a["out"], a["ne"], None)
    assert rc == 1


@pytest.mark.parametrize("case", ["logits", "uni", "stats", "tok", "R", "V", "T", "misaligned"])
def test_sample_rejects_bad_arguments(case):
    L = _lib()
    a = dict(logits=P, R=4, V=100, T=1.0, uni=P, stats=P, tok=P)
    if case == "R":
        a["R"] = 0
    elif case == "V":
        a["V"] = binding.SPEC_MAX_V + 1
    elif case == "T":
        a["T"] = 0.0
    elif case == "misaligned":
        a["tok"] = P + 1
    else:
        a[case] = None
    rc = L.spec_sample(a["logits"], 1, a["R"], a["V"], a["T"], a["uni"], a["stats"], a["tok"], None)
    assert rc == 1


@pytest.mark.parametrize("case", ["logits", "thr", "R", "V", "T", "top_k", "top_p0", "top_pnan",
                                  "misaligned_thr", "misaligned_out", "misaligned_stats",
                                  "overlap"])
def test_filter_rejects_bad_arguments(case):
    L = _lib()
    a = dict(logits=P, R=4, V=100, T=1.0, k=10, p=0.9, thr=P + 4096, stats=None, out=P + 65536)
    if case == "R":
        a["R"] = 0
    elif case == "V":
        a["V"] = binding.SPEC_MAX_V + 1
    elif case == "T":
        a["T"] = float("inf")
    elif case == "top_k":
        a["k"] = -1
    elif case == "top_p0":
        a["p"] = 0.0
    elif case == "top_pnan":
        a["p"] = math.nan
    elif case == "misaligned_thr":
        a["thr"] = P + 4098
    elif case == "misaligned_stats":
        a["stats"] = P + 8194
    elif case == "misaligned_out":
        a["out"] = P + 65537  # bf16 rows: odd byte address
    elif case == "overlap":
        a["out"] = P + 2  # shares all but one element with the input rows
    else:
        a[case] = None
    rc = L.spec_filter(a["logits"], 1, a["R"], a["V"], a["T"], a["k"], a["p"], a["thr"],
                       a["stats"], a["out"], None)
    assert rc == 1


@pytest.mark.parametrize("case", ["tgt", "dft", "tok", "uni", "ts", "ds", "nacc", "out", "K", "T",
                                  "misaligned"])
def test_verify_sample_rejects_bad_arguments(case):
    L = _lib()
    a = dict(tgt=P, dft=P, tok=P, uni=P, ts=P, ds=P, nacc=P, out=P, K=3, T=1.0, probs=None, ne=None)
    if case == "K":
        a["K"] = binding.SPEC_MAX_K + 1
    elif case == "T":
        a["T"] = -1.0
    elif case == "misaligned":
        a["ne"] = P + 3
    else:
        a[case] = None
    rc = L.spec_verify_sample(a["tgt"], a["dft"], 1, a["tok"], a["uni"], a["ts"], a["ds"], 2,
                              a["K"], 100, a["T"], a["nacc"], a["out"], a["probs"], a["ne"], None)
    assert rc == 1
