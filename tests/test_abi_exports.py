"""The C ABI library loads and exports every function include/vocab_ce.h
declares; host-only entry points and argument checks work without a GPU
(every call below returns before any HIP call is made)."""
import ctypes
import os
import re

import pytest

from vocab_softmax_cross_row_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vocab_ce.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ce_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from vocab_softmax_cross_row_amd import build
        build.build()
    return B.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_sizes_match_header():
    assert ctypes.sizeof(B.CEProblem) == 56
    assert B.ROW_STATS_DTYPE.itemsize == B.ROW_STATS_BYTES == 32
    assert B.ROW_FINAL_DTYPE.itemsize == B.ROW_FINAL_BYTES == 24


def test_host_only_calls(lib):
    assert B.ce_version() == 100
    assert B.ce_status_str(0) == "CE_OK"
    assert "label_smoothing" in B.ce_status_str(-3)
    p = B.make_problem(16384, 128256)
    assert B.ce_workspace_bytes(p, B.CE_OP_BACKWARD) == 0
    fused = B.ce_workspace_bytes(p, B.CE_OP_FUSED)
    assert fused >= 16384 * (32 + 24 + 4)
    small = B.make_problem(8, 128256)   # few rows: the split-V grid needs partials
    assert B.ce_workspace_bytes(small, B.CE_OP_FUSED) >= 8 * 32 * 2
    bad = B.make_problem(4, 10, label_smoothing=1.5)
    assert B.ce_workspace_bytes(bad, B.CE_OP_FUSED) == 0
    # the measurement entry point takes both events or neither (checked
    # before anything else, so nothing is launched here)
    nul = [None] * 9
    for ev in ((ctypes.c_void_p(16), None), (None, ctypes.c_void_p(16))):
        assert lib.ce_fused_fwd_bwd_timed(ctypes.byref(p), None, 1, None, None, None, None,
                                          None, None, None, 1, 16, None, 0, None, *ev) == -10
    del nul


@pytest.mark.parametrize("kw,status", [
    (dict(label_smoothing=1.0), -3), (dict(label_smoothing=-0.1), -3),
    (dict(reduction=7), -5), (dict(ld=5), -2), (dict(vocab_start=5), -2),
])
def test_argument_checks_before_any_launch(lib, kw, status):
    args = dict(T=4, V_local=10)
    args.update({k: v for k, v in kw.items() if k in ("ld",)})
    p = B.make_problem(args["T"], args["V_local"], args.get("ld"),
                       **{k: v for k, v in kw.items() if k != "ld"})
    rc = lib.ce_fused_fwd_bwd(ctypes.byref(p), None, 1, None, None, None, None, None, None,
                              None, 1, 10, None, 0, None)
    assert rc == status


def test_null_and_dtype_checks(lib):
    p = B.make_problem(4, 10)
    assert lib.ce_fused_fwd_bwd(None, None, 1, None, None, None, None, None, None, None, 1, 10,
                                None, 0, None) == -1
    assert lib.ce_fused_fwd_bwd(ctypes.byref(p), None, 1, None, None, None, None, None, None,
                                None, 1, 10, None, 0, None) == -1
    assert lib.ce_backward(ctypes.byref(p), None, 9, None, None, None, None, None, 1, 10,
                           None) == -4
    assert lib.ce_merge_shard_stats(ctypes.byref(p), 0, None, None, None, None, None, None,
                                    None, None, 0, None) == -7
    shard = B.make_problem(4, 5, vocab_start=5, V_total=10)
    one = ctypes.c_void_p(16)
    assert lib.ce_forward(ctypes.byref(shard), one, 1, one, one, None, one, None, None, None,
                          None, 0, None) == -10


def test_header_constants_match_the_binding():
    """The binding's copies of the header's #define constants."""
    hdr = open(os.path.join(ROOT, "include", "vocab_ce.h")).read()
    for name in ("CE_LINEAR_CHUNK", "CE_MAX_SHARDS"):
        m = re.search(r"#define\s+" + name + r"\s+(\d+)", hdr)
        assert m, name
        assert int(m.group(1)) == getattr(B, name), name
    m = re.search(r"#define CE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == B.CE_NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """Returns CE_ERR_WORKSPACE on the host, before any HIP call, when the
    fused workspace would not fit the static scratch array."""
    p = B.make_problem(200000, 1000)
    assert B.ce_workspace_bytes(p, B.CE_OP_FUSED) > B.CE_NOALLOC_SCRATCH_BYTES
    assert lib.ce_fused_fwd_bwd_noalloc(ctypes.byref(p), None, 1, None, None, None, None, None,
                                        None, None, 1, 1000, None) == -6
    bad = B.make_problem(4, 10, label_smoothing=2.0)
    assert lib.ce_fused_fwd_bwd_noalloc(ctypes.byref(bad), None, 1, None, None, None, None, None,
                                        None, None, 1, 10, None) == -3


def test_linear_problem_struct_and_workspace(lib):
    assert ctypes.sizeof(B.CELinearProblem) == 48
    p = B.make_linear_problem(8192, 2048, 128256)
    fwd = B.ce_linear_workspace_bytes(p, 0)
    both = B.ce_linear_workspace_bytes(p, 1)
    # forward: fragment-major E and C, 16-byte per-(256-class tile, row)
    # statistics
    assert fwd >= (8192 + 128256) * 2048 * 2 + 501 * 8192 * 16
    # backward adds E^T, C^T of one chunk and one chunk of G and G^T; at 8192
    # tokens a chunk is 8192 classes (G and G^T within 256 MiB), and the
    # whole workspace stays below 1 GB
    vc = 8192
    assert both >= fwd + 8192 * 2048 * 2 + 2048 * vc * 2 + 2 * 8192 * vc * 2
    assert both < 10 ** 9
    k = B.make_linear_problem(8192, 2048, 128256, accum="kahan")
    assert B.ce_linear_workspace_bytes(k, 1) >= both + 8192 * 2048 * 4
    assert B.ce_linear_workspace_bytes(B.make_linear_problem(4, 12, 10), 0) == 0  # D % 8
    assert B.ce_linear_workspace_bytes(B.make_linear_problem(4, 16, 10, accum=5), 0) == 0
    # gradient filtering adds its per-chunk flags and lists to the backward only
    f = B.make_linear_problem(8192, 2048, 128256, filter_eps=2.0 ** -8)
    tiles = (8192 // 256) * (8192 // 256)
    assert B.ce_linear_workspace_bytes(f, 1) >= both + tiles * (16 + 4)
    assert B.ce_linear_workspace_bytes(f, 0) == fwd


@pytest.mark.parametrize("kw,status", [
    (dict(D=12), -2), (dict(D=0), -2), (dict(V=0), -2), (dict(N=-1), -2),
    (dict(label_smoothing=1.0), -3), (dict(reduction=9), -5), (dict(accum=3), -10),
    (dict(filter_eps=-1.0), -10), (dict(filter_eps=float("nan")), -10),
    (dict(filter_eps=float("inf")), -10),
])
def test_linear_argument_checks_before_any_launch(lib, kw, status):
    args = dict(N=4, D=16, V=10)
    args.update({k: v for k, v in kw.items() if k in args})
    p = B.make_linear_problem(args["N"], args["D"], args["V"],
                              **{k: v for k, v in kw.items() if k not in args})
    one = ctypes.c_void_p(256)
    rc = lib.ce_linear_fwd_bwd(ctypes.byref(p), one, one, one, None, None, None, None, None,
                               None, None, one, 1 << 40, None)
    assert rc == status


def test_linear_null_and_pairing_checks(lib):
    p = B.make_linear_problem(4, 16, 10)
    one = ctypes.c_void_p(256)
    ws = B.ce_linear_workspace_bytes(p, 1)
    # E missing
    assert lib.ce_linear_fwd_bwd(ctypes.byref(p), None, one, one, None, None, None, None, None,
                                 None, None, one, ws, None) == -1
    # dE without dC
    assert lib.ce_linear_fwd_bwd(ctypes.byref(p), one, one, one, None, None, None, None, None,
                                 one, None, one, ws, None) == -1
    # workspace too small
    assert lib.ce_linear_fwd_bwd(ctypes.byref(p), one, one, one, None, None, None, None, None,
                                 None, None, one, 16, None) == -6
    # misaligned E
    assert lib.ce_linear_fwd_bwd(ctypes.byref(p), ctypes.c_void_p(258), one, one, None, None,
                                 None, None, None, None, None, one, ws, None) == -2


def test_alias_checks_before_any_launch(lib):
    """grad may be the logits exactly (same pointer, stride and dtype: an
    in-place gradient); any other overlap is CE_ERR_ALIAS, found on the host."""
    p = B.make_problem(4, 10, 16)
    ws_bytes = B.ce_workspace_bytes(p, B.CE_OP_FUSED)
    base = 1 << 20
    ws = ctypes.c_void_p(1 << 30)
    one = ctypes.c_void_p(256)
    # overlapping by two bytes
    rc = lib.ce_fused_fwd_bwd(ctypes.byref(p), ctypes.c_void_p(base), 1, one, None, None, None,
                              None, None, ctypes.c_void_p(base + 2), 1, 16, ws, ws_bytes, None)
    assert rc == -8
    # same pointer, other stride
    rc = lib.ce_fused_fwd_bwd(ctypes.byref(p), ctypes.c_void_p(base), 1, one, None, None, None,
                              None, None, ctypes.c_void_p(base), 1, 20, ws, ws_bytes, None)
    assert rc == -8
    # same pointer, other dtype
    rc = lib.ce_backward(ctypes.byref(p), ctypes.c_void_p(base), 1, one, one, one, None,
                         ctypes.c_void_p(base), 0, 16, None)
    assert rc == -8
