"""The e^z table compiled into the library (smoothed statistics of bf16 rows):
written by vocab_softmax_cross_row_amd/csrc/gen_exp_table.py at build time.
Checked here against the C library's exp through Python's math.exp (at most
one unit in the last place apart), at e and 1/e exactly, and for its layout:
entry 2 off + sign is the bf16 pattern (0x3780 + off) | sign << 15, then two
NaN entries."""
import importlib.util
import math
import os
import re
import struct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "vocab_softmax_cross_row_amd", "csrc", "gen_exp_table.py")
LAUNCH_H = os.path.join(ROOT, "vocab_softmax_cross_row_amd", "csrc", "ce_launch.h")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_exp_table", GEN)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def _ulps(a, b):
    ia = struct.unpack("<q", struct.pack("<d", a))[0]
    ib = struct.unpack("<q", struct.pack("<d", b))[0]
    return abs(ia - ib)


def _read(path):
    text = open(path).read()
    macros = dict(re.findall(r"#define (CE_EXP_TABLE_\w+) (\w+)", text))
    body = [l.strip().rstrip(",") for l in text.splitlines()
            if l.strip() and not l.startswith(("//", "#"))]
    return macros, body


def test_layout_matches_the_kernel_constants(tmp_path):
    g = _gen()
    h = open(LAUNCH_H).read()
    lo = int(re.search(r"kExpTabLo = (0x[0-9a-fA-F]+)", h).group(1), 16)
    half = int(re.search(r"kExpTabHalf = (\d+)", h).group(1))
    assert (g.LO, g.HALF) == (lo, half)
    macros, body = _read(g.write(str(tmp_path / "t.inc")))
    assert int(macros["CE_EXP_TABLE_LO"], 16) == lo
    assert int(macros["CE_EXP_TABLE_HALF"]) == half
    assert int(macros["CE_EXP_TABLE_ENTRIES"]) == len(body) == 2 * half + 2
    assert body[-2:] == ['__builtin_nan("")'] * 2


def test_values_against_the_c_library_exp(tmp_path):
    g = _gen()
    _, body = _read(g.write(str(tmp_path / "t.inc")))
    vals = [float.fromhex(v) for v in body[:-2]]
    worst = 0
    for i, v in enumerate(vals):
        off, sign = i >> 1, i & 1
        z = _bf16((g.LO + off) | (sign << 15))
        assert (z < 0) == bool(sign) and 2.0 ** -16 <= abs(z) < 512.0
        worst = max(worst, _ulps(v, math.exp(z)))
    assert worst <= 1
    # e and 1/e: bf16 1.0 is pattern 0x3f80
    i1 = 2 * (0x3F80 - g.LO)
    assert vals[i1] == math.e and vals[i1 + 1] == 0.36787944117144233
    # the two ends of the table: 2^-16 and the largest bf16 below 512
    # (e^x = 1 + x + x^2/2 + x^3/6 + ..., x = +-2^-16, to 17 digits)
    assert vals[0] == 1.0000152589054785 and vals[1] == 0.9999847413273523
    z_hi = _bf16(g.LO + g.HALF - 1)
    assert z_hi == 510.0 and _ulps(vals[-1], math.exp(-510.0)) <= 1
