"""Host-side logic of the matrix-core probes (no GPU): the operand lane map
is a bijection per lane half, packing places each logical K where the map
says, the code decoders agree with the oracle's format tables, and the probe
library (when built) exports its entry points."""
import ctypes
import os

import numpy as np
import pytest

from fp8_quantized_linear_mxq_amd.probe import mfma_probe as mp
from oracle import formats as fm


def test_kmap_is_a_bijection():
    for fp8 in (False, True):
        ks = sorted(mp._kmap(fp8, h, t) for h in (0, 1) for t in range(32))
        assert ks == list(range(64))
        # each lane's 32 slots cover both 32-blocks for E4M3, one for E2M1
        blocks = {mp._kmap(fp8, 0, t) // 32 for t in range(32)}
        assert blocks == ({0, 1} if fp8 else {0})


@pytest.mark.parametrize("kind", [0, 1, 2, 3, 4])
def test_pack_places_codes_by_the_map(kind):
    rng = np.random.default_rng(kind)
    K = mp._kdim(kind)
    codes = rng.integers(1, 15, size=(32, K)).tolist()
    ops = mp._pack(kind, codes, True).view(np.uint32)
    fp4 = kind == 1
    for lane in (0, 5, 33, 63):
        row, h = lane % 32, lane // 32
        for t in range(32 if kind in (0, 1, 2) else 8):
            if kind in (0, 1, 2):
                k = mp._kmap(not fp4, h, t)
                if fp4:
                    got = (int(ops[lane, t // 8]) >> (4 * (t % 8))) & 0xF
                else:
                    got = (int(ops[lane, t // 4]) >> (8 * (t % 4))) & 0xFF
            elif kind == 3:
                k = 8 * h + t
                got = (int(ops[lane, t // 4]) >> (8 * (t % 4))) & 0xFF
            else:
                k = 8 * h + t
                got = (int(ops[lane, t // 2]) >> (16 * (t % 2))) & 0xFFFF
            assert got == codes[row][k], (kind, lane, t)


def test_decoders_match_the_format_tables():
    e2 = fm.E2M1
    for c in range(16):
        assert float(mp.e2m1(c)) == float(e2.decode(np.array([c]))[0])
    e4 = fm.E4M3
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert float(mp.e4m3(c)) == float(e4.decode(np.array([c]))[0])


def test_probe_library_exports():
    if not os.path.exists(mp.LIB):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(mp.LIB)
    for sym in ("probe_mfma_rate", "probe_mfma_sum", "probe_cvt_scale"):
        assert hasattr(lib, sym)
