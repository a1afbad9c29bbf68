"""CPU tier: the streaming kernel's activation-tile waits count the loads issued after each tile
(an in-order counter), which is exact only if every prologue tile load is issued ahead of every
weight load.  The source pins that order with scheduling barriers; this test compiles two of
the six parts of the streaming kernel to gfx950 assembly and checks, in every instance that
loads activation tiles straight into LDS, that no weight load comes before the last prologue
tile load."""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from w4_groupwise_gemm_amd import build as B

PARTS = [(4, 2), (5, 1)]  # (code width, epilogue): the parts with the most ring instances


def _asm(part, tmp):
    bits, epi = part
    out = os.path.join(tmp, f"stream_{bits}_{epi}.s")
    cmd = [B.HIPCC] + B.COMMON + B.DEVICE_FLAGS + [f"-DW4_STREAM_BITS={bits}", f"-DW4_STREAM_EPI={epi}",
                                                   "--cuda-device-only", "-S", os.path.join(B.CSRC, "stream.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which(B.HIPCC) is None, reason="hipcc not available")
def test_tile_loads_precede_weight_loads():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(len(PARTS)) as ex:
            files = list(ex.map(lambda p: _asm(p, tmp), PARTS))
        checked = 0
        for f in files:
            s = open(f).read()
            for m in re.finditer(r"^(_ZN2w412_GLOBAL__N_113stream_kernel\S+):", s, re.M):
                end = s.index("s_endpgm", m.end())
                body = [line.strip() for line in s[m.end():end].splitlines()]
                lds_loads = [k for k, line in enumerate(body) if line.startswith("buffer_load") and line.endswith(" lds")]
                first_read = next((k for k, line in enumerate(body) if line.startswith("ds_read")), len(body))
                prologue = [k for k in lds_loads if k < first_read]
                if not prologue:
                    continue
                checked += 1
                early = [k for k, line in enumerate(body[:max(prologue)]) if line.startswith("global_load")]
                assert not early, f"{m.group(1)}: {len(early)} weight load(s) issued before a tile load"
        assert checked >= 60, checked
