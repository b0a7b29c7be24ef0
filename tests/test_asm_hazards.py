"""The attention's row loads and the long-row top-k's score pieces are written as inline
asm (global_load_lds_dwordx4), which the compiler's hazard recognizer does not see into.  The hardware needs 5 wait states
between a VALU write of an SGPR (v_readfirstlane of a row-table entry) and a vector-memory
instruction that reads it as its address, and 1 between a write of M0 and a load into LDS
that uses it.  This compiles both sources to gfx950 assembly exactly as the build does
and checks both distances before every such load (a load issued too early reads a stale
address word).  CPU only: hipcc cross-compiles."""

import os
import re
import shutil
import subprocess

import pytest

from compressed_sparse_kv_amd import build as B


def _asm(tmp_path, name):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    src = os.path.join(B.CSRC, name)
    out = tmp_path / name.replace(".hip", ".s")
    cmd = [B.HIPCC, *B.COMMON, *B.DEVICE_FLAGS, *B.PER_FILE.get(name, []), "--cuda-device-only", "-S",
           src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out.read_text()


def _wait_states_before(lines, k, writes):
    """Wait states between instruction k and the closest earlier instruction for which
    writes(instr) holds (s_nop N counts N + 1, any other instruction 1); None when none is
    found within 5, or when a label is reached first (counted as found at that point)."""
    ws = 0
    for ln in reversed(lines[:k]):
        if ln.endswith(":"):
            return ws
        if ln.startswith("s_nop"):
            ws += int(ln.split()[1]) + 1
        elif writes(ln):
            return ws
        else:
            ws += 1
        if ws >= 5:
            return None
    return ws


@pytest.mark.parametrize("name", ["attention.hip", "topk.hip"])
def test_row_loads_have_their_wait_states(tmp_path, name):
    text = _asm(tmp_path, name)
    lines = [ln.strip() for ln in text.splitlines()]
    lines = [ln for ln in lines if ln and not ln.startswith(";") and not ln.startswith(".")
             or re.match(r"^\.LBB\S+:$", ln or "")]
    n_loads = 0
    for k, ln in enumerate(lines):
        m = re.match(r"global_load_lds_dwordx4 v\d+, s\[(\d+):(\d+)\]", ln)
        if not m:
            continue
        n_loads += 1
        regs = {f"s{m.group(1)}", f"s{m.group(2)}", f"s[{m.group(1)}:{m.group(2)}]"}

        def valu_writes_addr(x):
            if not x.startswith("v_"):
                return False
            dst = x.split()[1].rstrip(",") if len(x.split()) > 1 else ""
            return dst in regs
        ws = _wait_states_before(lines, k, valu_writes_addr)
        assert ws is None or ws >= 5, f"row load {n_loads}: {ws} wait states after a VALU write of its address"
        ws_m0 = _wait_states_before(lines, k, lambda x: re.match(r"s_\w+ m0,", x) is not None)
        assert ws_m0 is None or ws_m0 >= 1, f"row load {n_loads}: M0 written right before it"
    assert n_loads > 0, f"no global_load_lds_dwordx4 found in {name}"
