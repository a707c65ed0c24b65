"""Code-generation properties of the attention kernels that their speed (and,
for the wait states, their correctness) depends on, checked on the gfx950
assembly hipcc emits for them (CPU only: hipcc cross-compiles).

* Every direct-to-LDS tile copy is issued from inline asm behind `s_nop 4`:
  the compiler's hazard checks do not look inside inline asm, and a VMEM
  instruction needs 5 wait states after a VALU write of an SGPR it reads.
* No compiler-inserted `s_waitcnt vmcnt(...)` sits directly before an LDS
  transpose read (`ds_read_b64_tr_b16`): with the copies tracked by the
  compiler, it waited there for the next tile's copy in every tile.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_context_parallelism_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["attn_fwd_bf16.hip", "attn_bwd_bf16.hip"]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def _asm(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text().splitlines()


def _instructions(lines):
    """(text, inside_inline_asm) for every instruction line, comments dropped."""
    inside = False
    out = []
    for ln in lines:
        t = ln.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
            continue
        if t.startswith(";;#ASMEND"):
            inside = False
            continue
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        out.append((t.split(";")[0].strip(), inside))
    return out


@pytest.mark.parametrize("src", SOURCES)
def test_lds_copies_are_asm_with_wait_states(src, tmp_path):
    ins = _instructions(_asm(src, tmp_path))
    loads = [i for i, (t, _) in enumerate(ins) if re.match(r"buffer_load_dword\w*\s.*\blds\b", t)]
    assert loads, "no direct-to-LDS loads found"
    for i in loads:
        assert ins[i][1], f"LDS copy outside inline asm: {ins[i][0]}"
        assert ins[i - 1] == ("s_nop 4", True), f"LDS copy without its wait states: {ins[i - 1]} / {ins[i][0]}"


@pytest.mark.parametrize("src", SOURCES)
def test_no_copy_wait_before_transpose_reads(src, tmp_path):
    ins = _instructions(_asm(src, tmp_path))
    reads = [i for i, (t, _) in enumerate(ins) if t.startswith("ds_read_b64_tr_b16")]
    assert reads, "no LDS transpose reads found"
    for i in reads:
        prev, in_asm = ins[i - 1]
        assert not (prev.startswith("s_waitcnt") and "vmcnt" in prev and not in_asm), \
            f"compiler wait for outstanding loads before a transpose read: {prev}"
