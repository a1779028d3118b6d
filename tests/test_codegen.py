"""Code generation checks of the hot kernels (CPU only: hipcc cross-compiles for gfx950).

The attention kernels wait for their asynchronous global->LDS copies with explicit
`s_waitcnt vmcnt` statements of their own: the compiler does not see those copies.  If the
compiler believes one of its own vector-memory loads is still pending when it reaches the
pipelined loop, it inserts a `vmcnt` wait there, and that wait also holds the wave until the
copies in flight for later tiles have landed: the pipeline silently serializes (a 7 % loss on
the 512-wide grouped kernel was found this way).  These tests compile the sources to assembly
and require that no MFMA block of a hot kernel carries a compiler-inserted `vmcnt` wait, except
the grouped kernel's first MFMA block (the prologue's scores of tile 0, which wait for the
queries).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_prefill_amd", "csrc")
HIPCC = os.environ.get("HIPCC") or (
    "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc"))

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def device_asm(src: str, tmp_path) -> str:
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", out, os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def mfma_blocks(asm: str, kernel_prefix: str):
    """{kernel symbol: [(block label, MFMA count, compiler vmcnt waits)]} for the kernels whose
    symbol starts with kernel_prefix; waits inside inline-asm regions are the kernel's own."""
    lines = asm.split("\n")
    res = {}
    for k, line in enumerate(lines):
        m = re.match(r"^(" + re.escape(kernel_prefix) + r"\S*):", line)
        if not m:
            continue
        blocks, cur, inasm = [], ["entry", 0, 0], False
        for line2 in lines[k + 1:]:
            if line2.startswith(".Lfunc_end"):
                break
            lab = re.match(r"^(\.LBB\S+):", line2)
            if lab:
                blocks.append(tuple(cur))
                cur = [lab.group(1), 0, 0]
                continue
            t = line2.strip()
            if t.startswith(";;#ASMSTART"):
                inasm = True
            elif t.startswith(";;#ASMEND"):
                inasm = False
            elif t.startswith("v_mfma"):
                cur[1] += 1
            elif t.startswith("s_waitcnt") and "vmcnt" in t and not inasm:
                cur[2] += 1
        blocks.append(tuple(cur))
        res[m.group(1)] = [b for b in blocks if b[1] >= 8]
    return res


def test_grouped_kernel_loop_has_no_compiler_vmcnt_waits(tmp_path):
    kernels = mfma_blocks(device_asm("grouped_attn.hip", tmp_path), "_ZN3dsa19rows128_attn_kernel")
    assert len(kernels) == 16, sorted(kernels)  # {576, 512} x {grouped, per-token} x {scaled} x {2 GiB}
    for name, blocks in kernels.items():
        assert blocks, name
        late = [b for b in blocks[1:] if b[2] > 0]
        assert not late, (name, late)


def test_pertoken_sorted_kernel_has_no_compiler_vmcnt_waits_in_mfma_blocks(tmp_path):
    # (the register-ring walk loads its rows with ordinary loads, whose waits are its design)
    kernels = mfma_blocks(device_asm("pertoken_attn.hip", tmp_path), "_ZN3dsa22pertoken_sorted_kernel")
    assert len(kernels) == 4, sorted(kernels)  # {576, 512} x {scaled}
    for name, blocks in kernels.items():
        assert blocks, name
        assert not [b for b in blocks if b[2] > 0], (name, blocks)


def test_masked_mha_kernel_has_no_compiler_vmcnt_waits_in_mfma_blocks(tmp_path):
    kernels = mfma_blocks(device_asm("masked_mha.hip", tmp_path), "_ZN3dsa17masked_mha_kernel")
    assert len(kernels) == 6, sorted(kernels)  # three geometries x {masked, dense}
    for name, blocks in kernels.items():
        assert blocks, name
        assert not [b for b in blocks if b[2] > 0], (name, blocks)
