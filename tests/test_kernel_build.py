"""Properties of the compiled gfx950 tile kernels that no GPU run shows directly (no GPU
needed: hipcc cross-compiles the device code to assembly here).

* M0: the global -> LDS copy helpers write M0 in inline asm and declare it clobbered,
  which the compiler does not honour by saving and restoring it.  The copies are only
  correct while the compiler keeps nothing of its own in M0 in these kernels, so the
  assembly must hold no M0 access outside those asm blocks.
* Registers: the kernels of the default plans (the fused block, GEMM alone, the partials
  mode and both producer tiles on 256 x 128 / 256 x 256) and the split schedule's
  128 x 128 tail tile must run without scratch, and the 8-wave ones within 256 registers,
  so that two waves fit on each SIMD.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "chunked_matmul_reduce_amd", "csrc", "tile_kernel.hip")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc is not installed")
    out = str(tmp_path_factory.mktemp("asm") / "tile_kernel.s")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-Xclang",
           "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", "-o", out, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


def _kernels(text):
    """name -> (agpr, vgpr incl. agpr, spilled vgprs, scratch bytes) from the metadata."""
    meta = text[text.index("amdhsa.kernels:"):]
    res = {}
    for blk in meta.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        res[name] = (int(blk.split("\n")[0]),
                     int(re.search(r"\.vgpr_count:\s+(\d+)", blk).group(1)),
                     int(re.search(r"\.vgpr_spill_count:\s+(\d+)", blk).group(1)),
                     int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", blk).group(1)))
    return res


def test_m0_only_inside_the_copy_asm(asm):
    outside, inside = [], 0
    in_asm = False
    for ln in asm.split("\n"):
        s = ln.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if s.startswith(";") or s.startswith("."):
            continue
        if re.search(r"\bm0\b", s):
            if in_asm:
                inside += 1
            else:
                outside.append(s)
    assert inside > 0, "the copy helpers' M0 writes were not found"
    assert outside == [], outside[:10]


# (mode, K step, W transposed, tile) of the kernels the default plans and the measurement
# legs launch, and whether they run 8 waves per workgroup
DEFAULT_KERNELS = [(0, 64, False, 0, True), (0, 64, True, 0, True), (1, 64, False, 0, True),
                   (1, 64, True, 0, True), (3, 64, False, 0, True), (4, 32, False, 0, True),
                   (2, 64, False, 0, False), (0, 32, False, 0, False), (0, 32, False, 1, False),
                   (0, 64, False, 2, True), (0, 32, False, 2, False)]


@pytest.mark.parametrize("mode,bk,wt,tile,eight", DEFAULT_KERNELS)
def test_default_kernels_fit_their_registers(asm, mode, bk, wt, tile, eight):
    ks = _kernels(asm)
    name = f"_ZN4mmar11tile_kernelILi{mode}ELi{bk}ELb{int(wt)}ELi{tile}EEEvNS_8TileArgsE"
    assert name in ks, sorted(ks)
    agpr, vgpr, spill, scratch = ks[name]
    if (mode, tile) == (0, 1):
        # the 256 x 192 fused tile: 512 registers of a lone wave, a few spills outside the
        # K loop (a tuner candidate, never the default)
        assert vgpr <= 512 and scratch <= 64, ks[name]
        return
    assert spill == 0 and scratch == 0, ks[name]
    if eight:
        assert vgpr <= 256, ks[name]
