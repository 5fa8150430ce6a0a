"""Shape of the compiled main loops, read from the gfx950 assembly that hipcc
makes of the kernel source here (device code only; no GPU needed).

Two properties that no numerical test can see, and that a small change far
from the main loop can break without a word from the compiler:

* No buffer descriptor of a stage load is taken for divergent.  The compiler
  then wraps the load in a loop over the lanes (v_readfirstlane, the load,
  s_cbranch_execnz), which costs 15-25 % of the kernel's time.
* Every instance's main loop is one straight-line block holding a whole trip
  of the ring: FM * FN * (BK / 16) * STAGES MFMAs of its configuration (and
  of the owned sub-tile configuration where the instance has one).
* No instance spills vector registers to scratch memory beyond the few
  listed below (two copies of a main loop body with its 256 accumulators
  have made the compiler spill a few hundred).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "gemm_reduce_scatter_amd", "csrc", "pk_gemm_rs.hip")

CFG = re.compile(r"Cfg<(\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)>")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc is not installed")
    from gemm_reduce_scatter_amd.build import HIPCC_FLAGS
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = str(tmp_path_factory.mktemp("isa") / "pk_gemm_rs.s")
    r = subprocess.run([hipcc, *flags, "-I", os.path.join(ROOT, "include"), "--cuda-device-only",
                        "-S", SRC, "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = open(out).read()
    names = re.findall(r"^(_Z\S+):", text, re.M)
    dem = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True,
                         text=True).stdout.splitlines()
    res = {}
    meta = text[text.index("amdhsa.kernels"):]
    for mangled, name in zip(names, dem):
        if "pk_gemm_rs_fused<" not in name:
            continue
        i = text.index(mangled + ":")
        body = text[i:text.index(".Lfunc_end", i)]
        j = meta.index(".name:           " + mangled + "\n")
        entry = meta[meta.rfind("\n  - ", 0, j):meta.find("\n  - ", j)]
        spill = re.search(r"\.vgpr_spill_count:\s+(\d+)", entry)
        res[name] = (re.split(r"\n\.LBB\S+:", body), int(spill.group(1)) if spill else -1)
    assert res, "no pk_gemm_rs_fused instance in the assembly"
    return res


def _trip_mfmas(cfg):
    bm, bn, wm, wn, bk, stages, _ = (int(x) for x in cfg)
    return (bm // wm // 32) * (bn // wn // 32) * (bk // 16) * stages


def test_no_lane_loop_around_stage_loads(kernels):
    bad = []
    for name, (blocks, _) in kernels.items():
        n = sum(1 for b in blocks
                if "offen lds" in b and "v_readfirstlane" in b and "s_cbranch_execnz" in b)
        if n:
            bad.append(f"{n} lane loops in {name}")
    assert not bad, "\n".join(bad)


def test_main_loop_trip_is_one_block(kernels):
    bad = []
    for name, (blocks, _) in kernels.items():
        counts = [b.count("v_mfma") for b in blocks]
        cs, co = CFG.findall(name)[:2]
        for cfg in {cs, co}:
            want = _trip_mfmas(cfg)
            if want not in counts:
                bad.append(f"{name}: no block of {want} MFMAs for Cfg<{', '.join(cfg)}> "
                           f"(largest {max(counts)})")
    assert not bad, "\n".join(bad)


# The multi-round walk of send tiles paired with owned sub-tiles (the owned
# split when it does not fit one round) spills 7 VGPRs, its scalar spills
# having taken vector lanes: 2 scratch loads per 128-MFMA trip of one of its
# main loops, the rest outside the loops (4 before the stage loads were issued
# ahead of the accumulator zeroing, with the same 2 per trip).  Every other
# instance spills none.
SPILL_ALLOWED = {"Cfg<256, 256, 2, 2, 32, 4, 1>, pk::Cfg<64, 128, 2, 2, 64, 4, 1>, 0, 7, 0>": 7}


def test_no_vector_register_spills(kernels):
    bad = []
    for name, (_, n) in kernels.items():
        allowed = max([v for k, v in SPILL_ALLOWED.items() if k in name], default=0)
        if n < 0 or n > allowed:
            bad.append(f"{name}: {n} VGPRs spilled (allowed {allowed})")
    assert not bad, "\n".join(bad)
