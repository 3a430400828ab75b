"""Wait-state hazards in the library's gfx950 device code, checked on the
assembly the compiler emits for it (no GPU needed).

Every kernel source is compiled with the library's own flags to device
assembly; the bounds come from the compiler's treatment of the probe kernels
in tests/isa/probe.hip; every producer/consumer pair of the kinds in
tests/isa_hazards.py must be at least that far apart.  The sources are also
checked for what the assembly check relies on: no inline assembly names a
matrix (XDL) instruction, and every inline LDS-DMA load begins with the
s_nop that covers the reads the compiler cannot see.  Planted mistakes in
assembly text show that each rule fires."""
import concurrent.futures as cf
import glob
import os
import re
import subprocess

import pytest

from tests import isa_hazards as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "non_prefix_kv_amd", "csrc")
PROBE = os.path.join(ROOT, "tests", "isa", "probe.hip")
HIPCC = "/opt/rocm/bin/hipcc"


def _flags():
    from non_prefix_kv_amd import build
    return [f for f in build.FLAGS if f != "-fPIC"]


def _asm(src, out_dir, flags):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return open(out).read()


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not present")
    d = str(tmp_path_factory.mktemp("isa"))
    flags = _flags()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(min(8, len(srcs) + 1)) as ex:
        probe = ex.submit(_asm, PROBE, d, ["--offload-arch=gfx950", "-O3"])
        outs = {os.path.basename(s): ex.submit(_asm, s, d, flags) for s in srcs}
        return probe.result(), {k: f.result() for k, f in outs.items()}


@pytest.fixture(scope="module")
def bounds(compiled):
    return H.calibrate(compiled[0])


def test_probe_bounds(bounds):
    """The compiler placed wait states for every probed pattern, and the
    accumulate form is the cheapest way to reuse a result."""
    for op in ("v_mfma_f32_16x16x32_bf16", "v_mfma_f32_32x32x16_bf16", "v_mfma_f32_16x16x4_f32"):
        assert bounds["raw"].get(op, 0) > 0, op
        assert bounds["srcc"][op] < bounds["raw"][op], op
    # the larger tile keeps its result longer in flight
    assert bounds["raw"]["v_mfma_f32_32x32x16_bf16"] > bounds["raw"]["v_mfma_f32_16x16x32_bf16"]
    for k in ("valu_xdl", "m0_dma", "valu_sgpr_vmem"):
        assert bounds[k] is not None and bounds[k] > 0, k


def test_library_device_code_has_no_wait_state_hazard(compiled, bounds):
    total_xdl, bad = 0, {}
    for name, asm in compiled[1].items():
        res, n = H.check_asm(asm, bounds)
        total_xdl += n
        for k, v in res.items():
            if v:
                bad[f"{name}:{k}"] = v[:5]
    assert total_xdl > 1000                   # the GEMMs and attention were seen
    assert not bad, "\n".join(f"{k}\n  " + "\n  ".join(v) for k, v in bad.items())


def _asm_statements(src):
    return re.findall(r"\basm\s+(?:volatile\s*)?\(\s*((?:\"(?:[^\"\\]|\\.)*\"\s*)+)", src)


def test_inline_assembly_rules_in_sources():
    n_dma = 0
    for path in glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")):
        src = re.sub(r"//[^\n]*", "", open(path).read())
        for text in _asm_statements(src):
            body = "".join(re.findall(r"\"((?:[^\"\\]|\\.)*)\"", text))
            assert "mfma" not in body, f"{path}: XDL op inside inline assembly"
            if "buffer_load" in body and " lds" in body:
                n_dma += 1
                assert body.startswith("s_nop "), f"{path}: LDS-DMA load without leading s_nop"
    assert n_dma == 3


PLANTED = [
    # XDL result read by a VALU instruction too early, then far enough
    ("v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]\n"
     "v_add_f32_e32 v30, v0, v1\n", 1),
    ("v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]\n"
     "s_nop 15\nv_add_f32_e32 v30, v0, v1\n", 0),
    # XDL result as the A operand of the next XDL op; accumulation is free
    ("v_mfma_f32_16x16x32_bf16 a[0:3], v[16:19], v[20:23], a[0:3]\n"
     "v_mfma_f32_16x16x32_bf16 a[4:7], a[0:3], v[20:23], a[4:7]\n", 1),
    ("v_mfma_f32_16x16x32_bf16 a[0:3], v[16:19], v[20:23], a[0:3]\n"
     "v_mfma_f32_16x16x32_bf16 a[0:3], v[24:27], v[20:23], a[0:3]\n", 0),
    # AGPR result copied out too early
    ("v_mfma_f32_16x16x32_bf16 a[0:3], v[16:19], v[20:23], a[0:3]\n"
     "s_nop 3\nv_accvgpr_read_b32 v5, a2\n", 1),
    # VALU write of an operand right before the XDL op
    ("v_mov_b32_e32 v17, 0\n"
     "v_mfma_f32_16x16x32_bf16 a[0:3], v[16:19], v[20:23], a[0:3]\n", 1),
    # M0 set right before a DMA load; one instruction in between is enough
    ("s_mov_b32 m0, s7\nbuffer_load_dwordx4 v2, s[0:3], s5 offen lds\n", 1),
    ("s_mov_b32 m0, s7\ns_nop 0\nbuffer_load_dwordx4 v2, s[0:3], s5 offen lds\n", 0),
    # descriptor word from v_readfirstlane, then the load
    ("v_readfirstlane_b32 s2, v7\ns_nop 1\nbuffer_load_dwordx4 v2, s[0:3], s5 offen lds\n", 1),
    ("v_readfirstlane_b32 s2, v7\ns_nop 4\nbuffer_load_dwordx4 v2, s[0:3], s5 offen lds\n", 0),
    # hazard across a loop back-edge: the loop's last XDL op, its first read
    ("s_mov_b32 s9, 0\n.LBB9_1:\nv_add_f32_e32 v30, v0, v1\ns_add_i32 s9, s9, 1\n"
     "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]\n"
     "s_cmp_lt_i32 s9, 4\ns_cbranch_scc1 .LBB9_1\ns_endpgm\n", 1),
]


@pytest.mark.parametrize("body,n_bad", PLANTED)
def test_checker_fires_on_planted_mistakes(bounds, body, n_bad):
    asm = "probe_fn:\n" + "".join("\t" + l + "\n" if not l.endswith(":") else l + "\n"
                                  for l in body.splitlines()) + ".Lfunc_end0:\n"
    res, _ = H.check_asm(asm, bounds)
    assert len(res["probe_fn"]) == n_bad, res["probe_fn"]


def test_checker_sees_the_dma_nops(compiled, bounds):
    """Taking the s_nop out of the GEMM's LDS-DMA loads makes the check
    fail: the wait states it relies on come from those statements."""
    asm = compiled[1]["gemm.hip"]
    stripped = re.sub(r"\n\ts_nop 0\n(\tbuffer_load_dwordx4 [^\n]* lds)", r"\n\1", asm)
    assert stripped != asm
    res, _ = H.check_asm(stripped, bounds, name_filter="gemm_mid_kernel")
    assert sum(len(v) for v in res.values()) > 0
