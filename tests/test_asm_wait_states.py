"""No inline-asm instruction of the library sits too close to an instruction
that depends on it, or that it depends on, in the compiled gfx950 code (see
asm_wait_states.py).  CPU only: every HIP source is compiled to assembly
with the library's flags."""
import concurrent.futures as cf
import glob
import importlib.util
import os
import subprocess
import tempfile

import pytest

from asm_wait_states import violations

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BAD = """
\tv_pk_mul_f16 v10, v1, v2
\ts_nop 0
\tv_mfma_f32_16x16x32_f16 v[20:23], v[10:13], v[14:17], v[20:23]
\tv_exp_f32_e32 v30, v31
\tv_fma_mix_f32 v32, v30, v33, 0 op_sel_hi:[1,0,0]
"""


def test_scanner_flags_planted_pairs():
    """The scanner finds an asm product read by an MFMA one wait state later
    and an asm mixed FMA reading a transcendental result at once, and
    nothing when the same instructions come from the compiler."""
    asm = BAD.replace("\tv_pk_mul_f16", ";;#ASMSTART\n\tv_pk_mul_f16").replace(
        "\ts_nop 0", ";;#ASMEND\n\ts_nop 0").replace(
        "\tv_fma_mix_f32", ";;#ASMSTART\n\tv_fma_mix_f32") + ";;#ASMEND\n"
    kinds = sorted(v[0] for v in violations(asm))
    assert kinds == ["asm VALU -> MFMA", "transcendental -> asm VALU"], kinds
    assert violations(BAD) == []


def test_library_has_no_inline_asm_hazards():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not installed")
    spec = importlib.util.spec_from_file_location(
        "_dqattn_build", os.path.join(ROOT, "dequant_decode_attention_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    srcs = sorted(glob.glob(os.path.join(build.CSRC, "*.hip")))
    with tempfile.TemporaryDirectory() as tmp:
        def asm(src):
            out = os.path.join(tmp, os.path.basename(src) + ".s")
            r = subprocess.run([hipcc] + build.DEVICE_FLAGS + ["--cuda-device-only", "-S", src, "-o", out],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            return src, open(out).read()
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            texts = list(ex.map(asm, srcs))
    bad = [(os.path.basename(src), v) for src, text in texts for v in violations(text)]
    assert not bad, "\n".join(f"{f}: {v[0]} at line {v[1]}: {v[2]} <- {v[3]} ({v[4]} wait states)"
                               for f, v in bad[:20])
