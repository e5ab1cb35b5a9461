"""Host-side checks of the prefill kernel's generated instruction blocks.

The per-tile steps are hand-scheduled asm written by
long_context_tiled_amd/csrc/gen_prefill_steps.py. They name fixed registers
(O^T and Q^T in AGPRs, two score buffers, fragments and P^T in VGPRs), and the
kernel limits the compiler to the low VGPRs / AGPRs (COMPILER_VGPRS). These tests check that the
committed blocks are the generator's output, that the compiled kernel keeps
that contract (no compiler instruction touches a reserved register), and that
every kernel is launched with the full register file it names."""
import os
import re
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_tiled_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
sys.path.insert(0, CSRC)
from gen_prefill_steps import COMPILER_VGPRS as RESERVED_FROM  # noqa: E402


def test_steps_inc_is_generator_output():
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "steps.inc")
        subprocess.run([sys.executable, os.path.join(CSRC, "gen_prefill_steps.py"), out], check=True)
        with open(out) as f:
            fresh = f.read()
    with open(os.path.join(CSRC, "prefill_steps.inc")) as f:
        committed = f.read()
    assert fresh == committed, "prefill_steps.inc is stale: rerun gen_prefill_steps.py"


@pytest.fixture(scope="module")
def device_asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "prefill.s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
               "--cuda-device-only", "-S", os.path.join(CSRC, "prefill.hip"), "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
        with open(out) as f:
            return f.read()


def _kernels(text):
    """name -> (list of (in_asm, instruction) lines, descriptor dict)"""
    out = {}
    cur = None
    in_asm = False
    for line in text.split("\n"):
        t = line.strip()
        m = re.match(r"^(_Z\w*prefill_kernel\w*):", t)
        if m:
            cur = m.group(1)
            out[cur] = ([], {})
            continue
        if cur is None:
            continue
        if t.startswith(".Lfunc_end"):
            cur = None
            continue
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if t and not t.startswith((";", ".")):
            out[cur][0].append((in_asm, t.split(";")[0]))
    for m in re.finditer(r"\.amdhsa_kernel (\w+)(.*?)\.end_amdhsa_kernel", text, re.S):
        if m.group(1) in out:
            for k, v in re.findall(r"\.amdhsa_(\w+) (\d+)", m.group(2)):
                out[m.group(1)][1][k] = int(v)
    return out


def test_compiler_keeps_out_of_reserved_registers(device_asm):
    kernels = _kernels(device_asm)
    # d x causal x heads-per-wave x (chunk x bf16 or fp8 QK, or SAS of degree 2 or 3,
    # or 8-bit P.V with bf16 or fp8 QK, or int8 QK)
    assert len(kernels) == 108
    for name, (lines, _) in kernels.items():
        bad = []
        for in_asm, ins in lines:
            if in_asm:
                continue
            for m in re.finditer(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]", ins):
                hi = int(m.group(2) or m.group(5))
                if hi >= RESERVED_FROM:
                    bad.append(ins)
        assert not bad, f"{name}: compiler code uses reserved registers: {bad[:5]}"
        assert not any(ins.startswith("scratch_") for _, ins in lines), f"{name} spills"


def test_kernels_get_the_register_file_they_name(device_asm):
    for name, (_, desc) in _kernels(device_asm).items():
        # template arguments: d, causal, heads per wave, stages, chunk, 8-bit QK (fp8,
        # or int8 with the last), SAS, 8-bit P.V, int8 QK
        m = re.search(r"ILi(\d+)ELb[01]ELi\dELi5ELb[01]ELb([01])ELi[023]ELb[01]ELb[01]E", name)
        d, f8 = int(m.group(1)), m.group(2) == "1"
        # AGPRs: O^T (d per lane) and Q^T (d / 2 bf16, d / 4 fp8) above a[64]
        want = 256 + 64 + d + (d // 4 if f8 else d // 2)
        assert desc["accum_offset"] == 256, name
        assert desc["next_free_vgpr"] == want, name
        assert desc["private_segment_fixed_size"] == 0, name


def test_int8_scores_as_offset_floats():
    # The int8 key loops start every S^T sum from the bits of the inline
    # constant 1/(2 pi) and read the int32 result as fp32: for every score
    # the int8 codes can give (|s| <= 127 * 127 * 128 at d = 128) the bits
    # 0x3e22f983 + s are exactly the float K0 + s 2^-26, their int32 order
    # is the order of s, and (bits - K0) * 2^26 gives s back exactly.
    import numpy as np
    k0_bits = 0x3E22F983
    k0 = np.array([k0_bits], np.uint32).view(np.float32)[0]
    assert k0 == np.float32(1.0 / (2.0 * np.pi))
    smax = 127 * 127 * 128
    assert smax < 2 ** 21
    s = np.arange(-smax, smax + 1, dtype=np.int64)
    f = (k0_bits + s).astype(np.uint32).view(np.float32)
    assert np.array_equal(f.astype(np.float64), np.float64(k0) + s * 2.0 ** -26)
    assert np.all(np.diff((k0_bits + s).astype(np.int32)) > 0)
    back = (f - k0) * np.float32(2.0 ** 26)          # fp32 operations, as the loop does
    assert np.array_equal(back.astype(np.int64), s)


def test_int8_loops_start_from_the_offset_and_convert_nothing():
    with open(os.path.join(CSRC, "prefill_steps.inc")) as f:
        text = f.read()
    for ns in ("d128i8", "d64i8"):
        body = text[text.index(f"namespace {ns} {{"):text.index(f"}}  // namespace {ns}")]
        mfma = re.findall(r"v_mfma_i32_32x32x32_i8 (v\[\d+:\d+\]), \S+, \S+, (\S+?)\\n", body)
        assert mfma, ns
        starts = [c for d, c in mfma if c != d]
        assert starts and set(starts) == {"0.15915494"}, (ns, set(starts))
        assert "v_cvt_f32_i32" not in body, ns
