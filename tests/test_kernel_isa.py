"""Checks on the gfx950 assembly of the HIP kernels (CPU only: hipcc
cross-compiles).  Every kernel must run from registers and LDS alone (no
scratch: no private segment, no vector-register spills; scalar registers
may only be parked in vector-register lanes, which the zero private
segment guarantees), and the deleted-decode floor
kernel of each decode matvec instance must issue exactly as many wide code
loads as the decode kernel itself, so the floor measures the same stream."""
import os
import re
import shutil
import subprocess

import pytest

import dequant_iqk_moe_amd.build as B

HIPCC = next((c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")) if c and os.path.exists(c)),
             None)
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def _device_asm(src: str, tmp_path) -> str:
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, *B.COMMON, *B.PER_FILE[src], *B.DEVICE, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _kernels(asm: str):
    """{kernel symbol: (body text, metadata dict)}"""
    lines = asm.splitlines()
    bodies = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S+):", l)
        if m and "kernel" in m.group(1):
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            bodies[m.group(1)] = "\n".join(lines[i:end])
    meta = {}
    for block in re.split(r"\n\s+- \.", asm.split("amdhsa.kernels:")[1]):
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        fields = dict(re.findall(r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count):\s+(\d+)", block))
        meta[name.group(1)] = {k: int(v) for k, v in fields.items()}
    return bodies, meta


@pytest.mark.parametrize("src", ["iqk_gemv.hip", "iqk_dequant.hip", "iqk_prefill.hip", "iqk_fused.hip", "iqk_glue.hip"])
def test_no_scratch(src, tmp_path):
    bodies, meta = _kernels(_device_asm(src, tmp_path))
    assert meta, "no kernels found"
    for name, m in meta.items():
        assert m.get("private_segment_fixed_size", 0) == 0, name
        assert m.get("vgpr_spill_count", 0) == 0, name


def test_floor_matvec_issues_the_same_code_loads(tmp_path):
    bodies, _ = _kernels(_device_asm("iqk_gemv.hip", tmp_path))
    pat = re.compile(r"gemv_kernelILi(\d)ELi(\d+)ELi(\d)ELb([01])ELi0E")
    counts = {}
    for name, body in bodies.items():
        m = pat.search(name)
        if m:
            fmt, n, xdt, floor = m.groups()
            wide = "buffer_load_dwordx2" if fmt == "3" else "buffer_load_dwordx4"
            counts[(fmt, n, xdt, floor)] = len(re.findall(wide + r"\b", body))
    pairs = [(k, k[:3] + ("1",)) for k in counts if k[3] == "0"]
    assert len(pairs) == 18
    for plain, floor in pairs:
        assert counts[plain] > 0 and counts[plain] == counts[floor], (plain, counts[plain], counts[floor])
