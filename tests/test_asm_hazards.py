"""The gfx950 device code, compiled to assembly on the CPU, checked for a
store-data hazard: a VMEM store of more than 8 bytes whose data registers
the very next VALU instruction overwrites.  This compiler does not separate
the two, and on the MI355X such a store wrote corrupted data (the split-KV
partials, before they were stored 8 bytes at a time)."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_15_amd", "csrc")

WIDE_STORE = re.compile(r"^(buffer|global|flat)_store_dwordx[34]\b")


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def _device_units():
    """The library's device compile units: (name, source, extra flags)."""
    import exact_tiled_attention_15_amd.build as b

    return [u for u in b.UNITS if u[1].endswith(".hip")]


def _asm(unit, out):
    import exact_tiled_attention_15_amd.build as b

    _, src, extra = unit
    cmd = [_hipcc(), "-O3", "-std=c++17", f"--offload-arch={b.ARCH}", "--cuda-device-only",
           "-S", *b.DEVICE_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def _regs(text):
    """(register file, first, last) of each v/a register operand in `text`."""
    out = []
    for m in REG.finditer(text):
        if m.group(1):
            out.append((m.group(1), int(m.group(2)), int(m.group(3))))
        else:
            out.append((m.group(4), int(m.group(5)), int(m.group(5))))
    return out


def _data_regs(line):
    """Register range of a wide store's data operand (VGPRs or AGPRs)."""
    ops = _regs(line.split(None, 1)[1])
    return ops[0] if line.startswith("buffer") else ops[1]


def hazards(asm_text):
    lines = [l.strip() for l in asm_text.split("\n")]
    found = []
    for i, s in enumerate(lines):
        if not WIDE_STORE.match(s):
            continue
        f, lo, hi = _data_regs(s)
        for n in lines[i + 1:i + 4]:
            if not n or n.startswith(";"):
                continue
            if n.startswith("v_"):  # a vector instruction: its first operand is the destination
                dst = _regs(n.split(None, 1)[1].split(",", 1)[0]) if " " in n else []
                if dst and dst[0][0] == f and dst[0][1] <= hi and lo <= dst[0][2]:
                    found.append((s, n))
            break
    return found


def test_scanner_catches_the_pattern():
    bad = "\tbuffer_store_dwordx4 v[2:5], v20, s[0:3], s4 offen\n\tv_mul_f32_e32 v2, v19, v6\n"
    ok = "\tbuffer_store_dwordx4 v[2:5], v20, s[0:3], s4 offen\n\ts_nop 0\n\tv_mul_f32_e32 v2, v19, v6\n"
    ok2 = "\tbuffer_store_dwordx2 v[2:3], v20, s[0:3], s4 offen\n\tv_mul_f32_e32 v2, v19, v6\n"
    g = "\tglobal_store_dwordx4 v[8:9], v[2:5], off\n\tv_add_f32_e32 v3, v1, v1\n"
    ga = "\tglobal_store_dwordx4 v[0:1], a[8:11], off offset:64\n\tv_accvgpr_write_b32 a9, v4\n"
    ga_ok = "\tglobal_store_dwordx4 v[0:1], a[8:11], off offset:64\n\tv_add_f32_e32 v9, v1, v1\n"
    wide = "\tbuffer_store_dwordx4 v[2:5], v20, s[0:3], s4 offen\n\tv_mov_b64_e32 v[4:5], v[8:9]\n"
    assert len(hazards(bad)) == 1 and not hazards(ok) and not hazards(ok2) and len(hazards(g)) == 1
    assert len(hazards(ga)) == 1 and not hazards(ga_ok) and len(hazards(wide)) == 1


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_device_code_has_no_wide_store_data_hazard():
    units = _device_units()
    assert len(units) >= 4
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(len(units)) as ex:
            texts = list(ex.map(lambda u: _asm(u, os.path.join(d, u[0] + ".s")), units))
    for (name, _, _), text in zip(units, texts):
        assert "v_mfma" in text, f"{name}: no device code?"
        h = hazards(text)
        assert not h, f"{name}: {len(h)} wide stores with their data overwritten next: {h[:3]}"
