"""Checks on the gfx950 assembly of the library's kernels, compiled here on the
CPU (hipcc cross-compiles; no GPU is needed).

* The attention kernel's global -> LDS copies (16 or 4 bytes per lane) are
  written as inline asm that sets M0 (the LDS destination) right before each
  buffer load.  M0 is a
  reserved register: the compiler does not save it around inline asm, so the
  asm is only safe while nothing else in the kernel keeps a value in M0.
  Every M0 reference must therefore be one of the asm's own pairs.
* Packed fp32 VALU instructions are disabled for all device code (the build
  passes -packed-fp32-ops); none may appear.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vision_encoder_varlen_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def _assemble(src, out_dir):
    from vision_encoder_varlen_amd import build
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [HIPCC, *[f for f in build.COMMON_FLAGS if f not in ("-fPIC", "-Wall")],
           "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("isa"))
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        outs = list(ex.map(lambda s: _assemble(s, d), srcs))
    return {os.path.basename(s): open(o).read().splitlines() for s, o in zip(srcs, outs)}


def _code(lines):
    return [l.split(";")[0].strip() for l in lines if l.strip() and not l.strip().startswith(";")]


ATTN_UNITS = ("attn_bf16.hip", "attn_bf16_fused.hip")


def test_m0_is_only_the_lds_copies_own(assembly):
    for unit in ATTN_UNITS:
        lines = _code(assembly[unit])
        copies = 0
        for i, l in enumerate(lines):
            if not re.search(r"\bm0\b", l):
                continue
            if l.startswith("s_mov_b32 m0,"):
                assert re.match(r"buffer_load_dword(x4)? ", lines[i + 1]) and \
                    lines[i + 1].endswith(" lds"), \
                    f"{unit}: M0 set without the LDS copy after it: {l!r} then {lines[i + 1]!r}"
                copies += 1
            else:
                pytest.fail(f"{unit}: M0 used outside the LDS copy asm: {l!r}")
        assert copies > 0, unit
    for name, src in assembly.items():
        if name not in ATTN_UNITS:
            assert not any(re.search(r"\bm0\b", l) for l in _code(src)), name


def test_no_packed_fp32_instructions(assembly):
    for name, src in assembly.items():
        bad = [l for l in _code(src) if re.match(r"v_pk_(fma|mul|add)_f32\b", l)]
        assert not bad, f"{name}: {bad[:3]}"
