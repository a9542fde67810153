"""The library's gfx950 machine code (built here from its sources and
disassembled on the CPU): no packed fp32 arithmetic anywhere, and no fp32 multiply-add in the
numeric chains.

Every elementwise stage is one rounded fp32 operation per eager op, so a
contracted multiply-add would change results; the only fp32 multiply-adds
the compiler may emit are those of its 64-bit integer division expansion,
which multiply by the constants 2^32 / -2^32 (0x4f800000 / 0xcf800000)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "dit_adaln_row_amd", "libditnorm.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
DIV_CONSTANTS = ("0x4f800000", "0xcf800000")


def _disassembly(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("the HIP library is not built")
    tools = [shutil.which("objcopy"), os.path.join(LLVM, "clang-offload-bundler"),
             os.path.join(LLVM, "llvm-objdump")]
    if not all(t and os.path.exists(t) for t in tools):
        pytest.skip("binutils / ROCm llvm tools not available")
    fat = tmp_path / "fat.bin"
    subprocess.check_call([tools[0], "--dump-section", f".hip_fatbin={fat}", LIB, str(tmp_path / "x.so")])
    data = fat.read_bytes()
    offs = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert offs, "no offload bundle in the library"
    text = []
    for i, o in enumerate(offs):
        chunk = tmp_path / f"b{i}.bin"
        chunk.write_bytes(data[o:offs[i + 1] if i + 1 < len(offs) else len(data)])
        code = tmp_path / f"c{i}.o"
        r = subprocess.run([tools[1], "--unbundle", "--type=o",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={chunk}",
                            f"--output={code}"], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        text.append(subprocess.check_output([tools[2], "-d", "--mcpu=gfx950", str(code)], text=True))
    return "\n".join(text)


def test_no_packed_fp32_and_no_contracted_fp32_fma(tmp_path):
    asm = _disassembly(tmp_path)
    lines = [l for l in asm.splitlines() if re.match(r"\s+v_", l)]
    assert len(lines) > 10000, "unexpectedly little device code"
    assert any("v_cvt_pk_bf16_f32" in l for l in lines), "expected bf16 rounding instructions"
    packed = [l.strip() for l in lines if re.match(r"\s+v_pk_(fma|mul|add)_f32", l)]
    assert not packed, f"packed fp32 arithmetic in the library: {packed[:3]}"
    fma = [l.strip() for l in lines
           if re.match(r"\s+v_(fma|fmac|fmamk|fmaak|mac|mad)_f32", l)
           and not any(c in l for c in DIV_CONSTANTS)]
    assert not fma, f"fp32 multiply-add outside the integer division expansion: {fma[:3]}"
