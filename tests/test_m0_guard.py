"""The direct-to-LDS loads and the M0 register, checked on the built code.

The production kernels issue ``global_load_lds_dwordx4`` from inline
assembly that first moves the wave's LDS destination into M0 and names M0 as
clobbered.  The compiler reserves M0 for itself and says that it may not
honour that clobber, so the kernels are correct only while the generated code
uses M0 for nothing else: in every kernel that contains the inline
sequence, no other instruction may write M0, and no other instruction that
reads M0 implicitly may appear.  These tests disassemble the gfx950 code
objects of this repository's own build and check exactly that, so a
toolchain that starts using M0 in these kernels fails here, on the CPU,
instead of producing wrong LDS contents on the GPU.  (Kernels that load
through the compiler's own ``__builtin_amdgcn_global_load_lds`` leave M0 to
the compiler and are not constrained.)
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(os.path.dirname(HERE), "tiled_fp32_gemm_03_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

# Instructions that read M0 without naming it (LDS DMA, messages, relative
# register moves, GWS and append/consume, thread-id addressed LDS, interpolation).
IMPLICIT_M0 = re.compile(r"^(s_sendmsg|s_movrel|v_movrel|ds_gws|ds_append|ds_consume|s_set_gpr_idx"
                         r"|ds_read_addtid|ds_write_addtid|v_interp|s_ttracedata|buffer_load_\S+\b.*\blds\b"
                         r"|buffer_store_lds|global_load_lds)")
MOV_M0 = re.compile(r"^s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$")
FUNC = re.compile(r"^[0-9a-f]+ <(.+)>:$")
# The inline sequence's load: a 32-bit lane offset from a scalar base.  (The
# compiler's builtin issues the 64-bit-address form, ``v[a:b], off``.)
SADDR_LOAD = re.compile(r"^global_load_lds_dwordx4 v\d+, s\[\d+:\d+\]")


def instructions(asm: str):
    """(function, instruction text) pairs of an llvm-objdump listing."""
    func = None
    for line in asm.splitlines():
        m = FUNC.match(line.strip())
        if m:
            func = m.group(1)
            continue
        text = line.split("//")[0].strip()
        if func is None or not text or text.endswith(":"):
            continue
        yield func, text


def _is_triple(insts, i) -> bool:
    """insts[i] starts the inline sequence s_mov_b32 m0, sN; s_nop 0;
    global_load_lds_dwordx4 vN, s[a:b] (all in one function)."""
    if i + 2 >= len(insts):
        return False
    func = insts[i][0]
    return bool(MOV_M0.match(insts[i][1]) and insts[i + 1] == (func, "s_nop 0")
                and insts[i + 2][0] == func
                and bool(SADDR_LOAD.match(insts[i + 2][1])))


def m0_violations(asm: str) -> list[str]:
    """In every function that contains the inline direct-load sequence
    ``s_mov_b32 m0, sN; s_nop 0; global_load_lds_dwordx4``, every M0 use that
    is not part of one."""
    insts = list(instructions(asm))
    asm_funcs = {insts[i][0] for i in range(len(insts)) if _is_triple(insts, i)}
    bad = []
    for i, (func, text) in enumerate(insts):
        if func not in asm_funcs:
            continue
        mnem = text.split()[0]
        if re.search(r"\bm0\b", text):
            ok = _is_triple(insts, i)
            if not ok:
                bad.append(f"{func}: M0 written or read outside a direct load: {text}")
        elif IMPLICIT_M0.match(text):
            ok = mnem == "global_load_lds_dwordx4" and i >= 2 and _is_triple(insts, i - 2)
            if not ok:
                bad.append(f"{func}: instruction reads M0 without setting it just before: {text}")
    return bad


def disassemble(obj: str, work: str) -> str:
    name = os.path.splitext(os.path.basename(obj))[0]
    fb = os.path.join(work, name + ".fb")
    co = os.path.join(work, name + ".co")
    subprocess.run(["objcopy", f"--dump-section", f".hip_fatbin={fb}", obj], check=True,
                   capture_output=True)
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fb}",
                    f"--targets={TARGET}", f"--output={co}"], check=True, capture_output=True)
    r = subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", co], check=True,
                       capture_output=True, text=True)
    return r.stdout


def device_objects() -> list[str]:
    objs = []
    for obj in sorted(glob.glob(os.path.join(BUILD, "*.o"))):
        r = subprocess.run(["objdump", "-h", obj], capture_output=True, text=True)
        if ".hip_fatbin" in r.stdout:
            objs.append(obj)
    return objs


def _tools_present() -> bool:
    return (shutil.which("objcopy") and shutil.which("objdump")
            and os.path.exists(f"{LLVM}/clang-offload-bundler") and os.path.exists(f"{LLVM}/llvm-objdump"))


@pytest.mark.skipif(not _tools_present(), reason="binutils or the ROCm LLVM tools are missing")
def test_m0_used_only_by_direct_loads(tmp_path):
    objs = device_objects()
    if not objs:
        pytest.skip("the library's objects are not built in this tree (run the build first)")
    total_loads = 0
    bad = []
    for obj in objs:
        asm = disassemble(obj, str(tmp_path))
        insts = list(instructions(asm))
        total_loads += sum(1 for i in range(len(insts)) if _is_triple(insts, i))
        bad += [f"{os.path.basename(obj)}: {b}" for b in m0_violations(asm)]
    assert not bad, "\n".join(bad[:20])
    # The inline-sequence kernels are in the build, so the check saw them.
    assert total_loads > 100


def test_checker_catches_foreign_m0_uses():
    good = """
0000000000001000 <k>:
\ts_mov_b32 m0, s4        // 000000001000: BEFC0004
\ts_nop 0                 // 000000001004: BF800000
\tglobal_load_lds_dwordx4 v1, s[2:3]   // 000000001008: DDF48000 00020001
\ts_endpgm
"""
    assert m0_violations(good) == []
    # The compiler sets M0 for something of its own.
    assert m0_violations(good.replace("\ts_endpgm", "\ts_mov_b32 m0, -1\n\ts_endpgm"))
    # A direct load whose M0 was not set just before it (next to a whole sequence).
    two = good.replace("\ts_endpgm", "\ts_mov_b32 m0, s5\n\tv_mov_b32 v2, 0\n"
                                     "\tglobal_load_lds_dwordx4 v1, s[2:3]\n\ts_endpgm")
    assert len(m0_violations(two)) == 2
    # Another instruction that reads M0 implicitly.
    assert m0_violations(good.replace("\ts_endpgm", "\ts_sendmsg sendmsg(MSG_INTERRUPT)\n\ts_endpgm"))
    assert m0_violations(good.replace("\ts_endpgm", "\tds_append v3\n\ts_endpgm"))
    # A kernel where the compiler manages M0 for its own builtin is not constrained ...
    builtin = """
0000000000002000 <b>:
\ts_mov_b32 m0, s2
\tv_mov_b32 v5, 0
\tglobal_load_lds_dwordx4 v[6:7], off
\ts_endpgm
"""
    assert m0_violations(builtin) == []
    # ... but the same compiler use of M0 inside an inline-sequence kernel is.
    assert m0_violations(good.replace("\ts_endpgm", builtin.split("<b>:\n")[1]))
