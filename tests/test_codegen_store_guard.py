"""The built library's gfx950 code, read back with the ROCm disassembler: no
store of more than 8 bytes may be followed, within two wait states, by a
vector instruction that overwrites one of the store's data registers.

Such a store reads its data registers after it has issued.  A build whose
weight-gradient epilogue put `v_mov_b32 v2, 0` (the next tile's accumulator
reset) or an address computation right behind `buffer_store_dwordx4
v[2:5]` stored, now and then and in some lanes, those new values as the
first word of the 16 bytes (zeros, or address bits read as bf16), so a few
4 x 8 blocks of dW1/dW3 came out wrong.  The stores that the kernels issue
through builtins are followed by a fixed wait (store_data_guard); this test
keeps the pattern out of every kernel of the library as built.  No GPU is
needed: the code object is taken out of libmoe.so and disassembled."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mixture_experts_layer_layout_amd", "lib", "libmoe.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

_WIDE = re.compile(r"^(buffer|global|flat)_store_(dwordx[34]|b96|b128)\b")
_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def vregs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def store_data(op, operands):
    """Data registers of a store: the first operand of a buffer store, the
    second of a global or flat store (the first is the address)."""
    parts = [p.strip() for p in operands.split(",")]
    return vregs(parts[0] if op.startswith("buffer") else parts[1])


def violations(lines, need=2):
    """(function, store, offending instruction) for every wide store whose
    data registers a vector instruction writes within `need` wait states
    (each instruction counts one, s_nop N counts N + 1)."""
    func, ins, out = None, [], []
    for line in lines:
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            func = m.group(1)
            ins.append((func, None))
            continue
        text = line.split("//")[0].strip()
        if text and not text.endswith(":"):
            ins.append((func, text))
    for k, (f, text) in enumerate(ins):
        if text is None:
            continue
        op, _, rest = text.partition(" ")
        if not _WIDE.match(op):
            continue
        data = store_data(op, rest)
        waits = 0
        for f2, t2 in ins[k + 1:k + 1 + need]:
            if t2 is None or f2 != f:
                break
            op2, _, rest2 = t2.partition(" ")
            if op2 == "s_nop":
                waits += int(rest2.split()[0], 0) + 1
            else:
                if op2.startswith("v_") and vregs(rest2.split(",")[0]) & data:
                    out.append((f, text, t2))
                    break
                waits += 1
            if waits >= need:
                break
    return out


def test_scanner_finds_the_pattern():
    code = ["0000000000001000 <k>:",
            "\tbuffer_store_dwordx4 v[2:5], v66, s[48:51], 0 offen nt // 0",
            "\tv_mov_b32_e32 v2, 0 // 8",
            "\tbuffer_store_dwordx4 v[6:9], v66, s[48:51], 0 offen nt // 0",
            "\ts_nop 3 // 8",
            "\tv_mov_b32_e32 v6, 0 // 8",
            "\tglobal_store_dwordx4 v[10:11], v[12:15], off // 0",
            "\tv_add_u32_e32 v20, 1, v20 // 8",
            "\tv_lshl_add_u64 v[14:15], v[0:1], 0, v[2:3] // 8",
            "\tglobal_store_dwordx2 v[10:11], v[16:17], off // 0",
            "\tv_mov_b32_e32 v16, 0 // 8"]
    found = violations(code)
    assert [v[2].split()[0] for v in found] == ["v_mov_b32_e32", "v_lshl_add_u64"]


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    if not os.path.exists(LIB):
        from mixture_experts_layer_layout_amd import build
        build.build()
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump of the ROCm toolchain not found")
    work = tmp_path_factory.mktemp("codeobj")
    lib = work / "libmoe.so"
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", str(lib)], check=True, capture_output=True, cwd=work)
    objs = [p for p in os.listdir(work) if p.endswith("gfx950")]
    assert objs, "no gfx950 code object in libmoe.so"
    res = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(work / objs[0])], check=True,
                         capture_output=True, text=True)
    return res.stdout.splitlines()


def test_no_wide_store_data_overwritten_right_after_the_store(disassembly):
    assert sum(1 for l in disassembly if "buffer_store_dwordx4" in l) > 100
    found = violations(disassembly)
    assert not found, "\n".join(f"{f}: {s}  ->  {t}" for f, s, t in found[:10])
