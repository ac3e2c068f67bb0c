"""Source rules for the hand-written gfx950 code (CPU only).

The compiler applies no hazard rules to the operands of inline assembly.  A
vector-memory instruction that reads an SGPR written by a VALU instruction
(the v_readfirstlane that makes descriptors and offsets scalar) needs 5 wait
states, and one that reads m0 after s_mov needs 1.  Without them the load can
use a stale descriptor: wrong data, or a lost range check and a memory fault.
So every inline-assembly memory instruction lives in the one helper that
carries those wait states (lds_dma16 in lds_dma.h), and these tests fail if an
`asm` statement anywhere else names a memory instruction.  They also keep
scalar-cache writes (scalar stores and atomics, cache write-back) out of the
sources altogether, and packed-fp32 instructions out of hand-written code.
"""
from __future__ import annotations

import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "transformer_block_amd", "csrc")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")))

# instructions that go through the vector memory pipeline (and read SGPR
# operands: descriptors, soffset) or through the scalar data cache
VMEM = re.compile(r"\b(buffer_|global_|flat_|scratch_|tbuffer_)\w*")
SCALAR_WRITE = re.compile(r"\bs_(store|buffer_store|atomic|buffer_atomic|dcache_wb|dcache_discard"
                          r"|scratch_store)\w*")
PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def strip_comments(src: str) -> str:
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    return re.sub(r"//[^\n]*", " ", src)


def asm_statements(src: str):
    """(line, text) of every asm statement: from the `asm`/`__asm__` keyword to
    its closing parenthesis."""
    out = []
    for m in re.finditer(r"\b(asm|__asm__|__asm)\b\s*(volatile|__volatile__)?\s*\(", src):
        depth, i = 1, m.end()
        while i < len(src) and depth:
            depth += {"(": 1, ")": -1}.get(src[i], 0)
            i += 1
        out.append((src.count("\n", 0, m.start()) + 1, src[m.start():i]))
    return out


def test_sources_found():
    assert "lds_dma.h" in SOURCES and "gemm.hip" in SOURCES


@pytest.mark.parametrize("name", SOURCES)
def test_memory_asm_only_in_the_dma_helper(name):
    src = strip_comments(open(os.path.join(CSRC, name)).read())
    for line, stmt in asm_statements(src):
        if VMEM.search(stmt) is None:
            continue
        assert name == "lds_dma.h", (
            f"{name}:{line}: inline-assembly memory instruction outside lds_dma16: {stmt[:120]}")


def test_dma_helper_carries_its_wait_states():
    src = strip_comments(open(os.path.join(CSRC, "lds_dma.h")).read())
    mem = [(line, s) for line, s in asm_statements(src) if VMEM.search(s)]
    assert len(mem) == 1, "lds_dma.h should hold exactly one inline-assembly load"
    stmt = mem[0][1]
    # m0 written, then 5 wait states (s_mov + s_nop 3), then the load
    order = [m.group(0) for m in re.finditer(r"s_mov_b32 m0|s_nop \d+|buffer_load\w*", stmt)]
    assert order[:3] == ["s_mov_b32 m0", "s_nop 3", "buffer_load_dwordx4"], order
    # the scalar operands are made uniform inside the helper, right before it
    body = src[src.index("void lds_dma16"):]
    body = body[:body.index("\n}\n")]
    assert body.count("__builtin_amdgcn_readfirstlane") >= 3


@pytest.mark.parametrize("name", SOURCES)
def test_no_scalar_cache_writes(name):
    src = strip_comments(open(os.path.join(CSRC, name)).read())
    for line, stmt in asm_statements(src):
        assert SCALAR_WRITE.search(stmt) is None, f"{name}:{line}: scalar-cache write in asm"
    assert "__builtin_amdgcn_s_dcache_wb" not in src


@pytest.mark.parametrize("name", SOURCES)
def test_no_hand_written_packed_fp32(name):
    src = strip_comments(open(os.path.join(CSRC, name)).read())
    for line, stmt in asm_statements(src):
        assert PACKED_F32.search(stmt) is None, f"{name}:{line}: packed fp32 in asm"


def test_planted_violation_is_caught():
    """The scanner itself: a load written in asm outside the helper is found."""
    bad = 'void f() { asm volatile("buffer_load_dword %0, %1, %2, 0 offen" : : "v"(a), "s"(d)); }'
    stmts = asm_statements(strip_comments(bad))
    assert len(stmts) == 1 and VMEM.search(stmts[0][1])
    ok = 'void f() { asm volatile("; masked key tile"); }'
    assert all(VMEM.search(s) is None for _, s in asm_statements(ok))
