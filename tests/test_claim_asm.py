"""The grouped GEMM's tile claim, checked in the gfx950 assembly the compiler
writes for it.

A claiming wave issues its atomic fetch-add in inline assembly and copies the
returned ticket into LDS, again in inline assembly, a few stages later.  In
between, the return is still in flight (nothing waits on it until the stage
waits cover it), so no other instruction may read or write the ticket's
register there.  The compiler does not know the register is busy, so this
test compiles the kernel source and checks, for every kernel that claims,
that the register's only references are the atomic and the LDS store.
Runs on the CPU (hipcc cross-compiles).  Without hipcc the library cannot be
built either, so a missing hipcc fails the test instead of skipping it: the
check must not go quiet while the kernels keep running."""
import os
import re
import shutil
import subprocess

import pytest

from token_routing_expert_amd import build as tre_build

GEMM = re.compile(r"^(_ZN3tre\S*k_grouped_gemm\S*):")
CLAIM = re.compile(r"global_atomic_add (v\d+), v\[\d+:\d+\], v\d+, off sc0")
VREF = re.compile(r"\bv(\d+)\b|v\[(\d+):(\d+)\]")


def ticket_references(asm: str):
    """{kernel: (ticket registers, [other instructions naming one of them])}"""
    lines = asm.split("\n")
    starts = [(i, m.group(1)) for i, l in enumerate(lines) if (m := GEMM.match(l))]
    out = {}
    for j, (a, name) in enumerate(starts):
        b = starts[j + 1][0] if j + 1 < len(starts) else len(lines)
        body = [l.split(";")[0].strip() for l in lines[a + 1:b]]
        regs = {int(m.group(1)[1:]) for l in body if (m := CLAIM.search(l))}
        other = []
        for n in regs:
            for ins in body:
                if not ins or ins.startswith(".") or ins.endswith(":"):
                    continue
                named = any((m.group(1) and int(m.group(1)) == n) or
                            (m.group(2) and int(m.group(2)) <= n <= int(m.group(3))) for m in VREF.finditer(ins))
                if not named or CLAIM.search(ins) or re.fullmatch(r"ds_write_b32 v\d+, v%d" % n, ins):
                    continue
                other.append(ins)
        out[name] = (regs, other)
    return out


def test_checker_sees_a_planted_reference():
    asm = "\n".join([
        "_ZN3tre12_GLOBAL__N_13dma14k_grouped_gemmILi1EEEv:",
        "  global_atomic_add v208, v[2:3], v12, off sc0",
        "  v_add_u32_e32 v1, v208, v2",
        "  ds_write_b32 v3, v208",
    ])
    regs, other = ticket_references(asm)["_ZN3tre12_GLOBAL__N_13dma14k_grouped_gemmILi1EEEv"]
    assert regs == {208} and other == ["v_add_u32_e32 v1, v208, v2"]


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    assert os.path.exists(hipcc), "hipcc not found: the claim check needs the kernels' gfx950 assembly"
    src = os.path.join(tre_build.CSRC, "grouped_ffn.hip")
    out = tmp_path_factory.mktemp("asm") / "grouped_ffn.s"
    r = subprocess.run([hipcc, *tre_build.FLAGS, "--cuda-device-only", "-S", src, "-o", str(out)],
                       capture_output=True, text=True, timeout=540)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


@pytest.mark.timeout(600)
def test_ticket_register_untouched_between_claim_and_post(gemm_asm):
    refs = ticket_references(gemm_asm)
    claiming = {k: v for k, v in refs.items() if v[0]}
    assert claiming, "no kernel claims tiles: the claim's instruction pattern changed"
    for name, (regs, other) in claiming.items():
        assert not other, f"{name}: ticket register v{sorted(regs)} also used by {other[:4]}"


@pytest.mark.timeout(600)
def test_gemm_kernels_do_not_spill(gemm_asm):
    # Spilled registers go through scratch memory: slow in the stage loop,
    # and scratch loads would join the vector-memory count that the stage
    # waits rely on.  Every instance of the grouped GEMM keeps all of its
    # state in registers.
    kernels = re.findall(r"\.amdhsa_kernel (\S*k_grouped_gemm\S*)\n(.*?)\.end_amdhsa_kernel", gemm_asm, re.S)
    assert len(kernels) >= 10
    for name, body in kernels:
        scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body).group(1))
        assert scratch == 0, f"{name} spills {scratch} bytes per lane"
