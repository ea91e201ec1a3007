"""The grouped GEMM's tile claim and register use, checked in the gfx950
assembly the compiler writes for it.

One lane of wave 0 claims a tile with an atomic fetch-add the compiler sees
(not inline assembly), so the compiler keeps the returned value's register
reserved until the return has landed.  The stage loads, however, are inline
assembly that the compiler does not count: before the ticket is first used,
only a full wait (vmcnt(0)) proves the return has arrived.  This test
compiles the kernel source and checks, for every kernel that claims, that
the compiler put one there; and that no instance of the grouped GEMM spills.
Runs on the CPU (hipcc cross-compiles).  Without hipcc the library cannot be
built either, so a missing hipcc fails the test instead of skipping it."""
import os
import re
import shutil
import subprocess

import pytest

from token_routing_expert_amd import build as tre_build

GEMM = re.compile(r"^(_ZN3tre\S*k_grouped_gemm\S*):")
CLAIM = re.compile(r"global_atomic_add(?:_u32)? (v\d+), .* sc0")
VREF = re.compile(r"\bv(\d+)\b|v\[(\d+):(\d+)\]")


def claims_without_wait(asm: str):
    """{kernel: number of claims} and [(kernel, first use) of a ticket read
    with no vmcnt(0) between the claim and that use]"""
    lines = asm.split("\n")
    starts = [(i, m.group(1)) for i, l in enumerate(lines) if (m := GEMM.match(l))]
    counts, bad = {}, []
    for j, (a, name) in enumerate(starts):
        b = starts[j + 1][0] if j + 1 < len(starts) else len(lines)
        body = [l.split(";")[0].strip() for l in lines[a + 1:b]]
        for i, ins in enumerate(body):
            m = CLAIM.search(ins)
            if not m:
                continue
            counts[name] = counts.get(name, 0) + 1
            n = int(m.group(1)[1:])
            waited = False
            for later in body[i + 1:]:
                if later.startswith("s_waitcnt") and "vmcnt(0)" in later:
                    waited = True
                if any((r.group(1) and int(r.group(1)) == n) or
                       (r.group(2) and int(r.group(2)) <= n <= int(r.group(3))) for r in VREF.finditer(later)):
                    if not waited:
                        bad.append((name, later))
                    break
    return counts, bad


def test_checker_sees_a_missing_wait():
    asm = "\n".join([
        "_ZN3tre12_GLOBAL__N_13dma14k_grouped_gemmILi1EEEv:",
        "  global_atomic_add v8, v1, v2, s[4:5] sc0",
        "  s_waitcnt vmcnt(2)",
        "  v_readfirstlane_b32 s3, v8",
        "_ZN3tre12_GLOBAL__N_13dma14k_grouped_gemmILi2EEEv:",
        "  global_atomic_add v8, v1, v2, s[4:5] sc0",
        "  s_waitcnt vmcnt(0)",
        "  v_readfirstlane_b32 s3, v8",
    ])
    counts, bad = claims_without_wait(asm)
    assert len(counts) == 2
    assert bad == [("_ZN3tre12_GLOBAL__N_13dma14k_grouped_gemmILi1EEEv", "v_readfirstlane_b32 s3, v8")]


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    assert os.path.exists(hipcc), "hipcc not found: the checks need the kernels' gfx950 assembly"
    src = os.path.join(tre_build.CSRC, "grouped_ffn.hip")
    out = tmp_path_factory.mktemp("asm") / "grouped_ffn.s"
    r = subprocess.run([hipcc, *tre_build.FLAGS, "--cuda-device-only", "-S", src, "-o", str(out)],
                       capture_output=True, text=True, timeout=540)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


@pytest.mark.timeout(600)
def test_ticket_read_only_after_a_full_wait(gemm_asm):
    counts, bad = claims_without_wait(gemm_asm)
    assert counts, "no kernel claims tiles: the claim's instruction pattern changed"
    assert not bad, f"a ticket is read before its return is waited for: {bad[:3]}"


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
