"""Code-generation checks of the streaming kernel (CPU only: hipcc cross-compiles).

The kernel keeps RING weight stages in flight per wave; each step must wait only
for its own stage (s_waitcnt vmcnt(N) with N = loads of the later stages). If
the register allocator moves a ring slot between registers on a loop pass, the
copy waits for every load in flight (vmcnt(0)) and the stream stalls every
RING steps; results stay correct, so only the generated code shows it. This
test compiles the kernels to gfx950 assembly and checks, for every variant on
the product path, that each group of matrix-core instructions in the step loop
is preceded by a wait that leaves the later stages in flight, and that no
streaming kernel spills to scratch (the offline packer keeps a block in private
memory; it is not on the timed path).  The persistent variant with two row
tiles is left out: one of its four steps waits for two of the three later
stages (a known slow spot).  The persistent launch always forms the min term
per step, so it has no sub-block-sum variant.  The
vector-unit variants (one per row count 1..4) are checked the same way on
their groups of dot-product instructions; there the compiler issues the
refill of a stage before the stage's dot products, so the wait may count the
refill's loads as well, but it must still leave the later stages in flight.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from weight_streaming_gemm_amd import build as B

RING = 4
LOADS_PER_STAGE = 3          # two quant halves and the header, one sub-tile per wave


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "k.s"
    cmd = [B.HIPCC, "-O3", "-std=c++17", f"--offload-arch={B.ARCH}", *B.DEVICE_FLAGS, "-x", "hip", "-S",
           "--cuda-device-only", os.path.join(B.CSRC, "qgemm_kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernel_body(asm: str, rt: int, nw: int, multi: bool, msum: bool, vr: int = 0) -> str:
    name = (f"_ZN2qg13stream_kernelILi{rt}ELi1ELi{nw}ELb{int(multi)}ELb{int(msum)}ELi{vr}"
            "EEEvNS_10StreamArgsEPKNS_8GemmDescE")
    start = asm.index(name + ":")
    return asm[start:asm.index("s_endpgm", start)]


def _mfma_groups(body: str, op: str = "v_mfma"):
    """(wait before the group, group size) for each run of `op` instructions with no vmcnt wait inside."""
    groups, last_wait, n = [], None, 0
    for line in body.splitlines():
        s = line.strip()
        if s.startswith("s_waitcnt") and "vmcnt" in s:
            if n:
                groups.append((last_wait, n))
                n = 0
            last_wait = int(re.search(r"vmcnt\((\d+)\)", s).group(1))
        elif re.match(op, s):
            n += 1
    if n:
        groups.append((last_wait, n))
    return groups


# (RT, waves) of the product variants, single-GEMM and persistent, both min-term forms
VARIANTS = [(1, 8), (2, 8), (3, 8), (4, 8)]


@pytest.mark.parametrize("rt,nw", VARIANTS)
@pytest.mark.parametrize("msum", [False, True])
def test_single_gemm_step_loop_keeps_ring_in_flight(asm, rt, nw, msum):
    body = _kernel_body(asm, rt, nw, False, msum)
    per_step = 8 * rt + (2 * rt if msum else 8 * rt)  # MFMAs of one step (sums: two fp32 products)
    steps = [(w, n) for w, n in _mfma_groups(body) if n >= per_step]
    assert steps, "no step loop found"
    for w, n in steps:
        assert n == per_step, f"{n} MFMAs under one wait: steps merged behind a full drain"
        assert w == (RING - 1) * LOADS_PER_STAGE, f"step waits vmcnt({w})"


@pytest.mark.parametrize("rt,nw", [(1, 8), (3, 8), (4, 8)])
def test_persistent_step_loop_keeps_ring_in_flight(asm, rt, nw):
    body = _kernel_body(asm, rt, nw, True, False)
    per_step = 16 * rt
    steps = [(w, n) for w, n in _mfma_groups(body) if n >= per_step]
    assert steps
    for w, n in steps:
        assert n == per_step and w == (RING - 1) * LOADS_PER_STAGE, (w, n)


@pytest.mark.parametrize("rt,nw", VARIANTS)
@pytest.mark.parametrize("multi,msum", [(False, False), (False, True), (True, False)])
def test_stream_kernels_do_not_spill(asm, rt, nw, multi, msum):
    body = _kernel_body(asm, rt, nw, multi, msum)
    assert "scratch_store" not in body and "scratch_load" not in body


@pytest.mark.parametrize("vr", [1, 2, 3, 4])
def test_vector_unit_step_loop_keeps_ring_in_flight(asm, vr):
    body = _kernel_body(asm, 1, 8, False, True, vr)
    per_step = 32 * vr                                   # 8 operand pairs x 4 dot products per row
    steps = [(w, n) for w, n in _mfma_groups(body, r"v_dot2c?_f32_f16") if n >= per_step]
    assert len(steps) >= RING, steps
    for w, n in steps:
        assert n == per_step, f"{n} dot products under one wait"
        assert (RING - 1) * LOADS_PER_STAGE <= w <= RING * LOADS_PER_STAGE, f"step waits vmcnt({w})"
    assert "scratch_store" not in body and "scratch_load" not in body
