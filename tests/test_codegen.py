"""Code-generation checks of the streaming and pass kernels (CPU only: hipcc
cross-compiles).

Both kernels keep RING weight stages in flight per wave; each step must wait
only for its own stage (s_waitcnt vmcnt(N) with N = loads of the later stages).
If the register allocator moves a ring slot between registers on a loop pass,
the copy waits for every load in flight (vmcnt(0)) and the stream stalls every
RING steps; results stay correct, so only the generated code shows it. These
tests compile the kernels to gfx950 assembly and check, for every variant on
the product path, that each group of matrix-core instructions in the step loop
is preceded by a wait that leaves the later stages in flight, and that no
streaming or pass kernel spills to scratch (the offline packer keeps a block in
private memory; it is not on the timed path).  The vector-unit variants (one
per row count 1..4) are checked the same way on their groups of dot-product
instructions; there the compiler issues the refill of a stage before the
stage's dot products, so the wait may count the refill's loads as well, but it
must still leave the later stages in flight.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from weight_streaming_gemm_amd import build as B

RING = 4
LOADS_PER_STAGE = 3          # two quant halves and the header, one sub-tile per wave


def _compile(tmp_path_factory, src: str) -> str:
    out = tmp_path_factory.mktemp("asm") / "k.s"
    cmd = [B.HIPCC, "-O3", "-std=c++17", f"--offload-arch={B.ARCH}", *B.DEVICE_FLAGS, "-x", "hip", "-S",
           "--cuda-device-only", os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return _compile(tmp_path_factory, "qgemm_kernels.hip")


@pytest.fixture(scope="module")
def pass_asm(tmp_path_factory):
    return _compile(tmp_path_factory, "pass.hip")


def _body(asm: str, name: str) -> str:
    start = asm.index(name + ":")
    return asm[start:asm.index("s_endpgm", start)]


def _kernel_body(asm: str, rt: int, nw: int, msum: bool, vr: int = 0) -> str:
    return _body(asm, f"_ZN2qg13stream_kernelILi{rt}ELi1ELi{nw}ELb{int(msum)}ELi{vr}EEEvNS_10StreamArgsE")


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


# (RT, waves) of the product variants, both min-term forms
VARIANTS = [(1, 8), (2, 8), (3, 8), (4, 8)]


@pytest.mark.parametrize("rt,nw", VARIANTS)
@pytest.mark.parametrize("msum", [False, True])
def test_single_gemm_step_loop_keeps_ring_in_flight(asm, rt, nw, msum):
    body = _kernel_body(asm, rt, nw, msum)
    per_step = 8 * rt + (rt if msum else 8 * rt)  # MFMAs of one step (sums: one fp16 product of their two parts)
    steps = [(w, n) for w, n in _mfma_groups(body) if n >= per_step]
    assert steps, "no step loop found"
    for w, n in steps:
        assert n == per_step, f"{n} MFMAs under one wait: steps merged behind a full drain"
        assert w == (RING - 1) * LOADS_PER_STAGE, f"step waits vmcnt({w})"


def _pass_ring(rt: int) -> int:
    """Ring depth of the pass kernel at rt row tiles (qgemm_internal.h: PASS_RING up to
    some row tiles, a shallower ring beyond, where the registers run short)."""
    text = open(os.path.join(B.CSRC, "qgemm_internal.h")).read()
    ring = int(re.search(r"constexpr int PASS_RING = (\d+);", text).group(1))
    upto, deep = re.search(r"pass_ring\(int RT\) \{ return RT <= (\d+) \? PASS_RING : (\d+); \}", text).groups()
    return ring if rt <= int(upto) else int(deep)


@pytest.mark.parametrize("rt,msum", [(1, False), (1, True), (2, True), (3, True)])
def test_pass_step_loop_keeps_ring_in_flight(pass_asm, msum, rt):
    """The pass kernel's step loop at rt 16-row tiles: RING steps per ring turn,
    each behind a wait that leaves the other RING - 1 stages in flight, and no
    spills to scratch.  From two row tiles on the kernel exists only with the
    sub-block sums (the products form is not instantiated there)."""
    ring = _pass_ring(rt)
    body = _body(pass_asm, f"_ZN2qg11pass_kernelILi{ring}ELb{int(msum)}ELi{rt}EEEvNS_8PassArgsE")
    per_step = rt * (8 + (1 if msum else 8))     # sums: one fp16 product of their two parts
    steps = [(w, n) for w, n in _mfma_groups(body) if n >= per_step]
    assert len(steps) == ring, steps
    for w, n in steps:
        assert n == per_step, f"{n} MFMAs under one wait: steps merged behind a full drain"
        assert w == (ring - 1) * LOADS_PER_STAGE, f"step waits vmcnt({w})"
    assert "scratch_store" not in body and "scratch_load" not in body


@pytest.mark.parametrize("rt,nw", VARIANTS)
@pytest.mark.parametrize("msum", [False, True])
def test_stream_kernels_do_not_spill(asm, rt, nw, msum):
    body = _kernel_body(asm, rt, nw, msum)
    assert "scratch_store" not in body and "scratch_load" not in body


@pytest.mark.parametrize("vr", [1, 2, 3, 4])
def test_vector_unit_step_loop_keeps_ring_in_flight(asm, vr):
    body = _kernel_body(asm, 1, 8, True, vr)
    per_step = 32 * vr                                   # 8 operand pairs x 4 dot products per row
    steps = [(w, n) for w, n in _mfma_groups(body, r"v_dot2c?_f32_f16") if n >= per_step]
    assert len(steps) >= RING, steps
    for w, n in steps:
        assert n == per_step, f"{n} dot products under one wait"
        assert (RING - 1) * LOADS_PER_STAGE <= w <= RING * LOADS_PER_STAGE, f"step waits vmcnt({w})"
    assert "scratch_store" not in body and "scratch_load" not in body
