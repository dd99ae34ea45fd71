"""Properties of the compiled gfx950 code that the kernels' correctness rests
on and that no source-level test can see (CPU only: hipcc compiles the
device code to assembly, nothing runs).

The streaming affine8 kernel issues its HBM -> LDS loads from inline asm, then
every code load as a buffer load, and then waits with vmcnt(number of code
loads): the wait covers the LDS loads only if the compiler keeps every code
load above it. If a later compiler moved one below, the count would let an
LDS load still be in flight when the barrier releases the waves."""
import os
import re
import shutil
import subprocess

import pytest

from weight_quantized_moe_amd import build as B

SRC = os.path.join(B.SRC, "misc.hip")


def _device_asm(src):
    if not os.path.exists(B.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    flags = [f for f in B.FLAGS if not f.startswith("-W")]
    r = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", "-"], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    return r.stdout


def _function(asm, mangled):
    m = re.search(rf"^{re.escape(mangled)}:[^\n]*\n(.*?)\ts_endpgm", asm, re.S | re.M)
    assert m, f"{mangled} not found"
    return m.group(1)


def test_affine8_stream_code_loads_precede_the_lds_wait():
    asm = _device_asm(SRC)
    for gw in range(1, 7):
        body = _function(asm, f"_ZN3moe21affine8_stream_kernelILi{gw}EEEvPKtPKhS2_S2_iiiPt")
        lines = body.splitlines()
        first_wait = next(i for i, l in enumerate(lines) if re.search(r"s_waitcnt\s+vmcnt", l))
        before = lines[:first_wait]
        n_buf = sum("buffer_load_dwordx4" in l for l in before)
        n_buf_all = sum("buffer_load" in l for l in lines)
        assert n_buf == n_buf_all == 2 * gw, (gw, n_buf, n_buf_all)
        assert re.search(rf"vmcnt\({2 * gw}\)", lines[first_wait]), lines[first_wait]
        # every HBM -> LDS load comes before the first code load
        first_buf = next(i for i, l in enumerate(lines) if "buffer_load" in l)
        assert not any("global_load_lds" in l for l in lines[first_buf:first_wait])
        assert any("global_load_lds" in l for l in lines[:first_buf])
        # no other vector-memory load between them
        assert not any(re.search(r"global_load_(?!lds)|scratch_", l) for l in before)


def test_affine8_gemm_dma_kernel_waits_are_its_own():
    """The HBM -> LDS GEMM's loop waits for its loads by count (vmcnt(4): the
    next group's activations may stay in flight). That count holds only if
    no compiled vector-memory load shares the counter: every load of the
    kernel must be one of its own HBM -> LDS loads, and every vmcnt wait one
    of its own."""
    asm = _device_asm(os.path.join(B.SRC, "affine8_gemm.hip"))
    body = _function(asm, "_ZN3moe23affine8_gemm_dma_kernelEPKtPKhS1_S1_iiiiiPtPf")
    lines = body.splitlines()
    assert sum("global_load_lds_dwordx4" in l for l in lines) >= 7
    assert not any(re.search(r"global_load_(?!lds)|buffer_load|scratch_|flat_load", l) for l in lines)
    waits = [int(m.group(1)) for l in lines for m in [re.search(r"s_waitcnt\s+vmcnt\((\d+)\)", l)] if m]
    assert waits and set(waits) <= {0, 4}, waits


def test_affine8_gemm_group_sums_read_all_four_words():
    """Each 16-byte piece's sum is four v_dot2 against (1, 1), one per word.
    Written with a bit cast of the vector's element accesses, this compiler
    read element 0 four times; the helper takes the words through an array.
    Every run of four accumulating v_dot2 into one register must read four
    different source registers."""
    asm = _device_asm(os.path.join(B.SRC, "affine8_gemm.hip"))
    for name in ("_ZN3moe19affine8_gemm_kernelEPKtPKhS1_S1_iiiiiPtPf", "_ZN3moe23affine8_gemm_dma_kernelEPKtPKhS1_S1_iiiiiPtPf"):
        dots = [m.groups() for l in _function(asm, name).splitlines()
                for m in [re.search(r"v_dot2c_f32_bf16_e32 (v\d+), 0x3f803f80, (v\d+)", l)] if m]
        assert len(dots) >= 8 and len(dots) % 4 == 0, (name, len(dots))
        by_dst = {}
        for dst, src in dots:
            by_dst.setdefault(dst, []).append(src)
        for dst, srcs in by_dst.items():
            for i in range(0, len(srcs) - 3, 4):
                assert len(set(srcs[i:i + 4])) == 4, (name, dst, srcs)


def test_vq_kernels_index_loads_precede_the_lds_wait():
    """The VQ gate/up and down kernels copy the codebook and their inputs HBM
    -> LDS from inline asm, then load their index groups into registers (the
    same number in every lane), then wait with vmcnt(number of index loads)
    before the barrier: the wait covers the copies only if every index load
    of the first pass sits between them and it, and no other vector-memory
    load shares the counter there."""
    asm = _device_asm(os.path.join(B.SRC, "vq.hip"))
    for name, n in (("_ZN3moe16vq_gateup_kernelENS_6VqArgsE", 20), ("_ZN3moe14vq_down_kernelENS_6VqArgsE", 5)):
        lines = _function(asm, name).splitlines()
        first_wait = next(i for i, l in enumerate(lines) if re.search(r"s_waitcnt\s+vmcnt", l))
        assert re.search(rf"vmcnt\({n}\)", lines[first_wait]), (name, lines[first_wait])
        assert "s_barrier" in "".join(lines[first_wait:first_wait + 4]), name
        before = lines[:first_wait]
        loads = [i for i, l in enumerate(before) if "global_load_dwordx3" in l]
        assert len(loads) == n, (name, len(loads))
        lds = [i for i, l in enumerate(before) if "global_load_lds" in l]
        assert lds and max(lds) < min(loads), name
        assert not any(re.search(r"global_load_(?!lds|dwordx3)|buffer_load|scratch_|flat_load", l) for l in before), name
