"""The C-ABI library loads, exports every function include/moe_mi355x.h
declares, and rejects bad arguments before it touches a GPU (these calls run
on a machine without one)."""
import ctypes as C
import os
import re

import pytest

import oracle
import weight_quantized_moe_amd as wq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_mi355x.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 17, names
    assert sorted(names) == sorted(wq.EXPORTS)
    L = C.CDLL(wq.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_record_sizes_match_oracle():
    for H, I in [(5120, 2560), (256, 128), (64, 64), (16, 32)]:
        _, nbytes, stride = oracle.record_layout(H, I)
        assert wq.moe_nvfp4_record_bytes(H, I) == nbytes
        assert wq.moe_nvfp4_record_stride(H, I) == stride
    assert wq.moe_nvfp4_record_bytes(24, 16) == 0


def test_bank_init_layout_and_errors():
    L = wq.lib()
    b = wq.moe_nvfp4_bank()
    assert L.moe_nvfp4_bank_init(C.byref(b), C.c_void_p(1 << 20), 5120, 2560, 256) == wq.MOE_OK
    off, nbytes, stride = oracle.record_layout(5120, 2560)
    assert list(b.part_off) == off and b.record_bytes == nbytes and b.stride == stride
    assert L.moe_nvfp4_bank_init(C.byref(b), C.c_void_p((1 << 20) + 256), 5120, 2560, 256) == wq.MOE_EALIGN
    assert L.moe_nvfp4_bank_init(C.byref(b), C.c_void_p(1 << 20), 5120, 2568, 256) == wq.MOE_ESHAPE
    assert L.moe_nvfp4_bank_init(C.byref(b), C.c_void_p(1 << 20), 5120, 2560, 0) == wq.MOE_ESHAPE
    assert L.moe_nvfp4_bank_init(C.byref(b), None, 5120, 2560, 16) == wq.MOE_EINVAL
    assert b"bank_init" in L.moe_last_error()


def _bank(H=256, I=128, E=16):
    b = wq.moe_nvfp4_bank()
    assert wq.lib().moe_nvfp4_bank_init(C.byref(b), C.c_void_p(1 << 24), H, I, E) == 0
    return b


def test_forward_validation_before_launch():
    L = wq.lib()
    b = _bank()
    fake = C.c_void_p(1 << 26)
    ws_need = L.moe_nvfp4_workspace_bytes(4, 2, 256, 128, 16)
    assert ws_need > 0
    args = lambda **kw: dict(dict(x=fake, T=4, idx=fake, w=fake, k=2, res=None, y=fake, flags=0, ws=fake,
                                  wsb=ws_need), **kw)

    def call(a, bank=b):
        return L.moe_nvfp4_forward(C.byref(bank), a["x"], a["T"], a["idx"], a["w"], a["k"], a["res"], a["y"],
                                   a["flags"], a["ws"], a["wsb"], None)

    assert call(args(k=0)) == wq.MOE_ESHAPE
    assert call(args(k=17)) == wq.MOE_ESHAPE
    assert call(args(T=-1)) == wq.MOE_ESHAPE
    assert call(args(x=None)) == wq.MOE_EINVAL
    assert call(args(wsb=ws_need - 1)) == wq.MOE_EWORKSPACE
    assert call(args(ws=C.c_void_p((1 << 26) + 16))) == wq.MOE_EALIGN
    assert call(args(x=C.c_void_p((1 << 26) + 2))) == wq.MOE_EALIGN
    assert call(args(y=C.c_void_p((1 << 26) + 8))) == wq.MOE_EALIGN
    assert call(args(res=C.c_void_p((1 << 26) + 4))) == wq.MOE_EALIGN
    assert call(args(flags=wq.MOE_FORCE_DECODE | wq.MOE_FORCE_PREFILL)) == wq.MOE_EINVAL
    assert call(args(flags=64)) == wq.MOE_EINVAL
    assert call(args(T=0)) == wq.MOE_OK  # nothing to do, nothing launched
    bad = _bank(H=256, I=96)  # I not a multiple of 64
    assert call(args(), bank=bad) == wq.MOE_ESHAPE
    broken = _bank()
    broken.part_off[2] += 4  # up.codes no longer 16-byte aligned
    assert call(args(), bank=broken) == wq.MOE_EALIGN
    broken = _bank()
    broken.stride = 4096
    assert call(args(), bank=broken) == wq.MOE_EINVAL


def test_layer_validation_before_launch():
    L = wq.lib()
    b = _bank()
    fake = C.c_void_p(1 << 26)
    ws_need = L.moe_nvfp4_workspace_bytes(1, 2, 256, 128, 16)
    args = lambda **kw: dict(dict(x=fake, wr=fake, T=1, k=2, res=None, lg=fake, idx=fake, w=fake, y=fake, flags=0,
                                  ws=fake, wsb=ws_need), **kw)

    def call(a, bank=b):
        return L.moe_nvfp4_layer(C.byref(bank), a["x"], a["wr"], a["T"], a["k"], a["res"], a["lg"], a["idx"],
                                 a["w"], a["y"], a["flags"], a["ws"], a["wsb"], None)

    assert call(args(k=0)) == wq.MOE_ESHAPE
    assert call(args(k=17)) == wq.MOE_ESHAPE
    assert call(args(T=-1)) == wq.MOE_ESHAPE
    assert call(args(wr=None)) == wq.MOE_EINVAL
    assert call(args(lg=None)) == wq.MOE_EINVAL
    assert call(args(idx=None)) == wq.MOE_EINVAL
    assert call(args(wsb=ws_need - 1)) == wq.MOE_EWORKSPACE
    assert call(args(wr=C.c_void_p((1 << 26) + 8))) == wq.MOE_EALIGN
    assert call(args(lg=C.c_void_p((1 << 26) + 2))) == wq.MOE_EALIGN
    assert call(args(x=C.c_void_p((1 << 26) + 2))) == wq.MOE_EALIGN
    assert call(args(flags=wq.MOE_FORCE_DECODE | wq.MOE_FORCE_PREFILL)) == wq.MOE_EINVAL
    assert call(args(T=0)) == wq.MOE_OK
    bad = _bank(H=256, I=96)
    assert call(args(), bank=bad) == wq.MOE_ESHAPE
    assert b"layer" in L.moe_last_error()


def test_route_sort_affine_rmsnorm_validation():
    L = wq.lib()
    fake = C.c_void_p(1 << 26)
    assert L.moe_route_topk(None, None, fake, 4, 256, 16, 0, fake, fake, None) == wq.MOE_ESHAPE
    assert L.moe_route_topk(None, None, fake, 4, 256, 16, 17, fake, fake, None) == wq.MOE_ESHAPE
    assert L.moe_route_topk(None, None, fake, 4, 256, 2048, 8, fake, fake, None) == wq.MOE_ESHAPE
    assert L.moe_route_topk(fake, None, fake, 4, 256, 16, 2, fake, fake, None) == wq.MOE_EINVAL
    assert L.moe_route_topk(fake, fake, fake, 4, 250, 16, 2, fake, fake, None) == wq.MOE_ESHAPE
    assert L.moe_route_topk(C.c_void_p((1 << 26) + 2), fake, fake, 4, 256, 16, 2, fake, fake, None) == wq.MOE_EALIGN
    assert L.moe_route_topk(None, None, fake, 0, 256, 16, 2, fake, fake, None) == wq.MOE_OK
    assert L.moe_sort_pairs(fake, 4, 0, 16, fake, fake, None) == wq.MOE_ESHAPE
    assert L.moe_sort_pairs(None, 4, 2, 16, fake, fake, None) == wq.MOE_EINVAL
    assert L.affine8_g64_linear(fake, fake, fake, fake, 2, 100, 64, fake, None) == wq.MOE_ESHAPE
    assert L.affine8_g64_linear(fake, C.c_void_p((1 << 26) + 4), fake, fake, 2, 128, 64, fake, None) == wq.MOE_EALIGN
    assert L.moe_rmsnorm(fake, 2, 0, C.c_float(1e-6), fake, None) == wq.MOE_ESHAPE
    assert L.moe_rmsnorm(fake, 2, 16, C.c_float(-1.0), fake, None) == wq.MOE_EINVAL
    b = _bank()
    assert L.moe_nvfp4_dequant(C.byref(b), 16, 0, fake, None, None) == wq.MOE_EINVAL
    assert L.moe_nvfp4_dequant(C.byref(b), 0, 3, fake, None, None) == wq.MOE_EINVAL
    assert L.moe_nvfp4_dequant(C.byref(b), 0, 0, None, None, None) == wq.MOE_EINVAL


def test_workspace_sizes_grow_with_pairs():
    L = wq.lib()
    a = L.moe_nvfp4_workspace_bytes(1, 8, 5120, 2560, 256)
    b = L.moe_nvfp4_workspace_bytes(8192, 8, 5120, 2560, 256)
    assert 0 < a < b
    # mids (bf16) and per-pair f32 rows dominate: P*(2I + 4H) bytes
    assert b >= 65536 * (2 * 2560 + 4 * 5120)


def test_pack_side_validation():
    L = wq.lib()
    b = _bank()
    fake = C.c_void_p(1 << 26)
    assert L.moe_nvfp4_record_sha256(C.byref(b), 15, 2, fake, None) == wq.MOE_EINVAL
    assert L.moe_nvfp4_record_sha256(C.byref(b), -1, 1, fake, None) == wq.MOE_EINVAL
    assert L.moe_nvfp4_record_sha256(C.byref(b), 0, 1, None, None) == wq.MOE_EINVAL
    assert L.moe_nvfp4_record_sha256(C.byref(b), 0, 1, C.c_void_p((1 << 26) + 2), None) == wq.MOE_EALIGN
    assert L.moe_nvfp4_record_sha256(None, 0, 1, fake, None) == wq.MOE_EINVAL
    assert L.moe_nvfp4_record_sha256(C.byref(b), 3, 0, None, None) == wq.MOE_OK


def test_manifest_part_table():
    from weight_quantized_moe_amd import manifest
    b = _bank(5120, 2560, 256)
    parts = manifest.part_table(b)
    assert [p[0] for p in parts] == ["gate.codes", "gate.scales", "up.codes", "up.scales", "down.codes",
                                     "down.scales", "gate.global", "up.global", "down.global"]
    # contiguous, ending at the record size
    end = 0
    for _, off, length in parts:
        assert off == end
        end = off + length
    assert end == b.record_bytes == 22118412


def test_cache_validation_before_any_hip_call():
    L = wq.lib()
    host = _bank(256, 128, 16)
    fake = C.c_void_p(1 << 26)
    h = C.c_void_p()
    assert L.moe_cache_create(C.byref(host), fake, 5, None) == wq.MOE_EINVAL
    assert L.moe_cache_create(C.byref(host), fake, 0, C.byref(h)) == wq.MOE_ESHAPE
    assert L.moe_cache_create(C.byref(host), fake, 17, C.byref(h)) == wq.MOE_ESHAPE
    assert L.moe_cache_create(C.byref(host), None, 5, C.byref(h)) == wq.MOE_EINVAL
    assert L.moe_cache_create(C.byref(host), C.c_void_p((1 << 26) + 256), 5, C.byref(h)) == wq.MOE_EALIGN
    assert L.moe_cache_create(None, fake, 5, C.byref(h)) == wq.MOE_EINVAL
    assert h.value is None
    assert L.moe_cache_prepare(None, None, 0, None, None) == wq.MOE_EINVAL
    assert L.moe_cache_bank(None, C.byref(host)) == wq.MOE_EINVAL
    assert L.moe_cache_stats(None, None, None, None) == wq.MOE_EINVAL


def test_vq_sizes_and_validation():
    L = wq.lib()
    for H, I in [(5120, 2560), (256, 128), (128, 64)]:
        _, nbytes, stride = oracle.vq_layout(H, I)
        assert wq.moe_vq_record_bytes(H, I) == nbytes and wq.moe_vq_record_stride(H, I) == stride
    assert wq.moe_vq_record_bytes(5120, 2576) == 0
    b = wq.moe_vq_bank()
    fake, cb = C.c_void_p(1 << 26), C.c_void_p(1 << 22)
    assert L.moe_vq_bank_init(C.byref(b), fake, cb, 5120, 2560, 256) == wq.MOE_OK
    off, nbytes, _ = oracle.vq_layout(5120, 2560)
    assert list(b.part_off) == off and b.record_bytes == nbytes
    assert L.moe_vq_bank_init(C.byref(b), fake, None, 5120, 2560, 256) == wq.MOE_EINVAL
    assert L.moe_vq_bank_init(C.byref(b), fake, C.c_void_p((1 << 22) + 8), 5120, 2560, 256) == wq.MOE_EALIGN
    assert L.moe_vq_bank_init(C.byref(b), fake, cb, 5120, 2560 + 16, 256) == wq.MOE_ESHAPE
    assert L.moe_vq_bank_init(C.byref(b), fake, cb, 5120, 2560, 256) == wq.MOE_OK
    ws = wq.moe_vq_workspace_bytes(1, 8, 5120, 2560)
    assert ws >= 8 * 2560 * 2 and wq.moe_vq_workspace_bytes(1, 17, 5120, 2560) == 0
    f = lambda **kw: L.moe_vq_forward(C.byref(b), kw.get("x", fake), kw.get("T", 1), fake, fake, kw.get("k", 8),
                                      None, fake, 0, fake, kw.get("wsb", ws), None)
    assert f(k=0) == wq.MOE_ESHAPE and f(k=17) == wq.MOE_ESHAPE
    assert f(T=-1) == wq.MOE_ESHAPE
    assert f(x=None) == wq.MOE_EINVAL
    assert f(x=C.c_void_p((1 << 26) + 8)) == wq.MOE_EALIGN
    assert f(wsb=ws - 1) == wq.MOE_EWORKSPACE
    assert f(T=0) == wq.MOE_OK
    assert L.moe_vq_dequant(C.byref(b), 256, 0, fake, None) == wq.MOE_EINVAL
    assert L.moe_vq_dequant(C.byref(b), 0, 3, fake, None) == wq.MOE_EINVAL


def test_layer_shapes_off_the_quad_grid_rejected():
    # A bank takes rows of any multiple of 16 inputs, the layer kernels walk
    # rows in 64-input quads: H or I of 16 * odd are refused before a launch.
    L = wq.lib()
    fake = C.c_void_p(1 << 26)
    for H, I in [(208, 112), (16 * 13, 128), (256, 16 * 9), (48, 64)]:
        b = wq.moe_nvfp4_bank()
        assert L.moe_nvfp4_bank_init(C.byref(b), C.c_void_p(1 << 24), H, I, 16) == wq.MOE_OK
        need = L.moe_nvfp4_workspace_bytes(4, 2, H, I, 16)
        rc = L.moe_nvfp4_forward(C.byref(b), fake, 4, fake, fake, 2, None, fake, 0, fake, need, None)
        assert rc == wq.MOE_ESHAPE and b"multiples of 64" in L.moe_last_error()
        rc = L.moe_nvfp4_layer(C.byref(b), fake, fake, 1, 2, None, fake, fake, fake, fake, 0, fake, need, None)
        assert rc == wq.MOE_ESHAPE


def test_status_word_calls_validate():
    L = wq.lib()
    v = C.c_uint32()
    assert L.moe_status_read(None, C.byref(v), None) == wq.MOE_EINVAL
    assert L.moe_status_read(C.c_void_p(1 << 26), None, None) == wq.MOE_EINVAL
    assert L.moe_status_read(C.c_void_p((1 << 26) + 64), C.byref(v), None) == wq.MOE_EALIGN
    assert L.moe_status_clear(None, None) == wq.MOE_EINVAL
    assert L.moe_status_clear(C.c_void_p((1 << 26) + 8), None) == wq.MOE_EALIGN
    assert wq.MOE_STATUS_OFFSET == 8 and (wq.MOE_STATUS_ROUTE_TIMEOUT, wq.MOE_STATUS_BAD_IDX) == (1, 2)


def test_binding_rejects_short_buffers_before_the_call():
    """The binding checks every tensor against the bytes the call's sizes
    imply (the library takes plain pointers and would access past a short
    buffer's end). Host tensors serve: the check raises before any library
    call."""
    import torch

    b = wq.moe_nvfp4_bank()
    b.H, b.I, b.E = 128, 64, 16
    T, k, H = 8, 4, 128

    def t(n, dtype=torch.int16):
        return torch.empty(n, dtype=dtype)

    ok = dict(x=t(T * H), idx=t(T * k, torch.int32), w=t(T * k, torch.float32), y=t(T * H))
    cases = [("x", t(T * H - 1)), ("idx", t(T * k - 1, torch.int32)), ("w", t(T * k - 1, torch.float32)),
             ("y", t(T * H - 1))]
    for name, short in cases:
        a = dict(ok, **{name: short})
        with pytest.raises(wq.MoeError) as e:
            wq.moe_nvfp4_forward(b, a["x"], T, a["idx"], a["w"], k, None, a["y"], 0, t(256, torch.uint8))
        assert e.value.code == wq.MOE_ESHAPE and name in str(e.value), (name, e.value)
    # an f32 output needs 4 bytes per value; a residual as many bytes as x
    with pytest.raises(wq.MoeError, match="y"):
        wq.moe_nvfp4_forward(b, ok["x"], T, ok["idx"], ok["w"], k, None, t(T * H), wq.MOE_F32_OUT, t(256, torch.uint8))
    with pytest.raises(wq.MoeError, match="residual"):
        wq.moe_nvfp4_forward(b, ok["x"], T, ok["idx"], ok["w"], k, t(T * H // 2), ok["y"], 0, t(256, torch.uint8))
    # the one-call layer also checks the router weights and the logits
    with pytest.raises(wq.MoeError, match="w_router"):
        wq.moe_nvfp4_layer(b, ok["x"], t(b.E * H - 1, torch.float32), T, k, None, t(T * b.E, torch.float32),
                           ok["idx"], ok["w"], ok["y"], 0, t(256, torch.uint8))
    with pytest.raises(wq.MoeError, match="logits"):
        wq.moe_route_topk(None, None, t(T * b.E - 1, torch.float32), T, H, b.E, k, ok["idx"], ok["w"])
    with pytest.raises(wq.MoeError, match="codes"):
        wq.affine8_g64_linear(t(T * H), t(H * H - 1, torch.uint8), t(H * 2), t(H * 2), T, H, H, t(T * H))
    with pytest.raises(wq.MoeError, match="y"):
        wq.moe_rmsnorm(t(T * H), T, H, 1e-6, t(T * H - 8))
