"""Python binding of libmoe_mi355x.so (see include/moe_mi355x.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch supplies device memory and the stream. The functions carry the
C entry points' names and take torch tensors (bf16 as torch.bfloat16 or
int16/uint16 bit patterns); outputs are caller-allocated unless a helper says
otherwise. A missing or unloadable library raises at import-time use; there is
no fallback path.
"""
import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EALIGN, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4, -5
MOE_F32_OUT, MOE_FORCE_DECODE, MOE_FORCE_PREFILL = 1, 2, 4
GATE, UP, DOWN = 0, 1, 2
MOE_STATUS_OFFSET, MOE_STATUS_ROUTE_TIMEOUT, MOE_STATUS_BAD_IDX = 8, 1, 2
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTS = [
    "moe_last_error", "moe_nvfp4_record_bytes", "moe_nvfp4_record_stride", "moe_nvfp4_bank_init",
    "moe_pack_nvfp4_bank", "moe_route_topk", "moe_sort_pairs", "moe_sort_workspace_bytes", "moe_sort_pairs_ws",
    "moe_nvfp4_workspace_bytes", "moe_nvfp4_forward", "moe_nvfp4_layer", "affine8_g64_linear", "moe_rmsnorm",
    "moe_nvfp4_dequant", "moe_profile_enable", "moe_profile_read", "moe_nvfp4_global_from_ws2",
    "moe_nvfp4_record_sha256", "moe_cache_create", "moe_cache_destroy", "moe_cache_prepare", "moe_cache_bank",
    "moe_cache_stats", "moe_vq_record_bytes", "moe_vq_record_stride", "moe_vq_bank_init", "moe_vq_pack_bank",
    "moe_vq_dequant", "moe_vq_workspace_bytes", "moe_vq_forward", "moe_status_read", "moe_status_clear",
    "moe_probe_hbm_read", "moe_probe_mfma_bf16", "moe_nvfp4_forward_noalloc",
]


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class moe_vq_bank(C.Structure):
    _fields_ = [("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32), ("reserved", C.c_int32),
                ("record_bytes", C.c_uint64), ("stride", C.c_uint64),
                ("part_off", C.c_uint64 * 6), ("base", C.c_void_p), ("codebook", C.c_void_p)]


class moe_nvfp4_bank(C.Structure):
    _fields_ = [("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32), ("reserved", C.c_int32),
                ("record_bytes", C.c_uint64), ("stride", C.c_uint64),
                ("part_off", C.c_uint64 * 9), ("base", C.c_void_p)]


_lib = None


def lib():
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(MOE_EINVAL, f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        vp, sz, i32 = C.c_void_p, C.c_size_t, C.c_int
        bankp = C.POINTER(moe_nvfp4_bank)
        L.moe_last_error.restype = C.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_nvfp4_record_bytes.restype = sz
        L.moe_nvfp4_record_bytes.argtypes = [i32, i32]
        L.moe_nvfp4_record_stride.restype = sz
        L.moe_nvfp4_record_stride.argtypes = [i32, i32]
        L.moe_nvfp4_bank_init.restype = i32
        L.moe_nvfp4_bank_init.argtypes = [bankp, vp, i32, i32, i32]
        L.moe_pack_nvfp4_bank.restype = i32
        L.moe_pack_nvfp4_bank.argtypes = [bankp, C.POINTER(vp), C.POINTER(vp), C.POINTER(vp), vp]
        L.moe_route_topk.restype = i32
        L.moe_route_topk.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
        L.moe_sort_pairs.restype = i32
        L.moe_sort_pairs.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.moe_sort_workspace_bytes.restype = sz
        L.moe_sort_workspace_bytes.argtypes = [i32, i32, i32]
        L.moe_sort_pairs_ws.restype = i32
        L.moe_sort_pairs_ws.argtypes = [vp, i32, i32, i32, vp, vp, vp, sz, vp]
        L.moe_nvfp4_workspace_bytes.restype = sz
        L.moe_nvfp4_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.moe_nvfp4_forward.restype = i32
        L.moe_nvfp4_forward.argtypes = [bankp, vp, i32, vp, vp, i32, vp, vp, C.c_uint, vp, sz, vp]
        L.moe_nvfp4_forward_noalloc.restype = i32
        L.moe_nvfp4_forward_noalloc.argtypes = [bankp, vp, i32, vp, vp, i32, vp, vp, C.c_uint, vp, vp]
        L.moe_nvfp4_layer.restype = i32
        L.moe_nvfp4_layer.argtypes = [bankp, vp, vp, i32, i32, vp, vp, vp, vp, vp, C.c_uint, vp, sz, vp]
        L.affine8_g64_linear.restype = i32
        L.affine8_g64_linear.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp]
        L.moe_rmsnorm.restype = i32
        L.moe_rmsnorm.argtypes = [vp, i32, i32, C.c_float, vp, vp]
        L.moe_nvfp4_dequant.restype = i32
        L.moe_nvfp4_dequant.argtypes = [bankp, i32, i32, vp, vp, vp]
        L.moe_nvfp4_global_from_ws2.restype = i32
        L.moe_nvfp4_global_from_ws2.argtypes = [vp, C.c_int64, vp, vp]
        L.moe_nvfp4_record_sha256.restype = i32
        L.moe_nvfp4_record_sha256.argtypes = [bankp, i32, i32, vp, vp]
        L.moe_cache_create.restype = i32
        L.moe_cache_create.argtypes = [bankp, vp, i32, C.POINTER(vp)]
        L.moe_cache_destroy.restype = i32
        L.moe_cache_destroy.argtypes = [vp]
        L.moe_cache_prepare.restype = i32
        L.moe_cache_prepare.argtypes = [vp, vp, i32, vp, vp]
        L.moe_cache_bank.restype = i32
        L.moe_cache_bank.argtypes = [vp, bankp]
        L.moe_cache_stats.restype = i32
        L.moe_cache_stats.argtypes = [vp, C.POINTER(C.c_int64), C.POINTER(C.c_int64), C.POINTER(C.c_int64)]
        vqp = C.POINTER(moe_vq_bank)
        L.moe_vq_record_bytes.restype = sz
        L.moe_vq_record_bytes.argtypes = [i32, i32]
        L.moe_vq_record_stride.restype = sz
        L.moe_vq_record_stride.argtypes = [i32, i32]
        L.moe_vq_bank_init.restype = i32
        L.moe_vq_bank_init.argtypes = [vqp, vp, vp, i32, i32, i32]
        L.moe_vq_pack_bank.restype = i32
        L.moe_vq_pack_bank.argtypes = [vqp, C.POINTER(vp), C.POINTER(vp), vp]
        L.moe_vq_dequant.restype = i32
        L.moe_vq_dequant.argtypes = [vqp, i32, i32, vp, vp]
        L.moe_vq_workspace_bytes.restype = sz
        L.moe_vq_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.moe_vq_forward.restype = i32
        L.moe_vq_forward.argtypes = [vqp, vp, i32, vp, vp, i32, vp, vp, C.c_uint, vp, sz, vp]
        L.moe_status_read.restype = i32
        L.moe_status_read.argtypes = [vp, C.POINTER(C.c_uint32), vp]
        L.moe_status_clear.restype = i32
        L.moe_status_clear.argtypes = [vp, vp]
        L.moe_probe_hbm_read.restype = i32
        L.moe_probe_hbm_read.argtypes = [vp, sz, i32, i32, vp, vp]
        L.moe_probe_mfma_bf16.restype = i32
        L.moe_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
        L.moe_profile_enable.restype = i32
        L.moe_profile_enable.argtypes = [i32]
        L.moe_profile_read.restype = i32
        L.moe_profile_read.argtypes = [C.c_char_p, C.POINTER(C.c_double), C.POINTER(C.c_int64)]
        _lib = L
    return _lib


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _need(what, t, nbytes):
    """Raises MOE_ESHAPE when the tensor t (if given) spans fewer than nbytes:
    the library takes plain pointers and reads or writes exactly the bytes
    its sizes imply, so a short buffer would be accessed past its end."""
    if t is None or nbytes <= 0:
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise MoeError(MOE_ESHAPE, f"{what}: {have} bytes, the call needs {int(nbytes)}")


def _need_tokens(T, H, E, k, flags=0, x=None, residual=None, y=None, idx=None, w=None, logits=None,
                 w_router=None):
    if T <= 0:
        return
    _need("x", x, T * H * 2)
    _need("residual", residual, T * H * 2)
    _need("y", y, T * H * (4 if flags & MOE_F32_OUT else 2))
    _need("idx", idx, T * k * 4)
    _need("w", w, T * k * 4)
    _need("logits", logits, T * E * 4)
    _need("w_router", w_router, E * H * 4)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# ---- sizes and the bank ----------------------------------------------------------
def moe_nvfp4_record_bytes(H, I):
    return lib().moe_nvfp4_record_bytes(H, I)


def moe_nvfp4_record_stride(H, I):
    return lib().moe_nvfp4_record_stride(H, I)


def moe_nvfp4_bank_init(base, H, I, E):
    """Descriptor for E records at the device tensor `base` (uint8, E*stride bytes)."""
    b = moe_nvfp4_bank()
    _check(lib().moe_nvfp4_bank_init(C.byref(b), C.c_void_p(base.data_ptr()), H, I, E))
    b._keep = base
    return b


def alloc_bank(H, I, E, device="cuda"):
    """Allocates a 4 KiB-aligned bank of E records on `device` and its descriptor."""
    stride = moe_nvfp4_record_stride(H, I)
    raw = torch.empty(E * stride + 4096, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 4096
    base = raw[off:off + E * stride]
    b = moe_nvfp4_bank_init(base, H, I, E)
    b._raw = raw
    return b, base


def moe_pack_nvfp4_bank(bank, codes, scales, g, stream=None):
    """codes[p]: int32/uint32 [E][out][in/8]; scales[p]: uint8 [E][out][in/16]; g[p]: f32 [E]."""
    for t in list(codes) + list(scales) + list(g):
        assert t.is_contiguous()
    cp = (C.c_void_p * 3)(*[t.data_ptr() for t in codes])
    sp = (C.c_void_p * 3)(*[t.data_ptr() for t in scales])
    gp = (C.c_void_p * 3)(*[t.data_ptr() for t in g])
    _check(lib().moe_pack_nvfp4_bank(C.byref(bank), cp, sp, gp, _stream(stream)))


# ---- routing ------------------------------------------------------------------------
def moe_route_topk(x, w_router, logits, T, H, E, k, idx, w, stream=None):
    _need_tokens(T, H, E, k, x=x, w_router=None if x is None else w_router, logits=logits, idx=idx, w=w)
    _check(lib().moe_route_topk(_ptr(x), _ptr(w_router), _ptr(logits), T, H, E, k, _ptr(idx), _ptr(w),
                                _stream(stream)))


def moe_sort_pairs(idx, T, k, E, offsets, sorted_, stream=None):
    if T > 0:
        _need("idx", idx, T * k * 4)
        _need("sorted", sorted_, T * k * 4)
        _need("offsets", offsets, (E + 1) * 4)
    _check(lib().moe_sort_pairs(_ptr(idx), T, k, E, _ptr(offsets), _ptr(sorted_), _stream(stream)))


def moe_sort_workspace_bytes(T, k, E):
    return lib().moe_sort_workspace_bytes(T, k, E)


def moe_sort_pairs_ws(idx, T, k, E, offsets, sorted_, workspace, stream=None):
    if T > 0:
        _need("idx", idx, T * k * 4)
        _need("sorted", sorted_, T * k * 4)
        _need("offsets", offsets, (E + 1) * 4)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_sort_pairs_ws(_ptr(idx), T, k, E, _ptr(offsets), _ptr(sorted_), _ptr(workspace), ws_bytes,
                                   _stream(stream)))


# ---- the layer ----------------------------------------------------------------------
def moe_nvfp4_workspace_bytes(T, k, H, I, E):
    return lib().moe_nvfp4_workspace_bytes(T, k, H, I, E)


def moe_nvfp4_forward(bank, x, T, idx, w, k, residual, y, flags, workspace, stream=None):
    _need_tokens(T, bank.H, bank.E, k, flags, x=x, residual=residual, y=y, idx=idx, w=w)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_nvfp4_forward(C.byref(bank), _ptr(x), T, _ptr(idx), _ptr(w), k, _ptr(residual), _ptr(y),
                                   flags, _ptr(workspace), ws_bytes, _stream(stream)))


def moe_nvfp4_forward_noalloc(bank, x, T, idx, w, k, residual, y, flags, status=None, stream=None):
    _need_tokens(T, bank.H, bank.E, k, flags, x=x, residual=residual, y=y, idx=idx, w=w)
    _check(lib().moe_nvfp4_forward_noalloc(C.byref(bank), _ptr(x), T, _ptr(idx), _ptr(w), k, _ptr(residual), _ptr(y),
                                           flags, _ptr(status), _stream(stream)))


def moe_nvfp4_layer(bank, x, w_router, T, k, residual, logits, idx, w, y, flags, workspace, stream=None):
    _need_tokens(T, bank.H, bank.E, k, flags, x=x, residual=residual, y=y, idx=idx, w=w, logits=logits,
                 w_router=w_router)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_nvfp4_layer(C.byref(bank), _ptr(x), _ptr(w_router), T, k, _ptr(residual), _ptr(logits),
                                 _ptr(idx), _ptr(w), _ptr(y), flags, _ptr(workspace), ws_bytes, _stream(stream)))


def affine8_g64_linear(x, codes, scales, biases, T, K, N, y, stream=None):
    if T > 0 and K > 0 and N > 0:
        _need("x", x, T * K * 2)
        _need("codes", codes, N * K)
        _need("scales", scales, N * (K // 64) * 2)
        _need("biases", biases, N * (K // 64) * 2)
        _need("y", y, T * N * 2)
    _check(lib().affine8_g64_linear(_ptr(x), _ptr(codes), _ptr(scales), _ptr(biases), T, K, N, _ptr(y),
                                    _stream(stream)))


def moe_rmsnorm(x, T, H, eps, y, stream=None):
    if T > 0 and H > 0:
        _need("x", x, T * H * 2)
        _need("y", y, T * H * 2)
    _check(lib().moe_rmsnorm(_ptr(x), T, H, float(eps), _ptr(y), _stream(stream)))


def moe_nvfp4_dequant(bank, expert, proj, out_f32, out_unit, stream=None):
    _need("out_f32", out_f32, bank.H * bank.I * 4)
    _need("out_unit", out_unit, bank.H * bank.I * 2)
    _check(lib().moe_nvfp4_dequant(C.byref(bank), expert, proj, _ptr(out_f32), _ptr(out_unit), _stream(stream)))


def moe_nvfp4_global_from_ws2(ws2):
    """g (f32) and the inexact flags (u8) for host f32 values ws2 (numpy)."""
    import numpy as np
    ws2 = np.ascontiguousarray(ws2, dtype=np.float32)
    g = np.empty_like(ws2)
    inexact = np.empty(ws2.shape, dtype=np.uint8)
    _check(lib().moe_nvfp4_global_from_ws2(ws2.ctypes.data_as(C.c_void_p), ws2.size,
                                           g.ctypes.data_as(C.c_void_p), inexact.ctypes.data_as(C.c_void_p)))
    return g, inexact


def moe_nvfp4_record_sha256(bank, e0, n, digests, stream=None):
    """digests: device uint8 [n][32]."""
    _need("digests", digests, n * 32)
    _check(lib().moe_nvfp4_record_sha256(C.byref(bank), e0, n, _ptr(digests), _stream(stream)))


def moe_cache_create(host_bank, slot_base, nslots):
    """host_bank: descriptor over pinned host memory; slot_base: device uint8
    tensor of nslots * stride bytes (4096-aligned). Returns the handle."""
    h = C.c_void_p()
    _check(lib().moe_cache_create(C.byref(host_bank), _ptr(slot_base), nslots, C.byref(h)))
    return h


def moe_cache_destroy(handle):
    _check(lib().moe_cache_destroy(handle))


def moe_cache_prepare(handle, ids, stream=None):
    """ids: host int sequence; returns the slots (numpy int32)."""
    import numpy as np
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    slot_of = np.empty_like(ids)
    _check(lib().moe_cache_prepare(handle, ids.ctypes.data_as(C.c_void_p), ids.size,
                                   slot_of.ctypes.data_as(C.c_void_p), _stream(stream)))
    return slot_of


def moe_cache_bank(handle):
    b = moe_nvfp4_bank()
    _check(lib().moe_cache_bank(handle, C.byref(b)))
    return b


def moe_cache_stats(handle):
    h, m, n = C.c_int64(), C.c_int64(), C.c_int64()
    _check(lib().moe_cache_stats(handle, C.byref(h), C.byref(m), C.byref(n)))
    return h.value, m.value, n.value


# ---- 8-dim VQ experts ---------------------------------------------------------------
def moe_vq_record_bytes(H, I):
    return lib().moe_vq_record_bytes(H, I)


def moe_vq_record_stride(H, I):
    return lib().moe_vq_record_stride(H, I)


def moe_vq_bank_init(base, codebook, H, I, E):
    b = moe_vq_bank()
    _check(lib().moe_vq_bank_init(C.byref(b), _ptr(base), _ptr(codebook), H, I, E))
    b._keep = (base, codebook)
    return b


def alloc_vq_bank(codebook, H, I, E, device="cuda"):
    """A 4 KiB-aligned bank of E VQ records on `device` over the device codebook
    (uint8 [4096][8]) and its descriptor."""
    stride = moe_vq_record_stride(H, I)
    raw = torch.empty(E * stride + 4096, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 4096
    base = raw[off:off + E * stride]
    b = moe_vq_bank_init(base, codebook, H, I, E)
    b._raw = raw
    return b, base


def moe_vq_pack_bank(bank, idx, gains, stream=None):
    ip = (C.c_void_p * 3)(*[t.data_ptr() for t in idx])
    gp = (C.c_void_p * 3)(*[t.data_ptr() for t in gains])
    _check(lib().moe_vq_pack_bank(C.byref(bank), ip, gp, _stream(stream)))


def moe_vq_dequant(bank, expert, proj, out_f32, stream=None):
    _need("out_f32", out_f32, bank.H * bank.I * 4)
    _check(lib().moe_vq_dequant(C.byref(bank), expert, proj, _ptr(out_f32), _stream(stream)))


def moe_vq_workspace_bytes(T, k, H, I):
    return lib().moe_vq_workspace_bytes(T, k, H, I)


def moe_vq_forward(bank, x, T, idx, w, k, residual, y, flags, ws, stream=None):
    _need_tokens(T, bank.H, bank.E, k, flags, x=x, residual=residual, y=y, idx=idx, w=w)
    _check(lib().moe_vq_forward(C.byref(bank), _ptr(x), T, _ptr(idx), _ptr(w), k, _ptr(residual), _ptr(y), flags,
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_probe_hbm_read(buf, nbytes, variant, blocks, sink, stream=None):
    _check(lib().moe_probe_hbm_read(_ptr(buf), nbytes, variant, blocks, _ptr(sink), _stream(stream)))


def moe_probe_mfma_bf16(blocks, iters, sink, stream=None):
    _check(lib().moe_probe_mfma_bf16(blocks, iters, _ptr(sink), _stream(stream)))


def moe_profile_enable(on):
    _check(lib().moe_profile_enable(1 if on else 0))


def moe_profile_read(name):
    ms, n = C.c_double(), C.c_int64()
    _check(lib().moe_profile_read(name.encode(), C.byref(ms), C.byref(n)))
    return ms.value, n.value


def moe_status_read(workspace, stream=None):
    """The workspace's status word (waits for the stream)."""
    v = C.c_uint32()
    _check(lib().moe_status_read(_ptr(workspace), C.byref(v), _stream(stream)))
    return v.value


def moe_status_clear(workspace, stream=None):
    _check(lib().moe_status_clear(_ptr(workspace), _stream(stream)))


def workspace(nbytes, device="cuda"):
    """A 256-byte aligned device workspace of at least nbytes (torch allocations
    are), its status word cleared."""
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    moe_status_clear(t)
    return t
