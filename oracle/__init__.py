"""ctypes wrapper of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the product library never does. Arrays are numpy;
bf16 values travel as uint16 bit patterns.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None

GATE, UP, DOWN = 0, 1, 2
ACC_F64, ACC_F32 = 0, 1


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        u8p, u16p, u32p = C.POINTER(C.c_uint8), C.POINTER(C.c_uint16), C.POINTER(C.c_uint32)
        i32p, f32p, u64p = C.POINTER(C.c_int32), C.POINTER(C.c_float), C.POINTER(C.c_uint64)
        L.orc_e2m1_value.restype = C.c_double
        L.orc_e2m1_value.argtypes = [C.c_uint]
        L.orc_e4m3_value.restype = C.c_double
        L.orc_e4m3_value.argtypes = [C.c_uint]
        L.orc_bf16_to_f32.restype = C.c_float
        L.orc_bf16_to_f32.argtypes = [C.c_uint16]
        L.orc_f64_to_bf16.restype = C.c_uint16
        L.orc_f64_to_bf16.argtypes = [C.c_double]
        L.orc_global_factor.restype = C.c_float
        L.orc_global_factor.argtypes = [C.c_float]
        L.orc_block_scale.restype = C.c_float
        L.orc_block_scale.argtypes = [C.c_uint, C.c_float]
        L.orc_weight.restype = C.c_float
        L.orc_weight.argtypes = [C.c_uint, C.c_uint, C.c_float]
        L.orc_record_layout.restype = C.c_int
        L.orc_record_layout.argtypes = [C.c_int, C.c_int, u64p, u64p, u64p]
        L.orc_pack_record.restype = None
        L.orc_pack_record.argtypes = [C.c_int, C.c_int, C.POINTER(u32p), C.POINTER(u8p), f32p, u8p]
        L.orc_dequant_projection.restype = None
        L.orc_dequant_projection.argtypes = [u8p, C.c_int, C.c_int, C.c_int, f32p, u16p]
        L.orc_router_logits.restype = None
        L.orc_router_logits.argtypes = [u16p, f32p, C.c_int, C.c_int, C.c_int, f32p]
        L.orc_route_topk.restype = C.c_int
        L.orc_route_topk.argtypes = [f32p, C.c_int, C.c_int, C.c_int, i32p, f32p]
        L.orc_sort_pairs.restype = C.c_int
        L.orc_sort_pairs.argtypes = [i32p, C.c_int, C.c_int, i32p, i32p]
        L.orc_moe_forward.restype = C.c_int
        L.orc_moe_forward.argtypes = [C.POINTER(u8p), C.c_int, C.c_int, C.c_int, u16p, C.c_int,
                                      i32p, f32p, C.c_int, u16p, C.c_int, f32p, u16p, u16p]
        L.orc_f16_value.restype = C.c_double
        L.orc_f16_value.argtypes = [C.c_uint16]
        L.orc_vq_index.restype = C.c_uint
        L.orc_vq_index.argtypes = [u8p, C.c_uint64]
        L.orc_vq_layout.restype = C.c_int
        L.orc_vq_layout.argtypes = [C.c_int, C.c_int, u64p, u64p, u64p]
        L.orc_vq_pack_record.restype = None
        L.orc_vq_pack_record.argtypes = [C.c_int, C.c_int, C.POINTER(u8p), C.POINTER(u16p), u8p]
        L.orc_vq_dequant_projection.restype = None
        L.orc_vq_dequant_projection.argtypes = [u8p, u8p, C.c_int, C.c_int, C.c_int, f32p]
        L.orc_vq_moe_forward.restype = C.c_int
        L.orc_vq_moe_forward.argtypes = [C.POINTER(u8p), u8p, C.c_int, C.c_int, C.c_int, u16p, C.c_int,
                                         i32p, f32p, C.c_int, u16p, C.c_int, f32p, u16p]
        L.orc_q8_quantize.restype = C.c_int
        L.orc_q8_quantize.argtypes = [u16p, C.c_int, C.c_int, u32p, u16p, u16p]
        L.orc_affine8_linear.restype = C.c_int
        L.orc_affine8_linear.argtypes = [u16p, u32p, u16p, u16p, C.c_int, C.c_int, C.c_int, f32p, u16p]
        L.orc_rmsnorm.restype = None
        L.orc_rmsnorm.argtypes = [u16p, C.c_int, C.c_int, C.c_double, u16p]
        _lib = L
    return _lib


def _p(a, ct):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.POINTER(ct))


# ---- number formats ------------------------------------------------------
def e2m1_value(code):
    return lib().orc_e2m1_value(int(code))


def e4m3_value(byte):
    return lib().orc_e4m3_value(int(byte))


def global_factor(g):
    return lib().orc_global_factor(float(g))


def block_scale(s_byte, g):
    return lib().orc_block_scale(int(s_byte), float(g))


def weight(code, s_byte, g):
    return lib().orc_weight(int(code), int(s_byte), float(g))


def f64_to_bf16(values):
    v = np.asarray(values, dtype=np.float64).ravel()
    f = lib().orc_f64_to_bf16
    return np.array([f(float(a)) for a in v], dtype=np.uint16).reshape(np.shape(values))


def bf16_to_f32(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---- record --------------------------------------------------------------
def record_layout(H, I):
    off = (C.c_uint64 * 9)()
    nb, st = C.c_uint64(), C.c_uint64()
    rc = lib().orc_record_layout(H, I, off, C.byref(nb), C.byref(st))
    if rc != 0:
        raise ValueError("bad shape")
    return [int(o) for o in off], int(nb.value), int(st.value)


def pack_record(H, I, codes, scales, g):
    """codes[p]: uint32 [out][in/8]; scales[p]: uint8 [out][in/16]; g: 3 floats."""
    _, _, stride = record_layout(H, I)
    codes = [np.ascontiguousarray(c, dtype=np.uint32) for c in codes]
    scales = [np.ascontiguousarray(s, dtype=np.uint8) for s in scales]
    cp = (C.POINTER(C.c_uint32) * 3)(*[_p(c, C.c_uint32) for c in codes])
    sp = (C.POINTER(C.c_uint8) * 3)(*[_p(s, C.c_uint8) for s in scales])
    gp = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty(stride, dtype=np.uint8)
    lib().orc_pack_record(H, I, cp, sp, _p(gp, C.c_float), _p(out, C.c_uint8))
    return out


def global_from_ws2(ws2):
    """The stored global g for each f32 weight_scale_2 value ("Beam 1.0 501B-A23B,
    streaming pack, NVFP4 experts / MLX 8-bit residents", "What this pack holds",
    global-scales bullet: the g with f32(g / 2688) equal to weight_scale_2, else
    the nearest g). Returns (g f32, inexact u8).

    Plainly: positive f32 values are ordered like their bit patterns and
    g -> f32(g / 2688) is monotone, so two bisections over the bit patterns find
    lo, the first g whose image is >= ws2, and hi, the first whose image is
    > ws2. The exact solutions are [lo, hi). If there are any, the pick is the one
    nearest to the exact product ws2 * 2688; if there are none, lo - 1 and lo
    (images below and above ws2) compete on the distance of their images to ws2,
    then on the distance to ws2 * 2688. Remaining ties go to the even bit
    pattern. Readings: "nearest" is taken on the image, and the tie rules are ours.
    """
    ws2 = np.ascontiguousarray(ws2, dtype=np.float32).ravel()
    n = ws2.size
    div = np.float32(2688.0)

    def image(bits):
        return (bits.astype(np.uint32).view(np.float32) / div).astype(np.float32)

    def first_at_least(strict):
        lo = np.ones(n, dtype=np.int64)              # smallest positive subnormal
        hi = np.full(n, 0x7F800000, dtype=np.int64)  # +inf: image compares as larger
        while np.any(lo < hi):
            mid = (lo + hi) // 2
            img = image(mid)
            ok = img > ws2 if strict else img >= ws2
            hi = np.where(ok & (lo < hi), mid, hi)
            lo = np.where(~ok & (lo < hi), mid + 1, lo)
        return lo

    lo = first_at_least(False)
    hi = first_at_least(True)
    target = ws2.astype(np.float64) * 2688.0
    g = np.empty(n, dtype=np.float32)
    inexact = np.zeros(n, dtype=np.uint8)
    for i in range(n):
        if hi[i] > lo[i]:
            cands = list(range(int(lo[i]), int(hi[i])))
        else:
            cands = [int(lo[i]) - 1, int(lo[i])]
            inexact[i] = 1
        best = None
        for c in cands:
            gv = np.array([c], dtype=np.uint32).view(np.float32)[0]
            if not np.isfinite(gv) or gv <= 0:
                continue
            err = abs(float(np.float32(gv / div)) - float(ws2[i]))
            dist = abs(float(gv) - float(target[i]))
            key = (err, dist, c & 1)
            if best is None or key < best[0]:
                best = (key, gv)
        g[i] = best[1]
    return g, inexact


def lru_slots(nslots, calls):
    """The expert cache's placement rule, step by step in plain Python: for each
    call (a list of expert ids) the slot of every id and the call's hits and
    misses. A resident id is a hit (also an id placed earlier in the same call);
    a miss takes, among the slots this call does not name, the one used longest
    ago (never-used slots first), the lowest slot on a tie. Returns
    [(slots, hits, misses)] per call. (The pages fix only that the cache is
    bounded and fed on demand; least-recently-used eviction is our reading.)"""
    holder = [None] * nslots       # expert in each slot
    last = [0] * nslots            # call number of each slot's last use
    where = {}
    out = []
    for t, ids in enumerate(calls, start=1):
        named = {where[e] for e in ids if e in where}
        slots, hits, misses = [], 0, 0
        for e in ids:
            if e in where:
                hits += 1
            else:
                free = [s for s in range(nslots) if s not in named]
                s = min(free, key=lambda q: (last[q], q))
                if holder[s] is not None:
                    del where[holder[s]]
                holder[s] = e
                where[e] = s
                named.add(s)
                misses += 1
            slots.append(where[e])
        for s in slots:
            last[s] = t
        out.append((slots, hits, misses))
    return out


def proj_shape(H, I, proj):
    return (H, I) if proj == DOWN else (I, H)


def dequant_projection(record, H, I, proj, want_unit=True):
    rows, cols = proj_shape(H, I, proj)
    rec = np.ascontiguousarray(record, dtype=np.uint8)
    w = np.empty((rows, cols), dtype=np.float32)
    u = np.empty((rows, cols), dtype=np.uint16) if want_unit else None
    lib().orc_dequant_projection(_p(rec, C.c_uint8), H, I, proj, _p(w, C.c_float), _p(u, C.c_uint16))
    return w, u


# ---- routing -------------------------------------------------------------
def router_logits(x_bf16, Wr):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    W = np.ascontiguousarray(Wr, dtype=np.float32)
    T, H = x.shape
    E = W.shape[0]
    assert W.shape[1] == H
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(_p(x, C.c_uint16), _p(W, C.c_float), T, H, E, _p(out, C.c_float))
    return out


def route_topk(logits, k):
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = lib().orc_route_topk(_p(lg, C.c_float), T, E, k, _p(idx, C.c_int32), _p(w, C.c_float))
    if rc != 0:
        raise ValueError("route_topk: bad k or NaN logit")
    return idx, w


def sort_pairs(idx, E):
    ix = np.ascontiguousarray(idx, dtype=np.int32).ravel()
    P = ix.size
    off = np.empty(E + 1, dtype=np.int32)
    srt = np.empty(max(P, 1), dtype=np.int32)
    rc = lib().orc_sort_pairs(_p(ix, C.c_int32), P, E, _p(off, C.c_int32), _p(srt, C.c_int32))
    if rc != 0:
        raise ValueError("sort_pairs: index out of range")
    return off, srt[:P]


# ---- the layer -----------------------------------------------------------
def moe_forward(records, E, H, I, x_bf16, idx, w, residual=None, acc=ACC_F64, want_mid=False):
    """records: dict or list mapping expert id -> uint8 record array (stride bytes)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T = x.shape[0]
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    wv = np.ascontiguousarray(w, dtype=np.float32)
    k = ix.shape[1]
    keep = []
    ptrs = (C.POINTER(C.c_uint8) * E)()
    items = records.items() if isinstance(records, dict) else enumerate(records)
    for e, r in items:
        if r is None:
            continue
        r = np.ascontiguousarray(r, dtype=np.uint8)
        keep.append(r)
        ptrs[int(e)] = _p(r, C.c_uint8)
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.uint16)
    yf = np.empty((T, H), dtype=np.float32)
    yb = np.empty((T, H), dtype=np.uint16)
    mid = np.empty((T * k, I), dtype=np.uint16) if want_mid else None
    rc = lib().orc_moe_forward(ptrs, E, H, I, _p(x, C.c_uint16), T, _p(ix, C.c_int32),
                               _p(wv, C.c_float), k, _p(res, C.c_uint16), acc,
                               _p(yf, C.c_float), _p(yb, C.c_uint16), _p(mid, C.c_uint16))
    if rc != 0:
        raise ValueError("moe_forward: bad argument or missing record")
    return (yf, yb, mid) if want_mid else (yf, yb)


# ---- 8-dim VQ experts ([VQ] "Recipe", routed-experts bullet) -----------------
def f16_value(bits):
    return lib().orc_f16_value(int(bits))


def vq_index(row_bytes, j):
    r = np.ascontiguousarray(row_bytes, dtype=np.uint8)
    return lib().orc_vq_index(_p(r, C.c_uint8), j)


def vq_layout(H, I):
    off = (C.c_uint64 * 6)()
    nb, st = C.c_uint64(), C.c_uint64()
    if lib().orc_vq_layout(H, I, off, C.byref(nb), C.byref(st)) != 0:
        raise ValueError("bad shape")
    return [int(o) for o in off], int(nb.value), int(st.value)


def vq_pack_record(H, I, idx, gains):
    """idx[p]: uint8 packed index rows [out][in*3/16]; gains[p]: f16 bits [out]."""
    _, _, stride = vq_layout(H, I)
    idx = [np.ascontiguousarray(a, dtype=np.uint8) for a in idx]
    gains = [np.ascontiguousarray(g, dtype=np.uint16) for g in gains]
    ip = (C.POINTER(C.c_uint8) * 3)(*[_p(a, C.c_uint8) for a in idx])
    gp = (C.POINTER(C.c_uint16) * 3)(*[_p(g, C.c_uint16) for g in gains])
    out = np.empty(stride, dtype=np.uint8)
    lib().orc_vq_pack_record(H, I, ip, gp, _p(out, C.c_uint8))
    return out


def vq_dequant_projection(record, codebook, H, I, proj):
    out, inn = proj_shape(H, I, proj)
    w = np.empty((out, inn), dtype=np.float32)
    r = np.ascontiguousarray(record, dtype=np.uint8)
    cb = np.ascontiguousarray(codebook, dtype=np.uint8).ravel()
    lib().orc_vq_dequant_projection(_p(r, C.c_uint8), _p(cb, C.c_uint8), H, I, proj, _p(w, C.c_float))
    return w


def vq_moe_forward(records, codebook, E, H, I, x_bf16, idx, w, residual=None, acc=ACC_F64):
    """moe_forward over VQ records (dict or list expert -> record bytes)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T = x.shape[0]
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    wv = np.ascontiguousarray(w, dtype=np.float32)
    k = ix.shape[1]
    keep = []
    ptrs = (C.POINTER(C.c_uint8) * E)()
    items = records.items() if isinstance(records, dict) else enumerate(records)
    for e, r in items:
        if r is None:
            continue
        r = np.ascontiguousarray(r, dtype=np.uint8)
        keep.append(r)
        ptrs[int(e)] = _p(r, C.c_uint8)
    cb = np.ascontiguousarray(codebook, dtype=np.uint8).ravel()
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.uint16)
    yf = np.empty((T, H), dtype=np.float32)
    yb = np.empty((T, H), dtype=np.uint16)
    rc = lib().orc_vq_moe_forward(ptrs, _p(cb, C.c_uint8), E, H, I, _p(x, C.c_uint16), T, _p(ix, C.c_int32),
                                  _p(wv, C.c_float), k, _p(res, C.c_uint16), acc, _p(yf, C.c_float),
                                  _p(yb, C.c_uint16))
    if rc != 0:
        raise ValueError("vq_moe_forward: bad argument or missing record")
    return yf, yb


# ---- residents -----------------------------------------------------------
def q8_quantize(v_bf16):
    v = np.ascontiguousarray(v_bf16, dtype=np.uint16)
    N, K = v.shape
    codes = np.zeros((N, K // 4), dtype=np.uint32)
    scales = np.empty((N, K // 64), dtype=np.uint16)
    biases = np.empty((N, K // 64), dtype=np.uint16)
    rc = lib().orc_q8_quantize(_p(v, C.c_uint16), N, K, _p(codes, C.c_uint32),
                               _p(scales, C.c_uint16), _p(biases, C.c_uint16))
    if rc != 0:
        raise ValueError("q8_quantize: bad shape")
    return codes, scales, biases


def affine8_linear(x_bf16, codes, scales, biases):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T, K = x.shape
    cd = np.ascontiguousarray(codes, dtype=np.uint32)
    N = cd.shape[0]
    sc = np.ascontiguousarray(scales, dtype=np.uint16)
    bi = np.ascontiguousarray(biases, dtype=np.uint16)
    yf = np.empty((T, N), dtype=np.float32)
    yb = np.empty((T, N), dtype=np.uint16)
    rc = lib().orc_affine8_linear(_p(x, C.c_uint16), _p(cd, C.c_uint32), _p(sc, C.c_uint16),
                                  _p(bi, C.c_uint16), T, K, N, _p(yf, C.c_float), _p(yb, C.c_uint16))
    if rc != 0:
        raise ValueError("affine8_linear: bad shape")
    return yf, yb


def rmsnorm(x_bf16, eps=1e-6):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T, H = x.shape
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x, C.c_uint16), T, H, float(eps), _p(y, C.c_uint16))
    return y
