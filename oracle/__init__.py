"""Plain fp64 CPU oracle for the CSA / HCA attention path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of bench.py, never by the product path.  It shares no code
with the HIP library and never imports it.

Each wrapper converts numpy arrays to the C calls in oracle.c; the arithmetic
and the readings of the pages are documented there.
"""
import ctypes as C
import os

import numpy as np

from .build import build_oracle, LIB_PATH

F32, BF16, FP8_E4M3, FP4_E2M1 = 0, 1, 2, 3

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build_oracle()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


class AttnParams(C.Structure):
    _fields_ = [("d", C.c_int), ("dr", C.c_int), ("window", C.c_int), ("m", C.c_int),
                ("base", C.c_double), ("scale", C.c_double), ("eps", C.c_double)]


_P = C.c_void_p


def _declare(L):
    L.orc_bf16_encode.restype = C.c_uint16
    L.orc_bf16_encode.argtypes = [C.c_float]
    L.orc_bf16_decode.restype = C.c_double
    L.orc_bf16_decode.argtypes = [C.c_uint16]
    L.orc_e4m3_encode.restype = C.c_uint8
    L.orc_e4m3_encode.argtypes = [C.c_float]
    L.orc_e4m3_decode.restype = C.c_double
    L.orc_e4m3_decode.argtypes = [C.c_uint8]
    L.orc_e2m1_encode.restype = C.c_uint8
    L.orc_e2m1_encode.argtypes = [C.c_float]
    L.orc_e2m1_decode.restype = C.c_double
    L.orc_e2m1_decode.argtypes = [C.c_uint8]
    L.orc_e8m0_decode.restype = C.c_double
    L.orc_e8m0_decode.argtypes = [C.c_uint8]
    L.orc_fp4_quant_row.restype = None
    L.orc_fp4_quant_row.argtypes = [_P, C.c_int, _P, _P]
    L.orc_kv_record_bytes.restype = C.c_int
    L.orc_kv_record_bytes.argtypes = [C.c_int, C.c_int, C.c_int]
    for name in ("orc_bf16_encode_n", "orc_e4m3_encode_n", "orc_e2m1_encode_n",
                 "orc_bf16_decode_n", "orc_e4m3_decode_n"):
        getattr(L, name).restype = None
        getattr(L, name).argtypes = [_P, C.c_long, _P]
    L.orc_kv_encode_n.argtypes = [_P, C.c_long, C.c_int, C.c_int, C.c_int, _P]
    L.orc_kv_encode_n.restype = None
    L.orc_kv_decode_n.argtypes = [_P, C.c_long, C.c_int, C.c_int, C.c_int, _P]
    L.orc_kv_decode_n.restype = None
    L.orc_idx_encode_n.argtypes = [_P, C.c_long, C.c_int, C.c_int, _P, _P]
    L.orc_idx_encode_n.restype = None
    L.orc_idx_decode_n.argtypes = [_P, _P, C.c_long, C.c_int, C.c_int, _P]
    L.orc_idx_decode_n.restype = None
    L.orc_pool.restype = None
    L.orc_pool.argtypes = [_P, C.c_int, C.c_int, _P, _P, _P, _P]
    L.orc_rmsnorm.restype = None
    L.orc_rmsnorm.argtypes = [_P, C.c_int, _P, C.c_double, _P]
    L.orc_rope.restype = None
    L.orc_rope.argtypes = [_P, C.c_int, C.c_int, C.c_double, C.c_double]
    L.orc_compress.restype = C.c_long
    L.orc_compress.argtypes = [_P, C.c_int, C.c_int, C.c_long, C.c_int, _P, C.c_int, _P, _P, _P,
                               C.c_float, C.c_int, C.c_float, C.c_int, C.c_int, _P, _P, C.c_long,
                               C.c_int, _P]
    L.orc_indexer_scores.restype = None
    L.orc_indexer_scores.argtypes = [_P, _P, C.c_int, C.c_int, _P, C.c_long, _P]
    L.orc_topk.restype = C.c_int
    L.orc_topk.argtypes = [_P, C.c_long, C.c_int, _P]
    L.orc_indexer_topk.restype = None
    L.orc_indexer_topk.argtypes = [_P, _P, C.c_int, _P, _P, C.c_int, C.c_int, C.c_int, _P, _P,
                                   C.c_int, C.c_long, C.c_int, C.c_int, _P, _P]
    L.orc_attention.restype = C.c_long
    L.orc_attention.argtypes = [_P, C.c_int, _P, C.c_int, C.c_int, _P, _P, C.POINTER(AttnParams),
                                _P, C.c_int, C.c_long, _P, C.c_int, C.c_long, _P, C.c_int, _P, _P, _P]
    L.orc_out_proj.restype = None
    L.orc_out_proj.argtypes = [_P, _P, C.c_long, C.c_int, C.c_int, C.c_int, _P]
    L.orc_fp8_rows_quant.restype = None
    L.orc_fp8_rows_quant.argtypes = [_P, C.c_long, C.c_int, _P, _P]
    L.orc_linear_fp8.restype = None
    L.orc_linear_fp8.argtypes = [_P, C.c_long, C.c_int, _P, _P, C.c_int, C.c_int, _P]


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats
def bf16_encode(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_encode_n(_p(x), x.size, _p(out))
    return out


def bf16_decode(b):
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().orc_bf16_decode_n(_p(b), b.size, _p(out))
    return out


def e4m3_encode(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_encode_n(_p(x), x.size, _p(out))
    return out


def e4m3_decode(c):
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3_decode_n(_p(c), c.size, _p(out))
    return out


def e2m1_encode(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e2m1_encode_n(_p(x), x.size, _p(out))
    return out


def e2m1_decode(c):
    return np.array([lib().orc_e2m1_decode(int(v)) for v in np.asarray(c).ravel()]).reshape(np.shape(c))


def kv_record_bytes(fmt, d, dr):
    return lib().orc_kv_record_bytes(fmt, d, dr)


def idx_row_bytes(fmt, di):
    return {F32: 4 * di, BF16: 2 * di, FP4_E2M1: di // 2}[fmt]


def kv_encode(v, fmt, dr):
    """v [..., d] -> uint8 records [..., rec_bytes]."""
    v = _c(v, np.float64)
    d = v.shape[-1]
    n = v.size // d
    rb = kv_record_bytes(fmt, d, dr)
    out = np.zeros(v.shape[:-1] + (rb,), np.uint8)
    lib().orc_kv_encode_n(_p(v), n, fmt, d, dr, _p(out))
    return out


def kv_decode(recs, fmt, d, dr):
    recs = _c(recs, np.uint8)
    n = recs.size // kv_record_bytes(fmt, d, dr)
    out = np.empty(recs.shape[:-1] + (d,), np.float64)
    lib().orc_kv_decode_n(_p(recs), n, fmt, d, dr, _p(out))
    return out


def idx_encode(v, fmt):
    """v [..., di] -> (codes uint8 [..., row_bytes], scales uint8 [..., di/32] or None)."""
    v = _c(v, np.float64)
    di = v.shape[-1]
    n = v.size // di
    codes = np.zeros(v.shape[:-1] + (idx_row_bytes(fmt, di),), np.uint8)
    scales = np.zeros(v.shape[:-1] + (di // 32,), np.uint8) if fmt == FP4_E2M1 else None
    lib().orc_idx_encode_n(_p(v), n, fmt, di, _p(codes), _p(scales))
    return codes, scales


def idx_decode(codes, scales, fmt, di):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n = codes.size // idx_row_bytes(fmt, di)
    out = np.empty(codes.shape[:-1] + (di,), np.float64)
    lib().orc_idx_decode_n(_p(codes), _p(scales), n, fmt, di, _p(out))
    return out


def fp4_quant_row(x):
    x = _c(x, np.float32)
    n = x.shape[-1]
    codes = np.zeros(n // 2, np.uint8)
    scales = np.zeros(n // 32, np.uint8)
    lib().orc_fp4_quant_row(_p(x), n, _p(codes), _p(scales))
    return codes, scales


# ---------------------------------------------------------- building blocks
def pool(x, b, u=None):
    x = _c(x, np.float64)
    m, d = x.shape
    b = _c(b, np.float64)
    u = _c(u, np.float64)
    c = np.empty(d)
    pi = np.empty(m)
    lib().orc_pool(_p(x), m, d, _p(b), _p(u), _p(c), _p(pi))
    return c, pi


def rmsnorm(v, gamma=None, eps=1e-6):
    v = _c(v, np.float64)
    g = _c(gamma, np.float64)
    out = np.empty_like(v)
    lib().orc_rmsnorm(_p(v), v.shape[-1], _p(g), eps, _p(out))
    return out


def rope(v, dr, pos, base=10000.0):
    v = np.array(v, dtype=np.float64, copy=True)
    lib().orc_rope(_p(v), v.shape[-1], dr, float(pos), float(base))
    return v


# ---------------------------------------------------------------- the calls
def compress(x, x_fmt, tok_start, m, b, u=None, gamma=None, eps=1e-6, dr=0, base=10000.0,
             out_kind=0, out_fmt=FP8_E4M3, cap=None, ring=False, want_pre=False):
    """x: [B][T][d] float32 (x_fmt F32) or uint16 bf16 bits (x_fmt BF16).
    Returns (codes, scales, pre_quant): codes [B][cap][rec] uint8."""
    x = _c(x, np.float32 if x_fmt == F32 else np.uint16)
    B, T, d = x.shape
    ts = _c(tok_start, np.int32)
    rb = kv_record_bytes(out_fmt, d, dr) if out_kind == 0 else idx_row_bytes(out_fmt, d)
    codes = np.zeros((B, cap, rb), np.uint8)
    scales = np.zeros((B, cap, d // 32), np.uint8) if (out_kind == 1 and out_fmt == FP4_E2M1) else None
    pre = np.full((B, cap, d), np.nan) if want_pre else None
    bb = _c(b, np.float32)
    uu = _c(u, np.float32)
    gg = _c(gamma, np.float32)
    lib().orc_compress(_p(x), x_fmt, B, T, d, _p(ts), m, _p(bb), _p(uu), _p(gg), eps, dr, base,
                       out_kind, out_fmt, _p(codes), _p(scales), cap, 1 if ring else 0, _p(pre))
    return codes, scales, pre


def indexer_scores(qI, w, keys):
    qI = _c(qI, np.float64)
    w = _c(w, np.float64)
    keys = _c(keys, np.float64)
    Hi, di = qI.shape
    S = np.empty(keys.shape[0])
    lib().orc_indexer_scores(_p(qI), _p(w), Hi, di, _p(keys), keys.shape[0], _p(S))
    return S


def topk(S, k):
    S = _c(S, np.float64)
    out = np.empty(k, np.int32)
    lib().orc_topk(_p(S), S.size, k, _p(out))
    return out


def indexer_topk(qI, qI_scales, q_fmt, w, q_pos, keys, key_scales, key_fmt, m, k,
                 want_scores=False):
    """One sequence.  qI [Tq][Hi][row] codes, w [Tq][Hi] f32, q_pos [Tq] int32,
    keys [cap][row] codes (+ scales).  Returns out [Tq][k] int32 (and scores)."""
    qI = _c(qI, np.uint8)
    qs = _c(qI_scales, np.uint8)
    w = _c(w, np.float32)
    q_pos = _c(q_pos, np.int32)
    keys = _c(keys, np.uint8)
    ks = _c(key_scales, np.uint8)
    Tq, Hi = w.shape
    cap = keys.shape[0]
    di = {F32: keys.shape[1] // 4, BF16: keys.shape[1] // 2, FP4_E2M1: keys.shape[1] * 2}[key_fmt]
    out = np.empty((Tq, k), np.int32)
    sc = np.full((Tq, cap), np.nan) if want_scores else None
    lib().orc_indexer_topk(_p(qI), _p(qs), q_fmt, _p(w), _p(q_pos), Tq, Hi, di, _p(keys), _p(ks),
                           key_fmt, cap, m, k, _p(out), _p(sc))
    return (out, sc) if want_scores else out


def attention(q, q_fmt, q_pos, gamma_q, sink, d, dr, window, m, base, scale, eps,
              comp, comp_fmt, win, win_fmt, topk_idx=None, want_p=False):
    """One sequence.  q [Tq][H][d] (float32 or bf16 bits); comp [cap][rec];
    win [wcap][rec]; topk_idx [Tq][k] or None (dense).  Returns out [Tq][H][d]
    fp64 (and the weights of query 0 / head 0 plus its sink weight)."""
    q = _c(q, np.float32 if q_fmt == F32 else np.uint16)
    Tq, H, _ = q.shape
    q_pos = _c(q_pos, np.int32)
    g = _c(gamma_q, np.float32)
    sink = _c(sink, np.float32)
    comp = _c(comp, np.uint8)
    win = _c(win, np.uint8)
    tk = _c(topk_idx, np.int32)
    k = 0 if tk is None else tk.shape[1]
    P = AttnParams(d, dr, window, m, base, scale, eps)
    out = np.empty((Tq, H, d))
    maxn = (k if tk is not None else comp.shape[0]) + window + 1
    p = np.empty(maxn) if want_p else None
    ps = np.empty(1) if want_p else None
    n = lib().orc_attention(_p(q), q_fmt, _p(q_pos), Tq, H, _p(g), _p(sink), C.byref(P), _p(comp),
                            comp_fmt, comp.shape[0], _p(win), win_fmt, win.shape[0], _p(tk), k,
                            _p(out), _p(p), _p(ps))
    if want_p:
        return out, p[:n] if Tq == 1 else p, ps[0]
    return out


def out_proj(o, W):
    """o [M][Hd] fp64, W [G][D/G][Hd/G] -> y [M][D]."""
    o = _c(o, np.float64)
    W = _c(W, np.float64)
    M, Hd = o.shape
    G, dg, cg = W.shape
    y = np.empty((M, G * dg))
    lib().orc_out_proj(_p(o), _p(W), M, Hd, G * dg, G, _p(y))
    return y


# ---------------------------------------------------------- FP8-weight projections
def fp8_rows_quant(W):
    """W [N][K] float -> (codes [N][K] uint8, scale [N] float32): per-row E4M3
    weights (weight preparation for tests, not a step of the path)."""
    W = _c(W, np.float32)
    N, K = W.shape
    codes = np.empty((N, K), np.uint8)
    scale = np.empty(N, np.float32)
    lib().orc_fp8_rows_quant(_p(W), N, K, _p(codes), _p(scale))
    return codes, scale


def linear_fp8(x, W, scale, G=1):
    """x [M][K] fp64 values, W [N][K/G] E4M3 codes, scale [N] -> y [M][N] fp64."""
    x = _c(x, np.float64)
    W = _c(W, np.uint8)
    scale = _c(scale, np.float32)
    M, K = x.shape
    N = W.shape[0]
    assert W.shape[1] * G == K and N % G == 0 and scale.shape == (N,)
    y = np.empty((M, N))
    lib().orc_linear_fp8(_p(x), M, K, _p(W), _p(scale), N, G, _p(y))
    return y


def layer_in_proj(h, Wq, sq, Wkv, skv, WkI, skI, WqI, sqI, Ww, sw, Hi):
    """The input projections of one layer from hidden states h [M][D] (values):
    q = h Wq^T, kv = h Wkv^T (the raw KV token), kI = h WkI^T (the raw indexer
    key), qI = h WqI^T, w = h Ww^T, every weight FP8 with per-row scales.
    Roundings of the outputs (the formats the next steps take): the projected
    value as an fp32 number, then q, kv, kI to bf16 (nearest even), w kept in
    fp32, qI quantised to FP4 per head row of di values by the indexer-key
    rule of fp4_quant_row.  Returns (q bf16 bits, kv bits, kI bits, qI codes
    [M][Hi][di/2], qI scales [M][Hi][di/32], w float32 [M][Hi])."""
    f32 = lambda W, s: linear_fp8(h, W, s).astype(np.float32)
    q, kv, kI = (bf16_encode(f32(W, s)) for W, s in ((Wq, sq), (Wkv, skv), (WkI, skI)))
    w = f32(Ww, sw)
    qI = f32(WqI, sqI)
    M = qI.shape[0]
    di = qI.shape[1] // Hi
    codes = np.empty((M, Hi, di // 2), np.uint8)
    scales = np.empty((M, Hi, di // 32), np.uint8)
    for r in range(M):
        for hh in range(Hi):
            codes[r, hh], scales[r, hh] = fp4_quant_row(qI[r, hh * di:(hh + 1) * di])
    return q, kv, kI, codes, scales, w
