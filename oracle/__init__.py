"""numpy front-end of the plain C oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding.
Every function here only marshals numpy arrays into the C routines declared
in oracle.h; all arithmetic is in oracle.c.

All arrays are C-contiguous numpy arrays: E4M3 codes as uint8, scales as
float32, bf16 values as uint16 bit patterns, indices as int32, results as
float64 (unrounded).
"""
import ctypes as _ct
import os as _os

import numpy as _np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _os.path.exists(_build.LIB):
        _build.build()
    lib = _ct.CDLL(_build.LIB)
    P = _ct.c_void_p
    I = _ct.c_int
    L = _ct.c_int64
    D = _ct.c_double
    sig = {
        "orc_e4m3_table": (None, [P]),
        "orc_e4m3_encode": (_ct.c_uint8, [_ct.c_float]),
        "orc_e4m3_encode_array": (None, [P, L, P]),
        "orc_block_scale": (_ct.c_float, [_ct.c_float]),
        "orc_quantize_1x128": (None, [P, I, I, I, P, P, I]),
        "orc_quantize_128x128": (None, [P, I, I, I, P, P]),
        "orc_block_scale_ue8m0": (_ct.c_float, [_ct.c_float]),
        "orc_quantize_1x128_ue8m0": (None, [P, I, I, I, P, P, I]),
        "orc_quantize_128x128_ue8m0": (None, [P, I, I, I, P, P]),
        "orc_bf16_to_double": (D, [_ct.c_uint16]),
        "orc_gemm_nt_elem": (D, [P, P, I, P, P, P, I, I, I, I, I]),
        "orc_gemm_nt": (None, [P, P, I, P, P, P, P, I, I, I]),
        "orc_gemm_nt_at": (None, [P, P, I, P, P, P, I, I, I, P, P, L, P]),
        "orc_block_dot": (D, [P, P]),
        "orc_m_grouped_contiguous": (None, [P, P, P, P, P, P, P, I, I, I, I]),
        "orc_m_grouped_contiguous_at": (None, [P, P, P, P, P, P, I, I, I, I, P, P, L, P]),
        "orc_m_grouped_masked": (None, [P, P, P, P, P, P, P, I, I, I, I]),
        "orc_m_grouped_masked_at": (None, [P, P, P, P, P, P, I, I, I, I, P, P, P, L, P]),
        "orc_k_grouped_tn": (None, [P, P, P, P, P, P, I, I, I, P]),
        "orc_k_grouped_tn_at": (None, [P, P, P, P, P, P, I, I, I, P, P, P, L, P]),
        "orc_mqa_logits": (None, [P, P, P, P, P, P, I, I, I, I, I, P]),
        "orc_mqa_logits_rows": (None, [P, P, P, P, P, P, I, I, I, I, P, I, P]),
        "orc_ue8m0_encode": (_ct.c_uint8, [_ct.c_float]),
        "orc_ue8m0_decode": (D, [_ct.c_uint8]),
        "orc_pack_ue8m0": (None, [P, I, I, I, P]),
        "orc_unpack_ue8m0": (None, [P, I, I, I, P]),
        "orc_num_threads": (I, []),
        "orc_set_num_threads": (None, [I]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(arr, dtype):
    if arr is None:
        return None
    assert isinstance(arr, _np.ndarray), type(arr)
    assert arr.dtype == dtype, (arr.dtype, dtype)
    assert arr.flags["C_CONTIGUOUS"]
    return arr.ctypes.data


def e4m3_table():
    out = _np.empty(256, dtype=_np.float64)
    _load().orc_e4m3_table(out.ctypes.data)
    return out


def e4m3_encode(x):
    x = _np.ascontiguousarray(x, dtype=_np.float32)
    q = _np.empty(x.shape, dtype=_np.uint8)
    _load().orc_e4m3_encode_array(x.ctypes.data, x.size, q.ctypes.data)
    return q


def block_scale(amax):
    return _np.float32(_load().orc_block_scale(float(amax)))


def sf_aligned(mn):
    return (mn + 3) // 4 * 4


def block_scale_ue8m0(amax):
    return _np.float32(_load().orc_block_scale_ue8m0(float(amax)))


def quantize_1x128(x, ld_sf=None, ue8m0=False):
    """x[groups, rows, K] (or [rows, K]) fp32 -> (q uint8 same shape, sf[groups, K/128, ld_sf]).
    ue8m0: power-of-two scales (the block scale rounded up to a power of two)."""
    x = _np.ascontiguousarray(x, dtype=_np.float32)
    squeeze = x.ndim == 2
    x3 = x[None] if squeeze else x
    groups, rows, K = x3.shape
    assert K % 128 == 0
    ld = sf_aligned(rows) if ld_sf is None else ld_sf
    q = _np.empty(x3.shape, dtype=_np.uint8)
    sf = _np.zeros((groups, K // 128, ld), dtype=_np.float32)
    f = _load().orc_quantize_1x128_ue8m0 if ue8m0 else _load().orc_quantize_1x128
    f(x3.ctypes.data, groups, rows, K, q.ctypes.data, sf.ctypes.data, ld)
    if squeeze:
        return q[0], sf[0]
    return q, sf


def quantize_128x128(x, ue8m0=False):
    """x[groups, rows, K] (or [rows, K]) -> (q, sf[groups, ceil(rows/128), K/128]).
    ue8m0: power-of-two scales."""
    x = _np.ascontiguousarray(x, dtype=_np.float32)
    squeeze = x.ndim == 2
    x3 = x[None] if squeeze else x
    groups, rows, K = x3.shape
    assert K % 128 == 0
    q = _np.empty(x3.shape, dtype=_np.uint8)
    sf = _np.empty((groups, (rows + 127) // 128, K // 128), dtype=_np.float32)
    f = _load().orc_quantize_128x128_ue8m0 if ue8m0 else _load().orc_quantize_128x128
    f(x3.ctypes.data, groups, rows, K, q.ctypes.data, sf.ctypes.data)
    if squeeze:
        return q[0], sf[0]
    return q, sf


def bf16_to_double(h):
    return _load().orc_bf16_to_double(int(h))


def block_dot(arow, brow):
    return _load().orc_block_dot(_p(arow, _np.uint8), _p(brow, _np.uint8))


def gemm_nt(a, sfa, b, sfb, c=None):
    """Dense D = C + A.B^T with block scales. a[M,K], sfa[K/128, ld], b[N,K], sfb[ceil(N/128), K/128]."""
    M, K = a.shape
    N = b.shape[0]
    d = _np.full((M, N), _np.nan, dtype=_np.float64)
    _load().orc_gemm_nt(_p(a, _np.uint8), _p(sfa, _np.float32), sfa.shape[-1],
                        _p(b, _np.uint8), _p(sfb, _np.float32), _p(c, _np.uint16),
                        d.ctypes.data, M, N, K)
    return d


def gemm_nt_elem(a, sfa, b, sfb, c, m, n):
    M, K = a.shape
    N = b.shape[0]
    return _load().orc_gemm_nt_elem(_p(a, _np.uint8), _p(sfa, _np.float32), sfa.shape[-1],
                                    _p(b, _np.uint8), _p(sfb, _np.float32), _p(c, _np.uint16),
                                    M, N, K, int(m), int(n))


def gemm_nt_at(a, sfa, b, sfb, c, ms, ns):
    M, K = a.shape
    N = b.shape[0]
    ms = _np.ascontiguousarray(ms, dtype=_np.int32)
    ns = _np.ascontiguousarray(ns, dtype=_np.int32)
    out = _np.empty(ms.size, dtype=_np.float64)
    _load().orc_gemm_nt_at(_p(a, _np.uint8), _p(sfa, _np.float32), sfa.shape[-1],
                           _p(b, _np.uint8), _p(sfb, _np.float32), _p(c, _np.uint16),
                           M, N, K, ms.ctypes.data, ns.ctypes.data, ms.size, out.ctypes.data)
    return out


def _logical(layout, a, b):
    """The stored operands of layout nt/nn/tn/tt as the logical A[M,K] and B[N,K]
    (GeekNews summary of the DeepGEMM README, layout section: the first letter
    tells whether A is stored as is ("n", [M,K]) or transposed ("t", [K,M]); the
    second whether B is stored transposed ("t", [N,K]) or as is ("n", [K,N]))."""
    if layout not in ("nt", "nn", "tn", "tt"):
        raise ValueError(layout)
    a_l = _np.ascontiguousarray(a if layout[0] == "n" else _np.asarray(a).T)
    b_l = _np.ascontiguousarray(b if layout[1] == "t" else _np.asarray(b).T)
    return a_l, b_l


def gemm_layout(layout, a, sfa, b, sfb, c=None):
    """D = C + A @ B for a stored layout: the NT definition on the logical operands."""
    a_l, b_l = _logical(layout, a, b)
    return gemm_nt(a_l, sfa, b_l, sfb, c)


def gemm_layout_at(layout, a, sfa, b, sfb, c, ms, ns):
    a_l, b_l = _logical(layout, a, b)
    return gemm_nt_at(a_l, sfa, b_l, sfb, c, ms, ns)


def m_grouped_contiguous(a, sfa, b, sfb, c, m_indices, d=None):
    """a[M_total,K], sfa[K/128, M_total], b[G,N,K], sfb[G, ceil(N/128), K/128], m_indices[M_total]."""
    M_total, K = a.shape
    G, N, _ = b.shape
    if d is None:
        d = _np.full((M_total, N), _np.nan, dtype=_np.float64)
    assert sfa.shape[-1] == M_total
    _load().orc_m_grouped_contiguous(_p(a, _np.uint8), _p(sfa, _np.float32), _p(b, _np.uint8),
                                     _p(sfb, _np.float32), _p(c, _np.uint16),
                                     _p(m_indices, _np.int32), _p(d, _np.float64),
                                     M_total, N, K, G)
    return d


def m_grouped_contiguous_at(a, sfa, b, sfb, c, m_indices, ms, ns):
    M_total, K = a.shape
    G, N, _ = b.shape
    ms = _np.ascontiguousarray(ms, dtype=_np.int32)
    ns = _np.ascontiguousarray(ns, dtype=_np.int32)
    out = _np.empty(ms.size, dtype=_np.float64)
    _load().orc_m_grouped_contiguous_at(_p(a, _np.uint8), _p(sfa, _np.float32), _p(b, _np.uint8),
                                        _p(sfb, _np.float32), _p(c, _np.uint16),
                                        _p(m_indices, _np.int32), M_total, N, K, G,
                                        ms.ctypes.data, ns.ctypes.data, ms.size, out.ctypes.data)
    return out


def m_grouped_masked(a, sfa, b, sfb, c, masked_m, d=None):
    """a[G,M_cap,K], sfa[G, K/128, round_up(M_cap,4)], b[G,N,K], sfb[G, ceil(N/128), K/128], masked_m[G]."""
    G, M_cap, K = a.shape
    N = b.shape[1]
    if d is None:
        d = _np.full((G, M_cap, N), _np.nan, dtype=_np.float64)
    assert sfa.shape[-1] == sf_aligned(M_cap)
    _load().orc_m_grouped_masked(_p(a, _np.uint8), _p(sfa, _np.float32), _p(b, _np.uint8),
                                 _p(sfb, _np.float32), _p(c, _np.uint16),
                                 _p(masked_m, _np.int32), _p(d, _np.float64), G, M_cap, N, K)
    return d


def m_grouped_masked_at(a, sfa, b, sfb, c, masked_m, gs, ms, ns):
    G, M_cap, K = a.shape
    N = b.shape[1]
    gs = _np.ascontiguousarray(gs, dtype=_np.int32)
    ms = _np.ascontiguousarray(ms, dtype=_np.int32)
    ns = _np.ascontiguousarray(ns, dtype=_np.int32)
    out = _np.empty(ms.size, dtype=_np.float64)
    _load().orc_m_grouped_masked_at(_p(a, _np.uint8), _p(sfa, _np.float32), _p(b, _np.uint8),
                                    _p(sfb, _np.float32), _p(c, _np.uint16),
                                    _p(masked_m, _np.int32), G, M_cap, N, K,
                                    gs.ctypes.data, ms.ctypes.data, ns.ctypes.data, ms.size,
                                    out.ctypes.data)
    return out


def _kg_args(a, sfa, b, sfb, ks, c):
    a = _np.ascontiguousarray(a, dtype=_np.uint8)
    b = _np.ascontiguousarray(b, dtype=_np.uint8)
    sfa = _np.ascontiguousarray(sfa, dtype=_np.float32)
    sfb = _np.ascontiguousarray(sfb, dtype=_np.float32)
    ks = _np.ascontiguousarray(ks, dtype=_np.int32)
    K, M = a.shape
    N = b.shape[1]
    assert b.shape[0] == K and sfa.shape == (K // 128, M) and sfb.shape == (K // 128, N)
    assert int(ks.sum()) <= K and _np.all(ks >= 0) and _np.all(ks % 128 == 0)
    G = ks.size
    cp = None
    if c is not None:
        c = _np.ascontiguousarray(c, dtype=_np.float32)
        assert c.shape == (G, M, N)
        cp = c.ctypes.data
    return a, sfa, b, sfb, ks, c, cp, G, M, N


def k_grouped_tn(a, sfa, b, sfb, ks, c=None):
    """K-grouped TN contiguous GEMM: a[K,M], b[K,N] E4M3, sfa[K/128,M], sfb[K/128,N],
    ks[G] group sizes (multiples of 128), c[G,M,N] fp32 or None -> d[G,M,N] fp64."""
    a, sfa, b, sfb, ks, c, cp, G, M, N = _kg_args(a, sfa, b, sfb, ks, c)
    d = _np.full((G, M, N), _np.nan, dtype=_np.float64)
    _load().orc_k_grouped_tn(a.ctypes.data, sfa.ctypes.data, b.ctypes.data, sfb.ctypes.data, ks.ctypes.data, cp,
                             G, M, N, d.ctypes.data)
    return d


def k_grouped_tn_at(a, sfa, b, sfb, ks, c, gs, ms, ns):
    a, sfa, b, sfb, ks, c, cp, G, M, N = _kg_args(a, sfa, b, sfb, ks, c)
    gs = _np.ascontiguousarray(gs, dtype=_np.int32)
    ms = _np.ascontiguousarray(ms, dtype=_np.int32)
    ns = _np.ascontiguousarray(ns, dtype=_np.int32)
    out = _np.empty(gs.size, dtype=_np.float64)
    _load().orc_k_grouped_tn_at(a.ctypes.data, sfa.ctypes.data, b.ctypes.data, sfb.ctypes.data, ks.ctypes.data, cp,
                                G, M, N, gs.ctypes.data, ms.ctypes.data, ns.ctypes.data, gs.size, out.ctypes.data)
    return out


def _mqa_args(q, kv, kv_scale, weights, k_start, k_end):
    q = _np.ascontiguousarray(q, dtype=_np.uint8)
    kv = _np.ascontiguousarray(kv, dtype=_np.uint8)
    kv_scale = _np.ascontiguousarray(kv_scale, dtype=_np.float32)
    weights = _np.ascontiguousarray(weights, dtype=_np.float32)
    k_start = _np.ascontiguousarray(k_start, dtype=_np.int32)
    k_end = _np.ascontiguousarray(k_end, dtype=_np.int32)
    S, H, D = q.shape
    Skv = kv.shape[0]
    assert kv.shape == (Skv, D) and kv_scale.shape == (Skv,) and weights.shape == (S, H)
    assert k_start.shape == (S,) and k_end.shape == (S,)
    return q, kv, kv_scale, weights, k_start, k_end, S, H, D, Skv


def mqa_logits(q, kv, kv_scale, weights, k_start, k_end, clean_logits):
    """FP8 MQA logits [S, Skv] in fp64; positions left untouched are NaN."""
    q, kv, kv_scale, weights, k_start, k_end, S, H, D, Skv = _mqa_args(q, kv, kv_scale, weights, k_start, k_end)
    out = _np.full((S, Skv), _np.nan, dtype=_np.float64)
    _load().orc_mqa_logits(q.ctypes.data, kv.ctypes.data, kv_scale.ctypes.data, weights.ctypes.data,
                           k_start.ctypes.data, k_end.ctypes.data, int(bool(clean_logits)), S, H, D, Skv,
                           out.ctypes.data)
    return out


def mqa_logits_rows(q, kv, kv_scale, weights, k_start, k_end, clean_logits, rows):
    """The listed query rows of mqa_logits: [len(rows), Skv] fp64 (untouched: NaN)."""
    q, kv, kv_scale, weights, k_start, k_end, S, H, D, Skv = _mqa_args(q, kv, kv_scale, weights, k_start, k_end)
    rows = _np.ascontiguousarray(rows, dtype=_np.int32)
    out = _np.full((rows.size, Skv), _np.nan, dtype=_np.float64)
    _load().orc_mqa_logits_rows(q.ctypes.data, kv.ctypes.data, kv_scale.ctypes.data, weights.ctypes.data,
                                k_start.ctypes.data, k_end.ctypes.data, int(bool(clean_logits)), H, D, Skv,
                                rows.ctypes.data, rows.size, out.ctypes.data)
    return out


def ue8m0_encode(s):
    return int(_load().orc_ue8m0_encode(float(s)))


def ue8m0_decode(e):
    return float(_load().orc_ue8m0_decode(int(e)))


def _axis_split(shape, k_axis):
    ax = k_axis % len(shape)
    outer = int(_np.prod(shape[:ax], dtype=_np.int64))
    inner = int(_np.prod(shape[ax + 1:], dtype=_np.int64))
    return ax, outer, shape[ax], inner


def pack_ue8m0(sf, k_axis):
    """Power-of-two fp32 scales -> uint32 words, four K blocks per word along `k_axis`
    (-2 for sfa [.., K/128, ld], -1 for sfb [.., ceil(N/128), K/128])."""
    sf = _np.ascontiguousarray(sf, dtype=_np.float32)
    ax, outer, kb, inner = _axis_split(sf.shape, k_axis)
    out = _np.empty(sf.shape[:ax] + ((kb + 3) // 4,) + sf.shape[ax + 1:], dtype=_np.uint32)
    _load().orc_pack_ue8m0(_p(sf, _np.float32), outer, kb, inner, _p(out, _np.uint32))
    return out


def unpack_ue8m0(w, kblocks, k_axis):
    """uint32 words -> the fp32 scales they encode ([.., kblocks, ..] along `k_axis`)."""
    w = _np.ascontiguousarray(w, dtype=_np.uint32)
    ax, outer, _, inner = _axis_split(w.shape, k_axis)
    out = _np.empty(w.shape[:ax] + (kblocks,) + w.shape[ax + 1:], dtype=_np.float32)
    _load().orc_unpack_ue8m0(_p(w, _np.uint32), outer, kblocks, inner, _p(out, _np.float32))
    return out


def num_threads():
    return _load().orc_num_threads()


def set_num_threads(n):
    """Threads of the oracle's parallel loops from here on (the same results with any count)."""
    _load().orc_set_num_threads(int(n))
