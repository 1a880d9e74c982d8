"""ctypes binding of libdg.so (C ABI in include/dg.h).

Argument marshalling only: the functions check that tensors have the dtype,
device, contiguity and shape the C ABI documents, then pass raw device
pointers, sizes and the current HIP stream.  Every step of the computation
runs in the library's HIP kernels.  There is no fallback: if libdg.so is
missing, loading raises.

E4M3 tensors may be torch.uint8 or torch.float8_e4m3fn; bf16 tensors are
torch.bfloat16; scales torch.float32; index tensors torch.int32.
"""
from __future__ import annotations

import ctypes as ct
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

DG_OK = 0
_STATUS = {0: "DG_OK", -1: "DG_ERR_NULL", -2: "DG_ERR_SHAPE", -3: "DG_ERR_ALIGN", -4: "DG_ERR_ARG",
           -5: "DG_ERR_UNSUPPORTED", -6: "DG_ERR_HIP", -7: "DG_ERR_SCRATCH"}

EXPORTS = {
    # name: (restype, argtypes)
    "dg_fp8_gemm_nt": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                  ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_fp8_gemm_nt_ws": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                     ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p, ct.c_size_t,
                                     ct.c_void_p]),
    "dg_fp8_gemm_nt_ue8m0_ws": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p,
                                           ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p,
                                           ct.c_size_t, ct.c_void_p]),
    "dg_get_workspace_size": (ct.c_int64, [ct.c_int, ct.c_int, ct.c_int]),
    "dg_fp8_gemm_nt_noalloc": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p,
                                          ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_m_grouped_fp8_gemm_nt_contiguous": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                       ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int,
                                                       ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_m_grouped_fp8_gemm_nt_masked": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                   ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int,
                                                   ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_quantize_e4m3_1x128": (ct.c_int, [ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p,
                                          ct.c_int, ct.c_void_p]),
    "dg_quantize_e4m3_128x128": (ct.c_int, [ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p,
                                            ct.c_void_p]),
    "dg_fp8_gemm_nt_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                        ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                             ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int,
                                                             ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_m_grouped_fp8_gemm_nt_masked_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                         ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int,
                                                         ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_quantize_e4m3_1x128_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p,
                                                ct.c_void_p, ct.c_int, ct.c_void_p]),
    "dg_quantize_e4m3_128x128_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p,
                                                  ct.c_void_p, ct.c_void_p]),
    "dg_fp8_gemm_nn": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                  ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_fp8_gemm_tn": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                  ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_fp8_gemm_tt": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                  ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_k_grouped_fp8_gemm_tn_contiguous": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                       ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int,
                                                       ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_fp8_gemm_nn_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                        ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_fp8_gemm_tn_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                        ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_fp8_gemm_tt_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                        ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                             ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_int,
                                                             ct.c_int, ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_fp8_gemm_nt_ue8m0_packed": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_void_p,
                                               ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_int, ct.c_int,
                                               ct.c_void_p, ct.c_size_t, ct.c_void_p]),
    "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_packed": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                                    ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                                    ct.c_void_p, ct.c_int, ct.c_int, ct.c_int,
                                                                    ct.c_int, ct.c_void_p]),
    "dg_m_grouped_fp8_gemm_nt_masked_ue8m0_packed": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                                ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                                                ct.c_void_p, ct.c_int, ct.c_int, ct.c_int,
                                                                ct.c_int, ct.c_int, ct.c_void_p]),
    "dg_pack_sf_ue8m0": (ct.c_int, [ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p]),
    "dg_fp8_mqa_logits": (ct.c_int, [ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                     ct.c_void_p, ct.c_int, ct.c_void_p, ct.c_int, ct.c_int, ct.c_int, ct.c_int,
                                     ct.c_void_p]),
    "dg_get_mk_alignment_for_contiguous_layout": (ct.c_int, []),
    "dg_set_mk_alignment_for_contiguous_layout": (ct.c_int, [ct.c_int]),
    "dg_get_sf_aligned_size": (ct.c_int, [ct.c_int]),
    "dg_set_num_cus": (ct.c_int, [ct.c_int]),
    "dg_get_num_cus": (ct.c_int, []),
    "dg_set_kernel_family": (ct.c_int, [ct.c_char_p]),
    "dg_get_kernel_family": (ct.c_char_p, []),
    "dg_status_string": (ct.c_char_p, [ct.c_int]),
    "dg_last_config": (ct.c_char_p, []),
}

_lib = None
_lock = threading.Lock()


class DGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({lib().dg_status_string(status).decode()})")


def lib() -> ct.CDLL:
    """The loaded libdg.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(f"{LIB_PATH} is missing: build it with "
                                      "`python -m moe_grouped_gemm_scaled_amd.build`")
                l = ct.CDLL(LIB_PATH)
                for name, (res, args) in EXPORTS.items():
                    f = getattr(l, name)
                    f.restype = res
                    f.argtypes = args
                _lib = l
    return _lib


def _check(status: int, where: str):
    if status != DG_OK:
        raise DGError(status, where)


def _stream(t: torch.Tensor):
    return ct.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


_FP8 = (torch.uint8, torch.float8_e4m3fn)


def _ptr(t, dtypes, name, shape=None):
    if t is None:
        return None
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ct.c_void_p(t.data_ptr())


def ceil_div(a: int, b: int) -> int:
    return (a + b - 1) // b


def _name(base: str, ue8m0: bool) -> str:
    return base + "_ue8m0" if ue8m0 else base


def get_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of split-K scratch dg_fp8_gemm_nt_ws needs for M x N x K on the current device (0: no split)."""
    v = lib().dg_get_workspace_size(int(M), int(N), int(K))
    if v < 0:
        raise DGError(int(v), "dg_get_workspace_size")
    return int(v)


def get_workspace(M: int, N: int, K: int, device=None):
    """A zero-filled uint8 device tensor of get_workspace_size(M, N, K) bytes (None when the problem does
    not split K).  It may serve any number of fp8_gemm_nt calls in stream order; calls that can run at
    the same time (other streams, graphs replayed concurrently) each need their own."""
    n = get_workspace_size(M, N, K)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device if device is not None else "cuda")


def fp8_gemm_nt(a, sfa, b, sfb, d, c=None, ue8m0=False, workspace="auto"):
    """D = C + A . B^T.  a[M,K], sfa[K/128, ld_sfa], b[N,K], sfb[ceil(N/128), K/128], d/c[M,N] bf16.
    ue8m0: every scale is a power of two (dg_fp8_gemm_nt_ue8m0[_ws]).
    workspace: a zeroed uint8 device tensor from get_workspace() (dg_fp8_gemm_nt_ws); None runs without
    split-K (dg_fp8_gemm_nt); "auto" takes a fresh zeroed one from torch's allocator for this call."""
    M, K = a.shape
    N = b.shape[0]
    if sfa.dim() != 2 or sfa.shape[0] != K // 128:
        raise ValueError(f"sfa: shape {tuple(sfa.shape)}, expected [K/128={K // 128}, ld_sfa]")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace {workspace!r}")
        workspace = get_workspace(M, N, K, d.device)
    args = (_ptr(a, _FP8, "a", (M, K)), _ptr(sfa, torch.float32, "sfa"), int(sfa.shape[1]),
            _ptr(b, _FP8, "b", (N, K)), _ptr(sfb, torch.float32, "sfb", (ceil_div(N, 128), K // 128)),
            _ptr(c, torch.bfloat16, "c", (M, N)), _ptr(d, torch.bfloat16, "d", (M, N)), M, N, K)
    if workspace is None:
        name = _name("dg_fp8_gemm_nt", ue8m0)
        _check(getattr(lib(), name)(*args, _stream(d)), name)
    else:
        name = "dg_fp8_gemm_nt_ue8m0_ws" if ue8m0 else "dg_fp8_gemm_nt_ws"
        ws = _ptr(workspace, torch.uint8, "workspace")
        _check(getattr(lib(), name)(*args, ws, int(workspace.numel()), _stream(d)), name)
    return d


def fp8_gemm_nt_noalloc(a, sfa, b, sfb, d, c=None):
    """D = C + A . B^T through dg_fp8_gemm_nt_noalloc: split-K scratch from the library's own device array,
    nothing allocated (not even by torch); calls that may overlap on one GPU race.  Arguments as for
    fp8_gemm_nt."""
    M, K = a.shape
    N = b.shape[0]
    if sfa.dim() != 2 or sfa.shape[0] != K // 128:
        raise ValueError(f"sfa: shape {tuple(sfa.shape)}, expected [K/128={K // 128}, ld_sfa]")
    args = (_ptr(a, _FP8, "a", (M, K)), _ptr(sfa, torch.float32, "sfa"), int(sfa.shape[1]),
            _ptr(b, _FP8, "b", (N, K)), _ptr(sfb, torch.float32, "sfb", (ceil_div(N, 128), K // 128)),
            _ptr(c, torch.bfloat16, "c", (M, N)), _ptr(d, torch.bfloat16, "d", (M, N)), M, N, K, _stream(d))
    _check(lib().dg_fp8_gemm_nt_noalloc(*args), "dg_fp8_gemm_nt_noalloc")
    return d


def fp8_gemm(layout, a, sfa, b, sfb, d, c=None, ue8m0=False):
    """D = C + A @ B in one of the layouts "nt", "nn", "tn", "tt" (dg_fp8_gemm_<layout>).
    The first letter is A's storage: "n" a[M,K], "t" a[K,M]; the second B's: "t" b[N,K], "n" b[K,N].
    Scales as for fp8_gemm_nt: sfa[K/128, ld_sfa], sfb[ceil(N/128), K/128]; d/c[M,N] bf16."""
    if layout not in ("nt", "nn", "tn", "tt"):
        raise ValueError(f"layout {layout!r}")
    M, N = d.shape
    K = a.shape[1] if layout[0] == "n" else a.shape[0]
    a_shape = (M, K) if layout[0] == "n" else (K, M)
    b_shape = (N, K) if layout[1] == "t" else (K, N)
    if sfa.dim() != 2 or sfa.shape[0] != K // 128:
        raise ValueError(f"sfa: shape {tuple(sfa.shape)}, expected [K/128={K // 128}, ld_sfa]")
    args = (_ptr(a, _FP8, "a", a_shape), _ptr(sfa, torch.float32, "sfa"), int(sfa.shape[1]),
            _ptr(b, _FP8, "b", b_shape), _ptr(sfb, torch.float32, "sfb", (ceil_div(N, 128), K // 128)),
            _ptr(c, torch.bfloat16, "c", (M, N)), _ptr(d, torch.bfloat16, "d", (M, N)), M, N, K, _stream(d))
    name = _name("dg_fp8_gemm_" + layout, ue8m0)
    _check(getattr(lib(), name)(*args), name)
    return d


def k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, ks, d, c=None, ue8m0=False):
    """K-grouped TN contiguous GEMM (dg_k_grouped_fp8_gemm_tn_contiguous): a[K,M], b[K,N] E4M3,
    sfa[K/128,M], sfb[K/128,N] fp32, ks[G] int32 device tensor of group sizes (multiples of 128),
    d (and c, optional, may be d) fp32 [G,M,N]:  D[g] = C[g] + A_g^T B_g."""
    K, M = a.shape
    N = b.shape[1]
    G = ks.shape[0]
    args = (_ptr(a, _FP8, "a", (K, M)), _ptr(sfa, torch.float32, "sfa", (K // 128, M)),
            _ptr(b, _FP8, "b", (K, N)), _ptr(sfb, torch.float32, "sfb", (K // 128, N)),
            _ptr(ks, torch.int32, "ks", (G,)), _ptr(c, torch.float32, "c", (G, M, N)),
            _ptr(d, torch.float32, "d", (G, M, N)), M, N, K, G, _stream(d))
    name = _name("dg_k_grouped_fp8_gemm_tn_contiguous", ue8m0)
    _check(getattr(lib(), name)(*args), name)
    return d


def m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, d, m_indices, c=None, ue8m0=False):
    """a[M_total,K], sfa[K/128, M_total], b[G,N,K], sfb[G, ceil(N/128), K/128], d/c[M_total,N], m_indices[M_total]."""
    M_total, K = a.shape
    G, N, _ = b.shape
    args = (_ptr(a, _FP8, "a", (M_total, K)), _ptr(sfa, torch.float32, "sfa", (K // 128, M_total)),
            _ptr(b, _FP8, "b", (G, N, K)), _ptr(sfb, torch.float32, "sfb", (G, ceil_div(N, 128), K // 128)),
            _ptr(c, torch.bfloat16, "c", (M_total, N)), _ptr(d, torch.bfloat16, "d", (M_total, N)),
            _ptr(m_indices, torch.int32, "m_indices", (M_total,)), M_total, N, K, G, _stream(d))
    name = _name("dg_m_grouped_fp8_gemm_nt_contiguous", ue8m0)
    _check(getattr(lib(), name)(*args), name)
    return d


def m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, d, masked_m, expected_m=0, c=None, ue8m0=False):
    """a[G,M_cap,K], sfa[G, K/128, round_up(M_cap,4)], b[G,N,K], sfb[G, ceil(N/128), K/128], d/c[G,M_cap,N]."""
    G, M_cap, K = a.shape
    N = b.shape[1]
    ld = (M_cap + 3) // 4 * 4
    args = (_ptr(a, _FP8, "a", (G, M_cap, K)), _ptr(sfa, torch.float32, "sfa", (G, K // 128, ld)),
            _ptr(b, _FP8, "b", (G, N, K)), _ptr(sfb, torch.float32, "sfb", (G, ceil_div(N, 128), K // 128)),
            _ptr(c, torch.bfloat16, "c", (G, M_cap, N)), _ptr(d, torch.bfloat16, "d", (G, M_cap, N)),
            _ptr(masked_m, torch.int32, "masked_m", (G,)), G, M_cap, N, K, int(expected_m), _stream(d))
    name = _name("dg_m_grouped_fp8_gemm_nt_masked", ue8m0)
    _check(getattr(lib(), name)(*args), name)
    return d


def quantize_e4m3_1x128(x, q=None, sf=None, ld_sf=None, ue8m0=False):
    """x[groups, rows, K] or [rows, K] fp32 -> (q uint8, sf[groups, K/128, ld_sf] or [K/128, ld_sf]).
    ue8m0: power-of-two scales (dg_quantize_e4m3_1x128_ue8m0)."""
    squeeze = x.dim() == 2
    groups, rows, K = (1,) + tuple(x.shape) if squeeze else tuple(x.shape)
    ld = (rows + 3) // 4 * 4 if ld_sf is None else int(ld_sf)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.zeros((K // 128, ld) if squeeze else (groups, K // 128, ld), dtype=torch.float32, device=x.device)
    _ptr(sf, torch.float32, "sf", (K // 128, ld) if squeeze else (groups, K // 128, ld))
    args = (_ptr(x, torch.float32, "x"), groups, rows, K, _ptr(q, _FP8, "q", tuple(x.shape)),
            ct.c_void_p(sf.data_ptr()), ld, _stream(x))
    name = _name("dg_quantize_e4m3_1x128", ue8m0)
    _check(getattr(lib(), name)(*args), name)
    return q, sf


def quantize_e4m3_128x128(x, q=None, sf=None, ue8m0=False):
    """x[groups, rows, K] or [rows, K] fp32 -> (q uint8, sf[groups, ceil(rows/128), K/128]).
    ue8m0: power-of-two scales (dg_quantize_e4m3_128x128_ue8m0)."""
    squeeze = x.dim() == 2
    groups, rows, K = (1,) + tuple(x.shape) if squeeze else tuple(x.shape)
    shape_sf = (ceil_div(rows, 128), K // 128) if squeeze else (groups, ceil_div(rows, 128), K // 128)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty(shape_sf, dtype=torch.float32, device=x.device)
    args = (_ptr(x, torch.float32, "x"), groups, rows, K, _ptr(q, _FP8, "q", tuple(x.shape)),
            _ptr(sf, torch.float32, "sf", shape_sf), _stream(x))
    name = _name("dg_quantize_e4m3_128x128", ue8m0)
    _check(getattr(lib(), name)(*args), name)
    return q, sf


def pack_sf_ue8m0(sf, k_axis, out=None):
    """Packs power-of-two fp32 scales four per 32-bit word along the K-block axis `k_axis`
    (dg_pack_sf_ue8m0): byte j of word q holds the exponent field of K block 4q + j.  sfa [.., K/128, ld]
    takes k_axis=-2, sfb [.., ceil(N/128), K/128] k_axis=-1.  Returns int32 words of sf's shape with
    ceil(K/512) along k_axis."""
    shape = tuple(sf.shape)
    ax = k_axis % len(shape)
    outer = 1
    for v in shape[:ax]:
        outer *= v
    inner = 1
    for v in shape[ax + 1:]:
        inner *= v
    kblocks = shape[ax]
    out_shape = shape[:ax] + (ceil_div(kblocks, 4),) + shape[ax + 1:]
    if out is None:
        out = torch.empty(out_shape, dtype=torch.int32, device=sf.device)
    _check(lib().dg_pack_sf_ue8m0(_ptr(sf, torch.float32, "sf"), outer, kblocks, inner,
                                  _ptr(out, torch.int32, "out", out_shape), _stream(sf)), "dg_pack_sf_ue8m0")
    return out


def fp8_gemm_nt_ue8m0_packed(a, sfa, b, sfb, d, c=None, workspace="auto"):
    """D = C + A . B^T on packed power-of-two scales (dg_fp8_gemm_nt_ue8m0_packed): sfa int32
    [ceil(K/512), ld_sfa], sfb int32 [ceil(N/128), ceil(K/512)] as pack_sf_ue8m0 writes them; the other
    arguments as for fp8_gemm_nt (workspace None: no split-K)."""
    M, K = a.shape
    N = b.shape[0]
    nkw = ceil_div(K // 128, 4)
    if sfa.dim() != 2 or sfa.shape[0] != nkw:
        raise ValueError(f"sfa: shape {tuple(sfa.shape)}, expected [ceil(K/512)={nkw}, ld_sfa]")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace {workspace!r}")
        workspace = get_workspace(M, N, K, d.device)
    ws = _ptr(workspace, torch.uint8, "workspace")
    args = (_ptr(a, _FP8, "a", (M, K)), _ptr(sfa, torch.int32, "sfa"), int(sfa.shape[1]),
            _ptr(b, _FP8, "b", (N, K)), _ptr(sfb, torch.int32, "sfb", (ceil_div(N, 128), nkw)),
            _ptr(c, torch.bfloat16, "c", (M, N)), _ptr(d, torch.bfloat16, "d", (M, N)), M, N, K,
            ws, int(workspace.numel()) if workspace is not None else 0, _stream(d))
    _check(lib().dg_fp8_gemm_nt_ue8m0_packed(*args), "dg_fp8_gemm_nt_ue8m0_packed")
    return d


def m_grouped_fp8_gemm_nt_contiguous_ue8m0_packed(a, sfa, b, sfb, d, m_indices, c=None):
    """Contiguous grouped GEMM on packed power-of-two scales: sfa int32 [ceil(K/512), M_total], sfb int32
    [G, ceil(N/128), ceil(K/512)]; the rest as m_grouped_fp8_gemm_nt_contiguous."""
    M_total, K = a.shape
    G, N, _ = b.shape
    nkw = ceil_div(K // 128, 4)
    args = (_ptr(a, _FP8, "a", (M_total, K)), _ptr(sfa, torch.int32, "sfa", (nkw, M_total)),
            _ptr(b, _FP8, "b", (G, N, K)), _ptr(sfb, torch.int32, "sfb", (G, ceil_div(N, 128), nkw)),
            _ptr(c, torch.bfloat16, "c", (M_total, N)), _ptr(d, torch.bfloat16, "d", (M_total, N)),
            _ptr(m_indices, torch.int32, "m_indices", (M_total,)), M_total, N, K, G, _stream(d))
    _check(lib().dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_packed(*args),
           "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_packed")
    return d


def m_grouped_fp8_gemm_nt_masked_ue8m0_packed(a, sfa, b, sfb, d, masked_m, expected_m=0, c=None):
    """Masked grouped GEMM on packed power-of-two scales: sfa int32 [G, ceil(K/512), round_up(M_cap,4)],
    sfb int32 [G, ceil(N/128), ceil(K/512)]; the rest as m_grouped_fp8_gemm_nt_masked."""
    G, M_cap, K = a.shape
    N = b.shape[1]
    ld = (M_cap + 3) // 4 * 4
    nkw = ceil_div(K // 128, 4)
    args = (_ptr(a, _FP8, "a", (G, M_cap, K)), _ptr(sfa, torch.int32, "sfa", (G, nkw, ld)),
            _ptr(b, _FP8, "b", (G, N, K)), _ptr(sfb, torch.int32, "sfb", (G, ceil_div(N, 128), nkw)),
            _ptr(c, torch.bfloat16, "c", (G, M_cap, N)), _ptr(d, torch.bfloat16, "d", (G, M_cap, N)),
            _ptr(masked_m, torch.int32, "masked_m", (G,)), G, M_cap, N, K, int(expected_m), _stream(d))
    _check(lib().dg_m_grouped_fp8_gemm_nt_masked_ue8m0_packed(*args), "dg_m_grouped_fp8_gemm_nt_masked_ue8m0_packed")
    return d


def fp8_mqa_logits(q, kv, kv_scale, weights, k_start, k_end, clean_logits=True, logits=None):
    """FP8 MQA logits (dg_fp8_mqa_logits).  q[S, H, D], kv[S_kv, D] E4M3, kv_scale[S_kv] fp32,
    weights[S, H] fp32, k_start/k_end[S] int32 -> logits[S, S_kv] fp32 (allocated when None; when
    clean_logits is false, positions outside a row's range keep what `logits` held)."""
    S, H, D = tuple(q.shape)
    S_kv = kv.shape[0]
    if logits is None:
        logits = torch.empty((S, S_kv), dtype=torch.float32, device=q.device)
    args = (_ptr(q, _FP8, "q"), _ptr(kv, _FP8, "kv", (S_kv, D)), _ptr(kv_scale, torch.float32, "kv_scale", (S_kv,)),
            _ptr(weights, torch.float32, "weights", (S, H)), _ptr(k_start, torch.int32, "k_start", (S,)),
            _ptr(k_end, torch.int32, "k_end", (S,)), int(bool(clean_logits)),
            _ptr(logits, torch.float32, "logits", (S, S_kv)), S, H, D, S_kv, _stream(q))
    _check(lib().dg_fp8_mqa_logits(*args), "dg_fp8_mqa_logits")
    return logits


def get_mk_alignment_for_contiguous_layout() -> int:
    return lib().dg_get_mk_alignment_for_contiguous_layout()


def set_mk_alignment_for_contiguous_layout(alignment: int):
    _check(lib().dg_set_mk_alignment_for_contiguous_layout(int(alignment)), "dg_set_mk_alignment_for_contiguous_layout")


def get_sf_aligned_size(mn: int) -> int:
    return lib().dg_get_sf_aligned_size(int(mn))


def set_num_cus(n: int):
    _check(lib().dg_set_num_cus(int(n)), "dg_set_num_cus")


def get_num_cus() -> int:
    v = lib().dg_get_num_cus()
    if v < 0:
        raise DGError(v, "dg_get_num_cus")
    return v


def set_kernel_family(name: str):
    """Kernel family of the GEMM entry points called from this thread: auto, pipe, persist, skinny or tiled."""
    _check(lib().dg_set_kernel_family(name.encode()), "dg_set_kernel_family")


def get_kernel_family() -> str:
    return lib().dg_get_kernel_family().decode()


def last_config() -> str:
    return lib().dg_last_config().decode()
