"""C ABI checks that need no GPU: the library loads, exports every function
that include/dg.h declares, and rejects invalid arguments on the host before
any HIP call (so these calls never reach the device)."""
import ctypes as ct
import os
import re

import pytest

from moe_grouped_gemm_scaled_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")

# Fake, 16-byte aligned, never dereferenced: validation fails before use.
P = ct.c_void_p(0x10000)
MIS = ct.c_void_p(0x10004)
NULL = None
S = None    # default stream


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from moe_grouped_gemm_scaled_amd import build
        build.build()
    return binding.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.EXPORTS), set(names) ^ set(binding.EXPORTS)


def test_utilities(lib):
    assert lib.dg_get_mk_alignment_for_contiguous_layout() == 128
    assert lib.dg_set_mk_alignment_for_contiguous_layout(128) == 0
    assert lib.dg_set_mk_alignment_for_contiguous_layout(64) == -4
    assert [lib.dg_get_sf_aligned_size(x) for x in (1, 4, 5, 128, 130)] == [4, 4, 8, 128, 132]
    assert lib.dg_set_num_cus(-1) == -4
    assert lib.dg_set_num_cus(0) == 0
    for s in range(-7, 1):
        assert lib.dg_status_string(s).decode().startswith(("DG_OK", "DG_ERR"))


def test_kernel_family_setting(lib):
    start = lib.dg_get_kernel_family().decode()
    try:
        for name in ("pipe", "persist", "skinny", "tiled", "auto"):
            assert lib.dg_set_kernel_family(name.encode()) == 0
            assert lib.dg_get_kernel_family().decode() == name
        assert lib.dg_set_kernel_family(b"cutlass") == -4
        assert lib.dg_set_kernel_family(None) == -1
        assert lib.dg_get_kernel_family().decode() == "auto"
    finally:
        lib.dg_set_kernel_family(start.encode())


def test_kernel_family_setting_is_per_thread(lib):
    """A thread's setting changes that thread's kernel choice only."""
    import threading
    seen = {}

    def worker():
        seen["before"] = lib.dg_get_kernel_family().decode()
        assert lib.dg_set_kernel_family(b"tiled") == 0
        seen["after"] = lib.dg_get_kernel_family().decode()

    start = lib.dg_get_kernel_family().decode()
    try:
        assert lib.dg_set_kernel_family(b"persist") == 0
        t = threading.Thread(target=worker)
        t.start()
        t.join()
        assert seen["after"] == "tiled"
        assert seen["before"] != "persist"          # the new thread starts from the environment, not from us
        assert lib.dg_get_kernel_family().decode() == "persist"
    finally:
        lib.dg_set_kernel_family(start.encode())


def test_workspace_entry_point_argument_errors(lib):
    f = lib.dg_fp8_gemm_nt_ws
    # a, sfa, ld_sfa, b, sfb, c, d, M, N, K, workspace, bytes, stream
    assert f(NULL, P, 64, P, P, NULL, P, 64, 64, 128, P, 1 << 20, S) == -1
    assert f(P, P, 64, P, P, NULL, P, 64, 64, 100, P, 1 << 20, S) == -2
    assert f(P, P, 64, P, P, NULL, P, 64, 64, 128, MIS, 1 << 20, S) == -3     # misaligned workspace
    assert lib.dg_fp8_gemm_nt_ue8m0_ws(P, P, 64, P, P, NULL, P, 64, 64, 128, MIS, 1 << 20, S) == -3
    assert lib.dg_get_workspace_size(64, 64, 100) == -2
    assert lib.dg_get_workspace_size(0, 64, 128) == -2


def test_noalloc_entry_point_argument_errors(lib):
    f = lib.dg_fp8_gemm_nt_noalloc
    # a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream
    assert f(NULL, P, 64, P, P, NULL, P, 64, 64, 128, S) == -1
    assert f(P, P, 64, P, P, NULL, P, 64, 64, 100, S) == -2
    assert f(P, P, 60, P, P, NULL, P, 64, 64, 128, S) == -3
    assert f(MIS, P, 64, P, P, NULL, P, 64, 64, 128, S) == -3
    assert lib.dg_status_string(-7).decode().startswith("DG_ERR_SCRATCH")


def test_dense_argument_errors(lib):
    f = lib.dg_fp8_gemm_nt
    # a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream
    assert f(NULL, P, 64, P, P, NULL, P, 64, 64, 128, S) == -1
    assert f(P, P, 64, P, P, NULL, NULL, 64, 64, 128, S) == -1
    assert f(P, P, 64, P, P, NULL, P, 64, 64, 100, S) == -2       # K % 128
    assert f(P, P, 64, P, P, NULL, P, 64, 64, 0, S) == -2
    assert f(P, P, 64, P, P, NULL, P, 0, 64, 128, S) == -2        # M < 1
    assert f(P, P, 64, P, P, NULL, P, 64, 0, 128, S) == -2        # N < 1
    assert f(P, P, 60, P, P, NULL, P, 64, 64, 128, S) == -3       # ld_sfa < M
    assert f(P, P, 66, P, P, NULL, P, 65, 64, 128, S) == -3       # ld_sfa % 4
    assert f(MIS, P, 64, P, P, NULL, P, 64, 64, 128, S) == -3     # misaligned a
    assert f(P, P, 64, P, P, MIS, P, 64, 64, 128, S) == -3        # misaligned c


def test_contiguous_argument_errors(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous
    # a, sfa, b, sfb, c, d, m_indices, M_total, N, K, G, stream
    assert f(P, P, P, P, NULL, P, NULL, 128, 64, 128, 2, S) == -1
    assert f(P, P, P, P, NULL, P, P, 100, 64, 128, 2, S) == -2     # M_total % 128
    assert f(P, P, P, P, NULL, P, P, 128, 64, 128, 0, S) == -2     # G < 1
    assert f(P, P, P, P, NULL, P, P, 128, 64, 129, 2, S) == -2
    assert f(P, P, P, P, NULL, P, MIS, 128, 64, 128, 2, S) == -3


def test_masked_argument_errors(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_masked
    # a, sfa, b, sfb, c, d, masked_m, G, M_cap, N, K, expected_m, stream
    assert f(P, P, P, P, NULL, P, NULL, 2, 64, 64, 128, 0, S) == -1
    assert f(P, P, P, P, NULL, P, P, 0, 64, 64, 128, 0, S) == -2
    assert f(P, P, P, P, NULL, P, P, 2, 0, 64, 128, 0, S) == -2
    assert f(P, P, P, P, NULL, P, P, 2, 64, 64, 64, 0, S) == -2
    assert f(P, MIS, P, P, NULL, P, P, 2, 64, 64, 128, 0, S) == -3


def test_quantiser_argument_errors(lib):
    f1 = lib.dg_quantize_e4m3_1x128
    # x, groups, rows, K, q, sf, ld_sf, stream
    assert f1(NULL, 1, 4, 128, P, P, 4, S) == -1
    assert f1(P, 1, 4, 130, P, P, 4, S) == -2
    assert f1(P, 0, 4, 128, P, P, 4, S) == -2
    assert f1(P, 1, 5, 128, P, P, 6, S) == -3
    assert f1(P, 1, 5, 128, P, P, 4, S) == -3
    f2 = lib.dg_quantize_e4m3_128x128
    assert f2(P, 1, 4, 128, NULL, P, S) == -1
    assert f2(P, 1, 0, 128, P, P, S) == -2
    assert f2(P, 1, 4, 128, MIS, P, S) == -3


def test_binding_rejects_wrong_tensors_on_host():
    import torch
    a = torch.zeros((4, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        binding._ptr(a, torch.uint8, "a")     # not a device tensor
    with pytest.raises(TypeError):
        binding._ptr(a, torch.float32, "a")


def test_mqa_logits_argument_errors(lib):
    f = lib.dg_fp8_mqa_logits
    # q, kv, kv_scale, weights, k_start, k_end, clean, logits, S, H, D, S_kv, stream
    ok = (P, P, P, P, P, P, 1, P, 64, 64, 128, 256, S)

    def call(**kw):
        a = list(ok)
        names = ["q", "kv", "sc", "w", "ks", "ke", "clean", "out", "S", "H", "D", "S_kv", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    for name in ("q", "kv", "sc", "w", "ks", "ke", "out"):
        assert call(**{name: NULL}) == -1, name
    assert call(S=0) == -2
    assert call(S_kv=0) == -2
    assert call(D=64) == -2 and call(D=256) == -2           # head dim 128 only
    assert call(H=8) == -2 and call(H=80) == -2 and call(H=24) == -2
    assert call(S_kv=1 << 24) == -2                         # S_kv * 128 reaches 2^31
    assert call(q=MIS) == -3 and call(kv=MIS) == -3 and call(w=MIS) == -3
    odd = ct.c_void_p(0x10002)
    for name in ("sc", "ks", "ke", "out"):
        assert call(**{name: odd}) == -3, name


def test_layout_argument_errors(lib):
    # a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream
    for name in ("dg_fp8_gemm_nn", "dg_fp8_gemm_tn", "dg_fp8_gemm_tt"):
        f = getattr(lib, name)
        assert f(NULL, P, 64, P, P, NULL, P, 64, 64, 128, S) == -1, name
        assert f(P, P, 64, P, P, NULL, P, 64, 64, 100, S) == -2, name        # K % 128
        assert f(P, P, 64, P, P, NULL, P, 0, 64, 128, S) == -2, name
        assert f(P, P, 60, P, P, NULL, P, 64, 64, 128, S) == -3, name        # ld_sfa < M
        assert f(MIS, P, 64, P, P, NULL, P, 64, 64, 128, S) == -3, name
        assert f(P, P, 1 << 20, P, P, NULL, P, 1 << 20, 64, 4096, S) == -2, name   # K * M reaches 2^31
    # an MN-major operand needs 16-byte rows
    assert lib.dg_fp8_gemm_tn(P, P, 72, P, P, NULL, P, 72, 64, 128, S) == -3      # M % 16
    assert lib.dg_fp8_gemm_tn(P, P, 64, P, P, NULL, P, 64, 72, 128, S) == -3      # N % 16
    assert lib.dg_fp8_gemm_tt(P, P, 72, P, P, NULL, P, 72, 64, 128, S) == -3      # M % 16
    assert lib.dg_fp8_gemm_nn(P, P, 64, P, P, NULL, P, 64, 72, 128, S) == -3      # N % 16


def test_k_grouped_argument_errors(lib):
    f = lib.dg_k_grouped_fp8_gemm_tn_contiguous
    # a, sfa, b, sfb, ks, c, d, M, N, K, G, stream
    assert f(NULL, P, P, P, P, NULL, P, 64, 64, 128, 2, S) == -1
    assert f(P, P, P, P, NULL, NULL, P, 64, 64, 128, 2, S) == -1
    assert f(P, P, P, P, P, NULL, NULL, 64, 64, 128, 2, S) == -1
    assert f(P, P, P, P, P, NULL, P, 64, 64, 100, 2, S) == -2        # K % 128
    assert f(P, P, P, P, P, NULL, P, 64, 64, 128, 0, S) == -2        # G < 1
    assert f(P, P, P, P, P, NULL, P, 0, 64, 128, 2, S) == -2
    assert f(P, P, P, P, P, NULL, P, 1 << 20, 64, 4096, 2, S) == -2  # K * M reaches 2^31
    assert f(P, P, P, P, P, NULL, P, 72, 64, 128, 2, S) == -3        # M % 16
    assert f(P, P, P, P, P, NULL, P, 64, 40, 128, 2, S) == -3        # N % 16
    assert f(MIS, P, P, P, P, NULL, P, 64, 64, 128, 2, S) == -3
    assert f(P, P, P, P, ct.c_void_p(0x10002), NULL, P, 64, 64, 128, 2, S) == -3


def test_ue8m0_layout_and_k_grouped_argument_errors(lib):
    for name in ("dg_fp8_gemm_nn_ue8m0", "dg_fp8_gemm_tn_ue8m0", "dg_fp8_gemm_tt_ue8m0"):
        f = getattr(lib, name)
        assert f(NULL, P, 64, P, P, NULL, P, 64, 64, 128, S) == -1, name
        assert f(P, P, 64, P, P, NULL, P, 64, 64, 100, S) == -2, name
    assert lib.dg_fp8_gemm_tn_ue8m0(P, P, 72, P, P, NULL, P, 72, 64, 128, S) == -3
    f = lib.dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0
    assert f(P, P, P, P, NULL, NULL, P, 64, 64, 128, 2, S) == -1
    assert f(P, P, P, P, P, NULL, P, 64, 40, 128, 2, S) == -3


def test_packed_ue8m0_argument_errors(lib):
    f = lib.dg_fp8_gemm_nt_ue8m0_packed
    assert f(NULL, P, 64, P, P, NULL, P, 64, 64, 128, NULL, 0, S) == -1
    assert f(P, P, 64, P, P, NULL, P, 64, 64, 200, NULL, 0, S) == -2
    assert f(P, P, 60, P, P, NULL, P, 64, 64, 128, NULL, 0, S) == -3       # ld_sfa < M
    assert f(P, MIS, 64, P, P, NULL, P, 64, 64, 128, NULL, 0, S) == -3
    assert f(P, P, 1 << 20, P, P, NULL, P, 1 << 20, 64, 1 << 12, NULL, 0, S) == -2   # K * M >= 2^31
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_packed
    assert f(P, P, P, P, NULL, P, NULL, 256, 64, 128, 2, S) == -1
    assert f(P, P, P, P, NULL, P, P, 200, 64, 128, 2, S) == -2
    assert f(P, P, P, P, NULL, P, P, 256, 1 << 20, 1 << 12, 2, S) == -2    # K * N >= 2^31
    f = lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0_packed
    assert f(P, P, P, P, NULL, P, NULL, 2, 64, 64, 128, 0, S) == -1
    assert f(P, P, P, P, NULL, P, P, 0, 64, 64, 128, 0, S) == -2
    assert f(P, P, P, P, NULL, MIS, P, 2, 64, 64, 128, 0, S) == -3
    f = lib.dg_pack_sf_ue8m0
    assert f(NULL, 1, 4, 8, P, S) == -1
    assert f(P, 1, 0, 8, P, S) == -2
    assert f(P, 1, 4, 8, ct.c_void_p(0x10002), S) == -3
    assert f(P, 1 << 30, 4, 1 << 30, P, S) == -2                          # too many workgroups
