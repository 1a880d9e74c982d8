"""GPU test of the allocation-free entry point dg_fp8_gemm_nt_noalloc: its
split-K scratch is the library's own device array, so nothing is allocated
per call.  Two calls in a row, the second on a smaller problem, must give
exactly what dg_fp8_gemm_nt_ws gives with a workspace of its own (the same
kernels and splits), and both must meet the GEMM bar against the oracle
(|D - D_ref| <= ulp_bf16(D_ref) + 1e-4 max|D_ref|, on sampled elements).
A problem whose split needs more scratch than the array holds is refused
before anything is launched.
"""
import ctypes as ct
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg

from helpers import Guarded, check_close, dense_problem, dev, sample_indices

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()
    dg.set_kernel_family("auto")
    yield
    torch.cuda.synchronize()


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    shapes = [(128, 7168, 8192, 501), (64, 2112, 4096, 502)]     # the second call is smaller
    for M, N, K, seed in shapes:
        announce(f"noalloc {M}x{N}x{K}")
        assert dg.get_workspace_size(M, N, K) > 0                  # a split-K configuration
        p = dense_problem(M, N, K, seed=seed, with_c=False)
        a, sfa, b, sfb = dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"])
        ref_out = Guarded((M, N))
        dg.fp8_gemm_nt(a, sfa, b, sfb, ref_out.t, workspace=dg.get_workspace(M, N, K))
        cfg_ws = dg.last_config()
        out = Guarded((M, N))
        torch.cuda.synchronize()
        dg.fp8_gemm_nt_noalloc(a, sfa, b, sfb, out.t)
        cfg_na = dg.last_config()
        torch.cuda.synchronize()
        assert cfg_na == cfg_ws and "splits=1 " not in cfg_na, (cfg_na, cfg_ws)
        assert out.guards_intact() and ref_out.guards_intact()
        got = out.bits()
        assert np.array_equal(got, ref_out.bits()), f"{M}x{N}x{K}: differs from dg_fp8_gemm_nt_ws"
        ms = sample_indices(M, 24, seed, stream=11)
        ns = sample_indices(N, 160, seed, stream=12)
        mm, nn = np.meshgrid(ms, ns, indexing="ij")
        ref = oracle.gemm_nt_at(p["a"], p["sfa"], p["b"], p["sfb"], None, mm.ravel(), nn.ravel())
        check_close(got[mm.ravel(), nn.ravel()], ref, f"noalloc {M}x{N}x{K}")


def test_noalloc_refuses_problems_beyond_its_scratch():
    """Stream-K over 512 column tiles of a 128 x 65536 x 16384 problem needs
    64 MiB of partials: refused with DG_ERR_SCRATCH on the host, nothing
    launched (the pointers are never dereferenced)."""
    P = ct.c_void_p(0x10000)
    dg.set_kernel_family("persist")
    try:
        st = dg.lib().dg_fp8_gemm_nt_noalloc(P, P, 128, P, P, None, P, 128, 65536, 16384, None)
    finally:
        dg.set_kernel_family("auto")
    assert st == -7, st
