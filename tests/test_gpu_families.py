"""GPU parity of every kernel family, each forced in turn through
dg_set_kernel_family: pipelined, persistent (stream-K for small-M dense),
skinny and tiled, on dense, contiguous and masked problems that span several
tiles with ragged tails, against the CPU oracle.  The default choice is
covered by test_gpu_parity.py; this module keeps the other families, which
stay reachable through the C ABI, under the same bar.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg

from helpers import SENTINEL, Guarded, check_close, contiguous_problem, dense_problem, dev, dev_bf16, masked_problem

pytestmark = pytest.mark.gpu

FAMILIES = ["pipe", "persist", "skinny", "tiled"]
DENSE_FAMILIES = FAMILIES + ["stream"]          # the streaming family takes dense problems only


def announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()
    yield
    dg.set_kernel_family("auto")
    torch.cuda.synchronize()


@pytest.fixture
def family(request):
    dg.set_kernel_family(request.param)
    assert dg.get_kernel_family() == request.param
    yield request.param
    dg.set_kernel_family("auto")


def _family_of(config):
    return config.split("family=")[1].split()[0]


# Dense shapes: small-M decode-like (split-K paths, odd and even K-block
# counts), and several-tile prefill-like with M and N tails.
DENSE = [(64, 2112, 2048, False), (128, 700, 1536, True), (33, 1000, 384, False), (96, 520, 1280, True),
         (300, 520, 768, True), (520, 300, 2048, False)]


@pytest.mark.parametrize("family", DENSE_FAMILIES, indirect=True)
@pytest.mark.parametrize("M,N,K,with_c", DENSE)
def test_dense_every_family(family, M, N, K, with_c):
    announce(f"family={family} dense M={M} N={N} K={K} C={with_c}")
    p = dense_problem(M, N, K, seed=M * 31 + N + K, with_c=with_c)
    out = Guarded((M, N))
    c = dev_bf16(p["c"]) if p["c"] is not None else None
    dg.fp8_gemm_nt(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t, c=c)
    torch.cuda.synchronize()
    cfg = dg.last_config()
    assert out.guards_intact()
    ref = oracle.gemm_nt(p["a"], p["sfa"], p["b"], p["sfb"], p["c"])
    check_close(out.bits(), ref, f"{family} dense {M}x{N}x{K} ({cfg})")
    # the forced family ran wherever it takes the problem
    takes = {"pipe": True, "tiled": True, "skinny": M <= 128, "stream": M <= 128,
             "persist": M > 128 or (K // 128) % 2 == 0}[family]
    if takes:
        assert _family_of(cfg) == family, cfg


@pytest.mark.parametrize("family", FAMILIES, indirect=True)
def test_masked_every_family(family):
    counts = [0, 1, 129, 256, 77, 300]
    G, M_cap, N, K = len(counts), 256, 392, 512
    announce(f"family={family} masked {counts}")
    p = masked_problem(G, M_cap, N, K, counts, seed=23, with_c=True)
    out = Guarded((G, M_cap, N))
    dg.m_grouped_fp8_gemm_nt_masked(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                    dev(p["masked_m"]), expected_m=128, c=dev_bf16(p["c"]))
    torch.cuda.synchronize()
    cfg = dg.last_config()
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_masked(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], p["masked_m"])
    for g, mm in enumerate(counts):
        mm = min(max(mm, 0), M_cap)
        if mm:
            check_close(got[g, :mm], ref[g, :mm], f"{family} masked group {g} ({cfg})")
        assert np.all(got[g, mm:] == SENTINEL), f"{family} group {g}: masked rows written"
    assert _family_of(cfg) == family, cfg


@pytest.mark.parametrize("family", FAMILIES, indirect=True)
def test_masked_padding_rows_are_inert(family):
    """Rows at or past masked_m hold E4M3 NaN codes in A and NaN scales in
    sfa: the valid rows still equal the oracle's (computed on the clean
    inputs) and no padding row of D is written."""
    counts = [0, 5, 64, 65, 130, 256]
    G, M_cap, N, K = len(counts), 256, 392, 512
    announce(f"family={family} masked with poisoned padding rows {counts}")
    p = masked_problem(G, M_cap, N, K, counts, seed=31, with_c=True)
    a, sfa = p["a"].copy(), p["sfa"].copy()
    for g, mm in enumerate(counts):
        a[g, mm:, :] = 0x7F                      # E4M3FN NaN
        sfa[g, :, mm:] = np.nan
    out = Guarded((G, M_cap, N))
    dg.m_grouped_fp8_gemm_nt_masked(dev(a), dev(sfa), dev(p["b"]), dev(p["sfb"]), out.t,
                                    dev(p["masked_m"]), expected_m=64, c=dev_bf16(p["c"]))
    torch.cuda.synchronize()
    cfg = dg.last_config()
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_masked(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], p["masked_m"])
    for g, mm in enumerate(counts):
        if mm:
            check_close(got[g, :mm], ref[g, :mm], f"{family} poisoned masked group {g} ({cfg})")
        assert np.all(got[g, mm:] == SENTINEL), f"{family} group {g}: padding rows written"
    assert _family_of(cfg) == family, cfg


@pytest.mark.parametrize("family", ["pipe", "persist", "tiled"], indirect=True)
def test_contiguous_every_family(family):
    counts = [130, 1, 0, 257, 128, 60]
    N, K = 520, 640
    announce(f"family={family} contiguous {counts}")
    p = contiguous_problem(counts, N, K, seed=29, with_c=True)
    out = Guarded((p["M_total"], N))
    dg.m_grouped_fp8_gemm_nt_contiguous(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                        dev(p["m_indices"]), c=dev_bf16(p["c"]))
    torch.cuda.synchronize()
    cfg = dg.last_config()
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_contiguous(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], p["m_indices"])
    valid = p["m_indices"] >= 0
    check_close(got[valid], ref[valid], f"{family} contiguous valid rows ({cfg})")
    assert np.all(got[~valid] == SENTINEL)
    assert _family_of(cfg) == family, cfg


@pytest.mark.parametrize("family", ["pipe", "persist", "tiled"], indirect=True)
def test_contiguous_padding_rows_are_inert(family):
    """Padding rows (m_indices = -1) hold E4M3 NaN codes in A and NaN scales
    in sfa: the valid rows still equal the oracle's (computed on the clean
    inputs) and no padding row of D is written."""
    counts = [130, 1, 0, 257, 128, 60]
    N, K = 520, 640
    announce(f"family={family} contiguous with poisoned padding rows {counts}")
    p = contiguous_problem(counts, N, K, seed=37, with_c=True)
    valid = p["m_indices"] >= 0
    a, sfa = p["a"].copy(), p["sfa"].copy()
    a[~valid, :] = 0x7F                          # E4M3FN NaN
    sfa[:, :p["M_total"]][:, ~valid] = np.nan
    out = Guarded((p["M_total"], N))
    dg.m_grouped_fp8_gemm_nt_contiguous(dev(a), dev(sfa), dev(p["b"]), dev(p["sfb"]), out.t,
                                        dev(p["m_indices"]), c=dev_bf16(p["c"]))
    torch.cuda.synchronize()
    cfg = dg.last_config()
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_contiguous(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], p["m_indices"])
    check_close(got[valid], ref[valid], f"{family} poisoned contiguous valid rows ({cfg})")
    assert np.all(got[~valid] == SENTINEL)
    assert _family_of(cfg) == family, cfg


@pytest.mark.parametrize("family", DENSE_FAMILIES, indirect=True)
def test_repeated_calls_leave_split_counters_clean(family):
    """Split-K and stream-K reset their per-tile counters; back-to-back calls
    of different shapes on one stream, all through one caller workspace, must
    all be right."""
    announce(f"family={family} repeated split calls")
    shapes = [(64, 700, 4096), (128, 300, 2048), (64, 700, 4096), (40, 1500, 1024)]
    need = max(dg.get_workspace_size(M, N, K) for M, N, K in shapes)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    for M, N, K in shapes:
        p = dense_problem(M, N, K, seed=M + N + K + 7, with_c=False)
        out = Guarded((M, N))
        dg.fp8_gemm_nt(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t, workspace=ws)
        torch.cuda.synchronize()
        assert out.guards_intact()
        ref = oracle.gemm_nt(p["a"], p["sfa"], p["b"], p["sfb"], None)
        check_close(out.bits(), ref, f"{family} repeated {M}x{N}x{K} ({dg.last_config()})")


@pytest.mark.parametrize("M,N,K,with_c", [(37, 4128, 512, True), (128, 4224, 640, False), (64, 24576, 256, True)])
def test_skinny_96_column_tiles(M, N, K, with_c):
    """Wide N where 96-column tiles leave fewer columns per CU than 128-column
    ones: tiles then start inside a 128-column scale block and reach into the
    next (tile t covers columns 96t .. 96t+95), so each wave takes the scale
    block of its own columns.  Full compare (with an N tail at 4128)."""
    announce(f"skinny 96-column tiles M={M} N={N} K={K} C={with_c}")
    dg.set_kernel_family("skinny")
    try:
        p = dense_problem(M, N, K, seed=M * 7 + N + K, with_c=with_c)
        out = Guarded((M, N))
        c = dev_bf16(p["c"]) if p["c"] is not None else None
        dg.fp8_gemm_nt(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t, c=c)
        torch.cuda.synchronize()
        cfg = dg.last_config()
    finally:
        dg.set_kernel_family("auto")
    assert "family=skinny" in cfg and "cols=96" in cfg, cfg
    assert out.guards_intact()
    ref = oracle.gemm_nt(p["a"], p["sfa"], p["b"], p["sfb"], p["c"])
    check_close(out.bits(), ref, f"skinny 96 {M}x{N}x{K} ({cfg})")
