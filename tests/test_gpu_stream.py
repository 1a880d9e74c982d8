"""GPU parity of the streaming decode family (all rows of A and a column
tile of B per workgroup, one K block per LDS stage filled by DMA, optional
split-K) against the CPU oracle: every tile configuration it takes (32-, 96-,
112- and 128-column tiles, up to 64 and up to 128 rows), M and N tails,
one-block and odd K, K ranges longer than one unrolled chunk, with and
without C, and C aliasing D.
Bar: |D - D_ref| <= ulp_bf16(D_ref) + 1e-4 max|D_ref|, every element.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg

from helpers import Guarded, check_close, dense_problem, dev, dev_bf16

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()
    dg.set_kernel_family("stream")
    yield
    dg.set_kernel_family("auto")
    dg.set_num_cus(0)
    torch.cuda.synchronize()


def run(M, N, K, with_c, seed, c_alias=False):
    p = dense_problem(M, N, K, seed=seed, with_c=with_c)
    out = Guarded((M, N))
    c = None
    if with_c:
        c = dev_bf16(p["c"])
        if c_alias:
            out.t.copy_(c)
            c = out.t
    dg.fp8_gemm_nt(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t, c=c)
    torch.cuda.synchronize()
    cfg = dg.last_config()
    assert cfg.startswith("family=stream"), cfg
    assert out.guards_intact(), cfg
    ref = oracle.gemm_nt(p["a"], p["sfa"], p["b"], p["sfb"], p["c"])
    check_close(out.bits(), ref, f"stream {M}x{N}x{K} ({cfg})")
    return cfg


# (M, N, K, with_c): narrow N (64-column tiles), wide N (96 or 128 columns),
# row tails against 64- and 128-row tiles, a single K block, odd block counts
SHAPES = [(64, 2112, 2048, False), (128, 2112, 1792, True), (1, 300, 384, False), (37, 520, 128, True),
          (65, 700, 1152, False), (100, 4100, 640, True), (128, 7168, 1536, False), (64, 7168, 2304, True),
          (16, 24576, 256, False), (128, 33000, 384, True), (96, 40000, 256, False)]


@pytest.mark.parametrize("M,N,K,with_c", SHAPES)
def test_stream_shapes(M, N, K, with_c):
    announce(f"stream {M}x{N}x{K} C={with_c}")
    run(M, N, K, with_c, seed=M * 7 + N + K)


@pytest.mark.parametrize("M,N,K,with_c", [(40, 7000, 4096, True), (128, 7000, 2048, False), (64, 7168, 1536, False)])
def test_stream_112_column_tiles(M, N, K, with_c):
    """Shapes where 112-column tiles give the busiest workgroup fewer bytes
    than 128-column ones (N = 7000 leaves a partial last tile, and tiles
    start inside 128-wide scale blocks)."""
    announce(f"stream 112 {M}x{N}x{K} C={with_c}")
    cfg = run(M, N, K, with_c, seed=M + N + K + 11)
    assert "cols=112" in cfg, cfg


def test_stream_c_aliases_d():
    announce("stream C aliasing D")
    run(64, 2112, 1024, True, seed=5, c_alias=True)


@pytest.mark.parametrize("cus,M,N,K", [(4, 64, 520, 5120), (8, 128, 1100, 8320), (3, 40, 300, 4224)])
def test_stream_k_longer_than_one_chunk(cus, M, N, K):
    """With few CUs planned for, the tiles alone fill them: no split, and each
    workgroup walks more K blocks than one unrolled chunk holds (32), so the
    pipeline restarts at chunk boundaries."""
    announce(f"stream chunks cus={cus} {M}x{N}x{K}")
    dg.set_num_cus(cus)
    try:
        cfg = run(M, N, K, False, seed=cus + K)
    finally:
        dg.set_num_cus(0)
    assert "splits=1 " in cfg, cfg
