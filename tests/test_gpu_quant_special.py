"""GPU quantisers on non-finite and signed-zero inputs, bit for bit against
the oracle: a NaN (of either sign) is left out of its block's maximum and
encodes as 0x7f; a block holding +-inf gets the scale inf, so its finite
values encode as zeros of their sign and the infinities (inf/inf) as 0x7f;
-0 keeps its sign.  Both block shapes, fp32 and power-of-two scales."""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg
from moe_grouped_gemm_scaled_amd import synth

from helpers import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()
    yield
    torch.cuda.synchronize()


def special_input(rows, K, seed):
    x = synth.normal_f32(seed, 0, (rows, K))
    bits = x.view(np.uint32)
    bits[0, 3] = 0x7FC00000           # +NaN
    bits[0, 77] = 0xFFC00001          # -NaN
    bits[1, 5] = 0x7F800000           # +inf
    bits[2, 130] = 0xFF800000         # -inf (second K block)
    bits[3, :128] = 0x80000000        # a block of -0
    bits[3, 200] = 0x80000000         # -0 among normal values
    bits[4, 1] = 0x7FA00000           # signalling-pattern NaN
    bits[5, 128:256] = 0x00000001     # a block of the smallest denormal
    return x


@pytest.mark.parametrize("ue8m0", [False, True])
def test_quantize_1x128_special_values(ue8m0):
    rows, K = 40, 384
    print(f"\n[case] 1x128 special ue8m0={ue8m0}", file=sys.stderr, flush=True)
    x = special_input(rows, K, 71)
    q_ref, sf_ref = oracle.quantize_1x128(x, ue8m0=ue8m0)
    q, sf = dg.quantize_e4m3_1x128(dev(x), ue8m0=ue8m0)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    assert np.array_equal(qh, q_ref), np.argwhere(qh != q_ref)[:8]
    assert np.array_equal(sf.cpu().numpy()[:, :rows].view(np.uint32), sf_ref[:, :rows].view(np.uint32))
    assert qh[0, 3] == 0x7F and qh[0, 77] == 0x7F and qh[1, 5] == 0x7F and qh[2, 130] == 0x7F
    assert qh[3, 200] == 0x80 and np.all(qh[3, :128] == 0x80)


@pytest.mark.parametrize("ue8m0", [False, True])
def test_quantize_128x128_special_values(ue8m0):
    rows, K = 130, 384
    print(f"\n[case] 128x128 special ue8m0={ue8m0}", file=sys.stderr, flush=True)
    x = special_input(rows, K, 72)
    q_ref, sf_ref = oracle.quantize_128x128(x, ue8m0=ue8m0)
    q, sf = dg.quantize_e4m3_128x128(dev(x), ue8m0=ue8m0)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    assert np.array_equal(qh, q_ref), np.argwhere(qh != q_ref)[:8]
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), sf_ref.view(np.uint32))
