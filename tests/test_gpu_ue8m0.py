"""GPU parity of the power-of-two (UE8M0) scale variants against the CPU
oracle: the *_ue8m0 quantisers bit for bit, and the *_ue8m0 GEMMs (whose
pipelined kernels hand the scales to the matrix cores as exponents) within
|D - D_ref| <= ulp_bf16(D_ref) + 1e-4 max|D_ref|, on the launch shapes of
every path: split-K decode tiles, 256x256 and 128x128 prefill tiles, the
contiguous and masked layouts, with M and N tails.  An identity case with
power-of-two scales must be bit-exact, which pins the per-lane scale operands
(which exponent applies to which row, column and K block).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg
from moe_grouped_gemm_scaled_amd import synth

from helpers import (SENTINEL, Guarded, check_close, contiguous_problem, dense_problem, dev, dev_bf16,
                     masked_problem, sample_indices)

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()
    yield
    torch.cuda.synchronize()


def _wide_range(seed, shape):
    """N(0,1) data scaled by 2^[-20, 20] per element: scales across many binades."""
    x = synth.normal_f32(seed, 0, shape)
    e = synth.randint(seed, 1, int(np.prod(shape)), -20, 20).reshape(shape)
    return (x * np.ldexp(np.float32(1.0), e)).astype(np.float32)


@pytest.mark.parametrize("groups,rows,K,ld", [(1, 37, 384, None), (3, 130, 256, 136), (1, 64, 7168, None)])
def test_quantize_1x128_ue8m0_bitexact(groups, rows, K, ld):
    announce(f"quantize_1x128_ue8m0 groups={groups} rows={rows} K={K}")
    x = _wide_range(40, (groups, rows, K))
    x[0, 0, :128] = 0.0
    q_ref, sf_ref = oracle.quantize_1x128(x, ld_sf=ld, ue8m0=True)
    q, sf = dg.quantize_e4m3_1x128(dev(x), ld_sf=ld, ue8m0=True)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    sfh = sf.cpu().numpy()
    assert np.array_equal(sfh[:, :, :rows].view(np.uint32), sf_ref[:, :, :rows].view(np.uint32))


@pytest.mark.parametrize("groups,rows,K", [(1, 300, 256), (4, 130, 384), (1, 2112, 1024)])
def test_quantize_128x128_ue8m0_bitexact(groups, rows, K):
    announce(f"quantize_128x128_ue8m0 groups={groups} rows={rows} K={K}")
    x = _wide_range(41, (groups, rows, K))
    x[0, :128, :128] = 0.0
    q_ref, sf_ref = oracle.quantize_128x128(x, ue8m0=True)
    q, sf = dg.quantize_e4m3_128x128(dev(x), ue8m0=True)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), sf_ref.view(np.uint32))


def run_dense(p):
    M, N = p["M"], p["N"]
    out = Guarded((M, N))
    c = dev_bf16(p["c"]) if p["c"] is not None else None
    dg.fp8_gemm_nt(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t, c=c, ue8m0=True)
    torch.cuda.synchronize()
    assert out.guards_intact()
    return out.bits()


# decode-shaped (split-K tiles, odd and even K-block counts), prefill-shaped
# (128x128 tiles for short K, 256x256 for long K), with M and N tails
DENSE = [(64, 2112, 2048, False), (128, 700, 1536, True), (33, 1000, 384, False), (300, 520, 768, True),
         (520, 600, 2304, True), (257, 300, 512, False)]


@pytest.mark.parametrize("M,N,K,with_c", DENSE)
def test_dense_ue8m0(M, N, K, with_c):
    announce(f"dense ue8m0 M={M} N={N} K={K} C={with_c}")
    p = dense_problem(M, N, K, seed=M * 13 + N + K, with_c=with_c, ue8m0=True)
    got = run_dense(p)
    ref = oracle.gemm_nt(p["a"], p["sfa"], p["b"], p["sfb"], p["c"])
    check_close(got, ref, f"dense ue8m0 {M}x{N}x{K} ({dg.last_config()})")


@pytest.mark.parametrize("M,K", [(96, 512), (300, 2304)])
def test_dense_ue8m0_identity_bitexact(M, K):
    """B = identity, power-of-two scales: every D[m,n] is one exactly
    representable product, so the scaled MFMA must give the oracle's value
    bit for bit; a wrong lane's exponent or a swapped operand shows here."""
    N = K
    announce(f"dense ue8m0 identity M={M} N=K={K}")
    a = synth.random_codes(42, 0, (M, K))
    b = np.zeros((N, K), dtype=np.uint8)
    b[np.arange(N), np.arange(N)] = 0x38
    ea = synth.randint(42, 4, (K // 128) * M, -8, 8).reshape(K // 128, M)
    eb = synth.randint(42, 5, (N // 128) * (K // 128), -8, 8).reshape(N // 128, K // 128)
    sfa = np.ldexp(np.float32(1.0), ea).astype(np.float32)
    sfb = np.ldexp(np.float32(1.0), eb).astype(np.float32)
    p = dict(a=a, sfa=sfa, b=b, sfb=sfb, c=None, M=M, N=N, K=K)
    got = run_dense(p)
    assert "scales=ue8m0" in dg.last_config(), dg.last_config()
    ref = oracle.gemm_nt(a, sfa, b, sfb, None)
    ref_bits = synth.f32_to_bf16_bits(ref.astype(np.float32))
    assert np.all(ref.astype(np.float32).astype(np.float64) == ref)
    eq = (got == ref_bits) | ((ref == 0) & ((got & 0x7FFF) == 0))
    assert np.all(eq), np.argwhere(~eq)[:5]


def test_contiguous_ue8m0():
    counts = [1, 128, 129, 0, 300, 5, 600]
    N, K = 264, 640
    announce(f"contiguous ue8m0 {counts}")
    p = contiguous_problem(counts, N, K, seed=43, with_c=True, ue8m0=True)
    out = Guarded((p["M_total"], N))
    dg.m_grouped_fp8_gemm_nt_contiguous(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                        dev(p["m_indices"]), c=dev_bf16(p["c"]), ue8m0=True)
    torch.cuda.synchronize()
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_contiguous(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], p["m_indices"])
    valid = p["m_indices"] >= 0
    check_close(got[valid], ref[valid], f"contiguous ue8m0 ({dg.last_config()})")
    assert np.all(got[~valid] == SENTINEL)


def test_masked_ue8m0():
    counts = [0, 1, 129, 256, 77, 300, -3]
    G, M_cap, N, K = len(counts), 256, 392, 512
    announce(f"masked ue8m0 {counts}")
    p = masked_problem(G, M_cap, N, K, counts, seed=44, with_c=True, ue8m0=True)
    out = Guarded((G, M_cap, N))
    dg.m_grouped_fp8_gemm_nt_masked(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                    dev(p["masked_m"]), expected_m=128, c=dev_bf16(p["c"]), ue8m0=True)
    torch.cuda.synchronize()
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_masked(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], p["masked_m"])
    for g, mm in enumerate(counts):
        mm = min(max(mm, 0), M_cap)
        if mm:
            check_close(got[g, :mm], ref[g, :mm], f"masked ue8m0 group {g}")
        assert np.all(got[g, mm:] == SENTINEL)


@pytest.mark.parametrize("cfg", synth.PREFILL, ids=lambda c: c["name"])
def test_prefill_ue8m0_full_size_sampled(cfg):
    """The prefill workloads with power-of-two scales, in the launch
    configuration the benchmark times, on sampled elements (N tail included)."""
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    announce(f"prefill ue8m0 full size {cfg['name']}")
    p = dense_problem(M, N, K, cfg["seed"], cfg["with_c"], ue8m0=True)
    got = run_dense(p)
    ms = sample_indices(M, 160, cfg["seed"], stream=10)
    ns = sample_indices(N, 160, cfg["seed"], stream=11)
    ns = np.unique(np.concatenate([ns, np.arange(max(0, N - 70), N)])).astype(np.int32)
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    ref = oracle.gemm_nt_at(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], mm.reshape(-1), nn.reshape(-1))
    check_close(got[mm, nn].reshape(-1), ref, cfg["name"] + " ue8m0")
    assert not np.any((got & 0x7F80) == 0x7F80), "non-finite output"


# ---- the other layouts and the K-grouped form with power-of-two scales

def _stored(layout, a, b):
    a_st = np.ascontiguousarray(a.T) if layout[0] == "t" else a
    b_st = np.ascontiguousarray(b.T) if layout[1] == "n" else b
    return a_st, b_st


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K,with_c", [(256, 384, 512, True), (304, 528, 2304, False)])
def test_layout_ue8m0(layout, M, N, K, with_c):
    announce(f"layout {layout} ue8m0 M={M} N={N} K={K}")
    p = dense_problem(M, N, K, seed=M + N + K + 5, with_c=with_c, ue8m0=True)
    a_st, b_st = _stored(layout, p["a"], p["b"])
    out = Guarded((M, N))
    c = dev_bf16(p["c"]) if p["c"] is not None else None
    dg.fp8_gemm(layout, dev(a_st), dev(p["sfa"]), dev(b_st), dev(p["sfb"]), out.t, c=c, ue8m0=True)
    torch.cuda.synchronize()
    assert out.guards_intact()
    cfg = dg.last_config()
    assert "scales=ue8m0" in cfg and f"layout={layout}" in cfg, cfg
    ref = oracle.gemm_layout(layout, a_st, p["sfa"], b_st, p["sfb"], p["c"])
    check_close(out.bits(), ref, f"{layout} ue8m0 {M}x{N}x{K} ({cfg})")


@pytest.mark.parametrize("ks,M,N", [([256, 0, 128, 384], 128, 144), ([512, 128, 640], 272, 400)])
def test_k_grouped_ue8m0(ks, M, N):
    """Power-of-two scales on both operands: the matrix instruction applies
    the A row's and the B column's exponents per lane."""
    announce(f"k-grouped ue8m0 ks={ks} M={M} N={N}")
    K = int(np.sum(ks))
    seed = 95 + M + N
    qa, sa = oracle.quantize_1x128(synth.normal_f32(seed, synth.STREAM_A, (M, K)), ld_sf=M, ue8m0=True)
    qb, sb = oracle.quantize_1x128(_wide_range(seed, (N, K)), ld_sf=N, ue8m0=True)
    a, b = np.ascontiguousarray(qa.T), np.ascontiguousarray(qb.T)
    sfa, sfb = sa[:, :M].copy(), sb[:, :N].copy()
    ksa = np.asarray(ks, np.int32)
    c = synth.normal_f32(seed, synth.STREAM_C, (len(ks), M, N))
    d = torch.full((len(ks), M, N), float("nan"), dtype=torch.float32, device="cuda")
    dg.k_grouped_fp8_gemm_tn_contiguous(dev(a), dev(sfa), dev(b), dev(sfb), dev(ksa), d, c=dev(c), ue8m0=True)
    torch.cuda.synchronize()
    assert "scales=ue8m0" in dg.last_config(), dg.last_config()
    got = d.cpu().numpy().astype(np.float64)
    ref = oracle.k_grouped_tn(a, sfa, b, sfb, ksa, c)
    for g in range(len(ks)):
        if ks[g] == 0:
            assert np.array_equal(got[g], c[g].astype(np.float64))
            continue
        scale = float(np.max(np.abs(ref[g])))
        tol = 2.0 ** -20 * np.abs(ref[g]) + 1e-4 * scale
        bad = ~(np.abs(got[g] - ref[g]) <= tol)
        assert not np.any(bad), (g, np.argwhere(bad)[:5], got[g][bad][:5], ref[g][bad][:5])
