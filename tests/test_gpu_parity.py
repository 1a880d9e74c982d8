"""GPU parity: the HIP path (called through the C ABI via the binding) against
the CPU oracle on the same seeded inputs.

Quantisers: bit-exact codes and scales.  GEMMs: within
|D - D_ref| <= ulp_bf16(D_ref) + 1e-4 max|D_ref| of the oracle's fp64 result;
outputs that must stay untouched (masked rows, padding rows, guard bands)
are checked bit for bit against the sentinel they were filled with.
Small problems are compared element by element; the full-size workloads are
compared on sampled elements plus properties that hold at any size.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg
from moe_grouped_gemm_scaled_amd import synth

from helpers import (SENTINEL, Guarded, check_close, contiguous_problem, dense_problem, dev, dev_bf16,
                     masked_problem, sample_indices, stratified_indices)

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


def run_dense(p, c_alias=False):
    M, N, K = p["M"], p["N"], p["K"]
    out = Guarded((M, N))
    if c_alias:
        out.t.copy_(dev_bf16(p["c"]))
        c = out.t
    else:
        c = dev_bf16(p["c"]) if p["c"] is not None else None
    dg.fp8_gemm_nt(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t, c=c)
    torch.cuda.synchronize()
    assert out.guards_intact()
    return out.bits()


# ---------------------------------------------------------------- quantisers


@pytest.mark.parametrize("groups,rows,K,ld", [(1, 128, 512, None), (1, 37, 384, None), (1, 64, 7168, None),
                                              (3, 130, 256, 136), (16, 256, 2048, None)])
def test_quantize_1x128_bitexact(groups, rows, K, ld):
    announce(f"quantize_1x128 groups={groups} rows={rows} K={K} ld={ld}")
    x = synth.normal_f32(7, 0, (groups, rows, K))
    x[0, 0, :128] = 0.0                               # an all-zero block (scale floor)
    x[-1, -1, -128:] *= 1e-6                          # a tiny block
    q_ref, sf_ref = oracle.quantize_1x128(x, ld_sf=ld)
    q, sf = dg.quantize_e4m3_1x128(dev(x), ld_sf=ld)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    sfh = sf.cpu().numpy()
    assert np.array_equal(sfh[:, :, :rows].view(np.uint32), sf_ref[:, :, :rows].view(np.uint32))


@pytest.mark.parametrize("groups,rows,K", [(1, 256, 512), (1, 2112, 1024), (1, 300, 256), (4, 130, 384)])
def test_quantize_128x128_bitexact(groups, rows, K):
    announce(f"quantize_128x128 groups={groups} rows={rows} K={K}")
    x = synth.normal_f32(8, 1, (groups, rows, K))
    x[0, :128, :128] = 0.0
    q_ref, sf_ref = oracle.quantize_128x128(x)
    q, sf = dg.quantize_e4m3_128x128(dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), sf_ref.view(np.uint32))


def test_encoder_every_fp32_in_range_via_unit_scale():
    """A 1x128 block whose first element is 448 has scale exactly 1, so its other
    127 codes are the encoder applied to the raw values.  Every fp32 with
    2^-12 <= |x| < 448, both signs, goes through the GPU encoder this way and
    is compared with the oracle encoder."""
    announce("encoder exhaustive via unit-scale blocks")
    total = 0
    for e in range(127 - 12, 127 + 9):
        bits = np.arange(e << 23, (e + 1) << 23, dtype=np.uint32)
        vals = bits.view(np.float32)
        vals = vals[vals < 448.0]
        vals = np.concatenate([vals, -vals])
        nrow = (vals.size + 126) // 127
        pad = nrow * 127 - vals.size
        body = np.concatenate([vals, np.zeros(pad, dtype=np.float32)]).reshape(nrow, 127)
        x = np.concatenate([np.full((nrow, 1), 448.0, dtype=np.float32), body], axis=1)
        q, sf = dg.quantize_e4m3_1x128(dev(x))
        torch.cuda.synchronize()
        assert np.all(sf.cpu().numpy()[0, :nrow] == 1.0)
        got = q.cpu().numpy()[:, 1:].reshape(-1)[:vals.size]
        ref = oracle.e4m3_encode(vals)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (e, vals[bad[:4]], got[bad[:4]], ref[bad[:4]])
        total += vals.size
        del q, sf
    assert total > 300_000_000


# ---------------------------------------------------------------- dense GEMM


def test_dense_small_config_full_compare():
    cfg = synth.DENSE_SMALL
    announce(f"dense {cfg['name']}")
    p = dense_problem(cfg["M"], cfg["N"], cfg["K"], cfg["seed"], cfg["with_c"])
    got = run_dense(p)
    ref = oracle.gemm_nt(p["a"], p["sfa"], p["b"], p["sfb"], p["c"])
    check_close(got, ref, cfg["name"])


@pytest.mark.parametrize("M,N,K,with_c", [(1, 2112, 256, False), (37, 200, 384, True), (129, 129, 128, True),
                                          (257, 300, 512, False), (64, 2112, 7168, False),
                                          (200, 1000, 1024, True), (5, 16, 128, True), (520, 600, 2304, True)])
def test_dense_shapes_and_tails_full_compare(M, N, K, with_c):
    announce(f"dense M={M} N={N} K={K} C={with_c}")
    p = dense_problem(M, N, K, seed=M * 7 + N, with_c=with_c)
    got = run_dense(p)
    ref = oracle.gemm_nt(p["a"], p["sfa"], p["b"], p["sfb"], p["c"])
    check_close(got, ref, f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("M,K", [(96, 512), (300, 2304)])
def test_dense_identity_power_of_two_scales_bitexact(M, K):
    """B = identity, power-of-two scales: each D[m,n] is one exactly
    representable product, so GPU and oracle agree bit for bit.  This pins
    the operand lane layout, the transposed sfa index, the per-block sfb index
    and the row/column mapping of the output, for a decode-shaped (split-K)
    and a prefill-shaped launch."""
    N = K
    announce(f"dense identity M={M} N=K={K}")
    a = synth.random_codes(3, 0, (M, K))
    b = np.zeros((N, K), dtype=np.uint8)
    b[np.arange(N), np.arange(N)] = 0x38
    ea = synth.randint(3, 4, (K // 128) * M, -8, 8).reshape(K // 128, M)
    eb = synth.randint(3, 5, (N // 128) * (K // 128), -8, 8).reshape(N // 128, K // 128)
    sfa = np.ldexp(np.float32(1.0), ea).astype(np.float32)
    sfb = np.ldexp(np.float32(1.0), eb).astype(np.float32)
    p = dict(a=a, sfa=sfa, b=b, sfb=sfb, c=None, M=M, N=N, K=K)
    got = run_dense(p)
    ref = oracle.gemm_nt(a, sfa, b, sfb, None)
    ref_bits = synth.f32_to_bf16_bits(ref.astype(np.float32))
    assert np.all(ref.astype(np.float32).astype(np.float64) == ref)      # exact in fp32 and in bf16
    eq = (got == ref_bits) | ((ref == 0) & ((got & 0x7FFF) == 0))
    assert np.all(eq), np.argwhere(~eq)[:5]


def test_dense_zero_a_gives_c_and_c_may_alias_d():
    M, N, K = 70, 260, 256
    announce("dense A=0 and C aliasing D")
    p = dense_problem(M, N, K, seed=5, with_c=True)
    p0 = dict(p, a=np.zeros_like(p["a"]))
    got = run_dense(p0)
    assert np.array_equal(got, p["c"])
    got_alias = run_dense(p, c_alias=True)
    got_plain = run_dense(p)
    assert np.array_equal(got_alias, got_plain)


# ---------------------------------------------------------------- grouped GEMM


def test_masked_edge_counts():
    counts = [0, 1, 127, 128, 129, 255, 256, 300, -5]
    G, M_cap, N, K = len(counts), 256, 200, 256
    announce(f"masked edges {counts}")
    p = masked_problem(G, M_cap, N, K, counts, seed=17, with_c=True)
    out = Guarded((G, M_cap, N))
    dg.m_grouped_fp8_gemm_nt_masked(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                    dev(p["masked_m"]), expected_m=128, c=dev_bf16(p["c"]))
    torch.cuda.synchronize()
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_masked(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], p["masked_m"])
    for g, mm in enumerate(counts):
        mm = min(max(mm, 0), M_cap)
        if mm:
            check_close(got[g, :mm], ref[g, :mm], f"masked group {g}")
        assert np.all(got[g, mm:] == SENTINEL), f"group {g}: masked rows written"


def test_contiguous_edge_counts():
    counts = [1, 128, 129, 0, 300, 5]
    N, K = 264, 384
    announce(f"contiguous edges {counts}")
    p = contiguous_problem(counts, N, K, seed=19, with_c=True)
    out = Guarded((p["M_total"], N))
    dg.m_grouped_fp8_gemm_nt_contiguous(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                        dev(p["m_indices"]), c=dev_bf16(p["c"]))
    torch.cuda.synchronize()
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_contiguous(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], p["m_indices"])
    valid = p["m_indices"] >= 0
    check_close(got[valid], ref[valid], "contiguous valid rows")
    assert np.all(got[~valid] == SENTINEL)
    # grouped == dense per group on the GPU too (within tolerance of the oracle's dense)
    for g, cnt in enumerate(counts):
        if cnt == 0:
            continue
        rows = np.nonzero(p["m_indices"] == g)[0]
        sub = dict(a=np.ascontiguousarray(p["a"][rows]),
                   sfa=np.ascontiguousarray(np.pad(p["sfa"][:, rows], ((0, 0), (0, (-rows.size) % 4)))),
                   b=np.ascontiguousarray(p["b"][g]), sfb=np.ascontiguousarray(p["sfb"][g]),
                   c=np.ascontiguousarray(p["c"][rows]), M=rows.size, N=N, K=K)
        dense = run_dense(sub)
        check_close(dense, ref[rows], f"dense on expert {g}")



def test_contiguous_many_experts():
    """More than 256 aligned 128-row blocks and many segments of one, two and
    three blocks, with empty experts between them: the unit scan of the
    256-row-tile path runs over several rounds, and units must neither mix
    experts nor skip any."""
    counts = [0 if g % 7 == 3 else int(c) for g, c in enumerate(synth.randint(31, 3, 300, 0, 300))]
    N, K = 136, 256
    announce(f"contiguous many experts G={len(counts)} rows={sum(counts)}")
    p = contiguous_problem(counts, N, K, seed=31, with_c=True)
    assert p["M_total"] // 128 > 256
    out = Guarded((p["M_total"], N))
    dg.m_grouped_fp8_gemm_nt_contiguous(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                        dev(p["m_indices"]), c=dev_bf16(p["c"]))
    torch.cuda.synchronize()
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_contiguous(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], p["m_indices"])
    valid = p["m_indices"] >= 0
    check_close(got[valid], ref[valid], f"contiguous many experts ({dg.last_config()})")
    assert np.all(got[~valid] == SENTINEL)

# ---------------------------------------------------------------- full-size workloads (sampled)


@pytest.mark.parametrize("cfg", synth.DECODE + synth.PREFILL, ids=lambda c: c["name"])
def test_dense_full_size_sampled(cfg):
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    announce(f"dense full size {cfg['name']}")
    p = dense_problem(M, N, K, cfg["seed"], cfg["with_c"])
    got = run_dense(p)
    # stratified: every 16-row and 16-column block, every position in it
    ms = stratified_indices(M, cfg["seed"], stream=10) if M > 128 else np.arange(M, dtype=np.int32)
    ns = stratified_indices(N, cfg["seed"], stream=11)
    ns = np.unique(np.concatenate([ns, np.arange(max(0, N - 70), N)])).astype(np.int32)   # N tail
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    ref = oracle.gemm_nt_at(p["a"], p["sfa"], p["b"], p["sfb"], p["c"], mm.reshape(-1), nn.reshape(-1))
    check_close(got[mm, nn].reshape(-1), ref, cfg["name"])
    assert not np.any((got & 0x7F80) == 0x7F80), "non-finite output"


def test_contiguous_full_size_sampled():
    cfg = synth.CONTIGUOUS
    counts = synth.contiguous_counts(cfg)
    announce(f"contiguous full size counts={counts.tolist()}")
    p = contiguous_problem(counts, cfg["N"], cfg["K"], cfg["seed"], with_c=False)
    out = Guarded((p["M_total"], cfg["N"]))
    dg.m_grouped_fp8_gemm_nt_contiguous(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                        dev(p["m_indices"]))
    torch.cuda.synchronize()
    assert out.guards_intact()
    got = out.bits()
    m_idx = p["m_indices"]
    assert np.all(got[m_idx < 0] == SENTINEL)
    assert not np.any((got[m_idx >= 0] & 0x7F80) == 0x7F80)
    rows = []
    for g in range(cfg["G"]):
        r = np.nonzero(m_idx == g)[0]
        rows += [r[0], r[-1], r[r.size // 2]]
    # stratified over the valid rows (every 16-row block of every expert) and
    # over the columns (every 16-column block, every position)
    valid_rows = np.nonzero(m_idx >= 0)[0].astype(np.int32)
    rows = np.unique(np.concatenate([np.array(rows, dtype=np.int32),
                                     stratified_indices(p["M_total"], cfg["seed"], stream=14, within=valid_rows)]))
    ns = stratified_indices(cfg["N"], cfg["seed"], stream=12)
    mm, nn = np.meshgrid(rows, ns, indexing="ij")
    ref = oracle.m_grouped_contiguous_at(p["a"], p["sfa"], p["b"], p["sfb"], None, m_idx,
                                         mm.reshape(-1), nn.reshape(-1))
    check_close(got[mm, nn].reshape(-1), ref, cfg["name"])


def test_masked_full_size_sampled():
    cfg = synth.MASKED
    mm_counts = synth.masked_counts(cfg)
    announce(f"masked full size masked_m={mm_counts.tolist()}")
    G, M_cap, N, K = cfg["G"], cfg["M_cap"], cfg["N"], cfg["K"]
    p = masked_problem(G, M_cap, N, K, mm_counts, cfg["seed"])
    out = Guarded((G, M_cap, N))
    dg.m_grouped_fp8_gemm_nt_masked(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                    dev(p["masked_m"]), expected_m=128)
    torch.cuda.synchronize()
    assert out.guards_intact()
    got = out.bits()
    gs, ms, ns = [], [], []
    col = stratified_indices(N, cfg["seed"], stream=13)
    for g in range(G):
        mmg = int(mm_counts[g])
        assert np.all(got[g, mmg:] == SENTINEL), f"group {g}: masked rows written"
        if mmg == 0:
            continue
        assert not np.any((got[g, :mmg] & 0x7F80) == 0x7F80)
        # every 16-row block of the valid rows, every position in it
        r = np.unique(np.concatenate([np.array([0, mmg - 1, mmg // 2]),
                                      stratified_indices(mmg, cfg["seed"] + g, stream=15)]))
        for rr in r:
            gs += [g] * col.size
            ms += [rr] * col.size
            ns += col.tolist()
    gs, ms, ns = (np.array(v, dtype=np.int32) for v in (gs, ms, ns))
    ref = oracle.m_grouped_masked_at(p["a"], p["sfa"], p["b"], p["sfb"], None, p["masked_m"], gs, ms, ns)
    check_close(got[gs, ms, ns], ref, cfg["name"])


def test_split_k_on_concurrent_streams():
    """Split-K decode GEMMs issued on three streams at once, repeated: each
    call brings its own workspace and counters, so concurrent calls must not
    disturb each other (every result to the oracle bar, every time)."""
    shapes = [(64, 2112, 7168), (128, 7168, 2048), (64, 7168, 4096)]
    announce(f"split-K on concurrent streams {shapes}")
    probs, outs, streams = [], [], []
    for k, (M, N, K) in enumerate(shapes):
        p = dense_problem(M, N, K, seed=300 + k, with_c=False)
        probs.append((p, dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"])))
        outs.append(Guarded((M, N)))
        streams.append(torch.cuda.Stream())
    torch.cuda.synchronize()
    refs = [oracle.gemm_nt(p["a"], p["sfa"], p["b"], p["sfb"], None) for p, *_ in probs]
    for rep in range(3):
        for (p, a, sfa, b, sfb), out, st in zip(probs, outs, streams):
            with torch.cuda.stream(st):
                dg.fp8_gemm_nt(a, sfa, b, sfb, out.t)
        torch.cuda.synchronize()
        for k, ((p, *_), out, ref) in enumerate(zip(probs, outs, refs)):
            assert out.guards_intact()
            check_close(out.bits(), ref, f"stream {k} rep {rep}")


@pytest.mark.parametrize("family", ["auto", "pipe", "persist", "tiled"])
def test_contiguous_invalid_expert_ids_are_padding(family):
    """A 128-row block whose id lies outside [0, G) (too large, or negative
    other than -1) is padding: never computed, never written, and b is never
    read past its last expert."""
    counts = [130, 128, 70]
    N, K = 256, 384
    announce(f"contiguous invalid ids, family {family}")
    p = contiguous_problem(counts, N, K, seed=23, with_c=False)
    G = len(counts)
    idx = p["m_indices"].copy()
    idx[256:384] = G + 3                  # expert 1's block: an id past the last expert
    idx[384:454] = -5                     # expert 2's rows: a negative id other than -1
    clean = np.where((idx >= 0) & (idx < G), idx, -1).astype(np.int32)
    out = Guarded((p["M_total"], N))
    dg.set_kernel_family(family)
    try:
        dg.m_grouped_fp8_gemm_nt_contiguous(dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"]), out.t,
                                            dev(idx))
        torch.cuda.synchronize()
    finally:
        dg.set_kernel_family("auto")
    assert out.guards_intact()
    got = out.bits()
    ref = oracle.m_grouped_contiguous(p["a"], p["sfa"], p["b"], p["sfb"], None, clean)
    valid = clean >= 0
    check_close(got[valid], ref[valid], f"contiguous valid rows ({family})")
    assert np.all(got[~valid] == SENTINEL)
