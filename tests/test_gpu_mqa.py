"""GPU parity of the FP8 MQA logits (dg_fp8_mqa_logits) against the CPU oracle.

Tolerance, derived from the arithmetic of gfx950's FP8 matrix instruction
(v_mfma_f32_16x16x128_f8f6f4), as measured on single products: within each
group of 8 consecutive head-dim elements the products are summed in a
fixed-point window 13 bits below the group's leading product bit
(truncating), and the 16 group sums are added in fp32.  With 7 products per
group cut by less than 2^(e_max - 13) each, a dot product is off by less
than 2^-10 * sum_d |q kv|; the weighted head sum and the scale add fp32
roundings far below that.  So with
    mag[i][j] = kv_scale[j] * sum_h |weights[i][h]| * sum_d |q[i,h,d] kv[j,d]|
(the oracle evaluated on absolute values) every computed logit satisfies
    |logit - exact| <= 2^-10 * mag[i][j].
Dots with a single non-zero product are exact (the one-hot test checks bits).
Positions outside a row's range must be exactly -inf (clean_logits) or keep
the caller's bits (otherwise).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg
from moe_grouped_gemm_scaled_amd import synth

pytestmark = pytest.mark.gpu

UNTOUCHED = np.uint32(0x7FC0DEAD)        # a NaN payload the kernel never writes


def announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()
    yield
    torch.cuda.synchronize()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run(q, kv, kv_scale, weights, ks, ke, clean, misalign=False):
    S, S_kv = q.shape[0], kv.shape[0]
    n = S * S_kv
    flat = torch.from_numpy(np.full(n + 8, UNTOUCHED, dtype=np.uint32).view(np.float32)).cuda()
    off = 1 if misalign else 4
    out = flat[off:off + n].view(S, S_kv)
    dg.fp8_mqa_logits(dev(q), dev(kv), dev(kv_scale), dev(weights), dev(ks), dev(ke), clean, logits=out)
    torch.cuda.synchronize()
    host = flat.cpu().numpy()
    guard = np.concatenate([host[:off], host[off + n:]]).view(np.uint32)
    assert np.all(guard == UNTOUCHED), "write outside the logits"
    return host[off:off + n].reshape(S, S_kv)


def magnitude(q, kv, kv_scale, weights, ks, ke, rows=None):
    qa, kva, wa = q & np.uint8(0x7F), kv & np.uint8(0x7F), np.abs(weights)
    if rows is None:
        return oracle.mqa_logits(qa, kva, kv_scale, wa, ks, ke, True)
    return oracle.mqa_logits_rows(qa, kva, kv_scale, wa, ks, ke, True, rows)


def check(got, ref, mag, clean, where):
    """got: fp32 rows from the GPU; ref: oracle fp64 rows (NaN = untouched);
    mag: the magnitude bound's rows."""
    assert got.shape == ref.shape
    outside = ~np.isfinite(ref)
    if clean:
        assert np.all(np.isneginf(ref[outside]))
        assert np.all(np.isneginf(got[outside])), f"{where}: outside positions not -inf"
    else:
        assert np.all(got[outside].view(np.uint32) == UNTOUCHED), f"{where}: outside positions written"
    inside = ~outside
    g = got[inside].astype(np.float64)
    r = ref[inside]
    tol = 2.0 ** -10 * mag[inside]
    err = np.abs(g - r)
    bad = ~(err <= tol)
    if np.any(bad):
        idx = np.argwhere(inside)[bad][:5]
        raise AssertionError(f"{where}: {int(bad.sum())} of {bad.size} outside tolerance; first {idx.tolist()}: "
                             f"got {g[bad][:5]}, ref {r[bad][:5]}, tol {tol[bad][:5]}")
    return float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0


def ragged_ranges(seed, S, S_kv):
    """Starts in [-3, S_kv), lengths in [-2, S_kv]: empty, clamped and
    full ranges all occur."""
    ks = synth.randint(seed, 20, S, -3, S_kv - 1).astype(np.int32)
    ke = (ks + synth.randint(seed, 21, S, -2, S_kv)).astype(np.int32)
    return ks, ke


SMALL = [(37, 64, 300, True), (37, 64, 300, False), (50, 32, 129, True), (9, 16, 1000, False),
         (70, 48, 260, True), (1, 64, 1, True), (1, 16, 5, False), (33, 64, 701, False)]


@pytest.mark.parametrize("S,H,S_kv,clean", SMALL)
def test_mqa_logits_small(S, H, S_kv, clean):
    """Every element, ragged ranges (empty, clamped, whole), every head count,
    S and S_kv off the tile sizes."""
    announce(f"mqa small S={S} H={H} S_kv={S_kv} clean={clean}")
    seed = 60 + S + H + S_kv
    q, kv, kv_scale, weights = synth.mqa_tensors(seed, S, H, S_kv)
    ks, ke = ragged_ranges(seed, S, S_kv)
    got = run(q, kv, kv_scale, weights, ks, ke, clean)
    ref = oracle.mqa_logits(q, kv, kv_scale, weights, ks, ke, clean)
    mag = magnitude(q, kv, kv_scale, weights, ks, ke)
    check(got, ref, mag, clean, f"S={S} H={H} S_kv={S_kv} ({dg.last_config()})")


@pytest.mark.parametrize("clean", [True, False])
def test_mqa_logits_scalar_store_path(clean):
    """Output not 16-byte aligned: the kernel falls back to 4-byte stores."""
    S, H, S_kv = 21, 64, 520
    announce(f"mqa misaligned output clean={clean}")
    q, kv, kv_scale, weights = synth.mqa_tensors(61, S, H, S_kv)
    ks, ke = ragged_ranges(61, S, S_kv)
    got = run(q, kv, kv_scale, weights, ks, ke, clean, misalign=True)
    assert "scalar-stores" in dg.last_config(), dg.last_config()
    ref = oracle.mqa_logits(q, kv, kv_scale, weights, ks, ke, clean)
    check(got, ref, magnitude(q, kv, kv_scale, weights, ks, ke), clean, "misaligned")


@pytest.mark.parametrize("clean", [True, False])
def test_mqa_logits_all_ranges_empty(clean):
    S, H, S_kv = 20, 64, 600
    announce(f"mqa empty ranges clean={clean}")
    q, kv, kv_scale, weights = synth.mqa_tensors(62, S, H, S_kv)
    ks = np.full(S, 100, np.int32)
    ke = np.array([100, 50, -1, 0] * 5, np.int32)
    got = run(q, kv, kv_scale, weights, ks, ke, clean)
    if clean:
        assert np.all(np.isneginf(got))
    else:
        assert np.all(got.view(np.uint32) == UNTOUCHED)


def test_mqa_logits_relu_and_identity_exact():
    """kv rows are +-(unit vectors), q[i,h] one-hot with a value of
    magnitude 0.5 .. 4, the scales and weights +-powers of two: every dot
    product is a single exact product, and each logit an fp32-exact sum, so
    the ReLU, the head/lane mapping and the key mapping are checked bit for
    bit."""
    S, H, S_kv = 40, 64, 256
    announce("mqa one-hot exact")
    kv = np.zeros((S_kv, 128), np.uint8)
    j = np.arange(S_kv)
    kv[j, j % 128] = np.where(j % 3 == 0, 0xB8, 0x38)          # -1 or +1 at position j % 128
    q = np.zeros((S, H, 128), np.uint8)
    pos = synth.randint(63, 0, S * H, 0, 127).reshape(S, H)
    code = synth.randint(63, 1, S * H, 0x30, 0x48).reshape(S, H).astype(np.uint8)   # 0.5 .. 4, +-
    sign = (synth.randint(63, 2, S * H, 0, 1).reshape(S, H) << 7).astype(np.uint8)
    for i in range(S):
        q[i, np.arange(H), pos[i]] = code[i] | sign[i]
    kv_scale = np.ldexp(np.float32(1.0), synth.randint(63, 3, S_kv, -3, 3)).astype(np.float32)
    weights = np.ldexp(np.float32(1.0), synth.randint(63, 4, S * H, -2, 2)).reshape(S, H).astype(np.float32)
    weights *= np.where(synth.randint(63, 5, S * H, 0, 3).reshape(S, H) == 0, -1, 1).astype(np.float32)
    ks = np.zeros(S, np.int32)
    ke = np.full(S, S_kv, np.int32)
    got = run(q, kv, kv_scale, weights, ks, ke, True)
    ref = oracle.mqa_logits(q, kv, kv_scale, weights, ks, ke, True)
    assert np.all(ref.astype(np.float32).astype(np.float64) == ref)
    assert np.array_equal(got.astype(np.float64), ref), np.argwhere(got != ref)[:5]


def test_mqa_logits_packed_sequences_sampled():
    """Sequences of mixed lengths packed back to back, causal within each;
    rows sampled around every sequence boundary and at random."""
    lengths = [700, 1, 333, 1200, 64, 900, 129]
    S = S_kv = sum(lengths)
    H = 64
    announce(f"mqa packed sequences {lengths}")
    q, kv, kv_scale, weights = synth.mqa_tensors(64, S, H, S_kv)
    ks, ke = synth.packed_ranges(lengths)
    for clean in (True, False):
        got = run(q, kv, kv_scale, weights, ks, ke, clean)
        bounds = np.cumsum([0] + lengths)
        rows = np.concatenate([bounds[:-1], bounds[1:] - 1, bounds[1:-1] - 2,
                               synth.randint(64, 30, 24, 0, S - 1)])
        rows = np.unique(np.clip(rows, 0, S - 1)).astype(np.int32)
        ref = oracle.mqa_logits_rows(q, kv, kv_scale, weights, ks, ke, clean, rows)
        mag = magnitude(q, kv, kv_scale, weights, ks, ke, rows)
        check(got[rows], ref, mag, clean, f"packed clean={clean} ({dg.last_config()})")


def test_mqa_logits_full_size_sampled():
    """The measured workload (4096 queries, 8192 keys, 64 heads, causal) in
    the launch configuration the benchmark times: sampled rows against the
    oracle, and on every row the -inf tail and finite range."""
    cfg = synth.MQA
    S, S_kv, H = cfg["S"], cfg["S_kv"], cfg["H"]
    announce(f"mqa full size {cfg['name']}")
    q, kv, kv_scale, weights = synth.mqa_tensors(cfg["seed"], S, H, S_kv)
    ks, ke = synth.causal_ranges(S, S_kv)
    got = run(q, kv, kv_scale, weights, ks, ke, True)
    rows = np.unique(np.concatenate([[0, 1, 7, 8, S - 1, S - 2],
                                     synth.randint(cfg["seed"], 30, 26, 0, S - 1)])).astype(np.int32)
    ref = oracle.mqa_logits_rows(q, kv, kv_scale, weights, ks, ke, True, rows)
    mag = magnitude(q, kv, kv_scale, weights, ks, ke, rows)
    check(got[rows], ref, mag, True, f"{cfg['name']} ({dg.last_config()})")
    cols = np.arange(S_kv)[None, :]
    inside = cols < ke[:, None]
    assert np.all(np.isfinite(got[inside]))
    assert np.all(np.isneginf(got[~inside]))


def test_mqa_logits_long_key_axis():
    """Few queries against 70 000 keys (137 chunks), ranges that start and end
    deep inside the key axis, and one range over all of it."""
    S, H, S_kv = 3, 64, 70000
    announce(f"mqa long key axis S={S} S_kv={S_kv}")
    q, kv, kv_scale, weights = synth.mqa_tensors(65, S, H, S_kv)
    ks = np.array([0, 33333, 69990], np.int32)
    ke = np.array([S_kv, 50001, 70100], np.int32)
    for clean in (True, False):
        got = run(q, kv, kv_scale, weights, ks, ke, clean)
        ref = oracle.mqa_logits(q, kv, kv_scale, weights, ks, ke, clean)
        check(got, ref, magnitude(q, kv, kv_scale, weights, ks, ke), clean, f"long keys clean={clean}")
