"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test names what it pins and where that fact comes from:
  * the E4M3FN codec against torch's float8_e4m3fn (a library routine) and
    the closed-form code table in tests/golden/e4m3fn_codes.txt;
  * the encoder's round-to-nearest-even against torch's cast over every fp32
    bit pattern in the E4M3 range, and against the midpoint definition;
  * the quantisers against inputs whose result is known in closed form
    (blocks of exactly representable values with a power-of-two amax);
  * the GEMM against numpy matmul of the de-scaled operands, against integer
    evaluation of a block sum, and against identity/one-hot products;
  * the grouped variants against per-group dense results.
A mistake such as a transposed scale index, a dropped C term or a wrong
tie rule fails at least one of them.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


# ---------------------------------------------------------------- codec


def test_table_equals_torch_float8_e4m3fn():
    table = oracle.e4m3_table()
    ref = torch_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(table), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(table[ok], ref[ok])
    # the sign of zero is part of the format
    assert np.signbit(table[0x80]) and not np.signbit(table[0x00])
    assert np.isnan(table[0x7F]) and np.isnan(table[0xFF])
    assert int(np.isnan(table).sum()) == 2


def test_table_matches_ocp_golden_values():
    table = oracle.e4m3_table()
    n = 0
    with open(os.path.join(GOLDEN, "e4m3fn_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code_s, val_s = line.split()
            code = int(code_s, 16)
            if val_s == "nan":
                assert np.isnan(table[code])
            else:
                v = float(val_s)
                assert table[code] == v, (hex(code), table[code], v)
                assert np.signbit(table[code]) == val_s.startswith("-")
            n += 1
    assert n >= 20


def test_table_monotone_and_symmetric():
    table = oracle.e4m3_table()
    pos = table[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(table[0x80:0xFF], -pos)


def test_encode_decode_roundtrip_all_finite_codes():
    table = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = oracle.e4m3_encode(table[codes].astype(np.float32))
    assert np.array_equal(back, codes)


def _binade_patterns(lo_exp: int, hi_exp: int) -> np.ndarray:
    """All fp32 bit patterns with biased exponent in [lo_exp, hi_exp]."""
    lo = np.uint32(lo_exp << 23)
    hi = np.uint32((hi_exp + 1) << 23)
    return np.arange(lo, hi, dtype=np.uint32)


def test_encode_equals_torch_on_every_fp32_in_range():
    """Every fp32 with 2^-12 <= |x| < 448 (both signs): the oracle encoder and
    torch's round-to-nearest-even cast agree bit for bit.  Above 448 torch does
    not saturate, so that range is pinned separately."""
    n_checked = 0
    for e in range(127 - 12, 127 + 9):          # binades [2^-12, 2^9)
        bits = _binade_patterns(e, e)
        x = bits.view(np.float32)
        x = x[x < 448.0]
        for sign in (1.0, -1.0):
            xs = (x * np.float32(sign)).astype(np.float32)
            got = oracle.e4m3_encode(xs)
            ref = torch_encode(xs)
            bad = np.nonzero(got != ref)[0]
            assert bad.size == 0, (e, xs[bad[:4]], got[bad[:4]], ref[bad[:4]])
            n_checked += xs.size
    assert n_checked > 300_000_000


def test_encode_saturates_and_tiny_values():
    big = np.array([448.0, 448.5, 463.99, 464.0, 479.0, 480.0, 1e6, 3.4e38, np.inf], dtype=np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    # |x| <= 2^-10 (half the smallest subnormal) rounds to zero, keeping the sign
    tiny = np.array([0.0, 2.0 ** -149, 1e-30, 2.0 ** -11, 2.0 ** -10], dtype=np.float32)
    assert np.all(oracle.e4m3_encode(tiny) == 0x00)
    assert np.all(oracle.e4m3_encode(-tiny) == 0x80)
    just_above = np.nextafter(np.float32(2.0 ** -10), np.float32(1.0))
    assert oracle.e4m3_encode(np.array([just_above]))[0] == 0x01
    assert oracle.e4m3_encode(np.array([np.nan], dtype=np.float32))[0] == 0x7F


def test_encode_midpoints_round_to_even():
    """Round to nearest, ties to even, by definition: the midpoint of two
    neighbouring codes goes to the one with an even mantissa; one fp32 ulp
    either side goes to the nearer one."""
    table = oracle.e4m3_table()
    for c in range(0x00, 0x7E):
        lo, hi = table[c], table[c + 1]
        mid = np.float32((lo + hi) / 2.0)
        assert float(mid) == (lo + hi) / 2.0          # midpoints are fp32-exact
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(mid, np.float32(-1.0))
        above = np.nextafter(mid, np.float32(1e9))
        got = oracle.e4m3_encode(np.array([mid, below, above], dtype=np.float32))
        assert list(got) == [even, c, c + 1], (hex(c), got)


# ---------------------------------------------------------------- quantisers


def _representable_blocks(rows, K, seed, block_rows):
    """x = dec(codes) * 2^j, one j per block, each block containing +-448:
    amax = 448 * 2^j, so the scale is exactly 2^j and the codes come back."""
    codes = synth.random_codes(seed, 0, (rows, K))
    nrb = (rows + block_rows - 1) // block_rows
    nkb = K // 128
    j = synth.randint(seed, 3, nrb * nkb, -20, 20).reshape(nrb, nkb)
    for rb in range(nrb):
        for kb in range(nkb):
            r0 = rb * block_rows
            codes[r0, kb * 128 + (rb * 7 + kb * 13) % 128] = 0x7E if (rb + kb) % 2 == 0 else 0xFE
    vals = torch_decode(codes)
    scale = np.ldexp(1.0, np.repeat(np.repeat(j, block_rows, axis=0)[:rows], 128, axis=1))
    x = (vals * scale).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), vals * scale)   # exact
    return codes, j, x


def test_quantize_1x128_exact_on_representable_blocks():
    rows, K = 37, 384
    codes, j, x = _representable_blocks(rows, K, seed=11, block_rows=1)
    q, sf = oracle.quantize_1x128(x)
    assert np.array_equal(q, codes)
    assert sf.shape == (K // 128, 40)       # transposed, rows padded to a multiple of 4
    assert np.array_equal(sf[:, :rows], np.ldexp(np.float32(1.0), j.T).astype(np.float32))


def test_quantize_128x128_exact_on_representable_blocks():
    rows, K = 300, 256                      # last row block is partial (44 rows)
    codes, j, x = _representable_blocks(rows, K, seed=12, block_rows=128)
    q, sf = oracle.quantize_128x128(x)
    assert np.array_equal(q, codes)
    assert sf.shape == (3, 2)
    assert np.array_equal(sf, np.ldexp(np.float32(1.0), j).astype(np.float32))


def test_quantize_zero_block_and_scale_floor():
    x = np.zeros((4, 256), dtype=np.float32)
    x[1, 130] = 2.0
    q, sf = oracle.quantize_1x128(x)
    floor_sf = np.float32(np.float32(1e-4) / np.float32(448.0))
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)
    assert sf[0, 0] == floor_sf and sf[1, 0] == floor_sf
    assert sf[1, 1] == np.float32(2.0) / np.float32(448.0)
    assert q[1, 130] == 0x7E


def _e4m3_half_spacing(y):
    ay = np.abs(y)
    e = np.floor(np.log2(np.maximum(ay, 2.0 ** -6)))
    return np.ldexp(1.0, (e - 3).astype(int)) / 2.0


@pytest.mark.parametrize("kind", ["1x128", "128x128"])
def test_quantize_invariants_on_normal_data(kind):
    x = synth.normal_f32(21, 0, (260, 512))
    if kind == "1x128":
        q, sf = oracle.quantize_1x128(x)
        s_full = np.repeat(sf[:, :260].T, 128, axis=1)
    else:
        q, sf = oracle.quantize_128x128(x)
        s_full = np.repeat(np.repeat(sf, 128, axis=0)[:260], 128, axis=1)
    vals = torch_decode(q)
    y = x.astype(np.float64) / s_full
    # round-to-nearest within half a spacing (+ the fp32 division's rounding)
    err = np.abs(vals - y)
    assert np.all(err <= _e4m3_half_spacing(y) + np.abs(y) * 2.0 ** -23)
    # the element of largest magnitude in each block maps to +-448
    blocks = np.abs(vals).reshape(-1) if kind == "1x128" else None
    if kind == "1x128":
        per_block = np.abs(vals).reshape(260, 4, 128).max(axis=2)
        assert np.all(per_block == 448.0)
    else:
        for rb in range(3):
            for kb in range(4):
                blk = np.abs(vals[rb * 128:(rb + 1) * 128, kb * 128:(kb + 1) * 128])
                assert blk.max() == 448.0
    del blocks


def test_quantize_groups_do_not_share_blocks_and_ld_padding_untouched():
    x = synth.normal_f32(22, 0, (2, 130, 256))
    x[1] *= 100.0
    q, sf = oracle.quantize_128x128(x)
    for g in range(2):
        qg, sfg = oracle.quantize_128x128(x[g])
        assert np.array_equal(q[g], qg) and np.array_equal(sf[g], sfg)
    q1, sf1 = oracle.quantize_1x128(x, ld_sf=136)
    assert np.all(sf1[:, :, 130:] == 0.0)        # zero-initialised padding stays
    for g in range(2):
        qg, sfg = oracle.quantize_1x128(x[g])
        assert np.array_equal(q1[g], qg) and np.array_equal(sf1[g][:, :130], sfg[:, :130])


@pytest.mark.parametrize("kind", ["1x128", "128x128"])
def test_quantize_ue8m0_scales_are_minimal_powers_of_two(kind):
    """Power-of-two scale variant: every scale is a power of two, at least
    the block's amax/448 (so nothing saturates) and less than twice it (the
    smallest such power).  Data spans many binades, including blocks whose
    amax/448 is itself a power of two and an all-zero block."""
    x = synth.normal_f32(23, 0, (260, 512)) * np.ldexp(np.float32(1.0), synth.randint(23, 1, 260 * 512, -20, 20).reshape(260, 512)).astype(np.float32)
    x[5, :128] = 0.0
    x[6, :128] = 0.0
    x[6, 7] = -448.0 * 2.0 ** -5
    if kind == "1x128":
        q, sf = oracle.quantize_1x128(x, ue8m0=True)
        amax = np.abs(x).reshape(260, 4, 128).max(axis=2).T            # [K/128, rows]
        sf = sf[:, :260]
    else:
        q, sf = oracle.quantize_128x128(x, ue8m0=True)
        amax = np.array([[np.abs(x[rb * 128:(rb + 1) * 128, kb * 128:(kb + 1) * 128]).max() for kb in range(4)]
                         for rb in range(3)])
    quot = np.maximum(amax, np.float32(1e-4)).astype(np.float32) / np.float32(448.0)
    mant, _ = np.frexp(sf)
    assert np.all(mant == 0.5)                       # powers of two
    assert np.all(sf >= quot) and np.all(sf / 2 < quot)
    if kind == "1x128":
        assert sf[0, 6] == np.float32(2.0 ** -5)    # amax/448 already a power of two: kept
        assert sf[0, 5] == np.float32(2.0 ** -22)   # zero block: 1e-4/448 rounded up


@pytest.mark.parametrize("kind", ["1x128", "128x128"])
def test_quantize_ue8m0_codes_are_the_e4m3_rounding_of_x_times_two_to_minus_e(kind):
    """Dividing by a power of two is exact, so the codes must equal torch's
    own E4M3 cast of x * 2^-e (an encoder that shares nothing with the
    oracle's), with no saturation."""
    x = synth.normal_f32(24, 0, (200, 384)) * np.float32(3.0)
    if kind == "1x128":
        q, sf = oracle.quantize_1x128(x, ue8m0=True)
        s_full = np.repeat(sf[:, :200].T, 128, axis=1)
    else:
        q, sf = oracle.quantize_128x128(x, ue8m0=True)
        s_full = np.repeat(np.repeat(sf, 128, axis=0)[:200], 128, axis=1)
    _, e = np.frexp(s_full)
    y = np.ldexp(x, 1 - e).astype(np.float32)       # x / s exactly (s = 2^(e-1))
    assert np.all(np.abs(y) <= 448.0)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


def _packed_golden():
    rows = []
    with open(os.path.join(GOLDEN, "ue8m0_packed_words.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                o, q, w0, w1 = line.split()
                rows.append((int(o), int(q), int(w0, 16), int(w1, 16)))
    words = np.zeros((2, 2, 2), dtype=np.uint32)
    for o, q, w0, w1 in rows:
        words[o, q] = (w0, w1)
    log2 = np.array([[[0, -3], [1, 5], [-1, 0], [-10, 12], [2, -126]],
                     [[127, 7], [-126, 7], [3, 7], [4, 7], [-20, 0]]], dtype=np.int32)   # [o][kb][i]
    return np.ldexp(np.float32(1.0), log2).astype(np.float32), words


def test_ue8m0_pack_matches_hand_worked_words():
    """Packing the hand-worked example of tests/golden/ue8m0_packed_words.txt
    (four K blocks per word, block 4q + j in byte j, zero high bytes in the
    last word) gives exactly the words derived there, and unpacking them
    returns the scales."""
    sf, words = _packed_golden()
    got = oracle.pack_ue8m0(sf, k_axis=1)
    assert got.shape == (2, 2, 2) and got.dtype == np.uint32
    assert np.array_equal(got, words), [hex(v) for v in got.reshape(-1)]
    assert np.array_equal(oracle.unpack_ue8m0(words, 5, k_axis=1), sf)


def test_ue8m0_code_is_the_ieee_exponent_field_of_every_normal_power_of_two():
    """A UE8M0 code (bias 127) of 2^k is the biased exponent field of the
    IEEE-754 single 2^k, read here from the bit pattern (a route that shares
    nothing with the oracle's frexp); decoding returns 2^k exactly."""
    for k in range(-126, 128):
        s = np.float32(np.ldexp(1.0, k))
        field = int(np.array([s], dtype=np.float32).view(np.uint32)[0] >> 23) & 0xFF
        assert oracle.ue8m0_encode(s) == field == k + 127
        assert oracle.ue8m0_decode(k + 127) == 2.0 ** k


@pytest.mark.parametrize("K", [128, 384, 512, 640, 1152])
def test_ue8m0_pack_round_trips_quantiser_scales_in_both_layouts(K):
    """The power-of-two quantisers' scales survive pack -> unpack in the
    layouts the GEMMs take them in (sfa [K/128][ld] packed along its first
    axis, sfb [G][N/128][K/128] along its last), for K-block counts that do
    and do not fill the last word (whose unused high bytes stay zero)."""
    x = synth.normal_f32(31, 0, (70, K)) * np.ldexp(np.float32(1.0), synth.randint(31, 1, 70 * K, -30, 30).reshape(70, K)).astype(np.float32)
    _, sfa = oracle.quantize_1x128(x, ue8m0=True)
    xb = synth.normal_f32(31, 2, (2, 200, K))
    _, sfb = oracle.quantize_128x128(xb, ue8m0=True)
    nkb = K // 128
    pa = oracle.pack_ue8m0(sfa[:, :70].copy(), k_axis=0)
    assert pa.shape == ((nkb + 3) // 4, 70)
    assert np.array_equal(oracle.unpack_ue8m0(pa, nkb, k_axis=0), sfa[:, :70])
    pb = oracle.pack_ue8m0(sfb, k_axis=-1)
    assert pb.shape == (2, 2, (nkb + 3) // 4)
    assert np.array_equal(oracle.unpack_ue8m0(pb, nkb, k_axis=-1), sfb)
    if nkb % 4:
        assert np.all(pb[..., -1] >> (8 * (nkb % 4)) == 0)


def test_quantize_ue8m0_equals_plain_when_scales_are_powers_of_two():
    """Blocks whose amax is 448 times a power of two have a power-of-two
    plain scale already: both quantisers give the same codes and scales."""
    x = synth.normal_f32(25, 0, (64, 256))
    for r in range(64):
        for kb in range(2):
            blk = x[r, kb * 128:(kb + 1) * 128]
            top = np.float32(448.0 * 2.0 ** ((r + kb) % 9 - 4))
            i = np.argmax(np.abs(blk))
            blk *= top / np.abs(blk[i])
            np.clip(blk, -top, top, out=blk)
            blk[i] = top if blk[i] > 0 else -top       # amax exactly 448 * 2^k
    q0, s0 = oracle.quantize_1x128(x)
    q1, s1 = oracle.quantize_1x128(x, ue8m0=True)
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


# ---------------------------------------------------------------- GEMM


def _expand_scales(sfa, sfb, M, N, K):
    SA = np.repeat(sfa[:, :M].astype(np.float64).T, 128, axis=1)          # [M, K]
    SB = np.repeat(np.repeat(sfb.astype(np.float64), 128, axis=0)[:N], 128, axis=1)  # [N, K]
    return SA, SB


def _random_problem(M, N, K, seed, with_c=True):
    a = synth.random_codes(seed, 0, (M, K))
    b = synth.random_codes(seed, 1, (N, K))
    ld = oracle.sf_aligned(M)
    sfa = np.zeros((K // 128, ld), dtype=np.float32)
    sfa[:, :M] = (synth.uniform(seed, 4, (K // 128) * M).reshape(K // 128, M) * 4 + 0.01).astype(np.float32)
    sfb = (synth.uniform(seed, 5, ((N + 127) // 128) * (K // 128)).reshape(-1, K // 128) * 4 + 0.01).astype(np.float32)
    c = synth.normal_bf16_bits(seed, 2, (M, N)) if with_c else None
    return a, sfa, b, sfb, c


@pytest.mark.parametrize("M,N,K,with_c", [(37, 200, 384, True), (5, 131, 256, False), (64, 1, 128, True)])
def test_gemm_equals_matmul_of_descaled_operands(M, N, K, with_c):
    """sum_kb sfa*sfb*blocksum == (dec(A)*SA) @ (dec(B)*SB)^T: scales are constant
    inside a block, so the two agree in exact arithmetic.  numpy's float64
    matmul is the library routine; the bound is its own rounding."""
    a, sfa, b, sfb, c = _random_problem(M, N, K, seed=M * 1000 + N)
    d = oracle.gemm_nt(a, sfa, b, sfb, c)
    SA, SB = _expand_scales(sfa, sfb, M, N, K)
    Ad = torch_decode(a) * SA
    Bd = torch_decode(b) * SB
    ref = Ad @ Bd.T
    if c is not None:
        ref = ref + synth.bf16_bits_to_f32(c).astype(np.float64)
    mag = np.abs(Ad) @ np.abs(Bd).T + (0 if c is None else np.abs(synth.bf16_bits_to_f32(c)))
    assert np.all(np.abs(d - ref) <= mag * 2.0 ** -48)


@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K", [(48, 160, 256), (128, 96, 128)])
def test_gemm_layouts_equal_matmul_in_the_stated_orientation(layout, M, N, K):
    """D = C + A @ B in each stored layout (nn: a[M,K], b[K,N]; tn: a[K,M],
    b[K,N]; tt: a[K,M], b[N,K]): numpy matmul of the de-scaled operands taken
    in the orientation the layout names (a.T where A is stored [K,M], b where
    B is stored [K,N]).  M == K in one case, so that reading a stored [K,M]
    as [M,K] would go unnoticed by the shapes alone."""
    a, sfa, b, sfb, c = _random_problem(M, N, K, seed=M + N + K + len(layout))
    a_st = np.ascontiguousarray(a.T) if layout[0] == "t" else a
    b_st = np.ascontiguousarray(b.T) if layout[1] == "n" else b
    d = oracle.gemm_layout(layout, a_st, sfa, b_st, sfb, c)
    SA, SB = _expand_scales(sfa, sfb, M, N, K)
    A_mk = (torch_decode(a_st).T if layout[0] == "t" else torch_decode(a_st)) * SA       # [M, K]
    B_kn = (torch_decode(b_st) if layout[1] == "n" else torch_decode(b_st).T) * SB.T     # [K, N]
    ref = A_mk @ B_kn + synth.bf16_bits_to_f32(c).astype(np.float64)
    mag = np.abs(A_mk) @ np.abs(B_kn) + np.abs(synth.bf16_bits_to_f32(c))
    assert np.all(np.abs(d - ref) <= mag * 2.0 ** -48)
    ms = np.array([0, M - 1, M // 2], np.int32)
    ns = np.array([N - 1, 0, N // 3], np.int32)
    assert np.array_equal(oracle.gemm_layout_at(layout, a_st, sfa, b_st, sfb, c, ms, ns), d[ms, ns])


def test_gemm_single_block_unit_scales_is_exact_matmul():
    M, N, K = 19, 23, 128
    a = synth.random_codes(31, 0, (M, K))
    b = synth.random_codes(31, 1, (N, K))
    sfa = np.ones((1, oracle.sf_aligned(M)), dtype=np.float32)
    sfb = np.ones((1, 1), dtype=np.float32)
    d = oracle.gemm_nt(a, sfa, b, sfb, None)
    ref = torch_decode(a) @ torch_decode(b).T          # every partial sum is exact
    assert np.array_equal(d, ref)


def test_block_dot_is_exact_integer_sum():
    """Block sum in units of 2^-18 from integer arithmetic on decoded values."""
    a = synth.random_codes(41, 0, (50, 128))
    b = synth.random_codes(41, 1, (50, 128))
    a[0, :] = 0x7E
    b[0, :] = 0x7E                       # largest magnitude products
    a[1, :] = 0x01
    b[1, :] = 0x81                       # smallest subnormal products
    ia = (torch_decode(a) * 512).astype(np.int64)
    ib = (torch_decode(b) * 512).astype(np.int64)
    assert np.array_equal(ia.astype(np.float64) / 512, torch_decode(a))
    for i in range(50):
        exact = int(np.sum(ia[i] * ib[i]))
        assert oracle.block_dot(a[i], b[i]) == exact / 2.0 ** 18


def test_gemm_identity_and_power_of_two_scales_exact():
    """B = identity (code 0x38 = 1.0 on the diagonal), power-of-two scales: every
    D[m,n] is the single product dec(A[m,n]) * sfa[n/128][m] * sfb[n/128][n/128]."""
    M, K = 40, 384
    N = K
    a = synth.random_codes(51, 0, (M, K))
    b = np.zeros((N, K), dtype=np.uint8)
    b[np.arange(N), np.arange(N)] = 0x38
    ea = synth.randint(51, 4, (K // 128) * M, -8, 8).reshape(K // 128, M)
    eb = synth.randint(51, 5, (N // 128) * (K // 128), -8, 8).reshape(N // 128, K // 128)
    sfa = np.zeros((K // 128, oracle.sf_aligned(M)), dtype=np.float32)
    sfa[:, :M] = np.ldexp(1.0, ea)
    sfb = np.ldexp(np.float32(1.0), eb).astype(np.float32)
    d = oracle.gemm_nt(a, sfa, b, sfb, None)
    av = torch_decode(a)
    for n in range(N):
        kb = n // 128
        expect = av[:, n] * sfa[kb, :M].astype(np.float64) * float(sfb[kb, kb])
        assert np.array_equal(d[:, n], expect)


def test_gemm_zero_a_returns_c_exactly():
    M, N, K = 9, 140, 256
    a = np.zeros((M, K), dtype=np.uint8)
    _, sfa, b, sfb, c = _random_problem(M, N, K, seed=61)
    d = oracle.gemm_nt(a, sfa, b, sfb, c)
    assert np.array_equal(d, synth.bf16_bits_to_f32(c).astype(np.float64))


def test_gemm_elem_at_and_full_agree():
    M, N, K = 33, 150, 256
    a, sfa, b, sfb, c = _random_problem(M, N, K, seed=71)
    d = oracle.gemm_nt(a, sfa, b, sfb, c)
    ms = synth.randint(71, 6, 100, 0, M - 1)
    ns = synth.randint(71, 7, 100, 0, N - 1)
    at = oracle.gemm_nt_at(a, sfa, b, sfb, c, ms, ns)
    assert np.array_equal(at, d[ms, ns])
    assert oracle.gemm_nt_elem(a, sfa, b, sfb, c, 5, 149) == d[5, 149]


# ---------------------------------------------------------------- grouped


def _contiguous_problem(counts, N, K, seed):
    m_idx = synth.contiguous_m_indices(counts)
    M_total = m_idx.size
    G = len(counts)
    a = synth.random_codes(seed, 0, (M_total, K))
    b = synth.random_codes(seed, 1, (G, N, K))
    sfa = (synth.uniform(seed, 4, (K // 128) * M_total).reshape(K // 128, M_total) + 0.5).astype(np.float32)
    sfb = (synth.uniform(seed, 5, G * ((N + 127) // 128) * (K // 128)).reshape(G, -1, K // 128) + 0.5).astype(np.float32)
    c = synth.normal_bf16_bits(seed, 2, (M_total, N))
    return a, sfa, b, sfb, c, m_idx


def test_contiguous_equals_per_group_dense_and_skips_padding():
    counts = [1, 128, 130, 0, 77]
    N, K = 136, 256
    a, sfa, b, sfb, c, m_idx = _contiguous_problem(counts, N, K, seed=81)
    assert m_idx.size % 128 == 0
    d = oracle.m_grouped_contiguous(a, sfa, b, sfb, c, m_idx)
    for g in range(len(counts)):
        rows = np.nonzero(m_idx == g)[0]
        assert rows.size == counts[g]
        if rows.size == 0:
            continue
        dense = oracle.gemm_nt(np.ascontiguousarray(a[rows]),
                               np.ascontiguousarray(np.pad(sfa[:, rows], ((0, 0), (0, (-rows.size) % 4)))),
                               np.ascontiguousarray(b[g]), np.ascontiguousarray(sfb[g]),
                               np.ascontiguousarray(c[rows]))
        assert np.array_equal(d[rows], dense)
    assert np.all(np.isnan(d[m_idx < 0]))
    ms = np.arange(m_idx.size, dtype=np.int32)
    ns = (ms * 7) % N
    at = oracle.m_grouped_contiguous_at(a, sfa, b, sfb, c, m_idx, ms, ns)
    assert np.array_equal(np.isnan(at), m_idx < 0)
    ok = m_idx >= 0
    assert np.array_equal(at[ok], d[ms[ok], ns[ok]])


def test_masked_equals_per_group_dense_and_leaves_rows_untouched():
    G, M_cap, N, K = 5, 130, 72, 256
    seed = 91
    a = synth.random_codes(seed, 0, (G, M_cap, K))
    b = synth.random_codes(seed, 1, (G, N, K))
    ld = oracle.sf_aligned(M_cap)
    sfa = (synth.uniform(seed, 4, G * (K // 128) * ld).reshape(G, K // 128, ld) + 0.5).astype(np.float32)
    sfb = (synth.uniform(seed, 5, G * 1 * (K // 128)).reshape(G, 1, K // 128) + 0.5).astype(np.float32)
    masked_m = np.array([0, 1, 129, 130, 500], dtype=np.int32)   # 500 clamps to M_cap
    d = oracle.m_grouped_masked(a, sfa, b, sfb, None, masked_m)
    for g in range(G):
        mm = min(max(int(masked_m[g]), 0), M_cap)
        if mm:
            dense = oracle.gemm_nt(np.ascontiguousarray(a[g, :mm]),
                                   np.ascontiguousarray(sfa[g]), np.ascontiguousarray(b[g]),
                                   np.ascontiguousarray(sfb[g]), None)
            assert np.array_equal(d[g, :mm], dense)
        assert np.all(np.isnan(d[g, mm:]))
    gs = np.repeat(np.arange(G), 3).astype(np.int32)
    ms = np.tile(np.array([0, 1, 129]), G).astype(np.int32)
    ns = np.tile(np.array([0, 33, 71]), G).astype(np.int32)
    at = oracle.m_grouped_masked_at(a, sfa, b, sfb, None, masked_m, gs, ms, ns)
    assert np.array_equal(np.isnan(at), np.isnan(d[gs, ms, ns]))
    ok = ~np.isnan(at)
    assert np.array_equal(at[ok], d[gs, ms, ns][ok])


def test_masked_negative_count_is_zero_rows():
    a = synth.random_codes(1, 0, (1, 8, 128))
    b = synth.random_codes(1, 1, (1, 16, 128))
    sfa = np.ones((1, 1, 8), dtype=np.float32)
    sfb = np.ones((1, 1, 1), dtype=np.float32)
    d = oracle.m_grouped_masked(a, sfa, b, sfb, None, np.array([-3], dtype=np.int32))
    assert np.all(np.isnan(d))


# ---------------------------------------------------------------- MQA logits
# The non-paged FP8 MQA logits of the DeepSeek v3.2 indexer (GeekNews summary
# of the DeepGEMM README, section on the MQA kernels for the v3.2 Indexer):
# for query token i and key token j in [k_start[i], k_end[i]), the logit is
# the weights[i]-weighted sum over heads of ReLU(kv_scale[j] * q[i,h].kv[j]).


def _mqa_inputs(seed, S, H, D, Skv):
    q = synth.random_codes(seed, 0, (S, H, D))
    kv = synth.random_codes(seed, 1, (Skv, D))
    kv_scale = (0.5 + synth.uniform(seed, 2, Skv)).astype(np.float32)
    weights = synth.normal_f32(seed, 3, (S, H))
    ks = synth.randint(seed, 4, S, -2, Skv // 2).astype(np.int32)
    ke = (ks + synth.randint(seed, 5, S, -1, Skv + 3)).astype(np.int32)
    return q, kv, kv_scale, weights, ks, ke


@pytest.mark.parametrize("clean", [True, False])
def test_mqa_logits_brute_force_over_torch_decode(clean):
    """Tiny case evaluated with torch's E4M3 decode and integer dot products
    (E4M3 values are multiples of 2^-9, so q.kv * 2^18 is an exact integer);
    the scale, ReLU, weighting and head sum follow in fp64, heads in order."""
    S, H, D, Skv = 6, 3, 256, 11
    q, kv, kv_scale, weights, ks, ke = _mqa_inputs(50, S, H, D, Skv)
    got = oracle.mqa_logits(q, kv, kv_scale, weights, ks, ke, clean)
    qi = (torch_decode(q) * 512).astype(np.int64)
    ki = (torch_decode(kv) * 512).astype(np.int64)
    for i in range(S):
        lo, hi = min(max(int(ks[i]), 0), Skv), min(max(int(ke[i]), 0), Skv)
        for j in range(Skv):
            if not (lo <= j < hi):
                if clean:
                    assert got[i, j] == -np.inf
                else:
                    assert np.isnan(got[i, j])
                continue
            want = 0.0
            for h in range(H):
                dot = float(int(np.dot(qi[i, h], ki[j]))) * 2.0 ** -18
                want += float(weights[i, h]) * max(float(kv_scale[j]) * dot, 0.0)
            assert got[i, j] == want, (i, j, got[i, j], want)


def test_mqa_logits_one_hot_closed_form():
    """q[i,h] has a single non-zero x_{i,h} at position p(i,h), kv[j] a single
    non-zero y_j at position r(j): the dot is x*y when the positions meet and
    0 otherwise, so each logit is a short sum fixed in advance."""
    S, H, D, Skv = 4, 2, 128, 5
    q = np.zeros((S, H, D), np.uint8)
    kv = np.zeros((Skv, D), np.uint8)
    pos_q = [[3, 7], [7, 3], [100, 3], [5, 5]]
    val_q = [[0x40, 0xC0], [0x38, 0x48], [0x30, 0x38], [0x38, 0xB8]]  # 2,-2 | 1,4 | 0.5,1 | 1,-1
    pos_kv = [3, 7, 5, 100, 3]
    val_kv = [0x38, 0x40, 0x44, 0xB8, 0xC0]                             # 1, 2, 3, -1, -2
    for i in range(S):
        for h in range(H):
            q[i, h, pos_q[i][h]] = val_q[i][h]
    for j in range(Skv):
        kv[j, pos_kv[j]] = val_kv[j]
    kv_scale = np.array([1.0, 0.5, 2.0, 4.0, 0.25], np.float32)
    weights = np.array([[1.0, 1.0], [0.5, 2.0], [1.0, -1.0], [3.0, 3.0]], np.float32)
    ks = np.zeros(S, np.int32)
    ke = np.full(S, Skv, np.int32)
    got = oracle.mqa_logits(q, kv, kv_scale, weights, ks, ke, True)
    want = np.array([
        # i=0: h0 (2 at 3), h1 (-2 at 7)
        [2 * 1 * 1.0, 0.0, 0.0, 0.0, 0.0],         # j=1: h1 gives -2*2*0.5<0; j=4: 2*-2*.25<0
        # i=1: h0 (1 at 7) w .5, h1 (4 at 3) w 2
        [2 * 4 * 1 * 1.0, 0.5 * 1 * 2 * 0.5, 0.0, 0.0, 0.0],   # j=4: 4*-2 <0
        # i=2: h0 (0.5 at 100) w 1, h1 (1 at 3) w -1
        [-1 * 1 * 1.0, 0.0, 0.0, 0.0, 0.0],        # j=3: 0.5*-1*4 <0 -> 0
        # i=3: h0 (1 at 5), h1 (-1 at 5), w 3
        [0.0, 0.0, 3 * 1 * 3 * 2.0, 0.0, 0.0],     # h1: -3*2 < 0 -> 0
    ])
    assert np.array_equal(got, want), got


def test_mqa_logits_relu_cuts_negative_heads_only():
    """kv = -q[i,0] makes head 0's product negative (dropped) and leaves a
    head whose q equals kv with its full square norm."""
    D = 128
    x = synth.random_codes(51, 0, (D,))
    neg = x ^ np.uint8(0x80)
    q = np.stack([x, neg])[None]                 # [1, 2, D]: head 0 = x, head 1 = -x
    kv = neg[None]                               # kv = -x
    norm2 = float(np.sum(torch_decode(x) ** 2))
    got = oracle.mqa_logits(q, kv, np.ones(1, np.float32), np.array([[5.0, 0.25]], np.float32),
                            np.zeros(1, np.int32), np.ones(1, np.int32), True)
    assert got[0, 0] == 0.25 * norm2


def test_mqa_logits_linear_in_weights_and_homogeneous_in_scale():
    S, H, D, Skv = 5, 4, 128, 7
    q, kv, kv_scale, weights, ks, ke = _mqa_inputs(52, S, H, D, Skv)
    ks[:] = 0
    ke[:] = Skv
    # weights that are small integers keep every sum exact
    w1 = synth.randint(52, 9, S * H, -4, 5).reshape(S, H).astype(np.float32)
    w2 = synth.randint(52, 10, S * H, -4, 5).reshape(S, H).astype(np.float32)
    sc = np.ldexp(np.float32(1.0), synth.randint(52, 11, Skv, -3, 4)).astype(np.float32)
    l1 = oracle.mqa_logits(q, kv, sc, w1, ks, ke, True)
    l2 = oracle.mqa_logits(q, kv, sc, w2, ks, ke, True)
    l12 = oracle.mqa_logits(q, kv, sc, w1 + w2, ks, ke, True)
    assert np.array_equal(l12, l1 + l2)
    l_half = oracle.mqa_logits(q, kv, (sc * 0.5).astype(np.float32), w1, ks, ke, True)
    assert np.array_equal(l_half * 2, l1)
    # a head with weight one and all others zero gives that head's ReLU(dot)
    dots = np.einsum("shd,kd->shk", torch_decode(q), torch_decode(kv))
    for h in range(H):
        w = np.zeros((S, H), np.float32)
        w[:, h] = 1.0
        lh = oracle.mqa_logits(q, kv, np.ones(Skv, np.float32), w, ks, ke, True)
        assert np.array_equal(lh, np.maximum(dots[:, h, :], 0.0))


def test_mqa_logits_ranges_clamped_and_rows_form_agrees():
    S, H, D, Skv = 7, 2, 128, 9
    q, kv, kv_scale, weights, _, _ = _mqa_inputs(53, S, H, D, Skv)
    ks = np.array([-5, 0, 3, 8, 9, 4, 20], np.int32)
    ke = np.array([2, 9, 3, 100, 12, 1, 30], np.int32)
    full = oracle.mqa_logits(q, kv, kv_scale, weights, np.zeros(S, np.int32), np.full(S, Skv, np.int32), True)
    for clean in (True, False):
        got = oracle.mqa_logits(q, kv, kv_scale, weights, ks, ke, clean)
        for i in range(S):
            lo, hi = min(max(ks[i], 0), Skv), min(max(ke[i], 0), Skv)
            inside = np.zeros(Skv, bool)
            inside[lo:max(lo, hi)] = True
            assert np.array_equal(got[i, inside], full[i, inside])
            if clean:
                assert np.all(got[i, ~inside] == -np.inf)
            else:
                assert np.all(np.isnan(got[i, ~inside]))
        # rows 2 (empty), 4 (start at Skv) and 5 (end before start) have no key
        assert not np.any(np.isfinite(got[[2, 4, 5]]))
        rows = np.array([6, 0, 3, 3], np.int32)
        sub = oracle.mqa_logits_rows(q, kv, kv_scale, weights, ks, ke, clean, rows)
        assert np.array_equal(sub, got[rows], equal_nan=True)


# ---------------------------------------------------------------- K-grouped TN
# MoE weight gradient (GeekNews summary of the DeepGEMM README, "Dense and
# Grouped GEMM": groups along K, M and N fixed): d[g] = c[g] + A_g^T B_g with
# A_g, B_g the K rows of group g, one scale per 128 K rows and per column.


def _kg_problem(seed, ks, M, N, with_c=True):
    K = int(np.sum(ks))
    a = synth.random_codes(seed, 0, (K, M))
    b = synth.random_codes(seed, 1, (K, N))
    sfa = (synth.uniform(seed, 4, (K // 128) * M).reshape(K // 128, M) * 4 + 0.01).astype(np.float32)
    sfb = (synth.uniform(seed, 5, (K // 128) * N).reshape(K // 128, N) * 4 + 0.01).astype(np.float32)
    c = synth.normal_f32(seed, 2, (len(ks), M, N)) if with_c else None
    return a, sfa, b, sfb, np.asarray(ks, np.int32), c


def test_k_grouped_equals_per_group_matmul_of_descaled_operands():
    ks = [256, 0, 128, 384]
    M, N = 40, 72
    a, sfa, b, sfb, ks, c = _kg_problem(70, ks, M, N)
    d = oracle.k_grouped_tn(a, sfa, b, sfb, ks, c)
    Ad = torch_decode(a) * np.repeat(sfa.astype(np.float64), 128, axis=0)       # [K, M]
    Bd = torch_decode(b) * np.repeat(sfb.astype(np.float64), 128, axis=0)       # [K, N]
    k0 = 0
    for g, kg in enumerate(ks):
        ref = Ad[k0:k0 + kg].T @ Bd[k0:k0 + kg] + c[g]
        mag = np.abs(Ad[k0:k0 + kg]).T @ np.abs(Bd[k0:k0 + kg]) + np.abs(c[g])
        assert np.all(np.abs(d[g] - ref) <= mag * 2.0 ** -48), g
        k0 += kg
    assert np.array_equal(d[1], c[1].astype(np.float64))            # empty group: D = C exactly


def test_k_grouped_reduces_to_the_nt_gemm_with_block_constant_column_scales():
    """With sfb constant over each 128 columns, group g is the NT GEMM of the
    transposed group rows with 128x128 B scales: same block sums, same order,
    so the two oracle functions agree bit for bit."""
    ks = [128, 256, 384]
    M, N = 24, 200
    a, sfa, b, sfb, ks, _ = _kg_problem(71, ks, M, N, with_c=False)
    s_nt = (synth.uniform(71, 8, ((N + 127) // 128) * (a.shape[0] // 128)).reshape(-1, a.shape[0] // 128) * 3
            + 0.1).astype(np.float32)                                # [ceil(N/128), K/128]
    sfb = np.ascontiguousarray(np.repeat(s_nt.T, 128, axis=1)[:, :N])   # [K/128, N]
    d = oracle.k_grouped_tn(a, sfa, b, sfb, ks, None)
    k0 = 0
    for g, kg in enumerate(ks):
        a_g = np.ascontiguousarray(a[k0:k0 + kg].T)                  # [M, kg]
        b_g = np.ascontiguousarray(b[k0:k0 + kg].T)                  # [N, kg]
        sfa_g = np.zeros((kg // 128, oracle.sf_aligned(M)), np.float32)
        sfa_g[:, :M] = sfa[k0 // 128:(k0 + kg) // 128]
        sfb_g = np.ascontiguousarray(s_nt[:, k0 // 128:(k0 + kg) // 128])
        assert np.array_equal(d[g], oracle.gemm_nt(a_g, sfa_g, b_g, sfb_g, None)), g
        k0 += kg


def test_k_grouped_split_group_sums_and_sampled_form():
    M, N = 16, 48
    a, sfa, b, sfb, _, _ = _kg_problem(72, [384], M, N, with_c=False)
    whole = oracle.k_grouped_tn(a, sfa, b, sfb, np.array([384], np.int32))
    parts = oracle.k_grouped_tn(a, sfa, b, sfb, np.array([128, 256], np.int32))
    mag = oracle.k_grouped_tn(a & np.uint8(0x7F), sfa, b & np.uint8(0x7F), sfb, np.array([384], np.int32))
    assert np.all(np.abs(parts[0] + parts[1] - whole[0]) <= 2.0 ** -48 * mag[0])
    gs = np.array([0, 1, 1, 0], np.int32)
    ms = np.array([0, 15, 3, 7], np.int32)
    ns = np.array([47, 0, 20, 9], np.int32)
    at = oracle.k_grouped_tn_at(a, sfa, b, sfb, np.array([128, 256], np.int32), None, gs, ms, ns)
    assert np.array_equal(at, parts[gs, ms, ns])


def test_block_scales_of_an_infinite_block_stay_infinite():
    """A block holding +-inf has the IEEE quotient inf / 448 = inf as its
    scale; there is no power of two above it, so the power-of-two form keeps
    inf as well (its codes are then zeros of the values' signs, and 0x7f for
    the infinities, inf / inf being NaN)."""
    assert oracle.block_scale(np.float32(np.inf)) == np.inf
    assert oracle.block_scale_ue8m0(np.float32(np.inf)) == np.inf
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, :4] = [np.inf, -1.5, 2.0, -0.0]
    for ue in (False, True):
        q, sf = oracle.quantize_1x128(x, ue8m0=ue)
        assert sf[0, 0] == np.inf
        assert list(q[0, :4]) == [0x7F, 0x80, 0x00, 0x80]
