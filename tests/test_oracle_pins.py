"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against what the pages or the mathematics fix:
spec values of the FP8 format, hand-derived closed forms (tests/golden/),
library routines for special cases (torch's float8_e4m3fn codec, numpy fp64
matmul), invariants of a rotation and of block quantisation, and brute force
on tiny inputs.  None of them re-types the oracle's own formula.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- helpers (independent routes)
def _all_codes():
    return np.arange(256, dtype=np.uint8)


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    """Library route: torch's float8_e4m3fn dtype."""
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def _finite_table():
    """(values, codes) of every finite code, sorted by value, from torch's decoder."""
    codes = _all_codes()
    vals = _torch_decode(codes).astype(np.float64)
    keep = np.isfinite(vals)
    return vals[keep], codes[keep]


def _nearest_even_by_search(x: np.ndarray) -> np.ndarray:
    """Brute force: nearest finite e4m3fn value by exhaustive search, ties to
    the code with an even mantissa LSB, saturating beyond 448.  Sign handled
    by symmetry so -0 keeps its sign."""
    vals, codes = _finite_table()
    pos = vals >= 0
    pv = vals[pos & ~((vals == 0) & (codes >= 0x80))]
    pc = codes[pos & ~((vals == 0) & (codes >= 0x80))]
    order = np.argsort(pv)
    pv, pc = pv[order], pc[order]
    a = np.abs(x.astype(np.float64))
    d = np.abs(a[:, None] - pv[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among ties prefer the even mantissa LSB (code & 1 == 0)
    even = (pc[None, :] & 1) == 0
    pick = np.where(cand & even, 1, 0) * 2 + np.where(cand, 1, 0)
    idx = pick.argmax(axis=1)
    out = pc[idx].astype(np.uint8)
    out = np.where(a >= 448.0, np.uint8(0x7E), out)
    sign = np.signbit(x.astype(np.float32))
    return np.where(sign, out | np.uint8(0x80), out).astype(np.uint8)


def _read_golden(name):
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ---------------------------------------------------------------- e4m3fn codec
def test_decode_spec_values(golden_dir):
    for row in _read_golden("e4m3fn_spec_values.txt"):
        code_s, val_s = row.split()
        code = int(code_s, 16)
        got = float(oracle.e4m3_decode(np.array([code], np.uint8))[0])
        if val_s == "nan":
            assert math.isnan(got), hex(code)
        else:
            want = float(val_s)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), hex(code)


def test_decode_matches_torch_all_codes():
    codes = _all_codes()
    a = oracle.e4m3_decode(codes)
    b = _torch_decode(codes)
    nan = np.isnan(b)
    assert np.array_equal(np.isnan(a), nan)
    assert np.array_equal(a[~nan].view(np.uint32), b[~nan].view(np.uint32))


def test_decode_structure():
    """Monotone positive half, mirror symmetry, 2 NaNs, max 448."""
    v = oracle.e4m3_decode(_all_codes()).astype(np.float64)
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    assert np.isnan(v).sum() == 2
    assert np.nanmax(v) == 448.0


def test_encode_roundtrip_every_finite_code():
    codes = _all_codes()
    vals = oracle.e4m3_decode(codes)
    fin = np.isfinite(vals)
    back = oracle.e4m3_encode(vals[fin])
    assert np.array_equal(back, codes[fin])


def test_encode_matches_bruteforce_search():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 30,
        rng.uniform(-448, 448, 20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-2).astype(np.float32),
        np.array([500.0, -1e30, 448.0, 464.0, 463.99, 447.0, -0.0, 0.0], np.float32),
    ])
    assert np.array_equal(oracle.e4m3_encode(x), _nearest_even_by_search(x))


def test_encode_every_midpoint_goes_to_even():
    vals, codes = _finite_table()
    pv = np.unique(vals[vals >= 0])
    mids = ((pv[:-1] + pv[1:]) / 2).astype(np.float32)  # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (pv[:-1] + pv[1:]) / 2)
    q = oracle.e4m3_encode(mids)
    assert np.all((q & 1) == 0)
    dq = oracle.e4m3_decode(q).astype(np.float64)
    lo, hi = pv[:-1], pv[1:]
    assert np.all((dq == lo) | (dq == hi))


def test_encode_matches_torch_in_range():
    """torch's fp32 -> float8_e4m3fn conversion rounds to nearest even; it does
    not saturate, so compare on |x| <= 448 only."""
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 200000), rng.standard_normal(200000) * 1e-2,
                        rng.standard_normal(200000)]).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), t)


def test_encode_saturates():
    x = np.array([448.0, 449.0, 464.0, 465.0, 480.0, 1e6, 3.4e38, -449.0, -1e6], np.float32)
    q = oracle.e4m3_encode(x)
    assert np.array_equal(q, np.array([0x7E] * 6 + [0x7E, 0xFE, 0xFE], np.uint8))


@pytest.mark.slow
def test_encode_exhaustive_fp32_window():
    """Every fp32 in [-1024, 1024] with the low 8 mantissa bits stepped: the
    encoder equals the exhaustive nearest-even search."""
    vals, codes = _finite_table()
    pv = np.unique(vals[vals > 0])
    bits = np.arange(0, 0x44800000, 251, dtype=np.uint32)  # 0 .. 1024
    x = bits.view(np.float32)
    q = oracle.e4m3_encode(x)
    # independent: bisect into the sorted positive values
    a = x.astype(np.float64)
    hi = np.searchsorted(pv, a, side="left")
    hi = np.clip(hi, 0, len(pv) - 1)
    lo = np.clip(hi - 1, 0, len(pv) - 1)
    vlo = np.where(a < pv[0], 0.0, pv[lo])
    vhi = pv[hi]
    dlo, dhi = a - vlo, vhi - a
    enc_lo = oracle.e4m3_encode(vlo.astype(np.float32))
    enc_hi = oracle.e4m3_encode(vhi.astype(np.float32))
    choose_hi = (dhi < dlo) | ((dhi == dlo) & ((enc_hi & 1) == 0))
    want = np.where(choose_hi, enc_hi, enc_lo)
    want = np.where(a >= 448.0, 0x7E, want).astype(np.uint8)
    assert np.array_equal(q, want)
    assert np.array_equal(oracle.e4m3_encode(-x), want | 0x80)


# ---------------------------------------------------------------- bf16 rounding, pow2
def test_f64_to_bf16_bruteforce():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(50000) * 10, rng.standard_normal(1000) * 1e-3,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)])])
    assert list(oracle.f64_to_bf16(np.array([0.0, -0.0]))) == [0x0000, 0x8000]
    h = oracle.f64_to_bf16(x)
    # independent: candidate bf16 patterns around the fp32 truncation, pick nearest, ties even
    base = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    cands = np.stack([base - 1, base, base + 1], axis=1)
    cv = ((cands.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    d = np.abs(cv - x[:, None])
    m = d.min(axis=1, keepdims=True)
    tie_even = (d == m) & ((cands & 1) == 0)
    pick = np.where(tie_even.any(axis=1), tie_even.argmax(axis=1), (d == m).argmax(axis=1))
    want = cands[np.arange(len(x)), pick].astype(np.uint16)
    assert np.array_equal(h, want)


def test_pow2_ceil_bruteforce():
    rng = np.random.default_rng(3)
    s = np.concatenate([np.exp(rng.uniform(-60, 20, 20000)), 2.0 ** np.arange(-40, 10)]).astype(np.float32)
    p = oracle.pow2_ceil(s)
    powers = 2.0 ** np.arange(-126, 127, dtype=np.float64)
    idx = np.searchsorted(powers, s.astype(np.float64), side="left")
    assert np.array_equal(p.astype(np.float64), powers[idx])


# ---------------------------------------------------------------- a1: inverse RoPE
def _table_row(c, s, rope=64):
    row = np.zeros((1, rope), np.float32)
    row[0, : rope // 2] = c
    row[0, rope // 2:] = s
    return row


def test_inverse_rope_golden_cases():
    for line in _read_golden("rope_inverse_cases.txt"):
        e, d, c, s, e2, d2 = (np.float32(v) for v in line.split())
        x = np.zeros((1, 1, 512), np.float32)
        x[0, 0, 448] = e
        x[0, 0, 449] = d
        x[0, 0, 510] = e  # last pair too
        x[0, 0, 511] = d
        tab = _table_row(c, s)
        out = oracle.rope_f32(x, np.array([0]), tab, 448, 64, inverse=True)
        assert out[0, 0, 448] == e2 and out[0, 0, 449] == d2, line
        assert out[0, 0, 510] == e2 and out[0, 0, 511] == d2, line


def _rand_rows(T, H, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, H, 512)).astype(np.float32)


def test_inverse_rope_position0_is_identity():
    tab = wl.cos_sin_table(16, 64)
    assert np.all(tab[0, :32] == 1.0) and np.all(tab[0, 32:] == 0.0)
    x = _rand_rows(3, 4, 4)
    out = oracle.rope_f32(x, np.zeros(3, np.int64), tab, 448, 64, inverse=True)
    assert np.array_equal(out.view(np.uint32), x.view(np.uint32))


def test_inverse_rope_complex_crosscheck():
    """Closed form in fp64 complex arithmetic: x * conj(cos + i sin)."""
    T, H = 7, 3
    x = _rand_rows(T, H, 5)
    tab = wl.cos_sin_table(4096, 64)
    pos = np.array([0, 1, 17, 999, 2048, 4095, 3], np.int64)
    out = oracle.rope_f32(x, pos, tab, 448, 64, inverse=True)
    z = x[..., 448::2].astype(np.float64) + 1j * x[..., 449::2].astype(np.float64)
    cs = tab[pos, :32].astype(np.float64) + 1j * tab[pos, 32:].astype(np.float64)
    want = z * np.conj(cs)[:, None, :]
    got = out[..., 448::2].astype(np.float64) + 1j * out[..., 449::2].astype(np.float64)
    err = np.abs(got - want) / np.maximum(np.abs(z), 1e-30)
    assert err.max() < 1e-6
    assert np.array_equal(out[..., :448], x[..., :448])


def test_forward_then_inverse_is_identity():
    T, H = 5, 2
    x = _rand_rows(T, H, 6)
    tab = wl.cos_sin_table(32768, 64)
    pos = np.array([1, 77, 4000, 20000, 32767], np.int64)
    f = oracle.rope_f32(x, pos, tab, 448, 64, inverse=False)
    b = oracle.rope_f32(f, pos, tab, 448, 64, inverse=True)
    e = b[..., 448:].reshape(T, H, 32, 2) - x[..., 448:].reshape(T, H, 32, 2)
    n = np.linalg.norm(x[..., 448:].reshape(T, H, 32, 2).astype(np.float64), axis=-1)
    rel = np.linalg.norm(e.astype(np.float64), axis=-1) / n
    assert rel.max() < 1e-6
    # forward alone is a real rotation (not the identity)
    assert np.abs(f[..., 448:] - x[..., 448:]).max() > 1e-2


def test_inverse_rope_preserves_pair_norm():
    x = _rand_rows(4, 4, 7)
    tab = wl.cos_sin_table(8192, 64)
    pos = np.array([5, 50, 500, 5000], np.int64)
    out = oracle.rope_f32(x, pos, tab, 448, 64, inverse=True)
    n0 = np.hypot(x[..., 448::2].astype(np.float64), x[..., 449::2].astype(np.float64))
    n1 = np.hypot(out[..., 448::2].astype(np.float64), out[..., 449::2].astype(np.float64))
    # table rows are unit vectors only to fp32 rounding: allow a few ulp
    assert np.abs(n1 / n0 - 1).max() < 4e-7


# ---------------------------------------------------------------- a2: block quant
def _parse_golden_quant():
    cases = []
    for line in _read_golden("quant_blocks.txt"):
        mode, ent, scale, codes = (p.strip() for p in line.split("|"))
        v = np.zeros(128, np.float32)
        for tok in ent.split():
            i, val = tok.split(":")
            v[int(i)] = np.float32(float(val))
        want = {int(t.split(":")[0]): int(t.split(":")[1], 16) for t in codes.split()}
        cases.append((mode, v, np.float32(float(scale)), want))
    return cases


def test_quant_golden_blocks():
    for mode, v, scale, want in _parse_golden_quant():
        q, s = oracle.block_quant_rows(v[None, :], 128, pow2=(mode == "pow2"))
        assert s[0, 0] == scale, (mode, s[0, 0], scale)
        for i, c in want.items():
            assert q[0, i] == c, (mode, i, hex(q[0, i]), hex(c))
        zero = np.ones(128, bool)
        zero[list(want)] = False
        zero &= v == 0
        assert np.all(q[0, zero] == 0)


def _rand_blocks(rows, seed, outliers=True):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, 1024)).astype(np.float32)
    if outliers:
        m = rng.uniform(size=v.shape) < 0.01
        v[m] *= 50
    v[0, :128] *= 1e-30  # tiny block
    v[1, 128:256] = 0.0  # all-zero block
    return v


def test_quant_fp32_scale_and_max_code():
    v = _rand_blocks(64, 8)
    q, s = oracle.block_quant_rows(v, 128, pow2=False)
    blocks = v.reshape(64, 8, 128)
    amax = np.maximum(np.abs(blocks).max(-1), np.float32(1e-10)).astype(np.float32)
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    dq = np.abs(oracle.e4m3_decode(q).reshape(64, 8, 128)).max(-1)
    nz = np.abs(blocks).max(-1) >= 1e-10
    assert np.all(dq[nz] == 448.0)
    assert np.all(dq[~nz] == 0.0)


def test_quant_pow2_scales():
    v = _rand_blocks(64, 9)
    q, s = oracle.block_quant_rows(v, 128, pow2=True)
    m, e = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5)  # exact powers of two
    blocks = v.reshape(64, 8, 128)
    amax = np.maximum(np.abs(blocks).max(-1), np.float32(1e-10)).astype(np.float32)
    ratio = (amax / np.float32(448.0)).astype(np.float32)
    assert np.all(s >= ratio) and np.all(s < 2 * ratio)
    dq = np.abs(oracle.e4m3_decode(q).reshape(64, 8, 128)).max(-1)
    nz = np.abs(blocks).max(-1) >= 1e-10
    assert np.all((dq[nz] >= 224.0) & (dq[nz] <= 448.0))


@pytest.mark.parametrize("pow2", [False, True])
def test_quant_dequant_error_bound(pow2):
    """|decode(q)*s - v| <= half the e4m3fn spacing at v/s, times s (plus the
    fp32 rounding of v/s)."""
    v = _rand_blocks(32, 10)
    q, s = oracle.block_quant_rows(v, 128, pow2=pow2)
    srep = np.repeat(s, 128, axis=1).astype(np.float64)
    r = v.astype(np.float64) / srep
    dq = oracle.e4m3_decode(q).astype(np.float64)
    # spacing of e4m3fn at |r|: 2^(floor(log2|r|) - 3) for normals, 2^-9 below 2^-6
    a = np.abs(r)
    ex = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    spacing = 2.0 ** (ex - 3)
    bound = 0.5 * spacing + a * 2.0 ** -23
    assert np.all(np.abs(dq - r) <= bound + 1e-300)


def test_quant_bruteforce_tiny():
    """Brute force on a tiny input: each code equals the search-based encoder
    applied to v / s, with s from the definition."""
    v = _rand_blocks(2, 11)
    q, s = oracle.block_quant_rows(v, 128, pow2=False)
    srep = np.repeat(s, 128, axis=1)
    want = _nearest_even_by_search((v / srep).astype(np.float32).ravel()).reshape(q.shape)
    assert np.array_equal(q, want)


def test_inv_rope_quant_matches_composition():
    """Fused a1+a2 equals rotating in fp32 and then quantising each group row;
    head h lives in group h // hpg at offset (h % hpg) * 512."""
    w = wl.WORKLOADS["tiny"]
    o = wl.attn_out(w)
    pos = wl.positions(w)
    tab = wl.table(w)
    q, s = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group)
    x = wl.bf16_bits_to_f32(o)
    r = oracle.rope_f32(x, pos, tab, 448, 64, inverse=True)
    rows = r.reshape(w.T * w.n_groups, w.D)
    q2, s2 = oracle.block_quant_rows(rows, 128)
    assert np.array_equal(q.reshape(-1, w.D), q2)
    assert np.array_equal(s.reshape(-1, w.KB), s2)
    # position 0 token: nope and rope dims both pass through unchanged
    pos0 = pos.copy()
    pos0[:] = 0
    q0, s0 = oracle.inv_rope_quant(o, pos0, tab, w.n_groups, w.heads_per_group)
    q3, s3 = oracle.block_quant_rows(x.reshape(w.T * w.n_groups, w.D), 128)
    assert np.array_equal(q0.reshape(-1, w.D), q3)


# ---------------------------------------------------------------- attention-epilogue producer (fp32 input)
def _f32_attn_out(T, H, seed):
    """fp32 attention output whose values are not bf16 values (low mantissa bits set)."""
    x = wl.normal(seed, T * H * 512).astype(np.float32).reshape(T, H, 512)
    assert np.any(wl.f32_to_bf16_bits(x).astype(np.uint32) << 16 != x.view(np.uint32))
    return x


def test_f32_producer_equals_the_bf16_path_on_bf16_values():
    """fp32 inputs that are exactly bf16 values give the a1+a2 result bit for bit."""
    w = wl.WORKLOADS["tiny"]
    o = wl.attn_out(w)
    pos, tab = wl.positions(w), wl.table(w)
    for pow2 in (False, True):
        q, s = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group, pow2=pow2)
        qf, sf = oracle.inv_rope_quant_f32(wl.bf16_bits_to_f32(o), pos, tab, w.n_groups, w.heads_per_group,
                                           pow2=pow2)
        assert np.array_equal(q, qf) and np.array_equal(s.view(np.uint32), sf.view(np.uint32))


def _torch_encode(v: np.ndarray) -> np.ndarray:
    """Library route: torch's float8_e4m3fn cast (nearest even) after clamping to +-448."""
    t = torch.from_numpy(np.clip(v, -448.0, 448.0).astype(np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_f32_producer_unrotated_blocks_are_plain_quantisation():
    """Blocks 0-2 of every head never see the rotation, and at position 0 none
    does (cos 1, sin 0): there each scale is max|x|/448 of the fp32 input block
    and each code is the e4m3fn value of x / scale (torch's codec)."""
    T, G, hpg = 5, 3, 2
    x = _f32_attn_out(T, G * hpg, 611)
    tab = wl.cos_sin_table(4096, 64)
    pos = np.array([0, 17, 4095, 1000, 0], np.int64)
    q, s = oracle.inv_rope_quant_f32(x, pos, tab, G, hpg)
    xb = x.reshape(T, G, hpg * 4, 128)          # [t, g, block, 128]
    sb = s.reshape(T, G, hpg * 4)
    qb = q.reshape(T, G, hpg * 4, 128)
    amax = np.abs(xb).max(axis=-1)
    want_s = (amax / np.float32(448.0)).astype(np.float32)
    plain = np.zeros((T, G, hpg * 4), bool)
    plain[:, :, [b for b in range(hpg * 4) if b % 4 != 3]] = True
    plain[pos == 0] = True
    assert np.array_equal(sb[plain].view(np.uint32), want_s[plain].view(np.uint32))
    want_q = _torch_encode(xb / sb[..., None])
    assert np.array_equal(qb[plain], want_q[plain])


def test_f32_producer_rotated_block_scale_within_the_fp64_bound():
    """Block 3 of each head (64 plain dims + the 32 rotated pairs): its scale is
    max|v|/448 of the exact (fp64) inverse rotation within the fp32 rounding of
    the rotation (|error| <= 2^-22 |v| per value) and of the division."""
    T, G, hpg = 4, 2, 4
    x = _f32_attn_out(T, G * hpg, 612)
    tab = wl.cos_sin_table(32768, 64)
    pos = np.array([3, 32767, 12345, 777], np.int64)
    _, s = oracle.inv_rope_quant_f32(x, pos, tab, G, hpg)
    c = tab[pos, :32].astype(np.float64)[:, None, :]
    sn = tab[pos, 32:].astype(np.float64)[:, None, :]
    e = x[:, :, 448::2].astype(np.float64)
    d = x[:, :, 449::2].astype(np.float64)
    er, dr = e * c + d * sn, d * c - e * sn    # rotation by -theta, pair (e, d)
    amax = np.maximum(np.abs(x[:, :, 384:448]).max(axis=-1),
                      np.maximum(np.abs(er).max(axis=-1), np.abs(dr).max(axis=-1)))
    want = (amax / 448.0).reshape(T, G, hpg)
    got = s.reshape(T, G, hpg, 4)[..., 3].astype(np.float64)
    assert np.all(np.abs(got - want) <= want * 2.0 ** -21)


# ---------------------------------------------------------------- weights
def test_weight_quant_and_dequant_blocks():
    rng = np.random.default_rng(12)
    wmat = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    q, s = oracle.quant_weight(wmat, 128)
    assert s.shape == (2, 3)
    for i in range(2):
        for b in range(3):
            tile = wmat[i * 128:(i + 1) * 128, b * 128:(b + 1) * 128]
            assert s[i, b] == np.float32(np.abs(tile).max()) / np.float32(448)
            dq = oracle.e4m3_decode(q[i * 128:(i + 1) * 128, b * 128:(b + 1) * 128])
            assert np.abs(dq).max() == 448.0
    # dequant is decode(q) * scale over 128x128 tiles (the scale multiplies)
    d = oracle.dequant_weight(q, s, 128)
    want = oracle.e4m3_decode(q).astype(np.float64) * np.kron(s.astype(np.float64), np.ones((128, 128)))
    assert np.array_equal(d, want)
    assert np.abs(d - wmat).max() <= np.abs(wmat).max() / 16 + 1e-12
    # 1x128 per-row mode, pow2
    q1, s1 = oracle.quant_weight(wmat, 1, pow2=True)
    assert s1.shape == (256, 3)
    d1 = oracle.dequant_weight(q1, s1, 1)
    want1 = oracle.e4m3_decode(q1).astype(np.float64) * np.kron(s1.astype(np.float64), np.ones((1, 128)))
    assert np.array_equal(d1, want1)


def _pow2_ceil_frexp(x: np.ndarray) -> np.ndarray:
    """Independent route to the power-of-two ceiling: frexp gives x = m * 2^e
    with m in [0.5, 1); x is a power of two exactly when m == 0.5."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.where(m == 0.5, x, np.ldexp(1.0, e)).astype(np.float32)


@pytest.mark.parametrize("pow2", [False, True])
def test_weight_quant_1x128_per_row_scales(pow2):
    """1x128 mode: each row's block scale comes from THAT row's 128 values
    (numpy's fp32 amax / 448, or its power-of-two ceiling), and each row's
    block decodes to a max |code| of 448 (fp32) or within [224, 448] (pow2).
    One large value planted in one row must change only that row's scale."""
    rng = np.random.default_rng(21)
    rows, K = 130, 384
    wmat = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    wmat[5, 130] = 3.0  # row 5, block 1 only
    q, s = oracle.quant_weight(wmat, 1, pow2=pow2)
    assert s.shape == (rows, K // 128)
    amax = np.abs(wmat.reshape(rows, K // 128, 128)).max(axis=2)
    want = amax.astype(np.float32) / np.float32(448)
    if pow2:
        want = _pow2_ceil_frexp(want)
    assert np.array_equal(s.view(np.uint32), want.view(np.uint32))
    assert s[5, 1] > 20 * s[4, 1] and s[5, 1] > 20 * s[6, 1]
    mx = np.abs(oracle.e4m3_decode(q).reshape(rows, K // 128, 128)).max(axis=2)
    if pow2:
        assert np.all((mx >= 224.0) & (mx <= 448.0))
    else:
        assert np.all(mx == 448.0)
    # the codes are the e4m3fn roundings of w / scale, by brute-force search
    quot = (wmat[3:6].reshape(3, K // 128, 128) / s[3:6, :, None]).astype(np.float32).ravel()
    assert np.array_equal(q[3:6].ravel(), _nearest_even_by_search(quot))


def test_weight_quant_1x128_golden_rows():
    for line in _read_golden("weight_rows_1x128.txt"):
        mode, ent, scl, codes = [p.strip() for p in line.split("|")]
        row = np.zeros((1, 256), np.float32)
        for kv in ent.split():
            i, v = kv.split(":")
            row[0, int(i)] = np.float32(float(v))
        q, s = oracle.quant_weight(row, 1, pow2=(mode == "pow2"))
        want_s = np.array([float(x) for x in scl.split()], np.float32)
        assert np.array_equal(s[0], want_s), (line, s[0], want_s)
        for kv in codes.split():
            i, c = kv.split(":")
            assert q[0, int(i)] == int(c, 16), (line, i, hex(q[0, int(i)]))
        assert np.all(q[0, [j for j in range(256) if row[0, j] == 0]] == 0)


# ---------------------------------------------------------------- a3: grouped contraction
def _tiny_operands(T, G, D, R, seed, pad=0, brows=128, pow2=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T * (G + pad), D)).astype(np.float32)
    qa, sa = oracle.block_quant_rows(x, 128, pow2=pow2)
    qa = qa.reshape(T, G + pad, D)
    sa = sa.reshape(T, G + pad, D // 128)
    wmat = (rng.standard_normal((G * R, D)) * 0.02).astype(np.float32)
    qw, sw = oracle.quant_weight(wmat, brows, pow2=pow2)
    return qa, sa, qw, sw


@pytest.mark.parametrize("brows,pow2", [(128, False), (1, True), (1, False)])
def test_grouped_gemm_equals_independent_matmuls(brows, pow2):
    T, G, D, R = 5, 3, 256, 128
    qa, sa, qw, sw = _tiny_operands(T, G, D, R, 13, brows=brows, pow2=pow2)
    z = oracle.grouped_gemm(qa, sa, qw, sw, G, R, brows)
    ad = oracle.e4m3_decode(qa).astype(np.float64) * np.repeat(sa.astype(np.float64), 128, axis=2)
    wd = oracle.e4m3_decode(qw).astype(np.float64) * np.kron(
        sw.astype(np.float64), np.ones((brows, 128)))[: G * R]
    for g in range(G):
        ref = ad[:, g, :] @ wd[g * R:(g + 1) * R, :].T
        assert np.allclose(z[:, g, :], ref, rtol=1e-12, atol=1e-12)


def test_grouped_gemm_r64_shares_weight_scale_rows():
    """R=64 < 128: 128x128 weight tiles cover the flat [G*R, D] matrix, so
    groups 0 and 1 share scale row 0."""
    T, G, D, R = 4, 2, 1024, 64
    qa, sa, qw, sw = _tiny_operands(T, G, D, R, 14)
    assert sw.shape == (1, 8)
    z = oracle.grouped_gemm(qa, sa, qw, sw, G, R, 128)
    ad = oracle.e4m3_decode(qa).astype(np.float64) * np.repeat(sa.astype(np.float64), 128, axis=2)
    wd = oracle.e4m3_decode(qw).astype(np.float64) * np.repeat(sw.astype(np.float64), 128, axis=1)
    for g in range(G):
        assert np.allclose(z[:, g, :], ad[:, g, :] @ wd[g * R:(g + 1) * R].T, rtol=1e-12, atol=1e-12)


def test_grouped_gemm_group_isolation():
    T, G, D, R = 3, 3, 256, 128
    qa, sa, qw, sw = _tiny_operands(T, G, D, R, 15)
    z = oracle.grouped_gemm(qa, sa, qw, sw, G, R)
    # zero every activation group except g=1 -> only z[:, 1] survives
    qa1 = qa.copy()
    qa1[:, [0, 2]] = 0
    z1 = oracle.grouped_gemm(qa1, sa, qw, sw, G, R)
    assert np.all(z1[:, [0, 2]] == 0) and np.array_equal(z1[:, 1], z[:, 1])
    # perturb weight rows outside group 1 -> z[:, 1] unchanged, others change
    qw2 = qw.copy()
    qw2[:R] ^= 0x01
    qw2[2 * R:] ^= 0x01
    z2 = oracle.grouped_gemm(qa, sa, qw2, sw, G, R)
    assert np.array_equal(z2[:, 1], z[:, 1])
    assert not np.array_equal(z2[:, 0], z[:, 0])


def test_grouped_gemm_reduces_to_plain_gemm():
    """G=1 and unit scales: plain product of the decoded codes."""
    rng = np.random.default_rng(16)
    T, D, R = 6, 256, 128
    qa = rng.integers(0, 256, (T, 1, D)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x00
    qw = rng.integers(0, 256, (R, D)).astype(np.uint8)
    qw[(qw & 0x7F) == 0x7F] = 0x01
    sa = np.ones((T, 1, D // 128), np.float32)
    sw = np.ones((1, D // 128), np.float32)
    z = oracle.grouped_gemm(qa, sa, qw, sw, 1, R)
    ref = _torch_decode(qa[:, 0]).astype(np.float64) @ _torch_decode(qw).astype(np.float64).T
    assert np.array_equal(z[:, 0], ref)


def test_grouped_gemm_padding_never_read():
    T, G, D, R = 4, 2, 256, 128
    qa, sa, qw, sw = _tiny_operands(T, G, D, R, 17, pad=2, pow2=True, brows=1)
    z = oracle.grouped_gemm(qa, sa, qw, sw, G, R, 1)
    qa[:, G:] = 0x7F  # NaN codes
    sa[:, G:] = np.nan
    zp = oracle.grouped_gemm(qa, sa, qw, sw, G, R, 1)
    assert np.all(np.isfinite(zp)) and np.array_equal(z, zp)
    z_live = oracle.grouped_gemm(np.ascontiguousarray(qa[:, :G]), np.ascontiguousarray(sa[:, :G]),
                                 qw, sw, G, R, 1)
    assert np.array_equal(z, z_live)


def test_grouped_gemm_sampled_equals_dense():
    T, G, D, R = 5, 2, 256, 128
    qa, sa, qw, sw = _tiny_operands(T, G, D, R, 18)
    z = oracle.grouped_gemm(qa, sa, qw, sw, G, R)
    idx = np.array([[0, 0, 0], [4, 1, 127], [2, 1, 5], [3, 0, 64]], np.int64)
    zs = oracle.grouped_gemm(qa, sa, qw, sw, G, R, idx=idx)
    assert np.array_equal(zs, z[idx[:, 0], idx[:, 1], idx[:, 2]])


@pytest.mark.parametrize("brows,pow2,pad", [(128, False, 0), (1, True, 2), (1, False, 1)])
def test_grouped_gemm_full_equals_elementwise(brows, pow2, pad):
    """The whole-tensor form (operands dequantised once, numpy fp64 product
    per group) against the element-by-element C loop; NaN padding groups
    must not reach it."""
    T, G, D, R = 37, 3, 512, 160
    qa, sa, qw, sw = _tiny_operands(T, G, D, R, 22, pad=pad, brows=brows, pow2=pow2)
    qa[:, G:] = 0x7F
    sa[:, G:] = np.nan
    z = oracle.grouped_gemm(qa, sa, qw, sw, G, R, brows)
    zf = oracle.grouped_gemm_full(qa, sa, qw, sw, G, R, brows)
    assert zf.shape == (T, G, R) and np.all(np.isfinite(zf))
    assert np.abs(zf - z).max() <= 1e-13 * np.abs(z).max()


def test_grouped_gemm_full_exact_on_integer_operands():
    """Codes of small integers and power-of-two scales make every partial sum
    exact in fp64, so any order gives the same bits: the two forms must agree
    exactly (a transposed operand or a wrong group slice cannot)."""
    rng = np.random.default_rng(23)
    T, G, D, R = 9, 2, 256, 128
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4], np.uint8)  # 0, +-1, +-2, 3, 4
    qa = ints[rng.integers(0, ints.size, (T, G, D))]
    qw = ints[rng.integers(0, ints.size, (G * R, D))]
    sa = (2.0 ** rng.integers(-3, 3, (T, G, D // 128))).astype(np.float32)
    sw = (2.0 ** rng.integers(-3, 3, (G * R // 128, D // 128))).astype(np.float32)
    z = oracle.grouped_gemm(qa, sa, qw, sw, G, R, 128)
    zf = oracle.grouped_gemm_full(qa, sa, qw, sw, G, R, 128)
    assert np.array_equal(z, zf)
    assert not np.array_equal(zf[:, 0], zf[:, 1])


def test_dense_gemm_bf16_full_equals_elementwise():
    rng = np.random.default_rng(24)
    x = wl.f32_to_bf16_bits(rng.standard_normal((33, 520)).astype(np.float32))
    w = wl.f32_to_bf16_bits((rng.standard_normal((70, 520)) * 0.02).astype(np.float32))
    y = oracle.dense_gemm_bf16(x, w)
    yf = oracle.dense_gemm_bf16_full(x, w)
    assert yf.shape == (33, 70)
    assert np.abs(yf - y).max() <= 1e-13 * np.abs(y).max()


# ---------------------------------------------------------------- a4: wo_b
def test_dense_bf16_gemm_matches_numpy():
    rng = np.random.default_rng(19)
    x = wl.f32_to_bf16_bits(rng.standard_normal((9, 300)).astype(np.float32))
    w = wl.f32_to_bf16_bits((rng.standard_normal((17, 300)) * 0.02).astype(np.float32))
    y = oracle.dense_gemm_bf16(x, w)
    ref = wl.bf16_bits_to_f32(x).astype(np.float64) @ wl.bf16_bits_to_f32(w).astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    idx = np.array([[0, 0], [8, 16], [3, 7]], np.int64)
    assert np.array_equal(oracle.dense_gemm_bf16(x, w, idx=idx), y[idx[:, 0], idx[:, 1]])


# ---------------------------------------------------------------- packed UE8M0 scales
def test_e8m0_pack_matches_torch_e8m0_codec():
    """Library route: torch's float8_e8m0fnu stores a power of two as its
    biased exponent byte; bytes land in memory order inside each word."""
    rng = np.random.default_rng(41)
    k = rng.integers(-127, 128, (5, 3, 8))
    s = np.ldexp(np.ones(k.shape), k).astype(np.float32)
    w = oracle.e8m0_pack(s)
    assert w.shape == (5, 3, 2) and w.dtype == np.uint32
    tb = torch.from_numpy(s.reshape(-1)).to(torch.float8_e8m0fnu).view(torch.uint8).numpy()
    assert np.array_equal(w.reshape(-1).view(np.uint8), tb)  # little-endian words = byte order
    assert np.array_equal(w.view(np.uint8).reshape(5, 3, 8).astype(np.int64) - 127, k)


def test_e8m0_pack_nan_and_rejects():
    s = np.array([[1.0, np.nan, 0.5, 2.0 ** 100]], np.float32)
    w = oracle.e8m0_pack(s)
    assert w.view(np.uint8).reshape(-1).tolist() == [127, 0xFF, 126, 227]
    for bad in (3.0, 0.0, -2.0):
        with pytest.raises(ValueError):
            oracle.e8m0_pack(np.array([[1.0, 1.0, 1.0, bad]], np.float32))


def test_e8m0_of_pow2_quant_scales_roundtrips():
    """The pow2 recipe's scales are exact powers of two: every one packs, and
    2^(byte-127) gives it back."""
    o = wl.normal_bf16(42, 3 * 4 * 512).reshape(3, 4, 512)
    tab = wl.cos_sin_table(4096, 64)
    _, sc = oracle.inv_rope_quant(o, np.array([0, 9, 4000], np.int64), tab, 2, 2, pow2=True)
    w = oracle.e8m0_pack(sc)
    back = np.ldexp(1.0, w.view(np.uint8).astype(np.int64) - 127).reshape(sc.shape)
    assert np.array_equal(back.astype(np.float32), sc)


# ---------------------------------------------------------------- unquantised path
def _bf16_rows(T, H, seed):
    return wl.normal_bf16(seed, T * H * 512).reshape(T, H, 512)


def test_inv_rope_bf16_position0_and_nope_passthrough():
    o = _bf16_rows(3, 4, 31)
    tab = wl.cos_sin_table(4096, 64)
    x0 = oracle.inv_rope_bf16(o, np.zeros(3, np.int64), tab)
    assert np.array_equal(x0, o)  # cos 0 = 1, sin 0 = 0: the identity, bit for bit
    x = oracle.inv_rope_bf16(o, np.array([7, 1000, 4095], np.int64), tab)
    assert np.array_equal(x[..., :448], o[..., :448])
    assert (x[..., 448:] != o[..., 448:]).mean() > 0.5


def test_inv_rope_bf16_is_the_fp32_rotation_rounded_by_torch():
    """Library route for the rounding: torch's fp32 -> bfloat16 conversion
    (nearest even) of the pinned fp32 rotation."""
    o = _bf16_rows(5, 3, 32)
    tab = wl.cos_sin_table(32768, 64)
    pos = np.array([1, 77, 4000, 20000, 32767], np.int64)
    x = oracle.inv_rope_bf16(o, pos, tab)
    r32 = oracle.rope_f32(wl.bf16_bits_to_f32(o), pos, tab, 448, 64, inverse=True)
    want = torch.from_numpy(np.ascontiguousarray(r32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(x.view(np.int16), want)


def test_inv_rope_bf16_error_bound_against_exact_rotation():
    """fp64 complex closed form; bf16 keeps 8 significant bits, so the result
    is within half a bf16 ulp of the exact value plus the fp32 rounding."""
    o = _bf16_rows(6, 2, 33)
    tab = wl.cos_sin_table(8192, 64)
    pos = np.array([0, 3, 33, 333, 3333, 8191], np.int64)
    x = wl.bf16_bits_to_f32(oracle.inv_rope_bf16(o, pos, tab)).astype(np.float64)
    of = wl.bf16_bits_to_f32(o).astype(np.float64)
    z = of[..., 448::2] + 1j * of[..., 449::2]
    cs = tab[pos, :32].astype(np.float64) + 1j * tab[pos, 32:].astype(np.float64)
    want = z * np.conj(cs)[:, None, :]
    for got, ref in ((x[..., 448::2], want.real), (x[..., 449::2], want.imag)):
        bound = np.abs(ref) * 2.0 ** -8 + np.abs(z) * 2.0 ** -21 + 1e-30
        assert np.all(np.abs(got - ref) <= bound)


def test_grouped_gemm_bf16_bruteforce_tiny():
    """Pure-Python fp64 loops over the definition, one matmul per group."""
    T, G, D, R = 3, 2, 16, 5
    x = wl.normal_bf16(34, T * G * D).reshape(T, G, D)
    w = wl.normal_bf16(35, G * R * D, std=0.02).reshape(G * R, D)
    xf, wf = wl.bf16_bits_to_f32(x), wl.bf16_bits_to_f32(w)
    z = oracle.grouped_gemm_bf16(x, w, G, R)
    for t in range(T):
        for g in range(G):
            for n in range(R):
                acc = 0.0
                for k in range(D):
                    acc += float(xf[t, g, k]) * float(wf[g * R + n, k])
                assert abs(z[t, g, n] - acc) <= 1e-12 * (1 + abs(acc))


def test_grouped_gemm_bf16_integer_operands_exact():
    """Small integers are exact in bf16 and in fp64 sums: closed form."""
    T, G, D, R = 4, 3, 64, 8
    rng = np.random.default_rng(36)
    xi = rng.integers(-8, 9, (T, G, D))
    wi = rng.integers(-8, 9, (G * R, D))
    x = wl.f32_to_bf16_bits(xi.astype(np.float32))
    w = wl.f32_to_bf16_bits(wi.astype(np.float32))
    z = oracle.grouped_gemm_bf16(x, w, G, R)
    want = np.einsum("tgk,gnk->tgn", xi, wi.reshape(G, R, D))
    assert np.array_equal(z, want.astype(np.float64))


def test_grouped_gemm_bf16_group_isolation_and_samples():
    T, G, D, R = 4, 3, 32, 6
    x = wl.normal_bf16(37, T * G * D).reshape(T, G, D)
    w = wl.normal_bf16(38, G * R * D, std=0.02).reshape(G * R, D)
    z = oracle.grouped_gemm_bf16(x, w, G, R)
    w2 = w.copy()
    w2[R:2 * R] = wl.f32_to_bf16_bits(np.full((R, D), 3.0, np.float32))  # rows of group 1 only
    z2 = oracle.grouped_gemm_bf16(x, w2, G, R)
    assert np.array_equal(z2[:, [0, 2]], z[:, [0, 2]]) and not np.array_equal(z2[:, 1], z[:, 1])
    idx = np.array([[0, 0, 0], [3, 2, 5], [1, 1, 3]], np.int64)
    assert np.array_equal(oracle.grouped_gemm_bf16(x, w, G, R, idx=idx), z[idx[:, 0], idx[:, 1], idx[:, 2]])


# ---------------------------------------------------------------- generator pins
def test_splitmix64_reference_outputs():
    """First outputs of SplitMix64 seeded with 0 (Vigna's reference generator)."""
    got = [int(v) for v in wl.splitmix64(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_bulk_generator_matches_numpy_statement():
    a = wl.normal_bf16(123, 50000, 1.0, 456, 0.01, 50.0)
    b = wl.normal_bf16_numpy(123, 50000, 1.0, 456, 0.01, 50.0)
    assert np.array_equal(a, b)
    c = wl.normal_f32_bulk(77, 50000, 0.02)
    d = wl.normal(77, 50000, 0.02).astype(np.float32)
    assert np.abs(c.view(np.int32).astype(np.int64) - d.view(np.int32)).max() <= 1


def test_workload_shapes():
    for name, w in wl.WORKLOADS.items():
        pos = wl.positions(w)
        assert pos.shape == (w.T,) and pos.min() >= 0 and pos.max() < w.max_pos, name
    full = wl.WORKLOADS["full"]
    pos = wl.positions(full)
    starts = np.flatnonzero(np.diff(pos) != 1)
    assert len(starts) <= full.n_seq - 1
