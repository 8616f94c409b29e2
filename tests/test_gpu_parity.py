"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: FP32 scales bit-exact; FP8 codes identical except <= 1e-4 of elements,
each at most one code step off; GEMM outputs E = max|y-r|/max|r| <= 1e-2
against the oracle's fp64 result.  Full-size workloads compare every code and
scale of the quantisation and a sample of GEMM outputs the oracle computes
one by one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_output_projection_amd as ap
import oracle
import workloads as wl
from tests import _util as U

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ap.load_library()
    yield
    torch.cuda.synchronize()


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _shape(w: wl.Workload, T: int | None = None) -> ap.Shape:
    return ap.Shape(T=w.T if T is None else T, n_groups=w.n_groups, heads_per_group=w.heads_per_group,
                    o_lora_rank=w.o_lora_rank, max_pos=w.max_pos)


def gpu_quant(w: wl.Workload, o: np.ndarray, pos: np.ndarray, tab: np.ndarray, pow2: bool):
    """GPU a1+a2 in the default layout -> token-major numpy codes/scales."""
    shp = _shape(w, o.shape[0])
    T = o.shape[0]
    d_o, d_pos, d_tab = _dev(o.view(np.int16)), _dev(pos), _dev(tab)
    codes, gc = U.guarded_empty((w.n_groups, T, w.D), torch.uint8, DEV)
    scales, gs = U.guarded_empty((w.n_groups, w.KB, T), torch.float32, DEV)
    ap.oproj_inv_rope_quant(shp, int(pow2), d_o, d_pos, d_tab, codes, scales)
    torch.cuda.synchronize()
    assert U.guard_intact(gc, codes) and U.guard_intact(gs, scales), "write past the end of an output"
    return U.group_major_to_token_major(_host(codes), _host(scales))


def gpu_weight(wmat: np.ndarray, brows: int, pow2: bool):
    rows, K = wmat.shape
    d_w = _dev(wmat)
    codes = torch.empty((rows, K), dtype=torch.uint8, device=DEV)
    scales = torch.empty(((rows + brows - 1) // brows, K // 128), dtype=torch.float32, device=DEV)
    blk = ap.OPROJ_WBLOCK_1x128 if brows == 1 else ap.OPROJ_WBLOCK_128x128
    ap.oproj_quantize_weight(rows, K, blk, int(pow2), d_w, codes, scales)
    return codes, scales


def gpu_gemm(w: wl.Workload, qa_tm: np.ndarray, sa_tm: np.ndarray, d_wq, d_ws, brows: int,
             pow2: bool) -> np.ndarray:
    """GPU a3 on token-major operands [T][Gp][D] (Gp >= G) passed with explicit strides."""
    T, Gp, D = qa_tm.shape
    KB = D // 128
    lay = ap.ActLayout(Gp * D, D, Gp * KB, KB, 1)
    z, gz = U.guarded_empty((T, w.n_groups, w.o_lora_rank), torch.int16, DEV)
    blk = ap.OPROJ_WBLOCK_1x128 if brows == 1 else ap.OPROJ_WBLOCK_128x128
    ap.oproj_grouped_wo_a(_shape(w, T), int(pow2), _dev(qa_tm), _dev(sa_tm), lay, d_wq, d_ws, blk, z)
    torch.cuda.synchronize()
    assert U.guard_intact(gz, z), "write past the end of z"
    return U.bf16_bits_to_f64(_host(z).view(np.uint16))


# ---------------------------------------------------------------- FP8 conversion sweep
def test_fp8_conversion_sweep_matches_oracle_encoder():
    """Rows whose block amax is exactly 448 get scale 1, so the weight
    quantiser's codes are the hardware conversion of the values themselves:
    sweep fp32 values over the whole e4m3fn range (normals, subnormals, every
    midpoint, the saturation edge)."""
    vals, _ = np.unique(oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)), return_index=True)
    vals = vals.astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(0)
    x = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, 448, 60000), np.exp(rng.uniform(-14, 6, 60000))]).astype(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448.0]
    per_row = 127
    n_rows = (x.size + per_row - 1) // per_row
    buf = np.zeros(n_rows * per_row, np.float32)
    buf[: x.size] = x
    rows = np.concatenate([np.full((n_rows, 1), 448.0, np.float32), buf.reshape(n_rows, per_row)], axis=1)
    codes, scales = gpu_weight(rows, 1, False)
    s = _host(scales)
    assert np.all(s == 1.0)
    got = _host(codes)[:, 1:].ravel()[: x.size]
    want = oracle.e4m3_encode(x)
    n_bad, n, adj = U.compare_codes(got, want)
    assert n_bad == 0, f"{n_bad}/{n} conversions differ from round-to-nearest-even"


# ---------------------------------------------------------------- weight quantisation
@pytest.mark.parametrize("brows,pow2", [(128, False), (1, True), (1, False), (128, True)])
def test_weight_quant_parity(brows, pow2):
    wmat = wl.normal_f32_bulk(wl.seed_of(90, brows + 2 * pow2), 640 * 1024, 0.02).reshape(640, 1024)
    wmat[3, 5] = 0.9  # an outlier block
    wmat[256:384, 128:256] = 0.0  # all-zero 128x128 block
    codes, scales = gpu_weight(wmat, brows, pow2)
    qr, sr = oracle.quant_weight(wmat, brows, pow2)
    U.assert_scales_bitexact(_host(scales), sr)
    U.assert_codes_parity(_host(codes), qr, frac=0.0)


# ---------------------------------------------------------------- a1 + a2
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "full"])
def test_inv_rope_quant_parity_workloads(name):
    w = wl.WORKLOADS[name]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    qg, sg = gpu_quant(w, o, pos, tab, pow2=w.pow2)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group, pow2=w.pow2)
    U.assert_scales_bitexact(sg, sr)
    U.assert_codes_parity(qg, qr)


@pytest.mark.parametrize("T,G,hpg,pow2", [(1, 1, 1, False), (3, 2, 2, True), (5, 3, 4, False),
                                          (77, 2, 8, False), (130, 1, 16, True), (257, 4, 8, True)])
def test_inv_rope_quant_ragged_shapes(T, G, hpg, pow2):
    w = wl.Workload(50 + T, f"r{T}", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=64,
                    max_pos=4096, positions="uniform", pow2=pow2)
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    pos[0] = 0
    pos[-1] = w.max_pos - 1
    qg, sg = gpu_quant(w, o, pos, tab, pow2)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, G, hpg, pow2=pow2)
    U.assert_scales_bitexact(sg, sr)
    U.assert_codes_parity(qg, qr)


def test_inv_rope_quant_beyond_4gib_input():
    """a1 + a2 on an input larger than 4 GiB (T = 4100 tokens of 1024 heads;
    token t starts at t MiB), so that rows past 2^31 and 2^32 bytes are read
    and group-major codes past 2^31 bytes are written.  Tokens on both sides
    of those offsets and at the end against the oracle."""
    w = wl.Workload(93, "big", T=4100, n_groups=128, heads_per_group=8, o_lora_rank=64, max_pos=32768,
                    positions="uniform")
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_o = _dev(o.view(np.int16))
    codes = torch.empty((w.n_groups, w.T, w.D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.n_groups, w.KB, w.T), dtype=torch.float32, device=DEV)
    ap.oproj_inv_rope_quant(_shape(w), 0, d_o, _dev(pos), _dev(tab), codes, scales)
    torch.cuda.synchronize()
    del d_o
    sel = np.array([0, 1, 2047, 2048, 2049, 4095, 4096, 4097, 4098, 4099], np.int64)
    tsel = torch.from_numpy(sel).to(DEV)
    qg, sg = U.group_major_to_token_major(_host(codes[:, tsel, :]), _host(scales[:, :, tsel]))
    qr, sr = oracle.inv_rope_quant(o[sel], pos[sel], tab, w.n_groups, w.heads_per_group)
    U.assert_scales_bitexact(sg, sr)
    U.assert_codes_parity(qg, qr)


def test_inv_rope_quant_degenerate_blocks():
    """All-zero blocks, tiny and huge magnitudes, exact ties."""
    w = wl.Workload(60, "deg", T=6, n_groups=2, heads_per_group=2, o_lora_rank=64, max_pos=64,
                    positions="uniform")
    o = wl.attn_out(w).copy()
    x = wl.bf16_bits_to_f32(o).copy()
    x[0] = 0.0  # whole token zero
    x[1, 0, :128] = 0.0  # one zero block
    x[2] *= 1e-30  # tiny values
    x[3] *= 1e30  # huge values
    x[4, :, ::2] = 0.5  # repeated values
    o = wl.f32_to_bf16_bits(x).reshape(o.shape)
    pos = np.array([0, 1, 2, 63, 5, 0], np.int64)
    tab = wl.cos_sin_table(64, 64)
    for pow2 in (False, True):
        qg, sg = gpu_quant(w, o, pos, tab, pow2)
        qr, sr = oracle.inv_rope_quant(o, pos, tab, 2, 2, pow2=pow2)
        U.assert_scales_bitexact(sg, sr)
        U.assert_codes_parity(qg, qr, frac=0.0)


def test_inv_rope_quant_bad_position_poisons_scales():
    w = wl.WORKLOADS["tiny"]
    o, pos, tab = wl.attn_out(w), wl.positions(w).copy(), wl.table(w)
    pos[1] = w.max_pos  # out of range
    pos[2] = -1
    qg, sg = gpu_quant(w, o, pos, tab, False)
    assert np.all(np.isnan(sg[1])) and np.all(np.isnan(sg[2]))
    ok = [0, 3]
    qr, sr = oracle.inv_rope_quant(o[ok], pos[ok], tab, w.n_groups, w.heads_per_group)
    U.assert_scales_bitexact(sg[ok], sr)
    U.assert_codes_parity(qg[ok], qr, frac=0.0)


def test_inv_rope_quant_t0_is_noop():
    w = wl.WORKLOADS["tiny"]
    ap.oproj_inv_rope_quant(_shape(w, 0), 0, None, None, None, None, None)


def test_inv_rope_quant_padded_layout_leaves_padding():
    """Writing into a [T, 10, D] buffer (8 live groups) touches only groups 0..7."""
    w = wl.WORKLOADS["pow2"].scaled(96)
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    Gp = w.n_groups + w.pad_groups
    codes = torch.full((w.T, Gp, w.D), 0x7F, dtype=torch.uint8, device=DEV)
    scales = torch.full((w.T, Gp, w.KB), float("nan"), dtype=torch.float32, device=DEV)
    lay = ap.ActLayout(Gp * w.D, w.D, Gp * w.KB, w.KB, 1)
    ap.oproj_inv_rope_quant(_shape(w), 1, _dev(o.view(np.int16)), _dev(pos), _dev(tab), codes, scales, lay)
    qg, sg = _host(codes), _host(scales)
    assert np.all(qg[:, w.n_groups:] == 0x7F) and np.all(np.isnan(sg[:, w.n_groups:]))
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group, pow2=True)
    U.assert_scales_bitexact(sg[:, : w.n_groups], sr)
    U.assert_codes_parity(qg[:, : w.n_groups], qr)


# ---------------------------------------------------------------- a3
def _weights_both(w: wl.Workload, wmat=None):
    wmat = wl.wo_a_f32(w) if wmat is None else wmat
    d_wq, d_ws = gpu_weight(wmat, w.w_block_rows, w.pow2)
    qr, sr = oracle.quant_weight(wmat, w.w_block_rows, w.pow2)
    return d_wq, d_ws, qr, sr


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_grouped_gemm_dense_parity(name):
    """Isolated (oracle codes into the GPU GEMM) and end-to-end, every output."""
    w = wl.WORKLOADS[name]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    U.assert_scales_bitexact(_host(d_ws), swr)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group)
    ref = oracle.grouped_gemm(qr, sr, qwr, swr, w.n_groups, w.o_lora_rank, w.w_block_rows)
    # isolated: identical operands
    zi = gpu_gemm(w, qr, sr, _dev(qwr), _dev(swr), w.w_block_rows, w.pow2)
    assert U.rel_max_err(zi, ref) <= TOL
    # end to end: GPU quantisation, GPU weights, default layout
    shp = _shape(w)
    codes = torch.empty((w.n_groups, w.T, w.D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.n_groups, w.KB, w.T), dtype=torch.float32, device=DEV)
    ap.oproj_inv_rope_quant(shp, 0, _dev(o.view(np.int16)), _dev(pos), _dev(tab), codes, scales)
    z = torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)
    ap.oproj_grouped_wo_a(shp, 0, codes, scales, None, d_wq, d_ws, ap.OPROJ_WBLOCK_128x128, z)
    ze = U.bf16_bits_to_f64(_host(z).view(np.uint16))
    e = U.rel_max_err(ze, ref)
    assert e <= TOL, e


@pytest.mark.parametrize("name,n_samples", [("prefill", 3000), ("full", 3000)])
def test_grouped_gemm_sampled_parity_full_size(name, n_samples):
    w = wl.WORKLOADS[name]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group)
    shp = _shape(w)
    codes = torch.empty((w.n_groups, w.T, w.D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.n_groups, w.KB, w.T), dtype=torch.float32, device=DEV)
    ap.oproj_inv_rope_quant(shp, 0, _dev(o.view(np.int16)), _dev(pos), _dev(tab), codes, scales)
    z = torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)
    ap.oproj_grouped_wo_a(shp, 0, codes, scales, None, d_wq, d_ws, ap.OPROJ_WBLOCK_128x128, z)
    zg = U.bf16_bits_to_f64(_host(z).view(np.uint16))
    idx = U.stratified_triples(np.random.default_rng(7), w.T, w.n_groups, w.o_lora_rank, extra=n_samples)
    ref = oracle.grouped_gemm(qr, sr, qwr, swr, w.n_groups, w.o_lora_rank, w.w_block_rows, idx=idx)
    e = U.rel_max_err(zg[idx[:, 0], idx[:, 1], idx[:, 2]], ref)
    assert e <= TOL, e
    assert np.all(np.isfinite(zg))


def test_grouped_gemm_at_the_offset_limit():
    """The largest activation operand the GEMM accepts: one group with D = 4096
    and T = 2^20 - 1 tokens, whose last row ends 4 KiB below 2^32 bytes (the
    kernels address each operand as a uniform base plus 32-bit lane offsets;
    one token more is refused).  Random FP8 codes and scales as inputs, outputs
    sampled against the oracle on both sides of the 2^31-byte offset and at the
    end of the operand."""
    T, D, R = (1 << 20) - 1, 4096, 256
    KB = D // 128
    qa = wl.fp8_codes(wl.seed_of(90, 0), T * D).reshape(T, 1, D)
    sa = (2.0 ** (-10.0 + 6.0 * wl.uniform(wl.seed_of(90, 1), T * KB))).astype(np.float32).reshape(T, 1, KB)
    qw = wl.fp8_codes(wl.seed_of(90, 2), R * D).reshape(R, D)
    sw = (2.0 ** (-12.0 + 4.0 * wl.uniform(wl.seed_of(90, 3), 2 * KB))).astype(np.float32).reshape(2, KB)
    shp = ap.Shape(T=T, n_groups=1, heads_per_group=8, o_lora_rank=R, max_pos=1)
    lay = ap.ActLayout(D, T * D, KB, T * KB, 1)  # token-major codes and scales
    d_qa = _dev(qa)
    z = torch.empty((T, 1, R), dtype=torch.int16, device=DEV)
    ap.oproj_grouped_wo_a(shp, 0, d_qa, _dev(sa), lay, _dev(qw), _dev(sw), ap.OPROJ_WBLOCK_128x128, z)
    torch.cuda.synchronize()
    del d_qa
    assert bool(torch.isfinite(z.view(torch.bfloat16)).all())
    rng = np.random.default_rng(11)
    idx = U.sample_triples(rng, T, 1, R, 3000)
    edge = np.array([1, (1 << 19) - 1, 1 << 19, (1 << 19) + 1, T - 256, T - 2], np.int64)
    idx[4:4 + edge.size, 0] = edge
    zs = z[torch.from_numpy(idx[:, 0]).to(DEV), 0, torch.from_numpy(idx[:, 2]).to(DEV)]
    got = U.bf16_bits_to_f64(_host(zs).view(np.uint16))
    ref = oracle.grouped_gemm(qa, sa, qw, sw, 1, R, 128, idx=idx)
    e = U.rel_max_err(got, ref)
    assert e <= TOL, e


def test_grouped_gemm_pow2_padded_input():
    """Pre-quantised [T, 10, D] input with NaN-poisoned padding groups, pow2
    scales and 1x128 weight blocks (block-scaled matrix-core path)."""
    w = wl.WORKLOADS["pow2"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    Gp = w.n_groups + w.pad_groups
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group, pow2=True)
    qpad = np.full((w.T, Gp, w.D), 0x7F, np.uint8)
    spad = np.full((w.T, Gp, w.KB), np.nan, np.float32)
    qpad[:, : w.n_groups], spad[:, : w.n_groups] = qr, sr
    d_wq, d_ws, qwr, swr = _weights_both(w)
    U.assert_scales_bitexact(_host(d_ws), swr)
    idx = U.stratified_triples(np.random.default_rng(8), w.T, w.n_groups, w.o_lora_rank, extra=1000)
    ref = oracle.grouped_gemm(qpad, spad, qwr, swr, w.n_groups, w.o_lora_rank, 1, idx=idx)
    zg = gpu_gemm(w, qpad, spad, d_wq, d_ws, 1, True)
    assert np.all(np.isfinite(zg))
    e = U.rel_max_err(zg[idx[:, 0], idx[:, 1], idx[:, 2]], ref)
    assert e <= TOL, e


@pytest.mark.parametrize("T,G,R,brows,pow2", [(1, 2, 64, 128, False), (3, 1, 128, 1, False),
                                              (65, 2, 192, 128, False), (100, 3, 128, 1, True),
                                              (128, 2, 320, 1, False), (128, 1, 64, 128, True),
                                              (160, 2, 192, 128, False), (256, 3, 320, 1, True),
                                              (129, 2, 128, 128, True), (300, 2, 320, 128, False),
                                              (513, 1, 256, 1, False)])
def test_grouped_gemm_ragged(T, G, R, brows, pow2):
    """Ragged token counts around both kernels' tile edges, R not a multiple
    of 128, both weight-scale layouts, both scale recipes (dense check)."""
    w = wl.Workload(70 + T, "rag", T=T, n_groups=G, heads_per_group=8, o_lora_rank=R, max_pos=4096,
                    positions="uniform", pow2=pow2, w_block_rows=brows)
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, G, 8, pow2=pow2)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    ref = oracle.grouped_gemm(qr, sr, qwr, swr, G, R, brows)
    zg = gpu_gemm(w, qr, sr, d_wq, d_ws, brows, pow2)
    e = U.rel_max_err(zg, ref)
    assert e <= TOL, e


def _random_tile_shapes(n: int, seed: int):
    """Seeded random shapes on the tile kernel (T > 256): ragged M- and N-tiles,
    K-block counts 4 to 16, both weight-block layouts and both scale recipes."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append((int(rng.integers(257, 701)), int(rng.integers(1, 4)), 64 * int(rng.integers(1, 6)),
                    int(rng.choice([1, 2, 4])), int(rng.choice([1, 128])), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("T,G,R,hpg,brows,pow2", _random_tile_shapes(12, 2024))
def test_grouped_gemm_random_tile_shapes(T, G, R, hpg, brows, pow2):
    """Every output of the tile kernel (all three wave roles of its K loop,
    the weights-as-rows promotion, the MX path) against the oracle."""
    w = wl.Workload(300 + T + G + R, "rnd", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R,
                    max_pos=4096, positions="uniform", pow2=pow2, w_block_rows=brows)
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, G, hpg, pow2=pow2)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    ref = oracle.grouped_gemm(qr, sr, qwr, swr, G, R, brows)
    zg = gpu_gemm(w, qr, sr, d_wq, d_ws, brows, pow2)
    e = U.rel_max_err(zg, ref)
    assert e <= TOL, e


# Tile walks of the persistent tile kernel (one workgroup per CU, several
# tiles each): 276 tiles (not a multiple of the XCD count: plain order), 320
# and 544 tiles (XCD order), a ragged last M-tile (the next tile's first
# stage is then copied by that tile itself), R = 320 (ragged N-tiles, no
# chaining at all), both recipes and both weight-block layouts (fp32 with
# per-row weight scales runs the one-tile-per-workgroup kernel).
@pytest.mark.parametrize("T,G,hpg,R,brows,pow2", [(5639, 3, 2, 1024, 128, False), (2404, 8, 2, 1024, 128, False),
                                                  (4100, 16, 2, 320, 128, False), (2404, 8, 2, 1024, 128, True),
                                                  (2404, 8, 2, 1024, 1, True), (2404, 8, 2, 1024, 1, False)])
def test_grouped_gemm_persistent_tile_walks(T, G, hpg, R, brows, pow2):
    """Every output against the oracle's whole-tensor GEMM."""
    w = wl.Workload(400 + T + G + R + brows, "walk", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R,
                    max_pos=4096, positions="uniform", pow2=pow2, w_block_rows=brows)
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, G, hpg, pow2=pow2)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    U.assert_scales_bitexact(_host(d_ws), swr)
    ref = oracle.grouped_gemm_full(qr, sr, qwr, swr, G, R, brows)
    zg = gpu_gemm(w, qr, sr, d_wq, d_ws, brows, pow2)
    e = U.rel_max_err(zg, ref)
    assert e <= TOL, e


def _random_walks(n: int, seed: int):
    """Seeded random shapes with more tiles than CUs (several tiles per
    workgroup of the persistent tile kernel): ragged M and N tiles, every
    scale recipe and weight-block layout."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.integers(1500, 9001))
        G = int(rng.integers(2, 17))
        R = 64 * int(rng.integers(2, 17))
        tiles = G * -(-T // 256) * -(-R // 256)
        if tiles <= 256 or T * G * R > 40_000_000:
            continue
        out.append((T, G, int(rng.choice([1, 2])), R, int(rng.choice([1, 128])), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("T,G,hpg,R,brows,pow2", _random_walks(6, 2027))
def test_grouped_gemm_random_persistent_walks(T, G, hpg, R, brows, pow2):
    """Every output against the oracle's whole-tensor GEMM."""
    w = wl.Workload(500 + T + G + R, "rwalk", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R,
                    max_pos=4096, positions="uniform", pow2=pow2, w_block_rows=brows)
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, G, hpg, pow2=pow2)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    ref = oracle.grouped_gemm_full(qr, sr, qwr, swr, G, R, brows)
    zg = gpu_gemm(w, qr, sr, d_wq, d_ws, brows, pow2)
    e = U.rel_max_err(zg, ref)
    assert e <= TOL, e


def test_grouped_gemm_group_isolation_on_gpu():
    """Changing weight rows of other groups leaves a group's output unchanged."""
    w = wl.Workload(80, "iso", T=40, n_groups=3, heads_per_group=8, o_lora_rank=128, max_pos=4096,
                    positions="uniform")
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, 3, 8)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    z1 = gpu_gemm(w, qr, sr, _dev(qwr), _dev(swr), 128, False)
    qw2 = qwr.copy()
    qw2[: w.o_lora_rank] ^= 0x01
    qw2[2 * w.o_lora_rank:] ^= 0x01
    z2 = gpu_gemm(w, qr, sr, _dev(qw2), _dev(swr), 128, False)
    assert np.array_equal(z1[:, 1], z2[:, 1])
    assert not np.array_equal(z1[:, 0], z2[:, 0])


def test_fused_at_the_head_limit():
    """The whole path at the most heads the library takes: 8192 groups of 8
    heads (65536 heads, 2 GiB of FP8 weights), three tokens.  Codes and scales
    in full, z sampled, against the oracle."""
    T, G, hpg, R = 3, 8192, 8, 64
    w = wl.Workload(94, "heads", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R, max_pos=4096,
                    positions="uniform")
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    D, KB = w.D, w.KB
    qw = wl.fp8_codes(wl.seed_of(94, 10), G * R * D).reshape(G * R, D)
    sw = (2.0 ** (-12.0 + 4.0 * wl.uniform(wl.seed_of(94, 11), (G * R // 128) * KB))).astype(
        np.float32).reshape(G * R // 128, KB)
    shp = _shape(w)
    nb = ap.oproj_fused_workspace_bytes(shp, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    z = torch.empty((T, G, R), dtype=torch.int16, device=DEV)
    ap.oproj_fused(shp, 0, _dev(o.view(np.int16)), _dev(pos), _dev(tab), _dev(qw), _dev(sw),
                   ap.OPROJ_WBLOCK_128x128, None, 0, ws, nb, z)
    torch.cuda.synchronize()
    ncode = T * G * D
    codes = ws[:ncode].view(G, T, D)
    soff = (ncode + 255) // 256 * 256
    scales = ws[soff:soff + G * KB * T * 4].view(torch.float32).view(G, KB, T)
    qg, sg = U.group_major_to_token_major(_host(codes), _host(scales))
    qr, sr = oracle.inv_rope_quant(o, pos, tab, G, hpg)
    U.assert_scales_bitexact(sg, sr)
    U.assert_codes_parity(qg, qr)
    idx = U.sample_triples(np.random.default_rng(14), T, G, R, 4000)
    idx[4:8, 1] = [0, 1, G - 2, G - 1]
    zg = U.bf16_bits_to_f64(_host(z).view(np.uint16))
    ref = oracle.grouped_gemm(qr, sr, qw, sw, G, R, 128, idx=idx)
    e = U.rel_max_err(zg[idx[:, 0], idx[:, 1], idx[:, 2]], ref)
    assert e <= TOL, e


# ---------------------------------------------------------------- a4 and the fused entry point
def test_dense_bf16_gemm_parity():
    rng = np.random.default_rng(9)
    M, N, K = 200, 7168, 2048
    x = wl.bf16_matrix(wl.seed_of(91, 1), M, K, 1.0)
    wb = wl.bf16_matrix(wl.seed_of(91, 2), N, K, 0.02)
    y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    ap.oproj_dense_bf16_gemm(M, N, K, _dev(x.view(np.int16)), _dev(wb.view(np.int16)), y)
    yg = U.bf16_bits_to_f64(_host(y).view(np.uint16))
    idx = np.stack([rng.integers(0, M, 4000), rng.integers(0, N, 4000)], axis=1)
    idx[:2] = [[0, 0], [M - 1, N - 1]]
    ref = oracle.dense_gemm_bf16(x, wb, idx=idx)
    e = U.rel_max_err(yg[idx[:, 0], idx[:, 1]], ref)
    assert e <= TOL, e


@pytest.mark.parametrize("M,N,K", [(600, 1040, 192), (1, 16, 64), (257, 272, 128), (513, 784, 320),
                                   (2048, 1792, 128), (1800, 1776, 192)])
def test_dense_bf16_gemm_ragged(M, N, K):
    """Several tiles with ragged M and N tails and odd step counts, checked
    densely; the last two shapes take the 256x224 tiles."""
    x = wl.bf16_matrix(wl.seed_of(92, M), M, K, 1.0)
    wb = wl.bf16_matrix(wl.seed_of(93, N), N, K, 0.02)
    y, gy = U.guarded_empty((M, N), torch.int16, DEV)
    ap.oproj_dense_bf16_gemm(M, N, K, _dev(x.view(np.int16)), _dev(wb.view(np.int16)), y)
    torch.cuda.synchronize()
    assert U.guard_intact(gy, y), "write past the end of y"
    yg = U.bf16_bits_to_f64(_host(y).view(np.uint16))
    ref = oracle.dense_gemm_bf16(x, wb)
    e = U.rel_max_err(yg, ref)
    assert e <= TOL, e


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_fused_equals_steps(name):
    w = wl.WORKLOADS[name]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    shp = _shape(w)
    d_o, d_pos, d_tab = _dev(o.view(np.int16)), _dev(pos), _dev(tab)
    nbytes = ap.oproj_fused_workspace_bytes(shp, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    zf = torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)
    ap.oproj_fused(shp, 0, d_o, d_pos, d_tab, d_wq, d_ws, 0, None, 0, ws, nbytes, zf)
    codes = torch.empty((w.n_groups, w.T, w.D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.n_groups, w.KB, w.T), dtype=torch.float32, device=DEV)
    ap.oproj_inv_rope_quant(shp, 0, d_o, d_pos, d_tab, codes, scales)
    zs = torch.empty_like(zf)
    ap.oproj_grouped_wo_a(shp, 0, codes, scales, None, d_wq, d_ws, 0, zs)
    assert torch.equal(zf, zs)
    # the workspace holds the same codes and scales (default layout, first two regions)
    ncode = w.n_groups * w.T * w.D
    assert torch.equal(ws[:ncode], codes.view(-1))
    soff = (ncode + 255) // 256 * 256
    assert torch.equal(ws[soff:soff + scales.numel() * 4].view(torch.int32), scales.view(-1).view(torch.int32))
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group)
    ref = oracle.grouped_gemm(qr, sr, qwr, swr, w.n_groups, w.o_lora_rank)
    assert U.rel_max_err(U.bf16_bits_to_f64(_host(zf).view(np.uint16)), ref) <= TOL


@pytest.mark.parametrize("T,G,hpg,R,pow2,brows", [(32, 4, 8, 256, True, 1), (17, 3, 1, 128, False, 128),
                                                  (9, 5, 2, 192, True, 128), (64, 2, 16, 64, False, 1)])
def test_fused_small_batches(T, G, hpg, R, pow2, brows):
    """oproj_fused on small batches equals the two separate calls bit for bit,
    for every scale recipe and head-chunk size, and matches the oracle."""
    w = wl.Workload(70 + T, f"f{T}", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R, max_pos=4096,
                    positions="uniform", pow2=pow2, w_block_rows=brows)
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    shp = _shape(w)
    mode = int(pow2)
    blk = ap.OPROJ_WBLOCK_1x128 if brows == 1 else ap.OPROJ_WBLOCK_128x128
    d_o, d_pos, d_tab = _dev(o.view(np.int16)), _dev(pos), _dev(tab)
    nbytes = ap.oproj_fused_workspace_bytes(shp, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    zf = torch.empty((T, G, R), dtype=torch.int16, device=DEV)
    ap.oproj_fused(shp, mode, d_o, d_pos, d_tab, d_wq, d_ws, blk, None, 0, ws, nbytes, zf)
    codes = torch.empty((G, T, w.D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((G, w.KB, T), dtype=torch.float32, device=DEV)
    ap.oproj_inv_rope_quant(shp, mode, d_o, d_pos, d_tab, codes, scales)
    zs = torch.empty_like(zf)
    ap.oproj_grouped_wo_a(shp, mode, codes, scales, None, d_wq, d_ws, blk, zs)
    assert torch.equal(zf, zs)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, G, hpg, pow2=pow2)
    ref = oracle.grouped_gemm(qr, sr, qwr, swr, G, R, brows)
    assert U.rel_max_err(U.bf16_bits_to_f64(_host(zf).view(np.uint16)), ref) <= TOL


def test_fused_decode_with_wo_b():
    """The decode batch through oproj_fused with wo_b (a1..a4 in one call)."""
    w = wl.WORKLOADS["decode"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    hidden = 512
    wob = wl.bf16_matrix(wl.seed_of(94, 1), hidden, w.n_groups * w.o_lora_rank, 0.02)
    shp = _shape(w)
    nbytes = ap.oproj_fused_workspace_bytes(shp, hidden)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    y = torch.empty((w.T, hidden), dtype=torch.int16, device=DEV)
    ap.oproj_fused(shp, 0, _dev(o.view(np.int16)), _dev(pos), _dev(tab), d_wq, d_ws, 0,
                   _dev(wob.view(np.int16)), hidden, ws, nbytes, y)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group)
    zb = oracle.f64_to_bf16(oracle.grouped_gemm(qr, sr, qwr, swr, w.n_groups, w.o_lora_rank))
    ref = oracle.dense_gemm_bf16(zb.reshape(w.T, -1), wob)
    assert U.rel_max_err(U.bf16_bits_to_f64(_host(y).view(np.uint16)), ref) <= TOL


def test_fused_decode_graph_replays():
    """oproj_fused on the decode batch captured in a HIP graph: every replay
    (with eager work and new inputs between replays) equals the eager result."""
    w = wl.WORKLOADS["decode"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws, _, _ = _weights_both(w)
    shp = _shape(w)
    d_o, d_pos, d_tab = _dev(o.view(np.int16)), _dev(pos), _dev(tab)
    nbytes = ap.oproj_fused_workspace_bytes(shp, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    z = torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)

    def run():
        ap.oproj_fused(shp, 0, d_o, d_pos, d_tab, d_wq, d_ws, 0, None, 0, ws, nbytes, z)

    run()
    ref0 = _host(z).copy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    o2 = o.copy()
    o2[::3] = o[::-1][::3]
    for rep in range(4):
        g.replay()
        assert np.array_equal(_host(z), ref0), f"replay {rep}"
        run()  # eager launch between replays
        assert np.array_equal(_host(z), ref0)
    d_o.copy_(_dev(o2.view(np.int16)))
    run()
    ref1 = _host(z).copy()
    assert not np.array_equal(ref1, ref0)
    for rep in range(2):
        g.replay()
        assert np.array_equal(_host(z), ref1), f"replay {rep} on new input"


def test_full_path_with_wo_b_sampled():
    """The whole path at its full size: a1..a4 through oproj_fused; sampled y
    against the oracle chain (oracle z rounded to bf16, then fp64 wo_b)."""
    w = wl.WORKLOADS["full"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    wob = wl.wo_b_bf16(w)
    shp = _shape(w)
    nbytes = ap.oproj_fused_workspace_bytes(shp, w.hidden)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    y = torch.empty((w.T, w.hidden), dtype=torch.int16, device=DEV)
    ap.oproj_fused(shp, 0, _dev(o.view(np.int16)), _dev(pos), _dev(tab), d_wq, d_ws, 0,
                   _dev(wob.view(np.int16)), w.hidden, ws, nbytes, y)
    yg = U.bf16_bits_to_f64(_host(y).view(np.uint16))
    assert np.all(np.isfinite(yg))
    rng = np.random.default_rng(10)
    toks = np.concatenate([[0, w.T - 1], rng.choice(w.T, 14, replace=False)])
    qr, sr = oracle.inv_rope_quant(o[toks], pos[toks], tab, w.n_groups, w.heads_per_group)
    zr = oracle.grouped_gemm(qr, sr, qwr, swr, w.n_groups, w.o_lora_rank)
    zb = oracle.f64_to_bf16(zr).reshape(len(toks), w.n_groups * w.o_lora_rank)
    cols = rng.integers(0, w.hidden, 128)
    idx = np.array([[i, c] for i in range(len(toks)) for c in cols], np.int64)
    ref = oracle.dense_gemm_bf16(zb, wob, idx=idx)
    got = yg[toks[idx[:, 0]], idx[:, 1]]
    e = U.rel_max_err(got, ref)
    assert e <= TOL, e


# ---------------------------------------------------------------- packed UE8M0 activation scales
def _quant_both_modes(w, o, pos, tab):
    """GPU a1+a2 in POW2 mode (fp32 scales) and in E8M0 mode (packed words), default layouts."""
    T = o.shape[0]
    shp = _shape(w, T)
    d_o, d_pos, d_tab = _dev(o.view(np.int16)), _dev(pos), _dev(tab)
    c2 = torch.empty((w.n_groups, T, w.D), dtype=torch.uint8, device=DEV)
    s2 = torch.empty((w.n_groups, w.KB, T), dtype=torch.float32, device=DEV)
    ap.oproj_inv_rope_quant(shp, ap.OPROJ_SCALE_POW2, d_o, d_pos, d_tab, c2, s2)
    c8 = torch.empty_like(c2)
    s8 = torch.empty((w.n_groups, w.KB // 4, T), dtype=torch.int32, device=DEV)
    ap.oproj_inv_rope_quant(shp, ap.OPROJ_SCALE_E8M0, d_o, d_pos, d_tab, c8, s8)
    return c2, s2, c8, s8


@pytest.mark.parametrize("name", ["tiny", "decode", "full"])
def test_inv_rope_quant_e8m0_words(name):
    """E8M0 mode: codes equal the POW2 mode's; the packed words are bit-exact
    against the oracle's packing of its pow2 scales."""
    w = wl.WORKLOADS[name]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    c2, s2, c8, s8 = _quant_both_modes(w, o, pos, tab)
    assert torch.equal(c2, c8)
    _, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group, pow2=True)
    want = oracle.e8m0_pack(sr)  # [T, G, KB/4]
    got = np.ascontiguousarray(np.transpose(_host(s8).view(np.uint32), (2, 0, 1)))
    assert np.array_equal(got, want)


def test_inv_rope_quant_e8m0_bad_position_is_ff():
    w = wl.WORKLOADS["tiny"]
    o, pos, tab = wl.attn_out(w), wl.positions(w).copy(), wl.table(w)
    pos[2] = -1
    _, _, _, s8 = _quant_both_modes(w, o, pos, tab)
    b = _host(s8).view(np.uint8).reshape(w.n_groups, w.KB // 4, w.T, 4)
    assert (b[:, :, 2, :] == 0xFF).all() and (b[:, :, [0, 1, 3], :] != 0xFF).all()


@pytest.mark.parametrize("T", [64, 300])
def test_grouped_gemm_e8m0_equals_pow2(T):
    """The GEMM fed packed UE8M0 words gives the same z, bit for bit, as with
    the fp32 powers of two (few-token and tile kernels), and meets the bar."""
    w = wl.WORKLOADS["decode"].scaled(T)
    o, tab = wl.attn_out(w), wl.table(w)
    pos = wl.uniform_int(wl.seed_of(77, T), T, 0, w.max_pos)
    c2, s2, c8, s8 = _quant_both_modes(w, o, pos, tab)
    wmat = wl.wo_a_f32(w)
    d_wq, d_ws = gpu_weight(wmat, 1, True)
    shp = _shape(w, T)
    z2 = torch.empty((T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)
    z8 = torch.empty_like(z2)
    ap.oproj_grouped_wo_a(shp, ap.OPROJ_SCALE_POW2, c2, s2, None, d_wq, d_ws, ap.OPROJ_WBLOCK_1x128, z2)
    ap.oproj_grouped_wo_a(shp, ap.OPROJ_SCALE_E8M0, c8, s8, None, d_wq, d_ws, ap.OPROJ_WBLOCK_1x128, z8)
    assert torch.equal(z2, z8)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group, pow2=True)
    qw, sw = oracle.quant_weight(wmat, 1, True)
    rng = np.random.default_rng(78)
    idx = U.sample_triples(rng, T, w.n_groups, w.o_lora_rank, 2000)
    ref = oracle.grouped_gemm(qr, sr, qw, sw, w.n_groups, w.o_lora_rank, 1, idx=idx)
    zg = U.bf16_bits_to_f64(_host(z8).view(np.uint16))
    assert U.rel_max_err(zg[idx[:, 0], idx[:, 1], idx[:, 2]], ref) <= TOL


def test_grouped_gemm_e8m0_token_major_layout():
    """Packed words in a token-major [T][G][KB/4] layout through the strides."""
    w = wl.WORKLOADS["tiny"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group, pow2=True)
    words = oracle.e8m0_pack(sr)  # [T, G, KB/4]
    wmat = wl.wo_a_f32(w)
    d_wq, d_ws = gpu_weight(wmat, 128, True)
    lay = ap.ActLayout(w.n_groups * w.D, w.D, w.n_groups * (w.KB // 4), w.KB // 4, 1)
    z = torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)
    ap.oproj_grouped_wo_a(_shape(w), ap.OPROJ_SCALE_E8M0, _dev(qr), _dev(words.view(np.int32)), lay,
                          d_wq, d_ws, ap.OPROJ_WBLOCK_128x128, z)
    qw, sw = oracle.quant_weight(wmat, 128, True)
    ref = oracle.grouped_gemm(qr, sr, qw, sw, w.n_groups, w.o_lora_rank, 128)
    assert U.rel_max_err(U.bf16_bits_to_f64(_host(z).view(np.uint16)), ref) <= TOL


def test_fused_e8m0_equals_steps():
    w = wl.WORKLOADS["decode"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws = gpu_weight(wl.wo_a_f32(w), 128, True)
    shp = _shape(w)
    d_o, d_pos, d_tab = _dev(o.view(np.int16)), _dev(pos), _dev(tab)
    nbytes = ap.oproj_fused_workspace_bytes(shp, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    zf = torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)
    ap.oproj_fused(shp, ap.OPROJ_SCALE_E8M0, d_o, d_pos, d_tab, d_wq, d_ws, 0, None, 0, ws, nbytes, zf)
    _, _, c8, s8 = _quant_both_modes(w, o, pos, tab)
    zs = torch.empty_like(zf)
    ap.oproj_grouped_wo_a(shp, ap.OPROJ_SCALE_E8M0, c8, s8, None, d_wq, d_ws, 0, zs)
    assert torch.equal(zf, zs)


# ---------------------------------------------------------------- packed UE8M0 weight scales
def _weight_ue8m0(wmat):
    rows, K = wmat.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device=DEV)
    words = torch.empty((rows, K // 512), dtype=torch.int32, device=DEV)
    ap.oproj_quantize_weight(rows, K, ap.OPROJ_WBLOCK_1x128_UE8M0, ap.OPROJ_SCALE_POW2, _dev(wmat), codes, words)
    return codes, words


def test_weight_quant_ue8m0_words():
    w = wl.WORKLOADS["decode"]
    wmat = wl.wo_a_f32(w)
    c8, w8 = _weight_ue8m0(wmat)
    c2, s2 = gpu_weight(wmat, 1, True)
    assert torch.equal(c8, c2)
    qr, sr = oracle.quant_weight(wmat, 1, True)
    assert np.array_equal(_host(w8).view(np.uint32), oracle.e8m0_pack(sr))


@pytest.mark.parametrize("T,amode", [(64, 1), (64, 2), (300, 2), (300, 1)])
def test_grouped_gemm_ue8m0_weights_equal_fp32_pow2(T, amode):
    """Packed UE8M0 weight scales give the same z, bit for bit, as the same
    powers of two stored as fp32 (few-token and tile kernels)."""
    w = wl.WORKLOADS["decode"].scaled(T)
    o, tab = wl.attn_out(w), wl.table(w)
    pos = wl.uniform_int(wl.seed_of(79, T), T, 0, w.max_pos)
    c2, s2, c8, s8 = _quant_both_modes(w, o, pos, tab)
    codes, scales = (c2, s2) if amode == 1 else (c8, s8)
    wmat = wl.wo_a_f32(w)
    wc, ws32 = gpu_weight(wmat, 1, True)
    wc8, ws8 = _weight_ue8m0(wmat)
    shp = _shape(w, T)
    za = torch.empty((T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)
    zb = torch.empty_like(za)
    ap.oproj_grouped_wo_a(shp, amode, codes, scales, None, wc, ws32, ap.OPROJ_WBLOCK_1x128, za)
    ap.oproj_grouped_wo_a(shp, amode, codes, scales, None, wc8, ws8, ap.OPROJ_WBLOCK_1x128_UE8M0, zb)
    assert torch.equal(za, zb)


# ---------------------------------------------------------------- every output at full size
# The whole-tensor oracle forms (each operand dequantised once, an fp64
# product per group) make every output of the full-size workloads checkable.
@pytest.mark.parametrize("name", ["prefill", "full"])
def test_grouped_gemm_every_output_full_size(name):
    """Every z of the prefill (T=8192) and full (T=4096) batches: end to end
    (GPU codes, GPU weights) and isolated (oracle codes and weights into the
    GPU GEMM), against the oracle chain."""
    w = wl.WORKLOADS[name]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    U.assert_scales_bitexact(_host(d_ws), swr)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group)
    ref = oracle.grouped_gemm_full(qr, sr, qwr, swr, w.n_groups, w.o_lora_rank, w.w_block_rows)
    shp = _shape(w)
    codes = torch.empty((w.n_groups, w.T, w.D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.n_groups, w.KB, w.T), dtype=torch.float32, device=DEV)
    ap.oproj_inv_rope_quant(shp, 0, _dev(o.view(np.int16)), _dev(pos), _dev(tab), codes, scales)
    z, gz = U.guarded_empty((w.T, w.n_groups, w.o_lora_rank), torch.int16, DEV)
    ap.oproj_grouped_wo_a(shp, 0, codes, scales, None, d_wq, d_ws, ap.OPROJ_WBLOCK_128x128, z)
    torch.cuda.synchronize()
    assert U.guard_intact(gz, z)
    del codes, scales
    e = U.rel_max_err(U.bf16_bits_to_f64(_host(z).view(np.uint16)), ref)
    assert e <= TOL, f"end to end: E = {e:.3e}"
    zi = gpu_gemm(w, qr, sr, _dev(qwr), _dev(swr), w.w_block_rows, w.pow2)
    e = U.rel_max_err(zi, ref)
    assert e <= TOL, f"isolated: E = {e:.3e}"


@pytest.mark.parametrize("T,G,pow2,brows", [(512, 16, False, 128), (513, 16, False, 128), (1000, 8, True, 1),
                                             (384, 16, True, 1), (200, 16, False, 128), (128, 16, True, 1)])
def test_grouped_gemm_every_output_both_tile_heights(T, G, pow2, brows):
    """Every z around the kernels' choice of tile at 16 and 8 groups of 1024
    columns.  Tile kernel: 512 tokens (16 groups) and 1000 tokens (8 groups)
    run 256 tiles of 128 rows, one per CU, in the XCD tile order; 513 tokens
    runs 192 tiles of 256 rows; 384 tokens 192 tiles of 128 rows.  Decode
    kernel with 128-token tiles: 200 tokens in two rounds of 256 workgroups,
    128 tokens in one.  Both scale recipes, against the oracle chain."""
    w = wl.Workload(900 + T, "heights", T=T, n_groups=G, heads_per_group=8, o_lora_rank=1024, max_pos=8192,
                    positions="uniform", pow2=pow2, w_block_rows=brows)
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, G, 8, pow2=pow2)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    ref = oracle.grouped_gemm_full(qr, sr, qwr, swr, G, 1024, brows)
    zg = gpu_gemm(w, qr, sr, d_wq, d_ws, brows, pow2)
    e = U.rel_max_err(zg, ref)
    assert e <= TOL, e


def test_grouped_gemm_every_output_pow2_padded():
    """Every z of the pow2 batch: the pre-quantised [T, 10, D] input (groups
    8-9 NaN) with 1x128 power-of-two weight scales."""
    w = wl.WORKLOADS["pow2"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    Gp = w.n_groups + w.pad_groups
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group, pow2=True)
    qpad = np.full((w.T, Gp, w.D), 0x7F, np.uint8)
    spad = np.full((w.T, Gp, w.KB), np.nan, np.float32)
    qpad[:, : w.n_groups], spad[:, : w.n_groups] = qr, sr
    d_wq, d_ws, qwr, swr = _weights_both(w)
    U.assert_scales_bitexact(_host(d_ws), swr)
    ref = oracle.grouped_gemm_full(qpad, spad, qwr, swr, w.n_groups, w.o_lora_rank, 1)
    zg = gpu_gemm(w, qpad, spad, d_wq, d_ws, 1, True)
    assert np.all(np.isfinite(zg))
    e = U.rel_max_err(zg, ref)
    assert e <= TOL, e


def test_full_path_every_output_with_wo_b():
    """The whole path at the full batch through oproj_fused with wo_b: every z
    (read from the workspace, where a3 leaves it for a4) and every y, against
    the oracle chain (oracle z rounded once to bf16, then fp64 wo_b)."""
    w = wl.WORKLOADS["full"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    d_wq, d_ws, qwr, swr = _weights_both(w)
    wob = wl.wo_b_bf16(w)
    shp = _shape(w)
    nbytes = ap.oproj_fused_workspace_bytes(shp, w.hidden)
    ws, gws = U.guarded_empty((nbytes,), torch.uint8, DEV)
    y, gy = U.guarded_empty((w.T, w.hidden), torch.int16, DEV)
    ap.oproj_fused(shp, 0, _dev(o.view(np.int16)), _dev(pos), _dev(tab), d_wq, d_ws, 0,
                   _dev(wob.view(np.int16)), w.hidden, ws, nbytes, y)
    torch.cuda.synchronize()
    assert U.guard_intact(gws, ws) and U.guard_intact(gy, y)
    rnd = lambda v: (v + 255) // 256 * 256
    zoff = rnd(w.T * w.n_groups * w.D) + rnd(w.T * w.n_groups * w.KB * 4)
    zb_gpu = _host(ws[zoff: zoff + w.T * w.n_groups * w.o_lora_rank * 2]).view(np.uint16)
    qr, sr = oracle.inv_rope_quant(o, pos, tab, w.n_groups, w.heads_per_group)
    zr = oracle.grouped_gemm_full(qr, sr, qwr, swr, w.n_groups, w.o_lora_rank)
    e = U.rel_max_err(U.bf16_bits_to_f64(zb_gpu).reshape(zr.shape), zr)
    assert e <= TOL, f"z: E = {e:.3e}"
    zb = oracle.f64_to_bf16(zr).reshape(w.T, w.n_groups * w.o_lora_rank)
    del zr
    yr = oracle.dense_gemm_bf16_full(zb, wob)
    yg = U.bf16_bits_to_f64(_host(y).view(np.uint16))
    assert np.all(np.isfinite(yg))
    e = U.rel_max_err(yg, yr)
    assert e <= TOL, f"y: E = {e:.3e}"
