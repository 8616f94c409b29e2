"""The attention-epilogue producer (oproj_inv_rope_quant_f32: inverse RoPE +
1x128 FP8 quantisation from fp32 attention output) against the oracle's
producer on the same seeded fp32 inputs: scales bit-exact, codes identical up
to the one-step tolerance, for every scale recipe, the decode batch, ragged
shapes, degenerate blocks and a strided output layout; and bit-identity with
the bf16 entry point on inputs that are bf16 values."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_output_projection_amd as ap
import oracle
import workloads as wl
from tests import _util as U

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ap.load_library()
    yield
    torch.cuda.synchronize()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _f32_out(T, H, seed):
    """fp32 attention output with low mantissa bits set (not bf16 values)."""
    return wl.normal(seed, T * H * 512).astype(np.float32).reshape(T, H, 512)


def gpu_quant_f32(x, pos, tab, G, hpg, mode):
    """GPU producer into the default group-major layout -> token-major codes and
    fp32 scales (UE8M0 words are returned as they are)."""
    T = x.shape[0]
    shp = ap.Shape(T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=64, max_pos=tab.shape[0])
    KB = hpg * 4
    codes = torch.empty((G, T, hpg * 512), dtype=torch.uint8, device=DEV)
    if mode == ap.OPROJ_SCALE_E8M0:
        scales = torch.empty((G, KB // 4, T), dtype=torch.int32, device=DEV)
    else:
        scales = torch.empty((G, KB, T), dtype=torch.float32, device=DEV)
    ap.oproj_inv_rope_quant_f32(shp, mode, _dev(x), _dev(pos), _dev(tab), codes, scales)
    torch.cuda.synchronize()
    q = codes.cpu().numpy().transpose(1, 0, 2)
    s = scales.cpu().numpy().transpose(2, 0, 1)
    return np.ascontiguousarray(q), np.ascontiguousarray(s)


@pytest.mark.parametrize("T,G,hpg", [(4, 2, 2), (64, 16, 8), (1, 1, 1), (37, 3, 4), (130, 2, 16)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_f32_producer_parity(T, G, hpg, mode):
    x = _f32_out(T, G * hpg, 700 + T + G + hpg)
    max_pos = 32768
    pos = wl.uniform_int(wl.seed_of(700 + T, 2), T, 0, max_pos).astype(np.int64)
    pos[0] = 0
    tab = wl.cos_sin_table(max_pos, 64)
    qg, sg = gpu_quant_f32(x, pos, tab, G, hpg, mode)
    qr, sr = oracle.inv_rope_quant_f32(x, pos, tab, G, hpg, pow2=mode != 0)
    U.assert_codes_parity(qg, qr)
    if mode == 2:
        assert np.array_equal(sg.view(np.uint32), oracle.e8m0_pack(sr))
    else:
        U.assert_scales_bitexact(sg, sr)


@pytest.mark.parametrize("mode", [0, 2])
def test_f32_producer_pipelined_launch(mode):
    """Enough items for the pipelined instance with four-head items and the
    fixed wave population that bench.py times at prefill (T=2048, 16 x 8
    heads), checked in full against the oracle."""
    T, G, hpg = 2048, 16, 8
    x = wl.normal_f32_bulk(wl.seed_of(750, 1), T * G * hpg * 512).reshape(T, G * hpg, 512)
    tab = wl.cos_sin_table(32768, 64)
    pos = wl.uniform_int(wl.seed_of(750, 2), T, 0, 32768).astype(np.int64)
    qg, sg = gpu_quant_f32(x, pos, tab, G, hpg, mode)
    qr, sr = oracle.inv_rope_quant_f32(x, pos, tab, G, hpg, pow2=mode != 0)
    U.assert_codes_parity(qg, qr)
    if mode == 2:
        assert np.array_equal(sg.view(np.uint32), oracle.e8m0_pack(sr))
    else:
        U.assert_scales_bitexact(sg, sr)


def test_f32_producer_equals_bf16_entry_point_on_bf16_values():
    w = wl.WORKLOADS["decode"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    shp = ap.Shape(T=w.T, n_groups=w.n_groups, heads_per_group=w.heads_per_group, o_lora_rank=w.o_lora_rank,
                   max_pos=w.max_pos)
    outs = []
    for f32 in (False, True):
        codes = torch.empty((w.n_groups, w.T, w.D), dtype=torch.uint8, device=DEV)
        scales = torch.empty((w.n_groups, w.KB, w.T), dtype=torch.float32, device=DEV)
        if f32:
            ap.oproj_inv_rope_quant_f32(shp, 0, _dev(wl.bf16_bits_to_f32(o)), _dev(pos), _dev(tab), codes, scales)
        else:
            ap.oproj_inv_rope_quant(shp, 0, _dev(o.view(np.int16)), _dev(pos), _dev(tab), codes, scales)
        outs.append((codes, scales))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))


def test_f32_producer_degenerate_blocks_and_bad_positions():
    """Zero blocks, tiny and huge magnitudes; a position outside the table
    gives NaN scales for its token only."""
    T, G, hpg = 6, 2, 2
    x = _f32_out(T, G * hpg, 731)
    x[0] = 0.0
    x[1, 0, :128] = 0.0
    x[2] *= 1e-30
    x[3] *= 1e30
    tab = wl.cos_sin_table(64, 64)
    pos = np.array([0, 1, 2, 63, 64, 5], np.int64)  # token 4 is out of range
    for mode in (0, 1):
        qg, sg = gpu_quant_f32(x, pos, tab, G, hpg, mode)
        ok = [0, 1, 2, 3, 5]
        qr, sr = oracle.inv_rope_quant_f32(x[ok], pos[ok], tab, G, hpg, pow2=mode == 1)
        U.assert_scales_bitexact(sg[ok], sr)
        U.assert_codes_parity(qg[ok], qr, frac=0.0)
        assert np.all(np.isnan(sg[4]))


def test_f32_producer_strided_layout_leaves_padding_alone():
    """Token-major output with two padding groups: only live groups are written."""
    T, G, hpg, Gp = 9, 3, 2, 5
    x = _f32_out(T, G * hpg, 741)
    tab = wl.cos_sin_table(4096, 64)
    pos = wl.uniform_int(wl.seed_of(741, 2), T, 0, 4096).astype(np.int64)
    D, KB = hpg * 512, hpg * 4
    codes = torch.full((T, Gp, D), 0x7F, dtype=torch.uint8, device=DEV)
    scales = torch.full((T, Gp, KB), float("nan"), dtype=torch.float32, device=DEV)
    lay = ap.ActLayout(Gp * D, D, Gp * KB, KB, 1)
    shp = ap.Shape(T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=64, max_pos=4096)
    ap.oproj_inv_rope_quant_f32(shp, 0, _dev(x), _dev(pos), _dev(tab), codes, scales, lay)
    torch.cuda.synchronize()
    qg, sg = codes.cpu().numpy(), scales.cpu().numpy()
    qr, sr = oracle.inv_rope_quant_f32(x, pos, tab, G, hpg)
    U.assert_scales_bitexact(sg[:, :G], sr)
    U.assert_codes_parity(qg[:, :G], qr)
    assert np.all(qg[:, G:] == 0x7F) and np.all(np.isnan(sg[:, G:]))


def test_f32_producer_beyond_4gib_input():
    """The producer on an fp32 input larger than 4 GiB (T = 2100 tokens of
    1024 heads; token t starts at 2t MiB), so that rows past 2^31 and 2^32
    bytes are read.  Tokens on both sides of those offsets and at the end
    against the oracle."""
    T, G, hpg = 2100, 128, 8
    x = wl.normal_f32_bulk(wl.seed_of(760, 1), T * G * hpg * 512).reshape(T, G * hpg, 512)
    tab = wl.cos_sin_table(32768, 64)
    pos = wl.uniform_int(wl.seed_of(760, 2), T, 0, 32768).astype(np.int64)
    shp = ap.Shape(T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=64, max_pos=tab.shape[0])
    d_x = _dev(x)
    codes = torch.empty((G, T, hpg * 512), dtype=torch.uint8, device=DEV)
    scales = torch.empty((G, hpg * 4, T), dtype=torch.float32, device=DEV)
    ap.oproj_inv_rope_quant_f32(shp, 0, d_x, _dev(pos), _dev(tab), codes, scales)
    torch.cuda.synchronize()
    del d_x
    sel = np.array([0, 1, 1023, 1024, 1025, 2047, 2048, 2049, 2098, 2099], np.int64)
    tsel = torch.from_numpy(sel).to(DEV)
    qg = np.ascontiguousarray(codes[:, tsel, :].cpu().numpy().transpose(1, 0, 2))
    sg = np.ascontiguousarray(scales[:, :, tsel].cpu().numpy().transpose(2, 0, 1))
    qr, sr = oracle.inv_rope_quant_f32(x[sel], pos[sel], tab, G, hpg)
    U.assert_codes_parity(qg, qr)
    U.assert_scales_bitexact(sg, sr)
