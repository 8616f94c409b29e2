"""GPU parity of the unquantised path (bf16 inverse RoPE -> grouped bf16
wo_a) through the C ABI against the CPU oracle on the same seeded inputs.

Bars: the bf16 rotation is bit-exact (both sides round the same fp32 value
to nearest even); the grouped GEMM meets E = max|y-r|/max|r| <= 1e-2 against
the oracle's fp64 result (dense at small sizes; every output of the prefill batch through the
oracle's whole-tensor product, sampled at the offset limits).
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


def _shape(w: wl.Workload, T: int | None = None, R: int | None = None) -> ap.Shape:
    return ap.Shape(T=w.T if T is None else T, n_groups=w.n_groups, heads_per_group=w.heads_per_group,
                    o_lora_rank=w.o_lora_rank if R is None else R, max_pos=w.max_pos)


def gpu_rope_bf16(w: wl.Workload, o, pos, tab, group_major: bool = False) -> np.ndarray:
    """GPU unquantised a1 -> token-major [T, G, D] bf16 bits."""
    T = o.shape[0]
    shp = _shape(w, T)
    if group_major:
        x = torch.empty((w.n_groups, T, w.D), dtype=torch.int16, device=DEV)
        lay = ap.Bf16Layout(w.D, T * w.D)
    else:
        x = torch.empty((T, w.n_groups, w.D), dtype=torch.int16, device=DEV)
        lay = None
    ap.oproj_inv_rope_bf16(shp, _dev(o.view(np.int16)), _dev(pos), _dev(tab), x, lay)
    h = _host(x).view(np.uint16)
    return np.ascontiguousarray(np.transpose(h, (1, 0, 2))) if group_major else h


@pytest.mark.parametrize("name", ["tiny", "decode", "full"])
def test_inv_rope_bf16_bitexact_workloads(name):
    w = wl.WORKLOADS[name]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    got = gpu_rope_bf16(w, o, pos, tab)
    ref = oracle.inv_rope_bf16(o, pos, tab).reshape(w.T, w.n_groups, w.D)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("T,G,hpg", [(1, 1, 1), (3, 2, 2), (5, 3, 4), (37, 2, 8), (130, 1, 16)])
def test_inv_rope_bf16_ragged_and_group_major(T, G, hpg):
    w = wl.Workload(40 + T, "r", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=64, max_pos=4096,
                    positions="uniform")
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    ref = oracle.inv_rope_bf16(o, pos, tab).reshape(T, G, w.D)
    assert np.array_equal(gpu_rope_bf16(w, o, pos, tab), ref)
    assert np.array_equal(gpu_rope_bf16(w, o, pos, tab, group_major=True), ref)


def test_inv_rope_bf16_bad_position_is_nan_and_t0_noop():
    w = wl.WORKLOADS["tiny"]
    o, pos, tab = wl.attn_out(w), wl.positions(w).copy(), wl.table(w)
    pos[1] = w.max_pos  # out of range
    got = gpu_rope_bf16(w, o, pos, tab).reshape(w.T, w.H, 512)
    f = U.bf16_bits_to_f64(got)
    assert np.isnan(f[1, :, 448:]).all() and np.isfinite(f[1, :, :448]).all()
    ok = np.array([0, 2, 3])
    ref = oracle.inv_rope_bf16(o[ok], pos[ok], tab)
    assert np.array_equal(got[ok], ref)
    ap.oproj_inv_rope_bf16(_shape(w, 0), None, None, None, None)  # T == 0: nothing to do


def gpu_gemm_bf16(w: wl.Workload, x_tgd, wq, R: int | None = None, group_major: bool = False) -> np.ndarray:
    T = x_tgd.shape[0]
    R = w.o_lora_rank if R is None else R
    shp = _shape(w, T, R)
    if group_major:
        d_x = _dev(np.ascontiguousarray(np.transpose(x_tgd, (1, 0, 2))).view(np.int16))
        lay = ap.Bf16Layout(w.D, T * w.D)
    else:
        d_x = _dev(x_tgd.view(np.int16))
        lay = None
    z, gz = U.guarded_empty((T, w.n_groups, R), torch.int16, DEV)
    ap.oproj_grouped_wo_a_bf16(shp, d_x, lay, _dev(wq.view(np.int16)), z)
    out = U.bf16_bits_to_f64(_host(z).view(np.uint16))
    assert U.guard_intact(gz, z), "bytes after z were written"
    return out


def test_grouped_wo_a_bf16_decode_dense_and_end_to_end():
    w = wl.WORKLOADS["decode"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    x = oracle.inv_rope_bf16(o, pos, tab).reshape(w.T, w.n_groups, w.D)
    wq = wl.wo_a_bf16(w)
    ref = oracle.grouped_gemm_bf16(x, wq, w.n_groups, w.o_lora_rank)
    # isolated: the GPU GEMM on the oracle's x
    e = U.rel_max_err(gpu_gemm_bf16(w, x, wq), ref)
    assert e <= TOL, e
    # end to end: the GPU's own x, fed on the device from one kernel to the next
    shp = _shape(w)
    d_x = torch.empty((w.T, w.n_groups, w.D), dtype=torch.int16, device=DEV)
    z = torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)
    ap.oproj_inv_rope_bf16(shp, _dev(o.view(np.int16)), _dev(pos), _dev(tab), d_x)
    ap.oproj_grouped_wo_a_bf16(shp, d_x, None, _dev(wq.view(np.int16)), z)
    e2 = U.rel_max_err(U.bf16_bits_to_f64(_host(z).view(np.uint16)), ref)
    assert e2 <= TOL, e2


@pytest.mark.parametrize("T,G,hpg,R,gm", [(1, 2, 2, 64, False), (3, 1, 1, 128, True), (257, 3, 2, 192, False),
                                          (600, 2, 4, 320, True), (130, 4, 8, 64, False)])
def test_grouped_wo_a_bf16_ragged(T, G, hpg, R, gm):
    """Ragged token tails, one and several tiles, both layouts, dense check."""
    w = wl.Workload(60 + T, "g", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R, max_pos=4096,
                    positions="uniform")
    x = wl.normal_bf16(wl.seed_of(w.wid, 9), T * G * w.D).reshape(T, G, w.D)
    wq = wl.wo_a_bf16(w)
    ref = oracle.grouped_gemm_bf16(x, wq, G, R)
    e = U.rel_max_err(gpu_gemm_bf16(w, x, wq, group_major=gm), ref)
    assert e <= TOL, e


def test_grouped_wo_a_bf16_prefill_every_output():
    """Full prefill size (T=8192, G=16, D=4096, R=1024): every output, against
    the oracle's whole-tensor bf16 product taken one group at a time."""
    w = wl.WORKLOADS["prefill"]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    x = oracle.inv_rope_bf16(o, pos, tab).reshape(w.T, w.n_groups, w.D)
    wq = wl.wo_a_bf16(w)
    zg = gpu_gemm_bf16(w, x, wq)
    R = w.o_lora_rank
    worst = 0.0
    for g in range(w.n_groups):
        ref = oracle.dense_gemm_bf16_full(np.ascontiguousarray(x[:, g, :]), wq[g * R:(g + 1) * R])
        e = U.rel_max_err(zg[:, g, :], ref)
        worst = max(worst, e)
        assert e <= TOL, (g, e)
    print(f"every output of the prefill batch: worst group E = {worst:.2e}")


def test_grouped_wo_a_bf16_at_the_offset_limit():
    """The largest bf16 activation operand the grouped GEMM accepts: one group
    with D = 4096 and T = 2^19 tokens, 4 GiB exactly (operands are addressed
    as a base plus 32-bit lane offsets; one token more is refused).  Sampled
    outputs against the oracle on both sides of the 2^31-byte offset and at
    the end."""
    T, D, R = 1 << 19, 4096, 128
    w = wl.Workload(91, "limit", T=T, n_groups=1, heads_per_group=8, o_lora_rank=R, max_pos=1,
                    positions="uniform")
    x = wl.normal_bf16(wl.seed_of(91, 0), T * D)
    wq = wl.wo_a_bf16(w)
    d_x = _dev(x.view(np.int16))
    z = torch.empty((T, 1, R), dtype=torch.int16, device=DEV)
    ap.oproj_grouped_wo_a_bf16(_shape(w), d_x, None, _dev(wq.view(np.int16)), z)
    torch.cuda.synchronize()
    del d_x
    assert bool(torch.isfinite(z.view(torch.bfloat16)).all())
    idx = U.sample_triples(np.random.default_rng(12), T, 1, R, 2000)
    edge = np.array([1, (1 << 18) - 1, 1 << 18, (1 << 18) + 1, T - 256, T - 2], np.int64)
    idx[4:4 + edge.size, 0] = edge
    zs = z[torch.from_numpy(idx[:, 0]).to(DEV), 0, torch.from_numpy(idx[:, 2]).to(DEV)]
    got = U.bf16_bits_to_f64(_host(zs).view(np.uint16))
    ref = oracle.grouped_gemm_bf16(x.reshape(T, 1, D), wq, 1, R, idx=idx)
    e = U.rel_max_err(got, ref)
    assert e <= TOL, e


def test_dense_bf16_gemm_at_the_offset_limit():
    """wo_b's kernel at its largest activation operand: M = 2^17 rows of
    K = 16384 (4 GiB exactly), sampled against the oracle."""
    M, N, K = 1 << 17, 64, 16384
    x = wl.normal_bf16(wl.seed_of(92, 0), M * K)
    wb = wl.bf16_matrix(wl.seed_of(92, 1), N, K, 0.02)
    d_x = _dev(x.view(np.int16))
    y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    ap.oproj_dense_bf16_gemm(M, N, K, d_x, _dev(wb.view(np.int16)), y)
    torch.cuda.synchronize()
    del d_x
    assert bool(torch.isfinite(y.view(torch.bfloat16)).all())
    rng = np.random.default_rng(13)
    m = rng.integers(0, M, 2000)
    m[:6] = [0, (1 << 16) - 1, 1 << 16, (1 << 16) + 1, M - 2, M - 1]
    j = rng.integers(0, N, 2000)
    pairs = np.stack([m, j], axis=1).astype(np.int64)
    ys = y[torch.from_numpy(m).to(DEV), torch.from_numpy(j).to(DEV)]
    got = U.bf16_bits_to_f64(_host(ys).view(np.uint16))
    ref = oracle.dense_gemm_bf16(x.reshape(M, K), wb, idx=pairs)
    e = U.rel_max_err(got, ref)
    assert e <= TOL, e


def test_grouped_wo_a_bf16_group_isolation():
    w = wl.Workload(70, "iso", T=40, n_groups=3, heads_per_group=2, o_lora_rank=64, max_pos=4096,
                    positions="uniform")
    x = wl.normal_bf16(wl.seed_of(70, 9), w.T * 3 * w.D).reshape(w.T, 3, w.D)
    wq = wl.wo_a_bf16(w)
    z = gpu_gemm_bf16(w, x, wq)
    wq2 = wq.copy()
    wq2[64:128] = wl.f32_to_bf16_bits(np.full((64, w.D), 0.5, np.float32))
    z2 = gpu_gemm_bf16(w, x, wq2)
    assert np.array_equal(z2[:, [0, 2]], z[:, [0, 2]]) and not np.array_equal(z2[:, 1], z[:, 1])


@pytest.mark.parametrize("name,with_wo_b", [("decode", False), ("tiny", False), ("decode", True)])
def test_fused_bf16_equals_steps(name, with_wo_b):
    """oproj_fused_bf16 equals the separate calls bit for bit; with wo_b the
    result also meets the bar against the oracle chain."""
    w = wl.WORKLOADS[name]
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    wq = wl.wo_a_bf16(w)
    shp = _shape(w)
    hidden = 512 if with_wo_b else 0
    wob = wl.bf16_matrix(wl.seed_of(w.wid, 12), hidden, w.n_groups * w.o_lora_rank, 0.02) if with_wo_b else None
    d_o, d_pos, d_tab, d_w = _dev(o.view(np.int16)), _dev(pos), _dev(tab), _dev(wq.view(np.int16))
    d_wob = _dev(wob.view(np.int16)) if with_wo_b else None
    nbytes = ap.oproj_fused_bf16_workspace_bytes(shp, hidden)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.empty((w.T, hidden) if with_wo_b else (w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16,
                      device=DEV)
    ap.oproj_fused_bf16(shp, d_o, d_pos, d_tab, d_w, d_wob, hidden, ws, nbytes, out)
    x = torch.empty((w.T, w.n_groups, w.D), dtype=torch.int16, device=DEV)
    z = torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=DEV)
    ap.oproj_inv_rope_bf16(shp, d_o, d_pos, d_tab, x)
    ap.oproj_grouped_wo_a_bf16(shp, x, None, d_w, z)
    if not with_wo_b:
        assert torch.equal(out, z)
        return
    y = torch.empty_like(out)
    ap.oproj_dense_bf16_gemm(w.T, hidden, w.n_groups * w.o_lora_rank, z, d_wob, y)
    assert torch.equal(out, y)
    xr = oracle.inv_rope_bf16(o, pos, tab).reshape(w.T, w.n_groups, w.D)
    zr = oracle.f64_to_bf16(oracle.grouped_gemm_bf16(xr, wq, w.n_groups, w.o_lora_rank))
    yr = oracle.dense_gemm_bf16(zr.reshape(w.T, -1), wob)
    e = U.rel_max_err(U.bf16_bits_to_f64(_host(out).view(np.uint16)), yr)
    assert e <= TOL, e
