"""Randomised parity sweep over small shapes and every mode combination: the
fused entry points (FP8 and unquantised) on seeded shapes with ragged token
counts, against the oracle chain, in one process."""
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


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _cases(n: int, seed: int):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([1, 2, 7, 31, 64, 65, 100, 129, 200, 257, 300]))
        G = int(rng.integers(1, 5))
        hpg = int(rng.choice([1, 2, 4, 8]))
        R = int(rng.choice([64, 128, 192, 256, 320]))
        mode = int(rng.integers(0, 3))  # FP32, POW2, E8M0 activation scales
        wblock = int(rng.integers(0, 3)) if mode else int(rng.integers(0, 2))
        if wblock == 2 and (hpg * 512) % 512:
            wblock = 1
        out.append((i, T, G, hpg, R, mode, wblock))
    return out


@pytest.mark.parametrize("i,T,G,hpg,R,mode,wblock", _cases(24, 2024))
def test_fused_fp8_sweep(i, T, G, hpg, R, mode, wblock):
    w = wl.Workload(200 + i, "sweep", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R, max_pos=8192,
                    positions="uniform")
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    wmat = wl.wo_a_f32(w)
    brows = 128 if wblock == 0 else 1
    pow2 = mode != 0
    rows, K = wmat.shape
    d_wq = torch.empty((rows, K), dtype=torch.uint8, device=DEV)
    if wblock == 2:
        d_ws = torch.empty((rows, K // 512), dtype=torch.int32, device=DEV)
    else:
        d_ws = torch.empty(((rows + brows - 1) // brows, K // 128), dtype=torch.float32, device=DEV)
    ap.oproj_quantize_weight(rows, K, wblock, mode, _dev(wmat), d_wq, d_ws)
    shp = ap.Shape(T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R, max_pos=w.max_pos)
    nbytes = ap.oproj_fused_workspace_bytes(shp, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    z = torch.empty((T, G, R), dtype=torch.int16, device=DEV)
    ap.oproj_fused(shp, mode, _dev(o.view(np.int16)), _dev(pos), _dev(tab), d_wq, d_ws, wblock, None, 0, ws,
                   nbytes, z)
    qa, sa = oracle.inv_rope_quant(o, pos, tab, G, hpg, pow2=pow2)
    qw, sw = oracle.quant_weight(wmat, brows, pow2)
    ref = oracle.grouped_gemm(qa, sa, qw, sw, G, R, brows)
    torch.cuda.synchronize()
    e = U.rel_max_err(U.bf16_bits_to_f64(z.cpu().numpy().view(np.uint16)), ref)
    assert e <= TOL, e


@pytest.mark.parametrize("i,T,G,hpg,R,mode,wblock", _cases(12, 2025))
def test_fused_bf16_sweep(i, T, G, hpg, R, mode, wblock):
    w = wl.Workload(300 + i, "sweep", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R, max_pos=8192,
                    positions="uniform")
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    wq = wl.wo_a_bf16(w)
    shp = ap.Shape(T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R, max_pos=w.max_pos)
    nbytes = ap.oproj_fused_bf16_workspace_bytes(shp, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    z = torch.empty((T, G, R), dtype=torch.int16, device=DEV)
    ap.oproj_fused_bf16(shp, _dev(o.view(np.int16)), _dev(pos), _dev(tab), _dev(wq.view(np.int16)), None, 0,
                        ws, nbytes, z)
    x = oracle.inv_rope_bf16(o, pos, tab).reshape(T, G, w.D)
    ref = oracle.grouped_gemm_bf16(x, wq, G, R)
    torch.cuda.synchronize()
    e = U.rel_max_err(U.bf16_bits_to_f64(z.cpu().numpy().view(np.uint16)), ref)
    assert e <= TOL, e
