"""Shared test helpers: parity metrics and layout conversions (no method arithmetic)."""
from __future__ import annotations

import numpy as np

import oracle


def rel_max_err(y: np.ndarray, r: np.ndarray) -> float:
    """E = max|y - r| / max|r| over one output tensor (the parity gate)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    denom = np.abs(r).max()
    return float(np.abs(y - r).max() / denom) if denom > 0 else float(np.abs(y - r).max())


def elem_rel_err(y: np.ndarray, r: np.ndarray) -> float:
    """Reported only: max |y-r| / (|r| + 1e-3 rms(r))."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    return float((np.abs(y - r) / (np.abs(r) + 1e-3 * rms + 1e-300)).max()) if r.size else 0.0


def compare_codes(gpu: np.ndarray, ref: np.ndarray):
    """FP8 code parity: returns (n_mismatch, n_total, all_within_one_step).

    Codes compare by value (+0 == -0); a mismatch is allowed only between
    adjacent representable magnitudes of the same sign."""
    gpu = np.ascontiguousarray(gpu, np.uint8).ravel()
    ref = np.ascontiguousarray(ref, np.uint8).ravel()
    diff = np.flatnonzero(gpu != ref)
    if diff.size == 0:
        return 0, gpu.size, True
    vg = oracle.e4m3_decode(gpu[diff])
    vr = oracle.e4m3_decode(ref[diff])
    same = (vg == vr) | (np.isnan(vg) & np.isnan(vr))
    bad = diff[~same]
    if bad.size == 0:
        return 0, gpu.size, True
    g, r = gpu[bad].astype(np.int32), ref[bad].astype(np.int32)
    mag_g, mag_r = g & 0x7F, r & 0x7F
    zero_g, zero_r = mag_g == 0, mag_r == 0
    sign_ok = ((g & 0x80) == (r & 0x80)) | zero_g | zero_r
    adjacent = (np.abs(mag_g - mag_r) == 1) & sign_ok
    return int(bad.size), int(gpu.size), bool(adjacent.all())


def assert_codes_parity(gpu, ref, frac: float = 1e-4):
    n_bad, n, adj = compare_codes(gpu, ref)
    assert adj, f"{n_bad} mismatching codes, some more than one step apart"
    assert n_bad <= frac * n, f"{n_bad}/{n} codes differ (> {frac})"
    return n_bad


def assert_scales_bitexact(gpu, ref):
    g = np.ascontiguousarray(gpu, np.float32)
    r = np.ascontiguousarray(ref, np.float32)
    assert g.shape == r.shape
    bad = g.view(np.uint32) != r.view(np.uint32)
    assert not bad.any(), f"{int(bad.sum())} scales differ, e.g. gpu={g[bad][:4]} ref={r[bad][:4]}"


def group_major_to_token_major(codes_gtd: np.ndarray, scales_gkt: np.ndarray):
    """[G][T][D] codes, [G][KB][T] scales -> [T][G][D], [T][G][KB]."""
    return (np.ascontiguousarray(np.transpose(codes_gtd, (1, 0, 2))),
            np.ascontiguousarray(np.transpose(scales_gkt, (2, 0, 1))))


def token_major_to_group_major(codes_tgd: np.ndarray, scales_tgk: np.ndarray):
    return (np.ascontiguousarray(np.transpose(codes_tgd, (1, 0, 2))),
            np.ascontiguousarray(np.transpose(scales_tgk, (1, 2, 0))))


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def sample_triples(rng: np.random.Generator, T: int, G: int, R: int, n: int) -> np.ndarray:
    """n (t, g, n) triples covering the first and last tokens and columns."""
    t = rng.integers(0, T, n)
    g = rng.integers(0, G, n)
    c = rng.integers(0, R, n)
    t[:4] = [0, T - 1, 0, T - 1]
    c[:4] = [0, R - 1, R - 1, 0]
    return np.stack([t, g, c], axis=1).astype(np.int64)


def stratified_triples(rng: np.random.Generator, T: int, G: int, R: int, bm: int = 128, bn: int = 64,
                       extra: int = 0) -> np.ndarray:
    """(t, g, n) triples with one random element in every bm x bn block of
    every group's [T, R] output (so every tile and every wave sub-tile of the
    GEMM kernels is sampled), the last row and last column of each group, and
    `extra` uniform draws."""
    out = []
    for g in range(G):
        for m0 in range(0, T, bm):
            for n0 in range(0, R, bn):
                t = m0 + int(rng.integers(0, min(bm, T - m0)))
                n = n0 + int(rng.integers(0, min(bn, R - n0)))
                out.append((t, g, n))
        out += [(T - 1, g, int(rng.integers(0, R))), (int(rng.integers(0, T)), g, R - 1),
                (T - 1, g, R - 1), (0, g, 0)]
    idx = np.array(out, np.int64)
    if extra:
        idx = np.concatenate([idx, sample_triples(rng, T, G, R, extra)])
    return idx


GUARD_BYTES = 4096
GUARD_FILL = 0xA5


def guarded_empty(shape, dtype, device):
    """A tensor of `shape` followed by GUARD_BYTES guard bytes in one
    allocation, every byte set to GUARD_FILL; returns (view, whole).  The
    kernels get the view; guard_intact(whole, view) checks that nothing was
    written past its end."""
    import torch

    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    whole = torch.full((nbytes + GUARD_BYTES,), GUARD_FILL, dtype=torch.uint8, device=device)
    return whole[:nbytes].view(dtype).view(*shape), whole


def guard_intact(whole, view) -> bool:
    nbytes = view.numel() * view.element_size()
    return bool((whole[nbytes:] == GUARD_FILL).all().item())
