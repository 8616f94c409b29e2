"""oproj_fused_noalloc: the whole path with the library's own scratch array as
its workspace (no allocation), through the C ABI, against oproj_fused with a
caller-allocated workspace: the same kernels, so z and y must be identical bit
for bit.  Two calls in a row, the second with a smaller input (and wo_b), so
the second reuses the array the first left behind."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_output_projection_amd as ap
import workloads as wl

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


def _case(w: wl.Workload, hidden: int):
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    wmat = wl.wo_a_f32(w)
    rows = w.n_groups * w.o_lora_rank
    wq = torch.empty((rows, w.D), dtype=torch.uint8, device=DEV)
    ws = torch.empty(((rows + 127) // 128, w.KB), dtype=torch.float32, device=DEV)
    ap.oproj_quantize_weight(rows, w.D, ap.OPROJ_WBLOCK_128x128, ap.OPROJ_SCALE_FP32, _dev(wmat), wq, ws)
    wob = _dev(wl.bf16_matrix(wl.seed_of(96, hidden), hidden, rows, 0.02).view(np.int16)) if hidden else None
    shp = ap.Shape(T=w.T, n_groups=w.n_groups, heads_per_group=w.heads_per_group, o_lora_rank=w.o_lora_rank,
                   max_pos=w.max_pos)
    args = (shp, ap.OPROJ_SCALE_FP32, _dev(o.view(np.int16)), _dev(pos), _dev(tab), wq, ws,
            ap.OPROJ_WBLOCK_128x128, wob, hidden)
    shape_out = (w.T, hidden) if hidden else (w.T, w.n_groups, w.o_lora_rank)
    return args, shape_out


def _both(args, shape_out):
    nb = ap.oproj_fused_workspace_bytes(args[0], args[-1])
    assert 0 < nb <= ap.OPROJ_NOALLOC_SCRATCH_BYTES
    ref = torch.empty(shape_out, dtype=torch.int16, device=DEV)
    ap.oproj_fused(*args, torch.empty(nb, dtype=torch.uint8, device=DEV), nb, ref)
    got = torch.full(shape_out, 0x7BAD, dtype=torch.int16, device=DEV)
    ap.oproj_fused_noalloc(*args, got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_fused_on_two_calls_second_smaller():
    big, out_big = _case(wl.WORKLOADS["decode"], 0)  # T=64, 16 groups x 8 heads: z
    small, out_small = _case(wl.Workload(97, "small", T=17, n_groups=4, heads_per_group=4, o_lora_rank=256,
                                         max_pos=4096, positions="uniform"), 512)  # y through wo_b
    assert ap.oproj_fused_workspace_bytes(small[0], 512) < ap.oproj_fused_workspace_bytes(big[0], 0)
    for args, shape_out in ((big, out_big), (small, out_small)):
        ref, got = _both(args, shape_out)
        assert torch.equal(got, ref)
        assert not bool((got == 0x7BAD).all())


def test_noalloc_refuses_more_than_its_scratch():
    w = wl.WORKLOADS["decode"].scaled(1024)  # 64 MiB of codes: more than the array holds
    args, shape_out = _case(w, 0)
    assert ap.oproj_fused_workspace_bytes(args[0], 0) > ap.OPROJ_NOALLOC_SCRATCH_BYTES
    z = torch.full(shape_out, 0x7BAD, dtype=torch.int16, device=DEV)
    with pytest.raises(ap.OprojError) as e:
        ap.oproj_fused_noalloc(*args, z)
    assert e.value.status == 6 and "scratch" in ap.oproj_status_string(6)
    torch.cuda.synchronize()
    assert bool((z == 0x7BAD).all())  # nothing was enqueued


def test_noalloc_t0_and_invalid_shape():
    ap.oproj_fused_noalloc(ap.Shape(T=0, n_groups=2, heads_per_group=2, o_lora_rank=64, max_pos=16),
                           0, None, None, None, None, None, 0, None, 0, None)
    with pytest.raises(ap.OprojError) as e:
        ap.oproj_fused_noalloc(ap.Shape(T=4, n_groups=2, heads_per_group=2, o_lora_rank=10, max_pos=16),
                               0, None, None, None, None, None, 0, None, 0, None)
    assert e.value.status == 2


def test_noalloc_replays_under_graph_capture():
    """The callers it is for: a HIP graph holding the call (captured after one
    eager call, which looks the array up), replayed four times with eager work
    between the replays, among it a call on another input that overwrites the
    array; every replay equals the eager result bit for bit."""
    args, shape_out = _case(wl.WORKLOADS["decode"], 0)
    other, other_out = _case(wl.Workload(98, "other", T=9, n_groups=2, heads_per_group=8, o_lora_rank=128,
                                         max_pos=4096, positions="uniform"), 0)
    ref = torch.empty(shape_out, dtype=torch.int16, device=DEV)
    ap.oproj_fused_noalloc(*args, ref)
    torch.cuda.synchronize()
    out = torch.full(shape_out, 0x7BAD, dtype=torch.int16, device=DEV)
    junk = torch.empty(other_out, dtype=torch.int16, device=DEV)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ap.oproj_fused_noalloc(*args, out)
    torch.cuda.synchronize()
    try:
        for rep in range(4):
            out.fill_(0x7BAD)                      # a fill kernel, eager
            ap.oproj_fused_noalloc(*other, junk)   # the array now holds another call's data
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"replay {rep} differs"
    finally:
        torch.cuda.synchronize()
        g.reset()
