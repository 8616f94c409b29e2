"""The one-launch decode entry point (quantisation, per-group barrier and
grouped GEMM in one kernel) against the two-launch oproj_fused, bit for bit,
and against the oracle chain: every scale recipe and weight-block mode,
ragged token counts, each supported head geometry, bad positions, calls
back to back with changing group sizes, calls overlapping on two streams with
their own workspaces, graph replays and the shapes it refuses."""
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


class _Case:
    """Inputs on the device, FP8 weights in the requested block mode, and a
    workspace for both entry points."""

    def __init__(self, seed, T, G, hpg, R, mode, wblock, max_pos=8192, bad_positions=False):
        self.w = wl.Workload(seed, "fdec", T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R,
                             max_pos=max_pos, positions="uniform")
        self.T, self.G, self.hpg, self.R, self.mode, self.wblock = T, G, hpg, R, mode, wblock
        self.o, self.pos, self.tab = wl.attn_out(self.w), wl.positions(self.w).copy(), wl.table(self.w)
        if bad_positions:
            self.pos[T // 2] = max_pos + 3
            self.pos[-1] = -1
        self.wmat = wl.wo_a_f32(self.w)
        rows, K = self.wmat.shape
        self.brows = 128 if wblock == ap.OPROJ_WBLOCK_128x128 else 1
        self.d_wq = torch.empty((rows, K), dtype=torch.uint8, device=DEV)
        if wblock == ap.OPROJ_WBLOCK_1x128_UE8M0:
            self.d_ws = torch.empty((rows, K // 512), dtype=torch.int32, device=DEV)
        else:
            self.d_ws = torch.empty(((rows + self.brows - 1) // self.brows, K // 128), dtype=torch.float32,
                                    device=DEV)
        ap.oproj_quantize_weight(rows, K, wblock, mode, _dev(self.wmat), self.d_wq, self.d_ws)
        self.shp = ap.Shape(T=T, n_groups=G, heads_per_group=hpg, o_lora_rank=R, max_pos=max_pos)
        self.nbytes = ap.oproj_fused_workspace_bytes(self.shp, 0)
        self.dbytes = ap.oproj_fused_decode_workspace_bytes(self.shp)
        self.d_o, self.d_pos, self.d_tab = _dev(self.o.view(np.int16)), _dev(self.pos), _dev(self.tab)

    def zbuf(self):
        return torch.full((self.T, self.G, self.R), 0x7BAD, dtype=torch.int16, device=DEV)

    def wsbuf(self):
        return torch.full((self.nbytes,), 0xA5, dtype=torch.uint8, device=DEV)

    def dwsbuf(self):
        """A one-launch workspace: garbage where the codes and scales go, the
        barrier words zeroed (as a caller does once per workspace)."""
        ws = torch.full((self.dbytes,), 0xA5, dtype=torch.uint8, device=DEV)
        ws[self.nbytes:].zero_()
        return ws

    def require_one_launch(self):
        why = ap.oproj_fused_decode_unsupported(self.shp, self.mode, self.wblock)
        if why is not None:  # e.g. a partitioned device with fewer compute units
            pytest.skip(f"one-launch path unavailable here: {why}")

    def one_launch(self, ws, z):
        ap.oproj_fused_decode(self.shp, self.mode, self.d_o, self.d_pos, self.d_tab, self.d_wq, self.d_ws,
                              self.wblock, ws, self.dbytes, z)

    def two_launch(self, ws, z):
        ap.oproj_fused(self.shp, self.mode, self.d_o, self.d_pos, self.d_tab, self.d_wq, self.d_ws,
                       self.wblock, None, 0, ws, self.nbytes, z)

    def oracle_z(self):
        pow2 = self.mode != 0
        qa, sa = oracle.inv_rope_quant(self.o, self.pos, self.tab, self.G, self.hpg, pow2=pow2)
        qw, sw = oracle.quant_weight(self.wmat, self.brows, pow2)
        return oracle.grouped_gemm(qa, sa, qw, sw, self.G, self.R, self.brows)


def _z64(z):
    torch.cuda.synchronize()
    return U.bf16_bits_to_f64(z.cpu().numpy().view(np.uint16))


F32, P2, E8 = ap.OPROJ_SCALE_FP32, ap.OPROJ_SCALE_POW2, ap.OPROJ_SCALE_E8M0
B128, B1, BU = ap.OPROJ_WBLOCK_128x128, ap.OPROJ_WBLOCK_1x128, ap.OPROJ_WBLOCK_1x128_UE8M0

CASES = [
    # T, G, hpg, R, mode, wblock
    (64, 16, 8, 1024, F32, B128),  # the decode batch of the DeepSeek-V4 O-projection
    (64, 16, 8, 1024, P2, B1),
    (64, 16, 8, 1024, E8, BU),
    (1, 16, 8, 1024, F32, B128),
    (17, 4, 8, 192, P2, B128),
    (33, 3, 16, 256, E8, B1),
    (5, 8, 4, 320, F32, B1),
    (64, 2, 2, 64, P2, BU),
    (63, 5, 2, 128, E8, B128),
    (64, 256, 2, 64, F32, B128),  # the most groups the one-launch path takes, one workgroup per CU
]


@pytest.mark.parametrize("T,G,hpg,R,mode,wblock", CASES)
def test_one_launch_equals_two_launches_and_oracle(T, G, hpg, R, mode, wblock):
    c = _Case(400 + T + 7 * G + hpg, T, G, hpg, R, mode, wblock)
    c.require_one_launch()
    ws1, z1 = c.dwsbuf(), c.zbuf()
    c.one_launch(ws1, z1)
    ws2, z2 = c.wsbuf(), c.zbuf()
    c.two_launch(ws2, z2)
    torch.cuda.synchronize()
    assert torch.equal(z1, z2)
    # the workspace regions the quantisation writes hold the same codes and scales
    ncode = T * G * hpg * 512
    nscale = T * G * hpg * (1 if mode == E8 else 4) * 4
    soff = (ncode + 255) // 256 * 256
    assert torch.equal(ws1[:ncode], ws2[:ncode])
    assert torch.equal(ws1[soff:soff + nscale], ws2[soff:soff + nscale])
    e = U.rel_max_err(_z64(z1), c.oracle_z())
    assert e <= TOL, e


def test_one_launch_bad_positions():
    """Positions outside the table give NaN scales: same bits as oproj_fused."""
    c = _Case(431, 24, 4, 8, 256, F32, B128, bad_positions=True)
    c.require_one_launch()
    z1, z2 = c.zbuf(), c.zbuf()
    c.one_launch(c.dwsbuf(), z1)
    c.two_launch(c.wsbuf(), z2)
    torch.cuda.synchronize()
    assert torch.equal(z1, z2)
    zz = _z64(z1)
    assert np.isnan(zz[c.T // 2]).all() and np.isnan(zz[-1]).all()
    assert not np.isnan(zz[0]).any()


def test_one_launch_back_to_back_changing_group_sizes():
    """Forty calls in a row on one stream, alternating shapes whose groups have
    16, 4 and 1 workgroups: the barrier words carry over from call to call."""
    cases = [_Case(440, 64, 16, 8, 1024, F32, B128), _Case(441, 9, 6, 4, 256, P2, B1),
             _Case(442, 40, 3, 2, 64, E8, BU)]
    for c in cases:
        c.require_one_launch()
    refs = []
    for c in cases:
        z = c.zbuf()
        c.two_launch(c.wsbuf(), z)
        refs.append(z)
    outs = [[c.zbuf() for _ in range(14)] for c in cases]
    wss = [c.dwsbuf() for c in cases]
    for i in range(14):
        for k, c in enumerate(cases):
            if k == 2 and i == 13:
                continue
            c.one_launch(wss[k], outs[k][i])
    torch.cuda.synchronize()
    for k in range(3):
        for i in range(14 if k < 2 else 13):
            assert torch.equal(outs[k][i], refs[k]), (k, i)


@pytest.mark.parametrize("spin", ["0", "1"])
def test_one_launch_fallback_path(spin, monkeypatch):
    """With the barrier's poll limit forced down from the host, every workgroup
    but a group's last arrival gives up waiting and quantises its whole group
    itself: the result is still bit-identical to the two-launch path."""
    c = _Case(445, 64, 16, 8, 1024, P2, B1)
    c.require_one_launch()
    ref = c.zbuf()
    c.two_launch(c.wsbuf(), ref)
    monkeypatch.setenv("OPROJ_FUSED_DECODE_SPIN_LIMIT", spin)
    outs = [c.zbuf() for _ in range(3)]
    ws = c.dwsbuf()
    for z in outs:
        c.one_launch(ws, z)
    monkeypatch.delenv("OPROJ_FUSED_DECODE_SPIN_LIMIT")
    z_after = c.zbuf()
    c.one_launch(ws, z_after)  # and the barrier words are left in order for normal calls
    torch.cuda.synchronize()
    for z in outs + [z_after]:
        assert torch.equal(z, ref)


def test_one_launch_graph_replays():
    """Captured in a HIP graph: every replay, with eager calls of the same
    entry point and new inputs between replays, equals the eager result."""
    c = _Case(450, 64, 16, 8, 1024, F32, B128)
    c.require_one_launch()
    ws, z = c.dwsbuf(), c.zbuf()
    c.one_launch(ws, z)
    torch.cuda.synchronize()
    ref0 = z.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c.one_launch(ws, z)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        c.one_launch(ws, z)
    torch.cuda.synchronize()
    o2 = wl.attn_out(wl.Workload(451, "fdec2", T=64, n_groups=16, heads_per_group=8, o_lora_rank=1024,
                                 max_pos=8192, positions="uniform"))
    alt = _dev(o2.view(np.int16))
    keep = c.d_o.clone()
    z_alt = c.zbuf()
    ap.oproj_fused(c.shp, c.mode, alt, c.d_pos, c.d_tab, c.d_wq, c.d_ws, c.wblock, None, 0, c.wsbuf(),
                   c.nbytes, z_alt)
    torch.cuda.synchronize()
    for r in range(5):
        c.d_o.copy_(alt if r % 2 else keep)
        z.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(z, z_alt if r % 2 else ref0), r
        c.one_launch(c.dwsbuf(), c.zbuf())  # eager work between replays
        torch.cuda.synchronize()


def test_eligibility_query_agrees_with_the_entry_point():
    """None for the decode batch; the compute-unit reason for a grid wider
    than the device, which the entry point refuses."""
    dec = ap.Shape(T=64, n_groups=16, heads_per_group=8, o_lora_rank=1024, max_pos=32768)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus >= 16 * 16:
        assert ap.oproj_fused_decode_unsupported(dec) is None
    else:
        assert "compute units" in ap.oproj_fused_decode_unsupported(dec)
    wide = ap.Shape(T=8, n_groups=cus // 16 + 1, heads_per_group=8, o_lora_rank=1024, max_pos=8192)
    assert "compute units" in ap.oproj_fused_decode_unsupported(wide)


def test_one_launch_refuses_shapes_that_do_not_fit():
    """More tokens than one tile, or more workgroups than compute units: an
    error, and the output is left untouched."""
    c = _Case(460, 8, 2, 8, 128, F32, B128)
    z = c.zbuf()
    big = ap.Shape(T=65, n_groups=2, heads_per_group=8, o_lora_rank=128, max_pos=8192)
    with pytest.raises(ap.OprojError) as ei:
        ap.oproj_fused_decode(big, F32, c.d_o, c.d_pos, c.d_tab, c.d_wq, c.d_ws, B128, c.dwsbuf(),
                              ap.oproj_fused_decode_workspace_bytes(big), z)
    assert ei.value.status == 2
    # buffers sized for the wide shape, so that nothing would be out of bounds
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    G, R, D = cus // 16 + 1, 1024, 8 * 512  # 16 workgroups per group
    wide = ap.Shape(T=8, n_groups=G, heads_per_group=8, o_lora_rank=R, max_pos=8192)
    nb = ap.oproj_fused_decode_workspace_bytes(wide)
    o = torch.zeros((8, G * 8, 512), dtype=torch.int16, device=DEV)
    wq = torch.zeros((G * R, D), dtype=torch.uint8, device=DEV)
    wsc = torch.ones((G * R // 128, D // 128), dtype=torch.float32, device=DEV)
    zw = torch.full((8, G, R), 0x7BAD, dtype=torch.int16, device=DEV)
    with pytest.raises(ap.OprojError) as ei:
        ap.oproj_fused_decode(wide, F32, o, c.d_pos, c.d_tab, wq, wsc, B128,
                              torch.zeros(nb, dtype=torch.uint8, device=DEV), nb, zw)
    assert ei.value.status == 2
    torch.cuda.synchronize()
    assert bool((z == 0x7BAD).all()) and bool((zw == 0x7BAD).all())


def test_two_launch_path_is_safe_on_concurrent_streams():
    """oproj_fused keeps no state between calls: calls on two streams at once,
    each with its own workspace, give the single-stream results."""
    cases = [_Case(470, 64, 16, 8, 1024, F32, B128), _Case(471, 48, 16, 8, 1024, P2, B1)]
    refs = []
    for c in cases:
        z = c.zbuf()
        c.two_launch(c.wsbuf(), z)
        refs.append(z)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[c.zbuf() for _ in range(8)] for c in cases]
    wss = [c.wsbuf() for c in cases]
    torch.cuda.synchronize()
    for i in range(8):
        for k, c in enumerate(cases):
            with torch.cuda.stream(streams[k]):
                ap.oproj_fused(c.shp, c.mode, c.d_o, c.d_pos, c.d_tab, c.d_wq, c.d_ws, c.wblock, None, 0,
                               wss[k], c.nbytes, outs[k][i], stream=streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        for i in range(8):
            assert torch.equal(outs[k][i], refs[k]), (k, i)


def test_one_launch_calls_overlapping_on_two_streams():
    """Two one-launch calls at a time, on two streams, each with its own
    workspace (and so its own barrier words): every result equals the
    single-stream two-launch result, call after call."""
    cases = [_Case(480, 64, 8, 8, 1024, F32, B128), _Case(481, 48, 4, 8, 1024, P2, B1)]  # 128 + 64 workgroups
    for c in cases:
        c.require_one_launch()
    if sum(c.G * ((c.R + 63) // 64) for c in cases) > torch.cuda.get_device_properties(0).multi_processor_count:
        pytest.skip("the two grids do not fit on the device together")
    refs = []
    for c in cases:
        z = c.zbuf()
        c.two_launch(c.wsbuf(), z)
        refs.append(z)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[c.zbuf() for _ in range(12)] for c in cases]
    wss = [c.dwsbuf() for c in cases]
    torch.cuda.synchronize()
    for i in range(12):
        for k, c in enumerate(cases):
            with torch.cuda.stream(streams[k]):
                ap.oproj_fused_decode(c.shp, c.mode, c.d_o, c.d_pos, c.d_tab, c.d_wq, c.d_ws, c.wblock, wss[k],
                                      c.dbytes, outs[k][i], stream=streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        for i in range(12):
            assert torch.equal(outs[k][i], refs[k]), (k, i)
