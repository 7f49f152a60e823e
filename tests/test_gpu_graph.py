"""The entry points launch only kernels on the caller's stream (no
allocation, no memset, no synchronisation), so they can be captured in a
HIP graph.  Each captured graph is replayed several times with eager work and
synchronisations in between, and every replay is checked against the eager
result."""
import numpy as np
import pytest

import synth
from synth.configs import DecodeConfig, ScanConfig
from tests.helpers import to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import selective_state_space_28_amd as ssm
    ssm.load()
    return torch.device("cuda:0")


@pytest.mark.parametrize("segs", ["1", "3"])
def test_scan_graph_replays(dev, segs, monkeypatch):
    import torch
    import selective_state_space_28_amd as ssm
    monkeypatch.setenv("SSM_SCAN_SEGMENTS", segs)
    inp = synth.make_scan_inputs(ScanConfig("g", 2, 96, 16, 300, "bf16", seed=31))
    t = {k: to_torch(inp[k], "bf16", dev) for k in ("u", "delta", "B", "C", "z")}
    A, D, bias = (to_torch(inp[k], "f32", dev) for k in ("A", "D", "delta_bias"))
    need = ssm.ssm_scan_fwd_workspace_bytes(2, 96, 16, 300, torch.bfloat16)
    ref = ssm.ssm_scan_fwd(t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias)
    torch.cuda.synchronize()
    y = torch.empty_like(t["u"])
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the default stream, as capture expects
        ssm.ssm_scan_fwd(t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ssm.ssm_scan_fwd(t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias, out=y, workspace=ws)
    other = synth.make_scan_inputs(ScanConfig("g2", 1, 64, 16, 100, "bf16", seed=32))
    o = {k: to_torch(other[k], "bf16", dev) for k in ("u", "delta", "B", "C", "z")}
    oA = to_torch(other["A"], "f32", dev)
    for i in range(4):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        # eager work between replays, on a workspace of its own
        ssm.ssm_scan_fwd(o["u"], o["delta"], oA, o["B"], o["C"], None, o["z"], None)
        torch.cuda.synchronize()


def test_decode_graph_replays(dev):
    import torch
    import selective_state_space_28_amd as ssm
    cfg = DecodeConfig("g", 4, 256, 16, 4, "bf16", seed=33)
    p = synth.make_decode_params(cfg)
    A, D, bias = (to_torch(p[k], "f32", dev) for k in ("A", "D", "delta_bias"))
    toks = [{k: to_torch(synth.make_decode_step(cfg, s)[k], "bf16", dev)
             for k in ("u", "delta", "B", "C", "z")} for s in range(cfg.steps)]
    h0 = to_torch(p["h0"], "f32", dev)
    st = h0.clone()
    ys_ref = [ssm.ssm_state_update(st, t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias)
              for t in toks]
    torch.cuda.synchronize()
    st_ref = st.clone()
    state = h0.clone()
    ys = [torch.empty_like(toks[0]["u"]) for _ in toks]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for t, yy in zip(toks, ys):
            ssm.ssm_state_update(state, t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias, out=yy)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        for t, yy in zip(toks, ys):
            ssm.ssm_state_update(state, t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias, out=yy)
    for i in range(3):
        state.copy_(h0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(cfg.steps):
            assert torch.equal(ys[s].view(torch.int16), ys_ref[s].view(torch.int16)), (i, s)
        assert torch.equal(state, st_ref), f"replay {i}"


def test_ssd_graph_replays(dev):
    """The SSD scan (prep kernel + chunked scan) captured and replayed."""
    import torch
    import selective_state_space_28_amd as ssm
    from synth.configs import SsdConfig
    inp = synth.make_ssd_inputs(SsdConfig("g", 2, 3, 64, 64, 300, "bf16", seed=34))
    t = {k: to_torch(inp[k], "bf16", dev) for k in ("x", "dt", "B", "C", "z")}
    A, D, bias = (to_torch(inp[k], "f32", dev) for k in ("A", "D", "dt_bias"))
    ref = ssm.ssm_ssd_scan_fwd(t["x"], t["dt"], A, t["B"], t["C"], D, t["z"], bias)
    torch.cuda.synchronize()
    y = torch.empty_like(t["x"])
    ws = torch.empty(ssm.ssm_ssd_scan_fwd_workspace_bytes(2, 64, 300, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    run = lambda: ssm.ssm_ssd_scan_fwd(t["x"], t["dt"], A, t["B"], t["C"], D, t["z"], bias, out=y, workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(4):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        ssm.ssm_ssd_scan_fwd(t["x"][:1].contiguous(), t["dt"][:1].contiguous(), A, t["B"][:1].contiguous(),
                             t["C"][:1].contiguous(), None, None, None)  # eager work in between
        torch.cuda.synchronize()


@pytest.mark.parametrize("bbar", ["euler", "zoh"])
def test_bwd_graph_replays(dev, bbar):
    """The backward (checkpoint pass, sweep, sums) captured and replayed; its
    outputs are bit-deterministic, so every replay must equal the eager call."""
    import torch
    import selective_state_space_28_amd as ssm
    inp = synth.make_scan_inputs(ScanConfig("g", 2, 96, 16, 300, "bf16", seed=35))
    t = {k: to_torch(inp[k], "bf16", dev) for k in ("u", "delta", "B", "C", "z")}
    A, D, bias = (to_torch(inp[k], "f32", dev) for k in ("A", "D", "delta_bias"))
    dy = torch.randn(t["u"].shape, generator=torch.Generator(device=dev).manual_seed(6), device=dev).to(torch.bfloat16)
    ws = torch.empty(ssm.ssm_scan_bwd_workspace_bytes(2, 96, 16, 300, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    run = lambda: ssm.ssm_scan_bwd(t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias, dy=dy, bbar=bbar,
                                   workspace=ws)
    ref = {k: (None if v is None else v.clone()) for k, v in run().items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = run()
    for i in range(3):
        for v in out.values():
            if v is not None:
                v.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            if v is not None:
                assert torch.equal(v, ref[k]), (i, k)
        ssm.ssm_scan_fwd(t["u"], t["delta"], A, t["B"], t["C"], None, None, None)  # eager work in between
        torch.cuda.synchronize()


def test_training_pair_graph_replays(dev):
    """ssm_scan_fwd_ckpt then ssm_scan_bwd_ckpt captured together (a training
    step): every replay rewrites y, last_state, the checkpoints and every
    gradient with the eager bits."""
    import torch
    import selective_state_space_28_amd as ssm
    b, d, n, L = 2, 96, 16, 300
    inp = synth.make_scan_inputs(ScanConfig("g", b, d, n, L, "bf16", seed=34))
    t = {k: to_torch(inp[k], "bf16", dev) for k in ("u", "delta", "B", "C", "z")}
    A, D, bias = (to_torch(inp[k], "f32", dev) for k in ("A", "D", "delta_bias"))
    dy = to_torch(synth.bf16_bits(np.random.default_rng(35).standard_normal((b, d, L), dtype=np.float32)),
                  "bf16", dev)
    args = (t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias)
    y_ref, last_ref, ck_ref = ssm.ssm_scan_fwd_ckpt(*args)
    g_ref = ssm.ssm_scan_bwd_ckpt(*args, ckpt=ck_ref, dy=dy)
    torch.cuda.synchronize()
    y, ck = torch.empty_like(y_ref), torch.empty_like(ck_ref)
    ws = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_bytes(b, d, n, L, torch.bfloat16)), dtype=torch.uint8,
                     device=dev)
    bws = torch.empty(max(1, ssm.ssm_scan_bwd_ckpt_workspace_bytes(b, d, n, L, torch.bfloat16)),
                      dtype=torch.uint8, device=dev)

    def step():
        _, last, _ = ssm.ssm_scan_fwd_ckpt(*args, out=y, ckpt=ck, workspace=ws)
        return last, ssm.ssm_scan_bwd_ckpt(*args, ckpt=ck, dy=dy, workspace=bws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the default stream, as capture expects
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        last, grads = step()

    def bits(x):
        return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)

    for i in range(4):
        for x in [y, ck, last] + [v for v in grads.values() if v is not None]:
            x.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y_ref)), f"replay {i}: y"
        assert torch.equal(bits(ck), bits(ck_ref)), f"replay {i}: checkpoints"
        assert torch.equal(bits(last), bits(last_ref)), f"replay {i}: last_state"
        for k, v in grads.items():
            if v is not None:
                assert torch.equal(bits(v), bits(g_ref[k])), f"replay {i}: {k}"
        # eager work between replays, with buffers of its own
        ssm.ssm_scan_bwd(*args, dy=dy)
        torch.cuda.synchronize()
