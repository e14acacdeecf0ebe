"""The single-launch decode layer (path "gemv_fused"): the same arithmetic as
the five-launch GEMV path, so its outputs, selection, permutation and h must
equal that path's bit for bit, every in-kernel wait must end normally (the
workspace's STATUS word is 0), and a captured HIP graph of it must replay
correctly (its flags are cleared within each call). It is also compared
with the oracle directly (test_gpu_parity.py's forward cases)."""
import pytest
import torch

import workloads as W
from parity import DevLayer, log

pytestmark = pytest.mark.gpu

C = W.CONFIGS

# (config, tokens, overrides)
CASES = [
    ("c1", 1, {}),
    ("c1", 2, {}),
    ("c1", 3, {}),
    ("c1", 4, {}),
    ("c1", 16, {}),
    ("c3", 1, {}),
    ("c3", 8, {}),
    ("c3", 16, {}),
    ("c0", 4, {}),                                    # fp32 activations
    ("c0", 16, {"experts": 512, "top_k": 16}),        # the most experts and choices
    ("c0", 9, {"experts": 100, "top_k": 3, "shared": True}),
    ("c0", 13, {"experts": 10, "top_k": 10}),         # every expert chosen, E not a multiple of 4
    ("c1", 7, {"bias": ("zipf", 1.1, 0.25)}),         # skewed routing
    ("c2", 16, {}),
]


def case_id(c):
    name, T, ov = c
    return f"{name}-T{T}" + ("-" + "-".join(sorted(ov)) if ov else "")


def run(layer, path, out_dtype=torch.float32, x=None):
    import block_fp8_routed_amd as moe
    s = layer.shape
    xx = layer.x if x is None else x
    cfg = moe.make_config(len(xx), s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                          xx.dtype, out_dtype, path)
    ws = moe.make_workspace(cfg, "cuda")
    out = moe.moe_forward(xx, layer.router_w, layer.bank, s.top_k, s.block, shared=layer.shared,
                          router_bias=layer.bias, out_dtype=out_dtype, path=path,
                          workspace=ws, cfg=cfg)
    torch.cuda.synchronize()
    return out, ws, cfg


def region(ws, cfg, r, dtype):
    import block_fp8_routed_amd as moe
    return moe.workspace_view(ws, cfg, r, dtype)


def status(ws, cfg):
    import block_fp8_routed_amd as moe
    return int(region(ws, cfg, moe.MOE_WS_STATUS, torch.int32).item())


@pytest.mark.parametrize("name,T,ov", CASES, ids=[case_id(c) for c in CASES])
def test_fused_equals_five_launch_path(name, T, ov):
    import block_fp8_routed_amd as moe
    shape = C[name].with_(**ov) if ov else C[name]
    layer = DevLayer(shape, tokens=T)
    log(f"fused vs gemv {case_id((name, T, ov))}")
    out_f, ws_f, cfg_f = run(layer, "gemv_fused")
    assert status(ws_f, cfg_f) == 0, "a wait of the single-launch layer gave up"
    out_g, ws_g, cfg_g = run(layer, "gemv")
    assert torch.equal(out_f, out_g)
    for r, dt in ((moe.MOE_WS_TOPK, torch.int32), (moe.MOE_WS_GATES, torch.int32),
                  (moe.MOE_WS_OFFSETS, torch.int32), (moe.MOE_WS_PAIR, torch.int32),
                  (moe.MOE_WS_INV, torch.int32), (moe.MOE_WS_H, torch.int32)):
        a, b = region(ws_f, cfg_f, r, dt), region(ws_g, cfg_g, r, dt)
        assert torch.equal(a, b), f"workspace region {r} differs"


@pytest.mark.parametrize("name,T", [("c1", 16), ("c3", 8)])
def test_fused_bf16_output(name, T):
    layer = DevLayer(C[name], tokens=T)
    out_f, ws, cfg = run(layer, "gemv_fused", out_dtype=torch.bfloat16)
    assert status(ws, cfg) == 0
    out_g, _, _ = run(layer, "gemv", out_dtype=torch.bfloat16)
    assert torch.equal(out_f, out_g)


def test_fused_back_to_back_calls_share_a_workspace():
    """Consecutive calls on one workspace (each with its own epoch, flags left
    cleared by the one before), different batches and token counts."""
    import block_fp8_routed_amd as moe
    shape = C["c1"]
    layer = DevLayer(shape, tokens=16)
    s = shape
    cfg16 = moe.make_config(16, s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                            layer.x.dtype, torch.float32, "gemv_fused")
    ws = moe.make_workspace(cfg16, "cuda")
    for b, T in enumerate([16, 16, 5, 1, 16, 9]):
        x = torch.from_numpy(W.gen_x(shape, 16, batch=b)[:T]).to(layer.x.dtype).cuda()
        cfg = moe.make_config(T, s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                              x.dtype, torch.float32, "gemv_fused")
        out = moe.moe_forward(x, layer.router_w, layer.bank, s.top_k, s.block, path="gemv_fused",
                              workspace=ws[:moe.workspace_bytes(cfg)], cfg=cfg)
        torch.cuda.synchronize()
        assert status(ws, cfg) == 0
        ref, _, _ = run(layer, "gemv", x=x)
        assert torch.equal(out, ref), f"call {b} (T={T})"


def test_fused_graph_replay():
    """A HIP graph holding the single-launch layer (one kernel, no memset
    nodes) replays with the epoch it was captured with; its flags are
    cleared inside every call, so each replay waits for that replay's own
    results. Replays with new inputs, eager work in between, each checked
    against the five-launch path."""
    import block_fp8_routed_amd as moe
    shape = C["c1"]
    layer = DevLayer(shape, tokens=16)
    s = shape
    cfg = moe.make_config(16, s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                          layer.x.dtype, torch.float32, "gemv_fused")
    ws = moe.make_workspace(cfg, "cuda")
    x_static = layer.x.clone()
    out_static = torch.empty((16, s.hidden), dtype=torch.float32, device="cuda")

    def call():
        moe.moe_forward(x_static, layer.router_w, layer.bank, s.top_k, s.block,
                        path="gemv_fused", out=out_static, workspace=ws, cfg=cfg)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for b in range(1, 5):
        x = torch.from_numpy(W.gen_x(shape, 16, batch=b)).to(layer.x.dtype).cuda()
        x_static.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        got = out_static.clone()
        assert status(ws, cfg) == 0, f"replay {b}"
        ref, _, _ = run(layer, "gemv", x=x)  # eager work between replays
        log(f"graph replay {b}: max |diff| {float((got - ref).abs().max()):.3g}")
        assert torch.equal(got, ref), f"replay {b}"
