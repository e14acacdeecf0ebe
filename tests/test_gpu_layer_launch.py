"""The grouped paths (bf16, and the FP8 variant) run their gate/up and down
passes as one launch: the down workgroups wait on per-tile counters for
their tile's gate/up workgroups. Its outputs must equal those of the two-launch form bit for bit
(moe_forward_streamed with every expert resident runs the same per-tile
arithmetic as two launches), every wait must end normally on the waiting
workgroup's own XCD (STATUS 0), consecutive calls on one workspace must not
see each other's counters (each call's permutation clears them), and a
captured HIP graph must replay correctly (no memset nodes: the clearing is
part of the permutation kernel). It is held to the oracle by
test_gpu_parity.py's grouped cases."""
import pytest
import torch

import workloads as W
from parity import DevLayer, host_bank, log

pytestmark = pytest.mark.gpu

C = W.CONFIGS

_PINNED = {}


def pinned_bank(shape):
    key = shape.with_(tokens=0)
    if key not in _PINNED:
        import block_fp8_routed_amd as moe
        bank, _ = host_bank(key)
        _PINNED.clear()
        _PINNED[key] = moe.Bank.pinned_from_numpy(bank)
    return _PINNED[key]


def forward(layer, T=None, x=None, ws=None, path="mfma"):
    """moe_forward on a grouped path; returns (out, status word)."""
    import block_fp8_routed_amd as moe
    s = layer.shape
    xx = layer.x if x is None else x
    cfg = moe.make_config(len(xx), s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                          xx.dtype, torch.float32, path)
    if ws is None:
        ws = moe.make_workspace(cfg, "cuda")
    out = moe.moe_forward(xx, layer.router_w, layer.bank, s.top_k, s.block, shared=layer.shared,
                          router_bias=layer.bias, path=path,
                          workspace=ws[:moe.workspace_bytes(cfg)], cfg=cfg)
    torch.cuda.synchronize()
    st = int(moe.workspace_view(ws, cfg, moe.MOE_WS_STATUS, torch.int32).item())
    return out, st


# (config, tokens, overrides): row tiles dealt round-robin over the XCDs and
# (8192 tokens: more than 512 tiles) in cost-balanced chunks; decode sizes
# (selection and permutation in one launch); a ragged tail; the shared
# expert; uniform routing
CASES = [
    ("c2", 512, {}, "mfma"),
    ("c2", 8192, {}, "mfma"),
    ("c2", 17, {}, "mfma"),
    ("c1", 5, {}, "mfma"),
    ("c2", 300, {"shared": True}, "mfma"),
    ("c2", 1000, {"bias": None}, "mfma"),
    ("c2", 512, {}, "mfma_fp8"),
    ("c2", 8192, {}, "mfma_fp8"),
    ("c1", 5, {}, "mfma_fp8"),
    ("c2", 300, {"shared": True}, "mfma_fp8"),
]


def case_id(c):
    name, T, ov, path = c
    return f"{name}-T{T}-{path}" + ("-" + "-".join(sorted(ov)) if ov else "")


@pytest.mark.parametrize("name,T,ov,path", CASES, ids=[case_id(c) for c in CASES])
def test_one_launch_equals_two_launches(name, T, ov, path):
    import block_fp8_routed_amd as moe
    shape = C[name].with_(**ov) if ov else C[name]
    layer = DevLayer(shape, tokens=T)
    log(f"one launch vs two {case_id((name, T, ov, path))}")
    got, st = forward(layer, path=path)
    assert st == 0, f"status {st:#x}: a wait gave up or ran on another XCD"
    cache = moe.ExpertCache(shape.experts)
    slot_bank = moe.Bank.empty_slots(shape.experts, shape.hidden, shape.inter, shape.block)
    want = moe.moe_forward_streamed(layer.x, layer.router_w, pinned_bank(shape), slot_bank, cache,
                                    shape.top_k, shape.block, shared=layer.shared,
                                    router_bias=layer.bias, path=path)
    torch.cuda.synchronize()
    assert cache.rounds_last == 1
    assert torch.equal(got, want)


def test_back_to_back_calls_share_a_workspace():
    """Calls of different sizes on one workspace: each equals a call on a
    fresh workspace, and its status is 0 (a later call with fewer tiles
    than the one before must not see that call's counters)."""
    import block_fp8_routed_amd as moe
    shape = C["c2"]
    layer = DevLayer(shape, tokens=2048)
    s = shape
    big = moe.make_config(2048, s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                          layer.x.dtype, torch.float32, "mfma")
    ws = moe.make_workspace(big, "cuda")
    for b, T in enumerate([2048, 512, 17, 3, 2048, 900]):
        x = torch.from_numpy(W.gen_x(shape, 2048, batch=b)[:T]).to(layer.x.dtype).cuda()
        got, st = forward(layer, x=x, ws=ws)
        assert st == 0, f"call {b} (T={T}): status {st:#x}"
        want, st2 = forward(layer, x=x)
        assert st2 == 0
        assert torch.equal(got, want), f"call {b} (T={T})"


@pytest.mark.parametrize("path", ["mfma", "mfma_fp8"])
def test_graph_replay(path):
    """A HIP graph holding the grouped path (router, selection, permutation,
    the activation quantiser of the FP8 variant, the one-launch passes,
    combine) replays with new inputs, eager work in between, each replay
    equal to an eager call and with status 0."""
    import block_fp8_routed_amd as moe
    shape = C["c2"]
    T = 512
    layer = DevLayer(shape, tokens=T)
    s = shape
    cfg = moe.make_config(T, s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                          layer.x.dtype, torch.float32, path)
    ws = moe.make_workspace(cfg, "cuda")
    x_static = layer.x.clone()
    out_static = torch.empty((T, s.hidden), dtype=torch.float32, device="cuda")

    def call():
        moe.moe_forward(x_static, layer.router_w, layer.bank, s.top_k, s.block,
                        router_bias=layer.bias, path=path, out=out_static, workspace=ws,
                        cfg=cfg)

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
        x = torch.from_numpy(W.gen_x(shape, T, batch=b)).to(layer.x.dtype).cuda()
        x_static.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        got = out_static.clone()
        st = int(moe.workspace_view(ws, cfg, moe.MOE_WS_STATUS, torch.int32).item())
        assert st == 0, f"replay {b}: status {st:#x}"
        ref, _ = forward(layer, x=x, path=path)  # eager work between replays
        log(f"graph replay {b}: max |diff| {float((got - ref).abs().max()):.3g}")
        assert torch.equal(got, ref), f"replay {b}"


def test_wait_give_up_is_reported_and_cleared():
    """With a poll bound of 1 (moe_set_wait_limit), down workgroups that do
    not see their tile complete at once give up, set STATUS bit 8 and skip
    their tile, and the call still ends. Two tokens on the 128-expert layer
    make at most 16 row tiles, so every gate/up and down workgroup is
    resident at once and the down workgroups start polling while their
    tiles' gate/up workgroups still run (on larger problems the down
    workgroups are dispatched only as gate/up ones finish, and rarely wait).
    The next call on the same workspace, with the default bound, waits
    normally (the selection kernel clears the give-up word and the status)
    and equals a call on a fresh workspace."""
    import block_fp8_routed_amd as moe
    shape = C["c1"]
    T = 2
    layer = DevLayer(shape, tokens=T)
    s = shape
    cfg = moe.make_config(T, s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                          layer.x.dtype, torch.float32, "mfma")
    ws = moe.make_workspace(cfg, "cuda")
    try:
        moe.set_wait_limit(1)
        _, st = forward(layer, ws=ws)
    finally:
        moe.set_wait_limit(0)
    log(f"poll bound 1: status {st:#x}")
    assert st & 8, f"status {st:#x}: no wait gave up"
    got, st2 = forward(layer, ws=ws)
    assert st2 == 0, f"status {st2:#x} after the default bound was restored"
    want, _ = forward(layer)
    assert torch.equal(got, want)
