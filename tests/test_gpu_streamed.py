"""moe_forward_streamed: routed experts in pinned host memory, streamed into
a bounded LRU cache of device expert slots (colizig page, "Features": the
bounded LRU expert cache and the GPU backend's LRU VRAM weight cache). Its
outputs must equal moe_forward's bit for bit (the same kernels compute each
group once), with caches smaller than one call's needed experts (several
rounds per call) and across calls whose needs overlap; one case is also held
to the oracle directly. The cache's bookkeeping is checked against the
routing (hits + misses = experts needed, distinct residents, LRU order)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import DevLayer, check_output, check_routing, host_bank, log

pytestmark = pytest.mark.gpu

_PINNED = {}


def pinned_bank(shape):
    key = shape.with_(tokens=0)
    if key not in _PINNED:
        import block_fp8_routed_amd as moe
        bank, _ = host_bank(key)
        _PINNED.clear()
        _PINNED[key] = moe.Bank.pinned_from_numpy(bank)
    return _PINNED[key]


def needed_experts(layer, accepted):
    return set(np.unique(accepted).tolist())


def streamed(layer, cache, slot_bank, path="auto"):
    import block_fp8_routed_amd as moe
    s = layer.shape
    return moe.moe_forward_streamed(layer.x, layer.router_w, pinned_bank(s), slot_bank, cache,
                                    s.top_k, s.block, shared=layer.shared,
                                    router_bias=layer.bias, path=path)


CASES = [  # (config, tokens per call, slots, path)
    ("c1", 16, 32, "auto"),      # 81 experts per call: three rounds
    ("c3", 8, 40, "auto"),       # shared expert, two rounds
    ("c2", 512, 48, "auto"),     # grouped MFMA family, all 128 experts: three rounds
    ("c2", 300, 100, "mfma_fp8"),
    ("c1", 4, 64, "auto"),       # the cache holds every call's experts
]


@pytest.mark.parametrize("name,T,slots,path", CASES,
                         ids=[f"{n}-T{t}-slots{s}-{p}" for n, t, s, p in CASES])
def test_streamed_matches_resident_forward(name, T, slots, path):
    import block_fp8_routed_amd as moe
    shape = W.CONFIGS[name]
    cache = moe.ExpertCache(slots)
    slot_bank = moe.Bank.empty_slots(slots, shape.hidden, shape.inter, shape.block)
    needs = []
    for call, batch in enumerate((0, 1, 1, 0)):
        layer = DevLayer(shape, tokens=T, batch=batch)
        want = layer.forward(path=path)
        got = streamed(layer, cache, slot_bank, path)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {call}: streamed output differs"
        idx, _ = layer.route()
        need = set(np.unique(idx.cpu().numpy()).tolist())
        needs.append(need)
        log(f"streamed {name} T={T} slots={slots} {path} call {call}: {len(need)} experts, "
            f"{cache.rounds_last} rounds, hits {cache.hits} misses {cache.misses}, "
            f"{cache.bytes_in / 1e6:.0f} MB in")
        assert cache.rounds_last == max(1, -(-len(need) // slots))
        res = cache.slot_expert[cache.slot_expert >= 0]
        assert len(set(res.tolist())) == len(res)
        assert cache.calls == call + 1
    assert cache.hits + cache.misses == sum(len(n) for n in needs)
    per_expert = shape.expert_bytes()
    assert cache.bytes_in == cache.misses * per_expert
    if len(needs[0] | needs[1]) <= slots:  # everything fits: each expert is copied once
        assert cache.misses == len(needs[0] | needs[1])


def test_streamed_against_the_oracle():
    """A cache of 20 slots for a 16-token call needing ~81 experts (five
    rounds), compared with the oracle directly."""
    import block_fp8_routed_amd as moe
    shape = W.CONFIGS["c1"]
    layer = DevLayer(shape, tokens=16, batch=2)
    idx, gates = layer.route()
    accepted, ties = check_routing(layer, idx, gates)
    cache = moe.ExpertCache(20)
    slot_bank = moe.Bank.empty_slots(20, shape.hidden, shape.inter, shape.block)
    out = streamed(layer, cache, slot_bank)
    torch.cuda.synchronize()
    ref = layer.oracle(routing=accepted)
    check_output(out, ref["out"], what=f"streamed c1 T=16 slots=20 ties={ties}")
    assert cache.rounds_last == -(-len(np.unique(accepted)) // 20)


def test_streamed_lru_order():
    """Least recently used out first: with 8 slots, a call needing experts
    A (8 of them) and then a call needing B (8 others, disjoint) evicts all
    of A; a third call needing 4 of B and 4 new ones keeps those 4 of B."""
    import block_fp8_routed_amd as moe
    shape = W.CONFIGS["c1"].with_(experts=24, top_k=8, name="c1e24")
    cache = moe.ExpertCache(8)
    slot_bank = moe.Bank.empty_slots(8, shape.hidden, shape.inter, shape.block)
    H = shape.hidden

    def layer_for(experts):
        # a router whose logits are 10 x (unit vector e) for the chosen experts
        x = np.zeros((1, H), np.float32)
        x[0, :24] = -5.0
        for j, e in enumerate(experts):
            x[0, e] = 8.0 - 0.5 * j
        x = W.round_to_bf16(x)
        lay = DevLayer(shape, x=x)
        wr = np.zeros((24, H), np.float32)
        wr[np.arange(24), np.arange(24)] = 1.0
        lay.router_host = wr
        lay.router_w = torch.from_numpy(wr).cuda()
        return lay

    for experts, want_hits in ((list(range(8)), 0), (list(range(8, 16)), 0),
                               ([8, 9, 10, 11, 16, 17, 18, 19], 4)):
        lay = layer_for(experts)
        h0 = cache.hits
        got = streamed(lay, cache, slot_bank)
        want = lay.forward()
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        assert set(cache.slot_expert.tolist()) == set(experts)
        assert cache.hits - h0 == want_hits
