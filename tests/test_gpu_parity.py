"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle on the same seeded inputs (MI355X only)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import DevLayer, check_output, check_routing, fp8_h_band, host_bank, log

pytestmark = pytest.mark.gpu

C = W.CONFIGS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import block_fp8_routed_amd as moe
    moe.load()
    yield
    torch.cuda.synchronize()


# --------------------------------------------------------------- dequant ---
def test_device_decode_all_256_codes():
    import block_fp8_routed_amd as moe
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)
    w = torch.from_numpy(codes).cuda()
    s = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    got = moe.moe_dequant_e4m3(w, s, 16).cpu().numpy().astype(np.float64)
    want = oracle.e4m3fn_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(want[fin]))


def test_device_dequant_block_grid():
    import block_fp8_routed_amd as moe
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, (64, 96)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    scales = rng.uniform(1e-4, 10, (2, 3)).astype(np.float32)
    got = moe.moe_dequant_e4m3(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), 32)
    want = oracle.dequantise(codes, scales, 32).astype(np.float32)  # one fp32 rounding
    assert np.array_equal(got.cpu().numpy(), want)


def _act_rows(rng):
    """bf16 rows that reach every branch of the activation quantiser: exact
    midpoints between neighbouring E4M3 values (ties), signed zeros, an
    all-zero block, blocks whose largest value sits at 448 * 2^k and just
    above it, blocks at the -127 exponent floor, subnormal E4M3 results."""
    mags = oracle.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2
    rows = []
    r = np.zeros(512)
    r[:126] = mids                      # block 0: max 440 -> e = 0, ties
    r[128:254] = -mids
    r[256:384] = 0.0                    # an all-zero block
    r[384] = 448.0 * 4                  # largest value exactly 448 * 2^2
    r[385:512] = -0.0
    rows.append(r)
    r = np.zeros(512)
    r[0] = 448.0 * 2 ** -3 * (1 + 2 ** -7)   # just above 448 * 2^-3 (a bf16 value)
    r[1:128] = rng.normal(0, 1e-3, 127)      # small values, E4M3 subnormals
    r[128:256] = rng.normal(0, 1e-37, 128)   # tiny block: the -127 floor
    r[256:384] = rng.normal(0, 1, 128) * 2.0 ** 60
    r[384:512] = rng.normal(0, 1, 128) * 2.0 ** -100
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("T,H", [(2, 512), (300, 2048), (4096, 4096)])
def test_activation_quantiser_matches_oracle(T, H):
    """E4M3 activation codes and E8M0 exponents bit-exact against the oracle
    (reading R10), on crafted edge rows and random bf16 rows at the prefill
    shapes."""
    import block_fp8_routed_amd as moe
    rng = np.random.default_rng(T + H)
    x = rng.normal(0, 1, (T, H))
    x[:, ::97] *= 50.0                                 # a few outliers per row
    if H == 512:
        x = _act_rows(rng)
    xb = torch.from_numpy(x).to(torch.bfloat16)       # the values both sides see
    codes, exps = moe.moe_quantize_act_e4m3(xb.cuda())
    torch.cuda.synchronize()
    r_codes, r_exps = oracle.quantise_activations(xb.to(torch.float64).numpy(), 128)
    assert np.array_equal(codes.cpu().numpy(), r_codes)
    assert np.array_equal(exps.cpu().numpy().astype(np.int64) - 127, r_exps)
    log(f"quantise activations T={T} H={H}: codes and exponents bit-exact")


# ---------------------------------------------------------------- router ---
# (the slices router takes T <= 16 or tokens x experts <= 32768: c1 17, c2
# 256, c3 64 and c0e1024k16 at 32 tokens are its largest batches; c2 512, c3
# 65 and c3 300 the MFMA router's)
ROUTE_CASES = [
    ("c0", None), ("c1", 1), ("c1", 4), ("c1", 16), ("c1", 17), ("c2", 256), ("c2", None),
    ("c3", None), ("c3", 64), ("c3", 65), ("c3", 300), ("c4", None), ("c0e1024k16", 16),
    ("c0e1024k16", 32), ("c0e1024k16", 37),
]


@pytest.mark.parametrize("name,T", ROUTE_CASES, ids=[f"{n}-T{t}" for n, t in ROUTE_CASES])
def test_route_matches_oracle(name, T):
    # routing needs no expert bank: build the inputs directly
    import block_fp8_routed_amd as moe
    shape = C[name] if name in C else C["c0"].with_(experts=1024, top_k=16, name=name)
    T = shape.tokens if T is None else T
    x = W.gen_x(shape, T)
    wr, b = W.gen_router(shape), W.gen_bias(shape)
    xdt = torch.bfloat16 if shape.x_dtype == "bf16" else torch.float32
    idx, gates, logits = moe.moe_route(
        torch.from_numpy(x).to(xdt).cuda(), torch.from_numpy(wr).cuda(), shape.top_k,
        shape.inter, shape.block,
        router_bias=None if b is None else torch.from_numpy(b).cuda(), with_logits=True)

    class L:  # the fields check_routing reads
        pass
    L.x_host, L.router_host, L.bias_host, L.shape = x, wr, b, shape
    _, ties = check_routing(L, idx, gates, logits)
    log(f"route {name} T={T}: ok, {ties} tie-flagged tokens")


# --------------------------------------------------------------- permute ---
PERM_CASES = [  # (T, E, k, shared, skew)
    (1, 8, 2, False, 0), (4, 8, 2, True, 0), (16, 128, 8, False, 0), (37, 16, 16, True, 0),
    (1, 1, 1, True, 0), (300, 512, 10, True, 0), (4096, 512, 10, True, 1),
    (2000, 1024, 4, False, 1), (1000, 513, 7, True, 0),
    # either side of the one-block counting limit (4096 slots), skewed so some
    # experts take many slots
    (512, 128, 8, False, 1), (513, 128, 8, True, 1),
]


@pytest.mark.parametrize("T,E,k,shared,skew", PERM_CASES)
def test_permute_matches_oracle(T, E, k, shared, skew):
    import block_fp8_routed_amd as moe
    rng = np.random.default_rng(T * 7919 + E)
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.3
        p /= p.sum()
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    else:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    off, pair, inv = moe.moe_permute(torch.from_numpy(idx.astype(np.int32)).cuda(), E, shared,
                                     hidden=64, inter=32, block=32)
    r_off, r_pair, r_inv = oracle.permutation(idx, E, shared)
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(pair.cpu().numpy(), r_pair)
    assert np.array_equal(inv.cpu().numpy(), r_inv)


# --------------------------------------------------------------- forward ---
FWD_CASES = [  # (config, tokens, path, overrides)
    ("c0", None, "auto", {}),
    ("c0", 33, "gemv", {}),
    ("c0", 5, "gemv", {"shared": True, "bias": ("zipf", 1.1, 0.5)}),
    ("c1", 1, "auto", {}),
    ("c1", 4, "auto", {}),
    ("c1", 16, "auto", {}),
    ("c1", 13, "gemv", {"experts": 16, "top_k": 4}),
    ("c1", 40, "gemv", {"experts": 8, "top_k": 8}),
    ("c3", None, "auto", {}),
    ("c3", 3, "auto", {}),
    # grouped bf16 MFMA family: several 64-row tiles per group, ragged tails
    ("c1", 5, "mfma", {}),
    ("c1", 37, "mfma", {}),
    ("c1", 300, "mfma", {"experts": 16, "top_k": 4}),
    ("c1", 70, "mfma", {"experts": 8, "top_k": 8}),
    ("c1", 130, "mfma", {"experts": 4, "top_k": 1}),
    ("c1", 10000, "mfma", {}),  # > 512 row tiles: tiles dealt to XCDs in chunks
    ("c2", None, "auto", {}),
    ("c3", 100, "mfma", {}),
    # the limits: top-16 (the most a token may choose) of 512 experts through the
    # one-workgroup decode selection, and 1024 experts (the most supported) with a
    # shared expert through the multi-block path
    ("c0", 16, "gemv", {"experts": 512, "top_k": 16}),
    ("c0", 20, "gemv", {"experts": 1024, "top_k": 16, "shared": True}),
    ("c0", 3, "gemv", {"experts": 1024, "top_k": 1}),
    # expert counts that leave part of a lane row empty in the one-workgroup
    # decode selection (two and four experts per lane); the first token count
    # past it (the GEMV family with the multi-kernel selection and
    # permutation), the last that AUTO gives the GEMV family, and the first it
    # sends to the grouped MFMA family
    ("c0", 9, "gemv", {"experts": 100, "top_k": 3, "shared": True}),
    ("c0", 16, "auto", {"experts": 200, "top_k": 5}),
    ("c1", 17, "auto", {}),
    ("c1", 48, "auto", {}),
    ("c1", 49, "auto", {}),
    # the single-launch decode layer
    ("c1", 1, "gemv_fused", {}),
    ("c1", 16, "gemv_fused", {}),
    ("c3", None, "gemv_fused", {}),
    ("c0", 16, "gemv_fused", {"experts": 512, "top_k": 16}),
    ("c0", 9, "gemv_fused", {"experts": 100, "top_k": 3, "shared": True}),
]


def fwd_id(c):
    name, T, path, ov = c
    return f"{name}-T{T}-{path}" + ("-" + "-".join(sorted(ov)) if ov else "")


@pytest.mark.parametrize("name,T,path,ov", FWD_CASES, ids=[fwd_id(c) for c in FWD_CASES])
def test_forward_matches_oracle(name, T, path, ov):
    shape = C[name].with_(**ov) if ov else C[name]
    layer = DevLayer(shape, tokens=T)
    log(f"forward {fwd_id((name, T, path, ov))}: T={layer.T}")
    idx, gates = layer.route()
    accepted, ties = check_routing(layer, idx, gates)
    out = layer.forward(path=path)
    torch.cuda.synchronize()
    ref = layer.oracle(routing=accepted)
    check_output(out, ref["out"], what=f"{name} T={layer.T} {path} ties={ties}")


def _constructed_routing_layer():
    """A 16-expert layer at the 2048/768 shape whose routing is fixed by
    construction: router row e is 10 * (unit vector e), so a token's logits
    are 10 * x[t, :16], and each token carries four chosen experts at
    x = 4, 3, 2, 1 (all other of the first 16 entries 0; the rest N(0,1)).
    Group sizes hit the grouped-MFMA tile edges: 129 and 128 (two tiles, the
    second of 1 / 0 rows), 65 and 64 (the full/thin boundary), 33 (two
    32-row MFMA tiles, the second of 1 row), 1, and ~38-row fill groups.
    Some block scales are 0 over nonzero codes (their weights dequantise
    to 0)."""
    shape = C["c1"].with_(experts=16, top_k=4, name="c1e16_tiles")
    T, E, k, H = 200, 16, 4, shape.hidden
    ranges = {0: (0, 129), 1: (0, 128), 2: (129, 194), 3: (0, 64), 4: (64, 97), 5: (197, 198)}
    rng = np.random.default_rng(5)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, :E] = 0.0
    fill = 6
    for t in range(T):
        chosen = [e for e, (lo, hi) in ranges.items() if lo <= t < hi]
        while len(chosen) < k:
            if fill not in chosen:
                chosen.append(fill)
            fill = 6 + (fill - 5) % 10
        for j, e in enumerate(chosen):
            x[t, e] = float(k - j)
    x = W.round_to_bf16(x)
    wr = np.zeros((E, H), np.float32)
    wr[np.arange(E), np.arange(E)] = 10.0
    bank, _ = host_bank(shape.with_(tokens=0))
    bank = {key: v.copy() for key, v in bank.items()}
    I = shape.inter
    bank["s_gate_up"][0, 1, 3] = 0.0            # gate rows 128..255, k 384..511
    bank["s_gate_up"][1, I // 128 + 2, 5] = 0.0  # up rows 256..383 of expert 1
    bank["s_gate_up"][6, 0, 0] = 0.0            # a thin fill group
    bank["s_down"][2, 4, 1] = 0.0
    return shape, x, wr, bank


@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_forward_tile_edges_and_zero_scales(path):
    import block_fp8_routed_amd as moe
    shape, x, wr, bank = _constructed_routing_layer()
    k = shape.top_k
    ref_idx = oracle.select_topk(oracle.router_logits(x, wr, None), k)
    counts = np.bincount(ref_idx.reshape(-1), minlength=shape.experts)
    assert list(counts[:6]) == [129, 128, 65, 64, 33, 1], counts
    out = moe.moe_forward(torch.from_numpy(x).to(torch.bfloat16).cuda(), torch.from_numpy(wr).cuda(),
                          moe.Bank.from_numpy(bank), k, shape.block, path=path)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(x, wr, None, lambda e: W.bank_expert(bank, e), k, shape.inter,
                           shape.block)
    check_output(out, ref["out"], what=f"constructed routing, zero scales, {path}")


@pytest.mark.parametrize("case", ["subnormal", "far_apart"])
@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_forward_subnormal_and_far_apart_block_scales(path, case):
    """Block scales that are subnormal fp32 numbers (first block of a row,
    mid-row, the smallest one), or a down row whose consecutive blocks differ
    by 10^30 (each case alone, so that its outputs are not hidden under the
    other's RMS): the grouped passes keep their accumulators in units of the
    current block's scale and move between blocks by the ratio of the scales,
    which must stay finite and exact in exponent (a reciprocal of a
    subnormal overflows)."""
    import block_fp8_routed_amd as moe
    shape, x, wr, bank = _constructed_routing_layer()
    k = shape.top_k
    if case == "subnormal":
        bank["s_gate_up"][0, 0, 0] = np.float32(1e-39)   # first block of its rows
        bank["s_gate_up"][1, 1, 2] = np.float32(3e-40)   # mid-row
        bank["s_gate_up"][4, 7, 9] = np.float32(2e-45)   # the smallest subnormal
        bank["s_down"][3, 5, 2] = np.float32(5e-39)
        assert bank["s_gate_up"][4, 7, 9] > 0
    else:
        far = np.array([1e-20, 1e10, 1e-20, 1e10, 1e-20, 1e10], np.float32)
        bank["s_down"][2, 3, :] = far[: bank["s_down"].shape[2]]
        bank["s_gate_up"][0, 2, :] = np.resize(far, bank["s_gate_up"].shape[2])
    out = moe.moe_forward(torch.from_numpy(x).to(torch.bfloat16).cuda(), torch.from_numpy(wr).cuda(),
                          moe.Bank.from_numpy(bank), k, shape.block, path=path)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite output"
    ref = oracle.moe_layer(x, wr, None, lambda e: W.bank_expert(bank, e), k, shape.inter,
                           shape.block)
    check_output(out, ref["out"], what=f"{case} block scales, {path}")


@pytest.mark.parametrize("T,path", [(16, "gemv"), (5, "mfma"), (40, "gemv")])
def test_exact_ties_go_to_the_lower_index(T, path):
    """A router of zeros, its odd rows -0, makes every logit exactly +0 or -0
    (the activations are positive): the selection is fixed by the tie rule
    alone (experts 0 .. k-1 in that order, -0 equal to +0, gates 1/k), and
    every token lands in the same k groups."""
    import block_fp8_routed_amd as moe
    shape = C["c1"].with_(experts=16, top_k=4, name="c1e16_ties")
    E, k, H = shape.experts, shape.top_k, shape.hidden
    x = np.abs(W.gen_x(shape, T))
    wr = np.zeros((E, H), np.float32)
    wr[1::2] = -0.0
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    idx, gates = moe.moe_route(xd, torch.from_numpy(wr).cuda(), k, shape.inter, shape.block)
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(k), (T, 1)))
    assert np.array_equal(gates.cpu().numpy(), np.full((T, k), 1.0 / k, np.float32))
    bank, _ = host_bank(shape.with_(tokens=0))
    out = moe.moe_forward(xd, torch.from_numpy(wr).cuda(), moe.Bank.from_numpy(bank), k,
                          shape.block, path=path)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(x, wr, None, lambda e: W.bank_expert(bank, e), k, shape.inter,
                           shape.block)
    assert np.array_equal(ref["topk_idx"], np.tile(np.arange(k), (T, 1)))
    check_output(out, ref["out"], what=f"exact ties T={T} {path}")


def test_forward_bf16_output():
    layer = DevLayer(C["c1"], tokens=16)
    idx, gates = layer.route()
    accepted, _ = check_routing(layer, idx, gates)
    out = layer.forward(out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    ref = layer.oracle(routing=accepted)
    check_output(out, ref["out"], bf16_out=True, what="c1 T=16 bf16 out")


def test_forward_is_deterministic():
    layer = DevLayer(C["c1"], tokens=16)
    a = layer.forward()
    b = layer.forward()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_token_subset_invariance_gemv():
    full = DevLayer(C["c1"], tokens=16)
    out = full.forward()
    for lo, hi in ((0, 4), (4, 5), (5, 16)):
        part = DevLayer(C["c1"], x=full.x_host[lo:hi].copy())
        assert torch.equal(part.forward(), out[lo:hi]), (lo, hi)


def test_expert_relabelling_invariance():
    shape = C["c0"].with_(shared=True, bias=("zipf", 1.1, 0.5))
    base = DevLayer(shape, tokens=7)
    out = base.forward()
    perm = np.random.default_rng(3).permutation(shape.experts)
    import block_fp8_routed_amd as moe
    bank = {k: v[perm].copy() for k, v in base.bank_host.items()}
    dbank = moe.Bank.from_numpy(bank)
    wr = torch.from_numpy(base.router_host[perm].copy()).cuda()
    bias = torch.from_numpy(base.bias_host[perm].copy()).cuda()
    out2 = moe.moe_forward(base.x, wr, dbank, shape.top_k, shape.block, shared=base.shared,
                           router_bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_prefill_e512_full_size():
    """The 512-expert prefill workload at full size (4096 tokens, 16 hot
    experts) in the launch configuration the benchmark uses: routing of every
    token and the whole permutation against the oracle, and every one of the
    4096 x 4096 outputs against the oracle."""
    import block_fp8_routed_amd as moe
    shape = C["c4"]
    layer = DevLayer(shape)
    log("c4: routing all 4096 tokens")
    idx, gates = layer.route()
    accepted, ties = check_routing(layer, idx, gates)
    off, pair, inv = moe.moe_permute(idx, shape.experts, True, shape.hidden, shape.inter,
                                     shape.block)
    r_off, r_pair, r_inv = oracle.permutation(accepted, shape.experts, True)
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(pair.cpu().numpy(), r_pair)
    assert np.array_equal(inv.cpu().numpy(), r_inv)
    out = layer.forward()
    torch.cuda.synchronize()
    counts = np.bincount(accepted.reshape(-1), minlength=shape.experts)
    log(f"c4: oracle on all {shape.tokens} tokens ({int((counts > 0).sum())} routed experts "
        f"+ shared), ties={ties}")
    ref = layer.oracle(routing=accepted)
    check_output(out, ref["out"], what="c4 T=4096 full")


def tile_boundary_tokens(accepted, experts, shared, tile_rows=128):
    """Tokens holding the first and the last row of every row tile of every
    group of the permutation (the grouped passes' tiles): comparing their
    outputs touches every tile, including each group's partial last tile."""
    T, k = accepted.shape
    off, pair, _ = oracle.permutation(accepted, experts, shared)
    toks = set()
    for g in range(experts + (1 if shared else 0)):
        lo, hi = int(off[g]), int(off[g + 1])
        for r0 in range(lo, hi, tile_rows):
            for row in (r0, min(r0 + tile_rows, hi) - 1):
                slot = int(pair[row])
                toks.add(slot // k if slot < T * k else slot - T * k)
    return np.array(sorted(toks))


FP8_CASES = [  # (config, tokens, overrides): the FP8 variant (E4M3 x and h)
    ("c1", 37, {}),                              # thin tiles, ragged tails
    ("c1", 300, {"experts": 16, "top_k": 4}),    # full and thin tiles, several per group
    ("c2", None, {}),                            # the 512-token layer at full size
    ("c3", 100, {}),                             # 4096 hidden, shared expert
    ("c1", 5, {}),                               # decode sizes: one-workgroup selection
    ("c3", None, {}),                            # 8 tokens, shared expert
    ("c1", 70, {"experts": 8, "top_k": 8}),      # every token in every group (k = E)
    ("c1", 130, {"experts": 4, "top_k": 1}),     # one expert per token, large groups
    ("c1", 200, {"experts": 16, "top_k": 16, "shared": True}),  # top-16 with a shared expert
    ("c1", 10000, {}),                           # > 512 row tiles: tiles dealt to XCDs in chunks
]


@pytest.mark.parametrize("name,T,ov", FP8_CASES, ids=[fwd_id((n, t, "mfma_fp8", o)) for n, t, o in FP8_CASES])
def test_forward_fp8_matches_oracle(name, T, ov):
    """The grouped family with E4M3 operands in both expert contractions
    against the oracle that quantises x and h the same way (readings R10 and
    R11, block 128): every h code the kernel wrote is admissible, and the
    outputs match the oracle evaluated on those codes within the layer
    tolerance; the router reads x itself on both sides."""
    shape = C[name].with_(**ov) if ov else C[name]
    layer = DevLayer(shape, tokens=T)
    log(f"forward fp8 {name}: T={layer.T}")
    layer.forward_fp8_checked(what=f"{name} T={layer.T} mfma_fp8")


@pytest.mark.parametrize("path", ["mfma_fp8", "mfma"])
def test_forward_scaled_and_zero_rows(path):
    """Rows at scales 2^-4 .. 2^3 of the usual activations (so the E4M3
    exponents of x and h vary from token to token), rows whose first 128
    columns are zero (an all-zero activation block: exponent 0, zero codes),
    and all-zero rows (h is zero too; the output row is exactly zero), on
    both grouped families against the oracle."""
    shape = C["c1"]
    T = 48
    x = W.gen_x(shape, T, 5).astype(np.float64)
    x *= (2.0 ** (np.arange(T) % 8 - 4))[:, None]
    x[1::6, :128] = 0.0
    zero = np.array([5, 23, 47])
    x[zero] = 0.0
    layer = DevLayer(shape, x=x.astype(np.float32))
    log(f"scaled and zero rows {path}: T={T}")
    rest = np.setdiff1d(np.arange(T), zero)
    if path == "mfma_fp8":
        layer.forward_fp8_checked(tokens=rest, what=f"scaled rows {path}")
    idx, gates = layer.route()
    accepted, ties = check_routing(layer, idx, gates)
    out = layer.forward(path=path)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert not got[zero].any()
    if path != "mfma_fp8":
        ref = layer.oracle(routing=accepted)
        assert not ref["out"][zero].any()
        check_output(out, ref["out"][rest], tokens=rest, what=f"scaled rows {path} ties={ties}")


def test_prefill_e512_fp8_full_size_tiles():
    """The FP8 variant on the 512-expert prefill workload at full size (4096
    tokens): outputs of the tokens that hold the first and the last row of
    every row tile of every group (so every tile of both passes is compared)
    against the oracle."""
    shape = C["c4"]
    layer = DevLayer(shape)
    idx, gates = layer.route()
    accepted, ties = check_routing(layer, idx, gates)
    sample = tile_boundary_tokens(accepted, shape.experts, True)
    log(f"c4 fp8: oracle on {len(sample)} tokens covering every row tile")
    layer.forward_fp8_checked(tokens=sample, what="c4 T=4096 mfma_fp8 tile rows")


RANGE_CASES = [("gemv", 16), ("mfma", 48), ("mfma_fp8", 48)]


@pytest.mark.parametrize("scale", ["large", "tiny", "mixed"])
@pytest.mark.parametrize("path,T", RANGE_CASES, ids=[f"{p}-T{t}" for p, t in RANGE_CASES])
def test_forward_far_outside_fp16_range(path, T, scale):
    """h and y are stored below fp32 between the passes; their power-of-two
    exponents must keep any magnitude. Activations scaled by 2^9 drive h and y
    far past fp16's largest value (65504), by 2^-14 far below its smallest
    normal (6.1e-5), and a mixed batch puts rows of both kinds (and 2^0) in the
    same expert groups; outputs against the oracle at the layer tolerance,
    whose per-token cosine sees each row at its own scale. The router weights
    take the inverse power of two (of the largest scale), so that the logits
    stay in the range whose absolute tolerances the routing check states:
    with a uniform scale they are exactly those of the unscaled rows."""
    shape = C["c1"]
    x = W.gen_x(shape, T, 7).astype(np.float64)
    if scale == "large":
        x *= 2.0 ** 9
        r = 2.0 ** -9
    elif scale == "tiny":
        x *= 2.0 ** -14
        r = 2.0 ** 14
    else:
        x *= (2.0 ** np.array([9, -14, 0])[np.arange(T) % 3])[:, None]
        r = 2.0 ** -9
    layer = DevLayer(shape, x=x.astype(np.float32))
    layer.router_host = (layer.router_host * np.float32(r)).astype(np.float32)
    layer.router_w = torch.from_numpy(layer.router_host).cuda()
    if path == "mfma_fp8":
        layer.forward_fp8_checked(what=f"{path} T={T} {scale} rows")
        return
    idx, gates = layer.route()
    accepted, ties = check_routing(layer, idx, gates)
    out = layer.forward(path=path)
    torch.cuda.synchronize()
    ref = layer.oracle(routing=accepted)
    check_output(out, ref["out"], what=f"{path} T={T} {scale} rows ties={ties}")


DECODE_PERM_CASES = [  # (config, tokens, overrides): the fused decode selection + permutation
    ("c1", 1, {}), ("c1", 4, {}), ("c1", 16, {}), ("c3", None, {}), ("c3", 3, {}),
    ("c0", 16, {"experts": 512, "top_k": 16}), ("c0", 9, {"experts": 100, "top_k": 3,
                                                          "shared": True}),
]


@pytest.mark.parametrize("name,T,ov", DECODE_PERM_CASES,
                         ids=[fwd_id((n, t, "auto", o)) for n, t, o in DECODE_PERM_CASES])
def test_decode_permutation_in_the_workspace(name, T, ov):
    """At decode sizes one kernel selects every token's experts and builds the
    permutation; after moe_forward its results are read from the workspace
    (moe_workspace_region) and compared bit-exactly with the oracle's
    selection and permutation, and the fp32 SwiGLU output h of every
    permuted row with the oracle's h of that (token, expert) pair."""
    import block_fp8_routed_amd as moe
    shape = C[name].with_(**ov) if ov else C[name]
    layer = DevLayer(shape, tokens=T)
    s = layer.shape
    T = layer.T
    cfg = moe.make_config(T, s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                          layer.x.dtype, torch.float32, "auto")
    ws = moe.make_workspace(cfg, "cuda")
    layer.forward(workspace=ws, cfg=cfg)
    torch.cuda.synchronize()

    def view(region, dtype):
        return moe.workspace_view(ws, cfg, region, dtype).cpu().numpy()
    topk = view(moe.MOE_WS_TOPK, torch.int32).reshape(T, s.top_k)
    gates = torch.from_numpy(view(moe.MOE_WS_GATES, torch.float32).reshape(T, s.top_k))
    accepted, ties = check_routing(layer, torch.from_numpy(topk), gates)
    r_off, r_pair, r_inv = oracle.permutation(accepted, s.experts, s.shared)
    assert np.array_equal(view(moe.MOE_WS_OFFSETS, torch.int32), r_off)
    assert np.array_equal(view(moe.MOE_WS_PAIR, torch.int32), r_pair)
    assert np.array_equal(view(moe.MOE_WS_INV, torch.int32), r_inv)
    # S4 alone: h of each permuted row (fp32 on this family)
    h = view(moe.MOE_WS_H, torch.float32).reshape(len(r_pair), s.inter).astype(np.float64)
    x = layer.x_host.astype(np.float64)
    worst = 0.0
    for row, slot in enumerate(r_pair):
        if slot < T * s.top_k:
            t, e = slot // s.top_k, int(accepted[slot // s.top_k, slot % s.top_k])
            wg, wu, _ = oracle.expert_matrices(layer.expert(e), s.inter, s.block)
        else:
            t = slot - T * s.top_k
            wg, wu, _ = oracle.expert_matrices(W.bank_expert(layer.shared_host, 0), s.inter,
                                               s.block)
        ref_h = oracle.silu(x[t] @ wg.T) * (x[t] @ wu.T)
        scale = np.abs(ref_h).max()
        worst = max(worst, float(np.abs(h[row] - ref_h).max() / scale))
    log(f"decode {name} T={T}: permutation bit-exact, h max rel err {worst:.2e}, ties={ties}")
    assert worst <= 1e-4, f"h error {worst:.2e} of the row's largest value"


WS_CASES = [("c1", 16, "auto"), ("c1", 4, "auto"), ("c0", 4, "auto"), ("c1", 16, "mfma"),
            ("c2", 512, "auto"), ("c3", 8, "auto"), ("c2", 512, "mfma_fp8"),
            ("c1", 37, "mfma_fp8"),
            # the single-launch decode layer: arbitrary flag words never pass a wait
            ("c1", 16, "gemv_fused"), ("c3", 8, "gemv_fused")]


@pytest.mark.parametrize("name,T,path", WS_CASES, ids=[f"{n}-T{t}-{p}" for n, t, p in WS_CASES])
def test_forward_does_not_depend_on_workspace_contents(name, T, path):
    """Every workspace byte the layer reads is written by the same call first,
    and nothing is written past the workspace: results are bit-identical for a
    zeroed and a garbage-filled workspace, and a canary band after the
    workspace is untouched."""
    import block_fp8_routed_amd as moe
    layer = DevLayer(C[name], tokens=T)
    s = layer.shape
    cfg = moe.make_config(T, s.hidden, s.experts, s.inter, s.top_k, s.block, s.shared,
                          layer.x.dtype, torch.float32, path)
    n = moe.workspace_bytes(cfg)
    guard = 1 << 20
    outs = []
    for fill in (0x00, 0xA5):
        buf = torch.full((n + guard,), fill, dtype=torch.uint8, device="cuda")
        ws = buf[:n]
        outs.append(layer.forward(path=path, workspace=ws).clone())
        torch.cuda.synchronize()
        assert bool((buf[n:] == fill).all()), "write past the end of the workspace"
    assert torch.equal(outs[0], outs[1])
