"""Pins of the CPU oracle to things other than itself (CPU only).

Each pin checks the oracle against something independent of its own code:
a library routine (torch's float8_e4m3fn conversion, torch's silu and matmul),
a published table (tests/golden/e4m3fn_anchors.txt, OCP OFP8), brute force
over all subsets, a scalar pure-Python evaluation of the definitions, or a
closed-form special case (one expert; all experts with equal gates). The
mutation test at the end plants plausible mistakes in copies of the oracle and
requires every one of them to fail at least one pin.
"""
import importlib.util
import itertools
import math
import os
import sys

import numpy as np
import pytest
import torch

from oracle import moe_oracle as ORACLE

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "moe_oracle.py")


# ---------------------------------------------------------------- helpers ---
def lib_decode(codes):
    """E4M3FN bytes -> fp64 through torch's own float8_e4m3fn conversion."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def lib_dequant(codes, scales, block):
    """Library dequantisation: torch fp8 decode times a Kronecker-expanded scale grid."""
    w = torch.from_numpy(lib_decode(codes))
    s = torch.from_numpy(np.asarray(scales, np.float64))
    return (w * torch.kron(s, torch.ones(block, block, dtype=torch.float64))).numpy()


def random_codes(rng, shape):
    """Random E4M3FN bytes excluding the two NaN codes."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def random_expert(rng, H, I, B, scale_lo=0.001, scale_hi=0.01):
    return {
        "w_gate_up": random_codes(rng, (2 * I, H)),
        "s_gate_up": rng.uniform(scale_lo, scale_hi, (2 * I // B, H // B)).astype(np.float32),
        "w_down": random_codes(rng, (H, I)),
        "s_down": rng.uniform(scale_lo, scale_hi, (H // B, I // B)).astype(np.float32),
    }


def torch_swiglu(x, expert, I, B):
    """Dense SwiGLU expert through torch library routines."""
    wgu = torch.from_numpy(lib_dequant(expert["w_gate_up"], expert["s_gate_up"], B))
    wd = torch.from_numpy(lib_dequant(expert["w_down"], expert["s_down"], B))
    xt = torch.from_numpy(np.asarray(x, np.float64))
    a = xt @ wgu[:I].T
    u = xt @ wgu[I:].T
    return (torch.nn.functional.silu(a) * u @ wd.T).numpy()


# ------------------------------------------------------------------- pins ---
def pin_decode_matches_library(O):
    codes = np.arange(256, dtype=np.uint8)
    ours, lib = O.e4m3fn_decode(codes), lib_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(lib)) and np.isnan(ours).sum() == 2
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], lib[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(lib[fin]))


def pin_decode_anchors(O):
    path = os.path.join(HERE, "golden", "e4m3fn_anchors.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        got = float(O.e4m3fn_decode(np.array([int(code, 16)], np.uint8))[0])
        if val == "nan":
            assert math.isnan(got), code
        else:
            want = float(val)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)
        n += 1
    assert n >= 10


def pin_dequant_bruteforce(O):
    rng = np.random.default_rng(1)
    B = 2
    codes = random_codes(rng, (6 * B, 4 * B))  # non-square block grid (6 x 4)
    scales = rng.uniform(0.5, 3.0, (6, 4)).astype(np.float32)
    ours = O.dequantise(codes, scales, B)
    dec = lib_decode(codes)
    for r in range(codes.shape[0]):
        for c in range(codes.shape[1]):
            assert ours[r, c] == dec[r, c] * float(scales[r // B, c // B])
    assert np.array_equal(ours, lib_dequant(codes, scales, B))


def brute_topk(l, k):
    """Max-sum k-subset, lexicographically lowest among ties, in slot order."""
    E = len(l)
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(range(E), k):  # lexicographic order
        s = sum(l[e] for e in sub)
        if s > best_sum:
            best, best_sum = sub, s
    return sorted(best, key=lambda e: (-l[e], e))


def pin_topk_bruteforce(O):
    rng = np.random.default_rng(2)
    for trial in range(300):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        # few distinct integer values: many exact ties, exactly summable
        l = rng.integers(-3, 4, size=(1, E)).astype(np.float64)
        got = list(O.select_topk(l, k)[0])
        assert got == brute_topk(list(l[0]), k), (l, k, got)


def pin_gates(O):
    rng = np.random.default_rng(3)
    for trial in range(100):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, E + 1))
        l = rng.normal(0, 3, (2, E))
        if trial % 3 == 0:
            l = np.round(l)  # ties
        idx = O.select_topk(l, k)
        g = O.gate_weights(l, idx)
        assert np.allclose(g.sum(axis=1), 1.0, atol=1e-12, rtol=0)
        for t in range(2):
            sel = np.array([l[t, e] for e in idx[t]])
            restricted = [math.exp(v - sel.max()) for v in sel]
            tot = math.fsum(restricted)
            assert np.allclose(g[t], [v / tot for v in restricted], atol=1e-12, rtol=0)
            # non-increasing in slot order, since slots follow descending logits
            assert all(g[t, j] >= g[t, j + 1] for j in range(k - 1))
        # a common shift of the logits changes nothing
        assert np.allclose(O.gate_weights(l + 7.25, idx), g, atol=1e-12, rtol=0)


def pin_permutation(O):
    rng = np.random.default_rng(4)
    for trial in range(50):
        T, E = int(rng.integers(1, 30)), int(rng.integers(1, 12))
        k = int(rng.integers(1, E + 1))
        shared = bool(trial % 2)
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        off, pair, inv = O.permutation(idx, E, shared)
        flat = idx.reshape(-1)
        want = sorted(range(T * k), key=lambda s: (flat[s], s // k))
        if shared:
            want += [T * k + t for t in range(T)]
        assert list(pair) == want
        counts = np.bincount(flat, minlength=E)
        assert off[0] == 0 and all(off[e + 1] - off[e] == counts[e] for e in range(E))
        assert off[E] == T * k and off[E + 1] == T * k + (T if shared else 0)
        assert np.array_equal(inv[pair], np.arange(len(pair)))
        for e in range(E):
            assert all(flat[s] == e for s in pair[off[e]:off[e + 1]])


def pin_single_expert_is_dense(O):
    rng = np.random.default_rng(5)
    H, I, B = 12, 8, 4  # H != I, non-square scale grids
    ex = random_expert(rng, H, I, B, 0.05, 0.5)
    x = rng.normal(0, 1, (5, H))
    wr = rng.normal(0, 1, (1, H))
    res = O.moe_layer(x, wr, None, lambda e: ex, top_k=1, inter=I, block=B)
    assert np.allclose(res["gates"], 1.0, atol=0, rtol=0)
    assert np.allclose(res["out"], torch_swiglu(x, ex, I, B), rtol=1e-12, atol=1e-12)


def pin_all_experts_equal_gates_is_dense_mean(O):
    rng = np.random.default_rng(6)
    H, I, B, E = 8, 4, 4, 5
    bank = [random_expert(rng, H, I, B, 0.05, 0.5) for _ in range(E)]
    shared = random_expert(rng, H, I, B, 0.05, 0.5)
    x = rng.normal(0, 1, (3, H))
    wr = np.zeros((E, H))
    res = O.moe_layer(x, wr, np.zeros(E), lambda e: bank[e], top_k=E, inter=I, block=B,
                      shared=shared)
    assert np.allclose(res["gates"], 1.0 / E, atol=1e-15, rtol=0)
    assert [list(r) for r in res["topk_idx"]] == [list(range(E))] * 3
    dense = sum(torch_swiglu(x, bank[e], I, B) for e in range(E)) / E
    dense = dense + torch_swiglu(x, shared, I, B)
    assert np.allclose(res["out"], dense, rtol=1e-12, atol=1e-12)


def scalar_layer(x, wr, bias, bank, shared, k, I, B):
    """The layer's definitions evaluated with Python scalars and loops."""
    T, H = len(x), len(x[0])
    E = len(wr)

    def weights(ex):
        dgu, dd = lib_decode(ex["w_gate_up"]), lib_decode(ex["w_down"])
        sgu, sd = ex["s_gate_up"], ex["s_down"]
        wgu = [[float(dgu[r][c]) * float(sgu[r // B][c // B]) for c in range(H)]
               for r in range(2 * I)]
        wdn = [[float(dd[r][c]) * float(sd[r // B][c // B]) for c in range(I)] for r in range(H)]
        return wgu, wdn

    def ffn(xt, w):
        wgu, wdn = w
        h = []
        for i in range(I):
            a = math.fsum(wgu[i][c] * xt[c] for c in range(H))
            u = math.fsum(wgu[I + i][c] * xt[c] for c in range(H))
            h.append(a / (1.0 + math.exp(-a)) * u)
        return [math.fsum(wdn[n][i] * h[i] for i in range(I)) for n in range(H)]

    cache = {}
    out = []
    for t in range(T):
        xt = [float(v) for v in x[t]]
        l = [math.fsum(xt[c] * float(wr[e][c]) for c in range(H))
             + (float(bias[e]) if bias is not None else 0.0) for e in range(E)]
        sel = brute_topk(l, k)
        m = max(l[e] for e in sel)
        den = math.fsum(math.exp(l[e] - m) for e in sel)
        o = [0.0] * H
        for e in sel:
            if e not in cache:
                cache[e] = weights(bank[e])
            y = ffn(xt, cache[e])
            g = math.exp(l[e] - m) / den
            o = [o[n] + g * y[n] for n in range(H)]
        if shared is not None:
            y = ffn(xt, weights(shared))
            o = [o[n] + y[n] for n in range(H)]
        out.append(o)
    return np.array(out)


def pin_whole_layer_scalar(O):
    import workloads as W
    for name, bias, shared in (("c0", None, False), ("c0", "zipf", True)):
        shape = W.CONFIGS[name]
        if bias:
            shape = shape.with_(bias=("zipf", 1.1, 0.5), shared=True)
        d = W.gen_layer(shape)
        bank = [W.bank_expert(d["bank"], e) for e in range(shape.experts)]
        sh = W.bank_expert(d["shared"], 0) if shared else None
        res = O.moe_layer(d["x"], d["router_w"], d["router_bias"], lambda e: bank[e],
                          top_k=shape.top_k, inter=shape.inter, block=shape.block, shared=sh)
        want = scalar_layer(d["x"], d["router_w"], d["router_bias"], bank, sh,
                            shape.top_k, shape.inter, shape.block)
        scale = np.sqrt(np.mean(want ** 2))
        assert np.max(np.abs(res["out"] - want)) <= 1e-12 * scale, name


def pin_tie_flags(O):
    l = np.array([[3.0, 2.0, 2.0 - 5e-6, 0.0],
                  [3.0, 2.0, 2.0 - 2e-5, 0.0],
                  [3.0, 3.0, 3.0, 3.0],
                  [4.0, 3.0, 3.0 - 1.5e-5, 0.0]])
    assert list(O.tie_flags(l, 2)) == [True, False, True, False]
    assert not O.tie_flags(l, 4).any()


# ------------------------------------------ E4M3 activations (reading R10) ---
def lib_round(v):
    """E4M3FN bytes of fp64 values through torch's own float8_e4m3fn cast."""
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def scalar_exponent(amax):
    """Smallest integer e >= -127 with amax <= 448 * 2^e, by counting up."""
    if amax == 0.0:
        return 0
    e = -127
    while amax > math.ldexp(448.0, e):
        e += 1
    return e


def pin_act_round_matches_library(O):
    rng = np.random.default_rng(10)
    mags = lib_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448, increasing
    mids = (mags[:-1] + mags[1:]) / 2                  # exact ties in fp64
    v = np.concatenate([mids, -mids, mags, -mags, rng.uniform(-448, 448, 4000),
                        rng.uniform(-2e-2, 2e-2, 4000), [0.0, -0.0, -1e-30]])
    assert np.array_equal(O.e4m3fn_round(v), lib_round(v))


def pin_act_scale_closed_form(O):
    for k in (-20, -1, 0, 3, 40):
        b = math.ldexp(448.0, k)
        got = O.act_scale_exponent(np.array([b, b * (1 + 2.0 ** -30), b * (1 - 2.0 ** -30)]))
        assert list(got) == [k, k + 1, k]
    assert list(O.act_scale_exponent(np.array([0.0, 1e-300, 1.0]))) == [0, -127, -8]


def pin_act_quantise_blocks_bruteforce(O):
    rng = np.random.default_rng(11)
    B = 32
    x = rng.normal(0, 1, (3, 4 * B)) * np.array([1e-3, 1.0, 1e3])[:, None]
    x[1, B:2 * B] = 0.0                                # an all-zero block
    x[2, 2 * B + 5] = 5e5                              # one large value: its block only
    codes, exps = O.quantise_activations(x, B)
    for t in range(x.shape[0]):
        for b in range(x.shape[1] // B):
            blk = x[t, b * B:(b + 1) * B]
            e = scalar_exponent(float(np.abs(blk).max()))
            assert exps[t, b] == e
            assert np.array_equal(codes[t, b * B:(b + 1) * B], lib_round(blk * 2.0 ** -e))
    xh = O.dequantise_activations(codes, exps, B)
    ok = np.abs(xh - x) <= np.maximum(2.0 ** -4 * np.abs(x),
                                      2.0 ** -10 * np.repeat(np.ldexp(1.0, exps), B, axis=1))
    assert ok.all()
    # idempotent in value (the exponent may drop by one when a block's
    # largest value rounds down to 448 * 2^(e-1); the values stay the same)
    assert np.array_equal(O.dequantise_activations(*O.quantise_activations(xh, B), B), xh)


def torch_quantise_rows(v, B):
    """Per row and block of B columns: scale exponent by counting up, E4M3 by
    torch's cast, back to fp64."""
    out = np.empty_like(v)
    for t in range(v.shape[0]):
        for b in range(v.shape[1] // B):
            blk = v[t, b * B:(b + 1) * B]
            e = scalar_exponent(float(np.abs(blk).max()))
            out[t, b * B:(b + 1) * B] = lib_decode(lib_round(blk * 2.0 ** -e)) * 2.0 ** e
    return out


def torch_swiglu_q(x, expert, I, B):
    """torch_swiglu with h quantised per row and B columns before the down
    product (the FP8 variant's down contraction)."""
    wgu = torch.from_numpy(lib_dequant(expert["w_gate_up"], expert["s_gate_up"], B))
    wd = torch.from_numpy(lib_dequant(expert["w_down"], expert["s_down"], B))
    xt = torch.from_numpy(np.asarray(x, np.float64))
    h = (torch.nn.functional.silu(xt @ wgu[:I].T) * (xt @ wgu[I:].T)).float().double().numpy()
    return (torch.from_numpy(torch_quantise_rows(h, B)) @ wd.T).numpy()


def pin_act_layer_uses_quantised_experts_only(O):
    """With act_block, the experts see E4M3 activations (x for gate/up, h for
    down) and the router the original x: against a torch evaluation that
    quantises with torch's cast."""
    rng = np.random.default_rng(12)
    H, I, B, E, k, T = 64, 32, 32, 4, 2, 5
    experts = [random_expert(rng, H, I, B) for _ in range(E)]
    shared = random_expert(rng, H, I, B)
    x = rng.normal(0, 1, (T, H))
    wr = rng.normal(0, 0.3, (E, H))
    res = O.moe_layer(x, wr, None, lambda e: experts[e], k, I, B, shared=shared, act_block=B)
    xh = torch_quantise_rows(x, B)
    logits = torch.from_numpy(x) @ torch.from_numpy(wr).T
    top = torch.topk(logits, k, dim=1).indices.numpy()
    assert np.array_equal(res["topk_idx"], top)
    want = torch_swiglu_q(xh, shared, I, B)
    for t in range(T):
        g = torch.softmax(logits[t, top[t]], 0).numpy()
        for j in range(k):
            want[t] += g[j] * torch_swiglu_q(xh[t:t + 1], experts[top[t, j]], I, B)[0]
    assert np.allclose(res["out"], want, rtol=1e-9, atol=1e-12)


# --------------------------- quantised h and its admissible flips (R11) ---
def pin_h_decided_in_fp32(O):
    """h = 1.0625 + 2^-30 (block maximum 448, exponent 0) is nearer 1.125 in
    fp64 but rounds to the midpoint 1.0625 in fp32, where the tie goes to the
    even code 1.0. silu(64) is exactly 64 in fp64, so h = 64 u exactly."""
    v = 1.0625 + 2.0 ** -30
    xs = np.array([[1.0]])
    wg = np.array([[64.0], [64.0]])
    wu = np.array([[7.0], [v / 64.0]])
    wd = np.array([[0.0, 1.0], [1.0, 0.0]])
    y = O.swiglu_expert(xs, wg, wu, wd, h_block=2)
    assert y.tolist() == [[1.0, 448.0]]
    assert lib_decode(lib_round(np.float32(v))) == 1.0  # the library's cast agrees


def pin_h_deviation_closed_form(O):
    """Hand-worked cases of the admissible deviation. Block [448, 1.0625,
    1.03, 0.0052] with a band of 1e-9: the maximum may cross 448, so the
    exponent may be 0 or 1; 1.0625 is a midpoint (1.0 by the even tie, 1.125
    just above it); 1.03 gives 1.0 either way; 0.0052 is subnormal, 3 * 2^-9
    under exponent 0 and 2 * 2^-9 under exponent 1. With a maximum of 300
    the exponent is 0 across the band; with no band nothing moves."""
    h = np.array([[448.0, 1.0625, 1.03, 0.0052, 300.0, 1.0625, 1.03, 0.0052]])
    dev = O.h_admissible_deviation(h, np.full(h.shape, 1e-9), 4)
    assert dev.tolist() == [[0.0, 0.125, 0.0, 2.0 ** -9, 0.0, 0.125, 0.0, 0.0]]
    assert not O.h_admissible_deviation(h, np.zeros(h.shape), 4).any()
    neg = O.h_admissible_deviation(-h, np.full(h.shape, 1e-9), 4)
    assert np.array_equal(neg, dev)


def pin_h_deviation_bruteforce(O):
    """Soundness by brute force: every h' in the band, quantised by the
    library's cast with the exponent its own block maximum gives, stays
    within the deviation of q(h). The h values sit on code midpoints and
    block maxima near 448 * 2^e, so flips of codes and of exponents occur."""
    rng = np.random.default_rng(21)
    B = 4
    mags = lib_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2
    n, I = 6, 8
    e = rng.integers(-3, 3, (n, I // B))
    h = rng.choice(mids[8:], (n, I)) * np.repeat(np.ldexp(1.0, e), B, axis=1)
    h[:, ::B] = np.ldexp(448.0, e)  # each block's maximum on the exponent boundary
    h *= rng.choice([-1.0, 1.0], h.shape)
    tau = np.abs(h) * 10.0 ** rng.uniform(-9, -3, h.shape)
    dev = O.h_admissible_deviation(h, tau, B)
    ref = torch_quantise_rows(h, B)
    seen = np.zeros_like(h)
    for blk in range(I // B):
        cols = slice(blk * B, (blk + 1) * B)
        for signs in itertools.product((-1.0, 0.0, 1.0), repeat=B):
            hp = h[:, cols] + np.array(signs) * tau[:, cols]
            seen[:, cols] = np.maximum(seen[:, cols], np.abs(torch_quantise_rows(hp, B) - ref[:, cols]))
    for _ in range(200):
        hp = h + rng.uniform(-1, 1, h.shape) * tau
        seen = np.maximum(seen, np.abs(torch_quantise_rows(hp, B) - ref))
    assert (seen <= dev).all()
    assert (seen > 0).sum() >= 0.5 * (dev > 0).sum() and (dev > 0).any()


def pin_h_admissible_codes_closed_form(O):
    """Hand-worked cases of the admissible codes, block [448, 1.0625, 1.03,
    0.0052] with a band of 1e-9 (as the deviation pin): the exponent may be 0
    or 1, not 2. Under exponent 0: 448 only as 448, 1.0625 (a midpoint) as
    1.0 or 1.125 but not 1.25, 1.03 only as 1.0, 0.0052 only as 3 * 2^-9.
    Under exponent 1 (values halved): 224, 0.5 or 0.5625 (0.53125 is a
    midpoint), 0.5, 1 * 2^-9. A block of maximum 300 takes exponent 0 only.
    With no band only the oracle's own codes pass (the tie goes to 1.0)."""
    h = np.array([[448.0, 1.0625, 1.03, 0.0052, 300.0, 1.0625, 1.03, 0.0052]])
    tau = np.full(h.shape, 1e-9)

    def ok(vals, e0, e1, t=tau):
        codes = lib_round(np.array([vals], np.float64))
        return O.h_admissible_codes(h, t, codes, np.array([[e0, e1]]), 4)[0].tolist()

    assert ok([448, 1.0, 1.0, 3 * 2.0 ** -9, 300, 1.0, 1.0, 3 * 2.0 ** -9], 0, 0) == [True] * 8
    assert ok([448, 1.125, 1.125, 2 * 2.0 ** -9, 320, 1.125, 1.125, 2 * 2.0 ** -9], 0, 0) == \
        [True, True, False, False, False, True, False, False]
    assert ok([416, 1.25, 0.875, 4 * 2.0 ** -9, 300, 1.25, 0.875, 3 * 2.0 ** -9], 0, 0) == \
        [False, False, False, False, True, False, False, True]
    assert ok([224, 0.5, 0.5, 2.0 ** -9, 300, 1.0, 1.0, 3 * 2.0 ** -9], 1, 0) == [True] * 8
    assert ok([224, 0.5625, 0.5625, 2 * 2.0 ** -9, 150, 0.5, 0.5, 2.0 ** -9], 1, 1) == \
        [True, True, False, False, False, False, False, False]
    # exponent 2 is outside the band: not even values that round alike pass
    assert ok([112, 0.25, 0.25, 2.0 ** -9, 300, 1.0, 1.0, 3 * 2.0 ** -9], 2, 0) == \
        [False] * 4 + [True] * 4
    zero = np.zeros(h.shape)
    assert ok([448, 1.0, 1.0, 3 * 2.0 ** -9, 300, 1.0, 1.0, 3 * 2.0 ** -9], 0, 0, zero) == [True] * 8
    assert ok([448, 1.125, 1.0, 3 * 2.0 ** -9, 300, 1.125, 1.0, 3 * 2.0 ** -9], 0, 0, zero) == \
        [True, False, True, True, True, False, True, True]
    assert ok([224, 0.5, 0.5, 2.0 ** -9, 300, 1.0, 1.0, 3 * 2.0 ** -9], 1, 0, zero)[:4] == [False] * 4
    # the sign is part of the value; -0 and +0 are one value
    neg = -h
    codes = lib_round(-np.array([[448, 1.0, 1.0, 3 * 2.0 ** -9, 300, 1.125, 1.0, 3 * 2.0 ** -9]]))
    assert O.h_admissible_codes(neg, tau, codes, np.array([[0, 0]]), 4).all()
    assert not O.h_admissible_codes(neg, tau, lib_round(np.abs(lib_decode(codes))),
                                    np.array([[0, 0]]), 4).any()
    tiny = np.array([[448.0, 2.0 ** -11, -2.0 ** -11, 0.0]])
    z = lib_round(np.array([[448.0, 0.0, -0.0, -0.0]]))
    assert O.h_admissible_codes(tiny, np.zeros(tiny.shape), z, np.array([[0]]), 4).all()


def pin_h_admissible_codes_bruteforce(O):
    """Against brute force: the codes and exponents reached by quantising
    (the library's cast, the exponent by counting up from each block's own
    maximum) points of the band, its corners and a dense sweep of each
    element at every exponent the band allows, are admissible; and at a
    fixed exponent every admissible value of an element is reached by the
    sweep (so the check is exact, not merely permissive). h sits on code
    midpoints and block maxima on exponent boundaries."""
    rng = np.random.default_rng(24)
    B, n, I = 4, 5, 8
    mags = lib_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2
    e = rng.integers(-3, 3, (n, I // B))
    h = rng.choice(mids[8:], (n, I)) * np.repeat(np.ldexp(1.0, e), B, axis=1)
    h[:, ::B] = np.ldexp(448.0, e)
    h *= rng.choice([-1.0, 1.0], h.shape)
    tau = np.abs(h) * 10.0 ** rng.uniform(-3, -1.3, h.shape)

    def quantise(hp):  # codes and exponents by counting up (independent of the oracle)
        codes = np.empty(hp.shape, np.uint8)
        ex = np.empty((hp.shape[0], hp.shape[1] // B), np.int64)
        for t in range(hp.shape[0]):
            for b in range(hp.shape[1] // B):
                blk = hp[t, b * B:(b + 1) * B]
                ex[t, b] = scalar_exponent(float(np.abs(blk).max()))
                codes[t, b * B:(b + 1) * B] = lib_round(blk * 2.0 ** -ex[t, b])
        return codes, ex

    for signs in itertools.product((-1.0, 1.0), repeat=B):
        hp = h + np.tile(np.array(signs), I // B) * tau
        assert O.h_admissible_codes(h, tau, *quantise(hp), B).all()
    for _ in range(100):
        hp = h + rng.uniform(-1, 1, h.shape) * tau
        assert O.h_admissible_codes(h, tau, *quantise(hp), B).all()
    # per element and exponent: the swept values are exactly the admissible ones
    sweep = np.linspace(-1.0, 1.0, 4001)
    for t in range(n):
        for b in range(I // B):
            blk = np.abs(h[t, b * B:(b + 1) * B])
            lo = scalar_exponent(float(np.maximum(blk - tau[t, b * B:(b + 1) * B], 0).max()))
            hi = scalar_exponent(float((blk + tau[t, b * B:(b + 1) * B]).max()))
            for ex in range(lo, hi + 1):
                for c in range(b * B, (b + 1) * B):
                    vals = h[t, c] + sweep * tau[t, c]
                    vals = np.clip(vals * 2.0 ** -ex, -448, 448)
                    reached = set(lib_decode(lib_round(vals)).tolist())
                    cand = np.arange(256, dtype=np.uint8)
                    cand = cand[(cand & 0x7F) != 0x7F]
                    hh = np.repeat(h[t:t + 1, b * B:(b + 1) * B], len(cand), axis=0)
                    tt = np.repeat(tau[t:t + 1, b * B:(b + 1) * B], len(cand), axis=0)
                    cc = np.tile(lib_round(hh[:1] * 2.0 ** -ex), (len(cand), 1))
                    cc[:, c - b * B] = cand
                    okc = O.h_admissible_codes(hh, tt, cc, np.full((len(cand), 1), ex), B)
                    adm = set(lib_decode(cand[okc[:, c - b * B]]).tolist())
                    assert adm == reached, (t, c, ex, sorted(adm), sorted(reached))
            # exponents outside the band's range are refused
            cc = lib_round(h[t:t + 1, b * B:(b + 1) * B] * 2.0 ** -(hi + 1))
            assert not O.h_admissible_codes(h[t:t + 1, b * B:(b + 1) * B],
                                            tau[t:t + 1, b * B:(b + 1) * B], cc,
                                            np.array([[hi + 1]]), B).any()


def pin_h_band_covers_fp32(O):
    """The band holds an fp32 evaluation of h: sums of 64 exact products
    rounded to fp32 and accumulated in fp32, then silu and the product in
    fp32 (numpy float32), against the fp64 value; with the band's
    accumulation term scaled as for those sums (2 (K/64 + K/128 + 2) 2^-24)."""
    rng = np.random.default_rng(22)
    n, K, I = 24, 512, 64
    xs = rng.normal(0, 1, (n, K))
    wg = rng.normal(0, 0.05, (I, K))
    wu = rng.normal(0, 0.05, (I, K))
    wu[:, : K // 2] *= 4.0

    def sum32(w):
        acc = np.zeros((n, I), np.float32)
        for c in range(0, K, 64):
            acc = acc + (xs[:, c:c + 64] @ w[:, c:c + 64].T).astype(np.float32)
        return acc

    a32, u32 = sum32(wg), sum32(wu)
    h32 = (a32 / (np.float32(1) + np.exp(-a32))) * u32
    a, u = xs @ wg.T, xs @ wu.T
    h = a / (1 + np.exp(-a)) * u
    tau = O.h_band_width(xs, wg, wu, 2 * (K / 64 + K / 128 + 2) * 2.0 ** -24, 4 * 2.0 ** -24)
    assert (np.abs(h32.astype(np.float64) - h) <= tau).all()
    assert (tau <= 1e-3 * np.abs(h).max()).all()  # and it is a narrow band


def pin_layer_flip_bound(O):
    """The layer's flip bound is sound: perturbing each expert's h anywhere in
    its band (fp32-rounded h, then re-quantised by the library's cast) moves
    the torch evaluation of the layer by no more than "flip"; and with a band
    of zero the bound vanishes."""
    rng = np.random.default_rng(23)
    H, I, B, E, k, T = 64, 32, 32, 4, 2, 5
    experts = [random_expert(rng, H, I, B) for _ in range(E)]
    shared = random_expert(rng, H, I, B)
    x = rng.normal(0, 1, (T, H))
    wr = rng.normal(0, 0.3, (E, H))
    band = (3e-3, 1e-3)
    res = O.moe_layer(x, wr, None, lambda e: experts[e], k, I, B, shared=shared, act_block=B,
                      h_band=band)
    zero = O.moe_layer(x, wr, None, lambda e: experts[e], k, I, B, shared=shared, act_block=B,
                       h_band=(0.0, 0.0))
    assert not zero["flip"].any() and np.array_equal(zero["out"], res["out"])
    xh = torch_quantise_rows(x, B)
    logits = torch.from_numpy(x) @ torch.from_numpy(wr).T
    top = torch.topk(logits, k, dim=1).indices.numpy()

    def h_tau_wd(ex, rows):
        wgu = lib_dequant(ex["w_gate_up"], ex["s_gate_up"], B)
        wd = lib_dequant(ex["w_down"], ex["s_down"], B)
        xt = torch.from_numpy(rows)
        h = (torch.nn.functional.silu(xt @ torch.from_numpy(wgu[:I]).T) *
             (xt @ torch.from_numpy(wgu[I:]).T)).float().double().numpy()
        a, u = rows @ wgu[:I].T, rows @ wgu[I:].T
        sa, su = np.abs(rows) @ np.abs(wgu[:I]).T, np.abs(rows) @ np.abs(wgu[I:]).T
        sig = 1 / (1 + np.exp(-a))
        tau = band[0] * (np.abs(sig * (1 + a * (1 - sig)) * u) * sa + np.abs(a * sig) * su) + \
            band[1] * (8 + np.abs(a)) * np.abs(a * sig * u)
        return h, tau, wd

    def perturbed(ex, rows, signs):
        h, tau, wd = h_tau_wd(ex, rows)
        return torch_quantise_rows(h + signs * tau, B) @ wd.T

    def bound(ex, rows):  # the deviation (pinned above) through |Wd|
        h, tau, wd = h_tau_wd(ex, rows)
        return O.h_admissible_deviation(h, tau, B) @ np.abs(wd).T

    want_flip = np.zeros((T, H))
    for t in range(T):
        g = torch.softmax(logits[t, top[t]], 0).numpy()
        want_flip[t] = bound(shared, xh[t:t + 1])[0] + sum(
            g[j] * bound(experts[top[t, j]], xh[t:t + 1])[0] for j in range(k))
    assert np.allclose(res["flip"], want_flip, rtol=1e-9, atol=1e-15)
    worst = 0.0
    for trial in range(40):
        want = np.zeros((T, H))
        for t in range(T):
            g = torch.softmax(logits[t, top[t]], 0).numpy()
            want[t] += perturbed(shared, xh[t:t + 1], rng.uniform(-1, 1, (1, I)) if trial else 0)[0]
            for j in range(k):
                s = rng.choice([-1.0, 1.0], (1, I)) if trial % 2 else rng.uniform(-1, 1, (1, I))
                want[t] += g[j] * perturbed(experts[top[t, j]], xh[t:t + 1], s if trial else 0)[0]
        dev = np.abs(want - res["out"])
        if trial == 0:
            assert np.allclose(want, res["out"], rtol=1e-9, atol=1e-12)
        assert (dev <= res["flip"] * (1 + 1e-9) + 1e-12).all()
        worst = max(worst, float((dev / np.maximum(res["flip"], 1e-300)).max()))
    assert worst > 0.05  # the bound is reached in part, not vacuous


def pin_layer_on_given_h_codes(O):
    """With h_codes the layer's down contraction reads the given codes: a
    torch evaluation of the layer on the same codes (routing and gates by
    torch, x quantised by the library's cast, h codes decoded by the
    library) matches; codes that are the quantisation of a point inside the
    band count as admissible, with their flips counted; a code off by a
    factor of two (the largest element's, halved) counts as inadmissible; the
    shared expert's codes are asked for with expert None."""
    rng = np.random.default_rng(25)
    H, I, B, E, k, T = 64, 32, 32, 4, 2, 6
    experts = [random_expert(rng, H, I, B) for _ in range(E)]
    shared = random_expert(rng, H, I, B)
    x = rng.normal(0, 1, (T, H))
    wr = rng.normal(0, 0.3, (E, H))
    band = (3e-3, 1e-3)
    xh = torch_quantise_rows(x, B)

    def h_of(ex, rows):
        wgu = lib_dequant(ex["w_gate_up"], ex["s_gate_up"], B)
        a = torch.from_numpy(xh[rows]) @ torch.from_numpy(wgu[:I]).T
        u = torch.from_numpy(xh[rows]) @ torch.from_numpy(wgu[I:]).T
        return (torch.nn.functional.silu(a) * u).numpy().astype(np.float32).astype(np.float64)

    def codes_of(hp):
        codes = np.empty(hp.shape, np.uint8)
        ex = np.empty((hp.shape[0], hp.shape[1] // B), np.int64)
        for t in range(hp.shape[0]):
            for b in range(hp.shape[1] // B):
                blk = hp[t, b * B:(b + 1) * B]
                ex[t, b] = scalar_exponent(float(np.abs(blk).max()))
                codes[t, b * B:(b + 1) * B] = lib_round(blk * 2.0 ** -ex[t, b])
        return codes, ex

    asked = []
    given = {}

    def h_codes_for(perturb, spoil):
        def cb(e, toks, js):
            ex = shared if e is None else experts[e]
            asked.append(e)
            h = h_of(ex, toks)
            wgu = lib_dequant(ex["w_gate_up"], ex["s_gate_up"], B)
            tau = O.h_band_width(xh[toks], wgu[:I], wgu[I:], *band)
            c, exps = codes_of(h + perturb * rng.uniform(-1, 1, h.shape) * tau)
            if spoil and e is not None:
                big = np.unravel_index(np.argmax(np.abs(h)), h.shape)
                c[big] = lib_round(0.5 * lib_decode(c[big[0]:big[0] + 1, big[1]:big[1] + 1]))[0, 0]
            given[(e, tuple(toks), None if js is None else tuple(js))] = (c, exps)
            return c, exps
        return cb

    for perturb, spoil in ((0.0, False), (1.0, False), (0.0, True)):
        asked.clear()
        given.clear()
        res = O.moe_layer(x, wr, None, lambda e: experts[e], k, I, B, shared=shared,
                          act_block=B, h_band=band, h_codes=h_codes_for(perturb, spoil))
        assert None in asked and "flip" not in res
        chk = res["h_check"]
        assert chk["elements"] == (T * k + T) * I
        if spoil:
            assert chk["inadmissible"] >= 1
        else:
            assert chk["inadmissible"] == 0
        if perturb == 0.0 and not spoil:
            assert chk["flips"] == 0
        logits = torch.from_numpy(x) @ torch.from_numpy(wr).T
        top = torch.topk(logits, k, dim=1).indices.numpy()
        want = np.zeros((T, H))
        for (e, toks, js), (c, exps) in given.items():
            ex = shared if e is None else experts[e]
            wd = lib_dequant(ex["w_down"], ex["s_down"], B)
            hq = lib_decode(c) * np.repeat(np.ldexp(1.0, exps), B, axis=1)
            y = (torch.from_numpy(hq) @ torch.from_numpy(wd).T).numpy()
            for r, t in enumerate(toks):
                if e is None:
                    want[t] += y[r]
                else:
                    j = js[r]
                    assert top[t, j] == e
                    g = torch.softmax(logits[t, top[t]], 0).numpy()
                    want[t] += g[j] * y[r]
        assert np.allclose(res["out"], want, rtol=1e-9, atol=1e-12)


PINS = [pin_decode_matches_library, pin_decode_anchors, pin_dequant_bruteforce,
        pin_topk_bruteforce, pin_gates, pin_permutation, pin_single_expert_is_dense,
        pin_all_experts_equal_gates_is_dense_mean, pin_whole_layer_scalar, pin_tie_flags,
        pin_act_round_matches_library, pin_act_scale_closed_form,
        pin_act_quantise_blocks_bruteforce, pin_act_layer_uses_quantised_experts_only,
        pin_h_decided_in_fp32, pin_h_deviation_closed_form, pin_h_deviation_bruteforce,
        pin_h_band_covers_fp32, pin_layer_flip_bound, pin_h_admissible_codes_closed_form,
        pin_h_admissible_codes_bruteforce, pin_layer_on_given_h_codes]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(ORACLE)


# ------------------------------------------------------------- mutations ---
# Plausible mistakes, each planted in a fresh copy of the oracle's source.
MUTATIONS = {
    "exponent_bias_8": ("(e - 7).astype", "(e - 8).astype"),
    "subnormal_scale": ("m * 2.0 ** -9", "m * 2.0 ** -10"),
    "sign_dropped": ("np.where(s == 1, -mag, mag)", "mag"),
    "gate_up_swapped": ("return wgu[:inter], wgu[inter:], wd", "return wgu[inter:], wgu[:inter], wd"),
    "scale_grid_transposed": ("s_full = np.repeat(np.repeat(s, block, axis=0), block, axis=1)",
                              "s_full = np.repeat(np.repeat(s.T, block, axis=0), block, axis=1)"),
    "bias_dropped": ("l = l + np.asarray(router_bias, np.float64)[None, :]", "l = l"),
    "ties_to_higher_index": ('order = np.argsort(-logits[t], kind="stable")',
                             'order = (len(logits[t]) - 1 - np.argsort(-logits[t][::-1], kind="stable"))'),
    "gates_not_renormalised": ("g[t] = sel / sel.sum()", "g[t] = sel"),
    "silu_sign": ("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
    "down_not_transposed": ("    return h @ wd.T", "    return h @ wd.T[::-1]"),
    "shared_dropped": ("        out += y\n", "        pass\n"),
    "permutation_ties_by_descending_slot": ('order = np.argsort(flat, kind="stable")',
                                            "order = np.lexsort((-np.arange(flat.size), flat))"),
    "tie_band_relative": ("return (srt[:, k - 1] - srt[:, k]) < band",
                          "return (srt[:, k - 1] - srt[:, k]) < band * np.abs(srt[:, k - 1])"),
    "act_ties_to_odd": ("((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
    "act_scale_one_too_large": ("e[nz] = np.maximum(est, -127)",
                                "e[nz] = np.maximum(est + 1, -127)"),
    "act_scale_floor_clamp": ("e[nz] = np.maximum(est, -127)", "e[nz] = np.maximum(est, -126)"),
    "act_sign_dropped": ("return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)",
                         "return code"),
    "experts_read_unquantised_x": ("y = expert_out(xe[rows[who]], wg, wu, wd, codes)",
                                   "y = expert_out(x[rows[who]], wg, wu, wd, codes)"),
    "h_not_quantised": ("y = dequantise_activations(*quantise_activations(h, h_block), h_block) @ wd.T",
                        "y = h @ wd.T"),
    "h_decided_in_fp64": ("    h = h.astype(np.float32).astype(np.float64)\n", ""),
    "flip_ignores_exponent_ambiguity": ("lo, hi = np.minimum(e_lo, e_hi), np.maximum(e_lo, e_hi)",
                                        "lo, hi = e, e"),
    "flip_one_sided": ("for side in (-1.0, 0.0, 1.0):", "for side in (0.0, 1.0):"),
    "band_drops_u_error": ("np.abs(dsilu * u) * sa + np.abs(a * sig) * su", "np.abs(dsilu * u) * sa"),
    "band_drops_a_error": ("np.abs(dsilu * u) * sa + np.abs(a * sig) * su", "np.abs(a * sig) * su"),
    "flip_gate_dropped": ("flip[i] += gates[rows[i], j] * bound[r]", "flip[i] += bound[r]"),
    "flip_shared_dropped": ("            flip += bound\n", ""),
    "admissible_any_exponent": ("ok = ok_e[:, :, None] & (v >= lo) & (v <= hi)",
                                "ok = (v >= lo) & (v <= hi)"),
    "admissible_one_sided": ("hi = e4m3fn_decode(e4m3fn_round(np.clip((hb + tb) * down",
                             "hi = e4m3fn_decode(e4m3fn_round(np.clip((hb + 0 * tb) * down"),
    "admissible_exponent_range_too_narrow": (
        "e_hi = act_scale_exponent((np.abs(hb) + tb).max(axis=2))\n    ok_e",
        "e_hi = act_scale_exponent(np.abs(hb).max(axis=2))\n    ok_e"),
    "given_codes_ignored": ("        return hq @ wd.T\n", "        return own @ wd.T\n"),
    "given_codes_unchecked": ('        check["inadmissible"] += int((~ok).sum())\n', ""),
}


def load_mutant(name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation {name}: anchor text not found exactly once"
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name):
    mod = load_mutant(name, *MUTATIONS[name])
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:  # AssertionError, shape errors, ...
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
