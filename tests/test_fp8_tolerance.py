"""The FP8 variant's parity check can tell a correct kernel from plausible
mistakes (CPU only).

A numpy emulation of what the kernels compute stands in for the GPU: the
gate/up sums taken as fp32 accumulations of 64-product steps, silu and the
product in fp32, h quantised to E4M3 per row and 128 columns with torch's
float8 cast (the exponent found by counting up), the down product and the
combine in fp64. Like the GPU test, the check reads the emulated kernel's h
codes and exponents: each must be admissible under reading R11 (the
oracle's h_admissible_codes, with the band of tests/parity.py), and the
outputs must match the oracle evaluated on those codes within the layer
tolerance. Evaluated correctly the emulation passes; with a mistake planted
in its quantisation of h (truncation instead of rounding, the sign dropped,
a block exponent one too large, blocks of 64 columns) its codes fail the
first part, and with one planted after it (the block scale not applied
back, h left unquantised in the down product) its outputs fail the second.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check_output, fp8_h_band

H, I, B, E, K, T = 256, 256, 128, 8, 2, 48
E4M3 = oracle.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448, increasing


def random_expert(rng):
    def codes(shape):
        c = rng.integers(0, 256, size=shape).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x7E
        return c
    return {"w_gate_up": codes((2 * I, H)),
            "s_gate_up": rng.uniform(1e-3, 1e-2, (2 * I // B, H // B)).astype(np.float32),
            "w_down": codes((H, I)),
            "s_down": rng.uniform(1e-3, 1e-2, (H // B, I // B)).astype(np.float32)}


def exponent(amax):
    if amax == 0.0:
        return 0
    e = -127
    while amax > np.ldexp(448.0, e):
        e += 1
    return e


def cast(v):
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def quantise_h(h, mistake):
    """codes [1][I], exponents [1][I/B] and the dequantised h the emulated
    down product reads."""
    codes = np.empty(h.shape, np.uint8)
    exps = np.empty((h.shape[0], h.shape[1] // B), np.int64)
    deq = np.empty(h.shape, np.float64)
    sub = 64 if mistake == "blocks_of_64" else B
    for r in range(h.shape[0]):
        for b0 in range(0, h.shape[1], sub):
            blk = h[r, b0:b0 + sub].astype(np.float64)
            e = exponent(float(np.abs(blk).max())) + (1 if mistake == "exponent_plus_one" else 0)
            v = blk * 2.0 ** -e
            if mistake == "truncate":
                mag = E4M3[np.searchsorted(E4M3, np.abs(v), side="right") - 1]
                c = cast(np.copysign(mag, v))
            else:
                c = cast(v)
            if mistake == "sign_dropped":
                c = c & 0x7F
            codes[r, b0:b0 + sub] = c
            exps[r, b0 // B] = e
            q = oracle.e4m3fn_decode(c)
            deq[r, b0:b0 + sub] = q * (1.0 if mistake == "scale_not_applied" else 2.0 ** e)
    return codes, exps, deq


def sum32(xs, w):
    acc = np.zeros((xs.shape[0], w.shape[0]), np.float32)
    for c in range(0, xs.shape[1], 64):
        acc = acc + (xs[:, c:c + 64] @ w[:, c:c + 64].T).astype(np.float32)
    return acc


def emulated_layer(x, experts, idx, gates, mistake):
    """Outputs and the h codes of every (token, slot) of an emulated kernel."""
    xh = oracle.dequantise_activations(*oracle.quantise_activations(x, B), B)
    out = np.zeros((T, H))
    codes = {}
    for t in range(T):
        for j in range(K):
            wg, wu, wd = oracle.expert_matrices(experts[idx[t, j]], I, B)
            a, u = sum32(xh[t:t + 1], wg), sum32(xh[t:t + 1], wu)
            h = (a / (np.float32(1) + np.exp(-a))) * u
            c, ex, hq = quantise_h(h, mistake)
            codes[(t, j)] = (c[0], ex[0])
            if mistake == "unquantised":
                hq = h.astype(np.float64)
            out[t] += gates[t, j] * (hq @ wd.T)[0]
    return out, codes


@pytest.fixture(scope="module")
def layer():
    rng = np.random.default_rng(31)
    experts = [random_expert(rng) for _ in range(E)]
    x = rng.normal(0, 1, (T, H)).astype(np.float32).astype(np.float64)
    wr = rng.normal(0, 0.1, (E, H))
    plain = oracle.moe_layer(x, wr, None, lambda e: experts[e], K, I, B, act_block=B)
    return x, wr, experts, plain


@pytest.mark.parametrize("mistake", [None, "truncate", "sign_dropped", "exponent_plus_one",
                                     "blocks_of_64", "scale_not_applied", "unquantised"])
def test_fp8_check_separates_mistakes(layer, mistake):
    x, wr, experts, plain = layer
    got, codes = emulated_layer(x, experts, plain["topk_idx"], plain["gates"], mistake)

    def h_codes(e, toks, js):
        c = np.stack([codes[(int(t), int(j))][0] for t, j in zip(toks, js)])
        ex = np.stack([codes[(int(t), int(j))][1] for t, j in zip(toks, js)])
        return c, ex

    ref = oracle.moe_layer(x, wr, None, lambda e: experts[e], K, I, B, act_block=B,
                           h_band=fp8_h_band(H), h_codes=h_codes)

    def run():
        assert ref["h_check"]["inadmissible"] == 0, "inadmissible h codes"
        check_output(torch.from_numpy(got), ref["out"], what=f"emulated {mistake}")

    if mistake is None:
        run()
        assert ref["h_check"]["flips"] < 0.01 * ref["h_check"]["elements"]
    else:
        with pytest.raises(AssertionError):
            run()
