"""The FP8 variant's output check can tell a correct kernel from plausible
mistakes (CPU only).

A numpy emulation of what the kernels compute stands in for the GPU: the
gate/up sums taken as fp32 accumulations of 64-product steps, silu and the
product in fp32, h quantised to E4M3 per row and 128 columns with torch's
float8 cast, the down product and the combine in fp64. Evaluated correctly
it must pass the FP8 parity check (layer tolerance plus the oracle's bound
for admissible h codes, reading R11); with a mistake planted in the
emulated quantisation of h (truncation instead of rounding, the sign
dropped, the block scale not applied back, no quantisation at all) it must
fail.

Some mistakes cannot be seen in the output at all, by any check: E4M3 is a
floating-point format, so choosing a block exponent one too large, or
blocks of 64 columns, changes only the values below 2^-6 of the block
scale (measured here: output changes of 1e-4 and 5e-5 x RMS). The oracle's
exponent rule is pinned on its own (tests/test_oracle_pins.py).
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


def quantise_h(h, mistake, block=B):
    out = np.empty(h.shape, np.float64)
    for r in range(h.shape[0]):
        for b0 in range(0, h.shape[1], block):
            blk = h[r, b0:b0 + block].astype(np.float64)
            e = exponent(float(np.abs(blk).max()))
            v = blk * 2.0 ** -e
            if mistake == "truncate":
                mag = E4M3[np.searchsorted(E4M3, np.abs(v), side="right") - 1]
                q = np.copysign(mag, v)
            else:
                q = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
            if mistake == "sign_dropped":
                q = np.abs(q)
            out[r, b0:b0 + block] = q * (1.0 if mistake == "scale_not_applied" else 2.0 ** e)
    return out


def sum32(xs, w):
    acc = np.zeros((xs.shape[0], w.shape[0]), np.float32)
    for c in range(0, xs.shape[1], 64):
        acc = acc + (xs[:, c:c + 64] @ w[:, c:c + 64].T).astype(np.float32)
    return acc


def emulated_layer(x, experts, idx, gates, mistake):
    xh = oracle.dequantise_activations(*oracle.quantise_activations(x, B), B)
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(K):
            wg, wu, wd = oracle.expert_matrices(experts[idx[t, j]], I, B)
            a, u = sum32(xh[t:t + 1], wg), sum32(xh[t:t + 1], wu)
            h = (a / (np.float32(1) + np.exp(-a))) * u
            if mistake == "unquantised":
                hq = h.astype(np.float64)
            else:
                hq = quantise_h(h, mistake)
            out[t] += gates[t, j] * (hq @ wd.T)[0]
    return out


@pytest.fixture(scope="module")
def layer():
    rng = np.random.default_rng(31)
    experts = [random_expert(rng) for _ in range(E)]
    x = rng.normal(0, 1, (T, H)).astype(np.float32).astype(np.float64)
    wr = rng.normal(0, 0.1, (E, H))
    ref = oracle.moe_layer(x, wr, None, lambda e: experts[e], K, I, B, act_block=B,
                           h_band=fp8_h_band(H))
    return x, experts, ref


@pytest.mark.parametrize("mistake", [None, "truncate", "sign_dropped", "scale_not_applied",
                                     "unquantised"])
def test_fp8_check_separates_mistakes(layer, mistake):
    x, experts, ref = layer
    got = emulated_layer(x, experts, ref["topk_idx"], ref["gates"], mistake)
    run = lambda: check_output(torch.from_numpy(got), ref["out"], what=f"emulated {mistake}",
                               flip=ref["flip"])
    if mistake is None:
        run()
    else:
        with pytest.raises(AssertionError):
            run()
