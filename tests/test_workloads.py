"""The seeded input generator: determinism, the quantiser's error bound and the
routing structure each workload is meant to have (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def lib_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_expert_streams_are_deterministic_and_independent():
    s = W.CONFIGS["c0"]
    a, b = W.gen_expert(s, 3), W.gen_expert(s, 3)
    for k in a:
        assert np.array_equal(a[k], b[k])
    c = W.gen_expert(s, 4)
    assert not np.array_equal(a["w_gate_up"], c["w_gate_up"])
    bank = W.gen_bank(s, threads=4)
    for e in range(s.experts):
        ex = W.gen_expert(s, e)
        for k in ex:
            assert np.array_equal(bank[k][e], ex[k])
    sh = W.gen_bank(s, shared=True)
    assert not np.array_equal(sh["w_gate_up"][0], bank["w_gate_up"][0])


def test_batch_prefixes_and_rotation():
    s = W.CONFIGS["c1"]
    x16 = W.gen_x(s)
    for T in (1, 4):
        assert np.array_equal(W.gen_x(s, tokens=T), x16[:T])
    assert not np.array_equal(W.gen_x(s, batch=1), x16)
    # bf16 layers: values are exactly bf16
    assert np.array_equal(W.round_to_bf16(x16), x16)


def test_quantiser_error_bound_and_range():
    s = W.CONFIGS["c0"]
    rng = np.random.default_rng(0)
    w = rng.normal(0, 0.02, (64, 96)).astype(np.float32)
    w[:32, :32] = 0.0  # an all-zero block gets scale 1
    q, sc = W.quantise_blocks(w, 32)
    assert q.dtype == np.uint8 and sc.shape == (2, 3)
    assert not np.any((q & 0x7F) == 0x7F), "NaN code emitted"
    assert sc[0, 0] == 1.0 and np.all(q[:32, :32] & 0x7F == 0)
    dec = lib_decode(q)
    for bi in range(2):
        for bj in range(3):
            blk = w[32 * bi:32 * bi + 32, 32 * bj:32 * bj + 32].astype(np.float64)
            if not blk.any():
                continue
            s_ = float(sc[bi, bj])
            assert s_ == np.float32(np.abs(blk).max() / np.float32(448.0))
            v = blk / s_
            d = dec[32 * bi:32 * bi + 32, 32 * bj:32 * bj + 32]
            assert np.abs(d).max() <= 448.0
            # half an ulp of E4M3: 2^-4 * 2^floor(log2|v|) for normals, 2^-10 below 2^-6
            ulp_half = np.where(np.abs(v) >= 2.0 ** -6,
                                2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 1e-30))) - 4),
                                2.0 ** -10)
            assert np.all(np.abs(d - v) <= ulp_half * (1 + 1e-6) + 1e-7)


def routing_counts(shape, tokens=None):
    x = W.gen_x(shape, tokens)
    logits = oracle.router_logits(x, W.gen_router(shape), W.gen_bias(shape))
    idx = oracle.select_topk(logits, shape.top_k)
    return np.bincount(idx.reshape(-1), minlength=shape.experts)


def test_c2_zipf_group_sizes():
    s = W.CONFIGS["c2"]
    b = W.gen_bias(s)
    assert sorted(np.round(np.exp(-b / (0.25 * 1.1))).astype(int)) == list(range(1, 129))
    n = routing_counts(s)
    assert n.sum() == 512 * 8
    assert 100 <= n.max() <= 200, n.max()


@pytest.mark.slow
def test_c4_skewed_structure():
    s = W.CONFIGS["c4"]
    b = W.gen_bias(s)
    assert int((b == 1.0).sum()) == 16
    n = routing_counts(s)
    T = s.tokens
    assert int((n > 0.2 * T).sum()) == 16, np.sort(n)[-20:]
    assert int((n == 0).sum()) > s.experts / 3


def test_uniform_decode_routing_spreads():
    s = W.CONFIGS["c1"]
    n = routing_counts(s)
    assert n.sum() == 128 and (n > 0).sum() >= 60
