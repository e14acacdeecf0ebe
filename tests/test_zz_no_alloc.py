"""moe_forward_static, the entry point that allocates nothing (its scratch is
a static device array inside the library): through the C ABI, on two calls in
a row (the second with a smaller input), its outputs equal moe_forward's with
a caller workspace bit for bit, on the decode (GEMV) and grouped (MFMA)
families and the single-launch decode layer (whose flags, in the static
array, must be left cleared by each call); a call too large for the array is
refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from parity import DevLayer, log

pytestmark = pytest.mark.gpu


def _static(layer, path):
    import block_fp8_routed_amd as moe
    return moe.moe_forward_static(layer.x, layer.router_w, layer.bank, layer.shape.top_k,
                                  layer.shape.block, shared=layer.shared,
                                  router_bias=layer.bias, path=path)


@pytest.mark.parametrize("name,tokens,path", [("c1", (16, 3), "auto"), ("c3", (8, 2), "auto"),
                                              ("c2", (512, 100), "mfma"),
                                              ("c2", (300, 40), "mfma_fp8"),
                                              ("c1", (16, 1), "gemv_fused")])
def test_static_scratch_matches_workspace_path(name, tokens, path):
    import block_fp8_routed_amd as moe
    moe.load()
    for i, T in enumerate(tokens):
        layer = DevLayer(W.CONFIGS[name], tokens=T, batch=i)
        want = layer.forward(path=path)
        got = _static(layer, path)
        torch.cuda.synchronize()
        log(f"static scratch {name} T={T} {path}: call {i + 1}")
        assert torch.equal(got, want), f"{name} T={T}: outputs differ"


def test_static_scratch_refuses_oversized_calls():
    import block_fp8_routed_amd as moe
    lib = moe.load()
    shape = W.CONFIGS["c4"]
    cfg = moe.make_config(shape.tokens, shape.hidden, shape.experts, shape.inter, shape.top_k,
                          shape.block, shape.shared, torch.bfloat16, torch.float32, "auto")
    assert moe.workspace_bytes(cfg) > moe.MOE_STATIC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the size check comes first
    bank = moe.MoeExpertBank(0x2000, 0x2000, 0x2000, 0x2000)
    st = lib.moe_forward_static(fake, fake, None, ctypes.byref(bank), ctypes.byref(bank),
                                shape.top_k, fake, ctypes.byref(cfg), None, None)
    assert st == moe.MOE_ERR_TOO_LARGE
