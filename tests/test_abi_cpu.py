"""The C ABI on the host (no GPU): the library loads, exports every function
include/moe_fp8.h declares, and rejects invalid calls with the documented
status before any HIP call is made (the pointers passed here are never
dereferenced, because validation fails first)."""
import ctypes
import os
import re

import pytest

import block_fp8_routed_amd as moe
from block_fp8_routed_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp8.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails before use


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(_lib.EXPORTS) <= set(names), names
    assert {"moe_forward", "moe_route", "moe_permute", "moe_workspace_bytes"} <= set(names)


def test_library_exports_every_declared_symbol():
    lib = moe.load()
    for name in declared_functions():
        assert hasattr(lib, name), f"libmoe_fp8.so does not export {name}"


def test_status_strings_and_version():
    for st in range(7):
        s = moe.status_string(st)
        assert isinstance(s, str) and s
    assert moe.status_string(99) == "unknown status"
    assert moe.version() >= 100


def test_wait_limit_setter_is_host_only():
    """moe_set_wait_limit only records the bound (no device call, so it
    runs without a GPU); 0 restores the default."""
    lib = moe.load()
    assert lib.moe_set_wait_limit(7) == _lib.MOE_OK
    assert lib.moe_set_wait_limit(0) == _lib.MOE_OK
    moe.set_wait_limit(0)


def cfg(**kw):
    base = dict(tokens=4, hidden=64, experts=8, inter=32, top_k=2, block=32, has_shared=False,
                x_dtype=_lib.torch.float32, out_dtype=_lib.torch.float32, path="auto")
    base.update(kw)
    return moe.make_config(**base)


def bank(null=False):
    b = _lib.MoeExpertBank()
    if not null:
        b.w_gate_up = b.w_down = b.s_gate_up = b.s_down = 0x2000
    return b


def forward(c, x=FAKE, wr=FAKE, bias=None, b=None, sh=None, top_k=None, out=FAKE, ws=FAKE,
            ws_bytes=None, cfgp=True):
    lib = moe.load()
    b = bank() if b is None else b
    top_k = c.top_k if top_k is None else top_k
    ws_bytes = moe.workspace_bytes(c) if ws_bytes is None else ws_bytes
    return lib.moe_forward(x, wr, bias, ctypes.byref(b), ctypes.byref(sh) if sh else None, top_k,
                           out, ctypes.byref(c) if cfgp else None, ws, ws_bytes, None, None)


def test_workspace_bytes():
    c = cfg()
    n = moe.workspace_bytes(c)
    assert n > 0 and n % 256 == 0
    big = cfg(tokens=4096, hidden=4096, experts=512, inter=1024, top_k=10, block=128,
              has_shared=True)
    P = 4096 * 11
    assert moe.workspace_bytes(big) >= P * 4096 * 2 + P * 1024 * 2  # y and h fp16
    small = cfg(tokens=16, hidden=4096, experts=512, inter=1024, top_k=10, block=128,
                has_shared=True)
    assert moe.workspace_bytes(small) >= 16 * 11 * (4096 + 1024) * 4  # y and h fp32
    assert moe.workspace_bytes(cfg(top_k=9)) == 0  # invalid config


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=9), _lib.MOE_ERR_SHAPE),
    (dict(top_k=0), _lib.MOE_ERR_SHAPE),
    (dict(tokens=-1), _lib.MOE_ERR_SHAPE),
    (dict(hidden=0), _lib.MOE_ERR_SHAPE),
    (dict(hidden=48), _lib.MOE_ERR_SHAPE),          # block does not divide hidden
    (dict(inter=40), _lib.MOE_ERR_SHAPE),           # block does not divide inter
    (dict(experts=2048, top_k=2), _lib.MOE_ERR_UNSUPPORTED),
    (dict(experts=64, top_k=17), _lib.MOE_ERR_UNSUPPORTED),
    (dict(hidden=128, inter=64), _lib.MOE_ERR_UNSUPPORTED),  # no kernel for this shape
    (dict(path="mfma"), _lib.MOE_ERR_UNSUPPORTED),  # MFMA needs bf16 activations
    # the single-launch decode layer: at most 16 tokens, at most 512 experts
    (dict(path="gemv_fused", tokens=17), _lib.MOE_ERR_UNSUPPORTED),
    (dict(path="gemv_fused", experts=513, top_k=2), _lib.MOE_ERR_UNSUPPORTED),
])
def test_forward_rejects_bad_configs(kw, status):
    assert forward(cfg(**kw)) == status


def test_forward_rejects_bad_enums():
    c = cfg()
    c.x_dtype = 7
    assert forward(c) == _lib.MOE_ERR_SHAPE
    c = cfg()
    c.path = 5
    assert forward(c) == _lib.MOE_ERR_SHAPE
    c = cfg()
    c.path = -1
    assert forward(c) == _lib.MOE_ERR_SHAPE
    c = cfg()
    c.has_shared = 2
    assert forward(c) == _lib.MOE_ERR_SHAPE


def test_forward_rejects_null_pointers():
    c = cfg()
    assert forward(c, cfgp=False) == _lib.MOE_ERR_NULL
    assert forward(c, x=None) == _lib.MOE_ERR_NULL
    assert forward(c, wr=None) == _lib.MOE_ERR_NULL
    assert forward(c, out=None) == _lib.MOE_ERR_NULL
    assert forward(c, b=bank(null=True)) == _lib.MOE_ERR_NULL
    assert forward(c, ws=None) == _lib.MOE_ERR_NULL
    cs = cfg(has_shared=True)
    assert forward(cs) == _lib.MOE_ERR_NULL          # shared bank required
    assert forward(cs, sh=bank(null=True)) == _lib.MOE_ERR_NULL


def test_forward_rejects_top_k_mismatch_and_workspace():
    c = cfg()
    assert forward(c, top_k=3) == _lib.MOE_ERR_SHAPE
    n = moe.workspace_bytes(c)
    assert forward(c, ws_bytes=n - 1) == _lib.MOE_ERR_WORKSPACE
    assert forward(c, ws=ctypes.c_void_p(0x1004)) == _lib.MOE_ERR_WORKSPACE  # misaligned


def test_zero_tokens_is_a_no_op():
    assert forward(cfg(tokens=0), ws=None, ws_bytes=0) == _lib.MOE_OK


def test_route_and_permute_validation():
    lib = moe.load()
    c = cfg()
    n = moe.workspace_bytes(c)
    assert lib.moe_route(None, FAKE, None, FAKE, FAKE, None, ctypes.byref(c), FAKE, n,
                         None) == _lib.MOE_ERR_NULL
    assert lib.moe_route(FAKE, FAKE, None, FAKE, FAKE, None, ctypes.byref(c), FAKE, n - 1,
                         None) == _lib.MOE_ERR_WORKSPACE
    bad = cfg(top_k=9)
    assert lib.moe_route(FAKE, FAKE, None, FAKE, FAKE, None, ctypes.byref(bad), FAKE, n,
                         None) == _lib.MOE_ERR_SHAPE
    assert lib.moe_permute(FAKE, None, FAKE, FAKE, ctypes.byref(c), FAKE, n,
                           None) == _lib.MOE_ERR_NULL
    assert lib.moe_permute(FAKE, FAKE, FAKE, FAKE, ctypes.byref(c), FAKE, 8,
                           None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_permute(FAKE, FAKE, FAKE, FAKE, None, FAKE, n, None) == _lib.MOE_ERR_NULL


def test_quantize_act_validation():
    lib = moe.load()
    q = lib.moe_quantize_act_e4m3
    assert q(None, 4, 256, FAKE, FAKE, None) == _lib.MOE_ERR_NULL
    assert q(FAKE, 4, 256, None, FAKE, None) == _lib.MOE_ERR_NULL
    assert q(FAKE, -1, 256, FAKE, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert q(FAKE, 4, 0, FAKE, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert q(FAKE, 4, 200, FAKE, FAKE, None) == _lib.MOE_ERR_UNSUPPORTED
    assert q(FAKE, 0, 256, FAKE, FAKE, None) == _lib.MOE_OK  # nothing enqueued


def test_fp8_path_validation_and_workspace():
    """The FP8 variant: bf16 activations only; against the bf16 grouped path
    its workspace adds the activation codes (T*H bytes) and their exponents
    (T*H/128 bytes), and holds h as one-byte codes instead of fp16 (P*I bytes
    fewer); both keep exponent bytes for h and y, and the per-tile counters
    and status word of their one-launch passes."""
    bf16 = _lib.torch.bfloat16
    shape = dict(tokens=300, hidden=2048, experts=128, inter=768, top_k=8, block=128)
    f32 = cfg(path="mfma_fp8", **shape)
    assert forward(f32) == _lib.MOE_ERR_UNSUPPORTED  # fp32 activations
    plain = cfg(path="mfma", x_dtype=bf16, **shape)
    f8 = cfg(path="mfma_fp8", x_dtype=bf16, **shape)
    extra = moe.workspace_bytes(f8) - moe.workspace_bytes(plain)
    T, H, I = shape["tokens"], shape["hidden"], shape["inter"]
    P = T * shape["top_k"] + (T if f8.has_shared else 0)
    want = T * H + T * H // 128 - P * I
    assert want - 3 * 256 <= extra <= want + 3 * 256  # region alignment
    auto = cfg(path="auto", x_dtype=bf16, **shape)
    assert moe.workspace_bytes(auto) == moe.workspace_bytes(plain)  # AUTO never picks FP8
    assert forward(f8, ws_bytes=moe.workspace_bytes(f8) - 256) == _lib.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("path,tokens", [("gemv", 16), ("auto", 8), ("mfma", 300),
                                         ("mfma_fp8", 300), ("gemv_fused", 16)])
def test_workspace_regions(path, tokens):
    """moe_workspace_region: every exported region is 256-byte aligned, lies
    inside moe_workspace_bytes and overlaps no other, and has the size its
    declaration gives for the path's kernel family (h and y in fp32 on the
    GEMV family; fp16 or E4M3 bytes plus exponent bytes per 128 columns on
    the grouped families)."""
    bf16 = _lib.torch.bfloat16
    T, H, E, I, k = tokens, 4096, 512, 1024, 10
    c = cfg(tokens=T, hidden=H, experts=E, inter=I, top_k=k, block=128, has_shared=True,
            x_dtype=bf16, path=path)
    total = moe.workspace_bytes(c)
    P = T * (k + 1)
    grouped = path in ("mfma", "mfma_fp8")
    h_elem = (1 if path == "mfma_fp8" else 2) if grouped else 4
    want = {moe.MOE_WS_TOPK: T * k * 4, moe.MOE_WS_GATES: T * k * 4,
            moe.MOE_WS_OFFSETS: (E + 2) * 4, moe.MOE_WS_PAIR: P * 4, moe.MOE_WS_INV: P * 4,
            moe.MOE_WS_H: P * I * h_elem, moe.MOE_WS_H_EXPS: P * I // 128 if grouped else 0,
            moe.MOE_WS_Y: P * H * (2 if grouped else 4),
            moe.MOE_WS_Y_EXPS: P * H // 128 if grouped else 0,
            # the status word of the single-launch decode layer and of the
            # grouped paths (their gate/up and down passes share a launch)
            moe.MOE_WS_STATUS: 4 if path in ("gemv_fused", "mfma", "mfma_fp8") else 0}
    spans = []
    for region, n in want.items():
        off, got = moe.workspace_region(c, region)
        assert got == n, (region, got, n)
        assert off % 256 == 0 and off + got <= total
        spans.append((off, off + got))
    spans.sort()
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0, "regions overlap"
    lib = moe.load()
    o, n = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.moe_workspace_region(ctypes.byref(c), moe.MOE_WS_COUNT,
                                    ctypes.byref(o), ctypes.byref(n)) == _lib.MOE_ERR_SHAPE
    assert lib.moe_workspace_region(ctypes.byref(c), -1, ctypes.byref(o),
                                    ctypes.byref(n)) == _lib.MOE_ERR_SHAPE
    assert lib.moe_workspace_region(ctypes.byref(c), 0, None, ctypes.byref(n)) == _lib.MOE_ERR_NULL
    assert lib.moe_workspace_region(None, 0, ctypes.byref(o), ctypes.byref(n)) == _lib.MOE_ERR_NULL


def test_streamed_forward_validation():
    """moe_forward_streamed refuses a missing cache, an empty cache, cache
    arrays that are NULL, and slot contents that do not name distinct routed
    experts, before anything is enqueued."""
    import numpy as np
    lib = moe.load()
    c = cfg()
    hb, sb = bank(), bank()
    n = moe.workspace_bytes(c)

    def call(cache):
        return lib.moe_forward_streamed(FAKE, FAKE, None, ctypes.byref(hb), ctypes.byref(sb),
                                        ctypes.byref(cache.c) if cache is not None else None,
                                        None, c.top_k, FAKE, ctypes.byref(c), FAKE, n, None)

    assert call(None) == _lib.MOE_ERR_NULL
    empty = moe.ExpertCache(1)
    empty.c.slots = 0
    assert call(empty) == _lib.MOE_ERR_SHAPE
    nulls = moe.ExpertCache(2)
    nulls.c.slot_used = ctypes.POINTER(ctypes.c_int64)()
    assert call(nulls) == _lib.MOE_ERR_NULL
    for bad in ([3, 3], [8, -1], [-2, 0]):  # duplicate, past E = 8, not -1
        ch = moe.ExpertCache(2)
        ch.slot_expert[:] = np.array(bad, np.int32)
        assert call(ch) == _lib.MOE_ERR_SHAPE, bad
    ok = moe.ExpertCache(2)
    ok.slot_expert[:] = np.array([5, -1], np.int32)
    null_bank = bank(null=True)
    assert lib.moe_forward_streamed(FAKE, FAKE, None, ctypes.byref(null_bank), ctypes.byref(sb),
                                    ctypes.byref(ok.c), None, c.top_k, FAKE, ctypes.byref(c),
                                    FAKE, n, None) == _lib.MOE_ERR_NULL


def test_static_scratch_entry_refuses_oversized_calls():
    """moe_forward_static (scratch in the library's static device array)
    refuses a call whose workspace would exceed MOE_STATIC_SCRATCH_BYTES with
    MOE_ERR_TOO_LARGE before touching the device, and a NULL config with
    MOE_ERR_NULL."""
    lib = moe.load()
    big = cfg(tokens=4096, hidden=4096, experts=512, inter=1024, top_k=10, block=128,
              has_shared=True, x_dtype=_lib.torch.bfloat16)
    assert moe.workspace_bytes(big) > moe.MOE_STATIC_SCRATCH_BYTES
    b = bank()
    assert lib.moe_forward_static(FAKE, FAKE, None, ctypes.byref(b), ctypes.byref(b), big.top_k,
                                  FAKE, ctypes.byref(big), None, None) == moe.MOE_ERR_TOO_LARGE
    assert lib.moe_forward_static(FAKE, FAKE, None, ctypes.byref(b), None, 2, FAKE, None, None,
                                  None) == _lib.MOE_ERR_NULL
    assert moe.status_string(moe.MOE_ERR_TOO_LARGE) != "unknown status"


@pytest.mark.parametrize("tokens,x_dtype,grouped", [(16, "bf16", False), (48, "bf16", False),
                                                    (49, "bf16", True), (4096, "bf16", True),
                                                    (4096, "f32", False)])
def test_auto_family_choice(tokens, x_dtype, grouped):
    """AUTO takes the wavefront GEMV family up to 48 tokens (bf16 x) or for
    fp32 x at any size, and the grouped bf16 MFMA family otherwise; the
    grouped families keep exponent bytes for h, which the layout shows."""
    xdt = _lib.torch.bfloat16 if x_dtype == "bf16" else _lib.torch.float32
    c = cfg(tokens=tokens, hidden=2048, experts=128, inter=768, top_k=8, block=128,
            x_dtype=xdt, path="auto")
    _, hexp_bytes = moe.workspace_region(c, moe.MOE_WS_H_EXPS)
    assert (hexp_bytes > 0) == grouped
