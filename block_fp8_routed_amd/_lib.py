"""ctypes binding of libmoe_fp8.so (the C ABI in include/moe_fp8.h).

Argument marshalling only: torch tensors supply device pointers, the current
HIP stream and workspace memory; every step of the layer runs in the HIP
library. There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_fp8.so")

(MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
 MOE_ERR_TOO_LARGE) = range(7)
MOE_STATIC_SCRATCH_BYTES = 64 << 20
MOE_F32, MOE_BF16 = 0, 1
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_MFMA, MOE_PATH_MFMA_FP8, MOE_PATH_GEMV_FUSED = range(5)
PATHS = {"auto": MOE_PATH_AUTO, "gemv": MOE_PATH_GEMV, "mfma": MOE_PATH_MFMA,
         "mfma_fp8": MOE_PATH_MFMA_FP8, "gemv_fused": MOE_PATH_GEMV_FUSED}
(MOE_EV_START, MOE_EV_ROUTED, MOE_EV_PERMUTED, MOE_EV_GATE_UP, MOE_EV_DOWN,
 MOE_EV_END, MOE_EV_COUNT) = range(7)

EXPORTS = ("moe_workspace_bytes", "moe_forward", "moe_forward_static", "moe_forward_streamed", "moe_route",
           "moe_permute",
           "moe_dequant_e4m3", "moe_quantize_act_e4m3", "moe_workspace_region",
           "moe_status_string", "moe_version", "moe_set_wait_limit")
(MOE_WS_TOPK, MOE_WS_GATES, MOE_WS_OFFSETS, MOE_WS_PAIR, MOE_WS_INV, MOE_WS_H, MOE_WS_H_EXPS,
 MOE_WS_Y, MOE_WS_Y_EXPS, MOE_WS_STATUS, MOE_WS_COUNT) = range(11)


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int32),
        ("experts", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("has_shared", ctypes.c_int32),
        ("x_dtype", ctypes.c_int),
        ("out_dtype", ctypes.c_int),
        ("path", ctypes.c_int),
    ]


class MoeExpertBank(ctypes.Structure):
    _fields_ = [
        ("w_gate_up", ctypes.c_void_p),
        ("w_down", ctypes.c_void_p),
        ("s_gate_up", ctypes.c_void_p),
        ("s_down", ctypes.c_void_p),
    ]


class MoeExpertCache(ctypes.Structure):
    _fields_ = [
        ("slots", ctypes.c_int32),
        ("slot_expert", ctypes.POINTER(ctypes.c_int32)),
        ("slot_used", ctypes.POINTER(ctypes.c_int64)),
        ("calls", ctypes.c_int64),
        ("hits", ctypes.c_int64),
        ("misses", ctypes.c_int64),
        ("bytes_in", ctypes.c_int64),
        ("rounds_last", ctypes.c_int32),
    ]


class MoePhaseEvents(ctypes.Structure):
    _fields_ = [("ev", ctypes.c_void_p * MOE_EV_COUNT)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe_fp8.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m block_fp8_routed_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    cfgp = ctypes.POINTER(MoeConfig)
    bankp = ctypes.POINTER(MoeExpertBank)
    lib.moe_workspace_bytes.argtypes = [cfgp]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_forward.argtypes = [P, P, P, bankp, bankp, ctypes.c_int32, P, cfgp, P,
                                ctypes.c_size_t, ctypes.POINTER(MoePhaseEvents), P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_static.argtypes = [P, P, P, bankp, bankp, ctypes.c_int32, P, cfgp,
                                       ctypes.POINTER(MoePhaseEvents), P]
    lib.moe_forward_static.restype = ctypes.c_int
    lib.moe_forward_streamed.argtypes = [P, P, P, bankp, bankp, ctypes.POINTER(MoeExpertCache),
                                         bankp, ctypes.c_int32, P, cfgp, P, ctypes.c_size_t, P]
    lib.moe_forward_streamed.restype = ctypes.c_int
    lib.moe_route.argtypes = [P, P, P, P, P, P, cfgp, P, ctypes.c_size_t, P]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_permute.argtypes = [P, P, P, P, cfgp, P, ctypes.c_size_t, P]
    lib.moe_permute.restype = ctypes.c_int
    lib.moe_dequant_e4m3.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P]
    lib.moe_dequant_e4m3.restype = ctypes.c_int
    lib.moe_quantize_act_e4m3.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P, P]
    lib.moe_quantize_act_e4m3.restype = ctypes.c_int
    lib.moe_workspace_region.argtypes = [cfgp, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t),
                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_workspace_region.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_int32
    lib.moe_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.moe_set_wait_limit.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def version() -> int:
    return int(load().moe_version())


def set_wait_limit(polls: int) -> None:
    """moe_set_wait_limit: the poll bound of the one-launch grouped passes'
    waits (0: the default); for tests of their give-up path."""
    st = load().moe_set_wait_limit(int(polls))
    if st != 0:
        raise MoeError(st, "moe_set_wait_limit")


def make_config(tokens: int, hidden: int, experts: int, inter: int, top_k: int, block: int,
                has_shared: bool = False, x_dtype=torch.bfloat16, out_dtype=torch.float32,
                path: str = "auto") -> MoeConfig:
    def code(dt):
        if dt == torch.float32:
            return MOE_F32
        if dt == torch.bfloat16:
            return MOE_BF16
        raise ValueError(f"unsupported dtype {dt}")
    return MoeConfig(int(tokens), int(hidden), int(experts), int(inter), int(top_k),
                     int(block), int(bool(has_shared)), code(x_dtype), code(out_dtype),
                     PATHS[path])


def workspace_bytes(cfg: MoeConfig) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(cfg)))


def workspace_region(cfg: MoeConfig, region: int):
    """(offset, bytes) of one intermediate result in the workspace of `cfg`."""
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    st = load().moe_workspace_region(ctypes.byref(cfg), int(region), ctypes.byref(off),
                                     ctypes.byref(n))
    if st != MOE_OK:
        raise MoeError(st, "moe_workspace_region")
    return off.value, n.value


def workspace_view(workspace: torch.Tensor, cfg: MoeConfig, region: int,
                   dtype=torch.uint8) -> torch.Tensor:
    """A flat view of one region of a workspace tensor, as `dtype`."""
    off, n = workspace_region(cfg, region)
    return workspace[off:off + n].view(dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_workspace(cfg: MoeConfig, device) -> torch.Tensor:
    """A workspace tensor for `cfg` (torch's allocator returns 256-byte aligned memory)."""
    return torch.empty(max(1, workspace_bytes(cfg)), dtype=torch.uint8, device=device)


class Bank:
    """A block-FP8 expert bank: n experts, layout of moe_expert_bank; on the
    device, or (host=True) in pinned host memory for moe_forward_streamed."""

    def __init__(self, w_gate_up: torch.Tensor, s_gate_up: torch.Tensor,
                 w_down: torch.Tensor, s_down: torch.Tensor, host: bool = False):
        if host:
            for t in (w_gate_up, s_gate_up, w_down, s_down):
                if t.is_cuda or not t.is_pinned() or not t.is_contiguous():
                    raise ValueError("a host bank needs contiguous pinned CPU tensors")
        else:
            _dev(w_gate_up, s_gate_up, w_down, s_down)
        if w_gate_up.dtype != torch.uint8 or w_down.dtype != torch.uint8:
            raise ValueError("E4M3 weights must be uint8 tensors")
        if s_gate_up.dtype != torch.float32 or s_down.dtype != torch.float32:
            raise ValueError("block scales must be float32 tensors")
        self.w_gate_up, self.s_gate_up, self.w_down, self.s_down = (
            w_gate_up, s_gate_up, w_down, s_down)
        self.c = MoeExpertBank(w_gate_up.data_ptr(), w_down.data_ptr(),
                               s_gate_up.data_ptr(), s_down.data_ptr())

    @classmethod
    def from_numpy(cls, bank: dict, device="cuda"):
        t = {k: torch.from_numpy(v).to(device) for k, v in bank.items()}
        return cls(t["w_gate_up"], t["s_gate_up"], t["w_down"], t["s_down"])

    @classmethod
    def pinned_from_numpy(cls, bank: dict):
        """A host bank in newly allocated pinned memory."""
        t = {k: torch.from_numpy(v).pin_memory() for k, v in bank.items()}
        return cls(t["w_gate_up"], t["s_gate_up"], t["w_down"], t["s_down"], host=True)

    @classmethod
    def empty_slots(cls, slots: int, H: int, I: int, B: int, device="cuda"):
        """A device bank of `slots` expert slots (the streamed cache)."""
        return cls(torch.empty((slots, 2 * I, H), dtype=torch.uint8, device=device),
                   torch.empty((slots, 2 * I // B, H // B), dtype=torch.float32, device=device),
                   torch.empty((slots, H, I), dtype=torch.uint8, device=device),
                   torch.empty((slots, H // B, I // B), dtype=torch.float32, device=device))

    @property
    def experts(self) -> int:
        return self.w_gate_up.shape[0]

    def check(self, n: int, H: int, I: int, B: int):
        want = {"w_gate_up": (n, 2 * I, H), "w_down": (n, H, I),
                "s_gate_up": (n, 2 * I // B, H // B), "s_down": (n, H // B, I // B)}
        for k, shp in want.items():
            if tuple(getattr(self, k).shape) != shp:
                raise ValueError(f"bank.{k} has shape {tuple(getattr(self, k).shape)}, want {shp}")


def moe_forward(x: torch.Tensor, router_w: torch.Tensor, bank: Bank, top_k: int, block: int,
                shared: Optional[Bank] = None, router_bias: Optional[torch.Tensor] = None,
                out_dtype=torch.float32, path: str = "auto", out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, events=None, stream=None,
                cfg: Optional[MoeConfig] = None) -> torch.Tensor:
    """The whole layer through moe_forward. `events` is an optional list of
    MOE_EV_COUNT raw hipEvent_t handles (ints or None)."""
    lib = load()
    T, H = x.shape
    E = router_w.shape[0]
    I = bank.w_gate_up.shape[1] // 2
    if cfg is None:
        cfg = make_config(T, H, E, I, top_k, block, shared is not None, x.dtype, out_dtype, path)
    _dev(x, router_w, router_bias)
    if router_w.dtype != torch.float32 or (router_bias is not None and router_bias.dtype != torch.float32):
        raise ValueError("router weight and bias must be float32")
    bank.check(E, H, I, block)
    if shared is not None:
        shared.check(1, H, I, block)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = make_workspace(cfg, x.device)
    evs = None
    if events is not None:
        evs = MoePhaseEvents()
        for i, e in enumerate(events):
            evs.ev[i] = e if e else None
    st = lib.moe_forward(_ptr(x), _ptr(router_w), _ptr(router_bias), ctypes.byref(bank.c),
                         ctypes.byref(shared.c) if shared is not None else None, int(top_k),
                         _ptr(out), ctypes.byref(cfg), _ptr(workspace), workspace.numel(),
                         ctypes.byref(evs) if evs is not None else None, _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_forward")
    return out


class ExpertCache:
    """Host-side state of a streamed expert cache of `slots` slots
    (moe_expert_cache), with the counters moe_forward_streamed keeps."""

    def __init__(self, slots: int):
        import numpy as np
        self.slot_expert = np.full(slots, -1, np.int32)
        self.slot_used = np.zeros(slots, np.int64)
        self.c = MoeExpertCache(slots, self.slot_expert.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                self.slot_used.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                0, 0, 0, 0, 0)

    def __getattr__(self, name):
        if name in ("slots", "calls", "hits", "misses", "bytes_in", "rounds_last"):
            return getattr(self.c, name)
        raise AttributeError(name)


def moe_forward_streamed(x: torch.Tensor, router_w: torch.Tensor, host_bank: Bank,
                         slot_bank: Bank, cache: ExpertCache, top_k: int, block: int,
                         shared: Optional[Bank] = None, router_bias: Optional[torch.Tensor] = None,
                         out_dtype=torch.float32, path: str = "auto",
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The whole layer through moe_forward_streamed: routed experts in pinned
    host memory (host_bank), streamed into the device slots of slot_bank."""
    lib = load()
    T, H = x.shape
    E = router_w.shape[0]
    I = host_bank.w_gate_up.shape[1] // 2
    cfg = make_config(T, H, E, I, top_k, block, shared is not None, x.dtype, out_dtype, path)
    _dev(x, router_w, router_bias)
    host_bank.check(E, H, I, block)
    slot_bank.check(cache.slots, H, I, block)
    if shared is not None:
        shared.check(1, H, I, block)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = make_workspace(cfg, x.device)
    st = lib.moe_forward_streamed(_ptr(x), _ptr(router_w), _ptr(router_bias),
                                  ctypes.byref(host_bank.c), ctypes.byref(slot_bank.c),
                                  ctypes.byref(cache.c),
                                  ctypes.byref(shared.c) if shared is not None else None,
                                  int(top_k), _ptr(out), ctypes.byref(cfg), _ptr(workspace),
                                  workspace.numel(), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_forward_streamed")
    return out


def moe_forward_static(x: torch.Tensor, router_w: torch.Tensor, bank: Bank, top_k: int,
                       block: int, shared: Optional[Bank] = None,
                       router_bias: Optional[torch.Tensor] = None, out_dtype=torch.float32,
                       path: str = "auto", out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """The whole layer through moe_forward_static (scratch in the library's
    static device array: no workspace is allocated). `out` may be given to
    avoid torch's own allocation of the result."""
    lib = load()
    T, H = x.shape
    E = router_w.shape[0]
    I = bank.w_gate_up.shape[1] // 2
    cfg = make_config(T, H, E, I, top_k, block, shared is not None, x.dtype, out_dtype, path)
    _dev(x, router_w, router_bias)
    bank.check(E, H, I, block)
    if shared is not None:
        shared.check(1, H, I, block)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    st = lib.moe_forward_static(_ptr(x), _ptr(router_w), _ptr(router_bias), ctypes.byref(bank.c),
                                ctypes.byref(shared.c) if shared is not None else None,
                                int(top_k), _ptr(out), ctypes.byref(cfg), None, _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_forward_static")
    return out


def moe_route(x: torch.Tensor, router_w: torch.Tensor, top_k: int, inter: int, block: int,
              router_bias: Optional[torch.Tensor] = None, with_logits: bool = False,
              workspace: Optional[torch.Tensor] = None, stream=None):
    """Router + top-k + gates through moe_route: (topk_idx, gates[, logits])."""
    lib = load()
    T, H = x.shape
    E = router_w.shape[0]
    cfg = make_config(T, H, E, inter, top_k, block, False, x.dtype, torch.float32)
    _dev(x, router_w, router_bias)
    idx = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
    gates = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if with_logits else None
    if workspace is None:
        workspace = make_workspace(cfg, x.device)
    st = lib.moe_route(_ptr(x), _ptr(router_w), _ptr(router_bias), _ptr(idx), _ptr(gates),
                       _ptr(logits), ctypes.byref(cfg), _ptr(workspace), workspace.numel(),
                       _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_route")
    return (idx, gates, logits) if with_logits else (idx, gates)


def moe_permute(topk_idx: torch.Tensor, experts: int, has_shared: bool, hidden: int,
                inter: int, block: int, workspace: Optional[torch.Tensor] = None, stream=None):
    """Token->expert permutation through moe_permute: (offsets, pair, inv)."""
    lib = load()
    T, k = topk_idx.shape
    _dev(topk_idx)
    if topk_idx.dtype != torch.int32:
        raise ValueError("topk_idx must be int32")
    cfg = make_config(T, hidden, experts, inter, k, block, has_shared)
    P = T * k + (T if has_shared else 0)
    dev = topk_idx.device
    offsets = torch.empty(experts + 2, dtype=torch.int32, device=dev)
    pair = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = make_workspace(cfg, dev)
    st = lib.moe_permute(_ptr(topk_idx), _ptr(offsets), _ptr(pair), _ptr(inv), ctypes.byref(cfg),
                         _ptr(workspace), workspace.numel(), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_permute")
    return offsets, pair[:P], inv[:P]


def moe_quantize_act_e4m3(x: torch.Tensor, stream=None):
    """bf16 activations [T][H] -> (E4M3 codes [T][H] uint8, E8M0 exponents
    [T][H/128] uint8, e + 127), one power-of-two scale per token and block of
    128 columns."""
    lib = load()
    _dev(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bf16 tensor")
    x = x.contiguous()
    T, H = x.shape
    codes = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    exps = torch.empty((T, max(H // 128, 1)), dtype=torch.uint8, device=x.device)
    st = lib.moe_quantize_act_e4m3(_ptr(x), T, H, _ptr(codes), _ptr(exps), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_quantize_act_e4m3")
    return codes, exps


def moe_dequant_e4m3(w: torch.Tensor, scales: torch.Tensor, block: int,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Expand a block-FP8 matrix [rows][cols] (uint8) with fp32 block scales to fp32."""
    lib = load()
    _dev(w, scales, out)
    rows, cols = w.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=w.device)
    st = lib.moe_dequant_e4m3(_ptr(w), _ptr(scales), rows, cols, int(block), _ptr(out),
                              _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_dequant_e4m3")
    return out
