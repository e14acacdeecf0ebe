"""CPU oracle of the block-FP8 routed MoE layer (fp64 NumPy).

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or run this module. The HIP library
never calls it and shares no code with it; inputs reach both sides from the
separate `workloads` generator.

It is plain and slow on purpose: every step is the textbook definition, in
fp64, one expert at a time, so that it can be checked against the pages by
eye. Sources, per function below:
  * colizig page, "What this project is trying to prove" (model table): both
    model families are natively block-FP8; top-8 of 128 experts with no shared
    expert, top-10 of 512 experts plus one shared expert.
  * colizig page, "Features": block-FP8 (E4M3) weights whose dequantisation is
    fused into the dot products; per-expert evaluation fanned out over workers,
    bit-identical to the serial path; an independent NumPy reference used as a
    correctness net for the engine.
  * colizig page, "Architecture & how it works": experts are the bulk of the
    parameters; the router is small and always resident.
  * ferrite page (both languages): the CPU backend is the golden standard that
    every other backend is validated against.
The pages never write the layer's formulas down. Readings taken where they are
silent (each restated at the function that uses it):
  R1 E4M3 is OCP E4M3FN: bias 7, subnormals, no infinities, 0x7F/0xFF are NaN,
     max finite 448 (consistent with scales of amax/448).
  R2 a block scale multiplies: W = dec(q) * scale[row // B, col // B].
  R3 gate/up are one [2I][H] matrix, gate rows first.
  R4 routing is softmax over all logits, top-k on the logits with ties to the
     lower expert index, slot order by descending logit, gates renormalised
     over the selected experts.
  R5 a router bias is added to the logits before selection and gating.
  R6 the expert FFN is SwiGLU: h = silu(x Wg^T) * (x Wu^T), y = h Wd^T.
  R7 the shared expert is always on with weight 1 and has the routed shape.
  R8 out_t = sum_j g_j y_{t,j} (+ y_shared,t).
  R9 a token is tie-flagged when its k-th and (k+1)-th largest logits differ by
     less than 1e-5 (absolute, on these fp64 logits); its selection is then not
     unique at the kernel's precision.
  R10 (a variant for prefill sizes, where both operands of the gate/up
     contraction are E4M3; the pages describe E4M3 weights only, so the
     activation side is this project's reading) each token's activation row
     is cut into blocks of `block` columns; a block's scale is 2^e with e the
     smallest integer such that its largest magnitude is at most 448 * 2^e
     (e = 0 for an all-zero block, never below -127), and each value becomes
     the nearest E4M3FN value of x * 2^-e (an exact tie goes to the even
     mantissa; the sign is kept, so negative values that round to zero give
     -0). The down contraction reads the SwiGLU output h quantised the same
     way (per expert row and block of `block` columns of h). Power-of-two
     scales are the block-scale form of gfx950's FP8 matrix instructions.
     The router still reads the unquantised x.
  R11 h is a computed value, so the decisions that quantise it (the block
     exponent from max|h|, then each code) are taken on h rounded to fp32,
     the precision the kernels compute h in. A kernel's own fp32 h still
     differs from that by its rounding error, so where h lies within that
     error of a decision boundary either side of the boundary is a correct
     result: h_admissible_deviation bounds how far the dequantised h can
     move over every such choice, and moe_layer (given h_band) turns that
     into a per-element bound on the output (the analogue of R9's tie band
     for selections). Given a kernel's own codes for h, h_admissible_codes
     decides element by element whether they are such a correct result, and
     moe_layer (given h_codes) evaluates the down contraction on them, as
     R9 re-runs the layer on an accepted selection.
Every function here is pinned by tests/test_oracle_pins.py; no function is
parity-unpinned.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

TIE_BAND = 1e-5


# --------------------------------------------------------------------------
# block-FP8 weights (R1, R2, R3)
# --------------------------------------------------------------------------
def e4m3fn_decode(codes) -> np.ndarray:
    """Value of each OCP E4M3FN byte, by the closed form (R1):
    sign s = b >> 7, exponent e = (b >> 3) & 15, mantissa m = b & 7;
    e == 0: (-1)^s * m * 2^-9 (subnormal); e == 15 and m == 7: NaN;
    otherwise (-1)^s * 2^(e - 7) * (1 + m / 8).
    The closed form is evaluated once for each of the 256 byte values and the
    codes index that table."""
    b = np.arange(256, dtype=np.int64)
    s = b >> 7
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    val = np.where(s == 1, -mag, mag)
    val = np.where((e == 15) & (m == 7), np.nan, val).astype(np.float64)
    return val[np.asarray(codes, dtype=np.uint8)]


def dequantise(codes: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """W[r, c] = dec(codes[r, c]) * scales[r // block, c // block] (R2), fp64."""
    w = e4m3fn_decode(codes)
    if np.isnan(w).any():
        raise ValueError("E4M3 NaN code in a weight matrix")
    s = np.asarray(scales, dtype=np.float64)
    s_full = np.repeat(np.repeat(s, block, axis=0), block, axis=1)
    assert s_full.shape == w.shape, (s_full.shape, w.shape)
    return w * s_full


# --------------------------------------------------------------------------
# E4M3 activations for the gate/up contraction (R10)
# --------------------------------------------------------------------------
def e4m3fn_round(v) -> np.ndarray:
    """The E4M3FN byte nearest to each finite v with |v| <= 448 (R10): the
    candidates are the values of the non-negative finite codes 0x00 .. 0x7E
    (increasing with the code), the nearest magnitude wins, an exact tie goes
    to the code whose mantissa is even, and the sign bit is v's sign bit."""
    v = np.asarray(v, np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > 448.0):
        raise ValueError("e4m3fn_round takes finite values of magnitude at most 448")
    mags = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))  # 0x00 .. 0x7E
    a = np.abs(v)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)  # first value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def act_scale_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, at least -127; 0 where
    amax is 0 (R10). A log2 estimate, corrected by exact comparisons."""
    amax = np.asarray(amax, np.float64)
    e = np.zeros(amax.shape, np.int64)
    nz = amax > 0
    a = amax[nz]
    est = np.ceil(np.log2(a / 448.0)).astype(np.int64)
    est = np.where(a > np.ldexp(448.0, est), est + 1, est)
    est = np.where(a <= np.ldexp(448.0, est - 1), est - 1, est)
    e[nz] = np.maximum(est, -127)
    return e


def quantise_activations(x: np.ndarray, block: int):
    """x [T][H] -> (codes [T][H] uint8, exponents [T][H/block] int64), one
    power-of-two scale per token and block of `block` columns (R10)."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    if H % block:
        raise ValueError("block must divide the row length")
    xb = x.reshape(T, H // block, block)
    e = act_scale_exponent(np.abs(xb).max(axis=2))
    scaled = xb * np.ldexp(1.0, -e)[:, :, None]  # exact: a power of two
    return e4m3fn_round(scaled).reshape(T, H), e


def dequantise_activations(codes: np.ndarray, exps: np.ndarray, block: int) -> np.ndarray:
    """x^[t, h] = dec(codes[t, h]) * 2^exps[t, h // block] (R10), fp64."""
    T, H = codes.shape
    v = e4m3fn_decode(codes).reshape(T, H // block, block)
    return (v * np.ldexp(1.0, np.asarray(exps, np.int64))[:, :, None]).reshape(T, H)


def expert_matrices(expert: dict, inter: int, block: int):
    """(Wg [I][H], Wu [I][H], Wd [H][I]) in fp64 from one expert's bytes and
    scales (R3: the first I rows of w_gate_up are the gate projection)."""
    wgu = dequantise(expert["w_gate_up"], expert["s_gate_up"], block)
    wd = dequantise(expert["w_down"], expert["s_down"], block)
    return wgu[:inter], wgu[inter:], wd


# --------------------------------------------------------------------------
# router and selection (R4, R5, R9)
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, router_w: np.ndarray,
                  router_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] Wr[e, h] (+ b[e]) in fp64 (R5)."""
    l = np.asarray(x, np.float64) @ np.asarray(router_w, np.float64).T
    if router_bias is not None:
        l = l + np.asarray(router_bias, np.float64)[None, :]
    return l


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k experts with the largest logits (R4): a full stable
    sort of the experts by descending logit, so equal logits keep ascending
    expert order; the first k are slots j = 0..k-1."""
    T, E = logits.shape
    assert 1 <= k <= E
    idx = np.empty((T, k), np.int64)
    for t in range(T):
        order = np.argsort(-logits[t], kind="stable")
        idx[t] = order[:k]
    return idx


def softmax(v: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax of a 1-D fp64 vector."""
    z = np.exp(v - v.max())
    return z / z.sum()


def gate_weights(logits: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    """g[t, j] = p[t, idx[t, j]] / sum_j' p[t, idx[t, j']] with p the softmax
    over all E logits of token t (R4)."""
    T, k = topk_idx.shape
    g = np.empty((T, k), np.float64)
    for t in range(T):
        p = softmax(logits[t])
        sel = p[topk_idx[t]]
        g[t] = sel / sel.sum()
    return g


def tie_flags(logits: np.ndarray, k: int, band: float = TIE_BAND) -> np.ndarray:
    """True for tokens whose k-th and (k+1)-th largest logits differ by less
    than `band` (R9). With k == E nothing can be swapped and no token is
    flagged."""
    T, E = logits.shape
    if k >= E:
        return np.zeros(T, bool)
    srt = -np.sort(-logits, axis=1)
    return (srt[:, k - 1] - srt[:, k]) < band


# --------------------------------------------------------------------------
# token -> expert permutation
# --------------------------------------------------------------------------
def permutation(topk_idx: np.ndarray, experts: int, shared: bool):
    """Group the slots s = t*k + j by expert: rows of expert e are its slots in
    ascending slot (hence token) order; the shared expert, if present, is group
    E holding slots T*k + t for t = 0..T-1. Returns (offsets [E+2], pair [P],
    inv [P]) with pair[row] = slot and inv[slot] = row."""
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1)
    order = np.argsort(flat, kind="stable")  # ascending expert, ties by slot
    counts = np.bincount(flat, minlength=experts)
    offsets = np.zeros(experts + 2, np.int64)
    offsets[1:experts + 1] = np.cumsum(counts)
    pair = list(order)
    if shared:
        pair += [T * k + t for t in range(T)]
    offsets[experts + 1] = len(pair)
    pair = np.asarray(pair, np.int64)
    inv = np.empty_like(pair)
    inv[pair] = np.arange(len(pair))
    return offsets, pair, inv


# --------------------------------------------------------------------------
# expert FFN and combine (R6, R7, R8)
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)), fp64."""
    return z / (1.0 + np.exp(-z))


def swiglu_expert(xs: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
                  h_block: Optional[int] = None, h_band: Optional[tuple] = None):
    """y = (silu(xs Wg^T) * (xs Wu^T)) Wd^T for rows xs [n][H] (R6); with
    h_block, h is rounded to fp32 and quantised to E4M3 in blocks of that many
    columns first (R10, R11). With h_band = (acc_rel, eval_rel) as well,
    returns (y, bound): bound [n][H] is the largest change of y that the
    admissible quantisations of h can make (R11), from the band h_band_width
    gives."""
    a = xs @ wg.T
    u = xs @ wu.T
    h = silu(a) * u
    if h_block is None:
        return h @ wd.T
    h = h.astype(np.float32).astype(np.float64)
    y = dequantise_activations(*quantise_activations(h, h_block), h_block) @ wd.T
    if h_band is None:
        return y
    tau = h_band_width(xs, wg, wu, *h_band)
    return y, h_admissible_deviation(h, tau, h_block) @ np.abs(wd).T


def h_band_width(xs: np.ndarray, wg: np.ndarray, wu: np.ndarray, acc_rel: float,
                 eval_rel: float) -> np.ndarray:
    """Per element of h = silu(a) * u (a = xs Wg^T, u = xs Wu^T), a bound on
    how far an fp32 evaluation can land from the exact value (R11): the sums
    err by at most acc_rel times the sum of their terms' magnitudes, which
    moves h by |silu'(a)| |u| da + |silu(a)| du to first order, and the
    pointwise steps (scaling, exponential, division, product) by at most
    eval_rel (8 + |a|) |h| (an exponential of a argument rounded to relative
    e errs by about |a| e)."""
    a = xs @ wg.T
    u = xs @ wu.T
    sa = np.abs(xs) @ np.abs(wg).T
    su = np.abs(xs) @ np.abs(wu).T
    sig = 1.0 / (1.0 + np.exp(-a))
    dsilu = sig * (1.0 + a * (1.0 - sig))
    h = a * sig * u
    return acc_rel * (np.abs(dsilu * u) * sa + np.abs(a * sig) * su) + \
        eval_rel * (8.0 + np.abs(a)) * np.abs(h)


def h_admissible_deviation(h: np.ndarray, tau: np.ndarray, block: int) -> np.ndarray:
    """For h [n][I] and a per-element band tau [n][I] (R11): the largest
    |q(h') - q(h)| over every h' with |h' - h| <= tau elementwise, where q is
    R10's quantise-then-dequantise in blocks of `block` columns. The block
    exponent of such an h' lies between those of the smallest and largest
    block maxima the band allows; under a fixed exponent the rounding is
    monotone, so the extremes are taken at h - tau and h + tau (values past
    448 under an exponent cannot occur with that exponent and are clipped)."""
    n, I = h.shape
    hb = np.asarray(h, np.float64).reshape(n, I // block, block)
    tb = np.asarray(tau, np.float64).reshape(n, I // block, block)
    codes, e = quantise_activations(h, block)
    ref = dequantise_activations(codes, e, block).reshape(hb.shape)
    e_lo = act_scale_exponent(np.maximum(np.abs(hb) - tb, 0.0).max(axis=2))
    e_hi = act_scale_exponent((np.abs(hb) + tb).max(axis=2))
    lo, hi = np.minimum(e_lo, e_hi), np.maximum(e_lo, e_hi)
    dev = np.zeros_like(hb)
    for step in range(int((hi - lo).max(initial=0)) + 1):
        ec = np.minimum(lo + step, hi)[:, :, None]
        for side in (-1.0, 0.0, 1.0):
            v = np.clip((hb + side * tb) * np.ldexp(1.0, -ec), -448.0, 448.0)
            q = e4m3fn_decode(e4m3fn_round(v)) * np.ldexp(1.0, ec)
            dev = np.maximum(dev, np.abs(q - ref))
    return dev.reshape(n, I)


def h_admissible_codes(h: np.ndarray, tau: np.ndarray, codes: np.ndarray, exps: np.ndarray,
                       block: int) -> np.ndarray:
    """For h [n][I], a per-element band tau [n][I] and a candidate
    quantisation of h (E4M3 codes [n][I], block exponents [n][I/block]):
    True where element (r, c) is one that an evaluation of h landing within
    tau of it produces under R10 (R11). The block's exponent must lie between
    those of the smallest and the largest block maximum the band allows
    (the exponent rule is monotone in the maximum), and under that exponent
    the element's value must lie between the values h - tau and h + tau
    round to (rounding is monotone, so every value between is reached).
    Values are compared, so +0 and -0 are the same result."""
    n, I = h.shape
    hb = np.asarray(h, np.float64).reshape(n, I // block, block)
    tb = np.asarray(tau, np.float64).reshape(n, I // block, block)
    ex = np.asarray(exps, np.int64).reshape(n, I // block)
    e_lo = act_scale_exponent(np.maximum(np.abs(hb) - tb, 0.0).max(axis=2))
    e_hi = act_scale_exponent((np.abs(hb) + tb).max(axis=2))
    ok_e = (ex >= np.minimum(e_lo, e_hi)) & (ex <= np.maximum(e_lo, e_hi))
    down = np.ldexp(1.0, -ex)[:, :, None]
    lo = e4m3fn_decode(e4m3fn_round(np.clip((hb - tb) * down, -448.0, 448.0)))
    hi = e4m3fn_decode(e4m3fn_round(np.clip((hb + tb) * down, -448.0, 448.0)))
    v = e4m3fn_decode(np.asarray(codes, np.uint8)).reshape(hb.shape)
    with np.errstate(invalid="ignore"):  # a NaN code compares false: not admissible
        ok = ok_e[:, :, None] & (v >= lo) & (v <= hi)
    return ok.reshape(n, I)


def moe_layer(x: np.ndarray, router_w: np.ndarray, router_bias: Optional[np.ndarray],
              expert: Callable[[int], dict], top_k: int, inter: int, block: int,
              shared: Optional[dict] = None, routing: Optional[np.ndarray] = None,
              tokens: Optional[np.ndarray] = None, act_block: Optional[int] = None,
              h_band: Optional[tuple] = None, h_codes: Optional[Callable] = None):
    """The whole layer in fp64.

    expert(e) returns expert e's block-FP8 dict (w_gate_up, s_gate_up, w_down,
    s_down); only experts some token selects are fetched. `routing` [T][k]
    overrides the selection (used to re-run the oracle with another valid set
    for a tie-flagged token); gates are then taken over those experts. With
    `tokens` given, only those rows of the output are computed (the logits of
    every token are still formed, since they are cheap). With `act_block`
    given, both expert contractions read E4M3 operands in blocks of that many
    columns (x for gate/up, h for down, R10); the router reads x as it is.
    With h_band = (acc_rel, eval_rel) as well, the result also holds
    "flip" [T'][H]: the bound on how far the admissible quantisations of h
    (R11) can move each output element, summed over the token's experts with
    their gates. With h_codes as well (a kernel's quantisation of h:
    h_codes(e, tokens, slots) returns (codes [n][I], block exponents) for
    expert e's rows of those tokens and slots j, and h_codes(None, tokens,
    None) for the shared expert's), the down contraction reads those codes
    instead of the oracle's own, "h_check" counts the elements whose codes
    are not admissible under R11 (h_admissible_codes, with the band h_band
    gives) and those whose value differs from the oracle's own, and no flip
    bound is formed: the output is the layer evaluated on the kernel's
    accepted codes, as R9 evaluates it on an accepted selection.

    Returns dict(out [T'][H], logits [T][E], topk_idx [T][k], gates [T][k],
    ties [T]) where T' = len(tokens) or T.
    """
    x = np.asarray(x, np.float64)
    logits = router_logits(x, router_w, router_bias)
    xe = x if act_block is None else dequantise_activations(
        *quantise_activations(x, act_block), act_block)
    idx = select_topk(logits, top_k) if routing is None else np.asarray(routing, np.int64)
    gates = gate_weights(logits, idx)
    rows = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens, np.int64)
    out = np.zeros((len(rows), x.shape[1]), np.float64)
    band = h_band if act_block is not None else None
    given = h_codes is not None and band is not None
    flip = np.zeros_like(out) if band is not None and not given else None
    check = {"inadmissible": 0, "flips": 0, "elements": 0}

    def expert_out(xs, wg, wu, wd, codes):
        if not given:
            return swiglu_expert(xs, wg, wu, wd, h_block=act_block, h_band=band)
        # R11: the kernel's codes, once each is admissible, feed the down contraction
        a, u = xs @ wg.T, xs @ wu.T
        h32 = (silu(a) * u).astype(np.float32).astype(np.float64)
        c, ex = codes
        ok = h_admissible_codes(h32, h_band_width(xs, wg, wu, *band), c, ex, act_block)
        hq = dequantise_activations(c, ex, act_block)
        own = dequantise_activations(*quantise_activations(h32, act_block), act_block)
        check["inadmissible"] += int((~ok).sum())
        check["flips"] += int(np.count_nonzero(hq != own))
        check["elements"] += hq.size
        return hq @ wd.T

    sub_idx = idx[rows]
    for e in np.unique(sub_idx):
        wg, wu, wd = expert_matrices(expert(int(e)), inter, block)
        who, slot = np.nonzero(sub_idx == e)
        codes = h_codes(int(e), rows[who], slot) if given else None
        y = expert_out(xe[rows[who]], wg, wu, wd, codes)
        if flip is not None:
            y, bound = y
        # each (token, slot) pair appears once; in fp64 the order of the k
        # terms of a token is immaterial at the tolerances this oracle serves
        for r, (i, j) in enumerate(zip(who, slot)):
            out[i] += gates[rows[i], j] * y[r]
            if flip is not None:
                flip[i] += gates[rows[i], j] * bound[r]
    if shared is not None:
        wg, wu, wd = expert_matrices(shared, inter, block)
        codes = h_codes(None, rows, None) if given else None
        y = expert_out(xe[rows], wg, wu, wd, codes)
        if flip is not None:
            y, bound = y
            flip += bound
        out += y
    res = {"out": out, "logits": logits, "topk_idx": idx, "gates": gates,
           "ties": tie_flags(logits, top_k)}
    if flip is not None:
        res["flip"] = flip
    if given:
        res["h_check"] = check
    return res
