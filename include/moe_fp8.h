/*
 * moe_fp8.h — C ABI of libmoe_fp8.so: one Mixture-of-Experts FFN layer whose
 * expert weights are stored as block-FP8 (OCP E4M3FN bytes with one fp32 scale
 * per square block), computed on one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes, per token t (x_t is one row of x):
 *   l      = x_t · Wrᵀ (+ b)                      router logits, fp32 accumulate
 *   S      = the top_k experts by l, ties to the lower expert index,
 *            in descending-logit order (slot j = 0 .. top_k-1)
 *   g_j    = exp(l_{S_j}) / Σ_{e∈S} exp(l_e)      softmax renormalised over S
 *   for each selected expert e (and, if present, the shared expert with weight 1):
 *     W    = dec(q) · scale[row/B][col/B]         block-FP8 dequantisation
 *     h    = silu(x_t · Wgᵀ) ⊙ (x_t · Wuᵀ)         SwiGLU, silu(z) = z / (1 + e^-z)
 *     y_e  = h · Wdᵀ
 *   out_t  = Σ_j g_j · y_{S_j} (+ y_shared)        fixed order j = 0..k-1, then shared
 *
 * Sources. The colizig page ("What this project is trying to prove", "Features",
 * "Status", "Architecture & how it works") names the pieces: natively block-FP8
 * (E4M3) expert weights, top-8-of-128 and top-10-of-512 routing with one
 * always-on shared expert, dequantisation fused into the dot product, per-expert
 * fan-out, and experts as the bulk of the parameters. The pages do not write
 * out the routing function, the FFN non-linearity, the block size, the E4M3
 * variant or the layout; the readings taken here are the ones stated above and
 * beside each field below (softmax over the logits, renormalised top-k gates,
 * SwiGLU, OCP E4M3FN with max 448, multiplicative fp32 block scales).
 *
 * Conventions for every entry point:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *    never frees, keeps or aliases it beyond the call's stream work.
 *  - The library allocates no memory; scratch lives in the caller's workspace,
 *    whose size moe_workspace_bytes() reports (256-byte aligned base required).
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *    legacy default stream) and the call returns without host synchronisation.
 *  - Arguments are validated on the host before anything is launched. A status
 *    other than MOE_OK from validation means nothing was enqueued. MOE_ERR_HIP
 *    means a launch failed; work enqueued before it may have run.
 *  - Results are deterministic: the same inputs give the same bits (no float
 *    atomics; sums are taken in a fixed order).
 *  - tokens == 0 is valid and enqueues nothing.
 *  - There is no CPU fallback: a layer shape without a compiled kernel returns
 *    MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                            */
  MOE_ERR_SHAPE = 2,       /* non-positive size, top_k outside [1, experts], block   */
                           /* not dividing hidden/inter, bad enum value             */
  MOE_ERR_UNSUPPORTED = 3, /* no kernel instantiated for this (hidden, inter, block, */
                           /* dtype, path) combination                              */
  MOE_ERR_WORKSPACE = 4,   /* workspace smaller than moe_workspace_bytes()          */
                           /* or not 256-byte aligned                               */
  MOE_ERR_HIP = 5,         /* a HIP launch or event call failed                     */
  MOE_ERR_TOO_LARGE = 6    /* moe_forward_static: the call needs more scratch than  */
                           /* MOE_STATIC_SCRATCH_BYTES                              */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Expert-pass kernel family. AUTO picks the wavefront GEMV family when
 * tokens <= 48 or x is fp32, and the bf16-MFMA grouped family otherwise.
 * The forced values exist so both families can be exercised at any size;
 * MFMA requires bf16 activations. MFMA_FP8 is the grouped family with both
 * expert contractions in E4M3 on both sides: x is quantised as
 * moe_quantize_act_e4m3 describes (the router still reads x itself), and
 * the SwiGLU output h, computed in fp32, is quantised by the same rule (per
 * expert row and 128 columns) before the down contraction. This changes the
 * layer's numerics (about 2^-4 relative per operand value); it requires bf16
 * x and H and I multiples of 128, and is not chosen by AUTO.
 * MFMA and MFMA_FP8 run their gate/up and down passes as one kernel launch
 * (not so moe_forward_streamed): a down workgroup waits for its row tile's gate/up
 * workgroups through a per-tile counter in the workspace, which the
 * permutation clears (no memset). Every wait is bounded; the STATUS region
 * reports one that gave up, or a tile whose two passes ran on different
 * XCDs (h goes between them through one XCD's L2); the output is then not
 * valid. Workgroups of a launch are dispatched in order on each XCD and a
 * gate/up workgroup never waits, so the waits end.
 * GEMV_FUSED runs the GEMV family's whole layer (router, selection,
 * permutation, gate/up, down, combine) as one kernel launch whose workgroups
 * hand results to each other through the workspace (flags holding a per-call
 * epoch, counters), instead of five launches: the fixed per-step operation
 * graph of decode that the ferrite page describes, without the kernel
 * boundaries. Same arithmetic as GEMV (the router's partial sums and the
 * combine's order included), so the two give identical outputs. It covers
 * 1 <= tokens <= 16, experts <= 512 and hidden < 512 or a multiple of 512,
 * on the GEMV shapes. AUTO does not take it: on MI355X its in-kernel
 * hand-offs cost more than the four kernel boundaries they replace. Its
 * workers wait for one another, so it expects the device to itself (they
 * are sized to fit on it at once); every wait is bounded, and the
 * workspace's STATUS region (moe_workspace_region) reports one that gave up
 * (the output is then not valid). */
typedef enum {
  MOE_PATH_AUTO = 0,
  MOE_PATH_GEMV = 1,
  MOE_PATH_MFMA = 2,
  MOE_PATH_MFMA_FP8 = 3,
  MOE_PATH_GEMV_FUSED = 4
} moe_path;

typedef struct {
  int64_t tokens;      /* T: rows of x and out                                    */
  int32_t hidden;      /* H                                                       */
  int32_t experts;     /* E: routed experts (1 .. 1024)                           */
  int32_t inter;       /* I: expert intermediate size                             */
  int32_t top_k;       /* k: experts selected per token, 1 .. min(E, 16)          */
  int32_t block;       /* B: square scale-block edge; must divide H and I         */
  int32_t has_shared;  /* 0 or 1: an always-on shared expert of the same shape    */
  moe_dtype x_dtype;   /* dtype of x (MOE_F32 or MOE_BF16)                        */
  moe_dtype out_dtype; /* dtype of out (MOE_F32 or MOE_BF16)                      */
  moe_path path;       /* expert kernel family                                    */
} moe_config;

/* One bank of n experts (n = E for the routed bank, 1 for the shared expert).
 * Row-major, contiguous, expert-major:
 *   w_gate_up [n][2I][H]     E4M3FN bytes; rows 0..I-1 are the gate projection,
 *                            rows I..2I-1 the up projection
 *   w_down    [n][H][I]      E4M3FN bytes
 *   s_gate_up [n][2I/B][H/B] fp32 scale of each B×B block of w_gate_up
 *   s_down    [n][H/B][I/B]  fp32 scale of each B×B block of w_down
 * A weight's value is dec(byte) · scale of its block, dec = OCP E4M3FN
 * (bias 7, no infinities, 0x7F/0xFF NaN, max finite 448). NaN bytes are not
 * supported inputs. */
typedef struct {
  const uint8_t* w_gate_up;
  const uint8_t* w_down;
  const float* s_gate_up;
  const float* s_down;
} moe_expert_bank;

/* Optional per-phase HIP events (hipEvent_t passed as void*). Each non-NULL
 * event is recorded on `stream` at the named phase boundary, so a caller can
 * time the phases of a call with hipEventElapsedTime. PERMUTED and GATE_UP
 * are attached to the gate/up kernel's own dispatch (hipExtLaunchKernel):
 * they take that kernel's start and end times, so the pair times the kernel
 * alone, without the dispatch gap before it (which falls in ROUTED ->
 * PERMUTED). NULL entries are skipped; pass NULL for the whole struct to
 * record nothing. */
typedef enum {
  MOE_EV_START = 0,        /* before the router                            */
  MOE_EV_ROUTED = 1,       /* after logits + top-k + gates (at decode sizes,  */
                           /* where selection and permutation share one      */
                           /* launch: after the logits)                      */
  MOE_EV_PERMUTED = 2,     /* start of the gate/up kernel (after the       */
                           /* token→expert permutation)                     */
  MOE_EV_GATE_UP = 3,      /* end of the gate/up + SwiGLU kernel (routed   */
                           /* and shared; on the MFMA paths that launch     */
                           /* also runs the down pass)                      */
  MOE_EV_DOWN = 4,         /* after the down projection                    */
  MOE_EV_END = 5,          /* after the combine                            */
  MOE_EV_COUNT = 6
} moe_phase;
typedef struct {
  void* ev[MOE_EV_COUNT];
} moe_phase_events;

/* Bytes of workspace moe_forward / moe_route / moe_permute need for `cfg`
 * (0 on an invalid cfg). The same workspace serves all three. */
size_t moe_workspace_bytes(const moe_config* cfg);

/* Whole layer (router, top-k, permutation, SwiGLU experts, combine).
 * Source: colizig page, "What this project is trying to prove" (model table:
 * top-8 of 128 experts; top-10 of 512 plus one always-on shared expert;
 * natively block-FP8 checkpoints), "Features" (E4M3 weights dequantised inside
 * the dot products; per-expert work fanned out, bit-identical to the serial
 * path) and "Architecture & how it works" (a small resident router in front of
 * the experts, which hold most of the parameters). The formulas are the
 * readings in this file's header.
 *   x           [T][H] of cfg->x_dtype
 *   router_w    [E][H] fp32
 *   router_bias [E] fp32 added to the logits (affects selection and gates),
 *               or NULL for none
 *   experts     routed bank, n = E (struct itself is read on the host)
 *   shared      shared bank, n = 1; required iff cfg->has_shared, else ignored
 *   top_k       must equal cfg->top_k
 *   out         [T][H] of cfg->out_dtype; written, never read
 *   workspace   device scratch of at least moe_workspace_bytes(cfg) bytes
 *   events      optional phase events (see moe_phase_events), or NULL        */
moe_status moe_forward(const void* x, const float* router_w, const float* router_bias,
                       const moe_expert_bank* experts, const moe_expert_bank* shared,
                       int32_t top_k, void* out, const moe_config* cfg,
                       void* workspace, size_t workspace_bytes,
                       const moe_phase_events* events, void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Its scratch is a static device array of
 * MOE_STATIC_SCRATCH_BYTES inside the library (each GPU it runs on holds one
 * copy until the process ends); the call allocates nothing, and everything
 * else (arguments, results, events, stream, errors) is as moe_forward.
 * Calls whose moe_workspace_bytes(cfg) exceeds MOE_STATIC_SCRATCH_BYTES
 * return MOE_ERR_TOO_LARGE before anything is enqueued (64 MiB hold the
 * decode layers and prefill batches of several hundred tokens). All calls on
 * one GPU share its array: calls that may overlap on one GPU (several
 * streams or host threads) race and must be serialised by the caller. The
 * first call on a device looks up the array's device address with that
 * device current (MOE_ERR_HIP if that fails). The STATUS word of the paths
 * with in-kernel waits stays inside that array, where the caller cannot
 * read it. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_static(const void* x, const float* router_w, const float* router_bias,
                              const moe_expert_bank* experts, const moe_expert_bank* shared,
                              int32_t top_k, void* out, const moe_config* cfg,
                              const moe_phase_events* events, void* stream);

/* ---- Routed experts streamed from host memory through an HBM cache ----
 * State of a bounded cache of expert slots in device memory, kept by the
 * caller in HOST memory and updated by moe_forward_streamed. Before the first
 * call: slot_expert[i] = -1 and slot_used[i] = 0 for every slot, counters 0.
 */
typedef struct {
  int32_t slots;         /* expert slots of the device bank (>= 1)                   */
  int32_t* slot_expert;  /* [slots] routed expert held by each slot, -1 = empty      */
  int64_t* slot_used;    /* [slots] value of `calls` when the slot was last used     */
  int64_t calls;         /* calls made with this cache                                */
  int64_t hits;          /* needed experts found resident, summed over calls         */
  int64_t misses;        /* needed experts copied in, summed over calls              */
  int64_t bytes_in;      /* expert bytes copied host -> device, summed over calls    */
  int32_t rounds_last;   /* expert-pass rounds of the last call                       */
} moe_expert_cache;

/* moe_forward with the routed experts kept in HOST memory and streamed on
 * demand into a bounded cache of device expert slots, least recently used
 * out first. Source: colizig page, "Features" (memory-tiered streaming with
 * a bounded LRU expert cache; the GPU backend's LRU VRAM weight cache) and
 * "What this project is trying to prove" (most of a 512-expert model is cold
 * at any instant, so its experts stream across memory tiers instead of all
 * being resident).
 *   host_experts  routed bank (n = E) in pinned host memory (hipHostMalloc or
 *                 equivalent), layout as moe_expert_bank
 *   slot_bank     device bank of n = cache->slots experts, the cache itself
 *   cache         host-memory state (above); read and updated by the call
 *   shared        the shared expert's bank in DEVICE memory (always resident)
 * Everything else as moe_forward (no phase events). The call routes on the
 * device, brings the group offsets back to name the experts it needs (it
 * waits for them), then runs the expert passes in rounds of at most `slots`
 * experts: experts already resident first, the missing ones copied into the
 * least recently used slots that the round does not use. A call needing
 * more experts than there are slots takes several rounds. The call returns
 * once its work has completed on `stream`. Outputs are bit-identical to
 * moe_forward's on the same inputs (the same kernels compute each group
 * once). The workspace is moe_forward's (moe_workspace_bytes). Errors: as
 * moe_forward; MOE_ERR_SHAPE also for slots < 1 or a slot_expert entry that
 * is not -1 or a distinct routed expert; MOE_ERR_NULL for NULL cache arrays. */
moe_status moe_forward_streamed(const void* x, const float* router_w, const float* router_bias,
                                const moe_expert_bank* host_experts,
                                const moe_expert_bank* slot_bank, moe_expert_cache* cache,
                                const moe_expert_bank* shared, int32_t top_k, void* out,
                                const moe_config* cfg, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Router and selection only (the first two steps of moe_forward).
 * Source: colizig page, "Architecture & how it works" (the router is small and
 * always resident) and "What this project is trying to prove" (top-8 / top-10
 * expert counts); the routing function (softmax, top-k with ties to the lower
 * expert index, gates renormalised over the chosen experts) is this file's
 * reading, the pages do not write it out.
 *   topk_idx [T][k] int32 expert ids, descending logit, ties to lower id
 *   gates    [T][k] fp32 renormalised softmax weights (sum to 1 per token)
 *   logits   [T][E] fp32 router logits, or NULL to keep them in the workspace */
moe_status moe_route(const void* x, const float* router_w, const float* router_bias,
                     int32_t* topk_idx, float* gates, float* logits,
                     const moe_config* cfg, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Token→expert permutation only (the third step of moe_forward), from a
 * given topk_idx [T][k]. Source: colizig page, "Features" (routed experts
 * evaluated per expert, the work fanned out over workers with results
 * bit-identical to the serial order): grouping every token's choices by
 * expert, stable in token order, is what lets each expert's weights stream
 * once for all of its tokens. Slot s = t·k + j is the j-th choice of token t;
 * when cfg->has_shared, slots T·k + t (t = 0..T-1) are the shared expert's.
 *   offsets [E+2] int32: rows of routed expert e are offsets[e] .. offsets[e+1]-1;
 *           the shared group is offsets[E] .. offsets[E+1]-1 (empty without one)
 *   pair    [P] int32, P = T·k (+T): pair[row] = slot, rows of one expert in
 *           ascending token order (stable by slot index)
 *   inv     [P] int32: inv[slot] = row                                       */
moe_status moe_permute(const int32_t* topk_idx, int32_t* offsets, int32_t* pair,
                       int32_t* inv, const moe_config* cfg, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Expand one block-FP8 matrix to fp32 on the device:
 *   out[r][c] = dec(w[r][c]) * scales[r / block][c / block]
 * with the same in-register E4M3FN decode the expert kernels use (colizig page,
 * "Features": block-FP8 E4M3 weights). w [rows][cols] uint8, scales
 * [rows/block][cols/block] fp32, out [rows][cols] fp32, all device memory.
 * block must divide rows and cols (else MOE_ERR_SHAPE); cols must be a
 * multiple of 16 (else MOE_ERR_UNSUPPORTED); rows == 0 enqueues nothing. */
moe_status moe_dequant_e4m3(const uint8_t* w, const float* scales, int64_t rows, int32_t cols,
                            int32_t block, float* out, void* stream);

/* E4M3 activations for the variant that runs both operands of both expert
 * contractions in FP8 (a reading of this project: the pages describe E4M3
 * weights only, colizig page, "What this project is trying to prove").
 * Each token's row of x is cut into blocks of 128 columns; block b of token t
 * gets the scale 2^e, e the smallest integer with max|x| <= 448 * 2^e over the
 * block (0 for an all-zero block, at least -127), and each value becomes the
 * nearest OCP E4M3FN value of x * 2^-e (ties to the even mantissa, sign
 * kept, so negatives that round to zero give 0x80).
 *   x      [tokens][hidden] bf16, finite values only (device)
 *   codes  [tokens][hidden] E4M3FN bytes (device, written)
 *   exps   [tokens][hidden/128] uint8 E8M0 exponents, e + 127 (device, written)
 * hidden must be a multiple of 128 (else MOE_ERR_UNSUPPORTED); tokens == 0
 * enqueues nothing. */
moe_status moe_quantize_act_e4m3(const void* x, int64_t tokens, int32_t hidden, uint8_t* codes,
                                 uint8_t* exps, void* stream);

/* Intermediate results of moe_forward, readable from its workspace once the
 * call's stream work has completed (the workspace is the caller's memory).
 * moe_workspace_region reports where one of them lies for `cfg`:
 *   *offset  byte offset from the workspace base (a multiple of 256)
 *   *bytes   its size in bytes (0 when the configuration does not use it)
 * Regions (P = T·k + T·has_shared rows; "row" = a row of the permuted
 * problem, whose order moe_permute defines; "slot" s = t·k + j, or T·k + t
 * for the shared expert):
 *   TOPK     int32 [T][k]   selected experts (as moe_route returns them)
 *   GATES    fp32  [T][k]   their gates
 *   OFFSETS  int32 [E+2]    group offsets (as moe_permute returns them)
 *   PAIR     int32 [P]      row -> slot
 *   INV      int32 [P]      slot -> row
 *   H        [P][I] SwiGLU output by row: fp32 (GEMV family); fp16 scaled by
 *            H_EXPS (MFMA family); E4M3 codes scaled by H_EXPS (MFMA_FP8)
 *   H_EXPS   uint8 [P][I/128] exponent bytes of H (MFMA families): element
 *            (r, c) of H is value(H[r][c]) * 2^(H_EXPS[r][c/128] - 127)
 *   Y        [P][H] expert outputs by slot: fp32 (GEMV family), fp16
 *            scaled by Y_EXPS (MFMA families)
 *   Y_EXPS   uint8 [P][H/128] exponent bytes of Y (MFMA families)
 *   STATUS   uint32 (single-launch decode layer and MFMA paths, else 0
 *            bytes): error bits of the call's in-kernel waits, 0 when every
 *            wait ended normally (decode layer: 1 router results, 2 the
 *            permutation, 4 gate/up results not seen within the bounded
 *            wait; MFMA paths: 8 a down workgroup's wait for its tile's
 *            gate/up results gave up, 16 a tile's gate/up and down passes
 *            ran on different XCDs); the output is then not valid
 * Returns MOE_ERR_NULL for a NULL pointer, MOE_ERR_SHAPE for an invalid cfg
 * or region. This call touches no device memory. It is what lets tests
 * compare each step's result with an independent evaluation. */
typedef enum {
  MOE_WS_TOPK = 0,
  MOE_WS_GATES = 1,
  MOE_WS_OFFSETS = 2,
  MOE_WS_PAIR = 3,
  MOE_WS_INV = 4,
  MOE_WS_H = 5,
  MOE_WS_H_EXPS = 6,
  MOE_WS_Y = 7,
  MOE_WS_Y_EXPS = 8,
  MOE_WS_STATUS = 9,
  MOE_WS_COUNT = 10
} moe_ws_region;
moe_status moe_workspace_region(const moe_config* cfg, int32_t region, size_t* offset,
                                size_t* bytes);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t moe_version(void);

/* Poll bound of the in-kernel waits of the MFMA paths' one launch (a
 * down workgroup waiting for its row tile's gate/up workgroups), for tests
 * of its give-up path: with a small bound, waits that do not see their tile
 * complete at once give up, set STATUS bit 8 and skip the tile, and every
 * workgroup still ends (the call's output is then not valid). polls = 0
 * restores the default bound (about a second). Process-wide; applies to
 * calls enqueued after it returns. Always MOE_OK. */
moe_status moe_set_wait_limit(uint32_t polls);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H */
