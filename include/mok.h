/*
 * mok.h -- libmok: one GPU's share of the Mixture-of-Kittens (MoK) forward
 * MoE layer on AMD Instinct MI355X (gfx950).
 *
 * The calls follow the pages' statement of the layer:
 *   route (tahou.com MoK article, routing paragraph)
 *   -> count per expert, plan expert-contiguous positions, build the pull
 *      table (article, layout-planning paragraph; PyTorchKR wiki summary,
 *      key point on the {src_rank, src_index} schedule built on the device
 *      without a sort)
 *   -> pull dispatch into a fixed ring token buffer (article, pull-dispatch
 *      and ring-buffer paragraphs)
 *   -> expert SwiGLU FFN as a grouped GEMM, optional MXFP8 activations
 *      (article, megakernel and state-machine paragraphs)
 *   -> push combine and final weighted merge (article, push-combine and
 *      benchmark-scope paragraphs)
 *   -> the fused layer (article, megakernel paragraph; wiki key points on
 *      the megakernel and on the SM split with local counters).
 * Cross-GPU traffic is not part of this library: the token "sources" are
 * partitions in this GPU's own HBM, addressed by (partition, row).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host".  Row-major.
 *   - bf16 tensors are passed as raw 16-bit patterns (void*).
 *   - The caller owns every buffer.  The library allocates nothing; scratch
 *     comes from a caller workspace sized by the matching *_workspace_size
 *     query.
 *   - Every call is asynchronous and stream-ordered on `stream`; none
 *     synchronises the host or copies device data to the host, except
 *     mok_device_status.
 *   - Synchronous argument errors return a mok_status and launch nothing.
 *     Conditions only the device can see (more routed rows than the
 *     capacity given) are reported through a device status word, read with
 *     mok_device_status (fused calls) or the optional `dev_status` int32
 *     (standalone calls; NULL = not reported).  Kernels never access memory
 *     outside the buffers described here, whatever the routing data holds.
 *   - Calls are stateless and may run concurrently on different streams
 *     with disjoint buffers.
 *   - The grouped GEMMs address the ring, the activation buffer and one
 *     expert's weights with 32-bit byte offsets: each must be smaller than
 *     4 GiB (ring_slots * H, act_rows * I and 2 * I * H elements), else the
 *     call returns MOK_ERR_UNSUPPORTED.
 *   - The ring and the activation buffer (the grouped GEMMs' token
 *     operands) are column-blocked: a buffer of `rows` rows of W values
 *     holds each row in 64-byte blocks (32 bf16 or 64 E4M3 values), block
 *     b of row r at byte (b * rows + r) * 64; its E8M0 scales (one per 32
 *     values) go in pairs, scale j of row r at byte
 *     (j / 2 * rows + r) * 2 + j % 2.  Sizes are those of the row-major
 *     [rows][W] arrays (rows * W values, rows * W / 32 scales).  A GEMM
 *     k-step of 256 rows is then 16 KiB of contiguous memory.
 */
#ifndef MOK_H
#define MOK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOK_OK = 0,
    MOK_ERR_INVALID_ARG = 1,  /* null pointer, bad size, k > E, ...            */
    MOK_ERR_UNSUPPORTED = 2,  /* shape outside what the kernels handle         */
    MOK_ERR_WORKSPACE = 3,    /* workspace smaller than the query returned     */
    MOK_ERR_HIP = 4,          /* a HIP runtime call or launch failed           */
    MOK_ERR_DEVICE = 5,       /* device-side wait gave up (persistent kernel)  */
    MOK_ERR_CAPACITY = 6      /* more routed rows than the capacity passed in  */
} mok_status;

typedef enum { MOK_ACT_BF16 = 0, MOK_ACT_MXFP8_E4M3 = 1 } mok_act_format;

/* Weight format of the grouped GEMMs.  MOK_W_MXFP8_E4M3: both weight matrices
 * quantised to OCP MX E4M3 with one E8M0 scale per 32 along the contraction
 * dimension (per row of W_gu and of W_d), by mok_pack_weights from the bf16
 * weights; needs act_format MOK_ACT_MXFP8_E4M3 and weights_packed = 1, and
 * runs both GEMMs on gfx950's block-scaled FP8 MFMA (both modes of the fused
 * calls and the standalone GEMM calls). */
typedef enum { MOK_W_BF16 = 0, MOK_W_MXFP8_E4M3 = 1 } mok_weight_format;

typedef enum {
    MOK_MODE_STREAM = 0,      /* one launch per step and per window           */
    MOK_MODE_PERSISTENT = 1   /* one cooperative kernel for all windows       */
} mok_mode;

/* One GPU's share of one MoE layer. */
typedef struct {
    int32_t hidden;       /* H; multiple of 64                                 */
    int32_t inter;        /* I (expert intermediate); multiple of 64           */
    int32_t n_experts;    /* E, experts routed over                            */
    int32_t top_k;        /* k                                                 */
    int32_t expert_base;  /* local experts are [expert_base, expert_base+n_local) */
    int32_t n_local;      /* 1..256                                            */
    int32_t act_format;   /* mok_act_format                                    */
    int32_t minibatch;    /* M rows per window; 0 = two-wave rule              */
    int32_t ring_slots;   /* S ring rows; 0 = 2*M; >= M (stream), >= 2*M (persistent) */
    int32_t max_rows;     /* capacity for routed rows R; 0 = T*k               */
    int32_t n_move_cus;   /* data-movement workgroups (persistent), which take
                             GEMM tiles once their gathers and merges are
                             done; 0 = auto: 1/4 of the CUs                  */
    int32_t mode;         /* mok_mode                                          */
    int32_t wait_timeout_us; /* bound of each device-side wait of the persistent
                                kernel; 0 = 2 s.  On expiry the kernel stops and
                                the status word becomes MOK_ERR_DEVICE.        */
    int32_t weights_packed; /* 0: w_gate_up / w_down in the documented layout;
                                1: both written by mok_pack_weights for this
                                hidden, inter, n_local and act_format.         */
    int32_t no_split_k;   /* 0: the grouped GEMMs (stream mode, and the
                             standalone GEMM calls given a workspace) cut the
                             tiles of a last, partial round along K over the
                             CUs that round would leave idle, adding fp32
                             partial sums in a fixed order; 1: every tile is
                             computed whole (results then bit-identical to
                             MOK_MODE_PERSISTENT).                           */
    int32_t weight_format; /* mok_weight_format                               */
} mok_layer_desc;

/* Tokens held in partitions: token t lives in partition t / part_rows at row
 * t % part_rows.  part_ptr is a DEVICE array of n_partitions DEVICE pointers,
 * each to bf16 [part_rows][H].  A plain x[T][H] is n_partitions = 1. */
typedef struct {
    void* const* part_ptr;
    int32_t n_partitions;
    int32_t part_rows;
} mok_tokens;

/* Top-k route (article, routing paragraph).  For each token t the k largest
 * logits[t][*] (fp32 [T][E]), equal values resolved to the lower expert id,
 * written in descending order to topk_idx (int32 [T][k]); topk_gate (fp32
 * [T][k]) = softmax over those k logits.  1 <= k <= min(E, 32), E <= 4096.
 * Logits must be finite. */
mok_status mok_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                          int32_t* topk_idx, float* topk_gate, hipStream_t stream);

/* Router GEMM fused with the route (article, routing paragraph: the router
 * scores every token against every expert, then picks).  logits[t][e] =
 * sum_h x[t][h] * w_router[e][h] over bf16 values with fp32 sums (products
 * exact, the sums' order the kernel's), then the picks and gates of
 * mok_route_topk.  The logits are never stored whole: per-split partial sums
 * go to ws and are added in split order, so results are deterministic.
 * x: bf16 [T][H]; w_router: bf16 [E][H] (nn.Linear layout); H a multiple of
 * 16; 1 <= k <= min(E, 32), E <= 4096.  ws: device scratch of
 * mok_route_gemm_workspace_size(T, E, H) bytes (MOK_ERR_WORKSPACE if
 * smaller); its contents on entry do not matter.  T = 0 does nothing. */
size_t mok_route_gemm_workspace_size(int32_t T, int32_t E, int32_t H);
mok_status mok_route_topk_gemm(const void* x, const void* w_router, int32_t T, int32_t H,
                               int32_t E, int32_t k, void* ws, size_t ws_bytes,
                               int32_t* topk_idx, float* topk_gate, hipStream_t stream);

/* Bytes of scratch mok_build_schedule needs. */
size_t mok_schedule_workspace_size(int64_t T, int32_t k, int32_t n_local);

/* Schedule (article, layout-planning paragraph; wiki key point on the pull
 * schedule).  Over the T*k assignments a = t*k + j of topk_idx (int32
 * [T][k]), local expert e = topk_idx - expert_base in [0, n_local):
 *   counts[e]  (int32 [n_local])    assignments to e
 *   offsets    (int32 [n_local+1])  exclusive prefix sum; R = offsets[n_local]
 *   slot_of_assign[a] (int32 [T*k]) offsets[e] + rank of a among e's
 *                                   assignments in increasing a; -1 if not local
 *   assign_of_slot[s] (int32 [T*k] capacity) inverse for s < R; entries >= R
 *                                   are left untouched.
 * The pull table entry of slot s is token assign_of_slot[s] / k, i.e.
 * (partition, row) = (token / part_rows, token % part_rows).
 * No sort and no host round trip.  T*k < 2^31. */
mok_status mok_build_schedule(const int32_t* topk_idx, int32_t T, int32_t k,
                              int32_t expert_base, int32_t n_local,
                              int32_t* counts, int32_t* offsets,
                              int32_t* slot_of_assign, int32_t* assign_of_slot,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* mok_build_schedule for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same schedule, bit for bit, with its scratch (the per-chunk
 * expert counts) in a fixed device array of the library, of
 * mok_schedule_noalloc_max_bytes() bytes (4 MiB) per GPU, held until the
 * process ends; its address on each device is looked up on the first call on
 * that device.  Calls nothing that allocates.  A schedule whose scratch
 * (mok_schedule_workspace_size) exceeds that size returns MOK_ERR_UNSUPPORTED
 * (e.g. more than 4.19 million assignments with 256 local experts).  All
 * calls on one GPU share the array: calls that overlap in time on one GPU
 * (concurrent streams) race and must not be issued.  Nothing in the array has
 * to start at zero; the last call's contents stay in it. */
size_t mok_schedule_noalloc_max_bytes(void);
mok_status mok_build_schedule_noalloc(const int32_t* topk_idx, int32_t T, int32_t k,
                                      int32_t expert_base, int32_t n_local, int32_t* counts,
                                      int32_t* offsets, int32_t* slot_of_assign,
                                      int32_t* assign_of_slot, hipStream_t stream);

/* Two-wave minibatch rule (article, minibatch paragraph; wiki key point on
 * minibatch size): M = 2 * n_cus * tile_m * tile_n / n_out rounded up to a
 * multiple of 64, clipped to `rows` when rows > 0.  Host only. */
int32_t mok_choose_minibatch(int32_t n_cus, int32_t tile_m, int32_t tile_n,
                             int32_t n_out, int64_t rows);

/* Minibatch windows.  win_seg (int32 [nwin][n_local+1]): for window b,
 * lo = min(b*M, R), hi = min((b+1)*M, R), win_seg[b][e] = clamp(offsets[e],
 * lo, hi); expert e's rows in window b are [win_seg[b][e], win_seg[b][e+1]). */
mok_status mok_build_windows(const int32_t* offsets, int32_t n_local, int32_t M,
                             int32_t nwin, int32_t* win_seg, hipStream_t stream);

/* mok_build_schedule and mok_build_windows in one call, as the fused layer
 * runs them (article, layout-planning and minibatch paragraphs): the same
 * counts, offsets, slot_of_assign, assign_of_slot and win_seg, bit for bit,
 * in two launches instead of three (the scatter's first block also writes
 * the window table once the offsets are known).  Arguments as in the two
 * calls; ws as for mok_build_schedule; nwin may be 0 (win_seg unused). */
mok_status mok_build_schedule_windows(const int32_t* topk_idx, int32_t T, int32_t k,
                                      int32_t expert_base, int32_t n_local, int32_t* counts,
                                      int32_t* offsets, int32_t* slot_of_assign,
                                      int32_t* assign_of_slot, int32_t M, int32_t nwin,
                                      int32_t* win_seg, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/* Pull dispatch (article, pull-dispatch paragraph).  For each slot s in
 * [slot_begin, min(slot_end, R)) with R = offsets[n_local]: ring row
 * s % ring_slots receives the row of token assign_of_slot[s] / k of src
 * (bf16, H values; H a multiple of 64).  MOK_ACT_BF16: ring holds
 * ring_slots x H bf16, a bit copy.  MOK_ACT_MXFP8_E4M3: ring holds
 * ring_slots x H E4M3 codes (u8) and ring_scales ring_slots x H/32 E8M0
 * scales (OCP MX v1.0 blocks of 32 along H).  Both column-blocked (see the
 * conventions above).
 * A token index outside src sets *dev_status = MOK_ERR_CAPACITY and the row
 * is skipped.  assign_of_slot is read at every slot of [slot_begin,
 * slot_end) (entries at or past R are ignored), so it holds slot_end
 * entries. */
mok_status mok_dispatch_gather(const mok_tokens* src, int32_t H, int32_t k,
                               const int32_t* assign_of_slot, const int32_t* offsets,
                               int32_t n_local, int32_t slot_begin, int32_t slot_end,
                               void* ring, uint8_t* ring_scales, int32_t ring_slots,
                               int32_t act_format, int32_t* dev_status,
                               hipStream_t stream);

/* Expert SwiGLU FFN as a grouped GEMM (article, layout-planning and
 * megakernel paragraphs; SwiGLU and MXFP8 in the state-machine paragraph).
 * For each slot s in [slot_begin, min(slot_end, R)) owned by local expert e
 * (offsets[e] <= s < offsets[e+1]), with x = ring row s % ring_slots:
 *   g = W_gu[e][0:I] . x,  u = W_gu[e][I:2I] . x      (fp32 accumulation)
 *   a = SiLU(g) * u  -> act row s % act_rows (bf16, or MXFP8 blocks of 32
 *                       along I into act and act_scales; both
 *                       column-blocked like the ring)
 *   y = W_d[e] . a   -> y row s % y_rows (bf16 [y_rows][H])
 * w_gate_up: bf16 [n_local][2I][H], rows 0..I-1 gate, I..2I-1 up; w_down:
 * bf16 [n_local][H][I]; no biases.  desc supplies H, I, n_local, act_format.
 * The ring and act formats follow desc->act_format.
 * ws / ws_bytes: optional workspace of mok_gemm_workspace_size() bytes for
 * the K split of a last, partial round of tiles (desc->no_split_k); NULL =
 * every tile whole.  Its contents must be zero before its first use; the
 * calls leave them zero, except after a device-side wait gave up (then the
 * workspace status word, read with mok_device_status, is MOK_ERR_DEVICE and
 * the workspace must be zeroed again).  One workspace serves one stream. */
mok_status mok_expert_ffn(const mok_layer_desc* desc, const void* ring,
                          const uint8_t* ring_scales, int32_t ring_slots,
                          const int32_t* offsets, int32_t slot_begin, int32_t slot_end,
                          const void* w_gate_up, const void* w_down,
                          void* act, uint8_t* act_scales, int32_t act_rows,
                          void* y, int32_t y_rows, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Bytes of the optional GEMM workspace of mok_expert_ffn, mok_expert_gate_up
 * and mok_expert_down on the current device: a status word, one counter and
 * one 256 x 256 fp32 partial tile per compute unit (64 MiB + 2 KiB on 256
 * CUs). */
size_t mok_gemm_workspace_size(void);

/* Weight packing (a layout of this library, not of the pages): one-time
 * rearrangement of w_gate_up and w_down into the tile order of the grouped
 * GEMMs, so that each load of a weight tile reads contiguous memory.  The
 * packed buffers (device, caller-owned, sizes from mok_packed_weights_size)
 * are then passed in place of the documented ones with desc->weights_packed
 * = 1; results are bit-identical.  The packed format depends on hidden,
 * inter, n_local, act_format and weight_format and is private to this
 * library version.  With desc->weight_format = MOK_W_MXFP8_E4M3 the packing
 * also quantises (OCP MX E4M3, blocks of 32 along the contraction dimension
 * of each weight row, the scale rule and rounding of the MXFP8 activations):
 * the results are then those of the quantised weights.
 * Either pair (source, packed) may be null to pack only the other; a pair
 * with one null pointer is MOK_ERR_INVALID_ARG.  Asynchronous on stream. */
mok_status mok_packed_weights_size(const mok_layer_desc* desc, size_t* gate_up_bytes,
                                   size_t* down_bytes);
mok_status mok_pack_weights(const mok_layer_desc* desc, const void* w_gate_up, const void* w_down,
                            void* packed_gate_up, void* packed_down, hipStream_t stream);

/* The two grouped GEMMs of mok_expert_ffn as separate calls, same layouts
 * and workspace rule: gate/up + SwiGLU (ring -> act) and down (act -> y). */
mok_status mok_expert_gate_up(const mok_layer_desc* desc, const void* ring,
                              const uint8_t* ring_scales, int32_t ring_slots,
                              const int32_t* offsets, int32_t slot_begin, int32_t slot_end,
                              const void* w_gate_up, void* act, uint8_t* act_scales,
                              int32_t act_rows, void* ws, size_t ws_bytes, hipStream_t stream);
mok_status mok_expert_down(const mok_layer_desc* desc, const void* act,
                           const uint8_t* act_scales, int32_t act_rows,
                           const int32_t* offsets, int32_t slot_begin, int32_t slot_end,
                           const void* w_down, void* y, int32_t y_rows, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Push combine + final weighted merge (article, push-combine and benchmark
 * scope paragraphs).  For each token t with at least one local assignment
 * (slot_of_assign[t*k+j] >= 0):
 *   out[t] = bf16( sum over j ascending, local, of gate[t][j] * y[slot] )
 * accumulated in fp32 fma from 0.  y is bf16 [y_rows][H] indexed by slot.
 * Rows of tokens with no local assignment are not written.  A slot >= y_rows
 * sets *dev_status = MOK_ERR_CAPACITY and contributes nothing. */
mok_status mok_combine(const void* y, int32_t y_rows, const int32_t* slot_of_assign,
                       const float* topk_gate, int32_t T, int32_t k, int32_t H,
                       const mok_tokens* out, int32_t* dev_status, hipStream_t stream);

/* The same merge driven by the routed slots: slot s < min(R, n_slots) merges
 * token assign_of_slot[s] / k when s is that token's smallest local slot, so
 * each token with a local assignment is written once and only R slots are
 * visited instead of all T tokens.  Output identical to mok_combine.
 * assign_of_slot is read at every slot s < n_slots, so it holds n_slots
 * entries.
 * offsets: int32 [n_local + 1] (R = offsets[n_local]). */
mok_status mok_combine_slots(const void* y, int32_t y_rows, const int32_t* assign_of_slot,
                             const int32_t* offsets, int32_t n_local, int32_t n_slots,
                             const int32_t* slot_of_assign, const float* topk_gate, int32_t k,
                             int32_t H, const mok_tokens* out, int32_t* dev_status,
                             hipStream_t stream);

/* The down GEMM with the merge of single-slot tokens in its epilogue (the
 * article's push combine: a result goes straight back to its token).  For
 * each slot s in [slot_begin, min(slot_end, R)) with a = assign_of_slot[s],
 * t = a / k (k = desc->top_k): if s is t's only local slot (exactly one
 * slot_of_assign[t][j] >= 0), out row t = bf16(fma(topk_gate[a], y_s, 0))
 * with y_s the bf16 result, which is what mok_combine_slots writes for a
 * single term; every other slot's y_s goes to y as mok_expert_down writes it.
 * mok_expert_down_merge over all routed slots followed by
 * mok_combine_slots_multi writes the same out, bit for bit, as
 * mok_expert_down followed by mok_combine_slots; y then holds only the rows
 * of tokens with several local slots (a forward whose y the backward reads
 * uses mok_expert_down).  Arguments as mok_expert_down and mok_combine_slots
 * (slot_of_assign: T x k, topk_gate: T x k, out: the tokens' output rows,
 * H = desc->hidden wide; slot_end <= y_rows).  merge_plan: caller scratch of
 * 16 * y_rows bytes (device), where a first launch writes, per slot, the
 * output row's address and the gate, which the GEMM's epilogue reads. */
mok_status mok_expert_down_merge(const mok_layer_desc* desc, const void* act,
                                 const uint8_t* act_scales, int32_t act_rows,
                                 const int32_t* offsets, int32_t slot_begin, int32_t slot_end,
                                 const void* w_down, void* y, int32_t y_rows,
                                 const int32_t* assign_of_slot, const int32_t* slot_of_assign,
                                 const float* topk_gate, const mok_tokens* out, void* merge_plan,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* mok_combine_slots for the tokens with at least two local slots only (the
 * others are written by mok_expert_down_merge).  A single-slot token outside
 * the out partitions still sets *dev_status = MOK_ERR_CAPACITY. */
mok_status mok_combine_slots_multi(const void* y, int32_t y_rows, const int32_t* assign_of_slot,
                                   const int32_t* offsets, int32_t n_local, int32_t n_slots,
                                   const int32_t* slot_of_assign, const float* topk_gate,
                                   int32_t k, int32_t H, const mok_tokens* out,
                                   int32_t* dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward of the layer's share (the pages report the backward pass next to
 * the forward; the reverse of pull dispatch and push combine).  bf16
 * activations and weights.  Per routed slot s of token t, pick j, local
 * expert e, gate w = topk_gate[t][j], with x_s the token's row,
 * h_s = W_gu[e] x_s = [g, u], a_s = SiLU(g) u, y_s = W_d[e] a_s and
 * out[t] = sum_j w y_s:
 *   dy_s    = w dout[t]                           (mok_combine_backward)
 *   dgate   = <dout[t], y_s>                      (mok_combine_backward)
 *   da_s    = W_d[e]^T dy_s
 *   dg = da u SiLU'(g),  du = da SiLU(g),  SiLU'(g) = s (1 + g (1 - s)),
 *   s = 1 / (1 + e^-g)                            (mok_expert_ffn_backward)
 *   dx_s    = W_gu[e]^T [dg, du]                  (mok_expert_ffn_backward)
 *   dx[t]   = sum_j dx_s                          (mok_dispatch_backward)
 *   dW_d[e] = sum_s dy_s a_s^T, dW_gu[e] = sum_s [dg, du]_s x_s^T
 *                                                 (mok_expert_wgrad)
 * Storage is bf16, sums fp32.
 * ------------------------------------------------------------------------ */

/* Bytes of the transposed packed weights the backward GEMMs read:
 * W_gu^T (n_local x H x 2I) and W_d^T (n_local x I x H).  The packing follows
 * desc->act_format (the backward GEMMs' k-step differs for MXFP8 tokens) and
 * desc->weight_format: with MOK_W_MXFP8_E4M3 (MXFP8 tokens, packed forward
 * weights) the transposed weights are quantised to OCP MX E4M3 along the
 * backward GEMMs' contraction dimension (W_d along H, W_gu along 2I: blocks of
 * 32 down each column of the forward's matrices), and the down and gate/up
 * dgrads run on the block-scaled FP8 MFMA. */
mok_status mok_packed_weights_bwd_size(const mok_layer_desc* desc, size_t* gate_up_t_bytes,
                                       size_t* down_t_bytes);
/* Packs them from the bf16 weights of mok_expert_ffn's layout (either pair of
 * pointers may be null; bf16 sources also for MXFP8 weights). */
mok_status mok_pack_weights_bwd(const mok_layer_desc* desc, const void* w_gate_up,
                                const void* w_down, void* packed_gate_up_t, void* packed_down_t,
                                hipStream_t stream);

/* Backward of the weighted merge: for each routed slot s < min(n_slots, R),
 * with a = assign_of_slot[s], t = a / k: dy row s % dy_rows = bf16(w dout[t])
 * (dy bf16, dy_rows x H, column-blocked like the ring) and dgate[a] =
 * sum_h dout[t][h] y[s][h] in fp32 (y: the forward's return area, bf16
 * [y_rows][H] indexed by slot).  dgate entries of non-local assignments are
 * not written.  dout: bf16 rows of the pool's tokens (mok_tokens).  H a
 * multiple of 64.  A token outside dout or s >= y_rows sets
 * *dev_status = MOK_ERR_CAPACITY and the slot is skipped. */
mok_status mok_combine_backward(const mok_tokens* dout, const void* y, int32_t y_rows,
                                const int32_t* assign_of_slot, const int32_t* offsets,
                                int32_t n_local, int32_t n_slots, const float* topk_gate,
                                int32_t k, int32_t H, void* dy, int32_t dy_rows, float* dgate,
                                int32_t* dev_status, hipStream_t stream);

/* Backward of the expert FFN for slots [slot_begin, min(slot_end, R)):
 * recomputes h (bf16, rows x 2I, row-major, row s % rows) from the ring (row
 * s % ring_slots) and w_gate_up (packed as desc->weights_packed says, as for
 * the forward), then da = dy W_d with the
 * SwiGLU backward in its epilogue (dh: bf16 rows x 2I, column-blocked), then
 * dx_s = dh W_gu (bf16 [rows][H], row-major, row s % rows).  h, dh and
 * dx_slots are caller scratch / output; the packed weights come from
 * mok_pack_weights_bwd.  Each buffer must stay below 4 GiB
 * (MOK_ERR_UNSUPPORTED). */
mok_status mok_expert_ffn_backward(const mok_layer_desc* desc, const void* ring,
                                   int32_t ring_slots, const void* dy, const int32_t* offsets,
                                   int32_t slot_begin, int32_t slot_end, const void* w_gate_up,
                                   const void* packed_gate_up_t, const void* packed_down_t,
                                   void* h, void* dh, void* dx_slots, int32_t rows,
                                   hipStream_t stream);

/* The forward's gate/up + SwiGLU (as mok_expert_gate_up, bf16 tokens and
 * weights only) that also stores h = [g, u]: bf16 [act_rows][2I], row-major,
 * row = the act row of the slot (s % act_rows), so the backward can take h
 * instead of recomputing it (mok_expert_ffn_backward_saved).  act is
 * bit-identical to mok_expert_gate_up's given the same workspace argument.
 * Without a workspace, h is bit-identical to the backward's recompute; with
 * one, tiles of a last, partial round may be split along K, and their h is
 * then the rounding of the pieces' fp32 partial sums added in piece order (a
 * different summation order, same bar).  Costs 2I bf16 per row of extra
 * writes.  Either buffer at 4 GiB or more: MOK_ERR_UNSUPPORTED. */
mok_status mok_expert_gate_up_save_h(const mok_layer_desc* desc, const void* ring,
                                     int32_t ring_slots, const int32_t* offsets,
                                     int32_t slot_begin, int32_t slot_end, const void* w_gate_up,
                                     void* act, int32_t act_rows, void* h, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* mok_expert_ffn_backward with h taken from mok_expert_gate_up_save_h
 * (rows = the forward's act_rows) instead of recomputed: the down dgrad with
 * the SwiGLU backward, then the gate/up dgrad; the same outputs, bit for bit,
 * when h was kept without a K-split workspace. */
mok_status mok_expert_ffn_backward_saved(const mok_layer_desc* desc, const void* dy,
                                         const int32_t* offsets, int32_t slot_begin,
                                         int32_t slot_end, const void* packed_gate_up_t,
                                         const void* packed_down_t, const void* h, void* dh,
                                         void* dx_slots, int32_t rows, hipStream_t stream);

/* Weight gradients over every routed slot s < R = offsets[n_local], per local
 * expert e (slots offsets[e] .. offsets[e+1] - 1):
 *   dW_down[e]    = sum_s dy_s a_s^T      bf16 [n_local][H][I]
 *   dW_gate_up[e] = sum_s dh_s x_s^T      bf16 [n_local][2I][H]
 * fp32 sums, bf16 results (either output may be null).  Inputs are the
 * forward's ring (x, row s % ring_slots) and act (a, row s % act_rows) and
 * the backward's dy (row s % rows, H) and dh (row s % rows, 2I), all
 * column-blocked.  ws: mok_wgrad_workspace_size(desc, rows) bytes of device
 * scratch (the operands transposed to slot-contiguous rows over a slot axis
 * padded to 32 per expert).  rows must be >= R; offsets that claim more
 * slots than rows allow leave every access in bounds, but the gradients are
 * then not meaningful. */
size_t mok_wgrad_workspace_size(const mok_layer_desc* desc, int32_t rows);
mok_status mok_expert_wgrad(const mok_layer_desc* desc, const void* ring, int32_t ring_slots,
                            const void* act, int32_t act_rows, const void* dy, const void* dh,
                            int32_t rows, const int32_t* offsets, void* dw_gate_up,
                            void* dw_down, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MXFP8 backward (the article reports the MXFP8 backward beside the bf16 one;
 * MXFP8 quantisation sits in the data path).  desc->act_format =
 * MOK_ACT_MXFP8_E4M3 with bf16 weights: the forward's ring and act are MXFP8,
 * and so are the backward's token operands dy (blocks of 32 along H) and dh
 * (blocks of 32 along 2I: the dg blocks, then the du blocks), each as E4M3
 * codes (u8, column-blocked like the ring) and E8M0 scales (pairs, as the
 * ring's).  h, dx_slots, dx and the weight gradients stay bf16, the sums
 * fp32.  The steps and their order are the bf16 backward's above.
 * ------------------------------------------------------------------------ */

/* mok_combine_backward with MXFP8 dy: the fp32 products w dout[t][h] of a
 * slot quantised per block of 32 along H (OCP MX v1.0: scale 2^E with E =
 * floor(log2 amax) - 8, codes rounded to nearest even, saturating at 448)
 * into dy (dy_rows x H codes) and dy_scales (dy_rows x H/32).  dgate as
 * mok_combine_backward. */
mok_status mok_combine_backward_mx(const mok_tokens* dout, const void* y, int32_t y_rows,
                                   const int32_t* assign_of_slot, const int32_t* offsets,
                                   int32_t n_local, int32_t n_slots, const float* topk_gate,
                                   int32_t k, int32_t H, void* dy, uint8_t* dy_scales,
                                   int32_t dy_rows, float* dgate, int32_t* dev_status,
                                   hipStream_t stream);

/* The forward's gate/up + SwiGLU with MXFP8 tokens and act (as
 * mok_expert_gate_up; bf16 or packed MXFP8 weights) that also stores
 * h = [g, u] in bf16 as mok_expert_gate_up_save_h does.  act and act_scales are bit-identical to
 * mok_expert_gate_up's given the same workspace argument; without a workspace
 * h is bit-identical to the backward's recompute. */
mok_status mok_expert_gate_up_save_h_mx(const mok_layer_desc* desc, const void* ring,
                                        const uint8_t* ring_scales, int32_t ring_slots,
                                        const int32_t* offsets, int32_t slot_begin,
                                        int32_t slot_end, const void* w_gate_up, void* act,
                                        uint8_t* act_scales, int32_t act_rows, void* h, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

/* mok_expert_ffn_backward (h_kept = 0: h recomputed from the MXFP8 ring and
 * w_gate_up) or mok_expert_ffn_backward_saved (h_kept != 0: h from
 * mok_expert_gate_up_save_h_mx, rows = its act_rows; ring, ring_scales and
 * w_gate_up are not read) with MXFP8 dy in and MXFP8 dh out: dh = [dg, du]
 * of the SwiGLU backward quantised per block of 32 along 2I (as dy) into dh
 * (rows x 2I codes) and dh_scales (rows x 2I/32); dx_s = dh W_gu in bf16.
 * The packed weights come from mok_pack_weights_bwd with this desc.  With
 * desc->weight_format = MOK_W_MXFP8_E4M3, w_gate_up is the forward's packed
 * MXFP8 gate/up (the recompute of h) and all three GEMMs run on the
 * block-scaled FP8 MFMA. */
mok_status mok_expert_ffn_backward_mx(const mok_layer_desc* desc, const void* ring,
                                      const uint8_t* ring_scales, int32_t ring_slots,
                                      const void* dy, const uint8_t* dy_scales,
                                      const int32_t* offsets, int32_t slot_begin, int32_t slot_end,
                                      const void* w_gate_up, const void* packed_gate_up_t,
                                      const void* packed_down_t, void* h, int32_t h_kept, void* dh,
                                      uint8_t* dh_scales, void* dx_slots, int32_t rows,
                                      hipStream_t stream);

/* mok_expert_wgrad over MXFP8 operands (the ring, act, dy and dh with their
 * scales): each operand's values, code x 2^E, enter the fp32 sums exactly
 * (converted to bf16 in the slot transposes: exact for every value of at
 * least 2^-133).  ws: mok_wgrad_workspace_size(desc, rows) bytes. */
mok_status mok_expert_wgrad_mx(const mok_layer_desc* desc, const void* ring,
                               const uint8_t* ring_scales, int32_t ring_slots, const void* act,
                               const uint8_t* act_scales, int32_t act_rows, const void* dy,
                               const uint8_t* dy_scales, const void* dh, const uint8_t* dh_scales,
                               int32_t rows, const int32_t* offsets, void* dw_gate_up,
                               void* dw_down, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of the pull dispatch (a push of gradients back to the tokens):
 * dx[t] = bf16(sum over t's local slots s, ascending j, of dx_slots row s)
 * in fp32, written at t's smallest local slot like mok_combine_slots (unit
 * gates).  Tokens without a local slot are not written. */
mok_status mok_dispatch_backward(const void* dx_slots, int32_t rows,
                                 const int32_t* assign_of_slot, const int32_t* offsets,
                                 int32_t n_local, int32_t n_slots, const int32_t* slot_of_assign,
                                 int32_t k, int32_t H, const mok_tokens* dx, int32_t* dev_status,
                                 hipStream_t stream);

/* Bytes of workspace mok_moe_forward, mok_moe_forward_routed and
 * mok_moe_forward_batches need for T source tokens per macrobatch and n_macro
 * macrobatches. */
size_t mok_forward_workspace_size(const mok_layer_desc* desc, int32_t T, int32_t n_macro);

/* The fused layer (article, routing, megakernel, minibatch and ring-buffer
 * paragraphs): route, schedule, windows, pull dispatch into the fixed ring,
 * grouped SwiGLU FFN, push of y into a return area indexed by slot, weighted
 * merge into out.  logits: fp32 [T][desc->n_experts] router scores of the T
 * tokens of x (finite; n_experts <= 4096); they are routed here as by
 * mok_route_topk (k = desc->top_k), into the workspace, and the route also
 * counts the picks of local experts for the schedule (one launch).
 * MOK_MODE_STREAM issues stream-ordered launches per window;
 * MOK_MODE_PERSISTENT runs the windows in one cooperative kernel whose
 * workgroups split into data movers and MFMA workers that signal through
 * device counters.  If R exceeds desc->max_rows the status word becomes
 * MOK_ERR_CAPACITY and out is left untouched.  T = 0 writes nothing (logits
 * may then be null). */
mok_status mok_moe_forward(const mok_layer_desc* desc, const float* logits, int32_t T,
                           const mok_tokens* x, const void* w_gate_up, const void* w_down,
                           const mok_tokens* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* The fused layer from the router weights (article, routing paragraph: the
 * router scores every token against every expert, then picks): the router
 * GEMM of the tokens' rows x with w_router (bf16 [n_experts][H], nn.Linear
 * layout; H a multiple of 16) as mok_route_topk_gemm computes it (fp32 sums,
 * splits of H added in split order), whose pick kernel also counts the local
 * picks for the schedule; then the steps of mok_moe_forward.  ws: at least
 * mok_forward_router_workspace_size(desc, T) bytes (the fused call's bytes
 * plus the router GEMM's partial sums). */
size_t mok_forward_router_workspace_size(const mok_layer_desc* desc, int32_t T);
mok_status mok_moe_forward_router(const mok_layer_desc* desc, const void* w_router, int32_t T,
                                  const mok_tokens* x, const void* w_gate_up, const void* w_down,
                                  const mok_tokens* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* The fused layer from routing decided elsewhere (one GPU's expert share:
 * the sources route their own tokens, and this GPU schedules every source's
 * picks of its local experts; article, routing and pull-dispatch
 * paragraphs).  topk_idx / topk_gate: int32 / fp32 [T][k] over the pool of T
 * tokens; otherwise as mok_moe_forward. */
mok_status mok_moe_forward_routed(const mok_layer_desc* desc, const int32_t* topk_idx,
                                  const float* topk_gate, int32_t T, const mok_tokens* x,
                                  const void* w_gate_up, const void* w_down,
                                  const mok_tokens* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* n_macro macrobatches through one ring (article, ring-buffer paragraph:
 * the next macrobatch's dispatch overlaps the previous one's combine).
 * topk_idx / topk_gate / out are HOST arrays of n_macro entries (device
 * pointers / host mok_tokens); all macrobatches share x, the weights and T. */
mok_status mok_moe_forward_batches(const mok_layer_desc* desc, int32_t n_macro,
                                   const int32_t* const* topk_idx,
                                   const float* const* topk_gate, int32_t T,
                                   const mok_tokens* x, const void* w_gate_up,
                                   const void* w_down, const mok_tokens* out,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Tuner of the fused call (article, minibatch paragraph: the minibatch, and
 * the share of CUs that move data, have to be retuned for every hidden size,
 * top-k and expert size).  For every candidate pair (minibatch[i],
 * n_move[j]) -- the other fields from desc; n_move applies in
 * MOK_MODE_PERSISTENT only, and n_n_move = 0 keeps desc->n_move_cus -- runs
 * mok_moe_forward_batches on the caller's inputs once untimed and `reps`
 * times between two HIP events, and writes the fastest candidate's
 * descriptor to *best and its mean time per call (ms) to *best_ms.
 * Candidates whose workspace exceeds ws_bytes, or whose calls fail or end
 * with a device status other than MOK_OK, are skipped; MOK_ERR_UNSUPPORTED
 * if none is left.  Synchronises `stream` (host-side timing); out is
 * written by every run.  Meant for set-up, not for the serving loop. */
mok_status mok_tune_forward(const mok_layer_desc* desc, const int32_t* minibatch,
                            int32_t n_minibatch, const int32_t* n_move, int32_t n_n_move,
                            int32_t reps, int32_t n_macro, const int32_t* const* topk_idx,
                            const float* const* topk_gate, int32_t T, const mok_tokens* x,
                            const void* w_gate_up, const void* w_down, const mok_tokens* out,
                            void* ws, size_t ws_bytes, mok_layer_desc* best, float* best_ms,
                            hipStream_t stream);

/* Synchronises `stream`, then copies the workspace status word to
 * *status_host (MOK_OK, MOK_ERR_CAPACITY or MOK_ERR_DEVICE). */
mok_status mok_device_status(const void* ws, int32_t* status_host, hipStream_t stream);

/* Minibatch the fused call uses for desc: desc->minibatch if set (clipped to
 * the row capacity), else the two-wave rule (mok_choose_minibatch) for each
 * of a window's GEMMs on this device's CUs with 256 x 256 tiles -- gate/up
 * (n_out = 2I) and down (n_out = H) -- the larger of the two, so that both
 * fill at least two waves.  Host only. */
int32_t mok_forward_minibatch(const mok_layer_desc* desc, int32_t T);

const char* mok_status_str(mok_status s);

/* Text of the last HIP error a call on this host thread turned into
 * MOK_ERR_HIP ("no error" if none). */
const char* mok_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOK_H */
