// mok_internal.h -- device helpers and launcher declarations shared by the
// libmok HIP sources (gfx950 / CDNA4, wave64).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mok.h"

namespace mok {

constexpr int kWave = 64;

// ----------------------------------------------------------------- bf16
// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32, two
// values per instruction.  (A bit-pattern rounding with a NaN test costs a
// branch per value; in the down GEMM's epilogue that was a sixth of the
// launch.)
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Streaming stores of rows that are written once and read by a later kernel.
// Non-temporal stores: with ordinary ones, rows written by one wave in pieces
// reach HBM as partial lines under eviction pressure (a row gather measured
// 1.84x its bytes written and ran at 4.2 TB/s; 1.00x and 6.5 TB/s with these).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_nt(uint4* p, uint4 v) {
  const u32x4_nt w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_nt*>(p));
}
__device__ __forceinline__ void st_nt(uint2* p, uint2 v) {
  const u32x2_nt w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2_nt*>(p));
}
// Streaming loads of rows read once (the gather's source rows): in the layer
// step the gather went 57 -> 51 us with these, the rows no longer pushing the
// GEMMs' operands out of the caches.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4_nt w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}

// ------------------------------------------------ column-blocked row buffers
// The buffers the grouped GEMMs read as their token operand (the ring and
// the activation buffer) hold each row in 64-byte column blocks, block-major:
// block b (32 bf16 or 64 E4M3 values) of row r sits at byte (b * rows + r) *
// 64.  A GEMM k-step of a 256-row tile is then 16 KiB of contiguous memory,
// fetched in whole 128-byte lines.  E8M0 scales go in pairs (the two blocks
// of 32 of a 64-value block): scale j of row r at byte (j / 2 * rows + r) *
// 2 + j % 2.
constexpr int kColBlock = 64;
__device__ __forceinline__ int64_t colblk_byte(int64_t r, int64_t rows, int64_t byte_in_row) {
  return ((byte_in_row >> 6) * rows + r) * kColBlock + (byte_in_row & 63);
}
__device__ __forceinline__ int64_t scale_byte(int64_t r, int64_t rows, int64_t j) {
  return ((j >> 1) * rows + r) * 2 + (j & 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt));
}

// --------------------------------------------------------- MXFP8 (E4M3)
// OCP MX v1.0 block scale from the block's largest magnitude (fp32):
// E = floor(log2 amax) - 8, clamped to [-127, 127]; zero block -> -127.
// Read off the exponent field: amax below 2^-126 clamps to -127 anyway.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  int ef = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);
  int E = ef - 127 - 8;
  return E < -127 ? -127 : E;
}

// E4M3 code of v * 2^-E: round to nearest even, saturate at 448, keep the
// sign of v (also for results that round to zero).
__device__ __forceinline__ uint32_t e4m3_code_scaled(float v, int E) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = __builtin_amdgcn_ldexpf(fabsf(v), -E);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7eu;
  } else if (a < 0.015625f) {              // below 2^-6: subnormal quantum 2^-9
    mag = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));  // 0..8; 8 == code of 2^-6
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7ffffu + ((u >> 20) & 1u);      // RNE to 3 mantissa bits
    mag = (u >> 20) - ((127u - 7u) << 3);  // rebias exponent 127 -> 7
    if (mag > 0x7eu) mag = 0x7eu;
  }
  return sign | mag;
}

// ------------------------------------------------------------ wave ops
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Lanes holding the same key as this lane (all 64 lanes must be active).
__device__ __forceinline__ uint64_t match_key(uint32_t key, int nbits) {
  uint64_t peers = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    uint64_t bal = __ballot((key >> b) & 1u);
    peers &= ((key >> b) & 1u) ? bal : ~bal;
  }
  return peers;
}

// --------------------------------------------------------- device status
__device__ __forceinline__ void set_status(int32_t* st, int32_t code) {
  if (st) __hip_atomic_fetch_max(st, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------- launchers
// All launchers return hipSuccess or the launch error.
int32_t route_gemm_splits(int32_t T, int32_t E, int32_t H);
// Counting of local picks into the schedule's chunk counts by a route kernel
// (blk_counts null: no counting).
struct RouteCount {
  int32_t base = 0, n_local = 0;
  int32_t* blk_counts = nullptr;
  int32_t nblk = 0;
};
// Router GEMM + pick; token rows from x [T][H] or, x_parts non-null, from
// partitions of x_part_rows rows.
hipError_t launch_route_topk_gemm(const uint16_t* x, void* const* x_parts, int32_t x_part_rows,
                                  const uint16_t* w_router, int32_t T, int32_t H, int32_t E,
                                  int32_t k, float* partial, int32_t* idx, float* gate,
                                  const RouteCount& rc, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                             int32_t* idx, float* gate, hipStream_t s);

// The schedule counts assignments in chunks of kSchedChunk (a = t*k + j):
// blk_counts[e][c] = local assignments to expert e in chunk c.
constexpr int kSchedChunk = 2048;
struct SchedWs {
  int32_t* blk_counts;  // [n_local][nblk]
  int32_t nblk;
};
size_t sched_ws_bytes(int64_t A, int32_t n_local);
SchedWs sched_ws_carve(void* ws, int64_t A, int32_t n_local);
hipError_t launch_schedule(const int32_t* idx, int64_t A, int32_t expert_base, int32_t n_local,
                           int32_t* counts, int32_t* offsets, int32_t* soa, int32_t* aos,
                           const SchedWs& w, hipStream_t s);
hipError_t launch_windows(const int32_t* offsets, int32_t n_local, int32_t M, int32_t nwin,
                          int32_t* win_seg, hipStream_t s);
// The fused layer's schedule.  route_logits non-null: the route of the T
// tokens from fp32 logits [T][E] writes idx / gate and counts its local picks
// into the chunk counts (zeroed by the caller beforehand) in the same launch;
// null: idx is given and counted by the count kernel (counted: the caller's
// route already filled the chunk counts).  Then the scatter,
// which also writes the window table (M, nwin) and raises MOK_ERR_CAPACITY in
// *status when R > cap.  Two launches either way.
hipError_t launch_route_schedule(const float* route_logits, int32_t E, float* gate,
                                 int32_t* idx, int64_t T, int32_t k, int32_t expert_base,
                                 int32_t n_local, int32_t* counts, int32_t* offsets, int32_t* soa,
                                 int32_t* aos, const SchedWs& w, int32_t M, int32_t nwin,
                                 int32_t* win_seg, int32_t cap, int32_t* status, hipStream_t s,
                                 bool counted = false);
hipError_t launch_route_count(const float* logits, int32_t T, int32_t E, int32_t k,
                              int32_t expert_base, int32_t n_local, int32_t* idx, float* gate,
                              int32_t* blk_counts, int32_t nblk, hipStream_t s);

hipError_t launch_gather(void* const* part_ptr, int32_t n_part, int32_t part_rows, int32_t H,
                         int32_t k, const int32_t* aos, const int32_t* offsets, int32_t n_local,
                         int32_t s_begin, int32_t s_end, void* ring, uint8_t* ring_scales,
                         int32_t ring_slots, int32_t act_format, int32_t* status, hipStream_t s);

hipError_t launch_combine(const void* y, int32_t y_rows, const int32_t* soa, const float* gate,
                          int32_t T, int32_t k, int32_t H, void* const* out_ptr, int32_t n_part,
                          int32_t part_rows, int32_t* status, bool abort_on_status,
                          hipStream_t s);

// Backward of the merge, one wave per routed slot: dy (column-blocked) and
// dgate.
hipError_t launch_unmerge_slots(void* const* dout_ptr, int32_t n_part, int32_t part_rows,
                                const void* y, int32_t y_rows, const int32_t* aos,
                                const int32_t* offsets, int32_t n_local, int32_t n_slots,
                                const float* gate, int32_t k, int32_t H, void* dy,
                                uint8_t* dy_scales, int32_t dy_rows, float* dgate, int32_t* status,
                                hipStream_t s);

// Merge driven by routed slots: each token merged at its smallest local slot
// (gate null: unit gates, i.e. the plain sum of the token's slot rows).
hipError_t launch_combine_slots(const void* y, int32_t y_rows, const int32_t* aos,
                                const int32_t* offsets, int32_t n_local, int32_t n_slots,
                                const int32_t* soa, const float* gate, int32_t k, int32_t H,
                                void* const* out_ptr, int32_t n_part, int32_t part_rows,
                                int32_t* status, bool abort_on_status, hipStream_t s,
                                bool multi_only = false);

// Workspace of the K split of the GEMMs' last, partial round of tiles:
// [n_cus arrival counters, padded to 256 bytes][n_cus fp32 partial tiles of
// 256 x 256].  Counters are zero between launches.
struct SplitWs {
  int32_t* cnt;
  float* part;              // null: no split
  int32_t n_cus;            // the device's CUs (set with or without a split)
};
size_t split_ws_bytes(int32_t n_cus);
SplitWs split_ws_carve(void* ws, int32_t n_cus);

// Grouped GEMM pair of the expert FFN over slots [s_begin, min(s_end, R)).
// The merge of single-slot tokens in the down GEMM's epilogue (aos null: none):
// launch_merge_plan writes a 16-byte record per slot into plan (y_rows of them),
// which the epilogue reads.
struct MergeArgs {
  const int32_t* aos; const int32_t* soa; const float* gate; int32_t k;
  void* const* out_parts; int32_t n_part, part_rows;
  void* plan;
  const int32_t* status;      // non-null: no output row is written once it is raised
};
hipError_t launch_merge_plan(const int32_t* aos, const int32_t* offsets, int32_t n_local,
                             int32_t s0, int32_t s1, const int32_t* soa, const float* gate,
                             int32_t k, int32_t H, void* const* out_parts, int32_t n_part,
                             int32_t part_rows, void* plan, hipStream_t s);
struct FfnArgs {
  const void* ring; const uint8_t* ring_scales; int32_t ring_slots;
  const int32_t* offsets; int32_t n_local; int32_t s_begin, s_end;
  const uint16_t* w_gu; const uint16_t* w_d;
  void* act; uint8_t* act_scales; int32_t act_rows;
  void* y; int32_t y_rows;
  int32_t H, I, act_format;
  int32_t w_packed;           // weights in the packed tile order (launch_pack_weights)
  int32_t weight_format;      // MOK_W_MXFP8_E4M3: packed MXFP8 weights, both GEMMs in MXFP8
  SplitWs split;              // split.part null: every tile whole
  void* h_out;                // non-null (bf16 weights): the gate/up also stores h = [g, u]
  MergeArgs merge;            // down: single-slot tokens straight to their output rows
};
hipError_t launch_gate_up(const FfnArgs& a, hipStream_t s);
hipError_t launch_down(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s);
// Backward of the expert FFN over slots [s_begin, min(s_end, R)): h = x W_gu^T
// (recomputed, bf16 [rows][2I]); da = dy W_d and dh = SwiGLU backward (dh
// column-blocked [rows][2I]); dx_s = dh W_gu (bf16 [rows][H]).  Rows of slot s:
// s % rows in every buffer; x from the ring (row s % ring_slots).
struct BwdArgs {
  const void* ring; int32_t ring_slots;
  const uint8_t* ring_scales;  // MXFP8 tokens (mx): the ring's, dy's and dh's E8M0 scales
  const uint8_t* dy_scales;
  uint8_t* dh_scales;
  int32_t mx;
  int32_t w_mx8;              // MXFP8 weights: the block-scaled FP8 tile (mx too)
  const int32_t* offsets; int32_t n_local; int32_t s_begin, s_end;
  const uint16_t* w_gu;       // the forward's gate/up weights (the recompute of h)
  int32_t w_gu_packed;        // ... in the packed tile order
  const uint16_t* w_gu_t;     // packed W_gu^T (launch_pack_weights_bwd)
  const uint16_t* w_d_t;      // packed W_d^T
  const void* dy;             // column-blocked [rows][H]
  void* h; void* dh; void* dx;
  int32_t h_saved;            // h already holds [g, u] from the forward: no recompute
  int32_t rows;
  int32_t H, I;
  int32_t n_cus;              // the device's CUs (the dx_s GEMM's half-width tail); 0: none
};
hipError_t launch_ffn_backward(const BwdArgs& a, hipStream_t s);
// Weight gradients over all slots [0, R): dW_d = sum dy a^T, dW_gu = sum dh x^T
// per expert (bf16 [n_local][H][I] and [n_local][2I][H]); slot s's rows are
// s % rows (dy, dh), s % act_rows (act), s % ring_slots (ring); all
// column-blocked.  ws: wgrad_ws_bytes(rows, H, I, n_local).
struct WgradArgs {
  const void* ring; int32_t ring_slots;
  const void* act; int32_t act_rows;
  const void* dy; const void* dh; int32_t rows;
  // MXFP8 operands: E8M0 scales of each (all null for bf16 operands)
  const uint8_t* ring_scales; const uint8_t* act_scales;
  const uint8_t* dy_scales; const uint8_t* dh_scales;
  const int32_t* offsets; int32_t n_local;
  void* dw_gu; void* dw_d;
  void* ws;
  int32_t H, I;
};
int32_t wgrad_kpad(int32_t rows, int32_t n_local);
size_t wgrad_ws_bytes(int32_t rows, int32_t H, int32_t I, int32_t n_local);
hipError_t launch_wgrad(const WgradArgs& a, hipStream_t s);
size_t packed_bwd_gate_up_bytes(int32_t H, int32_t I, int32_t n_local, int32_t weight_format);
size_t packed_bwd_down_bytes(int32_t H, int32_t I, int32_t n_local, int32_t weight_format);
hipError_t launch_pack_weights_bwd(const uint16_t* w_gu, const uint16_t* w_d, int32_t H, int32_t I,
                                   int32_t n_local, bool act_mx, bool w_mx8, uint16_t* packed_gu_t,
                                   uint16_t* packed_d_t, hipStream_t s);

// Packed weights: bytes, and the packing launch (either source may be null).
size_t packed_gate_up_bytes(int32_t H, int32_t I, int32_t n_local, int32_t weight_format);
size_t packed_down_bytes(int32_t H, int32_t I, int32_t n_local, int32_t weight_format);
hipError_t launch_pack_weights(const uint16_t* w_gu, const uint16_t* w_d, int32_t H, int32_t I,
                               int32_t n_local, int32_t act_format, int32_t weight_format,
                               uint16_t* packed_gu, uint16_t* packed_d, hipStream_t s);

}  // namespace mok
