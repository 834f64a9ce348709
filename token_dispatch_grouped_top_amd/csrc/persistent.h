// persistent.h -- the one-kernel pipeline of the fused layer (internal).
#pragma once

#include "mok_internal.h"

namespace mok {

// Device buffers of one macrobatch inside the fused call's workspace.
struct MacroBuffers {
  int32_t* counts;    // [n_local]
  int32_t* offsets;   // [n_local + 1]; R = offsets[n_local]
  int32_t* soa;       // slot_of_assign [T*k]
  int32_t* aos;       // assign_of_slot [T*k]
  int32_t* win;       // win_seg [nwin][n_local + 1]
  const float* gate;  // topk_gate [T*k]
  uint16_t* y;        // return area bf16 [cap][H], indexed by slot
  mok_tokens out;     // destination partitions
  void* plan;         // merge plan of the down GEMM's epilogue: 16 bytes per slot [cap]
};

struct PersistentArgs {
  int32_t n_macro;
  const MacroBuffers* mb;   // host array [n_macro]
  int32_t T, k, H, I, n_local, act_format;
  int32_t M, S, nwin, cap;
  mok_tokens x;
  const uint16_t* w_gu;
  const uint16_t* w_d;
  int32_t w_packed;         // weights in the packed tile order
  int32_t weight_format;    // mok_weight_format (MXFP8 weights: packed, MXFP8 activations)
  void* ring; uint8_t* ring_sc;
  void* act; uint8_t* act_sc; int32_t act_rows;
  int32_t* status;
  void* pers_ws;
  int32_t n_move;           // 0 = auto
  int32_t n_cus;
  int32_t timeout_us;       // bound of every device-side wait; 0 = 2 s
};

// Macrobatches handled by one persistent launch (more are run in groups).
constexpr int kPersistMaxMacro = 16;

size_t persistent_ws_bytes(int64_t total_windows);
mok_status launch_persistent(const PersistentArgs& a, hipStream_t s);

}  // namespace mok
