// abi.hip -- the extern "C" entry points of libmok: argument checks,
// workspace carving and the stream-ordered orchestration of the fused layer.
// The kernels live in route.hip, schedule.hip, movers.hip and gemm.hip; the
// persistent pipeline in persistent.hip.
#include <algorithm>
#include <atomic>
#include <cstring>

#include "mok_internal.h"
#include "persistent.h"

namespace mok {
namespace {

constexpr size_t kAlign = 256;
constexpr int kGemmTileM = 256, kGemmTileN = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Zeroes two ranges of int32 (the fused call's status word and counters).
__global__ void k_zero2(int32_t* a, int32_t na, int32_t* b, int32_t nb) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < na + nb; i += gridDim.x * blockDim.x) {
    if (i < na) a[i] = 0;
    else b[i - na] = 0;
  }
}

// Compute units of the current device, queried once per device.  Calls may
// run concurrently on several host threads: the cache is atomic, and two
// threads that both miss store the same value.
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

bool tokens_ok(const mok_tokens* t, int64_t T) {
  return t && t->part_ptr && t->n_partitions >= 1 && t->part_rows >= 1 &&
         static_cast<int64_t>(t->n_partitions) * t->part_rows >= T;
}

bool desc_ok(const mok_layer_desc* d) {
  if (!d) return false;
  if (d->hidden <= 0 || d->hidden % 64 != 0) return false;
  if (d->inter <= 0 || d->inter % 64 != 0) return false;
  if (d->weights_packed != 0 && d->weights_packed != 1) return false;
  if (d->n_local < 1 || d->n_local > 256) return false;
  if (d->top_k < 1 || d->top_k > 32 || d->top_k > d->n_experts) return false;
  if (d->expert_base < 0 || d->expert_base + d->n_local > d->n_experts) return false;
  if (d->act_format != MOK_ACT_BF16 && d->act_format != MOK_ACT_MXFP8_E4M3) return false;
  if (d->minibatch < 0 || d->ring_slots < 0 || d->max_rows < 0 || d->n_move_cus < 0 ||
      d->wait_timeout_us < 0)
    return false;
  if (d->mode != MOK_MODE_STREAM && d->mode != MOK_MODE_PERSISTENT) return false;
  if (d->no_split_k != 0 && d->no_split_k != 1) return false;
  if (d->weight_format != MOK_W_BF16 && d->weight_format != MOK_W_MXFP8_E4M3) return false;
  if (d->weight_format == MOK_W_MXFP8_E4M3 && d->act_format != MOK_ACT_MXFP8_E4M3) return false;
  return true;
}

// MXFP8 weights exist only in the packed form (mok_pack_weights quantises them).
bool weights_ok(const mok_layer_desc* d) {
  return d->weight_format == MOK_W_BF16 || d->weights_packed == 1;
}

// The GEMMs address their operands through raw buffer descriptors with
// 32-bit byte offsets: the ring, the activations and one expert's weights must
// each stay below 4 GiB (rows = 0: that operand is not used).
bool gemm_operands_fit(const mok_layer_desc* d, int64_t ring_rows, int64_t act_rows) {
  const int64_t eb = d->act_format == MOK_ACT_MXFP8_E4M3 ? 1 : 2;
  const int64_t lim = 1ll << 32;
  return ring_rows * d->hidden * eb < lim && act_rows * d->inter * eb < lim &&
         4ll * d->inter * d->hidden < lim;
}

// The K-split workspace of a standalone GEMM call: ws null = no split.  The
// CU count is passed either way (the down GEMM's half-width tail uses it).
mok_status gemm_split(const mok_layer_desc* d, void* ws, size_t ws_bytes, SplitWs& out) {
  out = SplitWs{};
  const int n_cus = device_cus();
  out.n_cus = n_cus;
  if (!ws || d->no_split_k) return MOK_OK;
  if (ws_bytes < split_ws_bytes(n_cus)) return MOK_ERR_WORKSPACE;
  out = split_ws_carve(ws, n_cus);
  return MOK_OK;
}

// Sizes of the fused call, derived from shapes only.
struct Plan {
  int64_t A;          // T*k assignments per macrobatch
  int32_t cap;        // row capacity (>= R expected)
  int32_t M, S;       // minibatch, ring rows
  int32_t nwin;       // windows planned per macrobatch
  int32_t act_rows;
  int32_t n_ybuf;     // return areas (2 when macrobatches overlap)
  bool split;         // stream mode with the GEMMs' K split (workspace at off_split)
  size_t off_status, off_split, off_sched, off_route_idx, off_route_gate, off_counts, off_offsets,
      off_soa, off_aos, off_win, off_ring, off_ring_sc, off_act, off_act_sc, off_y, off_plan,
      off_pers, total;
  size_t per_macro_counts, per_macro_offsets, per_macro_soa, per_macro_aos, per_macro_win;
};

// The two-wave rule for each of the window's GEMMs (gate/up: 2I output
// columns; down: H), the larger of the two: every GEMM of a window then fills
// at least two waves of the chip.
int32_t plan_minibatch(const mok_layer_desc* d, int64_t cap) {
  if (d->minibatch > 0) return static_cast<int32_t>(std::min<int64_t>(d->minibatch, std::max<int64_t>(cap, 1)));
  const int n = device_cus();
  const int32_t m = std::max(mok_choose_minibatch(n, kGemmTileM, kGemmTileN, 2 * d->inter, cap),
                             mok_choose_minibatch(n, kGemmTileM, kGemmTileN, d->hidden, cap));
  return std::max<int32_t>(m, 1);
}

bool make_plan(const mok_layer_desc* d, int32_t T, int32_t n_macro, Plan& p) {
  p.A = static_cast<int64_t>(T) * d->top_k;
  if (p.A >= (1ll << 31)) return false;
  int64_t cap = d->max_rows > 0 ? d->max_rows : p.A;
  if (cap < 1) cap = 1;
  p.cap = static_cast<int32_t>(cap);
  p.M = plan_minibatch(d, cap);
  p.S = d->ring_slots > 0 ? d->ring_slots : 2 * p.M;
  if (p.S < p.M) return false;
  if (d->mode == MOK_MODE_PERSISTENT && p.S < 2 * static_cast<int64_t>(p.M)) return false;
  p.nwin = static_cast<int32_t>((cap + p.M - 1) / p.M);
  p.act_rows = p.S;
  if (!gemm_operands_fit(d, p.S, p.act_rows)) return false;
  p.n_ybuf = n_macro > 1 ? 2 : 1;
  const bool mx = d->act_format == MOK_ACT_MXFP8_E4M3;
  const int64_t H = d->hidden, I = d->inter, nl = d->n_local;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  p.split = d->mode == MOK_MODE_STREAM && !d->no_split_k;
  p.off_status = take(kAlign);
  p.off_split = take(p.split ? split_ws_bytes(device_cus()) : 0);  // right after the status word
  p.off_sched = take(sched_ws_bytes(p.A, d->n_local));
  // routing of the logits-taking call (T x k ids and gates of one macrobatch)
  p.off_route_idx = take(static_cast<size_t>(std::max<int64_t>(p.A, 1)) * 4);
  p.off_route_gate = take(static_cast<size_t>(std::max<int64_t>(p.A, 1)) * 4);
  p.per_macro_counts = align_up(nl * 4);
  p.per_macro_offsets = align_up((nl + 1) * 4);
  p.per_macro_soa = align_up(std::max<int64_t>(p.A, 1) * 4);
  p.per_macro_aos = align_up(std::max<int64_t>(std::max<int64_t>(p.A, p.cap), 1) * 4);
  p.per_macro_win = align_up(static_cast<size_t>(p.nwin) * (nl + 1) * 4);
  p.off_counts = take(p.per_macro_counts * n_macro);
  p.off_offsets = take(p.per_macro_offsets * n_macro);
  p.off_soa = take(p.per_macro_soa * n_macro);
  p.off_aos = take(p.per_macro_aos * n_macro);
  p.off_win = take(p.per_macro_win * n_macro);
  p.off_ring = take(static_cast<size_t>(p.S) * H * (mx ? 1 : 2));
  p.off_ring_sc = take(mx ? static_cast<size_t>(p.S) * (H / 32) : 0);
  p.off_act = take(static_cast<size_t>(p.act_rows) * I * (mx ? 1 : 2));
  p.off_act_sc = take(mx ? static_cast<size_t>(p.act_rows) * (I / 32) : 0);
  p.off_y = take(static_cast<size_t>(p.n_ybuf) * p.cap * H * 2);
  // merge plans of the down GEMM's epilogue: 16 bytes per slot and macrobatch
  p.off_plan = take(static_cast<size_t>(n_macro) * p.cap * 16);
  p.off_pers = take(persistent_ws_bytes(p.nwin * static_cast<int64_t>(n_macro)));
  p.total = o;
  return true;
}

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off); }

thread_local hipError_t g_last_hip_error = hipSuccess;

mok_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOK_OK;
  g_last_hip_error = e;
  return MOK_ERR_HIP;
}

}  // namespace
}  // namespace mok

using namespace mok;

extern "C" {

const char* mok_status_str(mok_status s) {
  switch (s) {
    case MOK_OK: return "ok";
    case MOK_ERR_INVALID_ARG: return "invalid argument";
    case MOK_ERR_UNSUPPORTED: return "unsupported shape or option";
    case MOK_ERR_WORKSPACE: return "workspace too small";
    case MOK_ERR_HIP: return "HIP runtime or launch error";
    case MOK_ERR_DEVICE: return "device-side wait gave up";
    case MOK_ERR_CAPACITY: return "more routed rows than the capacity";
  }
  return "unknown status";
}

mok_status mok_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
                          float* topk_gate, hipStream_t stream) {
  if (T < 0 || E < 1 || E > 4096 || k < 1 || k > 32 || k > E) return MOK_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !topk_idx || !topk_gate)) return MOK_ERR_INVALID_ARG;
  return hip_status(launch_route_topk(logits, T, E, k, topk_idx, topk_gate, stream));
}

size_t mok_route_gemm_workspace_size(int32_t T, int32_t E, int32_t H) {
  if (T < 0 || E < 1 || H < 16) return 0;
  return static_cast<size_t>(route_gemm_splits(T, E, H)) * static_cast<size_t>(T) * E * sizeof(float);
}

mok_status mok_route_topk_gemm(const void* x, const void* w_router, int32_t T, int32_t H, int32_t E,
                               int32_t k, void* ws, size_t ws_bytes, int32_t* topk_idx,
                               float* topk_gate, hipStream_t stream) {
  if (T < 0 || H < 16 || H % 16 != 0 || E < 1 || E > 4096 || k < 1 || k > 32 || k > E)
    return MOK_ERR_INVALID_ARG;
  if (T == 0) return MOK_OK;
  if (!x || !w_router || !topk_idx || !topk_gate || !ws) return MOK_ERR_INVALID_ARG;
  if (ws_bytes < mok_route_gemm_workspace_size(T, E, H)) return MOK_ERR_WORKSPACE;
  return hip_status(launch_route_topk_gemm(static_cast<const uint16_t*>(x), nullptr, 0,
                                           static_cast<const uint16_t*>(w_router), T, H, E, k,
                                           static_cast<float*>(ws), topk_idx, topk_gate,
                                           RouteCount{}, stream));
}

size_t mok_schedule_workspace_size(int64_t T, int32_t k, int32_t n_local) {
  if (T < 0 || k < 1 || n_local < 1) return 0;
  return sched_ws_bytes(T * k, n_local);
}

mok_status mok_build_schedule(const int32_t* topk_idx, int32_t T, int32_t k, int32_t expert_base,
                              int32_t n_local, int32_t* counts, int32_t* offsets,
                              int32_t* slot_of_assign, int32_t* assign_of_slot, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || k < 1 || n_local < 1 || n_local > 256) return MOK_ERR_INVALID_ARG;
  const int64_t A = static_cast<int64_t>(T) * k;
  if (A >= (1ll << 31)) return MOK_ERR_UNSUPPORTED;
  if (!counts || !offsets || !ws) return MOK_ERR_INVALID_ARG;
  if (A > 0 && (!topk_idx || !slot_of_assign || !assign_of_slot)) return MOK_ERR_INVALID_ARG;
  if (ws_bytes < sched_ws_bytes(A, n_local)) return MOK_ERR_WORKSPACE;
  SchedWs w = sched_ws_carve(ws, A, n_local);
  return hip_status(launch_schedule(topk_idx, A, expert_base, n_local, counts, offsets,
                                    slot_of_assign, assign_of_slot, w, stream));
}

}  // extern "C"

// ---------------------------------------------- schedule with no allocation
// The schedule's per-chunk counts live in a fixed device array instead of a
// caller workspace, for callers that cannot allocate.  In host code the
// array's name is only a stand-in: its device address, one per GPU, comes
// from hipGetSymbolAddress on the first call on that device and is what the
// kernels receive.
namespace {
constexpr size_t kNoAllocScratchBytes = 4u << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

void* noalloc_scratch(mok_status* st) {
  static std::atomic<void*> ptr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { *st = hip_status(e); return nullptr; }
  if (dev < 0 || dev >= 64) { *st = MOK_ERR_UNSUPPORTED; return nullptr; }
  void* p = ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) { *st = hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol); return nullptr; }
    ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}
}  // namespace

extern "C" {

size_t mok_schedule_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

mok_status mok_build_schedule_noalloc(const int32_t* topk_idx, int32_t T, int32_t k,
                                      int32_t expert_base, int32_t n_local, int32_t* counts,
                                      int32_t* offsets, int32_t* slot_of_assign,
                                      int32_t* assign_of_slot, hipStream_t stream) {
  if (T < 0 || k < 1 || n_local < 1 || n_local > 256) return MOK_ERR_INVALID_ARG;
  const int64_t A = static_cast<int64_t>(T) * k;
  if (A >= (1ll << 31)) return MOK_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOK_ERR_INVALID_ARG;
  if (A > 0 && (!topk_idx || !slot_of_assign || !assign_of_slot)) return MOK_ERR_INVALID_ARG;
  if (sched_ws_bytes(A, n_local) > kNoAllocScratchBytes) return MOK_ERR_UNSUPPORTED;
  mok_status st = MOK_OK;
  void* ws = noalloc_scratch(&st);
  if (!ws) return st;
  // every chunk count the scatter reads is written by the count launch first:
  // nothing in the array has to start at zero
  SchedWs w = sched_ws_carve(ws, A, n_local);
  return hip_status(launch_schedule(topk_idx, A, expert_base, n_local, counts, offsets,
                                    slot_of_assign, assign_of_slot, w, stream));
}

int32_t mok_choose_minibatch(int32_t n_cus, int32_t tile_m, int32_t tile_n, int32_t n_out,
                             int64_t rows) {
  if (n_cus < 1 || tile_m < 1 || tile_n < 1 || n_out < 1) return 0;
  int64_t need = 2ll * n_cus * tile_m * tile_n;
  int64_t m = (need + n_out - 1) / n_out;
  m = (m + 63) / 64 * 64;
  if (rows > 0 && m > rows) m = rows;
  return static_cast<int32_t>(m);
}

mok_status mok_build_schedule_windows(const int32_t* topk_idx, int32_t T, int32_t k,
                                      int32_t expert_base, int32_t n_local, int32_t* counts,
                                      int32_t* offsets, int32_t* slot_of_assign,
                                      int32_t* assign_of_slot, int32_t M, int32_t nwin,
                                      int32_t* win_seg, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  if (T < 0 || k < 1 || n_local < 1 || n_local > 256 || M < 1 || nwin < 0)
    return MOK_ERR_INVALID_ARG;
  const int64_t A = static_cast<int64_t>(T) * k;
  if (A >= (1ll << 31)) return MOK_ERR_UNSUPPORTED;
  if (!counts || !offsets || !ws || (nwin > 0 && !win_seg)) return MOK_ERR_INVALID_ARG;
  if (A > 0 && (!topk_idx || !slot_of_assign || !assign_of_slot)) return MOK_ERR_INVALID_ARG;
  if (ws_bytes < sched_ws_bytes(A, n_local)) return MOK_ERR_WORKSPACE;
  SchedWs w = sched_ws_carve(ws, A, n_local);
  // the fused layer's two launches: count, then the scatter whose block 0
  // also writes the window table (no capacity bound here)
  return hip_status(launch_route_schedule(nullptr, 0, nullptr, const_cast<int32_t*>(topk_idx), T, k,
                                          expert_base, n_local, counts, offsets, slot_of_assign,
                                          assign_of_slot, w, M, nwin, win_seg, 0x7fffffff, nullptr,
                                          stream, false));
}

mok_status mok_build_windows(const int32_t* offsets, int32_t n_local, int32_t M, int32_t nwin,
                             int32_t* win_seg, hipStream_t stream) {
  if (!offsets || n_local < 1 || M < 1 || nwin < 0) return MOK_ERR_INVALID_ARG;
  if (nwin > 0 && !win_seg) return MOK_ERR_INVALID_ARG;
  return hip_status(launch_windows(offsets, n_local, M, nwin, win_seg, stream));
}

mok_status mok_dispatch_gather(const mok_tokens* src, int32_t H, int32_t k,
                               const int32_t* assign_of_slot, const int32_t* offsets,
                               int32_t n_local, int32_t slot_begin, int32_t slot_end, void* ring,
                               uint8_t* ring_scales, int32_t ring_slots, int32_t act_format,
                               int32_t* dev_status, hipStream_t stream) {
  if (!tokens_ok(src, 0) || H <= 0 || H % 64 != 0 || k < 1 || !assign_of_slot || !offsets ||
      n_local < 1 || slot_begin < 0 || slot_end < slot_begin || !ring || ring_slots < 1)
    return MOK_ERR_INVALID_ARG;
  if (act_format == MOK_ACT_MXFP8_E4M3) {
    if (!ring_scales) return MOK_ERR_INVALID_ARG;
  } else if (act_format != MOK_ACT_BF16) {
    return MOK_ERR_INVALID_ARG;
  }
  return hip_status(launch_gather(src->part_ptr, src->n_partitions, src->part_rows, H, k,
                                  assign_of_slot, offsets, n_local, slot_begin, slot_end, ring,
                                  ring_scales, ring_slots, act_format, dev_status, stream));
}

mok_status mok_packed_weights_size(const mok_layer_desc* desc, size_t* gate_up_bytes,
                                   size_t* down_bytes) {
  if (!desc_ok(desc)) return MOK_ERR_INVALID_ARG;
  if (gate_up_bytes)
    *gate_up_bytes = packed_gate_up_bytes(desc->hidden, desc->inter, desc->n_local, desc->weight_format);
  if (down_bytes)
    *down_bytes = packed_down_bytes(desc->hidden, desc->inter, desc->n_local, desc->weight_format);
  return MOK_OK;
}

mok_status mok_pack_weights(const mok_layer_desc* desc, const void* w_gate_up, const void* w_down,
                            void* packed_gate_up, void* packed_down, hipStream_t stream) {
  if (!desc_ok(desc)) return MOK_ERR_INVALID_ARG;
  if (!w_gate_up != !packed_gate_up || !w_down != !packed_down) return MOK_ERR_INVALID_ARG;
  if (!w_gate_up && !w_down) return MOK_ERR_INVALID_ARG;
  return hip_status(launch_pack_weights(static_cast<const uint16_t*>(w_gate_up),
                                        static_cast<const uint16_t*>(w_down), desc->hidden,
                                        desc->inter, desc->n_local, desc->act_format,
                                        desc->weight_format, static_cast<uint16_t*>(packed_gate_up),
                                        static_cast<uint16_t*>(packed_down), stream));
}

mok_status mok_expert_ffn(const mok_layer_desc* desc, const void* ring, const uint8_t* ring_scales,
                          int32_t ring_slots, const int32_t* offsets, int32_t slot_begin,
                          int32_t slot_end, const void* w_gate_up, const void* w_down, void* act,
                          uint8_t* act_scales, int32_t act_rows, void* y, int32_t y_rows,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!desc_ok(desc) || !ring || ring_slots < 1 || !offsets || slot_begin < 0 ||
      slot_end < slot_begin || !w_gate_up || !w_down || !act || act_rows < 1 || !y || y_rows < 1)
    return MOK_ERR_INVALID_ARG;
  const bool mx = desc->act_format == MOK_ACT_MXFP8_E4M3;
  if (mx && (!ring_scales || !act_scales)) return MOK_ERR_INVALID_ARG;
  if (!weights_ok(desc)) return MOK_ERR_INVALID_ARG;
  if (!gemm_operands_fit(desc, ring_slots, act_rows)) return MOK_ERR_UNSUPPORTED;
  FfnArgs a{};
  if (mok_status st = gemm_split(desc, ws, ws_bytes, a.split)) return st;
  a.ring = ring; a.ring_scales = ring_scales; a.ring_slots = ring_slots;
  a.offsets = offsets; a.n_local = desc->n_local; a.s_begin = slot_begin; a.s_end = slot_end;
  a.w_gu = static_cast<const uint16_t*>(w_gate_up); a.w_d = static_cast<const uint16_t*>(w_down);
  a.act = act; a.act_scales = act_scales; a.act_rows = act_rows;
  a.y = y; a.y_rows = y_rows;
  a.H = desc->hidden; a.I = desc->inter; a.act_format = desc->act_format;
  a.w_packed = desc->weights_packed; a.weight_format = desc->weight_format;
  return hip_status(launch_ffn(a, stream));
}

mok_status mok_expert_gate_up(const mok_layer_desc* desc, const void* ring,
                              const uint8_t* ring_scales, int32_t ring_slots,
                              const int32_t* offsets, int32_t slot_begin, int32_t slot_end,
                              const void* w_gate_up, void* act, uint8_t* act_scales,
                              int32_t act_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!desc_ok(desc) || !ring || ring_slots < 1 || !offsets || slot_begin < 0 ||
      slot_end < slot_begin || !w_gate_up || !act || act_rows < 1)
    return MOK_ERR_INVALID_ARG;
  if (desc->act_format == MOK_ACT_MXFP8_E4M3 && (!ring_scales || !act_scales))
    return MOK_ERR_INVALID_ARG;
  if (!weights_ok(desc)) return MOK_ERR_INVALID_ARG;
  if (!gemm_operands_fit(desc, ring_slots, 0)) return MOK_ERR_UNSUPPORTED;
  FfnArgs a{};
  if (mok_status st = gemm_split(desc, ws, ws_bytes, a.split)) return st;
  a.ring = ring; a.ring_scales = ring_scales; a.ring_slots = ring_slots;
  a.offsets = offsets; a.n_local = desc->n_local; a.s_begin = slot_begin; a.s_end = slot_end;
  a.w_gu = static_cast<const uint16_t*>(w_gate_up);
  a.act = act; a.act_scales = act_scales; a.act_rows = act_rows;
  a.H = desc->hidden; a.I = desc->inter; a.act_format = desc->act_format;
  a.w_packed = desc->weights_packed; a.weight_format = desc->weight_format;
  return hip_status(launch_gate_up(a, stream));
}

mok_status mok_expert_gate_up_save_h(const mok_layer_desc* desc, const void* ring,
                                     int32_t ring_slots, const int32_t* offsets,
                                     int32_t slot_begin, int32_t slot_end, const void* w_gate_up,
                                     void* act, int32_t act_rows, void* h, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!desc_ok(desc) || desc->act_format != MOK_ACT_BF16 || desc->weight_format != MOK_W_BF16 ||
      !ring || ring_slots < 1 || !offsets || slot_begin < 0 || slot_end < slot_begin ||
      !w_gate_up || !act || act_rows < 1 || !h)
    return MOK_ERR_INVALID_ARG;
  if (!weights_ok(desc)) return MOK_ERR_INVALID_ARG;
  if (!gemm_operands_fit(desc, ring_slots, act_rows) ||
      static_cast<int64_t>(act_rows) * 2 * desc->inter * 2 >= (1ll << 32))
    return MOK_ERR_UNSUPPORTED;
  FfnArgs a{};
  if (mok_status st = gemm_split(desc, ws, ws_bytes, a.split)) return st;
  a.ring = ring; a.ring_scales = nullptr; a.ring_slots = ring_slots;
  a.offsets = offsets; a.n_local = desc->n_local; a.s_begin = slot_begin; a.s_end = slot_end;
  a.w_gu = static_cast<const uint16_t*>(w_gate_up);
  a.act = act; a.act_scales = nullptr; a.act_rows = act_rows;
  a.H = desc->hidden; a.I = desc->inter; a.act_format = MOK_ACT_BF16;
  a.w_packed = desc->weights_packed; a.weight_format = MOK_W_BF16;
  a.h_out = h;
  return hip_status(launch_gate_up(a, stream));
}

mok_status mok_expert_gate_up_save_h_mx(const mok_layer_desc* desc, const void* ring,
                                        const uint8_t* ring_scales, int32_t ring_slots,
                                        const int32_t* offsets, int32_t slot_begin,
                                        int32_t slot_end, const void* w_gate_up, void* act,
                                        uint8_t* act_scales, int32_t act_rows, void* h, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  if (!desc_ok(desc) || desc->act_format != MOK_ACT_MXFP8_E4M3 || !ring || !ring_scales ||
      ring_slots < 1 || !offsets || slot_begin < 0 || slot_end < slot_begin || !w_gate_up || !act ||
      !act_scales || act_rows < 1 || !h)
    return MOK_ERR_INVALID_ARG;
  if (!weights_ok(desc)) return MOK_ERR_INVALID_ARG;
  if (!gemm_operands_fit(desc, ring_slots, act_rows) ||
      static_cast<int64_t>(act_rows) * 2 * desc->inter * 2 >= (1ll << 32))
    return MOK_ERR_UNSUPPORTED;
  FfnArgs a{};
  if (mok_status st = gemm_split(desc, ws, ws_bytes, a.split)) return st;
  a.ring = ring; a.ring_scales = ring_scales; a.ring_slots = ring_slots;
  a.offsets = offsets; a.n_local = desc->n_local; a.s_begin = slot_begin; a.s_end = slot_end;
  a.w_gu = static_cast<const uint16_t*>(w_gate_up);
  a.act = act; a.act_scales = act_scales; a.act_rows = act_rows;
  a.H = desc->hidden; a.I = desc->inter; a.act_format = MOK_ACT_MXFP8_E4M3;
  a.w_packed = desc->weights_packed; a.weight_format = desc->weight_format;
  a.h_out = h;
  return hip_status(launch_gate_up(a, stream));
}

mok_status mok_expert_down(const mok_layer_desc* desc, const void* act, const uint8_t* act_scales,
                           int32_t act_rows, const int32_t* offsets, int32_t slot_begin,
                           int32_t slot_end, const void* w_down, void* y, int32_t y_rows,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!desc_ok(desc) || !act || act_rows < 1 || !offsets || slot_begin < 0 ||
      slot_end < slot_begin || !w_down || !y || y_rows < 1)
    return MOK_ERR_INVALID_ARG;
  if (desc->act_format == MOK_ACT_MXFP8_E4M3 && !act_scales) return MOK_ERR_INVALID_ARG;
  if (!weights_ok(desc)) return MOK_ERR_INVALID_ARG;
  if (!gemm_operands_fit(desc, 0, act_rows)) return MOK_ERR_UNSUPPORTED;
  FfnArgs a{};
  if (mok_status st = gemm_split(desc, ws, ws_bytes, a.split)) return st;
  a.offsets = offsets; a.n_local = desc->n_local; a.s_begin = slot_begin; a.s_end = slot_end;
  a.w_d = static_cast<const uint16_t*>(w_down);
  a.act = const_cast<void*>(act); a.act_scales = const_cast<uint8_t*>(act_scales);
  a.act_rows = act_rows; a.y = y; a.y_rows = y_rows;
  a.H = desc->hidden; a.I = desc->inter; a.act_format = desc->act_format;
  a.w_packed = desc->weights_packed; a.weight_format = desc->weight_format;
  return hip_status(launch_down(a, stream));
}

mok_status mok_expert_down_merge(const mok_layer_desc* desc, const void* act,
                                 const uint8_t* act_scales, int32_t act_rows,
                                 const int32_t* offsets, int32_t slot_begin, int32_t slot_end,
                                 const void* w_down, void* y, int32_t y_rows,
                                 const int32_t* assign_of_slot, const int32_t* slot_of_assign,
                                 const float* topk_gate, const mok_tokens* out, void* merge_plan,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!desc_ok(desc) || !act || act_rows < 1 || !offsets || slot_begin < 0 ||
      slot_end < slot_begin || !w_down || !y || y_rows < 1 || !assign_of_slot ||
      !slot_of_assign || !topk_gate || !tokens_ok(out, 0) || !merge_plan || slot_end > y_rows)
    return MOK_ERR_INVALID_ARG;
  if (desc->act_format == MOK_ACT_MXFP8_E4M3 && !act_scales) return MOK_ERR_INVALID_ARG;
  if (!weights_ok(desc)) return MOK_ERR_INVALID_ARG;
  if (!gemm_operands_fit(desc, 0, act_rows)) return MOK_ERR_UNSUPPORTED;
  FfnArgs a{};
  if (mok_status st = gemm_split(desc, ws, ws_bytes, a.split)) return st;
  a.offsets = offsets; a.n_local = desc->n_local; a.s_begin = slot_begin; a.s_end = slot_end;
  a.w_d = static_cast<const uint16_t*>(w_down);
  a.act = const_cast<void*>(act); a.act_scales = const_cast<uint8_t*>(act_scales);
  a.act_rows = act_rows; a.y = y; a.y_rows = y_rows;
  a.H = desc->hidden; a.I = desc->inter; a.act_format = desc->act_format;
  a.w_packed = desc->weights_packed; a.weight_format = desc->weight_format;
  a.merge.aos = assign_of_slot; a.merge.soa = slot_of_assign; a.merge.gate = topk_gate;
  a.merge.k = desc->top_k; a.merge.out_parts = out->part_ptr; a.merge.n_part = out->n_partitions;
  a.merge.part_rows = out->part_rows; a.merge.plan = merge_plan; a.merge.status = nullptr;
  return hip_status(launch_down(a, stream));
}

mok_status mok_combine(const void* y, int32_t y_rows, const int32_t* slot_of_assign,
                       const float* topk_gate, int32_t T, int32_t k, int32_t H,
                       const mok_tokens* out, int32_t* dev_status, hipStream_t stream) {
  if (T < 0 || k < 1 || k > 32 || H <= 0 || H % 8 != 0 || !tokens_ok(out, T)) return MOK_ERR_INVALID_ARG;
  if (T > 0 && (!y || y_rows < 1 || !slot_of_assign || !topk_gate)) return MOK_ERR_INVALID_ARG;
  return hip_status(launch_combine(y, y_rows, slot_of_assign, topk_gate, T, k, H, out->part_ptr,
                                   out->n_partitions, out->part_rows, dev_status, false, stream));
}

mok_status mok_combine_slots(const void* y, int32_t y_rows, const int32_t* assign_of_slot,
                             const int32_t* offsets, int32_t n_local, int32_t n_slots,
                             const int32_t* slot_of_assign, const float* topk_gate, int32_t k,
                             int32_t H, const mok_tokens* out, int32_t* dev_status,
                             hipStream_t stream) {
  if (k < 1 || k > 32 || H <= 0 || H % 8 != 0 || n_local < 1 || n_slots < 0 || !tokens_ok(out, 0))
    return MOK_ERR_INVALID_ARG;
  if (n_slots > 0 && (!y || y_rows < 1 || !assign_of_slot || !offsets || !slot_of_assign ||
                      !topk_gate))
    return MOK_ERR_INVALID_ARG;
  return hip_status(launch_combine_slots(y, y_rows, assign_of_slot, offsets, n_local, n_slots,
                                         slot_of_assign, topk_gate, k, H, out->part_ptr,
                                         out->n_partitions, out->part_rows, dev_status, false,
                                         stream));
}

mok_status mok_combine_slots_multi(const void* y, int32_t y_rows, const int32_t* assign_of_slot,
                                   const int32_t* offsets, int32_t n_local, int32_t n_slots,
                                   const int32_t* slot_of_assign, const float* topk_gate,
                                   int32_t k, int32_t H, const mok_tokens* out,
                                   int32_t* dev_status, hipStream_t stream) {
  if (k < 1 || k > 32 || H <= 0 || H % 8 != 0 || n_local < 1 || n_slots < 0 || !tokens_ok(out, 0))
    return MOK_ERR_INVALID_ARG;
  if (n_slots > 0 && (!y || y_rows < 1 || !assign_of_slot || !offsets || !slot_of_assign ||
                      !topk_gate))
    return MOK_ERR_INVALID_ARG;
  return hip_status(launch_combine_slots(y, y_rows, assign_of_slot, offsets, n_local, n_slots,
                                         slot_of_assign, topk_gate, k, H, out->part_ptr,
                                         out->n_partitions, out->part_rows, dev_status, false,
                                         stream, true));
}

// ------------------------------------------------------------ backward
namespace {
// bf16 tokens and weights
bool bwd_desc_ok(const mok_layer_desc* d) {
  return desc_ok(d) && d->act_format == MOK_ACT_BF16 && d->weight_format == MOK_W_BF16;
}
// MXFP8 tokens; bf16 weights, or MXFP8 weights (packed, as the forward needs them)
bool bwd_desc_mx_ok(const mok_layer_desc* d) {
  return desc_ok(d) && d->act_format == MOK_ACT_MXFP8_E4M3 &&
         (d->weight_format == MOK_W_BF16 || (d->weight_format == MOK_W_MXFP8_E4M3 && d->weights_packed));
}
}  // namespace

mok_status mok_packed_weights_bwd_size(const mok_layer_desc* desc, size_t* gate_up_t_bytes,
                                       size_t* down_t_bytes) {
  if (!bwd_desc_ok(desc) && !bwd_desc_mx_ok(desc)) return MOK_ERR_INVALID_ARG;
  if (gate_up_t_bytes)
    *gate_up_t_bytes = packed_bwd_gate_up_bytes(desc->hidden, desc->inter, desc->n_local, desc->weight_format);
  if (down_t_bytes)
    *down_t_bytes = packed_bwd_down_bytes(desc->hidden, desc->inter, desc->n_local, desc->weight_format);
  return MOK_OK;
}

mok_status mok_pack_weights_bwd(const mok_layer_desc* desc, const void* w_gate_up, const void* w_down,
                                void* packed_gate_up_t, void* packed_down_t, hipStream_t stream) {
  if (!bwd_desc_ok(desc) && !bwd_desc_mx_ok(desc)) return MOK_ERR_INVALID_ARG;
  if ((w_gate_up == nullptr) != (packed_gate_up_t == nullptr) ||
      (w_down == nullptr) != (packed_down_t == nullptr))
    return MOK_ERR_INVALID_ARG;
  return hip_status(launch_pack_weights_bwd(static_cast<const uint16_t*>(w_gate_up),
                                            static_cast<const uint16_t*>(w_down), desc->hidden,
                                            desc->inter, desc->n_local, bwd_desc_mx_ok(desc),
                                            desc->weight_format == MOK_W_MXFP8_E4M3,
                                            static_cast<uint16_t*>(packed_gate_up_t),
                                            static_cast<uint16_t*>(packed_down_t), stream));
}

mok_status mok_combine_backward(const mok_tokens* dout, const void* y, int32_t y_rows,
                                const int32_t* assign_of_slot, const int32_t* offsets,
                                int32_t n_local, int32_t n_slots, const float* topk_gate, int32_t k,
                                int32_t H, void* dy, int32_t dy_rows, float* dgate,
                                int32_t* dev_status, hipStream_t stream) {
  if (k < 1 || k > 32 || H <= 0 || H % 64 != 0 || n_local < 1 || n_slots < 0 || !tokens_ok(dout, 0))
    return MOK_ERR_INVALID_ARG;
  if (n_slots > 0 && (!y || y_rows < 1 || !assign_of_slot || !offsets || !topk_gate || !dy ||
                      dy_rows < 1 || !dgate))
    return MOK_ERR_INVALID_ARG;
  return hip_status(launch_unmerge_slots(dout->part_ptr, dout->n_partitions, dout->part_rows, y,
                                         y_rows, assign_of_slot, offsets, n_local, n_slots,
                                         topk_gate, k, H, dy, nullptr, dy_rows, dgate, dev_status,
                                         stream));
}

mok_status mok_combine_backward_mx(const mok_tokens* dout, const void* y, int32_t y_rows,
                                   const int32_t* assign_of_slot, const int32_t* offsets,
                                   int32_t n_local, int32_t n_slots, const float* topk_gate,
                                   int32_t k, int32_t H, void* dy, uint8_t* dy_scales,
                                   int32_t dy_rows, float* dgate, int32_t* dev_status,
                                   hipStream_t stream) {
  if (k < 1 || k > 32 || H <= 0 || H % 64 != 0 || n_local < 1 || n_slots < 0 || !tokens_ok(dout, 0))
    return MOK_ERR_INVALID_ARG;
  if (n_slots > 0 && (!y || y_rows < 1 || !assign_of_slot || !offsets || !topk_gate || !dy ||
                      !dy_scales || dy_rows < 1 || !dgate))
    return MOK_ERR_INVALID_ARG;
  return hip_status(launch_unmerge_slots(dout->part_ptr, dout->n_partitions, dout->part_rows, y,
                                         y_rows, assign_of_slot, offsets, n_local, n_slots,
                                         topk_gate, k, H, dy, dy_scales, dy_rows, dgate,
                                         dev_status, stream));
}

mok_status mok_expert_ffn_backward(const mok_layer_desc* desc, const void* ring, int32_t ring_slots,
                                   const void* dy, const int32_t* offsets, int32_t slot_begin,
                                   int32_t slot_end, const void* w_gate_up,
                                   const void* packed_gate_up_t, const void* packed_down_t, void* h,
                                   void* dh, void* dx_slots, int32_t rows, hipStream_t stream) {
  if (!bwd_desc_ok(desc) || !ring || ring_slots < 1 || !dy || !offsets || slot_begin < 0 ||
      slot_end < slot_begin || !w_gate_up || !packed_gate_up_t || !packed_down_t || !h || !dh ||
      !dx_slots || rows < 1)
    return MOK_ERR_INVALID_ARG;
  const int64_t lim = 1ll << 32, H = desc->hidden, I = desc->inter;
  if (static_cast<int64_t>(ring_slots) * H * 2 >= lim || static_cast<int64_t>(rows) * 2 * I * 2 >= lim ||
      static_cast<int64_t>(rows) * H * 2 >= lim || 4ll * I * H >= lim)
    return MOK_ERR_UNSUPPORTED;
  BwdArgs a{};
  a.ring = ring; a.ring_slots = ring_slots;
  a.offsets = offsets; a.n_local = desc->n_local; a.s_begin = slot_begin; a.s_end = slot_end;
  a.w_gu = static_cast<const uint16_t*>(w_gate_up); a.w_gu_packed = desc->weights_packed;
  a.w_gu_t = static_cast<const uint16_t*>(packed_gate_up_t);
  a.w_d_t = static_cast<const uint16_t*>(packed_down_t);
  a.dy = dy; a.h = h; a.dh = dh; a.dx = dx_slots; a.rows = rows;
  a.H = desc->hidden; a.I = desc->inter; a.n_cus = device_cus();
  return hip_status(launch_ffn_backward(a, stream));
}

mok_status mok_expert_ffn_backward_saved(const mok_layer_desc* desc, const void* dy,
                                         const int32_t* offsets, int32_t slot_begin,
                                         int32_t slot_end, const void* packed_gate_up_t,
                                         const void* packed_down_t, const void* h, void* dh,
                                         void* dx_slots, int32_t rows, hipStream_t stream) {
  if (!bwd_desc_ok(desc) || !dy || !offsets || slot_begin < 0 || slot_end < slot_begin ||
      !packed_gate_up_t || !packed_down_t || !h || !dh || !dx_slots || rows < 1)
    return MOK_ERR_INVALID_ARG;
  const int64_t lim = 1ll << 32, H = desc->hidden, I = desc->inter;
  if (static_cast<int64_t>(rows) * 2 * I * 2 >= lim || static_cast<int64_t>(rows) * H * 2 >= lim ||
      4ll * I * H >= lim)
    return MOK_ERR_UNSUPPORTED;
  BwdArgs a{};
  a.offsets = offsets; a.n_local = desc->n_local; a.s_begin = slot_begin; a.s_end = slot_end;
  a.w_gu_t = static_cast<const uint16_t*>(packed_gate_up_t);
  a.w_d_t = static_cast<const uint16_t*>(packed_down_t);
  a.dy = dy; a.h = const_cast<void*>(h); a.dh = dh; a.dx = dx_slots; a.rows = rows;
  a.h_saved = 1;
  a.H = desc->hidden; a.I = desc->inter; a.n_cus = device_cus();
  return hip_status(launch_ffn_backward(a, stream));
}

mok_status mok_expert_ffn_backward_mx(const mok_layer_desc* desc, const void* ring,
                                      const uint8_t* ring_scales, int32_t ring_slots,
                                      const void* dy, const uint8_t* dy_scales,
                                      const int32_t* offsets, int32_t slot_begin, int32_t slot_end,
                                      const void* w_gate_up, const void* packed_gate_up_t,
                                      const void* packed_down_t, void* h, int32_t h_kept, void* dh,
                                      uint8_t* dh_scales, void* dx_slots, int32_t rows,
                                      hipStream_t stream) {
  if (!bwd_desc_mx_ok(desc) || !dy || !dy_scales || !offsets || slot_begin < 0 ||
      slot_end < slot_begin || !packed_gate_up_t || !packed_down_t || !h || !dh || !dh_scales ||
      !dx_slots || rows < 1)
    return MOK_ERR_INVALID_ARG;
  if (!h_kept && (!ring || !ring_scales || ring_slots < 1 || !w_gate_up)) return MOK_ERR_INVALID_ARG;
  const int64_t lim = 1ll << 32, H = desc->hidden, I = desc->inter;
  if ((!h_kept && static_cast<int64_t>(ring_slots) * H >= lim) ||
      static_cast<int64_t>(rows) * 2 * I * 2 >= lim || static_cast<int64_t>(rows) * H * 2 >= lim ||
      4ll * I * H >= lim)
    return MOK_ERR_UNSUPPORTED;
  BwdArgs a{};
  a.ring = ring; a.ring_scales = ring_scales; a.ring_slots = ring_slots;
  a.offsets = offsets; a.n_local = desc->n_local; a.s_begin = slot_begin; a.s_end = slot_end;
  a.w_gu = static_cast<const uint16_t*>(w_gate_up); a.w_gu_packed = desc->weights_packed;
  a.w_gu_t = static_cast<const uint16_t*>(packed_gate_up_t);
  a.w_d_t = static_cast<const uint16_t*>(packed_down_t);
  a.dy = dy; a.dy_scales = dy_scales; a.h = h; a.dh = dh; a.dh_scales = dh_scales;
  a.dx = dx_slots; a.rows = rows; a.h_saved = h_kept ? 1 : 0; a.mx = 1;
  a.w_mx8 = desc->weight_format == MOK_W_MXFP8_E4M3 ? 1 : 0;
  a.H = desc->hidden; a.I = desc->inter; a.n_cus = device_cus();
  return hip_status(launch_ffn_backward(a, stream));
}

size_t mok_wgrad_workspace_size(const mok_layer_desc* desc, int32_t rows) {
  if ((!bwd_desc_ok(desc) && !bwd_desc_mx_ok(desc)) || rows < 1) return 0;
  return wgrad_ws_bytes(rows, desc->hidden, desc->inter, desc->n_local);
}

mok_status mok_expert_wgrad(const mok_layer_desc* desc, const void* ring, int32_t ring_slots,
                            const void* act, int32_t act_rows, const void* dy, const void* dh,
                            int32_t rows, const int32_t* offsets, void* dw_gate_up, void* dw_down,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!bwd_desc_ok(desc) || !ring || ring_slots < 1 || !act || act_rows < 1 || !dy || !dh ||
      rows < 1 || !offsets || (!dw_gate_up && !dw_down) || !ws)
    return MOK_ERR_INVALID_ARG;
  if (ws_bytes < mok_wgrad_workspace_size(desc, rows)) return MOK_ERR_WORKSPACE;
  const int64_t lim = 1ll << 32, H = desc->hidden, I = desc->inter;
  const int64_t kp = wgrad_kpad(rows, desc->n_local);
  if (kp * H * 2 >= lim || kp * 2 * I * 2 >= lim || static_cast<int64_t>(ring_slots) * H * 2 >= lim ||
      static_cast<int64_t>(act_rows) * I * 2 >= lim || static_cast<int64_t>(rows) * 2 * I * 2 >= lim)
    return MOK_ERR_UNSUPPORTED;
  WgradArgs a{};
  a.ring = ring; a.ring_slots = ring_slots; a.act = act; a.act_rows = act_rows;
  a.dy = dy; a.dh = dh; a.rows = rows; a.offsets = offsets; a.n_local = desc->n_local;
  a.dw_gu = dw_gate_up; a.dw_d = dw_down; a.ws = ws; a.H = desc->hidden; a.I = desc->inter;
  return hip_status(launch_wgrad(a, stream));
}

mok_status mok_expert_wgrad_mx(const mok_layer_desc* desc, const void* ring,
                               const uint8_t* ring_scales, int32_t ring_slots, const void* act,
                               const uint8_t* act_scales, int32_t act_rows, const void* dy,
                               const uint8_t* dy_scales, const void* dh, const uint8_t* dh_scales,
                               int32_t rows, const int32_t* offsets, void* dw_gate_up,
                               void* dw_down, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!bwd_desc_mx_ok(desc) || !ring || !ring_scales || ring_slots < 1 || !act || !act_scales ||
      act_rows < 1 || !dy || !dy_scales || !dh || !dh_scales || rows < 1 || !offsets ||
      (!dw_gate_up && !dw_down) || !ws)
    return MOK_ERR_INVALID_ARG;
  if (ws_bytes < mok_wgrad_workspace_size(desc, rows)) return MOK_ERR_WORKSPACE;
  const int64_t lim = 1ll << 32, H = desc->hidden, I = desc->inter;
  const int64_t kp = wgrad_kpad(rows, desc->n_local);
  if (kp * H * 2 >= lim || kp * 2 * I * 2 >= lim || static_cast<int64_t>(ring_slots) * H >= lim ||
      static_cast<int64_t>(act_rows) * I >= lim || static_cast<int64_t>(rows) * 2 * I >= lim ||
      static_cast<int64_t>(rows) * H >= lim)
    return MOK_ERR_UNSUPPORTED;
  WgradArgs a{};
  a.ring = ring; a.ring_slots = ring_slots; a.act = act; a.act_rows = act_rows;
  a.dy = dy; a.dh = dh; a.rows = rows; a.offsets = offsets; a.n_local = desc->n_local;
  a.ring_scales = ring_scales; a.act_scales = act_scales; a.dy_scales = dy_scales;
  a.dh_scales = dh_scales;
  a.dw_gu = dw_gate_up; a.dw_d = dw_down; a.ws = ws; a.H = desc->hidden; a.I = desc->inter;
  return hip_status(launch_wgrad(a, stream));
}

mok_status mok_dispatch_backward(const void* dx_slots, int32_t rows, const int32_t* assign_of_slot,
                                 const int32_t* offsets, int32_t n_local, int32_t n_slots,
                                 const int32_t* slot_of_assign, int32_t k, int32_t H,
                                 const mok_tokens* dx, int32_t* dev_status, hipStream_t stream) {
  if (k < 1 || k > 32 || H <= 0 || H % 8 != 0 || n_local < 1 || n_slots < 0 || !tokens_ok(dx, 0))
    return MOK_ERR_INVALID_ARG;
  if (n_slots > 0 && (!dx_slots || rows < 1 || !assign_of_slot || !offsets || !slot_of_assign))
    return MOK_ERR_INVALID_ARG;
  return hip_status(launch_combine_slots(dx_slots, rows, assign_of_slot, offsets, n_local, n_slots,
                                         slot_of_assign, nullptr, k, H, dx->part_ptr,
                                         dx->n_partitions, dx->part_rows, dev_status, false, stream));
}

size_t mok_gemm_workspace_size(void) { return split_ws_bytes(device_cus()); }

size_t mok_forward_workspace_size(const mok_layer_desc* desc, int32_t T, int32_t n_macro) {
  Plan p;
  if (!desc_ok(desc) || T < 0 || n_macro < 1 || !make_plan(desc, T, n_macro, p)) return 0;
  return p.total;
}

int32_t mok_forward_minibatch(const mok_layer_desc* desc, int32_t T) {
  Plan p;
  if (!desc_ok(desc) || T < 0 || !make_plan(desc, T, 1, p)) return 0;
  return p.M;
}

}  // extern "C"

namespace mok {
namespace {

// The fused layer.  logits non-null (then n_macro = 1): the routing of the T
// tokens is computed here, from fp32 logits [T][n_experts], into the
// workspace; w_router non-null (then n_macro = 1): from the router GEMM of
// the tokens' rows x with the bf16 router rows w_router [n_experts][H], its
// per-split partial sums in the workspace past the plan's bytes; otherwise
// topk_idx / topk_gate hold each macrobatch's routing.
mok_status forward_impl(const mok_layer_desc* desc, int32_t n_macro, const float* logits,
                        const void* w_router, const int32_t* const* topk_idx,
                        const float* const* topk_gate, int32_t T, const mok_tokens* x,
                        const void* w_gate_up, const void* w_down, const mok_tokens* out,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!desc_ok(desc) || n_macro < 1 || T < 0 || !tokens_ok(x, T) || !w_gate_up || !w_down ||
      !out || !ws || !weights_ok(desc))
    return MOK_ERR_INVALID_ARG;
  const bool route_here = logits || w_router;
  if (route_here ? (n_macro != 1 || desc->n_experts > 4096)
                 : (!topk_idx || !topk_gate))
    return MOK_ERR_INVALID_ARG;
  for (int m = 0; m < n_macro; ++m) {
    if (T > 0 && !route_here && (!topk_idx[m] || !topk_gate[m])) return MOK_ERR_INVALID_ARG;
    if (!tokens_ok(&out[m], T)) return MOK_ERR_INVALID_ARG;
  }
  Plan p;
  if (!make_plan(desc, T, n_macro, p)) return MOK_ERR_UNSUPPORTED;
  const size_t router_bytes =
      w_router && T > 0 ? mok_route_gemm_workspace_size(T, desc->n_experts, desc->hidden) : 0;
  if (ws_bytes < p.total + router_bytes) return MOK_ERR_WORKSPACE;

  const mok_layer_desc& d = *desc;
  const bool mx = d.act_format == MOK_ACT_MXFP8_E4M3;
  int32_t* status = at<int32_t>(ws, p.off_status);
  hipError_t err = hipSuccess;
  // the status word and, with the K split, its counters (which follow it);
  // with logits also the schedule's chunk counts, which the route adds into
  const int n_cus = device_cus();
  const int32_t n_clear = static_cast<int32_t>(kAlign / 4) + (p.split ? n_cus : 0);
  SchedWs sw = sched_ws_carve(at<void>(ws, p.off_sched), p.A, d.n_local);
  const int32_t n_clear2 = route_here ? sw.nblk * d.n_local : 0;
  hipLaunchKernelGGL(k_zero2, dim3(n_clear2 > 4096 ? 16 : 1), dim3(256), 0, stream, status, n_clear,
                     sw.blk_counts, n_clear2);
  if ((err = hipGetLastError()) != hipSuccess) return hip_status(err);
  SplitWs split = p.split ? split_ws_carve(at<void>(ws, p.off_split), n_cus) : SplitWs{};
  split.n_cus = n_cus;
  int32_t* route_idx = at<int32_t>(ws, p.off_route_idx);
  float* route_gate = at<float>(ws, p.off_route_gate);

  MacroBuffers mb[64];
  const int nm_buf = n_macro < 64 ? n_macro : 64;
  if (n_macro > 64) return MOK_ERR_UNSUPPORTED;
  for (int m = 0; m < nm_buf; ++m) {
    mb[m].counts = at<int32_t>(ws, p.off_counts + m * p.per_macro_counts);
    mb[m].offsets = at<int32_t>(ws, p.off_offsets + m * p.per_macro_offsets);
    mb[m].soa = at<int32_t>(ws, p.off_soa + m * p.per_macro_soa);
    mb[m].aos = at<int32_t>(ws, p.off_aos + m * p.per_macro_aos);
    mb[m].win = at<int32_t>(ws, p.off_win + m * p.per_macro_win);
    mb[m].gate = route_here ? route_gate : topk_gate[m];
    mb[m].y = at<uint16_t>(ws, p.off_y + static_cast<size_t>(m % p.n_ybuf) * p.cap * d.hidden * 2);
    mb[m].out = out[m];
    mb[m].plan = at<void>(ws, p.off_plan + static_cast<size_t>(m) * p.cap * 16);
  }
  // Route (logits form), schedule, windows and capacity check for every
  // macrobatch first: two launches each, reading only routing.
  if (w_router && T > 0) {   // router GEMM + pick, counting the local picks as it goes
    RouteCount rc;
    rc.base = d.expert_base; rc.n_local = d.n_local; rc.blk_counts = sw.blk_counts; rc.nblk = sw.nblk;
    err = launch_route_topk_gemm(nullptr, x->part_ptr, x->part_rows,
                                 static_cast<const uint16_t*>(w_router), T, d.hidden, d.n_experts,
                                 d.top_k, at<float>(ws, p.total), route_idx, route_gate, rc, stream);
    if (err != hipSuccess) return hip_status(err);
  }
  for (int m = 0; m < n_macro; ++m) {
    int32_t* idx = route_here ? route_idx : const_cast<int32_t*>(T > 0 ? topk_idx[m] : nullptr);
    err = launch_route_schedule(logits, d.n_experts, route_gate, idx, T, d.top_k, d.expert_base,
                                d.n_local, mb[m].counts, mb[m].offsets, mb[m].soa, mb[m].aos, sw,
                                p.M, p.nwin, mb[m].win, p.cap, status, stream, w_router != nullptr);
    if (err != hipSuccess) return hip_status(err);
  }

  void* ring = at<void>(ws, p.off_ring);
  uint8_t* ring_sc = mx ? at<uint8_t>(ws, p.off_ring_sc) : nullptr;
  void* act = at<void>(ws, p.off_act);
  uint8_t* act_sc = mx ? at<uint8_t>(ws, p.off_act_sc) : nullptr;

  if (d.mode == MOK_MODE_PERSISTENT) {
    PersistentArgs pa{};
    pa.n_macro = n_macro; pa.mb = mb; pa.T = T; pa.k = d.top_k;
    pa.H = d.hidden; pa.I = d.inter; pa.n_local = d.n_local; pa.act_format = d.act_format;
    pa.M = p.M; pa.S = p.S; pa.nwin = p.nwin; pa.cap = p.cap;
    pa.x = *x; pa.w_gu = static_cast<const uint16_t*>(w_gate_up);
    pa.w_d = static_cast<const uint16_t*>(w_down);
    pa.w_packed = d.weights_packed; pa.weight_format = d.weight_format;
    pa.ring = ring; pa.ring_sc = ring_sc; pa.act = act; pa.act_sc = act_sc; pa.act_rows = p.act_rows;
    pa.status = status; pa.pers_ws = at<void>(ws, p.off_pers);
    pa.n_move = d.n_move_cus; pa.n_cus = device_cus(); pa.timeout_us = d.wait_timeout_us;
    mok_status st = launch_persistent(pa, stream);
    return st;
  }

  for (int m = 0; m < n_macro; ++m) {
    for (int b = 0; b < p.nwin; ++b) {
      const int32_t s0 = b * p.M;
      const int32_t s1 = static_cast<int32_t>(std::min<int64_t>(static_cast<int64_t>(s0) + p.M, p.cap));
      err = launch_gather(x->part_ptr, x->n_partitions, x->part_rows, d.hidden, d.top_k,
                          mb[m].aos, mb[m].offsets, d.n_local, s0, s1, ring, ring_sc, p.S,
                          d.act_format, status, stream);
      if (err != hipSuccess) return hip_status(err);
      FfnArgs a{};
      a.ring = ring; a.ring_scales = ring_sc; a.ring_slots = p.S;
      a.offsets = mb[m].offsets; a.n_local = d.n_local; a.s_begin = s0; a.s_end = s1;
      a.w_gu = static_cast<const uint16_t*>(w_gate_up); a.w_d = static_cast<const uint16_t*>(w_down);
      a.act = act; a.act_scales = act_sc; a.act_rows = p.act_rows;
      a.y = mb[m].y; a.y_rows = p.cap;
      a.H = d.hidden; a.I = d.inter; a.act_format = d.act_format;
      a.w_packed = d.weights_packed; a.weight_format = d.weight_format;
      a.split = split;
      // single-slot tokens merged in the down GEMM's epilogue; the rest below
      a.merge.aos = mb[m].aos; a.merge.soa = mb[m].soa; a.merge.gate = mb[m].gate;
      a.merge.k = d.top_k; a.merge.out_parts = mb[m].out.part_ptr;
      a.merge.n_part = mb[m].out.n_partitions; a.merge.part_rows = mb[m].out.part_rows;
      a.merge.plan = mb[m].plan; a.merge.status = status;
      if ((err = launch_ffn(a, stream)) != hipSuccess) return hip_status(err);
    }
    err = launch_combine_slots(mb[m].y, p.cap, mb[m].aos, mb[m].offsets, d.n_local, p.cap,
                               mb[m].soa, mb[m].gate, d.top_k, d.hidden, mb[m].out.part_ptr,
                               mb[m].out.n_partitions, mb[m].out.part_rows, status, true, stream,
                               true);
    if (err != hipSuccess) return hip_status(err);
  }
  return MOK_OK;
}

}  // namespace
}  // namespace mok

extern "C" {

mok_status mok_moe_forward_batches(const mok_layer_desc* desc, int32_t n_macro,
                                   const int32_t* const* topk_idx, const float* const* topk_gate,
                                   int32_t T, const mok_tokens* x, const void* w_gate_up,
                                   const void* w_down, const mok_tokens* out, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  return mok::forward_impl(desc, n_macro, nullptr, nullptr, topk_idx, topk_gate, T, x, w_gate_up,
                           w_down, out, ws, ws_bytes, stream);
}

mok_status mok_moe_forward_routed(const mok_layer_desc* desc, const int32_t* topk_idx,
                                  const float* topk_gate, int32_t T, const mok_tokens* x,
                                  const void* w_gate_up, const void* w_down, const mok_tokens* out,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  return mok::forward_impl(desc, 1, nullptr, nullptr, &topk_idx, &topk_gate, T, x, w_gate_up,
                           w_down, out, ws, ws_bytes, stream);
}

mok_status mok_moe_forward(const mok_layer_desc* desc, const float* logits, int32_t T,
                           const mok_tokens* x, const void* w_gate_up, const void* w_down,
                           const mok_tokens* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T > 0 && !logits) return MOK_ERR_INVALID_ARG;
  static const float kNoLogits = 0.0f;     // T = 0: nothing is read
  return mok::forward_impl(desc, 1, T > 0 ? logits : &kNoLogits, nullptr, nullptr, nullptr, T, x,
                           w_gate_up, w_down, out, ws, ws_bytes, stream);
}

size_t mok_forward_router_workspace_size(const mok_layer_desc* desc, int32_t T) {
  const size_t base = mok_forward_workspace_size(desc, T, 1);
  if (base == 0) return 0;
  return base + (T > 0 ? mok_route_gemm_workspace_size(T, desc->n_experts, desc->hidden) : 0);
}

mok_status mok_moe_forward_router(const mok_layer_desc* desc, const void* w_router, int32_t T,
                                  const mok_tokens* x, const void* w_gate_up, const void* w_down,
                                  const mok_tokens* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (!desc || (T > 0 && !w_router)) return MOK_ERR_INVALID_ARG;
  if (desc->hidden % 16 != 0) return MOK_ERR_INVALID_ARG;
  static const float kNoLogits = 0.0f;     // T = 0: no route at all
  return mok::forward_impl(desc, 1, T > 0 ? nullptr : &kNoLogits, T > 0 ? w_router : nullptr,
                           nullptr, nullptr, T, x, w_gate_up, w_down, out, ws, ws_bytes, stream);
}

mok_status mok_tune_forward(const mok_layer_desc* desc, const int32_t* minibatch,
                            int32_t n_minibatch, const int32_t* n_move, int32_t n_n_move,
                            int32_t reps, int32_t n_macro, const int32_t* const* topk_idx,
                            const float* const* topk_gate, int32_t T, const mok_tokens* x,
                            const void* w_gate_up, const void* w_down, const mok_tokens* out,
                            void* ws, size_t ws_bytes, mok_layer_desc* best, float* best_ms,
                            hipStream_t stream) {
  if (!desc || !minibatch || n_minibatch < 1 || n_n_move < 0 || (n_n_move > 0 && !n_move) ||
      reps < 1 || n_macro < 1 || !best || !best_ms || !ws)
    return MOK_ERR_INVALID_ARG;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return MOK_ERR_HIP;
  }
  bool found = false;
  float best_t = 0.0f;
  mok_layer_desc best_d = *desc;
  const int nm = n_n_move > 0 ? n_n_move : 1;
  for (int i = 0; i < n_minibatch; ++i) {
    for (int j = 0; j < nm; ++j) {
      mok_layer_desc d = *desc;
      d.minibatch = minibatch[i];
      if (n_n_move > 0) d.n_move_cus = n_move[j];
      if (d.mode != MOK_MODE_PERSISTENT && j > 0) continue;   // movers only in persistent mode
      const size_t need = mok_forward_workspace_size(&d, T, n_macro);
      if (need == 0 || need > ws_bytes) continue;
      // one untimed call, then `reps` timed ones
      if (mok_moe_forward_batches(&d, n_macro, topk_idx, topk_gate, T, x, w_gate_up, w_down, out,
                                  ws, ws_bytes, stream) != MOK_OK)
        continue;
      bool ok = hipEventRecord(e0, stream) == hipSuccess;
      for (int r = 0; ok && r < reps; ++r)
        ok = mok_moe_forward_batches(&d, n_macro, topk_idx, topk_gate, T, x, w_gate_up, w_down,
                                     out, ws, ws_bytes, stream) == MOK_OK;
      ok = ok && hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
      int32_t dev = MOK_OK;
      ok = ok && mok_device_status(ws, &dev, stream) == MOK_OK && dev == MOK_OK;
      float ms = 0.0f;
      ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
      if (!ok) continue;
      ms /= static_cast<float>(reps);
      if (!found || ms < best_t) { found = true; best_t = ms; best_d = d; }
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (!found) return MOK_ERR_UNSUPPORTED;
  *best = best_d;
  *best_ms = best_t;
  return MOK_OK;
}

mok_status mok_device_status(const void* ws, int32_t* status_host, hipStream_t stream) {
  if (!ws || !status_host) return MOK_ERR_INVALID_ARG;
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(status_host, ws, sizeof(int32_t), hipMemcpyDeviceToHost);
  return hip_status(e);
}

const char* mok_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

}  // extern "C"
