// movers.hip -- standalone pull dispatch (gather into the ring) and push
// combine with the final weighted merge; the row routines are in
// movers_dev.h.  Both kernels are HBM-bound row copies / reductions: the
// gather takes two consecutive slots per wave, the merge one token per wave,
// 4 waves per 256-thread workgroup.
#include "movers_dev.h"

namespace mok {

namespace {

using namespace movers;

constexpr int kRowsPerBlock = 4;   // waves per block (merge: one token each)
constexpr int kGatherWaves = 4;    // waves per block (gather)
// Waves per slot pair, each moving a contiguous share of the pair's pieces:
// 2 for the bf16 copy, 4 for the MXFP8 gather, whose quantisation keeps each
// wave longer between its loads and stores (measured inside the bench step
// on the Kimi-shaped share: bf16 53.5 -> 50 us with 2, MXFP8 62 -> 51 us
// with 4, against one wave per pair).
template <bool MX> struct GatherShape { static constexpr int kWavesPerPair = MX ? 4 : 2; };

// The wave's slots s and s + 1, their tokens t1, t2 (t2 = -1 when s + 1 is
// past the end) and its share [p_lo, p_hi) of the pair's 16-byte pieces
// (whole 2 G-piece groups, G = 4 bf16 / 8 E4M3); false: nothing to do.
template <bool MX>
__device__ __forceinline__ bool gather_slots(const int32_t* __restrict__ aos,
                                             const int32_t* __restrict__ offsets, int32_t n_local,
                                             int32_t k, int32_t H, int32_t s_begin, int32_t s_end,
                                             int64_t& s, int64_t& t1, int64_t& t2, int& p_lo,
                                             int& p_hi) {
  constexpr int G = MX ? 8 : 4, kWavesPerPair = GatherShape<MX>::kWavesPerPair;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * kGatherWaves + threadIdx.x / kWave;
  s = static_cast<int64_t>(s_begin) + 2 * (wid / kWavesPerPair);
  const int npc = 2 * (H / 8);
  const int share = (npc / (2 * G) + kWavesPerPair - 1) / kWavesPerPair * (2 * G);
  p_lo = static_cast<int>(wid % kWavesPerPair) * share;
  p_hi = p_lo + share < npc ? p_lo + share : npc;
  if (p_lo >= p_hi) return false;
  if (s >= s_end) return false;
  const int32_t a1 = aos[s];                             // aos holds s_end entries: both are
  const int32_t a2 = s + 1 < s_end ? aos[s + 1] : 0;     // issued together with R
  const int32_t R = offsets[n_local];
  if (s >= R) return false;
  t1 = a1 / k;
  t2 = s + 1 < s_end && s + 1 < R ? a2 / k : -1;
  return true;
}

__global__ __launch_bounds__(kGatherWaves * kWave)
void k_gather_bf16(void* const* __restrict__ parts, int32_t n_part, int32_t part_rows,
                   int32_t H, int32_t k, const int32_t* __restrict__ aos,
                   const int32_t* __restrict__ offsets, int32_t n_local, int32_t s_begin,
                   int32_t s_end, uint16_t* __restrict__ ring, int32_t ring_slots,
                   int32_t* status) {
  int64_t s, t1, t2;
  int p_lo, p_hi;
  if (!gather_slots<false>(aos, offsets, n_local, k, H, s_begin, s_end, s, t1, t2, p_lo, p_hi)) return;
  gather_pair_bf16(parts, n_part, part_rows, H, t1, t2, ring, s % ring_slots, (s + 1) % ring_slots,
                   ring_slots, p_lo, p_hi, status);
}

__global__ __launch_bounds__(kGatherWaves * kWave)
void k_gather_mxfp8(void* const* __restrict__ parts, int32_t n_part, int32_t part_rows,
                    int32_t H, int32_t k, const int32_t* __restrict__ aos,
                    const int32_t* __restrict__ offsets, int32_t n_local, int32_t s_begin,
                    int32_t s_end, uint8_t* __restrict__ ring, uint8_t* __restrict__ scales,
                    int32_t ring_slots, int32_t* status) {
  int64_t s, t1, t2;
  int p_lo, p_hi;
  if (!gather_slots<true>(aos, offsets, n_local, k, H, s_begin, s_end, s, t1, t2, p_lo, p_hi)) return;
  gather_pair_mxfp8(parts, n_part, part_rows, H, t1, t2, ring, scales, s % ring_slots,
                    (s + 1) % ring_slots, ring_slots, p_lo, p_hi, status);
}

__global__ __launch_bounds__(kRowsPerBlock * kWave)
void k_combine(const uint16_t* __restrict__ y, int32_t y_rows, const int32_t* __restrict__ soa,
               const float* __restrict__ gate, int32_t T, int32_t k, int32_t H,
               void* const* __restrict__ out_parts, int32_t n_part, int32_t part_rows,
               int32_t* status, bool abort_on_status) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  if (abort_on_status && *status != 0) return;   // capacity exceeded: leave out untouched
  combine_token(y, y_rows, soa, gate, t, k, H, out_parts, n_part, part_rows, status);
}

// Slot-driven variant: one wave per routed slot s < min(R, n_slots).
__global__ __launch_bounds__(kRowsPerBlock * kWave)
void k_combine_slots(const uint16_t* __restrict__ y, int32_t y_rows,
                     const int32_t* __restrict__ aos, const int32_t* __restrict__ offsets,
                     int32_t n_local, int32_t n_slots, const int32_t* __restrict__ soa,
                     const float* __restrict__ gate, int32_t k, int32_t H,
                     void* const* __restrict__ out_parts, int32_t n_part, int32_t part_rows,
                     int32_t* status, bool abort_on_status, bool multi_only) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kWave;
  if (s >= n_slots) return;
  const int32_t a = aos[s];                 // issued together with R (aos holds n_slots entries)
  const int32_t R = offsets[n_local];
  if (s >= R) return;
  if (abort_on_status && *status != 0) return;
  merge_slot(y, y_rows, a, soa, gate, s, k, H, out_parts, n_part, part_rows, status, multi_only);
}

// One wave per routed slot s < min(R, n_slots): the backward of the merge.
__global__ __launch_bounds__(kRowsPerBlock * kWave)
void k_unmerge_slots(void* const* __restrict__ dout_parts, int32_t n_part, int32_t part_rows,
                     const uint16_t* __restrict__ y, int32_t y_rows,
                     const int32_t* __restrict__ aos, const int32_t* __restrict__ offsets,
                     int32_t n_local, int32_t n_slots, const float* __restrict__ gate, int32_t k,
                     int32_t H, uint8_t* __restrict__ dy, uint8_t* __restrict__ dy_scales,
                     int32_t dy_rows, float* __restrict__ dgate, int32_t* status) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kWave;
  if (s >= n_slots) return;
  const int32_t a = aos[s];                 // issued together with R (aos holds n_slots entries)
  const int32_t R = offsets[n_local];
  if (s >= R) return;
  if (dy_scales)                            // MXFP8 dy (uniform over the launch)
    unmerge_slot_mx(dout_parts, n_part, part_rows, y, y_rows, a, gate, s, k, H, dy, dy_scales,
                    dy_rows, dgate, status);
  else
    unmerge_slot(dout_parts, n_part, part_rows, y, y_rows, a, gate, s, k, H, dy, dy_rows, dgate,
                 status);
}

// Merge plan of the slots [s0, min(s1, R)): plan[s] = {address of token t's
// output row (lo, hi), gate bits, 0} when s is the only local slot of its
// token t (exactly one slot_of_assign[t][j] >= 0) and t lies in the output
// partitions, else zeros.  One thread per slot; read by the down GEMM's
// merging epilogue.
__global__ __launch_bounds__(256)
void k_merge_plan(const int32_t* __restrict__ aos, const int32_t* __restrict__ offsets,
                  int32_t n_local, int32_t s0, int32_t s1, const int32_t* __restrict__ soa,
                  const float* __restrict__ gate, int32_t k, int32_t H,
                  void* const* __restrict__ out_parts, int32_t n_part, int32_t part_rows,
                  uint4* __restrict__ plan) {
  const int64_t s = s0 + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int32_t R = offsets[n_local];
  if (s >= s1 || s >= R) return;
  const int32_t a = aos[s];
  const int64_t t = a / k;
  int live = 0;
  for (int j = 0; j < k; ++j) live += soa[t * k + j] >= 0 ? 1 : 0;
  uint4 rec = make_uint4(0, 0, 0, 0);
  const int64_t part = t / part_rows;
  if (live == 1 && part < n_part) {
    const uint64_t addr = reinterpret_cast<uint64_t>(static_cast<uint16_t*>(out_parts[part]) +
                                                     (t % part_rows) * static_cast<int64_t>(H));
    rec = make_uint4(static_cast<uint32_t>(addr), static_cast<uint32_t>(addr >> 32),
                     __float_as_uint(gate[a]), 0u);
  }
  plan[s] = rec;
}

}  // namespace

hipError_t launch_merge_plan(const int32_t* aos, const int32_t* offsets, int32_t n_local,
                             int32_t s0, int32_t s1, const int32_t* soa, const float* gate,
                             int32_t k, int32_t H, void* const* out_parts, int32_t n_part,
                             int32_t part_rows, void* plan, hipStream_t s) {
  if (s1 <= s0) return hipSuccess;
  const int64_t n = static_cast<int64_t>(s1) - s0;
  hipLaunchKernelGGL(k_merge_plan, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     aos, offsets, n_local, s0, s1, soa, gate, k, H, out_parts, n_part, part_rows,
                     static_cast<uint4*>(plan));
  return hipGetLastError();
}

hipError_t launch_unmerge_slots(void* const* dout_ptr, int32_t n_part, int32_t part_rows,
                                const void* y, int32_t y_rows, const int32_t* aos,
                                const int32_t* offsets, int32_t n_local, int32_t n_slots,
                                const float* gate, int32_t k, int32_t H, void* dy,
                                uint8_t* dy_scales, int32_t dy_rows, float* dgate, int32_t* status,
                                hipStream_t s) {
  if (n_slots <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((static_cast<int64_t>(n_slots) + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(k_unmerge_slots, grid, dim3(kRowsPerBlock * kWave), 0, s, dout_ptr, n_part,
                     part_rows, static_cast<const uint16_t*>(y), y_rows, aos, offsets, n_local,
                     n_slots, gate, k, H, static_cast<uint8_t*>(dy), dy_scales, dy_rows, dgate,
                     status);
  return hipGetLastError();
}

hipError_t launch_gather(void* const* part_ptr, int32_t n_part, int32_t part_rows, int32_t H,
                         int32_t k, const int32_t* aos, const int32_t* offsets, int32_t n_local,
                         int32_t s_begin, int32_t s_end, void* ring, uint8_t* ring_scales,
                         int32_t ring_slots, int32_t act_format, int32_t* status, hipStream_t s) {
  int64_t rows = static_cast<int64_t>(s_end) - s_begin;
  if (rows <= 0) return hipSuccess;
  const bool mx = act_format == MOK_ACT_MXFP8_E4M3;
  const int64_t waves = (rows + 1) / 2 * (mx ? GatherShape<true>::kWavesPerPair
                                              : GatherShape<false>::kWavesPerPair);
  dim3 grid(static_cast<unsigned>((waves + kGatherWaves - 1) / kGatherWaves));
  if (mx) {
    hipLaunchKernelGGL(k_gather_mxfp8, grid, dim3(kGatherWaves * kWave), 0, s, part_ptr, n_part,
                       part_rows, H, k, aos, offsets, n_local, s_begin, s_end,
                       static_cast<uint8_t*>(ring), ring_scales, ring_slots, status);
  } else {
    hipLaunchKernelGGL(k_gather_bf16, grid, dim3(kGatherWaves * kWave), 0, s, part_ptr, n_part,
                       part_rows, H, k, aos, offsets, n_local, s_begin, s_end,
                       static_cast<uint16_t*>(ring), ring_slots, status);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, int32_t y_rows, const int32_t* soa, const float* gate,
                          int32_t T, int32_t k, int32_t H, void* const* out_ptr, int32_t n_part,
                          int32_t part_rows, int32_t* status, bool abort_on_status,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((static_cast<int64_t>(T) + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(k_combine, grid, dim3(kRowsPerBlock * kWave), 0, s,
                     static_cast<const uint16_t*>(y), y_rows, soa, gate, T, k, H, out_ptr,
                     n_part, part_rows, status, abort_on_status && status != nullptr);
  return hipGetLastError();
}

hipError_t launch_combine_slots(const void* y, int32_t y_rows, const int32_t* aos,
                                const int32_t* offsets, int32_t n_local, int32_t n_slots,
                                const int32_t* soa, const float* gate, int32_t k, int32_t H,
                                void* const* out_ptr, int32_t n_part, int32_t part_rows,
                                int32_t* status, bool abort_on_status, hipStream_t s,
                                bool multi_only) {
  if (n_slots <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((static_cast<int64_t>(n_slots) + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(k_combine_slots, grid, dim3(kRowsPerBlock * kWave), 0, s,
                     static_cast<const uint16_t*>(y), y_rows, aos, offsets, n_local, n_slots, soa,
                     gate, k, H, out_ptr, n_part, part_rows, status,
                     abort_on_status && status != nullptr, multi_only);
  return hipGetLastError();
}

}  // namespace mok
