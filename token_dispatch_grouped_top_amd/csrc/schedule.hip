// schedule.hip -- per-expert counts, offsets and the pull table, on device.
//
// tahou.com MoK article, layout-planning paragraph: count the tokens per
// expert, then plan positions so that one expert's tokens are contiguous for
// the grouped GEMM.  PyTorchKR wiki summary, key point on scheduling: the
// {src_rank, src_index} pull schedule is built on the device with no sort and
// no CPU-GPU exchange.  Reading of the slot order (not fixed by the pages):
// stable in assignment id a = t*k + j, i.e. a counting sort.
//
// Two launches, no atomics on the data path, so the result is unique:
//   count   -- each block takes a chunk of 2048 assignments; each wave takes
//              512 consecutive ones in 8 steps of 64 and groups equal keys
//              with ballots on the key bits (match_key); the lowest lane of a
//              group adds the group size to the wave's LDS histogram.
//   scatter -- every block sums the per-block counts into the expert totals
//              and its own block prefix (a wave per expert), scans
//              the totals into offsets (block 0 writes counts and offsets),
//              recounts per wave; wave cursor = offsets[e] + block prefix +
//              prefix over the block's waves; each lane's slot = wave cursor
//              + popcount(group & lanes below).
// A wave loads the keys of all its steps before the first ballot.
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kSchedThreads = 256;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kStepsPerWave = 8;    // 8: 14.6 us for the two launches at 589,824 ids; 16: 19.2
constexpr int kChunk = kSchedThreads * kStepsPerWave;  // 2048 assignments per block
static_assert(kChunk == kSchedChunk, "chunk of the route's counts");
constexpr int kMaxLocal = 256;

__device__ __forceinline__ int key_bits(int32_t n_local) { return 32 - __clz(n_local); }

// The keys of a wave's 1024 assignments, all loaded before any is used: the
// loads are unconditional (index clamped into [0, A)), so they are issued
// back to back instead of one guarded load and wait per step.  A >= 1.
__device__ __forceinline__ void load_keys(const int32_t* __restrict__ idx, int64_t A, int32_t base,
                                          int32_t n_local, int64_t a0, uint32_t (&keys)[kStepsPerWave]) {
  const int lane = lane_id();
  int32_t v[kStepsPerWave];
#pragma unroll
  for (int it = 0; it < kStepsPerWave; ++it) {
    const int64_t a = a0 + it * kWave + lane;
    v[it] = idx[a < A ? a : A - 1];
  }
#pragma unroll
  for (int it = 0; it < kStepsPerWave; ++it) {
    const int64_t a = a0 + it * kWave + lane;
    const int32_t e = v[it] - base;
    keys[it] = (a < A && e >= 0 && e < n_local) ? static_cast<uint32_t>(e)
                                                 : static_cast<uint32_t>(n_local);
  }
}

// Per-wave histogram of the block's chunk into h[wave][e].
__device__ void wave_histogram(const uint32_t (&keys)[kStepsPerWave], int32_t n_local,
                               int32_t (*h)[kMaxLocal]) {
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int nbits = key_bits(n_local);
  for (int e = lane; e < n_local; e += kWave) h[w][e] = 0;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int it = 0; it < kStepsPerWave; ++it) {
    uint32_t key = keys[it];
    uint64_t peers = match_key(key, nbits);
    bool leader = (peers & lanemask_lt()) == 0;
    if (leader && key < static_cast<uint32_t>(n_local)) h[w][key] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(kSchedThreads)
void k_sched_count(const int32_t* __restrict__ idx, int64_t A, int32_t base, int32_t n_local,
                   int32_t nblk, int32_t* __restrict__ blk_counts) {
  __shared__ int32_t h[kSchedWaves][kMaxLocal];
  uint32_t keys[kStepsPerWave];
  if (A > 0) {
    load_keys(idx, A, base, n_local,
              static_cast<int64_t>(blockIdx.x) * kChunk + (threadIdx.x / kWave) * (kWave * kStepsPerWave),
              keys);
  } else {
#pragma unroll
    for (int it = 0; it < kStepsPerWave; ++it) keys[it] = static_cast<uint32_t>(n_local);
  }
  wave_histogram(keys, n_local, h);
  __syncthreads();
  for (int e = threadIdx.x; e < n_local; e += kSchedThreads) {
    int32_t c = 0;
#pragma unroll
    for (int w = 0; w < kSchedWaves; ++w) c += h[w][e];
    blk_counts[static_cast<int64_t>(e) * nblk + blockIdx.x] = c;
  }
}

__global__ __launch_bounds__(kSchedThreads)
void k_sched_scatter(const int32_t* __restrict__ idx, int64_t A, int32_t base, int32_t n_local,
                     int32_t nblk, const int32_t* __restrict__ blk_counts,
                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                     int32_t* __restrict__ soa, int32_t* __restrict__ aos, int32_t M,
                     int32_t nwin, int32_t* __restrict__ win_seg, int32_t cap,
                     int32_t* __restrict__ status) {
  __shared__ int32_t h[kSchedWaves][kMaxLocal];
  __shared__ int32_t cur[kSchedWaves][kMaxLocal];
  __shared__ int32_t tot[kMaxLocal], pre[kMaxLocal], off[kMaxLocal + 1];
  const int64_t a0w =
      static_cast<int64_t>(blockIdx.x) * kChunk + (threadIdx.x / kWave) * (kWave * kStepsPerWave);
  uint32_t keys[kStepsPerWave];
  if (A > 0) {
    load_keys(idx, A, base, n_local, a0w, keys);
  } else {
#pragma unroll
    for (int it = 0; it < kStepsPerWave; ++it) keys[it] = static_cast<uint32_t>(n_local);
  }
  const int w = threadIdx.x / kWave, lane = lane_id();
  // per expert: total over all blocks and prefix over the blocks before this
  // one; one wave per expert, lanes striding over the blocks
  for (int e = w; e < n_local; e += kSchedWaves) {
    const int32_t* bc = blk_counts + static_cast<int64_t>(e) * nblk;
    int32_t t = 0, p = 0;
    for (int j = lane; j < nblk; j += kWave) {
      const int32_t v = bc[j];
      t += v;
      p += j < static_cast<int>(blockIdx.x) ? v : 0;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      t += __shfl_xor(t, o);
      p += __shfl_xor(p, o);
    }
    if (lane == 0) { tot[e] = t; pre[e] = p; }
  }
  wave_histogram(keys, n_local, h);
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int e = 0; e < n_local; ++e) { off[e] = acc; acc += tot[e]; }
    off[n_local] = acc;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e <= n_local; e += kSchedThreads) {
      offsets[e] = off[e];
      if (e < n_local) counts[e] = tot[e];
    }
    // the fused layer's window table and capacity check (win_seg null: not asked)
    if (win_seg) {
      const int64_t R = off[n_local];
      const int64_t n = static_cast<int64_t>(nwin) * (n_local + 1);
      for (int64_t i = threadIdx.x; i < n; i += kSchedThreads) {
        const int64_t b = i / (n_local + 1), e = i % (n_local + 1);
        int64_t lo = b * M, hi = lo + M;
        if (lo > R) lo = R;
        if (hi > R) hi = R;
        int64_t v = off[e];
        win_seg[i] = static_cast<int32_t>(v < lo ? lo : (v > hi ? hi : v));
      }
      if (threadIdx.x == 0 && R > cap) set_status(status, MOK_ERR_CAPACITY);
    }
  }
  for (int e = threadIdx.x; e < n_local; e += kSchedThreads) {
    int32_t b = off[e] + pre[e];
#pragma unroll
    for (int w = 0; w < kSchedWaves; ++w) { cur[w][e] = b; b += h[w][e]; }
  }
  __syncthreads();
  const int nbits = key_bits(n_local);
#pragma unroll
  for (int it = 0; it < kStepsPerWave; ++it) {
    const int64_t a = a0w + it * kWave + lane;
    uint32_t key = keys[it];
    uint64_t peers = match_key(key, nbits);
    bool local = key < static_cast<uint32_t>(n_local);
    int32_t c = local ? cur[w][key] : 0;
    int32_t slot = c + __popcll(peers & lanemask_lt());
    if (a < A) {
      soa[a] = local ? slot : -1;
      if (local) aos[slot] = static_cast<int32_t>(a);
    }
    __builtin_amdgcn_wave_barrier();
    if (local && (peers & lanemask_lt()) == 0) cur[w][key] = c + __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ void k_windows(const int32_t* __restrict__ offsets, int32_t n_local, int32_t M,
                          int32_t nwin, int32_t* __restrict__ win_seg) {
  const int64_t R = offsets[n_local];
  const int64_t n = static_cast<int64_t>(nwin) * (n_local + 1);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    int64_t b = i / (n_local + 1), e = i % (n_local + 1);
    int64_t lo = b * M, hi = lo + M;
    if (lo > R) lo = R;
    if (hi > R) hi = R;
    int64_t v = offsets[e];
    v = v < lo ? lo : (v > hi ? hi : v);
    win_seg[i] = static_cast<int32_t>(v);
  }
}

}  // namespace

size_t sched_ws_bytes(int64_t A, int32_t n_local) {
  int64_t nblk = (A + kChunk - 1) / kChunk;
  if (nblk < 1) nblk = 1;
  return static_cast<size_t>(2 * nblk * n_local) * sizeof(int32_t) + 256;
}

SchedWs sched_ws_carve(void* ws, int64_t A, int32_t n_local) {
  SchedWs w;
  int64_t nblk = (A + kChunk - 1) / kChunk;
  if (nblk < 1) nblk = 1;
  w.nblk = static_cast<int32_t>(nblk);
  w.blk_counts = static_cast<int32_t*>(ws);
  return w;
}

hipError_t launch_schedule(const int32_t* idx, int64_t A, int32_t expert_base, int32_t n_local,
                           int32_t* counts, int32_t* offsets, int32_t* soa, int32_t* aos,
                           const SchedWs& w, hipStream_t s) {
  if (n_local > kMaxLocal) return hipErrorInvalidValue;
  if (A > 0) {
    hipLaunchKernelGGL(k_sched_count, dim3(w.nblk), dim3(kSchedThreads), 0, s, idx, A,
                       expert_base, n_local, w.nblk, w.blk_counts);
  } else {
    hipLaunchKernelGGL(k_sched_count, dim3(1), dim3(kSchedThreads), 0, s, idx, A, expert_base,
                       n_local, w.nblk, w.blk_counts);
  }
  hipLaunchKernelGGL(k_sched_scatter, dim3(A > 0 ? w.nblk : 1), dim3(kSchedThreads), 0, s, idx, A,
                     expert_base, n_local, w.nblk, w.blk_counts, counts, offsets, soa, aos, 0, 0,
                     nullptr, 0, nullptr);
  return hipGetLastError();
}

hipError_t launch_route_schedule(const float* route_logits, int32_t E, float* gate,
                                 int32_t* idx, int64_t T, int32_t k, int32_t expert_base,
                                 int32_t n_local, int32_t* counts, int32_t* offsets, int32_t* soa,
                                 int32_t* aos, const SchedWs& w, int32_t M, int32_t nwin,
                                 int32_t* win_seg, int32_t cap, int32_t* status, hipStream_t s,
                                 bool counted) {
  if (n_local > kMaxLocal) return hipErrorInvalidValue;
  const int64_t A = T * k;
  hipError_t e = hipSuccess;
  if (counted && T > 0) {
    // the chunk counts come from the caller's route
  } else if (route_logits && T > 0) {
    e = launch_route_count(route_logits, static_cast<int32_t>(T), E, k, expert_base, n_local, idx,
                           gate, w.blk_counts, w.nblk, s);
  } else {
    hipLaunchKernelGGL(k_sched_count, dim3(A > 0 ? w.nblk : 1), dim3(kSchedThreads), 0, s, idx, A,
                       expert_base, n_local, w.nblk, w.blk_counts);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sched_scatter, dim3(A > 0 ? w.nblk : 1), dim3(kSchedThreads), 0, s, idx, A,
                     expert_base, n_local, w.nblk, w.blk_counts, counts, offsets, soa, aos, M,
                     nwin, win_seg, cap, status);
  return hipGetLastError();
}

hipError_t launch_windows(const int32_t* offsets, int32_t n_local, int32_t M, int32_t nwin,
                          int32_t* win_seg, hipStream_t s) {
  int64_t n = static_cast<int64_t>(nwin) * (n_local + 1);
  if (n == 0) return hipSuccess;
  int blocks = static_cast<int>((n + 255) / 256);
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_windows, dim3(blocks), dim3(256), 0, s, offsets, n_local, M, nwin,
                     win_seg);
  return hipGetLastError();
}

}  // namespace mok
