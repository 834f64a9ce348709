// route.hip -- top-k routing with softmax gates over the picks.
//
// tahou.com MoK article, routing paragraph: the router assigns each token to
// experts.  Reading used (the pages fix no details): the k largest logits,
// equal logits resolved to the lower expert id, picks in descending order,
// gates = softmax over the k picked logits.
//
// One wave per token.  Lane l holds logits l, l+64, l+128, ... in registers;
// each of the k rounds is a lane-local argmax, then the best of each 16-lane
// row by DPP moves (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row half-mirror,
// row mirror), then the four rows' bests read with readlane.  Every step keeps
// the better pair under one total order (value descending, expert id
// ascending), so the pick does not depend on the order of the steps.  Gates:
// lanes 0..k-1 hold the picked logits; e_j = exp(l_j - l_0) in fp32, summed
// by a butterfly, divided.
//
// k_route_count (the fused layer): the same route, and each lane holding a
// pick of a local expert adds one to that expert's count of the pick's
// schedule chunk (integer atomics: the counts do not depend on their order),
// so the schedule's separate count launch is not needed.
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kRouteWaves = 4;

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

// (bv, be) <- the better of its own pair and the pair of the lane that DPP
// control CTRL names (every lane has a source under the row patterns used).
template <int CTRL>
__device__ __forceinline__ void best_dpp(float& bv, int& be) {
  const float ov = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bv), CTRL, 0xF, 0xF, false));
  const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xF, 0xF, false);
  if (better(ov, oe, bv, be)) { bv = ov; be = oe; }
}

// Picks and gates of token t from its logits v (lane l holds logits l,
// l + 64, ...; -inf past E).  All 64 lanes call it.
template <int VPL>
__device__ __forceinline__ int pick_topk(const float (&v)[VPL], int32_t E, int32_t k, int64_t t,
                                         int32_t* __restrict__ idx, float* __restrict__ gate) {
  const int lane = lane_id();
  uint64_t taken = 0;  // bit i: v[i] already picked
  float mine = 0.0f;   // lane j keeps the j-th picked logit
  int mine_e = 0;

  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      int e = lane + kWave * i;
      if (!((taken >> i) & 1ull) && e < E && better(v[i], e, bv, be)) { bv = v[i]; be = e; }
    }
    // best of the wave: within each 16-lane row by DPP (xor 1, xor 2, then
    // lane i with 7 - i and with 15 - i), then the four rows' results read
    // into scalars.  `better` is a total order, so the steps' order does not
    // change the pick.
    best_dpp<0xB1>(bv, be);                              // quad_perm [1,0,3,2]
    best_dpp<0x4E>(bv, be);                              // quad_perm [2,3,0,1]
    best_dpp<0x141>(bv, be);                             // row_half_mirror
    best_dpp<0x140>(bv, be);                             // row_mirror
    {
      float rv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 0));
      int re = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
      for (int row = 1; row < 4; ++row) {
        const float ov = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 16 * row));
        const int oe = __builtin_amdgcn_readlane(be, 16 * row);
        if (better(ov, oe, rv, re)) { rv = ov; re = oe; }
      }
      bv = rv; be = re;
    }
    if ((be & (kWave - 1)) == lane) taken |= 1ull << (be / kWave);
    if (lane == j) { mine = bv; mine_e = be; }
  }

  const float l0 = __shfl(mine, 0);
  float ex = lane < k ? expf(mine - l0) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    idx[t * k + lane] = mine_e;
    gate[t * k + lane] = ex / sum;
  }
  return mine_e;                 // lane j < k: the j-th pick
}

template <int VPL>
__global__ __launch_bounds__(kRouteWaves * kWave)
void k_route_topk(const float* __restrict__ logits, int32_t T, int32_t E, int32_t k,
                  int32_t* __restrict__ idx, float* __restrict__ gate) {
  const int lane = lane_id();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteWaves + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = logits + t * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + kWave * i;
    v[i] = e < E ? row[e] : -__builtin_inff();
  }
  pick_topk<VPL>(v, E, k, t, idx, gate);
}

template <int VPL>
__global__ __launch_bounds__(kRouteWaves * kWave)
void k_route_count(const float* __restrict__ logits, int32_t T, int32_t E, int32_t k, int32_t base,
                   int32_t n_local, int32_t* __restrict__ idx, float* __restrict__ gate,
                   int32_t* __restrict__ blk_counts, int32_t nblk) {
  const int lane = lane_id();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteWaves + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = logits + t * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + kWave * i;
    v[i] = e < E ? row[e] : -__builtin_inff();
  }
  const int e = pick_topk<VPL>(v, E, k, t, idx, gate) - base;
  if (lane < k && e >= 0 && e < n_local) {
    const int64_t chunk = (t * k + lane) / kSchedChunk;
    __hip_atomic_fetch_add(blk_counts + static_cast<int64_t>(e) * nblk + chunk, 1,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------- router GEMM + top-k
// logits = x . w_r^T (bf16 inputs, fp32 sums), never stored whole.
// Pass 1 (k_router_partial): a workgroup takes 64 tokens x 128 experts x one
// split of H, in k-steps of 64.  Each k-step's 64 + 128 rows of 128 bytes go
// global -> registers -> LDS with 16-byte loads, 8 lanes per 128-byte line,
// the next k-step's loads in flight while the current one is multiplied;
// chunks are XOR-swizzled per row so the fragment reads of 8 rows hit
// distinct banks.  Wave w multiplies tokens 32 (w % 2) .. + 31 against
// experts 64 (w / 2) .. + 63 with v_mfma_f32_32x32x16_bf16 (slice s of a
// k-step: lane l reads row l % 32, chunk 2 s + l / 32).  Fed (router rows,
// tokens), lane l ends with token t0 + 32 (w % 2) + l % 32 and experts
// e0 + 64 (w / 2) + 32 ni + 8 (q / 4) + 4 (l / 32) + q % 4, stored to
// partial[split][t][e].  Pass 2 (k_route_topk_sum): one wave per token adds
// the splits in split order (so the result does not depend on timing) and
// picks as k_route_topk.
typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x16_t __attribute__((ext_vector_type(16)));
constexpr int kRgTok = 64, kRgExp = 128, kRgK = 64, kRgRowB = kRgK * 2;
constexpr int kRgRows = kRgTok + kRgExp;                   // LDS rows per buffer
constexpr int kRgLoads = kRgRows * kRgRowB / (256 * 16);   // 16-byte loads per thread: 6

__global__ __launch_bounds__(4 * kWave)
void k_router_partial(const uint16_t* __restrict__ x, void* const* __restrict__ x_parts,
                      int32_t x_part_rows, const uint16_t* __restrict__ wr,
                      int32_t T, int32_t H, int32_t E, int32_t kchunk,
                      float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kRgRows * kRgRowB];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int t0 = blockIdx.x * kRgTok, e0 = blockIdx.y * kRgExp;
  const int split = blockIdx.z;
  const int kb = split * kchunk, ke = kb + kchunk < H ? kb + kchunk : H;
  const int nks = ke > kb ? (ke - kb + kRgK - 1) / kRgK : 0;
  // loader: thread tid moves chunk tid % 8 of LDS rows tid / 8 + 32 j
  // (rows 0..63 tokens, 64..191 router rows; rows past T or E repeat the
  // last one, k past ke reads zeros)
  const int lc = tid & 7;
  const uint16_t* src[kRgLoads];
  int dst[kRgLoads];
#pragma unroll
  for (int j = 0; j < kRgLoads; ++j) {
    const int row = tid / 8 + 32 * j;
    const uint16_t* base;
    if (row < kRgTok) {
      const int t = t0 + row < T ? t0 + row : T - 1;
      // token rows: one array x[T][H], or partitions (row t % part_rows of
      // partition t / part_rows)
      base = x_parts ? static_cast<const uint16_t*>(x_parts[t / x_part_rows]) +
                           static_cast<int64_t>(t % x_part_rows) * H
                     : x + static_cast<int64_t>(t) * H;
    } else {
      const int e = e0 + row - kRgTok < E ? e0 + row - kRgTok : E - 1;
      base = wr + static_cast<int64_t>(e) * H;
    }
    src[j] = base + 8 * lc;
    dst[j] = row * kRgRowB + ((lc ^ (row & 7)) << 4);
  }
  auto load = [&](int ks, uint4 (&r)[kRgLoads]) {
    const int k = kb + ks * kRgK;
#pragma unroll
    for (int j = 0; j < kRgLoads; ++j)
      r[j] = k + 8 * lc < ke ? *reinterpret_cast<const uint4*>(src[j] + k) : make_uint4(0, 0, 0, 0);
  };
  auto store = [&](int buf, const uint4 (&r)[kRgLoads]) {
#pragma unroll
    for (int j = 0; j < kRgLoads; ++j) *reinterpret_cast<uint4*>(&lds[buf][dst[j]]) = r[j];
  };
  const int tb = wave & 1, eb = wave >> 1, fr = lane & 31, kh = lane >> 5;
  rf32x16_t acc[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[ni][q] = 0.0f;
  // two k-steps of loads in flight: registers ra / rb alternate between the
  // step being loaded (ks + 2) and the one waiting for its LDS buffer (ks + 1)
  auto mma = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kRgK / 16; ++s) {
      const int c = 2 * s + kh;
      const int xr = 32 * tb + fr;
      const rbf16x8_t xf = *reinterpret_cast<const rbf16x8_t*>(&lds[buf][xr * kRgRowB + ((c ^ (xr & 7)) << 4)]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int wrow = kRgTok + 64 * eb + 32 * ni + fr;
        const rbf16x8_t wf =
            *reinterpret_cast<const rbf16x8_t*>(&lds[buf][wrow * kRgRowB + ((c ^ (wrow & 7)) << 4)]);
        acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf, acc[ni], 0, 0, 0);
      }
    }
  };
  uint4 ra[kRgLoads], rb[kRgLoads];
  if (nks > 0) load(0, ra);
  if (nks > 1) load(1, rb);
  if (nks > 0) store(0, ra);
  __syncthreads();
  for (int ks = 0; ks < nks; ks += 2) {
    if (ks + 2 < nks) load(ks + 2, ra);
    mma(0);
    if (ks + 1 < nks) store(1, rb);
    __syncthreads();
    if (ks + 1 >= nks) break;
    if (ks + 3 < nks) load(ks + 3, rb);
    mma(1);
    if (ks + 2 < nks) store(0, ra);
    __syncthreads();
  }
  const int t = t0 + 32 * tb + fr;
  if (t >= T) return;
  float* out = partial + (static_cast<int64_t>(split) * T + t) * E;
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int e = e0 + 64 * eb + 32 * ni + 8 * g + 4 * kh;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (e + q < E) out[e + q] = acc[ni][4 * g + q];
    }
}

template <int VPL>
__global__ __launch_bounds__(kRouteWaves * kWave)
void k_route_topk_sum(const float* __restrict__ partial, int32_t n_split, int32_t T, int32_t E,
                      int32_t k, int32_t* __restrict__ idx, float* __restrict__ gate, int32_t base,
                      int32_t n_local, int32_t* __restrict__ blk_counts, int32_t nblk) {
  const int lane = lane_id();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteWaves + threadIdx.x / kWave;
  if (t >= T) return;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = 0.0f;
  // splits in groups of 4: a group's loads are issued together, then added in
  // split order
  for (int sp0 = 0; sp0 < n_split; sp0 += 4) {
    float tmp[4][VPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* row = partial + (static_cast<int64_t>(sp0 + u) * T + t) * E;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        tmp[u][i] = sp0 + u < n_split && e < E ? row[e] : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (sp0 + u < n_split) v[i] += tmp[u][i];
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (lane + kWave * i >= E) v[i] = -__builtin_inff();
  const int e = pick_topk<VPL>(v, E, k, t, idx, gate) - base;
  // the fused layer's schedule counts (as k_route_count)
  if (blk_counts && lane < k && e >= 0 && e < n_local) {
    const int64_t chunk = (t * k + lane) / kSchedChunk;
    __hip_atomic_fetch_add(blk_counts + static_cast<int64_t>(e) * nblk + chunk, 1,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int VPL>
hipError_t launch_vpl(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* idx,
                      float* gate, hipStream_t s) {
  dim3 grid((T + kRouteWaves - 1) / kRouteWaves);
  hipLaunchKernelGGL(k_route_topk<VPL>, grid, dim3(kRouteWaves * kWave), 0, s, logits, T, E, k,
                     idx, gate);
  return hipGetLastError();
}

template <int VPL>
hipError_t launch_count_vpl(const float* logits, int32_t T, int32_t E, int32_t k, int32_t base,
                            int32_t n_local, int32_t* idx, float* gate, int32_t* blk_counts,
                            int32_t nblk, hipStream_t s) {
  dim3 grid((T + kRouteWaves - 1) / kRouteWaves);
  hipLaunchKernelGGL(k_route_count<VPL>, grid, dim3(kRouteWaves * kWave), 0, s, logits, T, E, k,
                     base, n_local, idx, gate, blk_counts, nblk);
  return hipGetLastError();
}

template <int VPL>
hipError_t launch_sum_vpl(const float* partial, int32_t n_split, int32_t T, int32_t E, int32_t k,
                          int32_t* idx, float* gate, const RouteCount& rc, hipStream_t s) {
  dim3 grid((T + kRouteWaves - 1) / kRouteWaves);
  hipLaunchKernelGGL(k_route_topk_sum<VPL>, grid, dim3(kRouteWaves * kWave), 0, s, partial, n_split,
                     T, E, k, idx, gate, rc.base, rc.n_local, rc.blk_counts, rc.nblk);
  return hipGetLastError();
}

}  // namespace

// Splits of H for the router GEMM: about one workgroup per CU of a 256-CU
// part in all (more splits cost partial-sum traffic), each split at least 256
// of H and a whole number of 64-wide k-steps.
int32_t route_gemm_splits(int32_t T, int32_t E, int32_t H) {
  if (T < 1 || E < 1 || H < 16) return 1;
  const int64_t tiles = static_cast<int64_t>((T + kRgTok - 1) / kRgTok) * ((E + kRgExp - 1) / kRgExp);
  int64_t ks = (256 + tiles - 1) / tiles;
  const int64_t kmax = H / 256 > 1 ? H / 256 : 1;
  if (ks > kmax) ks = kmax;
  return static_cast<int32_t>(ks < 1 ? 1 : ks);
}

hipError_t launch_route_topk_gemm(const uint16_t* x, void* const* x_parts, int32_t x_part_rows,
                                  const uint16_t* w_router, int32_t T, int32_t H, int32_t E,
                                  int32_t k, float* partial, int32_t* idx, float* gate,
                                  const RouteCount& rc, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int32_t ks = route_gemm_splits(T, E, H);
  const int32_t kchunk = ((H + ks - 1) / ks + kRgK - 1) / kRgK * kRgK;
  dim3 grid((T + kRgTok - 1) / kRgTok, (E + kRgExp - 1) / kRgExp, ks);
  hipLaunchKernelGGL(k_router_partial, grid, dim3(4 * kWave), 0, s, x, x_parts, x_part_rows,
                     w_router, T, H, E, kchunk, partial);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (E <= 64) return launch_sum_vpl<1>(partial, ks, T, E, k, idx, gate, rc, s);
  if (E <= 128) return launch_sum_vpl<2>(partial, ks, T, E, k, idx, gate, rc, s);
  if (E <= 256) return launch_sum_vpl<4>(partial, ks, T, E, k, idx, gate, rc, s);
  if (E <= 512) return launch_sum_vpl<8>(partial, ks, T, E, k, idx, gate, rc, s);
  if (E <= 1024) return launch_sum_vpl<16>(partial, ks, T, E, k, idx, gate, rc, s);
  if (E <= 2048) return launch_sum_vpl<32>(partial, ks, T, E, k, idx, gate, rc, s);
  return launch_sum_vpl<64>(partial, ks, T, E, k, idx, gate, rc, s);
}

hipError_t launch_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                             int32_t* idx, float* gate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E <= 64) return launch_vpl<1>(logits, T, E, k, idx, gate, s);
  if (E <= 128) return launch_vpl<2>(logits, T, E, k, idx, gate, s);
  if (E <= 256) return launch_vpl<4>(logits, T, E, k, idx, gate, s);
  if (E <= 512) return launch_vpl<8>(logits, T, E, k, idx, gate, s);
  if (E <= 1024) return launch_vpl<16>(logits, T, E, k, idx, gate, s);
  if (E <= 2048) return launch_vpl<32>(logits, T, E, k, idx, gate, s);
  return launch_vpl<64>(logits, T, E, k, idx, gate, s);
}

hipError_t launch_route_count(const float* logits, int32_t T, int32_t E, int32_t k,
                              int32_t base, int32_t n_local, int32_t* idx, float* gate,
                              int32_t* blk_counts, int32_t nblk, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E <= 64) return launch_count_vpl<1>(logits, T, E, k, base, n_local, idx, gate, blk_counts, nblk, s);
  if (E <= 128) return launch_count_vpl<2>(logits, T, E, k, base, n_local, idx, gate, blk_counts, nblk, s);
  if (E <= 256) return launch_count_vpl<4>(logits, T, E, k, base, n_local, idx, gate, blk_counts, nblk, s);
  if (E <= 512) return launch_count_vpl<8>(logits, T, E, k, base, n_local, idx, gate, blk_counts, nblk, s);
  if (E <= 1024) return launch_count_vpl<16>(logits, T, E, k, base, n_local, idx, gate, blk_counts, nblk, s);
  if (E <= 2048) return launch_count_vpl<32>(logits, T, E, k, base, n_local, idx, gate, blk_counts, nblk, s);
  return launch_count_vpl<64>(logits, T, E, k, base, n_local, idx, gate, blk_counts, nblk, s);
}

}  // namespace mok
