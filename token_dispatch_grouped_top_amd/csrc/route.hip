// route.hip -- top-k routing with softmax gates over the picks.
//
// tahou.com MoK article, routing paragraph: the router assigns each token to
// experts.  Reading used (the pages fix no details): the k largest logits,
// equal logits resolved to the lower expert id, picks in descending order,
// gates = softmax over the k picked logits.
//
// One wave per token.  Lane l holds logits l, l+64, l+128, ... in registers;
// each of the k rounds is a lane-local argmax followed by a 6-step butterfly
// over the wave with the (value desc, id asc) order, so the result does not
// depend on the reduction order.  Gates: lanes 0..k-1 hold the picked
// logits; e_j = exp(l_j - l_0) in fp32, summed by a butterfly, divided.
#include "mok_internal.h"

namespace mok {

namespace {

constexpr int kRouteWaves = 4;

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
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
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      float ov = __shfl_xor(bv, off);
      int oe = __shfl_xor(be, off);
      if (better(ov, oe, bv, be)) { bv = ov; be = oe; }
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
}

template <int VPL>
hipError_t launch_vpl(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* idx,
                      float* gate, hipStream_t s) {
  dim3 grid((T + kRouteWaves - 1) / kRouteWaves);
  hipLaunchKernelGGL(k_route_topk<VPL>, grid, dim3(kRouteWaves * kWave), 0, s, logits, T, E, k,
                     idx, gate);
  return hipGetLastError();
}

}  // namespace

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

}  // namespace mok
