// movers_dev.h -- wave-level row movement of the layer (device code shared by
// the standalone dispatch/combine kernels and the persistent pipeline).
//
// tahou.com MoK article: the receiver pulls each token by (source, offset)
// and lays it out per expert itself (pull-dispatch paragraph); the results
// go straight back to their token (push-combine paragraph); the measured
// layer ends with the weighted merge (benchmark-scope paragraph); MXFP8 is
// fused into dispatch (state-machine paragraph).  With the sources being
// HBM partitions of this GPU, the pull is a gather of whole rows.
//
// One wave per row.  Lane l moves the 16-byte pieces l, l+64, ... of the row,
// so every wave instruction touches 1 KiB of contiguous memory; loads of a row
// are issued in batches before any store to keep many requests in flight.
#pragma once

#include "mok_internal.h"

namespace mok {
namespace movers {

constexpr int kBatch = 8;          // 16-byte pieces in flight per lane (gather)
constexpr int kCombPieces = 4;     // 16-byte pieces per lane per batch (several local slots:
                                   // fp32 accumulators; kept small for occupancy)
constexpr int kMergeFast = 8;      // 16-byte pieces per lane per batch (single local slot)

__device__ __forceinline__ const uint4* token_row(void* const* parts, int32_t n_part,
                                                  int32_t part_rows, int64_t t, int32_t H) {
  int64_t p = t / part_rows, r = t % part_rows;
  if (t < 0 || p >= n_part) return nullptr;
  return reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(parts[p]) + r * H);
}

// Pull the row of token t into ring row dst_row: bf16 bit copy.
__device__ __forceinline__ void gather_row_bf16(void* const* __restrict__ parts, int32_t n_part,
                                                int32_t part_rows, int32_t H, int64_t t,
                                                uint16_t* __restrict__ ring, int64_t dst_row,
                                                int32_t* status) {
  const int lane = lane_id();
  const uint4* src = token_row(parts, n_part, part_rows, t, H);
  if (!src) { if (lane == 0) set_status(status, MOK_ERR_CAPACITY); return; }
  uint4* dst = reinterpret_cast<uint4*>(ring + dst_row * static_cast<int64_t>(H));
  const int nvec = H / 8;
  for (int v0 = lane; v0 < nvec; v0 += kWave * kBatch) {
    uint4 buf[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      int v = v0 + u * kWave;
      if (v < nvec) buf[u] = src[v];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      int v = v0 + u * kWave;
      if (v < nvec) st_nt(dst + v, buf[u]);
    }
  }
}

// Pull of rows s = first, first + step, ... < end, two rows per wave at a
// time: both rows' indices are read first, then kBatch 16-byte pieces of each
// row are loaded before any is stored, so a wave keeps 2 x kBatch pieces per
// lane in flight.  Destination row of slot s: (dst_base + s) % ring_slots.
__device__ __forceinline__ void gather_rows_bf16_x2(void* const* __restrict__ parts,
                                                    int32_t n_part, int32_t part_rows, int32_t H,
                                                    int32_t k, const int32_t* __restrict__ aos,
                                                    int64_t first, int64_t step, int64_t end,
                                                    uint16_t* __restrict__ ring, int64_t dst_base,
                                                    int32_t ring_slots, int32_t* status) {
  const int lane = lane_id();
  const int nvec = H / 8;
  for (int64_t s = first; s < end; s += 2 * step) {
    const int64_t s2 = s + step < end ? s + step : s;   // odd tail: copy row s twice
    const uint4* src1 = token_row(parts, n_part, part_rows, aos[s] / k, H);
    const uint4* src2 = token_row(parts, n_part, part_rows, aos[s2] / k, H);
    if (!src1 || !src2) { if (lane == 0) set_status(status, MOK_ERR_CAPACITY); continue; }
    uint4* d1 = reinterpret_cast<uint4*>(ring + ((dst_base + s) % ring_slots) * static_cast<int64_t>(H));
    uint4* d2 = reinterpret_cast<uint4*>(ring + ((dst_base + s2) % ring_slots) * static_cast<int64_t>(H));
    for (int v0 = lane; v0 - lane < nvec; v0 += kWave * kBatch) {
      uint4 b1[kBatch], b2[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int v = v0 + u * kWave;
        if (v < nvec) { b1[u] = src1[v]; b2[u] = src2[v]; }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int v = v0 + u * kWave;
        if (v < nvec) { st_nt(d1 + v, b1[u]); st_nt(d2 + v, b2[u]); }
      }
    }
  }
}

// Same with MXFP8 quantisation on the way: a block of 32 values is 4
// consecutive 16-byte pieces, i.e. 4 consecutive lanes; amax by two
// xor-shuffles.  All 64 lanes must call it (wave-uniform loop).
__device__ __forceinline__ void gather_row_mxfp8(void* const* __restrict__ parts, int32_t n_part,
                                                 int32_t part_rows, int32_t H, int64_t t,
                                                 uint8_t* __restrict__ ring,
                                                 uint8_t* __restrict__ scales, int64_t dst_row,
                                                 int32_t* status) {
  const int lane = lane_id();
  const uint4* src = token_row(parts, n_part, part_rows, t, H);
  if (!src) { if (lane == 0) set_status(status, MOK_ERR_CAPACITY); return; }
  const int64_t rr = dst_row;
  uint2* dst = reinterpret_cast<uint2*>(ring + rr * static_cast<int64_t>(H));
  uint8_t* sdst = scales + rr * static_cast<int64_t>(H / 32);
  const int nvec = H / 8;   // H % 32 == 0, so nvec % 4 == 0: blocks never straddle lane groups
  for (int v0 = lane; v0 - lane < nvec; v0 += kWave * kBatch) {
    uint4 buf[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      int v = v0 + u * kWave;
      if (v < nvec) buf[u] = src[v];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      int v = v0 + u * kWave;
      if (v0 - lane + u * kWave >= nvec) break;      // wave-uniform
      const bool ok = v < nvec;
      float f[8];
      const uint32_t w[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(w[q] << 16);
        f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      }
      float amax = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(f[q]));
      if (!ok) amax = 0.0f;
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      const int E = mx_scale_exp(amax);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo |= e4m3_code_scaled(f[q], E) << (8 * q);
        hi |= e4m3_code_scaled(f[q + 4], E) << (8 * q);
      }
      if (ok) {
        st_nt(dst + v, make_uint2(lo, hi));
        if ((v & 3) == 0) sdst[v >> 2] = static_cast<uint8_t>(E + 127);
      }
    }
  }
}

// Weighted merge of token t.  The k slots and gates are read by lanes 0..k-1
// and broadcast; accumulation per element in fp32 fma in ascending j from 0.
// A column chunk of 64 lanes x 16 pieces x 8 values (8192 values) is held in
// registers across the k rows.  All 64 lanes must call it.
// kFast: single-local-slot fast path and small accumulator batches (the
// standalone merge: high occupancy).  The persistent kernel's movers use the
// plain path with large batches: faster movers there steal the HBM / L2
// bandwidth of the GEMM workers running beside them (measured: slower layer).
template <bool kFast = true>
__device__ __forceinline__ void combine_token(const uint16_t* __restrict__ y, int32_t y_rows,
                                              const int32_t* __restrict__ soa,
                                              const float* __restrict__ gate, int64_t t, int32_t k,
                                              int32_t H, void* const* __restrict__ out_parts,
                                              int32_t n_part, int32_t part_rows, int32_t* status) {
  const int lane = lane_id();
  int32_t my_s = -1;
  float my_g = 0.0f;
  if (lane < k) {
    my_s = soa[t * k + lane];
    my_g = gate[t * k + lane];
    if (my_s >= y_rows) { set_status(status, MOK_ERR_CAPACITY); my_s = -1; }
  }
  const uint64_t live = __ballot(my_s >= 0);
  if (live == 0) return;
  const int64_t p = t / part_rows, r = t % part_rows;
  if (p >= n_part) { if (lane == 0) set_status(status, MOK_ERR_CAPACITY); return; }
  uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out_parts[p]) + r * H);
  const int nvec = H / 8;
  if (kFast && __popcll(live) == 1) {
    // one local slot (most tokens): out = bf16(fma(g, y, 0)), as the general
    // sum gives for a single term, with no accumulators held
    const int j = __ffsll(static_cast<long long>(live)) - 1;
    const int32_t s = __shfl(my_s, j);
    const float g = __shfl(my_g, j);
    const uint4* src = reinterpret_cast<const uint4*>(y + static_cast<int64_t>(s) * H);
    for (int c0 = 0; c0 < nvec; c0 += kWave * kMergeFast) {
      uint4 buf[kMergeFast];
#pragma unroll
      for (int u = 0; u < kMergeFast; ++u) {
        const int v = c0 + lane + u * kWave;
        if (v < nvec) buf[u] = src[v];
      }
#pragma unroll
      for (int u = 0; u < kMergeFast; ++u) {
        const int v = c0 + lane + u * kWave;
        if (v < nvec) {
          const uint32_t w[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
          uint32_t o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = pack_bf16x2(fmaf(g, __uint_as_float(w[q] << 16), 0.0f),
                               fmaf(g, __uint_as_float(w[q] & 0xffff0000u), 0.0f));
          st_nt(dst + v, make_uint4(o[0], o[1], o[2], o[3]));
        }
      }
    }
    return;
  }
  constexpr int kPieces = kFast ? kCombPieces : 16;
  for (int c0 = 0; c0 < nvec; c0 += kWave * kPieces) {
    float acc[kPieces][8];
#pragma unroll
    for (int u = 0; u < kPieces; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
    for (int j = 0; j < k; ++j) {
      if (!((live >> j) & 1ull)) continue;
      const int32_t s = __shfl(my_s, j);
      const float g = __shfl(my_g, j);
      const uint4* src = reinterpret_cast<const uint4*>(y + static_cast<int64_t>(s) * H);
      uint4 buf[kPieces];
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        int v = c0 + lane + u * kWave;
        if (v < nvec) buf[u] = src[v];
      }
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        const uint32_t w[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[u][2 * q] = fmaf(g, __uint_as_float(w[q] << 16), acc[u][2 * q]);
          acc[u][2 * q + 1] = fmaf(g, __uint_as_float(w[q] & 0xffff0000u), acc[u][2 * q + 1]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      int v = c0 + lane + u * kWave;
      if (v < nvec) {
        uint4 o;
        o.x = pack_bf16x2(acc[u][0], acc[u][1]);
        o.y = pack_bf16x2(acc[u][2], acc[u][3]);
        o.z = pack_bf16x2(acc[u][4], acc[u][5]);
        o.w = pack_bf16x2(acc[u][6], acc[u][7]);
        st_nt(dst + v, o);
      }
    }
  }
}

// Slot-driven merge: slot s (s < R) merges its token t = assign_of_slot[s] / k
// when s is t's smallest local slot, so every token with a local assignment is
// merged exactly once while only the R routed slots (not all pool tokens) are
// visited.  All 64 lanes must call it.
// a_s = assign_of_slot[s] (the caller loads it early).
template <bool kFast = true>
__device__ __forceinline__ void merge_slot(const uint16_t* __restrict__ y, int32_t y_rows,
                                           int32_t a_s, const int32_t* __restrict__ soa,
                                           const float* __restrict__ gate, int64_t s, int32_t k,
                                           int32_t H, void* const* __restrict__ out_parts,
                                           int32_t n_part, int32_t part_rows, int32_t* status) {
  const int lane = lane_id();
  const int64_t t = a_s / k;
  int32_t mine = 0x7fffffff;
  if (lane < k) {
    const int32_t v = soa[t * k + lane];
    if (v >= 0) mine = v;
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) mine = min(mine, __shfl_xor(mine, off));
  if (mine != s) return;
  combine_token<kFast>(y, y_rows, soa, gate, t, k, H, out_parts, n_part, part_rows, status);
}

}  // namespace movers
}  // namespace mok
