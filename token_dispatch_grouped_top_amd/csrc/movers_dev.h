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
// The gather moves two rows per wave, the merge one token per wave; loads are
// issued in batches before any store to keep many requests in flight.
#pragma once

#include "mok_internal.h"

namespace mok {
namespace movers {

constexpr int kCombPieces = 4;     // 16-byte pieces per lane per batch (several local slots:
                                   // fp32 accumulators; kept small for occupancy)
constexpr int kMergeFast = 8;      // 16-byte pieces per lane per batch (single local slot)

__device__ __forceinline__ const uint4* token_row(void* const* parts, int32_t n_part,
                                                  int32_t part_rows, int64_t t, int32_t H) {
  int64_t p = t / part_rows, r = t % part_rows;
  if (t < 0 || p >= n_part) return nullptr;
  return reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(parts[p]) + r * H);
}

// Pull of two ring rows per wave: the rows of tokens t1 and t2 into ring rows
// rr1 and rr2 (t2 < 0: t1 alone).  The ring is column-blocked (block b of
// row r at byte (b * rows + r) * 64), so block b of two consecutive ring rows
// is one 128-byte line.  Lane l of wave instruction u takes piece p = 64 u + l
// of the pair, 16 source bytes (8 bf16): G consecutive lanes fill one 64-byte
// destination block and the two rows alternate every G lanes, so an
// instruction reads 512 contiguous source bytes of each row and writes
// 64-byte blocks that pair up into whole lines.  A call moves the pieces
// [p_lo, p_hi) of the pair (both multiples of 2 G, or p_hi = 2 H / 8);
// kPairBatch pieces per lane (16 bf16, 8 MXFP8) are loaded before any is
// stored.
template <int G>
__device__ __forceinline__ void pair_piece(int p, int& sel, int& v) {
  sel = (p / G) & 1;                      // which row of the pair
  v = (p / (2 * G)) * G + p % G;          // 16-byte source piece of that row
}

// bf16: a bit copy, G = 4 (a 64-byte block is 4 source pieces).
__device__ __forceinline__ void gather_pair_bf16(void* const* __restrict__ parts, int32_t n_part,
                                                 int32_t part_rows, int32_t H, int64_t t1,
                                                 int64_t t2, uint16_t* __restrict__ ring,
                                                 int64_t rr1, int64_t rr2, int32_t rows,
                                                 int p_lo, int p_hi, int32_t* status) {
  constexpr int kPairBatch = 16;
  const int lane = lane_id();
  const uint4* src1 = token_row(parts, n_part, part_rows, t1, H);
  const uint4* src2 = t2 >= 0 ? token_row(parts, n_part, part_rows, t2, H) : src1;
  if (!src1 || !src2) { if (lane == 0) set_status(status, MOK_ERR_CAPACITY); return; }
  if (t2 < 0) rr2 = rr1;                  // the second half repeats row 1's copy
  uint8_t* ringb = reinterpret_cast<uint8_t*>(ring);
  const int npc = p_hi;
  for (int p0 = p_lo; p0 < npc; p0 += kWave * kPairBatch) {
    uint4 buf[kPairBatch];
#pragma unroll
    for (int u = 0; u < kPairBatch; ++u) {
      const int p = p0 + u * kWave + lane;
      int sel, v;
      pair_piece<4>(p, sel, v);
      if (p < npc) buf[u] = ld_nt((sel ? src2 : src1) + v);
    }
#pragma unroll
    for (int u = 0; u < kPairBatch; ++u) {
      const int p = p0 + u * kWave + lane;
      int sel, v;
      pair_piece<4>(p, sel, v);
      if (p < npc) st_nt(reinterpret_cast<uint4*>(ringb + colblk_byte(sel ? rr2 : rr1, rows, 16 * v)), buf[u]);
    }
  }
}

// MXFP8 quantisation on the way, G = 8 (64 codes are 8 source pieces).  A
// block of 32 values is 4 consecutive pieces, i.e. 4 consecutive lanes of one
// row; its amax by two xor-shuffles.  Lane v % 4 == 0 of a block writes its
// E8M0 scale.  All 64 lanes must call it (wave-uniform loop).
__device__ __forceinline__ void gather_pair_mxfp8(void* const* __restrict__ parts, int32_t n_part,
                                                  int32_t part_rows, int32_t H, int64_t t1,
                                                  int64_t t2, uint8_t* __restrict__ ring,
                                                  uint8_t* __restrict__ scales, int64_t rr1,
                                                  int64_t rr2, int32_t rows, int p_lo, int p_hi,
                                                  int32_t* status) {
  constexpr int kPairBatch = 8;
  const int lane = lane_id();
  const uint4* src1 = token_row(parts, n_part, part_rows, t1, H);
  const uint4* src2 = t2 >= 0 ? token_row(parts, n_part, part_rows, t2, H) : src1;
  if (!src1 || !src2) { if (lane == 0) set_status(status, MOK_ERR_CAPACITY); return; }
  if (t2 < 0) rr2 = rr1;
  const int npc = p_hi;                   // H % 64 == 0: groups of 8 lanes are whole
  for (int p0 = p_lo; p0 < npc; p0 += kWave * kPairBatch) {
    uint4 buf[kPairBatch];
#pragma unroll
    for (int u = 0; u < kPairBatch; ++u) {
      const int p = p0 + u * kWave + lane;
      int sel, v;
      pair_piece<8>(p, sel, v);
      if (p < npc) buf[u] = ld_nt((sel ? src2 : src1) + v);
    }
#pragma unroll
    for (int u = 0; u < kPairBatch; ++u) {
      if (p0 + u * kWave >= npc) break;   // wave-uniform
      const int p = p0 + u * kWave + lane;
      const bool ok = p < npc;
      int sel, v;
      pair_piece<8>(p, sel, v);
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
        const int64_t rr = sel ? rr2 : rr1;
        st_nt(reinterpret_cast<uint2*>(ring + colblk_byte(rr, rows, 8 * v)), make_uint2(lo, hi));
        if ((v & 3) == 0) scales[scale_byte(rr, rows, v >> 2)] = static_cast<uint8_t>(E + 127);
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
    my_g = gate ? gate[t * k + lane] : 1.0f;                // null: unit gates (plain sum)
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

// Backward of the weighted merge for slot s (token t = a_s / k, pick
// j = a_s % k, gate w = gate[a_s]): dy[s] = bf16(w * dout[t]) into the
// column-blocked dy (row s % dy_rows), and dgate[a_s] = sum_h dout[t][h] *
// y[s][h] in fp32 (each lane sums its pieces in order, then a fixed
// butterfly).  All 64 lanes must call it.
__device__ __forceinline__ void unmerge_slot(void* const* __restrict__ dout_parts, int32_t n_part,
                                             int32_t part_rows, const uint16_t* __restrict__ y,
                                             int32_t y_rows, int32_t a_s,
                                             const float* __restrict__ gate, int64_t s, int32_t k,
                                             int32_t H, uint8_t* __restrict__ dy, int32_t dy_rows,
                                             float* __restrict__ dgate, int32_t* status) {
  const int lane = lane_id();
  const uint4* src = token_row(dout_parts, n_part, part_rows, a_s / k, H);
  if (!src || s >= y_rows) { if (lane == 0) set_status(status, MOK_ERR_CAPACITY); return; }
  const float w = gate[a_s];
  const uint4* yrow = reinterpret_cast<const uint4*>(y + s * static_cast<int64_t>(H));
  const int64_t drow = s % dy_rows;
  const int nvec = H / 8;
  float part = 0.0f;
  for (int v0 = 0; v0 < nvec; v0 += kWave * kMergeFast) {
    uint4 bd[kMergeFast], by[kMergeFast];
#pragma unroll
    for (int u = 0; u < kMergeFast; ++u) {
      const int v = v0 + u * kWave + lane;
      if (v < nvec) { bd[u] = src[v]; by[u] = yrow[v]; }
    }
#pragma unroll
    for (int u = 0; u < kMergeFast; ++u) {
      const int v = v0 + u * kWave + lane;
      if (v >= nvec) continue;
      const uint32_t d4[4] = {bd[u].x, bd[u].y, bd[u].z, bd[u].w};
      const uint32_t y4[4] = {by[u].x, by[u].y, by[u].z, by[u].w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float dlo = __uint_as_float(d4[q] << 16), dhi = __uint_as_float(d4[q] & 0xffff0000u);
        part = fmaf(dlo, __uint_as_float(y4[q] << 16), part);
        part = fmaf(dhi, __uint_as_float(y4[q] & 0xffff0000u), part);
        o[q] = pack_bf16x2(w * dlo, w * dhi);
      }
      *reinterpret_cast<uint4*>(dy + colblk_byte(drow, dy_rows, 16 * static_cast<int64_t>(v))) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if (lane == 0) dgate[a_s] = part;
}

// unmerge_slot with MXFP8 dy: the fp32 products w * dout[t] quantised in
// blocks of 32 along H (E4M3 codes column-blocked like the ring, E8M0 scales
// in pairs).  A block is 4 consecutive pieces, i.e. 4 consecutive lanes of
// one instruction: its amax by two xor-shuffles, as in the MXFP8 gather.
// dgate as unmerge_slot (the same fp32 sum order).  All 64 lanes must call it.
__device__ __forceinline__ void unmerge_slot_mx(void* const* __restrict__ dout_parts, int32_t n_part,
                                                int32_t part_rows, const uint16_t* __restrict__ y,
                                                int32_t y_rows, int32_t a_s,
                                                const float* __restrict__ gate, int64_t s, int32_t k,
                                                int32_t H, uint8_t* __restrict__ dy,
                                                uint8_t* __restrict__ dy_scales, int32_t dy_rows,
                                                float* __restrict__ dgate, int32_t* status) {
  const int lane = lane_id();
  const uint4* src = token_row(dout_parts, n_part, part_rows, a_s / k, H);
  if (!src || s >= y_rows) { if (lane == 0) set_status(status, MOK_ERR_CAPACITY); return; }
  const float w = gate[a_s];
  const uint4* yrow = reinterpret_cast<const uint4*>(y + s * static_cast<int64_t>(H));
  const int64_t drow = s % dy_rows;
  const int nvec = H / 8;                 // H % 64 == 0: groups of 4 lanes are whole
  float part = 0.0f;
  for (int v0 = 0; v0 < nvec; v0 += kWave * kMergeFast) {
    uint4 bd[kMergeFast], by[kMergeFast];
#pragma unroll
    for (int u = 0; u < kMergeFast; ++u) {
      const int v = v0 + u * kWave + lane;
      if (v < nvec) { bd[u] = src[v]; by[u] = yrow[v]; }
    }
#pragma unroll
    for (int u = 0; u < kMergeFast; ++u) {
      if (v0 + u * kWave >= nvec) break;  // wave-uniform
      const int v = v0 + u * kWave + lane;
      const bool ok = v < nvec;
      const uint32_t d4[4] = {ok ? bd[u].x : 0u, ok ? bd[u].y : 0u, ok ? bd[u].z : 0u, ok ? bd[u].w : 0u};
      const uint32_t y4[4] = {ok ? by[u].x : 0u, ok ? by[u].y : 0u, ok ? by[u].z : 0u, ok ? by[u].w : 0u};
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float dlo = __uint_as_float(d4[q] << 16), dhi = __uint_as_float(d4[q] & 0xffff0000u);
        part = fmaf(dlo, __uint_as_float(y4[q] << 16), part);
        part = fmaf(dhi, __uint_as_float(y4[q] & 0xffff0000u), part);
        f[2 * q] = w * dlo;
        f[2 * q + 1] = w * dhi;
      }
      float amax = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(f[q]));
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
        *reinterpret_cast<uint2*>(dy + colblk_byte(drow, dy_rows, 8 * static_cast<int64_t>(v))) =
            make_uint2(lo, hi);
        if ((v & 3) == 0) dy_scales[scale_byte(drow, dy_rows, v >> 2)] = static_cast<uint8_t>(E + 127);
      }
    }
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if (lane == 0) dgate[a_s] = part;
}

// Slot-driven merge: slot s (s < R) merges its token t = assign_of_slot[s] / k
// when s is t's smallest local slot, so every token with a local assignment is
// merged exactly once while only the R routed slots (not all pool tokens) are
// visited.  All 64 lanes must call it.
// a_s = assign_of_slot[s] (the caller loads it early).  multi_only: tokens
// with a single local slot are skipped (the down GEMM's merging epilogue has
// written them); an index outside the partitions still raises the status.
template <bool kFast = true>
__device__ __forceinline__ void merge_slot(const uint16_t* __restrict__ y, int32_t y_rows,
                                           int32_t a_s, const int32_t* __restrict__ soa,
                                           const float* __restrict__ gate, int64_t s, int32_t k,
                                           int32_t H, void* const* __restrict__ out_parts,
                                           int32_t n_part, int32_t part_rows, int32_t* status,
                                           bool multi_only = false) {
  const int lane = lane_id();
  const int64_t t = a_s / k;
  int32_t mine = 0x7fffffff;
  bool local = false;
  if (lane < k) {
    const int32_t v = soa[t * k + lane];
    if (v >= 0) { mine = v; local = true; }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) mine = min(mine, __shfl_xor(mine, off));
  if (mine != s) return;
  if (multi_only && __popcll(__ballot(local)) == 1) {
    if (lane == 0 && t / part_rows >= n_part) set_status(status, MOK_ERR_CAPACITY);
    return;
  }
  combine_token<kFast>(y, y_rows, soa, gate, t, k, H, out_parts, n_part, part_rows, status);
}

}  // namespace movers
}  // namespace mok
