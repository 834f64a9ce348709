// gemm_tile_mx8.h -- the grouped GEMM tile with both operands in MXFP8: E4M3
// codes with one E8M0 scale per 32 along K for the tokens (ring / act rows)
// and for the weights (packed by launch_pack_weights_mx8), multiplied by
// gfx950's block-scaled v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Operand layout of that MFMA (checked on the GPU against E4M3 x E4M3 with
// random codes and scales): lane l feeds row l % 32 with 32 bytes; bytes 0..15
// belong to k-block 0 and bytes 16..31 to k-block 1 of the 64-wide k-step,
// and the lane's scale operand is the E8M0 of block l / 32.  Lane half h =
// l / 32 therefore takes chunk h (codes 16h..16h+15 of block 0) and chunk
// 2 + h (the same of block 1) of a 64-byte row, for both operands alike; the
// products are summed over all 64 k, so which 16 codes of a block a lane
// brings does not matter as long as both operands agree.
//
// Tile, waves, tile order, split and epilogue are those of gemm_tile.h (the
// accumulator layout of the 32x32x64 MFMA equals that of the bf16 32x32x16).
// Per k-step of 64: 16 KiB of token codes, 16 KiB of weight codes and 2
// scale bytes per row of each, 16 MFMAs per wave.
#pragma once

#include "gemm_tile.h"

namespace mok {
namespace gemm {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct GeoMX8 {
  static constexpr int BK = 64, NS = 4;
  static constexpr int ROWB = BK, CPR = ROWB / 16, TILE = BM * ROWB;   // 16 KiB of codes
  static constexpr int SCALEB = BM * 4;                  // 4-byte slot per row, 2 bytes used
  // stage: [token codes][weight codes][token scales][weight scales]
  static constexpr int STAGEB = 2 * TILE + 2 * SCALEB;
  static constexpr int NLOAD = TILE / 4096;              // 1-KiB wave loads per operand
  static constexpr int RSTEP = 4 * 1024 / ROWB;          // rows per round of four waves
  static constexpr int LOOP_LDS = NS * STAGEB;
  static constexpr int LDS = LOOP_LDS > kEpiLds ? LOOP_LDS : kEpiLds;
  // packed weights: per (expert, column tile, k-step) the LDS image of the
  // codes, then 2 scale bytes per row
  static constexpr int WBLOCK = TILE + BM * 2;
  static __device__ __forceinline__ int off(int row, int chunk) {
    return row * ROWB + ((chunk ^ chunk_key<CPR>(row)) << 4);
  }
};
static_assert(GeoMX8::LDS <= 160 * 1024, "LDS budget");

// TN = 128: a half-width tail tile (job.half), the y-storing epilogues only.
template <int EPI, int TN = BN>
__device__ __forceinline__ void gemm_tile_mx8(const GemmParams& p, const TileJob& job,
                                              uint8_t* __restrict__ lds) {
  using G = GeoMX8;
  constexpr int BK = G::BK, NS = G::NS;
  static_assert(TN == BN || (TN == BN / 2 && (EPI == EPI_STORE_BF16 || EPI == EPI_DOWN_MERGE)),
                "half-width tiles store y only");
  constexpr int NB = TN / 64;                   // 32-column fragments per wave
  constexpr int NLB = G::NLOAD * TN / BN;       // weight code loads per stage and thread
  // first weight row of a half-width tile within its column tile
  const int hrow = TN == BN ? 0 : (job.half - 1) * TN;
  __syncthreads();
  const int e = job.e, row0 = job.row0, nrows = job.nrows, ntile = job.ntile;
  const int tid = threadIdx.x, lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;
  const int K = p.K;
  const int nk_all = K / BK;
  const int kt0 = job.kt0;
  const int nk = job.nkt > 0 ? job.nkt : nk_all;

  // weights: the tile's blocks from k-step kt0 on; load j of a wave reads the
  // contiguous KiB (4 j + wave) of a block, the scales 2 bytes per thread (a
  // half-width tile: the half's rows, one contiguous half of the codes; its
  // threads 128..255 load the half's scales again, into slots nobody reads)
  const uint8_t* Wq = reinterpret_cast<const uint8_t*>(p.W) +
                      ((static_cast<int64_t>(e) * p.n_tiles + ntile) * nk_all + kt0) * G::WBLOCK;
  uint32_t boff[G::NLOAD];
#pragma unroll
  for (int j = 0; j < NLB; ++j) boff[j] = (4 * j + wave) * 1024 + lane * 16 + hrow * G::ROWB;
  const uint32_t wsoff = G::TILE + 2 * (hrow + (TN == BN ? tid : (tid & (TN - 1))));
  // tokens: ring rows, tail rows clamped to the last valid one; lane l of load
  // j lands at physical chunk l % 4 of row tid / 4 + RSTEP j.  The ring is
  // column-blocked: a k-step is one 64-byte block per row, a_kstep bytes
  // apart, and scale pairs a_rows * 2 bytes apart.
  const ARows a_ring_row(p, row0, nrows);
  const uint32_t a_kstep = static_cast<uint32_t>(p.a_rows) * kColBlock;
  const int lrow = tid / G::CPR;
  const int lchunk = (lane % G::CPR) ^ chunk_key<G::CPR>(lrow);
  uint32_t aoff[G::NLOAD];
#pragma unroll
  for (int j = 0; j < G::NLOAD; ++j)
    aoff[j] = a_ring_row(lrow + G::RSTEP * j) * kColBlock + lchunk * 16 + static_cast<uint32_t>(kt0) * a_kstep;
  const uint32_t soff = a_ring_row(tid) * 2u + static_cast<uint32_t>(kt0) * p.a_rows * 2u;
  auto extent = [](int64_t bytes) -> int32_t {
    return static_cast<int32_t>(bytes < 0xffffffffll ? bytes : 0xffffffffll);
  };
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wq), 0, extent(static_cast<int64_t>(nk_all - kt0) * G::WBLOCK), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.A), 0, extent(static_cast<int64_t>(p.a_rows) * K), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.A_scales), 0, extent(static_cast<int64_t>(p.a_rows) * (K / 32)), kRsrcWord3);

  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  auto tileA = [&](int buf) { return lds + buf * G::STAGEB; };
  auto tileB = [&](int buf) { return lds + buf * G::STAGEB + G::TILE; };
  auto tileSA = [&](int buf) { return lds + buf * G::STAGEB + 2 * G::TILE; };
  auto tileSB = [&](int buf) { return lds + buf * G::STAGEB + 2 * G::TILE + G::SCALEB; };

  f32x16_t acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int frag_row = lane & 31;
  const int khalf = lane >> 5;

  // A stage's loads in two halves (as in gemm_tile.h): weights (codes +
  // scales) and tokens (codes + scales); the 2-byte scale loads land in
  // 4-byte slots, lane i at slot base + 4 i, i.e. row tid at 4 tid.
// Weights with the non-temporal policy (aux bit 1), as the bf16 tile's.
#define MX8_ISSUE_W(kt, buf)                                                                 \
  do {                                                                                       \
    uint8_t* Bs_ = tileB(buf);                                                               \
    _Pragma("unroll") for (int j = 0; j < NLB; ++j)                                          \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_ptr_t)(Bs_ + (4 * j + wave) * 1024), 16, \
                                               boff[j], static_cast<uint32_t>(kt) * G::WBLOCK, 0, 2); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_ptr_t)(tileSB(buf) + wave * 256), 2,   \
                                             wsoff, static_cast<uint32_t>(kt) * G::WBLOCK, 0, 2); \
  } while (0)
#define MX8_ISSUE_A(kt, buf)                                                                 \
  do {                                                                                       \
    uint8_t* As_ = tileA(buf);                                                               \
    _Pragma("unroll") for (int j = 0; j < G::NLOAD; ++j)                                     \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(As_ + (4 * j + wave) * 1024), 16, \
                                               aoff[j], static_cast<uint32_t>(kt) * a_kstep, 0, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_ptr_t)(tileSA(buf) + wave * 256), 2,   \
                                             soff, static_cast<uint32_t>(kt) * p.a_rows * 2u, 0, 0); \
  } while (0)

  // Fragments of one k-step into register set `set`: rows of the wave's token
  // and weight blocks, chunks khalf and 2 + khalf, and the block scale khalf.
  // Row 128 w + 32 i + frag_row of a block has the swizzle key of frag_row
  // (the key is bits 2..3 of the row), so a fragment sits at a wave-uniform
  // base + 2048 i + a per-lane offset: one address per chunk serves all four
  // row groups, i goes into the instruction's offset field, and the loop
  // needs no address arithmetic per read.
  i32x8_t tf[2][4], wf[2][NB];
  int ts[2][4], wsc[2][NB];
  const int key = chunk_key<G::CPR>(frag_row);
  const int lane_lo = frag_row * G::ROWB + ((khalf ^ key) << 4);
  const int lane_hi = frag_row * G::ROWB + (((2 + khalf) ^ key) << 4);
  const int lane_sc = 4 * frag_row + khalf;
  auto frag = [&](const uint8_t* lo_p, const uint8_t* hi_p, int i) -> i32x8_t {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(lo_p + 32 * G::ROWB * i);  // vector-typed:
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(hi_p + 32 * G::ROWB * i);  // see lds_read16
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
#define MX8_FRAGS(set, buf)                                                                  \
  do {                                                                                       \
    const uint8_t* At_ = tileA(buf) + 128 * G::ROWB * wm;                                    \
    const uint8_t* Bt_ = tileB(buf) + (TN / 2) * G::ROWB * wn;                               \
    const uint8_t* Sa_ = tileSA(buf) + 512 * wm + lane_sc;                                   \
    const uint8_t* Sb_ = tileSB(buf) + (TN / 2) * 4 * wn + lane_sc;                          \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                       \
      if (i_ < NB) wf[set][i_ < NB ? i_ : 0] = frag(Bt_ + lane_lo, Bt_ + lane_hi, i_);        \
      tf[set][i_] = frag(At_ + lane_lo, At_ + lane_hi, i_);                                  \
      if (i_ < NB) wsc[set][i_ < NB ? i_ : 0] = Sb_[128 * i_];                               \
      ts[set][i_] = Sa_[128 * i_];                                                           \
    }                                                                                        \
  } while (0)
  // The MFMAs of token row groups mi0, mi0 + 1 (fed weights, tokens, as in
  // gemm_tile.h; both formats E4M3 = 0).
#define MX8_MMA(set, mi0)                                                                    \
  do {                                                                                       \
    _Pragma("unroll") for (int mi = (mi0); mi < (mi0) + 2; ++mi)                              \
      _Pragma("unroll") for (int ni = 0; ni < NB; ++ni)                                      \
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                       \
            wf[set][ni], tf[set][mi], acc[mi][ni], 0, 0, 0, wsc[set][ni], 0, ts[set][mi]);   \
  } while (0)

  // Pipeline as in gemm_tile.h, with one MFMA k-slice per k-step: phase A runs
  // the MFMAs of row groups 0, 1 and issues the token half of stage kt-1+NS;
  // after the barrier (stage kt+1 landed, buffer kt % NS free) phase B reads
  // all fragments of step kt+1 into the other register set, issues the weight
  // half of stage kt+NS and runs the MFMAs of row groups 2, 3.  The loop is
  // unrolled by two so the register sets alternate at compile time.
  constexpr int LW = NLB + 1, LA = G::NLOAD + 1, LPS = LW + LA;
  // scheduling groups: phase A's MFMAs paired with the token loads, phase B's
  // with the fragment reads (3 per row group: two code chunks and a scale)
  constexpr int kMP = 2 * NB;                                // MFMAs per phase
  constexpr int kVA = LA < kMP ? LA : kMP;
  constexpr int kRB = 3 * (4 + NB), kRPer = kRB / kMP;
  MergeRow mr;                                               // EPI_DOWN_MERGE, as gemm_tile
  if constexpr (EPI == EPI_DOWN_MERGE) merge_row_load(p, job.row0, job.nrows, mr);
#pragma unroll
  for (int s0 = 0; s0 < NS; ++s0) {
    const int ks0 = s0 < nk ? s0 : nk - 1;
    MX8_ISSUE_W(ks0, s0);
    if (s0 + 1 < NS) MX8_ISSUE_A(ks0, s0);
  }
  wait_vm<(NS - 2) * LPS + LW>();                            // stage 0 landed
  __syncthreads();
  MX8_FRAGS(0, 0);
  int buf = 0, kt = 0;
#define MX8_STEP(cur, nxt)                                                                   \
  do {                                                                                       \
    const int nbuf_ = buf + 1 == NS ? 0 : buf + 1;                                           \
    MX8_MMA(cur, 0);                                                                         \
    {                                                                                        \
      const int kp_ = kt - 1 + NS < nk ? kt - 1 + NS : nk - 1;                               \
      MX8_ISSUE_A(kp_, buf == 0 ? NS - 1 : buf - 1);                                         \
    }                                                                                        \
    _Pragma("unroll") for (int i_ = 0; i_ < kVA; ++i_) {                                     \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                     \
    }                                                                                        \
    if (kMP - kVA > 0) __builtin_amdgcn_sched_group_barrier(0x008, kMP - kVA, 0);            \
    if (LA - kVA > 0) __builtin_amdgcn_sched_group_barrier(0x020, LA - kVA, 0);              \
    __builtin_amdgcn_sched_barrier(0);                                                       \
    wait_vm<(NS - 2) * LPS>();                                                               \
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                          \
    __builtin_amdgcn_sched_barrier(0);                                                       \
    const int kn_ = kt + NS < nk ? kt + NS : nk - 1;                                         \
    MX8_FRAGS(nxt, nbuf_);                                                                   \
    MX8_ISSUE_W(kn_, buf);                                                                   \
    MX8_MMA(cur, 2);                                                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < kMP; ++i_) {                                     \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
      __builtin_amdgcn_sched_group_barrier(0x100, kRPer, 0);                                 \
    }                                                                                        \
    if (kRB - kRPer * kMP > 0) __builtin_amdgcn_sched_group_barrier(0x100, kRB - kRPer * kMP, 0); \
    __builtin_amdgcn_sched_group_barrier(0x020, LW, 0);                                      \
    __builtin_amdgcn_sched_barrier(0);                                                       \
    buf = nbuf_;                                                                             \
    ++kt;                                                                                    \
  } while (0)
  const int pairs = (nk - 1) / 2;
  for (int i = 0; i < pairs; ++i) {
    MX8_STEP(0, 1);
    MX8_STEP(1, 0);
  }
  if ((nk - 1) & 1) {                                        // odd: one more step, set 1 -> 0
    MX8_STEP(0, 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) { tf[0][i] = tf[1][i]; ts[0][i] = ts[1][i]; }
#pragma unroll
    for (int i = 0; i < NB; ++i) { wf[0][i] = wf[1][i]; wsc[0][i] = wsc[1][i]; }
  }
  MX8_MMA(0, 0);                                             // last k-step
  MX8_MMA(0, 2);
#undef MX8_STEP
#undef MX8_MMA
#undef MX8_FRAGS
#undef MX8_ISSUE_A
#undef MX8_ISSUE_W
  wait_vm<0>();                                              // clamped tail loads still land in LDS
  __syncthreads();
  if constexpr (TN == BN) {
    tile_finish<EPI>(p, job, acc, lds, mr);
  } else {
    tile_finish_half<EPI>(p, job, acc, lds, mr);
  }
}

// A whole tile (all k-steps).
template <int EPI>
__device__ __forceinline__ void gemm_tile_mx8(const GemmParams& p, int e, int row0, int nrows,
                                              int ntile, uint8_t* __restrict__ lds) {
  TileJob j;
  j.e = e; j.row0 = row0; j.nrows = nrows; j.ntile = ntile;
  j.kt0 = 0; j.nkt = 0; j.role = kWhole; j.slot = 0; j.slot0 = 0; j.npieces = 0; j.cnt = nullptr;
  j.half = 0;
  gemm_tile_mx8<EPI>(p, j, lds);
}

}  // namespace gemm
}  // namespace mok
