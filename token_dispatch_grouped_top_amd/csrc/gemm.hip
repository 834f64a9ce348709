// gemm.hip -- the expert SwiGLU FFN as two grouped bf16 MFMA GEMMs.
//
// tahou.com MoK article: same-expert tokens are laid out contiguously so a
// grouped GEMM can run over them (layout-planning paragraph); the expert FFN
// is SwiGLU and MXFP8 activation quantisation is fused into the grouped GEMM
// and SwiGLU instead of separate kernels (state-machine paragraph).
//
//   gate/up:  h = x . W_gu[e]^T  (K = H),  a = SiLU(h_gate) * h_up -> act
//   down:     y = a . W_d[e]^T   (K = I)                          -> y
//
// Both operands are K-contiguous (token rows, nn.Linear weight rows), which is
// what v_mfma_f32_32x32x16_bf16 wants: lane l feeds row (l % 32), k-run
// 8*(l / 32) .. +7 of both operands as one 16-byte LDS read.
//
// Tiling (gfx950: 160 KiB LDS, wave64, 4 SIMDs per CU):
//   workgroup tile 256 x 256, 256 threads = 4 waves in 2 x 2, each wave
//   128 x 128 = 4 x 4 MFMA tiles of 32 x 32 (256 fp32 accumulators per lane).
//   Operand tiles stream through an LDS ring of NS k-steps, NS-1 of them in
//   flight while one is consumed:
//     bf16 tokens:  BK = 32, NS = 4 (4 x 32 KiB = 128 KiB);
//     E4M3 tokens:  BK = 64, NS = 3, codes and E8M0 scales loaded into LDS
//                   and converted to bf16 in registers per k-slice;
//     E4M3 tokens and weights: gemm_tile_mx8.h (block-scaled FP8 MFMA).
//   Loads go global -> LDS directly (buffer_load ... lds, a per-lane offset
//   fixed for the tile plus a per-k-step scalar offset): no staging registers,
//   no ds_write.  Weights come packed in the LDS image order, tokens from the
//   column-blocked ring / act, so a k-step of either operand is one contiguous
//   16 KiB block.  Rows keep their 16-byte chunks XOR-swizzled so the fragment
//   reads of 16 consecutive rows hit distinct banks; the swizzle is applied on
//   the global side of the loads.
// Grouped M: the window's rows [s_begin, min(s_end, R)) are cut per expert
// segment (offsets) into 256-row tiles; the grid is sized from the window
// length (never from counts), and blocks past the last tile exit at once.
// Ragged tails load a clamped valid row and mask the stores.
// SwiGLU fusion: a gate/up tile takes 128 gate rows and the 128 up rows of the
// same intermediate columns (64 + 64 per wave column), so each lane holds g and
// u of the same (row, i) in accumulators (mi, ni) and (mi, ni + 2).
// The backward's GEMMs reuse the tile with other epilogues: g and u stored
// (EPI_STORE_GU), the SwiGLU backward (EPI_SWIGLU_BWD).
#include "gemm_tile.h"
#include "gemm_tile_mx8.h"

namespace mok {

namespace {

using namespace gemm;

template <bool A_MX, int EPI>
__global__ __launch_bounds__(kThreads)
void k_ffn_gemm(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kernel_lds<Geo<A_MX>::LDS, EPI>()];
  constexpr bool halves = EPI == EPI_STORE_BF16 || EPI == EPI_DOWN_MERGE;
  TileJob j;
  if (!decode_job(p, p.K / Geo<A_MX>::BK, blockIdx.x, j, halves)) return;
  if constexpr (halves) {
    if (j.half != 0) {
      gemm_tile<A_MX, EPI, BN / 2>(p, j, lds);
      return;
    }
  }
  gemm_tile<A_MX, EPI>(p, j, lds);
}

template <int EPI>
__global__ __launch_bounds__(kThreads)
void k_ffn_gemm_mx8(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kernel_lds<GeoMX8::LDS, EPI>()];
  constexpr bool halves = EPI == EPI_STORE_BF16 || EPI == EPI_DOWN_MERGE;
  TileJob j;
  if (!decode_job(p, p.K / GeoMX8::BK, blockIdx.x, j, halves)) return;
  if constexpr (halves) {
    if (j.half != 0) {
      gemm_tile_mx8<EPI, BN / 2>(p, j, lds);
      return;
    }
  }
  gemm_tile_mx8<EPI>(p, j, lds);
}

// MXFP8 packing: one thread per (expert, column tile, k-step, weight row).  The
// row's 64 weights of the k-step are quantised as two OCP MX blocks of 32
// (the quantiser of the MXFP8 activations) and written where the MXFP8 tile's
// loads land them: codes in the LDS image of the block (chunk swizzle
// included), then the 2 scale bytes of row r at TILE + 2 r.
__global__ __launch_bounds__(256)
void k_pack_weights_mx8(const uint16_t* __restrict__ W, int64_t expert_stride, int32_t K, int32_t I,
                        int32_t N, int32_t swiglu, int32_t n_tiles, int32_t n_local,
                        uint8_t* __restrict__ out) {
  using G = GeoMX8;
  const int nk = K / G::BK;
  const int64_t total = static_cast<int64_t>(n_local) * n_tiles * nk * BM;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < total;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int row = static_cast<int>(u % BM);
    const int64_t blk = u / BM;                            // (e * n_tiles + nt) * nk + kt
    const int kt = static_cast<int>(blk % nk);
    const int64_t et = blk / nk;
    const int nt = static_cast<int>(et % n_tiles), e = static_cast<int>(et / n_tiles);
    const int wrow = w_row_of(row, nt, swiglu != 0, I, N);
    const uint4* src = reinterpret_cast<const uint4*>(W + e * expert_stride + static_cast<int64_t>(wrow) * K +
                                                      kt * G::BK);
    uint8_t* dst = out + blk * G::WBLOCK;
#pragma unroll
    for (int b = 0; b < 2; ++b) {                          // two blocks of 32
      float v[32];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 w = src[4 * b + c];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[8 * c + 2 * q] = __uint_as_float(ws[q] << 16);
          v[8 * c + 2 * q + 1] = __uint_as_float(ws[q] & 0xffff0000u);
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
      const int E = mx_scale_exp(amax);
#pragma unroll
      for (int h = 0; h < 2; ++h) {                        // 16-byte chunks 2 b + h of the row
        uint32_t c4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float* t = v + 16 * h + 4 * q;
          c4[q] = e4m3_code_scaled(t[0], E) | (e4m3_code_scaled(t[1], E) << 8) |
                  (e4m3_code_scaled(t[2], E) << 16) | (e4m3_code_scaled(t[3], E) << 24);
        }
        *reinterpret_cast<uint4*>(dst + G::off(row, 2 * b + h)) = make_uint4(c4[0], c4[1], c4[2], c4[3]);
      }
      dst[G::TILE + 2 * row + b] = static_cast<uint8_t>(E + 127);
    }
  }
}

// MXFP8 packing of a transposed weight (a backward GEMM's B with MXFP8 weights):
// weight row n, k-value k is src[e][k][n] of a source stored [K][N] row-major
// per expert, quantised along k like k_pack_weights_mx8 (two blocks of 32 per
// k-step of 64).  Adjacent threads take adjacent rows n, so each of their 2-byte
// reads is coalesced across the wave.  Rows past N repeat the last one.
__global__ __launch_bounds__(256)
void k_pack_weights_mx8_t(const uint16_t* __restrict__ W, int64_t expert_stride, int32_t K,
                          int32_t N, int32_t n_tiles, int32_t n_local, uint8_t* __restrict__ out) {
  using G = GeoMX8;
  const int nk = K / G::BK;
  const int64_t total = static_cast<int64_t>(n_local) * n_tiles * nk * BM;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < total;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int row = static_cast<int>(u % BM);
    const int64_t blk = u / BM;                            // (e * n_tiles + nt) * nk + kt
    const int kt = static_cast<int>(blk % nk);
    const int64_t et = blk / nk;
    const int nt = static_cast<int>(et % n_tiles), e = static_cast<int>(et / n_tiles);
    const int n = nt * BN + row < N ? nt * BN + row : N - 1;
    const uint16_t* src = W + e * expert_stride + static_cast<int64_t>(kt * G::BK) * N + n;
    uint8_t* dst = out + blk * G::WBLOCK;
#pragma unroll
    for (int b = 0; b < 2; ++b) {                          // two blocks of 32
      float v[32];
#pragma unroll
      for (int q = 0; q < 32; ++q)
        v[q] = __uint_as_float(static_cast<uint32_t>(src[static_cast<int64_t>(32 * b + q) * N]) << 16);
      float amax = 0.0f;
#pragma unroll
      for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
      const int E = mx_scale_exp(amax);
#pragma unroll
      for (int h = 0; h < 2; ++h) {                        // 16-byte chunks 2 b + h of the row
        uint32_t c4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float* t = v + 16 * h + 4 * q;
          c4[q] = e4m3_code_scaled(t[0], E) | (e4m3_code_scaled(t[1], E) << 8) |
                  (e4m3_code_scaled(t[2], E) << 16) | (e4m3_code_scaled(t[3], E) << 24);
        }
        *reinterpret_cast<uint4*>(dst + G::off(row, 2 * b + h)) = make_uint4(c4[0], c4[1], c4[2], c4[3]);
      }
      dst[G::TILE + 2 * row + b] = static_cast<uint8_t>(E + 127);
    }
  }
}

// Packing: one thread per 16-byte piece of the packed weights.  Block
// (e, column tile, k-step) holds the tile's 256 weight rows x BK in the byte
// order the GEMM's direct-to-LDS loads land them (chunk swizzle included).
template <bool A_MX>
__global__ __launch_bounds__(256)
void k_pack_weights(const uint16_t* __restrict__ W, int64_t expert_stride, int32_t K, int32_t I,
                    int32_t N, int32_t swiglu, int32_t n_tiles, int32_t n_local,
                    uint16_t* __restrict__ out) {
  using G = Geo<A_MX>;
  constexpr int BK = G::BK;
  constexpr int64_t kPieces = BM * BK / 8;                 // 16-byte pieces per block
  const int nk = K / BK;
  const int64_t total = static_cast<int64_t>(n_local) * n_tiles * nk * kPieces;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < total;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t blk = u / kPieces;
    const int o = static_cast<int>(u % kPieces) * 16;      // byte offset in the block
    const int kt = static_cast<int>(blk % nk);
    const int64_t et = blk / nk;
    const int nt = static_cast<int>(et % n_tiles), e = static_cast<int>(et / n_tiles);
    const int row = o / G::ROWB_B;
    const int chunk = ((o % G::ROWB_B) >> 4) ^ chunk_key<G::CPR_B>(row);
    const int wrow = w_row_of(row, nt, swiglu != 0, I, N);
    reinterpret_cast<uint4*>(out)[u] = *reinterpret_cast<const uint4*>(
        W + e * expert_stride + static_cast<int64_t>(wrow) * K + kt * BK + chunk * 8);
  }
}

// Packing of a transposed weight (the backward GEMMs' B): the GEMM's weight
// row n, k-value k is src[e][k][n] of a source stored [K][N] row-major per
// expert.  One thread per 16-byte piece, as k_pack_weights; the 8 values of a
// piece are 8 source rows apart by N.  Rows past N repeat the last one.  A_MX:
// the k-step and LDS layout of the GEMMs whose token operand is MXFP8.
template <bool A_MX>
__global__ __launch_bounds__(256)
void k_pack_weights_t(const uint16_t* __restrict__ W, int64_t expert_stride, int32_t K, int32_t N,
                      int32_t n_tiles, int32_t n_local, uint16_t* __restrict__ out) {
  using G = Geo<A_MX>;
  constexpr int BK = G::BK;
  constexpr int64_t kPieces = BM * BK / 8;
  const int nk = K / BK;
  const int64_t total = static_cast<int64_t>(n_local) * n_tiles * nk * kPieces;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < total;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t blk = u / kPieces;
    const int o = static_cast<int>(u % kPieces) * 16;
    const int kt = static_cast<int>(blk % nk);
    const int64_t et = blk / nk;
    const int nt = static_cast<int>(et % n_tiles), e = static_cast<int>(et / n_tiles);
    const int row = o / G::ROWB_B;
    const int chunk = ((o % G::ROWB_B) >> 4) ^ chunk_key<G::CPR_B>(row);
    const int n = nt * BN + row < N ? nt * BN + row : N - 1;
    const uint16_t* src = W + e * expert_stride + static_cast<int64_t>(kt * BK + chunk * 8) * N + n;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = static_cast<uint32_t>(src[(2 * q) * static_cast<int64_t>(N)]) |
             (static_cast<uint32_t>(src[(2 * q + 1) * static_cast<int64_t>(N)]) << 16);
    reinterpret_cast<uint4*>(out)[u] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <bool A_MX>
hipError_t pack_one(const uint16_t* W, int64_t stride, int32_t K, int32_t I, int32_t N, bool swiglu,
                    int32_t n_tiles, int32_t n_local, uint16_t* out, hipStream_t s) {
  const int64_t pieces = static_cast<int64_t>(n_local) * n_tiles * (K / Geo<A_MX>::BK) *
                         (BM * Geo<A_MX>::BK / 8);
  const int64_t blocks = (pieces + 255) / 256;
  hipLaunchKernelGGL(k_pack_weights<A_MX>, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)),
                     dim3(256), 0, s, W, stride, K, I, N, swiglu ? 1 : 0, n_tiles, n_local, out);
  return hipGetLastError();
}

// Grid: an upper bound of the window's tiles (its rows plus one partial tile
// per expert), plus (tail split) n_cus / 32 more workgroups per XCD for the
// pieces of the last round.  Workgroups without work exit at once, but each
// still waits for a CU with the kernel's LDS free, so the spare count is kept
// small: the pieces also use the bound's slack.
template <bool A_MX, int EPI>
hipError_t launch_one(GemmParams gp, int n_tiles, int m_tiles, hipStream_t s) {
  gp.n_tiles = n_tiles;
  int64_t grid = static_cast<int64_t>(n_tiles) * m_tiles;
  if (gp.part) grid = ((grid + kXcds - 1) / kXcds + gp.n_cus / (4 * kXcds)) * kXcds;
  hipLaunchKernelGGL((k_ffn_gemm<A_MX, EPI>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, gp);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_one_mx8(GemmParams gp, int n_tiles, int m_tiles, hipStream_t s) {
  gp.n_tiles = n_tiles;
  int64_t grid = static_cast<int64_t>(n_tiles) * m_tiles;
  if (gp.part) grid = ((grid + kXcds - 1) / kXcds + gp.n_cus / (4 * kXcds)) * kXcds;
  hipLaunchKernelGGL((k_ffn_gemm_mx8<EPI>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, gp);
  return hipGetLastError();
}

hipError_t pack_one_mx8(const uint16_t* W, int64_t stride, int32_t K, int32_t I, int32_t N, bool swiglu,
                        int32_t n_tiles, int32_t n_local, uint8_t* out, hipStream_t s) {
  const int64_t threads = static_cast<int64_t>(n_local) * n_tiles * (K / GeoMX8::BK) * BM;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(k_pack_weights_mx8, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)),
                     dim3(256), 0, s, W, stride, K, I, N, swiglu ? 1 : 0, n_tiles, n_local, out);
  return hipGetLastError();
}

// The device's CUs (the half-width tail) and, with a workspace, the K split.
void set_split(GemmParams& g, const FfnArgs& a) {
  g.n_cus = a.split.n_cus;
  if (!a.split.part || a.split.n_cus < kXcds) return;
  g.part = a.split.part; g.part_cnt = a.split.cnt;
}

}  // namespace

size_t split_ws_bytes(int32_t n_cus) {
  return ((static_cast<size_t>(n_cus) * 4 + 255) / 256) * 256 +
         static_cast<size_t>(n_cus) * BM * BN * sizeof(float);
}

SplitWs split_ws_carve(void* ws, int32_t n_cus) {
  SplitWs w{};
  uint8_t* b = static_cast<uint8_t*>(ws);
  w.cnt = reinterpret_cast<int32_t*>(b);
  w.part = reinterpret_cast<float*>(b + ((static_cast<size_t>(n_cus) * 4 + 255) / 256) * 256);
  w.n_cus = n_cus;
  return w;
}

hipError_t launch_gate_up(const FfnArgs& a, hipStream_t s) {
  const int64_t span = static_cast<int64_t>(a.s_end) - a.s_begin;
  if (span <= 0) return hipSuccess;
  const int m_tiles = static_cast<int>((span + BM - 1) / BM) + a.n_local;
  GemmParams g{};
  g.offsets = a.offsets; g.n_local = a.n_local; g.s_begin = a.s_begin; g.s_end = a.s_end;
  g.A = a.ring; g.A_scales = a.ring_scales; g.a_rows = a.ring_slots;
  g.W = a.w_gu; g.w_expert_stride = static_cast<int64_t>(2) * a.I * a.H; g.K = a.H;
  g.N = a.I; g.I = a.I;
  g.C = a.act; g.C_scales = a.act_scales; g.c_rows = a.act_rows;
  g.w_packed = a.w_packed;
  set_split(g, a);
  const int n1 = (a.I + BN / 2 - 1) / (BN / 2);
  if (a.h_out) g.H_out = static_cast<uint16_t*>(a.h_out);
  if (a.weight_format == MOK_W_MXFP8_E4M3)
    return a.h_out ? launch_one_mx8<EPI_SWIGLU_MX_H>(g, n1, m_tiles, s)
                   : launch_one_mx8<EPI_SWIGLU_MX>(g, n1, m_tiles, s);
  if (a.h_out) {                   // the gate/up also keeps h = [g, u]
    return a.act_format == MOK_ACT_MXFP8_E4M3 ? launch_one<true, EPI_SWIGLU_MX_H>(g, n1, m_tiles, s)
                                               : launch_one<false, EPI_SWIGLU_BF16_H>(g, n1, m_tiles, s);
  }
  return a.act_format == MOK_ACT_MXFP8_E4M3 ? launch_one<true, EPI_SWIGLU_MX>(g, n1, m_tiles, s)
                                             : launch_one<false, EPI_SWIGLU_BF16>(g, n1, m_tiles, s);
}

hipError_t launch_down(const FfnArgs& a, hipStream_t s) {
  const int64_t span = static_cast<int64_t>(a.s_end) - a.s_begin;
  if (span <= 0) return hipSuccess;
  const int m_tiles = static_cast<int>((span + BM - 1) / BM) + a.n_local;
  GemmParams g{};
  g.offsets = a.offsets; g.n_local = a.n_local; g.s_begin = a.s_begin; g.s_end = a.s_end;
  g.A = a.act; g.A_scales = a.act_scales; g.a_rows = a.act_rows;
  g.W = a.w_d; g.w_expert_stride = static_cast<int64_t>(a.H) * a.I; g.K = a.I;
  g.N = a.H; g.I = 0;
  g.C = a.y; g.C_scales = nullptr; g.c_rows = a.y_rows;
  g.w_packed = a.w_packed;
  set_split(g, a);
  const int n2 = (a.H + BN - 1) / BN;
  const bool mx = a.act_format == MOK_ACT_MXFP8_E4M3;
  if (a.merge.aos) {               // single-slot tokens merged in the epilogue
    const hipError_t e = launch_merge_plan(a.merge.aos, a.offsets, a.n_local, a.s_begin, a.s_end,
                                           a.merge.soa, a.merge.gate, a.merge.k, a.H,
                                           a.merge.out_parts, a.merge.n_part, a.merge.part_rows,
                                           a.merge.plan, s);
    if (e != hipSuccess) return e;
    g.m_plan = static_cast<const uint4*>(a.merge.plan); g.m_status = a.merge.status;
    if (a.weight_format == MOK_W_MXFP8_E4M3) return launch_one_mx8<EPI_DOWN_MERGE>(g, n2, m_tiles, s);
    return mx ? launch_one<true, EPI_DOWN_MERGE>(g, n2, m_tiles, s)
              : launch_one<false, EPI_DOWN_MERGE>(g, n2, m_tiles, s);
  }
  if (a.weight_format == MOK_W_MXFP8_E4M3) return launch_one_mx8<EPI_STORE_BF16>(g, n2, m_tiles, s);
  return mx ? launch_one<true, EPI_STORE_BF16>(g, n2, m_tiles, s)
            : launch_one<false, EPI_STORE_BF16>(g, n2, m_tiles, s);
}

// ------------------------------------------------------------ backward
// h = x . W_gu^T, stored whole (bf16 [rows][2I], row-major) for the SwiGLU
// backward: the forward's gate/up GEMM (packed or not) with g and u stored.
hipError_t launch_recompute_h(const BwdArgs& a, hipStream_t s) {
  const int64_t span = static_cast<int64_t>(a.s_end) - a.s_begin;
  if (span <= 0) return hipSuccess;
  const int m_tiles = static_cast<int>((span + BM - 1) / BM) + a.n_local;
  GemmParams g{};
  g.offsets = a.offsets; g.n_local = a.n_local; g.s_begin = a.s_begin; g.s_end = a.s_end;
  g.A = a.ring; g.A_scales = a.ring_scales; g.a_rows = a.ring_slots;
  g.W = a.w_gu; g.w_expert_stride = static_cast<int64_t>(2) * a.I * a.H; g.K = a.H;
  g.N = a.I; g.I = a.I;
  g.C = a.h; g.c_rows = a.rows;
  g.w_packed = a.w_gu_packed;
  const int nt = (a.I + BN / 2 - 1) / (BN / 2);
  if (a.w_mx8) return launch_one_mx8<EPI_STORE_GU>(g, nt, m_tiles, s);   // forward-packed W_gu
  return a.mx ? launch_one<true, EPI_STORE_GU>(g, nt, m_tiles, s)
              : launch_one<false, EPI_STORE_GU>(g, nt, m_tiles, s);
}

// da = dy . W_d (dy column-blocked, K = H), then dh = SwiGLU'(h) . da in the
// epilogue (column-blocked, 2I wide; MXFP8 dy in, MXFP8 dh out when a.mx).
// B: W_d^T packed [n_local][I][H].
hipError_t launch_down_dgrad(const BwdArgs& a, hipStream_t s) {
  const int64_t span = static_cast<int64_t>(a.s_end) - a.s_begin;
  if (span <= 0) return hipSuccess;
  const int m_tiles = static_cast<int>((span + BM - 1) / BM) + a.n_local;
  GemmParams g{};
  g.offsets = a.offsets; g.n_local = a.n_local; g.s_begin = a.s_begin; g.s_end = a.s_end;
  g.A = a.dy; g.A_scales = a.dy_scales; g.a_rows = a.rows;
  g.W = a.w_d_t; g.w_expert_stride = static_cast<int64_t>(a.H) * a.I; g.K = a.H;
  g.N = a.I; g.I = 0;
  g.C = a.dh; g.C_scales = a.dh_scales; g.c_rows = a.rows;
  g.H_src = static_cast<const uint16_t*>(a.h);
  g.w_packed = 1;
  const int nt = (a.I + BN - 1) / BN;
  if (a.w_mx8) return launch_one_mx8<EPI_SWIGLU_BWD_MX>(g, nt, m_tiles, s);
  return a.mx ? launch_one<true, EPI_SWIGLU_BWD_MX>(g, nt, m_tiles, s)
              : launch_one<false, EPI_SWIGLU_BWD>(g, nt, m_tiles, s);
}

// dx_s = dh . W_gu (dh column-blocked, K = 2I) -> bf16 [rows][H], row-major.
// B: W_gu^T packed [n_local][H][2I].
hipError_t launch_gate_up_dgrad(const BwdArgs& a, hipStream_t s) {
  const int64_t span = static_cast<int64_t>(a.s_end) - a.s_begin;
  if (span <= 0) return hipSuccess;
  const int m_tiles = static_cast<int>((span + BM - 1) / BM) + a.n_local;
  GemmParams g{};
  g.offsets = a.offsets; g.n_local = a.n_local; g.s_begin = a.s_begin; g.s_end = a.s_end;
  g.A = a.dh; g.A_scales = a.dh_scales; g.a_rows = a.rows;
  g.W = a.w_gu_t; g.w_expert_stride = static_cast<int64_t>(2) * a.I * a.H; g.K = 2 * a.I;
  g.N = a.H; g.I = 0;
  g.C = a.dx; g.c_rows = a.rows;
  g.w_packed = 1;
  g.n_cus = a.n_cus;
  const int nt = (a.H + BN - 1) / BN;
  if (a.w_mx8) return launch_one_mx8<EPI_STORE_BF16>(g, nt, m_tiles, s);
  return a.mx ? launch_one<true, EPI_STORE_BF16>(g, nt, m_tiles, s)
              : launch_one<false, EPI_STORE_BF16>(g, nt, m_tiles, s);
}

hipError_t launch_ffn_backward(const BwdArgs& a, hipStream_t s) {
  hipError_t e = a.h_saved ? hipSuccess : launch_recompute_h(a, s);
  if (e == hipSuccess) e = launch_down_dgrad(a, s);
  if (e == hipSuccess) e = launch_gate_up_dgrad(a, s);
  return e;
}

size_t packed_bwd_gate_up_bytes(int32_t H, int32_t I, int32_t n_local, int32_t weight_format) {
  const size_t tiles = static_cast<size_t>(n_local) * ((H + BN - 1) / BN);
  if (weight_format == MOK_W_MXFP8_E4M3) return tiles * (2 * I / GeoMX8::BK) * GeoMX8::WBLOCK;
  return tiles * BM * (2 * static_cast<size_t>(I)) * 2;
}
size_t packed_bwd_down_bytes(int32_t H, int32_t I, int32_t n_local, int32_t weight_format) {
  const size_t tiles = static_cast<size_t>(n_local) * ((I + BN - 1) / BN);
  if (weight_format == MOK_W_MXFP8_E4M3) return tiles * (H / GeoMX8::BK) * GeoMX8::WBLOCK;
  return tiles * BM * static_cast<size_t>(H) * 2;
}

hipError_t launch_pack_weights_bwd(const uint16_t* w_gu, const uint16_t* w_d, int32_t H, int32_t I,
                                   int32_t n_local, bool act_mx, bool w_mx8, uint16_t* packed_gu_t,
                                   uint16_t* packed_d_t, hipStream_t s) {
  auto pack_t = [&](const uint16_t* W, int64_t stride, int32_t K, int32_t N, uint16_t* out) {
    const int n_tiles = (N + BN - 1) / BN;
    if (w_mx8) {                   // MXFP8: quantised along k, the backward GEMM's contraction
      const int64_t threads = static_cast<int64_t>(n_local) * n_tiles * (K / GeoMX8::BK) * BM;
      const int64_t blocks = (threads + 255) / 256;
      hipLaunchKernelGGL(k_pack_weights_mx8_t, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)),
                         dim3(256), 0, s, W, stride, K, N, n_tiles, n_local,
                         reinterpret_cast<uint8_t*>(out));
      return hipGetLastError();
    }
    // the same number of 16-byte pieces for either k-step (K % 64 == 0)
    const int64_t pieces = static_cast<int64_t>(n_local) * n_tiles * K * BM / 8;
    const int64_t blocks = (pieces + 255) / 256;
    const dim3 grid(static_cast<unsigned>(blocks < 65536 ? blocks : 65536));
    if (act_mx)
      hipLaunchKernelGGL(k_pack_weights_t<true>, grid, dim3(256), 0, s, W, stride, K, N, n_tiles,
                         n_local, out);
    else
      hipLaunchKernelGGL(k_pack_weights_t<false>, grid, dim3(256), 0, s, W, stride, K, N, n_tiles,
                         n_local, out);
    return hipGetLastError();
  };
  hipError_t e = hipSuccess;
  if (w_gu && packed_gu_t) e = pack_t(w_gu, static_cast<int64_t>(2) * I * H, 2 * I, H, packed_gu_t);
  if (e == hipSuccess && w_d && packed_d_t) e = pack_t(w_d, static_cast<int64_t>(H) * I, H, I, packed_d_t);
  return e;
}

size_t packed_gate_up_bytes(int32_t H, int32_t I, int32_t n_local, int32_t weight_format) {
  const size_t tiles = static_cast<size_t>(n_local) * ((I + BN / 2 - 1) / (BN / 2));
  if (weight_format == MOK_W_MXFP8_E4M3) return tiles * (H / GeoMX8::BK) * GeoMX8::WBLOCK;
  return tiles * BM * H * 2;
}
size_t packed_down_bytes(int32_t H, int32_t I, int32_t n_local, int32_t weight_format) {
  const size_t tiles = static_cast<size_t>(n_local) * ((H + BN - 1) / BN);
  if (weight_format == MOK_W_MXFP8_E4M3) return tiles * (I / GeoMX8::BK) * GeoMX8::WBLOCK;
  return tiles * BM * I * 2;
}

hipError_t launch_pack_weights(const uint16_t* w_gu, const uint16_t* w_d, int32_t H, int32_t I,
                               int32_t n_local, int32_t act_format, int32_t weight_format,
                               uint16_t* packed_gu, uint16_t* packed_d, hipStream_t s) {
  const bool mx = act_format == MOK_ACT_MXFP8_E4M3;
  const int n1 = (I + BN / 2 - 1) / (BN / 2), n2 = (H + BN - 1) / BN;
  hipError_t err = hipSuccess;
  if (weight_format == MOK_W_MXFP8_E4M3) {
    if (w_gu && packed_gu)
      err = pack_one_mx8(w_gu, static_cast<int64_t>(2) * I * H, H, I, 0, true, n1, n_local,
                         reinterpret_cast<uint8_t*>(packed_gu), s);
    if (err == hipSuccess && w_d && packed_d)
      err = pack_one_mx8(w_d, static_cast<int64_t>(H) * I, I, 0, H, false, n2, n_local,
                         reinterpret_cast<uint8_t*>(packed_d), s);
    return err;
  }
  if (w_gu && packed_gu)
    err = mx ? pack_one<true>(w_gu, static_cast<int64_t>(2) * I * H, H, I, 0, true, n1, n_local, packed_gu, s)
             : pack_one<false>(w_gu, static_cast<int64_t>(2) * I * H, H, I, 0, true, n1, n_local, packed_gu, s);
  if (err == hipSuccess && w_d && packed_d)
    err = mx ? pack_one<true>(w_d, static_cast<int64_t>(H) * I, I, 0, H, false, n2, n_local, packed_d, s)
             : pack_one<false>(w_d, static_cast<int64_t>(H) * I, I, 0, H, false, n2, n_local, packed_d, s);
  return err;
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  hipError_t err = launch_gate_up(a, s);
  return err != hipSuccess ? err : launch_down(a, s);
}

}  // namespace mok
