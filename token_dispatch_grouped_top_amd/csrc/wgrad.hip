// wgrad.hip -- weight gradients of the expert FFN (the backward layer's
// GEMMs that contract over each expert's slots):
//   dW_d[e]  = sum_{s of e} dy_s a_s^T   (H x I)
//   dW_gu[e] = sum_{s of e} dh_s x_s^T   (2I x H)
//
// The forward's grouped GEMM tile runs them unchanged once both operands are
// slot-contiguous: a transpose (through LDS) turns each slot-row buffer into
// feature rows over a padded slot axis, where expert e owns the padded
// positions [poff[e], poff[e+1]), a whole number of 32-slot k-steps (at least
// one, zero-filled past its count).  The A operand (dy^T, dh^T) is
// column-blocked over that axis like the ring, the B operand (a^T, x^T) is
// row-major like unpacked weights.  One tile per (expert, 256 feature rows,
// 256 output columns); its row wraps modulo the feature count in A, and the
// output row is e * M + feature.
#include "gemm_tile.h"

namespace mok {

namespace {

using namespace gemm;

constexpr int kPadK = 32;         // padded slot axis granularity (one bf16 k-step)

// poff[e] = sum over e' < e of max(32, 32 * ceil(count_e' / 32)); one thread.
__global__ void k_pad_offsets(const int32_t* __restrict__ offsets, int32_t n_local, int32_t kpad,
                              int32_t* __restrict__ poff) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int32_t acc = 0;
  bool fits = true;
  for (int e = 0; e < n_local && fits; ++e) {
    const int32_t c = offsets[e + 1] - offsets[e];
    if (c > kpad) { fits = false; break; }
    acc += c > 0 ? (c + kPadK - 1) / kPadK * kPadK : kPadK;
    fits = acc <= kpad;
  }
  // Counts past the padded axis (offsets claiming more than rows slots) give
  // every expert one segment of kPadK slots, so no read leaves the buffers.
  acc = 0;
  for (int e = 0; e < n_local; ++e) {
    poff[e] = acc;
    const int32_t c = offsets[e + 1] - offsets[e];
    acc += fits && c > 0 ? (c + kPadK - 1) / kPadK * kPadK : kPadK;
  }
  poff[n_local] = acc;
}

// Transpose of a column-blocked slot-row buffer (rows s % src_rows, F bf16
// features) into feature rows over the padded slot axis: 64 positions x 64
// features per workgroup, through an LDS tile.  dst_blocked: column-blocked
// (64-byte block kb of feature row f at (kb * F + f) * 64); else row-major
// [F][kpad].  Positions past a segment's count, and past poff[n_local], get
// zeros.  MX: the source holds E4M3 codes (one byte per feature) and E8M0
// scales (pairs); each value is converted to bf16 on the way, code x 2^E,
// which bf16 holds exactly for every code whose value is at least 2^-133.
template <bool MX>
__global__ __launch_bounds__(256)
void k_slot_transpose(const uint8_t* __restrict__ src, const uint8_t* __restrict__ src_scales,
                      int32_t src_rows, int32_t F,
                      const int32_t* __restrict__ offsets, const int32_t* __restrict__ poff,
                      int32_t n_local, int32_t kpad, int32_t dst_blocked,
                      uint8_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][64 + 2];
  __shared__ int32_t s_poff[257], s_off[257];
  const int tid = threadIdx.x;
  for (int e = tid; e <= n_local; e += 256) { s_poff[e] = poff[e]; s_off[e] = offsets[e]; }
  __syncthreads();
  const int q0 = blockIdx.x * 64, f0 = blockIdx.y * 64;
  // load: thread -> (position q0 + tid / 8 + 32 j, 8 features at chunk tid % 8)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ql = tid / 8 + 32 * j, c = tid % 8, q = q0 + ql;
    int lo = 0, hi = n_local - 1;                      // last e with poff[e] <= q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_poff[mid] <= q) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int32_t jj = q - s_poff[e], cnt = s_off[e + 1] - s_off[e];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (q < s_poff[n_local] && jj >= 0 && jj < cnt) {
      const int64_t s = s_off[e] + jj;
      if (MX) {
        const int64_t row = s % src_rows;
        const uint2 c8 = *reinterpret_cast<const uint2*>(src + colblk_byte(row, src_rows, f0 + 8 * c));
        const uint32_t S = src_scales[scale_byte(row, src_rows, (f0 + 8 * c) >> 5)];
        const float sc = __uint_as_float(S ? S << 23 : 0x00400000u);      // 2^(S - 127)
        v = make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.x, sc, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.x, sc, true)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.y, sc, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.y, sc, true)));
      } else {
        v = *reinterpret_cast<const uint4*>(src + colblk_byte(s % src_rows, src_rows, 2 * (f0 + 8 * c)));
      }
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      tile[ql][8 * c + 2 * t] = static_cast<uint16_t>(w[t] & 0xffffu);
      tile[ql][8 * c + 2 * t + 1] = static_cast<uint16_t>(w[t] >> 16);
    }
  }
  __syncthreads();
  // store: thread -> (feature f0 + tid / 8 + 32 j, 8 positions at chunk tid % 8)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int fl = tid / 8 + 32 * j, c = tid % 8;
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      w[t] = static_cast<uint32_t>(tile[8 * c + 2 * t][fl]) |
             (static_cast<uint32_t>(tile[8 * c + 2 * t + 1][fl]) << 16);
    const int64_t f = f0 + fl, q = q0 + 8 * c;
    uint8_t* d = dst_blocked ? dst + colblk_byte(f, F, 2 * q) : dst + (f * kpad + q) * 2;
    *reinterpret_cast<uint4*>(d) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// One tile per (expert, 256 feature rows, 256 output columns).
__global__ __launch_bounds__(kThreads)
void k_wgrad(const GemmParams p, const int32_t* __restrict__ poff, int32_t M, int32_t mt, int32_t nt) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[Geo<false>::LDS];
  const int bid = blockIdx.x;
  const int e = bid / (mt * nt), rem = bid % (mt * nt);
  if (e >= p.n_local) return;
  const int mtile = rem / nt, ntile = rem % nt;
  TileJob j;
  j.e = 0;                                   // B is one matrix over the padded slot axis
  j.row0 = e * M + mtile * BM;
  j.nrows = M - mtile * BM < BM ? M - mtile * BM : BM;
  j.ntile = ntile;
  j.kt0 = poff[e] / kPadK;
  j.nkt = (poff[e + 1] - poff[e]) / kPadK;   // >= 1
  j.role = kWhole; j.slot = 0; j.slot0 = 0; j.npieces = 0; j.cnt = nullptr; j.half = 0;
  gemm_tile<false, EPI_STORE_BF16>(p, j, lds);
}

// Launch of one weight gradient: dW [n_local][M][N] = A^T-slots x B^T-slots.
hipError_t launch_wgrad_one(const void* at, const void* bt, int32_t M, int32_t N, int32_t kpad,
                            const int32_t* offsets, const int32_t* poff, int32_t n_local, void* dw,
                            hipStream_t s) {
  GemmParams g{};
  g.A = at; g.a_rows = M; g.a_row_base = 0;
  g.W = static_cast<const uint16_t*>(bt); g.w_expert_stride = static_cast<int64_t>(N) * kpad;
  g.K = kpad; g.N = N; g.I = 0;
  g.C = dw; g.c_rows = n_local * M; g.c_row_base = 0;
  g.offsets = offsets; g.n_local = n_local;
  g.w_packed = 0;
  const int mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
  g.n_tiles = nt;
  hipLaunchKernelGGL(k_wgrad, dim3(static_cast<unsigned>(n_local * mt * nt)), dim3(kThreads), 0, s, g,
                     poff, M, mt, nt);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, const uint8_t* scales, int32_t src_rows, int32_t F,
                            const int32_t* offsets, const int32_t* poff, int32_t n_local,
                            int32_t kpad, bool blocked, void* dst, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(kpad / 64), static_cast<unsigned>(F / 64));
  if (scales)
    hipLaunchKernelGGL(k_slot_transpose<true>, grid, dim3(256), 0, s, static_cast<const uint8_t*>(src),
                       scales, src_rows, F, offsets, poff, n_local, kpad, blocked ? 1 : 0,
                       static_cast<uint8_t*>(dst));
  else
    hipLaunchKernelGGL(k_slot_transpose<false>, grid, dim3(256), 0, s, static_cast<const uint8_t*>(src),
                       scales, src_rows, F, offsets, poff, n_local, kpad, blocked ? 1 : 0,
                       static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

}  // namespace

int32_t wgrad_kpad(int32_t rows, int32_t n_local) {
  const int64_t k = static_cast<int64_t>(rows) + static_cast<int64_t>(kPadK) * n_local;
  return static_cast<int32_t>((k + 63) / 64 * 64);
}

size_t wgrad_ws_bytes(int32_t rows, int32_t H, int32_t I, int32_t n_local) {
  const size_t kp = static_cast<size_t>(wgrad_kpad(rows, n_local));
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  return al(static_cast<size_t>(n_local + 1) * 4) + al(kp * H * 2) * 2 + al(kp * 2 * I * 2) +
         al(kp * I * 2);
}

hipError_t launch_wgrad(const WgradArgs& a, hipStream_t s) {
  const int32_t kp = wgrad_kpad(a.rows, a.n_local);
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  uint8_t* w = static_cast<uint8_t*>(a.ws);
  int32_t* poff = reinterpret_cast<int32_t*>(w);
  w += al(static_cast<size_t>(a.n_local + 1) * 4);
  void* dyT = w; w += al(static_cast<size_t>(kp) * a.H * 2);
  void* xT = w; w += al(static_cast<size_t>(kp) * a.H * 2);
  void* dhT = w; w += al(static_cast<size_t>(kp) * 2 * a.I * 2);
  void* aT = w;
  hipLaunchKernelGGL(k_pad_offsets, dim3(1), dim3(64), 0, s, a.offsets, a.n_local, kp, poff);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess)
    e = launch_transpose(a.dy, a.dy_scales, a.rows, a.H, a.offsets, poff, a.n_local, kp, true, dyT, s);
  if (e == hipSuccess)
    e = launch_transpose(a.act, a.act_scales, a.act_rows, a.I, a.offsets, poff, a.n_local, kp, false, aT, s);
  if (e == hipSuccess)
    e = launch_transpose(a.dh, a.dh_scales, a.rows, 2 * a.I, a.offsets, poff, a.n_local, kp, true, dhT, s);
  if (e == hipSuccess)
    e = launch_transpose(a.ring, a.ring_scales, a.ring_slots, a.H, a.offsets, poff, a.n_local, kp, false, xT, s);
  if (e == hipSuccess && a.dw_d) e = launch_wgrad_one(dyT, aT, a.H, a.I, kp, a.offsets, poff, a.n_local, a.dw_d, s);
  if (e == hipSuccess && a.dw_gu)
    e = launch_wgrad_one(dhT, xT, 2 * a.I, a.H, kp, a.offsets, poff, a.n_local, a.dw_gu, s);
  return e;
}

}  // namespace mok
