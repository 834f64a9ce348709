// gemm_tile.h -- the grouped bf16 MFMA GEMM tile of the expert FFN (device
// code shared by the standalone GEMM kernels and the persistent pipeline).
// See gemm.hip for the design notes.
#pragma once

#include "mok_internal.h"

namespace mok {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes of LDS through a vector-typed load.  A struct copy (uint4) carries
// no type-based alias information, and without it the compiler makes the read
// wait for every direct-to-LDS load in flight (vmcnt(0), the newest stages
// included); the pipelines' own vmcnt waits and barriers order the reads.
__device__ __forceinline__ uint4 lds_read16(const uint8_t* p) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int BM = 256, BN = 256;
constexpr int kThreads = 256;
constexpr int kEpiLds = BM * BN * 2;           // epilogue staging: 256 x 256 bf16 / 256 x 128 fp32
constexpr int kMergeLds = kEpiLds + BM * 12;   // EPI_DOWN_MERGE: + a destination and a gate per row

// Pipeline shape per A-operand format.
#ifndef MOK_BF16_BK
#define MOK_BF16_BK 32
#endif
#ifndef MOK_BF16_NS
#define MOK_BF16_NS 4
#endif
template <bool A_MX> struct Pipe;
template <> struct Pipe<false> { static constexpr int BK = MOK_BF16_BK, NS = MOK_BF16_NS; };
template <> struct Pipe<true> { static constexpr int BK = 64, NS = 3; };

// Chunk XOR key of an LDS row of `cpr` 16-byte chunks: the b128 fragment reads
// of 16 consecutive rows at one logical chunk hit distinct banks.
template <int cpr> __device__ __forceinline__ int chunk_key(int row) {
  return cpr == 8 ? ((row & 7) ^ ((row >> 3) & 1)) : ((row >> 2) & 3);
}

// LDS geometry of one pipeline stage: [A tile][B tile][A scales].
//   B (weights, bf16): 256 rows of BK * 2 bytes.
//   A: bf16 rows like B, or E4M3 codes (BK bytes per row) plus one 4-byte
//      slot per row holding the row's two E8M0 block scales of the k-step.
template <bool A_MX> struct Geo {
  static constexpr int BK = Pipe<A_MX>::BK, NS = Pipe<A_MX>::NS;
  static constexpr int ROWB_B = BK * 2, CPR_B = ROWB_B / 16, TILE_B = BM * ROWB_B;
  static constexpr int ROWB_A = A_MX ? BK : BK * 2, CPR_A = ROWB_A / 16, TILE_A = BM * ROWB_A;
  static constexpr int SCALEB = A_MX ? BM * 4 : 0;
  static constexpr int STAGEB = TILE_A + TILE_B + SCALEB;
  // one wave instruction fills 1 KiB; four waves cover RSTEP rows per round
  static constexpr int NLOAD_B = TILE_B / 4096, RSTEP_B = 4 * 1024 / ROWB_B;
  static constexpr int NLOAD_A = TILE_A / 4096, RSTEP_A = 4 * 1024 / ROWB_A;
  static constexpr int LOOP_LDS = NS * STAGEB;
  static constexpr int LDS = LOOP_LDS > kEpiLds ? LOOP_LDS : kEpiLds;
  static __device__ __forceinline__ int offA(int row, int chunk) {
    return row * ROWB_A + ((chunk ^ chunk_key<CPR_A>(row)) << 4);
  }
  static __device__ __forceinline__ int offB(int row, int chunk) {
    return row * ROWB_B + ((chunk ^ chunk_key<CPR_B>(row)) << 4);
  }
};
static_assert(Geo<false>::LDS <= 160 * 1024 && Geo<true>::LDS <= 160 * 1024, "LDS budget");

// EPI_SWIGLU_BWD: the backward of SwiGLU on the down GEMM's gradient (da):
// reads g, u of the same (row, i) from H_src and writes dh = [dg, du] (bf16;
// EPI_SWIGLU_BWD_MX: MXFP8, blocks of 32 along 2I, into C and C_scales).
// EPI_STORE_GU: a gate/up tile stores g and u themselves (h = [g, u], bf16
// [c_rows][2 N] row-major) for that backward.  EPI_SWIGLU_BF16_H and
// EPI_SWIGLU_MX_H: the forward's SwiGLU epilogues that also store h so.
// EPI_DOWN_MERGE: the down GEMM's store with the merge of single-slot tokens
// (a slot that is its token's only local slot goes to the token's output row
// as bf16(gate * y); every other slot's y to C as EPI_STORE_BF16).
enum Epi { EPI_SWIGLU_BF16 = 0, EPI_SWIGLU_MX = 1, EPI_STORE_BF16 = 2, EPI_SWIGLU_BWD = 3,
           EPI_STORE_GU = 4, EPI_SWIGLU_BF16_H = 5, EPI_SWIGLU_BWD_MX = 6, EPI_SWIGLU_MX_H = 7,
           EPI_DOWN_MERGE = 8 };
// LDS of a GEMM kernel: the pipeline's (with the usual epilogue's), or the
// merging epilogue's if larger.
template <int LOOP, int EPI> constexpr int kernel_lds() {
  return EPI == EPI_DOWN_MERGE && kMergeLds > LOOP ? kMergeLds : LOOP;
}
// Whether an epilogue pairs gate and up columns (the gate/up weight order).
template <int EPI> constexpr bool epi_swiglu() {
  return EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_MX || EPI == EPI_STORE_GU ||
         EPI == EPI_SWIGLU_BF16_H || EPI == EPI_SWIGLU_MX_H;
}

struct GemmParams {
  const void* A;              // bf16 or E4M3 codes, a_rows x K, column-blocked
  const uint8_t* A_scales;    // a_rows x K/32 scale pairs (column-blocked) when A is MXFP8
  int32_t a_rows;
  const uint16_t* W;          // [n_local][w_rows][K]
  int64_t w_expert_stride;    // elements
  int32_t K;
  int32_t N;                  // output columns (I for gate/up, H for down)
  int32_t I;                  // up-row offset for gate/up
  void* C;                    // y: bf16 [c_rows][N]; act: bf16 or E4M3 codes, column-blocked
  uint8_t* C_scales;          // act scale pairs, c_rows x N/32 (column-blocked)
  int32_t c_rows;
  const int32_t* offsets;
  int32_t n_local;
  int32_t s_begin, s_end;
  int32_t n_tiles;            // output column tiles
  int32_t w_packed;           // W in the packed tile order written by launch_pack_weights
  int32_t a_row_base;         // A row of slot s: (s + a_row_base) % a_rows
  int32_t c_row_base;         // C row of slot s: (s + c_row_base) % c_rows
  const uint16_t* H_src;      // EPI_SWIGLU_BWD: h = [g, u] bf16 [c_rows][2 N], row-major
  uint16_t* H_out;            // EPI_SWIGLU_BF16_H: h = [g, u] bf16 [c_rows][2 N], row-major
  // EPI_DOWN_MERGE: per slot s, m_plan[s] = {output row address (lo, hi), gate
  // bits, 0}, address 0 for a slot whose y goes to C (launch_merge_plan)
  const uint4* m_plan;
  const int32_t* m_status;    // non-null: a raised status word stops the output stores
  // Split of the last, partial round of tiles along K (standalone launches):
  float* part;                // [n_cus][BM * BN] fp32 partial tiles; null = no split
  int32_t* part_cnt;          // [n_cus] arrival counters, zero before and after a launch
  int32_t n_cus;
};

// What one workgroup computes: a whole tile, or the k-steps [kt0, kt0 + nkt)
// of a tile split into npieces pieces, whose fp32 sums go to slot (piece
// slot0 + piece number) and whose arrivals are counted in *cnt.
enum TileRole { kWhole = 0, kPiece = 1 };
struct TileJob {
  int e, row0, nrows, ntile;
  int kt0, nkt;               // nkt = 0: all k-steps
  int role, slot, slot0, npieces;
  int32_t* cnt;
  int half;                   // 0: the whole column tile; 1, 2: its first or second 128 columns
};

// Tile order and placement.  Tiles are numbered expert by expert; inside an
// expert, n-tile major and m-tile minor, so the workgroups running at the same
// time share the expert's A rows and a few weight tiles.  Workgroup ids are
// dealt to the 8 XCDs round-robin (id % 8); each XCD is given a contiguous run
// of tile numbers, so an expert's operands are fetched into one XCD's L2
// instead of all eight.  Returns false for workgroups past the last tile.
constexpr int kXcds = 8;

// m-tiles of the window [w0, w1) (already clipped to R), summed over experts.
__device__ __forceinline__ int window_mtiles(const int32_t* __restrict__ offsets, int32_t n_local,
                                             int32_t w0, int32_t w1) {
  int total = 0;
  for (int e = 0; e < n_local; ++e) {
    const int32_t lo = offsets[e] < w0 ? w0 : offsets[e];
    const int32_t hi = offsets[e + 1] > w1 ? w1 : offsets[e + 1];
    if (hi > lo) total += (hi - lo + BM - 1) / BM;
  }
  return total;
}

// Tile t of the window in (expert, n-tile, m-tile) order.
__device__ __forceinline__ bool tile_of(const int32_t* __restrict__ offsets, int32_t n_local,
                                        int32_t w0, int32_t w1, int n_tiles, int t, int& e_out,
                                        int& row0, int& nrows, int& ntile) {
  for (int e = 0; e < n_local; ++e) {
    const int32_t lo = offsets[e] < w0 ? w0 : offsets[e];
    const int32_t hi = offsets[e + 1] > w1 ? w1 : offsets[e + 1];
    if (hi <= lo) continue;
    const int mt = (hi - lo + BM - 1) / BM;
    if (t < mt * n_tiles) {
      const int m = t % mt;
      ntile = t / mt;
      e_out = e;
      row0 = lo + m * BM;
      nrows = (hi - row0) < BM ? (hi - row0) : BM;
      return true;
    }
    t -= mt * n_tiles;
  }
  return false;
}

// Tile of workgroup `bid` in a standalone launch: XCD x = bid % 8 takes the
// x-th contiguous eighth of the window's tiles.
__device__ __forceinline__ bool decode_tile(const int32_t* __restrict__ offsets, int32_t n_local,
                                            int32_t s_begin, int32_t s_end, int n_tiles, int bid,
                                            int& e_out, int& row0, int& nrows, int& ntile) {
  const int32_t R = offsets[n_local];
  const int32_t w0 = s_begin, w1 = s_end < R ? s_end : R;
  if (w1 <= w0) return false;
  const int total = window_mtiles(offsets, n_local, w0, w1) * n_tiles;
  const int q = total / kXcds, r = total % kXcds;
  const int x = bid % kXcds, i = bid / kXcds;
  if (i >= q + (x < r ? 1 : 0)) return false;
  return tile_of(offsets, n_local, w0, w1, n_tiles, x * q + (x < r ? x : r) + i, e_out, row0, nrows,
                 ntile);
}

// Workgroup `bid` of a standalone launch with the tail split.  Per XCD x (its
// contiguous share of c tiles, run by P = n_cus / 8 CUs in rounds), the last
// r = c % P tiles would make a round of their own with P - r CUs idle.  They
// are cut into s pieces of k-steps instead, run by the workgroups that follow
// the whole tiles in dispatch order, where
//   s = min(P / r, nk / 8, 8, 1 + (workgroups of XCD x - c) / r)
// and s >= 3: a round half full of whole tiles runs each tile faster than a
// full one (more L2 and memory bandwidth per CU), and two pieces did not win
// back the partial sums' traffic (measured: 250 -> 262 us on a down GEMM with
// 16 of 32 CUs per XCD in its last round).  Slots and counters of XCD x are
// [x * P, (x + 1) * P).
// Half-width tail (`halves`, the y-storing epilogues): where no split into
// pieces is taken and the r tail tiles fill at most half of the XCD's CUs,
// each is run as two tiles of 128 columns instead (the first half of these
// jobs before the whole tiles, the rest after them).  A round of tiles runs as
// long as a full one however
// few of them there are (measured on the Kimi-shaped down GEMM, 256 tiles per
// round: 3.5 rounds took as long as 4); a half-width tile does half the MFMAs
// on the same token panel and needs no partial sums.  Every output element is
// summed by the same MFMAs in the same order either way.
constexpr int kSplitMinSteps = 8, kSplitMax = 8, kSplitMinPieces = 3;
__device__ __forceinline__ bool decode_job(const GemmParams& p, int nk, int bid, TileJob& j,
                                           bool halves = false) {
  const int32_t R = p.offsets[p.n_local];
  const int32_t w0 = p.s_begin, w1 = p.s_end < R ? p.s_end : R;
  if (w1 <= w0) return false;
  const int total = window_mtiles(p.offsets, p.n_local, w0, w1) * p.n_tiles;
  const int q = total / kXcds, r = total % kXcds;
  const int x = bid % kXcds, i = bid / kXcds;
  const int c = q + (x < r ? 1 : 0), start = x * q + (x < r ? x : r);
  j.kt0 = 0; j.nkt = 0; j.role = kWhole; j.slot = 0; j.slot0 = 0; j.npieces = 0; j.cnt = nullptr;
  j.half = 0;
  int t = i;
  bool pieces = false;
  if (p.part != nullptr && p.n_cus >= kXcds) {
    const int P = p.n_cus / kXcds, rx = c % P;
    const int gx = (static_cast<int>(gridDim.x) - x + kXcds - 1) / kXcds;  // >= c
    int sp = rx > 0 ? P / rx : 0;
    if (sp > nk / kSplitMinSteps) sp = nk / kSplitMinSteps;
    if (sp > kSplitMax) sp = kSplitMax;
    if (rx > 0 && sp > 1 + (gx - c) / rx) sp = 1 + (gx - c) / rx;
    pieces = sp >= kSplitMinPieces;
    if (sp >= kSplitMinPieces && i >= c - rx) {
      const int u = i - (c - rx), tt = u / sp, piece = u % sp;
      if (tt >= rx) return false;
      t = c - rx + tt;
      j.kt0 = piece * nk / sp;
      j.nkt = (piece + 1) * nk / sp - j.kt0;
      j.role = kPiece;
      j.slot0 = x * P + tt * sp;
      j.slot = j.slot0 + piece;
      j.npieces = sp;
      j.cnt = p.part_cnt + x * P + tt;
    }
  }
  if (halves && !pieces && p.n_cus >= kXcds) {
    const int P = p.n_cus / kXcds, rx = c % P;
    const int gx = (static_cast<int>(gridDim.x) - x + kXcds - 1) / kXcds;  // workgroups of XCD x
    if (rx > 0 && 2 * rx <= P && gx >= c + rx) {
      // Dispatch order of XCD x: the first rx half-width jobs, the c - rx
      // whole tiles, then the other rx half-width jobs (u = 0 .. 2 rx - 1
      // numbers the halves of the tail tiles).  The CUs that start with a
      // half-width job stay half a tile ahead of the others until the end,
      // so the rounds' epilogue stores and first loads are spread over two
      // half-size bursts instead of one that all CUs of the XCD wait on.
      int u = -1;
      if (i < rx) u = i;
      else if (i >= c) u = i - c + rx;
      else t = i - rx;
      if (u >= 2 * rx) return false;
      if (u >= 0) {
        t = c - rx + (u >> 1);
        j.half = 1 + (u & 1);
      }
    }
  }
  if (t >= c) return false;
  return tile_of(p.offsets, p.n_local, w0, w1, p.n_tiles, start + t, j.e, j.row0, j.nrows, j.ntile);
}

// Weight row held by row nb (0..255) of the B tile of output column tile
// `ntile`.  gate/up (swiglu): B rows 0..127 feed wave column 0, 128..255 wave
// column 1; in each, 64 gate rows then the 64 up rows of the same
// intermediate columns, so a lane's accumulators hold g and u of one (row, i).
// Columns past the end are clamped to the last one (masked at the store).
__device__ __forceinline__ int w_row_of(int nb, int ntile, bool swiglu, int32_t I, int32_t N) {
  if (swiglu) {
    const int wc = nb >> 7, q = nb & 127;
    int icol = ntile * (BN / 2) + 64 * wc + (q & 63);
    if (icol >= I) icol = I - 1;
    return (q < 64) ? icol : I + icol;
  }
  const int wrow = ntile * BN + nb;
  return wrow < N ? wrow : N - 1;
}

// Fourth word of a raw buffer descriptor on gfx9 (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// EPI_DOWN_MERGE: row tid's plan record (slot row0 + tid), loaded at the
// start of the tile so that it lands under the main loop.  The records are
// contiguous by slot (a wave's 64 rows are 1 KiB); looking the token up in
// the epilogue instead (assign_of_slot, then k slot_of_assign entries and the
// gate, scattered by token, again in each of a row block's column tiles) added
// about 15 % to the down GEMM's L2 requests, which bound it.
struct MergeRow {
  uint4 rec;
};
__device__ __forceinline__ void merge_row_load(const GemmParams& p, int row0, int nrows, MergeRow& m) {
  m.rec = static_cast<int>(threadIdx.x) < nrows ? p.m_plan[row0 + threadIdx.x] : make_uint4(0, 0, 0, 0);
}

// C row of tile row r, for tiles starting at window row row0: one modulo per
// tile, then a compare per row (a modulo per 16-byte store cost a third of
// the down GEMM's time).
struct CRows {
  int64_t base, rows;
  __device__ __forceinline__ CRows(const GemmParams& p, int row0)
      : base((static_cast<int64_t>(row0) + p.c_row_base) % p.c_rows), rows(p.c_rows) {}
  __device__ __forceinline__ int64_t operator()(int r) const {
    const int64_t c = base + r;
    return c < rows ? c : (rows >= BM ? c - rows : c % rows);
  }
};

// A (token) row of tile row r, tail rows clamped to the last valid one: one
// 32-bit modulo per tile, then a compare per row (a 64-bit modulo per row
// kept every tile's first loads waiting behind a few hundred instructions).
// Row numbers and the base are non-negative int32, so their sum fits in 32
// bits; a tile row beyond the ring's size takes the modulo again.
struct ARows {
  uint32_t base, rows;
  int nrows;
  __device__ __forceinline__ ARows(const GemmParams& p, int row0, int nrows_)
      : base((static_cast<uint32_t>(row0) + static_cast<uint32_t>(p.a_row_base)) %
             static_cast<uint32_t>(p.a_rows)),
        rows(static_cast<uint32_t>(p.a_rows)), nrows(nrows_) {}
  __device__ __forceinline__ uint32_t operator()(int r) const {
    uint32_t c = base + static_cast<uint32_t>(r < nrows ? r : nrows - 1);
    if (c >= rows) c -= rows;
    if (c >= rows) c %= rows;
    return c;
  }
};

// The y store of EPI_STORE_BF16 / EPI_DOWN_MERGE for a tile TN columns wide
// (256, or a half-width tail tile of 128) starting at output column n0.
// vals(mi, tv) gives the wave's accumulators of fragment row group mi as TN/16
// float4 (u = 4 ni + g: columns 8 g .. 8 g + 3 of tile (mi, ni)).  Staged
// through LDS for 16-byte global stores: accumulator element q of tile (mi, ni)
// is token row 32 mi + lane % 32 and column 32 ni + 8 (q / 4) + 4 (lane / 32) +
// q % 4 of the wave's 128 x TN/2 block, so each lane writes 4 consecutive
// columns of one row with one 8-byte store; staged rows keep their 16-byte
// chunk k at k ^ (row % 16), so the writes of 16 rows and the row-wise reads
// back are both free of bank conflicts.
template <int EPI, int TN, typename Vals>
__device__ __forceinline__ void store_y(const GemmParams& p, const TileJob& job, int n0, Vals&& vals,
                                        uint8_t* __restrict__ lds, const MergeRow& mr) {
  constexpr int NB = TN / 64, RB = TN * 2;                 // fragments per wave row, bytes per staged row
  const int nrows = job.nrows;
  const int tid = threadIdx.x, lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;
  const int erow = 128 * wm + (lane & 31), khalf = lane >> 5;
  const CRows c_row_of(p, job.row0);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int r = erow + 32 * mi;
    float4 tv[4 * NB];
    vals(mi, tv);
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = (TN / 2) * wn + 32 * ni + 8 * g + 4 * khalf;
        const float4 t = tv[4 * ni + g];
        const uint2 v = make_uint2(pack_bf16x2(t.x, t.y), pack_bf16x2(t.z, t.w));
        *reinterpret_cast<uint2*>(lds + r * RB + (((n >> 3) ^ (r & 15)) << 4) + ((n >> 2) & 1) * 8) = v;
      }
  }
  // EPI_DOWN_MERGE: where each row goes, one thread per row.  A slot that is
  // its token's only local slot (its plan record holds the token's output row)
  // goes there as bf16(fma(g, y, 0)) of the bf16 y: the slot-driven merge's
  // value for a single term, bit for bit.  Every other slot (and every slot
  // once m_status is raised) stores y in C.
  uint16_t** m_dst = reinterpret_cast<uint16_t**>(lds + kEpiLds);
  float* m_g = reinterpret_cast<float*>(lds + kEpiLds + BM * 8);
  if constexpr (EPI == EPI_DOWN_MERGE) {
    if (tid < nrows) {
      const bool go = p.m_status == nullptr || *p.m_status == 0;
      const uint64_t addr = static_cast<uint64_t>(mr.rec.x) | (static_cast<uint64_t>(mr.rec.y) << 32);
      m_dst[tid] = go ? reinterpret_cast<uint16_t*>(addr) : nullptr;
      m_g[tid] = __uint_as_float(mr.rec.z);
    }
  }
  __syncthreads();
  uint16_t* C = static_cast<uint16_t*>(p.C);
  const int k = tid % (TN / 8), col = n0 + k * 8;           // fixed 16-byte column per thread
  if (col < p.N) {
    for (int r = tid / (TN / 8); r < nrows; r += kThreads / (TN / 8)) {
      const uint4 v = *reinterpret_cast<const uint4*>(lds + r * RB + ((k ^ (r & 15)) << 4));
      if constexpr (EPI == EPI_DOWN_MERGE) {
        uint16_t* d = m_dst[r];
        if (d != nullptr) {
          const float g = m_g[r];
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
          uint32_t o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = pack_bf16x2(fmaf(g, __uint_as_float(w[q] << 16), 0.0f),
                               fmaf(g, __uint_as_float(w[q] & 0xffff0000u), 0.0f));
          // the token's row is read by no later kernel of the layer: streaming store
          st_nt(reinterpret_cast<uint4*>(d + col), make_uint4(o[0], o[1], o[2], o[3]));
          continue;
        }
      }
      *reinterpret_cast<uint4*>(C + c_row_of(r) * p.N + col) = v;
    }
  }
}

// A half-width tail tile (columns [n0, n0 + 128) of its column tile): the y
// store only (such tiles are never split into pieces).
template <int EPI>
__device__ __forceinline__ void tile_finish_half(const GemmParams& p, const TileJob& job,
                                                 f32x16_t (&acc)[4][2], uint8_t* __restrict__ lds,
                                                 const MergeRow& mr) {
  static_assert(EPI == EPI_STORE_BF16 || EPI == EPI_DOWN_MERGE, "half-width tiles store y only");
  const int n0 = job.ntile * BN + (job.half - 1) * (BN / 2);
  auto vals = [&](const int mi, float4 (&tv)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      tv[u] = make_float4(acc[mi][u >> 2][4 * (u & 3)], acc[mi][u >> 2][4 * (u & 3) + 1],
                          acc[mi][u >> 2][4 * (u & 3) + 2], acc[mi][u >> 2][4 * (u & 3) + 3]);
  };
  store_y<EPI, BN / 2>(p, job, n0, vals, lds, mr);
}

// After the main loop (LDS free, every load landed): the K-split exchange of
// a piece and the epilogue.  acc holds the wave's 128 x 128 block: element q of
// tile (mi, ni) is token row 32 mi + lane % 32, output column 32 ni + 8 (q / 4)
// + 4 (lane / 32) + q % 4.  Shared by every operand format.
template <int EPI>
__device__ __forceinline__ void tile_finish(const GemmParams& p, const TileJob& job,
                                            f32x16_t (&acc)[4][4], uint8_t* __restrict__ lds,
                                            const MergeRow& mr) {
  const int row0 = job.row0, nrows = job.nrows, ntile = job.ntile;
  const int tid = threadIdx.x, lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;
  constexpr bool swiglu = epi_swiglu<EPI>();
  const int n0 = ntile * (swiglu ? BN / 2 : BN);
  const int frag_row = lane & 31;
  const int khalf = lane >> 5;
  // ---- split tiles.  Every piece stores its fp32 sums in its slot (float4 i
  // of thread tid at slot + i * kThreads + tid: each instruction covers 4 KiB
  // of contiguous memory) and counts itself in; the piece that arrives last
  // adds the slots of all pieces in piece order and runs the epilogue.  No
  // workgroup ever waits for another.
  if (job.role == kPiece) {
    float4* dst = reinterpret_cast<float4*>(p.part) + static_cast<int64_t>(job.slot) * (BM * BN / 4) + tid;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          dst[((mi * 4 + ni) * 4 + g) * kThreads] =
              make_float4(acc[mi][ni][4 * g], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]);
    }
    // publish: each wave waits until its stores have reached L2 (a workgroup
    // fence would not wait for them), then the release half of thread 0's add
    // writes the L2 back; the acquire half, taken by the last piece, makes
    // the other pieces' slots visible to it
    wait_vm<0>();
    __syncthreads();
    int32_t* flag = reinterpret_cast<int32_t*>(lds);
    if (tid == 0) {
      const int32_t before = __hip_atomic_fetch_add(job.cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const int32_t last = before == job.npieces - 1;
      if (last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(job.cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next launch
      }
      *flag = last;
    }
    __syncthreads();
    const bool last = *flag != 0;
    __syncthreads();                                         // the epilogue overwrites the flag
    if (!last) return;
  }
  // Accumulator values of fragment row group mi, as 16 float4 (u = 4 ni + g:
  // columns 8 g .. 8 g + 3 of tile (mi, ni)): the registers of a whole tile,
  // or for a split one the sum over its pieces' slots, in piece order, loaded
  // right before the epilogue consumes them.
  const float4* red = reinterpret_cast<const float4*>(p.part) +
                      static_cast<int64_t>(job.slot0) * (BM * BN / 4) + tid;
  const bool split = job.role == kPiece;
  auto tile_vals = [&](const int mi, float4 (&tv)[16]) {
    if (split) {
#pragma unroll
      for (int u = 0; u < 16; ++u) tv[u] = red[(mi * 16 + u) * kThreads];
      for (int q = 1; q < job.npieces; ++q) {
        const float4* rq = red + static_cast<int64_t>(q) * (BM * BN / 4);
        float4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = rq[(mi * 16 + u) * kThreads];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          tv[u].x += v[u].x; tv[u].y += v[u].y; tv[u].z += v[u].z; tv[u].w += v[u].w;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 16; ++u)
        tv[u] = make_float4(acc[mi][u >> 2][4 * (u & 3)], acc[mi][u >> 2][4 * (u & 3) + 1],
                            acc[mi][u >> 2][4 * (u & 3) + 2], acc[mi][u >> 2][4 * (u & 3) + 3]);
    }
  };

  // ---- epilogue, staged through LDS for 16-byte global stores.
  // The MFMA is fed (weights, tokens), i.e. it computes the tile transposed:
  // accumulator element q of tile (mi, ni) is token row 32mi + lane%32 and
  // output column 32ni + 8(q/4) + 4(lane/32) + q%4 of the wave's 128 x 128
  // block, so each lane holds 4 consecutive columns of one row and writes
  // them to LDS with one 8-byte (bf16) or 16-byte (fp32) store.  Staged rows
  // keep their 16-byte chunk k at k ^ (row % 16): the writes of 16 rows and
  // the row-wise reads back are both free of bank conflicts.
  const CRows c_row_of(p, row0);
  const int erow = 128 * wm + frag_row;                  // + 32 mi
  if (EPI == EPI_STORE_GU) {
    // gate column i pairs with up column i in tile (mi, ni + 2), as in the
    // SwiGLU epilogue; both go out as bf16, 4 columns per 8-byte store
    uint16_t* C = static_cast<uint16_t*>(p.C);
    const int64_t N2 = 2 * static_cast<int64_t>(p.N);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = erow + 32 * mi;
      float4 tv[16];
      tile_vals(mi, tv);
      if (r >= nrows) continue;
      uint16_t* hrow = C + c_row_of(r) * N2;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + 64 * wn + 32 * ni + 8 * g + 4 * khalf;
          if (col >= p.N) continue;
          const float4 g4 = tv[4 * ni + g], u4 = tv[4 * (ni + 2) + g];
          *reinterpret_cast<uint2*>(hrow + col) = make_uint2(pack_bf16x2(g4.x, g4.y), pack_bf16x2(g4.z, g4.w));
          *reinterpret_cast<uint2*>(hrow + p.N + col) = make_uint2(pack_bf16x2(u4.x, u4.y), pack_bf16x2(u4.z, u4.w));
        }
    }
  } else if (EPI == EPI_SWIGLU_BWD || EPI == EPI_SWIGLU_BWD_MX) {
    // da of 4 consecutive columns per lane and (mi, ni, g); with g, u of the
    // same (row, i) from H_src: dg = da u SiLU'(g), du = da SiLU(g), where
    // SiLU(g) = g s, SiLU'(g) = s (1 + g (1 - s)), s = 1 / (1 + e^-g).  dh is
    // column-blocked (the next GEMM's token operand), 2 N wide.
    // MXFP8: the 32 columns of (mi, ni) are one block of dg and one of du (N
    // a multiple of 32); lane l holds 16 of them (4 columns at 8 g + 4 (l /
    // 32)) and lane l ^ 32 the other 16, so the block amax takes one
    // shuffle; two more swap code words so that each lane stores 16
    // consecutive codes.  Lanes l and l ^ 32 share the row and the block, so
    // the skips below never split a pair.
    constexpr bool MXO = EPI == EPI_SWIGLU_BWD_MX;
    uint8_t* C = static_cast<uint8_t*>(p.C);
    const int64_t N2 = 2 * static_cast<int64_t>(p.N);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = erow + 32 * mi;
      float4 tv[16];
      tile_vals(mi, tv);
      if (r >= nrows) continue;
      const int64_t crow = c_row_of(r);
      const uint16_t* hrow = p.H_src + crow * N2;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int cb = n0 + 128 * wn + 32 * ni;              // first column of the block
        if (cb >= p.N) continue;
        float dg[4][4], du[4][4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = cb + 8 * g + 4 * khalf;
          const uint2 gb = *reinterpret_cast<const uint2*>(hrow + col);
          const uint2 ub = *reinterpret_cast<const uint2*>(hrow + p.N + col);
          const float gv[4] = {__uint_as_float(gb.x << 16), __uint_as_float(gb.x & 0xffff0000u),
                               __uint_as_float(gb.y << 16), __uint_as_float(gb.y & 0xffff0000u)};
          const float uv[4] = {__uint_as_float(ub.x << 16), __uint_as_float(ub.x & 0xffff0000u),
                               __uint_as_float(ub.y << 16), __uint_as_float(ub.y & 0xffff0000u)};
          const float4 t = tv[4 * ni + g];
          const float da[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[q]));
            du[g][q] = da[q] * gv[q] * sg;
            dg[g][q] = da[q] * uv[q] * sg * (1.0f + gv[q] * (1.0f - sg));
          }
          if (!MXO) {
            *reinterpret_cast<uint2*>(C + colblk_byte(crow, p.c_rows, 2 * col)) =
                make_uint2(pack_bf16x2(dg[g][0], dg[g][1]), pack_bf16x2(dg[g][2], dg[g][3]));
            *reinterpret_cast<uint2*>(C + colblk_byte(crow, p.c_rows, 2 * (p.N + col))) =
                make_uint2(pack_bf16x2(du[g][0], du[g][1]), pack_bf16x2(du[g][2], du[g][3]));
          }
        }
        if (MXO) {
          float mg = 0.0f, mu = 0.0f;
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) { mg = fmaxf(mg, fabsf(dg[g][q])); mu = fmaxf(mu, fabsf(du[g][q])); }
          mg = fmaxf(mg, __shfl_xor(mg, 32));
          mu = fmaxf(mu, __shfl_xor(mu, 32));
          const int Eg = mx_scale_exp(mg), Eu = mx_scale_exp(mu);
          uint32_t cg[4], cu[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            cg[g] = e4m3_code_scaled(dg[g][0], Eg) | (e4m3_code_scaled(dg[g][1], Eg) << 8) |
                    (e4m3_code_scaled(dg[g][2], Eg) << 16) | (e4m3_code_scaled(dg[g][3], Eg) << 24);
            cu[g] = e4m3_code_scaled(du[g][0], Eu) | (e4m3_code_scaled(du[g][1], Eu) << 8) |
                    (e4m3_code_scaled(du[g][2], Eu) << 16) | (e4m3_code_scaled(du[g][3], Eu) << 24);
          }
          // half 0 keeps columns 0-3 and 8-11 and takes 4-7 and 12-15; half 1
          // keeps 20-23 and 28-31 and takes 16-19 and 24-27
          const uint32_t xg0 = __shfl_xor(khalf ? cg[0] : cg[2], 32);
          const uint32_t xg1 = __shfl_xor(khalf ? cg[1] : cg[3], 32);
          const uint32_t xu0 = __shfl_xor(khalf ? cu[0] : cu[2], 32);
          const uint32_t xu1 = __shfl_xor(khalf ? cu[1] : cu[3], 32);
          const uint4 og = khalf ? make_uint4(xg0, cg[2], xg1, cg[3]) : make_uint4(cg[0], xg0, cg[1], xg1);
          const uint4 ou = khalf ? make_uint4(xu0, cu[2], xu1, cu[3]) : make_uint4(cu[0], xu0, cu[1], xu1);
          *reinterpret_cast<uint4*>(C + colblk_byte(crow, p.c_rows, cb + 16 * khalf)) = og;
          *reinterpret_cast<uint4*>(C + colblk_byte(crow, p.c_rows, p.N + cb + 16 * khalf)) = ou;
          if (khalf == 0) {
            p.C_scales[scale_byte(crow, p.c_rows, cb / 32)] = static_cast<uint8_t>(Eg + 127);
            p.C_scales[scale_byte(crow, p.c_rows, (p.N + cb) / 32)] = static_cast<uint8_t>(Eu + 127);
          }
        }
      }
    }
  } else if (EPI == EPI_STORE_BF16 || EPI == EPI_DOWN_MERGE) {
    store_y<EPI, BN>(p, job, n0, tile_vals, lds, mr);
  } else {
    // SwiGLU: gate column i pairs with up column i in tile (mi, ni + 2).
    // SiLU(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal.
    constexpr bool MXO = EPI == EPI_SWIGLU_MX || EPI == EPI_SWIGLU_MX_H;
    constexpr int RB = MXO ? (BN / 2) * 4 : (BN / 2) * 2;  // staged row: 128 fp32 or bf16
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = erow + 32 * mi;
      float4 tv[16];
      tile_vals(mi, tv);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 g4 = tv[4 * ni + g], u4 = tv[4 * (ni + 2) + g];
          const float gvs[4] = {g4.x, g4.y, g4.z, g4.w}, uvs[4] = {u4.x, u4.y, u4.z, u4.w};
          float a[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gv = gvs[j], uv = uvs[j];
            a[j] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          }
          const int i = 64 * wn + 32 * ni + 8 * g + 4 * khalf;
          if constexpr (EPI == EPI_SWIGLU_BF16_H || EPI == EPI_SWIGLU_MX_H) {  // h kept for the backward
            if (r < nrows && n0 + i < p.N) {
              uint16_t* hrow = p.H_out + c_row_of(r) * (2 * static_cast<int64_t>(p.N));
              *reinterpret_cast<uint2*>(hrow + n0 + i) =
                  make_uint2(pack_bf16x2(g4.x, g4.y), pack_bf16x2(g4.z, g4.w));
              *reinterpret_cast<uint2*>(hrow + p.N + n0 + i) =
                  make_uint2(pack_bf16x2(u4.x, u4.y), pack_bf16x2(u4.z, u4.w));
            }
          }
          if (MXO) {
            *reinterpret_cast<float4*>(lds + r * RB + (((i >> 2) ^ (r & 15)) << 4)) =
                make_float4(a[0], a[1], a[2], a[3]);
          } else {
            *reinterpret_cast<uint2*>(lds + r * RB + (((i >> 3) ^ (r & 15)) << 4) + ((i >> 2) & 1) * 8) =
                make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
          }
        }
    }
    __syncthreads();
    // act is column-blocked (the down GEMM's token operand): 64-byte block
    // b of act row c at byte (b * c_rows + c) * 64
    if (!MXO) {
      uint8_t* C = static_cast<uint8_t*>(p.C);
      const int k = tid & 15, col = n0 + k * 8;             // fixed 16-byte column per thread
      if (col < p.N) {
        for (int r = tid >> 4; r < nrows; r += kThreads / 16) {
          const int64_t crow = c_row_of(r);
          *reinterpret_cast<uint4*>(C + colblk_byte(crow, p.c_rows, 2 * col)) =
              *reinterpret_cast<const uint4*>(lds + r * RB + ((k ^ (r & 15)) << 4));
        }
      }
    } else {
      uint8_t* C = static_cast<uint8_t*>(p.C);
      const int b = tid & 3, col = n0 + b * 32;               // fixed 32-column block per thread
      for (int r = tid >> 2; r < nrows && col < p.N; r += kThreads / 4) {
        float v[32];
#pragma unroll
        for (int c4 = 0; c4 < 8; ++c4) {
          const float4 f = *reinterpret_cast<const float4*>(lds + r * RB + (((8 * b + c4) ^ (r & 15)) << 4));
          v[4 * c4] = f.x; v[4 * c4 + 1] = f.y; v[4 * c4 + 2] = f.z; v[4 * c4 + 3] = f.w;
        }
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
        const int E = mx_scale_exp(amax);
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          w[q] = e4m3_code_scaled(v[4 * q], E) | (e4m3_code_scaled(v[4 * q + 1], E) << 8) |
                 (e4m3_code_scaled(v[4 * q + 2], E) << 16) | (e4m3_code_scaled(v[4 * q + 3], E) << 24);
        const int64_t crow = c_row_of(r);
        uint4* d = reinterpret_cast<uint4*>(C + colblk_byte(crow, p.c_rows, col));
        d[0] = make_uint4(w[0], w[1], w[2], w[3]);
        d[1] = make_uint4(w[4], w[5], w[6], w[7]);
        p.C_scales[scale_byte(crow, p.c_rows, col / 32)] = static_cast<uint8_t>(E + 127);
      }
    }
  }
}

// One 256-row x (256 | 128 SwiGLU) output tile of expert e, rows
// [row0, row0 + nrows) of the window, column tile `ntile`.  Called by all 256
// threads of a workgroup; `lds` is the workgroup's LDS (Geo<A_MX>::LDS bytes).
// Starts with a barrier, so it can be called back to back on the same LDS.
// TN = 128: a half-width tail tile (job.half), the y-storing epilogues only.
template <bool A_MX, int EPI, int TN = BN>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const TileJob& job,
                                          uint8_t* __restrict__ lds) {
  using G = Geo<A_MX>;
  constexpr int BK = G::BK, NS = G::NS;
  static_assert(TN == BN || (TN == BN / 2 && (EPI == EPI_STORE_BF16 || EPI == EPI_DOWN_MERGE)),
                "half-width tiles store y only");
  constexpr int NB = TN / 64;                   // 32-column fragments per wave
  constexpr int NLB = G::NLOAD_B * TN / BN;     // weight loads per stage and thread
  // first weight row of a half-width tile within its column tile
  const int hrow = TN == BN ? 0 : (job.half - 1) * TN;
  __syncthreads();
  const int e = job.e, row0 = job.row0, nrows = job.nrows, ntile = job.ntile;
  // the wave index is uniform: in an SGPR the LDS destinations of the direct
  // loads (M0) are scalar arithmetic, with no v_readfirstlane per load
  const int tid = threadIdx.x, lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;
  constexpr bool swiglu = epi_swiglu<EPI>();
  const int K = p.K;
  const int nk_all = K / BK;
  // k-steps of this job: the operand bases below start at k-step kt0
  const int kt0 = job.kt0;
  const int nk = job.nkt > 0 ? job.nkt : nk_all;

  // ---- operand tiles.  A wave load instruction fills 1 KiB of LDS: lane l
  // lands at physical chunk l % CPR of row l / CPR of that KiB, so it fetches
  // the logical chunk (l % CPR) ^ key(row).  Thread rows: tid / CPR + RSTEP * j
  // (the key repeats every 16 rows and RSTEP is a multiple of 16).
  // Weights: load j of k-step kt reads Wbase + kt * wkstride + boff[j].
  //   documented layout: the thread's row and swizzled chunk of expert e;
  //   packed layout: the tile's blocks are stored in LDS-image order, so a
  //   wave instruction reads 1 KiB of contiguous memory.
  const uint16_t* Wbase;
  int32_t wkstride;
  // (fixed-size arrays: a template-dependent bound here made the host pass
  // drop the kernel's launch stub)
  uint32_t boff[8];
  if (p.w_packed) {
    Wbase = p.W + ((static_cast<int64_t>(e) * p.n_tiles + ntile) * nk_all + kt0) * (BM * BK);
    wkstride = BM * BK;
    // (the LDS image is row-major: a half's rows are one contiguous half of it)
#pragma unroll
    for (int j = 0; j < NLB; ++j) boff[j] = (4 * j + wave) * 512 + lane * 8 + hrow * BK;
  } else {
    Wbase = p.W + static_cast<int64_t>(e) * p.w_expert_stride + kt0 * BK;
    wkstride = BK;
    const int lrowB = tid / G::CPR_B;
    const int lchunkB = (lane % G::CPR_B) ^ chunk_key<G::CPR_B>(lrowB);
#pragma unroll
    for (int j = 0; j < NLB; ++j)
      boff[j] = static_cast<uint32_t>(w_row_of(hrow + lrowB + G::RSTEP_B * j, ntile, swiglu, p.I, p.N)) *
                    static_cast<uint32_t>(K) + lchunkB * 8;
  }
  // A rows (slots) -> ring rows, tail rows clamped to the last valid one.
  // The A buffer is column-blocked (a k-step of either format is one 64-byte
  // block per row, block-major): load j of k-step kt reads byte aoff[j] +
  // kt * a_kstep, and the tile's rows of a k-step are contiguous memory.
  const ARows a_ring_row(p, row0, nrows);
  const uint32_t a_kstep = static_cast<uint32_t>(p.a_rows) * kColBlock;
  const int lrowA = tid / G::CPR_A;
  const int lchunkA = (lane % G::CPR_A) ^ chunk_key<G::CPR_A>(lrowA);
  uint32_t aoff[8];                                           // byte offsets
#pragma unroll
  for (int j = 0; j < G::NLOAD_A; ++j)
    aoff[j] = a_ring_row(lrowA + G::RSTEP_A * j) * kColBlock + lchunkA * 16 +
              static_cast<uint32_t>(kt0) * a_kstep;
  // E4M3 A: thread tid fetches the scale pair of row tid for each k-step
  // (pairs are block-major too: k-step kt's pairs are a_rows * 2 bytes apart)
  const uint32_t soff = A_MX ? a_ring_row(tid) * 2u + static_cast<uint32_t>(kt0) * p.a_rows * 2u : 0;
  // Raw buffer descriptors over the operands (byte extents below 4 GiB, which
  // the launchers check); a load past an extent reads zero.
  auto extent = [](int64_t bytes) -> int32_t {
    return static_cast<int32_t>(bytes < 0xffffffffll ? bytes : 0xffffffffll);
  };
  const int64_t w_left = p.w_packed
      ? static_cast<int64_t>(nk_all - kt0) * (BM * BK) * 2
      : (p.w_expert_stride - static_cast<int64_t>(kt0) * BK) * 2;
  const __amdgpu_buffer_rsrc_t rW =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Wbase), 0, extent(w_left), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.A), 0, extent(static_cast<int64_t>(p.a_rows) * K * (A_MX ? 1 : 2)), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.A_scales), 0, extent(A_MX ? static_cast<int64_t>(p.a_rows) * (K / 32) : 0),
      kRsrcWord3);

  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  auto tileA = [&](int buf) { return lds + buf * G::STAGEB; };
  auto tileB = [&](int buf) { return lds + buf * G::STAGEB + G::TILE_A; };
  auto tileS = [&](int buf) { return lds + buf * G::STAGEB + G::TILE_A + G::TILE_B; };

  // (zeroed after the prologue's loads are issued: 256 accumulator writes
  // per lane would otherwise sit in front of them)
  f32x16_t acc[4][NB];

  const int frag_row = lane & 31;
  const int khalf = lane >> 5;

  // Buffer loads: a per-lane byte offset that is fixed for the tile (VGPR)
  // plus a per-k-step offset (SGPR), so no address arithmetic per load.
  // Weights are loaded with the non-temporal policy (aux bit 1): each is read
  // by one XCD's tiles in a short span, and streaming them this way keeps the
  // caches for the token operands and y (the layer step 6 us faster).
#define MOK_LD_W(j, kt, dst)                                                                 \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_ptr_t)(dst), 16, boff[j] * 2u,            \
                                           static_cast<uint32_t>(kt) * wkstride * 2u, 0, 2)
#define MOK_LD_A(j, kt, dst)                                                                 \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(dst), 16, aoff[j],                 \
                                           static_cast<uint32_t>(kt) * a_kstep, 0, 0)
  // The two halves of a stage's direct loads: weights; tokens (+ E4M3 scales,
  // 2 bytes per lane, which land in 4-byte slots: lane i at slot base + 4 i).
#define MOK_ISSUE_W(kt, buf)                                                                 \
  do {                                                                                       \
    uint8_t* Bs_ = tileB(buf);                                                               \
    _Pragma("unroll") for (int j = 0; j < NLB; ++j)                                          \
      MOK_LD_W(j, kt, Bs_ + (4 * j + wave) * 1024);                                          \
  } while (0)
#define MOK_ISSUE_A(kt, buf)                                                                 \
  do {                                                                                       \
    uint8_t* As_ = tileA(buf);                                                               \
    if (A_MX) {                                                                              \
      _Pragma("unroll") for (int j = 0; j < G::NLOAD_A; ++j)                                 \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(As_ + (4 * j + wave) * 1024), \
                                                 16, aoff[j], static_cast<uint32_t>(kt) * a_kstep, 0, 0); \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_ptr_t)(tileS(buf) + wave * 256), 2, soff, \
                                               static_cast<uint32_t>(kt) * p.a_rows * 2u, 0, 0); \
    } else {                                                                                 \
      _Pragma("unroll") for (int j = 0; j < G::NLOAD_A; ++j)                                 \
        MOK_LD_A(j, kt, As_ + (4 * j + wave) * 1024);                                        \
    }                                                                                        \
  } while (0)

  // Fragments.  v_mfma_f32_32x32x16_bf16: lane l feeds row l % 32 with 8
  // consecutive k.  bf16 A: slice ks of a k-step takes k-chunk 2 ks + l / 32 of
  // both operands.  E4M3 A: the k order inside a k-step of 64 is permuted the
  // same way for both operands -- slice ks of lane half h takes k 32 h + 8 ks
  // .. +7 -- so one 16-byte code chunk holds a lane's k of two slices and one
  // E8M0 block scale (block h of the step) covers all four: per k-step a lane
  // reads two code chunks and one scale per A fragment row, and converts each
  // slice right before it is used (v_cvt_scalef32_pk_bf16_fp8: exact
  // bf16 rounding of code x 2^E).
  bf16x8_t af[2][4], bfr[2][NB];
  uint4 araw[4][2];
  float ascale[4];
#define MOK_FRAGS_B(dst, pb, ks_)                                                            \
  do {                                                                                       \
    const int kc_ = A_MX ? 4 * khalf + (ks_) : 2 * (ks_) + khalf;                            \
    _Pragma("unroll") for (int ni = 0; ni < NB; ++ni)                                        \
      bfr[dst][ni] = *reinterpret_cast<const bf16x8_t*>((pb) + G::offB((TN / 2) * wn + 32 * ni + frag_row, kc_)); \
  } while (0)
#define MOK_FRAGS(dst, pa, pb, ks_)                                                          \
  do {                                                                                       \
    if (A_MX) {                                                                              \
      MOK_CVT(dst, ks_);                                                                     \
    } else {                                                                                 \
      const int kc_ = 2 * (ks_) + khalf;                                                     \
      _Pragma("unroll") for (int mi = 0; mi < 4; ++mi)                                       \
        af[dst][mi] = *reinterpret_cast<const bf16x8_t*>((pa) + G::offA(128 * wm + 32 * mi + frag_row, kc_)); \
    }                                                                                        \
    MOK_FRAGS_B(dst, pb, ks_);                                                               \
  } while (0)
  // E4M3 A: the raw code chunks and scales of a whole k-step
#define MOK_RAW_A(pa, ps)                                                                    \
  do {                                                                                       \
    _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) {                                       \
      const int r_ = 128 * wm + 32 * mi + frag_row;                                          \
      araw[mi][0] = lds_read16((pa) + G::offA(r_, 2 * khalf));                               \
      araw[mi][1] = lds_read16((pa) + G::offA(r_, 2 * khalf + 1));                           \
      const uint32_t e_ = (ps)[r_ * 4 + khalf];                                              \
      ascale[mi] = __uint_as_float(e_ ? e_ << 23 : 0x00400000u);                             \
    }                                                                                        \
  } while (0)
#define MOK_CVT(dst, ks_)                                                                    \
  do {                                                                                       \
    _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) {                                       \
      const uint4 c_ = araw[mi][(ks_) >> 1];                                                 \
      const uint32_t w0_ = ((ks_) & 1) ? c_.z : c_.x, w1_ = ((ks_) & 1) ? c_.w : c_.y;        \
      const bf16x2_t p0_ = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0_, ascale[mi], false); \
      const bf16x2_t p1_ = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0_, ascale[mi], true);  \
      const bf16x2_t p2_ = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1_, ascale[mi], false); \
      const bf16x2_t p3_ = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1_, ascale[mi], true);  \
      af[dst][mi] = bf16x8_t{p0_[0], p0_[1], p1_[0], p1_[1], p2_[0], p2_[1], p3_[0], p3_[1]}; \
    }                                                                                        \
  } while (0)
  // first fragments of a k-step (E4M3: raw codes + scales; slice 0 converted later)
#define MOK_FRAGS0(pa, pb, ps)                                                               \
  do {                                                                                       \
    if (A_MX) {                                                                              \
      MOK_RAW_A(pa, ps);                                                                     \
      MOK_FRAGS_B(0, pb, 0);                                                                 \
    } else {                                                                                 \
      MOK_FRAGS(0, pa, pb, 0);                                                               \
    }                                                                                        \
  } while (0)
#define MOK_MMA(src)                                                                         \
  do {                                                                                       \
    _Pragma("unroll") for (int mi = 0; mi < 4; ++mi)                                         \
      _Pragma("unroll") for (int ni = 0; ni < NB; ++ni)                                      \
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[src][ni], af[src][mi], acc[mi][ni], 0, 0, 0); \
  } while (0)

  // Pipeline.  Stage s lives in LDS buffer s % NS.  In k-step kt the barrier
  // sits after every wave holds its last fragments of kt and before their
  // MFMAs: then buffer kt % NS is free for stage kt + NS, and the first
  // fragments of kt + 1 are read while the last MFMAs of kt run.  Before that
  // barrier a thread waits until its loads of stage kt + 1 have landed: the
  // NS - 2 newer stages may still fly.
  // A stage's loads are issued in two halves, so no phase of a k-step issues
  // them in one burst (a burst from all four waves right after the barrier
  // filled the load queues and stalled the MFMA stream behind it): the weight
  // half of stage kt + NS after the barrier of kt, the token half before the
  // barrier of kt + 1.  The prologue issues stages 0 .. NS-2 and the weight
  // half of NS-1, so every k-step has the same shape.  Past the end, loads are
  // clamped re-loads of the last stage into buffers nobody reads again, which
  // keeps the per-thread load count -- and so the vmcnt bookkeeping -- the
  // same in every step.
  constexpr int LW = NLB, LA = G::NLOAD_A + (A_MX ? 1 : 0), LPS = LW + LA;
  // EPI_DOWN_MERGE: the plan record of this thread's row is loaded before the
  // prologue's loads (it only makes the first waits below stricter)
  MergeRow mr;
  if constexpr (EPI == EPI_DOWN_MERGE) merge_row_load(p, job.row0, job.nrows, mr);
#pragma unroll
  for (int s0 = 0; s0 < NS; ++s0) {
    const int ks0 = s0 < nk ? s0 : nk - 1;
    MOK_ISSUE_W(ks0, s0);
    if (s0 + 1 < NS) MOK_ISSUE_A(ks0, s0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  wait_vm<(NS - 2) * LPS + LW>();                            // stage 0 landed
  __syncthreads();

  MOK_FRAGS0(tileA(0), tileB(0), tileS(0));
  constexpr int KS = BK / 16;                                // k-slices per k-step
  int buf = 0;
  // Steady state: every k-step but the last, with no branch in the body, so
  // the wait counters stay exact.  Two phases per k-step, pinned with
  // scheduling barriers (the compiler otherwise moves MFMAs, which touch no
  // memory, across the workgroup barrier and leaves LDS latency exposed):
  //   A: MFMAs of slices 0 .. KS-2, with the fragment reads of the next slices
  //      and then the token half of a stage's loads interleaved one per MFMA;
  //   barrier (stage kt+1 landed everywhere; buffer kt % NS free);
  //   B: MFMAs of the last slice, with the fragment reads of step kt+1 and
  //      then the weight half of stage kt+NS interleaved the same way.
  constexpr int MPS = 4 * NB;                                // MFMAs per k-slice
  constexpr int kReadsA = A_MX ? NB * (KS - 1) : (4 + NB) * (KS - 1);  // fragment reads in phase A
  constexpr int kReadsB = A_MX ? NB + 12 : 4 + NB;           // E4M3: NB B + 8 codes + 4 scales
  constexpr int kMA = MPS * (KS - 1);                        // MFMAs in phase A
  constexpr int kRA1 = kReadsA < kMA ? kReadsA : kMA;        // reads paired one per MFMA
  constexpr int kVA = kMA - kRA1 < LA ? kMA - kRA1 : LA;     // loads paired after them
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const uint8_t* As = tileA(buf);
    const uint8_t* Bs = tileB(buf);
    const int nbuf = buf + 1 == NS ? 0 : buf + 1;
    if (A_MX) MOK_CVT(0, 0);
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      MOK_FRAGS((ks + 1) & 1, As, Bs, ks + 1);
      MOK_MMA(ks & 1);
    }
    {                                                        // token half of stage kt-1+NS
      const int kp = kt - 1 + NS < nk ? kt - 1 + NS : nk - 1;
      MOK_ISSUE_A(kp, buf == 0 ? NS - 1 : buf - 1);
    }
#pragma unroll
    for (int i = 0; i < kRA1; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // one fragment read
    }
#pragma unroll
    for (int i = 0; i < kVA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // one global -> LDS load
    }
    if (kMA - kRA1 - kVA > 0) __builtin_amdgcn_sched_group_barrier(0x008, kMA - kRA1 - kVA, 0);
    if (kReadsA - kRA1 > 0) __builtin_amdgcn_sched_group_barrier(0x100, kReadsA - kRA1, 0);
    if (LA - kVA > 0) __builtin_amdgcn_sched_group_barrier(0x020, LA - kVA, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<(NS - 2) * LPS>();                               // stage kt+1 landed
    // Barrier without a fence: a workgroup fence here would wait for every
    // direct-to-LDS load in flight (vmcnt(0)), the newest stages included.
    // Each wave's own loads of stage kt+1 are covered by the wait above, and
    // its fragment reads of buffer buf by lgkmcnt(0), before buf is refilled.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const int kn = kt + NS < nk ? kt + NS : nk - 1;
    MOK_FRAGS0(tileA(nbuf), tileB(nbuf), tileS(nbuf));
    MOK_ISSUE_W(kn, buf);                                    // weight half of stage kt+NS
    MOK_MMA((KS - 1) & 1);
    constexpr int kRB1 = kReadsB < MPS ? kReadsB : MPS;      // reads paired one per MFMA
    constexpr int kVB = MPS - kRB1 < LW ? MPS - kRB1 : LW;   // loads paired after them
#pragma unroll
    for (int i = 0; i < kRB1; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // one fragment read
    }
#pragma unroll
    for (int i = 0; i < kVB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // one global -> LDS load
    }
    if (MPS - kRB1 - kVB > 0) __builtin_amdgcn_sched_group_barrier(0x008, MPS - kRB1 - kVB, 0);
    if (kReadsB - kRB1 > 0) __builtin_amdgcn_sched_group_barrier(0x100, kReadsB - kRB1, 0);
    if (LW - kVB > 0) __builtin_amdgcn_sched_group_barrier(0x020, LW - kVB, 0);
    __builtin_amdgcn_sched_barrier(0);
    buf = nbuf;
  }
  {                                                          // last k-step
    const uint8_t* As = tileA(buf);
    const uint8_t* Bs = tileB(buf);
    if (A_MX) MOK_CVT(0, 0);
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      MOK_FRAGS((ks + 1) & 1, As, Bs, ks + 1);
      MOK_MMA(ks & 1);
    }
    MOK_MMA((KS - 1) & 1);
  }
#undef MOK_ISSUE_W
#undef MOK_ISSUE_A
#undef MOK_LD_W
#undef MOK_LD_A
#undef MOK_FRAGS_B
#undef MOK_FRAGS
#undef MOK_RAW_A
#undef MOK_CVT
#undef MOK_FRAGS0
#undef MOK_MMA
  wait_vm<0>();                                              // clamped tail loads still land in LDS
  __syncthreads();                                           // LDS is reused by the epilogue

  if constexpr (TN == BN) {
    tile_finish<EPI>(p, job, acc, lds, mr);
  } else {
    tile_finish_half<EPI>(p, job, acc, lds, mr);
  }
}

// A whole tile (all k-steps).
template <bool A_MX, int EPI>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int e, int row0, int nrows, int ntile,
                                          uint8_t* __restrict__ lds) {
  TileJob j;
  j.e = e; j.row0 = row0; j.nrows = nrows; j.ntile = ntile;
  j.kt0 = 0; j.nkt = 0; j.role = kWhole; j.slot = 0; j.slot0 = 0; j.npieces = 0; j.cnt = nullptr;
  j.half = 0;
  gemm_tile<A_MX, EPI>(p, j, lds);
}

}  // namespace gemm
}  // namespace mok
