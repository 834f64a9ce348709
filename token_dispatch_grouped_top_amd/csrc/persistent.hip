// persistent.hip -- the fused layer as one cooperative kernel.
//
// tahou.com MoK article, megakernel paragraph: the GPU's compute units are
// split into a group that moves tokens (dispatch, combine, bookkeeping) and a
// group that runs the expert FFN; each side tells the other through local
// counters when a batch of tokens is ready or done.  Minibatch paragraph: a
// minibatch (window) is what the FFN side gets at once.  Ring-buffer
// paragraph: tokens land in a fixed buffer that is reused as soon as the
// expert computation has consumed them, and the next macrobatch's dispatch
// overlaps the previous one's combine; state-machine paragraph: the GPU, not
// the CPU, decides what runs next.  PyTorchKR wiki summary, key point on the
// SM split: the two groups signal through local counters.
//
// Shape on MI355X:
//   - one 256-thread workgroup per CU (160 KiB LDS), launched cooperatively so
//     all are resident; workgroups 0 .. n_move-1 are movers (ids are dealt to
//     the 8 XCDs round-robin, so a multiple of 8 spreads them evenly), the rest
//     are MFMA workers;
//   - windows are numbered across macrobatches; window w uses ring half w % 2
//     (rows (w % 2) * M + s - s0) and the same half of the activation buffer;
//   - movers walk an item list: gather window w (after the gate/up tiles of
//     window w - 2 freed the ring half), and merge macrobatch m (after every
//     down tile of m); merges of m are placed after the second window of m + 1
//     so they run while the workers compute m + 1;
//   - workers take tiles from a per-XCD queue over the sequence
//     G1(0), G1(1), G2(0), G1(2), G2(1), ..., G2(W-1) (G1 = gate/up + SwiGLU,
//     G2 = down); each XCD owns a contiguous eighth of every window's tiles so
//     an expert's operands stay in one L2.  A G1 tile waits for its window's
//     gather and for the G2 tiles of w - 2 (activation half); a G2 tile waits
//     for all G1 tiles of its window and for the merge of macrobatch m - 2
//     (return area m % 2).
//   - every dependency points at earlier items of the same sequences, so the
//     waits cannot cycle; every wait is bounded by a timeout after which the
//     kernel sets MOK_ERR_DEVICE, raises an abort flag seen by all waits, and
//     every workgroup returns.
// Counters live in the workspace and are cleared by a fill kernel before the
// plan kernel.  Each XCD has its own L2, so an agent-scope release writes the
// XCD's dirty L2 lines back and an agent-scope acquire invalidates the XCD's
// L2: both are paid once per signal / satisfied wait, never per poll.  A
// producer workgroup publishes with a barrier and one release add by thread 0;
// a consumer polls with relaxed (coherent, non-invalidating) loads, then takes
// one acquire fence.  A worker remembers the last window whose dependencies it
// has acquired, so consecutive tiles of one window wait (and invalidate) once.
#include "gemm_tile.h"
#include "gemm_tile_mx8.h"
#include "movers_dev.h"
#include "persistent.h"

namespace mok {

namespace {

using namespace gemm;
using namespace movers;

constexpr int kMaxMacro = kPersistMaxMacro;

struct PMacro {
  const int32_t* offsets;
  const int32_t* aos;
  const int32_t* soa;
  const float* gate;
  uint16_t* y;
  void* const* out_parts;
  int32_t out_n_part, out_part_rows;
};

struct PKArgs {
  PMacro mb[kMaxMacro];
  int32_t n_macro, T, k, H, I, n_local, act_format, M, S, cap, n_move, max_win;
  void* const* x_parts;
  int32_t x_n_part, x_part_rows;
  const uint16_t* w_gu;
  const uint16_t* w_d;
  int32_t w_packed;
  void* ring;
  uint8_t* ring_sc;
  void* act;
  uint8_t* act_sc;
  int32_t act_rows;
  int32_t* status;
  int32_t* ctl;
  uint64_t timeout_ticks;
};

// Control block (int32 words) for at most W windows.
struct CtlView {
  int32_t *tile_ctr, *abort, *n_windows, *n_items;
  int32_t *win_m, *win_s0, *win_s1, *win_nt1, *win_nt2;
  int32_t *gathered, *gu_done, *dn_done, *merged;
  int32_t* xseq;   // [8][2W + 1] per-XCD prefix of tile shares over the sequence
  int32_t* ent;    // [2W] sequence entries: 2 * window + (0 gate/up, 1 down)
  int32_t* items;  // [W + kMaxMacro] mover items: window >= 0, merge m as -m - 1
  PMacro* pm;      // [kMaxMacro] per-macrobatch buffers (copied from the kernel arguments,
                   // so runtime indexing does not force the arguments into scratch)
  int xstride;
  __host__ __device__ static size_t int_words(int W) {
    return 16 + 5 * W + 3 * W + kMaxMacro + 8 * (2 * W + 1) + 2 * W + W + kMaxMacro;
  }
  __host__ __device__ static size_t words(int W) {
    return (int_words(W) + 3) / 4 * 4 + kMaxMacro * sizeof(PMacro) / sizeof(int32_t);
  }
  __device__ CtlView(int32_t* b, int W) {
    tile_ctr = b; abort = b + 8; n_windows = b + 9; n_items = b + 10;
    int32_t* p = b + 16;
    win_m = p; p += W; win_s0 = p; p += W; win_s1 = p; p += W; win_nt1 = p; p += W;
    win_nt2 = p; p += W; gathered = p; p += W; gu_done = p; p += W; dn_done = p; p += W;
    merged = p; p += kMaxMacro; xseq = p; p += 8 * (2 * W + 1); ent = p; p += 2 * W; items = p;
    pm = reinterpret_cast<PMacro*>(b + (int_words(W) + 3) / 4 * 4);
    xstride = 2 * W + 1;
  }
};

__global__ void k_fill(int32_t* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

// Builds windows, the worker tile sequence and the mover item list on the
// device from the schedules (no host round trip).
// Plan of one launch, built in LDS (a chain of dependent global reads and
// writes by one thread took up to 120 us): the macrobatches' offsets are
// staged by all threads, thread 0 plans windows, the G1/G2 sequence and the
// mover items, threads 0..7 build the per-XCD prefix tables, and all threads
// copy the plan out.  Dynamic LDS: plan_lds_bytes().
constexpr int kPlanMaxWin = 1024;

__host__ __device__ inline size_t plan_lds_words(int n_macro, int n_local, int max_win) {
  return static_cast<size_t>(n_macro) * (n_local + 1) + 8 * static_cast<size_t>(max_win) + kMaxMacro;
}

__global__ __launch_bounds__(256) void k_plan(const PKArgs a) {
  extern __shared__ int32_t plan_lds[];
  __shared__ int32_t sh_w, sh_ne, sh_ni, sh_fail;
  const int tid = threadIdx.x, nl1 = a.n_local + 1, MW = a.max_win;
  int32_t* offs = plan_lds;                                   // [n_macro][n_local + 1]
  int32_t* wm = offs + a.n_macro * nl1;                       // windows: macrobatch,
  int32_t* ws0 = wm + MW;                                     //   first slot,
  int32_t* ws1 = ws0 + MW;                                    //   end slot,
  int32_t* wn1 = ws1 + MW;                                    //   gate/up tiles,
  int32_t* wn2 = wn1 + MW;                                    //   down tiles
  int32_t* ent = wn2 + MW;                                    // [2 MW] sequence
  int32_t* items = ent + 2 * MW;                              // [MW + kMaxMacro] mover items
  CtlView c(a.ctl, MW);
#pragma unroll
  for (int m = 0; m < kMaxMacro; ++m) {                       // compile-time indices into the args
    if (m < a.n_macro) {
      for (int e = tid; e < nl1; e += blockDim.x) offs[m * nl1 + e] = a.mb[m].offsets[e];
      if (tid == 0) c.pm[m] = a.mb[m];
    }
  }
  __syncthreads();
  if (tid == 0) {
    int fail = 0;
    for (int m = 0; m < a.n_macro; ++m)
      if (offs[m * nl1 + a.n_local] > a.cap) fail = 1;       // more rows than the capacity
    const int n1 = (a.I + BN / 2 - 1) / (BN / 2), n2 = (a.H + BN - 1) / BN;
    int W = 0, ne = 0, ni = 0;
    if (!fail) {
      for (int m = 0; m < a.n_macro; ++m) {
        const int32_t R = offs[m * nl1 + a.n_local];
        for (int32_t s0 = 0; s0 < R && W < MW; s0 += a.M) {
          const int32_t s1 = s0 + a.M < R ? s0 + a.M : R;
          const int mt = window_mtiles(offs + m * nl1, a.n_local, s0, s1);
          wm[W] = m; ws0[W] = s0; ws1[W] = s1; wn1[W] = mt * n1; wn2[W] = mt * n2;
          ++W;
        }
      }
      for (int w = 0; w < W; ++w) {
        ent[ne++] = 2 * w;
        if (w >= 1) ent[ne++] = 2 * (w - 1) + 1;
      }
      if (W >= 1) ent[ne++] = 2 * (W - 1) + 1;
      int next_merge = 0, w = 0;
      for (int m = 0; m < a.n_macro; ++m) {
        const int32_t R = offs[m * nl1 + a.n_local];
        const int nw = (R + a.M - 1) / a.M;
        for (int b = 0; b < nw; ++b, ++w) {
          items[ni++] = w;
          if (b >= 1 || nw == 1)
            while (next_merge < m) items[ni++] = -(next_merge++) - 1;
        }
      }
      while (next_merge < a.n_macro) items[ni++] = -(next_merge++) - 1;
    }
    sh_fail = fail; sh_w = W; sh_ne = ne; sh_ni = ni;
  }
  __syncthreads();
  if (sh_fail) {
    if (tid == 0) {
      set_status(a.status, MOK_ERR_CAPACITY);
      *c.n_windows = 0;
      *c.n_items = 0;
    }
    return;
  }
  const int W = sh_w, ne = sh_ne, ni = sh_ni;
  if (tid < kXcds) {                                          // XCD tid's share prefix
    int32_t acc = 0;
    for (int q = 0; q < ne; ++q) {
      const int w = ent[q] >> 1;
      const int32_t tk = (ent[q] & 1) ? wn2[w] : wn1[w];
      c.xseq[tid * c.xstride + q] = acc;
      acc += tk / kXcds + (tid < tk % kXcds ? 1 : 0);
    }
    c.xseq[tid * c.xstride + ne] = acc;
  }
  for (int i = tid; i < W; i += blockDim.x) {
    c.win_m[i] = wm[i]; c.win_s0[i] = ws0[i]; c.win_s1[i] = ws1[i];
    c.win_nt1[i] = wn1[i]; c.win_nt2[i] = wn2[i];
  }
  for (int i = tid; i < ne; i += blockDim.x) c.ent[i] = ent[i];
  for (int i = tid; i < ni; i += blockDim.x) c.items[i] = items[i];
  if (tid == 0) { *c.n_windows = W; *c.n_items = ni; }
}

// Bounded wait by thread 0 for *ctr >= target: relaxed polls, then one
// agent-scope acquire fence; the result is broadcast to the workgroup.  False
// when the kernel is aborting.
__device__ __forceinline__ bool wait_geq(int32_t* ctr, int32_t target, const CtlView& c,
                                         const PKArgs& a, int32_t* sh_flag) {
  if (threadIdx.x == 0) {
    int ok = 1;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(c.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) { ok = 0; break; }
      if (__builtin_amdgcn_s_memrealtime() - t0 > a.timeout_ticks) {
        __hip_atomic_store(c.abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        set_status(a.status, MOK_ERR_DEVICE);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *sh_flag = ok;
  }
  __syncthreads();
  const bool ok = *sh_flag != 0;
  __syncthreads();
  return ok;
}

// Publishes this workgroup's writes, then bumps the counter: every wave
// waits until its stores have reached the XCD's L2 (vmcnt(0); a workgroup
// fence does not wait for global stores), the barrier joins the waves, and
// thread 0's release add writes that L2 back before the increment becomes
// visible.
__device__ __forceinline__ void signal_add(int32_t* ctr) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Gather of window w by the waves first, first + step, ...: wave i takes
// the slot pairs (s0 + 2 q, s0 + 2 q + 1), q = i, i + step, ...
template <bool A_MX>
__device__ __forceinline__ void gather_window(const PKArgs& a, const CtlView& c, int w,
                                              int64_t first, int64_t step) {
  const PMacro pm = c.pm[c.win_m[w]];
  const int32_t s0 = c.win_s0[w], s1 = c.win_s1[w];
  const int64_t base = static_cast<int64_t>(w & 1) * a.M - s0;
  for (int64_t s = s0 + 2 * first; s < s1; s += 2 * step) {
    const int64_t t1 = pm.aos[s] / a.k;
    const int64_t t2 = s + 1 < s1 ? pm.aos[s + 1] / a.k : -1;
    if (A_MX)
      gather_pair_mxfp8(a.x_parts, a.x_n_part, a.x_part_rows, a.H, t1, t2,
                        static_cast<uint8_t*>(a.ring), a.ring_sc, base + s, base + s + 1, a.S, 0,
                        a.H / 4, a.status);
    else
      gather_pair_bf16(a.x_parts, a.x_n_part, a.x_part_rows, a.H, t1, t2,
                       static_cast<uint16_t*>(a.ring), base + s, base + s + 1, a.S, 0, a.H / 4,
                       a.status);
  }
}

// Merge of macrobatch m by the waves first, first + step, ... after every
// down tile of its windows is done.  kFast: see combine_token.
template <bool kFast>
__device__ __forceinline__ bool merge_macro(const PKArgs& a, const CtlView& c, int32_t* sh, int m,
                                            int64_t first, int64_t step) {
  const int W = *c.n_windows;
  for (int w = 0; w < W; ++w)
    if (c.win_m[w] == m && !wait_geq(&c.dn_done[w], c.win_nt2[w], c, a, sh)) return false;
  const PMacro pm = c.pm[m];
  const int32_t R = pm.offsets[a.n_local];
  for (int64_t s = first; s < R; s += step)
    merge_slot<kFast>(pm.y, a.cap, pm.aos[s], pm.soa, pm.gate, s, a.k, a.H, pm.out_parts,
                      pm.out_n_part, pm.out_part_rows, a.status);
  return true;
}

// Movers: the item list in order, except window 0 (gathered by every
// workgroup at the start) and the last macrobatch's merge, which they share
// with the workers once the GEMMs are done (nothing else runs then, so it is
// spread over all CUs).  Between those two points the movers run beside the
// GEMM workers and keep a moderate pace: faster movers there took HBM / L2
// bandwidth from the workers' operand stream and slowed the layer.
template <bool A_MX>
__device__ __forceinline__ void mover(const PKArgs& a, const CtlView& c, int32_t* sh) {
  const int wave = threadIdx.x / kWave;
  const int64_t mw = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const int64_t nmw = static_cast<int64_t>(a.n_move) * 4;
  const int ni = *c.n_items;
  for (int it = 0; it < ni; ++it) {
    const int item = c.items[it];
    if (item >= 0) {
      const int w = item;
      if (w == 0) continue;
      if (w >= 2 && !wait_geq(&c.gu_done[w - 2], c.win_nt1[w - 2], c, a, sh)) return;
      gather_window<A_MX>(a, c, w, mw, nmw);
      signal_add(&c.gathered[w]);
    } else {
      const int m = -item - 1;
      if (m == a.n_macro - 1) {
        merge_macro<true>(a, c, sh, m, mw, static_cast<int64_t>(gridDim.x) * 4);
      } else {
        if (!merge_macro<false>(a, c, sh, m, mw, nmw)) return;
        signal_add(&c.merged[m]);
      }
    }
  }
}

// Operand formats of a persistent launch: bf16 activations and weights;
// MXFP8 activations with bf16 weights; MXFP8 activations and weights.
enum PFormat { kPBf16 = 0, kPMxAct = 1, kPMx8 = 2 };

// Workers: GEMM tiles from the XCD's queue; false when the kernel aborts.
template <int F>
__device__ __forceinline__ bool worker_tiles(const PKArgs& a, const CtlView& c, int32_t* sh,
                                             uint8_t* lds) {
  const int x = blockIdx.x % kXcds;
  const int W = *c.n_windows, ne = 2 * W;
  const int32_t* xs = c.xseq + x * c.xstride;
  const int32_t total = W > 0 ? xs[ne] : 0;
  const int n1 = (a.I + BN / 2 - 1) / (BN / 2), n2 = (a.H + BN - 1) / BN;
  int ready_g1 = -1, ready_g2 = -1;   // last window whose G1 / G2 dependencies were acquired
  while (true) {
    if (threadIdx.x == 0)
      sh[1] = __hip_atomic_fetch_add(&c.tile_ctr[x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int32_t lt = sh[1];
    __syncthreads();
    if (lt >= total) return true;
    int lo = 0, hi = ne - 1;                     // last entry whose prefix <= lt
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (xs[mid] <= lt) lo = mid; else hi = mid - 1;
    }
    const int w = c.ent[lo] >> 1, down = c.ent[lo] & 1;
    const int32_t tk = down ? c.win_nt2[w] : c.win_nt1[w];
    const int32_t q = tk / kXcds, r = tk % kXcds;
    const int te = x * q + (x < r ? x : r) + (lt - xs[lo]);
    const int m = c.win_m[w];
    bool ok = true;
    if (!down && w != ready_g1) {
      ok = wait_geq(&c.gathered[w], w == 0 ? static_cast<int32_t>(gridDim.x) : a.n_move, c, a, sh) &&
           (w < 2 || wait_geq(&c.dn_done[w - 2], c.win_nt2[w - 2], c, a, sh));
      ready_g1 = w;
    } else if (down && w != ready_g2) {
      ok = wait_geq(&c.gu_done[w], c.win_nt1[w], c, a, sh) &&
           (m < 2 || wait_geq(&c.merged[m - 2], a.n_move, c, a, sh));
      ready_g2 = w;
    }
    if (!ok) return false;
    const PMacro pm = c.pm[m];
    const int32_t s0 = c.win_s0[w], s1 = c.win_s1[w];
    int e, row0, nrows, ntile;
    if (!tile_of(pm.offsets, a.n_local, s0, s1, down ? n2 : n1, te, e, row0, nrows, ntile)) {
      signal_add(down ? &c.dn_done[w] : &c.gu_done[w]);   // cannot happen: counts come from the plan
      continue;
    }
    const int32_t rb = static_cast<int32_t>(
        ((static_cast<int64_t>(w & 1) * a.M - s0) % a.S + a.S) % a.S);
    GemmParams g{};
    g.offsets = pm.offsets; g.n_local = a.n_local; g.s_begin = s0; g.s_end = s1;
    if (!down) {
      g.A = a.ring; g.A_scales = a.ring_sc; g.a_rows = a.S; g.a_row_base = rb;
      g.W = a.w_gu; g.w_expert_stride = static_cast<int64_t>(2) * a.I * a.H; g.K = a.H;
      g.N = a.I; g.I = a.I;
      g.C = a.act; g.C_scales = a.act_sc; g.c_rows = a.act_rows; g.c_row_base = rb;
      g.n_tiles = n1; g.w_packed = a.w_packed;
      if constexpr (F == kPMx8)
        gemm_tile_mx8<EPI_SWIGLU_MX>(g, e, row0, nrows, ntile, lds);
      else
        gemm_tile<F == kPMxAct, F == kPMxAct ? EPI_SWIGLU_MX : EPI_SWIGLU_BF16>(g, e, row0, nrows, ntile, lds);
      signal_add(&c.gu_done[w]);
    } else {
      g.A = a.act; g.A_scales = a.act_sc; g.a_rows = a.act_rows; g.a_row_base = rb;
      g.W = a.w_d; g.w_expert_stride = static_cast<int64_t>(a.H) * a.I; g.K = a.I;
      g.N = a.H; g.I = 0;
      g.C = pm.y; g.C_scales = nullptr; g.c_rows = a.cap; g.c_row_base = 0;
      g.n_tiles = n2; g.w_packed = a.w_packed;
      if constexpr (F == kPMx8)
        gemm_tile_mx8<EPI_STORE_BF16>(g, e, row0, nrows, ntile, lds);
      else
        gemm_tile<F == kPMxAct, EPI_STORE_BF16>(g, e, row0, nrows, ntile, lds);
      signal_add(&c.dn_done[w]);
    }
  }
}

template <int F>
__global__ __launch_bounds__(256)
void k_persist(const PKArgs a) {
  constexpr bool A_MX = F != kPBf16;
  constexpr int kLds0 = Geo<false>::LDS > Geo<true>::LDS ? Geo<false>::LDS : Geo<true>::LDS;
  constexpr int kLds = kLds0 > GeoMX8::LDS ? kLds0 : GeoMX8::LDS;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  // The broadcast words share the first 16 bytes of the GEMM's LDS: every
  // use is fenced by workgroup barriers from the tile that overwrites them
  // (gemm_tile opens with one; signal_add closes each tile with one).
  int32_t* sh = reinterpret_cast<int32_t*>(lds);
  CtlView c(a.ctl, a.max_win);
  const int wave = threadIdx.x / kWave;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + wave, ngw = static_cast<int64_t>(gridDim.x) * 4;
  // nothing can run before window 0 is in the ring: every workgroup gathers it
  if (*c.n_windows > 0) {
    gather_window<A_MX>(a, c, 0, gw, ngw);
    signal_add(&c.gathered[0]);
  }
  if (static_cast<int>(blockIdx.x) < a.n_move) {
    mover<A_MX>(a, c, sh);
  } else if (worker_tiles<F>(a, c, sh, lds) && *c.n_items > 0) {
    // GEMMs done: help the movers with the last macrobatch's merge
    merge_macro<true>(a, c, sh, a.n_macro - 1, gw, ngw);
  }
}

}  // namespace

size_t persistent_ws_bytes(int64_t total_windows) {
  int W = static_cast<int>(total_windows > 0 ? total_windows : 1);
  return CtlView::words(W) * sizeof(int32_t) + 256;
}

mok_status launch_persistent(const PersistentArgs& a, hipStream_t s) {
  // automatic split (measured on 256 CUs, Kimi-shaped share): 1/8 of the CUs
  // move data for one macrobatch, 3/16 when several stream through the ring
  // (the movers then also carry the merges that overlap the next gathers)
  const int n_move = a.n_move > 0 ? a.n_move
                                  : (a.n_macro > 1 ? (3 * a.n_cus) / 16 : a.n_cus / 8) > 8
                                        ? (a.n_macro > 1 ? (3 * a.n_cus) / 16 : a.n_cus / 8)
                                        : 8;
  if (n_move < 1 || n_move > a.n_cus - kXcds) return MOK_ERR_INVALID_ARG;
  const bool mx = a.act_format == MOK_ACT_MXFP8_E4M3;
  const void* fn = !mx ? reinterpret_cast<const void*>(&k_persist<kPBf16>)
                   : a.weight_format == MOK_W_MXFP8_E4M3 ? reinterpret_cast<const void*>(&k_persist<kPMx8>)
                                                         : reinterpret_cast<const void*>(&k_persist<kPMxAct>);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess || per_cu < 1)
    return MOK_ERR_HIP;
  const uint64_t timeout_us = a.timeout_us > 0 ? static_cast<uint64_t>(a.timeout_us) : 2000000ull;
  if (a.nwin > kPlanMaxWin) return MOK_ERR_UNSUPPORTED;      // minibatch tiny for the capacity
  const int group = kPlanMaxWin / a.nwin < kMaxMacro ? kPlanMaxWin / a.nwin : kMaxMacro;
  for (int g0 = 0; g0 < a.n_macro; g0 += group) {
    const int gn = a.n_macro - g0 < group ? a.n_macro - g0 : group;
    PKArgs k{};
    for (int m = 0; m < gn; ++m) {
      const MacroBuffers& b = a.mb[g0 + m];
      k.mb[m] = PMacro{b.offsets, b.aos, b.soa, b.gate, b.y, b.out.part_ptr, b.out.n_partitions,
                       b.out.part_rows};
    }
    k.n_macro = gn; k.T = a.T; k.k = a.k; k.H = a.H; k.I = a.I; k.n_local = a.n_local;
    k.act_format = a.act_format; k.M = a.M; k.S = a.S; k.cap = a.cap; k.n_move = n_move;
    k.max_win = gn * a.nwin;
    k.x_parts = a.x.part_ptr; k.x_n_part = a.x.n_partitions; k.x_part_rows = a.x.part_rows;
    k.w_gu = a.w_gu; k.w_d = a.w_d; k.w_packed = a.w_packed;
    k.ring = a.ring; k.ring_sc = a.ring_sc; k.act = a.act; k.act_sc = a.act_sc;
    k.act_rows = a.act_rows; k.status = a.status; k.ctl = static_cast<int32_t*>(a.pers_ws);
    k.timeout_ticks = timeout_us * 100;           // s_memrealtime runs at 100 MHz
    const int64_t words = static_cast<int64_t>(CtlView::words(k.max_win));
    hipLaunchKernelGGL(k_fill, dim3(static_cast<unsigned>((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                       dim3(256), 0, s, k.ctl, words);
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(256),
                       plan_lds_words(gn, a.n_local, k.max_win) * sizeof(int32_t), s, k);
    if (hipGetLastError() != hipSuccess) return MOK_ERR_HIP;
    void* args[] = {&k};
    if (hipLaunchCooperativeKernel(fn, dim3(a.n_cus), dim3(256), args, 0, s) != hipSuccess)
      return MOK_ERR_HIP;
  }
  return MOK_OK;
}

}  // namespace mok
