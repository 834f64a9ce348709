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
//     down tile of m), in the order in which the workers free them, so each
//     gather starts as soon as its ring half is free and each merge runs
//     while the workers compute the next macrobatch;
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
// Counters live in the workspace and are cleared by the set-up launch
// (k_setup) before it plans.  Each XCD has its own L2, so an agent-scope release writes the
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
  uint4* plan;              // merge plan of the down tiles' epilogue [cap]
};

struct PKArgs {
  PMacro mb[kMaxMacro];
  int32_t n_macro, T, k, H, I, n_local, act_format, M, S, cap, n_move, max_win, n_cus;
  int32_t halves;           // the last down phase's tail may run as half-width tiles
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

// Control block (int32 words) for at most W windows.  The view holds only
// the base and W; every member is an offset computed where it is used, so the
// workers do not keep a dozen pointers live in scalar registers across a GEMM
// tile (with them live, the tile's main loop ran short of SGPRs and the
// compiler rebuilt a buffer descriptor with v_readfirstlane in every k-step).
struct CtlView {
  int32_t* b;
  int W;
  __host__ __device__ static size_t int_words(int W) {
    return 16 + 5 * W + 3 * W + kMaxMacro + 8 * (2 * W + 1) + 2 * W + W + kMaxMacro + 16 * W;
  }
  __host__ __device__ static size_t words(int W) {
    return (int_words(W) + 3) / 4 * 4 + kMaxMacro * sizeof(PMacro) / sizeof(int32_t);
  }
  __device__ CtlView(int32_t* base, int W_) : b(base), W(W_) {}
  __device__ int32_t* tile_ctr() const { return b; }
  __device__ int32_t* abort() const { return b + 8; }
  __device__ int32_t* n_windows() const { return b + 9; }
  __device__ int32_t* n_items() const { return b + 10; }
  __device__ int32_t* win_m() const { return b + 16; }
  __device__ int32_t* win_s0() const { return b + 16 + W; }
  __device__ int32_t* win_s1() const { return b + 16 + 2 * W; }
  __device__ int32_t* win_nt1() const { return b + 16 + 3 * W; }
  __device__ int32_t* win_nt2() const { return b + 16 + 4 * W; }
  __device__ int32_t* gathered() const { return b + 16 + 5 * W; }
  __device__ int32_t* gu_done() const { return b + 16 + 6 * W; }
  __device__ int32_t* dn_done() const { return b + 16 + 7 * W; }
  __device__ int32_t* merged() const { return b + 16 + 8 * W; }
  // [8][2W + 1] per-XCD prefix of tile shares over the sequence
  __device__ int32_t* xseq() const { return b + 16 + 8 * W + kMaxMacro; }
  __device__ int xstride() const { return 2 * W + 1; }
  // [2W] sequence entries: 2 * window + (0 gate/up, 1 down)
  __device__ int32_t* ent() const { return xseq() + 8 * (2 * W + 1); }
  // [W + kMaxMacro] mover items: window w >= 1, merge of m < n_macro - 1 as -m - 1
  __device__ int32_t* items() const { return ent() + 2 * W; }
  // [W][2][8] tiles done per window, phase (gate/up, down) and XCD
  __device__ int32_t* xdone() const { return items() + W + kMaxMacro; }
  // [kMaxMacro] per-macrobatch buffers (copied from the kernel arguments, so
  // runtime indexing does not force the arguments into scratch)
  __device__ PMacro* pm() const { return reinterpret_cast<PMacro*>(b + (int_words(W) + 3) / 4 * 4); }
};


// XCD x's share of a phase of `tiles` tiles (a contiguous run of the tile list).
__host__ __device__ __forceinline__ int32_t share_of(int32_t tiles, int x) {
  return tiles / kXcds + (x < tiles % kXcds ? 1 : 0);
}

// Half-width tail of a one-window launch.  Its sequence is G1(0), G2(0): the
// down tiles start together on an XCD's P = n_cus / 8 workgroups once every
// gate/up tile is done, and the last r = c % P of the XCD's c down tiles would
// make a round of their own with P - r CUs idle until the kernel ends.  Where
// that round fills at most half of the CUs, its r tiles run as 2 r tiles of
// 128 columns, as the standalone y-storing GEMMs do: the round takes half as
// long, and every output element is summed by the same MFMAs in the same
// order.  With several windows the down phases interleave with gate/up tiles
// and the rounds do not start together: the same rule there (on the last two
// down phases) measured 1.6 % slower at two windows and no faster at eight,
// while one window gained 2.3 % (the Kimi-shaped share at M = 4096 / 8192,
// A/B in one box).  Returns r (the tiles split), or 0.
__host__ __device__ __forceinline__ int32_t tail_halves(int W, int32_t nt_down, int x, int P) {
  if (W != 1 || P <= 0) return 0;
  const int32_t c = share_of(nt_down, x), rx = c % P;
  return (rx > 0 && 2 * rx <= P) ? rx : 0;
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

// Block 0 of k_setup: clears the control block (every counter at zero), then
// plans into it.
__device__ __forceinline__ void plan_block(const PKArgs& a, int32_t* plan_lds) {
  __shared__ int32_t sh_w, sh_ne, sh_ni, sh_fail;
  const int tid = threadIdx.x, nl1 = a.n_local + 1, MW = a.max_win;
  {
    const int64_t words = static_cast<int64_t>(CtlView::words(MW));
    for (int64_t i = tid; i < words; i += blockDim.x) a.ctl[i] = 0;
    __syncthreads();                 // the plan below writes into the cleared block
  }
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
      if (tid == 0) c.pm()[m] = a.mb[m];
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
      // Mover items in the order in which the worker sequence frees them:
      // the gather of w waits for G1(w - 2) (its ring half), the merge of m
      // for G2 of m's last window.  A mover then never waits on an item
      // while a later one of its list is ready, and every gather starts as
      // soon as its ring half is free.  Positions in the sequence: G1(0) at
      // 0, G1(v) at 2v - 1, G2(v) at 2v + 2, the last G2 at 2W - 1.
      auto g1pos = [](int v) { return v == 0 ? 0 : 2 * v - 1; };
      auto g2pos = [W](int v) { return v == W - 1 ? 2 * W - 1 : 2 * v + 2; };
      int gw = 0, mm = 0, wi = 0;
      while (gw < W || mm < a.n_macro) {
        while (wi < W && wm[wi] <= mm) ++wi;          // windows of macrobatches <= mm
        const int kg = gw >= W ? 0x7fffffff : gw < 2 ? -1 : g1pos(gw - 2);
        const int km = mm >= a.n_macro ? 0x7fffffff : wi > 0 ? g2pos(wi - 1) : -1;
        // window 0 is gathered before the kernel, the last macrobatch merged
        // after it (launches of their own at full occupancy)
        if (kg <= km) {
          if (gw > 0) items[ni++] = gw;
          ++gw;
        } else {
          if (mm < a.n_macro - 1) items[ni++] = -mm - 1;
          ++mm;
        }
      }
    }
    sh_fail = fail; sh_w = W; sh_ne = ne; sh_ni = ni;
  }
  __syncthreads();
  if (sh_fail) {
    if (tid == 0) {
      set_status(a.status, MOK_ERR_CAPACITY);
      *c.n_windows() = 0;
      *c.n_items() = 0;
    }
    return;
  }
  const int W = sh_w, ne = sh_ne, ni = sh_ni;
  if (tid < kXcds) {                                          // XCD tid's share prefix
    // the last entry (G2(W - 1)) holds r more jobs where its tail runs as halves
    const int32_t hx = W > 0 && a.halves ? tail_halves(W, wn2[W - 1], tid, a.n_cus / kXcds) : 0;
    int32_t acc = 0;
    for (int q = 0; q < ne; ++q) {
      const int w = ent[q] >> 1;
      const int32_t tk = (ent[q] & 1) ? wn2[w] : wn1[w];
      c.xseq()[tid * c.xstride() + q] = acc;
      acc += share_of(tk, tid) + (q == ne - 1 ? hx : 0);
    }
    c.xseq()[tid * c.xstride() + ne] = acc;
  }
  for (int i = tid; i < W; i += blockDim.x) {
    c.win_m()[i] = wm[i]; c.win_s0()[i] = ws0[i]; c.win_s1()[i] = ws1[i];
    c.win_nt1()[i] = wn1[i]; c.win_nt2()[i] = wn2[i];
  }
  for (int i = tid; i < ne; i += blockDim.x) c.ent()[i] = ent[i];
  for (int i = tid; i < ni; i += blockDim.x) c.items()[i] = items[i];
  if (tid == 0) { *c.n_windows() = W; *c.n_items() = ni; }
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
      if (__hip_atomic_load(c.abort(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) { ok = 0; break; }
      if (__builtin_amdgcn_s_memrealtime() - t0 > a.timeout_ticks) {
        __hip_atomic_store(c.abort(), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// A pointer the whole wave holds (its two halves moved to scalar registers).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Completion of a GEMM tile of one phase (gate/up or down) of a window.
// Each XCD has its own L2, and an agent-scope release writes back all of it:
// paying that per tile stalled every tile for the write-back of its whole
// XCD's dirty lines.  So a tile only counts itself in per XCD (every wave
// first waits until its stores are in the XCD's L2), and the tile that
// completes its XCD's share of the phase does the one release add on the
// phase counter, whose write-back covers every tile of that XCD: their stores
// reached the same L2 before their counts did.  Consumers wait for the number
// of XCDs that hold tiles of the phase (xcds_of).
__device__ __forceinline__ int32_t xcds_of(int32_t tiles) {
  return tiles < kXcds ? tiles : kXcds;
}
__device__ __forceinline__ void signal_tile(int32_t* xcnt, int32_t share, int32_t* done) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t before = __hip_atomic_fetch_add(xcnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before + 1 == share)
      __hip_atomic_fetch_add(done, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Gather of window w by the waves first, first + step, ...: wave i takes
// the slot pairs (s0 + 2 q, s0 + 2 q + 1), q = i, i + step, ...
template <bool A_MX>
__device__ __forceinline__ void gather_window(const PKArgs& a, const CtlView& c, int w,
                                              int64_t first, int64_t step) {
  const PMacro pm = c.pm()[c.win_m()[w]];
  const int32_t s0 = c.win_s0()[w], s1 = c.win_s1()[w];
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

// Merge of macrobatch m by the waves first, first + step, ... once every
// down tile of its windows is done (item_ready).  kFast: see combine_token.
template <bool kFast>
__device__ __forceinline__ void merge_macro(const PKArgs& a, const CtlView& c, int m,
                                            int64_t first, int64_t step) {
  const PMacro pm = c.pm()[m];
  const int32_t R = pm.offsets[a.n_local];
  for (int64_t s = first; s < R; s += step)             // single-slot tokens: by the down tiles
    merge_slot<kFast>(pm.y, a.cap, pm.aos[s], pm.soa, pm.gate, s, a.k, a.H, pm.out_parts,
                      pm.out_n_part, pm.out_part_rows, a.status, true);
}

__device__ __forceinline__ int32_t ld_relaxed(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0, no wait: whether mover item `item` can start (window >= 0: its
// ring half was freed by G1(w - 2); merge -m - 1: every down tile of m is
// done; the windows of m are contiguous).
__device__ __forceinline__ bool item_ready(const PKArgs& a, const CtlView& c, int item) {
  if (item >= 0)
    return item < 2 || ld_relaxed(&c.gu_done()[item - 2]) >= xcds_of(c.win_nt1()[item - 2]);
  const int m = -item - 1, W = *c.n_windows();
  int lo = 0, hi = W;                            // first window of m
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (c.win_m()[mid] < m) lo = mid + 1; else hi = mid;
  }
  for (int w = lo; w < W && c.win_m()[w] == m; ++w)
    if (ld_relaxed(&c.dn_done()[w]) < xcds_of(c.win_nt2()[w])) return false;
  return true;
}

// Thread 0, no wait: whether every dependency of a tile of entry (w, down) is
// met.  G1(w): the gather of w (window 0 is in the ring before the kernel)
// and G2(w - 2) (activation half).  G2(w): G1(w) and the merge of m - 2
// (return area).
__device__ __forceinline__ bool deps_met(const PKArgs& a, const CtlView& c, int w, int down) {
  if (!down)
    return (w == 0 || ld_relaxed(&c.gathered()[w]) >= a.n_move) &&
           (w < 2 || ld_relaxed(&c.dn_done()[w - 2]) >= xcds_of(c.win_nt2()[w - 2]));
  const int m = c.win_m()[w];
  return ld_relaxed(&c.gu_done()[w]) >= xcds_of(c.win_nt1()[w]) &&
         (m < 2 || ld_relaxed(&c.merged()[m - 2]) >= a.n_move);
}

// Last sequence entry whose prefix (in the XCD's share table xs) is <= lt.
__device__ __forceinline__ int entry_of(const int32_t* xs, int ne, int32_t lt) {
  int lo = 0, hi = ne - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (xs[mid] <= lt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Operand formats of a persistent launch: bf16 activations and weights;
// MXFP8 activations with bf16 weights; MXFP8 activations and weights.
enum PFormat { kPBf16 = 0, kPMxAct = 1, kPMx8 = 2 };

// One loop per workgroup.
//   Movers (workgroups 0 .. n_move - 1) walk the item list, except window 0
//   (gathered by a launch of its own before the kernel) and the last
//   macrobatch's merge (a launch of its own after it: nothing else runs
//   then, so it gets every CU at full occupancy).  While their next item is
//   not ready they take the XCD's next tile if it is a down tile whose
//   dependencies are all met (a compare-and-swap on the queue counter, so a
//   mover never holds a tile it would have to wait for, and its item waits
//   at most one tile), else they poll.  Down tiles only: gate/up tiles are
//   the next step after a gather on the workers' path, and with the Kimi-
//   shaped share (K = 7168 against the down GEMM's 2048) each is 3.5 times
//   longer; a mover that took them delayed the gathers of later windows.
//   Beside the GEMM workers the movers keep a moderate pace: faster movers
//   took HBM / L2 bandwidth from the workers' operand stream and slowed the
//   layer.  After their last item (with a single window they have none) they
//   take tiles like the workers.
//   Workers take the XCD's next tile and wait for its dependencies.
template <int F>
__global__ __launch_bounds__(256)
void k_persist(const PKArgs a) {
  constexpr bool A_MX = F != kPBf16;
  // Half-width tail tiles (tail_halves) with bf16 or full-MXFP8 operands: with
  // MXFP8 activations and bf16 weights the second tile variant took the loop
  // past 256 VGPRs (12 bytes of scratch per lane), so that format keeps whole
  // tiles (the host sets PKArgs::halves to match).
  constexpr bool kHalves = F != kPMxAct;
  constexpr int kLds0 = Geo<false>::LDS > Geo<true>::LDS ? Geo<false>::LDS : Geo<true>::LDS;
  constexpr int kLds1 = kLds0 > GeoMX8::LDS ? kLds0 : GeoMX8::LDS;
  constexpr int kLds = kLds1 > kMergeLds ? kLds1 : kMergeLds;     // the merging down epilogue
  // One LDS array: with a second __shared__ object the compiler could no
  // longer tell the GEMM's LDS reads from its direct-to-LDS loads and made
  // every k-step wait for all loads in flight (vmcnt(0)).
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds + 16];
  // The broadcast words share the first 16 bytes of the GEMM's LDS: every
  // use is fenced by workgroup barriers from the tile that overwrites them
  // (gemm_tile opens with one; signal_add / signal_tile close with one).
  int32_t* sh = reinterpret_cast<int32_t*>(lds);
  CtlView c(a.ctl, a.max_win);
  const int x = blockIdx.x % kXcds;
  // loop state in scalar registers (readfirstlane): the GEMM tile inside the
  // loop needs every vector register
  const int W = __builtin_amdgcn_readfirstlane(*c.n_windows()), ne = 2 * W;
  const int32_t* xs = c.xseq() + x * c.xstride();
  const int32_t total = W > 0 ? __builtin_amdgcn_readfirstlane(xs[ne]) : 0;
  const int n1 = (a.I + BN / 2 - 1) / (BN / 2), n2 = (a.H + BN - 1) / BN;
  int ready_g1 = -1, ready_g2 = -1;   // last window whose G1 / G2 dependencies were acquired
  // A mover's next item and its last progress (for the wait bound) stay in
  // the 16 bytes past the GEMM's LDS, so no register holds them across a
  // GEMM tile.  Thread 0 writes both.
  int32_t& sh_it = *reinterpret_cast<int32_t*>(lds + kLds);
  uint64_t& sh_t0 = *reinterpret_cast<uint64_t*>(lds + kLds + 8);
  if (threadIdx.x == 0) { sh_it = 0; sh_t0 = __builtin_amdgcn_s_memrealtime(); }
  __syncthreads();
  while (true) {
    int32_t lt;
    bool met = false;                 // the tile's dependencies are met and acquired
    const int ni = static_cast<int>(blockIdx.x) < a.n_move
                       ? __builtin_amdgcn_readfirstlane(*c.n_items()) : 0;
    const int it = ni > 0 ? __builtin_amdgcn_readfirstlane(sh_it) : 0;
    if (it < ni) {
      const int item = __builtin_amdgcn_readfirstlane(c.items()[it]);
      constexpr int32_t kItem = -1, kIdle = -2, kAbort = -3;
      if (threadIdx.x == 0) {
        int32_t r = kIdle;
        if (item_ready(a, c, item)) {
          r = kItem;
        } else {
          const int32_t cur = ld_relaxed(&c.tile_ctr()[x]);
          if (cur < total) {
            const int q = entry_of(xs, ne, cur);
            const int ent = c.ent()[q];
            int32_t expect = cur;
            if ((ent & 1) && deps_met(a, c, ent >> 1, 1) &&
                __hip_atomic_compare_exchange_strong(&c.tile_ctr()[x], &expect, cur + 1,
                                                     __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT))
              r = cur;
          }
        }
        const uint64_t now = __builtin_amdgcn_s_memrealtime();
        if (r != kIdle) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          sh_t0 = now;
        } else if (ld_relaxed(c.abort())) {
          r = kAbort;
        } else if (now - sh_t0 > a.timeout_ticks) {
          __hip_atomic_store(c.abort(), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          set_status(a.status, MOK_ERR_DEVICE);
          r = kAbort;
        } else {
          __builtin_amdgcn_s_sleep(1);
        }
        sh[1] = r;
      }
      __syncthreads();
      const int32_t r = __builtin_amdgcn_readfirstlane(sh[1]);
      __syncthreads();
      if (r == kAbort) return;
      if (r == kIdle) continue;
      if (r == kItem) {
        // every wave read sh_it before the barriers above; the next read
        // follows the item's closing barrier (signal_add)
        if (threadIdx.x == 0) sh_it = it + 1;
        const int64_t mw = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
        const int64_t nmw = static_cast<int64_t>(a.n_move) * 4;
        if (item >= 0) {
          gather_window<A_MX>(a, c, item, mw, nmw);
          signal_add(&c.gathered()[item]);
        } else {
          // 4 pieces per lane and slot (kFast): the 16 of the plain merge held
          // 128 accumulators per lane in this loop beside the GEMM's state and
          // pushed registers of every tile to scratch; the sums are the same
          merge_macro<true>(a, c, -item - 1, mw, nmw);
          signal_add(&c.merged()[-item - 1]);
        }
        continue;
      }
      lt = r;
      met = true;
    } else {
      if (threadIdx.x == 0)
        sh[1] = __hip_atomic_fetch_add(&c.tile_ctr()[x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      // uniform by construction (one value broadcast through LDS); saying so
      // keeps everything derived from it -- tile coordinates, operand bases and
      // the buffer descriptors -- in scalar registers, where the GEMM's main
      // loop wants them (with a vector value the compiler re-derived the
      // descriptors with v_readfirstlane in every k-step)
      lt = __builtin_amdgcn_readfirstlane(sh[1]);
      __syncthreads();
      if (lt >= total) return;
    }
    const int lo = entry_of(xs, ne, lt);
    const int w = c.ent()[lo] >> 1, down = c.ent()[lo] & 1;
    const int32_t tk = down ? c.win_nt2()[w] : c.win_nt1()[w];
    const int32_t q = tk / kXcds, r = tk % kXcds;
    // the last entry's tail as half-width jobs (tail_halves): dispatch order
    // of XCD x is the first hx halves, the c - hx whole tiles, then the other
    // hx halves, as in the standalone GEMM (the CUs that start with a half
    // stay half a tile ahead, so the round's stores and loads come in two
    // half-size bursts)
    const int32_t hx = kHalves && lo == ne - 1
        ? tail_halves(W, tk, x, static_cast<int>(gridDim.x) / kXcds) : 0;
    int32_t u = lt - xs[lo];
    int half = 0;
    if (hx > 0) {
      const int32_t cx = share_of(tk, x);
      const int32_t v = u < hx ? u : u >= cx ? u - cx + hx : -1;
      if (v >= 0) {
        u = cx - hx + (v >> 1);
        half = 1 + (v & 1);
      } else {
        u -= hx;
      }
    }
    half = __builtin_amdgcn_readfirstlane(half);
    const int te = x * q + (x < r ? x : r) + u;
    const int m = c.win_m()[w];
    bool ok = true;
    if (!met && !down && w != ready_g1) {
      ok = (w == 0 || wait_geq(&c.gathered()[w], a.n_move, c, a, sh)) &&
           (w < 2 || wait_geq(&c.dn_done()[w - 2], xcds_of(c.win_nt2()[w - 2]), c, a, sh));
      ready_g1 = w;
    } else if (!met && down && w != ready_g2) {
      ok = wait_geq(&c.gu_done()[w], xcds_of(c.win_nt1()[w]), c, a, sh) &&
           (m < 2 || wait_geq(&c.merged()[m - 2], a.n_move, c, a, sh));
      ready_g2 = w;
    }
    int32_t* xcnt = c.xdone() + (2 * w + down) * kXcds + x;
    const int32_t xshare = share_of(tk, x) + hx;
    if (!ok) return;
    // The control block is written during the kernel, so its loads are vector
    // loads, whose results the compiler keeps in VGPRs: every value the tile
    // derives from them (operand bases, buffer descriptors) would then be
    // re-read with v_readfirstlane inside the GEMM's k-loop.  They are uniform;
    // moving them to scalar registers here keeps the k-loop as in the
    // standalone GEMM kernels.
    const PMacro pm = c.pm()[m];
    const int32_t* offs = uniform_ptr(pm.offsets);
    const int32_t s0 = __builtin_amdgcn_readfirstlane(c.win_s0()[w]);
    const int32_t s1 = __builtin_amdgcn_readfirstlane(c.win_s1()[w]);
    int e, row0, nrows, ntile;
    const bool have = tile_of(offs, a.n_local, s0, s1, down ? n2 : n1, te, e, row0, nrows, ntile);
    e = __builtin_amdgcn_readfirstlane(e);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    ntile = __builtin_amdgcn_readfirstlane(ntile);
    if (!have) {
      signal_tile(xcnt, xshare, down ? &c.dn_done()[w] : &c.gu_done()[w]);   // cannot happen: counts
      continue;                                                          // come from the plan
    }
    const int32_t rb = static_cast<int32_t>(
        ((static_cast<int64_t>(w & 1) * a.M - s0) % a.S + a.S) % a.S);
    GemmParams g{};
    g.offsets = offs; g.n_local = a.n_local; g.s_begin = s0; g.s_end = s1;
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
      signal_tile(xcnt, xshare, &c.gu_done()[w]);
    } else {
      g.A = a.act; g.A_scales = a.act_sc; g.a_rows = a.act_rows; g.a_row_base = rb;
      g.W = a.w_d; g.w_expert_stride = static_cast<int64_t>(a.H) * a.I; g.K = a.I;
      g.N = a.H; g.I = 0;
      g.C = uniform_ptr(pm.y); g.C_scales = nullptr; g.c_rows = a.cap; g.c_row_base = 0;
      g.n_tiles = n2; g.w_packed = a.w_packed;
      g.m_plan = uniform_ptr(pm.plan); g.m_status = a.status;     // single-slot tokens merged here
      if (kHalves && half != 0) {
        TileJob j{};
        j.e = e; j.row0 = row0; j.nrows = nrows; j.ntile = ntile; j.role = kWhole; j.half = half;
        if constexpr (F == kPMx8)
          gemm_tile_mx8<EPI_DOWN_MERGE, BN / 2>(g, j, lds);
        else if constexpr (F == kPBf16)
          gemm_tile<false, EPI_DOWN_MERGE, BN / 2>(g, j, lds);
      } else if constexpr (F == kPMx8) {
        gemm_tile_mx8<EPI_DOWN_MERGE>(g, e, row0, nrows, ntile, lds);
      } else {
        gemm_tile<F == kPMxAct, EPI_DOWN_MERGE>(g, e, row0, nrows, ntile, lds);
      }
      signal_tile(xcnt, xshare, &c.dn_done()[w]);
    }
  }
}

}  // namespace

// Merge plan record of slot s of one macrobatch (launch_merge_plan's records;
// k_setup writes those of all the group's macrobatches).  Slots s < min(R,
// cap): a plan holds cap records (with R > cap the set-up plans nothing and
// raises the capacity status; records past cap would overwrite the next
// workspace region, the control block).
__device__ __forceinline__ void merge_plan_slot(const PKArgs& a, const PMacro& pm, int64_t s) {
  if (s >= pm.offsets[a.n_local] || s >= a.cap) return;
  const int32_t asg = pm.aos[s];
  const int64_t t = asg / a.k;
  int live = 0;
  for (int j = 0; j < a.k; ++j) live += pm.soa[t * a.k + j] >= 0 ? 1 : 0;
  uint4 rec = make_uint4(0, 0, 0, 0);
  const int64_t part = t / pm.out_part_rows;
  if (live == 1 && part < pm.out_n_part) {
    const uint64_t addr = reinterpret_cast<uint64_t>(static_cast<uint16_t*>(pm.out_parts[part]) +
                                                     (t % pm.out_part_rows) * static_cast<int64_t>(a.H));
    rec = make_uint4(static_cast<uint32_t>(addr), static_cast<uint32_t>(addr >> 32),
                     __float_as_uint(pm.gate[asg]), 0u);
  }
  pm.plan[s] = rec;
}

// The set-up of a group of macrobatches in one launch: block 0 clears the
// control block and plans the windows, the worker tile sequence and the mover
// items (plan_block); blocks 1 .. gn * mb_blocks write the merge plans,
// mb_blocks blocks of 256 slots per macrobatch.  (Three launches before:
// a fill, the plan, the merge plans.)
__global__ __launch_bounds__(256)
void k_setup(const PKArgs a, int32_t mb_blocks) {
  extern __shared__ int32_t plan_lds[];
  if (blockIdx.x == 0) {
    plan_block(a, plan_lds);
    return;
  }
  const int b = static_cast<int>(blockIdx.x) - 1, m = b / mb_blocks;
  if (m >= a.n_macro) return;
  const PMacro pm = a.mb[m];
  merge_plan_slot(a, pm, static_cast<int64_t>(b % mb_blocks) * blockDim.x + threadIdx.x);
}

size_t persistent_ws_bytes(int64_t total_windows) {
  int W = static_cast<int>(total_windows > 0 ? total_windows : 1);
  return CtlView::words(W) * sizeof(int32_t) + 256;
}

mok_status launch_persistent(const PersistentArgs& a, hipStream_t s) {
  // automatic split: a quarter of the CUs move data.  Movers take GEMM tiles
  // once their gathers and merges are done, so more of them cost the GEMMs
  // little, while fewer slow every window's gather (measured on 256 CUs, the
  // Kimi-shaped share at M = 4096: 8 movers 1.68 ms, 16 1.13, 64 0.83).
  const int n_move = a.n_move > 0 ? a.n_move : (a.n_cus / 4 > 8 ? a.n_cus / 4 : 8);
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
                       b.out.part_rows, static_cast<uint4*>(b.plan)};
    }
    k.n_macro = gn; k.T = a.T; k.k = a.k; k.H = a.H; k.I = a.I; k.n_local = a.n_local;
    k.act_format = a.act_format; k.M = a.M; k.S = a.S; k.cap = a.cap; k.n_move = n_move;
    k.n_cus = a.n_cus;
    k.halves = (!mx || a.weight_format == MOK_W_MXFP8_E4M3) ? 1 : 0;   // as kHalves of k_persist
    k.max_win = gn * a.nwin;
    k.x_parts = a.x.part_ptr; k.x_n_part = a.x.n_partitions; k.x_part_rows = a.x.part_rows;
    k.w_gu = a.w_gu; k.w_d = a.w_d; k.w_packed = a.w_packed;
    k.ring = a.ring; k.ring_sc = a.ring_sc; k.act = a.act; k.act_sc = a.act_sc;
    k.act_rows = a.act_rows; k.status = a.status; k.ctl = static_cast<int32_t*>(a.pers_ws);
    k.timeout_ticks = timeout_us * 100;           // s_memrealtime runs at 100 MHz
    const int32_t mb_blocks = static_cast<int32_t>((a.cap + 255) / 256);
    hipLaunchKernelGGL(k_setup, dim3(static_cast<unsigned>(1 + static_cast<int64_t>(gn) * mb_blocks)),
                       dim3(256), plan_lds_words(gn, a.n_local, k.max_win) * sizeof(int32_t), s, k,
                       mb_blocks);
    if (hipGetLastError() != hipSuccess) return MOK_ERR_HIP;
    // window 0 of the group: the first macrobatch's slots [0, M) into ring half 0
    const MacroBuffers& b0 = a.mb[g0];
    if (launch_gather(a.x.part_ptr, a.x.n_partitions, a.x.part_rows, a.H, a.k, b0.aos, b0.offsets,
                      a.n_local, 0, a.M < a.cap ? a.M : a.cap, a.ring, a.ring_sc, a.S,
                      a.act_format, a.status, s) != hipSuccess)
      return MOK_ERR_HIP;
    void* args[] = {&k};
    if (hipLaunchCooperativeKernel(fn, dim3(a.n_cus), dim3(256), args, 0, s) != hipSuccess)
      return MOK_ERR_HIP;
    // the group's last macrobatch, merged once every down tile is done
    const MacroBuffers& bl = a.mb[g0 + gn - 1];
    if (launch_combine_slots(bl.y, a.cap, bl.aos, bl.offsets, a.n_local, a.cap, bl.soa, bl.gate,
                             a.k, a.H, bl.out.part_ptr, bl.out.n_partitions, bl.out.part_rows,
                             a.status, true, s, true) != hipSuccess)
      return MOK_ERR_HIP;
  }
  return MOK_OK;
}

}  // namespace mok
