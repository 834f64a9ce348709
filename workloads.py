"""Seeded synthetic inputs for the MoE forward layer (one GPU's share).

This module only draws numbers.  It holds none of the layer's arithmetic:
no top-k, no schedule, no quantiser, no FFN, no combine.  Both the CPU
oracle (``oracle/``) and the HIP library (``token_dispatch_grouped_top_amd``)
consume exactly the bits produced here.

Every array comes from ``numpy.random.Generator(PCG64)`` streams derived
from one integer seed through ``SeedSequence``: child 0 draws the token
activations ``x``, child 1 the gate/up weights, child 2 the down weights,
child 3 the routing (logits or routed ids and gates).  Large arrays are drawn
in fixed 4 Mi-element chunks, each chunk with its own spawned stream, so the
bits do not depend on the number of threads used.  fp32 draws become bf16
by round-to-nearest-even on the bit pattern (input preparation only).

Workload shapes follow the Mixture-of-Kittens pages (tahou.com article and
the PyTorchKR wiki summary): a hidden size 7168 / expert intermediate 2048
expert share fed by 72 source partitions, plus a tiny and a Mixtral-shaped
case.  Routing statistics (balanced, Zipf-skewed) are synthetic stand-ins;
no dataset or trained weight is used.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional

import numpy as np

_CHUNK = 1 << 22

ACT_BF16 = 0
ACT_MXFP8 = 1


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _bf16_bits(a32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = a32.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def normal_bf16(seed_seq: np.random.SeedSequence, n: int, std: float) -> np.ndarray:
    """n draws of N(0, std^2) as bf16 bits (uint16), chunked and threaded."""
    out = np.empty(n, np.uint16)
    nch = (n + _CHUNK - 1) // _CHUNK
    kids = seed_seq.spawn(nch)

    def work(i: int) -> None:
        g = np.random.Generator(np.random.PCG64(kids[i]))
        m = min(_CHUNK, n - i * _CHUNK)
        a = g.standard_normal(m, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        out[i * _CHUNK:i * _CHUNK + m] = _bf16_bits(a)

    if nch == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nch)))
    return out


def small_int_bf16(seed: int, shape, lo: int, hi: int) -> np.ndarray:
    """Integers drawn uniformly from [lo, hi] as bf16 bits (exact for |v| <= 256)."""
    g = np.random.default_rng(seed)
    return _bf16_bits(g.integers(lo, hi + 1, size=shape).astype(np.float32))


def router_inputs(seed: int, T: int, H: int, E: int):
    """Tokens x ~ N(0, 1) bf16 [T][H] and router weights W_r ~ N(0, 1/H) bf16
    [E][H] (nn.Linear layout) for the router GEMM."""
    ss = np.random.SeedSequence(seed).spawn(2)
    x = normal_bf16(ss[0], T * H, 1.0).reshape(T, H)
    w = normal_bf16(ss[1], E * H, float(1.0 / np.sqrt(H))).reshape(E, H)
    return x, w


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> fp32 values (exact widening)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One synthetic instance of the layer on one GPU.

    Token t of the pool lives in source partition ``t // part_rows`` at row
    ``t % part_rows``.  ``x`` holds the pool flattened as [T, H] bf16 bits;
    the GPU side places each partition in its own allocation.
    """
    name: str
    seed: int
    T: int                 # pool tokens whose routing is given
    H: int
    I: int
    E: int                 # experts routed over
    k: int
    expert_base: int
    n_local: int
    n_partitions: int
    part_rows: int
    act_format: int
    x: np.ndarray          # uint16 [T, H]
    w_gu: np.ndarray       # uint16 [n_local, 2I, H]; rows 0..I-1 gate, I..2I-1 up
    w_d: np.ndarray        # uint16 [n_local, H, I]
    logits: np.ndarray     # float32 [T_route, E]; routed by the route step
    topk_idx: Optional[np.ndarray] = None   # int32 [T, k] given routing (pool cases)
    topk_gate: Optional[np.ndarray] = None  # float32 [T, k]
    minibatches: List[int] = dataclasses.field(default_factory=list)
    macrobatch: int = 0
    weight_format: int = 0  # 0: bf16 weights; 1: weights quantised to MXFP8 (act_format 1)

    @property
    def routing_from_logits(self) -> bool:
        return self.topk_idx is None


def _weights(ss_gu, ss_d, n_local: int, H: int, I: int, std: float):
    w_gu = normal_bf16(ss_gu, n_local * 2 * I * H, std).reshape(n_local, 2 * I, H)
    w_d = normal_bf16(ss_d, n_local * H * I, std).reshape(n_local, H, I)
    return w_gu, w_d


def logits_workload(name: str, seed: int, T: int, H: int, I: int, E: int, k: int,
                    x_std: float, w_std: float, router: str = "normal",
                    expert_base: int = 0, n_local: Optional[int] = None,
                    n_partitions: int = 1, act_format: int = ACT_BF16,
                    minibatches=()) -> Workload:
    """Tokens routed by the route step from fp32 logits.

    router="normal": logits ~ N(0, 1) fp32 [T, E].
    router="gaussian_weights": logits = x . W_r with W_r ~ N(0, 1/H) fp32
    [H, E], formed once on the host in fp64 and stored as fp32 (the router
    projection is harness work, not part of the layer here).
    router="ties": logits drawn from {-1, 0, 1} to force equal keys.
    """
    n_local = E if n_local is None else n_local
    ss = np.random.SeedSequence(seed).spawn(4)
    x = normal_bf16(ss[0], T * H, x_std).reshape(T, H)
    w_gu, w_d = _weights(ss[1], ss[2], n_local, H, I, w_std)
    g = np.random.Generator(np.random.PCG64(ss[3]))
    if router == "normal":
        logits = g.standard_normal((T, E), dtype=np.float32)
    elif router == "gaussian_weights":
        w_r = g.standard_normal((H, E), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
        logits = (bf16_to_f32(x).astype(np.float64) @ w_r.astype(np.float64)).astype(np.float32)
    elif router == "ties":
        logits = g.integers(-1, 2, size=(T, E)).astype(np.float32)
    else:
        raise ValueError(router)
    assert T % n_partitions == 0
    return Workload(name=name, seed=seed, T=T, H=H, I=I, E=E, k=k,
                    expert_base=expert_base, n_local=n_local,
                    n_partitions=n_partitions, part_rows=T // n_partitions,
                    act_format=act_format, x=x, w_gu=w_gu, w_d=w_d,
                    logits=np.ascontiguousarray(logits),
                    minibatches=list(minibatches))


def pool_routing(g: np.random.Generator, T: int, E: int, k: int, expert_base: int,
                 counts) -> tuple:
    """Routing of a pool of T source tokens, as the sources' routers produced it.

    Local expert e (global id expert_base + e) receives exactly counts[e]
    distinct pool tokens, chosen uniformly without replacement.  Each token's
    k routed ids are its local picks plus distinct random non-local ids, in
    random slot order.  Gates per token: softmax of k N(0,1) draws sorted in
    descending order (slot 0 carries the largest gate).
    """
    n_local = len(counts)
    picks = np.zeros((T, n_local), dtype=bool)
    for e, c in enumerate(counts):
        picks[g.choice(T, size=int(c), replace=False), e] = True
    nloc = picks.sum(1)
    if nloc.max() > k:
        raise ValueError("a token picked by more local experts than k")
    non_local = np.array([e for e in range(E)
                          if not (expert_base <= e < expert_base + n_local)], np.int32)
    # first k entries of a per-token random permutation of the non-local ids
    keys = g.random((T, non_local.size), dtype=np.float32)
    extra = non_local[np.argpartition(keys, k - 1, axis=1)[:, :k]]
    idx = np.empty((T, k), np.int32)
    local_ids = np.arange(n_local, dtype=np.int32) + expert_base
    for L in range(0, k + 1):
        rows = np.nonzero(nloc == L)[0]
        if rows.size == 0:
            continue
        loc = np.where(picks[rows], local_ids[None, :], -1)
        loc = -np.sort(-loc, axis=1)[:, :L]   # the L local ids of each row
        idx[rows, :L] = loc
        idx[rows, L:] = extra[rows, :k - L]
    perm = np.argsort(g.random((T, k)), axis=1)
    idx = np.take_along_axis(idx, perm, axis=1)
    z = -np.sort(-g.standard_normal((T, k)), axis=1)
    z = np.exp(z - z[:, :1])
    gate = (z / z.sum(1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(idx), np.ascontiguousarray(gate)


def pool_workload(name: str, seed: int, n_partitions: int, part_rows: int, H: int, I: int,
                  E: int, k: int, expert_base: int, counts, x_std: float, w_std: float,
                  route_share: int, act_format: int = ACT_BF16, minibatches=(),
                  routing_seed: Optional[int] = None, macrobatch: int = 0,
                  base: Optional[Workload] = None) -> Workload:
    """Expert share fed by a pool of n_partitions x part_rows source tokens.

    The route step is exercised on this GPU's own share of source tokens:
    logits ~ N(0,1) fp32 [route_share, E].  ``base`` reuses an earlier
    workload's pool and weights (same seed) with a new routing seed.
    """
    n_local = len(counts)
    T = n_partitions * part_rows
    ss = np.random.SeedSequence(seed).spawn(4)
    if base is not None:
        x, w_gu, w_d = base.x, base.w_gu, base.w_d
    else:
        x = normal_bf16(ss[0], T * H, x_std).reshape(T, H)
        w_gu, w_d = _weights(ss[1], ss[2], n_local, H, I, w_std)
    rs = ss[3] if routing_seed is None else np.random.SeedSequence(routing_seed).spawn(4)[3]
    g = np.random.Generator(np.random.PCG64(rs))
    idx, gate = pool_routing(g, T, E, k, expert_base, counts)
    logits = g.standard_normal((route_share, E), dtype=np.float32)
    return Workload(name=name, seed=seed, T=T, H=H, I=I, E=E, k=k,
                    expert_base=expert_base, n_local=n_local,
                    n_partitions=n_partitions, part_rows=part_rows,
                    act_format=act_format, x=x, w_gu=w_gu, w_d=w_d, logits=logits,
                    topk_idx=idx, topk_gate=gate, minibatches=list(minibatches),
                    macrobatch=macrobatch)


# Local-expert loads for the skewed case: Zipf s = 1.2 over global expert
# ranks, this GPU holding the experts at ranks 1,2,3,4,6,8,10,12 of 8192
# routed rows (max/min about 20x).
ZIPF_COUNTS = [3715, 1617, 994, 704, 433, 306, 235, 188]
BALANCED_COUNTS = [1024] * 8
MINIBATCH_SWEEP = [512, 1024, 2368, 2560, 4096]


def tiny(seed: int = 1001) -> Workload:
    """T=256, hidden 256, 8 experts, top-2, intermediate 512; x, W ~ N(0, 0.02)."""
    return logits_workload("tiny_T256_H256_I512_E8_k2", seed, T=256, H=256, I=512, E=8,
                           k=2, x_std=0.02, w_std=0.02, minibatches=[512])


def mixtral(seed: int = 1002) -> Workload:
    """T=4096, hidden 4096, 8 experts, top-2, intermediate 14336, Gaussian router."""
    return logits_workload("mixtral_T4096_H4096_I14336_E8_k2", seed, T=4096, H=4096,
                           I=14336, E=8, k=2, x_std=1.0, w_std=0.02,
                           router="gaussian_weights", minibatches=[8192])


def kimi_share(seed: int = 1003, counts=None, act_format: int = ACT_BF16,
               name: str = "kimi_share_R8192_H7168_I2048_E384_k8_local8") -> Workload:
    """8192 routed rows from 72 source partitions of 1024 tokens; 8 of 384 experts."""
    counts = BALANCED_COUNTS if counts is None else counts
    return pool_workload(name, seed, n_partitions=72, part_rows=1024, H=7168, I=2048,
                         E=384, k=8, expert_base=40, counts=counts, x_std=1.0,
                         w_std=0.02, route_share=1024, act_format=act_format,
                         minibatches=MINIBATCH_SWEEP)


def kimi_zipf_mxfp8(seed: int = 1004) -> Workload:
    return kimi_share(seed, counts=ZIPF_COUNTS, act_format=ACT_MXFP8,
                      name="kimi_zipf_mxfp8_R8192_H7168_I2048_E384_k8_local8")


def kimi_full_mxfp8(seed: int = 1003, counts=None, name: str = "") -> Workload:
    """The Kimi-shaped share with MXFP8 activations and MXFP8 weights (both GEMMs on the
    block-scaled FP8 MFMA); balanced counts unless given."""
    counts = BALANCED_COUNTS if counts is None else counts
    wl = kimi_share(seed, counts=counts, act_format=ACT_MXFP8,
                    name=name or "kimi_full_mxfp8_R8192_H7168_I2048_E384_k8_local8")
    wl.weight_format = 1
    return wl


def kimi_zipf_full_mxfp8(seed: int = 1004) -> Workload:
    return kimi_full_mxfp8(seed, counts=ZIPF_COUNTS,
                           name="kimi_zipf_full_mxfp8_R8192_H7168_I2048_E384_k8_local8")


def streaming(n_macro: int = 8, seed: int = 1005) -> List[Workload]:
    """n_macro macrobatches sharing one pool and one set of weights."""
    first = kimi_share(seed, name="stream_m0")
    out = [first]
    for m in range(1, n_macro):
        out.append(pool_workload(f"stream_m{m}", seed, n_partitions=72, part_rows=1024,
                                 H=7168, I=2048, E=384, k=8, expert_base=40,
                                 counts=BALANCED_COUNTS, x_std=1.0, w_std=0.02,
                                 route_share=1024, minibatches=[2560],
                                 routing_seed=seed + 100 * m, macrobatch=m, base=first))
    return out


def small_pool(seed: int, n_partitions: int, part_rows: int, H: int, I: int, E: int, k: int,
               expert_base: int, counts, act_format: int = ACT_BF16,
               x_std: float = 1.0) -> Workload:
    """Scaled-down pool case for parity tests (ragged tiles, several partitions)."""
    return pool_workload(f"pool_P{n_partitions}x{part_rows}_H{H}_I{I}", seed, n_partitions,
                         part_rows, H, I, E, k, expert_base, counts, x_std=x_std,
                         w_std=0.02, route_share=min(256, n_partitions * part_rows),
                         act_format=act_format)
