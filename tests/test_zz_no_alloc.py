"""GPU test of mok_build_schedule_noalloc: the schedule with its scratch in
the library's fixed device array (for callers that cannot allocate) equals
mok_build_schedule with a caller workspace, bit for bit, on two calls in a
row -- the second with a smaller input, so stale contents of the array from
the first call would show."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import DeviceWorkload, gpu_schedule, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _noalloc(idx, T, k, base, n_local):
    import token_dispatch_grouped_top_amd as mok
    A = T * k
    counts = torch.full((n_local,), -3, dtype=torch.int32, device="cuda")
    offsets = torch.full((n_local + 1,), -3, dtype=torch.int32, device="cuda")
    soa = torch.full((max(A, 1),), -3, dtype=torch.int32, device="cuda")
    aos = torch.full((max(A, 1),), -7, dtype=torch.int32, device="cuda")
    mok.mok_build_schedule_noalloc(idx, T, k, base, n_local, counts, offsets, soa, aos)
    return dict(counts=counts, offsets=offsets, soa=soa, aos=aos)


def test_noalloc_schedule_matches_workspace_schedule_twice():
    big = W.kimi_share()                                   # 589,824 ids, 8 local experts
    small = W.small_pool(27, n_partitions=2, part_rows=300, H=128, I=128, E=16, k=4,
                         expert_base=3, counts=[100, 0, 250, 7, 60])
    for wl in (big, small):
        print(f"[no-alloc] {wl.name}: T={wl.T} k={wl.k} n_local={wl.n_local}", flush=True)
        dw = DeviceWorkload(wl)
        got = _noalloc(dw.topk_idx, wl.T, wl.k, wl.expert_base, wl.n_local)
        ref = gpu_schedule(dw.topk_idx, wl.T, wl.k, wl.expert_base, wl.n_local)
        torch.cuda.synchronize()
        for key in ("counts", "offsets", "soa"):
            assert torch.equal(got[key], ref[key]), (wl.name, key)
        R = int(to_host(ref["offsets"])[-1])
        assert torch.equal(got["aos"][:R], ref["aos"][:R])
        assert bool((got["aos"][R:] == -7).all())            # untouched past R
        orc = oracle.build_schedule(wl.topk_idx, wl.expert_base, wl.n_local)
        assert np.array_equal(to_host(got["aos"])[:R], orc["assign_of_slot"])
        del dw
