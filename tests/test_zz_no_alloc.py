"""dsa_topk_noalloc (the entry point for callers that cannot allocate) against dsa_topk with a
caller workspace: identical indices on two calls in a row, the second with a smaller input,
on shapes whose paths use scratch memory (the filtered path of few long rows, the two-stage
path when forced), and the oracle's selection for the same scores."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import binding, dev, host

pytestmark = pytest.mark.gpu
import torch  # noqa: E402


def _both(scores: np.ndarray, top_k: int):
    L = binding()
    rows, n = scores.shape
    need = L.dsa_topk_workspace_size(rows, n, top_k)
    assert 0 < need <= L.TOPK_NOALLOC_SCRATCH_BYTES, need
    s = dev(scores)
    a = torch.full((rows, top_k), -7, dtype=torch.int32, device="cuda")
    b = torch.full((rows, top_k), -9, dtype=torch.int32, device="cuda")
    L.dsa_topk_noalloc(s, a, top_k)
    L.dsa_topk(s, b, top_k, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    ga, gb = host(a), host(b)
    assert np.array_equal(ga, gb), "dsa_topk_noalloc differs from dsa_topk"
    want = oracle.topk(scores, top_k)
    bad = np.nonzero((ga != want).any(axis=1))[0]
    assert bad.size == 0, f"rows {bad[:4]} differ from the oracle"


@pytest.mark.parametrize("path", [0, 2], ids=["automatic", "two_stage"])
def test_noalloc_matches_workspace_call_twice(path):
    L = binding()
    L.dsa_set_tuning("topk_path", path)
    try:
        # first call: 32 rows x 32768 (the batched-decode top-k), then a smaller one; the
        # second reads scratch that still holds the first call's candidates
        big = workloads.random_scores(32, 32768, seed=41, tie_frac=0.05, neg_inf_frac=0.02)
        _both(big, 2048)
        small = workloads.random_scores(8, 16384, seed=42, quantize=0.125)
        _both(small, 1000)
    finally:
        L.dsa_set_tuning("topk_path", 0)


def test_noalloc_rejects_oversized_on_host():
    L = binding()
    rows, n, k = 256, 1 << 20, 2048
    assert L.dsa_topk_workspace_size(rows, n, k) > L.TOPK_NOALLOC_SCRATCH_BYTES
    s = torch.empty((1, n), dtype=torch.float32, device="cuda").expand(rows, n)
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    # the binding needs contiguous tensors: call the C entry point directly with the sizes
    st = L.lib.dsa_topk_noalloc(s.data_ptr(), idx.data_ptr(), rows, n, k, None)
    assert st == -5 and b"static array" in L.lib.dsa_last_error()
