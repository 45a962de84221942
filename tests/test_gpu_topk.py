"""dsa_topk on the GPU: bit-exact against the oracle when fed the same fp32 scores, on
both paths (one workgroup per row, two-stage), with ties, signed zeros, NaN and -inf."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import binding, check_topk_properties, dev, host

pytestmark = pytest.mark.gpu
import torch  # noqa: E402


@pytest.fixture(params=[1, 2], ids=["one_pass", "two_stage"])
def path(request):
    L = binding()
    L.dsa_set_tuning("topk_path", request.param)
    yield request.param
    L.dsa_set_tuning("topk_path", 0)


def _run(scores: np.ndarray, top_k: int):
    L = binding()
    rows, n = scores.shape
    idx = torch.full((rows, top_k), -7, dtype=torch.int32, device="cuda")
    s = dev(scores)
    L.dsa_topk(s, idx, top_k)
    torch.cuda.synchronize()
    got = host(idx)
    want = oracle.topk(scores, top_k)
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"rows {bad[:4]} differ; first: got {got[bad[0]][:8]} want {want[bad[0]][:8]}"
    check_topk_properties(s, idx, top_k, "topk")
    return got


@pytest.mark.parametrize("n", [1, 7, 63, 64, 65, 255, 256, 1000, 2049, 8192, 8193, 20000, 32768, 40000])
def test_sizes(path, n):
    for top_k in sorted({1, 64, min(n, 2048), n, n + 7}):
        _run(workloads.random_scores(3, n, seed=n + top_k), top_k)


@pytest.mark.parametrize("n,top_k", [(300, 64), (9000, 2048), (33000, 2048), (70000, 1000)])
def test_ties_signed_zeros_nan_neginf(path, n, top_k):
    s = workloads.random_scores(5, n, seed=11, tie_frac=0.2, neg_inf_frac=0.1, nan_frac=0.05)
    _run(s, top_k)
    q = workloads.random_scores(4, n, seed=12, quantize=0.25)  # few distinct values: long ties
    _run(q, top_k)


def test_all_invalid_and_few_valid(path):
    s = np.full((3, 5000), -np.inf, np.float32)
    s[1, [7, 4000]] = [0.5, -0.0]
    s[2, :] = np.nan
    s[2, 4999] = 1.0
    got = _run(s, 64)
    assert np.all(got[0] == -1)
    assert list(got[1][:3]) == [7, 4000, -1]


def test_many_rows_prefill_shape(path):
    # rows of a causal prefill: valid prefix lengths differ per row
    rows, n = 64, 16384
    s = workloads.random_scores(rows, n, seed=13)
    for r in range(rows):
        s[r, 12288 + r * 64 + 1:] = -np.inf
    _run(s, 2048)


def test_paths_agree_bitwise():
    L = binding()
    s = workloads.random_scores(8, 131072, seed=14, tie_frac=0.01)
    outs = []
    for p in (1, 2, 0):
        L.dsa_set_tuning("topk_path", p)
        idx = torch.empty((8, 2048), dtype=torch.int32, device="cuda")
        L.dsa_topk(dev(s), idx, 2048)
        outs.append(host(idx))
    L.dsa_set_tuning("topk_path", 0)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    assert np.array_equal(outs[0], oracle.topk(s, 2048))


def test_oracle_scores_of_a_workload(path):
    wl = workloads.GLM_DECODE_8K.scaled(B=2, n_kv=9000)
    inp = workloads.gen_all(wl, 3, parts=("q", "k", "w"))
    S = oracle.index_score(inp["q"], inp["k"], inp["w"], None, None, 1.0, wl.idx_dtype, wl.idx_dtype)
    _run(S.reshape(-1, wl.n_kv), wl.top_k)
