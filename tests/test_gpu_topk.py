"""dsa_topk on the GPU: bit-exact against the oracle when fed the same fp32 scores, on
every path (one workgroup per row, two-stage, filtered), with ties, signed zeros, NaN and
-inf, and inputs that push the filtered path into its whole-row fallback."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import binding, check_guards, check_topk_properties, dev, guarded, guarded_workspace, host

pytestmark = pytest.mark.gpu
import torch  # noqa: E402


@pytest.fixture(params=[1, 2, 3], ids=["one_pass", "two_stage", "filtered"])
def path(request):
    L = binding()
    L.dsa_set_tuning("topk_path", request.param)
    yield request.param
    L.dsa_set_tuning("topk_path", 0)


def _run(scores: np.ndarray, top_k: int):
    L = binding()
    rows, n = scores.shape
    idx = guarded((rows, top_k), torch.int32, fill=-7)
    s = dev(scores)
    L.dsa_topk(s, idx, top_k, workspace=guarded_workspace(L.dsa_topk_workspace_size(rows, n, top_k)))
    check_guards(f"top-k {rows} x {n}, k {top_k}")
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
    for p in (1, 2, 3, 0):
        L.dsa_set_tuning("topk_path", p)
        idx = torch.empty((8, 2048), dtype=torch.int32, device="cuda")
        L.dsa_topk(dev(s), idx, 2048)
        outs.append(host(idx))
    L.dsa_set_tuning("topk_path", 0)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert np.array_equal(outs[0], oracle.topk(s, 2048))


def test_oracle_scores_of_a_workload(path):
    wl = workloads.GLM_DECODE_8K.scaled(B=2, n_kv=9000)
    inp = workloads.gen_all(wl, 3, parts=("q", "k", "w"))
    S = oracle.index_score(inp["q"], inp["k"], inp["w"], None, None, 1.0, wl.idx_dtype, wl.idx_dtype)
    _run(S.reshape(-1, wl.n_kv), wl.top_k)


# The filtered path takes its threshold from a sample of the row: the whole row up to 2048
# entries, else 512 runs of 4 consecutive entries starting at floor(r * (n - 4) / 511).
def _sampled(n):
    if n <= 2048:
        return np.arange(n)
    r = np.arange(512, dtype=np.int64)
    return ((r * (n - 4)) // 511)[:, None] + np.arange(4)[None, :]


def test_filtered_sample_overestimates():
    """Sampled positions hold the largest scores, so the sample's threshold admits fewer than
    top_k entries of the row: the selection must come from the whole-row fallback."""
    L = binding()
    L.dsa_set_tuning("topk_path", 3)
    try:
        for n, top_k in [(32768, 2048), (131072, 2048), (20000, 1000)]:
            s = workloads.random_scores(4, n, seed=n)
            s[:, _sampled(n)] += 100.0
            _run(s, top_k)
    finally:
        L.dsa_set_tuning("topk_path", 0)


def test_filtered_sample_sees_no_valid():
    """Only unsampled positions are valid: the threshold falls to "every valid key", which is
    more candidates than one select holds, so the fallback runs; with few valid keys the
    candidates fit and the filtered select itself answers."""
    L = binding()
    L.dsa_set_tuning("topk_path", 3)
    try:
        n = 32768
        s = workloads.random_scores(3, n, seed=21, tie_frac=0.05)
        s[:, _sampled(n)] = -np.inf
        s[1, :] = -np.inf
        s[1, 5::97] = 1.5  # 338 valid, all tied
        s[2, 8000:] = np.nan
        _run(s, 2048)
    finally:
        L.dsa_set_tuning("topk_path", 0)


@pytest.mark.parametrize("rows,n,top_k", [(1, 8192, 2048), (32, 32768, 2048), (8, 131072, 2048),
                                          (3, 4097, 64), (200, 12000, 4096), (2, 2047, 100)])
def test_filtered_shapes(rows, n, top_k):
    L = binding()
    L.dsa_set_tuning("topk_path", 3)
    try:
        _run(workloads.random_scores(rows, n, seed=rows * n + top_k, tie_frac=0.01), top_k)
    finally:
        L.dsa_set_tuning("topk_path", 0)
