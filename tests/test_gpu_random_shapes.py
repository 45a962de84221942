"""Seeded random shapes through the whole path on the GPU against the oracle.

Twenty-four cases are drawn once from a fixed seed over the sizes the kernels branch on:
sequences, queries per sequence (decode rows and a few prefill-sized chunks), cached rows with
ragged kv_len, indexer heads, bf16 or f16 indexer, top_k below and above the valid rows, MLA
heads 16-64, 512- and 576-wide rows, and part counts (automatic, one, a few, sixteen). Each
case runs the three calls in the bench's launch configuration and the fused score -> top-k
call, and is checked by the chain's rules: S1 scores within tolerance, S3 indices by the
end-to-end rule, S5 outputs and lse within tolerance of the oracle on the GPU's indices, the
fused call equal to the three calls bit for bit, and no write past any output or workspace.
Three fixed cases add a batch holding an empty sequence (kv_len 0) beside a one-row and a full
one.
"""
import numpy as np
import pytest

import workloads
from gpu_util import (binding, check_guards, check_topk_properties, dev, guarded, guarded_workspace, host,
                      run_chain, to_device_inputs)
from test_gpu_chain import _compare_rows

pytestmark = pytest.mark.gpu
import torch  # noqa: E402


def _cases():
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(24):
        B = int(rng.integers(1, 5))
        n_q = int(rng.choice([1, 1, 1, 2, 3, 7, 9]))
        n_kv = int(rng.integers(max(n_q, 2), 6000))
        top_k = int(rng.choice([1, 16, 100, 513, 2048, 3000]))
        n_split = int(rng.choice([0, 0, 1, 3, 16]))
        if top_k > 2048 and n_split == 1:
            n_split = 0  # one part holds at most 2048 slots
        kv_len = rng.integers(n_q, n_kv + 1, size=B).astype(np.int32)
        kv_len[0] = n_kv  # one sequence fills the cache
        out.append(dict(i=i, B=B, n_q=n_q, n_kv=n_kv, H=int(rng.choice([8, 17, 32])), top_k=top_k,
                        Hm=int(rng.choice([16, 32, 48, 64])), d_rope=int(rng.choice([0, 64])),
                        idx_dtype=int(rng.choice([workloads.BF16, workloads.F16])), n_split=n_split,
                        kv_len=kv_len))
    return out


CASES = _cases()


# sequences with no cached row (a padded batch slot), one row, and a full cache, through the
# decode and the prefill-sized query counts
EDGE = [dict(i=100 + j, B=3, n_q=n_q, n_kv=3000, H=32, top_k=2048, Hm=64, d_rope=64, idx_dtype=workloads.BF16,
             n_split=0, kv_len=np.array([0, n_q, 3000], np.int32)) for j, n_q in enumerate((1, 2, 9))]
CASES = CASES + EDGE


@pytest.mark.parametrize("c", CASES, ids=[f"case{c['i']}_B{c['B']}_q{c['n_q']}_kv{c['n_kv']}_k{c['top_k']}"
                                          f"_Hm{c['Hm']}_r{c['d_rope']}_s{c['n_split']}" for c in CASES])
def test_random_shape(c):
    L = binding()
    wl = workloads.GLM_DECODE_8K.scaled(B=c["B"], n_q=c["n_q"], n_kv=c["n_kv"], H=c["H"], top_k=c["top_k"],
                                        Hm=c["Hm"], d_rope=c["d_rope"], idx_dtype=c["idx_dtype"])
    print(f"[random] case {c['i']}: B={wl.B} n_q={wl.n_q} n_kv={wl.n_kv} H={wl.H} top_k={wl.top_k} Hm={wl.Hm} "
          f"Dc={wl.Dc} dtype={wl.idx_dtype} n_split={c['n_split']} kv_len={c['kv_len'].tolist()}", flush=True)
    inp = workloads.gen_all(wl, 100 + c["i"])
    inp["kv_len"] = c["kv_len"]
    # the queries are the last n_q cached rows of each sequence (the default the calls apply)
    inp["q_pos"] = (c["kv_len"][:, None] - wl.n_q + np.arange(wl.n_q)[None, :]).astype(np.int32)
    d = to_device_inputs(wl, inp)
    scores_t, idx_t, out_t, lse_t = run_chain(wl, d, n_split=c["n_split"])
    check_topk_properties(scores_t, idx_t, wl.top_k, f"case {c['i']}")
    # the fused call: the same scores and indices
    f_idx = guarded(tuple(idx_t.shape), torch.int32, fill=-3)
    f_sc = guarded(tuple(scores_t.shape), torch.float32, fill=-3.0)
    L.dsa_index_score_topk(d["q"], d["k"], d["w"], f_idx, wl.top_k, scores=f_sc, kv_len=d["kv_len"], scale=wl.scale,
                           workspace=guarded_workspace(L.dsa_index_score_topk_workspace_size(
                               wl.B, wl.n_q, wl.H, wl.D, wl.n_kv, wl.top_k, wl.idx_dtype)))
    check_guards(f"case {c['i']} fused score -> top-k")
    assert torch.equal(f_sc.view(torch.int32), scores_t.view(torch.int32)), "fused scores differ"
    assert torch.equal(f_idx, idx_t), "fused indices differ"
    scores, idx, out, lse = (host(t) for t in (scores_t, idx_t, out_t, lse_t))
    for _ in _compare_rows(wl, inp, scores, idx, out, lse, range(wl.B), range(wl.n_q)):
        pass
    for b in np.nonzero(c["kv_len"] == 0)[0]:  # an empty sequence selects nothing and attends to nothing
        assert np.all(np.isneginf(scores[b])) and np.all(idx[b] == -1)
        assert np.all(out[b] == 0.0) and np.all(np.isneginf(lse[b]))
