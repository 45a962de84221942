"""The whole chain (score -> top-k -> sparse MLA) on the GPU against the oracle.

Small cases are compared in full. The five workloads run at full size in the launch
configuration the bench times: every sequence of the decode workloads, and for the chunked
prefill the first 64 queries, the last 64 and every 32nd, are compared with the oracle; every
row is checked for the properties a correct selection has at any size; the fused score ->
top-k call the bench times gives the same scores and indices as the two calls.
Rules: S1 scores within tolerance; S2 top-k fed the oracle's scores is bit-exact; S3 an
end-to-end index may differ only where its oracle score is within 1e-4 relative of the
k-th; S5 outputs within tolerance of the oracle evaluated on the GPU's own indices.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (RTOL, assert_rowwise, binding, check_guards, check_index_rule, check_topk_properties, dev,
                      guarded, guarded_workspace, host, run_chain, to_device_inputs)

pytestmark = pytest.mark.gpu
import torch  # noqa: E402


def _compare_rows(wl, inp, scores, idx, out, lse, sel_b, sel_i):
    """Oracle on sequences sel_b and queries sel_i only."""
    sl_q = np.asarray(sel_i)
    for b in sel_b:
        q = inp["q"][b:b + 1][:, sl_q]
        w = inp["w"][b:b + 1][:, sl_q]
        qp = inp["q_pos"][b:b + 1][:, sl_q]
        S = oracle.index_score(q, inp["k"][b:b + 1], w, inp["kv_len"][b:b + 1], qp, wl.scale,
                               wl.idx_dtype, wl.idx_dtype)
        g_s = scores[b:b + 1][:, sl_q]
        assert_rowwise(g_s, S, RTOL[wl.idx_dtype], f"{wl.name} scores b={b}")            # S1
        o_idx = oracle.topk(S.reshape(-1, wl.n_kv), wl.top_k).reshape(1, len(sl_q), wl.top_k)
        g_idx = idx[b:b + 1][:, sl_q]
        check_index_rule(g_idx, o_idx, S, f"{wl.name} idx b={b}")                         # S3
        o_out, o_lse = oracle.sparse_mla(inp["qa"][b:b + 1][:, sl_q], inp["latent"][b:b + 1], g_idx,
                                         wl.sm_scale, wl.d_latent, wl.mla_dtype, inp["kv_len"][b:b + 1])
        assert_rowwise(out[b:b + 1][:, sl_q], o_out, RTOL[wl.mla_dtype], f"{wl.name} out b={b}")  # S5
        assert_rowwise(lse[b:b + 1][:, sl_q], o_lse, RTOL[wl.mla_dtype], f"{wl.name} lse b={b}")
        yield b, S, o_idx


SMALL = [
    workloads.TINY_FP32,
    workloads.GLM_DECODE_8K.scaled(B=2, n_kv=3000, top_k=512),
    workloads.LONG_DECODE_128K.scaled(B=3, n_kv=5000, top_k=700),
    workloads.CHUNKED_PREFILL_16K.scaled(n_q=40, n_kv=900, q_pos_start=860 - 40, top_k=256),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name + "_small" for w in SMALL])
def test_chain_small(wl):
    L = binding()
    inp = workloads.gen_all(wl, 0)
    d = to_device_inputs(wl, inp)
    scores, idx, out, lse = (host(t) for t in run_chain(wl, d))
    for b, S, o_idx in _compare_rows(wl, inp, scores, idx, out, lse, range(wl.B), range(wl.n_q)):
        # S2: the selection kernel fed the oracle's scores returns the oracle's indices exactly
        g = torch.empty((wl.n_q, wl.top_k), dtype=torch.int32, device="cuda")
        L.dsa_topk(dev(np.ascontiguousarray(S.reshape(-1, wl.n_kv))), g, wl.top_k)
        torch.cuda.synchronize()
        assert np.array_equal(host(g), o_idx.reshape(-1, wl.top_k))


def _full(name, sel_b, sel_i):
    L = binding()
    wl = workloads.WORKLOADS[name]
    print(f"[full-size] {name}: generating inputs", flush=True)
    inp = workloads.gen_all(wl, 0)
    d = to_device_inputs(wl, inp)
    print(f"[full-size] {name}: running the chain", flush=True)
    scores_t, idx_t, out_t, lse_t = run_chain(wl, d)
    torch.cuda.synchronize()
    check_topk_properties(scores_t, idx_t, wl.top_k, name)
    # the fused score -> top-k call of the bench's step: the same scores and indices, bit for bit
    f_idx = guarded(tuple(idx_t.shape), torch.int32, fill=-3)
    f_sc = guarded(tuple(scores_t.shape), torch.float32, fill=-3.0)
    q_pos = d["q_pos"] if wl.q_pos_start is not None else None
    L.dsa_index_score_topk(d["q"], d["k"], d["w"], f_idx, wl.top_k, scores=f_sc, kv_len=d["kv_len"], q_pos=q_pos,
                           scale=wl.scale,
                           workspace=guarded_workspace(L.dsa_index_score_topk_workspace_size(
                               wl.B, wl.n_q, wl.H, wl.D, wl.n_kv, wl.top_k, wl.idx_dtype)))
    check_guards(f"{name} fused score -> top-k")
    assert torch.equal(f_sc.view(torch.int32), scores_t.view(torch.int32)), f"{name}: fused scores differ"
    assert torch.equal(f_idx, idx_t), f"{name}: fused indices differ"
    del f_idx, f_sc
    assert torch.isfinite(out_t).all() and torch.isfinite(lse_t).all()
    scores, idx, out, lse = (host(t) for t in (scores_t, idx_t, out_t, lse_t))
    print(f"[full-size] {name}: oracle on the sample", flush=True)
    rows = []
    for b, S, o_idx in _compare_rows(wl, inp, scores, idx, out, lse, sel_b, sel_i):
        rows.append((b, S, o_idx))
    # S2 in the same launch configuration: oracle rows substituted into the full score array
    mixed = scores.copy()
    for b, S, _ in rows:
        mixed[b][np.asarray(sel_i)] = S[0]
    g = torch.empty_like(idx_t)
    L.dsa_topk(dev(mixed), g, wl.top_k)
    torch.cuda.synchronize()
    g = host(g)
    for b, S, o_idx in rows:
        assert np.array_equal(g[b][np.asarray(sel_i)], o_idx[0]), f"{name}: S2 fails in sequence {b}"


def test_full_glm_decode_b1_8k():
    _full("glm_decode_b1_8k", [0], [0])


def test_full_batched_decode_b32_32k():
    _full("batched_decode_b32_32k", range(32), [0])


def test_full_long_decode_b8_128k():
    _full("long_decode_b8_128k", range(8), [0])


def test_full_chunked_prefill():
    # the first 64 queries, the last 64 and every 32nd (252 of the 4096)
    sel = sorted(set(range(64)) | set(range(4032, 4096)) | set(range(0, 4096, 32)))
    _full("chunked_prefill_4096_after_12288", [0], sel)


def test_full_tiny():
    _full("tiny_fp32_decode_256", [0], [0])


def test_indexshare_shared_layer_reuses_indices():
    """A shared layer (IndexShare) attends over the indices of the last full layer: its own
    queries and latent cache, the full layer's selection."""
    L = binding()
    wl = workloads.GLM_DECODE_8K.scaled(B=2, n_kv=3000, top_k=512)
    full = workloads.gen_all(wl, 0)
    shared = workloads.gen_all(wl, 1, parts=("qa", "latent"))
    d = to_device_inputs(wl, full)
    _, idx, _, _ = run_chain(wl, d)
    out = torch.empty((wl.B, wl.n_q, wl.Hm, wl.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((wl.B, wl.n_q, wl.Hm), dtype=torch.float32, device="cuda")
    src = L.dsa_topk_source_layer(5)
    assert L.dsa_layer_computes_topk(src) and not L.dsa_layer_computes_topk(5)
    L.dsa_sparse_mla_attn(dev(shared["qa"], wl.mla_dtype), dev(shared["latent"], wl.mla_dtype), idx, out,
                          wl.d_latent, wl.sm_scale, lse=lse, kv_len=d["kv_len"])
    torch.cuda.synchronize()
    o_out, o_lse = oracle.sparse_mla(shared["qa"], shared["latent"], host(idx), wl.sm_scale, wl.d_latent,
                                     wl.mla_dtype, full["kv_len"])
    assert_rowwise(host(out), o_out, RTOL[wl.mla_dtype], "shared layer out")
    assert_rowwise(host(lse), o_lse, RTOL[wl.mla_dtype], "shared layer lse")


@pytest.mark.parametrize("fused,B", [(False, 4), (True, 4), (True, 2)])
def test_graph_replays_match_eager(fused, B):
    """The chain captured in a HIP graph (how the bench times it) gives, on every replay, the
    bits of the eager run: the library records no memset nodes and keeps no state between
    calls. Eager work and synchronisations run between the replays. fused: the fused score ->
    top-k call and the attention (the bench's step); two sequences take 16 parts, whose merge
    gives each slot four threads."""
    L = binding()
    wl = workloads.BATCHED_DECODE_32K.scaled(B=B, n_kv=8192)
    inp = workloads.gen_all(wl, 3)
    d = to_device_inputs(wl, inp)
    rows = wl.B * wl.n_q
    ws_t = torch.empty(max(1, L.dsa_topk_workspace_size(rows, wl.n_kv, wl.top_k)), dtype=torch.uint8, device="cuda")
    ns = L.dsa_sparse_mla_num_splits(wl.B, wl.n_q, wl.top_k)
    ws_m = torch.empty(max(1, L.dsa_sparse_mla_workspace_size(wl.B, wl.n_q, wl.Hm, wl.top_k, wl.d_latent, ns)),
                       dtype=torch.uint8, device="cuda")
    scores = torch.empty((wl.B, wl.n_q, wl.n_kv), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.B, wl.n_q, wl.top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.B, wl.n_q, wl.Hm, wl.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((wl.B, wl.n_q, wl.Hm), dtype=torch.float32, device="cuda")

    ws_f = torch.empty(max(1, L.dsa_index_score_topk_workspace_size(wl.B, wl.n_q, wl.H, wl.D, wl.n_kv, wl.top_k,
                                                                      wl.idx_dtype)), dtype=torch.uint8, device="cuda")

    def step():
        if fused:
            L.dsa_index_score_topk(d["q"], d["k"], d["w"], idx, wl.top_k, scores=scores, kv_len=d["kv_len"],
                                   scale=wl.scale, workspace=ws_f)
        else:
            L.dsa_index_score(d["q"], d["k"], d["w"], scores, kv_len=d["kv_len"], scale=wl.scale)
            L.dsa_topk(scores, idx, wl.top_k, workspace=ws_t)
        L.dsa_sparse_mla_attn(d["qa"], d["latent"], idx, out, wl.d_latent, wl.sm_scale, lse=lse,
                              kv_len=d["kv_len"], n_split=ns, workspace=ws_m)

    step()
    torch.cuda.synchronize()
    ref = [host(t).copy() for t in (scores, idx, out, lse)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (scores, idx, out, lse):
            t.fill_(0)  # eager work between replays; the replay must rewrite everything
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("scores", "idx", "out", "lse"), (scores, idx, out, lse), ref):
            assert np.array_equal(host(t).view(np.uint32) if t.dtype != torch.int32 else host(t),
                                  r.view(np.uint32) if r.dtype != np.int32 else r), f"replay {rep}: {name}"
