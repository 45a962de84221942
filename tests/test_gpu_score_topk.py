"""dsa_index_score_topk (fused score -> top-k) on the GPU: its scores equal dsa_index_score's
bit for bit, its indices equal dsa_topk's over those scores bit for bit, and both meet the
oracle's rules (scores within the dtype's tolerance, indices by the end-to-end rule). Cases
cover the candidate path at the decode workloads' shapes, ragged caches and rows, several
queries per sequence, fewer heads, top_k above n_kv, rows whose answer sits in a few key
ranges (the re-read of a range), rows of nearly equal scores (a range's cut inside one 16-bit
bin) and rows of equal scores (the whole-row fallback)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (RTOL, assert_rowwise, binding, check_guards, check_index_rule, check_topk_properties, dev,
                      guarded, guarded_workspace, host)

pytestmark = pytest.mark.gpu
import torch  # noqa: E402


def _fused_vs_separate(wl, inp, top_k, kv_len=None, q_pos=None, scores_out=True, oracle_rows=None):
    L = binding()
    q, k, w = dev(inp["q"], wl.idx_dtype), dev(inp["k"], wl.idx_dtype), dev(inp["w"])
    kv = dev(np.asarray(kv_len, np.int32)) if kv_len is not None else None
    qp = dev(np.asarray(q_pos, np.int32)) if q_pos is not None else None
    B, n_q, n_kv = wl.B, wl.n_q, wl.n_kv
    idx = guarded((B, n_q, top_k), torch.int32, fill=-7)
    sc = guarded((B, n_q, n_kv), torch.float32, fill=3.0) if scores_out else None
    ws = guarded_workspace(L.dsa_index_score_topk_workspace_size(B, n_q, wl.H, wl.D, n_kv, top_k, wl.idx_dtype,
                                                                 not scores_out))
    L.dsa_index_score_topk(q, k, w, idx, top_k, scores=sc, kv_len=kv, q_pos=qp, scale=wl.scale, workspace=ws)
    ref_sc = guarded((B, n_q, n_kv), torch.float32, fill=5.0)
    L.dsa_index_score(q, k, w, ref_sc, kv_len=kv, q_pos=qp, scale=wl.scale)
    ref_idx = guarded((B, n_q, top_k), torch.int32, fill=-9)
    L.dsa_topk(ref_sc, ref_idx, top_k, workspace=guarded_workspace(L.dsa_topk_workspace_size(B * n_q, n_kv, top_k)))
    check_guards(f"{wl.name} fused score -> top-k")
    if sc is not None:
        assert torch.equal(sc.view(torch.int32), ref_sc.view(torch.int32)), "fused scores differ from dsa_index_score"
    g_idx = host(idx)
    assert np.array_equal(g_idx, host(ref_idx)), "fused indices differ from dsa_topk over the same scores"
    check_topk_properties(ref_sc, idx, top_k, "fused")
    rows = range(B) if oracle_rows is None else oracle_rows
    kvn = np.full(B, n_kv, np.int32) if kv_len is None else np.asarray(kv_len, np.int32)
    for b in rows:
        sl = slice(b, b + 1)
        want = oracle.index_score(inp["q"][sl], inp["k"][sl], inp["w"][sl], kvn[sl],
                                  None if q_pos is None else np.asarray(q_pos)[sl], wl.scale, wl.idx_dtype,
                                  wl.idx_dtype)
        assert_rowwise(host(ref_sc[sl]), want, RTOL[wl.idx_dtype], f"{wl.name} seq {b}")
        check_index_rule(g_idx[sl], oracle.topk(want.reshape(-1, n_kv), top_k).reshape(1, n_q, top_k), want,
                         f"{wl.name} seq {b}")
    return g_idx


DEC = workloads.GLM_DECODE_8K


def test_glm_decode_8k():
    wl = DEC
    _fused_vs_separate(wl, workloads.gen_all(wl, 0, parts=("q", "k", "w")), wl.top_k)


def test_batched_decode_32k_full_shape():
    """The batched workload's shape (32 x 32768, top-k 2048); sequences 0, 13 and 31 drawn from
    their own streams and compared with the oracle, the rest hold zero keys."""
    wl = workloads.BATCHED_DECODE_32K
    seqs = (0, 13, 31)
    parts = [workloads.gen_seq(wl, 0, b, ("q", "k", "w")) if b in seqs else None for b in range(wl.B)]
    z = {n: np.zeros_like(parts[0][n]) for n in ("q", "k", "w")}
    inp = {n: np.stack([(p if p is not None else z)[n] for p in parts]) for n in ("q", "k", "w")}
    _fused_vs_separate(wl, inp, wl.top_k, oracle_rows=seqs)


def test_long_decode_128k_shape():
    wl = workloads.LONG_DECODE_128K.scaled(B=2)
    _fused_vs_separate(wl, workloads.gen_all(wl, 3, parts=("q", "k", "w")), wl.top_k, oracle_rows=(1,))


@pytest.mark.parametrize("B,n_q,n_kv,H,top_k", [(1, 1, 1, 32, 1), (2, 1, 63, 32, 8), (3, 1, 1000, 32, 100),
                                                (1, 1, 4099, 17, 5000), (2, 3, 2113, 32, 500),
                                                (1, 7, 9000, 8, 2048), (4, 1, 20000, 32, 2048)])
def test_shapes(B, n_q, n_kv, H, top_k):
    wl = DEC.scaled(B=B, n_q=n_q, n_kv=n_kv, H=H)
    _fused_vs_separate(wl, workloads.gen_all(wl, B * 7 + n_q, parts=("q", "k", "w")), top_k)


def test_ragged_kv_len_and_positions_f16():
    wl = workloads.LONG_DECODE_128K.scaled(B=3, n_q=2, n_kv=12000)
    inp = workloads.gen_all(wl, 4, parts=("q", "k", "w"))
    kv = [12000, 7001, 300]
    qp = [[11998, 11999], [5000, 7000], [10, 299]]
    _fused_vs_separate(wl, inp, 2048, kv_len=kv, q_pos=qp)


def test_scores_kept_in_workspace():
    wl = DEC.scaled(B=3, n_kv=16384)
    _fused_vs_separate(wl, workloads.gen_all(wl, 8, parts=("q", "k", "w")), 2048, scores_out=False)


def test_concentrated_answer_rereads_ranges():
    """Keys 1000..1599 score far above the rest, so the waves holding them keep fewer keys than
    they hold of the answer: the selection re-reads those ranges."""
    wl = DEC.scaled(B=2, n_kv=16384)
    inp = workloads.gen_all(wl, 9, parts=("q", "k", "w"))
    k = oracle.decode(inp["k"], wl.idx_dtype)
    q = oracle.decode(inp["q"], wl.idx_dtype)
    k[:, 1000:1600] += 2.0 * q[:, 0, 0][:, None, :]   # aligned with head 0 of the query
    inp["k"] = workloads.round_to(k, wl.idx_dtype)
    inp["w"] = inp["w"].copy()
    inp["w"][:, :, 0] = 1.0
    _fused_vs_separate(wl, inp, 512)


def test_equal_scores_fall_back_to_whole_rows():
    """All scores equal (zero queries): every range is truncated at the threshold, the re-read set
    is the whole row; beyond one workgroup's capacity the streaming select takes over."""
    for n_kv in (5000, 20000):
        wl = DEC.scaled(B=2, n_kv=n_kv)
        inp = workloads.gen_all(wl, 10, parts=("q", "k", "w"))
        inp["q"] = np.zeros_like(inp["q"])
        idx = _fused_vs_separate(wl, inp, 2048)
        assert np.array_equal(idx[0, 0], np.arange(2048))  # ties go to the lowest indices


@pytest.mark.parametrize("noise", [0.002, 0.01, 0.05])
@pytest.mark.parametrize("B,n_kv", [(2, 16384), (8, 32768)])
def test_near_equal_scores_share_the_cut_bin(B, n_kv, noise):
    """Keys are one shared key plus a little noise, so scores differ by a fraction of a percent
    and most of a range's keys share the upper 16 bits of its m-th key: each range keeps part
    of that bin in index order, not by value (at 1 % noise every range's kept set differs from
    its m largest keys while the bin's top stays below the row's K-th key, checked with the
    oracle's scores on the host), or, at 0.2 %, every range's bound reaches that key and the
    ranges are re-read. The indices must still equal dsa_topk's."""
    wl = DEC.scaled(B=B, n_kv=n_kv)
    inp = workloads.gen_all(wl, 13, parts=("q", "k", "w"))
    k = oracle.decode(inp["k"], wl.idx_dtype)
    inp["k"] = workloads.round_to(k[:, :1, :] + noise * k, wl.idx_dtype)
    _fused_vs_separate(wl, inp, 2048, oracle_rows=(0,))


@pytest.mark.parametrize("B,n_kv", [(2, 16384), (2, 131072)])
def test_nonfinite_scores(B, n_kv):
    """Non-finite scores: sequence 0 weighs head 0 by +inf, so its scores are +inf where that
    head's relu is positive and NaN (inf x 0) where it is zero, many +inf ties and NaN (invalid)
    keys; sequence 1 holds key rows whose head-0 dot overflows to +inf among finite scores, and
    NaN key rows. The fused call's indices must equal dsa_topk's over the same scores (no oracle
    comparison: its rules are stated for finite inputs)."""
    L = binding()
    wl = DEC.scaled(B=B, n_kv=n_kv)
    inp = workloads.gen_all(wl, 15, parts=("q", "k", "w"))
    k = oracle.decode(inp["k"], wl.idx_dtype)
    rng = np.random.default_rng(15)
    rows = rng.choice(n_kv, size=64, replace=False)
    q0 = oracle.decode(inp["q"], wl.idx_dtype)[1, 0, 0, :]
    k[1, rows[:32]] = 1e38 * np.sign(q0)[None, :]  # head 0's dot overflows to +inf
    k[1, rows[32:]] = np.nan
    inp["k"] = workloads.round_to(k, wl.idx_dtype)
    w_np = inp["w"].copy()
    w_np[0, 0, 0] = np.inf
    q, kk, w = dev(inp["q"], wl.idx_dtype), dev(inp["k"], wl.idx_dtype), dev(w_np)
    idx = guarded((B, 1, 2048), torch.int32, fill=-7)
    sc = guarded((B, 1, n_kv), torch.float32, fill=3.0)
    L.dsa_index_score_topk(q, kk, w, idx, 2048, scores=sc, scale=wl.scale,
                           workspace=guarded_workspace(L.dsa_index_score_topk_workspace_size(
                               B, 1, wl.H, wl.D, n_kv, 2048, wl.idx_dtype)))
    ref_sc = guarded((B, 1, n_kv), torch.float32, fill=5.0)
    L.dsa_index_score(q, kk, w, ref_sc, scale=wl.scale)
    ref_idx = guarded((B, 1, 2048), torch.int32, fill=-9)
    L.dsa_topk(ref_sc, ref_idx, 2048, workspace=guarded_workspace(L.dsa_topk_workspace_size(B, n_kv, 2048)))
    check_guards("non-finite scores")
    h = host(ref_sc)
    print(f"[nonfinite] seq 0: +inf {int(np.isposinf(h[0]).sum())}, NaN {int(np.isnan(h[0]).sum())}; "
          f"seq 1: +inf {int(np.isposinf(h[1]).sum())}, NaN {int(np.isnan(h[1]).sum())}", flush=True)
    assert np.isposinf(h[0]).sum() > 2048 and np.isnan(h[0]).any(), "sequence 0 should hold +inf ties and NaN"
    assert np.isposinf(h[1]).any(), "sequence 1 should hold +inf scores"
    assert torch.equal(sc.view(torch.int32), ref_sc.view(torch.int32))
    assert torch.equal(idx, ref_idx), "fused indices differ from dsa_topk over the same scores"
    check_topk_properties(ref_sc, idx, 2048, "non-finite scores")
    g = host(idx)
    assert np.all(np.isposinf(h[0, 0, g[0, 0]])), "sequence 0 keeps +inf keys only"
    assert np.array_equal(g[0, 0], np.nonzero(np.isposinf(h[0, 0]))[0][:2048]), "+inf ties go to the lowest indices"


@pytest.mark.parametrize("kind", ["plain", "concentrated", "near_equal", "equal"])
def test_wide_select_128k_rows(kind):
    """Rows of 131072 keys: 1024 ranges of 12 candidates, more than 8192, so the select holds 16
    per thread. Plain rows, an answer concentrated in a few ranges (re-read), nearly equal scores
    (cut inside a 16-bit bin) and equal scores (re-read set larger than the workgroup: the
    streaming select)."""
    wl = workloads.LONG_DECODE_128K.scaled(B=2)
    inp = workloads.gen_all(wl, 14, parts=("q", "k", "w"))
    if kind == "concentrated":
        k = oracle.decode(inp["k"], wl.idx_dtype)
        q = oracle.decode(inp["q"], wl.idx_dtype)
        k[:, 70000:70600] += 2.0 * q[:, 0, 0][:, None, :]
        inp["k"] = workloads.round_to(k, wl.idx_dtype)
        inp["w"] = inp["w"].copy()
        inp["w"][:, :, 0] = 1.0
    elif kind == "near_equal":
        k = oracle.decode(inp["k"], wl.idx_dtype)
        inp["k"] = workloads.round_to(k[:, :1, :] + 0.01 * k, wl.idx_dtype)
    elif kind == "equal":
        inp["q"] = np.zeros_like(inp["q"])
    _fused_vs_separate(wl, inp, wl.top_k, oracle_rows=(0,))


@pytest.mark.parametrize("block", [256, 512, 1024])
def test_select_block_sizes(block):
    """Every select workgroup size gives the same answer, on the plain path, the re-read path and
    the whole-row fallback."""
    L = binding()
    L.dsa_set_tuning("topk_cand_block", block)
    try:
        wl = DEC.scaled(B=3, n_kv=16384)
        inp = workloads.gen_all(wl, 11, parts=("q", "k", "w"))
        _fused_vs_separate(wl, inp, 2048)
        k = oracle.decode(inp["k"], wl.idx_dtype)
        q = oracle.decode(inp["q"], wl.idx_dtype)
        k[:, 3000:3700] += 2.0 * q[:, 0, 0][:, None, :]
        inp2 = dict(inp, k=workloads.round_to(k, wl.idx_dtype), w=inp["w"].copy())
        inp2["w"][:, :, 0] = 1.0
        _fused_vs_separate(wl, inp2, 512)
        wl3 = DEC.scaled(B=2, n_kv=20000)
        inp3 = workloads.gen_all(wl3, 12, parts=("q", "k", "w"))
        inp3["q"] = np.zeros_like(inp3["q"])
        _fused_vs_separate(wl3, inp3, 2048)
    finally:
        L.dsa_set_tuning("topk_cand_block", 0)
