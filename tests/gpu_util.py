"""Helpers of the GPU parity tests: host arrays -> device tensors, the comparison rules,
and the whole chain through the C ABI in the launch configuration the bench uses."""
from __future__ import annotations

import numpy as np
import torch

import workloads

RTOL = {workloads.F32: 1e-5, workloads.BF16: 2e-3, workloads.F16: 2e-3}
EDGE_RTOL = 1e-4  # end-to-end index rule: oracle score within 1e-4 relative of the k-th


# Guard zones: outputs and workspaces of the parity tests are carved out of larger buffers
# whose first and last 4 KiB hold a canary byte; after the calls every canary must be intact,
# so a kernel that writes past either end of what it was given fails the test.
_GUARD = 4096
_CANARY = 0xA5
_guarded = []


def guarded(shape, dtype, fill=None) -> torch.Tensor:
    """A contiguous device tensor with 4 KiB of canary bytes before and after it (checked and
    forgotten by check_guards). fill: the tensor's own initial value (else the canary bytes)."""
    shape = tuple(int(x) for x in shape)
    es = torch.empty((), dtype=dtype).element_size()
    n = int(np.prod(shape)) if shape else 1
    raw = torch.full((n * es + 2 * _GUARD,), _CANARY, dtype=torch.uint8, device="cuda")
    t = raw[_GUARD:_GUARD + n * es].view(dtype).view(shape)
    if fill is not None:
        t.fill_(fill)
    _guarded.append(raw)
    return t


def guarded_workspace(nbytes: int) -> torch.Tensor:
    return guarded((max(1, int(nbytes)),), torch.uint8)


def check_guards(what: str) -> None:
    """Every canary zone handed out since the last check is intact."""
    torch.cuda.synchronize()
    bad = [i for i, raw in enumerate(_guarded)
           if not (bool((raw[:_GUARD] == _CANARY).all()) and bool((raw[-_GUARD:] == _CANARY).all()))]
    _guarded.clear()
    assert not bad, f"{what}: a kernel wrote past the end of an output or workspace ({len(bad)} buffers)"


def binding():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; none is visible")
    from sparse_attention_10_amd import dsa
    return dsa


def dev(a: np.ndarray, dtype_code: int = None) -> torch.Tensor:
    """numpy -> contiguous device tensor; uint16 arrays are bf16/f16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
        t = t.view(torch.bfloat16 if dtype_code == workloads.BF16 else torch.float16)
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_rowwise(got: np.ndarray, want: np.ndarray, rtol: float, what: str) -> None:
    """Per row (last axis): -inf pattern identical, max |g - o| <= rtol * max |o| over finite o."""
    g = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    o = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    assert g.shape == o.shape, f"{what}: shapes {g.shape} vs {o.shape}"
    fin = np.isfinite(o)
    bad_pattern = np.nonzero((np.isfinite(g) != fin).any(axis=1))[0]
    assert bad_pattern.size == 0, f"{what}: finite pattern differs in rows {bad_pattern[:5]}"
    assert np.array_equal(g[~fin], o[~fin]), f"{what}: non-finite values differ"
    err = np.where(fin, np.abs(g - np.where(fin, o, 0)), 0).max(axis=1)
    ref = np.where(fin, np.abs(np.where(fin, o, 0)), 0).max(axis=1)
    worst = np.argmax(err - rtol * ref)
    assert np.all(err <= rtol * ref + 1e-30), (
        f"{what}: row {worst}: max err {err[worst]:.3e} > {rtol:.1e} * {ref[worst]:.3e}")


def check_index_rule(gpu_idx: np.ndarray, ora_idx: np.ndarray, ora_scores: np.ndarray, what: str) -> None:
    """End-to-end selection rule: equal sizes; every index in the symmetric difference has an
    oracle score within 1e-4 relative of the oracle's K-th largest score."""
    gi = gpu_idx.reshape(-1, gpu_idx.shape[-1])
    oi = ora_idx.reshape(-1, ora_idx.shape[-1])
    sc = ora_scores.reshape(-1, ora_scores.shape[-1])
    for r in range(gi.shape[0]):
        a = gi[r][gi[r] >= 0]
        b = oi[r][oi[r] >= 0]
        assert a.size == b.size, f"{what}: row {r}: sizes {a.size} vs {b.size}"
        assert np.all(np.diff(a) > 0), f"{what}: row {r} not ascending"
        if a.size == 0:
            continue
        T = float(sc[r][b].min())
        diff = np.setxor1d(a, b)
        if diff.size:
            dev_ = np.abs(sc[r][diff].astype(np.float64) - T)
            assert np.all(dev_ <= EDGE_RTOL * abs(T)), (
                f"{what}: row {r}: index {diff[np.argmax(dev_)]} differs, |S - T| = {dev_.max():.3e}, T = {T:.6e}")


def check_topk_properties(scores: torch.Tensor, idx: torch.Tensor, top_k: int, what: str) -> None:
    """Properties of a correct selection that hold at any size (checked on the device):
    ascending distinct indices, size min(top_k, n_valid), every chosen score >= every unchosen
    valid score, and ties at the threshold resolved toward lower indices."""
    s = scores.reshape(-1, scores.shape[-1]).float()
    ix = idx.reshape(-1, idx.shape[-1]).long()
    rows, n = s.shape
    valid = ~(torch.isnan(s) | torch.isneginf(s))
    n_valid = valid.sum(dim=1)
    K = torch.clamp(n_valid, max=top_k)
    cnt = (ix >= 0).sum(dim=1)
    assert torch.equal(cnt, K), f"{what}: selection sizes differ from min(top_k, n_valid)"
    pos = torch.arange(top_k, device=ix.device)[None, :]
    assert torch.all((ix >= 0) == (pos < K[:, None])), f"{what}: -1 padding not at the end"
    d = ix[:, 1:] - ix[:, :-1]
    both = (ix[:, 1:] >= 0)
    assert torch.all(d[both] > 0), f"{what}: indices not ascending / distinct"
    # padding slots scatter into a spare column n that is dropped afterwards
    chosen = torch.zeros((rows, n + 1), dtype=torch.bool, device=s.device)
    safe = torch.where(ix >= 0, ix, torch.full_like(ix, n))
    chosen.scatter_(1, safe, torch.ones_like(safe, dtype=torch.bool))
    chosen = chosen[:, :n]
    # canonical value (-0 == +0) for comparisons
    sv = torch.where(valid, s + 0.0, torch.full_like(s, -float("inf")))
    min_chosen = torch.where(chosen, sv, torch.full_like(sv, float("inf"))).min(dim=1).values
    max_other = torch.where(valid & ~chosen, sv, torch.full_like(sv, -float("inf"))).max(dim=1).values
    has = K > 0
    assert torch.all(min_chosen[has] >= max_other[has]), f"{what}: an unchosen score beats a chosen one"
    tie = has & (min_chosen == max_other)
    if tie.any():
        ar = torch.arange(n, device=s.device)[None, :].expand(rows, n)
        last_tie_chosen = torch.where(chosen & (sv == min_chosen[:, None]), ar, torch.full_like(ar, -1)).max(dim=1).values
        first_tie_other = torch.where(valid & ~chosen & (sv == min_chosen[:, None]), ar, torch.full_like(ar, n)).min(dim=1).values
        assert torch.all(last_tie_chosen[tie] < first_tie_other[tie]), f"{what}: ties not resolved to lower index"


def run_chain(wl: workloads.Workload, d: dict, ws_topk=None, ws_mla=None, n_split: int = 0):
    """Scores -> top-k -> sparse MLA through the C ABI, default (bench) launch configuration."""
    L = binding()
    B, n_q = wl.B, wl.n_q
    scores = guarded((B, n_q, wl.n_kv), torch.float32)
    idx = guarded((B, n_q, wl.top_k), torch.int32)
    out = guarded((B, n_q, wl.Hm, wl.d_latent), torch.float32)
    lse = guarded((B, n_q, wl.Hm), torch.float32)
    if ws_topk is None:
        ws_topk = guarded_workspace(L.dsa_topk_workspace_size(B * n_q, wl.n_kv, wl.top_k))
    if ws_mla is None:
        ws_mla = guarded_workspace(L.dsa_sparse_mla_workspace_size(B, n_q, wl.Hm, wl.top_k, wl.d_latent, n_split))
    q_pos = d.get("q_pos") if wl.q_pos_start is not None else None
    L.dsa_index_score(d["q"], d["k"], d["w"], scores, kv_len=d.get("kv_len"), q_pos=q_pos, scale=wl.scale)
    L.dsa_topk(scores, idx, wl.top_k, workspace=ws_topk)
    L.dsa_sparse_mla_attn(d["qa"], d["latent"], idx, out, wl.d_latent, wl.sm_scale, lse=lse,
                          kv_len=d.get("kv_len"), n_split=n_split, workspace=ws_mla)
    check_guards(f"{wl.name} chain")
    return scores, idx, out, lse


def to_device_inputs(wl: workloads.Workload, inp: dict) -> dict:
    return {"q": dev(inp["q"], wl.idx_dtype), "k": dev(inp["k"], wl.idx_dtype), "w": dev(inp["w"]),
            "qa": dev(inp["qa"], wl.mla_dtype), "latent": dev(inp["latent"], wl.mla_dtype),
            "kv_len": dev(inp["kv_len"]), "q_pos": dev(inp["q_pos"])}
