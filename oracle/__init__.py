"""CPU oracle for the DSA hot path: indexer score -> top-k -> sparse absorbed MLA.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(``sparse_attention_10_amd``, the HIP kernels and the C ABI) never imports,
links or calls it, and shares no code with it.

Every function computes the plain definition of its step in float64 with
numpy (a matmul, an exp and a stable sort are the only library steps), with no
blocking, fusion or reordering beyond the definition, and rounds results to
float32 (round to nearest even) at the end. Inputs are decoded exactly: bf16
and f16 bit patterns convert exactly to float64.

Sources (web pages; cited by title and section):

* ik_llama_opt squash-commit log, sub-commit "Add GLM-5.2/DeepSeek-V3.2 DSA
  lightning indexer": the score is relu(k . q) per indexer head, scaled by the
  per-head weights, summed over heads, plus the causal mask; then top_k of
  min(top_k, n_tokens). The selection is used only as a set (a mask scatter).
* same log, "decode-correct via persistent indexer-K cache": queries are
  scored against all cached indexer keys; q and k are Hadamard-rotated, which
  leaves the scores unchanged; the selection is a descending argsort (same set).
* ds4 "hy3: Metal decode path" PR, GLM CPU oracle section: MLA over cached
  576-wide rows (512 latent + 64 already-rotated rope), score over qk_nope +
  qk_rope = 256 dims, one softmax over the candidate rows, values from the
  latent part.
* ds4 "Hy3 (295B): CUDA backend support" PR, online-softmax commit: the
  single-pass online softmax equals the two-pass one (split-K + merge here).

Readings where the pages are silent or garbled:
the indexer ``scale`` is an explicit factor applied after the head sum; relu
is applied per head before the weight; masked keys score exactly -inf; a
decode query sits at cache position kv_len - 1; NaN and -inf scores are never
selected and do not count as valid, +inf is valid; -0.0 equals +0.0; ties go
to the lower index and the selection is returned in ascending index order,
padded with -1; the attention value is the 512-wide latent part only; an
empty selection gives out = 0 and lse = -inf.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

F32, BF16, F16 = 0, 1, 2


# ----------------------------------------------------------------------------
# exact decoding of the storage dtypes
# ----------------------------------------------------------------------------
def decode(x: np.ndarray, dtype: int) -> np.ndarray:
    """Storage array -> float64, exactly. bf16/f16 arrive as uint16 bit patterns."""
    x = np.asarray(x)
    if dtype == F32:
        return x.astype(np.float64)
    if dtype == BF16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == F16:
        return x.view(np.float16).astype(np.float64)
    if dtype == -1:  # float64 passthrough, used by the invariance pins
        return x.astype(np.float64)
    raise ValueError(f"unknown dtype code {dtype}")


def _default_q_pos(kv_len: np.ndarray, n_q: int) -> np.ndarray:
    return (kv_len[:, None].astype(np.int64) - n_q + np.arange(n_q)[None, :])


# ----------------------------------------------------------------------------
# 1. lightning-indexer score
# ----------------------------------------------------------------------------
def index_score_f64(q, k, w, kv_len=None, q_pos=None, scale: float = 1.0,
                    q_dtype: int = F32, k_dtype: int = F32, block: int = 32) -> np.ndarray:
    """S[b,i,t] = scale * sum_h w[b,i,h] * max(0, sum_d q[b,i,h,d] * k[b,t,d]),
    and S = -inf where t > q_pos[b,i] or t >= kv_len[b].

    ik_llama_opt "DSA lightning indexer" sub-commit (score = relu(k.q) per
    head, scaled per-head weights, summed over heads, + causal mask) and the
    "persistent indexer-K cache" sub-commit (each query against every cached
    key). q [B][n_q][H][D], k [B][n_kv][D], w [B][n_q][H]; float64 result.
    """
    qd = decode(q, q_dtype)
    kd = decode(k, k_dtype)
    wd = np.asarray(w, dtype=np.float64)
    B, n_q, H, D = qd.shape
    n_kv = kd.shape[1]
    kv_len = np.full((B,), n_kv, np.int64) if kv_len is None else np.asarray(kv_len, np.int64)
    q_pos = _default_q_pos(kv_len, n_q) if q_pos is None else np.asarray(q_pos, np.int64)
    S = np.empty((B, n_q, n_kv), dtype=np.float64)
    t = np.arange(n_kv)
    for b in range(B):
        for i0 in range(0, n_q, block):
            i1 = min(n_q, i0 + block)
            # logits[i, h, t] = sum_d q[i,h,d] k[t,d]
            logits = (qd[b, i0:i1].reshape(-1, D) @ kd[b].T).reshape(i1 - i0, H, n_kv)
            per_head = np.maximum(logits, 0.0)                      # relu per head
            s = (wd[b, i0:i1, :, None] * per_head).sum(axis=1)      # weight, then head sum
            s = scale * s
            masked = (t[None, :] > q_pos[b, i0:i1, None]) | (t[None, :] >= kv_len[b])
            s[masked] = -np.inf
            S[b, i0:i1] = s
    return S


def index_score(q, k, w, kv_len=None, q_pos=None, scale: float = 1.0,
                q_dtype: int = F32, k_dtype: int = F32) -> np.ndarray:
    """The oracle score array: index_score_f64 rounded to float32 (nearest even)."""
    return index_score_f64(q, k, w, kv_len, q_pos, scale, q_dtype, k_dtype).astype(np.float32)


def index_score_sink(q, k, w, kv_len=None, q_pos=None, scale: float = 1.0, q_dtype: int = F32,
                     k_dtype: int = F32, sink_start=None, n_sink: int = 0, sink_boost: float = 1e20) -> np.ndarray:
    """index_score with the attention-sink boost: the float32 boost is added (in float32) to the
    float32 scores of keys sink_start[b] <= t < sink_start[b] + n_sink that are not masked
    (ik_llama_opt log: "DSA_SINK" force-inclusion, a boost so the sink always survives top-k;
    "per-sequence attention sink": only the query's own sequence's sink, as an additive F32
    input; "UPDATE 6": anchored on the sequence's first present position). sink_start [B] or
    None (0 for every sequence)."""
    S = index_score(q, k, w, kv_len, q_pos, scale, q_dtype, k_dtype)
    if n_sink <= 0:
        return S
    B, n_q, n_kv = S.shape
    start = np.zeros(B, np.int64) if sink_start is None else np.asarray(sink_start, np.int64)
    t = np.arange(n_kv)
    for b in range(B):
        in_sink = (t >= start[b]) & (t < start[b] + n_sink)
        # masked keys are -inf, and -inf + boost stays -inf
        S[b][:, in_sink] = S[b][:, in_sink] + np.float32(sink_boost)
    return S


# ----------------------------------------------------------------------------
# 2. top-k selection
# ----------------------------------------------------------------------------
def topk(scores: np.ndarray, top_k: int) -> np.ndarray:
    """Per row: the min(top_k, n_valid) largest valid scores.

    ik_llama_opt "DSA lightning indexer" sub-commit: top_k of
    min(top_k, n_tokens), used as a set. Rank by a stable sort on (score
    descending, index ascending) comparing values numerically (-0.0 == +0.0);
    NaN and -inf are not valid. The chosen indices are returned in ascending
    order and padded with -1 to top_k. scores [rows][n] float32 -> [rows][top_k] int32.
    """
    s = np.asarray(scores, dtype=np.float32)
    rows, n = s.shape
    out = np.full((rows, top_k), -1, dtype=np.int32)
    for r in range(rows):
        row = s[r]
        valid = np.nonzero(~np.isnan(row) & (row != -np.inf))[0]   # ascending indices
        order = valid[np.argsort(-row[valid], kind="stable")]      # ties keep ascending index
        K = min(top_k, valid.size)
        out[r, :K] = np.sort(order[:K])
    return out


# ----------------------------------------------------------------------------
# 3. sparse absorbed MLA over the selected latent rows
# ----------------------------------------------------------------------------
def _attend(qa_bi: np.ndarray, rows: np.ndarray, sm_scale: float, d_latent: int):
    """One query, all heads, over the given rows (float64).

    z[h,j] = sm_scale * qa[h,:] . row_j[:];  p = softmax_j(z);
    out[h,:] = sum_j p[h,j] * row_j[:d_latent];  lse[h] = log sum_j exp(z[h,j]).
    ds4 "hy3: Metal decode path" PR, GLM CPU oracle: one softmax over the
    candidate rows, score over the full 576 (latent + rope) row, values from
    the latent part.
    """
    Hm = qa_bi.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((Hm, d_latent)), np.full((Hm,), -np.inf)
    z = sm_scale * (qa_bi @ rows.T)                 # [Hm][J]
    M = z.max(axis=1, keepdims=True)
    e = np.exp(z - M)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    out = p @ rows[:, :d_latent]
    lse = M[:, 0] + np.log(l[:, 0])
    return out, lse


def sparse_mla_f64(qa, latent, idx, sm_scale: float, d_latent: int, dtype: int = F32,
                   kv_len=None) -> Tuple[np.ndarray, np.ndarray]:
    """qa [B][n_q][Hm][Dc], latent [B][n_kv][Dc], idx [B][n_q][top_k] int32.

    Index entries outside [0, kv_len[b]) (in particular the -1 padding) are
    skipped. Returns out [B][n_q][Hm][d_latent] and lse [B][n_q][Hm], float64.
    """
    idx = np.asarray(idx)
    B, n_q, Hm, Dc = qa.shape
    n_kv = latent.shape[1]
    kv_len = np.full((B,), n_kv, np.int64) if kv_len is None else np.asarray(kv_len, np.int64)
    out = np.zeros((B, n_q, Hm, d_latent))
    lse = np.zeros((B, n_q, Hm))
    for b in range(B):
        for i in range(n_q):
            sel = idx[b, i]
            sel = sel[(sel >= 0) & (sel < kv_len[b])]
            rows = decode(latent[b, sel], dtype)
            out[b, i], lse[b, i] = _attend(decode(qa[b, i], dtype), rows, sm_scale, d_latent)
    return out, lse


def sparse_mla(qa, latent, idx, sm_scale: float, d_latent: int, dtype: int = F32,
               kv_len=None) -> Tuple[np.ndarray, np.ndarray]:
    """sparse_mla_f64 rounded to float32."""
    out, lse = sparse_mla_f64(qa, latent, idx, sm_scale, d_latent, dtype, kv_len)
    return out.astype(np.float32), lse.astype(np.float32)


def dense_mla_f64(qa, latent, sm_scale: float, d_latent: int, dtype: int = F32,
                  kv_len=None, q_pos=None) -> Tuple[np.ndarray, np.ndarray]:
    """Dense causal MLA: every query attends to cache rows 0..q_pos[b,i] (< kv_len).

    Used only as a check: with top_k >= n_kv the sparse path must equal it
    (ik_llama_opt sub-commits report DSA-on identical to dense when
    top_k >= n_kv). Written head by head, independently of _attend.
    """
    B, n_q, Hm, Dc = qa.shape
    n_kv = latent.shape[1]
    kv_len = np.full((B,), n_kv, np.int64) if kv_len is None else np.asarray(kv_len, np.int64)
    q_pos = _default_q_pos(kv_len, n_q) if q_pos is None else np.asarray(q_pos, np.int64)
    out = np.zeros((B, n_q, Hm, d_latent))
    lse = np.full((B, n_q, Hm), -np.inf)
    for b in range(B):
        for i in range(n_q):
            last = min(int(q_pos[b, i]), int(kv_len[b]) - 1)
            if last < 0:
                continue
            rows = decode(latent[b, :last + 1], dtype)
            qb = decode(qa[b, i], dtype)
            for h in range(Hm):
                z = np.array([sm_scale * float(np.dot(qb[h], rows[j])) for j in range(rows.shape[0])])
                zmax = z.max()
                wts = np.exp(z - zmax)
                tot = wts.sum()
                out[b, i, h] = (wts[:, None] * rows[:, :d_latent]).sum(axis=0) / tot
                lse[b, i, h] = zmax + math.log(tot)
    return out, lse


def sparse_mla_split_merge_f64(qa, latent, idx, sm_scale: float, d_latent: int, dtype: int,
                               n_split: int, kv_len=None) -> Tuple[np.ndarray, np.ndarray]:
    """Split-K partials and their log-sum-exp merge, in float64.

    Split s covers index slots [s*c, (s+1)*c) with c = ceil(top_k / n_split):
    m_s = max z, l_s = sum exp(z - m_s), o_s = sum exp(z - m_s) row[:d_latent];
    merge: M = max_s m_s, L = sum_s exp(m_s - M) l_s,
    out = sum_s exp(m_s - M) o_s / L, lse = M + log L. Empty splits carry
    m = -inf, l = 0. ds4 "Hy3 (295B)" online-softmax commit: the running
    max/denominator rescale reproduces the single softmax.
    """
    idx = np.asarray(idx)
    B, n_q, Hm, Dc = qa.shape
    top_k = idx.shape[2]
    n_kv = latent.shape[1]
    kv_len = np.full((B,), n_kv, np.int64) if kv_len is None else np.asarray(kv_len, np.int64)
    c = -(-top_k // n_split)
    out = np.zeros((B, n_q, Hm, d_latent))
    lse = np.full((B, n_q, Hm), -np.inf)
    for b in range(B):
        for i in range(n_q):
            qb = decode(qa[b, i], dtype)
            ms, ls, os_ = [], [], []
            for s in range(n_split):
                sel = idx[b, i, s * c:(s + 1) * c]
                sel = sel[(sel >= 0) & (sel < kv_len[b])]
                if sel.size == 0:
                    ms.append(np.full((Hm,), -np.inf)); ls.append(np.zeros(Hm)); os_.append(np.zeros((Hm, d_latent)))
                    continue
                rows = decode(latent[b, sel], dtype)
                z = sm_scale * (qb @ rows.T)
                m = z.max(axis=1)
                e = np.exp(z - m[:, None])
                ms.append(m); ls.append(e.sum(axis=1)); os_.append(e @ rows[:, :d_latent])
            m_all = np.stack(ms)                      # [S][Hm]
            M = m_all.max(axis=0)
            if not np.isfinite(M).any():
                continue
            f = np.where(np.isfinite(m_all), np.exp(m_all - M[None, :]), 0.0)
            L = (f * np.stack(ls)).sum(axis=0)
            out[b, i] = (f[:, :, None] * np.stack(os_)).sum(axis=0) / L[:, None]
            lse[b, i] = M + np.log(L)
    return out, lse


# ----------------------------------------------------------------------------
# 4. indexer-input preparation: RoPE, Hadamard rotation, cache append
# ----------------------------------------------------------------------------
def encode(x64: np.ndarray, dtype: int) -> np.ndarray:
    """float64 -> storage: float32, or bf16 / f16 bit patterns (uint16), each by rounding
    to float32 first and then to the 16-bit format, to nearest even."""
    x32 = np.asarray(x64, np.float64).astype(np.float32)
    if dtype == F32:
        return x32
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x32.view(np.uint32).astype(np.uint64)
        out = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        out[np.isnan(x32)] = 0x7FC0
        return out
    raise ValueError(f"unknown dtype code {dtype}")


def rope_neox_f64(x: np.ndarray, pos: np.ndarray, rope_base: float, n_rope: int = 64) -> np.ndarray:
    """NeoX rotary embedding of the first n_rope dims of the last axis (ik_llama_opt log,
    "Add GLM-5.2/DeepSeek-V3.2 DSA lightning indexer": the indexer q and k are split into a
    64-dim rope part and a 64-dim nope part, the rope part is NeoX-roped, the two are
    concatenated again). NeoX pairs dim i with dim i + n_rope/2 (rotate-half):
        theta_i = pos * rope_base^(-2 i / n_rope),  i < n_rope / 2
        y_i = x_i cos theta_i - x_{i+h} sin theta_i,  y_{i+h} = x_{i+h} cos theta_i + x_i sin theta_i
    pos broadcasts against x[..., 0]; dims from n_rope on pass through."""
    x = np.asarray(x, np.float64)
    h = n_rope // 2
    i = np.arange(h, dtype=np.float64)
    theta = np.asarray(pos, np.float64)[..., None] * np.power(float(rope_base), -2.0 * i / n_rope)
    c, s = np.cos(theta), np.sin(theta)
    a, b = x[..., :h], x[..., h:n_rope]
    y = x.copy()
    y[..., :h] = a * c - b * s
    y[..., h:n_rope] = b * c + a * s
    return y


def hadamard_f64(x: np.ndarray) -> np.ndarray:
    """Orthonormal Walsh-Hadamard rotation of the last axis (ik_llama_opt log, "decode-correct
    via persistent indexer-K cache": the indexer q and k are Hadamard-rotated, which keeps
    (Hq).(Hk) = q.k). The matrix is Sylvester's, H_1 = [1], H_2n = [[H, H], [H, -H]], scaled
    by 1/sqrt(n); it is symmetric, so x H = H x per row."""
    x = np.asarray(x, np.float64)
    n = x.shape[-1]
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == n, "length must be a power of two"
    return x @ (H / math.sqrt(n))


def indexer_prep_f64(q_in, k_in, pos, rope_base: float, hadamard: bool = True):
    """Indexer inputs of the new tokens, before scoring: RoPE on the rope part, then the
    Hadamard rotation (same two log entries as above; the rotation acts on the roped vector).
    q_in [B][n][H][128], k_in [B][n][128] (either may be None), pos [B][n] the new tokens'
    positions. Returns (q, k) in float64."""
    pos = np.asarray(pos)
    q = k = None
    if q_in is not None:
        q = rope_neox_f64(q_in, pos[:, :, None], rope_base)
        if hadamard:
            q = hadamard_f64(q)
    if k_in is not None:
        k = rope_neox_f64(k_in, pos, rope_base)
        if hadamard:
            k = hadamard_f64(k)
    return q, k


def indexer_prep(q_in, k_in, pos, rope_base: float, out_dtype: int, hadamard: bool = True):
    """indexer_prep_f64 rounded to the cache dtype (see encode)."""
    q, k = indexer_prep_f64(q_in, k_in, pos, rope_base, hadamard)
    return (None if q is None else encode(q, out_dtype)), (None if k is None else encode(k, out_dtype))


def cache_append(cache: np.ndarray, rows: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """A copy of cache [B][n_kv][...] with row pos[b][i] replaced by rows[b][i] (ik_llama_opt
    log, "decode-correct via persistent indexer-K cache": the batch's indexer keys are
    written to the cache at kv_head; the same holds for the latent rows of the MLA cache).
    Positions outside [0, n_kv) write nothing."""
    out = np.array(cache, copy=True)
    pos = np.asarray(pos)
    for b in range(pos.shape[0]):
        for i in range(pos.shape[1]):
            p = int(pos[b, i])
            if 0 <= p < out.shape[1]:
                out[b, p] = rows[b, i]
    return out


# ----------------------------------------------------------------------------
# the whole chain, as one decode/prefill step of one DSA layer
# ----------------------------------------------------------------------------
def dsa_step(inp: dict, wl) -> dict:
    """Scores -> selection -> attention for one workload's inputs (see workloads.gen_all)."""
    S = index_score(inp["q"], inp["k"], inp["w"], inp["kv_len"], inp["q_pos"], wl.scale,
                    wl.idx_dtype, wl.idx_dtype)
    idx = topk(S.reshape(-1, S.shape[-1]), wl.top_k).reshape(wl.B, wl.n_q, wl.top_k)
    out, lse = sparse_mla(inp["qa"], inp["latent"], idx, wl.sm_scale, wl.d_latent, wl.mla_dtype,
                          inp["kv_len"])
    return {"scores": S, "idx": idx, "out": out, "lse": lse}


# ----------------------------------------------------------------------------
# 5. pooled (kpool) indexer: pool compression, pool scores, token selection
# ----------------------------------------------------------------------------
# vllm-rdna "Glm5Next (GLM-5.3-Flash) on gfx1030" PR, architecture section and the DSA
# attention and first-cut kernel commit bodies: the indexer cache holds one packed row per
# token (257 = k | gate | valid for 128-dim keys), groups of kpool = 4 tokens are compressed
# into one pool key with softmax(gate + ape) weights, queries score pool keys (relu per head,
# weighted head sum), top-k runs caller-side over pools, and the last incomplete pool (the
# tail, at most 3 tokens) is always selected, so 2048 selected tokens plus the tail give an
# attended width of 2051. Readings: the softmax runs per dimension over
# the pool's tokens, ape[j][d] is indexed by the token's slot j in its pool; a token whose
# valid entry is zero takes no part in its pool's softmax and is never attended; a pool with
# no valid token has the zero key; a pool is visible to a query once its last token is
# (kpool p + kpool - 1 <= pos and < kv_len); top_k counts tokens, so top_k / kpool pools
# are kept.
def packed_fields(packed, D: int, row_dtype: int):
    """Packed rows [B][n_kv][>= 2 D + 1] -> (k [B][n_kv][D], gate [B][n_kv][D], valid
    [B][n_kv] bool), decoded exactly. valid is any nonzero value (+0 and -0 are not valid)."""
    x = decode(packed, row_dtype)
    return x[..., :D], x[..., D:2 * D], x[..., 2 * D] != 0


def kpool_compress_f64(packed, ape, D: int, kpool: int, row_dtype: int) -> np.ndarray:
    """Pool keys [B][n_kv // kpool][D] in float64: for pool p and dim d, over the valid tokens
    t = kpool p + j of the pool, a = gate[t][d] + ape[j][d], wts = softmax_j(a),
    key[p][d] = sum_j wts_j k[t][d]. A pool with no valid token has the zero key."""
    k, gate, valid = packed_fields(packed, D, row_dtype)
    ape = np.asarray(ape, np.float64)
    B, n_kv = valid.shape
    n_pool = n_kv // kpool
    out = np.zeros((B, n_pool, D))
    for b in range(B):
        for p in range(n_pool):
            toks = [kpool * p + j for j in range(kpool) if valid[b, kpool * p + j]]
            if not toks:
                continue
            a = np.stack([gate[b, t] + ape[t - kpool * p] for t in toks])  # [n][D]
            e = np.exp(a - a.max(axis=0, keepdims=True))
            wts = e / e.sum(axis=0, keepdims=True)
            out[b, p] = (wts * np.stack([k[b, t] for t in toks])).sum(axis=0)
    return out


def kpool_compress(packed, ape, D: int, kpool: int, row_dtype: int, out_dtype: int) -> np.ndarray:
    """kpool_compress_f64 rounded to the pool-cache dtype (see encode)."""
    return encode(kpool_compress_f64(packed, ape, D, kpool, row_dtype), out_dtype)


def kpool_positions(kv_len, q_pos, n_q: int, kpool: int):
    """Token-level (kv_len [B], q_pos [B][n_q] or None) -> pool-level ones: pools wholly
    inside the cache, and the last pool whose final token is at or before the query."""
    kv_len = np.asarray(kv_len, np.int64)
    qp = _default_q_pos(kv_len, n_q) if q_pos is None else np.asarray(q_pos, np.int64)
    return kv_len // kpool, (qp + 1) // kpool - 1


def kpool_scores(q, pooled, w, kv_len, q_pos, scale: float, kpool: int, q_dtype: int, k_dtype: int):
    """Scores of every pool key [B][n_q][n_pool] fp32: the plain indexer score of section 1
    over the pool keys, with pool-level visibility (kpool_positions)."""
    n_q = np.asarray(q).shape[1]
    pl, pp = kpool_positions(kv_len, q_pos, n_q, kpool)
    return index_score(q, pooled, w, pl, pp, scale, q_dtype, k_dtype)


def kpool_select(pool_scores, packed_valid, kv_len, q_pos, top_k: int, kpool: int) -> np.ndarray:
    """Token indices [B][n_q][kpool * (top_k // kpool) + kpool - 1] int32: the top_k // kpool
    best pools (section 2's rule: ties to the lower pool, ascending, -1 padded), each
    expanded to its kpool tokens in order, then the tail tokens kpool * floor((pos + 1) /
    kpool) .. pos, always selected; -1 for padding, tokens whose valid entry is zero and
    tail slots past the query."""
    S = np.asarray(pool_scores)
    B, n_q, n_pool = S.shape
    kp = top_k // kpool
    width = kpool * kp + kpool - 1
    kv_len = np.asarray(kv_len, np.int64)
    qp = _default_q_pos(kv_len, n_q) if q_pos is None else np.asarray(q_pos, np.int64)
    pidx = topk(S.reshape(-1, n_pool), kp).reshape(B, n_q, kp)
    out = np.full((B, n_q, width), -1, np.int32)
    for b in range(B):
        for i in range(n_q):
            for s in range(kp):
                p = int(pidx[b, i, s])
                if p < 0:
                    continue
                for j in range(kpool):
                    t = kpool * p + j
                    if packed_valid[b, t]:
                        out[b, i, kpool * s + j] = t
            pos = int(qp[b, i])
            t0 = kpool * ((pos + 1) // kpool)
            for j in range(kpool - 1):
                t = t0 + j
                if 0 <= t <= pos and t < min(int(kv_len[b]), packed_valid.shape[1]) and packed_valid[b, t]:
                    out[b, i, kpool * kp + j] = t
    return out


def kpool_step(inp: dict, wl) -> dict:
    """The pooled chain of one decode step: compress every complete pool of the cache, score
    the pools, select tokens, attend (NoPE latent rows)."""
    pooled = kpool_compress(inp["packed"], inp["ape"], wl.D, wl.kpool, wl.idx_dtype, wl.idx_dtype)
    S = kpool_scores(inp["q"], pooled, inp["w"], inp["kv_len"], inp["q_pos"], wl.scale, wl.kpool,
                     wl.idx_dtype, wl.idx_dtype)
    _, _, valid = packed_fields(inp["packed"], wl.D, wl.idx_dtype)
    idx = kpool_select(S, valid, inp["kv_len"], inp["q_pos"], wl.top_k, wl.kpool)
    out, lse = sparse_mla(inp["qa"], inp["latent"], idx, wl.sm_scale, wl.d_latent, wl.mla_dtype,
                          inp["kv_len"])
    return {"pooled": pooled, "scores": S, "idx": idx, "out": out, "lse": lse}
