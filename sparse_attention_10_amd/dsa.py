"""ctypes binding of libdsa.so: the three DSA calls with the C names.

Argument marshalling only: each function checks dtypes, shapes and contiguity of the
torch tensors it is given, passes their device pointers and the current HIP stream to
the C ABI (include/dsa.h) and raises DsaError on a nonzero status. Every step of the
hot path runs in the HIP kernels of libdsa.so; there is no fallback. PyTorch only
provides device memory and the stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_F32, DSA_BF16, DSA_F16 = 0, 1, 2
_DTYPE = {torch.float32: DSA_F32, torch.bfloat16: DSA_BF16, torch.float16: DSA_F16}

EXPORTED = ("dsa_index_score", "dsa_index_score_sink", "dsa_topk_workspace_size", "dsa_topk", "dsa_sparse_mla_num_splits",
            "dsa_sparse_mla_workspace_size", "dsa_sparse_mla_attn", "dsa_indexer_prep", "dsa_layer_computes_topk", "dsa_topk_source_layer", "dsa_set_tuning",
            "dsa_kpool_compress", "dsa_kpool_index_score", "dsa_kpool_expand", "dsa_kpool_sparse_mla_attn",
            "dsa_topk_noalloc", "dsa_index_score_topk_workspace_size", "dsa_index_score_topk",
            "dsa_status_string", "dsa_last_error", "dsa_version")


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where} failed with status {status}: {detail}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_attention_10_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.dsa_index_score.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, P]
    lib.dsa_index_score.restype = I
    lib.dsa_index_score_sink.argtypes = [P, P, P, P, P, P, I, F, P, I, I, I, I, I, I, I, F, P]
    lib.dsa_index_score_sink.restype = I
    lib.dsa_topk_workspace_size.argtypes = [I, I, I]
    lib.dsa_topk_workspace_size.restype = S
    lib.dsa_topk.argtypes = [P, P, I, I, I, P, S, P]
    lib.dsa_topk.restype = I
    lib.dsa_topk_noalloc.argtypes = [P, P, I, I, I, P]
    lib.dsa_topk_noalloc.restype = I
    lib.dsa_index_score_topk_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
    lib.dsa_index_score_topk_workspace_size.restype = S
    lib.dsa_index_score_topk.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P, S, P]
    lib.dsa_index_score_topk.restype = I
    lib.dsa_sparse_mla_num_splits.argtypes = [I, I, I]
    lib.dsa_sparse_mla_num_splits.restype = I
    lib.dsa_sparse_mla_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.dsa_sparse_mla_workspace_size.restype = S
    lib.dsa_sparse_mla_attn.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P, S, P]
    lib.dsa_sparse_mla_attn.restype = I
    lib.dsa_indexer_prep.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P]
    lib.dsa_indexer_prep.restype = I
    lib.dsa_kpool_compress.argtypes = [P, I, I, P, P, I, I, I, I, I, I, I, P]
    lib.dsa_kpool_compress.restype = I
    lib.dsa_kpool_index_score.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P]
    lib.dsa_kpool_index_score.restype = I
    lib.dsa_kpool_expand.argtypes = [P, P, I, I, I, P, P, P, I, I, I, I, I, P]
    lib.dsa_kpool_expand.restype = I
    lib.dsa_kpool_sparse_mla_attn.argtypes = [P, P, P, P, I, I, I, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, P,
                                              S, P]
    lib.dsa_kpool_sparse_mla_attn.restype = I
    lib.dsa_layer_computes_topk.argtypes = [I]
    lib.dsa_layer_computes_topk.restype = I
    lib.dsa_topk_source_layer.argtypes = [I]
    lib.dsa_topk_source_layer.restype = I
    lib.dsa_set_tuning.argtypes = [ctypes.c_char_p, I]
    lib.dsa_set_tuning.restype = I
    lib.dsa_status_string.argtypes = [I]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_version.argtypes = []
    lib.dsa_version.restype = I
    return lib


lib = _load()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DsaError(status, where, lib.dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _opt(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape) -> None:
    """An optional device tensor of exactly this dtype and shape (or None)."""
    if t is None:
        return
    _dev(t, name)
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)} (got {t.dtype} {tuple(t.shape)})")


def _workspace_bytes(workspace: Optional[torch.Tensor]) -> int:
    if workspace is None:
        return 0
    _dev(workspace, "workspace")
    return workspace.numel() * workspace.element_size()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def dsa_index_score(q: torch.Tensor, k_cache: torch.Tensor, w: torch.Tensor, scores: torch.Tensor,
                    kv_len: Optional[torch.Tensor] = None, q_pos: Optional[torch.Tensor] = None,
                    scale: float = 1.0, stream=None, n_sink: int = 0,
                    sink_start: Optional[torch.Tensor] = None, sink_boost: float = 1e20) -> torch.Tensor:
    """q [B][n_q][H][D], k_cache [B][n_kv][D] (same dtype), w [B][n_q][H] fp32,
    scores [B][n_q][n_kv] fp32 (output); kv_len [B] / q_pos [B][n_q] int32 or None.
    n_sink > 0 adds sink_boost to the first n_sink keys from sink_start [B] int32 (or 0)."""
    B, n_q, H, D = q.shape
    n_kv = k_cache.shape[1]
    for t, n in ((q, "q"), (k_cache, "k_cache"), (w, "w"), (scores, "scores")):
        _dev(t, n)
    if tuple(k_cache.shape) != (B, n_kv, D) or tuple(w.shape) != (B, n_q, H) \
            or tuple(scores.shape) != (B, n_q, n_kv):
        raise ValueError("dsa_index_score: inconsistent shapes")
    if w.dtype != torch.float32 or scores.dtype != torch.float32:
        raise ValueError("w and scores must be float32")
    _opt(kv_len, "kv_len", torch.int32, (B,))
    _opt(q_pos, "q_pos", torch.int32, (B, n_q))
    if n_sink:
        if sink_start is not None:
            _dev(sink_start, "sink_start")
            if sink_start.dtype != torch.int32 or tuple(sink_start.shape) != (B,):
                raise ValueError("sink_start must be int32 [B]")
        _check(lib.dsa_index_score_sink(q.data_ptr(), k_cache.data_ptr(), w.data_ptr(), _ptr(kv_len),
                                        _ptr(q_pos), _ptr(sink_start), int(n_sink), float(sink_boost),
                                        scores.data_ptr(), B, n_q, H, D, n_kv, _DTYPE[q.dtype],
                                        _DTYPE[k_cache.dtype], float(scale), _stream(stream)), "dsa_index_score_sink")
        return scores
    _check(lib.dsa_index_score(q.data_ptr(), k_cache.data_ptr(), w.data_ptr(), _ptr(kv_len), _ptr(q_pos),
                               scores.data_ptr(), B, n_q, H, D, n_kv, _DTYPE[q.dtype], _DTYPE[k_cache.dtype],
                               float(scale), _stream(stream)), "dsa_index_score")
    return scores


def dsa_index_score_topk_workspace_size(B: int, n_q: int, H: int, D: int, n_kv: int, top_k: int, dtype,
                                        scores_in_workspace: bool = False) -> int:
    code = _DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib.dsa_index_score_topk_workspace_size(B, n_q, H, D, n_kv, top_k, code, 1 if scores_in_workspace else 0))


def dsa_index_score_topk(q: torch.Tensor, k_cache: torch.Tensor, w: torch.Tensor, idx: torch.Tensor, top_k: int,
                         scores: Optional[torch.Tensor] = None, kv_len: Optional[torch.Tensor] = None,
                         q_pos: Optional[torch.Tensor] = None, scale: float = 1.0,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Scores and top-k in one call: q [B][n_q][H][D], k_cache [B][n_kv][D] (same dtype), w [B][n_q][H]
    fp32, idx [B][n_q][top_k] int32 (output); scores [B][n_q][n_kv] fp32 (output) or None (kept in
    the workspace); kv_len [B] / q_pos [B][n_q] int32 or None."""
    B, n_q, H, D = q.shape
    n_kv = k_cache.shape[1]
    for t, n in ((q, "q"), (k_cache, "k_cache"), (w, "w"), (idx, "idx")):
        _dev(t, n)
    if tuple(k_cache.shape) != (B, n_kv, D) or tuple(w.shape) != (B, n_q, H) \
            or tuple(idx.shape) != (B, n_q, top_k) or idx.dtype != torch.int32 or w.dtype != torch.float32:
        raise ValueError("dsa_index_score_topk: inconsistent shapes or dtypes")
    _opt(scores, "scores", torch.float32, (B, n_q, n_kv))
    _opt(kv_len, "kv_len", torch.int32, (B,))
    _opt(q_pos, "q_pos", torch.int32, (B, n_q))
    need = dsa_index_score_topk_workspace_size(B, n_q, H, D, n_kv, top_k, q.dtype, scores is None)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.dsa_index_score_topk(q.data_ptr(), k_cache.data_ptr(), w.data_ptr(), _ptr(kv_len), _ptr(q_pos),
                                    _ptr(scores), idx.data_ptr(), B, n_q, H, D, n_kv, int(top_k), _DTYPE[q.dtype],
                                    _DTYPE[k_cache.dtype], float(scale), workspace.data_ptr(),
                                    _workspace_bytes(workspace), _stream(stream)), "dsa_index_score_topk")
    return idx


def dsa_topk_workspace_size(rows: int, n_kv: int, top_k: int) -> int:
    return int(lib.dsa_topk_workspace_size(rows, n_kv, top_k))


def dsa_topk(scores: torch.Tensor, idx: torch.Tensor, top_k: int,
             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """scores [rows][n_kv] fp32 (any leading shape, flattened), idx [rows][top_k] int32 (output)."""
    _dev(scores, "scores")
    _dev(idx, "idx")
    n_kv = scores.shape[-1]
    rows = scores.numel() // n_kv
    if idx.numel() != rows * top_k or idx.dtype != torch.int32 or scores.dtype != torch.float32:
        raise ValueError("dsa_topk: idx must be int32 [rows][top_k], scores float32")
    need = dsa_topk_workspace_size(rows, n_kv, top_k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wbytes = _workspace_bytes(workspace)
    _check(lib.dsa_topk(scores.data_ptr(), idx.data_ptr(), rows, n_kv, top_k, _ptr(workspace), wbytes,
                        _stream(stream)), "dsa_topk")
    return idx


TOPK_NOALLOC_SCRATCH_BYTES = 16 << 20  # DSA_TOPK_NOALLOC_SCRATCH_BYTES


def dsa_topk_noalloc(scores: torch.Tensor, idx: torch.Tensor, top_k: int, stream=None) -> torch.Tensor:
    """dsa_topk without a workspace: the library's static per-GPU scratch array is used, and
    nothing is allocated (for callers under graph capture or that cannot allocate). Calls that
    overlap on one GPU share that array and race."""
    _dev(scores, "scores")
    _dev(idx, "idx")
    n_kv = scores.shape[-1]
    rows = scores.numel() // n_kv
    if idx.numel() != rows * top_k or idx.dtype != torch.int32 or scores.dtype != torch.float32:
        raise ValueError("dsa_topk_noalloc: idx must be int32 [rows][top_k], scores float32")
    _check(lib.dsa_topk_noalloc(scores.data_ptr(), idx.data_ptr(), rows, n_kv, top_k, _stream(stream)),
           "dsa_topk_noalloc")
    return idx


def dsa_sparse_mla_num_splits(B: int, n_q: int, top_k: int) -> int:
    return int(lib.dsa_sparse_mla_num_splits(B, n_q, top_k))


def dsa_sparse_mla_workspace_size(B: int, n_q: int, Hm: int, top_k: int, d_latent: int, n_split: int) -> int:
    return int(lib.dsa_sparse_mla_workspace_size(B, n_q, Hm, top_k, d_latent, n_split))


def dsa_sparse_mla_attn(q_abs: torch.Tensor, latent: torch.Tensor, idx: torch.Tensor, out: torch.Tensor,
                        d_latent: int, sm_scale: float, lse: Optional[torch.Tensor] = None,
                        kv_len: Optional[torch.Tensor] = None, n_split: int = 0,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q_abs [B][n_q][Hm][Dc], latent [B][n_kv][Dc] (same dtype), idx [B][n_q][top_k] int32,
    out [B][n_q][Hm][d_latent] fp32 (output), lse [B][n_q][Hm] fp32 or None."""
    B, n_q, Hm, Dc = q_abs.shape
    n_kv = latent.shape[1]
    top_k = idx.shape[-1]
    for t, n in ((q_abs, "q_abs"), (latent, "latent"), (idx, "idx"), (out, "out")):
        _dev(t, n)
    if tuple(latent.shape) != (B, n_kv, Dc) or tuple(idx.shape) != (B, n_q, top_k) \
            or tuple(out.shape) != (B, n_q, Hm, d_latent) or latent.dtype != q_abs.dtype:
        raise ValueError("dsa_sparse_mla_attn: inconsistent shapes or dtypes")
    if idx.dtype != torch.int32 or out.dtype != torch.float32:
        raise ValueError("idx must be int32 and out float32")
    _opt(lse, "lse", torch.float32, (B, n_q, Hm))
    _opt(kv_len, "kv_len", torch.int32, (B,))
    need = dsa_sparse_mla_workspace_size(B, n_q, Hm, top_k, d_latent, n_split)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_abs.device)
    wbytes = _workspace_bytes(workspace)
    _check(lib.dsa_sparse_mla_attn(q_abs.data_ptr(), latent.data_ptr(), idx.data_ptr(), _ptr(kv_len),
                                   out.data_ptr(), _ptr(lse), B, n_q, Hm, n_kv, top_k, d_latent,
                                   Dc - d_latent, float(sm_scale), _DTYPE[q_abs.dtype], int(n_split),
                                   _ptr(workspace), wbytes, _stream(stream)), "dsa_sparse_mla_attn")
    return out


def dsa_indexer_prep(pos: torch.Tensor, q_in: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                     k_in: Optional[torch.Tensor] = None, k_cache: Optional[torch.Tensor] = None,
                     latent_in: Optional[torch.Tensor] = None, latent_cache: Optional[torch.Tensor] = None,
                     rope_base: float = 10000.0, hadamard: bool = True, stream=None) -> None:
    """pos [B][n_new] int32; q_in [B][n_new][H][128] fp32 -> q_out (same shape, bf16/f16/fp32);
    k_in [B][n_new][128] fp32 -> rows pos of k_cache [B][n_kv][128]; latent_in [B][n_new][R]
    -> rows pos of latent_cache [B][n_kv][R] (copied)."""
    _dev(pos, "pos")
    if pos.dtype != torch.int32 or pos.dim() != 2:
        raise ValueError("pos must be int32 [B][n_new]")
    B, n_new = pos.shape
    H, n_kv, row_bytes, out_dtype = 1, None, 0, None
    if (q_in is None) != (q_out is None) or (k_in is None) != (k_cache is None) \
            or (latent_in is None) != (latent_cache is None):
        raise ValueError("dsa_indexer_prep: inputs and outputs come in pairs")
    if q_in is not None:
        _dev(q_in, "q_in"); _dev(q_out, "q_out")
        if q_in.dtype != torch.float32 or tuple(q_in.shape[:2]) != (B, n_new) or q_in.shape[-1] != 128 \
                or q_in.dim() != 4 or tuple(q_out.shape) != tuple(q_in.shape):
            raise ValueError("q_in must be fp32 [B][n_new][H][128] and q_out of the same shape")
        H = q_in.shape[2]
        out_dtype = _DTYPE[q_out.dtype]
    if k_in is not None:
        _dev(k_in, "k_in"); _dev(k_cache, "k_cache")
        if k_in.dtype != torch.float32 or tuple(k_in.shape) != (B, n_new, 128) or k_cache.dim() != 3 \
                or k_cache.shape[0] != B or k_cache.shape[2] != 128:
            raise ValueError("k_in must be fp32 [B][n_new][128], k_cache [B][n_kv][128]")
        if out_dtype is not None and _DTYPE[k_cache.dtype] != out_dtype:
            raise ValueError("q_out and k_cache must share a dtype")
        out_dtype = _DTYPE[k_cache.dtype]
        n_kv = k_cache.shape[1]
    if latent_in is not None:
        _dev(latent_in, "latent_in"); _dev(latent_cache, "latent_cache")
        if latent_in.dim() != 3 or tuple(latent_in.shape[:2]) != (B, n_new) or latent_cache.dim() != 3 \
                or latent_cache.shape[0] != B or latent_cache.shape[2] != latent_in.shape[2] \
                or latent_cache.dtype != latent_in.dtype:
            raise ValueError("latent_in [B][n_new][R] and latent_cache [B][n_kv][R] of one dtype")
        if n_kv is not None and latent_cache.shape[1] != n_kv:
            raise ValueError("k_cache and latent_cache must have the same n_kv")
        n_kv = latent_cache.shape[1]
        row_bytes = latent_in.shape[2] * latent_in.element_size()
    if n_kv is None:
        n_kv = 1
    _check(lib.dsa_indexer_prep(_ptr(q_in), _ptr(k_in), _ptr(latent_in), pos.data_ptr(), _ptr(q_out),
                                _ptr(k_cache), _ptr(latent_cache), B, n_new, H, n_kv, row_bytes,
                                DSA_BF16 if out_dtype is None else out_dtype, float(rope_base),
                                1 if hadamard else 0, _stream(stream)), "dsa_indexer_prep")


def dsa_layer_computes_topk(layer: int) -> bool:
    r = lib.dsa_layer_computes_topk(int(layer))
    if r < 0:
        _check(r, "dsa_layer_computes_topk")
    return r == 1


def dsa_topk_source_layer(layer: int) -> int:
    r = lib.dsa_topk_source_layer(int(layer))
    if r < 0:
        _check(r, "dsa_topk_source_layer")
    return r


def dsa_set_tuning(key: str, value: int) -> None:
    _check(lib.dsa_set_tuning(key.encode(), int(value)), "dsa_set_tuning")


def dsa_kpool_compress(packed: torch.Tensor, ape: torch.Tensor, pooled: torch.Tensor, D: int, kpool: int,
                       pool_begin: int = 0, pool_end: Optional[int] = None, stream=None) -> torch.Tensor:
    """packed [B][n_kv][row_stride] (k | gate | valid, row_stride >= 2 D + 1), ape [kpool][D] fp32,
    pooled [B][n_kv // kpool][D] (output; pools [pool_begin, pool_end) are written)."""
    B, n_kv, stride = packed.shape
    for t, n in ((packed, "packed"), (ape, "ape"), (pooled, "pooled")):
        _dev(t, n)
    if tuple(ape.shape) != (kpool, D) or ape.dtype != torch.float32 or tuple(pooled.shape) != (B, n_kv // kpool, D):
        raise ValueError("dsa_kpool_compress: inconsistent shapes or dtypes")
    end = n_kv // kpool if pool_end is None else pool_end
    _check(lib.dsa_kpool_compress(packed.data_ptr(), stride, _DTYPE[packed.dtype], ape.data_ptr(), pooled.data_ptr(),
                                  _DTYPE[pooled.dtype], B, n_kv, D, kpool, int(pool_begin), int(end),
                                  _stream(stream)), "dsa_kpool_compress")
    return pooled


def dsa_kpool_index_score(q: torch.Tensor, pooled: torch.Tensor, w: torch.Tensor, scores: torch.Tensor, kpool: int,
                          kv_len: Optional[torch.Tensor] = None, q_pos: Optional[torch.Tensor] = None,
                          scale: float = 1.0, stream=None) -> torch.Tensor:
    """q [B][n_q][H][D], pooled [B][n_pool][D] (same dtype), w [B][n_q][H] fp32, scores [B][n_q][n_pool]
    fp32 (output); kv_len [B] and q_pos [B][n_q] int32 in tokens, or None."""
    B, n_q, H, D = q.shape
    n_pool = pooled.shape[1]
    for t, n in ((q, "q"), (pooled, "pooled"), (w, "w"), (scores, "scores")):
        _dev(t, n)
    if tuple(pooled.shape) != (B, n_pool, D) or tuple(w.shape) != (B, n_q, H) \
            or tuple(scores.shape) != (B, n_q, n_pool) or w.dtype != torch.float32 or scores.dtype != torch.float32:
        raise ValueError("dsa_kpool_index_score: inconsistent shapes or dtypes")
    _opt(kv_len, "kv_len", torch.int32, (B,))
    _opt(q_pos, "q_pos", torch.int32, (B, n_q))
    _check(lib.dsa_kpool_index_score(q.data_ptr(), pooled.data_ptr(), w.data_ptr(), _ptr(kv_len), _ptr(q_pos),
                                     scores.data_ptr(), B, n_q, H, D, n_pool, int(kpool), _DTYPE[q.dtype],
                                     _DTYPE[pooled.dtype], float(scale), _stream(stream)), "dsa_kpool_index_score")
    return scores


def dsa_kpool_expand(pool_idx: torch.Tensor, packed: torch.Tensor, D: int, tok_idx: torch.Tensor, kpool: int,
                     kv_len: Optional[torch.Tensor] = None, q_pos: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """pool_idx [B][n_q][top_pools] int32, packed [B][n_kv][row_stride], tok_idx
    [B][n_q][kpool * top_pools + kpool - 1] int32 (output)."""
    B, n_q, top_pools = pool_idx.shape
    n_kv, stride = packed.shape[1], packed.shape[2]
    for t, n in ((pool_idx, "pool_idx"), (packed, "packed"), (tok_idx, "tok_idx")):
        _dev(t, n)
    if pool_idx.dtype != torch.int32 or tok_idx.dtype != torch.int32 or packed.shape[0] != B \
            or tuple(tok_idx.shape) != (B, n_q, kpool * top_pools + kpool - 1):
        raise ValueError("dsa_kpool_expand: inconsistent shapes or dtypes")
    _opt(kv_len, "kv_len", torch.int32, (B,))
    _opt(q_pos, "q_pos", torch.int32, (B, n_q))
    _check(lib.dsa_kpool_expand(pool_idx.data_ptr(), packed.data_ptr(), stride, _DTYPE[packed.dtype], D,
                                _ptr(kv_len), _ptr(q_pos), tok_idx.data_ptr(), B, n_q, n_kv, top_pools, int(kpool),
                                _stream(stream)), "dsa_kpool_expand")
    return tok_idx


def dsa_kpool_sparse_mla_attn(q_abs: torch.Tensor, latent: torch.Tensor, pool_idx: torch.Tensor,
                              packed: torch.Tensor, D: int, kpool: int, out: torch.Tensor, d_latent: int,
                              sm_scale: float, lse: Optional[torch.Tensor] = None,
                              kv_len: Optional[torch.Tensor] = None, q_pos: Optional[torch.Tensor] = None,
                              n_split: int = 0, workspace: Optional[torch.Tensor] = None,
                              stream=None) -> torch.Tensor:
    """dsa_kpool_expand + dsa_sparse_mla_attn in one call: q_abs [B][n_q][Hm][Dc] bf16, latent
    [B][n_kv][Dc] bf16, pool_idx [B][n_q][top_pools] int32, packed [B][n_kv][row_stride],
    out [B][n_q][Hm][d_latent] fp32 (output), lse [B][n_q][Hm] fp32 or None."""
    B, n_q, Hm, Dc = q_abs.shape
    n_kv = latent.shape[1]
    top_pools = pool_idx.shape[-1]
    for t, n in ((q_abs, "q_abs"), (latent, "latent"), (pool_idx, "pool_idx"), (packed, "packed"), (out, "out")):
        _dev(t, n)
    if tuple(latent.shape) != (B, n_kv, Dc) or tuple(pool_idx.shape) != (B, n_q, top_pools) \
            or tuple(out.shape) != (B, n_q, Hm, d_latent) or latent.dtype != q_abs.dtype \
            or packed.dim() != 3 or tuple(packed.shape[:2]) != (B, n_kv):
        raise ValueError("dsa_kpool_sparse_mla_attn: inconsistent shapes or dtypes")
    if pool_idx.dtype != torch.int32 or out.dtype != torch.float32:
        raise ValueError("pool_idx must be int32 and out float32")
    _opt(lse, "lse", torch.float32, (B, n_q, Hm))
    _opt(kv_len, "kv_len", torch.int32, (B,))
    _opt(q_pos, "q_pos", torch.int32, (B, n_q))
    width = kpool * top_pools + kpool - 1
    need = dsa_sparse_mla_workspace_size(B, n_q, Hm, width, d_latent, n_split)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_abs.device)
    wbytes = _workspace_bytes(workspace)
    _check(lib.dsa_kpool_sparse_mla_attn(q_abs.data_ptr(), latent.data_ptr(), pool_idx.data_ptr(), packed.data_ptr(),
                                         packed.shape[2], _DTYPE[packed.dtype], D, _ptr(kv_len), _ptr(q_pos),
                                         out.data_ptr(), _ptr(lse), B, n_q, Hm, n_kv, top_pools, int(kpool),
                                         d_latent, Dc - d_latent, float(sm_scale), _DTYPE[q_abs.dtype],
                                         int(n_split), _ptr(workspace), wbytes, _stream(stream)),
           "dsa_kpool_sparse_mla_attn")
    return out
