"""libdsa: DeepSeek Sparse Attention hot path (indexer score -> top-k -> sparse absorbed
MLA) as hand-written HIP kernels for MI355X (gfx950) behind a C ABI (include/dsa.h).

The binding lives in ``sparse_attention_10_amd.dsa`` and loads ``libdsa.so`` on import
(it raises ImportError when the library has not been built)."""
