"""cache_aware_attention_amd -- MI355X (gfx950) kernels for the per-step hot path
of KV-cached masked-autoregressive (MAR) image decoding.

The computation lives in libmarca.so (hand-written HIP kernels behind a C ABI,
declared in include/mar_cache_attn.h); this package only binds it.  Importing
the package loads the library and raises ImportError when it is not built.
"""
from ._lib import (  # noqa: F401
    MAR_BF16, MAR_CFG_REUSE, MAR_CFG_STORE, MAR_F32, MAR_LAYER_CACHE, MAR_LAYER_GATE,
    MAR_LAYER_SELECT, MAR_REFRESH_TOPK_SCRATCH_BYTES, MarError, Prepared, StepPlan, load_library,
    mar_cache_attn_fwd, mar_cache_attn_fwd_ragged, mar_cache_attn_fwd_ragged_update,
    mar_cache_attn_fwd_scores,
    mar_cache_attn_fwd_update, mar_cfg_residual,
    mar_cos_gate, mar_kv_scatter_refresh, mar_layer_flags, mar_plan_step, mar_refresh_select,
    mar_refresh_topk, mar_refresh_topk_noalloc, mar_refresh_topk_workspace, prepare)

load_library()
