"""MI355X-native per-token mixed-precision KV transfer path (SpectrumKV).

The path - importance score, tier assignment, quantize + pack, dense or paged
unpack - runs in hand-written HIP kernels for gfx950 behind the C ABI in
``include/sk.h`` (``libsk.so``).  :mod:`serving_sk_score_amd.sk` is the thin
Python binding; PyTorch only provides device memory and streams.
"""

from .sk import (  # noqa: F401
    OVERFLOW_DROP, OVERFLOW_FALLBACK, OVERFLOW_REJECT, SCORE_SCRATCH_BYTES, SK_E_WORKSPACE,
    TIER_DROP, Plan, Policy, Shape,
    SkError, assign_tiers, balanced_keys, colsum_workspace_bytes, decode_attention,
    decode_workspace_bytes, lib, pack,
    plan_make, recency_weight, score, score_colsum, score_kvnorm, score_noalloc, score_rowlse,
    colsum_layers_workspace_bytes, score_colsum_layers, score_layers,
    score_layers_workspace_bytes, score_rowlse_layers, score_workspace_bytes, unpack, unpack_paged, upgrade_bytes, upgrade_pack, upgrade_unpack,
    upgrade_unpack_paged,
)
