"""Biased, soft-capped multi-query attention for AMD Instinct MI355X.

AlphaGenome-style sequence attention (8 query heads sharing one K/V head,
head dim 128, a compact pair bias repeated 16x along both axes, tanh
soft-cap) as a HIP library for gfx950 with a C ABI (include/abg.h) and this
thin Python binding.

    from long_context_biased_amd import pair_bias_project, biased_mqa_fwd
    bias = pair_bias_project(pair, weight)          # [8, P, P] float32
    out = biased_mqa_fwd(q, k, v, bias, softcap=5.0)
    out = pair_biased_mqa_fwd(q, k, v, pair, weight)  # the projection inside
"""

from ._lib import (  # noqa: F401
    ABG_BF16,
    ABG_F32,
    EXPORTS,
    LIB_PATH,
    AbgError,
    auto_kv_splits,
    NOALLOC_SCRATCH_BYTES,
    biased_mqa_fwd,
    biased_mqa_fwd_ex_noalloc,
    load,
    pair_bias_project,
    pair_biased_mqa_fwd,
    raw_biased_mqa_fwd,
    raw_biased_mqa_fwd_ex,
    raw_biased_mqa_fwd_ex_noalloc,
    raw_pair_bias_project,
    raw_pair_biased_mqa_fwd,
    workspace_bytes,
)
