"""Plain float64 CPU oracle for biased, soft-capped multi-query attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call, link or execute anything in this
package.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the GPU
path: no kernels, headers, helpers, constants or pre/post-processing.

Citations in this package:
  [AG3090] web page "Making Full-Context AlphaGenome Fit on an RTX 3090"
           (twigslot.github.io, 2026-08-19).
  [AGDNA]  web page "From Code to Cure: How AlphaGenome Decodes the 'Dark
           Matter' of DNA" (sterlites.com), section "The Architecture".
"""

from .biased_mqa import (  # noqa: F401
    BIAS_BLOCK,
    as_f64,
    attention,
    attention_row_given_bias_row,
    attention_rows,
    expand_bias,
    logits,
    project_pair_bias,
    soft_cap,
    softmax_two_pass,
    tiled_attention,
)
from .brute import attention_brute, project_brute  # noqa: F401
