"""CPU oracle for the HySparse / HySparse2 hybrid-block attention hot path.

THIS PACKAGE IS TEST INFRASTRUCTURE.  It exists to check the HIP library.
Only the tests, the smoke entry point and the benchmark's CPU-baseline leg
may import or run it; the library and its Python binding never do, and the
product path has no CPU fallback.

What it is: plain float64 numpy definitions of each step, written from the
HySparse and HySparse2 pages (QbitAI HySparse article; TechWalker HySparse
write-up; airebao HySparse2 news; demingchina HySparse2 commentary), with no
blocking, fusion or reordering beyond evaluating query rows independently.
It shares no code with the HIP path; both consume the seeded bytes of the
`synth` input generator.

Pins (tests/test_oracle*.py, run with -m "not gpu"): brute force in pure
Python loops, torch's CPU float64 scaled_dot_product_attention, closed forms,
invariants, hand-derived golden values under tests/golden/, the fp8
decode table against torch.float8_e4m3fn, the fp8 encoder of the KV
Bridging projection (bridge.py) against torch's CPU float8 conversion, and
the HySparse decode step with ring window caches (hysparse_decode.py)
against the prefill block evaluated at its last row, and the backward pass
(hysparse_bwd.py) against central finite differences of the forward
definitions.

Parity unpinned (against the real HySparse/HySparse2, whose pages leave these
open): the head reduction of importance scores (max over all query heads),
the gate's form (one sigmoid scalar per token and head, no bias), the empty
sparse set rule, the per-tile token-score reading, the per-query forced
window and the decode-time ring window cache.  They are pinned only to this
package's stated readings.
"""
from . import bridge, fp8, hysparse_bwd, hysparse_decode  # noqa: F401
from .hysparse import (  # noqa: F401
    NEG_INF, attend, block_scores, block_scores_per_group, decode_full, decode_sparse, decode_step,
    expand_blocks, full_attention, gate_merge, hysparse2_block, hysparse2_gated_window_layer, hysparse_block,
    logits, sparse_block_attention, sparse_block_attention_grouped, sparse_token_attention, tile_block_scores,
    tile_token_scores, topk_rows, topk_select, window_attention,
)

import numpy as _np


def as_f64(t, dtype: str, scale: float = 1.0) -> _np.ndarray:
    """Stored tensor -> float64 values the oracle computes on.

    fp32 and bf16 are upcast exactly; fp8 e4m3fn bytes are decoded with this
    package's own table and multiplied by the per-tensor scale.
    """
    import torch
    if dtype == "fp8":
        return fp8.dequantize(t.view(torch.uint8).numpy(), scale)
    return t.to(torch.float64).numpy()
