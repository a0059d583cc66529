"""CPU oracle for exact tiled attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and nothing
here imports the product path.

What it computes is the plain definition of scaled-dot-product attention in
float64 numpy: full score rows, masks, softcap and ALiBi applied, softmax,
times V, plus the analytic backward.  There is no tiling, no online softmax
and no KV split here: the pages state that the tiled method returns the same
numbers as standard attention (page "FlashAttention 实战指南：如何把训练内存省
20 倍、速度提 4 倍", section "FlashAttention 的做法是三个手段配合": output
numerically identical to standard attention), so the oracle is that standard
attention written out.

Modules
-------
attention : dense forward / backward (GQA, causal, window, softcap, ALiBi)
varlen    : packed variable-length forward / backward (per-sequence slices)
kvcache   : rotary embedding, paged-cache append and decode attention
dropout   : Philox4x32-10 and the attention-dropout keep mask

Every function is pinned by CPU tests (``tests/test_oracle_*.py``) against
library routines, closed forms, invariants, brute force and finite
differences; none of it is "parity unpinned".
"""
from .attention import attention_fwd, attention_bwd, allowed_mask, score_transform  # noqa: F401
from .varlen import varlen_fwd, varlen_bwd  # noqa: F401
from .kvcache import rotary_apply, round_bf16, kvcache_fwd, gather_logical_cache  # noqa: F401
from .dropout import philox4, keep_mask, keep_scale, threshold  # noqa: F401
