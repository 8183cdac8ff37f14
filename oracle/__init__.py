"""fp64 CPU oracle for chunk-windowed softmax attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this package.  It shares no code with the HIP path.
"""

from .window_attention import (  # noqa: F401
    Geometry,
    PlanGroup,
    chunk_span_rows,
    kept_pairs_per_head,
    kept_set,
    masked_dense_attention,
    plan_groups,
    plan_kv_indices,
    window_attention_reference,
    window_attention_rows,
    window_bounds,
    window_mask,
)
from .causal_attention import (  # noqa: F401
    causal_attention_reference,
    causal_attention_rows,
    causal_mask,
    causal_pairs_per_head,
)
from .qk_norm_rope import (  # noqa: F401
    qk_norm_rope_reference,
    rms_norm,
    rope,
)
from .block_mask import block_mask, block_mask_brute_force, block_sparse_computed_pairs  # noqa: F401
from .fp8 import (  # noqa: F401
    decode_e4m3,
    fp8_causal_attention_reference,
    fp8_causal_attention_rows,
    fp8_window_attention_reference,
    fp8_window_attention_rows,
)
