"""float64 CPU oracle: test infrastructure, never part of the product path.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.  See
``oracle/attention.py`` (forward, decode), ``oracle/attention_bwd.py``
(gradients) and ``oracle/fp8_quant.py`` (incoherent processing and e4m3
quantisation) for what each function computes and which passage of the
pages it follows.
"""

from .attention import (allowed_keys, attention_head_ref, attention_ref,
                        merge_partials, merge_ref, online_ref)
from .attention_bwd import attention_bwd_head_ref, attention_bwd_ref
from .fp8_quant import (e4m3_decode_ref, e4m3_round_ref, e4m3_values, hadamard_ref,
                        rotate_quantize_ref, rotate_ref)

__all__ = ["allowed_keys", "attention_head_ref", "attention_ref",
           "merge_partials", "merge_ref", "online_ref",
           "attention_bwd_head_ref", "attention_bwd_ref",
           "e4m3_decode_ref", "e4m3_round_ref", "e4m3_values", "hadamard_ref",
           "rotate_quantize_ref", "rotate_ref"]
