"""CPU oracle for decode-phase paged attention (fp64) and for appending a decode
step's K/V rows to the paged cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``, never by the library.
"""

from .decode import (  # noqa: F401
    attend,
    decode_attention,
    dequantize_rows,
    gather_sequence,
    kv_head_of,
)
from .append import append_kv, quantize_row, quantize_row_fp8  # noqa: F401
from .prefill import prefill_attention  # noqa: F401
from .formats import (  # noqa: F401
    bf16_to_float64,
    e4m3_from_float32,
    e4m3_to_float64,
    element_values,
)
