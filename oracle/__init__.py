"""Float64 CPU oracle for grouped-query decode attention (one or several query
rows per slot).

Test infrastructure only.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, tables or helpers with the HIP
library under ``long_context_decode_kv_amd/``.
"""

from .kvdec_oracle import (  # noqa: F401
    F16,
    Q8_B32,
    Q4_B32,
    BLOCK,
    RECORD_CELLS,
    f16_bits_to_f64,
    dequantize,
    row_elems,
    attend_row,
    partial_row,
    merge_partials,
    decode_attention,
    decode_attention_multi,
    compact_plan,
)
