"""Float64 CPU oracle for paged MLA decode — test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. It shares no code with the HIP path.
"""
from .mla_oracle import (D_QK, D_V, E4M3FN_TABLE, absorb_out, absorb_q, attend,  # noqa: F401
                         bf16_bits_to_f64,
                         combine_partials, cos_diff, decode_rows, e4m3fn_to_f64,
                         e4m3fn_value, gather_keys, kv_append, mla_decode, quantize_e4m3fn,
                         rel_fro, round_bf16, visible_keys)
