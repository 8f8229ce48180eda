"""fp64 CPU oracle for split-KV decode attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP product path never imports it and shares no
code with it.
"""

from .decode_attention import (  # noqa: F401
    LOG2E,
    bf16_round_fp64,
    combine_fp64,
    decode_attention_fp64,
    decode_attention_splitk_fp64,
    equal_share_pieces,
    fp8_e4m3_to_fp64,
    partition_partials_fp64,
    range_partials_fp64,
)
