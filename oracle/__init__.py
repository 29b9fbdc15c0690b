"""CPU float64 oracle for the fp8 MQA indexer (logits + top-k + index map).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the tests, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP
library: it decodes fp8 from the bit layout itself and evaluates the
definitions literally in float64 with numpy.
"""

from .indexer_oracle import (  # noqa: F401
    e4m3fn_value_table,
    decode_e4m3fn,
    scores,
    mqa_logits,
    gather_paged_kv,
    paged_mqa_logits,
    topk_indices,
    map_token_table,
    map_block_table,
    ragged_topk_mapped,
    paged_topk_mapped,
    rows_per_chunk,
    encode_e4m3fn,
)
from .sparse_mla_oracle import (  # noqa: F401
    MLA_DQK,
    MLA_DV,
    decode_bf16,
    sparse_mla,
)
