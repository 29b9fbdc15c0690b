"""Seeded synthetic inputs for the fp8 MQA indexer (logits + top-k).

This package is shared by the tests, the benchmark and the oracle's callers.
It holds none of the method's arithmetic: it draws random tensors, casts them
to fp8 e4m3fn with torch's own cast (the same recipe as the chunking
micro-benchmark's ``_build`` on the bench_mqa_logits_chunking.py page), and
lays out the index arrays (ks, ke, block tables).  Everything is returned as
numpy arrays on the host; callers upload them to the device themselves.
"""

from .generate import (  # noqa: F401
    H,
    D,
    RaggedInputs,
    PagedInputs,
    ragged_inputs,
    paged_inputs,
    config_inputs,
    CONFIGS,
)
