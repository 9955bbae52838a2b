"""Seeded synthetic decode batches shared by the tests, the benchmark and smoke().

This package only draws random numbers and lays out block tables; it holds
none of the attention, append or copy arithmetic, so it can feed both the
HIP library and the oracle without coupling them.
"""

from .decode import (  # noqa: F401
    Batch,
    SCALE_D128,
    config1,
    config2,
    config3,
    config4,
    config5,
    custom,
    make_config,
)
from .extend import ExtendBatch, extend_batch, prefill_chunk_batch, verify_batch  # noqa: F401
