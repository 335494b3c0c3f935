"""fp64 CPU oracle for the W4A16 group-quantised decode GEMV.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
bench's CPU-baseline leg may import this package. The product path (the C-ABI
library and its Python binding) never imports, calls or links anything here,
and nothing here imports the product path.
"""
from .w4a16_ref import (  # noqa: F401
    ATOL,
    GROUP,
    RTOL,
    dequantise,
    gemv,
    gemv_rows,
    quantise,
    tolerance,
    unpack_codes,
    within_tolerance,
)
from . import codecs_ref  # noqa: F401,E402  (weight-code variants)
from . import kv_attention_ref  # noqa: F401,E402  (decode attention over a quantised KV cache)
