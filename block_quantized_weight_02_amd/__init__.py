"""MI355X (gfx950) Q8_0 weight product: y = x . W over int8 values with one
fp32 scale per 32 rows of each column, for 1..32 activation rows (bf16 or
their per-32-block int8 form), the weight streamed once for all rows.

The compute is the HIP library ``libq8gemv.so`` (C ABI: include/q8gemv.h);
``binding`` exposes it to Python under the same names.  ``inputs`` draws the
seeded synthetic workloads.  Build with ``python -m block_quantized_weight_02_amd.build``.
"""
from .binding import *  # noqa: F401,F403
from .binding import Q8Error, lib, q8_plan  # noqa: F401
