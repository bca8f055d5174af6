"""MI355X-native batched verifier / lossless rejection sampler for speculative decoding.

The verify step (target softmax, accept test against min(1, p/q), first
rejection, residual or bonus draw, greedy variant) runs in hand-written HIP
kernels for gfx950 behind a C ABI (include/spec_verify.h); this package is
the thin Python binding over it.
"""

from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    SV_BF16,
    SV_F32,
    SVArgs,
    SVConfig,
    SpecVerify,
    SpecVerifyError,
    load_library,
    status_string,
)
from .device import DeviceBatch, upload  # noqa: F401
