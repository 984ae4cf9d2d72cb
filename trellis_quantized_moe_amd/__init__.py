"""trellis_quantized_moe_amd: routed-expert GEMV/GEMM over T16 trellis-coded and MXFP4
expert weights, decoded on the fly by hand-written gfx950 (MI355X) kernels.

The compute lives in libtq.so (C ABI in include/tq.h, sources in csrc/). This package
only marshals PyTorch device tensors and streams to it; importing ``ops`` fails loudly
if the library is missing.
"""

from ._lib import (TQ_AUTO, TQ_COMBINE, TQ_EALIGN, TQ_EHIP, TQ_EINVAL, TQ_EUNSUPPORTED,  # noqa: F401
                   TQ_EWORKSPACE, TQ_GEMM, TQ_GEMV, TQ_OK, TQ_STATUS_BAD_EXPERT,
                   TQ_STATUS_BAD_UNIT, TQError, LIB_PATH, load)
