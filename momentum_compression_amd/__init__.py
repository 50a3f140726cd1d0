"""MI355X-native error-compensated 1-bit / INT8 compression stage of
1-bit Adam and 1-bit LAMB.

The compute lives in libonebit.so (hand-written HIP for gfx950, C ABI in
include/onebit.h); ``momentum_compression_amd.onebit`` is its ctypes binding
and ``momentum_compression_amd.state`` allocates the buffers one simulated
data-parallel group needs and drives one step through the binding.
"""

from . import onebit  # noqa: F401
from .onebit import (  # noqa: F401
    OnebitError,
    frozen_v_step,
    int8_quantize,
    int8_sr_quantize,
    lamb_layer_scale,
    onebit_compress,
    onebit_compress_ex,
    onebit_compress_grad,
    onebit_decompress,
    onebit_error_materialize,
    onebit_server_reduce,
    onebit_server_reduce_ex,
    workspace_bytes,
    frozen_v_workspace_bytes,
    lamb_momentum_scale,
    warmup_adam_step,
    warmup_lamb_step,
    warmup_workspace_bytes,
)
