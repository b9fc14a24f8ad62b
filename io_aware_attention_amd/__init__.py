"""MI355X-native FlashAttention forward and backward passes (libfa355) and their
Python binding."""
from .fa355 import (BF16, F16, F32, NOALLOC_SCRATCH_BYTES, FA355Error, Plan, bwd,  # noqa: F401
                    decode_noalloc_bytes, decode_split_count, fwd, fwd_bias, fwd_decode,
                    fwd_decode_noalloc, fwd_fp8, fwd_split, lib, plan, split_count, status_str,
                    use_library)

__version__ = "0.3.0"
