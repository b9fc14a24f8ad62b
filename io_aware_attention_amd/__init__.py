"""MI355X-native FlashAttention forward pass (libfa355) and its Python binding."""
from .fa355 import (BF16, F16, F32, FA355Error, Plan, fwd, lib, plan,  # noqa: F401
                    status_str)

__version__ = "0.1.0"
