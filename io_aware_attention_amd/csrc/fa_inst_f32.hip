// Kernel variants for fp32 inputs, head dim 64.
#include "fa_launch.hpp"

FA355_VARIANTS_F32(FA355_INSTANTIATE_F32)
