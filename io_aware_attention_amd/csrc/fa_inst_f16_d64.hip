// Kernel variants for f16 inputs, head dim 64.
#include "fa_launch.hpp"

FA355_VARIANTS_D64_D128(FA355_INSTANTIATE, F16, 64)
FA355_SPLIT_VARIANTS(FA355_INSTANTIATE_SPLIT, F16, 64)
