// Kernel variants for f16 inputs, head dim 256.
#include "fa_launch.hpp"

FA355_PAIR_VARIANTS(FA355_INSTANTIATE_PAIR, F16)
FA355_ROLE_VARIANTS(FA355_INSTANTIATE_ROLE, F16)
