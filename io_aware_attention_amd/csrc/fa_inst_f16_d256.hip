// Kernel variants for f16 inputs, head dim 256.
#include "fa_launch.hpp"

FA355_VARIANTS_D256(FA355_INSTANTIATE, F16)
FA355_PAIR_VARIANTS(FA355_INSTANTIATE_PAIR, F16)
