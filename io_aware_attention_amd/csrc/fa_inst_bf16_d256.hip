// Kernel variants for bf16 inputs, head dim 256.
#include "fa_launch.hpp"

FA355_PAIR_VARIANTS(FA355_INSTANTIATE_PAIR, BF16)
FA355_ROLE_VARIANTS(FA355_INSTANTIATE_ROLE, BF16)
