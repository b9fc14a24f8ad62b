// Backward kernel variants for bf16 inputs.
#include "fa_bwd_launch.hpp"

FA355_BWD_VARIANTS(FA355_INSTANTIATE_BWD, BF16)
