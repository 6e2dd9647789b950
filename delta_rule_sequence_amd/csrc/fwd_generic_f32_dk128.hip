// fwd_generic_f32_dk128.hip - the generic forward for f32 I/O and key width 128: every
// value width (16, 32, 64, 128) and chunk size (16, 32, 64) whose tiles fit a CU's LDS.
#include "prism_generic_launch.h"

PRISM_DEFINE_GENERIC(launch_generic_f32_dk128, float, 128)
