// kernels_f32.hip -- every kernel variant for f32 storage.
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(float, 0, f32)
