// kernels_f32.hip -- every kernel variant for fp32 data.
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(f32, rmsn::add_full<float>(v, rmsn::Types{0, 0, 0}))
