// kernels_f16.hip -- every kernel variant for fp16 data.
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(f16, rmsn::add_full<_Float16>(v, rmsn::Types{1, 1, 1}))
