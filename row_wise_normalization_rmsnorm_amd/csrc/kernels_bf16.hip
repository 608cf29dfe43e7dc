// kernels_bf16.hip -- every kernel variant for bf16 data.
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(bf16, rmsn::add_full<__bf16>(v, rmsn::Types{2, 2, 2}))
