// kernels_ag_f16.hip -- the fused form with an all-gather epilogue for f16
// data (add_rmsnorm_ag_fwd).
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(ag_f16, rmsn::add_ag<_Float16>(v, rmsn::Types{1, 1, 1}))
