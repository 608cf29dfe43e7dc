// kernels_ag_bf16.hip -- the fused form with an all-gather epilogue for bf16
// data (add_rmsnorm_ag_fwd).
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(ag_bf16, rmsn::add_ag<__bf16>(v, rmsn::Types{2, 2, 2}))
