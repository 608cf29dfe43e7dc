// kernels_ag_f32.hip -- the fused form with an all-gather epilogue for f32
// data (add_rmsnorm_ag_fwd).
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(ag_f32, rmsn::add_ag<float>(v, rmsn::Types{0, 0, 0}))
