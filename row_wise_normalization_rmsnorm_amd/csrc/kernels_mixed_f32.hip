// kernels_mixed_f32.hip -- the general interface for fp32 data: fp16 or
// bf16 output (gamma is fp32).
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(mixed_f32,
                  rmsn::add_mixed<float, float, _Float16>(v, rmsn::Types{0, 0, 1});
                  rmsn::add_mixed<float, float, __bf16>(v, rmsn::Types{0, 0, 2}))
