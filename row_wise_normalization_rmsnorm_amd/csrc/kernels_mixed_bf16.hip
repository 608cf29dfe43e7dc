// kernels_mixed_bf16.hip -- the general interface for bf16 data: bf16 or
// fp32 gamma, and every output dtype other than the single-dtype case.
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(mixed_bf16,
                  rmsn::add_mixed<__bf16, __bf16, float>(v, rmsn::Types{2, 2, 0});
                  rmsn::add_mixed<__bf16, __bf16, _Float16>(v, rmsn::Types{2, 2, 1});
                  rmsn::add_mixed<__bf16, float, float>(v, rmsn::Types{2, 0, 0});
                  rmsn::add_mixed<__bf16, float, _Float16>(v, rmsn::Types{2, 0, 1});
                  rmsn::add_mixed<__bf16, float, __bf16>(v, rmsn::Types{2, 0, 2}))
