// kernels_mixed_f16.hip -- the general interface for fp16 data: fp16 or
// fp32 gamma, and every output dtype other than the single-dtype case.
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(mixed_f16,
                  rmsn::add_mixed<_Float16, _Float16, float>(v, rmsn::Types{1, 1, 0});
                  rmsn::add_mixed<_Float16, _Float16, __bf16>(v, rmsn::Types{1, 1, 2});
                  rmsn::add_mixed<_Float16, float, float>(v, rmsn::Types{1, 0, 0});
                  rmsn::add_mixed<_Float16, float, _Float16>(v, rmsn::Types{1, 0, 1});
                  rmsn::add_mixed<_Float16, float, __bf16>(v, rmsn::Types{1, 0, 2}))
