// kernels_bf16.hip -- every kernel variant for bf16 storage.
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(__bf16, 2, bf16)
