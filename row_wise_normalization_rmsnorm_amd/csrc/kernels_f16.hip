// kernels_f16.hip -- every kernel variant for f16 storage.
#include "rmsnorm_table.hpp"

RMSN_DEFINE_TABLE(_Float16, 1, f16)
