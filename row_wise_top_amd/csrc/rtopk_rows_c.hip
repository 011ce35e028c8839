// Instantiates the register-resident row kernels for Q = 24, 32 slots.
#include "rtopk_rows.hpp"

namespace rtopk {
template RowsKernel rows_kernel<24>(bool, Mode, bool, int);
template RowsKernel rows_kernel<32>(bool, Mode, bool, int);
}  // namespace rtopk
