// Instantiates the register-resident row kernels for Q = 128 slots.
#include "rtopk_rows.hpp"

namespace rtopk {
template RowsKernel rows_kernel<128>(bool, Mode, bool, int);
}  // namespace rtopk
