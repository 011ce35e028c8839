// Instantiates the register-resident row kernels for Q = 96 slots.
#include "rtopk_rows.hpp"

namespace rtopk {
template RowsKernel rows_kernel<96>(bool, Mode, bool, int);
}  // namespace rtopk
