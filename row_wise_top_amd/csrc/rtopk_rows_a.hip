// Instantiates the register-resident row kernels for Q = 1, 2, 3, 4 slots.
#include "rtopk_rows.hpp"

namespace rtopk {
template RowsKernel rows_kernel<1>(bool, Mode, bool, int);
template RowsKernel rows_kernel<2>(bool, Mode, bool, int);
template RowsKernel rows_kernel<3>(bool, Mode, bool, int);
template RowsKernel rows_kernel<4>(bool, Mode, bool, int);
}  // namespace rtopk
