// Instantiates the register-resident row kernels for Q = 6, 8, 12, 16 slots.
#include "rtopk_rows.hpp"

namespace rtopk {
template RowsKernel rows_kernel<6>(bool, Mode, bool, int);
template RowsKernel rows_kernel<8>(bool, Mode, bool, int);
template RowsKernel rows_kernel<12>(bool, Mode, bool, int);
template RowsKernel rows_kernel<16>(bool, Mode, bool, int);
}  // namespace rtopk
