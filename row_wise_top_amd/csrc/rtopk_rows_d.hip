// Instantiates the register-resident row kernels for Q = 48, 64 slots.
#include "rtopk_rows.hpp"

namespace rtopk {
template RowsKernel rows_kernel<48>(bool, Mode, bool, int);
template RowsKernel rows_kernel<64>(bool, Mode, bool, int);
}  // namespace rtopk
