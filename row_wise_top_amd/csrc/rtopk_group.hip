// Instantiates the row-group exact and capped kernels (four waves per row)
// for rows of up to 6,144 and 8,192 columns (24 and 32 slots per lane per
// wave).
#include "rtopk_group.hpp"

namespace rtopk {
template RowsKernel group_kernel<24>(bool, bool, int, bool);
template RowsKernel group_kernel<32>(bool, bool, int, bool);
}  // namespace rtopk
