// Stack kernel variant with 1 hidden chunk and 2 intermediate chunks per lane.
// (With two intermediate chunks a lane group covers one down row, so J >= 2
// rows need RD >= 2; hidden sizes needing two chunks give J >= 10 on 256
// compute units, beyond RD 2: those shapes use the per-layer kernels.)
#include "persist.h"

namespace moe {
MOE_STACK_INSTANTIATE(1, 2, 2)
}  // namespace moe
