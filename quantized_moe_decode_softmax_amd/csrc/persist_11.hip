// Stack kernel variants with 1 hidden chunk(s) and 1 intermediate chunk(s) per lane.
#include "persist.h"

namespace moe {
MOE_STACK_INSTANTIATE(1, 1, 1)
MOE_STACK_INSTANTIATE(1, 1, 2)
MOE_STACK_INSTANTIATE(1, 1, 4)
MOE_STACK_INSTANTIATE(1, 1, 8)
}  // namespace moe
