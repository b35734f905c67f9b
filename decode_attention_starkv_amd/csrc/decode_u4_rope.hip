// Instantiations of the split kernel for the uniform 4-bit cache that read
// precomputed rotary scores (see split_q43.h and rope.hip); kept in their
// own translation unit so they compile in parallel with the others.
#include "split_q43.h"

namespace starkv {

SplitFn u4_rope_kernel(const Dims& d) { return q43_kernel_select<true, true>(d); }

}  // namespace starkv
