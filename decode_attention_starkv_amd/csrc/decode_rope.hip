// Instantiations of the 4/3-bit split kernel that read precomputed rotary
// scores (see split_q43.h and rope.hip); kept in their own translation unit
// so they compile in parallel with the latent-score kernels of decode.hip.
#include "split_q43.h"

namespace starkv {

SplitFn q43_rope_kernel(const Dims& d) { return q43_kernel_select<true, false>(d); }

}  // namespace starkv
