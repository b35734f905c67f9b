// Instantiations of the split kernel for the uniform 4-bit cache (both
// precision blocks at 4 bits; see split_q43.h), scoring latent keys; kept in
// their own translation unit so they compile in parallel with the others.
#include "split_q43.h"

namespace starkv {

SplitFn u4_kernel(const Dims& d) { return q43_kernel_select<false, true>(d); }

}  // namespace starkv
