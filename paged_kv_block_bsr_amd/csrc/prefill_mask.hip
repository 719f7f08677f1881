// prefill_mask.hip -- the batch-prefill kernels with a tree mask
// (prefill_kernel.h), built apart from the others so that the variants
// compile in parallel.
#include "prefill_kernel.h"

namespace fi {

int launch_prefill_mask(const RunArgs& r, const PrefillParams& p) { return launch_mode<false, false, true>(r, p); }

}  // namespace fi
