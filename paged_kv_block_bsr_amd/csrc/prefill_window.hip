// prefill_window.hip -- the batch-prefill kernels with a sliding window
// (prefill_kernel.h), built apart from the others so that both halves
// compile in parallel.
#include "prefill_kernel.h"

namespace fi {

int launch_prefill_window(const RunArgs& r, const PrefillParams& p) { return launch_mode<true, false>(r, p); }

}  // namespace fi
