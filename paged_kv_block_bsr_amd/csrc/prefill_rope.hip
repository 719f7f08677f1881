// prefill_rope.hip -- the batch-prefill kernels with the fused rotary
// embedding (prefill_kernel.h), built apart from the others so that the
// variants compile in parallel.  They are the windowed kernels too: without
// a window they run with one longer than any request, which hides nothing.
#include <climits>

#include "prefill_kernel.h"

namespace fi {

int launch_prefill_rope(const RunArgs& r, const PrefillParams& p) {
  PrefillParams q = p;
  if (q.window < 0) q.window = INT_MAX;
  return launch_mode<true, true>(r, q);
}

}  // namespace fi
