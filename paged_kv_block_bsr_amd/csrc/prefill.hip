// prefill.hip -- placeholder until the MFMA prefill kernel lands: plans with
// prefill tiles are rejected by the API layer.
#include "device_common.h"
#include "fi_internal.h"

namespace fi {
int launch_prefill(const RunArgs&) { return FI_OK; }
}  // namespace fi
