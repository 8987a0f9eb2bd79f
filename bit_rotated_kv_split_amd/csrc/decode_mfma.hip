// Matrix-core (MFMA) history kernel: not built yet; the vector-ALU kernel
// serves every shape until it is.
#include "oscar_internal.h"

namespace oscar {

bool hist_mfma_supported(const oscar_dims&) { return false; }

hipError_t launch_hist_mfma(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace oscar
