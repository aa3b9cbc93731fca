// decode_mfma.hip -- matrix-core split-K decode attention for wide head folds.
#include "da_device.h"

namespace da {

int mfma_rows_per_block() { return 16; }
int mfma_step_keys() { return 32; }

hipError_t launch_decode_mfma(const DecodeParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace da
