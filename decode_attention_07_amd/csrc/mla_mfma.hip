// mla_mfma.hip -- matrix-core MLA decode (depth 576, V = K[..., :512]).
#include "da_device.h"

namespace da {

int mla_rows_per_block(int, int) { return 128; }
int mla_step_keys(int) { return 32; }

hipError_t launch_mla(const DecodeParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace da
