// Decode kernel instantiations: 40-head (three row block) latent rows.
#include "kk_decode_kernel.h"

namespace kk {
template hipError_t launch_decode_items<3, kFull>(const DecodeArgs&, int, int, hipStream_t);
}  // namespace kk
