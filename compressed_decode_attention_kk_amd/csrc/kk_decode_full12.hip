// Decode kernel instantiations: one and two row block latent rows.
#include "kk_decode_kernel.h"

namespace kk {
template hipError_t launch_decode_items<1, kFull>(const DecodeArgs&, int, int, hipStream_t);
template hipError_t launch_decode_items<2, kFull>(const DecodeArgs&, int, int, hipStream_t);
}  // namespace kk
