// Decode kernel instantiations: narrow latent tables (d <= 256).
#include "kk_decode_kernel.h"

namespace kk {
template hipError_t launch_decode_items<1, kLean>(const DecodeArgs&, int, int, hipStream_t);
template hipError_t launch_decode_items<2, kLean>(const DecodeArgs&, int, int, hipStream_t);
}  // namespace kk
