// Decode kernel instantiations: grouped-query rows.
#include "kk_decode_kernel.h"

namespace kk {
template hipError_t launch_decode_items<1, kGqa>(const DecodeArgs&, int, int, hipStream_t);
template hipError_t launch_decode_items<2, kGqa>(const DecodeArgs&, int, int, hipStream_t);
}  // namespace kk
