// Quantize-and-pack cache writer for gfx950.
//
// Precision axis of KV-Kaizen ("Three Non-Eviction Compression Axes", item 3
// of the picx.dev summary page): one symmetric uniform scale per token; the
// rank axis (item 2) keeps the first d latent coordinates plus the RoPE key.
//
// One wave quantizes one token.  Lane w owns 32-bit word w of the packed row
// (32/b consecutive fields), so the packed stores are fully coalesced.  For
// b = 16 the row is two byte planes (the K high bytes, then the K low bytes
// with bit 7 flipped): lane w's two fields go to 16-bit slots of each plane.  The
// absmax is a wave max (exact, order independent); scale and codes use
// IEEE fp32 division with round-to-nearest-even and rint (ties to even), so
// the result is bit-identical to any other correct implementation of the
// same definition.
#include <hip/hip_runtime.h>

#include "kk_internal.h"

namespace kk {
namespace {

__device__ inline float load_src(const void* p, int64_t idx, int bf16) {
  if (bf16) {
    uint32_t h = ((const uint16_t*)p)[idx];
    return __uint_as_float(h << 16);
  }
  return ((const float*)p)[idx];
}

template <int BITS>
__global__ void __launch_bounds__(256) write_kernel(WriteArgs a) {
  constexpr int kFields = 32 / BITS;              // fields per 32-bit word
  constexpr int kMaxWords = (640 * BITS / 32 + 63) / 64;   // words per lane (K <= 640)
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= a.n_tokens) return;
  const int64_t src = a.src_index ? (int64_t)a.src_index[tok] : tok;
  const int64_t slot = a.dst_slot[tok];
  if (src < 0 || src >= a.n_src || slot < 0 || slot >= a.n_slots) return;

  const int K = a.d + a.d_rope;
  const int words = a.row_stride >> 2;
  float v[kMaxWords][kFields];
  float amax = 0.0f;
#pragma unroll
  for (int wi = 0; wi < kMaxWords; ++wi) {
    const int w = lane + 64 * wi;
#pragma unroll
    for (int f = 0; f < kFields; ++f) {
      const int j = w * kFields + f;
      float x = 0.0f;
      if (w < words && j < K) {
        x = j < a.d ? load_src(a.latent, src * a.latent_ld + j, a.src_bf16)
                    : load_src(a.rope, src * a.rope_ld + (j - a.d), a.src_bf16);
      }
      v[wi][f] = x;
      amax = fmaxf(amax, fabsf(x));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));

  const float qmax = (float)((1 << (BITS - 1)) - 1);
  const float scale = __fdiv_rn(amax, qmax);
  uint8_t* row = a.codes + slot * a.row_stride;
#pragma unroll
  for (int wi = 0; wi < kMaxWords; ++wi) {
    const int w = lane + 64 * wi;
    if (w >= words) continue;
    uint32_t word = 0;
#pragma unroll
    for (int f = 0; f < kFields; ++f) {
      const int j = w * kFields + f;
      int c = 0;
      if (amax > 0.0f && j < K) {
        float q = rintf(__fdiv_rn(v[wi][f], scale));
        q = fminf(fmaxf(q, -qmax), qmax);
        c = (int)q;
      }
      word |= ((uint32_t)c & ((1u << BITS) - 1u)) << (f * BITS);
    }
    if constexpr (BITS == 16) {
      // word = (code 2w+1 << 16) | code 2w: high bytes to plane 0, low bytes ^ 0x80 to plane 1
      if (2 * w < K) {
        ((uint16_t*)row)[w] = (uint16_t)(((word >> 8) & 0xFFu) | ((word >> 16) & 0xFF00u));
        ((uint16_t*)(row + K))[w] = (uint16_t)(((word & 0xFFu) | ((word >> 8) & 0xFF00u)) ^ 0x8080u);
      }
    } else {
      ((uint32_t*)row)[w] = word;
    }
  }
  if (lane == 0) a.scales[slot] = scale;
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, hipStream_t stream) {
  if (a.n_tokens <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.n_tokens + 3) / 4)), block(256);
  switch (a.bits) {
    case 2: hipLaunchKernelGGL(write_kernel<2>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(write_kernel<4>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(write_kernel<8>, grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL(write_kernel<16>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kk
