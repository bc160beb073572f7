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

// Quantizes one token (the wave's 64 lanes) from its source rows and packs it
// into `row` with its scale at *scale_out.  The source rows hold the latent
// (first d used) and the RoPE key (d_rope), fp32 or bf16.  amax_in >= 0 gives
// the absmax the scale is taken from (a token whose scale covers more than
// this row); otherwise it is the row's own.
template <int BITS>
__device__ inline void quantize_token(const void* lat_row, const void* rope_row, int bf16, int d, int d_rope,
                                      int row_stride, uint8_t* row, float* scale_out, int lane,
                                      float amax_in = -1.0f) {
  constexpr int kFields = 32 / BITS;              // fields per 32-bit word
  constexpr int kMaxWords = (640 * BITS / 32 + 63) / 64;   // words per lane (K <= 640)
  const int K = d + d_rope;
  const int words = row_stride >> 2;
  float v[kMaxWords][kFields];
  float amax = 0.0f;
#pragma unroll
  for (int wi = 0; wi < kMaxWords; ++wi) {
    const int w = lane + 64 * wi;
#pragma unroll
    for (int f = 0; f < kFields; ++f) {
      const int j = w * kFields + f;
      float x = 0.0f;
      if (w < words && j < K) x = j < d ? load_src(lat_row, j, bf16) : load_src(rope_row, j - d, bf16);
      v[wi][f] = x;
      amax = fmaxf(amax, fabsf(x));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (amax_in >= 0.0f) amax = amax_in;

  const float qmax = (float)((1 << (BITS - 1)) - 1);
  const float scale = __fdiv_rn(amax, qmax);
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
  if (lane == 0) *scale_out = scale;
}

template <int BITS>
__global__ void __launch_bounds__(256) write_kernel(WriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= a.n_tokens) return;
  const int64_t src = a.src_index ? (int64_t)a.src_index[tok] : tok;
  const int64_t slot = a.dst_slot[tok];
  if (src < 0 || src >= a.n_src || slot < 0 || slot >= a.n_slots) return;
  const size_t es = a.src_bf16 ? 2 : 4;
  quantize_token<BITS>((const char*)a.latent + src * a.latent_ld * es, (const char*)a.rope + src * a.rope_ld * es,
                       a.src_bf16, a.d, a.d_rope, a.row_stride, a.codes + slot * a.row_stride, a.scales + slot, lane);
}

// Append: one wave per (anchor, sequence) writes the sequence's new token at
// row seq_lens[s] - 1 of the anchor's cache (nothing when that is outside
// [0, t_cap)).  The bit width is uniform per wave.
__global__ void __launch_bounds__(256) append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)a.n_anchors * a.batch) return;
  const int j = (int)(w / a.batch), s = (int)(w - (int64_t)j * a.batch);
  const int pos = a.seq_lens[s] - 1;
  if (pos < 0 || pos >= a.t_cap) return;
  const AppendAnchor& A = a.anchors[j];
  const size_t es = a.src_bf16 ? 2 : 4;
  const int64_t src = (int64_t)A.layer * a.batch + s;
  const char* lat = (const char*)a.latent + src * a.latent_ld * es;
  const char* rope = (const char*)a.rope + src * a.rope_ld * es;
  const int64_t slot = (int64_t)s * a.t_cap + pos;
  uint8_t* row = A.codes + slot * A.row_stride;
  switch (A.bits) {
    case 2: quantize_token<2>(lat, rope, a.src_bf16, A.d, a.d_rope, A.row_stride, row, A.scales + slot, lane); break;
    case 4: quantize_token<4>(lat, rope, a.src_bf16, A.d, a.d_rope, A.row_stride, row, A.scales + slot, lane); break;
    case 8: quantize_token<8>(lat, rope, a.src_bf16, A.d, a.d_rope, A.row_stride, row, A.scales + slot, lane); break;
    default: quantize_token<16>(lat, rope, a.src_bf16, A.d, a.d_rope, A.row_stride, row, A.scales + slot, lane); break;
  }
}

// Grouped-query write: one wave per token.  The absmax runs over the token's
// K and V of every KV head (one scale per token), then each KV head's row
// [V_g || K_g] is packed like a latent row with values first.
template <int BITS>
__global__ void __launch_bounds__(256) gqa_write_kernel(GqaWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= a.n_tokens) return;
  const int64_t src = a.src_index ? (int64_t)a.src_index[tok] : tok;
  const int64_t slot = a.dst_slot[tok];
  if (src < 0 || src >= a.n_src || slot < 0 || slot >= a.n_slots) return;
  const int64_t per = (int64_t)a.n_kv * a.d_head;
  const int64_t base = src * per;
  float amax = 0.0f;
  for (int64_t j = lane; j < per; j += 64)
    amax = fmaxf(amax, fmaxf(fabsf(load_src(a.k, base + j, a.src_bf16)), fabsf(load_src(a.v, base + j, a.src_bf16))));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const int64_t seq = slot / a.t_cap, pos = slot - seq * a.t_cap;
  const size_t es = a.src_bf16 ? 2 : 4;
  for (int g = 0; g < a.n_kv; ++g) {
    const int64_t r = (seq * a.n_kv + g) * a.t_cap + pos;
    const int64_t so = (base + (int64_t)g * a.d_head) * es;
    quantize_token<BITS>((const char*)a.v + so, (const char*)a.k + so, a.src_bf16, a.d_head, a.d_head, a.row_stride,
                         a.codes + r * a.row_stride, a.scales + r, lane, amax);
  }
}

}  // namespace

hipError_t launch_gqa_write(const GqaWriteArgs& a, hipStream_t stream) {
  if (a.n_tokens <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.n_tokens + 3) / 4)), block(256);
  switch (a.bits) {
    case 2: hipLaunchKernelGGL(gqa_write_kernel<2>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(gqa_write_kernel<4>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(gqa_write_kernel<8>, grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL(gqa_write_kernel<16>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

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

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.n_anchors * a.batch;
  if (waves <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kk
