// Split-T merge, plan upload and the launch dispatcher of the decode step
// (gfx950).  The decode kernel itself is in kk_decode_kernel.h; its variants
// are instantiated in kk_decode_full3.hip, kk_decode_full12.hip,
// kk_decode_lean.hip and kk_decode_gqa.hip.
#include "kk_decode_kernel.h"

namespace kk {
// The decode kernel variants are instantiated in their own translation units
// only (this one sees the template's definition but must not compile it again).
extern template hipError_t launch_decode_items<1, kFull>(const DecodeArgs&, int, int, hipStream_t);
extern template hipError_t launch_decode_items<2, kFull>(const DecodeArgs&, int, int, hipStream_t);
extern template hipError_t launch_decode_items<3, kFull>(const DecodeArgs&, int, int, hipStream_t);
extern template hipError_t launch_decode_items<1, kLean>(const DecodeArgs&, int, int, hipStream_t);
extern template hipError_t launch_decode_items<2, kLean>(const DecodeArgs&, int, int, hipStream_t);
extern template hipError_t launch_decode_items<1, kGqa>(const DecodeArgs&, int, int, hipStream_t);
extern template hipError_t launch_decode_items<2, kGqa>(const DecodeArgs&, int, int, hipStream_t);

namespace {
// Merge the split partials of one (entry, sequence, chunk) in a fixed order.
// A merge may be cut into A.merge_parts workgroups, each owning a contiguous
// range of the 8-feature vectors of every row (and computing the rows' split
// weights itself); every output sums its splits in the same order either way.
__global__ void __launch_bounds__(256) merge_kernel(DecodeArgs) {
  __shared__ float wgt[kMaxMergeSplits][64];
  KArgs& A = kernel_args();
  const int blk = blockIdx.x;
  KEntry* ents = entry_array(A);
  KEntry& E = ents[find_entry<true>(A, ents, blk)];
  const int parts = A.merge_parts;
  const int local = (blk - E.merge_base) / parts, part = (blk - E.merge_base) - local * parts;
  if (E.splits <= 1 || local >= E.n_seq * E.nrc) return;
  const int s = local / E.nrc, chunk = local - s * E.nrc;
  const int d = E.d, S = E.splits;
  const int r0 = E.row_begin + chunk * E.chunk_rows;
  const int nrows = min(E.chunk_rows, E.row_end - r0);
  const int64_t slotf = partial_slot_floats(d);
  const float* base = A.ws + E.ws_off + (int64_t)(s * S) * E.nrc * slotf + chunk * slotf;
  const int64_t kstride = E.nrc * slotf;
  // o = sum_k w_k (O/l)_k with w_k = l_k 2^(m_k - M) / sum_j l_j 2^(m_j - M);
  // the stored (O/l)_k are in units of the slot scale, folded into w_k.
  // (one pass over the splits with a running maximum; loads of 8 splits at a time)
  for (int rl = threadIdx.x; rl < nrows; rl += 256) {
    float M = -INFINITY, L = 0.0f;
    for (int k0 = 0; k0 < S; k0 += 8) {
      float mk[8], lk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float* p = base + min(k0 + j, S - 1) * kstride + partial_ml_offset(d);
        mk[j] = p[rl];
        lk[j] = k0 + j < S ? p[64 + rl] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (lk[j] > 0.0f) {
          const float Mn = fmaxf(M, mk[j]);
          L = L * exp2f(M - Mn) + lk[j] * exp2f(mk[j] - Mn);
          M = Mn;
        }
      }
    }
    // weights: again 8 splits' loads issued before any is used
    for (int k0 = 0; k0 < S; k0 += 8) {
      float mk[8], lk[8], uk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float* p = base + min(k0 + j, S - 1) * kstride + partial_ml_offset(d);
        mk[j] = p[rl];
        lk[j] = p[64 + rl];
        uk[j] = p[128];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < S) wgt[k0 + j][rl] = (L > 0.0f && lk[j] > 0.0f) ? lk[j] * exp2f(mk[j] - M) / L * uk[j] : 0.0f;
    }
  }
  __syncthreads();
  // Each thread merges two 8-feature vectors per pass (16-byte loads) and
  // issues the loads of kSplitBatch splits before using any of them; every
  // output still sums its splits in order k = 0 .. S-1.
  const int d8 = d >> 3;
  const int v0 = (part * d8) / parts, nv = ((part + 1) * d8) / parts - v0;   // this part's vectors of a row
  constexpr int kMergeVec = 2;
  constexpr int kSplitBatch = 4;
  const int total = nrows * nv;
  for (int i0 = threadIdx.x; i0 < total; i0 += kMergeVec * 256) {
    int rl[kMergeVec], f[kMergeVec];
    f4 acc[kMergeVec][2];
#pragma unroll
    for (int j = 0; j < kMergeVec; ++j) {
      const int idx = min(i0 + 256 * j, total - 1);
      rl[j] = idx / nv;
      f[j] = (v0 + idx - rl[j] * nv) * 8;
      acc[j][0] = acc[j][1] = f4{0.f, 0.f, 0.f, 0.f};
    }
    for (int k0 = 0; k0 < S; k0 += kSplitBatch) {
      h8 h[kSplitBatch][kMergeVec];
#pragma unroll
      for (int kb = 0; kb < kSplitBatch; ++kb) {
        const _Float16* pk = (const _Float16*)(base + min(k0 + kb, S - 1) * kstride);
#pragma unroll
        for (int j = 0; j < kMergeVec; ++j) h[kb][j] = *(const h8*)(pk + (int64_t)rl[j] * d + f[j]);
      }
#pragma unroll
      for (int kb = 0; kb < kSplitBatch; ++kb) {
        if (k0 + kb < S) {
#pragma unroll
          for (int j = 0; j < kMergeVec; ++j) {
            const float wk = wgt[k0 + kb][rl[j]];
            acc[j][0] += f4{(float)h[kb][j][0], (float)h[kb][j][1], (float)h[kb][j][2], (float)h[kb][j][3]} * wk;
            acc[j][1] += f4{(float)h[kb][j][4], (float)h[kb][j][5], (float)h[kb][j][6], (float)h[kb][j][7]} * wk;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kMergeVec; ++j) {
      if (i0 + 256 * j < total) {
        const int gr = r0 + rl[j];
        const int layer = group_layer_at(A, E.lay_begin + gr / A.heads), head = gr % A.heads;
        float* dst = A.out + layer_at(A, layer).out_off + ((int64_t)s * A.heads + head) * d + f[j];
        *(f4*)dst = acc[j][0];
        *(f4*)(dst + 4) = acc[j][1];
      }
    }
  }
}

// Plan upload: each launch carries up to kStoreWords words in its arguments
// and writes them to device memory.
constexpr int kStoreWords = 1800;
struct StoreArgs {
  uint32_t* dst;
  int32_t n;
  int32_t pad_;
  uint32_t w[kStoreWords];
};
typedef __attribute__((address_space(4))) const StoreArgs KStore;

__global__ void __launch_bounds__(256) store_kernel(StoreArgs) {
  KStore& a = *(KStore*)(__builtin_amdgcn_kernarg_segment_ptr());
  for (int i = threadIdx.x; i < a.n; i += 256) a.dst[i] = a.w[i];
}

}  // namespace

// Tile buffers per workgroup: as many as fit in the workgroup's share of the
// 160 KB LDS, 3 to 12 (two tiles are in use, the rest in flight).
hipError_t launch_decode(const DecodeArgs& a, const DecodeLaunch& L, hipStream_t stream) {
  static_assert(sizeof(DecodeArgs) < 7600, "kernel argument block too large");
  if (L.items > 0) {
    hipError_t e;
    if (L.variant == kGqa) {          // grouped-query rows: <= 32 per KV head, <= 2 row blocks
      if (L.row_blocks > 2) return hipErrorInvalidValue;
      e = L.row_blocks == 1 ? launch_decode_items<1, kGqa>(a, L.items, L.lds_bytes, stream)
                            : launch_decode_items<2, kGqa>(a, L.items, L.lds_bytes, stream);
    } else if (L.variant == kLean) {  // <= 2 row blocks
      if (L.row_blocks > 2) return hipErrorInvalidValue;
      e = L.row_blocks == 1 ? launch_decode_items<1, kLean>(a, L.items, L.lds_bytes, stream)
                            : launch_decode_items<2, kLean>(a, L.items, L.lds_bytes, stream);
    } else {
      switch (L.row_blocks) {
        case 1: e = launch_decode_items<1, kFull>(a, L.items, L.lds_bytes, stream); break;
        case 2: e = launch_decode_items<2, kFull>(a, L.items, L.lds_bytes, stream); break;
        case 3: e = launch_decode_items<3, kFull>(a, L.items, L.lds_bytes, stream); break;
        default: return hipErrorInvalidValue;   // at most kMaxRowBlocks (3) row blocks
      }
    }
    if (e != hipSuccess) return e;
  }
  if (L.merge_blocks > 0) {
    hipLaunchKernelGGL(merge_kernel, dim3(L.merge_blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_store(uint32_t* dst, const uint32_t* words, int64_t n_words, hipStream_t stream) {
  static_assert(sizeof(StoreArgs) < 7600, "kernel argument block too large");
  StoreArgs a;
  for (int64_t o = 0; o < n_words; o += kStoreWords) {
    const int m = (int)(n_words - o < kStoreWords ? n_words - o : kStoreWords);
    a.dst = dst + o;
    a.n = m;
    a.pad_ = 0;
    std::memcpy(a.w, words + o, (size_t)m * sizeof(uint32_t));
    hipLaunchKernelGGL(store_kernel, dim3(1), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kk
