// Latent epilogue of absorbed-MLA decode for gfx950 (MI355X): the value
// up-projection of each head and the output projection of each layer.
//
// The MLA cache holds a shared latent c^KV (KV-Kaizen summary page, "Three
// Non-Eviction Compression Axes", rank item), so decode attention returns,
// per head, a weighted sum of latents o_h in the kept coordinates.  The head's
// value is its block of the up-projection W_UV on those coordinates,
// v_h = W_UV[h] o_h (attention is linear in its values), and the layer output
// mixes the heads, y = W_O [v_1; ...; v_H].
//
// Both are skinny products (the batch is the short side): Y[b][n] =
// sum_k X[b][k] W[n][k] with bf16 weights W [N][K] streamed from HBM once, fp32
// activations X read through L2.  On the bf16 MFMA (16x16x32) a weight tile is
// the A operand (16 rows n x 32 k) and the activations the B operand; the
// activations are split into bf16 high and low parts (x = hi + lo to 16
// significant bits) so that the bf16 weights are used exactly.  Each wave
// owns 64 output rows of one (layer, head) and the whole batch (<= 64 rows
// per pass) and keeps kStages k-steps of loads in flight.
#include <hip/hip_runtime.h>

#include <cstring>

#include "kk_internal.h"

namespace kk {
namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(4))) const EpiArgs KEpi;
typedef __attribute__((address_space(4))) const GemmProblem KProb;

constexpr int kStages = 4;       // k-steps of 32 in flight per wave
constexpr int kRowBlocks = 4;    // 16-row output blocks per wave (64 rows)

__device__ inline f4 mfma_bf16(bf8 a, bf8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

// One k-step of operands: 4 weight tiles and, per 16-token block, 8 fp32
// activations of this lane.
template <int BB>
struct Stage {
  u4 w[kRowBlocks];
  f4 x[BB][2];
};

template <int BB>
__device__ __forceinline__ void load_stage(Stage<BB>& st, KProb& P, const uint16_t* const (&wrow)[kRowBlocks],
                                           const float* xbase, int step, int lane, int b0, int batch) {
  const int g = lane >> 4, i = lane & 15;
  int k = step * 32 + 8 * g;
  k = k < P.k ? k : P.k - 8;                            // past the end: re-read the last valid 8 (masked)
#pragma unroll
  for (int nb = 0; nb < kRowBlocks; ++nb) st.w[nb] = *(const u4*)(wrow[nb] + k);
#pragma unroll
  for (int bb = 0; bb < BB; ++bb) {
    int b = b0 + 16 * bb + i;
    b = b < batch ? b : batch - 1;
    const float* xp = xbase + (int64_t)b * P.ldx + k;
    st.x[bb][0] = *(const f4*)xp;
    st.x[bb][1] = *(const f4*)(xp + 4);
  }
}

template <int BB>
__device__ __forceinline__ void mma_stage(const Stage<BB>& st, f4 (&acc)[kRowBlocks][BB], bool valid) {
  bf8 a[kRowBlocks];
#pragma unroll
  for (int nb = 0; nb < kRowBlocks; ++nb) {
    const u4 w = valid ? st.w[nb] : u4{0u, 0u, 0u, 0u};
    a[nb] = __builtin_bit_cast(bf8, w);
  }
#pragma unroll
  for (int bb = 0; bb < BB; ++bb) {
    const f8 x = {st.x[bb][0][0], st.x[bb][0][1], st.x[bb][0][2], st.x[bb][0][3],
                  st.x[bb][1][0], st.x[bb][1][1], st.x[bb][1][2], st.x[bb][1][3]};
    const bf8 hi = __builtin_convertvector(x, bf8);
    const f8 rest = x - __builtin_convertvector(hi, f8);       // exact in fp32
    const bf8 lo = __builtin_convertvector(rest, bf8);
#pragma unroll
    for (int nb = 0; nb < kRowBlocks; ++nb) {
      acc[nb][bb] = mfma_bf16(a[nb], hi, acc[nb][bb]);
      acc[nb][bb] = mfma_bf16(a[nb], lo, acc[nb][bb]);
    }
  }
}

__device__ inline int find_problem(KEpi& A, int wave) {
  int lo = 0, hi = A.n_probs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (A.p[mid].wave_base <= wave) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int BB>
__global__ void __launch_bounds__(256) gemm_kernel(EpiArgs) {
  KEpi& A = *(KEpi*)(__builtin_amdgcn_kernarg_segment_ptr());
  const int lane = threadIdx.x & 63;
  // Blocks in launch order: the hardware deals them round-robin to the 8
  // XCDs, which spreads the layers (whose cost grows with their width d)
  // evenly; a head's activations are read only by its own workgroup, so a
  // contiguous run of layers per XCD would buy no L2 reuse, only imbalance.
  const int lblock = blockIdx.x;
  const int wave = lblock * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  if (wave >= A.total_waves) return;
  KProb& P = A.p[find_problem(A, wave)];
  const int local = wave - P.wave_base;
  const int head = local / P.n_tiles, tile = local - head * P.n_tiles;
  const int n0 = tile * 64;
  const int g = lane >> 4, i = lane & 15;
  // this lane's weight row in block nb is n0 + 16 nb + i, clamped to the last
  // row (rows past N are computed from a valid row and never stored)
  const uint16_t* wrow[kRowBlocks];
#pragma unroll
  for (int nb = 0; nb < kRowBlocks; ++nb) {
    const int n = min(n0 + 16 * nb + i, P.n - 1);
    wrow[nb] = P.w + (int64_t)head * P.w_hs + (int64_t)n * P.ldw;
  }
  const float* xbase = P.x + (int64_t)head * P.x_hs;
  float* ybase = P.y + (int64_t)head * P.y_hs;
  const int steps = (P.k + 31) / 32;
  const int steps_p = (steps + kStages - 1) / kStages * kStages;
  for (int b0 = 0; b0 < A.batch; b0 += 16 * BB) {
    f4 acc[kRowBlocks][BB];
#pragma unroll
    for (int nb = 0; nb < kRowBlocks; ++nb)
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) acc[nb][bb] = f4{0.f, 0.f, 0.f, 0.f};
    Stage<BB> ring[kStages];
#pragma unroll
    for (int s = 0; s < kStages; ++s) load_stage<BB>(ring[s], P, wrow, xbase, s, lane, b0, A.batch);
    for (int s0 = 0; s0 < steps_p; s0 += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        const int s = s0 + j;
        mma_stage<BB>(ring[j], acc, s * 32 + 8 * g < P.k);
        const int nx = s + kStages < steps ? s + kStages : steps - 1;
        load_stage<BB>(ring[j], P, wrow, xbase, nx, lane, b0, A.batch);
      }
    }
    // C layout: lane (i, g) holds column b = 16 bb + i, rows 4g..4g+3 of block nb
#pragma unroll
    for (int nb = 0; nb < kRowBlocks; ++nb) {
      const int n = n0 + 16 * nb + 4 * g;
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) {
        const int b = b0 + 16 * bb + i;
        if (b < A.batch && n < P.n) *(f4*)(ybase + (int64_t)b * P.ldy + n) = acc[nb][bb];
      }
    }
  }
}

// Wide products (one copy per problem, N >= 256, e.g. the output projection):
// a workgroup of 4 waves owns 256 output rows and shares the activations.
// They are staged per 256-wide k chunk in LDS, already split into bf16
// hi/lo and laid out as MFMA B operands, so the activations cross L2 once per
// workgroup instead of once per wave (double-buffered: the next chunk's
// loads are in flight while the current chunk is used).
constexpr int kChunk = 256;
constexpr int kChunkSteps = kChunk / 32;
constexpr int kWideStages = 4;   // stages of weights in flight per wave: one per row block
static_assert(kChunkSteps % kWideStages == 0 && kWideStages == 4, "ring slots must map to the 4 row blocks");
static_assert(kChunk == 256, "the chunk staging maps 32 threads to one row's 256 values");

template <int BB>
__device__ __forceinline__ int xbuf_off(int buf, int t, int bb, int limb, int lane) {
  return ((((buf * kChunkSteps + t) * BB + bb) * 2 + limb) * 64 + lane) * 16;
}

// Chunk c of the activations, rows b0 .. b0 + 16 BB: 2 BB groups of 8 values
// per thread (32 threads cover one row's 256 values, 1 KB contiguous).
template <int BB>
__device__ __forceinline__ void load_x_chunk(f4 (&xr)[2 * BB][2], KProb& P, const float* xbase, int c, int b0,
                                             int batch) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 2 * BB; ++j) {
    int b = b0 + (tid >> 5) + 8 * j;
    b = b < batch ? b : batch - 1;
    int k = c * kChunk + 8 * (tid & 31);
    k = k < P.k ? k : P.k - 8;
    const float* xp = xbase + (int64_t)b * P.ldx + k;
    xr[j][0] = *(const f4*)xp;
    xr[j][1] = *(const f4*)(xp + 4);
  }
}

template <int BB>
__device__ __forceinline__ void store_x_chunk(char* lds, int buf, const f4 (&xr)[2 * BB][2], KProb& P, int c) {
  const int tid = threadIdx.x;
  const int kg = tid & 31, t = kg >> 2, g = kg & 3;
  const bool in = c * kChunk + 8 * kg < P.k;                // past K: zeros (the weights are masked too)
#pragma unroll
  for (int j = 0; j < 2 * BB; ++j) {
    const int bl = (tid >> 5) + 8 * j, bb = bl >> 4, i = bl & 15;
    const f8 x = in ? f8{xr[j][0][0], xr[j][0][1], xr[j][0][2], xr[j][0][3],
                         xr[j][1][0], xr[j][1][1], xr[j][1][2], xr[j][1][3]}
                    : f8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const bf8 hi = __builtin_convertvector(x, bf8);
    const bf8 lo = __builtin_convertvector(x - __builtin_convertvector(hi, f8), bf8);
    const int lane = 16 * g + i;
    *(bf8*)(lds + xbuf_off<BB>(buf, t, bb, 0, lane)) = hi;
    *(bf8*)(lds + xbuf_off<BB>(buf, t, bb, 1, lane)) = lo;
  }
}

// Stage order: stage x streams 16 rows x 128 k of one row block (rb = x & 3,
// k block x >> 2) as four 16 x 32 MFMA tiles, so each row's 256 bytes are
// requested back to back (4 KB per stage per wave, as 64 rows x 32 k would
// be, but in runs of 256 contiguous bytes instead of 64: 15-20 % more HBM
// throughput).  Ring slot x % 4 therefore always holds the same row block.
__device__ __forceinline__ void load_wide_stage(u4 (&slot)[kRowBlocks], const uint16_t* const (&wrow)[kRowBlocks],
                                                int x, int g, int K) {
  const int m = x >> 2, rb = x & 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) slot[j] = *(const u4*)(wrow[rb] + min(128 * m + 32 * j + 8 * g, K - 8));
}

template <int BB>
__global__ void __launch_bounds__(256) gemm_lds_kernel(EpiArgs) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  KEpi& A = *(KEpi*)(__builtin_amdgcn_kernarg_segment_ptr());
  const int per_xcd = gridDim.x >> 3;
  // XCD-aware numbering: blocks are dealt round-robin to the 8 XCDs, so
  // logical block (b % 8) * (grid / 8) + b / 8 gives each XCD a contiguous run
  // of workgroups of one layer, whose activations then stay in that XCD's L2
  // (every layer costs the same here: K = n_heads * d_v).
  const int lblock = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lblock >= A.total_waves) return;                      // here total_waves counts workgroups
  KProb& P = A.p[find_problem(A, lblock)];
  const int local = lblock - P.wave_base;
  const int tile = local;                                   // heads == 1
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i = lane & 15;
  const int n0 = tile * 256 + 64 * wave;
  const uint16_t* wrow[kRowBlocks];
#pragma unroll
  for (int nb = 0; nb < kRowBlocks; ++nb) wrow[nb] = P.w + (int64_t)min(n0 + 16 * nb + i, P.n - 1) * P.ldw;
  const int chunks = (P.k + kChunk - 1) / kChunk;
  const int last = 4 * ((P.k + 127) / 128) - 1;             // last stage that holds valid k
  for (int b0 = 0; b0 < A.batch; b0 += 16 * BB) {
    f4 acc[kRowBlocks][BB];
#pragma unroll
    for (int nb = 0; nb < kRowBlocks; ++nb)
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) acc[nb][bb] = f4{0.f, 0.f, 0.f, 0.f};
    f4 xr[2 * BB][2];
    load_x_chunk<BB>(xr, P, P.x, 0, b0, A.batch);
    u4 ring[kWideStages][kRowBlocks];
#pragma unroll
    for (int x = 0; x < kWideStages; ++x) {
      load_wide_stage(ring[x], wrow, min(x, last), g, P.k);
      __builtin_amdgcn_sched_barrier(0);          // issue in ring order, as the loop refills it
    }
    store_x_chunk<BB>(lds, 0, xr, P, 0);
    __syncthreads();
    for (int c = 0; c < chunks; ++c) {
      const bool more = c + 1 < chunks;
      if (more) load_x_chunk<BB>(xr, P, P.x, c + 1, b0, A.batch);
      const int buf = c & 1;
#pragma unroll
      for (int t = 0; t < kChunkSteps; ++t) {
        const int x = c * kChunkSteps + t;                  // stage: row block t & 3, k block x >> 2
        constexpr int kSlots = kWideStages;
        const int sl = t % kSlots;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tk = 4 * (t >> 2) + j;                  // k-step within the chunk
          const bool valid = 128 * (x >> 2) + 32 * j + 8 * g < P.k;
          const bf8 a = __builtin_bit_cast(bf8, valid ? ring[sl][j] : u4{0u, 0u, 0u, 0u});
#pragma unroll
          for (int bb = 0; bb < BB; ++bb) {
            const bf8 hi = *(const bf8*)(lds + xbuf_off<BB>(buf, tk, bb, 0, lane));
            const bf8 lo = *(const bf8*)(lds + xbuf_off<BB>(buf, tk, bb, 1, lane));
            acc[t & 3][bb] = mfma_bf16(a, hi, acc[t & 3][bb]);
            acc[t & 3][bb] = mfma_bf16(a, lo, acc[t & 3][bb]);
          }
        }
        load_wide_stage(ring[sl], wrow, min(x + kSlots, last), g, P.k);
        // keep the refill of the slot after its use: hoisting it would need
        // new registers and a copy (with a full wait) at the loop's back edge
        __builtin_amdgcn_sched_barrier(0);
      }
      if (more) store_x_chunk<BB>(lds, buf ^ 1, xr, P, c + 1);
      __syncthreads();
    }
#pragma unroll
    for (int nb = 0; nb < kRowBlocks; ++nb) {
      const int n = n0 + 16 * nb + 4 * g;
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) {
        const int b = b0 + 16 * bb + i;
        if (b < A.batch && n < P.n) *(f4*)(P.y + (int64_t)b * P.ldy + n) = acc[nb][bb];
      }
    }
  }
}

}  // namespace

int epilogue_lds_bytes(int batch) {
  const int bb = batch >= 64 ? 4 : (batch + 15) / 16;
  return 2 * kChunkSteps * bb * 2 * 64 * 16;
}

hipError_t launch_epilogue_gemm_wide(const EpiArgs& a, hipStream_t stream) {
  if (a.total_waves <= 0) return hipSuccess;
  const int blocks = (a.total_waves + 7) / 8 * 8;           // total_waves counts workgroups here
  const int bb = a.batch >= 64 ? 4 : (a.batch + 15) / 16;
  const int lds = epilogue_lds_bytes(a.batch);
  hipError_t e = hipSuccess;
  switch (bb) {
#define KK_LAUNCH_WIDE(B)                                                                                   \
  case B:                                                                                                   \
    e = hipFuncSetAttribute((const void*)gemm_lds_kernel<B>, hipFuncAttributeMaxDynamicSharedMemorySize, lds); \
    if (e != hipSuccess) return e;                                                                          \
    hipLaunchKernelGGL(gemm_lds_kernel<B>, dim3(blocks), dim3(256), lds, stream, a);                         \
    break;
    KK_LAUNCH_WIDE(1)
    KK_LAUNCH_WIDE(2)
    KK_LAUNCH_WIDE(3)
    default:
    KK_LAUNCH_WIDE(4)
#undef KK_LAUNCH_WIDE
  }
  return hipGetLastError();
}

hipError_t launch_epilogue_gemm(const EpiArgs& a, hipStream_t stream) {
  static_assert(sizeof(EpiArgs) < 7600, "kernel argument block too large");
  if (a.total_waves <= 0) return hipSuccess;
  const int blocks = (a.total_waves + 3) / 4;
  const int bb = a.batch >= 64 ? 4 : (a.batch + 15) / 16;
  switch (bb) {
    case 1: hipLaunchKernelGGL(gemm_kernel<1>, dim3(blocks), dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(gemm_kernel<2>, dim3(blocks), dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(gemm_kernel<3>, dim3(blocks), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(gemm_kernel<4>, dim3(blocks), dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace kk
