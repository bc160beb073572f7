// Split-T flash-decoding of absorbed-MLA attention over a per-layer
// compressed cache, for gfx950 (MI355X).
//
// What is computed (KV-Kaizen, picx.dev summary page): each layer's cache is
// its anchor's ("Three Non-Eviction Compression Axes", depth item), holding the
// first d latent coordinates plus the RoPE key (rank item) as b-bit symmetric
// codes with one scale per token (precision item).  Per query head:
//   z_t = sm_scale * (q_lat[:d] . c_t[:d] + q_rope . kR_t),  o = sum_t softmax(z)_t c_t[:d].
// Decode reads the whole cache for every token ("Background: The KV Cache
// Bottleneck"), so the kernel is built around streaming the packed codes once.
//
// Work item = (anchor-group chunk of <= 64 query rows, sequence, token split).
// A workgroup of 4 waves processes one item in 32-token tiles:
//   1. the tile's packed rows and scales are copied HBM -> LDS with direct
//      loads (global_load_lds_dwordx4), double-buffered one tile ahead;
//   2. Q.K: the 32-wide contraction chunks are split over the 4 waves; each
//      wave dequantizes its chunks of the codes to exact fp16 integers
//      (magic-number conversion) and runs v_mfma_f32_16x16x32_f16 against its
//      q fragments held in registers; partial scores go through LDS;
//   3. online softmax: the wave owning a 16-row block sums the partials,
//      applies sm_scale * per-token scale, keeps a lazily moved running max
//      (log2 domain), and writes P' = exp2(z - m) * scale_t * 2^-E as fp16;
//   4. P.V: the output features are split over the waves in 32-wide units;
//      codes are read transposed with ds_read_b64_tr_b{4,8,16}, dequantized
//      and multiplied by P' with MFMA into fp32 accumulators.
// Inheriting layers of a group add query rows to the same item, so one read
// of the anchor cache serves the whole group.  Items that were split write
// (m, l, O) partials; a second small kernel merges them in a fixed order.
//
// Exactness: codes are exact fp16 integers (|c| <= 127; b = 16 codes are split
// as hi*256 + lo with both halves exact), bf16 queries are exact in fp16 after
// a power-of-two row prescale, products are exact in the fp32 accumulators.
// The only rounding besides fp32 accumulation is P' to fp16 (2^-11 relative).
#include <hip/hip_runtime.h>

#include "kk_internal.h"

namespace kk {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef int i2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// The launch descriptor, read in place from the kernarg segment (constant
// address space, scalar loads).
typedef __attribute__((address_space(4))) const DecodeArgs KArgs;
typedef __attribute__((address_space(4))) const EntryArg KEntry;

constexpr float kLog2e = 1.4426950408889634f;

// ---- LDS map (bytes, dynamic shared memory) ----------------------------------
//  [0, 2*buf)            two tile buffers: codes of token block 0 | block 1 | scales | slack
//  sbuf                  Q.K partials   [wave][row block][token block][64 lanes] f4
//  pbuf                  P' fragments   [row block][64 lanes] h8
//  alpha / flags / rowmax / final (m, l)
constexpr int kSbufBytes = kWaves * kMaxRowBlocks * 2 * 64 * 16;
constexpr int kPbufBytes = kMaxRowBlocks * 64 * 16;
constexpr int kMiscBytes = 64 * 4 /*alpha*/ + 16 /*flags*/ + kWaves * 64 * 4 /*rowmax*/ +
                           64 * 8 /*m,l*/ + 64 /*reduce*/;

__host__ __device__ inline int nseg_of(int row_stride) { return row_stride >> 4; }
__host__ __device__ inline int chunks_of(int K) { return (K + 31) >> 5; }
__host__ __device__ inline int nsegpad_of(int K, int bits) { return (chunks_of(K) * bits + 3) >> 2; }
// one tile buffer: two token blocks of nseg segments, over-read slack, then 128 B of scales
__host__ __device__ inline int tilebuf_bytes(int row_stride, int K, int bits) {
  int nseg = nseg_of(row_stride), pad = nsegpad_of(K, bits);
  return (nseg + (pad > nseg ? pad : nseg)) * 256 + 256;
}

// ---- dequantization to exact fp16 integers ------------------------------------
__device__ inline h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }
__device__ inline uint32_t perm(uint32_t a, uint32_t b, uint32_t sel) { return __builtin_amdgcn_perm(a, b, sel); }

__device__ inline h8 pack8(h2 a, h2 b, h2 c, h2 d) {
  h8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 signed bytes (x0: elements 0..3, x1: 4..7) -> fp16 in element order.
// fp16 0x64XX = 1024 + XX; the byte is offset by 128 first (xor of its sign bit).
__device__ inline h8 cvt_b8(uint32_t x0, uint32_t x1) {
  const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  x0 ^= 0x80808080u; x1 ^= 0x80808080u;
  return pack8(as_h2(perm(0x64646464u, x0, 0x04010400u)) + bias, as_h2(perm(0x64646464u, x0, 0x04030402u)) + bias,
               as_h2(perm(0x64646464u, x1, 0x04010400u)) + bias, as_h2(perm(0x64646464u, x1, 0x04030402u)) + bias);
}

// 8 signed nibbles of x (element k at bits 4k) -> fp16 in order (0,4,1,5,2,6,3,7).
__device__ inline h8 cvt_b4(uint32_t x) {
  const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  x ^= 0x88888888u;
  return pack8(as_h2((x & 0x000F000Fu) | 0x64006400u) + bias, as_h2(((x >> 4) & 0x000F000Fu) | 0x64006400u) + bias,
               as_h2(((x >> 8) & 0x000F000Fu) | 0x64006400u) + bias, as_h2(((x >> 12) & 0x000F000Fu) | 0x64006400u) + bias);
}

// 8 signed 2-bit fields of the low 16 bits of x (element k at bits 2k) -> fp16
// in order (0,4,1,5,2,6,3,7).
__device__ inline h8 cvt_b2(uint32_t x) {
  const h2 bias = {(_Float16)-1026.0f, (_Float16)-1026.0f};
  uint32_t y = (x ^ 0xAAAAu) & 0xFFFFu;
  y |= (y >> 8) << 16;
  return pack8(as_h2((y & 0x00030003u) | 0x64006400u) + bias, as_h2(((y >> 2) & 0x00030003u) | 0x64006400u) + bias,
               as_h2(((y >> 4) & 0x00030003u) | 0x64006400u) + bias, as_h2(((y >> 6) & 0x00030003u) | 0x64006400u) + bias);
}

// 2-bit fields of nibble-packed data from a 4-bit transpose read: element e at
// bits 4e (even field) or 4e + 2 (odd field); result order (0,4,1,5,2,6,3,7).
__device__ inline h8 cvt_b2_nib(uint32_t x, int odd) {
  const h2 bias = {(_Float16)-1026.0f, (_Float16)-1026.0f};
  uint32_t y = (x ^ 0xAAAAAAAAu) >> (odd ? 2 : 0);
  return pack8(as_h2((y & 0x00030003u) | 0x64006400u) + bias, as_h2(((y >> 4) & 0x00030003u) | 0x64006400u) + bias,
               as_h2(((y >> 8) & 0x00030003u) | 0x64006400u) + bias, as_h2(((y >> 12) & 0x00030003u) | 0x64006400u) + bias);
}

// 8 int16 codes (w0..w3 little-endian) -> hi (signed high byte) and lo/256
// (unsigned low byte scaled by 2^-8, exact: fp16 0x44XX = 4 + XX/256).
__device__ inline void cvt_b16(u4 w, h8& hi, h8& lo) {
  const h2 bh = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const h2 bl = {(_Float16)-4.0f, (_Float16)-4.0f};
  u4 x = w ^ 0x80008000u;
  hi = pack8(as_h2(perm(0x64646464u, x[0], 0x04030401u)) + bh, as_h2(perm(0x64646464u, x[1], 0x04030401u)) + bh,
             as_h2(perm(0x64646464u, x[2], 0x04030401u)) + bh, as_h2(perm(0x64646464u, x[3], 0x04030401u)) + bh);
  lo = pack8(as_h2(perm(0x44444444u, w[0], 0x04020400u)) + bl, as_h2(perm(0x44444444u, w[1], 0x04020400u)) + bl,
             as_h2(perm(0x44444444u, w[2], 0x04020400u)) + bl, as_h2(perm(0x44444444u, w[3], 0x04020400u)) + bl);
}

__device__ inline f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

__device__ inline float wave_max_xor_16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ inline float wave_sum_xor_16_32(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Byte offset of (token block tb, segment seg, token-in-block t) inside a tile
// buffer.  Token block 1 swaps slot groups of 4 (t ^ 4) so that the transposed
// P.V reads of tokens {4g..4g+3} of both blocks land in different LDS banks.
__device__ inline int tile_off(int pitch, int tb, int seg, int t) { return tb * pitch + seg * 256 + ((t ^ (tb << 2)) << 4); }

// ---- per-item decode, specialised on the bit width ------------------------------
template <int BITS>
__device__ void run_item(KArgs& A, KEntry& E, int s, int ksplit, int chunk, char* lds) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, n = lane & 15;
  const int d = E.d, K = d + A.d_rope, KC = chunks_of(K);
  const int NSEG = nseg_of(E.row_stride), PITCH = NSEG * 256;
  const int bufbytes = tilebuf_bytes(E.row_stride, K, BITS);
  char* sbuf = lds + 2 * bufbytes;
  char* pbuf = sbuf + kSbufBytes;
  float* alpha_lds = (float*)(pbuf + kPbufBytes);
  int* flag_lds = (int*)(alpha_lds + 64);
  float* rowmax_lds = (float*)(flag_lds + 4);
  float* ml_lds = rowmax_lds + kWaves * 64;
  float* red_lds = ml_lds + 128;

  // rows of this chunk
  const int r0 = E.row_begin + chunk * E.chunk_rows;
  const int nrows = min(E.chunk_rows, E.row_end - r0);
  const int RB = (nrows + 15) >> 4;

  // token range of this split
  int len = A.seq_lens[s];
  len = len < 0 ? 0 : (len > A.t_cap ? A.t_cap : len);
  const int tps = ((len + E.splits - 1) / E.splits + kTile - 1) / kTile * kTile;
  const int t0 = ksplit * tps;
  const int t1 = min(len, t0 + tps);
  const int ntok = t1 > t0 ? t1 - t0 : 0;
  const int ntiles = (ntok + kTile - 1) / kTile;
  const int64_t row0 = (int64_t)s * A.t_cap + t0;    // first cache row of this item

  // ---- scale exponent E: s_t * 2^-E <= 1 for every token of the item -------------
  float smax = 0.0f;
  for (int t = tid; t < ntok; t += kThreads) smax = fmaxf(smax, E.scales[row0 + t]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) smax = fmaxf(smax, __shfl_xor(smax, o));
  if (lane == 0) red_lds[wave] = smax;

  // ---- q fragments (registers), with a power-of-two prescale per row ---------------
  // fragment (ci, rb): chunk c = wave + 4*ci, lane (g, n): row 16*rb + n, features
  // 32c + 8g + slot order (identity for b >= 8, (0,4,1,5,2,6,3,7) for b <= 4).
  float qv[kMaxChunksPerWave][kMaxRowBlocks][8];
  float rmax[kMaxRowBlocks];
  int row_layer[kMaxRowBlocks], row_head[kMaxRowBlocks];
#pragma unroll
  for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
    rmax[rb] = 0.0f;
    const int rl = 16 * rb + n;
    row_layer[rb] = -1;
    row_head[rb] = 0;
    if (rl < nrows) {
      const int gr = r0 + rl;
      row_layer[rb] = A.group_layers[E.lay_begin + gr / A.heads];
      row_head[rb] = gr % A.heads;
    }
  }
#pragma unroll
  for (int ci = 0; ci < kMaxChunksPerWave; ++ci) {
    const int c = wave + kWaves * ci;
    const int f0 = 32 * c + 8 * g;
#pragma unroll
    for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.0f;
      if (c < KC && row_layer[rb] >= 0 && f0 < K) {
        const int64_t qrow = ((int64_t)row_layer[rb] * A.batch + s) * A.heads + row_head[rb];
        const bool lat = f0 < d;
        const int64_t off = lat ? qrow * A.r + f0 : qrow * A.d_rope + (f0 - d);
        const void* base = lat ? A.q_lat : A.q_rope;
        if (A.q_is_f32) {
          const f4* p = (const f4*)((const float*)base + off);
          f4 a = p[0], b = p[1];
#pragma unroll
          for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
        } else {
          u4 w = *(const u4*)((const uint16_t*)base + off);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int src = BITS <= 4 ? ((i & 1) ? 4 + (i >> 1) : (i >> 1)) : i;
        qv[ci][rb][i] = x[src];
        rmax[rb] = fmaxf(rmax[rb], fabsf(x[i]));
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
    rmax[rb] = wave_max_xor_16_32(rmax[rb]);
    if (g == 0) rowmax_lds[wave * 64 + 16 * rb + n] = rmax[rb];
  }
  __syncthreads();
  float item_smax = fmaxf(fmaxf(red_lds[0], red_lds[1]), fmaxf(red_lds[2], red_lds[3]));
  int Eexp = 0;
  if (item_smax > 0.0f) (void)frexpf(item_smax, &Eexp);     // item_smax * 2^-Eexp in [0.5, 1)
  h8 qf[kMaxChunksPerWave][kMaxRowBlocks];
  float rowf[kMaxRowBlocks];                                  // used by the softmax wave
  constexpr float kBitScale = BITS == 16 ? 256.0f : 1.0f;
#pragma unroll
  for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
    float m = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, rowmax_lds[w * 64 + 16 * rb + n]);
    int e = 0;
    if (m > 0.0f) (void)frexpf(m, &e);
    const float pre = ldexpf(1.0f, -e);
#pragma unroll
    for (int ci = 0; ci < kMaxChunksPerWave; ++ci)
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[ci][rb][i] = (_Float16)(qv[ci][rb][i] * pre);
    rowf[rb] = row_layer[rb] >= 0 ? A.layers[row_layer[rb]].sm_scale * kLog2e * ldexpf(kBitScale, e) : 0.0f;
  }

  // ---- tile loader: direct HBM -> LDS copies ---------------------------------------
  const uint8_t* codes = E.codes;
  const float* scales = E.scales;
  auto issue_tile = [&](int it) {
    char* buf = lds + (it & 1) * bufbytes;
    const int tok0 = it * kTile;
    const int tvalid = min(kTile, ntok - tok0);
    const int npos = 32 * NSEG;                  // 16-byte pieces of codes in the tile
    const int ninst = (npos + 63) >> 6;
    for (int i = wave; i < ninst; i += kWaves) {
      const int p = i * 64 + lane;
      const int tb = p / (NSEG * 16);
      const int rem = p - tb * NSEG * 16;
      const int seg = rem >> 4, slot = rem & 15;
      const int t = 16 * tb + (slot ^ (tb << 2));
      if (p < npos && t < tvalid) {
        const uint8_t* gp = codes + (row0 + tok0 + t) * (int64_t)E.row_stride + seg * 16;
        __builtin_amdgcn_global_load_lds(gp, LDS_PTR(void, buf + i * 1024), 16, 0, 0);
      }
    }
    if (wave == kWaves - 1 && lane < kTile && lane < tvalid) {
      __builtin_amdgcn_global_load_lds(scales + row0 + tok0 + lane, LDS_PTR(void, buf + 2 * PITCH), 4, 0, 0);
    }
  };

  // ---- accumulators -------------------------------------------------------------
  f4 oacc[kMaxUnitsPerWave][2][kMaxRowBlocks];
#pragma unroll
  for (int u = 0; u < kMaxUnitsPerWave; ++u)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int rb = 0; rb < kMaxRowBlocks; ++rb) oacc[u][f][rb] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.0f;     // softmax state of row 16*wave + n (wave < RB)
  const float sprime = ldexpf(1.0f, -Eexp);
  const int NU = (d + 31) >> 5;               // 32-feature output units
  const int nqk = min(kWaves, KC);             // waves holding Q.K chunks

  if (ntiles > 0) issue_tile(0);
  for (int it = 0; it < ntiles; ++it) {
    __builtin_amdgcn_s_waitcnt(0x3f70);        // vmcnt(0): this tile's copies have landed
    __syncthreads();                            // (A) tile visible; previous P.V finished
    if (it + 1 < ntiles) issue_tile(it + 1);
    const char* buf = lds + (it & 1) * bufbytes;
    const float* sc = (const float*)(buf + 2 * PITCH);
    const int tvalid = min(kTile, ntok - it * kTile);

    // ---- Q.K partial over this wave's chunks ----
    f4 sacc[kMaxRowBlocks][2];
#pragma unroll
    for (int rb = 0; rb < kMaxRowBlocks; ++rb) sacc[rb][0] = sacc[rb][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int ci = 0; ci < kMaxChunksPerWave; ++ci) {
        const int c = wave + kWaves * ci;
        if (c < KC) {
        const int piece = 4 * c + g;                 // 8 fields of BITS bits = BITS bytes
        const int byte = piece * BITS;
        const char* p = buf + tile_off(PITCH, tb, byte >> 4, n) + (byte & 15);
        if constexpr (BITS == 16) {
          h8 hi, lo;
          cvt_b16(*(const u4*)p, hi, lo);
#pragma unroll
          for (int rb = 0; rb < kMaxRowBlocks; ++rb)
            if (rb < RB) {
              sacc[rb][tb] = mfma(hi, qf[ci][rb], sacc[rb][tb]);
              sacc[rb][tb] = mfma(lo, qf[ci][rb], sacc[rb][tb]);
            }
        } else {
          h8 a;
          if constexpr (BITS == 8) { u2 x = *(const u2*)p; a = cvt_b8(x[0], x[1]); }
          if constexpr (BITS == 4) { a = cvt_b4(*(const uint32_t*)p); }
          if constexpr (BITS == 2) { a = cvt_b2(*(const uint16_t*)p); }
#pragma unroll
          for (int rb = 0; rb < kMaxRowBlocks; ++rb)
            if (rb < RB) sacc[rb][tb] = mfma(a, qf[ci][rb], sacc[rb][tb]);
        }
        }
      }
    }
    if (wave < nqk) {
#pragma unroll
      for (int rb = 0; rb < kMaxRowBlocks; ++rb)
        if (rb < RB)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            ((f4*)sbuf)[((wave * kMaxRowBlocks + rb) * 2 + tb) * 64 + lane] = sacc[rb][tb];
    }
    __syncthreads();                            // (B) partial scores visible

    // ---- online softmax for row block `wave` ----
    if (wave < RB) {
      const int rb = wave;
      float rf = 0.0f;
#pragma unroll
      for (int q = 0; q < kMaxRowBlocks; ++q) if (q == rb) rf = rowf[q];
      float z[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        f4 acc = ((const f4*)sbuf)[((0 * kMaxRowBlocks + rb) * 2 + tb) * 64 + lane];
        for (int w = 1; w < nqk; ++w) acc += ((const f4*)sbuf)[((w * kMaxRowBlocks + rb) * 2 + tb) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * tb + 4 * g + j;
          z[tb][j] = t < tvalid ? acc[j] * rf * sc[t] : -INFINITY;
          tmax = fmaxf(tmax, z[tb][j]);
        }
      }
      tmax = wave_max_xor_16_32(tmax);
      const bool need = tmax > m_run + kLazyRescale;
      int flag = 0;
      if (__any(need)) {
        const float mnew = fmaxf(m_run, tmax);
        const float alpha = exp2f(m_run - mnew);
        l_lane *= alpha;
        m_run = mnew;
        if (g == 0) alpha_lds[16 * rb + n] = alpha;
        flag = 1;
      }
      if (lane == 0) flag_lds[rb] = flag;
      h8 pf;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * tb + 4 * g + j;
          const float e = exp2f(z[tb][j] - m_run);
          l_lane += e;
          pf[4 * tb + j] = (_Float16)(t < tvalid ? e * (sc[t] * sprime) : 0.0f);
        }
      ((h8*)pbuf)[rb * 64 + lane] = pf;
    }
    __syncthreads();                            // (C) P' and rescale factors visible

    // ---- P.V over this wave's output units ----
    h8 pfr[kMaxRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
      if (rb < RB) {
        pfr[rb] = ((const h8*)pbuf)[rb * 64 + lane];
        if (flag_lds[rb]) {
          const float al = alpha_lds[16 * rb + n];
#pragma unroll
          for (int u = 0; u < kMaxUnitsPerWave; ++u)
#pragma unroll
            for (int f = 0; f < 2; ++f) oacc[u][f][rb] *= al;
        }
      }
    }
#pragma unroll
    for (int ui = 0; ui < kMaxUnitsPerWave; ++ui) {
      const int u = wave + kWaves * ui;
      if (u < NU) {
      h8 a[2], alo[2];
      if constexpr (BITS == 8) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int e = n >> 1, h = n & 1, tb = e >> 2;
          const char* p = buf + tile_off(PITCH, tb, 2 * u + f, 4 * g + (e & 3)) + 8 * h;
          i2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i2, p));
          a[f] = cvt_b8((uint32_t)x[0], (uint32_t)x[1]);
        }
      }
      if constexpr (BITS == 4 || BITS == 2) {
        const int e = n & 7, half = n >> 3;
        const int tb = (e >> 1) & 1, t = 4 * g + 2 * (e & 1) + (e >> 2);
        const char* p = BITS == 4 ? buf + tile_off(PITCH, tb, u, t) + 8 * half
                                  : buf + tile_off(PITCH, tb, u >> 1, t) + 8 * (u & 1);
        i2 x = __builtin_amdgcn_ds_read_tr4_b64_v2i32(LDS_PTR(i2, p));
        if constexpr (BITS == 4) { a[0] = cvt_b4((uint32_t)x[0]); a[1] = cvt_b4((uint32_t)x[1]); }
        else { a[0] = cvt_b2_nib((uint32_t)x[0], 0); a[1] = cvt_b2_nib((uint32_t)x[0], 1); }
      }
      if constexpr (BITS == 16) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int fb = 2 * u + f, e = n >> 2, q = n & 3;
          const int seg = 2 * fb + (q >> 1), off = 8 * (q & 1);
          s4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s4, buf + tile_off(PITCH, 0, seg, 4 * g + e) + off));
          s4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s4, buf + tile_off(PITCH, 1, seg, 4 * g + e) + off));
          u2 y0 = __builtin_bit_cast(u2, x0), y1 = __builtin_bit_cast(u2, x1);
          cvt_b16(u4{y0[0], y0[1], y1[0], y1[1]}, a[f], alo[f]);
        }
      }
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int rb = 0; rb < kMaxRowBlocks; ++rb)
          if (rb < RB) {
            oacc[ui][f][rb] = mfma(a[f], pfr[rb], oacc[ui][f][rb]);
            if constexpr (BITS == 16) oacc[ui][f][rb] = mfma(alo[f], pfr[rb], oacc[ui][f][rb]);
          }
      }
    }
  }

  // ---- finish: row sums, then normalized output or split partial -----------------
  if (wave < RB) {
    const float lrow = wave_sum_xor_16_32(l_lane);
    if (g == 0) { ml_lds[2 * (16 * wave + n)] = m_run; ml_lds[2 * (16 * wave + n) + 1] = lrow; }
  }
  __syncthreads();
  const float outscale = ldexpf(kBitScale, Eexp);
  const bool split = E.splits > 1;
  float* part = nullptr;
  if (split) {
    const int64_t slot = ((int64_t)(s * E.splits + ksplit) * E.nrc + chunk);
    part = A.ws + E.ws_off + slot * partial_slot_floats(d);
    if (tid < 64) {
      part[64 * (int64_t)d + tid] = ml_lds[2 * tid];
      part[64 * (int64_t)d + 64 + tid] = ml_lds[2 * tid + 1];
    }
  }
#pragma unroll
  for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
    const int rl = 16 * rb + n;
    if (rb < RB && rl < nrows) {
      const float lrow = ml_lds[2 * rl + 1];
      const float fac = split ? outscale : (lrow > 0.0f ? outscale / lrow : 0.0f);
      float* dst = split ? part + (int64_t)rl * d
                         : A.out + A.layers[row_layer[rb]].out_off + ((int64_t)s * A.heads + row_head[rb]) * d;
#pragma unroll
      for (int ui = 0; ui < kMaxUnitsPerWave; ++ui) {
        const int u = wave + kWaves * ui;
        if constexpr (BITS == 2) {
          const int fbase = 32 * u + 8 * g;
          if (u < NU && fbase < d) {
            f4 e0 = oacc[ui][0][rb] * fac, e1 = oacc[ui][1][rb] * fac;
            *(f4*)(dst + fbase) = f4{e0[0], e1[0], e0[1], e1[1]};
            *(f4*)(dst + fbase + 4) = f4{e0[2], e1[2], e0[3], e1[3]};
          }
        } else {
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const int fbase = 32 * u + 16 * f + 4 * g;
            if (u < NU && fbase < d) *(f4*)(dst + fbase) = oacc[ui][f][rb] * fac;
          }
        }
      }
    }
  }
}

__device__ inline int find_entry(KArgs& A, int item) {
  int lo = 0, hi = A.n_entries - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (A.entries[mid].item_base <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The argument block is read in place from the kernarg segment (a by-value
// parameter that is referenced would be copied to scratch memory).
__device__ inline KArgs& kernel_args() {
  return *(KArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
}

// One kernel per bit width (entries are ordered by bit width on the host, so
// each launch covers a contiguous item range): each specialisation is
// register-allocated on its own.
template <int BITS>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(DecodeArgs, int item_begin) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  KArgs& A = kernel_args();
  const int item = item_begin + blockIdx.x;
  const int ei = find_entry(A, item);
  KEntry& E = A.entries[ei];
  // item numbering: chunks of one (sequence, split) pair sit 8 blocks apart, so
  // they are dispatched to the same XCD at about the same time and share its L2.
  const int local = item - E.item_base;
  const int J = A.batch * E.splits, nrc = E.nrc;
  const int q8 = J >> 3, r8 = J & 7;
  int chunk, j;
  if (local < 8 * q8 * nrc) {
    const int blk = local / (8 * nrc), rem = local - blk * 8 * nrc;
    chunk = rem >> 3;
    j = blk * 8 + (rem & 7);
  } else {
    const int rem = local - 8 * q8 * nrc;
    chunk = rem / r8;
    j = 8 * q8 + rem % r8;
  }
  const int s = j / E.splits, ks = j - s * E.splits;
  run_item<BITS>(A, E, s, ks, chunk, lds);
}

// Merge split partials of one (entry, sequence, chunk): fixed split order.
__global__ void __launch_bounds__(256) merge_kernel(DecodeArgs) {
  KArgs& A = kernel_args();
  const int blk = blockIdx.x;
  int ei = -1;
  for (int e = 0; e < A.n_entries; ++e)
    if (A.entries[e].splits > 1 && A.entries[e].merge_base <= blk) ei = e;
  if (ei < 0) return;
  KEntry& E = A.entries[ei];
  const int local = blk - E.merge_base;
  if (local >= A.batch * E.nrc) return;
  const int s = local / E.nrc, chunk = local - s * E.nrc;
  const int d = E.d;
  const int r0 = E.row_begin + chunk * E.chunk_rows;
  const int nrows = min(E.chunk_rows, E.row_end - r0);
  const int64_t slotf = partial_slot_floats(d);
  const float* base = A.ws + E.ws_off + (int64_t)(s * E.splits) * E.nrc * slotf + chunk * slotf;
  const int64_t kstride = E.nrc * slotf;
  for (int idx = threadIdx.x; idx < nrows * d; idx += 256) {
    const int rl = idx / d, f = idx - rl * d;
    float M = -INFINITY;
    for (int k = 0; k < E.splits; ++k) {
      const float* p = base + k * kstride;
      if (p[64 * (int64_t)d + 64 + rl] > 0.0f) M = fmaxf(M, p[64 * (int64_t)d + rl]);
    }
    float L = 0.0f, acc = 0.0f;
    for (int k = 0; k < E.splits; ++k) {
      const float* p = base + k * kstride;
      const float l = p[64 * (int64_t)d + 64 + rl];
      if (l > 0.0f) {
        const float w = exp2f(p[64 * (int64_t)d + rl] - M);
        L += l * w;
        acc += p[(int64_t)rl * d + f] * w;
      }
    }
    const int gr = r0 + rl;
    const int layer = A.group_layers[E.lay_begin + gr / A.heads], head = gr % A.heads;
    A.out[A.layers[layer].out_off + ((int64_t)s * A.heads + head) * d + f] = L > 0.0f ? acc / L : 0.0f;
  }
}

}  // namespace

int decode_lds_bytes(int row_stride, int K, int bits) {
  return 2 * tilebuf_bytes(row_stride, K, bits) + kSbufBytes + kPbufBytes + kMiscBytes;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodeLaunch& L, hipStream_t stream) {
  static_assert(sizeof(DecodeArgs) < 7600, "kernel argument block too large");
  for (int c = 0; c < 4; ++c) {
    const int n = L.item_end[c] - L.item_begin[c];
    if (n <= 0) continue;
    const void* fn = c == 0 ? (const void*)decode_kernel<2> : c == 1 ? (const void*)decode_kernel<4>
                   : c == 2 ? (const void*)decode_kernel<8> : (const void*)decode_kernel<16>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L.lds_bytes[c]);
    if (e != hipSuccess) return e;
    switch (c) {
      case 0: hipLaunchKernelGGL(decode_kernel<2>, dim3(n), dim3(kThreads), L.lds_bytes[c], stream, a, L.item_begin[c]); break;
      case 1: hipLaunchKernelGGL(decode_kernel<4>, dim3(n), dim3(kThreads), L.lds_bytes[c], stream, a, L.item_begin[c]); break;
      case 2: hipLaunchKernelGGL(decode_kernel<8>, dim3(n), dim3(kThreads), L.lds_bytes[c], stream, a, L.item_begin[c]); break;
      default: hipLaunchKernelGGL(decode_kernel<16>, dim3(n), dim3(kThreads), L.lds_bytes[c], stream, a, L.item_begin[c]); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (L.merge_blocks > 0) {
    hipLaunchKernelGGL(merge_kernel, dim3(L.merge_blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace kk
