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
// Work item = (chunk of <= 16*RB query rows of one anchor group, sequence,
// token split).  A workgroup of 4 waves processes one item in tiles of 32
// tokens (16 for b = 16), two to four workgroups per CU (by the register budget
// of the kernel variant):
//   1. the tile's packed rows and scales are copied HBM -> LDS with direct
//      loads (global_load_lds), several tiles ahead (explicit vmcnt waits);
//   2. Q.K on the integer MFMA: wave w < RB owns query rows 16w..16w+15.  The
//      codes are used as int8 operands directly (b = 8), after a shift/mask
//      that moves each field to the top of its byte (b = 4, 2), or (b = 16)
//      as the row's two byte planes: signed high bytes and offset-binary low
//      bytes, with an exact integer bias correction.
//      Each part of a query row is a fixed-point number relative to its own
//      largest magnitude (15 bits latent, 22 bits RoPE) held as int8 limbs, so
//      scores accumulate exactly in int32;
//   3. online softmax in the same wave (no exchange): per-token scale and
//      sm_scale applied in fp32, running max in the log2 domain moved lazily,
//      P' = exp2(z - m - E) * scale_t written to LDS as fp16, with E a
//      lazily raised power-of-two bound of the scales seen;
//   4. P.V on the fp16 MFMA, output features split over the waves in 32-wide
//      units; codes are read transposed with ds_read_b64_tr_b{4,8} and
//      converted to fp16: exact integers for b <= 8 (magic-number conversion),
//      int16 rebuilt from the two planes and rounded to 11 significant bits
//      for b = 16.
// Each stage runs P.V of tile t and Q.K + softmax of tile t+1 between two
// barriers.  Inheriting layers of a group are extra query rows of the same
// items.  Items that were split write (m, l, O) partials; a small kernel
// merges them.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstring>
#include <type_traits>

#include "kk_internal.h"

namespace kk {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef int i2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// The launch descriptor, read in place from the kernarg segment (constant
// address space, scalar loads).
typedef __attribute__((address_space(4))) const DecodeArgs KArgs;
typedef __attribute__((address_space(4))) const EntryArg KEntry;
typedef __attribute__((address_space(4))) const LayerArg KLayer;
typedef __attribute__((address_space(4))) const uint16_t KU16;

// Plan arrays: in the launch arguments (one table) or in device memory
// (several tables); both are read-only for the launch, so scalar loads.
__device__ inline KEntry* entry_array(KArgs& A) { return A.plan.entries ? (KEntry*)A.plan.entries : A.entries; }
__device__ inline KLayer& layer_at(KArgs& A, int i) {
  return A.plan.entries ? ((KLayer*)A.plan.layers)[i] : A.layers[i];
}
__device__ inline int group_layer_at(KArgs& A, int i) {
  return A.plan.entries ? ((KU16*)A.plan.group_layers)[i] : A.group_layers[i];
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kQMax = 16256.0f;    // latent query fixed point: |q'| <= 127 * 128, two int8 limbs
constexpr float kQMaxRope = 16256.0f * 128.0f;   // RoPE query: |q'| <= 127 * 128^2, three int8 limbs
constexpr int kMaxRopeChunks = 2;    // d_R <= 128
constexpr int kScaleHeadroom = 6;    // scales may exceed 2^E by 2^6 before E is raised
// Copy instructions (1 KB each) per tile: a tile holds at most 32 * K bytes of
// codes (32 tokens of 8-bit codes or 16 tokens of 16-bit codes), shared
// round-robin by the waves, so each wave issues at most kCopyRounds of them.
constexpr int kCopyRounds = 5;
static_assert((32 * kMaxK / 1024 + kWaves - 1) / kWaves <= kCopyRounds, "copy rounds too few for K");

// The LDS map (tile buffers, P' fragments, softmax state) and its sizes are in
// kk_internal.h, shared with the host planner.

// ---- operand conversions ------------------------------------------------------
__device__ inline h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }
__device__ inline uint32_t perm(uint32_t a, uint32_t b, uint32_t sel) { return __builtin_amdgcn_perm(a, b, sel); }

__device__ inline h8 pack8(h2 a, h2 b, h2 c, h2 d) {
  h8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// fp16 exact integers for the P.V operand.  fp16 0x64XX = 1024 + XX.
// 8 signed bytes (x0: elements 0..3, x1: 4..7) -> fp16 in element order.
__device__ inline h8 cvt_b8(uint32_t x0, uint32_t x1) {
  const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  x0 ^= 0x80808080u; x1 ^= 0x80808080u;
  return pack8(as_h2(perm(0x64646464u, x0, 0x04010400u)) + bias, as_h2(perm(0x64646464u, x0, 0x04030402u)) + bias,
               as_h2(perm(0x64646464u, x1, 0x04010400u)) + bias, as_h2(perm(0x64646464u, x1, 0x04030402u)) + bias);
}
// 8 signed nibbles of x (element k at bits 4k) -> fp16 in order (0,4,1,5,2,6,3,7).
// (nibble & 15) ^ 8 is the offset-binary code c + 8; the exponent bits 0x6400
// are merged by the same xor (they are zero after the mask): 1024 + c + 8.
__device__ inline h8 cvt_b4(uint32_t x) {
  const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  return pack8(as_h2((x & 0x000F000Fu) ^ 0x64086408u) + bias, as_h2(((x >> 4) & 0x000F000Fu) ^ 0x64086408u) + bias,
               as_h2(((x >> 8) & 0x000F000Fu) ^ 0x64086408u) + bias, as_h2(((x >> 12) & 0x000F000Fu) ^ 0x64086408u) + bias);
}
// 2-bit fields of nibble-packed data from a 4-bit transpose read: element e at
// bits 4e (even field) or 4e + 2 (odd field); result order (0,4,1,5,2,6,3,7).
template <int ODD>
__device__ inline h8 cvt_b2_nib(uint32_t x) {
  const h2 bias = {(_Float16)-1026.0f, (_Float16)-1026.0f};
  const uint32_t y = x >> (2 * ODD);
  return pack8(as_h2((y & 0x00030003u) ^ 0x64026402u) + bias, as_h2(((y >> 4) & 0x00030003u) ^ 0x64026402u) + bias,
               as_h2(((y >> 8) & 0x00030003u) ^ 0x64026402u) + bias, as_h2(((y >> 12) & 0x00030003u) ^ 0x64026402u) + bias);
}

// int8 operands for the Q.K MFMA (16 features per lane).  A b-bit two's
// complement field moved to the top of its byte, with the bits below cleared,
// is the signed byte 2^(8-b) * code exactly, so no offset or bias correction
// is needed; the factor 2^(8-b) is divided out with the row scale.
// b = 4: 16 nibbles (x0: 0..7, x1: 8..15) -> 16 * code,
//        slot order 0,2,4,6 | 1,3,5,7 | 8,10,12,14 | 9,11,13,15.
__device__ inline i4 qk_b4(uint32_t x0, uint32_t x1) {
  return i4{(int)((x0 << 4) & 0xF0F0F0F0u), (int)(x0 & 0xF0F0F0F0u), (int)((x1 << 4) & 0xF0F0F0F0u), (int)(x1 & 0xF0F0F0F0u)};
}
// b = 2: 16 fields of x -> 64 * code; slot 4j + k holds field 4k + j.
__device__ inline i4 qk_b2(uint32_t x) {
  return i4{(int)((x << 6) & 0xC0C0C0C0u), (int)((x << 4) & 0xC0C0C0C0u), (int)((x << 2) & 0xC0C0C0C0u), (int)(x & 0xC0C0C0C0u)};
}
// Q.K operand scale of b-bit codes (see qk_b4 / qk_b2)
template <int BITS>
constexpr float qk_code_scale() { return BITS == 4 ? 1.0f / 16.0f : BITS == 2 ? 1.0f / 64.0f : 1.0f; }
// feature (within a lane's 16) held by operand slot i
template <int BITS>
__device__ constexpr int qk_slot_feature(int i) {
  return BITS == 4 ? ((i >> 3) << 3) + ((i & 3) << 1) + ((i >> 2) & 1)
       : BITS == 2 ? ((i & 3) << 2) + (i >> 2)
       : i;
}

__device__ inline f4 mfma_f16(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ inline i4 mfma_i8(i4 a, i4 b, i4 c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }

// Reductions over the four 16-lane rows of a wave (lanes n, n+16, n+32, n+48)
// with the gfx950 row-swap instructions: v_permlane16_swap exchanges odd and
// even 16-lane rows, v_permlane32_swap the two 32-lane halves.  Called with
// both operands equal, they return (row 0, row 0, row 2, row 2) and
// (row 1, row 1, row 3, row 3) (resp. (half 0, half 0), (half 1, half 1)), so
// op(r[0], r[1]) is the pairwise result, in the same operand order on every lane.
// v_max_f32 on values known to be ordinary floats or infinities: fmaxf would
// first canonicalize operands that arrive through an integer bit cast.
__device__ inline float max_plain(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float max_xor_16_32(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = max_plain(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t y = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return max_plain(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_xor_16_32(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t y = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Workgroup barrier for LDS hand-offs.  __syncthreads() also fences memory,
// which drains every outstanding HBM -> LDS copy (they count as LDS stores) and
// so would serialize the tile pipeline; here only the LDS operations of the
// calling wave are waited for, and copies are waited for explicitly (vm_wait).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// HBM -> LDS copies (global_load_lds): lane i writes LDS at lds_base + i*16
// (dwordx4) or lds_base + i*4 (dword).  Written as asm so that the compiler's
// wait insertion does not see them: it cannot tell that they never alias the
// LDS reads of the tile being computed and would drain every copy in flight
// before each such read.  All waits for them are explicit (vm_wait).  M0 holds
// the LDS base; the nop covers the M0-write hazard.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Address = 64-bit scalar base + 32-bit per-lane byte offset (SADDR form).
__device__ inline void copy16_to_lds(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
__device__ inline void copy4_to_lds(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ inline uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)LDS_PTR(const void, p));
}
__device__ inline const void* uniform_ptr(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x), hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Waits until at most n (wave-uniform, clamped to 0..63) vector memory
// operations of this wave are outstanding.  s_waitcnt only takes an immediate,
// so this jumps into a table of 64 "s_waitcnt vmcnt(k); s_branch end" pairs
// (8 bytes each) at 8*k bytes past its start: two jumps per call, where a
// compare-and-branch tree over the same cases costs five or six.  s_getpc
// yields the address of the instruction after it, which is where the
// label-difference offset is measured from.
#define KK_VMW(k) "s_waitcnt vmcnt(" #k ")\n\ts_branch .Lend%=\n\t"
#define KK_VMW10(a) \
  KK_VMW(a##0) KK_VMW(a##1) KK_VMW(a##2) KK_VMW(a##3) KK_VMW(a##4) KK_VMW(a##5) KK_VMW(a##6) KK_VMW(a##7) KK_VMW(a##8) KK_VMW(a##9)
__device__ inline void vm_wait(int n) {
  const int k = __builtin_amdgcn_readfirstlane(n < 0 ? 0 : n > 63 ? 63 : n);
  asm volatile(
      "s_getpc_b64 s[98:99]\n"
      ".Lpc%=:\n\t"
      "s_lshl_b32 s97, %0, 3\n\t"
      "s_add_u32 s98, s98, s97\n\t"
      "s_addc_u32 s99, s99, 0\n\t"
      "s_add_u32 s98, s98, .Ltab%=-.Lpc%=\n\t"
      "s_addc_u32 s99, s99, 0\n\t"
      "s_setpc_b64 s[98:99]\n"
      ".Ltab%=:\n\t"
      KK_VMW(0) KK_VMW(1) KK_VMW(2) KK_VMW(3) KK_VMW(4) KK_VMW(5) KK_VMW(6) KK_VMW(7) KK_VMW(8) KK_VMW(9)
      KK_VMW10(1) KK_VMW10(2) KK_VMW10(3) KK_VMW10(4) KK_VMW10(5)
      KK_VMW(60) KK_VMW(61) KK_VMW(62) KK_VMW(63)
      ".Lend%=:\n" ::"s"(k)
      : "s97", "s98", "s99", "scc", "memory");
}
#undef KK_VMW10
#undef KK_VMW

__device__ inline int isum_xor_16_32(int v) {
  const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = (int)a[0] + (int)a[1];
  const auto b = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)b[0] + (int)b[1];
}

// Byte offset of (token block tb, segment seg, token-in-block t) inside a tile
// buffer.  Token block 1 swaps the two halves of each 256-byte segment
// (t ^ 8): a transposed P.V read takes tokens 4g..4g+3 of both blocks, and with
// the swap the 32 lanes of g = 0, 1 (and of g = 2, 3) cover all 64 banks once;
// with a swap of groups of 4 (t ^ 4) they would hit 32 banks twice (measured:
// two-way conflicts on gfx950, which serves 32 lanes x 8 bytes per pass).
__device__ inline int tile_off(int pitch, int tb, int seg, int t) { return tb * pitch + seg * 256 + ((t ^ (tb << 3)) << 4); }

// ---- per-item decode ----------------------------------------------------------
// Tiles hold 2 token blocks of 16 (32 tokens) for b <= 8 and 1 block (16
// tokens) for b = 16, whose rows are up to 8x longer, so that every entry keeps
// three or more tiles in LDS (two in use, the rest in flight).
template <int BITS>
constexpr int tile_blocks() { return BITS == 16 ? 1 : 2; }
static_assert(tile_blocks<16>() == 1 && tile_blocks<8>() == 2, "tile_blocks and tile_blocks_of differ");

// P.V output units (32 features) per wave.  Q.K waves take a few units; the
// waves without Q.K rows take the rest, so that no wave idles while Q.K runs.
// Kernel variants (register budgets): kFull, any row; kLean, rows with K <= 320
// and d <= 256 in items of at most 2 row blocks (3 workgroups per CU);
// kGqa, grouped-query rows [V || K] with d = d_h <= 128 (4 workgroups per
// CU).  Lean and grouped-query rows have at most 8 and 4 output units.  (A
// lean 3-row-block item spills: it is left to the full variant.)
template <int RB, int V>
constexpr int qk_units_max() { return V == kGqa ? 1 : V == kLean ? 1 : 3; }
template <int RB, int V>
constexpr int pv_units_max() { return V == kGqa ? 2 : V == kLean ? 4 : RB == 3 ? 7 : 5; }
// 64-field chunks of a row that enter Q.K
template <int V>
constexpr int max_chunks() { return V == kGqa ? 4 : V == kLean ? 5 : (kMaxK + 63) / 64; }

__device__ inline f4 mfma_f16_k16(h4 a, h4 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0); }

// 4 int16 codes (w0, w1 little-endian) -> fp16, rounded to nearest even (11
// significant bits; relative error <= 2^-11, the same size as the fp16 P').
__device__ inline h4 cvt_i16x4(u2 w) {
  return h4{(_Float16)(short)(w[0] & 0xFFFFu), (_Float16)(short)(w[0] >> 16), (_Float16)(short)(w[1] & 0xFFFFu),
            (_Float16)(short)(w[1] >> 16)};
}

// One work item: a chunk of <= 16*RB query rows of one anchor group, one
// sequence, one token split.  Stage st (st = -1 .. ntiles-1) runs Q.K and the
// softmax of tile st+1 on the Q.K waves and P.V of tile st on every wave, with
// one barrier per stage (P.V first, so that after its rescale branch the two
// halves form one region the compiler can interleave); P', the rescale factors
// and the flags are double buffered by tile parity.
// GQA: grouped-query rows [V || K] (values first; Q.K skips the value
// chunks, the first half of the row) and sequence s reading seq_lens[s / n_kv].
template <int BITS, int RB, int V>
__device__ __forceinline__ void run_item(KArgs& A, KEntry& E, int s, int ksplit, int chunk, char* lds) {
  constexpr int TB = tile_blocks<BITS>();
  constexpr int kMaxC = max_chunks<V>();
  constexpr bool GQA = V == kGqa;
  constexpr int TILE = 16 * TB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, n = lane & 15;
  const int d = E.d, K = d + A.d_rope;
  // Q.K chunks: NRq RoPE chunks (three query limbs, fields from d), then NLq
  // latent chunks (two query limbs, fields from 0).  Grouped-query rows [V || K]
  // have one part only, the keys: two-limb chunks from field d.
  const int NRq = GQA ? 0 : (A.d_rope + 63) >> 6, NLq = GQA ? (A.d_rope + 63) >> 6 : (d + 63) >> 6, KC = NLq + NRq;
  const int NSEG = nseg_of(E.row_stride), PITCH = NSEG * 256;
  const int bufbytes = tilebuf_bytes(E.row_stride, d, A.d_rope, BITS);
  const int nbuf = E.nbuf;                    // >= 3 tile buffers
  constexpr int PSLOT = 8 * TB;               // P' bytes per lane and row block
  constexpr int PPAR = RB * 64 * PSLOT;       // P' bytes per tile parity
  char* pbuf = lds + nbuf * bufbytes;         // [2][RB][64 lanes] PSLOT bytes
  float* alpha_lds = (float*)(pbuf + 2 * PPAR);     // [2][64]
  int* flag_lds = (int*)(alpha_lds + 128);          // [2][4]
  float* ml_lds = (float*)(flag_lds + 8);           // [64][2]
  int* misc_lds = (int*)(ml_lds + 128);

  // rows of this chunk (at most 16 * RB); wave < RB owns rows 16*wave + n
  const int r0 = E.row_begin + chunk * E.chunk_rows;
  const int nrows = min(E.chunk_rows, E.row_end - r0);

  // token range of this split
  int len = A.seq_lens[GQA ? (E.seq_base + s) / A.seq_div : E.seq_base + s];
  len = len < 0 ? 0 : (len > A.t_cap ? A.t_cap : len);
  const int tps = ((len + E.splits - 1) / E.splits + kTile - 1) / kTile * kTile;
  const int t0 = ksplit * tps;
  const int t1 = min(len, t0 + tps);
  const int ntok = t1 > t0 ? t1 - t0 : 0;
  const int ntiles = (ntok + TILE - 1) / TILE;
  const int64_t row0 = (int64_t)s * A.t_cap + t0;    // first cache row of this item

  // ---- tile loader: direct HBM -> LDS copies ---------------------------------------
  // Every wave issues the same number of copy instructions for every tile
  // (rows past the valid tokens re-read the last valid row), so "tile t has
  // landed" is a fixed count of this wave's outstanding copies.
  const uint8_t* codes = E.codes;
  const float* scales = E.scales;
  const int block_pieces = NSEG * 16;
  const int npos = TB * block_pieces;            // 16-byte pieces of codes in a tile
  const int ninst = (npos + 63) >> 6;            // 64-lane copy instructions per tile
  // The copy loop runs on scalar registers: wave index, tile base address and
  // LDS addresses are wave-uniform; each lane only adds its 32-bit offset.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Copy i of a tile goes to wave i mod 4, except with two or three Q.K
  // waves, whose stages are the longest: the waves without Q.K rows take the
  // first n_pv copies of each tile (wave RB + j takes i = j, j + npv, ...) and
  // Q.K wave w the copies n_pv + w, n_pv + w + RB, ...  n_pv follows the
  // measured balance of the stage: with two Q.K waves, and for b <= 4 (the
  // narrow codes' short Q.K stages), every copy (the other waves still idle
  // otherwise); else half, which leaves each of the three Q.K waves one copy
  // in six.
  constexpr bool kPvCopies = RB >= 2;
  constexpr int kNpv = kWaves - RB;
  const int n_pv = !kPvCopies ? 0 : (BITS <= 4 || RB == 2) ? ninst : ninst / 2;
  int my_copies;
  if constexpr (kPvCopies) {
    const int n_qk = ninst - n_pv;
    my_copies = wave_u < RB ? (n_qk > wave_u ? (n_qk - wave_u + RB - 1) / RB : 0)
                            : (n_pv > wave_u - RB ? (n_pv - (wave_u - RB) + kNpv - 1) / kNpv : 0);
  } else {
    my_copies = ninst > wave_u ? (ninst - wave_u + kWaves - 1) / kWaves : 0;
  }
  // copy rounds of each role (straight-line code): at most 18 copies per tile,
  // at most 9 of them for b <= 4
  constexpr int kMaxCopies = 32 * kMaxK / 1024;
  constexpr int kQkRounds = kPvCopies ? (RB == 3 ? (kMaxCopies - kMaxCopies / 2 + RB - 1) / RB : 0) : kCopyRounds;
  constexpr int kPvRounds = kPvCopies ? ((RB == 3 ? kMaxCopies / 2 : kMaxCopies) + kNpv - 1) / kNpv : kCopyRounds;
  static_assert(kMaxCopies == 18 && 32 * 4 * kMaxK / 8 / 1024 <= 9, "copy rounds sized for K = 576");
  const int copies = __builtin_amdgcn_readfirstlane(my_copies + (wave_u == kWaves - 1 ? 1 : 0));
  const uint32_t lds0 = lds_addr(lds);
  const int rstride = E.row_stride;
  const uint8_t* item_codes = (const uint8_t*)uniform_ptr(codes + row0 * (int64_t)rstride);
  const float* item_scales = (const float*)uniform_ptr(scales + row0);
  auto issue_tile = [&](int it, int slotb, auto qk_tag) {
    constexpr bool QK_ROLE = decltype(qk_tag)::value;      // issued by a wave with Q.K rows
    const uint32_t buf = lds0 + slotb * bufbytes;
    const int tok0 = it * TILE;
    const int tlast = min(TILE, ntok - tok0) - 1;
    const void* tbase = item_codes + (int64_t)tok0 * rstride;
    // the per-copy lane offsets are recomputed at each issue (a few VALU ops)
    // rather than hoisted out of the stage loop, where they would hold
    // registers for the whole loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < (QK_ROLE ? kQkRounds : kPvRounds); ++k) {   // straight-line: one exit branch
      const int i = !kPvCopies ? wave_u + kWaves * k
                               : QK_ROLE ? n_pv + wave_u + RB * k : (wave_u - RB) + kNpv * k;   // increasing in k
      if (!kPvCopies || QK_ROLE ? i >= ninst : i >= n_pv) break;
      const int p = i * 64 + ln;
      const int tb = (TB == 2 && p >= block_pieces) ? 1 : 0;
      const int rem = p - tb * block_pieces;
      const int seg = rem >> 4, slot = rem & 15;
      // token held by this slot: block 1 of a two-block tile swaps segment
      // halves (slot ^ 8), as does the low-byte plane of b = 16
      const int swz = BITS == 16 ? (seg >= (NSEG >> 1) ? 8 : 0) : (tb << 3);
      const int t = min(16 * tb + (slot ^ swz), tlast);
      if (p < npos)                              // lane 0 always copies: the instruction is issued
        copy16_to_lds(__umul24(t, rstride) + seg * 16, tbase, buf + i * 1024);   // t < 32, stride <= 1152
    }
    if (wave_u == kWaves - 1 && lane < TILE)
      copy4_to_lds((uint32_t)(min(lane, tlast) * 4), item_scales + tok0, buf + TB * PITCH);
  };
  // prologue: tiles 0 .. nbuf-3; stage st issues tile st + nbuf - 1
  // (the prologue copies, tiles 0 .. nbuf-3, are issued by each role at the
  // start of its pipeline below)

  // ---- P.V output units of this wave ---------------------------------------------
  const int NU = (d + 31) >> 5;
  int ubase, ucount;
  static_assert(RB < kWaves, "at least one wave without Q.K rows");
  {
    const int npv = kWaves - RB;
    // Q.K waves carry the longer stage, so they take output units only when
    // the other waves cannot hold them all (the full variant keeps at least
    // 3/16 of them on the Q.K waves: its P.V wave's registers are the limit)
    int uq = (NU - npv * pv_units_max<RB, V>() + RB - 1) / RB;
    if constexpr (V != kLean) uq = max((NU * 3) / 16, uq);
    uq = min(max(uq, 0), qk_units_max<RB, V>());
    const int rest = NU - RB * uq;
    const int per = (rest + npv - 1) / npv;
    if (wave < RB) {
      ubase = wave * uq;
      ucount = uq;
    } else {
      ubase = RB * uq + (wave - RB) * per;
      ucount = max(0, min(per, rest - (wave - RB) * per));
    }
  }

  float m_run = -INFINITY, l_lane = 0.0f;     // softmax state of row 16*wave + n (Q.K waves)
  // E before an item's first tile: any scale above 2^-94 raises it there; a
  // first tile of all-zero tokens (scale 0) keeps it, and its exponentials,
  // at most 2^100 each, stay finite in P' (= 0) and in l (< 2^114 over 8192
  // tokens); a later raise rescales both like any other.
  int Ecur = -100;                             // scales so far are <= 2^(Ecur + headroom)

  // The stage loop of one wave role.  QKW: this wave owns Q.K rows; UMAX: its
  // largest unit count (each role is register-allocated for its own arrays).
  auto pipeline = [&](auto qkw_tag, auto umax_tag) {
    constexpr bool QKW = decltype(qkw_tag)::value;
    constexpr int UMAX = decltype(umax_tag)::value;
    // prologue: tiles 0 .. nbuf-3; stage st issues tile st + nbuf - 1
    for (int it = 0; it < nbuf - 2 && it < ntiles; ++it) issue_tile(it, it, qkw_tag);
    const int my_row = 16 * wave + n;
    const int rope_field0 = d + 16 * g;           // first RoPE field of this lane's Q.K features
    const int lat_field0 = (GQA ? d : 0) + 16 * g;  // first field of its two-limb chunks

    // ---- q as int8 limbs of a fixed-point number per row and part -------------------
    // Q.K chunk c < NRq covers RoPE features 64c + 16g + qk_slot_feature(i) (q = 0
    // past d_R), read from the row at field d + 64c + ...; chunk NRq + c' covers
    // latent features 64c' + 16g + ... (q = 0 at and past d).  The two parts of a
    // row each get their own prescale: the latent part is a 15-bit number (two
    // limbs), the RoPE part a 22-bit one (three limbs: hi, mid, lo), so that a
    // RoPE query far larger than the latent one (or the reverse) keeps its
    // logits accurate.  The integer scores of the parts are joined in fp32
    // (S = S_lat + ratio * S_rope, in units of the latent prescale).
    i4 qh[QKW ? kMaxC : 1], ql[QKW ? kMaxC : 1], qm[QKW ? kMaxRopeChunks : 1];
    float rowf = 1.0f, ratio = 0.0f;
    int qbiasL = 0, qbiasR = 0;
    if constexpr (QKW) {
      int my_layer = -1, my_head = 0;
      if (my_row < nrows) {
        const int gr = r0 + my_row;
        my_layer = group_layer_at(A, E.lay_begin + gr / A.heads);
        my_head = gr % A.heads;
      }
      // The loads of every chunk are issued before any of them is used, so the
      // query costs one memory round trip: a chunk outside the row or past the
      // part's width reads the (valid) first query element and is zeroed afterwards.
      const bool row_ok = my_layer >= 0;
      const int64_t qrow =
          row_ok ? ((int64_t)(my_layer - E.layer_base) * A.batch + E.seq_base + s) * A.heads + my_head : 0;
      bool ok[kMaxC], lat[kMaxC];
      int64_t off[kMaxC];
#pragma unroll
      for (int c = 0; c < kMaxC; ++c) {
        lat[c] = c >= NRq;
        const int f0 = lat[c] ? 64 * (c - NRq) + 16 * g : 64 * c + 16 * g;
        ok[c] = row_ok && c < KC && f0 < (lat[c] && !GQA ? d : A.d_rope);
        off[c] = !ok[c] ? 0 : lat[c] && !GQA ? qrow * A.r + f0 : qrow * A.d_rope + f0;
      }
      // Two passes over the query: the part maxima, then the limbs.  bf16 queries
      // are loaded once and kept packed (8 dwords per chunk); fp32 queries are
      // loaded again for the second pass (a second round trip, which keeps 16
      // floats per chunk out of the registers).  Each dtype has its own
      // straight-line copy of the code.
      const float sm = my_layer >= 0 ? layer_at(A, my_layer).sm_scale : 0.0f;
      float preL = 0.0f, preR = 0.0f, mxL = 0.0f, mxR = 0.0f;
      int qsumL = 0, qsumR = 0;                   // sums of the fixed-point q per part
      // NRQ >= 0: the RoPE chunk count known at compile time (bf16 queries), so
      // that each chunk's limb code is its own; NRQ < 0: NRq at run time
      auto quantize = [&](auto f32_tag, auto nrq_tag) {
        constexpr bool F32 = decltype(f32_tag)::value;
        constexpr int NRQ = decltype(nrq_tag)::value;
        auto is_lat = [&](int c) { return NRQ >= 0 ? c >= NRQ : lat[c]; };
        u4 raw[F32 ? 1 : kMaxC][2];
        auto get = [&](int c, float (&x)[16]) {
          if constexpr (F32) {
            const f4* p = (const f4*)((const float*)(is_lat(c) && !GQA ? A.q_lat : A.q_rope) + off[c]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const f4 t = p[v];
#pragma unroll
              for (int i = 0; i < 4; ++i) x[4 * v + i] = ok[c] ? t[i] : 0.0f;
            }
          } else {
#pragma unroll
            for (int v = 0; v < 2; ++v)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                x[8 * v + 2 * i] = ok[c] ? __uint_as_float(raw[c][v][i] << 16) : 0.0f;
                x[8 * v + 2 * i + 1] = ok[c] ? __uint_as_float(raw[c][v][i] & 0xFFFF0000u) : 0.0f;
              }
          }
        };
        if constexpr (!F32) {
#pragma unroll
          for (int c = 0; c < kMaxC; ++c) {
            const u4* p = (const u4*)((const uint16_t*)(is_lat(c) && !GQA ? A.q_lat : A.q_rope) + off[c]);
#pragma unroll
            for (int v = 0; v < 2; ++v) raw[c][v] = p[v];
          }
        }
        if constexpr (!F32) {
          // bf16: |x| orders as its bit pattern without the sign, so the maxima
          // are taken two elements at a time on the packed words
          us2 m2L = us2{0, 0}, m2R = us2{0, 0};
#pragma unroll
          for (int c = 0; c < kMaxC; ++c) {
            const uint32_t msk = ok[c] ? 0x7FFF7FFFu : 0u;
#pragma unroll
            for (int v = 0; v < 2; ++v)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const us2 t = __builtin_bit_cast(us2, raw[c][v][i] & msk);
                if (is_lat(c)) m2L = __builtin_elementwise_max(m2L, t);
                else m2R = __builtin_elementwise_max(m2R, t);
              }
          }
          mxL = __uint_as_float((uint32_t)(m2L[0] > m2L[1] ? m2L[0] : m2L[1]) << 16);
          mxR = __uint_as_float((uint32_t)(m2R[0] > m2R[1] ? m2R[0] : m2R[1]) << 16);
        } else {
#pragma unroll
          for (int c = 0; c < kMaxC; ++c) {
            float x[16];
            get(c, x);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              if (is_lat(c)) mxL = fmaxf(mxL, fabsf(x[i]));
              else mxR = fmaxf(mxR, fabsf(x[i]));
            }
          }
        }
        mxL = max_xor_16_32(mxL);
        mxR = max_xor_16_32(mxR);
        // A negative softmax scale is carried by q (z = |scale| * (-q) . k), so the
        // row factor below is positive, as the softmax needs.
        const float sgn = sm < 0.0f ? -1.0f : 1.0f;
        preL = mxL > 0.0f ? sgn * (kQMax / mxL) : 0.0f;
        preR = mxR > 0.0f ? sgn * (kQMaxRope / mxR) : 0.0f;
#pragma unroll
        for (int c = 0; c < kMaxC; ++c) {
          float x[16];
          get(c, x);
          uint32_t hw[4] = {0, 0, 0, 0}, mw[4] = {0, 0, 0, 0}, lw[4] = {0, 0, 0, 0};
          const float pre = is_lat(c) ? preL : preR;
          if (BITS != 16 && is_lat(c)) {
            // Latent part, codes of b <= 8: base-256 limbs, qi = 256 hi + lo with
            // lo in [-128, 127] and hi = floor((qi + 128) / 256) in [-63, 64].
            // One fma rounds x * pre to the nearest integer (ties to even) in
            // the low bits of a float near 1.5 * 2^23: its bits are
            // 0x4B400000 + qi + 128, so byte 0 is lo + 128 and byte 1 is hi
            // (two's complement), and v_perm gathers them four at a time.
            uint32_t zb[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) zb[i] = __float_as_uint(fmaf(x[qk_slot_feature<BITS>(i)], pre, 12583040.0f));
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t a = perm(zb[4 * w + 1], zb[4 * w], 0x05010400u);       // lo0 lo1 hi0 hi1
              const uint32_t b = perm(zb[4 * w + 3], zb[4 * w + 2], 0x05010400u);   // lo2 lo3 hi2 hi3
              lw[w] = perm(b, a, 0x05040100u) ^ 0x80808080u;
              hw[w] = perm(b, a, 0x07060302u);
            }
          } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // latent (b = 16): qi = 128 hi + lo, |qi| <= 16256; RoPE: qi = 16384 hi + 128 mid + lo,
            // |qi| <= 16256 * 128 (floor divisions: hi in [-127, 127], mid in [-64, 64],
            // lo in [-64, 63])
            const int qi = (int)rintf(x[qk_slot_feature<BITS>(i)] * pre);
            const int hi = is_lat(c) ? (qi + 64) >> 7 : (qi + 8192) >> 14;
            const int rest = is_lat(c) ? 0 : qi - (hi << 14);
            const int mid = (rest + 64) >> 7;
            const int lo = is_lat(c) ? qi - (hi << 7) : rest - (mid << 7);
            if (is_lat(c)) qsumL += qi; else qsumR += qi;
            hw[i >> 2] |= ((uint32_t)hi & 0xFFu) << (8 * (i & 3));
            mw[i >> 2] |= ((uint32_t)mid & 0xFFu) << (8 * (i & 3));
            lw[i >> 2] |= ((uint32_t)lo & 0xFFu) << (8 * (i & 3));
          }
          }
          qh[c] = i4{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3]};
          ql[c] = i4{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3]};
          if (c < kMaxRopeChunks) qm[c < kMaxRopeChunks ? c : 0] = i4{(int)mw[0], (int)mw[1], (int)mw[2], (int)mw[3]};
        }
      };
      if (A.q_is_f32) quantize(std::true_type{}, std::integral_constant<int, -1>{});
      else if constexpr (GQA) quantize(std::false_type{}, std::integral_constant<int, 0>{});
      else if (NRq == 1) quantize(std::false_type{}, std::integral_constant<int, 1>{});
      else quantize(std::false_type{}, std::integral_constant<int, 2>{});
      // scores are taken in units of the latent prescale (the RoPE one when the
      // latent part is zero); rowf >= FLT_MIN: a zero scale (or a padding row,
      // q = 0) still maps the masked tokens' t = -inf to z = -inf.
      const float pref = fabsf(mxL > 0.0f ? preL : preR);
      ratio = mxR > 0.0f ? fabsf(pref / preR) : 0.0f;
      rowf = fmaxf(pref > 0.0f ? fabsf(sm) * kLog2e * qk_code_scale<BITS>() / pref : 0.0f, FLT_MIN);
      // b = 16: offset-binary bias of the low-byte operand (exact integer correction)
      if constexpr (BITS == 16) {
        qbiasL = isum_xor_16_32(qsumL);
        qbiasR = isum_xor_16_32(qsumR);
      }
    }

    f4 oacc[UMAX][2][RB];
#pragma unroll
    for (int u = 0; u < UMAX; ++u)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) oacc[u][f][rb] = f4{0.f, 0.f, 0.f, 0.f};

    int slot_qk = 0, slot_pv = nbuf - 1, slot_issue = nbuf - 2;   // buffers of tiles st+1, st, st+nbuf-1
    // The stage loop is instantiated for the common row shapes with the unit
    // count UC and the chunk counts NC (NR of them RoPE) as compile-time
    // constants, so that a stage is one block of straight-line code the
    // scheduler can interleave; UC < 0 is the generic loop (runtime counts).
    auto stage_loop = [&](auto nc_tag, auto nr_tag, auto uc_tag) {
      constexpr int NC_CT = decltype(nc_tag)::value, NR_CT = decltype(nr_tag)::value;
      constexpr int UC_CT = decltype(uc_tag)::value;
    for (int st = -1; st < ntiles; ++st) {
      if (st + 1 < ntiles) vm_wait(min(nbuf - 3, ntiles - 2 - st) * copies);  // tile st+1 has landed
      lds_barrier();                  // tile st+1 visible; P'(st) written; P.V(st-1) done everywhere
      if (st + nbuf - 1 < ntiles) issue_tile(st + nbuf - 1, slot_issue, qkw_tag);
      slot_issue = slot_issue + 1 == nbuf ? 0 : slot_issue + 1;

      // ---- P.V of tile st (every wave, its own output units) ----
      if (st >= 0) {
        const char* buf = lds + slot_pv * bufbytes;
        const int par = st & 1;
        const char* psrc = pbuf + par * PPAR;
        // Rescale flags of this tile's rows: read here, tested only after the
        // P.V operand reads are issued, so that the two LDS round trips overlap.
        // One uniform test for the rare rescale (a branch per row block costs more).
        int fl[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) fl[rb] = flag_lds[4 * par + rb];
        auto rescale = [&](auto uw) {
          constexpr int UW = decltype(uw)::value;
          int fany = 0;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) fany |= fl[rb];
          if (__builtin_amdgcn_readfirstlane(fany))
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              if (fl[rb]) {
                const float al = alpha_lds[64 * par + 16 * rb + n];
#pragma unroll
                for (int u = 0; u < UW; ++u)
#pragma unroll
                  for (int f = 0; f < 2; ++f) oacc[u][f][rb] *= al;
              }
            }
        };
        auto pv_units = [&](auto uw) {
          constexpr int UW = decltype(uw)::value;
          if constexpr (TB == 2) {
            h8 pfr[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) pfr[rb] = *(const h8*)(psrc + (rb * 64 + lane) * PSLOT);
            u2 rv[UW][BITS == 16 ? 4 : BITS == 8 ? 2 : 1];
#pragma unroll
            for (int ui = 0; ui < UW; ++ui) {
              const int u = ubase + ui;
              if constexpr (BITS == 8) {
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                  const int e = n >> 1, h = n & 1, tb = e >> 2;
                  const char* p = buf + tile_off(PITCH, tb, 2 * u + f, 4 * g + (e & 3)) + 8 * h;
                  rv[ui][f] = __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i2, p)));
                }
              }
              if constexpr (BITS == 4 || BITS == 2) {
                const int e = n & 7, half = n >> 3;
                const int tb = (e >> 1) & 1, t = 4 * g + 2 * (e & 1) + (e >> 2);
                const char* p = BITS == 4 ? buf + tile_off(PITCH, tb, u, t) + 8 * half
                                          : buf + tile_off(PITCH, tb, u >> 1, t) + 8 * (u & 1);
                rv[ui][0] = __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr4_b64_v2i32(LDS_PTR(i2, p)));
              }
            }
            rescale(uw);
#pragma unroll
            for (int ui = 0; ui < UW; ++ui) {
              h8 a[2];
              if constexpr (BITS == 8) {
                a[0] = cvt_b8(rv[ui][0][0], rv[ui][0][1]);
                a[1] = cvt_b8(rv[ui][1][0], rv[ui][1][1]);
              }
              if constexpr (BITS == 4) { a[0] = cvt_b4(rv[ui][0][0]); a[1] = cvt_b4(rv[ui][0][1]); }
              if constexpr (BITS == 2) { a[0] = cvt_b2_nib<0>(rv[ui][0][0]); a[1] = cvt_b2_nib<1>(rv[ui][0][0]); }
#pragma unroll
              for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) oacc[ui][f][rb] = mfma_f16(a[f], pfr[rb], oacc[ui][f][rb]);
            }
          } else {
            // b = 16, 16-token tiles: k = 16 MFMAs on the codes rounded to fp16
            h4 pfr[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) pfr[rb] = *(const h4*)(psrc + (rb * 64 + lane) * PSLOT);
            u2 rv[UW][2];
#pragma unroll
            for (int ui = 0; ui < UW; ++ui) {
              const int u = ubase + ui;
#pragma unroll
              for (int f = 0; f < 2; ++f) {
                // transposed byte read of 8 rows: high-plane rows of tokens
                // 4g..4g+3, then the low-plane rows of the same tokens; lane n
                // gets feature 16*fb + n: high bytes in rv[0], low bytes in rv[1]
                const int fb = 2 * u + f, k = n >> 1, h = n & 1;
                const int seg = k < 4 ? fb : (NSEG >> 1) + fb, slot = k < 4 ? 4 * g + k : (4 * g + k - 4) ^ 8;
                rv[ui][f] = __builtin_bit_cast(
                    u2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i2, buf + tile_off(PITCH, 0, seg, slot) + 8 * h)));
              }
            }
            rescale(uw);
#pragma unroll
            for (int ui = 0; ui < UW; ++ui) {
#pragma unroll
              for (int f = 0; f < 2; ++f) {
                // int16 codes of tokens (t0, t1), (t2, t3): low byte (bit 7 restored), high byte
                const uint32_t w0 = perm(rv[ui][f][1], rv[ui][f][0], 0x01050004u) ^ 0x00800080u;
                const uint32_t w1 = perm(rv[ui][f][1], rv[ui][f][0], 0x03070206u) ^ 0x00800080u;
                const h4 a = cvt_i16x4(u2{w0, w1});
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) oacc[ui][f][rb] = mfma_f16_k16(a, pfr[rb], oacc[ui][f][rb]);
              }
            }
          }
        };
        if constexpr (UC_CT == 0) {
        } else if constexpr (UC_CT > 0) pv_units(std::integral_constant<int, UC_CT>{});
        else switch (ucount) {
          case 0: break;
          case 1: pv_units(std::integral_constant<int, 1>{}); break;
          case 2: if constexpr (UMAX >= 2) pv_units(std::integral_constant<int, 2>{}); break;
          case 3: if constexpr (UMAX >= 3) pv_units(std::integral_constant<int, 3>{}); break;
          case 4: if constexpr (UMAX >= 4) pv_units(std::integral_constant<int, 4>{}); break;
          case 5: if constexpr (UMAX >= 5) pv_units(std::integral_constant<int, 5>{}); break;
          case 6: if constexpr (UMAX >= 6) pv_units(std::integral_constant<int, 6>{}); break;
          default: if constexpr (UMAX >= 7) pv_units(std::integral_constant<int, 7>{}); break;
        }
      }
      // ---- Q.K and softmax of tile st+1 (Q.K waves) ----
      if constexpr (QKW) {
        if (st + 1 < ntiles) {
          const int tq = st + 1;
          const char* buf = lds + slot_qk * bufbytes;
          const float* sc = (const float*)(buf + TB * PITCH);
          const int tvalid = min(TILE, ntok - tq * TILE);
          // Latent chunks: code x q_hi, code x q_lo; b = 16: high byte x (q_hi, q_lo) and
          // low byte x q_hi (the low byte x q_lo product is left out: its weight is
          // 2^-15 of the leading term, the size of the 15-bit rounding of q).
          // RoPE chunks: code x (q_hi, q_mid, q_lo); b = 16: high byte x (q_hi, q_mid,
          // q_lo) and low byte x (q_hi, q_mid) (left out: 2^-22 of the leading term).
          constexpr int NACC_L = BITS == 16 ? 3 : 2, NACC_R = BITS == 16 ? 5 : 3;
          float sqv[TB][4];                         // scores in units of the latent prescale
          f4 scv[TB];                               // this lane's 4 token scales per token block
          // NC chunks, of which the first NR are RoPE chunks: compile-time counts in
          // each case below, so every LDS read of the tile is straight-line code
          // the scheduler can hoist ahead of the MFMAs that consume it.
          auto qk_chunks = [&](auto nc_tag, auto nr_tag) {
            constexpr int NC = decltype(nc_tag)::value, NR = decltype(nr_tag)::value, NL = NC - NR;
            // the scales are read with the codes, not after the MFMAs
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) scv[tb] = *(const f4*)(sc + 16 * tb + 4 * g);
            // RoPE chunks first: their integer score is turned into fp32 before
            // the latent chunks run, so the two parts never hold accumulators
            // at the same time
            auto run_chunks = [&](auto c_begin, auto c_end, auto rope_tag, auto& acc) {
              constexpr int CB = decltype(c_begin)::value, CE = decltype(c_end)::value;
              constexpr bool ROPE = decltype(rope_tag)::value;
#pragma unroll
              for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int k = 0; k < (ROPE ? NACC_R : NACC_L); ++k) acc[tb][k] = i4{0, 0, 0, 0};
#pragma unroll
              for (int c = CB; c < CE; ++c) {
                // first field of this lane's 16 features in the row
                const int field = ROPE ? rope_field0 + 64 * c : lat_field0 + 64 * (c - NR);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                  if constexpr (BITS == 16) {
                    // byte planes: signed high bytes and offset-binary low bytes of
                    // these 16 features are each one 16-byte row (low plane: slot n ^ 8)
                    const i4 hi = *(const i4*)(buf + tile_off(PITCH, 0, field >> 4, n));
                    const i4 lo = *(const i4*)(buf + tile_off(PITCH, 0, (K >> 4) + (field >> 4), n ^ 8));
                    acc[tb][0] = mfma_i8(hi, qh[c], acc[tb][0]);
                    acc[tb][1] = mfma_i8(hi, ql[c], acc[tb][1]);
                    acc[tb][2] = mfma_i8(lo, qh[c], acc[tb][2]);
                    if constexpr (ROPE) {
                      acc[tb][3] = mfma_i8(hi, qm[c < kMaxRopeChunks ? c : 0], acc[tb][3]);
                      acc[tb][4] = mfma_i8(lo, qm[c < kMaxRopeChunks ? c : 0], acc[tb][4]);
                    }
                  } else {
                    const int fbyte = field * BITS / 8;   // first byte of this lane's 16 features
                    const char* p = buf + tile_off(PITCH, tb, fbyte >> 4, n) + (fbyte & 15);
                    i4 a;
                    if constexpr (BITS == 8) a = *(const i4*)p;
                    else if constexpr (BITS == 4) { const u2 x = *(const u2*)p; a = qk_b4(x[0], x[1]); }
                    else a = qk_b2(*(const uint32_t*)p);
                    acc[tb][0] = mfma_i8(a, qh[c], acc[tb][0]);
                    acc[tb][1] = mfma_i8(a, ql[c], acc[tb][1]);
                    if constexpr (ROPE) acc[tb][2] = mfma_i8(a, qm[c < kMaxRopeChunks ? c : 0], acc[tb][2]);
                  }
                }
              }
            };
            // the parts are exact integers (b = 16: up to the left-out products),
            // joined in fp32: S = S_lat + ratio * S_rope
            float sr[TB][4];
            if constexpr (NR == 0) {
#pragma unroll
              for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int j = 0; j < 4; ++j) sr[tb][j] = 0.0f;
            } else {
              i4 acc[TB][NACC_R];
              run_chunks(std::integral_constant<int, 0>{}, std::integral_constant<int, NR>{}, std::true_type{}, acc);
#pragma unroll
              for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  float v;
                  if constexpr (BITS == 16)   // 2^22 hh + 2^15 hm + 2^8 hl + 2^14 lh + 2^7 (lm + sum q)
                    v = fmaf(4194304.0f, (float)acc[tb][0][j],
                             fmaf(256.0f, (float)(128 * acc[tb][3][j] + acc[tb][1][j]),
                                  fmaf(16384.0f, (float)acc[tb][2][j], 128.0f * (float)(acc[tb][4][j] + qbiasR))));
                  else                        // 2^14 hi + 2^7 mid + lo
                    v = fmaf(16384.0f, (float)acc[tb][0][j], (float)(128 * acc[tb][2][j] + acc[tb][1][j]));
                  sr[tb][j] = v * ratio;
                }
            }
            if constexpr (NL > 0) {
              // keep the two phases apart: interleaved, their accumulators would
              // be live at the same time
              if constexpr (NR > 0) __builtin_amdgcn_sched_barrier(0);
              i4 acc[TB][NACC_L];
              run_chunks(std::integral_constant<int, NR>{}, std::integral_constant<int, NC>{}, std::false_type{}, acc);
#pragma unroll
              for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  float v;
                  if constexpr (BITS == 16)   // 2^8 (2^7 hi + lo) + 2^7 (lh + sum q)
                    v = fmaf(256.0f, (float)(128 * acc[tb][0][j] + acc[tb][1][j]), 128.0f * (float)(acc[tb][2][j] + qbiasL));
                  else                        // base-256 limbs: |256 hi + lo| < 2^31 up to d = 512
                    v = (float)(256 * acc[tb][0][j] + acc[tb][1][j]);
                  sqv[tb][j] = v + sr[tb][j];
                }
            } else {
#pragma unroll
              for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int j = 0; j < 4; ++j) sqv[tb][j] = sr[tb][j];
            }
          };
          if constexpr (GQA) {
            if (KC == 1) qk_chunks(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});   // d_h = 64
            else qk_chunks(std::integral_constant<int, 2>{}, std::integral_constant<int, 0>{});           // d_h = 128
          } else {
#define KK_QK_CASE(k)                                                                           \
  case k:                                                                                       \
    if constexpr (kMaxC >= k) {                                                                 \
      if (NRq == 1 || k < 3) qk_chunks(std::integral_constant<int, k>{}, std::integral_constant<int, 1>{}); \
      else qk_chunks(std::integral_constant<int, k>{}, std::integral_constant<int, (k >= 3 ? 2 : 1)>{});    \
    }                                                                                           \
    break;
            if constexpr (NC_CT > 0) {
              qk_chunks(std::integral_constant<int, NC_CT>{}, std::integral_constant<int, NR_CT>{});
            } else {
              switch (KC) {
                KK_QK_CASE(2) KK_QK_CASE(3) KK_QK_CASE(4) KK_QK_CASE(5) KK_QK_CASE(6) KK_QK_CASE(7) KK_QK_CASE(8)
                default: KK_QK_CASE(9)
              }
            }
#undef KK_QK_CASE
          }

          // ---- online softmax for these rows ----
          // t = integer score x token scale; the log2-domain logit is z = t * rowf
          // with rowf > 0, so the row maximum of z is rowf times that of t.
          float t[TB][4];
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int j = 0; j < 4; ++j) t[tb][j] = sqv[tb][j] * scv[tb][j];
          if (tvalid < TILE) {        // an item's last tile: tokens past the end get z = -inf
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (16 * tb + 4 * g + j >= tvalid) t[tb][j] = -INFINITY;
          }
          // (scales past the end repeat the last valid token's, so smax is unchanged)
          float smax = 0.0f, tmax = -INFINITY;
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              smax = fmaxf(smax, scv[tb][j]);
              tmax = fmaxf(tmax, t[tb][j]);
            }
          // The running max and E usually stay: the exponentials are taken
          // with them right away, and only a lane-local test decides whether any
          // row must move them (the row reductions run in that rare stage only,
          // which also redoes the exponentials).
          float e[TB][4];
          {
            const float mE0 = m_run + (float)Ecur;    // P~ = 2^(z - m - E), P' = P~ * scale_t
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
              for (int j = 0; j < 4; ++j) e[tb][j] = __builtin_amdgcn_exp2f(fmaf(t[tb][j], rowf, -mE0));
          }
          const float e_limit = ldexpf(1.0f, Ecur + kScaleHeadroom);
          const bool upd = __any(smax > e_limit || tmax * rowf > m_run + kLazyRescale);   // wave-uniform
          const int par = tq & 1;
          if (upd) {
            // every row of a wave sees the same tokens, so smax is wave-uniform
            smax = max_xor_16_32(smax);
            tmax = max_xor_16_32(tmax) * rowf;
            const bool raise_e = smax > e_limit;
            const float mnew = max_plain(m_run, tmax);
            int es = Ecur;
            (void)frexpf(smax, &es);
            const int enew = raise_e ? es : Ecur;
            // l is kept in units of 2^-E like O, so one factor rescales both
            // (one v_exp: m_run - mnew <= 0, Ecur - enew <= 0; results below 2^-126 are 0)
            const float alpha = __builtin_amdgcn_exp2f((m_run - mnew) + (float)(Ecur - enew));
            l_lane *= alpha;
            m_run = mnew;
            Ecur = enew;
            if (g == 0) alpha_lds[64 * par + my_row] = alpha;
            const float mE = m_run + (float)Ecur;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
              for (int j = 0; j < 4; ++j) e[tb][j] = __builtin_amdgcn_exp2f(fmaf(t[tb][j], rowf, -mE));
          }
          if (lane == 0) flag_lds[4 * par + wave] = upd ? 1 : 0;
          char* pdst = pbuf + par * PPAR + (wave * 64 + lane) * PSLOT;
          if constexpr (TB == 2) {
            h8 pf;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                l_lane += e[tb][j];
                pf[4 * tb + j] = (_Float16)(e[tb][j] * scv[tb][j]);
              }
            *(h8*)pdst = pf;
          } else {
            h4 pf;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              l_lane += e[0][j];
              pf[j] = (_Float16)(e[0][j] * scv[0][j]);
            }
            *(h4*)pdst = pf;
          }
        }
      }

      slot_qk = slot_qk + 1 == nbuf ? 0 : slot_qk + 1;
      slot_pv = slot_pv + 1 == nbuf ? 0 : slot_pv + 1;
    }
    };
    using I0 = std::integral_constant<int, 0>;
    using IG = std::integral_constant<int, -1>;
    bool done = false;
    if constexpr (QKW) {
      // the Q.K waves of 40-head rows with d = 128, 256, 384, 512 and d_R <= 64
      // (chunks 3, 5, 7, 9; output units 0, 1, 2, 3)
      if constexpr (RB == 3 && V == kFull) {
        if (NRq == 1 && KC == 3 && ucount == 0) { stage_loop(std::integral_constant<int, 3>{}, std::integral_constant<int, 1>{}, I0{}); done = true; }
        else if (NRq == 1 && KC == 5 && ucount == 1) { stage_loop(std::integral_constant<int, 5>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}); done = true; }
        else if (NRq == 1 && KC == 7 && ucount == 2) { stage_loop(std::integral_constant<int, 7>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{}); done = true; }
        else if (NRq == 1 && KC == 9 && ucount == 3) { stage_loop(std::integral_constant<int, 9>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, 3>{}); done = true; }
      }
      if (!done && NRq == 1 && KC == kMaxC && ucount == UMAX) {
        stage_loop(std::integral_constant<int, kMaxC>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, UMAX>{});
        done = true;
      }
      if constexpr (V == kLean) {
        // lean Q.K waves without output units (their P.V waves hold them all)
        if (!done && NRq == 1 && KC == kMaxC && ucount == 0) {
          stage_loop(std::integral_constant<int, kMaxC>{}, std::integral_constant<int, 1>{}, I0{});
          done = true;
        }
      }
    } else {
      // waves without Q.K rows: one loop per unit count
      switch (ucount) {
        case 0: stage_loop(I0{}, I0{}, I0{}); done = true; break;
        case 1: stage_loop(I0{}, I0{}, std::integral_constant<int, 1>{}); done = true; break;
        case 2: if constexpr (UMAX >= 2) { stage_loop(I0{}, I0{}, std::integral_constant<int, 2>{}); done = true; } break;
        case 3: if constexpr (UMAX >= 3) { stage_loop(I0{}, I0{}, std::integral_constant<int, 3>{}); done = true; } break;
        case 4: if constexpr (UMAX >= 4) { stage_loop(I0{}, I0{}, std::integral_constant<int, 4>{}); done = true; } break;
        case 5: if constexpr (UMAX >= 5) { stage_loop(I0{}, I0{}, std::integral_constant<int, 5>{}); done = true; } break;
        case 6: if constexpr (UMAX >= 6) { stage_loop(I0{}, I0{}, std::integral_constant<int, 6>{}); done = true; } break;
        case 7: if constexpr (UMAX >= 7) { stage_loop(I0{}, I0{}, std::integral_constant<int, 7>{}); done = true; } break;
        default: break;
      }
    }
    if (!done) stage_loop(I0{}, I0{}, IG{});

    // ---- finish: row sums, then normalized output or split partial -----------------
    if constexpr (QKW) {
      const float lrow = sum_xor_16_32(l_lane);
      if (g == 0) { ml_lds[2 * my_row] = m_run; ml_lds[2 * my_row + 1] = lrow; }
      if (wave == 0 && lane == 0) misc_lds[0] = Ecur;
    }
    lds_barrier();
    // O and l are in units of 2^-E: the normalized output is O / l.  A split
    // writes O / l as fp16 in units of 2^(E+6) (|O / l| <= qmax * 2^(E+6), so
    // it stays below 2^15), l in true units (l * 2^E) and m, for the merge.
    const int Eitem = misc_lds[0];
    const bool split = E.splits > 1;
    _Float16* part = nullptr;
    if (split) {
      const int64_t slotp = ((int64_t)(s * E.splits + ksplit) * E.nrc + chunk);
      float* slot = A.ws + E.ws_off + slotp * partial_slot_floats(d);
      part = (_Float16*)slot;
      float* ml = slot + partial_ml_offset(d);
      if (tid < 16 * RB) {
        ml[tid] = ml_lds[2 * tid];
        ml[64 + tid] = ntiles > 0 ? ldexpf(ml_lds[2 * tid + 1], Eitem) : 0.0f;
      }
      if (tid == 0) ml[128] = ntiles > 0 ? ldexpf(1.0f, Eitem + 6) : 0.0f;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rl = 16 * rb + n;
      if (rl < nrows) {
        const int gr = r0 + rl;
        const int layer = group_layer_at(A, E.lay_begin + gr / A.heads), head = gr % A.heads;
        const float lrow = ml_lds[2 * rl + 1];
        const float inv = lrow > 0.0f ? 1.0f / lrow : 0.0f;
        const float fac = split ? (lrow > 0.0f ? ldexpf(inv, -(Eitem + 6)) : 0.0f) : inv;
        float* dst = split ? nullptr : A.out + layer_at(A, layer).out_off + ((int64_t)s * A.heads + head) * d;
        _Float16* dsth = split ? part + (int64_t)rl * d : nullptr;
#pragma unroll
        for (int ui = 0; ui < UMAX; ++ui) {
          const int u = ubase + ui;
          if (ui < ucount) {
            if constexpr (BITS == 2) {
              const int fbase = 32 * u + 8 * g;
              if (fbase < d) {
                const f4 e0 = oacc[ui][0][rb] * fac, e1 = oacc[ui][1][rb] * fac;
                if (split) {
                  *(h8*)(dsth + fbase) = h8{(_Float16)e0[0], (_Float16)e1[0], (_Float16)e0[1], (_Float16)e1[1],
                                            (_Float16)e0[2], (_Float16)e1[2], (_Float16)e0[3], (_Float16)e1[3]};
                } else {
                  *(f4*)(dst + fbase) = f4{e0[0], e1[0], e0[1], e1[1]};
                  *(f4*)(dst + fbase + 4) = f4{e0[2], e1[2], e0[3], e1[3]};
                }
              }
            } else {
#pragma unroll
              for (int f = 0; f < 2; ++f) {
                const int fbase = 32 * u + 16 * f + 4 * g;
                if (fbase < d) {
                  const f4 e = oacc[ui][f][rb] * fac;
                  if (split) *(h4*)(dsth + fbase) = h4{(_Float16)e[0], (_Float16)e[1], (_Float16)e[2], (_Float16)e[3]};
                  else *(f4*)(dst + fbase) = e;
                }
              }
            }
          }
        }
      }
    }
  };

  if (wave < RB)
    pipeline(std::true_type{}, std::integral_constant<int, qk_units_max<RB, V>()>{});
  else
    pipeline(std::false_type{}, std::integral_constant<int, pv_units_max<RB, V>()>{});
}

// Last entry whose first decode block (merge: first merge block) is <= blk;
// both are monotone over the entries.
template <bool MERGE>
__device__ inline int find_entry(KArgs& A, KEntry* ents, int blk) {
  int lo = 0, hi = A.n_entries - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((MERGE ? ents[mid].merge_base : ents[mid].item_base) <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The argument block is read in place from the kernarg segment (a by-value
// parameter that is referenced would be copied to scratch memory).
__device__ inline KArgs& kernel_args() {
  return *(KArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
}

// One launch covers the items of every bit width, interleaved by the host so
// that each CU runs a mix of bandwidth-bound (wide codes) and arithmetic-bound
// (narrow codes) items; the bit width is uniform per workgroup.
template <int RB, int V>
__global__ void __launch_bounds__(kThreads, decode_wg_per_cu(V)) decode_kernel(DecodeArgs) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  KArgs& A = kernel_args();
  const int item = blockIdx.x;
  KEntry* ents = entry_array(A);
  KEntry& E = ents[find_entry<false>(A, ents, item)];
  // item numbering: chunks of one (sequence, split) pair sit 8 blocks apart, so
  // they are dispatched to the same XCD at about the same time and share its L2.
  const int local = item - E.item_base;
  const int J = E.n_seq * E.splits, nrc = E.nrc;
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
  switch (E.bits) {
    case 2: run_item<2, RB, V>(A, E, s, ks, chunk, lds); break;
    case 4: run_item<4, RB, V>(A, E, s, ks, chunk, lds); break;
    case 8: run_item<8, RB, V>(A, E, s, ks, chunk, lds); break;
    default: run_item<16, RB, V>(A, E, s, ks, chunk, lds); break;
  }
}

}  // namespace

// Launch of the decode kernel variant (RB row blocks, register budget V); each
// variant is instantiated in a translation unit of its own (kk_decode_*.hip).
template <int RB, int V>
hipError_t launch_decode_items(const DecodeArgs& a, int n, int lds, hipStream_t stream) {
  hipError_t e =
      hipFuncSetAttribute((const void*)decode_kernel<RB, V>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<RB, V>), dim3(n), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace kk
