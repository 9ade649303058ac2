// Fused transform + quantize (encode) and fused reconstruct (decode) kernels
// for gfx950.
//
// Method: "Beyond Compression Ratio: High-Throughput KV Compression for
// Disaggregated LLM Serving" (FastKVComp), Sec. 4.1.  The encoder applies a
// seeded sign flip and a Hadamard transform over head_dim, computes per-group
// min/max, derives fp16 (scale, minimum) parameters and writes packed 2/4/8-bit
// codes, all in one pass over the input; no transformed tensor is written to
// HBM.  The decoder dequantizes, applies the inverse transform, normalizes,
// restores the signs and writes 16-bit values, in the order the page lists
// the steps of its fused reconstruction.
//
// Arithmetic (fixed so that results are reproducible bit for bit):
//   z      = unnormalized Walsh-Hadamard transform of d*x in binary32, stages
//            with pair distance 1, 2, 4, ..., 64 in that order;
//   lo, hi = c*min z rounded down, c*max z rounded up (binary32);
//   m      = lo rounded down to fp16;  s = ((hi - m) rounded up) / (2^b - 1)
//            rounded up to binary32, then up to fp16;  inv = 1/s (0 if s = 0);
//   q      = round-half-even( fma(z, c, -m) * inv ), product exact;
//   decode = d * fl( c * FWHT( fma(q, s, m) ) ), rounded to nearest-even
//            (the sign commutes with round-to-nearest-even, so it is applied
//            to the 16-bit result).
// Directed roundings use error-free transforms (TwoProduct with fma, TwoSum).
//
// Work layout.  A head vector (128 channels) is held by two lanes, 64 values
// each (lane L and L+32 of a wavefront of 64).  Inputs are read with
// bounds-checked 16-byte buffer loads (out-of-range lanes read zero, so there
// is no branch per load), sign-flipped in the 16-bit domain and transposed
// through a wave-private LDS tile whose 272-byte row pitch keeps both the
// row-major writes and the per-lane reads free of bank conflicts.  Six
// butterfly stages run in registers; the seventh pairs the two lanes with
// v_permlane32_swap, which also leaves each lane holding whole 32-channel
// groups.  Per-channel groups (keys) are reduced through a second LDS
// transpose so that one thread owns one channel of one token group.
#include <algorithm>
#include <type_traits>

#include "kvc_internal.h"
#include "kvc_xpose.h"

namespace kvc {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Element i of a table that no wave of the running launch writes (chunk
// sizes and offsets, request descriptors, block tables: all written by earlier
// launches or the host), for an i that is the same in every lane of the wave
// (the index is taken from the first active lane).  It is read through the scalar
// cache: waiting for a scalar load does not wait for the wave's outstanding
// vector stores, as waiting for a vector load would (one counter covers both),
// so a tile's table lookups never drain the previous tile's stores.
template <typename T>
__device__ __forceinline__ T uniform_load(const T* base, int64_t i) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)i);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)i >> 32));
  const int64_t iu = (int64_t)(((uint64_t)hi << 32) | lo);
  static_assert(sizeof(T) % 4 == 0 && alignof(T) >= 4, "tables of whole dwords");
  typedef const __attribute__((address_space(4))) uint32_t cdword;
  cdword* src = (cdword*)base + iu * (int64_t)(sizeof(T) / 4);
  uint32_t w[sizeof(T) / 4];
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 4); ++k) w[k] = src[k];
  return __builtin_bit_cast(T, w);
}

typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));

// Raw buffer resource over [p, p + bytes): loads past the end return zero and
// stores past the end are dropped.  The range check covers the VGPR offset
// (and the instruction's immediate) but not the SGPR offset, so every
// position that must be checked goes in the VGPR offset; callers pass 0 as
// the SGPR offset.
// Cache policy bits of the streaming buffer accesses (2 = non-temporal).
// Every input and output byte of these kernels is touched once.
#ifndef KVC_LOAD_POLICY
#define KVC_LOAD_POLICY 0
#endif
#ifndef KVC_STORE_POLICY
#define KVC_STORE_POLICY 2
#endif
#ifndef KVC_NARROW_STORE_POLICY
#define KVC_NARROW_STORE_POLICY 0
#endif
constexpr int kLoadPol = KVC_LOAD_POLICY;
// The per-channel encoder's input tiles are loaded non-temporal: measured on
// the 70B shape, its kernel time drops 2-4 % (32768 tokens, bf16: 1.312 ->
// 1.289 ms; half-zero input 1.258 -> 1.213 ms; 131072 tokens, fp16: 5.26 ->
// 5.20 ms), while the same policy on the other kernels' loads slows them
// (per-token decode 1.181 -> 1.201 ms, half-zero 1.213 -> 1.343 ms).
#ifndef KVC_KEY_TILE_LOAD_POLICY
#define KVC_KEY_TILE_LOAD_POLICY 2
#endif
constexpr int kKeyTileLoadPol = KVC_KEY_TILE_LOAD_POLICY;
// Grid sizes of the fused kernels: at most KVC_*_BLOCKS blocks, and for the
// per-token ones at least KVC_*_MIN_TILES tiles per wave.  Chosen by
// measurement on the 70B shape (80 x 32768 x 8 x 128): every kernel runs
// fastest with many short-lived blocks, whose loads overlap the arithmetic of
// the other blocks resident on a CU (per-channel encode 1.44 ms at 8192
// blocks, 1.30 at 65536; per-channel decode 1.41 at 4096, 1.30-1.34 at 65536;
// per-token decode 1.26 at 2048, 1.21-1.25 at 32768; per-token encode 1.28 at
// 2048, 1.20 at 65536).  The per-token encoder's waves prefetch their next
// tile, so it keeps at least two tiles per wave: one layer (8192 tiles) takes
// 41 us in 1024 blocks against 53 us in 2048 blocks of one tile per wave.
#ifndef KVC_ET_BLOCKS
#define KVC_ET_BLOCKS 65536     // per-token encoder
#endif
#ifndef KVC_ET_MIN_TILES
#define KVC_ET_MIN_TILES 2
#endif
#ifndef KVC_DT_BLOCKS
#define KVC_DT_BLOCKS 32768     // per-token decoder
#endif
#ifndef KVC_DT_MIN_TILES
#define KVC_DT_MIN_TILES 1
#endif
#ifndef KVC_EK_BLOCKS
#define KVC_EK_BLOCKS 65536     // per-channel encoder (two-wave blocks)
#endif
#ifndef KVC_DC_BLOCKS
#define KVC_DC_BLOCKS 65536     // per-channel decoder
#endif
#ifndef KVC_DC_MIN_TILES
#define KVC_DC_MIN_TILES 1
#endif
#ifndef KVC_EC_WAVES
#define KVC_EC_WAVES 4   // waves per SIMD the complete-tile channel encoder is built for
#endif
constexpr int kStorePol = KVC_STORE_POLICY;          // 16-byte stores
constexpr int kNarrowStorePol = KVC_NARROW_STORE_POLICY;   // 4- and 8-byte stores

// Every resource here describes a per-wave (or per-block) range, so its base
// and size are wave-uniform; reading them through readfirstlane puts the
// descriptor in scalar registers, which buffer instructions require (a
// descriptor in vector registers makes the compiler loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* q = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
template <int POL = kLoadPol>
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const int4v x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, POL);
  return make_uint4((uint32_t)x.x, (uint32_t)x.y, (uint32_t)x.z, (uint32_t)x.w);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kLoadPol);
}
__device__ __forceinline__ void bstore16(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  int4v x = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)voff, (int)soff, kStorePol);
}
__device__ __forceinline__ void bstore8(uint2 v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  int2v x = {(int)v.x, (int)v.y};
  __builtin_amdgcn_raw_buffer_store_b64(x, r, (int)voff, (int)soff, kNarrowStorePol);
}
__device__ __forceinline__ void bstore4(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32((int)v, r, (int)voff, (int)soff, kNarrowStorePol);
}

__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const int2v x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, kLoadPol);
  return make_uint2((uint32_t)x.x, (uint32_t)x.y);
}

__device__ __forceinline__ uint32_t h16_from(float f) {
  _Float16 h = (_Float16)f;                     // v_cvt_f16_f32, round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f_from_h16(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Directed rounding through the MODE register: bits [1:0] hold the binary32
// rounding mode and bits [3:2] the fp16/fp64 one (0 nearest-even, 1 toward
// +inf, 2 toward -inf).  Each statement sets both fields, runs its
// instructions and restores nearest-even; being one asm statement, nothing
// else is scheduled while the mode differs.  The wait state before the
// restore keeps it from overtaking the last arithmetic instruction.
// lo = RD32(a*b), h = RD16(lo) (in the low 16 bits; the high bits are zero)
__device__ __forceinline__ void mul_cvt_rd(float a, float b, float& lo, uint32_t& h) {
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 10\n\t"
      "v_mul_f32 %0, %2, %3\n\t"
      "v_cvt_f16_f32 %1, %0\n\t"
      "s_nop 0\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 0"
      : "=&v"(lo), "=&v"(h)
      : "v"(a), "v"(b));
}
// hi = RU32(a*b), r = RU32(hi - m)
__device__ __forceinline__ void mul_sub_ru(float a, float b, float m, float& hi, float& r) {
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 5\n\t"
      "v_mul_f32 %0, %2, %3\n\t"
      "v_sub_f32 %1, %0, %4\n\t"
      "s_nop 0\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 0"
      : "=&v"(hi), "=&v"(r)
      : "v"(a), "v"(b), "v"(m));
}
// RU16(x) in the low 16 bits
__device__ __forceinline__ uint32_t cvt_f16_ru(float x) {
  uint32_t h;
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 5\n\t"
      "v_cvt_f16_f32 %0, %1\n\t"
      "s_nop 0\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 0"
      : "=v"(h)
      : "v"(x));
  return h;
}

// RN32(1 / (2^b - 1))
template <int BITS>
__device__ __forceinline__ constexpr float rcp_levels() {
  return BITS == 2 ? 0x1.555556p-2f : BITS == 4 ? 0x1.111112p-4f : 0x1.010102p-8f;
}

// Smallest binary32 >= r / k for finite r >= 0 and k = 2^b - 1: q1 is the
// correctly rounded quotient (one Markstein correction of r * RN(1/k), with
// exact fma residuals), then the residual's sign decides one step up.  The
// sequence was checked against the exact result for every binary32 r >= 0
// and k in {3, 15, 255}.
template <int BITS>
__device__ __forceinline__ float div_levels_ru(float r) {
  constexpr float k = (float)((1 << BITS) - 1);
  constexpr float rk = rcp_levels<BITS>();
  const float q0 = r * rk;
  const float e1 = __builtin_fmaf(-q0, k, r);
  const float q1 = __builtin_fmaf(e1, rk, q0);
  const float e2 = __builtin_fmaf(-q1, k, r);
  return (e2 > 0.0f) ? u2f(f2u(q1) + 1u) : q1;
}

// RN32(1 / s) for a positive fp16 value s: hardware reciprocal refined by one
// Newton step with an exact fma residual (equal to the IEEE quotient for every
// positive finite fp16 value, checked exhaustively).
__device__ __forceinline__ float rcp_rn_f16val(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}

struct GroupQ {
  float neg_m;      // -m as binary32
  float inv;        // 1/s or 0
  uint32_t packed;  // s | m << 16 (stream parameter word)
  bool bad;         // a parameter is not a finite fp16
};

template <int BITS>
__device__ __forceinline__ GroupQ group_params(float zmin, float zmax, float c) {
  // -0 and +0 are one real value; the group extremes use +0 for it
  zmin = zmin + 0.0f;
  zmax = zmax + 0.0f;
  float lo, hi, range;
  uint32_t m16;
  mul_cvt_rd(zmin, c, lo, m16);
  const float mf = f_from_h16(m16);
  mul_sub_ru(zmax, c, mf, hi, range);
  const uint32_t s16 = cvt_f16_ru(div_levels_ru<BITS>(range));
  const float sf = f_from_h16(s16);
  GroupQ g;
  g.neg_m = -mf;
  g.inv = (sf == 0.0f) ? 0.0f : rcp_rn_f16val(sf);
  g.packed = s16 | (m16 << 16);
  // a NaN or infinite extreme makes m or s NaN or infinite
  g.bad = ((s16 & 0x7c00u) == 0x7c00u) || ((m16 & 0x7c00u) == 0x7c00u);
  return g;
}

// min / max in the sense of IEEE 754-2019 minimum / maximum (gfx950's
// v_minimum3_f32 / v_maximum3_f32): a NaN operand gives NaN, so one
// non-finite transform output anywhere in a group makes its parameters
// non-finite and the group is reported as out of range; -0 orders below +0.
__device__ __forceinline__ float vmin3(float a, float b, float c) {
  float r;
  asm("v_minimum3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_maximum3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmin(float a, float b) { return vmin3(a, b, b); }
__device__ __forceinline__ float vmax(float a, float b) { return vmax3(a, b, b); }
// min and max of n >= 1 values
template <int N>
__device__ __forceinline__ void minmax_n(const float* x, float& mn, float& mx) {
  mn = x[0];
  mx = x[0];
  int i = 1;
#pragma unroll
  for (; i + 1 < N; i += 2) { mn = vmin3(mn, x[i], x[i + 1]); mx = vmax3(mx, x[i], x[i + 1]); }
  if (i < N) { mn = vmin(mn, x[i]); mx = vmax(mx, x[i]); }
}

// Code of one value: fl(fl(z*c - m) * inv + 2^23) carries round-half-even(t*inv)
// in its low mantissa bits (exact product, one rounding); bits 8..23 are zero.
__device__ __forceinline__ uint32_t quant_code(float z, float c, const GroupQ& g) {
  const float t = __builtin_fmaf(z, c, g.neg_m);
  return f2u(__builtin_fmaf(t, g.inv, 0x1p23f));
}

// Merge codes held in the low byte of each word (bits 8..23 zero) into packed
// BITS-bit fields, LSB first: 32/BITS codes -> one dword.
template <int BITS>
__device__ __forceinline__ uint32_t pack_dword(const uint32_t* q) {
  if constexpr (BITS == 8) {
    const uint32_t a = (q[1] << 8) | q[0], b = (q[3] << 8) | q[2];
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
  } else if constexpr (BITS == 4) {
    // even codes to the low nibbles of four bytes, odd codes to the high ones
    const uint32_t e = __builtin_amdgcn_perm(__builtin_amdgcn_perm(q[6], q[4], 0x0c0c0400u),
                                             __builtin_amdgcn_perm(q[2], q[0], 0x0c0c0400u), 0x05040100u);
    const uint32_t o = __builtin_amdgcn_perm(__builtin_amdgcn_perm(q[7], q[5], 0x0c0c0400u),
                                             __builtin_amdgcn_perm(q[3], q[1], 0x0c0c0400u), 0x05040100u);
    return (o << 4) | e;
  } else {
    // code pairs as 4-bit values in the low byte (bits 8..23 still zero),
    // packed as 4-bit codes; the byte selections keep the compiler from
    // re-associating the whole merge into one shift per code
    uint32_t t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = (q[2 * k + 1] << 2) | q[2 * k];
    return pack_dword<4>(t);
  }
}

template <int BITS>
__device__ __forceinline__ float unpack_code(const uint32_t* w, int i) {
  if constexpr (BITS == 4) return (float)((w[i >> 3] >> (4 * (i & 7))) & 15u);
  else if constexpr (BITS == 2) return (float)((w[i >> 4] >> (2 * (i & 15))) & 3u);
  else return (float)((w[i >> 2] >> (8 * (i & 3))) & 255u);
}

// Codes spread one per byte, so that each converts with one v_cvt_f32_ubyteN:
// for a dword of packed codes, mask k holds codes k, k + K, k + 2K, k + 3K in
// its four bytes (K = 8 / BITS masks per dword; the 8-bit codes are their own).
template <int BITS>
__device__ __forceinline__ void code_masks(const uint32_t* w, int ndw, uint32_t* m) {
#pragma unroll
  for (int d = 0; d < ndw; ++d) {
    if constexpr (BITS == 8) {
      m[d] = w[d];
    } else if constexpr (BITS == 4) {
      m[2 * d] = w[d] & 0x0F0F0F0Fu;
      m[2 * d + 1] = (w[d] >> 4) & 0x0F0F0F0Fu;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) m[4 * d + k] = (w[d] >> (2 * k)) & 0x03030303u;
    }
  }
  // opaque to the compiler: otherwise it folds each byte's extraction back
  // into a bit-field extract per code (v_bfe + v_cvt_f32_ubyte0)
#pragma unroll
  for (int k = 0; k < ndw * (8 / BITS); ++k) asm volatile("" : "+v"(m[k]));
}
// code i as binary32, from code_masks
template <int BITS>
__device__ __forceinline__ float code_of(const uint32_t* m, int i) {
  constexpr int K = 8 / BITS;                         // codes per byte
  const int d = i / (4 * K), r = i % (4 * K);
  return (float)((m[K * d + r % K] >> (8 * (r / K))) & 255u);
}

// 16-bit pair -> two binary32 values
template <bool BF16>
__device__ __forceinline__ void unpack16(uint32_t u, float& lo, float& hi) {
  if constexpr (BF16) {
    lo = u2f(u << 16);
    hi = u2f(u & 0xffff0000u);
  } else {
    lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
    hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
  }
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

// two binary32 values -> 16-bit pair, round to nearest even
template <bool BF16>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
  float2v f = {lo, hi};
  if constexpr (BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf162v));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, half2v));
}

// Sign-flip masks for the 8 channels [8*slot, 8*slot + 8) of a 16-byte slot:
// dword j flips channels 8*slot + 2j (bit 15) and 8*slot + 2j + 1 (bit 31).
__device__ __forceinline__ void slot_sign_masks(const uint32_t* signs, int slot, uint32_t* m) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch = 8 * slot + 2 * j;
    const uint32_t b0 = (signs[ch >> 5] >> (ch & 31)) & 1u;
    const uint32_t b1 = (signs[(ch + 1) >> 5] >> ((ch + 1) & 31)) & 1u;
    m[j] = (b0 << 15) | (b1 << 31);
  }
}

// One butterfly (a, b) -> (a + b, a - b), each result rounded once.  Written
// as a fixed two-instruction sequence so that the register allocator updates
// the pair in place (one temporary) instead of keeping every stage's inputs
// and outputs alive; that halves the registers the transform needs.
__device__ __forceinline__ void bfly(float& a, float& b) {
  float t;
  asm volatile("v_sub_f32 %0, %1, %2\n\tv_add_f32 %1, %1, %2" : "=&v"(t), "+v"(a) : "v"(b));
  b = t;
}

// Butterfly stages 1..32 on a lane's 64 values (register r <-> local channel r).
__device__ __forceinline__ void fwht64_inreg(float* v) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      if (!(r & h)) bfly(v[r], v[r + h]);
    }
  }
}

// Stage 64 across the lane pair (L, L+32).  Before: lane half hf holds
// channels [64 hf, 64 hf + 64).  After: register r < 32 holds channel
// 32 hf + r and register 32 + r holds channel 64 + 32 hf + r.
__device__ __forceinline__ void fwht_cross(float* v) {
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    auto p = __builtin_amdgcn_permlane32_swap(f2u(v[r]), f2u(v[r + 32]), false, false);
    float a = u2f(p[0]), b = u2f(p[1]);
    bfly(a, b);
    v[r] = a;
    v[r + 32] = b;
  }
}

// Normalization of a lane's 64 inverse-transform outputs: the product with
// c = fl32(1/sqrt(128)), rounded once.
__device__ __forceinline__ void normalize64(float* v, float c) {
#pragma unroll
  for (int r = 0; r < 64; ++r) v[r] = v[r] * c;
}

// value of the partner lane (L xor 32)
__device__ __forceinline__ float pair_xchg(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return u2f((__lane_id() < 32) ? p[1] : p[0]);
}

template <typename T>
__device__ __forceinline__ T pick(int which, const T (&a)[2]) { return which ? a[1] : a[0]; }

// chunk holding byte off of a codes section (chunk sizes are multiples of 4 KiB)
__device__ __forceinline__ int64_t chunk_of(const CallDesc& c, int64_t off) {
  if (c.chunk_shift >= 0) return off >> c.chunk_shift;
  return (int64_t)((uint64_t)(off >> 12) / (c.chunk_bytes >> 12));
}

__device__ __forceinline__ void set_status(Control* ctl, uint32_t bit) {
  __hip_atomic_fetch_or(&ctl->status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ ReqDesc load_req(const CallDesc& c, int r) {
  return (c.R == 1) ? c.one : uniform_load(c.reqs, r);
}

__device__ __forceinline__ int find_req_by_tile(const CallDesc& c, int which, int64_t tile) {
  if (c.R == 1) return 0;
  // the table brackets the request; the search is usually over one or two
  const int64_t q = tile >> c.req_shift[which];
  const int32_t* tab = which ? c.req_tab[1] : c.req_tab[0];
  int lo = uniform_load(tab, q), hi = uniform_load(tab, q + 1);
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const ReqDesc rm = uniform_load(c.reqs, mid);
    const int64_t b = which ? rm.tile_begin[1] : rm.tile_begin[0];
    if (b <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Paged: base (in 16-bit elements) of vectors [vstart, vstart + 32) of layer l
// of request rq, which lie inside one page.  ok = false flags a bad block id.
__device__ __forceinline__ int64_t page_run_base(const CallDesc& c, const ReqDesc& rq, int l, int64_t vstart,
                                                 bool& ok) {
  const int64_t vpp = (int64_t)c.page_tokens * c.heads;     // vectors per page
  const int64_t page = vstart / vpp;
  const int64_t voff = vstart - page * vpp;
  const int32_t blk = uniform_load(c.block_table, (int64_t)rq.row * c.max_blocks + page);
  ok = blk >= 0 && blk < c.num_blocks;
  if (!ok) return 0;
  return (((int64_t)l * c.num_blocks + blk) * c.page_tokens * c.heads + voff) * kHeadDim;
}

constexpr int RP = 68;               // LDS row pitch in dwords (272 bytes)
constexpr int kWaveLds = 32 * RP;    // dwords of one wave's staging tile

// 16-bit pair -> two binary32 values with the sign bits set in m (bits 15
// and 31) flipped.  For bfloat16 the flip rides on the unpacking: adding
// bit 15 toggles it modulo 2^16 (the carry leaves with the shift), and the
// high half takes an exclusive or before its mask.
template <bool BF16>
__device__ __forceinline__ void unpack16_signed(uint32_t u, uint32_t m, float& lo, float& hi) {
  if constexpr (BF16) {
    lo = u2f((u + m) << 16);
    hi = u2f((u ^ m) & 0xffff0000u);
  } else {
    unpack16<false>(u ^ m, lo, hi);
  }
}

// Stage 32 head vectors (256 bytes each, consecutive vectors vstride bytes
// apart) through LDS and return this lane's 64 values: lane half hf gets
// channels [64 hf, 64 hf + 64) of vector (lane & 31), sign-flipped with the
// table smt (32 words per lane half, word j covering channels 64 hf + 2 j, +1).
template <bool BF16>
__device__ __forceinline__ void stage_in(__amdgpu_buffer_rsrc_t src, uint32_t vstride, uint32_t* wl,
                                         const uint32_t* smt, float* f) {
  const int lane = __lane_id();
  uint32_t voff = (uint32_t)(lane >> 4) * vstride + (uint32_t)(lane & 15) * 16;
  asm volatile("" : "+v"(voff));   // one offset register: the per-load offsets are added here, not kept
  uint4 d[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) d[k] = bload16<kKeyTileLoadPol>(src, voff + (uint32_t)k * 4 * vstride, 0);
  uint32_t* wrow = wl + (lane >> 4) * RP + (lane & 15) * 4;
#pragma unroll
  for (int k = 0; k < 8; ++k) *(uint4*)(wrow + k * 4 * RP) = d[k];
  wave_sync();
  const uint32_t* rrow = wl + (lane & 31) * RP + (lane >> 5) * 32;
  const uint32_t* mrow = smt + (lane >> 5) * 32;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 x = *(const uint4*)(rrow + 4 * j);
    const uint4 m = *(const uint4*)(mrow + 4 * j);
    unpack16_signed<BF16>(x.x, m.x, f[8 * j + 0], f[8 * j + 1]);
    unpack16_signed<BF16>(x.y, m.y, f[8 * j + 2], f[8 * j + 3]);
    unpack16_signed<BF16>(x.z, m.z, f[8 * j + 4], f[8 * j + 5]);
    unpack16_signed<BF16>(x.w, m.w, f[8 * j + 6], f[8 * j + 7]);
  }
  wave_sync();
}

// Convert the lane's 64 reconstructed values (layout after fwht_cross) to
// 16-bit, transpose through LDS and store 32 vectors (vstride bytes apart),
// restoring signs; stores past the resource end are dropped.
template <bool BF16>
__device__ __forceinline__ void stage_out(const float* f, uint32_t* wl, const uint32_t* sm,
                                          __amdgpu_buffer_rsrc_t dst, uint32_t vstride) {
  const int lane = __lane_id();
  const int hf = lane >> 5;
  uint32_t* wrow = wl + (lane & 31) * RP + hf * 16;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int r0 = 32 * half + 8 * s4;
      uint4 x;
      x.x = pack16<BF16>(f[r0 + 0], f[r0 + 1]);
      x.y = pack16<BF16>(f[r0 + 2], f[r0 + 3]);
      x.z = pack16<BF16>(f[r0 + 4], f[r0 + 5]);
      x.w = pack16<BF16>(f[r0 + 6], f[r0 + 7]);
      *(uint4*)(wrow + half * 32 + s4 * 4) = x;
    }
  }
  wave_sync();
  const uint32_t* rrow = wl + (lane >> 4) * RP + (lane & 15) * 4;
  uint32_t voff = (uint32_t)(lane >> 4) * vstride + (uint32_t)(lane & 15) * 16;
  asm volatile("" : "+v"(voff));   // one offset register: the per-store offsets are added here, not kept
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint4 x = *(const uint4*)(rrow + k * 4 * RP);
    x.x ^= sm[0]; x.y ^= sm[1]; x.z ^= sm[2]; x.w ^= sm[3];
    bstore16(x, dst, voff + (uint32_t)k * 4 * vstride, 0);
  }
  wave_sync();
}


// ------------------------------------------------------------------
// Lossless size contribution of freshly packed codes.  For TUPL8_1 -> BIT_8
// -> RZE_2 the non-zero RZE words of a chunk number, over its aligned
// 1 KiB regions (128 words) and the 8 residues kk of the word index mod 8,
// the sum of popcount(OR of the region's 16 words of residue kk); for
// TUPL8_1 -> RZE_2, the non-zero bytes of the OR of the two words of each
// aligned 16-byte unit.  Both are sums of terms local to aligned pieces, so
// a wave adds the terms of the codes it wrote to the chunk's counter.
// ------------------------------------------------------------------
// value of lane ^ K (K < 32)
template <int K>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (K == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  else if constexpr (K == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  else if constexpr (K == 8) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
  else return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (K << 10));
}
template <int K>
__device__ __forceinline__ uint64_t or_lane_xor(uint64_t x) {
  const uint32_t lo = lane_xor<K>((uint32_t)x), hi = lane_xor<K>((uint32_t)(x >> 32));
  return x | (((uint64_t)hi << 32) | lo);
}
// OR over the lanes that differ only in lane-index bits LO .. HI-1 (HI <= 5)
template <int LO, int HI>
__device__ __forceinline__ uint64_t or_lane_bits(uint64_t x) {
  if constexpr (LO <= 0 && 0 < HI) x = or_lane_xor<1>(x);
  if constexpr (LO <= 1 && 1 < HI) x = or_lane_xor<2>(x);
  if constexpr (LO <= 2 && 2 < HI) x = or_lane_xor<4>(x);
  if constexpr (LO <= 3 && 3 < HI) x = or_lane_xor<8>(x);
  if constexpr (LO <= 4 && 4 < HI) x = or_lane_xor<16>(x);
  return x;
}
__device__ __forceinline__ uint32_t popc64(uint64_t x) { return (uint32_t)__builtin_popcountll(x); }
// non-zero bytes of a 64-bit word
__device__ __forceinline__ uint32_t nz_bytes64(uint64_t x) {
  const uint32_t a = (uint32_t)x, b = (uint32_t)(x >> 32);
  const uint32_t za = ~(((a & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | a | 0x7F7F7F7Fu);   // 0x80 in each zero byte
  const uint32_t zb = ~(((b & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | b | 0x7F7F7F7Fu);
  return 8u - (uint32_t)__builtin_popcount(za) - (uint32_t)__builtin_popcount(zb);
}
// sum over the wavefront (all lanes active): row sums by DPP, then the four rows
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);    // lane ^ 1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);    // lane ^ 2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false);   // row_ror:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);   // row_ror:8
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}
// counter slot of this wave: the waves writing one chunk's codes spread over
// kNnzSlots addresses
__device__ __forceinline__ uint32_t* nnz_slot(const CallDesc& c, int64_t gci) {
  const uint32_t w = (uint32_t)blockIdx.x * (blockDim.x >> 6) + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return c.chunk_counts + gci * kNnzSlots + (w & (kNnzSlots - 1));
}
__device__ __forceinline__ void add_chunk_nnz(const CallDesc& c, int64_t gci, uint32_t v) {
  const uint32_t t = wave_sum(v);
  if (__lane_id() == 0 && t) __hip_atomic_fetch_add(nnz_slot(c, gci), t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// as add_chunk_nnz when only lanes L0..L3 hold non-zero counts
template <int L0, int L1, int L2, int L3>
__device__ __forceinline__ void add_chunk_nnz4(const CallDesc& c, int64_t gci, uint32_t v) {
  const uint32_t t = __builtin_amdgcn_readlane(v, L0) + __builtin_amdgcn_readlane(v, L1) +
                     __builtin_amdgcn_readlane(v, L2) + __builtin_amdgcn_readlane(v, L3);
  if (__lane_id() == 0 && t) __hip_atomic_fetch_add(nnz_slot(c, gci), t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t u64of(uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; }

// ------------------------------------------------------------------
// Tile loads straight into LDS.  A wavefront's tile is 32 head vectors of 256
// bytes; the 16-byte loads of one instruction land in LDS at consecutive
// lanes (lane i at base + 16 i), so four rows per instruction.  Lanes fetch
// the global chunk that makes the LDS tile XOR-swizzled: row r's chunk j sits
// in slot j ^ (r & 15).  Rows then start on the same bank but the per-lane
// reads of (row, chunk) pairs spread over all banks.
// ------------------------------------------------------------------
constexpr int kTileBytes = 32 * 256;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;     // low half of a shared-aperture address is the LDS offset
}

// One 16-byte load per lane into LDS at m0 + 16 * lane.  Issued from asm so
// that the compiler's wait insertion does not add a wait for all outstanding
// memory operations before every LDS read; the caller waits explicitly.  A
// load to LDS that reads m0 needs one wait state after the scalar write of
// m0, which the compiler cannot add inside an asm statement: hence the nop.
#ifndef KVC_DMA_NT
#define KVC_DMA_NT 1
#endif
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
#if KVC_DMA_NT
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
#else
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
#endif
               :
               : "v"(voff), "s"(r), "s"(lds)
               : "memory");
}

// Wait until at most N vector memory operations are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Loads of 32 rows (vstride bytes apart) of one tile into a wave's LDS tile.
__device__ __forceinline__ void tile_dma(__amdgpu_buffer_rsrc_t src, uint32_t vstride, uint32_t lds) {
  const int lane = __lane_id();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t r = 4 * k + (lane >> 4);
    const uint32_t j = (uint32_t)(lane & 15) ^ (r & 15);
    dma16(src, r * vstride + j * 16, lds + 1024 * k);
  }
}

// This lane's 64 values of its vector from a loaded LDS tile: lane half hf
// gets channels [64 hf, 64 hf + 64) of row (lane & 31), sign-flipped with the
// table of per-chunk masks (16 chunks x 4 dwords).
template <bool BF16>
__device__ __forceinline__ void tile_read(const uint32_t* tile, const uint32_t* masks, float* f) {
  const int lane = __lane_id();
  const int v = lane & 31, hf = lane >> 5;
  const uint32_t x = (uint32_t)(8 * hf) ^ (uint32_t)(v & 15);
  const uint32_t base = (uint32_t)v * 256u + x * 16u;             // byte offset of chunk 8 hf
  const uint4* mk = (const uint4*)(masks + 32 * hf);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    uint4 d = *(const uint4*)((const char*)tile + (base ^ (uint32_t)(16 * jj)));
    const uint4 m = mk[jj];
    d.x ^= m.x; d.y ^= m.y; d.z ^= m.z; d.w ^= m.w;
    unpack16<BF16>(d.x, f[8 * jj + 0], f[8 * jj + 1]);
    unpack16<BF16>(d.y, f[8 * jj + 2], f[8 * jj + 3]);
    unpack16<BF16>(d.z, f[8 * jj + 4], f[8 * jj + 5]);
    unpack16<BF16>(d.w, f[8 * jj + 6], f[8 * jj + 7]);
  }
}

// Sign-mask table: dword 4 g + j flips channels 8 g + 2 j (bit 15) and
// 8 g + 2 j + 1 (bit 31).
__device__ __forceinline__ void fill_mask_table(const uint32_t* signs, uint32_t* table) {
  if (threadIdx.x < 64) {
    const int g = threadIdx.x >> 2, j = threadIdx.x & 3;
    const int ch = 8 * g + 2 * j;
    const uint32_t b0 = (signs[ch >> 5] >> (ch & 31)) & 1u;
    const uint32_t b1 = (signs[(ch + 1) >> 5] >> ((ch + 1) & 31)) & 1u;
    table[threadIdx.x] = (b0 << 15) | (b1 << 31);
  }
}

// Where a per-token tile's vectors and outputs live.
struct TokTile {
  const uint16_t* src;     // first input vector
  uint32_t vstride;        // bytes between consecutive input vectors
  int nv;                  // vectors present (0..32)
  int64_t vg0;             // index of the first vector within its request
  uint8_t* codes_base;
  uint8_t* params_base;
};

template <bool PAGED>
__device__ __forceinline__ TokTile enc_token_tile(const CallDesc& c, int which, int64_t tile, const uint16_t* in) {
  TokTile t;
  t.vstride = 256u;
  if constexpr (!PAGED) {
    if (c.mixed) {
      // 32 tokens of one (layer, head) slab; its codes and parameters are a
      // one-head run inside the section
      const int T = c.one.T;
      const int64_t tps = (T + 31) >> 5;
      const int sl = (int)(tile / tps);
      const int64_t t0 = (tile - (int64_t)sl * tps) * 32;
      const SlabDesc sd = uniform_load(c.slabs, sl);
      t.vg0 = t0;
      t.nv = (int)std::max<int64_t>(0, std::min<int64_t>(32, T - t0));
      t.src = in + (((int64_t)sd.l * T + t0) * c.heads + sd.h) * kHeadDim;
      t.vstride = (uint32_t)c.heads * 256u;
      t.codes_base = c.codes + pick(which, c.one.codes_off) + sd.codes_off;
      t.params_base = c.stream + pick(which, c.one.params_off) + sd.params_off;
      return t;
    }
    const int64_t nvec = (int64_t)c.layers * c.one.T * c.heads;
    t.vg0 = tile * 32;
    t.nv = (int)std::max<int64_t>(0, std::min<int64_t>(32, nvec - t.vg0));
    t.src = in + t.vg0 * kHeadDim;
    t.codes_base = c.codes + pick(which, c.one.codes_off);
    t.params_base = c.stream + pick(which, c.one.params_off);
  } else {
    const int r = find_req_by_tile(c, which, tile);
    const ReqDesc rq = load_req(c, r);
    const int64_t vpl = (int64_t)rq.T * c.heads;               // vectors per layer
    const int64_t tpl = (vpl + 31) >> 5;                        // tiles per layer
    const int64_t tr = tile - pick(which, rq.tile_begin);
    const int l = (int)(tr / tpl);
    const int64_t vstart = (tr - (int64_t)l * tpl) * 32;
    t.nv = (int)std::max<int64_t>(0, std::min<int64_t>(32, vpl - vstart));
    t.vg0 = (int64_t)l * vpl + vstart;
    bool ok;
    const int64_t base = page_run_base(c, rq, l, vstart, ok);
    if (!ok) {
      if (__lane_id() == 0) set_status(c.ctl, kStBadBlock);
      t.nv = 0;
    }
    t.src = in + base;
    t.codes_base = c.codes + pick(which, rq.codes_off);
    t.params_base = c.params_ws + pick(which, rq.params_ws_off);
  }
  return t;
}

// ===================================================================
// Encode, per-token groups.  One wavefront encodes 32 consecutive head
// vectors (a tile); 4 wavefronts per block.  Dense calls treat all L*T*H
// vectors as one run (codes and parameters follow the same order); paged
// calls decompose tiles by request, layer and page.  The loads of a wave's
// next tile are issued as soon as the current tile has been read out of LDS,
// so they are in flight while the current tile is transformed, quantized and
// stored.
// ===================================================================
template <int BITS, int G, bool BF16, bool PAGED>
__global__ __launch_bounds__(256, 4) void k_encode_token(CallDesc c, int which) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[4 * kTileBytes / 4 + 64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint32_t* wl = lds + wave * (kTileBytes / 4);
  uint32_t* masks = lds + 4 * (kTileBytes / 4);
  const uint32_t wl_lds = lds_addr(wl);
  const TensorPol pol = which ? c.pol[1] : c.pol[0];
  const float cc = pol.c;
  fill_mask_table(c.signs, masks);
  __syncthreads();
  const uint16_t* in = (const uint16_t*)(which ? c.in_kv[1] : c.in_kv[0]);
  const int64_t ntiles = which ? c.tiles[1] : c.tiles[0];
  const int v = lane & 31, hf = lane >> 5;
  constexpr int LG = (G < 32) ? G : 32;          // group size held in one lane
  constexpr int NLG = 64 / LG;
  constexpr int CB = kHeadDim * BITS / 8;        // code bytes per vector
  constexpr int NGV = kHeadDim / G;              // groups per vector
  // vector memory operations issued after a tile's loads: the code stores
  // (one per half, two for 8-bit codes) and the parameter stores; all are
  // unconditional so the count is exact
  constexpr int NPST = 1;
  constexpr int NST = ((BITS == 2) ? 1 : (BITS == 4) ? 2 : 4) + NPST;

  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t tile = (int64_t)blockIdx.x * 4 + wave;
  if (tile >= ntiles) return;
  TokTile cur = enc_token_tile<PAGED>(c, which, tile, in);
  tile_dma(make_rsrc(cur.src, cur.nv ? (uint32_t)(cur.nv - 1) * cur.vstride + 256u : 0u), cur.vstride, wl_lds);
  bool first = true;
  for (; tile < ntiles; tile += stride) {
    if (first) wait_vmcnt<0>();
    else wait_vmcnt<NST>();
    first = false;
    float f[64];
    tile_read<BF16>(wl, masks, f);
    wait_lgkm0();                                  // reads done before the tile is reloaded
    const TokTile t = cur;
    if (tile + stride < ntiles) {
      cur = enc_token_tile<PAGED>(c, which, tile + stride, in);
      tile_dma(make_rsrc(cur.src, cur.nv ? (uint32_t)(cur.nv - 1) * cur.vstride + 256u : 0u), cur.vstride, wl_lds);
    }
    fwht64_inreg(f);
    fwht_cross(f);
    // register r: channel (r < 32 ? 32 hf + r : 64 + 32 hf + r - 32)

    float mn[NLG], mx[NLG];
#pragma unroll
    for (int j = 0; j < NLG; ++j) minmax_n<LG>(f + j * LG, mn[j], mx[j]);
    if constexpr (G == 128) {
      mn[0] = vmin(mn[0], mn[1]); mx[0] = vmax(mx[0], mx[1]);
      mn[0] = vmin(mn[0], pair_xchg(mn[0])); mx[0] = vmax(mx[0], pair_xchg(mx[0]));
      mn[1] = mn[0]; mx[1] = mx[0];
    } else if constexpr (G == 64) {
#pragma unroll
      for (int j = 0; j < 2; ++j) { mn[j] = vmin(mn[j], pair_xchg(mn[j])); mx[j] = vmax(mx[j], pair_xchg(mx[j])); }
    }
    GroupQ gq[NLG];
    bool bad = false;
    if constexpr (G == 128) {
      gq[0] = group_params<BITS>(mn[0], mx[0], cc);
      gq[1] = gq[0];
      bad = gq[0].bad;
    } else {
#pragma unroll
      for (int j = 0; j < NLG; ++j) { gq[j] = group_params<BITS>(mn[j], mx[j], cc); bad |= gq[j].bad; }
    }

    const __amdgpu_buffer_rsrc_t crs = make_rsrc(t.codes_base + t.vg0 * CB, (uint32_t)t.nv * CB);
    uint32_t wv[2][BITS];                                         // packed codes of register halves 0, 1
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      constexpr int PER = 32 / BITS;                              // codes per dword
#pragma unroll
      for (int dw = 0; dw < BITS; ++dw) {
        uint32_t q[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int r2 = 32 * half + dw * PER + i;
          q[i] = quant_code(f[r2], cc, gq[r2 / LG]);
        }
        wv[half][dw] = pack_dword<BITS>(q);
      }
    }
    if constexpr (BITS == 2) {
      // lane half hf holds the 8-byte code runs of channels [32 hf, 32 hf + 32)
      // and [64 + 32 hf, ...); swapping the second run of the lower lane with the
      // first run of the upper lane gives each lane 16 contiguous bytes
#pragma unroll
      for (int dw = 0; dw < 2; ++dw) {
        auto p = __builtin_amdgcn_permlane32_swap(wv[0][dw], wv[1][dw], false, false);
        wv[0][dw] = p[0];
        wv[1][dw] = p[1];
      }
      bstore16(make_uint4(wv[0][0], wv[0][1], wv[1][0], wv[1][1]), crs, (uint32_t)v * CB + 16 * hf, 0);
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t off = (uint32_t)v * CB + (64 * half + 32 * hf) * BITS / 8;
        if constexpr (BITS == 4) bstore16(make_uint4(wv[half][0], wv[half][1], wv[half][2], wv[half][3]), crs, off, 0);
        else {
          bstore16(make_uint4(wv[half][0], wv[half][1], wv[half][2], wv[half][3]), crs, off, 0);
          bstore16(make_uint4(wv[half][4], wv[half][5], wv[half][6], wv[half][7]), crs, off + 16, 0);
        }
      }
    }
    if (c.nnz_pipe && c.nnz_sec[which]) {
      // wv[h][*]: this lane's codes of register half h (for 2 bits, after the
      // swap, the lane's 16 contiguous bytes are wv[0][0..1], wv[1][0..1])
      uint32_t cnt = 0;
      const bool live = v < t.nv;
      if (c.nnz_pipe == 1) {
        if constexpr (BITS == 2) {
          // words 4v + 2hf, +1 of a 1 KiB region: residues 4 (v & 1) + 2 hf, +1;
          // the same residue recurs in lanes differing in v bits 1..4
          uint64_t x0 = live ? u64of(wv[0][0], wv[0][1]) : 0ull, x1 = live ? u64of(wv[1][0], wv[1][1]) : 0ull;
          x0 = or_lane_bits<1, 5>(x0); x1 = or_lane_bits<1, 5>(x1);
          cnt = ((v >> 1) == 0) ? popc64(x0) + popc64(x1) : 0u;
        } else if constexpr (BITS == 4) {
          // words 8v + 4h + 2hf, +1: residues 4h + 2hf, +1; regions of 16 vectors
          uint64_t x[4];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            x[2 * h] = live ? u64of(wv[h][0], wv[h][1]) : 0ull;
            x[2 * h + 1] = live ? u64of(wv[h][2], wv[h][3]) : 0ull;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = or_lane_bits<0, 4>(x[i]);
          cnt = ((v & 15) == 0) ? popc64(x[0]) + popc64(x[1]) + popc64(x[2]) + popc64(x[3]) : 0u;
        } else {
          // words 16v + 8h + 4hf + m: residues 4hf + m (both halves); regions of 8 vectors
          uint64_t x[4];
#pragma unroll
          for (int m = 0; m < 4; ++m)
            x[m] = live ? (u64of(wv[0][2 * m], wv[0][2 * m + 1]) | u64of(wv[1][2 * m], wv[1][2 * m + 1])) : 0ull;
#pragma unroll
          for (int m = 0; m < 4; ++m) x[m] = or_lane_bits<0, 3>(x[m]);
          cnt = ((v & 7) == 0) ? popc64(x[0]) + popc64(x[1]) + popc64(x[2]) + popc64(x[3]) : 0u;
        }
      } else if (live) {
        if constexpr (BITS == 2) {
          cnt = nz_bytes64(u64of(wv[0][0], wv[0][1]) | u64of(wv[1][0], wv[1][1]));
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int u = 0; u < BITS / 4; ++u)
              cnt += nz_bytes64(u64of(wv[h][4 * u], wv[h][4 * u + 1]) | u64of(wv[h][4 * u + 2], wv[h][4 * u + 3]));
        }
      }
      const int64_t coff = t.vg0 * CB;
      const int64_t ci = chunk_of(c, coff);
      if constexpr (PAGED) {
        const int r = find_req_by_tile(c, which, tile);
        const ReqDesc rq = load_req(c, r);
        const int64_t cbase = rq.chunk_begin + (which ? rq.nchunks[0] : 0);
        // a tile may cover two chunks: a lane counts for the chunk of its vector
        const int64_t vb = ((ci + 1) * (int64_t)c.chunk_bytes - coff) / CB;
        if (vb < t.nv) {
          add_chunk_nnz(c, cbase + ci, v < vb ? cnt : 0u);
          add_chunk_nnz(c, cbase + ci + 1, v < vb ? 0u : cnt);
        } else {
          add_chunk_nnz(c, cbase + ci, cnt);
        }
      } else {
        add_chunk_nnz(c, (which ? c.one.nchunks[0] : 0) + ci, cnt);
      }
    }
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(t.params_base + t.vg0 * NGV * 4, (uint32_t)t.nv * NGV * 4);
    const uint32_t prow = (uint32_t)v * NGV * 4;
    if constexpr (G == 32) {
      // groups 2 hf and 2 + hf; after the swap the lower lane holds groups 0, 1
      // and the upper lane groups 2, 3
      auto p = __builtin_amdgcn_permlane32_swap(gq[0].packed, gq[1].packed, false, false);
      bstore8(make_uint2(p[0], p[1]), prs, prow + 8 * hf, 0);
    } else if constexpr (G == 16) {
      // groups {2 hf, 2 hf + 1} and {4 + 2 hf, 5 + 2 hf}, swapped the same way
      auto p0 = __builtin_amdgcn_permlane32_swap(gq[0].packed, gq[2].packed, false, false);
      auto p1 = __builtin_amdgcn_permlane32_swap(gq[1].packed, gq[3].packed, false, false);
      bstore16(make_uint4(p0[0], p1[0], p0[1], p1[1]), prs, prow + 16 * hf, 0);
    } else if constexpr (G == 64) {
      bstore4(hf ? gq[1].packed : gq[0].packed, prs, prow + hf * 4, 0);
    } else {
      // one parameter word per vector: the upper lane's store is pushed out of range
      bstore4(gq[0].packed, prs, hf ? 0x7ffffff0u : prow, 0);
    }
    if (bad && v < t.nv) set_status(c.ctl, kStRange);
  }
}

// ===================================================================
// Decode, per-token groups: the mirror image of k_encode_token.  A wave's
// next tile's codes and parameters (a few registers per lane) are loaded
// before the current tile is transformed and stored.
// ===================================================================
struct DecTok {
  const uint8_t* csrc;    // the tile's codes
  uint32_t cbytes;        // bytes readable there
  const uint8_t* psrc;    // the tile's parameter words
  uint32_t pbytes;
  uint16_t* dst;          // first output vector
  uint32_t vstride;       // bytes between consecutive output vectors
  int nvo;                // output vectors to store
  // a TUPL8_1 -> BIT_8 -> RZE_2 chunk decoded by the block (2-bit codes): csrc
  // is the stored chunk (cbytes readable), p1_n its raw size, the tile quarter
  // p1_q of 4 KiB block p1_gi, p1_pref the non-zero words before each bitmap
  // dword of the chunk
  int p1, p1_n, p1_gi, p1_q;
  const uint32_t* p1_pref;
};

template <int BITS, int G, bool PAGED, bool MIRROR = false>
__device__ __forceinline__ DecTok dec_token_tile(const CallDesc& c, int which, int64_t tile, uint16_t* out) {
  constexpr int CB = kHeadDim * BITS / 8;
  constexpr int NGV = kHeadDim / G;
  DecTok d;
  d.vstride = 256u;
  d.p1 = 0;
  int64_t vg0;
  int nv;
  const uint8_t* params_base;
  if constexpr (!PAGED) {
    if (c.mixed) {
      const int T = c.one.T;
      const int64_t tps = (T + 31) >> 5;
      const int sl = (int)(tile / tps);
      const int64_t t0 = (tile - (int64_t)sl * tps) * 32;
      const SlabDesc sd = uniform_load(c.slabs, sl);
      nv = (int)std::max<int64_t>(0, std::min<int64_t>(32, T - t0));
      d.nvo = nv;
      d.csrc = c.codes + pick(which, c.one.codes_off) + sd.codes_off + t0 * CB;
      d.cbytes = (uint32_t)nv * CB;
      d.psrc = c.stream + pick(which, c.one.params_off) + sd.params_off + t0 * NGV * 4;
      d.pbytes = (uint32_t)nv * NGV * 4;
      d.dst = out + (((int64_t)sd.l * T + t0) * c.heads + sd.h) * kHeadDim;
      d.vstride = (uint32_t)c.heads * 256u;
      return d;
    }
    const int64_t nvec = (int64_t)c.layers * c.one.T * c.heads;
    vg0 = tile * 32;
    nv = (int)std::max<int64_t>(0, std::min<int64_t>(32, nvec - vg0));
    d.nvo = nv;
    const int64_t coff = vg0 * CB;
    d.csrc = c.codes + pick(which, c.one.codes_off) + coff;
    d.cbytes = (uint32_t)nv * CB;
    if (c.direct[which]) {
      // a tile never straddles chunks here; a raw chunk is read in place
      const int64_t ci = chunk_of(c, coff);
      const int64_t gci = (which ? (int64_t)c.one.nchunks[0] : 0) + ci;
      const uint32_t e = uniform_load(c.chunk_sizes, gci);
      if (e >> 31) {
        const uint64_t pos = (uint64_t)c.one.payload_off + uniform_load(c.chunk_offs, gci) + (uint64_t)(coff - ci * c.chunk_bytes);
        d.csrc = c.stream + pos;
        d.cbytes = (pos >= c.stream_bytes) ? 0u : (uint32_t)std::min<uint64_t>(d.cbytes, c.stream_bytes - pos);
      } else if (MIRROR && BITS == 2 && c.mirror[which]) {
        const int64_t n = std::min<int64_t>((int64_t)c.chunk_bytes, pick(which, c.one.codes_bytes) - ci * (int64_t)c.chunk_bytes);
        if ((n & 4095) == 0) {
          const uint64_t pos = (uint64_t)c.one.payload_off + uniform_load(c.chunk_offs, gci);
          const int64_t toff = coff - ci * (int64_t)c.chunk_bytes;
          d.p1 = 1;
          d.p1_n = (int)n;
          d.p1_gi = (int)(toff >> 12);
          d.p1_q = (int)((toff >> 10) & 3);
          d.p1_pref = (const uint32_t*)(c.codes + pick(which, c.one.codes_off) + ci * (int64_t)c.chunk_bytes);
          d.csrc = c.stream + pos;
          // the chunk with its zero padding to 16 bytes: the word loads are
          // whole dwords, and the last word may end 2 bytes short of one
          d.cbytes = (pos >= c.stream_bytes)
                         ? 0u
                         : (uint32_t)std::min<uint64_t>(((e & 0x7fffffffu) + 15u) & ~15u, c.stream_bytes - pos);
        }
      }
    }
    params_base = c.stream + pick(which, c.one.params_off);
    d.dst = out + vg0 * kHeadDim;
  } else {
    const int r = find_req_by_tile(c, which, tile);
    const ReqDesc rq = load_req(c, r);
    const int64_t vpl = (int64_t)rq.T * c.heads;
    const int64_t tpl = (vpl + 31) >> 5;
    const int64_t tr = tile - pick(which, rq.tile_begin);
    const int l = (int)(tr / tpl);
    const int64_t vstart = (tr - (int64_t)l * tpl) * 32;
    nv = (int)std::max<int64_t>(0, std::min<int64_t>(32, vpl - vstart));
    vg0 = (int64_t)l * vpl + vstart;
    // this request's parameters must lie inside the input
    const uint64_t off = c.req_offsets[r];
    const bool pok =
        off + (uint64_t)pick(which, rq.params_off) + (uint64_t)pick(which, rq.params_bytes) <= c.stream_bytes;
    if (!pok) { if (__lane_id() == 0) set_status(c.ctl, kStCorrupt); nv = 0; }
    d.csrc = c.codes + pick(which, rq.codes_off) + vg0 * CB;
    d.cbytes = (uint32_t)nv * CB;
    if (c.direct[which] && nv > 0) {
      // the tile covers one or two chunks; when all are raw it reads the
      // stream, where consecutive raw chunks lie back to back
      const int64_t coff = vg0 * CB;
      const int64_t ci0 = chunk_of(c, coff), ci1 = chunk_of(c, coff + d.cbytes - 1);
      const int64_t g0 = rq.chunk_begin + (which ? rq.nchunks[0] : 0);
      const uint32_t e0 = uniform_load(c.chunk_sizes, g0 + ci0);
      const uint32_t e1 = (ci1 != ci0) ? uniform_load(c.chunk_sizes, g0 + ci1) : e0;
      if ((e0 & e1) >> 31) {
        const uint64_t pos = off + (uint64_t)rq.payload_off +
                             (uniform_load(c.chunk_offs, g0 + ci0) - uniform_load(c.chunk_offs, rq.chunk_begin)) +
                             (uint64_t)(coff - ci0 * c.chunk_bytes);
        d.csrc = c.stream + pos;
        d.cbytes = (pos >= c.stream_bytes) ? 0u : (uint32_t)std::min<uint64_t>(d.cbytes, c.stream_bytes - pos);
      }
    }
    params_base = c.stream + (pok ? off : 0) + pick(which, rq.params_off);
    bool ok;
    const int64_t base = page_run_base(c, rq, l, vstart, ok);
    if (!ok && __lane_id() == 0) set_status(c.ctl, kStBadBlock);
    d.nvo = ok ? (int)std::max<int64_t>(0, std::min<int64_t>(32, vpl - vstart)) : 0;
    d.dst = out + base;
  }
  d.psrc = params_base + vg0 * NGV * 4;
  d.pbytes = (uint32_t)nv * NGV * 4;
  return d;
}

// a lane's codes of channels [64 hf, 64 hf + 64) and its group parameter words
template <int BITS, int G>
struct DecRegs {
  static constexpr int LG = (G < 64) ? G : 64;
  static constexpr int NLG = 64 / LG;
  uint32_t w[4 * ((2 * BITS + 3) / 4)];
  uint32_t pw[NLG];
};

template <int BITS, int G>
__device__ __forceinline__ void dec_token_params(const DecTok& t, DecRegs<BITS, G>& R);

// codes and parameters of a tile; for a tile the block decodes from a
// TUPL8_1 -> BIT_8 -> RZE_2 chunk, in place of the codes the two bitmap dwords
// this lane expands and the non-zero words before each
template <int BITS, int G, bool MIRROR = false>
__device__ __forceinline__ void dec_token_load(const DecTok& t, DecRegs<BITS, G>& R) {
  constexpr int CB = kHeadDim * BITS / 8;
  const int lane = __lane_id();
  const int v = lane & 31, hf = lane >> 5;
  if (MIRROR && t.p1) {
    const uint32_t d0 = (uint32_t)((lane >> 3) * (t.p1_n >> 9) + 8 * t.p1_gi + 2 * t.p1_q);
    const uint2 b = bload8(make_rsrc(t.csrc, t.cbytes), 4u * d0);
    const uint2 p = bload8(make_rsrc(t.p1_pref, (uint32_t)t.p1_n / 16u), 4u * d0);
    R.w[0] = b.x; R.w[1] = b.y; R.w[2] = p.x; R.w[3] = p.y;
  } else {
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(t.csrc, t.cbytes);
    const uint32_t coff = (uint32_t)v * CB + 64 * hf * BITS / 8;
#pragma unroll
    for (int i = 0; i < 2 * BITS; i += 4) {
      const uint4 x = bload16(crs, coff + 4 * i, 0);
      R.w[i] = x.x; R.w[i + 1] = x.y; R.w[i + 2] = x.z; R.w[i + 3] = x.w;
    }
  }
  dec_token_params(t, R);
}

template <int BITS, int G>
__device__ __forceinline__ void dec_token_params(const DecTok& t, DecRegs<BITS, G>& R) {
  constexpr int NGV = kHeadDim / G;
  const int lane = __lane_id();
  const int v = lane & 31, hf = lane >> 5;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(t.psrc, t.pbytes);
#pragma unroll
  for (int j = 0; j < DecRegs<BITS, G>::NLG; ++j)
    R.pw[j] = bload4(prs, (uint32_t)v * NGV * 4 + ((64 * hf + j * DecRegs<BITS, G>::LG) / G) * 4, 0);
}

template <int BITS, int G, bool BF16, bool PAGED>
__global__ __launch_bounds__(256, 4) void k_decode_token(CallDesc c, int which) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[4 * kWaveLds];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint32_t* wl = lds + wave * kWaveLds;
  const TensorPol pol = which ? c.pol[1] : c.pol[0];
  const float cc = pol.c;
  uint32_t sm[4];
  slot_sign_masks(c.signs, lane & 15, sm);
  uint16_t* out = (uint16_t*)(which ? c.out_kv[1] : c.out_kv[0]);
  const int64_t ntiles = which ? c.tiles[1] : c.tiles[0];
  constexpr int LG = DecRegs<BITS, G>::LG;
  constexpr int NLG = DecRegs<BITS, G>::NLG;

  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t tile = (int64_t)blockIdx.x * 4 + wave;
  if (tile >= ntiles) return;
  DecTok cur = dec_token_tile<BITS, G, PAGED>(c, which, tile, out);
  DecRegs<BITS, G> R;
  dec_token_load(cur, R);
  for (; tile < ntiles; tile += stride) {
    const DecTok t = cur;
    const DecRegs<BITS, G> q = R;
    if (tile + stride < ntiles) {
      cur = dec_token_tile<BITS, G, PAGED>(c, which, tile + stride, out);
      dec_token_load(cur, R);
    }
    float sg[NLG], mu[NLG];
#pragma unroll
    for (int j = 0; j < NLG; ++j) {
      sg[j] = f_from_h16(q.pw[j] & 0xffffu);
      mu[j] = f_from_h16(q.pw[j] >> 16);
    }
    float f[64];
    uint32_t cm[16];                               // 2 BITS dwords of codes, 8 / BITS masks each
    code_masks<BITS>(q.w, 2 * BITS, cm);
#pragma unroll
    for (int r2 = 0; r2 < 64; ++r2) f[r2] = __builtin_fmaf(code_of<BITS>(cm, r2), sg[r2 / LG], mu[r2 / LG]);

    fwht64_inreg(f);
    fwht_cross(f);
    normalize64(f, cc);
    stage_out<BF16>(f, wl, sm, make_rsrc(t.dst, t.nvo ? (uint32_t)(t.nvo - 1) * t.vstride + 256u : 0u), t.vstride);
  }
}

// -------------------------------------------------------------------
// Per-token decode that also decodes TUPL8_1 -> BIT_8 -> RZE_2 chunks of 2-bit
// codes (the mirror of the single-pass placement).  A stored chunk of n bytes
// is the RZE bitmap (n / 16 bytes; bit r of dword d = j dpj + 8 gi + kk,
// dpj = n / 512, marks 16-bit quarter r % 4 of row 8 j + r / 4 of the (4 KiB
// block gi, kk) transpose) followed by the non-zero words in order;
// k_ll_decode_raw leaves the count of non-zero words before each bitmap dword
// in the chunk's codes slot.  A block's four tiles are one 4 KiB block: wave w
// gathers rows of transposes kk = 2 w, 2 w + 1 (lane c row c), transposes
// them back (lane i then holds input word 8 i + kk) and puts them in LDS; each
// wave then reads its tile's codes from there.  Reads are buffer loads bounded
// by the stored size: a set bit over a zero word marks a corrupt stream.
// -------------------------------------------------------------------
// The nibble's non-zero words are consecutive in the stream: three dword
// loads from the one holding its first word cover them, and the nibble's
// entry of `nibtab` (rze_nibble_entry) spreads them to their places.
__device__ __forceinline__ uint32_t p1_block_to_lds(const DecTok& t, const uint32_t* seg, uint32_t* blk,
                                                   const uint4* nibtab) {
  const int lane = __lane_id();
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(t.csrc, t.cbytes);
  const uint32_t words = (uint32_t)t.p1_n / 16u;
  const uint32_t sh = 4u * (uint32_t)(lane & 7);
  const rze_u16x2 one2 = opaque_one2();
  uint32_t bad = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t kb = seg[h];                 // bitmap dword of transpose kk = 2 p1_q + h
    const uint32_t nib = (kb >> sh) & 15u;
    const uint32_t r0 = seg[2 + h] + (uint32_t)__builtin_popcount(kb & ((1u << sh) - 1u));
    // bytes past the stored size read zero (a set bit there is a corrupt stream)
    const uint32_t off = words + 2u * (r0 & ~1u);
    const uint32_t d0 = bload4(rs, off, 0), d1 = bload4(rs, off + 4u, 0), d2 = bload4(rs, off + 8u, 0);
    const uint32_t s16 = (r0 & 1u) << 4;
    const uint32_t p01 = __builtin_amdgcn_alignbit(d1, d0, s16), p23 = __builtin_amdgcn_alignbit(d2, d1, s16);
    const uint4 e = nibtab[nib];
    uint32_t lo = __builtin_amdgcn_perm(p23, p01, e.x), hi = __builtin_amdgcn_perm(p23, p01, e.y);
    bad |= (nz_halves(lo, one2) ^ e.z) | (nz_halves(hi, one2) ^ e.w);
    xpose64_lean(lo, hi);
    *(uint2*)(blk + 2 * (8 * lane + 2 * t.p1_q + h)) = make_uint2(lo, hi);
  }
  return bad;
}

template <int G, bool BF16>
__global__ __launch_bounds__(256, 4) void k_decode_token_m(CallDesc c, int which) {
  constexpr int BITS = 2;
  __shared__ __attribute__((aligned(16))) uint32_t lds[4 * kWaveLds];
  __shared__ __attribute__((aligned(16))) uint32_t blk[1024];      // one decoded 4 KiB block
  __shared__ __attribute__((aligned(16))) uint4 nibtab[16];         // RZE_2 nibble expansion
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (threadIdx.x < 16) nibtab[threadIdx.x] = rze_nibble_entry(threadIdx.x);   // read after a barrier
  uint32_t* wl = lds + wave * kWaveLds;
  const TensorPol pol = which ? c.pol[1] : c.pol[0];
  const float cc = pol.c;
  uint32_t sm[4];
  slot_sign_masks(c.signs, lane & 15, sm);
  uint16_t* out = (uint16_t*)(which ? c.out_kv[1] : c.out_kv[0]);
  const int64_t ntiles = which ? c.tiles[1] : c.tiles[0];
  constexpr int LG = DecRegs<BITS, G>::LG;
  constexpr int NLG = DecRegs<BITS, G>::NLG;
  const int v = lane & 31, hf = lane >> 5;

  // every wave runs the block's iterations (block barriers around the shared
  // decode); a wave past the last tile stores nothing
  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t b0 = (int64_t)blockIdx.x * 4;
  if (b0 >= ntiles) return;
  auto tile_at = [&](int64_t base) {
    const int64_t tl = base + wave;
    DecTok d = dec_token_tile<BITS, G, false, true>(c, which, tl < ntiles ? tl : base, out);
    if (tl >= ntiles) d.nvo = 0;
    d.p1_q = wave;                               // the wave's quarter (also past the end)
    return d;
  };
  DecTok cur = tile_at(b0);
  DecRegs<BITS, G> R;
  dec_token_load<BITS, G, true>(cur, R);
  for (; b0 < ntiles; b0 += stride) {
    const DecTok t = cur;
    DecRegs<BITS, G> q = R;
    if (b0 + stride < ntiles) {
      cur = tile_at(b0 + stride);
      dec_token_load<BITS, G, true>(cur, R);
    }
    if (t.p1) {                                  // the same for the block's four tiles
      __syncthreads();                           // the previous block's readers are done
      const uint32_t bad = p1_block_to_lds(t, q.w, blk, nibtab);
      if (bad) set_status(c.ctl, kStCorrupt);
      __syncthreads();
      const uint4 x = *(const uint4*)(blk + 256 * t.p1_q + 8 * v + 4 * hf);
      q.w[0] = x.x; q.w[1] = x.y; q.w[2] = x.z; q.w[3] = x.w;
    }
    float sg[NLG], mu[NLG];
#pragma unroll
    for (int j = 0; j < NLG; ++j) {
      sg[j] = f_from_h16(q.pw[j] & 0xffffu);
      mu[j] = f_from_h16(q.pw[j] >> 16);
    }
    float f[64];
    uint32_t cm[16];                               // 2 BITS dwords of codes, 8 / BITS masks each
    code_masks<BITS>(q.w, 2 * BITS, cm);
#pragma unroll
    for (int r2 = 0; r2 < 64; ++r2) f[r2] = __builtin_fmaf(code_of<BITS>(cm, r2), sg[r2 / LG], mu[r2 / LG]);

    fwht64_inreg(f);
    fwht_cross(f);
    normalize64(f, cc);
    stage_out<BF16>(f, wl, sm, make_rsrc(t.dst, t.nvo ? (uint32_t)(t.nvo - 1) * t.vstride + 256u : 0u), t.vstride);
  }
}

// ===================================================================
// Per-channel groups (keys), dense calls.  A block of two wavefronts handles
// one tile of 64 tokens x 1 head of one layer (one group of 64 or two groups
// of 32).  LDS tile z[64 tokens][64 channels] (pitch 68), channels of rows
// 32..63 XOR-swizzled by 32 so that the two token halves read distinct banks;
// each wave's staging tile aliases its own 32 rows.
// ===================================================================
__device__ __forceinline__ int64_t pc_layer_bytes(int T, int G, int H, int bits) {
  const int ng = (T + G - 1) / G;
  const int glast = T - (ng - 1) * G;
  return (int64_t)(ng - 1) * H * kHeadDim * (G * bits / 8) + (int64_t)H * kHeadDim * ((glast * bits + 7) / 8);
}
// byte offset of the (l, g, h) block and the column bytes of that group
__device__ __forceinline__ int64_t pc_block(int T, int G, int H, int bits, int l, int g, int h, int& colb) {
  const int ng = (T + G - 1) / G;
  const int gg = (g == ng - 1) ? T - g * G : G;
  colb = (gg * bits + 7) / 8;
  return (int64_t)l * pc_layer_bytes(T, G, H, bits) + (int64_t)g * H * kHeadDim * (G * bits / 8) +
         (int64_t)h * kHeadDim * colb;
}

// TAIL = false: the complete 64-token groups; TAIL = true: the last,
// incomplete group of every (layer, head) when T is not a multiple of 64.
template <int BITS, int G, bool BF16, bool TAIL>
__global__ __launch_bounds__(128, TAIL ? 4 : KVC_EC_WAVES) void k_encode_channel(CallDesc c, int which) {
  __shared__ __attribute__((aligned(16))) float zb[64 * RP];
  __shared__ __attribute__((aligned(16))) uint32_t smt[64];
  // 2-bit groups of 64: per pass and wave, the ORs of the 8 residues of the
  // 8-byte word index over the wave's channels (a 1 KiB region spans both waves)
  __shared__ __attribute__((aligned(16))) uint64_t part2[(BITS == 2 && G == 64 && !TAIL) ? 2 * 2 * 8 : 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const TensorPol pol = which ? c.pol[1] : c.pol[0];
  const float cc = pol.c;
  if (threadIdx.x < 64) {
    // sign words of channel pairs (2 t, 2 t + 1) at bits 15 and 31
    const int ch = 2 * threadIdx.x;
    smt[threadIdx.x] = (((c.signs[ch >> 5] >> (ch & 31)) & 1u) << 15) | (((c.signs[ch >> 5] >> ((ch & 31) + 1)) & 1u) << 31);
  }
  const uint16_t* in = (const uint16_t*)(which ? c.in_kv[1] : c.in_kv[0]);
  uint32_t* stg = (uint32_t*)(zb + 32 * wave * RP);          // this wave's staging (aliases its z rows)
  const int v = lane & 31, hf = lane >> 5;
  const int H = c.heads;
  const int T = c.one.T;
  const int n64 = TAIL ? 1 : T / 64;                   // groups this kernel walks per layer
  // mixed precision: the launch covers c.nslabs (layer, head) slabs of one width
  const int64_t ntiles = c.mixed ? (int64_t)c.nslabs * n64 : (int64_t)c.layers * n64 * H;
  const int ngr = (T + G - 1) / G;
  uint8_t* codes_sec = c.codes + pick(which, c.one.codes_off);
  uint32_t* prm = (uint32_t*)(c.stream + pick(which, c.one.params_off));
  const uint32_t vstride = (uint32_t)H * 256u;

  // Tile order.  Workgroups are handed to the eight XCDs in turn, so the
  // blocks one XCD receives are those with the same blockIdx mod 8.  Virtual
  // tile v = 8 r + x (v below `full`) is head r mod H of 64-token group
  // 8 (r / H) + x: an XCD takes all heads of a group one after another and
  // reads whole token rows of the layer.  The last ngroups mod 8 groups
  // (v >= full) go in plain order.  Group index = l * n64 + g64.
  const int tw0 = 32 * wave;                           // this wave's first token in a tile
  const int ngroups = (int)(ntiles / H);
  const int full = (ngroups / 8) * 8 * H;
  auto decode_tile = [&](int vt, int& l_, int& g_, int& h_) {
    int gidx;
    if (vt < full) {
      const int r = vt >> 3;
      h_ = r % H;
      gidx = (r / H) * 8 + (vt & 7);
    } else {
      h_ = (vt - full) % H;
      gidx = full / H + (vt - full) / H;
    }
    l_ = gidx / n64;
    g_ = gidx % n64;
  };
  // advancing v by a grid size that is a multiple of 8 keeps x: r grows by
  // step / 8 = dq H + dh, the group index by 8 dq (+ 8 when the head wraps)
  const int step = (int)gridDim.x;
  const bool stepwise = (step & 7) == 0;
  const int dh = (step >> 3) % H, dq = (step >> 3) / H;
  const int dgA = (8 * dq) % n64, dlA = (8 * dq) / n64;
  const int dgB = (8 * dq + 8) % n64, dlB = (8 * dq + 8) / n64;
  int l, g64, h;
  decode_tile((int)blockIdx.x, l, g64, h);
  if constexpr (TAIL) g64 = T / 64;
  // the sign table is written; from here on each pass ends with a barrier, so
  // a tile's staging writes never meet the previous tile's readers
  __syncthreads();
  for (int tile = blockIdx.x; tile < (int)ntiles; tile += step) {
    // output addressing: (layer, head) within the section layout, and its base
    int lo = l, ho = h, Ho = H;
    uint8_t* csec = codes_sec;
    uint32_t* psec = prm;
    if (c.mixed) {
      const int sl = tile / n64;
      const SlabDesc sd = uniform_load(c.slabs, sl);
      l = sd.l;
      h = sd.h;
      g64 = TAIL ? T / 64 : tile - sl * n64;
      lo = 0; ho = 0; Ho = 1;
      csec = codes_sec + sd.codes_off;
      psec = (uint32_t*)((uint8_t*)prm + sd.params_off);
    }
    const int t0 = g64 * 64;
    const int gg = TAIL ? T - t0 : 64;                 // valid tokens in this tile
    const int nvw = TAIL ? max(0, min(32, gg - tw0)) : 32;

    float f[64];
    const uint16_t* src = in + (((int64_t)l * T + t0 + tw0) * H + h) * kHeadDim;
    stage_in<BF16>(make_rsrc(src, nvw ? (uint32_t)(nvw - 1) * vstride + 256u : 0u), vstride, stg, smt, f);
    fwht64_inreg(f);
    fwht_cross(f);

    // two passes of 64 channels: pass p holds channels [64p, 64p + 64)
    uint32_t tile_cnt = 0;                             // this lane's RZE word counts, both passes
    int64_t tile_gci = 0;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float* wrow = zb + (tw0 + v) * RP + ((32 * hf) ^ (32 * wave));   // rows >= 32 swizzled by 32
#pragma unroll
      for (int s4 = 0; s4 < 8; ++s4)
        *(float4*)(wrow + 4 * s4) = make_float4(f[32 * p + 4 * s4], f[32 * p + 4 * s4 + 1],
                                                f[32 * p + 4 * s4 + 2], f[32 * p + 4 * s4 + 3]);
      __syncthreads();
      // channel phase: this thread owns channel chl of token half th
      const int chl = 32 * wave + (lane & 31);
      const int th = lane >> 5;
      const int ch = 64 * p + chl;
      float zc[32];
      const float* rcol = zb + 32 * th * RP + (chl ^ (32 * th));
#pragma unroll
      for (int i = 0; i < 32; ++i) zc[i] = rcol[i * RP];
      // FULL: all 64 tokens of the tile exist (every group is complete)
      auto pass = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int nvt = FULL ? 32 : max(0, min(32, gg - 32 * th));   // valid tokens of this half
        float a, b;
        if constexpr (FULL) {
          minmax_n<32>(zc, a, b);
        } else {
          a = __builtin_inff(); b = -__builtin_inff();
#pragma unroll
          for (int i = 0; i < 32; ++i) if (i < nvt) { a = vmin(a, zc[i]); b = vmax(b, zc[i]); }
        }
        int grp, ntok;
        if constexpr (G == 64) {
          a = vmin(a, pair_xchg(a));
          b = vmax(b, pair_xchg(b));
          grp = g64; ntok = gg;
        } else {
          grp = 2 * g64 + th; ntok = nvt;
        }
        const GroupQ gq = group_params<BITS>(a, b, cc);
        if (gq.bad && nvt > 0) set_status(c.ctl, kStRange);
        uint32_t w[BITS];
        constexpr int PER = 32 / BITS;
#pragma unroll
        for (int dw = 0; dw < BITS; ++dw) {
          uint32_t q[PER];
#pragma unroll
          for (int i = 0; i < PER; ++i) {
            const int t2 = dw * PER + i;
            q[i] = (FULL || t2 < nvt) ? quant_code(zc[t2], cc, gq) : 0x4b000000u;
          }
          w[dw] = pack_dword<BITS>(q);
        }
        int colb;
        // complete tiles: the block of the tile's first group (both halves of a
        // G = 32 tile are complete groups, the second one block further on)
        const int64_t boff = pc_block(T, G, Ho, BITS, lo, FULL ? ((G == 64) ? g64 : 2 * g64) : grp, ho, colb);
        const int tok0 = (G == 64) ? 32 * th : 0;        // first token of this thread in its group
        if constexpr (FULL) {
          const uint32_t gstride = (G == 64) ? 0u : (uint32_t)Ho * kHeadDim * colb;
          const __amdgpu_buffer_rsrc_t crs = make_rsrc(csec + boff, gstride + (uint32_t)kHeadDim * colb);
          const uint32_t co = (uint32_t)th * gstride + (uint32_t)ch * colb + (uint32_t)(tok0 * BITS / 8);
          if constexpr (BITS == 2) bstore8(make_uint2(w[0], w[1]), crs, co, 0);
          else if constexpr (BITS == 4) bstore16(make_uint4(w[0], w[1], w[2], w[3]), crs, co, 0);
          else {
            bstore16(make_uint4(w[0], w[1], w[2], w[3]), crs, co, 0);
            bstore16(make_uint4(w[4], w[5], w[6], w[7]), crs, co + 16, 0);
          }
        } else if (nvt == 32 && colb == G * BITS / 8) {
          uint8_t* dst = csec + boff + (int64_t)ch * colb + tok0 * BITS / 8;
          if constexpr (BITS == 2) *(uint2*)dst = make_uint2(w[0], w[1]);
          else if constexpr (BITS == 4) *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
          else {
            *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
            *(uint4*)(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
          }
        } else if (ntok > 0 && nvt > 0) {
          uint8_t* dst = csec + boff + (int64_t)ch * colb + tok0 * BITS / 8;
          // partial group: this thread's codes start at byte tok0 * BITS / 8
          const int nbytes = (nvt * BITS + 7) / 8;
#pragma unroll
          for (int i = 0; i < 4 * BITS; ++i)
            if (i < nbytes) dst[i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
        }
        const bool writer = (G == 64) ? (th == 0) : true;
        if constexpr (FULL) {
          const int grp0 = (G == 64) ? g64 : 2 * g64;
          const uint32_t pstride = (G == 64) ? 0u : (uint32_t)Ho * kHeadDim;  // next group, in words
          const __amdgpu_buffer_rsrc_t prs =
              make_rsrc(psec + (((int64_t)lo * ngr + grp0) * Ho + ho) * kHeadDim, 4u * (pstride + kHeadDim));
          if (writer) bstore4(gq.packed, prs, 4u * ((uint32_t)th * pstride + (uint32_t)ch), 0);
        } else if (writer && ntok > 0) {
          psec[(((int64_t)lo * ngr + grp) * Ho + ho) * kHeadDim + ch] = gq.packed;
        }
        if constexpr (G == 64 && FULL && BITS >= 4) {
          if (c.nnz_pipe && c.nnz_sec[which]) {
            // this thread's codes: 4 * BITS bytes at ch * 8 BITS + th * 4 BITS of
            // the group block, i.e. words (4 BITS ch + 2 BITS th) / 4 + m
            uint32_t cnt = 0;
            if (c.nnz_pipe == 1) {
              if constexpr (BITS == 4) {
                // residues 4 (ch & 1) + 2 th, +1; a 1 KiB region is this wave's 32 channels
                uint64_t x0 = u64of(w[0], w[1]), x1 = u64of(w[2], w[3]);
                x0 = or_lane_bits<1, 5>(x0); x1 = or_lane_bits<1, 5>(x1);
                cnt = popc64(x0) + popc64(x1);               // the sum of lanes 0, 1, 32 and 33
              } else {
                // residues 4 th + m; regions of 16 channels
                uint64_t x[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) x[m] = or_lane_bits<0, 4>(u64of(w[2 * m], w[2 * m + 1]));
                cnt = popc64(x[0]) + popc64(x[1]) + popc64(x[2]) + popc64(x[3]);   // lanes 0, 16, 32, 48
              }
            } else {
#pragma unroll
              for (int u = 0; u < BITS / 4; ++u)
                cnt += nz_bytes64(u64of(w[4 * u], w[4 * u + 1]) | u64of(w[4 * u + 2], w[4 * u + 3]));
            }
            // both passes' codes lie in the same group block, hence the same
            // chunk: one atomic per tile
            tile_cnt += cnt;
            tile_gci = (which ? (int64_t)c.one.nchunks[0] : 0) + chunk_of(c, boff);
          }
        }
        if constexpr (G == 64 && FULL && BITS == 2) {
          if (c.nnz_pipe && c.nnz_sec[which]) {
            // this thread's codes: the 8-byte word 2 ch + th of the group block
            const uint64_t x = u64of(w[0], w[1]);
            if (c.nnz_pipe == 1) {
              // residue 2 (ch & 3) + th; the pass's 64 channels are one 1 KiB
              // region: OR over this wave's lanes of equal (ch & 3, th), the
              // other wave's half joins through LDS after the pass
              const uint64_t y = or_lane_bits<2, 5>(x);
              if ((lane & 28) == 0) part2[(2 * p + wave) * 8 + 2 * (lane & 3) + th] = y;
            } else {
              // the channel's aligned 16-byte unit is the words of th = 0 and 1
              const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
              auto plo = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
              auto phi = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
              const uint64_t o = u64of(th ? plo[0] : plo[1], th ? phi[0] : phi[1]);
              if (th == 0) tile_cnt += nz_bytes64(x | o);
            }
            tile_gci = (which ? (int64_t)c.one.nchunks[0] : 0) + chunk_of(c, boff);
          }
        }
      };
      if constexpr (TAIL) pass(std::false_type{});
      else pass(std::true_type{});
      __syncthreads();                                   // before the next pass overwrites zb
    }
    if constexpr (G == 64 && !TAIL && BITS == 2) {
      if (c.nnz_pipe && c.nnz_sec[which]) {
        if (c.nnz_pipe == 1) {
          // both passes' regions lie in the tile's group block, hence one chunk
          if (wave == 0) {
            const int q = lane & 15;
            const uint32_t cnt = (lane < 16) ? popc64(part2[(2 * (q >> 3)) * 8 + (q & 7)] |
                                                       part2[(2 * (q >> 3) + 1) * 8 + (q & 7)]) : 0u;
            add_chunk_nnz(c, tile_gci, cnt);
          }
        } else {
          add_chunk_nnz(c, tile_gci, tile_cnt);
        }
      }
    }
    if constexpr (G == 64 && !TAIL && BITS >= 4) {
      if (c.nnz_pipe && c.nnz_sec[which]) {
        if (c.nnz_pipe == 1) {
          if constexpr (BITS == 4) add_chunk_nnz4<0, 1, 32, 33>(c, tile_gci, tile_cnt);
          else add_chunk_nnz4<0, 16, 32, 48>(c, tile_gci, tile_cnt);
        } else {
          add_chunk_nnz(c, tile_gci, tile_cnt);
        }
      }
    }
    const int nt = tile + step;
    if (stepwise && nt < full) {
      h += dh;
      const bool cy = h >= H;
      if (cy) h -= H;
      g64 += cy ? dgB : dgA;
      l += cy ? dlB : dlA;
      if (g64 >= n64) { g64 -= n64; ++l; }
    } else {
      decode_tile(nt, l, g64, h);
    }
    if constexpr (TAIL) g64 = T / 64;
  }
}

// Per-channel decode.  A wave reconstructs 32 tokens x 1 head (half of a
// 64-token tile) on its own LDS region, with no block barriers: in pass p
// lane c dequantizes channel 64 p + c of its 32 tokens into column c of a
// 32 x 64 tile, and the lanes of half p read their rows back.  The next
// wave-tile's codes and parameters are loaded before the current one is
// transformed and stored.
template <int BITS>
struct ChRegs {
  uint32_t w[2][BITS];   // codes of channel 64 p + lane for the wave's 32 tokens
  uint32_t pw[2];        // its group parameter word
};

// A wave-tile: 32 tokens (half `half` of 64-token group g64 of layer l) of head h.
struct WaveTile {
  int l, g64, h, half;
  int k;                 // 2 h + half
  int sl;                // mixed precision: index of the (layer, head) slab in the launch, else -1
};

// Wave-tile order of the per-channel decoder.  Workgroups go to the eight
// XCDs in turn (blockIdx mod 8), four wave-tiles per block.  Wave-tile
// u = 4 b + w with b = 8 r + x (u below `full`) is entry k = s mod 2H,
// s = 4 r + w, of 64-token group 8 (s / 2H) + x: the blocks of one XCD walk
// all heads and halves of a group before the next.  The rest goes in plain
// order.  Group index = l * n64 + g64.
struct ChDecOrder {
  int H, n64, full;
  int dk, dgA, dlA, dgB, dlB;
  bool stepwise;
  const SlabDesc* slabs;   // mixed precision: the launch's slabs, wave-tiles in plain order
  __device__ ChDecOrder(int H_, int n64_, int64_t ntiles, int grid, const SlabDesc* slabs_)
      : H(H_), n64(n64_), slabs(slabs_) {
    const int ngroups = (int)(ntiles / H);
    full = (H % 2 == 0 && !slabs) ? (ngroups / 8) * 8 * 2 * H : 0;
    stepwise = (grid & 7) == 0;
    const int ds = grid / 2;                         // s advance per grid stride of wave-tiles
    dk = ds % (2 * H);
    const int dq = ds / (2 * H);
    dgA = (8 * dq) % n64; dlA = (8 * dq) / n64;
    dgB = (8 * dq + 8) % n64; dlB = (8 * dq + 8) / n64;
  }
  __device__ WaveTile decode(int64_t u) const {
    WaveTile o;
    o.sl = -1;
    if (slabs) {
      const int tile = (int)(u >> 1);
      o.sl = tile / n64;
      const SlabDesc sd = uniform_load(slabs, o.sl);
      o.l = sd.l; o.h = sd.h; o.g64 = tile - o.sl * n64; o.half = (int)(u & 1);
      o.k = 2 * o.h + o.half;
      return o;
    }
    int grp;
    if (u < full) {
      const int b = (int)(u >> 2);
      const int sidx = 4 * (b >> 3) + (int)(u & 3);
      o.k = sidx % (2 * H);
      grp = 8 * (sidx / (2 * H)) + (b & 7);
    } else {
      const int64_t w = u - full;
      o.k = (int)(w % (2 * H));
      grp = full / (2 * H) + (int)(w / (2 * H));
    }
    o.h = o.k >> 1; o.half = o.k & 1;
    o.l = grp / n64; o.g64 = grp % n64;
    return o;
  }
  // wave-tile u, given o = wave-tile u - stride
  __device__ WaveTile advance(int64_t u, WaveTile o) const {
    if (stepwise && u < full && !slabs) {
      o.k += dk;
      const bool cy = o.k >= 2 * H;
      if (cy) o.k -= 2 * H;
      o.g64 += cy ? dgB : dgA;
      o.l += cy ? dlB : dlA;
      if (o.g64 >= n64) { o.g64 -= n64; ++o.l; }
      o.h = o.k >> 1; o.half = o.k & 1;
      return o;
    }
    return decode(u);
  }
};

template <int BITS, int G>
__device__ __forceinline__ void ch_dec_load(const CallDesc& c, int which, WaveTile wt, ChRegs<BITS>& R) {
  const int lane = __lane_id();
  const int H = c.heads, T = c.one.T;
  const int ngr = (T + G - 1) / G;
  const int half = wt.half, g64 = wt.g64;
  const int gg = min(64, T - g64 * 64);
  const int nvw = max(0, min(32, gg - 32 * half));            // tokens of this wave-tile
  const int grp = (G == 64) ? g64 : 2 * g64 + half;
  const int tok0 = (G == 64) ? 32 * half : 0;                 // first token of the wave in its group
  const uint8_t* codes_sec = c.codes + pick(which, c.one.codes_off);
  const uint32_t* prm = (const uint32_t*)(c.stream + pick(which, c.one.params_off));
  // (layer, head) within the section layout: a mixed slab is a one-layer, one-head run
  int l = wt.l, h = wt.h, Ho = H;
  if (wt.sl >= 0) {
    const SlabDesc sd = uniform_load(c.slabs, wt.sl);
    codes_sec += sd.codes_off;
    prm = (const uint32_t*)((const uint8_t*)prm + sd.params_off);
    l = 0; h = 0; Ho = 1;
  }
  int colb;
  const int64_t boff = pc_block(T, G, Ho, BITS, l, grp, h, colb);
  // a group block never straddles chunks here: a raw chunk is read in place
  int64_t rawpos = -1;
  if (nvw > 0 && c.direct[which]) {
    const int64_t ci = chunk_of(c, boff);
    const int64_t gci = (which ? (int64_t)c.one.nchunks[0] : 0) + ci;
    const uint32_t e = uniform_load(c.chunk_sizes, gci);
    if (e >> 31)
      rawpos = (int64_t)((uint64_t)c.one.payload_off + uniform_load(c.chunk_offs, gci) + (uint64_t)(boff - ci * c.chunk_bytes));
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int ch = 64 * p + lane;
#pragma unroll
    for (int i = 0; i < BITS; ++i) R.w[p][i] = 0;
    R.pw[p] = 0;
    if (nvw > 0) {
      const uint8_t* col = codes_sec + boff + (int64_t)ch * colb;
      bool have = true;
      if (rawpos >= 0) {
        const uint64_t pos = (uint64_t)rawpos + (uint64_t)ch * colb;
        have = pos + (uint64_t)colb <= c.stream_bytes;
        col = c.stream + pos;
      }
      const uint8_t* s = col + tok0 * BITS / 8;
      if (!have) {
        // past the end of a damaged stream (already flagged): zero codes
      } else if (nvw == 32 && colb == G * BITS / 8) {
        if constexpr (BITS == 2) { const uint2 x = *(const uint2*)s; R.w[p][0] = x.x; R.w[p][1] = x.y; }
        else {
#pragma unroll
          for (int i = 0; i < BITS; i += 4) {
            const uint4 x = *(const uint4*)(s + 4 * i);
            R.w[p][i] = x.x; R.w[p][i + 1] = x.y; R.w[p][i + 2] = x.z; R.w[p][i + 3] = x.w;
          }
        }
      } else {
        const int nbytes = (nvw * BITS + 7) / 8;
#pragma unroll
        for (int i = 0; i < 4 * BITS; ++i)
          if (i < nbytes) R.w[p][i >> 2] |= (uint32_t)s[i] << (8 * (i & 3));
      }
      R.pw[p] = prm[(((int64_t)l * ngr + grp) * Ho + h) * kHeadDim + ch];
    }
  }
}

template <int BITS, int G, bool BF16>
__global__ __launch_bounds__(256, 4) void k_decode_channel(CallDesc c, int which) {
  __shared__ __attribute__((aligned(16))) float lds[4 * 32 * RP];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  float* zw = lds + wave * 32 * RP;
  uint32_t* stg = (uint32_t*)zw;                                  // output staging aliases it
  const TensorPol pol = which ? c.pol[1] : c.pol[0];
  const float cc = pol.c;
  uint32_t sm[4];
  slot_sign_masks(c.signs, lane & 15, sm);
  uint16_t* out = (uint16_t*)(which ? c.out_kv[1] : c.out_kv[0]);
  const int64_t nwt = 2 * (which ? c.tiles[1] : c.tiles[0]);
  const int v = lane & 31, hf = lane >> 5;
  const int H = c.heads, T = c.one.T;
  const int n64 = (T + 63) / 64;
  const uint32_t vstride = (uint32_t)H * 256u;

  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t wt = (int64_t)blockIdx.x * 4 + wave;
  if (wt >= nwt) return;
  const ChDecOrder order(H, n64, nwt / 2, (int)gridDim.x, c.mixed ? c.slabs : nullptr);
  WaveTile nxt = order.decode(wt);
  ChRegs<BITS> R;
  ch_dec_load<BITS, G>(c, which, nxt, R);
  for (; wt < nwt; wt += stride) {
    const ChRegs<BITS> q = R;
    const WaveTile cur = nxt;
    nxt = order.advance(wt + stride, nxt);
    if (wt + stride < nwt) ch_dec_load<BITS, G>(c, which, nxt, R);
    const int h = cur.h, g64 = cur.g64, l = cur.l;
    const int t0 = g64 * 64 + 32 * cur.half;
    const int nvw = max(0, min(32, T - t0));

    float f[64];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float sg = f_from_h16(q.pw[p] & 0xffffu);
      const float mu = f_from_h16(q.pw[p] >> 16);
      // rows of tokens past the end hold finite filler that is never stored
      uint32_t cm[8];                              // BITS dwords of codes, 8 / BITS masks each
      code_masks<BITS>(q.w[p], BITS, cm);
#pragma unroll
      for (int i = 0; i < 32; ++i) zw[i * RP + lane] = __builtin_fmaf(code_of<BITS>(cm, i), sg, mu);
      wave_sync();
      if (hf == p) {
        const float* rrow = zw + v * RP;
#pragma unroll
        for (int s4 = 0; s4 < 16; ++s4) {
          const float4 x = *(const float4*)(rrow + 4 * s4);
          f[4 * s4] = x.x; f[4 * s4 + 1] = x.y; f[4 * s4 + 2] = x.z; f[4 * s4 + 3] = x.w;
        }
      }
      wave_sync();
    }
    fwht64_inreg(f);
    fwht_cross(f);
    normalize64(f, cc);
    uint16_t* dst = out + (((int64_t)l * T + t0) * H + h) * kHeadDim;
    stage_out<BF16>(f, stg, sm, make_rsrc(dst, nvw ? (uint32_t)(nvw - 1) * vstride + 256u : 0u), vstride);
  }
}

// ------------------------------------------------------------------ launch

static int grid_for(int64_t blocks_needed, int cap) {
  return (int)std::max<int64_t>(1, std::min<int64_t>(blocks_needed, (int64_t)cap));
}

// -------------------------------------------------------------------
// Token delta (KVServe Sec. 5.1 lists Delta, after CacheGen, among the
// transforms applied before quantization).  In each (layer, head) the tokens
// form runs of `run` (a power of two) from token 0; a run's first token is
// kept, every other token is replaced by its binary32 difference from it,
// rounded to the 16-bit type (forward), and decoding adds the anchor back the
// same way (inverse, in place: anchors are never written there).  A thread
// takes 8 channels (16 bytes) of one head over 32 consecutive tokens; threads
// of a wave cover consecutive 16-byte slots of a token, so every step of the
// token loop is a contiguous 1 KiB access per wave.  Memory-bound: forward
// reads 2 bytes and writes 2 per value, inverse reads 2 and writes 2 per
// non-anchor value (anchors come from cache).
// -------------------------------------------------------------------
template <bool BF16, bool FWD>
__global__ __launch_bounds__(256) void k_delta(const uint16_t* x, uint16_t* y, int L, int T, int H, int run) {
  const int64_t slots = (int64_t)H * 16;             // 16-byte slots per token
  const int64_t nblk = (T + 31) / 32;
  const int64_t total = (int64_t)L * nblk * slots;
  const int64_t vec = slots * 8;                     // values per token
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t slot = i % slots;
    const int64_t r = i / slots;
    const int64_t l = r / nblk;
    const int t0 = (int)(r - l * nblk) * 32;
    const int t1 = std::min(T, t0 + 32);
    const int64_t base = l * (int64_t)T * vec + slot * 8;
    uint4 anc = make_uint4(0, 0, 0, 0);
    int acur = -1;
    for (int t = t0; t < t1; ++t) {
      const int a = t & ~(run - 1);
      const uint4 v = *(const uint4*)(x + base + (int64_t)t * vec);
      if (a == t) {
        anc = v;
        acur = a;
        if constexpr (FWD) *(uint4*)(y + base + (int64_t)t * vec) = v;
        continue;
      }
      if (a != acur) {
        anc = *(const uint4*)(x + base + (int64_t)a * vec);
        acur = a;
      }
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w}, aw[4] = {anc.x, anc.y, anc.z, anc.w};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float v0, v1, a0, a1;
        unpack16<BF16>(vw[k], v0, v1);
        unpack16<BF16>(aw[k], a0, a1);
        o[k] = FWD ? pack16<BF16>(v0 - a0, v1 - a1) : pack16<BF16>(v0 + a0, v1 + a1);
      }
      *(uint4*)(y + base + (int64_t)t * vec) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_delta(const CallDesc& c, int which, int T, bool forward, const void* x, void* y, hipStream_t s) {
  const int run = c.pol[which].delta;
  const int64_t threads = (int64_t)c.layers * ((T + 31) / 32) * c.heads * 16;
  const int grid = grid_for((threads + 255) / 256, 256 * 64);
  const uint16_t* xi = (const uint16_t*)x;
  uint16_t* yo = (uint16_t*)y;
  if (c.dtype == 1) {
    if (forward) k_delta<true, true><<<grid, 256, 0, s>>>(xi, yo, c.layers, T, c.heads, run);
    else k_delta<true, false><<<grid, 256, 0, s>>>(xi, yo, c.layers, T, c.heads, run);
  } else {
    if (forward) k_delta<false, true><<<grid, 256, 0, s>>>(xi, yo, c.layers, T, c.heads, run);
    else k_delta<false, false><<<grid, 256, 0, s>>>(xi, yo, c.layers, T, c.heads, run);
  }
  return hipGetLastError();
}

#define KVC_TOKEN_CASES_P(KERNEL, BITS, BF, PG)                                    \
  switch (pol.group) {                                                             \
    case 16: KERNEL<BITS, 16, BF, PG><<<grid, block, 0, s>>>(c, which); break;    \
    case 32: KERNEL<BITS, 32, BF, PG><<<grid, block, 0, s>>>(c, which); break;    \
    case 64: KERNEL<BITS, 64, BF, PG><<<grid, block, 0, s>>>(c, which); break;    \
    default: KERNEL<BITS, 128, BF, PG><<<grid, block, 0, s>>>(c, which); break;   \
  }
#define KVC_TOKEN_CASES(KERNEL, BITS, BF)                                          \
  if (c.page_tokens) { KVC_TOKEN_CASES_P(KERNEL, BITS, BF, true) }                 \
  else { KVC_TOKEN_CASES_P(KERNEL, BITS, BF, false) }
#define KVC_ENC_CHANNEL_CASES(BF, BITS, TAIL)                                      \
  switch (pol.group) {                                                             \
    case 32: k_encode_channel<BITS, 32, BF, TAIL><<<grid, block, 0, s>>>(c, which); break; \
    default: k_encode_channel<BITS, 64, BF, TAIL><<<grid, block, 0, s>>>(c, which); break; \
  }
#define KVC_CHANNEL_CASES(KERNEL, BITS, BF)                                        \
  switch (pol.group) {                                                             \
    case 32: KERNEL<BITS, 32, BF><<<grid, block, 0, s>>>(c, which); break;        \
    default: KERNEL<BITS, 64, BF><<<grid, block, 0, s>>>(c, which); break;        \
  }
#define KVC_BITS_CASES(CASES, KERNEL, BF)                                          \
  switch (pol.bits) {                                                              \
    case 2: CASES(KERNEL, 2, BF) break;                                            \
    case 4: CASES(KERNEL, 4, BF) break;                                            \
    default: CASES(KERNEL, 8, BF) break;                                           \
  }

hipError_t launch_encode_fused(const CallDesc& c, int which, hipStream_t s) {
  const TensorPol& pol = which ? c.pol[1] : c.pol[0];
  const int64_t tiles = which ? c.tiles[1] : c.tiles[0];
  if (tiles == 0) return hipSuccess;
  if (pol.axis == 0) {
    const dim3 block(256);
    const int grid = grid_for((tiles + 4 * KVC_ET_MIN_TILES - 1) / (4 * KVC_ET_MIN_TILES), KVC_ET_BLOCKS);
    if (c.dtype == 1) { KVC_BITS_CASES(KVC_TOKEN_CASES, k_encode_token, true) }
    else { KVC_BITS_CASES(KVC_TOKEN_CASES, k_encode_token, false) }
  } else {
    const dim3 block(128);
    const int T = c.one.T;
    const int64_t units = c.mixed ? (int64_t)c.nslabs : (int64_t)c.layers * c.heads;   // (layer, head) pairs
    if (T >= 64) {
      const int grid = grid_for(units * (T / 64), KVC_EK_BLOCKS);
      if (c.dtype == 1) { KVC_BITS_CASES(KVC_ENC_CHANNEL_CASES, true, false) }
      else { KVC_BITS_CASES(KVC_ENC_CHANNEL_CASES, false, false) }
    }
    if (T % 64) {
      const int grid = grid_for(units, 256 * 32);
      if (c.dtype == 1) { KVC_BITS_CASES(KVC_ENC_CHANNEL_CASES, true, true) }
      else { KVC_BITS_CASES(KVC_ENC_CHANNEL_CASES, false, true) }
    }
  }
  return hipGetLastError();
}

// 16-bit passthrough slabs: slab i of the launch holds the T x head_dim values
// of its (layer, head) in token order; one 16-byte piece per thread.
__global__ __launch_bounds__(256) void k_slab_copy(CallDesc c, int which, int encode) {
  const int T = c.one.T, H = c.heads;
  const int64_t per = (int64_t)T * 16;                     // 16-byte pieces per slab
  const int64_t n = (int64_t)c.nslabs * per;
  uint8_t* sec = c.codes + pick(which, c.one.codes_off);
  uint16_t* x = (uint16_t*)(encode ? const_cast<void*>(c.in_kv[which]) : c.out_kv[which]);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int sl = (int)(i / per);
    const int64_t r = i - (int64_t)sl * per;
    const int64_t t = r >> 4;
    const int q = (int)(r & 15);
    const SlabDesc sd = c.slabs[sl];
    uint4* a = (uint4*)(sec + sd.codes_off) + r;
    uint4* b = (uint4*)(x + (((int64_t)sd.l * T + t) * H + sd.h) * kHeadDim) + q;
    if (encode) *a = *b;
    else *b = *a;
  }
}

hipError_t launch_slab_copy(const CallDesc& c, int which, bool encode, hipStream_t s) {
  const int64_t n = (int64_t)c.nslabs * c.one.T * 16;
  if (n == 0) return hipSuccess;
  k_slab_copy<<<grid_for((n + 255) / 256, 256 * 32), 256, 0, s>>>(c, which, encode ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_decode_fused(const CallDesc& c, int which, hipStream_t s) {
  const TensorPol& pol = which ? c.pol[1] : c.pol[0];
  const int64_t tiles = which ? c.tiles[1] : c.tiles[0];
  if (tiles == 0) return hipSuccess;
  if (pol.axis == 0) {
    const dim3 block(256);
    const int grid = grid_for((tiles + 4 * KVC_DT_MIN_TILES - 1) / (4 * KVC_DT_MIN_TILES), KVC_DT_BLOCKS);
    if (c.mirror[which] && pol.bits == 2 && c.page_tokens == 0) {
#define KVC_TOKEN_M_CASES(BF)                                                       \
  switch (pol.group) {                                                              \
    case 16: k_decode_token_m<16, BF><<<grid, block, 0, s>>>(c, which); break;      \
    case 32: k_decode_token_m<32, BF><<<grid, block, 0, s>>>(c, which); break;      \
    case 64: k_decode_token_m<64, BF><<<grid, block, 0, s>>>(c, which); break;      \
    default: k_decode_token_m<128, BF><<<grid, block, 0, s>>>(c, which); break;     \
  }
      if (c.dtype == 1) { KVC_TOKEN_M_CASES(true) }
      else { KVC_TOKEN_M_CASES(false) }
#undef KVC_TOKEN_M_CASES
    } else if (c.dtype == 1) { KVC_BITS_CASES(KVC_TOKEN_CASES, k_decode_token, true) }
    else { KVC_BITS_CASES(KVC_TOKEN_CASES, k_decode_token, false) }
  } else {
    const dim3 block(256);
    const int grid = grid_for((2 * tiles + 4 * KVC_DC_MIN_TILES - 1) / (4 * KVC_DC_MIN_TILES), KVC_DC_BLOCKS);
    if (c.dtype == 1) { KVC_BITS_CASES(KVC_CHANNEL_CASES, k_decode_channel, true) }
    else { KVC_BITS_CASES(KVC_CHANNEL_CASES, k_decode_channel, false) }
  }
  return hipGetLastError();
}

}  // namespace kvc
