// 64x64 bit-matrix transpose across a wavefront (gfx950) and the RZE_2
// nibble helpers, shared by the word-parallel lossless kernels and the
// reconstruct kernels that decode TUPL8_1 -> BIT_8 -> RZE_2 chunks
// themselves.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

__device__ __forceinline__ uint32_t rotr32(uint32_t x, uint32_t s) { return __builtin_amdgcn_alignbit(x, x, s); }
// (m & a) | (~m & b) in one instruction: v_bitop3_b32's table is indexed by
// (m << 2) | (a << 1) | b, and 0xCA is "m ? a : b"
__device__ __forceinline__ uint32_t bfi32(uint32_t m, uint32_t a, uint32_t b) {
  return __builtin_amdgcn_bitop3_b32(m, a, b, 0xCA);
}

// Lane constants of the 64x64 bit transpose.  The rounds exchanging with
// lane ^ 16 and lane ^ 8 move whole bytes, so each is one v_perm_b32 of the
// lane's word and its partner's (sel16, sel8); the rounds with lane ^ 4, ^ 2
// and ^ 1 keep the bits mk[r] and rotate the partner's by sh[r].
struct XposeLane {
  uint32_t sel16, sel8;
  uint32_t mk[3];
  uint32_t sh[3];
};
// v_perm_b32 selectors of a byte-moving round, the partner's word being the
// high operand (bytes 4..7): lane ^ 16 (lower lanes keep their two low bytes
// and take the partner's two low ones above them; upper lanes the mirror
// image) and lane ^ 8 (the same with bytes 0, 2 and 1, 3)
__device__ __forceinline__ uint32_t xpose_sel16(int lane) { return (lane & 16) ? 0x03020706u : 0x05040100u; }
__device__ __forceinline__ uint32_t xpose_sel8(int lane) { return (lane & 8) ? 0x03070105u : 0x06020400u; }
__device__ __forceinline__ XposeLane xpose_lane() {
  XposeLane x;
  const int lane = __lane_id();
  x.sel16 = xpose_sel16(lane);
  x.sel8 = xpose_sel8(lane);
  const uint32_t m[3] = {0x0F0F0F0Fu, 0x33333333u, 0x55555555u};
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int j = 4 >> r;
    const bool lower = (lane & j) == 0;
    x.mk[r] = lower ? m[r] : ~m[r];
    x.sh[r] = lower ? (uint32_t)(32 - j) : (uint32_t)j;
  }
  return x;
}
// partner values: lane ^ 16 and lane ^ 4 through the swizzle unit, lane ^ 8
// (rotate a 16-lane row by 8), lane ^ 2 and lane ^ 1 (quad permutes) by DPP.
// Every source lane of these DPP patterns lies in the wave, so no old value
// is needed (bound_ctrl: an inactive source would read 0).
__device__ __forceinline__ uint32_t xchg16(uint32_t v) { return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F); }
__device__ __forceinline__ uint32_t xchg8(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true); }
__device__ __forceinline__ uint32_t xchg4(uint32_t v) { return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F); }
__device__ __forceinline__ uint32_t xchg2(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true); }
__device__ __forceinline__ uint32_t xchg1(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true); }

// Lane i holds row i of a 64x64 bit matrix (lo: bits 0..31, hi: 32..63);
// afterwards lane c holds column c.  Each round swaps the off-diagonal
// blocks of one bit of the row and column index.
__device__ __forceinline__ void xpose64(uint32_t& lo, uint32_t& hi, const XposeLane& X) {
  {
    auto p = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
    lo = p[0];
    hi = p[1];
  }
  uint32_t a, b;
  a = xchg16(lo); b = xchg16(hi);
  lo = __builtin_amdgcn_perm(a, lo, X.sel16); hi = __builtin_amdgcn_perm(b, hi, X.sel16);
  a = xchg8(lo); b = xchg8(hi);
  lo = __builtin_amdgcn_perm(a, lo, X.sel8); hi = __builtin_amdgcn_perm(b, hi, X.sel8);
  a = xchg4(lo); b = xchg4(hi);
  lo = bfi32(X.mk[0], lo, rotr32(a, X.sh[0])); hi = bfi32(X.mk[0], hi, rotr32(b, X.sh[0]));
  a = xchg2(lo); b = xchg2(hi);
  lo = bfi32(X.mk[1], lo, rotr32(a, X.sh[1])); hi = bfi32(X.mk[1], hi, rotr32(b, X.sh[1]));
  a = xchg1(lo); b = xchg1(hi);
  lo = bfi32(X.mk[2], lo, rotr32(a, X.sh[2])); hi = bfi32(X.mk[2], hi, rotr32(b, X.sh[2]));
}

// N transposes at once, round by round, so that each round's exchanges
// (swizzles with their LDS latency, DPP moves with their wait states) are
// issued together
template <int N>
__device__ __forceinline__ void xpose64_n(uint32_t* lo, uint32_t* hi, const XposeLane& X) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    auto p = __builtin_amdgcn_permlane32_swap(lo[i], hi[i], false, false);
    lo[i] = p[0];
    hi[i] = p[1];
  }
  uint32_t a[N], b[N];
#define KVC_XN_EXCHANGE(XCHG)                                                   \
  _Pragma("unroll") for (int i = 0; i < N; ++i) { a[i] = XCHG(lo[i]); b[i] = XCHG(hi[i]); }
  KVC_XN_EXCHANGE(xchg16)
#pragma unroll
  for (int i = 0; i < N; ++i) {
    lo[i] = __builtin_amdgcn_perm(a[i], lo[i], X.sel16); hi[i] = __builtin_amdgcn_perm(b[i], hi[i], X.sel16);
  }
  KVC_XN_EXCHANGE(xchg8)
#pragma unroll
  for (int i = 0; i < N; ++i) {
    lo[i] = __builtin_amdgcn_perm(a[i], lo[i], X.sel8); hi[i] = __builtin_amdgcn_perm(b[i], hi[i], X.sel8);
  }
#define KVC_XN_BITS(XCHG, R)                                                     \
  KVC_XN_EXCHANGE(XCHG)                                                          \
  _Pragma("unroll") for (int i = 0; i < N; ++i) {                                \
    lo[i] = bfi32(X.mk[R], lo[i], rotr32(a[i], X.sh[R]));                        \
    hi[i] = bfi32(X.mk[R], hi[i], rotr32(b[i], X.sh[R]));                        \
  }
  KVC_XN_BITS(xchg4, 0)
  KVC_XN_BITS(xchg2, 1)
  KVC_XN_BITS(xchg1, 2)
#undef KVC_XN_BITS
#undef KVC_XN_EXCHANGE
}

// xpose64 with the lane constants derived in place (for kernels with no
// registers to spare for XposeLane)
__device__ __forceinline__ void xpose64_lean(uint32_t& lo, uint32_t& hi) {
  {
    auto p = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
    lo = p[0];
    hi = p[1];
  }
  // opaque: the constants below are derived at each use, not hoisted out of
  // the caller's loop into registers
  uint32_t lane = (uint32_t)__lane_id();
  asm volatile("" : "+v"(lane));
  uint32_t a, b, mk, sh, sel;
  sel = xpose_sel16((int)lane);
  a = xchg16(lo); b = xchg16(hi);
  lo = __builtin_amdgcn_perm(a, lo, sel); hi = __builtin_amdgcn_perm(b, hi, sel);
  sel = xpose_sel8((int)lane);
  a = xchg8(lo); b = xchg8(hi);
  lo = __builtin_amdgcn_perm(a, lo, sel); hi = __builtin_amdgcn_perm(b, hi, sel);
#define KVC_XROUND(J, M, XCHG)                                            \
  mk = (lane & (J)) ? ~(uint32_t)(M) : (uint32_t)(M);                     \
  sh = (lane & (J)) ? (uint32_t)(J) : (uint32_t)(32 - (J));               \
  a = XCHG(lo); b = XCHG(hi);                                             \
  lo = bfi32(mk, lo, rotr32(a, sh)); hi = bfi32(mk, hi, rotr32(b, sh));
  KVC_XROUND(4, 0x0F0F0F0Fu, xchg4)
  KVC_XROUND(2, 0x33333333u, xchg2)
  KVC_XROUND(1, 0x55555555u, xchg1)
#undef KVC_XROUND
}

// ---- RZE_2 nibbles (4 words of 16 bits under 4 bits of the bitmap)

// (1, 1) as two 16-bit halves, opaque to the compiler: min(x, one) on the
// halves stays one v_pk_min_u16 instead of becoming compares and selects
typedef unsigned short rze_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ rze_u16x2 opaque_one2() {
  uint32_t w = 0x00010001u;
  asm volatile("" : "+v"(w));
  return __builtin_bit_cast(rze_u16x2, w);
}
// per 16-bit half of x: 1 if non-zero, else 0
__device__ __forceinline__ uint32_t nz_halves(uint32_t x, rze_u16x2 one2) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(rze_u16x2, x), one2));
}
// bit q: 16-bit word q of (lo, hi) is non-zero
__device__ __forceinline__ uint32_t nz_quarters(uint32_t lo, uint32_t hi, rze_u16x2 one2) {
  const uint32_t q = nz_halves(lo, one2) | (nz_halves(hi, one2) << 2);   // bits 0, 2, 16, 18
  return (q | (q >> 15)) & 15u;
}

// RZE_2 expansion of a nibble of the bitmap (4 words): the nibble's non-zero
// words lie consecutively in the stream; entry `nib` of this table holds the
// v_perm_b32 selectors that place them (from the 8 bytes starting at the
// first one) into words 0, 1 (.x) and 2, 3 (.y), zero bytes elsewhere, and
// the words that must be non-zero, as a 1 per 16-bit half (.z, .w).
__device__ __forceinline__ uint4 rze_nibble_entry(uint32_t nib) {
  uint32_t sel[2] = {0, 0}, ex[2] = {0, 0}, k = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bool present = (nib >> u) & 1u;
    const uint32_t half = present ? ((2u * k) | ((2u * k + 1u) << 8)) : 0x0C0Cu;   // 0x0C: a zero byte
    sel[u >> 1] |= half << (16 * (u & 1));
    ex[u >> 1] |= (present ? 1u : 0u) << (16 * (u & 1));
    k += present ? 1u : 0u;
  }
  return make_uint4(sel[0], sel[1], ex[0], ex[1]);
}

// RZE_2 compaction of a nibble: the v_perm_b32 selectors that gather its
// non-zero words (of the 8 bytes lo, hi) to the front, words 0, 1 (.x) and
// 2, 3 (.y), in order; the rest is don't-care.
__device__ __forceinline__ uint2 rze_compact_entry(uint32_t nib) {
  uint32_t sel[2] = {0x0C0C0C0Cu, 0x0C0C0C0Cu}, k = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if ((nib >> u) & 1u) {
      const uint32_t half = (2u * u) | ((2u * u + 1u) << 8);
      sel[k >> 1] = (sel[k >> 1] & ~(0xFFFFu << (16 * (k & 1)))) | (half << (16 * (k & 1)));
      ++k;
    }
  }
  return make_uint2(sel[0], sel[1]);
}

}  // namespace kvc
