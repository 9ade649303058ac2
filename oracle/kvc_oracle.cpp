/*
 * kvc_oracle.cpp -- plain, slow, single-threaded CPU reference of the
 * KV-cache compression path.  TEST INFRASTRUCTURE ONLY (see kvc_oracle.h).
 *
 * Build: g++ -std=c++17 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * fp-contract must stay off: every fp32 operation below is meant to round on
 * its own; the single place an fused multiply-add is meant, fmaf() is called.
 *
 * Method (FastKVComp, "Beyond Compression Ratio: High-Throughput KV Compression
 * for Disaggregated LLM Serving", Sec. 4.1 and 4.2; pipeline abstraction
 * BS = C(Q(T(X))) from "KVServe", Sec. 5.1):
 *   T  deterministic randomized Hadamard over head_dim (signs from a seed),
 *   Q  asymmetric min-max quantization to 2/4/8 bits; keys may be grouped per
 *      channel (groups of tokens), values per token (groups of channels),
 *   C  chunked lossless backend composed of tuple reordering (TUPL), bit
 *      shuffling (BIT), word differencing (DIFF) and zero elimination (RZE).
 * Decoding is the mirror image: lossless decode, dequantization, inverse
 * Hadamard, normalization, sign restoration (FastKVComp Sec. 4.1, "Fused
 * Reconstruction").
 */
#include "kvc_oracle.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

/* ======================================================================
 * Scalar number formats
 * ====================================================================== */

static uint32_t f2u(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

/* IEEE binary16 -> binary32, exact (normals, subnormals, inf, NaN). */
extern "C" float kvco_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h >> 15) & 1u;
  int exp = (h >> 10) & 0x1f;
  uint32_t man = h & 0x3ffu;
  double mag;
  if (exp == 0) {
    mag = std::ldexp((double)man, -24);                 /* subnormal: man * 2^-24 */
  } else if (exp == 31) {
    if (man == 0) return sign ? -INFINITY : INFINITY;
    return u2f((sign << 31) | 0x7fc00000u | (man << 13));
  } else {
    mag = std::ldexp((double)(1024 + man), exp - 25);   /* (1.man) * 2^(exp-15) */
  }
  float f = (float)mag;                                  /* exact: 11 significant bits */
  return sign ? -f : f;
}

/* binary32 -> binary16, round to nearest, ties to even (IEEE 754 default
 * rounding), done on the bit fields.  The binary32 value is
 * (1.M) * 2^(E-127) for 0 < E < 255; binary16 normals have exponent field
 * E - 112 in [1, 30] and keep the top 10 of M's 23 bits, subnormals are
 * integer multiples of 2^-24.  Rounding looks at the dropped bits: above half
 * of the kept unit rounds up, exactly half rounds to the even neighbour.  A
 * carry out of the mantissa moves to the next exponent (or from the largest
 * subnormal to the smallest normal), which is what the bit layout gives. */
extern "C" uint16_t kvco_f32_to_f16_rn(float f) {
  const uint32_t u = f2u(f);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t E = (u >> 23) & 0xffu, M = u & 0x7fffffu;
  if (E == 0xffu && M != 0) return (uint16_t)(sign | 0x7e00u);            /* NaN -> quiet NaN */
  /* |f| >= 65520 = 65504 + half an ulp rounds to infinity (the tie goes to the
   * even neighbour 65536, which does not exist as a finite fp16) */
  if ((u & 0x7fffffffu) >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);
  if (E >= 113) {                                   /* binary16 normal range */
    uint32_t h = ((E - 112) << 10) | (M >> 13);
    const uint32_t rem = M & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;
    return (uint16_t)(sign | h);
  }
  /* subnormal (or zero) result: n = |f| / 2^-24 = (1.M) * 2^(E - 103), an
   * integer part of (2^23 + M) >> s with s = 126 - E, rounded */
  if (E < 102) return sign;                         /* |f| < 2^-25: below half the smallest subnormal */
  const uint32_t mant = M | 0x800000u;
  const uint32_t s = 126 - E;                       /* 14 .. 24 */
  uint32_t n = mant >> s;
  const uint32_t rem = mant & ((1u << s) - 1u), half = 1u << (s - 1);
  if (rem > half || (rem == half && (n & 1u))) n += 1;
  return (uint16_t)(sign | n);
}

/* next representable fp16 toward +inf / -inf */
static uint16_t f16_next_up(uint16_t h) {
  if (h == 0x7c00) return h;
  if (h == 0x8000) return 0x0001;
  if (h & 0x8000) return (uint16_t)(h - 1);
  return (uint16_t)(h + 1);
}
static uint16_t f16_next_down(uint16_t h) {
  if (h == 0xfc00) return h;
  if (h == 0x0000) return 0x8001;
  if (h & 0x8000) return (uint16_t)(h + 1);
  return (uint16_t)(h - 1);
}

/* largest fp16 <= f */
extern "C" uint16_t kvco_f32_to_f16_rd(float f) {
  uint16_t h = kvco_f32_to_f16_rn(f);
  if (std::isnan(f)) return h;
  if ((double)kvco_f16_to_f32(h) > (double)f) h = f16_next_down(h);
  return h;
}
/* smallest fp16 >= f */
extern "C" uint16_t kvco_f32_to_f16_ru(float f) {
  uint16_t h = kvco_f32_to_f16_rn(f);
  if (std::isnan(f)) return h;
  if ((double)kvco_f16_to_f32(h) < (double)f) h = f16_next_up(h);
  return h;
}

extern "C" float kvco_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even (on the exact value). */
extern "C" uint16_t kvco_f32_to_bf16_rn(float f) {
  uint32_t u = f2u(f);
  if (std::isnan(f)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lower = u & 0xffffu;
  uint32_t upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;  /* carries into exponent correctly */
  return (uint16_t)upper;
}

static float load16(uint16_t bits, int dtype) {
  return dtype == 0 ? kvco_f16_to_f32(bits) : kvco_bf16_to_f32(bits);
}
static uint16_t store16(float f, int dtype) {
  return dtype == 0 ? kvco_f32_to_f16_rn(f) : kvco_f32_to_bf16_rn(f);
}

/* Directed rounding of exact real values to binary32.
 * A product of two binary32 values is exact in binary64, so it is formed
 * there and then rounded in the wanted direction. */
static float rd32_mul(float a, float b) {
  double p = (double)a * (double)b;
  float f = (float)p;
  if ((double)f > p) f = std::nextafter(f, -INFINITY);
  return f;
}
static float ru32_mul(float a, float b) {
  double p = (double)a * (double)b;
  float f = (float)p;
  if ((double)f < p) f = std::nextafter(f, INFINITY);
  return f;
}
/* Smallest binary32 >= a + b (exact real sum).  The binary64 sum s plus the
 * TwoSum error term e equals a + b exactly. */
static float ru32_add(float a, float b) {
  double s = (double)a + (double)b;
  double bb = s - (double)a;
  double e = ((double)a - (s - bb)) + ((double)b - bb);
  float f = (float)s;
  if ((double)f < s || ((double)f == s && e > 0)) f = std::nextafter(f, INFINITY);
  return f;
}
/* Smallest binary32 f with f * k >= r (k a small positive integer). */
static float ru32_div_int(float r, int k) {
  float f = (float)((double)r / (double)k);
  while ((double)f * k < (double)r) f = std::nextafter(f, INFINITY);
  for (;;) {
    float p = std::nextafter(f, -INFINITY);
    if ((double)p * k >= (double)r) f = p; else break;
  }
  return f;
}

/* ======================================================================
 * T: deterministic randomized Hadamard
 * ====================================================================== */

/* splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014; Vigna's public-domain formulation): the state
 * advances by the golden-ratio increment and the output is the mixed state. */
extern "C" uint64_t kvco_splitmix64(uint64_t* state) {
  *state += 0x9E3779B97F4A7C15ull;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Sign vector d in {+1,-1}^n.  The pages describe the rotation as a Hadamard
 * transform randomized by signs that are fixed (deterministic) and cached for
 * reuse over layers and requests (FastKVComp Sec. 4.1), but not how the signs
 * are drawn.  Reading: one vector per stream,
 * shared by K, V, every layer and head; d_i = -1 iff the top bit of the i-th
 * splitmix64 output (state started at the seed) is set. */
extern "C" int kvco_signs(uint64_t seed, int n, int8_t* out) {
  if (n <= 0 || !out) return KVCO_ERR_INVALID_ARG;
  uint64_t st = seed;
  for (int i = 0; i < n; ++i) out[i] = (kvco_splitmix64(&st) >> 63) ? -1 : 1;
  return KVCO_OK;
}

/* Orthonormal scale c = 1/sqrt(n), rounded once to binary32. */
extern "C" float kvco_norm_const(int n) { return (float)(1.0 / std::sqrt((double)n)); }

/* Unnormalized fast Walsh-Hadamard transform in Sylvester (natural) order,
 * binary32, in place.  Stage order is fixed: pair distance h = 1, 2, 4, ...,
 * n/2; each butterfly (a, b) -> (a + b, a - b) rounds each result once.
 * Reading: the pages name the Hadamard transform (KVServe Sec. 5.1 cites
 * QuaRot's rotation) but not its ordering or evaluation order; the Sylvester
 * order and this stage order are ours and fix every rounding. */
extern "C" int kvco_fwht(float* v, int n) {
  if (!v || n < 1 || (n & (n - 1))) return KVCO_ERR_INVALID_ARG;
  for (int h = 1; h < n; h *= 2) {
    for (int j = 0; j < n; j += 2 * h) {
      for (int k = j; k < j + h; ++k) {
        float a = v[k], b = v[k + h];
        v[k] = a + b;
        v[k + h] = a - b;
      }
    }
  }
  return KVCO_OK;
}

/* ======================================================================
 * Q: asymmetric min-max quantization
 * ====================================================================== */

/* Parameters of one group of unnormalized transform outputs z (the normalized
 * values are y = c * z).  The pages keep KVServe's min-max rule unchanged
 * (FastKVComp Sec. 4.1) without giving its arithmetic.  Readings:
 *  - two 16-bit parameters per group (scale s, minimum m): the only metadata
 *    size consistent with KIVI's ~5.33x ceiling at 2 bits quoted in KVServe
 *    Sec. 7.3 (16 / (2 + 32/32) = 5.33);
 *  - both stored as fp16 and rounded outward so the grid [m, m + (2^b-1) s]
 *    covers [c*min z, c*max z] exactly:
 *       lo = RD32(c * min z),  hi = RU32(c * max z),
 *       m  = RD16(lo),
 *       s  = RU16( RU32( RU32(hi - m) / (2^b - 1) ) ),
 *       inv = 1/s rounded to nearest binary32 (0 when s == 0).
 * Returns KVCO_ERR_RANGE when m or s is not a finite fp16, and when any z is
 * infinite or NaN (the pages define no codes for such values; with the
 * Hadamard on, one non-finite input value makes every transform output of
 * its head vector non-finite, so every group it reaches reports it). */
extern "C" int kvco_group_params(const float* z, int count, int bits, float c,
                                 uint16_t* s_out, uint16_t* m_out, float* inv_out) {
  if (!z || count < 1 || !(bits == 2 || bits == 4 || bits == 8)) return KVCO_ERR_INVALID_ARG;
  float zmin = z[0], zmax = z[0];
  bool nonfinite = false;
  for (int i = 0; i < count; ++i) {
    if (!std::isfinite(z[i])) nonfinite = true;
    if (z[i] < zmin) zmin = z[i];
    if (z[i] > zmax) zmax = z[i];
  }
  /* -0 and +0 are one real value; the group extremes use +0 for it */
  if (zmin == 0.0f) zmin = 0.0f;
  if (zmax == 0.0f) zmax = 0.0f;
  const int levels = (1 << bits) - 1;
  float lo = rd32_mul(zmin, c);
  float hi = ru32_mul(zmax, c);
  uint16_t m = kvco_f32_to_f16_rd(lo);
  float mf = kvco_f16_to_f32(m);
  float range = ru32_add(hi, -mf);
  float s32 = ru32_div_int(range, levels);
  uint16_t s = kvco_f32_to_f16_ru(s32);
  float sf = kvco_f16_to_f32(s);
  if (s_out) *s_out = s;
  if (m_out) *m_out = m;
  if (inv_out) *inv_out = (sf == 0.0f) ? 0.0f : 1.0f / sf;
  if (nonfinite || !std::isfinite(mf) || !std::isfinite(sf) || std::isnan(lo) || std::isnan(hi)) return KVCO_ERR_RANGE;
  return KVCO_OK;
}

/* Codes of one group: q = round-half-even( fl32(c*z - m) * inv ), where the
 * first rounding is a single fused multiply-add and the product with inv is
 * taken exactly.  Reading: the pages do not state the rounding rule; this is
 * round-to-nearest-even.  Outward-rounded parameters make 0 <= q <= 2^b - 1
 * without clamping; a value outside that range is reported as an internal
 * error so the range invariant is tested, not enforced. */
extern "C" int kvco_quantize_group(const float* z, int count, int bits, float c,
                                   uint16_t s, uint16_t m, float inv, uint8_t* codes_out) {
  if (!z || !codes_out || count < 1) return KVCO_ERR_INVALID_ARG;
  (void)s;
  const float mf = kvco_f16_to_f32(m);
  const int levels = (1 << bits) - 1;
  for (int i = 0; i < count; ++i) {
    float t = std::fmaf(z[i], c, -mf);
    double q = std::nearbyint((double)t * (double)inv);
    if (!(q >= 0.0 && q <= (double)levels)) return KVCO_ERR_INTERNAL;
    codes_out[i] = (uint8_t)q;
  }
  return KVCO_OK;
}

/* ======================================================================
 * Tensor layouts
 *   input / output:  x[l][t][h][d], 16-bit
 *   per-token axis:  groups of G consecutive channels of one (l,t,h) vector;
 *                    codes [L][T][H][D] packed along d (LSB-first);
 *                    params [L][T][H][D/G] of (s, m) fp16 pairs.
 *   per-channel axis: groups of G consecutive tokens of one (l,h,channel);
 *                    codes [L][ceil(T/G)][H][D][ceil(Gg*b/8)] packed along the
 *                    group's tokens (LSB-first), Gg = tokens in that group;
 *                    params [L][ceil(T/G)][H][D] of (s, m) fp16 pairs.
 * FastKVComp Sec. 4.1: channel-wise quantization for keys, token-wise for
 * values.  The byte layouts are this project's format.
 * ====================================================================== */

struct Pol { int bits, axis, group, had; };

static Pol policy(const kvco_cfg* cfg, int which) {
  Pol p;
  if (which == 0) { p.bits = cfg->k_bits; p.axis = cfg->k_axis; p.group = cfg->k_group; p.had = cfg->k_hadamard; }
  else { p.bits = cfg->v_bits; p.axis = cfg->v_axis; p.group = cfg->v_group; p.had = cfg->v_hadamard; }
  return p;
}

static bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
static int which_delta(const kvco_cfg* cfg, int which) { return which == 0 ? cfg->k_delta : cfg->v_delta; }

static int check_cfg(const kvco_cfg* cfg) {
  if (!cfg) return KVCO_ERR_INVALID_ARG;
  if (cfg->layers < 1 || cfg->layers > 4096 || cfg->heads < 1 || cfg->heads > 1024 ||
      !is_pow2(cfg->head_dim) || cfg->head_dim < 16 || cfg->head_dim > 256)
    return KVCO_ERR_INVALID_ARG;
  if (cfg->dtype != 0 && cfg->dtype != 1) return KVCO_ERR_INVALID_ARG;
  for (int w = 0; w < 2; ++w) {
    Pol p = policy(cfg, w);
    if (!(p.bits == 2 || p.bits == 4 || p.bits == 8)) return KVCO_ERR_INVALID_ARG;
    if (p.axis != 0 && p.axis != 1) return KVCO_ERR_INVALID_ARG;
    if (p.had != 0 && p.had != 1) return KVCO_ERR_INVALID_ARG;
    if (!is_pow2(p.group)) return KVCO_ERR_INVALID_ARG;
    if (p.axis == 0 && (p.group < 8 || p.group > cfg->head_dim)) return KVCO_ERR_INVALID_ARG;
    if (p.axis == 1 && (p.group < 16 || p.group > 256)) return KVCO_ERR_INVALID_ARG;
    const int dr = which_delta(cfg, w);
    if (dr != 0 && (!is_pow2(dr) || dr < 2 || dr > 32768)) return KVCO_ERR_INVALID_ARG;
  }
  if (cfg->chunk_bytes < 4096 || cfg->chunk_bytes > (1u << 20) || (cfg->chunk_bytes % 4096) != 0)
    return KVCO_ERR_INVALID_ARG;
  bool seen_rze = false;
  for (int i = 0; i < 4 && cfg->stages[i]; ++i) {
    int s = cfg->stages[i];
    if (s < KVCO_TUPL2_1 || s > KVCO_RZE_8) return KVCO_ERR_INVALID_ARG;
    if (seen_rze) return KVCO_ERR_UNSUPPORTED;          /* zero elimination must come last */
    if (s >= KVCO_RZE_1) seen_rze = true;
  }
  return KVCO_OK;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* bytes of packed codes for one (l, g, h, channel) column of a per-channel group */
static int64_t col_bytes(int gg, int bits) { return ceil_div((int64_t)gg * bits, 8); }

static int64_t layer_codes_bytes(const kvco_cfg* cfg, const Pol& p, int T) {
  const int64_t H = cfg->heads, D = cfg->head_dim;
  if (p.axis == 0) return (int64_t)T * H * D * p.bits / 8;
  int64_t total = 0;
  for (int g0 = 0; g0 < T; g0 += p.group) {
    int gg = (T - g0 < p.group) ? (T - g0) : p.group;
    total += H * D * col_bytes(gg, p.bits);
  }
  return total;
}

extern "C" int64_t kvco_codes_bytes(const kvco_cfg* cfg, int which, int tokens) {
  if (check_cfg(cfg) != KVCO_OK || tokens < 0) return -1;
  Pol p = policy(cfg, which);
  return (int64_t)cfg->layers * layer_codes_bytes(cfg, p, tokens);
}

extern "C" int64_t kvco_params_bytes(const kvco_cfg* cfg, int which, int tokens) {
  if (check_cfg(cfg) != KVCO_OK || tokens < 0) return -1;
  Pol p = policy(cfg, which);
  const int64_t L = cfg->layers, H = cfg->heads, D = cfg->head_dim;
  if (p.axis == 0) return L * tokens * H * (D / p.group) * 4;
  return L * ceil_div(tokens, p.group) * H * D * 4;
}

/* Forward transform of one head vector: v = d * x (binary32), z = FWHT(v). */
static void forward_vector(const uint16_t* x, int D, int dtype, const Pol& p,
                           const int8_t* signs, float* z) {
  for (int i = 0; i < D; ++i) {
    float f = load16(x[i], dtype);
    z[i] = p.had ? f * (float)signs[i] : f;
  }
  if (p.had) kvco_fwht(z, D);
}

static void put_code(uint8_t* base, int64_t index, int bits, uint8_t q) {
  int64_t bit = index * bits;
  base[bit >> 3] |= (uint8_t)(q << (bit & 7));
}
static uint8_t get_code(const uint8_t* base, int64_t index, int bits) {
  int64_t bit = index * bits;
  return (uint8_t)((base[bit >> 3] >> (bit & 7)) & ((1 << bits) - 1));
}
static void put_params(uint8_t* params, int64_t g, uint16_t s, uint16_t m) {
  params[4 * g + 0] = (uint8_t)(s & 0xff);
  params[4 * g + 1] = (uint8_t)(s >> 8);
  params[4 * g + 2] = (uint8_t)(m & 0xff);
  params[4 * g + 3] = (uint8_t)(m >> 8);
}
static void get_params(const uint8_t* params, int64_t g, uint16_t* s, uint16_t* m) {
  *s = (uint16_t)(params[4 * g] | (params[4 * g + 1] << 8));
  *m = (uint16_t)(params[4 * g + 2] | (params[4 * g + 3] << 8));
}

extern "C" int kvco_quantize_tensor(const kvco_cfg* cfg, int which, const uint16_t* x, int tokens,
                                    uint8_t* codes, uint8_t* params) {
  int st = check_cfg(cfg);
  if (st != KVCO_OK) return st;
  if (tokens < 0 || (tokens > 0 && (!x || !codes || !params))) return KVCO_ERR_INVALID_ARG;
  const Pol p = policy(cfg, which);
  const int L = cfg->layers, T = tokens, H = cfg->heads, D = cfg->head_dim;
  const int levels_bits = p.bits;
  std::vector<int8_t> signs(D);
  kvco_signs(cfg->seed, D, signs.data());
  const float c = p.had ? kvco_norm_const(D) : 1.0f;
  const int64_t ncodes = kvco_codes_bytes(cfg, which, tokens);
  if (ncodes > 0) std::memset(codes, 0, (size_t)ncodes);
  int status = KVCO_OK;
  std::vector<float> z(D);
  std::vector<uint8_t> q(256);

  if (p.axis == 0) {
    const int G = p.group, NGv = D / G;
    for (int64_t vec = 0; vec < (int64_t)L * T * H; ++vec) {
      forward_vector(x + vec * D, D, cfg->dtype, p, signs.data(), z.data());
      uint8_t* row = codes + vec * D * levels_bits / 8;
      for (int g = 0; g < NGv; ++g) {
        uint16_t s, m; float inv;
        int r = kvco_group_params(&z[g * G], G, p.bits, c, &s, &m, &inv);
        if (r == KVCO_ERR_RANGE) status = KVCO_ERR_RANGE;
        else if (r != KVCO_OK) return r;
        put_params(params, vec * NGv + g, s, m);
        int qr = kvco_quantize_group(&z[g * G], G, p.bits, c, s, m, inv, q.data());
        if (qr != KVCO_OK && r == KVCO_OK) return qr;
        for (int i = 0; i < G; ++i) put_code(row, g * G + i, p.bits, q[i]);
      }
    }
    return status;
  }

  /* per-channel: a group is G consecutive tokens of one (layer, head, channel) */
  const int G = p.group;
  const int NG = (int)ceil_div(T, G);
  std::vector<float> zt((size_t)G * D);
  std::vector<float> col(G);
  int64_t off = 0;
  for (int l = 0; l < L; ++l) {
    for (int g = 0; g < NG; ++g) {
      const int gg = (T - g * G < G) ? (T - g * G) : G;
      const int64_t cb = col_bytes(gg, p.bits);
      for (int h = 0; h < H; ++h) {
        for (int tt = 0; tt < gg; ++tt) {
          const int64_t vec = ((int64_t)l * T + (int64_t)g * G + tt) * H + h;
          forward_vector(x + vec * D, D, cfg->dtype, p, signs.data(), &zt[(size_t)tt * D]);
        }
        for (int ch = 0; ch < D; ++ch) {
          for (int tt = 0; tt < gg; ++tt) col[tt] = zt[(size_t)tt * D + ch];
          uint16_t s, m; float inv;
          int r = kvco_group_params(col.data(), gg, p.bits, c, &s, &m, &inv);
          if (r == KVCO_ERR_RANGE) status = KVCO_ERR_RANGE;
          else if (r != KVCO_OK) return r;
          const int64_t gidx = (((int64_t)l * NG + g) * H + h) * D + ch;
          put_params(params, gidx, s, m);
          int qr = kvco_quantize_group(col.data(), gg, p.bits, c, s, m, inv, q.data());
          if (qr != KVCO_OK && r == KVCO_OK) return qr;
          uint8_t* dst = codes + off + ((int64_t)h * D + ch) * cb;
          for (int tt = 0; tt < gg; ++tt) put_code(dst, tt, p.bits, q[tt]);
        }
      }
      off += (int64_t)H * D * cb;
    }
  }
  return status;
}

/* Reconstruction of one head vector from its dequantized values w (in the
 * transform domain, unnormalized grid: w = q*s + m): the inverse of the
 * orthonormal rotation c*H*diag(d) is diag(d)*c*H, applied as the pages list
 * the fused reconstruction's steps (FastKVComp Sec. 4.1, "Fused
 * Reconstruction": dequantization, inverse Hadamard transformation,
 * normalization, sign restoration): the FWHT in the same fixed stage order as
 * the forward transform, then the product with c (rounded once), then the
 * sign, then rounding to the 16-bit dtype (nearest, ties to even). */
static void inverse_vector(float* w, int D, int dtype, const Pol& p, float c, const int8_t* signs, uint16_t* out) {
  if (p.had) kvco_fwht(w, D);
  for (int i = 0; i < D; ++i) {
    float f = w[i];
    if (p.had) {
      f = f * c;                                   /* normalization */
      f = f * (float)signs[i];                     /* sign restoration (exact) */
    }
    out[i] = store16(f, dtype);
  }
}

/* Dequantization of one group's parameters: the stored fp16 scale and
 * minimum as binary32 (exact). */
static void dequant_params(const uint8_t* params, int64_t g, float* sigma, float* mu) {
  uint16_t s, m;
  get_params(params, g, &s, &m);
  *sigma = kvco_f16_to_f32(s);
  *mu = kvco_f16_to_f32(m);
}

extern "C" int kvco_dequantize_tensor(const kvco_cfg* cfg, int which, const uint8_t* codes,
                                      const uint8_t* params, int tokens, uint16_t* x) {
  int st = check_cfg(cfg);
  if (st != KVCO_OK) return st;
  if (tokens < 0 || (tokens > 0 && (!x || !codes || !params))) return KVCO_ERR_INVALID_ARG;
  const Pol p = policy(cfg, which);
  const int L = cfg->layers, T = tokens, H = cfg->heads, D = cfg->head_dim;
  std::vector<int8_t> signs(D);
  kvco_signs(cfg->seed, D, signs.data());
  const float c = p.had ? kvco_norm_const(D) : 1.0f;
  std::vector<float> w(D);

  if (p.axis == 0) {
    const int G = p.group, NGv = D / G;
    for (int64_t vec = 0; vec < (int64_t)L * T * H; ++vec) {
      const uint8_t* row = codes + vec * D * p.bits / 8;
      for (int g = 0; g < NGv; ++g) {
        float sigma, mu;
        dequant_params(params, vec * NGv + g, &sigma, &mu);
        for (int i = 0; i < G; ++i)
          w[g * G + i] = std::fmaf((float)get_code(row, g * G + i, p.bits), sigma, mu);
      }
      inverse_vector(w.data(), D, cfg->dtype, p, c, signs.data(), x + vec * D);
    }
    return KVCO_OK;
  }

  const int G = p.group;
  const int NG = (int)ceil_div(T, G);
  std::vector<float> sig(D), mus(D);
  int64_t off = 0;
  for (int l = 0; l < L; ++l) {
    for (int g = 0; g < NG; ++g) {
      const int gg = (T - g * G < G) ? (T - g * G) : G;
      const int64_t cb = col_bytes(gg, p.bits);
      for (int h = 0; h < H; ++h) {
        for (int ch = 0; ch < D; ++ch)
          dequant_params(params, (((int64_t)l * NG + g) * H + h) * D + ch, &sig[ch], &mus[ch]);
        for (int tt = 0; tt < gg; ++tt) {
          for (int ch = 0; ch < D; ++ch) {
            const uint8_t* src = codes + off + ((int64_t)h * D + ch) * cb;
            w[ch] = std::fmaf((float)get_code(src, tt, p.bits), sig[ch], mus[ch]);
          }
          const int64_t vec = ((int64_t)l * T + (int64_t)g * G + tt) * H + h;
          inverse_vector(w.data(), D, cfg->dtype, p, c, signs.data(), x + vec * D);
        }
      }
      off += (int64_t)H * D * cb;
    }
  }
  return KVCO_OK;
}

/* ======================================================================
 * C: lossless components.  FastKVComp Sec. 4.2 builds its backend from
 * composable primitives (reordering of byte tuples, shuffling of bits, and
 * elimination of zero words) and selects the pipeline TUPL8_1 -> BIT_8 ->
 * RZE_2.  The pages give names, not formats;
 * the definitions below are this project's (LC-style, not LC's formats):
 *   TUPLk_1: n bytes seen as m = floor(n/k) k-tuples of bytes; out[j*m + i] =
 *            in[i*k + j]; the n - m*k tail bytes are copied.
 *   DIFFw:   w-byte little-endian words; out[0] = in[0], out[i] = in[i] -
 *            in[i-1] mod 2^(8w); tail bytes copied.
 *   BITw:    groups of B = 8w words form a B x B bit matrix that is
 *            transposed: output word j bit i = bit j of input word i;
 *            incomplete trailing group copied.
 *   RZEw:    bitmap of ceil((n/w)/8) bytes (bit i, LSB-first, set iff word i
 *            is non-zero), then the non-zero words in order, then the tail.
 * ====================================================================== */

static int stage_kind(int s) {   /* 0 TUPL, 1 DIFF, 2 BIT, 3 RZE */
  if (s >= KVCO_TUPL2_1 && s <= KVCO_TUPL8_1) return 0;
  if (s >= KVCO_DIFF1 && s <= KVCO_DIFF8) return 1;
  if (s >= KVCO_BIT_1 && s <= KVCO_BIT_8) return 2;
  if (s >= KVCO_RZE_1 && s <= KVCO_RZE_8) return 3;
  return -1;
}
static int stage_width(int s) {
  switch (s) {
    case KVCO_TUPL2_1: return 2; case KVCO_TUPL4_1: return 4; case KVCO_TUPL8_1: return 8;
    case KVCO_DIFF1: case KVCO_BIT_1: case KVCO_RZE_1: return 1;
    case KVCO_DIFF2: case KVCO_BIT_2: case KVCO_RZE_2: return 2;
    case KVCO_DIFF4: case KVCO_BIT_4: case KVCO_RZE_4: return 4;
    case KVCO_DIFF8: case KVCO_BIT_8: case KVCO_RZE_8: return 8;
  }
  return 0;
}

static uint64_t get_word(const uint8_t* p, int w) {
  uint64_t v = 0;
  for (int b = 0; b < w; ++b) v |= (uint64_t)p[b] << (8 * b);
  return v;
}
static void put_word(uint8_t* p, int w, uint64_t v) {
  for (int b = 0; b < w; ++b) p[b] = (uint8_t)(v >> (8 * b));
}
static uint64_t word_mask(int w) { return w == 8 ? ~0ull : ((1ull << (8 * w)) - 1); }

extern "C" int kvco_stage_encode(int stage, const uint8_t* in, size_t n, uint8_t* out, size_t cap, size_t* out_n) {
  const int kind = stage_kind(stage), w = stage_width(stage);
  if (kind < 0 || !out_n || (n > 0 && (!in || !out))) return KVCO_ERR_INVALID_ARG;
  if (kind == 0) {
    if (cap < n) return KVCO_ERR_BUFFER_TOO_SMALL;
    const size_t k = (size_t)w, m = n / k;
    for (size_t i = 0; i < m; ++i)
      for (size_t j = 0; j < k; ++j) out[j * m + i] = in[i * k + j];
    for (size_t p = m * k; p < n; ++p) out[p] = in[p];
    *out_n = n;
    return KVCO_OK;
  }
  if (kind == 1) {
    if (cap < n) return KVCO_ERR_BUFFER_TOO_SMALL;
    const size_t nw = n / w;
    uint64_t prev = 0;
    for (size_t i = 0; i < nw; ++i) {
      uint64_t cur = get_word(in + i * w, w);
      put_word(out + i * w, w, (cur - prev) & word_mask(w));
      prev = cur;
    }
    for (size_t p = nw * w; p < n; ++p) out[p] = in[p];
    *out_n = n;
    return KVCO_OK;
  }
  if (kind == 2) {
    if (cap < n) return KVCO_ERR_BUFFER_TOO_SMALL;
    const int B = 8 * w;
    const size_t gbytes = (size_t)w * B, ng = n / gbytes;
    for (size_t g = 0; g < ng; ++g) {
      const uint8_t* src = in + g * gbytes;
      uint8_t* dst = out + g * gbytes;
      for (int j = 0; j < B; ++j) {
        uint64_t o = 0;
        for (int i = 0; i < B; ++i) o |= ((get_word(src + (size_t)i * w, w) >> j) & 1ull) << i;
        put_word(dst + (size_t)j * w, w, o);
      }
    }
    for (size_t p = ng * gbytes; p < n; ++p) out[p] = in[p];
    *out_n = n;
    return KVCO_OK;
  }
  /* RZE */
  const size_t nw = n / w, bm = (nw + 7) / 8, tail = n - nw * w;
  size_t nnz = 0;
  for (size_t i = 0; i < nw; ++i) if (get_word(in + i * w, w) != 0) ++nnz;
  const size_t need = bm + nnz * w + tail;
  if (cap < need) return KVCO_ERR_BUFFER_TOO_SMALL;
  std::memset(out, 0, bm);
  size_t pos = bm;
  for (size_t i = 0; i < nw; ++i) {
    uint64_t v = get_word(in + i * w, w);
    if (v != 0) {
      out[i / 8] |= (uint8_t)(1u << (i % 8));
      put_word(out + pos, w, v);
      pos += w;
    }
  }
  for (size_t p = nw * w; p < n; ++p) out[pos++] = in[p];
  *out_n = pos;
  return KVCO_OK;
}

/* Inverse of one stage; n is the decoded length (known from chunk position). */
extern "C" int kvco_stage_decode(int stage, const uint8_t* in, size_t in_n, uint8_t* out, size_t n) {
  const int kind = stage_kind(stage), w = stage_width(stage);
  if (kind < 0 || (n > 0 && !out) || (in_n > 0 && !in)) return KVCO_ERR_INVALID_ARG;
  if (kind != 3 && in_n != n) return KVCO_ERR_CORRUPT_STREAM;
  if (kind == 0) {
    const size_t k = (size_t)w, m = n / k;
    for (size_t i = 0; i < m; ++i)
      for (size_t j = 0; j < k; ++j) out[i * k + j] = in[j * m + i];
    for (size_t p = m * k; p < n; ++p) out[p] = in[p];
    return KVCO_OK;
  }
  if (kind == 1) {
    const size_t nw = n / w;
    uint64_t acc = 0;
    for (size_t i = 0; i < nw; ++i) {
      acc = (acc + get_word(in + i * w, w)) & word_mask(w);
      put_word(out + i * w, w, acc);
    }
    for (size_t p = nw * w; p < n; ++p) out[p] = in[p];
    return KVCO_OK;
  }
  if (kind == 2) {   /* a square bit transpose is its own inverse */
    size_t on = 0;
    return kvco_stage_encode(stage, in, n, out, n, &on);
  }
  const size_t nw = n / w, bm = (nw + 7) / 8, tail = n - nw * w;
  if (in_n < bm + tail) return KVCO_ERR_CORRUPT_STREAM;
  size_t nnz = 0;
  for (size_t i = 0; i < nw; ++i) if (in[i / 8] & (1u << (i % 8))) ++nnz;
  for (size_t i = nw; i < bm * 8; ++i) if (in[i / 8] & (1u << (i % 8))) return KVCO_ERR_CORRUPT_STREAM;
  if (in_n != bm + nnz * w + tail) return KVCO_ERR_CORRUPT_STREAM;
  size_t pos = bm;
  for (size_t i = 0; i < nw; ++i) {
    if (in[i / 8] & (1u << (i % 8))) {
      uint64_t v = get_word(in + pos, w);
      if (v == 0) return KVCO_ERR_CORRUPT_STREAM;      /* a flagged word must be non-zero */
      put_word(out + i * w, w, v);
      pos += w;
    } else {
      put_word(out + i * w, w, 0);
    }
  }
  for (size_t p = nw * w; p < n; ++p) out[p] = in[pos++];
  return KVCO_OK;
}

/* One chunk through the whole pipeline.  If the result is not smaller than
 * the input, the chunk is stored raw (the backend never expands data). */
extern "C" int kvco_chunk_encode(const uint8_t* stages, const uint8_t* in, size_t n,
                                 uint8_t* out, size_t* stored, int* raw) {
  if (!stages || !stored || !raw || (n > 0 && (!in || !out))) return KVCO_ERR_INVALID_ARG;
  std::vector<uint8_t> a(in, in + n), b(n + 64);
  size_t cur = n;
  for (int i = 0; i < 4 && stages[i]; ++i) {
    size_t on = 0;
    size_t cap = b.size();
    int r = kvco_stage_encode(stages[i], a.data(), cur, b.data(), cap, &on);
    if (r == KVCO_ERR_BUFFER_TOO_SMALL) { cur = n + 1; break; }   /* would expand: store raw */
    if (r != KVCO_OK) return r;
    a.assign(b.begin(), b.begin() + on);
    b.assign(n + 64, 0);
    cur = on;
  }
  if (cur >= n) {
    if (n) std::memcpy(out, in, n);
    *stored = n;
    *raw = 1;
  } else {
    std::memcpy(out, a.data(), cur);
    *stored = cur;
    *raw = 0;
  }
  return KVCO_OK;
}

extern "C" int kvco_chunk_decode(const uint8_t* stages, const uint8_t* in, size_t stored, int raw,
                                 uint8_t* out, size_t n) {
  if (!stages || (n > 0 && !out) || (stored > 0 && !in)) return KVCO_ERR_INVALID_ARG;
  if (raw) {
    if (stored != n) return KVCO_ERR_CORRUPT_STREAM;
    if (n) std::memcpy(out, in, n);
    return KVCO_OK;
  }
  int ns = 0;
  while (ns < 4 && stages[ns]) ++ns;
  if (ns == 0 || stored >= n) return KVCO_ERR_CORRUPT_STREAM;
  std::vector<uint8_t> a(in, in + stored), b(n);
  size_t cur = stored;
  for (int i = ns - 1; i >= 0; --i) {
    int r = kvco_stage_decode(stages[i], a.data(), cur, b.data(), n);
    if (r != KVCO_OK) return r;
    a = b;
    cur = n;
  }
  std::memcpy(out, a.data(), n);
  return KVCO_OK;
}

/* ======================================================================
 * Token delta.  KVServe Sec. 5.1 lists Delta (from CacheGen) among the
 * transformer modules that reshape the value distribution before
 * quantization, and names it only.  The reading taken here: in each (layer,
 * head) the tokens form runs of D consecutive tokens from token 0 (the last
 * run may be shorter); a run's first token, its anchor, is kept, and every
 * other token is replaced, channel by channel, by its difference from the
 * anchor, formed in binary32 from the two 16-bit values and rounded to the
 * tensor's 16-bit type (nearest, ties to even).  The result is quantized like
 * any input.  Decoding reverses it on the reconstructed 16-bit tensor: a
 * non-anchor value becomes the rounded binary32 sum of itself and its anchor.
 * ====================================================================== */
extern "C" int kvco_delta_forward(const kvco_cfg* cfg, int which, const uint16_t* x, int tokens, uint16_t* y) {
  if (check_cfg(cfg) != KVCO_OK || (which != 0 && which != 1) || tokens < 0) return KVCO_ERR_INVALID_ARG;
  const int64_t H = cfg->heads, D = cfg->head_dim, run = which_delta(cfg, which);
  const int64_t n = (int64_t)cfg->layers * tokens * H * D;
  if (n > 0 && (!x || !y)) return KVCO_ERR_INVALID_ARG;
  for (int l = 0; l < cfg->layers; ++l)
    for (int t = 0; t < tokens; ++t)
      for (int h = 0; h < H; ++h) {
        const int a = run ? (int)(t - t % run) : t;           /* the anchor of token t */
        const int64_t xi = (((int64_t)l * tokens + t) * H + h) * D;
        const int64_t ai = (((int64_t)l * tokens + a) * H + h) * D;
        for (int d = 0; d < D; ++d) {
          if (a == t) { y[xi + d] = x[xi + d]; continue; }
          const float diff = load16(x[xi + d], cfg->dtype) - load16(x[ai + d], cfg->dtype);
          y[xi + d] = store16(diff, cfg->dtype);
        }
      }
  return KVCO_OK;
}

extern "C" int kvco_delta_inverse(const kvco_cfg* cfg, int which, uint16_t* x, int tokens) {
  if (check_cfg(cfg) != KVCO_OK || (which != 0 && which != 1) || tokens < 0) return KVCO_ERR_INVALID_ARG;
  const int64_t H = cfg->heads, D = cfg->head_dim, run = which_delta(cfg, which);
  if (!run) return KVCO_OK;
  if ((int64_t)cfg->layers * tokens * H * D > 0 && !x) return KVCO_ERR_INVALID_ARG;
  for (int l = 0; l < cfg->layers; ++l)
    for (int t = 0; t < tokens; ++t) {
      const int a = (int)(t - t % run);
      if (a == t) continue;                                  /* anchors are stored as they are */
      for (int h = 0; h < H; ++h) {
        const int64_t xi = (((int64_t)l * tokens + t) * H + h) * D;
        const int64_t ai = (((int64_t)l * tokens + a) * H + h) * D;
        for (int d = 0; d < D; ++d)
          x[xi + d] = store16(load16(x[xi + d], cfg->dtype) + load16(x[ai + d], cfg->dtype), cfg->dtype);
      }
    }
  return KVCO_OK;
}

/* ======================================================================
 * Stream format (this project's; little-endian)
 *   [0,64)   header: magic "KVC1", u16 version 1, u8 dtype, u8 flags (bit 0:
 *            mixed precision, below; other bits 0),
 *            i32 layers, tokens, heads, head_dim,
 *            K policy {u8 bits, u8 axis, u8 hadamard, u8 0, u16 group,
 *            u16 token-delta run length (0 = none)},
 *            V policy (same), u64 seed, u8 stages[4], u32 chunk_bytes,
 *            u64 total_bytes
 *   [64, 64 + 4*nc) chunk table, K chunks then V chunks: bit 31 = stored raw,
 *            bits 0..30 = stored bytes
 *   align16: K params, align16: V params, align16: payload; chunk i starts at
 *            payload + sum over j < i of align16(stored_j); padding is zero.
 * FastKVComp Sec. 4.2 sends only the compressed size to the host during
 * encoding; total_bytes is that scalar.
 * ====================================================================== */

static const uint32_t MAGIC = 0x3143564Bu;   /* "KVC1" */
static int64_t align16(int64_t x) { return (x + 15) & ~(int64_t)15; }

struct Layout {
  int64_t codes[2], params[2], nchunks[2];
  int64_t table_off, map_off, params_off[2], payload_off, max_total;
};

/* ======================================================================
 * Mixed precision per (layer, head).  KVServe Sec. 5.1 (MixHQ, and its
 * layer-wise generalization) keeps some heads at high precision and others at
 * very low bit widths; the mechanism here takes the width of every (tensor,
 * layer, head) as input: 2, 4 or 8 bits through the quantizer, or 16 to keep
 * the head's 16-bit values unchanged.  Stream: flags bit 0 set; right after
 * the header the 2 * layers * heads widths (K then V, layer-major,
 * head-minor), then, 16-byte aligned, the chunk table; every codes and
 * parameter section is the
 * concatenation, in the same (layer, head) order, of the sections a
 * one-layer, one-head uniform stream with that head's width would hold
 * (width 16: the tokens x head_dim 16-bit values, no parameters).
 * ====================================================================== */
static kvco_cfg slab_cfg(const kvco_cfg* cfg, int which, int bits) {
  kvco_cfg s = *cfg;
  s.layers = 1;
  s.heads = 1;
  if (which == 0) s.k_bits = bits; else s.v_bits = bits;
  return s;
}

static int64_t slab_codes_bytes(const kvco_cfg* cfg, int which, int bits, int tokens) {
  if (bits == 16) return (int64_t)tokens * cfg->head_dim * 2;
  const kvco_cfg s = slab_cfg(cfg, which, bits);
  return kvco_codes_bytes(&s, which, tokens);
}

static int64_t slab_params_bytes(const kvco_cfg* cfg, int which, int bits, int tokens) {
  if (bits == 16) return 0;
  const kvco_cfg s = slab_cfg(cfg, which, bits);
  return kvco_params_bytes(&s, which, tokens);
}

static int check_bits_map(const kvco_cfg* cfg, const uint8_t* bits) {
  if (!bits) return KVCO_ERR_INVALID_ARG;
  for (int64_t i = 0; i < 2 * (int64_t)cfg->layers * cfg->heads; ++i) {
    const int b = bits[i];
    if (b != 2 && b != 4 && b != 8 && b != 16) return KVCO_ERR_INVALID_ARG;
    if (b != 16) {
      const int which = i < (int64_t)cfg->layers * cfg->heads ? 0 : 1;
      const kvco_cfg s = slab_cfg(cfg, which, b);
      if (check_cfg(&s) != KVCO_OK) return KVCO_ERR_INVALID_ARG;
    }
  }
  return KVCO_OK;
}

/* bits == NULL: uniform layout */
static Layout layout_of(const kvco_cfg* cfg, int tokens, const uint8_t* bits = nullptr) {
  Layout L;
  const int64_t LH = (int64_t)cfg->layers * cfg->heads;
  for (int w = 0; w < 2; ++w) {
    if (!bits) {
      L.codes[w] = kvco_codes_bytes(cfg, w, tokens);
      L.params[w] = kvco_params_bytes(cfg, w, tokens);
    } else {
      L.codes[w] = L.params[w] = 0;
      for (int64_t i = 0; i < LH; ++i) {
        L.codes[w] += slab_codes_bytes(cfg, w, bits[w * LH + i], tokens);
        L.params[w] += slab_params_bytes(cfg, w, bits[w * LH + i], tokens);
      }
    }
    L.nchunks[w] = ceil_div(L.codes[w], cfg->chunk_bytes);
  }
  L.map_off = 64;
  L.table_off = bits ? align16(64 + 2 * LH) : 64;
  L.params_off[0] = align16(L.table_off + 4 * (L.nchunks[0] + L.nchunks[1]));
  L.params_off[1] = align16(L.params_off[0] + L.params[0]);
  L.payload_off = align16(L.params_off[1] + L.params[1]);
  int64_t pay = 0;
  for (int w = 0; w < 2; ++w)
    for (int64_t i = 0; i < L.nchunks[w]; ++i) {
      int64_t n = L.codes[w] - i * cfg->chunk_bytes;
      if (n > cfg->chunk_bytes) n = cfg->chunk_bytes;
      pay += align16(n);
    }
  L.max_total = L.payload_off + pay;
  return L;
}

extern "C" int64_t kvco_max_stream_bytes(const kvco_cfg* cfg, int tokens) {
  if (check_cfg(cfg) != KVCO_OK || tokens < 0) return -1;
  return layout_of(cfg, tokens).max_total;
}

static void w16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void w32(uint8_t* p, uint32_t v) { for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static void w64(uint8_t* p, uint64_t v) { for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static uint16_t r16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t r32(const uint8_t* p) { uint32_t v = 0; for (int i = 0; i < 4; ++i) v |= (uint32_t)p[i] << (8 * i); return v; }
static uint64_t r64(const uint8_t* p) { uint64_t v = 0; for (int i = 0; i < 8; ++i) v |= (uint64_t)p[i] << (8 * i); return v; }

static void write_header(uint8_t* o, const kvco_cfg* cfg, int tokens, uint64_t total, int flags = 0) {
  std::memset(o, 0, 64);
  w32(o + 0, MAGIC);
  w16(o + 4, 1);
  o[6] = (uint8_t)cfg->dtype;
  o[7] = (uint8_t)flags;
  w32(o + 8, (uint32_t)cfg->layers);
  w32(o + 12, (uint32_t)tokens);
  w32(o + 16, (uint32_t)cfg->heads);
  w32(o + 20, (uint32_t)cfg->head_dim);
  for (int w = 0; w < 2; ++w) {
    Pol p = policy(cfg, w);
    uint8_t* q = o + 24 + 8 * w;
    q[0] = (uint8_t)p.bits; q[1] = (uint8_t)p.axis; q[2] = (uint8_t)p.had;
    w16(q + 4, (uint16_t)p.group);
    w16(q + 6, (uint16_t)which_delta(cfg, w));
  }
  w64(o + 40, cfg->seed);
  for (int i = 0; i < 4; ++i) o[48 + i] = cfg->stages[i];
  w32(o + 52, cfg->chunk_bytes);
  w64(o + 56, total);
}

/* Codes and parameters of one tensor of a mixed stream: each (layer, head)
 * slab is gathered into a one-layer, one-head tensor and quantized as a
 * uniform stream of its width would be, or copied for width 16. */
static int quantize_mixed(const kvco_cfg* cfg, const uint8_t* bits, int which, const uint16_t* x, int T,
                          uint8_t* codes, uint8_t* params) {
  const int H = cfg->heads, D = cfg->head_dim;
  const int64_t LH = (int64_t)cfg->layers * H;
  std::vector<uint16_t> slab((size_t)T * D);
  int status = KVCO_OK;
  int64_t co = 0, po = 0;
  for (int l = 0; l < cfg->layers; ++l)
    for (int h = 0; h < H; ++h) {
      const int b = bits[which * LH + (int64_t)l * H + h];
      for (int t = 0; t < T; ++t)
        std::memcpy(&slab[(size_t)t * D], x + (((int64_t)l * T + t) * H + h) * D, (size_t)D * 2);
      if (b == 16) {
        std::memcpy(codes + co, slab.data(), (size_t)T * D * 2);
      } else {
        const kvco_cfg sc = slab_cfg(cfg, which, b);
        const int r = kvco_quantize_tensor(&sc, which, slab.data(), T, codes + co, params + po);
        if (r == KVCO_ERR_RANGE) status = KVCO_ERR_RANGE;
        else if (r != KVCO_OK) return r;
      }
      co += slab_codes_bytes(cfg, which, b, T);
      po += slab_params_bytes(cfg, which, b, T);
    }
  return status;
}

static int dequantize_mixed(const kvco_cfg* cfg, const uint8_t* bits, int which, const uint8_t* codes,
                            const uint8_t* params, int T, uint16_t* x) {
  const int H = cfg->heads, D = cfg->head_dim;
  const int64_t LH = (int64_t)cfg->layers * H;
  std::vector<uint16_t> slab((size_t)T * D);
  int64_t co = 0, po = 0;
  for (int l = 0; l < cfg->layers; ++l)
    for (int h = 0; h < H; ++h) {
      const int b = bits[which * LH + (int64_t)l * H + h];
      if (b == 16) {
        std::memcpy(slab.data(), codes + co, (size_t)T * D * 2);
      } else {
        const kvco_cfg sc = slab_cfg(cfg, which, b);
        const int r = kvco_dequantize_tensor(&sc, which, codes + co, params + po, T, slab.data());
        if (r != KVCO_OK) return r;
      }
      for (int t = 0; t < T; ++t)
        std::memcpy(x + (((int64_t)l * T + t) * H + h) * D, &slab[(size_t)t * D], (size_t)D * 2);
      co += slab_codes_bytes(cfg, which, b, T);
      po += slab_params_bytes(cfg, which, b, T);
    }
  return KVCO_OK;
}

extern "C" int64_t kvco_max_stream_bytes_mixed(const kvco_cfg* cfg, const uint8_t* bits, int tokens) {
  if (check_cfg(cfg) != KVCO_OK || tokens < 0 || check_bits_map(cfg, bits) != KVCO_OK) return -1;
  return layout_of(cfg, tokens, bits).max_total;
}

static int encode_stream(const kvco_cfg* cfg, const uint8_t* bits, const uint16_t* k, const uint16_t* v,
                         int tokens, uint8_t* out, size_t cap, size_t* out_bytes) {
  int st = check_cfg(cfg);
  if (st != KVCO_OK) return st;
  if (tokens < 0 || !out || !out_bytes || (tokens > 0 && (!k || !v))) return KVCO_ERR_INVALID_ARG;
  if (bits && check_bits_map(cfg, bits) != KVCO_OK) return KVCO_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg, tokens, bits);
  if ((int64_t)cap < L.max_total) return KVCO_ERR_BUFFER_TOO_SMALL;
  std::memset(out, 0, (size_t)L.max_total);
  int status = KVCO_OK;
  std::vector<uint8_t> codes[2];
  std::vector<uint16_t> delta;
  for (int w = 0; w < 2; ++w) {
    codes[w].assign((size_t)L.codes[w], 0);
    const uint16_t* x = w == 0 ? k : v;
    if (which_delta(cfg, w) && tokens > 0) {
      delta.assign((size_t)cfg->layers * tokens * cfg->heads * cfg->head_dim, 0);
      const int r = kvco_delta_forward(cfg, w, x, tokens, delta.data());
      if (r != KVCO_OK) return r;
      x = delta.data();
    }
    int r = bits ? quantize_mixed(cfg, bits, w, x, tokens, codes[w].data(), out + L.params_off[w])
                 : kvco_quantize_tensor(cfg, w, x, tokens, codes[w].data(), out + L.params_off[w]);
    if (r == KVCO_ERR_RANGE) status = KVCO_ERR_RANGE;
    else if (r != KVCO_OK) return r;
  }
  if (bits) std::memcpy(out + L.map_off, bits, (size_t)(2 * (int64_t)cfg->layers * cfg->heads));
  int64_t pos = L.payload_off, ci = 0;
  std::vector<uint8_t> buf(cfg->chunk_bytes);
  for (int w = 0; w < 2; ++w) {
    for (int64_t i = 0; i < L.nchunks[w]; ++i, ++ci) {
      int64_t n = L.codes[w] - i * cfg->chunk_bytes;
      if (n > cfg->chunk_bytes) n = cfg->chunk_bytes;
      size_t stored = 0; int raw = 0;
      int r = kvco_chunk_encode(cfg->stages, codes[w].data() + i * cfg->chunk_bytes, (size_t)n,
                                buf.data(), &stored, &raw);
      if (r != KVCO_OK) return r;
      std::memcpy(out + pos, buf.data(), stored);
      w32(out + L.table_off + 4 * ci, (uint32_t)stored | (raw ? 0x80000000u : 0u));
      pos += align16((int64_t)stored);
    }
  }
  write_header(out, cfg, tokens, (uint64_t)pos, bits ? 1 : 0);
  *out_bytes = (size_t)pos;
  return status;
}

extern "C" int kvco_encode(const kvco_cfg* cfg, const uint16_t* k, const uint16_t* v, int tokens,
                           uint8_t* out, size_t cap, size_t* out_bytes) {
  return encode_stream(cfg, nullptr, k, v, tokens, out, cap, out_bytes);
}

extern "C" int kvco_encode_mixed(const kvco_cfg* cfg, const uint8_t* bits, const uint16_t* k, const uint16_t* v,
                                 int tokens, uint8_t* out, size_t cap, size_t* out_bytes) {
  if (!bits) return KVCO_ERR_INVALID_ARG;
  return encode_stream(cfg, bits, k, v, tokens, out, cap, out_bytes);
}

/* The width map of a mixed stream (NULL for a uniform one), after checking
 * that it lies inside the stream and holds valid widths. */
static int stream_bits(const uint8_t* in, size_t in_bytes, const kvco_cfg* cfg, const uint8_t** bits) {
  *bits = nullptr;
  if (!(in[7] & 1)) return KVCO_OK;
  if ((int64_t)in_bytes < 64 + 2 * (int64_t)cfg->layers * cfg->heads) return KVCO_ERR_CORRUPT_STREAM;
  if (check_bits_map(cfg, in + 64) != KVCO_OK) return KVCO_ERR_CORRUPT_STREAM;
  *bits = in + 64;
  return KVCO_OK;
}

extern "C" int kvco_stream_info(const uint8_t* in, size_t in_bytes, kvco_cfg* cfg, int* tokens) {
  if (!in || !cfg || !tokens) return KVCO_ERR_INVALID_ARG;
  if (in_bytes < 64 || r32(in) != MAGIC || r16(in + 4) != 1 || (in[7] & ~1)) return KVCO_ERR_CORRUPT_STREAM;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->dtype = in[6];
  cfg->layers = (int32_t)r32(in + 8);
  *tokens = (int32_t)r32(in + 12);
  cfg->heads = (int32_t)r32(in + 16);
  cfg->head_dim = (int32_t)r32(in + 20);
  cfg->k_bits = in[24]; cfg->k_axis = in[25]; cfg->k_hadamard = in[26]; cfg->k_group = r16(in + 28);
  cfg->k_delta = r16(in + 30);
  cfg->v_bits = in[32]; cfg->v_axis = in[33]; cfg->v_hadamard = in[34]; cfg->v_group = r16(in + 36);
  cfg->v_delta = r16(in + 38);
  cfg->seed = r64(in + 40);
  for (int i = 0; i < 4; ++i) cfg->stages[i] = in[48 + i];
  cfg->chunk_bytes = r32(in + 52);
  if (check_cfg(cfg) != KVCO_OK || *tokens < 0 || *tokens > (1 << 26)) return KVCO_ERR_CORRUPT_STREAM;
  const uint8_t* bits = nullptr;
  if (stream_bits(in, in_bytes, cfg, &bits) != KVCO_OK) return KVCO_ERR_CORRUPT_STREAM;
  const Layout L = layout_of(cfg, *tokens, bits);
  const uint64_t total = r64(in + 56);
  if ((int64_t)total < L.payload_off || (int64_t)total > L.max_total || total > in_bytes)
    return KVCO_ERR_CORRUPT_STREAM;
  return KVCO_OK;
}

extern "C" int kvco_decode(const uint8_t* in, size_t in_bytes, uint16_t* k, uint16_t* v, size_t elems_cap) {
  kvco_cfg cfg; int tokens = 0;
  int st = kvco_stream_info(in, in_bytes, &cfg, &tokens);
  if (st != KVCO_OK) return st;
  const size_t elems = (size_t)cfg.layers * tokens * cfg.heads * cfg.head_dim;
  if (elems > elems_cap) return KVCO_ERR_BUFFER_TOO_SMALL;
  if (elems > 0 && (!k || !v)) return KVCO_ERR_INVALID_ARG;
  const uint8_t* bits = nullptr;
  stream_bits(in, in_bytes, &cfg, &bits);       /* checked by kvco_stream_info */
  const Layout L = layout_of(&cfg, tokens, bits);
  const uint64_t total = r64(in + 56);
  int64_t pos = L.payload_off, ci = 0;
  for (int w = 0; w < 2; ++w) {
    std::vector<uint8_t> codes((size_t)L.codes[w]);
    for (int64_t i = 0; i < L.nchunks[w]; ++i, ++ci) {
      int64_t n = L.codes[w] - i * cfg.chunk_bytes;
      if (n > cfg.chunk_bytes) n = cfg.chunk_bytes;
      uint32_t e = r32(in + L.table_off + 4 * ci);
      const int raw = (e >> 31) & 1;
      const int64_t stored = e & 0x7fffffff;
      if (stored > n || pos + stored > (int64_t)total) return KVCO_ERR_CORRUPT_STREAM;
      int r = kvco_chunk_decode(cfg.stages, in + pos, (size_t)stored, raw,
                                codes.data() + i * cfg.chunk_bytes, (size_t)n);
      if (r != KVCO_OK) return r == KVCO_ERR_INVALID_ARG ? KVCO_ERR_CORRUPT_STREAM : r;
      pos += align16(stored);
    }
    int r = bits ? dequantize_mixed(&cfg, bits, w, codes.data(), in + L.params_off[w], tokens, w == 0 ? k : v)
                 : kvco_dequantize_tensor(&cfg, w, codes.data(), in + L.params_off[w], tokens, w == 0 ? k : v);
    if (r != KVCO_OK) return r;
    r = kvco_delta_inverse(&cfg, w, w == 0 ? k : v, tokens);
    if (r != KVCO_OK) return r;
  }
  if (pos != (int64_t)total) return KVCO_ERR_CORRUPT_STREAM;
  return KVCO_OK;
}

/* ======================================================================
 * Paged pools.  One stream per request, each laid out as above with
 * tokens = that request's length; request r's stream starts at
 * req_offsets[r] (an exclusive scan of the stream sizes, which are multiples
 * of 16).  Token t of request r lives in pool block
 * block_table[r * max_blocks_per_req + t / page_tokens], slot t % page_tokens.
 * ====================================================================== */

static int check_pages(int64_t num_blocks, int page_tokens, const int32_t* bt, int maxb,
                       const int32_t* seq_lens, int nreq) {
  if (num_blocks < 0 || page_tokens < 1 || nreq < 0 || maxb < 0 || (nreq > 0 && (!bt || !seq_lens)))
    return KVCO_ERR_INVALID_ARG;
  for (int r = 0; r < nreq; ++r) {
    if (seq_lens[r] < 0 || ceil_div(seq_lens[r], page_tokens) > maxb) return KVCO_ERR_INVALID_ARG;
    for (int64_t b = 0; b < ceil_div(seq_lens[r], page_tokens); ++b) {
      int32_t blk = bt[(int64_t)r * maxb + b];
      if (blk < 0 || blk >= num_blocks) return KVCO_ERR_INVALID_ARG;
    }
  }
  return KVCO_OK;
}

static void gather_request(const kvco_cfg* cfg, const uint16_t* pool, int64_t num_blocks, int page_tokens,
                           const int32_t* bt_row, int T, uint16_t* dense) {
  const int64_t vec_elems = (int64_t)cfg->heads * cfg->head_dim;
  for (int l = 0; l < cfg->layers; ++l)
    for (int t = 0; t < T; ++t) {
      const int64_t blk = bt_row[t / page_tokens];
      const uint16_t* src = pool + (((int64_t)l * num_blocks + blk) * page_tokens + t % page_tokens) * vec_elems;
      std::memcpy(dense + ((int64_t)l * T + t) * vec_elems, src, (size_t)vec_elems * 2);
    }
}

static void scatter_request(const kvco_cfg* cfg, uint16_t* pool, int64_t num_blocks, int page_tokens,
                            const int32_t* bt_row, int T, const uint16_t* dense) {
  const int64_t vec_elems = (int64_t)cfg->heads * cfg->head_dim;
  for (int l = 0; l < cfg->layers; ++l)
    for (int t = 0; t < T; ++t) {
      const int64_t blk = bt_row[t / page_tokens];
      uint16_t* dst = pool + (((int64_t)l * num_blocks + blk) * page_tokens + t % page_tokens) * vec_elems;
      std::memcpy(dst, dense + ((int64_t)l * T + t) * vec_elems, (size_t)vec_elems * 2);
    }
}

extern "C" int kvco_encode_paged(const kvco_cfg* cfg, const uint16_t* k_pool, const uint16_t* v_pool,
                                 int64_t num_blocks, int page_tokens, const int32_t* block_table,
                                 int max_blocks_per_req, const int32_t* seq_lens, int num_requests,
                                 uint8_t* out, size_t cap, uint64_t* req_offsets, size_t* out_bytes) {
  int st = check_cfg(cfg);
  if (st != KVCO_OK) return st;
  st = check_pages(num_blocks, page_tokens, block_table, max_blocks_per_req, seq_lens, num_requests);
  if (st != KVCO_OK) return st;
  if (!out || !req_offsets || !out_bytes) return KVCO_ERR_INVALID_ARG;
  int status = KVCO_OK;
  uint64_t pos = 0;
  for (int r = 0; r < num_requests; ++r) {
    const int T = seq_lens[r];
    const size_t elems = (size_t)cfg->layers * T * cfg->heads * cfg->head_dim;
    std::vector<uint16_t> kd(elems), vd(elems);
    const int32_t* row = block_table + (int64_t)r * max_blocks_per_req;
    gather_request(cfg, k_pool, num_blocks, page_tokens, row, T, kd.data());
    gather_request(cfg, v_pool, num_blocks, page_tokens, row, T, vd.data());
    req_offsets[r] = pos;
    size_t nb = 0;
    if (pos > cap) return KVCO_ERR_BUFFER_TOO_SMALL;
    int e = kvco_encode(cfg, kd.data(), vd.data(), T, out + pos, cap - pos, &nb);
    if (e == KVCO_ERR_RANGE) status = KVCO_ERR_RANGE;
    else if (e != KVCO_OK) return e;
    pos += nb;
  }
  req_offsets[num_requests] = pos;
  *out_bytes = (size_t)pos;
  return status;
}

extern "C" int kvco_decode_paged(const uint8_t* in, const uint64_t* req_offsets, int num_requests,
                                 uint16_t* k_pool, uint16_t* v_pool, int64_t num_blocks, int page_tokens,
                                 const int32_t* block_table, int max_blocks_per_req, const int32_t* seq_lens) {
  int st = check_pages(num_blocks, page_tokens, block_table, max_blocks_per_req, seq_lens, num_requests);
  if (st != KVCO_OK) return st;
  if (!in || !req_offsets) return KVCO_ERR_INVALID_ARG;
  for (int r = 0; r < num_requests; ++r) {
    const uint8_t* s = in + req_offsets[r];
    const size_t avail = (size_t)(req_offsets[r + 1] - req_offsets[r]);
    kvco_cfg cfg; int T = 0;
    int e = kvco_stream_info(s, avail, &cfg, &T);
    if (e != KVCO_OK) return e;
    if (T != seq_lens[r]) return KVCO_ERR_PLAN_MISMATCH;
    const size_t elems = (size_t)cfg.layers * T * cfg.heads * cfg.head_dim;
    std::vector<uint16_t> kd(elems), vd(elems);
    e = kvco_decode(s, avail, kd.data(), vd.data(), elems);
    if (e != KVCO_OK) return e;
    const int32_t* row = block_table + (int64_t)r * max_blocks_per_req;
    scatter_request(&cfg, k_pool, num_blocks, page_tokens, row, T, kd.data());
    scatter_request(&cfg, v_pool, num_blocks, page_tokens, row, T, vd.data());
  }
  return KVCO_OK;
}
