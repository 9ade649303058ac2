/*
 * kvc_oracle.h -- plain, slow CPU reference of the KV-cache compression path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product library
 * (kv_cache_compression_kvc_amd) never calls it and shares no code with it.
 *
 * What it computes follows "Beyond Compression Ratio: High-Throughput KV
 * Compression for Disaggregated LLM Serving" (FastKVComp), Sec. 4.1 (fused
 * randomized-Hadamard + min-max quantization; fused reconstruction doing
 * dequantization, inverse Hadamard, normalization and sign restoration) and
 * Sec. 4.2 (chunked lossless backend built from tuple reordering, bit
 * shuffling and zero-oriented encoding, pipeline TUPL8_1 -> BIT_8 -> RZE_2).
 * Where the pages leave a step open, the reading taken is stated next to the
 * function that implements it.
 *
 * Conventions: all buffers are host memory owned by the caller; 16-bit KV
 * values are passed as their raw bit patterns (uint16_t) and interpreted as
 * fp16 or bf16 according to the config; every function returns a status code
 * (KVCO_OK = 0) and never reads or writes outside the sizes it is given.
 *
 * Every arithmetic function here is pinned by a test under tests/ that does
 * not re-use it (test_oracle_*.py).
 */
#ifndef KVC_ORACLE_H
#define KVC_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KVCO_OK = 0,
  KVCO_ERR_INVALID_ARG = 1,
  KVCO_ERR_UNSUPPORTED = 2,
  KVCO_ERR_NO_MEMORY = 3,
  KVCO_ERR_BUFFER_TOO_SMALL = 4,
  KVCO_ERR_CORRUPT_STREAM = 5,
  KVCO_ERR_PLAN_MISMATCH = 6,
  KVCO_ERR_RANGE = 7,
  KVCO_ERR_INTERNAL = 99
};

/* Lossless stage identifiers (the byte values stored in a stream header). */
enum {
  KVCO_STAGE_END = 0,
  KVCO_TUPL2_1 = 1, KVCO_TUPL4_1 = 2, KVCO_TUPL8_1 = 3,
  KVCO_DIFF1 = 4, KVCO_DIFF2 = 5, KVCO_DIFF4 = 6, KVCO_DIFF8 = 7,
  KVCO_BIT_1 = 8, KVCO_BIT_2 = 9, KVCO_BIT_4 = 10, KVCO_BIT_8 = 11,
  KVCO_RZE_1 = 12, KVCO_RZE_2 = 13, KVCO_RZE_4 = 14, KVCO_RZE_8 = 15
};

typedef struct {
  int32_t layers, heads, head_dim;
  int32_t dtype;                       /* 0 = fp16, 1 = bf16 */
  int32_t k_bits, k_axis, k_group, k_hadamard;   /* axis 0 = per-token, 1 = per-channel */
  int32_t v_bits, v_axis, v_group, v_hadamard;
  uint64_t seed;
  uint8_t stages[4];                   /* 0-terminated lossless pipeline */
  uint32_t chunk_bytes;
  int32_t k_delta, v_delta;            /* token-delta run length: 0 = none, else a power of two in [2, 32768] */
} kvco_cfg;

/* ---- scalar building blocks (exported so tests can pin them) ---- */
uint64_t kvco_splitmix64(uint64_t* state);
int kvco_signs(uint64_t seed, int n, int8_t* out);
float kvco_norm_const(int n);
int kvco_fwht(float* v, int n);
float kvco_f16_to_f32(uint16_t h);
uint16_t kvco_f32_to_f16_rn(float f);
uint16_t kvco_f32_to_f16_rd(float f);
uint16_t kvco_f32_to_f16_ru(float f);
float kvco_bf16_to_f32(uint16_t h);
uint16_t kvco_f32_to_bf16_rn(float f);
int kvco_group_params(const float* z, int count, int bits, float c,
                      uint16_t* s_out, uint16_t* m_out, float* inv_out);
int kvco_quantize_group(const float* z, int count, int bits, float c,
                        uint16_t s, uint16_t m, float inv, uint8_t* codes_out);

/* ---- whole tensors (one of K or V: which = 0 for K, 1 for V) ---- */
int64_t kvco_codes_bytes(const kvco_cfg* cfg, int which, int tokens);
int64_t kvco_params_bytes(const kvco_cfg* cfg, int which, int tokens);
int kvco_quantize_tensor(const kvco_cfg* cfg, int which, const uint16_t* x, int tokens,
                         uint8_t* codes, uint8_t* params);
int kvco_dequantize_tensor(const kvco_cfg* cfg, int which, const uint8_t* codes,
                           const uint8_t* params, int tokens, uint16_t* x);

/* ---- token delta (a pre-transform; identity when the tensor's run length is 0) ---- */
int kvco_delta_forward(const kvco_cfg* cfg, int which, const uint16_t* x, int tokens, uint16_t* y);
int kvco_delta_inverse(const kvco_cfg* cfg, int which, uint16_t* x, int tokens);

/* ---- lossless components ---- */
int kvco_stage_encode(int stage, const uint8_t* in, size_t n, uint8_t* out, size_t cap, size_t* out_n);
int kvco_stage_decode(int stage, const uint8_t* in, size_t in_n, uint8_t* out, size_t n);
int kvco_chunk_encode(const uint8_t* stages, const uint8_t* in, size_t n,
                      uint8_t* out, size_t* stored, int* raw);
int kvco_chunk_decode(const uint8_t* stages, const uint8_t* in, size_t stored, int raw,
                      uint8_t* out, size_t n);

/* ---- whole streams ---- */
int64_t kvco_max_stream_bytes(const kvco_cfg* cfg, int tokens);
int kvco_encode(const kvco_cfg* cfg, const uint16_t* k, const uint16_t* v, int tokens,
                uint8_t* out, size_t cap, size_t* out_bytes);
int kvco_stream_info(const uint8_t* in, size_t in_bytes, kvco_cfg* cfg_out, int* tokens_out);

/* ---- mixed precision per (layer, head): bits[2][layers][heads] holds 2, 4 or
 * 8 (that width through the quantizer) or 16 (values kept); kvco_decode reads
 * both kinds of stream ---- */
int64_t kvco_max_stream_bytes_mixed(const kvco_cfg* cfg, const uint8_t* bits, int tokens);
int kvco_encode_mixed(const kvco_cfg* cfg, const uint8_t* bits, const uint16_t* k, const uint16_t* v,
                      int tokens, uint8_t* out, size_t cap, size_t* out_bytes);
int kvco_decode(const uint8_t* in, size_t in_bytes, uint16_t* k, uint16_t* v, size_t elems_cap);

/* ---- paged pools: [layers][num_blocks][page_tokens][heads][head_dim] ---- */
int kvco_encode_paged(const kvco_cfg* cfg, const uint16_t* k_pool, const uint16_t* v_pool,
                      int64_t num_blocks, int page_tokens, const int32_t* block_table,
                      int max_blocks_per_req, const int32_t* seq_lens, int num_requests,
                      uint8_t* out, size_t cap, uint64_t* req_offsets, size_t* out_bytes);
int kvco_decode_paged(const uint8_t* in, const uint64_t* req_offsets, int num_requests,
                      uint16_t* k_pool, uint16_t* v_pool, int64_t num_blocks, int page_tokens,
                      const int32_t* block_table, int max_blocks_per_req, const int32_t* seq_lens);

#ifdef __cplusplus
}
#endif
#endif
