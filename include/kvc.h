/*
 * kvc.h -- C ABI of libkvc, an MI355X (gfx950) implementation of the KV-cache
 * compression data path described in "Beyond Compression Ratio:
 * High-Throughput KV Compression for Disaggregated LLM Serving" (FastKVComp):
 *
 *   encode:  fused randomized-Hadamard + min-max quantize-and-pack kernel
 *            (Sec. 4.1, fused transform-quantization), then a chunked lossless
 *            backend over the packed codes (Sec. 4.2, pipeline TUPL8_1 ->
 *            BIT_8 -> RZE_2 by default), a device-wide scan of the chunk sizes
 *            and a compacted write of the final stream;
 *   decode:  lossless decode, then a fused dequantize + inverse Hadamard +
 *            normalization + sign restoration kernel (Sec. 4.1, fused
 *            reconstruction), applied in that order: x = d * fl32(c * H w),
 *            w = q * s + m (one fused multiply-add), c = fl32(1/sqrt(128)),
 *            rounded to the 16-bit type to nearest-even.
 *
 * FastKVComp Sec. 4.2 describes the runtime as device-pointer encode/decode
 * calls that keep the bitstream on the GPU, reuse persistent scratch and send
 * only the compressed size to the host; this ABI follows that shape.
 *
 * Conventions for every entry point:
 *   - Pointers named d_* are device pointers (HIP device memory of the current
 *     device); h_* are host pointers.  The caller owns all of them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All device work is enqueued on it; calls return without synchronizing
 *     unless stated otherwise.
 *   - KV tensors are fp16 or bf16, contiguous, laid out [layers][tokens]
 *     [kv_heads][head_dim] (dense) or, for paged calls, pools laid out
 *     [layers][num_blocks][page_tokens][kv_heads][head_dim].
 *   - Argument errors are detected on the host and returned before anything
 *     is enqueued.  Errors only the device can see (corrupt stream, fp16
 *     parameter overflow, non-finite input values) are recorded in a status
 *     word inside the workspace;
 *     they are returned by kvc_encode when h_out_bytes is non-NULL and
 *     otherwise by kvc_query_status.
 *   - No exceptions cross the ABI.  kvc_last_error() returns a thread-local
 *     description of the last failure of the calling thread.
 *   - Plans are immutable after kvc_plan() and may be used from several
 *     threads and streams at once, provided each in-flight call has its own
 *     workspace.  Two calls that share a workspace race.
 *
 * Stream format (version 1, little-endian), produced by kvc_encode and read
 * by kvc_decode:
 *   [0,64)          header: u32 magic 0x3143564B ("KVC1"), u16 version = 1,
 *                   u8 dtype, u8 flags (bit 0: mixed precision, see
 *                   kvc_plan_mixed; other bits 0), i32 layers, tokens, kv_heads, head_dim,
 *                   K policy {u8 bits, u8 axis, u8 hadamard, u8 0, u16 group,
 *                   u16 token-delta run length}, V policy (same), u64 sign_seed,
 *                   u8 lossless[4],
 *                   u32 chunk_bytes, u64 total_bytes
 *   [64, 64+4n)     chunk table for the K code chunks then the V code chunks:
 *                   bit 31 = stored raw, bits 0..30 = stored bytes
 *   align 16        K parameters, then (align 16) V parameters, each an array
 *                   of (scale, minimum) fp16 pairs
 *   align 16        code chunks; chunk i starts at the sum over j < i of
 *                   align16(stored_j); all padding bytes are zero
 *   Mixed-precision streams insert the 2 * L * H widths (K then V, layer-major)
 *   at [64, 64 + 2LH) and start the chunk table at align16(64 + 2LH); each
 *   codes / parameter section is then the concatenation over (layer, head) of
 *   the sections a one-layer, one-head stream of that head's width holds
 *   (width 16: the T x D 16-bit values, no parameters).
 *   Codes: per-token policy -> [L][T][H][D] packed along head_dim, LSB
 *   first; per-channel policy -> [L][ceil(T/G)][H][D][ceil(Gg*bits/8)]
 *   packed along the group's Gg tokens.  Parameters: per-token ->
 *   [L][T][H][D/G]; per-channel -> [L][ceil(T/G)][H][D].
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvc_plan_s* kvc_plan_t;

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = 1,      /* NULL pointer, bad shape, bad policy value */
  KVC_ERR_UNSUPPORTED = 2,      /* valid policy the GPU kernels do not implement */
  KVC_ERR_NO_MEMORY = 3,        /* host allocation failed */
  KVC_ERR_BUFFER_TOO_SMALL = 4, /* output capacity or workspace too small */
  KVC_ERR_CORRUPT_STREAM = 5,   /* stream fails validation (device-detected) */
  KVC_ERR_PLAN_MISMATCH = 6,    /* stream header differs from the plan / tokens */
  KVC_ERR_RANGE = 7,            /* a quantization parameter is not a finite fp16, or an
                                   input value is infinite or NaN (device-detected: the
                                   stream is then not decodable) */
  KVC_ERR_HIP = 8               /* a HIP runtime call failed */
} kvc_status;

enum { KVC_F16 = 0, KVC_BF16 = 1 };
enum { KVC_PER_TOKEN = 0, KVC_PER_CHANNEL = 1 };

/* Lossless stage identifiers (bytes of kvc_config.lossless and of the header). */
enum {
  KVC_STAGE_END = 0,
  KVC_TUPL2_1 = 1, KVC_TUPL4_1 = 2, KVC_TUPL8_1 = 3,
  KVC_DIFF1 = 4, KVC_DIFF2 = 5, KVC_DIFF4 = 6, KVC_DIFF8 = 7,
  KVC_BIT_1 = 8, KVC_BIT_2 = 9, KVC_BIT_4 = 10, KVC_BIT_8 = 11,
  KVC_RZE_1 = 12, KVC_RZE_2 = 13, KVC_RZE_4 = 14, KVC_RZE_8 = 15
};

/* Quantization policy of one tensor (FastKVComp Sec. 4.1: channel-wise for
 * keys, token-wise for values, min-max rule, randomized Hadamard). */
typedef struct {
  uint8_t bits;       /* 2, 4 or 8 */
  uint8_t axis;       /* KVC_PER_TOKEN: groups of `group` channels of one head vector;
                         KVC_PER_CHANNEL: groups of `group` tokens of one channel */
  uint8_t hadamard;   /* 1: randomized Hadamard over head_dim; 0: none (stream format
                         only: kvc_plan returns KVC_ERR_UNSUPPORTED for it) */
  uint8_t reserved0;
  uint16_t group;     /* power of two */
  uint16_t delta;     /* token delta before the transform (KVServe Sec. 5.1, the Delta
                         transformer module, after CacheGen): 0 = none; else a power of
                         two D in [2, 32768].  In each (layer, head) the tokens form runs
                         of D from token 0; a run's first token is kept and every other
                         token is replaced by its binary32 difference from it, rounded
                         to the 16-bit type; decoding adds the anchor back with the same
                         rounding.  Dense calls only (the paged calls return
                         KVC_ERR_UNSUPPORTED); an encode needs 2 bytes of workspace per
                         value of each tensor that uses it. */
} kvc_tensor_policy;

typedef struct {
  uint32_t struct_size;        /* sizeof(kvc_config) */
  int32_t layers;
  int32_t max_tokens;          /* largest token count a dense call may pass */
  int32_t kv_heads;
  int32_t head_dim;            /* power of two; the GPU kernels run head_dim 128 */
  int32_t dtype;               /* KVC_F16 or KVC_BF16 */
  kvc_tensor_policy k, v;
  uint64_t sign_seed;          /* seeds the Hadamard sign vector (splitmix64) */
  uint8_t lossless[4];         /* 0-terminated stage list; zero elimination must be last */
  uint32_t chunk_bytes;        /* lossless chunk size: multiple of 4096, at most 65536 */
  int32_t page_tokens;         /* tokens per page for the paged calls; 0 = dense only */
} kvc_config;

/* Validate a configuration and build a plan (host only; allocates no device
 * memory and needs no GPU).  FastKVComp Sec. 4.1 caches signs, precision
 * assignments and workspaces across layers and requests; the plan holds the
 * first two.  Returns KVC_ERR_INVALID_ARG for malformed values and
 * KVC_ERR_UNSUPPORTED for valid policies the GPU kernels do not implement
 * (head_dim != 128, per-channel groups other than 32/64, per-token groups
 * other than 16..128, kv_heads not dividing 32 for per-token policies). */
kvc_status kvc_plan(const kvc_config* cfg, kvc_plan_t* out);

/* A plan with mixed precision per (layer, head) (KVServe Sec. 5.1: head-wise
 * and layer-wise mixed precision, e.g. retrieval heads at high precision and
 * streaming heads at very low bit widths).  h_bits is a host array
 * [2][layers][kv_heads] (K then V): 0 = the tensor policy's bits, 2 / 4 / 8 =
 * that width for the head's quantizer (same axis, group and Hadamard), 16 =
 * the head's 16-bit values kept as they are.  The plan copies it.  Dense
 * calls only (page_tokens must be 0; paged calls return KVC_ERR_UNSUPPORTED).
 * Errors as kvc_plan, and KVC_ERR_INVALID_ARG for other width values. */
kvc_status kvc_plan_mixed(const kvc_config* cfg, const uint8_t* h_bits, kvc_plan_t* out);

/* Release a plan (host memory only).  NULL is accepted.  Calls still in
 * flight on a stream keep no reference to the plan. */
kvc_status kvc_plan_destroy(kvc_plan_t plan);

/* Exact sizes for a dense call with `tokens` tokens: the largest stream
 * kvc_encode can produce (chunks stored raw) and the workspace bytes both
 * kvc_encode and kvc_decode need.  Host only.  FastKVComp Sec. 4.2 keeps the
 * persistent scratch and a reusable staging buffer with the runtime; here the
 * caller allocates both once from these sizes and reuses them across calls.
 * KVC_ERR_INVALID_ARG if tokens is outside [0, max_tokens]. */
kvc_status kvc_plan_sizes(kvc_plan_t plan, int64_t tokens,
                          size_t* max_stream_bytes, size_t* workspace_bytes);

/* Same for a paged call: the sum of the per-request maximum stream sizes and
 * the workspace for encode_paged / decode_paged.  h_seq_lens[num_requests]
 * (host array).  The lengths themselves, not only their total, are needed:
 * every request's stream is chunked on its own, so the exact sizes depend on
 * each length.  KVC_ERR_INVALID_ARG for a negative count, a missing array or
 * a length outside [0, 2^26]. */
kvc_status kvc_plan_sizes_paged(kvc_plan_t plan, const int32_t* h_seq_lens, int32_t num_requests,
                                size_t* max_total_bytes, size_t* workspace_bytes);

/* Encode K and V ([layers][tokens][kv_heads][head_dim], plan dtype) into one
 * stream at d_out (capacity out_capacity >= max_stream_bytes): the fused
 * rotation + quantize + pack of FastKVComp Sec. 4.1 over every token vector,
 * then its LC-style lossless stage per chunk (Sec. 4.2).  d_k, d_v, d_out and
 * d_ws are device pointers the caller owns; d_ws is the workspace
 * (>= workspace_bytes, 256-byte aligned), reused across calls.  If h_out_bytes is non-NULL the call synchronizes the stream, copies
 * back the 8-byte compressed size (the only device-to-host transfer) and
 * returns any device-detected status; with NULL the call is fully
 * asynchronous and the size is the header's total_bytes field.  With the
 * stream synchronized, the result is reproducible bit-for-bit. */
kvc_status kvc_encode(kvc_plan_t plan, const void* d_k, const void* d_v, int32_t tokens,
                      void* d_out, size_t out_capacity, void* d_ws, size_t ws_bytes,
                      size_t* h_out_bytes, void* stream);

/* kvc_encode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a fixed array of
 * KVC_NOALLOC_SCRATCH_BYTES inside the library's device code; each device
 * that runs this call holds its own copy until the process ends.  The call
 * allocates nothing (no hipMalloc / hipFree); the caller passes the inputs
 * and d_out as for kvc_encode, with the same stream format and results.
 * Returns KVC_ERR_BUFFER_TOO_SMALL, before enqueuing anything, when the call's
 * workspace (kvc_plan_sizes) exceeds the array (e.g. more than one layer of
 * 131072 tokens of 8 KV heads at 2 bits), and KVC_ERR_UNSUPPORTED for
 * mixed-precision plans.  Every call on one device shares that device's
 * array: calls that overlap in time on one device (two streams, two threads)
 * race and must be ordered by the caller.  The array keeps the last call's
 * contents; each call clears what must start at zero itself.  Device-detected
 * errors are returned when h_out_bytes is non-NULL (the call then
 * synchronizes as kvc_encode does); with NULL the call is asynchronous, the
 * size is the header's total_bytes field and the device status is not
 * reported. */
#define KVC_NOALLOC_SCRATCH_BYTES (128u << 20)
kvc_status kvc_encode_noalloc(kvc_plan_t plan, const void* d_k, const void* d_v, int32_t tokens,
                              void* d_out, size_t out_capacity, size_t* h_out_bytes, void* stream);

/* Decode a stream of in_bytes bytes holding `tokens` tokens into d_k and d_v
 * ([layers][tokens][kv_heads][head_dim]): lossless decode per chunk, then the
 * fused reconstruction of FastKVComp Sec. 4.1 (dequantization, inverse
 * Hadamard, normalization, sign restoration).  `tokens` is the length the
 * caller sized d_k and d_v for; the header must state the same (so the
 * launch shapes are known on the host, with no read-back of the header, and
 * a stream of another length is reported rather than written past the
 * buffers).  The device validates the header against the plan and every
 * chunk against in_bytes; failures are recorded as KVC_ERR_PLAN_MISMATCH or
 * KVC_ERR_CORRUPT_STREAM (read them with kvc_query_status), in which case the
 * output contents are unspecified but no read or write leaves the given
 * buffers.  Host-detected errors (NULL or misaligned pointers, tokens outside
 * [0, max_tokens], in_bytes shorter than the fixed sections, ws_bytes too
 * small) return before anything is enqueued. */
kvc_status kvc_decode(kvc_plan_t plan, const void* d_in, size_t in_bytes, int32_t tokens,
                      void* d_k, void* d_v, void* d_ws, size_t ws_bytes, void* stream);

/* Paged encode (FastKVComp Sec. 4.2: the runtime consumes the frontend's
 * device buffers, here a paged pool): request r (length h_seq_lens[r]) has token t in pool block
 * d_block_table[r * max_blocks_per_req + t / page_tokens], slot
 * t % page_tokens.  Each request becomes its own stream (format above, tokens
 * = its length); request r's stream starts at d_req_offsets[r] within d_out and
 * d_req_offsets[num_requests] is the total (device array of num_requests + 1,
 * written by the call).  The block-table gather is fused into the quantize
 * kernel.  Block ids are validated on the device (KVC_ERR_INVALID_ARG in the
 * status word if out of range).  Supports per-token policies. */
kvc_status kvc_encode_paged(kvc_plan_t plan, const void* d_k_pool, const void* d_v_pool,
                            int64_t num_blocks, const int32_t* d_block_table, int32_t max_blocks_per_req,
                            const int32_t* h_seq_lens, int32_t num_requests,
                            void* d_out, size_t out_capacity, uint64_t* d_req_offsets,
                            void* d_ws, size_t ws_bytes, size_t* h_out_bytes, void* stream);

/* Paged decode: the mirror image; the reconstruction kernel scatters each
 * request's tokens into the pools through d_block_table (which may differ
 * from the one used to encode).  d_req_offsets[num_requests + 1] is the
 * device array kvc_encode_paged wrote; each request's header is checked
 * against the plan and its length, and its chunks against in_bytes, with
 * errors recorded in the workspace status as for kvc_decode. */
kvc_status kvc_decode_paged(kvc_plan_t plan, const void* d_in, size_t in_bytes,
                            const uint64_t* d_req_offsets, const int32_t* h_seq_lens, int32_t num_requests,
                            void* d_k_pool, void* d_v_pool, int64_t num_blocks,
                            const int32_t* d_block_table, int32_t max_blocks_per_req,
                            void* d_ws, size_t ws_bytes, void* stream);

/* Synchronize `stream`, return the device status recorded in the workspace by
 * the last call that used it, and clear it.  FastKVComp Sec. 4.2 returns only
 * a size scalar to the host; the status word is the other value that stays
 * on the device until asked for. */
kvc_status kvc_query_status(kvc_plan_t plan, const void* d_ws, void* stream);

/* Static name of a status code. */
const char* kvc_status_string(kvc_status s);
/* Detail of the calling thread's last host-detected error (thread-local,
 * valid until that thread's next call). */
const char* kvc_last_error(void);

/* Optional per-kernel timing.  While enabled, every kernel launch of the
 * library is bracketed by HIP events on its stream; kvc_profile_query
 * synchronizes those events and returns the accumulated milliseconds and
 * launch count of one kernel kind since the last reset. */
typedef enum {
  KVC_KERNEL_ENCODE_K = 0,     /* fused transform + quantize, K */
  KVC_KERNEL_ENCODE_V = 1,     /* fused transform + quantize, V */
  KVC_KERNEL_LOSSLESS_ENC = 2,
  KVC_KERNEL_SCAN = 3,
  KVC_KERNEL_COMPACT = 4,      /* single-pass placement of the chunks (and, paged, the headers and parameters) */
  KVC_KERNEL_LOSSLESS_DEC = 5,
  KVC_KERNEL_DECODE_K = 6,     /* fused reconstruct, K */
  KVC_KERNEL_DECODE_V = 7,     /* fused reconstruct, V */
  KVC_KERNEL_AUX = 8,          /* header, validation and status kernels */
  KVC_KERNEL_DELTA = 9,        /* token delta: forward before encoding, inverse after decoding */
  KVC_KERNEL_COUNT = 10
} kvc_kernel_kind;

kvc_status kvc_profile_enable(int on);
kvc_status kvc_profile_reset(void);
kvc_status kvc_profile_query(int kind, double* total_ms, int64_t* launches);

/* Bandwidth reference for the measurements (no part of the compression
 * path): enqueue on `stream` a streaming kernel over `items` items, each
 * reading `reads` 16-byte lines of d_src (items * reads * 16 bytes) and
 * writing `writes` 16-byte lines of d_dst (items * writes * 16 bytes), with
 * 16-byte buffer accesses, non-temporal stores and no other work.  With
 * flags 0 it loads with the default cache policy from a capped grid of
 * looping waves, as most fused kernels do; KVC_PROBE_NT_LOADS makes the
 * loads non-temporal, KVC_PROBE_SHORT_WAVES launches one wave per 256 items
 * (each wave handles its items once and exits).  (reads, writes) is one of (1,0), (0,1),
 * (1,1), (2,1), (4,1), (1,4); other pairs return KVC_ERR_UNSUPPORTED, other
 * flag bits KVC_ERR_INVALID_ARG.  d_sink is a 4-byte device word the
 * read-only form may write.  Time it with events on `stream`. */
enum { KVC_PROBE_NT_LOADS = 1, KVC_PROBE_SHORT_WAVES = 2 };
kvc_status kvc_probe_bandwidth(const void* d_src, void* d_dst, int64_t items, int reads, int writes, int flags,
                               uint32_t* d_sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif
