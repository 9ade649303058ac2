// Internal declarations shared by libkvc's translation units (host API and
// kernels).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr int kHeadDim = 128;          // head_dim the kernels are written for
constexpr uint32_t kMagic = 0x3143564Bu;
constexpr int kHeaderBytes = 64;
constexpr uint32_t kRawFlag = 0x80000000u;
// Non-zero-word counters per chunk that the fused encoders add to (a wave
// picks one by its index), so that the waves of one chunk spread their
// atomics over several addresses; the scan and the size pass sum them.
constexpr int kNnzSlots = 16;

// Status word bits recorded by kernels in the workspace control block.
enum : uint32_t {
  kStCorrupt = 1u << 0,
  kStMismatch = 1u << 1,
  kStRange = 1u << 2,
  kStBadBlock = 1u << 3,
  kStStall = 1u << 4,        // a bounded wait of the single-pass placement ran out
};

// Workspace control block (first 256 bytes of every workspace).
struct Control {
  uint32_t status;
  uint32_t pad0;
  uint64_t total;        // dense encode: stream bytes
  uint64_t pad[30];
};
static_assert(sizeof(Control) == 256, "control block is 256 bytes");

// Quantization policy of one tensor as the kernels see it.
struct TensorPol {
  int bits;
  int axis;              // 0 per-token, 1 per-channel
  int group;
  int hadamard;
  float c;               // 1/sqrt(head_dim) rounded to binary32 (1 if no transform)
  int delta;             // token-delta run length (0 = none)
};

// One (layer, head) slab of a mixed-precision tensor: its codes and
// parameters start codes_off / params_off bytes into the tensor's sections.
struct SlabDesc {
  int32_t l, h;
  int64_t codes_off, params_off;
};

// One request of a call; a dense call is a single request.
struct ReqDesc {
  int32_t T;                 // tokens
  int32_t row;               // block-table row (paged)
  int32_t nchunks[2];        // code chunks of K and V
  int64_t chunk_begin;       // global index of the first chunk (K chunks, then V chunks)
  int64_t tile_begin[2];     // first fused-kernel tile of K and of V
  int64_t codes_off[2];      // code sections in the workspace codes area
  int64_t codes_bytes[2];
  int64_t params_ws_off[2];  // parameter staging in the workspace (paged encode), -1 if direct
  int64_t params_off[2];     // parameter sections inside this request's stream
  int64_t params_bytes[2];
  int64_t table_off;         // chunk table offset inside this request's stream
  int64_t payload_off;       // payload offset inside this request's stream
  int64_t max_stream;        // stream bytes with every chunk raw
  int64_t piece_begin;       // first parameter-copy piece (paged encode)
  int64_t raw_base;          // paged encode: where this request's stream would start if every
                             //   earlier request's chunks were raw (sum of their max_stream)
  int64_t fixed_before;      // paged encode: payload_off summed over the earlier requests
};

// Where the requests live and where their data goes.
// Entries of a paged call's tile -> request table, per tensor (R > 1).
constexpr int kReqTableMax = 4096;

struct CallDesc {
  int R;                     // requests
  const ReqDesc* reqs;       // device array [R] (R > 1)
  ReqDesc one;               // the request when R == 1
  // R > 1: req_tab[w][i] = the last request whose first tile of tensor w is at
  // or before tile i << req_shift[w] (i up to tiles >> req_shift, inclusive),
  // which brackets the request of any tile to [req_tab[i], req_tab[i + 1]]
  const int32_t* req_tab[2];
  int req_shift[2];
  int layers, heads;
  int dtype;                 // 0 fp16, 1 bf16
  TensorPol pol[2];
  uint32_t signs[4];         // bit i set: sign of channel i is -1
  uint8_t stages[4];
  uint32_t chunk_bytes;
  int chunk_shift;           // log2(chunk_bytes) when it is a power of two, else -1
  uint64_t seed;
  // paged addressing (page_tokens == 0: dense)
  int page_tokens;
  int64_t num_blocks;
  const int32_t* block_table;
  int max_blocks;
  // buffers
  const void* in_kv[2];      // encode: K, V inputs (dense tensors or pools)
  void* out_kv[2];           // decode: K, V outputs (dense tensors or pools)
  uint8_t* codes;            // packed codes: the workspace codes area, or (dense encode) the
                             // stream's payload laid out as if every chunk were raw
  uint8_t* codes_out;        // encode: where compressed chunk bytes go (== codes: in place)
  int direct[2];             // decode: reconstruct kernels read raw chunks of K / V from the stream
  int mirror[2];             // decode: ... and decode TUPL8_1 -> BIT_8 -> RZE_2 chunks of 2-bit
  int straddle;              // decode (paged): a reconstruct tile may cover two chunks; it reads the
                             //   stream only if both are raw, so raw chunks next to a compressed one
                             //   are still copied to the codes area
                             //   per-token codes themselves, from per-segment word counts that
                             //   k_ll_decode_raw leaves in the chunk's slot of the codes area
  int place;                 // encode: 1 = dense, finish the stream in one in-place pass (k_place);
                             //   2 = paged, chunks placed from the workspace (k_place_paged)
  uint32_t* place_flags;     //   [total chunks] read announcements, then [ceil(total / 64)] group counts
  uint64_t* scan_state;      // dense calls: look-back words of the chunk-size scan, one per 1024 chunks
  int counts_to_sizes;       // dense encode: every chunk is counted by the fused kernels and
                             //   encoded by the placement, so the scan turns counts into sizes
                             //   itself (no size pass)
  int validate_in_reset;     // dense decode: the reset kernel also checks the header
  int nnz_pipe;              // encode: 1 or 2 when the fused kernels count the non-zero RZE
  int nnz_sec[2];            //   words of pipeline P1 / P2 per chunk (into chunk_sizes), per section
  uint8_t* params_ws;        // workspace parameter staging area (paged encode)
  uint8_t* stream;           // dense: the stream; paged: base of all streams
  const uint64_t* req_offsets;  // paged: stream offsets (device)
  uint64_t* req_offsets_out;    // paged encode: written by the scan
  uint64_t stream_bytes;     // decode: bytes available in the input
  uint32_t* chunk_sizes;     // [total chunks] stored sizes | raw flag
  uint32_t* chunk_counts;    // encode: [total chunks][kNnzSlots] non-zero RZE word counts of the fused encoders
  uint64_t* chunk_offs;      // [total chunks + 1] exclusive scan of align16(stored)
  Control* ctl;
  int64_t total_chunks;
  int64_t total_pieces;      // paged encode: parameter copy pieces
  int64_t tiles[2];          // fused-kernel tiles of K and V over all requests
  // mixed precision per (layer, head): codes and parameters are (layer, head)
  // slabs; each fused launch covers the `nslabs` slabs of `slabs` (one width)
  int mixed;
  const SlabDesc* slabs;
  int nslabs;
  const uint8_t* width_map;  // device copy of the 2 * L * H widths (header)
};

// Kernel launch wrappers (defined in the .hip files).  Each returns the HIP
// error of its launch.
hipError_t launch_reset(const CallDesc& c, hipStream_t s);
hipError_t launch_encode_fused(const CallDesc& c, int which, hipStream_t s);
hipError_t launch_decode_fused(const CallDesc& c, int which, hipStream_t s);
hipError_t launch_lossless_encode(const CallDesc& c, hipStream_t s);
hipError_t launch_scan(const CallDesc& c, bool from_table, hipStream_t s);
// Token delta over a dense [layers][T][heads][128] tensor of 16-bit values:
// forward (x -> y, out of place) or inverse (in place, x == y).
hipError_t launch_delta(const CallDesc& c, int which, int T, bool forward, const void* x, void* y, hipStream_t s);
hipError_t launch_compact(const CallDesc& c, hipStream_t s);
hipError_t launch_place(const CallDesc& c, hipStream_t s);
hipError_t launch_validate(const CallDesc& c, hipStream_t s);
// classified: the chunks were classified by launch_dec_front_small
hipError_t launch_lossless_decode(const CallDesc& c, bool classified, hipStream_t s);
// One-request decodes of at most kFrontChunks chunks: reset, header check,
// chunk-offset scan and classification in one single-block launch (in place
// of launch_reset, launch_scan and the classification).
constexpr int kFrontChunks = 1024;
hipError_t launch_dec_front_small(const CallDesc& c, hipStream_t s);
// Whether a one-request call's chunks all go to the word-parallel kernels (a
// standard pipeline and every chunk size a multiple of its block).
bool all_word_parallel(const CallDesc& c);
// 16-bit passthrough slabs of a mixed tensor: gather into the codes section
// (encode) or scatter back into the tensor (decode)
hipError_t launch_slab_copy(const CallDesc& c, int which, bool encode, hipStream_t s);

// Bandwidth reference kernel: `items` items, each reading `reads` and writing
// `writes` 16-byte lines (kvc_probe.hip); flags as kvc_probe_bandwidth's.
hipError_t launch_probe(const void* src, void* dst, int64_t items, int reads, int writes, int flags,
                        uint32_t* sink, hipStream_t s);

// Per-kernel timing hooks (kvc_api.cpp).
void prof_begin(int kind, hipStream_t s);
void prof_end(int kind, hipStream_t s);

}  // namespace kvc
