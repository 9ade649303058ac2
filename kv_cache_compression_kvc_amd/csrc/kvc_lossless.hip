// Chunked lossless backend over the packed codes, its scan and compaction,
// stream headers and validation, for gfx950.
//
// FastKVComp ("Beyond Compression Ratio: High-Throughput KV Compression for
// Disaggregated LLM Serving") Sec. 4.2 composes reordering of byte tuples,
// shuffling of bits and elimination of zero words into one pipeline
// (TUPL8_1 -> BIT_8 -> RZE_2).  Stage definitions used here:
//   TUPLk_1  m = n/k tuples: out[j*m + i] = in[i*k + j]; tail copied;
//   DIFFw    w-byte words: out[i] = in[i] - in[i-1] mod 2^(8w); tail copied;
//   BITw     8w words of w bytes form a square bit matrix that is transposed;
//            incomplete trailing group copied;
//   RZEw     bitmap (bit i set iff word i != 0, LSB first), the non-zero
//            words, then the tail bytes.
// A chunk whose result is not smaller than its input is stored raw.
//
// Encode: every chunk's exact compressed size comes first, without
// materializing the transform: for the two standard pipelines a 2-byte RZE
// word of the output is zero exactly when a fixed set of input bits is zero,
// so the count of non-zero output words is a popcount of OR-reductions of the
// input words (the fused encoders usually count it while the codes are in
// registers).  Chunks of other pipelines, and partial chunks, go on a
// worklist for the stage engine, which runs the stages in LDS (two 64 KiB
// buffers) and writes the result into the chunk's staging slot.  A scan turns
// stored sizes into 16-byte aligned offsets.  A dense encode then ends with
// one in-place pass (k_place) that encodes the chunks of the two standard
// pipelines and puts every chunk at its final offset; a paged encode places
// its chunks the same way from the workspace (k_place_paged) while the
// compaction kernel copies the parameter pieces.  Headers and chunk tables
// are written along the way.
#include <algorithm>

#include "kvc_internal.h"
#include "kvc_xpose.h"

namespace kvc {

__device__ __forceinline__ void set_status2(Control* ctl, uint32_t bit) {
  __hip_atomic_fetch_or(&ctl->status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ ReqDesc req_at(const CallDesc& c, int r) { return (c.R == 1) ? c.one : c.reqs[r]; }

__device__ __forceinline__ int find_req_by_chunk(const CallDesc& c, int64_t chunk) {
  if (c.R == 1) return 0;
  int lo = 0, hi = c.R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (c.reqs[mid].chunk_begin <= chunk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct ChunkLoc {
  int r, w;
  int64_t index;    // within its section
  int64_t n;        // raw bytes
  int64_t src;      // byte offset in the codes area
};

__device__ __forceinline__ ChunkLoc locate_chunk(const CallDesc& c, const ReqDesc& rq, int r, int64_t chunk) {
  ChunkLoc L;
  L.r = r;
  const int64_t k = chunk - rq.chunk_begin;
  L.w = (k < rq.nchunks[0]) ? 0 : 1;
  L.index = (L.w == 0) ? k : k - rq.nchunks[0];
  const int64_t rem = rq.codes_bytes[L.w] - L.index * (int64_t)c.chunk_bytes;
  L.n = rem < (int64_t)c.chunk_bytes ? rem : (int64_t)c.chunk_bytes;
  L.src = rq.codes_off[L.w] + L.index * (int64_t)c.chunk_bytes;
  return L;
}

__device__ __forceinline__ int64_t align16(int64_t x) { return (x + 15) & ~(int64_t)15; }

// Raw buffer access (wave-uniform base and size; out-of-range lanes read zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ll_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 ll_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef int int4v_ __attribute__((ext_vector_type(4)));
  const int4v_ x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4((uint32_t)x.x, (uint32_t)x.y, (uint32_t)x.z, (uint32_t)x.w);
}

// non-zero RZE words the fused encoders counted for chunk k (the sum of its slots)
__device__ __forceinline__ uint32_t chunk_count(const CallDesc& c, int64_t k) {
  const uint4* q = (const uint4*)(c.chunk_counts + k * kNnzSlots);
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < kNnzSlots / 4; ++i) {
    const uint4 x = q[i];
    t += x.x + x.y + x.z + x.w;
  }
  return t;
}

__device__ __forceinline__ uint64_t stream_base(const CallDesc& c, int r, bool encode) {
  if (c.R == 1 && c.req_offsets == nullptr && c.req_offsets_out == nullptr) return 0;
  return encode ? c.req_offsets_out[r] : c.req_offsets[r];
}

// ------------------------------------------------------------------ reset

__device__ void validate_request(const CallDesc& c, int r);

__global__ void k_reset(CallDesc c) {
  Control* ctl = c.ctl;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ctl->status = 0;
    ctl->pad0 = 0;
    ctl->total = 0;
    ctl->pad[0] = 0;   // header-field diagnosis bits
    ctl->pad[1] = 0;   // worklist entries for the general stage engine (from the back)
    ctl->pad[2] = 0;   // tickets of the single-pass placement
    ctl->pad[3] = ~0ull;  // first chunk with placement work (a minimum)
    ctl->pad[4] = 0;   // tickets of the dense scan
    ctl->pad[5] = 0;   // compressed chunks left to the word-parallel decode kernels
    ctl->pad[6] = 0;   // chunks listed for a whole block (front of the worklist)
  }
  if (c.validate_in_reset && blockIdx.x == 0) {
    __syncthreads();                                   // the status word is clear before any check sets it
    if (threadIdx.x < 64) validate_request(c, 0);
  }
  if (c.scan_state && blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i <= c.total_chunks / 1024; i += blockDim.x) c.scan_state[i] = 0;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, di = (int64_t)gridDim.x * blockDim.x;
  // the fused encoders accumulate per-chunk non-zero word counts here
  if (c.nnz_pipe)
    for (int64_t i = i0; i < c.total_chunks * (kNnzSlots / 4); i += di) ((uint4*)c.chunk_counts)[i] = make_uint4(0, 0, 0, 0);
  if (c.place_flags)
    for (int64_t i = i0; i < c.total_chunks + (c.total_chunks + 63) / 64; i += di) c.place_flags[i] = 0;
}

hipError_t launch_reset(const CallDesc& c, hipStream_t s) {
  const bool wide = c.nnz_pipe || c.place;
  const int grid = wide ? (int)std::max<int64_t>(1, std::min<int64_t>((c.total_chunks + 255) / 256, 1024)) : 1;
  k_reset<<<grid, 256, 0, s>>>(c);
  return hipGetLastError();
}

// ------------------------------------------------------------------ block helpers

template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T x, T* sh, T& total) {
  // sh: blockDim.x entries
  const int t = threadIdx.x, nt = blockDim.x;
  sh[t] = x;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    T y = (t >= off) ? sh[t - off] : (T)0;
    __syncthreads();
    sh[t] += y;
    __syncthreads();
  }
  total = sh[nt - 1];
  const T incl = sh[t];
  __syncthreads();
  return incl - x;
}

// Inclusive prefix sum over a wavefront (all lanes active): prefix sums within
// each 16-lane row by DPP row shifts, then the rows joined through the row
// broadcasts of lane 15 and lane 31.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive prefix sum over a block of NW wavefronts (blockDim.x == 64 NW):
// wave scans by DPP, the wave totals through sh[NW]; two barriers.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t x, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan_u32(x);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = sh[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  total = tot;
  __syncthreads();                                   // sh is reused by the next scan
  return before + inc - x;
}

__device__ __forceinline__ uint64_t ld_word(const uint8_t* p, int w) {
  uint64_t v = 0;
  for (int b = 0; b < w; ++b) v |= (uint64_t)p[b] << (8 * b);
  return v;
}
__device__ __forceinline__ void st_word(uint8_t* p, int w, uint64_t v) {
  for (int b = 0; b < w; ++b) p[b] = (uint8_t)(v >> (8 * b));
}

__device__ __forceinline__ int stage_kind(int s) {
  if (s >= KVC_TUPL2_1 && s <= KVC_TUPL8_1) return 0;
  if (s >= KVC_DIFF1 && s <= KVC_DIFF8) return 1;
  if (s >= KVC_BIT_1 && s <= KVC_BIT_8) return 2;
  return 3;
}
__device__ __forceinline__ int stage_width(int s) {
  const int k = stage_kind(s);
  if (k == 0) return 2 << (s - KVC_TUPL2_1);
  if (k == 1) return 1 << (s - KVC_DIFF1);
  if (k == 2) return 1 << (s - KVC_BIT_1);
  return 1 << (s - KVC_RZE_1);
}

// One forward stage, block-cooperative, LDS in -> LDS out.  Returns the output size.
__device__ int stage_forward(int stage, const uint8_t* in, uint8_t* out, int n, uint32_t* sh32) {
  const int kind = stage_kind(stage), w = stage_width(stage);
  const int t = threadIdx.x, nt = blockDim.x;
  if (kind == 0) {
    const int m = n / w;
    for (int p = t; p < n; p += nt) {
      if (p < m * w) { const int j = p / m, i = p - j * m; out[p] = in[i * w + j]; }
      else out[p] = in[p];
    }
    __syncthreads();
    return n;
  }
  if (kind == 1) {
    const int nw = n / w;
    const uint64_t mask = (w == 8) ? ~0ull : ((1ull << (8 * w)) - 1);
    for (int i = t; i < nw; i += nt) {
      const uint64_t cur = ld_word(in + i * w, w);
      const uint64_t prev = i ? ld_word(in + (i - 1) * w, w) : 0ull;
      st_word(out + i * w, w, (cur - prev) & mask);
    }
    for (int p = nw * w + t; p < n; p += nt) out[p] = in[p];
    __syncthreads();
    return n;
  }
  if (kind == 2) {
    const int B = 8 * w, gb = w * B, ng = n / gb;
    for (int o = t; o < ng * B; o += nt) {
      const int g = o / B, j = o - g * B;
      const uint8_t* src = in + g * gb;
      uint64_t acc = 0;
      for (int i = 0; i < B; ++i) acc |= ((ld_word(src + i * w, w) >> j) & 1ull) << i;
      st_word(out + g * gb + j * w, w, acc);
    }
    for (int p = ng * gb + t; p < n; p += nt) out[p] = in[p];
    __syncthreads();
    return n;
  }
  // RZE: each thread owns a contiguous range of words
  const int nw = n / w, bm = (nw + 7) / 8, tail = n - nw * w;
  const int per = (nw + nt - 1) / nt;
  const int i0 = min(nw, t * per), i1 = min(nw, i0 + per);
  uint32_t cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += ld_word(in + i * w, w) != 0ull;
  uint32_t total;
  const uint32_t before = block_exclusive_scan<uint32_t>(cnt, sh32, total);
  // zero elimination is the last stage: a result that does not shrink the
  // chunk means the chunk is stored raw, so nothing is written (and the
  // output buffer cannot overflow)
  if ((int64_t)bm + (int64_t)total * w + tail >= n) return n;
  for (int b = t; b < bm; b += nt) {
    uint32_t byte = 0;
    for (int k = 0; k < 8; ++k) {
      const int i = 8 * b + k;
      if (i < nw && ld_word(in + i * w, w) != 0ull) byte |= 1u << k;
    }
    out[b] = (uint8_t)byte;
  }
  int pos = bm + (int)before * w;
  for (int i = i0; i < i1; ++i) {
    const uint64_t v = ld_word(in + i * w, w);
    if (v) { st_word(out + pos, w, v); pos += w; }
  }
  const int tpos = bm + (int)total * w;
  for (int p = t; p < tail; p += nt) out[tpos + p] = in[nw * w + p];
  __syncthreads();
  return tpos + tail;
}

// Inverse of one stage; n is the decoded length.  Returns false on a corrupt input.
__device__ bool stage_inverse(int stage, const uint8_t* in, int in_n, uint8_t* out, int n,
                              uint32_t* sh32, uint64_t* sh64) {
  const int kind = stage_kind(stage), w = stage_width(stage);
  const int t = threadIdx.x, nt = blockDim.x;
  if (kind != 3 && in_n != n) return false;
  if (kind == 0) {
    const int m = n / w;
    for (int p = t; p < n; p += nt) {
      if (p < m * w) { const int i = p / w, j = p - i * w; out[p] = in[j * m + i]; }
      else out[p] = in[p];
    }
    __syncthreads();
    return true;
  }
  if (kind == 1) {
    const int nw = n / w;
    const uint64_t mask = (w == 8) ? ~0ull : ((1ull << (8 * w)) - 1);
    const int per = (nw + nt - 1) / nt;
    const int i0 = min(nw, t * per), i1 = min(nw, i0 + per);
    uint64_t sum = 0;
    for (int i = i0; i < i1; ++i) sum += ld_word(in + i * w, w);
    uint64_t total;
    uint64_t acc = block_exclusive_scan<uint64_t>(sum, sh64, total);
    for (int i = i0; i < i1; ++i) {
      acc += ld_word(in + i * w, w);
      st_word(out + i * w, w, acc & mask);
    }
    for (int p = nw * w + t; p < n; p += nt) out[p] = in[p];
    __syncthreads();
    return true;
  }
  if (kind == 2) {
    stage_forward(stage, in, out, n, sh32);
    return true;
  }
  const int nw = n / w, bm = (nw + 7) / 8, tail = n - nw * w;
  if (in_n < bm + tail) return false;
  const int per = (nw + nt - 1) / nt;
  const int i0 = min(nw, t * per), i1 = min(nw, i0 + per);
  uint32_t cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += (in[i >> 3] >> (i & 7)) & 1u;
  uint32_t total;
  const uint32_t before = block_exclusive_scan<uint32_t>(cnt, sh32, total);
  // stray bitmap bits past the last word, or a size mismatch, mean corruption
  bool okk = (int)(bm + total * w + tail) == in_n;
  if (bm * 8 > nw) {
    const uint32_t last = in[bm - 1];
    if (last >> (nw - (bm - 1) * 8)) okk = false;
  }
  if (!okk) return false;
  int pos = bm + (int)before * w;
  uint32_t zero_flag = 0;
  for (int i = i0; i < i1; ++i) {
    if ((in[i >> 3] >> (i & 7)) & 1u) {
      const uint64_t v = ld_word(in + pos, w);
      zero_flag |= (v == 0ull);
      st_word(out + i * w, w, v);
      pos += w;
    } else {
      st_word(out + i * w, w, 0ull);
    }
  }
  for (int p = t; p < tail; p += nt) out[nw * w + p] = in[bm + total * w + p];
  const int any_zero = __syncthreads_or((int)zero_flag);
  return any_zero == 0;
}

// ------------------------------------------------------------------ worklist

// Chunks that need the stage engines.  Chunks of the two standard pipelines
// whose size is a multiple of the kernels' block go to the word-parallel
// kernels (entries from the front of the list); all others go to the general
// engine (entries from the back).  The list has one entry per chunk.
__device__ __forceinline__ uint32_t* generic_count(const CallDesc& c) { return (uint32_t*)&c.ctl->pad[1]; }
// Chunks that need a whole block (a reduction or a copy) are listed from the
// front of the worklist by the one-thread-per-chunk classification passes;
// the stage engine's chunks fill it from the back.  A chunk is in at most
// one of the two lists, so they never meet.
__device__ __forceinline__ uint32_t* block_count(const CallDesc& c) { return (uint32_t*)&c.ctl->pad[6]; }
__device__ __forceinline__ void push_block(const CallDesc& c, uint32_t* worklist, int64_t ch) {
  const uint32_t k = __hip_atomic_fetch_add(block_count(c), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  worklist[k] = (uint32_t)ch;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += (uint32_t)__shfl_xor((int)x, o);
  return x;
}

__device__ __forceinline__ int fast_pipeline(const CallDesc& c) {
  if (c.stages[0] == KVC_TUPL8_1 && c.stages[1] == KVC_BIT_8 && c.stages[2] == KVC_RZE_2 && c.stages[3] == 0) return 1;
  if (c.stages[0] == KVC_TUPL8_1 && c.stages[1] == KVC_RZE_2 && c.stages[2] == 0) return 2;
  return 0;
}
__device__ __forceinline__ bool fast_eligible(int pipe, int64_t n) {
  return (pipe == 1 && n % 4096 == 0) || (pipe == 2 && n % 1024 == 0);
}
// a chunk for the stage engine (entries from the back of the list)
__device__ __forceinline__ void push_work(const CallDesc& c, uint32_t* worklist, int64_t ch) {
  const uint32_t k = __hip_atomic_fetch_add(generic_count(c), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  worklist[c.total_chunks - 1 - k] = (uint32_t)ch;
}

// ------------------------------------------------------------------ encode: sizes

// Non-zero 2-byte words after TUPL8_1 -> BIT_8 -> RZE_2, for a full chunk of
// n bytes (n a multiple of 4096).  Word (stream j, block gi, byte kk, bit b,
// quarter u) is zero iff bit b of byte j of the input words
// gi*512 + i*8 + kk, i in [16u, 16u+16), are all zero.
__device__ uint32_t nnz_tupl8_bit8_rze2(const uint64_t* src, int n, uint32_t* sh32) {
  const int nr = (n / 4096) * 32;                 // (gi, u, kk) triples
  uint32_t cnt = 0;
  for (int e = threadIdx.x; e < nr; e += blockDim.x) {
    const int kk = e & 7, u = (e >> 3) & 3, gi = e >> 5;
    uint64_t acc = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc |= src[gi * 512 + (16 * u + i) * 8 + kk];
    cnt += __popcll(acc);
  }
  uint32_t total;
  block_exclusive_scan<uint32_t>(cnt, sh32, total);
  return total;
}

// Non-zero 2-byte words after TUPL8_1 -> RZE_2: word (stream j, pair p) is
// byte j of input words 2p and 2p+1.
__device__ uint32_t nnz_tupl8_rze2(const uint64_t* src, int n, uint32_t* sh32) {
  const int np = n / 16;
  uint32_t cnt = 0;
  for (int p = threadIdx.x; p < np; p += blockDim.x) {
    const uint64_t x = src[2 * p] | src[2 * p + 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) cnt += ((x >> (8 * j)) & 0xffull) != 0ull;
  }
  uint32_t total;
  block_exclusive_scan<uint32_t>(cnt, sh32, total);
  return total;
}

// Encode sizes, one thread per chunk: a counted chunk of a standard pipeline
// gets its size from the fused encoders' counts (raw when that does not
// shrink it); an uncounted one is listed for k_ll_sizes; other pipelines'
// chunks go to the stage engine; with no lossless stage every chunk is raw.
__global__ __launch_bounds__(256) void k_ll_classify_enc(CallDesc c, uint32_t* worklist) {
  const int pipe = fast_pipeline(c);
  for (int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ch < c.total_chunks;
       ch += (int64_t)gridDim.x * blockDim.x) {
    const int r = find_req_by_chunk(c, ch);
    const ReqDesc rq = req_at(c, r);
    const ChunkLoc L = locate_chunk(c, rq, r, ch);
    const int n = (int)L.n;
    if (fast_eligible(pipe, n)) {
      if (c.nnz_pipe == pipe && c.nnz_sec[L.w]) {
        const int64_t size = n / 16 + 2 * (int64_t)chunk_count(c, ch);
        c.chunk_sizes[ch] = (size >= n) ? ((uint32_t)n | kRawFlag) : (uint32_t)size;
      } else {
        push_block(c, worklist, ch);
      }
    } else if (c.stages[0] == 0) {
      c.chunk_sizes[ch] = (uint32_t)n | kRawFlag;
    } else {
      push_work(c, worklist, ch);
    }
  }
}

// The listed chunks' sizes, one block per chunk: the exact non-zero word count
// without the transform (a compressible chunk is encoded by the placement,
// which needs only its size).
__global__ __launch_bounds__(256) void k_ll_sizes(CallDesc c, const uint32_t* worklist) {
  __shared__ uint32_t sh32[256];
  const int pipe = fast_pipeline(c);
  const uint32_t count = __hip_atomic_load(block_count(c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (uint32_t item = blockIdx.x; item < count; item += gridDim.x) {
    const int64_t ch = worklist[item];
    const int r = find_req_by_chunk(c, ch);
    const ReqDesc rq = req_at(c, r);
    const ChunkLoc L = locate_chunk(c, rq, r, ch);
    const int n = (int)L.n;
    const uint64_t* src = (const uint64_t*)(c.codes + L.src);
    const uint32_t nnz = (pipe == 1) ? nnz_tupl8_bit8_rze2(src, n, sh32) : nnz_tupl8_rze2(src, n, sh32);
    const int64_t size = n / 16 + 2 * (int64_t)nnz;
    if (threadIdx.x == 0) c.chunk_sizes[ch] = (size >= n) ? ((uint32_t)n | kRawFlag) : (uint32_t)size;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_ll_encode_generic(CallDesc c, const uint32_t* worklist) {
  __shared__ __attribute__((aligned(16))) uint8_t bufA[65536];
  __shared__ __attribute__((aligned(16))) uint8_t bufB[65536];
  __shared__ uint32_t sh32[256];
  const uint32_t count = *generic_count(c);
  for (uint32_t item = blockIdx.x; item < count; item += gridDim.x) {
    const int64_t ch = worklist[c.total_chunks - 1 - item];
    const int r = find_req_by_chunk(c, ch);
    const ReqDesc rq = req_at(c, r);
    const ChunkLoc L = locate_chunk(c, rq, r, ch);
    const int n = (int)L.n;
    uint8_t* slot = c.codes + L.src;
    for (int p = threadIdx.x; p < n; p += blockDim.x) bufA[p] = slot[p];
    __syncthreads();
    uint8_t* cur = bufA;
    uint8_t* alt = bufB;
    int size = n;
    for (int s = 0; s < 4 && c.stages[s]; ++s) {
      size = stage_forward(c.stages[s], cur, alt, size, sh32);
      uint8_t* tmp = cur; cur = alt; alt = tmp;
    }
    if (size >= n) {
      if (threadIdx.x == 0) c.chunk_sizes[ch] = (uint32_t)n | kRawFlag;
    } else {
      uint8_t* oslot = c.codes_out + L.src;
      for (int p = threadIdx.x; p < size; p += blockDim.x) oslot[p] = cur[p];
      if (threadIdx.x == 0) c.chunk_sizes[ch] = (uint32_t)size;
    }
    __syncthreads();
  }
}


// ------------------------------------------------------------------ word-parallel kernels

// For the two standard pipelines on chunks of n bytes (P1: TUPL8_1 -> BIT_8 ->
// RZE_2, n a multiple of 4096; P2: TUPL8_1 -> RZE_2, n a multiple of 1024)
// the stages reduce to word operations.  With input words w[0 .. n/8) and
// m = n/8:
//  P1: the BIT_8 output is, for every gi < n/4096 and kk < 8, the transpose
//      of the 64x64 bit matrix whose row i is w[512 gi + 8 i + kk]; its row c
//      is the 8-byte word at byte offset (c/8) m + 512 gi + 64 kk + 8 (c%8).
//      The RZE_2 words are the four 16-bit quarters of those rows.
//  P2: the RZE_2 word (j, p), index j m/2 + p, is byte j of w[2p] followed
//      by byte j of w[2p+1].
// Every 32 consecutive RZE words share one bitmap dword.  The placement
// builds the bitmap, scans its popcounts for the word offsets and writes the
// words; the decode kernels below read them back.

// 8x8 transpose of nibbles over each aligned group of 8 lanes: nibble c of
// lane 8 g + r becomes nibble r of lane 8 g + c.  Three rounds swap the
// off-diagonal blocks: 16-bit halves with lane ^ 4, bytes with lane ^ 2
// (one v_perm_b32 each), nibbles with lane ^ 1.
__device__ __forceinline__ uint32_t nibble_xpose8(uint32_t x, int lane) {
  uint32_t p = xchg4(x);
  x = __builtin_amdgcn_perm(p, x, (lane & 4) ? 0x03020706u : 0x05040100u);
  p = xchg2(x);
  x = __builtin_amdgcn_perm(p, x, (lane & 2) ? 0x03070105u : 0x06020400u);
  p = xchg1(x);
  return bfi32((lane & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu, x, rotr32(p, (lane & 1) ? 4u : 28u));
}

// Block scan of the popcounts of nd <= 1024 bitmap dwords: offs[d] = number
// of set bits before dword d; returns the total.  64 NW threads.
template <int NW>
__device__ __forceinline__ uint32_t scan_bitmap(const uint32_t* bm, uint32_t* offs, int nd, uint32_t* sh32) {
  constexpr int PT = 1024 / (64 * NW);               // dwords per thread
  const int t = threadIdx.x;
  uint32_t cnt[PT], sum = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int d = PT * t + i;
    cnt[i] = (d < nd) ? (uint32_t)__builtin_popcount(bm[d]) : 0u;
    sum += cnt[i];
  }
  uint32_t total;
  uint32_t run = block_excl_scan_u32<NW>(sum, sh32, total);
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int d = PT * t + i;
    if (d < nd) offs[d] = run;
    run += cnt[i];
  }
  __syncthreads();
  return total;
}

// Copy nv <= 4096 16-byte lines from global memory to LDS with 64 NW threads:
// every load of a thread is issued before the first LDS store, so a block has
// the whole chunk in flight at once.  Lines past `avail` bytes read as zero.
template <int NW>
__device__ __forceinline__ void stage_lines(const uint4* src, int nv, uint64_t avail, uint4* dst) {
  constexpr int NT = 64 * NW, PT = 4096 / NT;
  uint4 x[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int k = (int)threadIdx.x + NT * u;
    x[u] = make_uint4(0, 0, 0, 0);
    if (k < nv && (uint64_t)(16 * k + 16) <= avail) x[u] = src[k];
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int k = (int)threadIdx.x + NT * u;
    if (k < nv) dst[k] = x[u];
  }
}

// Stage a compressed chunk into LDS and check that its bitmap accounts for
// its length.  Returns false (and flags the stream) if not.
template <int NW>
__device__ __forceinline__ bool load_compressed(const CallDesc& c, uint64_t pos, int stored, int n, uint4* buf,
                                                uint32_t* offs, uint32_t* sh32, uint32_t& nnz) {
  const uint64_t avail = (c.stream_bytes > pos) ? c.stream_bytes - pos : 0;
  const int nv = (stored + 15) / 16;
  const uint4* src = (const uint4*)(c.stream + pos);
  stage_lines<NW>(src, nv, avail, buf);
  __syncthreads();
  // bytes of the last 16-byte line past the stored length are ignored
  if (stored < n / 16) return false;
  nnz = scan_bitmap<NW>((const uint32_t*)buf, offs, n / 64, sh32);
  return n / 16 + 2 * (int)nnz == stored && (uint64_t)(16 * nv) <= avail + 15;
}

// Decode: whether chunk ch is a well-formed compressed chunk of a standard
// pipeline, which the word-parallel kernels decode.  They take every such
// chunk by index (a shared worklist counter would serialize thousands of
// atomics); the stage engine takes the other compressed chunks from its
// worklist.
__device__ __forceinline__ bool wp_decode_chunk(const CallDesc& c, int64_t ch, int pipe, ChunkLoc& L, uint64_t& pos,
                                                int& stored) {
  const int r = find_req_by_chunk(c, ch);
  const ReqDesc rq = req_at(c, r);
  L = locate_chunk(c, rq, r, ch);
  const uint32_t e = c.chunk_sizes[ch];
  stored = (int)(e & 0x7fffffffu);
  if ((e >> 31) || !fast_eligible(pipe, L.n) || c.mirror[L.w]) return false;   // mirror: the reconstruct kernel
  const uint64_t base = c.req_offsets ? c.req_offsets[r] : 0;
  pos = base + (uint64_t)rq.payload_off + (c.chunk_offs[ch] - c.chunk_offs[rq.chunk_begin]);
  return stored < L.n && stored > 0 && pos + (uint64_t)stored <= c.stream_bytes && (pos & 15) == 0;
}

// Waves per block of the placement and of the TUPL8_1 -> RZE_2 decode.  A
// chunk is one block's work; more waves split its 4 KiB (or 1 KiB) pieces
// finer, so a chunk's loads, transposes and stores run on more waves at once.
// Both hold a 64 KiB LDS buffer, so two blocks fit a CU.  Measured on the 70B
// shape with half of the 64-token blocks zero: placement 1.21 ms at 4 waves,
// 0.98 ms at 8 (4 waves per SIMD, a few registers spilled), 1.33 ms at 16 (one
// block per CU).
#ifndef KVC_PLACE_WAVES
#define KVC_PLACE_WAVES 8
#endif
#ifndef KVC_DEC_WAVES
#define KVC_DEC_WAVES 4
#endif

constexpr int kPlaceWaves = KVC_PLACE_WAVES;
constexpr int kPlaceThreads = 64 * kPlaceWaves;
constexpr int kDecWaves = KVC_DEC_WAVES;

// first candidate at or after i (NT when none), the same in every thread
template <int NT>
__device__ __forceinline__ int next_cand(const uint32_t* cand, int i) {
  while (i < NT && !cand[i]) ++i;
  return i;
}

// P1 decode staged in phases.  Output group gi (4 KiB) reads, in every bit
// plane j, the words of bitmap dwords [j dpj + 8 gi, j dpj + 8 gi + 8), so
// the groups [g0, g1) of a phase read one contiguous run of stored words per
// plane.  Only those eight runs are staged (the 16-byte lines that cover
// them, run after run), a phase at a time: a block holds 1/PH of a chunk and
// more blocks fit a CU than with whole chunks, and the next phase's lines
// load while the current one decodes.  A wave's decoded group goes out
// through LDS so that every store instruction writes 1 KiB of whole lines:
// straight from the transposes, each store would cover a quarter of 32
// lines, which measured about 18 % slower with default stores and five
// times slower with non-temporal ones.
#ifndef KVC_P1_PHASES
#define KVC_P1_PHASES 4
#endif
constexpr int kP1Phases = KVC_P1_PHASES;
constexpr int kP1Gpp = 16 / kP1Phases;               // groups per phase of a 64 KiB chunk
// a phase's lines for any bitmap: 256 words per group and plane, two lines of
// slack per run for its unaligned ends
constexpr int kP1SegLines = 32 * kP1Gpp + 2;
constexpr int kP1CapLines = 8 * kP1SegLines;
// LDS per block: the phase's lines, the bitmap and its offsets, and a 4 KiB
// output staging area per wave: about 57 KB (two blocks per CU) at two
// phases, 40 KB (four) at four
constexpr int kP1BlocksPerCu = kP1Phases == 2 ? 2 : 4;
static_assert(kP1Phases == 2 || kP1Phases == 4, "two or four phases");

// The decode reads bitmap dwords j dpj + c and their offsets for the eight
// bit planes j at once; padded by 4 dwords (bitmap) and 8 halfwords (offsets)
// per plane, the eight reads fall on eight different banks.  dpj is a
// multiple of 8, so (dpj + 4) mod 32 is an odd multiple of 4.
__device__ __forceinline__ int bm_pad(int d, int dpj) { return d + 4 * (d / dpj); }
__device__ __forceinline__ int offs_pad(int d, int dpj) { return d + 8 * (d / dpj); }

// bitmap popcount scan into 16-bit offsets (a chunk has at most 32768 words),
// both arrays padded per plane; offs at offs_pad(nd) = total
template <int NW>
__device__ __forceinline__ uint32_t scan_bitmap16(const uint32_t* bm, uint16_t* offs, int nd, int dpj, uint32_t* sh32) {
  constexpr int PT = 1024 / (64 * NW);
  const int t = threadIdx.x;
  const int pj = (PT * t) / dpj;                     // a thread's PT dwords lie in one plane (dpj % PT == 0)
  uint32_t cnt[PT], sum = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int d = PT * t + i;
    cnt[i] = (d < nd) ? (uint32_t)__builtin_popcount(bm[d + 4 * pj]) : 0u;
    sum += cnt[i];
  }
  uint32_t total;
  uint32_t run = block_excl_scan_u32<NW>(sum, sh32, total);
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int d = PT * t + i;
    if (d < nd) offs[d + 8 * pj] = (uint16_t)run;
    run += cnt[i];
  }
  if (t == 0) offs[offs_pad(nd, dpj)] = (uint16_t)total;
  __syncthreads();
  return total;
}

// orders a wave's LDS writes before its lanes read each other's (and those
// reads before the next writes)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// first set flag at or after i in the 64 NW-bit mask m (64 NW when none)
template <int NW>
__device__ __forceinline__ int next_flag(const uint64_t* m, int i) {
  while (i < 64 * NW) {
    const uint64_t x = m[i >> 6] >> (i & 63);
    if (x) return i + (int)__builtin_ctzll(x);
    i = (i | 63) + 1;
  }
  return 64 * NW;
}

template <int NW>
__global__ __launch_bounds__(64 * NW, kP1BlocksPerCu) void k_ll_decode_p1(CallDesc c, const uint32_t* worklist) {
  constexpr int NT = 64 * NW, PH = kP1Phases;
  static_assert(NT == 256, "one bitmap line per thread");
  constexpr int SPT = NT / 8;                          // loader threads per run
  __shared__ __attribute__((aligned(16))) uint4 buf[kP1CapLines + 1];   // a lane reads 3 dwords from its first word's
  __shared__ __attribute__((aligned(16))) uint32_t bm[1024 + 32];   // padded per plane (bm_pad)
  __shared__ uint16_t offs[1024 + 64 + 1];                             // (offs_pad)
  __shared__ __attribute__((aligned(16))) uint4 seg[PH * 8];   // per (phase, plane): first LDS line, first stored line, lines, word shift
  __shared__ uint32_t sh32[NW];
  __shared__ __attribute__((aligned(16))) uint4 nibtab[16];
  __shared__ uint64_t candm[NW];
  // a wave's decoded 4 KiB group, so that its stores cover whole lines: lane i
  // decodes bytes [64 i, 64 i + 64) of the group; store q of lane L writes
  // bytes 1024 q + 16 L.  16-byte slot s of lane i sits at slot s ^ ((i >> 1) & 3)
  // of its 64 bytes, which spreads both access patterns over all banks.
  __shared__ __attribute__((aligned(16))) uint4 ostage[NW * 256];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const XposeLane X = xpose_lane();
  if (threadIdx.x < 16) nibtab[threadIdx.x] = rze_nibble_entry(threadIdx.x);
  if (__hip_atomic_load((const uint32_t*)&c.ctl->pad[5], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) return;
  for (int64_t r0 = 0; (int64_t)blockIdx.x + (int64_t)gridDim.x * r0 < c.total_chunks; r0 += NT) {
    {
      const int64_t mine = (int64_t)blockIdx.x + (int64_t)gridDim.x * (r0 + threadIdx.x);
      ChunkLoc L;
      uint64_t pos;
      int stored;
      const bool f = mine < c.total_chunks && wp_decode_chunk(c, mine, 1, L, pos, stored);
      const uint64_t b = __ballot(f);
      if (lane == 0) candm[wave] = b;
    }
    __syncthreads();
    ChunkLoc L;
    uint64_t pos = 0;
    int stored = 0;
    // x: the lines of a phase in flight, or (x[0]) line threadIdx.x of the next chunk's bitmap
    constexpr int PTL = (kP1SegLines + SPT - 1) / SPT;   // lines per loader thread, at most
    uint4 x[PTL];
    auto load_bitmap = [&]() {
      const uint64_t avail = (c.stream_bytes > pos) ? c.stream_bytes - pos : 0;
      const int t = threadIdx.x;
      x[0] = make_uint4(0, 0, 0, 0);
      if (t < (int)(L.n / 256) && (uint64_t)(16 * t + 16) <= avail) x[0] = ((const uint4*)(c.stream + pos))[t];
    };
    int i = next_flag<NW>(candm, 0);
    if (i < NT) {
      wp_decode_chunk(c, (int64_t)blockIdx.x + (int64_t)gridDim.x * (r0 + i), 1, L, pos, stored);
      load_bitmap();
    }
    while (i < NT) {
      const int n = (int)L.n;
      const int64_t dst0 = L.src;
      const int sc = stored;
      const uint64_t cpos = pos;
      const uint64_t avail = (c.stream_bytes > cpos) ? c.stream_bytes - cpos : 0;
      const int dpj = n / 512;                          // bitmap dwords per bit plane
      if ((int)threadIdx.x < n / 256) *(uint4*)(bm + bm_pad(4 * threadIdx.x, dpj)) = x[0];
      __syncthreads();
      i = next_flag<NW>(candm, i + 1);
      if (i < NT) wp_decode_chunk(c, (int64_t)blockIdx.x + (int64_t)gridDim.x * (r0 + i), 1, L, pos, stored);
      // bytes of the last 16-byte line past the stored length are ignored
      bool ok = sc >= n / 16;
      const int nd = n / 64;
      uint32_t nnz = 0;
      if (ok) {
        nnz = scan_bitmap16<NW>(bm, offs, nd, dpj, sh32);
        ok = n / 16 + 2 * (int)nnz == sc && (uint64_t)(16 * ((sc + 15) / 16)) <= avail + 15;
      }
      if (!ok) {
        if (threadIdx.x == 0) set_status2(c.ctl, kStCorrupt);
        __syncthreads();
        if (i < NT) load_bitmap();
        continue;
      }
      const int ngi = n / 4096;
      const int gpp = (ngi + PH - 1) / PH;
      if (wave == 0) {
        // run of plane j in phase h (lane 8 h + j): words [A, B), lines A / 8 .. (B + 7) / 8
        const int h = lane >> 3, j = lane & 7;
        const int g0 = min(ngi, h * gpp), g1 = min(ngi, g0 + gpp);
        uint32_t A = 0, B = 0;
        if (h < PH) { A = offs[offs_pad(j * dpj + 8 * g0, dpj)]; B = offs[offs_pad(j * dpj + 8 * g1, dpj)]; }
        const uint32_t cnt = (B > A) ? ((B + 7) >> 3) - (A >> 3) : 0u;
        uint32_t s = cnt;
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
          const uint32_t y = (uint32_t)__shfl_up((int)s, o, 8);
          if (j >= o) s += y;
        }
        const uint32_t lb = s - cnt;
        if (h < PH) seg[lane] = make_uint4(lb, A >> 3, cnt, 8u * lb - 8u * (A >> 3));
      }
      __syncthreads();
      const uint4* src = (const uint4*)(c.stream + cpos);
      const uint32_t wline = (uint32_t)(n / 256);        // first line of the words
      auto load_phase = [&](int h) {
        const uint4 sg = seg[8 * h + (int)threadIdx.x / SPT];
        const int k0 = (int)threadIdx.x % SPT;
#pragma unroll
        for (int u = 0; u < PTL; ++u) {
          const int k = k0 + SPT * u;
          const uint32_t l = wline + sg.y + (uint32_t)k;
          x[u] = make_uint4(0, 0, 0, 0);
          if (k < (int)sg.z && (uint64_t)(16 * l + 16) <= avail) x[u] = src[l];
        }
      };
      // A set bitmap bit must mark a non-zero word.  The size check has
      // matched the set bits one to one with the stored words, so that holds
      // when every stored word is non-zero: checked on the staged lines
      // (each line of a run once; words past the last stored one excluded).
      const rze_u16x2 one2 = opaque_one2();
      uint32_t bad = 0;
      auto store_phase = [&](int h) {
        const uint4 sg = seg[8 * h + (int)threadIdx.x / SPT];
        const int k0 = (int)threadIdx.x % SPT;
#pragma unroll
        for (int u = 0; u < PTL; ++u) {
          const int k = k0 + SPT * u;
          if (k < (int)sg.z) {
            buf[sg.x + k] = x[u];
            uint4 y = x[u];
            const int past = 8 * (int)(sg.y + (uint32_t)k) + 8 - (int)nnz;   // words of the line past the end
            if (past > 0) {
              // the chunk's last line: its words from 8 - past on are not stored words
              const uint32_t keep = 8 - past;
              y.x |= keep < 1 ? 0xFFFFu : 0u; y.x |= keep < 2 ? 0xFFFF0000u : 0u;
              y.y |= keep < 3 ? 0xFFFFu : 0u; y.y |= keep < 4 ? 0xFFFF0000u : 0u;
              y.z |= keep < 5 ? 0xFFFFu : 0u; y.z |= keep < 6 ? 0xFFFF0000u : 0u;
              y.w |= keep < 7 ? 0xFFFFu : 0u; y.w |= 0xFFFF0000u;
            }
            bad |= (nz_halves(y.x, one2) & nz_halves(y.y, one2) & nz_halves(y.z, one2) & nz_halves(y.w, one2)) ^
                   0x00010001u;
          }
        }
      };
      const uint32_t* buf32 = (const uint32_t*)buf;
      const int j = lane >> 3, bb = lane & 7;
      const uint32_t below = (1u << (4 * bb)) - 1u;     // bitmap bits of the nibbles before this lane's
      load_phase(0);
#pragma unroll 1
      for (int h = 0; h < PH; ++h) {
        store_phase(h);
        __syncthreads();
        if (h + 1 < PH) load_phase(h + 1);
        else if (i < NT) load_bitmap();                   // the next chunk's bitmap goes out now
        const uint32_t shift = seg[8 * h + j].w;         // stored word index -> LDS word index
        const int g1 = min(ngi, h * gpp + gpp);
        for (int gi = h * gpp + wave; gi < g1; gi += NW) {
          uint4* os = ostage + 256 * wave;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
          uint32_t w[4], wl[2], wh[2];
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int kk = 2 * q + k2;
            const int d = 8 * gi + kk;                      // within plane j
            const uint32_t bits = bm[j * (dpj + 4) + d];
            const uint32_t nib = (bits >> (4 * bb)) & 15u;
            // index of the nibble's first non-zero word; every word this
            // nibble can mark lies in the phase's run of plane j
            const uint32_t rr = (uint32_t)offs[j * (dpj + 8) + d] + (uint32_t)__builtin_popcount(bits & below);
            const uint32_t di = min((rr + shift) >> 1, 4u * (uint32_t)kP1CapLines + 1u);
            const uint32_t d0 = buf32[di], d1 = buf32[di + 1], d2 = buf32[di + 2];
            const uint32_t sh = (rr & 1u) << 4;
            const uint32_t p01 = __builtin_amdgcn_alignbit(d1, d0, sh), p23 = __builtin_amdgcn_alignbit(d2, d1, sh);
            const uint4 e = nibtab[nib];
            uint32_t lo = __builtin_amdgcn_perm(p23, p01, e.x), hi = __builtin_amdgcn_perm(p23, p01, e.y);
            wl[k2] = lo;
            wh[k2] = hi;
          }
          xpose64_n<2>(wl, wh, X);
          w[0] = wl[0]; w[1] = wh[0]; w[2] = wl[1]; w[3] = wh[1];
          os[4 * lane + (q ^ ((lane >> 1) & 3))] = make_uint4(w[0], w[1], w[2], w[3]);
          }
          wave_lds_sync();
          uint4* dst = (uint4*)(c.codes + dst0 + (int64_t)gi * 4096);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i2 = 16 * q + (lane >> 2), s2 = lane & 3;
            dst[64 * q + lane] = os[4 * i2 + (s2 ^ ((i2 >> 1) & 3))];
          }
          wave_lds_sync();                                 // the next group's writes follow these reads
        }
        if (h + 1 < PH) __syncthreads();                 // the block is done with this phase's lines
      }
      // a set bitmap bit must mark a non-zero word (and the block is done with buf, bm, offs)
      if (__syncthreads_or((int)bad) && threadIdx.x == 0) set_status2(c.ctl, kStCorrupt);
    }
    __syncthreads();                                   // candm is rewritten next round
  }
}

template <int NW>
__global__ __launch_bounds__(64 * NW, NW / 2 < 4 ? NW / 2 : 4) void k_ll_decode_p2(CallDesc c, const uint32_t* worklist) {
  constexpr int NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) uint4 buf[4096];
  __shared__ uint32_t offs[1024];
  __shared__ uint32_t sh32[NW];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // this block's chunks are blockIdx.x + gridDim.x * i; NT at a time are
  // checked in parallel and the block then works through those to decode
  __shared__ uint32_t cand[NT];
  // nothing to decode (e.g. every chunk raw): leave at once
  if (__hip_atomic_load((const uint32_t*)&c.ctl->pad[5], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) return;
  for (int64_t r0 = 0; (int64_t)blockIdx.x + (int64_t)gridDim.x * r0 < c.total_chunks; r0 += NT) {
  {
    const int64_t mine = (int64_t)blockIdx.x + (int64_t)gridDim.x * (r0 + threadIdx.x);
    ChunkLoc L;
    uint64_t pos;
    int stored;
    cand[threadIdx.x] = (mine < c.total_chunks && wp_decode_chunk(c, mine, 2, L, pos, stored)) ? 1u : 0u;
  }
  __syncthreads();
  for (int i = 0; i < NT; ++i) {
    if (!cand[i]) continue;
    const int64_t ch = (int64_t)blockIdx.x + (int64_t)gridDim.x * (r0 + i);
    ChunkLoc L;
    uint64_t pos;
    int stored;
    wp_decode_chunk(c, ch, 2, L, pos, stored);
    const int n = (int)L.n;
    uint32_t nnz = 0;
    const bool ok = load_compressed<NW>(c, pos, stored, n, buf, offs, sh32, nnz);
    if (!ok) {
      if (threadIdx.x == 0) set_status2(c.ctl, kStCorrupt);
      __syncthreads();
      continue;
    }
    const uint32_t* bm = (const uint32_t*)buf;
    const uint16_t* words = (const uint16_t*)buf + n / 32;
    const int nblk = n / 1024, dpj = n / 512;
    const int rr = lane & 31;
    uint32_t bad = 0;
    for (int blk = wave; blk < nblk; blk += NW) {
      uint32_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = j * dpj + 2 * blk + (lane >> 5);
        const uint32_t bits = bm[d];
        const uint32_t set = (bits >> rr) & 1u;
        const uint32_t rk = offs[d] + (uint32_t)__builtin_popcount(bits & ((1u << rr) - 1u));
        const uint32_t x = set ? (uint32_t)words[min(rk, nnz - 1u)] : 0u;
        bad |= set & (uint32_t)(x == 0u);
        v[j] = x;
      }
      // byte j of w[2p] is the low byte of word j, byte j of w[2p+1] its high byte
      const uint32_t p01 = v[0] | (v[1] << 16), p23 = v[2] | (v[3] << 16);
      const uint32_t p45 = v[4] | (v[5] << 16), p67 = v[6] | (v[7] << 16);
      uint4 x;
      x.x = __builtin_amdgcn_perm(p23, p01, 0x06040200u);
      x.y = __builtin_amdgcn_perm(p67, p45, 0x06040200u);
      x.z = __builtin_amdgcn_perm(p23, p01, 0x07050301u);
      x.w = __builtin_amdgcn_perm(p67, p45, 0x07050301u);
      ((uint4*)(c.codes + L.src))[64 * blk + lane] = x;
    }
    if (__syncthreads_or((int)bad) && threadIdx.x == 0) set_status2(c.ctl, kStCorrupt);
  }
  __syncthreads();                                   // cand is rewritten next round
  }
}

// Whether every chunk of a one-request call goes to the word-parallel
// kernels (a standard pipeline, and every chunk size a multiple of its
// block): then the stage engine's worklist stays empty and it is not launched.
bool all_word_parallel(const CallDesc& c) {
  const bool p1 = c.stages[0] == KVC_TUPL8_1 && c.stages[1] == KVC_BIT_8 && c.stages[2] == KVC_RZE_2 && c.stages[3] == 0;
  const bool p2 = c.stages[0] == KVC_TUPL8_1 && c.stages[1] == KVC_RZE_2 && c.stages[2] == 0;
  if (c.R != 1 || !(p1 || p2)) return false;
  const int64_t blk = p1 ? 4096 : 1024;
  for (int w = 0; w < 2; ++w) {
    const int64_t cb = c.one.codes_bytes[w];
    if (cb == 0) continue;
    const int64_t last = cb - (int64_t)(c.one.nchunks[w] - 1) * c.chunk_bytes;
    if (last % blk) return false;
  }
  return true;
}

hipError_t launch_lossless_encode(const CallDesc& c, hipStream_t s) {
  if (c.total_chunks == 0) return hipSuccess;
  uint32_t* worklist = (uint32_t*)(c.chunk_offs + c.total_chunks + 1);
  k_ll_classify_enc<<<(int)std::min<int64_t>((c.total_chunks + 255) / 256, 4096), 256, 0, s>>>(c, worklist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_ll_sizes<<<(int)std::min<int64_t>(c.total_chunks, 256 * 8), 256, 0, s>>>(c, worklist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (all_word_parallel(c)) return hipSuccess;
  k_ll_encode_generic<<<(int)std::min<int64_t>(c.total_chunks, 512), 256, 0, s>>>(c, worklist);
  return hipGetLastError();
}

// ------------------------------------------------------------------ scan

// Exclusive scan of align16(stored size) over all chunks of a call (one
// request or many, the requests' chunks one after another), one block per
// 1024 chunks, chained by decoupled look-back: a block publishes its sum,
// then walks back over earlier blocks' words (sum, or running total once a
// block has one) until it meets a running total.  Blocks take their index
// from a ticket counter in the order they start, so a block waits only on
// blocks already running; the wait is bounded all the same (kStStall).  For
// decode the stored sizes come from the streams' chunk tables (bounds
// checked) and are copied to chunk_sizes.  A dense encode also gets the first
// chunk that is not raw at its all-raw place (the minimum over blocks) for
// the placement.
constexpr int kScanPer = 1024;
constexpr uint64_t kLbAgg = 1ull << 62, kLbIncl = 2ull << 62, kLbVal = (1ull << 62) - 1;

__global__ __launch_bounds__(256) void k_scan_chunks(CallDesc c, int from_table) {
  __shared__ uint32_t sh32[4];
  __shared__ int64_t sb[2];
  const int t = threadIdx.x;
  const int64_t N = c.total_chunks;
  if (t == 0) sb[0] = (int64_t)__hip_atomic_fetch_add((uint32_t*)&c.ctl->pad[4], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int64_t vb = sb[0];
  const int64_t k0 = vb * kScanPer + 4 * t;
  // the request of each of the thread's chunks (consecutive)
  int r = (k0 < N) ? find_req_by_chunk(c, k0) : 0;
  ReqDesc rq = req_at(c, r);
  uint32_t e[4];
  uint64_t sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t k = k0 + i;
    e[i] = 0;
    if (k < N) {
      while (r + 1 < c.R && k >= rq.chunk_begin + rq.nchunks[0] + rq.nchunks[1]) rq = req_at(c, ++r);
      if (from_table) {
        const uint64_t base = c.req_offsets ? c.req_offsets[r] : 0;
        const uint64_t pos = base + (uint64_t)rq.table_off + 4 * (uint64_t)(k - rq.chunk_begin);
        if (pos + 4 <= c.stream_bytes && pos + 4 <= base + (uint64_t)rq.payload_off) e[i] = *(const uint32_t*)(c.stream + pos);
        else set_status2(c.ctl, kStCorrupt);
        c.chunk_sizes[k] = e[i];
      } else if (c.counts_to_sizes) {
        // a counted chunk of a standard pipeline: its encoded size, or raw
        // when that does not shrink it (the size pass's rule)
        const int64_t n = locate_chunk(c, rq, r, k).n;
        const int64_t size = n / 16 + 2 * (int64_t)chunk_count(c, k);
        e[i] = (size >= n) ? ((uint32_t)n | kRawFlag) : (uint32_t)size;
        c.chunk_sizes[k] = e[i];
      } else {
        e[i] = c.chunk_sizes[k];
      }
    }
    sum += (uint64_t)align16(e[i] & 0x7fffffffu);
  }
  // a block's 1024 chunks hold at most 64 MiB: the block-local scan fits 32 bits
  uint32_t agg32;
  const uint64_t ex = block_excl_scan_u32<4>((uint32_t)sum, sh32, agg32);
  const uint64_t agg = agg32;
  if (t == 0) {
    uint64_t* st = c.scan_state;
    uint64_t prefix = 0;
    if (vb == 0) {
      __hip_atomic_store(st, kLbIncl | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __hip_atomic_store(st + vb, kLbAgg | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int64_t j = vb - 1; j >= 0; --j) {
        uint64_t w = __hip_atomic_load(st + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (w == 0) {
          const uint64_t t0 = wall_clock64();
          while ((w = __hip_atomic_load(st + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0) {
            if (wall_clock64() - t0 > (1ull << 27)) break;
            __builtin_amdgcn_s_sleep(2);
          }
          if (w == 0) { set_status2(c.ctl, kStStall); break; }
        }
        prefix += w & kLbVal;
        if (w & kLbIncl) break;
      }
      __hip_atomic_store(st + vb, kLbIncl | (prefix + agg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sb[1] = (int64_t)prefix;
  }
  __syncthreads();
  uint64_t acc = (uint64_t)sb[1] + ex;
  int64_t first_work = N;
  // the placement's first chunk that is not raw at its all-raw place
  // (positions relative to c.codes: dense, the payload; paged, the output)
  const bool track = !from_table && c.place != 0;
  r = (k0 < N) ? find_req_by_chunk(c, k0) : 0;
  rq = req_at(c, r);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t k = k0 + i;
    if (k < N) {
      c.chunk_offs[k] = acc;
      if (track && first_work == N) {
        while (r + 1 < c.R && k >= rq.chunk_begin + rq.nchunks[0] + rq.nchunks[1]) rq = req_at(c, ++r);
        const uint64_t fin = (c.place == 2 ? (uint64_t)(rq.fixed_before + rq.payload_off) : 0) + acc;
        if (!((e[i] >> 31) && fin == (uint64_t)locate_chunk(c, rq, r, k).src)) first_work = k;
      }
      acc += (uint64_t)align16(e[i] & 0x7fffffffu);
    }
  }
  if (track && first_work < N)
    __hip_atomic_fetch_min(&c.ctl->pad[3], (uint64_t)first_work, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t == 0 && (vb + 1) * kScanPer >= N) {
    const uint64_t total = (uint64_t)sb[1] + agg;
    c.chunk_offs[N] = total;
    if (!from_table && c.req_offsets_out == nullptr) c.ctl->total = (uint64_t)c.one.payload_off + total;
  }
}

// Paged encode, after the chunk scan: each request's stream size (its fixed
// sections plus its chunks' aligned sizes) scanned into req_offsets_out, and
// the call's total.
__global__ __launch_bounds__(1024) void k_req_offsets(CallDesc c) {
  __shared__ uint64_t sh[1024];
  const int t = threadIdx.x, nt = blockDim.x;
  const int R = c.R;
  const int rper = (R + nt - 1) / nt;
  const int r0 = min(R, t * rper), r1 = min(R, r0 + rper);
  auto size_of = [&](int r) {
    const ReqDesc rq = req_at(c, r);
    const int64_t cend = rq.chunk_begin + rq.nchunks[0] + rq.nchunks[1];
    return (uint64_t)rq.payload_off + (c.chunk_offs[cend] - c.chunk_offs[rq.chunk_begin]);
  };
  uint64_t rs = 0;
  for (int r = r0; r < r1; ++r) rs += size_of(r);
  uint64_t rtotal;
  uint64_t racc = block_exclusive_scan<uint64_t>(rs, sh, rtotal);
  for (int r = r0; r < r1; ++r) {
    c.req_offsets_out[r] = racc;
    racc += size_of(r);
  }
  if (t == 0) { c.req_offsets_out[R] = rtotal; c.ctl->total = rtotal; }
}

hipError_t launch_scan(const CallDesc& c, bool from_table, hipStream_t s) {
  const int64_t nb = std::max<int64_t>(1, (c.total_chunks + kScanPer - 1) / kScanPer);
  k_scan_chunks<<<(int)nb, 256, 0, s>>>(c, from_table ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || from_table || c.req_offsets_out == nullptr) return e;
  k_req_offsets<<<1, 1024, 0, s>>>(c);
  return hipGetLastError();
}


// ------------------------------------------------------------------ compaction

__device__ void write_header(const CallDesc& c, const ReqDesc& rq, uint8_t* o, uint64_t total) {
  // threads 0..63 of the block each write one byte
  const int t = threadIdx.x;
  if (t >= 64) return;
  uint8_t b = 0;
  auto byte_of = [](uint64_t v, int k) { return (uint8_t)(v >> (8 * k)); };
  if (t < 4) b = byte_of(kMagic, t);
  else if (t < 6) b = byte_of(1, t - 4);
  else if (t == 6) b = (uint8_t)c.dtype;
  else if (t == 7) b = c.mixed ? 1 : 0;              // flags: bit 0 = mixed precision
  else if (t < 12) b = byte_of((uint32_t)c.layers, t - 8);
  else if (t < 16) b = byte_of((uint32_t)rq.T, t - 12);
  else if (t < 20) b = byte_of((uint32_t)c.heads, t - 16);
  else if (t < 24) b = byte_of((uint32_t)kHeadDim, t - 20);
  else if (t < 40) {
    const int w = (t - 24) / 8, k = (t - 24) % 8;
    const TensorPol& p = c.pol[w];
    if (k == 0) b = (uint8_t)p.bits;
    else if (k == 1) b = (uint8_t)p.axis;
    else if (k == 2) b = (uint8_t)p.hadamard;
    else if (k == 4) b = byte_of((uint32_t)p.group, 0);
    else if (k == 5) b = byte_of((uint32_t)p.group, 1);
    else if (k == 6) b = byte_of((uint32_t)p.delta, 0);
    else if (k == 7) b = byte_of((uint32_t)p.delta, 1);
  } else if (t < 48) b = byte_of(c.seed, t - 40);
  else if (t < 52) b = c.stages[t - 48];
  else if (t < 56) b = byte_of(c.chunk_bytes, t - 52);
  else b = byte_of(total, t - 56);
  o[t] = b;
}

// zero the alignment gaps between table, parameter sections and payload; a
// mixed-precision stream also gets its width map after the header
__device__ void zero_gaps(const CallDesc& c, const ReqDesc& rq, uint8_t* o) {
  const int64_t tend = rq.table_off + 4 * (int64_t)(rq.nchunks[0] + rq.nchunks[1]);
  const int64_t mapn = c.mixed ? 2 * (int64_t)c.layers * c.heads : 0;
  for (int64_t p = threadIdx.x; p < mapn; p += blockDim.x) o[64 + p] = c.width_map[p];
  const int64_t g0[4] = {64 + mapn, tend, rq.params_off[0] + rq.params_bytes[0], rq.params_off[1] + rq.params_bytes[1]};
  const int64_t g1[4] = {rq.table_off, rq.params_off[0], rq.params_off[1], rq.payload_off};
  for (int k = 0; k < 4; ++k)
    for (int64_t p = g0[k] + threadIdx.x; p < g1[k]; p += blockDim.x) o[p] = 0;
}

__device__ __forceinline__ int find_req_by_piece(const CallDesc& c, int64_t piece) {
  int lo = 0, hi = c.R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (c.reqs[mid].piece_begin <= piece) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void k_compact(CallDesc c) {
  const int64_t items = c.total_chunks + c.R + c.total_pieces;
  if (c.place == 2) {
    // the chunk tables of a paged encode, after its placement
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < c.total_chunks;
         k += (int64_t)gridDim.x * blockDim.x) {
      const int r = find_req_by_chunk(c, k);
      const ReqDesc rq = req_at(c, r);
      *(uint32_t*)(c.stream + stream_base(c, r, true) + rq.table_off + 4 * (k - rq.chunk_begin)) = c.chunk_sizes[k];
    }
  }
  // with the paged placement (place == 2) the chunks are placed there
  for (int64_t it = blockIdx.x + (c.place == 2 ? c.total_chunks : 0); it < items; it += gridDim.x) {
    if (it < c.total_chunks) {
      const int64_t ch = it;
      const int r = find_req_by_chunk(c, ch);
      const ReqDesc rq = req_at(c, r);
      const ChunkLoc L = locate_chunk(c, rq, r, ch);
      const uint32_t e = c.chunk_sizes[ch];
      const int64_t stored = e & 0x7fffffffu;
      const uint64_t base = stream_base(c, r, true);
      uint8_t* out = c.stream + base;
      const uint64_t fin = c.chunk_offs[ch] - c.chunk_offs[rq.chunk_begin];
      uint8_t* dst = out + rq.payload_off + fin;
      const uint8_t* src = c.codes + L.src;
      if (c.codes_out != c.codes) {
        // codes were written where an all-raw stream keeps them: a raw chunk
        // whose offset did not change is in place (only its alignment padding
        // is written); every other chunk comes from the staging area
        if ((e >> 31) && fin == (uint64_t)L.src) {
          const int64_t pad = align16(stored) - stored;
          if (threadIdx.x < pad) dst[stored + threadIdx.x] = 0;
          if (threadIdx.x == 0) *(uint32_t*)(out + rq.table_off + 4 * (ch - rq.chunk_begin)) = e;
          continue;
        }
        src = c.codes_out + L.src;
      }
      const int64_t nv = align16(stored) / 16;
      for (int64_t k = threadIdx.x; k < nv; k += blockDim.x) {
        uint4 x = ((const uint4*)src)[k];
        const int64_t lim = stored - 16 * k;
        if (lim < 16) {
          uint8_t* xb = (uint8_t*)&x;
          for (int b = 0; b < 16; ++b) if (b >= lim) xb[b] = 0;
        }
        ((uint4*)dst)[k] = x;
      }
      if (threadIdx.x == 0) *(uint32_t*)(out + rq.table_off + 4 * (ch - rq.chunk_begin)) = e;
    } else if (it < c.total_chunks + c.R) {
      const int r = (int)(it - c.total_chunks);
      const ReqDesc rq = req_at(c, r);
      const uint64_t base = stream_base(c, r, true);
      const uint64_t total = (c.req_offsets_out != nullptr) ? c.req_offsets_out[r + 1] - c.req_offsets_out[r]
                                                            : c.ctl->total;
      write_header(c, rq, c.stream + base, total);
      zero_gaps(c, rq, c.stream + base);
    } else {
      const int64_t piece = it - c.total_chunks - c.R;
      const int r = find_req_by_piece(c, piece);
      const ReqDesc rq = req_at(c, r);
      int64_t k = piece - rq.piece_begin;
      const int64_t p0 = (rq.params_bytes[0] + 65535) / 65536;
      const int w = (k < p0) ? 0 : 1;
      if (w == 1) k -= p0;
      const int64_t off = k * 65536;
      const int64_t len = min<int64_t>(65536, rq.params_bytes[w] - off);
      // both ends are 16-byte aligned (256-byte staging offsets, 16-byte
      // sections and streams): 16-byte lines, then the last dwords
      const uint32_t* src = (const uint32_t*)(c.params_ws + rq.params_ws_off[w] + off);
      uint32_t* dst = (uint32_t*)(c.stream + stream_base(c, r, true) + rq.params_off[w] + off);
      const int64_t n16 = len / 16;
      for (int64_t i = threadIdx.x; i < n16; i += blockDim.x) ((uint4*)dst)[i] = ((const uint4*)src)[i];
      for (int64_t i = 4 * n16 + threadIdx.x; i < len / 4; i += blockDim.x) dst[i] = src[i];
    }
  }
}

hipError_t launch_compact(const CallDesc& c, hipStream_t s) {
  const int64_t items = c.total_chunks + c.R + c.total_pieces;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(items, 256 * 16));
  k_compact<<<grid, 256, 0, s>>>(c);
  return hipGetLastError();
}

// ------------------------------------------------------------------ single-pass placement

// Dense encode, after the sizes and their scan: one in-place pass writes every
// chunk to its final offset.  The fused encoders left the codes where a stream
// whose chunks are all raw keeps them, so a raw chunk whose offset did not
// change needs nothing; a chunk of TUPL8_1 -> BIT_8 -> RZE_2 (whole 4 KiB
// blocks) or TUPL8_1 -> RZE_2 (whole 1 KiB blocks) is read once, transformed
// in registers, assembled in LDS and written once; a raw chunk that moves is
// read into LDS and written; a chunk the stage engines encoded (other
// pipelines, partial chunks) is copied from the staging area.  A chunk's final offset never exceeds its codes' offset,
// so its output can only cover codes of itself and of earlier chunks.  Blocks
// take chunks in index order from a ticket counter (the leading raw chunks
// that keep their place, found by the scan, go 64 to a ticket and need only
// their table entries); every chunk announces once it has read its codes (a
// raw chunk at its place needs none), and a chunk writes only
// after all earlier chunks whose codes its output covers have announced.  A
// chunk waits only on earlier chunks, whose blocks already run, so the waits
// end; they are bounded all the same (kStStall, and every later write is
// skipped).  The last ticket writes the header and the gaps between the
// sections.
// Bound of one wait, in ticks of the 100 MHz real-time counter (about 1.3 s).
constexpr uint64_t kPlaceWaitTicks = 1ull << 27;

__device__ __forceinline__ uint32_t ld_flag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// first chunk whose codes end after payload offset `fin` (dense stream)
__device__ __forceinline__ int64_t first_covered(const CallDesc& c, uint64_t fin) {
  const ReqDesc& rq = c.one;
  if ((int64_t)fin < rq.codes_bytes[0]) return (int64_t)(fin / c.chunk_bytes);
  if ((int64_t)fin < rq.codes_off[1]) return rq.nchunks[0];
  return rq.nchunks[0] + (int64_t)((fin - (uint64_t)rq.codes_off[1]) / c.chunk_bytes);
}

// first chunk whose codes, at their all-raw places, end after position `pos`
// of the output buffer (paged encode)
__device__ __forceinline__ int64_t first_covered_paged(const CallDesc& c, uint64_t pos) {
  int lo = 0, hi = c.R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((uint64_t)c.reqs[mid].raw_base <= pos) lo = mid; else hi = mid - 1;
  }
  const ReqDesc rq = req_at(c, lo);
  const int64_t rel = (int64_t)pos - rq.codes_off[0];       // from the request's K codes
  if (rel < 0) return rq.chunk_begin;
  if (rel < rq.codes_bytes[0]) return rq.chunk_begin + rel / c.chunk_bytes;
  const int64_t v0 = rq.codes_off[1] - rq.codes_off[0];
  if (rel < v0) return rq.chunk_begin + rq.nchunks[0];
  return rq.chunk_begin + rq.nchunks[0] + min((rel - v0) / (int64_t)c.chunk_bytes, (int64_t)rq.nchunks[1]);
}

// Block-wide: wait until every chunk in [j0, k) has announced.  Whole groups
// of 64 chunks are checked through their counters, the ragged ends chunk by
// chunk.  Returns false if a wait ran out or an earlier one did (kStStall).
__device__ bool wait_announced(const CallDesc& c, const uint32_t* ann, const uint32_t* grp, int64_t j0, int64_t k) {
  bool ok = true;
  if (j0 < k) {
    const int64_t ga = (j0 + 63) >> 6, gb = k >> 6;
    const int64_t h1 = min(k, ga * 64);                  // head chunks [j0, h1)
    const int64_t ng = (ga < gb) ? gb - ga : 0;          // groups [ga, gb)
    const int64_t t0 = max(h1, gb * 64);                 // tail chunks [t0, k)
    const int64_t nh = h1 - j0, nt = k - t0, items = nh + ng + nt;
    for (int64_t i = threadIdx.x; i < items && ok; i += blockDim.x) {
      const uint32_t* f;
      uint32_t want;
      if (i < nh) { f = ann + j0 + i; want = 1; }
      else if (i < nh + ng) { f = grp + ga + (i - nh); want = 64; }
      else { f = ann + t0 + (i - nh - ng); want = 1; }
      if (ld_flag(f) >= want) continue;
      const uint64_t t_start = wall_clock64();
      while (ld_flag(f) < want) {
        if ((ld_flag(&c.ctl->status) & kStStall) || wall_clock64() - t_start > kPlaceWaitTicks) { ok = false; break; }
        __builtin_amdgcn_s_sleep(2);
      }
    }
  }
  return __syncthreads_and(ok ? 1 : 0) != 0;
}

// PIPE: the plan's pipeline when it is one of the two encoded here (1:
// TUPL8_1 -> BIT_8 -> RZE_2, 2: TUPL8_1 -> RZE_2), else 0; one instantiation
// each, so none carries the other's registers.  NW waves per block.
// One chunk of the placement (dense: k at or past the first chunk with work,
// in ticket order; paged: any order, written to the request's own stream).
template <int PIPE, bool PAGED, int NW>
__device__ __forceinline__ void place_chunk(const CallDesc& c, int64_t k, int64_t kf, uint32_t* ann, uint32_t* grp,
                                            const XposeLane& X, int wave, int lane, uint32_t* ob, uint32_t* bm,
                                            uint32_t* offs, uint32_t* sh32, const uint2* cmptab) {
  constexpr int pipe = PIPE;
  constexpr int NS = 16 / NW;                          // 4 KiB blocks per wave (mode 2)
  constexpr int NU = 64 / NW;                          // 1 KiB blocks per wave (mode 4)
  const int r = PAGED ? find_req_by_chunk(c, k) : 0;
  const ReqDesc rq = req_at(c, r);
  const ChunkLoc L = locate_chunk(c, rq, r, k);
  const uint32_t e = c.chunk_sizes[k];
  const int64_t stored = e & 0x7fffffffu;
  // final position relative to c.codes (dense: the payload; paged: the output
  // buffer, whose request r starts at fixed_before + chunk_offs[chunk_begin])
  const uint64_t fin = (PAGED ? (uint64_t)(rq.fixed_before + rq.payload_off) : 0) + c.chunk_offs[k];
  uint8_t* dst = c.codes + fin;
  const uint8_t* slot = c.codes + L.src;
  // 0: raw, in place; 1: raw, moves; 2: TUPL8_1 -> BIT_8 -> RZE_2 here;
  // 3: from the staging area; 4: TUPL8_1 -> RZE_2 here
  const int mode = (e >> 31) ? ((fin == (uint64_t)L.src) ? 0 : 1)
                             : ((pipe == 0 || !fast_eligible(pipe, L.n)) ? 3 : (pipe == 1 ? 2 : 4));
  const int n = (int)L.n;
  const int ngi = n >> 12, nd = n >> 6, dpj = n >> 9;
  // R: this lane's 64 bytes of each of the wave's pieces of the chunk.
  // Mode 2: R[16 s4 .. 16 s4 + 15] = bytes 64 lane .. 64 lane + 63 of 4 KiB
  // block gi = wave + NW s4, input word 8 lane + kk at R[16 s4 + 2 kk],
  // transposed there in place.  Mode 4: R[4 u .. 4 u + 3] = 16-byte unit
  // `lane` of 1 KiB block wave + NW u.
  uint32_t R[16 * NS];
  if (mode == 4) {
    // every load first, so the whole chunk is in flight at once: buffer
    // loads with one lane offset and wave-uniform block offsets (blocks past
    // the chunk read zero)
    const __amdgpu_buffer_rsrc_t rs = ll_rsrc(slot, (uint32_t)n);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const uint4 x = ll_load16(rs, 16u * (uint32_t)lane, 1024u * (uint32_t)(wave + NW * u));
      R[4 * u] = x.x; R[4 * u + 1] = x.y; R[4 * u + 2] = x.z; R[4 * u + 3] = x.w;
    }
  }
  if (mode == 2) {
    const rze_u16x2 one2 = opaque_one2();
#pragma unroll
    for (int s4 = 0; s4 < NS; ++s4) {
      const int gi = wave + NW * s4;
      if (gi < ngi) {
        // block by block (measured faster than issuing all of a wave's loads first)
        const uint4* src = (const uint4*)(slot + (int64_t)gi * 4096 + 64 * lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 x = src[q];
          R[16 * s4 + 4 * q] = x.x; R[16 * s4 + 4 * q + 1] = x.y; R[16 * s4 + 4 * q + 2] = x.z; R[16 * s4 + 4 * q + 3] = x.w;
        }
        uint32_t qs = 0;                                 // nibble kk: non-zero words of this lane's row kk
#pragma unroll
        for (int k2 = 0; k2 < 8; k2 += 2) {
          uint32_t lo[2] = {R[16 * s4 + 2 * k2], R[16 * s4 + 2 * k2 + 2]};
          uint32_t hi[2] = {R[16 * s4 + 2 * k2 + 1], R[16 * s4 + 2 * k2 + 3]};
          xpose64_n<2>(lo, hi, X);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int kk = k2 + u;
            R[16 * s4 + 2 * kk] = lo[u];
            R[16 * s4 + 2 * kk + 1] = hi[u];
            qs |= nz_quarters(lo[u], hi[u], one2) << (4 * kk);
          }
        }
        // bitmap dword (j, kk) is nibble kk of lanes 8 j + bb, bb = 0..7, placed
        // at nibble bb: after the transpose lane 8 j + kk holds it
        bm[(lane >> 3) * dpj + 8 * gi + (lane & 7)] = nibble_xpose8(qs, lane);
      }
    }
  } else if (mode == 4) {
    // RZE word (j, p) is byte j of input words 2 p and 2 p + 1; lane `lane`
    // of block blk holds pair p = 64 blk + lane, and the 64 pairs of a block
    // and byte j make two bitmap dwords (ballot)
    const int nblk = n >> 10;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int blk = wave + NW * u;
      if (blk < nblk) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t a = (j < 4) ? R[4 * u] : R[4 * u + 1], b = (j < 4) ? R[4 * u + 2] : R[4 * u + 3];
          const uint32_t jj = (uint32_t)(j & 3);
          const uint32_t word = __builtin_amdgcn_perm(b, a, 0x0C0C0000u | ((4u + jj) << 8) | jj);
          const uint64_t m = __ballot(word != 0u);
          if (lane == 0) {
            bm[j * dpj + 2 * blk] = (uint32_t)m;
            bm[j * dpj + 2 * blk + 1] = (uint32_t)(m >> 32);
          }
        }
      }
    }
  } else if (mode == 1) {
    const int64_t nv = align16(stored) / 16;
    for (int64_t q = threadIdx.x; q < nv; q += blockDim.x) ((uint4*)ob)[q] = ((const uint4*)slot)[q];
  }
  __syncthreads();
  // every load of this chunk's codes has returned: announce
  if (threadIdx.x == 0) {
    __hip_atomic_store(ann + k, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(grp + (k >> 6), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  bool consistent = true;
  if (mode == 2 || mode == 4) {
    const uint32_t nnz = scan_bitmap<NW>(bm, offs, nd, sh32);
    consistent = n / 16 + 2 * (int64_t)nnz == stored;    // the size the scan used
    if (!consistent && threadIdx.x == 0) set_status2(c.ctl, kStStall);
  }
  if (mode == 2 && consistent) {
    for (int d = threadIdx.x; d < nd; d += blockDim.x) ob[d] = bm[d];
    uint16_t* ow = (uint16_t*)(ob + nd);
    const int j = lane >> 3, r4 = 4 * (lane & 7);
    const uint32_t below = (1u << r4) - 1u;            // bitmap bits of the nibbles before this lane's
#pragma unroll
    for (int s4 = 0; s4 < NS; ++s4) {
      const int gi = wave + NW * s4;
      if (gi < ngi) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int d = j * dpj + 8 * gi + kk;
          const uint32_t bits = bm[d];
          const uint32_t nib = (bits >> r4) & 15u;
          // the nibble's non-zero words, in order, go to consecutive words
          // from its first index
          const uint32_t rr = offs[d] + (uint32_t)__builtin_popcount(bits & below);
          const uint32_t lo = R[16 * s4 + 2 * kk], hi = R[16 * s4 + 2 * kk + 1];
          const uint2 sel = cmptab[nib];
          const uint32_t c01 = __builtin_amdgcn_perm(hi, lo, sel.x), c23 = __builtin_amdgcn_perm(hi, lo, sel.y);
          const uint32_t pc = (uint32_t)__builtin_popcount(nib);
          uint16_t* p = ow + rr;
          if (pc > 0) p[0] = (uint16_t)c01;
          if (pc > 1) p[1] = (uint16_t)(c01 >> 16);
          if (pc > 2) p[2] = (uint16_t)c23;
          if (pc > 3) p[3] = (uint16_t)(c23 >> 16);
        }
      }
    }
  } else if (mode == 4 && consistent) {
    for (int d = threadIdx.x; d < nd; d += blockDim.x) ob[d] = bm[d];
    uint16_t* ow = (uint16_t*)(ob + nd);
    const int nblk = n >> 10;
    const uint32_t rr = (uint32_t)(lane & 31);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int blk = wave + NW * u;
      if (blk < nblk) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t a = (j < 4) ? R[4 * u] : R[4 * u + 1], b = (j < 4) ? R[4 * u + 2] : R[4 * u + 3];
          const uint32_t jj = (uint32_t)(j & 3);
          const uint32_t word = __builtin_amdgcn_perm(b, a, 0x0C0C0000u | ((4u + jj) << 8) | jj);
          const int d = j * dpj + 2 * blk + (lane >> 5);
          const uint32_t bits = bm[d];
          if ((bits >> rr) & 1u) ow[offs[d] + (uint32_t)__builtin_popcount(bits & ((1u << rr) - 1u))] = (uint16_t)word;
        }
      }
    }
  }
  if (mode == 0) {
    const int64_t pad = align16(stored) - stored;
    if (threadIdx.x < pad) dst[stored + threadIdx.x] = 0;
  } else if (consistent) {
    // the output [fin, fin + align16(stored)) covers the codes of chunks j0 .. j1
    // (and its own); chunks below kf are raw at their places: their codes are
    // never covered
    const uint64_t end = fin + (uint64_t)align16(stored);
    auto cover = [&](uint64_t x) { return PAGED ? first_covered_paged(c, x) : first_covered(c, x); };
    const int64_t j0 = min(max(cover(fin), kf), k);
    const int64_t j1 = (end == fin) ? j0 : max(j0, min(cover(end - 1) + 1, k));
    if (!wait_announced(c, ann, grp, j0, j1)) {
      if (threadIdx.x == 0) set_status2(c.ctl, kStStall);
    } else {
      const uint4* src = (mode == 3) ? (const uint4*)(c.codes_out + L.src) : (const uint4*)ob;
      const int64_t nv = align16(stored) / 16;
      for (int64_t q = threadIdx.x; q < nv; q += blockDim.x) {
        uint4 x = src[q];
        const int64_t lim = stored - 16 * q;
        if (lim < 16) {
          uint8_t* xb = (uint8_t*)&x;
          for (int b = 0; b < 16; ++b) if (b >= lim) xb[b] = 0;
        }
        ((uint4*)dst)[q] = x;
      }
    }
  }
  // a paged table may cover codes of earlier requests still to move: the
  // compaction writes those after the placement
  if (!PAGED && threadIdx.x == 0) *(uint32_t*)(c.stream + rq.table_off + 4 * k) = e;
  __syncthreads();                                     // LDS reused by the next chunk
}

template <int PIPE, bool PAGED>
__global__ __launch_bounds__(kPlaceThreads, kPlaceWaves / 2 < 4 ? kPlaceWaves / 2 : 4) void k_place(CallDesc c) {
  __shared__ __attribute__((aligned(16))) uint32_t ob[16384];   // output assembly / raw chunk (64 KiB)
  __shared__ uint32_t bm[1024];
  __shared__ uint32_t offs[1024];
  __shared__ uint32_t sh32[kPlaceWaves];
  __shared__ int64_t tk[1];
  __shared__ uint2 cmptab[16];
  if (threadIdx.x < 16) cmptab[threadIdx.x] = rze_compact_entry(threadIdx.x);   // read after the first barrier
  const int64_t N = c.total_chunks;
  uint32_t* ann = c.place_flags;
  uint32_t* grp = c.place_flags + N;
  // tickets: batches of 64 chunks below the first chunk with work (table
  // entries only), then every chunk from there on, then the header
  const int64_t kf = (int64_t)min<uint64_t>(c.ctl->pad[3], (uint64_t)N);
  const int64_t nb0 = (kf + 63) / 64, last = nb0 + (N - kf);
  // there are last + 1 tickets: the blocks past them leave without taking one
  // (one atomic counter that every block of a large grid hit was the cost of
  // small calls whose chunks all stay in place)
  if ((int64_t)blockIdx.x > last) return;
  const XposeLane X = xpose_lane();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint32_t* ticket = (uint32_t*)&c.ctl->pad[2];
  // A ticket is taken only when its work can start: every chunk waits for its
  // predecessor's read, so a ticket held while the block finishes another
  // chunk would delay the whole chain behind it.
  for (;;) {
    if (threadIdx.x == 0) tk[0] = (int64_t)__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int64_t t = tk[0];
    __syncthreads();
    if (t > last) break;
    if (t == last) {
      // dense: the header and the gaps (paged: the compaction, afterwards)
      if (!PAGED) {
        write_header(c, c.one, c.stream, c.ctl->total);
        zero_gaps(c, c.one, c.stream);
      }
      __syncthreads();
      continue;
    }
    if (t < nb0) {
      // raw chunks at their all-raw places: padding (and dense table
      // entries); nothing waits on them (no later output reaches their codes)
      const int64_t k = 64 * t + threadIdx.x;
      if (threadIdx.x < 64 && k < kf) {
        const int r = PAGED ? find_req_by_chunk(c, k) : 0;
        const ReqDesc rq = req_at(c, r);
        const ChunkLoc L = locate_chunk(c, rq, r, k);
        uint8_t* dst = c.codes + L.src;
        for (int64_t b = L.n; b < align16(L.n); ++b) dst[b] = 0;
        if (!PAGED) *(uint32_t*)(c.stream + rq.table_off + 4 * k) = c.chunk_sizes[k];
      }
      __syncthreads();
      continue;
    }
    place_chunk<PIPE, PAGED, kPlaceWaves>(c, kf + (t - nb0), kf, ann, grp, X, wave, lane, ob, bm, offs, sh32, cmptab);
  }
}

hipError_t launch_place(const CallDesc& c, hipStream_t s) {
  const int grid = (int)std::min<int64_t>(c.total_chunks + 1, 512);
  const bool p1 = c.stages[0] == KVC_TUPL8_1 && c.stages[1] == KVC_BIT_8 && c.stages[2] == KVC_RZE_2 && c.stages[3] == 0;
  const bool p2 = c.stages[0] == KVC_TUPL8_1 && c.stages[1] == KVC_RZE_2 && c.stages[2] == 0;
  if (c.place == 2) {
    if (c.total_chunks == 0) return hipSuccess;
    if (p1) k_place<1, true><<<grid, kPlaceThreads, 0, s>>>(c);
    else if (p2) k_place<2, true><<<grid, kPlaceThreads, 0, s>>>(c);
    else k_place<0, true><<<grid, kPlaceThreads, 0, s>>>(c);
  } else if (p1) {
    k_place<1, false><<<grid, kPlaceThreads, 0, s>>>(c);
  } else if (p2) {
    k_place<2, false><<<grid, kPlaceThreads, 0, s>>>(c);
  } else {
    k_place<0, false><<<grid, kPlaceThreads, 0, s>>>(c);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode

// Check request r's header against the plan and the bytes available (64 threads).
__device__ void validate_request(const CallDesc& c, int r) {
    const ReqDesc rq = req_at(c, r);
    const uint64_t base = c.req_offsets ? c.req_offsets[r] : 0;
    const int t = threadIdx.x;
    uint32_t bad = 0;
    if (base + (uint64_t)rq.payload_off > c.stream_bytes) {
      bad = kStCorrupt;
    } else {
      const uint8_t* h = c.stream + base;
      if (t == 0) {
        if (*(const uint32_t*)h != kMagic || *(const uint16_t*)(h + 4) != 1) bad |= kStCorrupt;
        else {
          uint32_t diag = 0;
          diag |= (h[6] != (uint8_t)c.dtype) << 0;
          diag |= (*(const int32_t*)(h + 8) != c.layers) << 1;
          diag |= (*(const int32_t*)(h + 12) != rq.T) << 2;
          diag |= (*(const int32_t*)(h + 16) != c.heads) << 3;
          diag |= (*(const int32_t*)(h + 20) != kHeadDim) << 4;
          diag |= (*(const uint64_t*)(h + 40) != c.seed) << 5;
          diag |= (*(const uint32_t*)(h + 52) != c.chunk_bytes) << 6;
          for (int w = 0; w < 2; ++w) {
            const uint8_t* p = h + 24 + 8 * w;
            diag |= (p[0] != c.pol[w].bits || p[1] != c.pol[w].axis || p[2] != c.pol[w].hadamard ||
                     *(const uint16_t*)(p + 4) != c.pol[w].group ||
                     *(const uint16_t*)(p + 6) != c.pol[w].delta) << (7 + w);
          }
          for (int k = 0; k < 4; ++k) diag |= (h[48 + k] != c.stages[k]) << (9 + k);
          diag |= (h[7] != (c.mixed ? 1 : 0)) << 13;
          if (diag) {
            bad |= kStMismatch;
            // which header fields differ (bit per field), kept for diagnosis
            __hip_atomic_fetch_or((uint32_t*)&c.ctl->pad[0], diag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          const uint64_t total = *(const uint64_t*)(h + 56);
          if (total < (uint64_t)rq.payload_off || total > (uint64_t)rq.max_stream || base + total > c.stream_bytes)
            bad |= kStCorrupt;
        }
      }
    }
    if (!bad && c.mixed) {
      // the width map must be the plan's
      const uint8_t* h = c.stream + base;
      const int64_t mapn = 2 * (int64_t)c.layers * c.heads;
      for (int64_t p = t; p < mapn; p += 64)
        if (h[64 + p] != c.width_map[p]) bad = kStMismatch;
    }
    if (bad) set_status2(c.ctl, bad);
}

// Check each request's header against the plan and the bytes available.
__global__ __launch_bounds__(64) void k_validate(CallDesc c) {
  for (int r = blockIdx.x; r < c.R; r += gridDim.x) validate_request(c, r);
}

hipError_t launch_validate(const CallDesc& c, hipStream_t s) {
  k_validate<<<(int)std::min(c.R, 1024), 64, 0, s>>>(c);
  return hipGetLastError();
}

// Decode classification, one thread per chunk (and per request: each
// stream's chunk sizes must add up to its header's total).  A chunk whose
// size, place or alignment is impossible marks the stream corrupt.  A raw
// chunk the reconstruct kernels read in place needs nothing; a raw chunk they
// cannot (paged tiles may cover it with a compressed neighbour) and a
// compressed chunk they decode themselves are listed for k_ll_decode_raw; a
// compressed chunk of a standard pipeline is left to the word-parallel
// kernels (which find it by index; only the count is kept here), and any
// other goes to the stage engine.
// request r's chunk sizes must add up to its header's total
__device__ __forceinline__ void check_request_total(const CallDesc& c, int64_t r) {
  const ReqDesc rq = req_at(c, (int)r);
  const uint64_t base = c.req_offsets ? c.req_offsets[r] : 0;
  const int64_t cend = rq.chunk_begin + rq.nchunks[0] + rq.nchunks[1];
  const uint64_t want = (uint64_t)rq.payload_off + (c.chunk_offs[cend] - c.chunk_offs[rq.chunk_begin]);
  if (base + 64 > c.stream_bytes || *(const uint64_t*)(c.stream + base + 56) != want)
    set_status2(c.ctl, kStCorrupt);
}
// classify chunk ch; returns 1 for a chunk left to the word-parallel kernels
__device__ __forceinline__ uint32_t classify_dec_chunk(const CallDesc& c, uint32_t* worklist, int pipe, int64_t ch) {
  const int r = find_req_by_chunk(c, ch);
  const ReqDesc rq = req_at(c, r);
  const ChunkLoc L = locate_chunk(c, rq, r, ch);
  const uint32_t e = c.chunk_sizes[ch];
  const int64_t stored = e & 0x7fffffffu;
  const bool raw = (e >> 31) != 0;
  const uint64_t base = c.req_offsets ? c.req_offsets[r] : 0;
  const uint64_t pos = base + (uint64_t)rq.payload_off + (c.chunk_offs[ch] - c.chunk_offs[rq.chunk_begin]);
  const bool ok = (raw ? stored == L.n : (stored < L.n && stored > 0)) && pos + (uint64_t)stored <= c.stream_bytes &&
                  (pos & 15) == 0;
  if (!ok) {
    set_status2(c.ctl, kStCorrupt);
    return 0;
  }
  bool in_place = raw && c.direct[L.w];
  if (in_place && c.straddle) {
    // a tile that also covers a compressed neighbour reads both from the codes area
    const int64_t s0 = rq.chunk_begin + (L.w ? rq.nchunks[0] : 0), s1 = s0 + rq.nchunks[L.w];
    const bool prev_c = ch > s0 && !(c.chunk_sizes[ch - 1] >> 31);
    const bool next_c = ch + 1 < s1 && !(c.chunk_sizes[ch + 1] >> 31);
    in_place = !(prev_c || next_c);
  }
  if (in_place) {
    // the reconstruct kernels read this chunk from the stream
  } else if (raw || (c.mirror[L.w] && fast_eligible(1, L.n))) {
    push_block(c, worklist, ch);
  } else if (!fast_eligible(pipe, L.n)) {
    push_work(c, worklist, ch);                      // the stage engine
  } else {
    return 1;                                        // the word-parallel kernels find theirs by index
  }
  return 0;
}
__device__ __forceinline__ void count_word_parallel(const CallDesc& c, uint32_t wp) {
  wp = wave_sum_u32(wp);
  if ((threadIdx.x & 63) == 0 && wp)
    __hip_atomic_fetch_add((uint32_t*)&c.ctl->pad[5], wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void k_ll_classify_dec(CallDesc c, uint32_t* worklist) {
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, dt = (int64_t)gridDim.x * blockDim.x;
  for (int64_t r = t0; r < c.R; r += dt) check_request_total(c, r);
  const int pipe = fast_pipeline(c);
  uint32_t wp = 0;                                   // compressed chunks left to the word-parallel kernels
  for (int64_t ch = t0; ch < c.total_chunks; ch += dt) wp += classify_dec_chunk(c, worklist, pipe, ch);
  count_word_parallel(c, wp);
}

// Small one-request decodes (at most kFrontChunks chunks, one per thread):
// the reset, the header check, the chunk-offset scan over the stream's table
// and the classification in one launch instead of three, which a layer-by-
// layer pipeline pays once per layer.
__global__ __launch_bounds__(kFrontChunks) void k_dec_front_small(CallDesc c, uint32_t* worklist) {
  __shared__ uint32_t sh32[kFrontChunks / 64];
  const int t = threadIdx.x;
  Control* ctl = c.ctl;
  if (t == 0) {
    ctl->status = 0;
    ctl->pad0 = 0;
    ctl->total = 0;
    for (int i = 0; i < 7; ++i) ctl->pad[i] = 0;
    ctl->pad[3] = ~0ull;
    __threadfence();
  }
  __syncthreads();                                   // the status word is clear before any check sets it
  if (t < 64) validate_request(c, 0);
  const int64_t N = c.total_chunks;
  const ReqDesc& rq = c.one;
  uint32_t e = 0;
  if (t < N) {
    const uint64_t pos = (uint64_t)rq.table_off + 4 * (uint64_t)t;
    if (pos + 4 <= c.stream_bytes && pos + 4 <= (uint64_t)rq.payload_off) e = *(const uint32_t*)(c.stream + pos);
    else set_status2(ctl, kStCorrupt);
    c.chunk_sizes[t] = e;
  }
  // kFrontChunks chunks hold at most 64 MiB of stored bytes: the scan fits 32 bits
  uint32_t total;
  const uint32_t ex = block_excl_scan_u32<kFrontChunks / 64>((uint32_t)align16(e & 0x7fffffffu), sh32, total);
  if (t < N) c.chunk_offs[t] = ex;
  if (t == 0) c.chunk_offs[N] = total;
  __threadfence_block();
  __syncthreads();                                   // every size and offset is written
  if (t == 0) check_request_total(c, 0);
  count_word_parallel(c, (t < N) ? classify_dec_chunk(c, worklist, fast_pipeline(c), t) : 0u);
}

hipError_t launch_dec_front_small(const CallDesc& c, hipStream_t s) {
  uint32_t* worklist = (uint32_t*)(c.chunk_offs + c.total_chunks + 1);
  k_dec_front_small<<<1, kFrontChunks, 0, s>>>(c, worklist);
  return hipGetLastError();
}

// The listed chunks, one block each: a raw chunk is copied to its code slot;
// for a compressed chunk the reconstruct kernel decodes itself, the number of
// non-zero words before each bitmap dword (n / 64 words in the chunk's codes
// slot), checked against the stored size.
__global__ __launch_bounds__(256) void k_ll_decode_raw(CallDesc c, const uint32_t* worklist) {
  __shared__ uint32_t sh32[256];
  const uint32_t count = __hip_atomic_load(block_count(c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (uint32_t item = blockIdx.x; item < count; item += gridDim.x) {
    const int64_t ch = worklist[item];
    const int r = find_req_by_chunk(c, ch);
    const ReqDesc rq = req_at(c, r);
    const ChunkLoc L = locate_chunk(c, rq, r, ch);
    const uint32_t e = c.chunk_sizes[ch];
    const int64_t stored = e & 0x7fffffffu;
    const uint64_t base = c.req_offsets ? c.req_offsets[r] : 0;
    const uint64_t pos = base + (uint64_t)rq.payload_off + (c.chunk_offs[ch] - c.chunk_offs[rq.chunk_begin]);
    if (!(e >> 31)) {
      const int n = (int)L.n, nd = n / 64;
      if (stored < n / 16) {
        if (threadIdx.x == 0) set_status2(c.ctl, kStCorrupt);
        continue;
      }
      const uint32_t* bmg = (const uint32_t*)(c.stream + pos);
      uint32_t* pref = (uint32_t*)(c.codes + L.src);
      uint32_t cnt[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 4 * (int)threadIdx.x + i;
        cnt[i] = (d < nd) ? (uint32_t)__builtin_popcount(bmg[d]) : 0u;
        sum += cnt[i];
      }
      uint32_t total;
      uint32_t run = block_exclusive_scan<uint32_t>(sum, sh32, total);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 4 * (int)threadIdx.x + i;
        if (d < nd) pref[d] = run;
        run += cnt[i];
      }
      if (n / 16 + 2 * (int64_t)total != stored && threadIdx.x == 0) set_status2(c.ctl, kStCorrupt);
    } else {
      const uint4* src = (const uint4*)(c.stream + pos);
      uint4* dst = (uint4*)(c.codes + L.src);
      const int64_t nv = L.n / 16;
      for (int64_t k = threadIdx.x; k < nv; k += blockDim.x) dst[k] = src[k];
      for (int64_t p = nv * 16 + threadIdx.x; p < L.n; p += blockDim.x) c.codes[L.src + p] = c.stream[pos + p];
    }
    __syncthreads();                                 // sh32 is reused by the next chunk
  }
}

__global__ __launch_bounds__(256) void k_ll_decode_generic(CallDesc c, const uint32_t* worklist) {
  __shared__ __attribute__((aligned(16))) uint8_t bufA[65536];
  __shared__ __attribute__((aligned(16))) uint8_t bufB[65536];
  __shared__ uint32_t sh32[256];
  __shared__ uint64_t sh64[256];
  const uint32_t count = *generic_count(c);
  for (uint32_t item = blockIdx.x; item < count; item += gridDim.x) {
    const int64_t ch = worklist[c.total_chunks - 1 - item];
    const int r = find_req_by_chunk(c, ch);
    const ReqDesc rq = req_at(c, r);
    const ChunkLoc L = locate_chunk(c, rq, r, ch);
    const uint32_t e = c.chunk_sizes[ch];
    const int stored = (int)(e & 0x7fffffffu);
    const uint64_t base = c.req_offsets ? c.req_offsets[r] : 0;
    const uint64_t pos = base + (uint64_t)rq.payload_off + (c.chunk_offs[ch] - c.chunk_offs[rq.chunk_begin]);
    const int n = (int)L.n;
    for (int p = threadIdx.x; p < stored; p += blockDim.x) bufA[p] = c.stream[pos + p];
    __syncthreads();
    int ns = 0;
    while (ns < 4 && c.stages[ns]) ++ns;
    uint8_t* cur = bufA;
    uint8_t* alt = bufB;
    int size = stored;
    bool ok = true;
    for (int s = ns - 1; s >= 0 && ok; --s) {
      ok = stage_inverse(c.stages[s], cur, size, alt, n, sh32, sh64);
      uint8_t* tmp = cur; cur = alt; alt = tmp;
      size = n;
    }
    if (!ok) {
      if (threadIdx.x == 0) set_status2(c.ctl, kStCorrupt);
    } else {
      for (int p = threadIdx.x; p < n; p += blockDim.x) c.codes[L.src + p] = cur[p];
    }
    __syncthreads();
  }
}

hipError_t launch_lossless_decode(const CallDesc& c, bool classified, hipStream_t s) {
  if (c.total_chunks == 0) return hipSuccess;
  uint32_t* worklist = (uint32_t*)(c.chunk_offs + c.total_chunks + 1);
  hipError_t e = hipSuccess;
  if (!classified) {
    k_ll_classify_dec<<<(int)std::min<int64_t>((std::max<int64_t>(c.total_chunks, c.R) + 255) / 256, 4096), 256, 0, s>>>(
        c, worklist);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  k_ll_decode_raw<<<(int)std::min<int64_t>(c.total_chunks, 256 * 8), 256, 0, s>>>(c, worklist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool p1 = c.stages[0] == KVC_TUPL8_1 && c.stages[1] == KVC_BIT_8 && c.stages[2] == KVC_RZE_2 && c.stages[3] == 0;
  const bool p2 = c.stages[0] == KVC_TUPL8_1 && c.stages[1] == KVC_RZE_2 && c.stages[2] == 0;
  const int fgrid = (int)std::min<int64_t>(c.total_chunks, 512);
  if (p1) k_ll_decode_p1<4><<<(int)std::min<int64_t>(c.total_chunks, 256 * kP1BlocksPerCu), 256, 0, s>>>(c, worklist);
  else if (p2) k_ll_decode_p2<kDecWaves><<<fgrid, 64 * kDecWaves, 0, s>>>(c, worklist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (all_word_parallel(c)) return hipSuccess;
  k_ll_decode_generic<<<(int)std::min<int64_t>(c.total_chunks, 512), 256, 0, s>>>(c, worklist);
  return hipGetLastError();
}

}  // namespace kvc
