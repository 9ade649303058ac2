// Host side of libkvc: plan validation, stream and workspace layouts, launch
// sequences for encode / decode (dense and paged), device status, profiling.
//
// FastKVComp ("Beyond Compression Ratio: High-Throughput KV Compression for
// Disaggregated LLM Serving") Sec. 4.2: the runtime consumes device buffers,
// keeps the compressed stream on the GPU, reuses persistent scratch and
// returns only the compressed size to the host.  Sec. 4.1: signs and
// precision assignments are computed once and reused (the plan).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kvc_internal.h"

using namespace kvc;

struct kvc_plan_s {
  kvc_config cfg;
  TensorPol pol[2];
  uint32_t signs[4];
  bool mixed = false;
  std::vector<uint8_t> widths;   // mixed: [2][layers][kv_heads] of 2, 4, 8 or 16
};

namespace {

thread_local std::string g_last_error;

kvc_status fail(kvc_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kvc_status fail(kvc_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kvc_status hip_fail(hipError_t e, const char* what) {
  return fail(KVC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t a16(int64_t x) { return (x + 15) & ~int64_t(15); }
int64_t a256(int64_t x) { return (x + 255) & ~int64_t(255); }

// splitmix64 output stream (Steele, Lea, Flood, OOPSLA 2014): the i-th sign
// is -1 when the top bit of the i-th output, state started at the seed, is set.
uint64_t splitmix_next(uint64_t& st) {
  st += 0x9E3779B97F4A7C15ull;
  uint64_t z = st;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int64_t codes_bytes_of(const TensorPol& p, int L, int T, int H) {
  if (T == 0) return 0;
  if (p.axis == 0) return (int64_t)L * T * H * kHeadDim * p.bits / 8;
  const int64_t ng = cdiv(T, p.group);
  const int64_t glast = T - (ng - 1) * p.group;
  const int64_t per_layer = (ng - 1) * H * kHeadDim * (p.group * p.bits / 8) +
                            (int64_t)H * kHeadDim * cdiv(glast * p.bits, 8);
  return (int64_t)L * per_layer;
}

int64_t params_bytes_of(const TensorPol& p, int L, int T, int H) {
  if (p.axis == 0) return (int64_t)L * T * H * (kHeadDim / p.group) * 4;
  return (int64_t)L * cdiv(T, p.group) * H * kHeadDim * 4;
}

// Fused-kernel tiles.  Per-token tiles are 32 head vectors: a dense call maps
// them over all L*T*H vectors as one run; a paged request maps them per layer
// so that no tile crosses a page.  Per-channel tiles are 64 tokens x 1 head.
int64_t tiles_of(const TensorPol& p, int L, int T, int H, bool paged) {
  if (T == 0) return 0;
  if (p.axis == 0) return paged ? (int64_t)L * cdiv((int64_t)T * H, 32) : cdiv((int64_t)L * T * H, 32);
  return (int64_t)L * cdiv(T, 64) * H;
}

// Whether every reconstruct tile's codes of a dense call lie inside one chunk
// (then raw chunks can be read straight from the stream): per-token tiles
// are 32 vectors at multiples of their size; per-channel tiles read blocks of
// 128 columns of one token group, uniform in size only when no group is partial.
bool tiles_within_chunks(const TensorPol& p, int T, uint32_t chunk_bytes) {
  if (p.axis == 0) return chunk_bytes % (32 * kHeadDim * p.bits / 8) == 0;
  if (T % p.group) return false;
  return chunk_bytes % (kHeadDim * p.group * p.bits / 8) == 0;
}

// The two lossless pipelines with word-parallel kernels: 1 = TUPL8_1 -> BIT_8 ->
// RZE_2, 2 = TUPL8_1 -> RZE_2, 0 = other.
int lossless_pipe(const uint8_t* st) {
  if (st[0] == KVC_TUPL8_1 && st[1] == KVC_BIT_8 && st[2] == KVC_RZE_2 && st[3] == 0) return 1;
  if (st[0] == KVC_TUPL8_1 && st[1] == KVC_RZE_2 && st[2] == 0) return 2;
  return 0;
}

// Whether the fused encoders of a dense call can count a section's non-zero
// RZE words: every wave's codes must cover whole aligned 1 KiB regions of one
// chunk.  Per-token tiles always do; per-channel kernels count groups of 64
// tokens (2, 4 or 8 bits) when no group is partial.
bool fused_count_ok(const TensorPol& p, int T, uint32_t chunk_bytes) {
  if (p.axis == 0) return true;
  return p.group == 64 && T % 64 == 0 && chunk_bytes % (kHeadDim * 64 * p.bits / 8) == 0;
}

// Whether the fused encoders of a paged call can count a section's non-zero
// RZE words.  TUPL8_1 -> RZE_2 counts per aligned 16-byte unit, which every
// tile covers whole.  TUPL8_1 -> BIT_8 -> RZE_2 counts per aligned 1 KiB
// region, which a tile covers whole only if every layer of every request
// starts on a region boundary.  A tile that covers two chunks splits its
// count between them.
bool paged_count_ok(const TensorPol& p, int pipe, int H, const int32_t* lens, int R) {
  if (p.axis != 0) return false;
  if (pipe == 2) return true;
  if (pipe != 1) return false;
  const int64_t layer_vec_bytes = (int64_t)H * kHeadDim * p.bits / 8;
  for (int r = 0; r < R; ++r)
    if (((int64_t)lens[r] * layer_vec_bytes) % 1024) return false;
  return true;
}

// Codes / parameter bytes of one (layer, head) slab of width `bits` (16:
// the 16-bit values themselves): the sections of a one-layer, one-head
// uniform stream of that width.
int64_t slab_codes_bytes(const TensorPol& p, int bits, int T) {
  if (bits == 16) return (int64_t)T * kHeadDim * 2;
  TensorPol q = p;
  q.bits = bits;
  return codes_bytes_of(q, 1, T, 1);
}
int64_t slab_params_bytes(const TensorPol& p, int bits, int T) {
  if (bits == 16) return 0;
  return params_bytes_of(p, 1, T, 1);
}

// Fill the stream layout of one request with T tokens (offsets inside its stream).
void request_layout(const kvc_plan_s* p, int T, ReqDesc& rq) {
  const kvc_config& c = p->cfg;
  std::memset(&rq, 0, sizeof(rq));
  rq.T = T;
  int64_t nch = 0;
  const int64_t LH = (int64_t)c.layers * c.kv_heads;
  for (int w = 0; w < 2; ++w) {
    if (!p->mixed) {
      rq.codes_bytes[w] = codes_bytes_of(p->pol[w], c.layers, T, c.kv_heads);
      rq.params_bytes[w] = params_bytes_of(p->pol[w], c.layers, T, c.kv_heads);
    } else {
      for (int64_t i = 0; i < LH; ++i) {
        rq.codes_bytes[w] += slab_codes_bytes(p->pol[w], p->widths[w * LH + i], T);
        rq.params_bytes[w] += slab_params_bytes(p->pol[w], p->widths[w * LH + i], T);
      }
    }
    rq.nchunks[w] = (int32_t)cdiv(rq.codes_bytes[w], c.chunk_bytes);
    nch += rq.nchunks[w];
    rq.params_ws_off[w] = -1;
  }
  // mixed streams carry the width map right after the header
  rq.table_off = p->mixed ? a16(kHeaderBytes + 2 * LH) : kHeaderBytes;
  rq.params_off[0] = a16(rq.table_off + 4 * nch);
  rq.params_off[1] = a16(rq.params_off[0] + rq.params_bytes[0]);
  rq.payload_off = a16(rq.params_off[1] + rq.params_bytes[1]);
  int64_t pay = 0;
  for (int w = 0; w < 2; ++w)
    for (int64_t i = 0; i < rq.nchunks[w]; ++i)
      pay += a16(std::min<int64_t>(c.chunk_bytes, rq.codes_bytes[w] - i * c.chunk_bytes));
  rq.max_stream = rq.payload_off + pay;
}

// Workspace carving shared by all calls.
struct WsLayout {
  int64_t ctl, sizes, offs, worklist, flags, scan, counts, codes, params, reqs, slabs, delta, total;
};

// Bytes of the token-delta area of a dense encode: the transformed copy of
// each tensor that uses the delta.
int64_t delta_area(const kvc_plan_s* p, int64_t T, int64_t* k_bytes = nullptr) {
  const int64_t one = a256((int64_t)p->cfg.layers * T * p->cfg.kv_heads * kHeadDim * 2);
  const int64_t k = p->pol[0].delta ? one : 0, v = p->pol[1].delta ? one : 0;
  if (k_bytes) *k_bytes = k;
  return k + v;
}

// Bytes of the slab tables (a SlabDesc per (tensor, layer, head)) and the width
// map that a mixed call uploads into its workspace.
int64_t slab_area(const kvc_plan_s* p) {
  if (!p->mixed) return 0;
  const int64_t n = 2 * (int64_t)p->cfg.layers * p->cfg.kv_heads;
  return a256(n * (int64_t)sizeof(SlabDesc)) + a256(n);
}

// Request area of a paged call (R > 1): the descriptors, then the two tile ->
// request tables (kReqTableMax + 1 entries each).
int64_t req_table_off(int64_t R) { return a256(R * (int64_t)sizeof(ReqDesc)); }
int64_t req_area(int64_t R) { return req_table_off(R) + 2 * 4 * (int64_t)(kReqTableMax + 1); }

WsLayout ws_layout(int64_t nchunks, int64_t codes_area, int64_t params_area, int64_t R, int64_t slabs = 0,
                   int64_t delta = 0) {
  WsLayout w;
  w.ctl = 0;
  w.sizes = 256;
  w.offs = w.sizes + a256(4 * std::max<int64_t>(nchunks, 1));
  // the worklist follows the offsets directly (kernels locate it there)
  w.worklist = w.offs + 8 * (nchunks + 1);
  // read announcements of the single-pass placement: one word per chunk, one per 64 chunks
  w.flags = a256(w.worklist + 4 * std::max<int64_t>(nchunks, 1));
  // look-back words of the dense scan: one per 1024 chunks
  w.scan = a256(w.flags + 4 * (nchunks + (nchunks + 63) / 64 + 1));
  // the fused encoders' non-zero word counters: kNnzSlots per chunk
  w.counts = a256(w.scan + 8 * (nchunks / 1024 + 1));
  w.codes = a256(w.counts + 4 * (int64_t)kNnzSlots * std::max<int64_t>(nchunks, 1));
  w.params = a256(w.codes + codes_area);
  w.reqs = a256(w.params + params_area);
  w.slabs = a256(w.reqs + (R > 1 ? req_area(R) : 0));
  w.delta = a256(w.slabs + slabs);
  w.total = a256(w.delta + delta);
  return w;
}

// Slab tables of a mixed dense call with T tokens, grouped per tensor and width
// (2, 4, 8, 16) in (layer, head) order, followed by the width map; first[w][k]
// and count[w][k] index the group of width {2, 4, 8, 16}[k].
struct SlabTables {
  std::vector<uint8_t> bytes;
  int first[2][4], count[2][4];
  int64_t map_off;
};

SlabTables slab_tables(const kvc_plan_s* p, int T) {
  static const int kW[4] = {2, 4, 8, 16};
  SlabTables t;
  const int L = p->cfg.layers, H = p->cfg.kv_heads;
  const int64_t LH = (int64_t)L * H;
  std::vector<SlabDesc> all;
  for (int w = 0; w < 2; ++w) {
    std::vector<int64_t> co(LH), po(LH);
    int64_t c = 0, q = 0;
    for (int64_t i = 0; i < LH; ++i) {
      co[i] = c;
      po[i] = q;
      c += slab_codes_bytes(p->pol[w], p->widths[w * LH + i], T);
      q += slab_params_bytes(p->pol[w], p->widths[w * LH + i], T);
    }
    for (int k = 0; k < 4; ++k) {
      t.first[w][k] = (int)all.size();
      for (int64_t i = 0; i < LH; ++i)
        if (p->widths[w * LH + i] == kW[k]) all.push_back(SlabDesc{(int32_t)(i / H), (int32_t)(i % H), co[i], po[i]});
      t.count[w][k] = (int)all.size() - t.first[w][k];
    }
  }
  t.map_off = a256((int64_t)all.size() * (int64_t)sizeof(SlabDesc));
  t.bytes.assign((size_t)(t.map_off + 2 * LH), 0);
  std::memcpy(t.bytes.data(), all.data(), all.size() * sizeof(SlabDesc));
  std::memcpy(t.bytes.data() + t.map_off, p->widths.data(), (size_t)(2 * LH));
  return t;
}

// ---------------------------------------------------------------- profiling

struct ProfRec { int kind; hipEvent_t a, b; };
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_open;      // recorded, not yet harvested
std::vector<hipEvent_t> g_prof_pool;
double g_prof_ms[KVC_KERNEL_COUNT];
int64_t g_prof_n[KVC_KERNEL_COUNT];
thread_local hipEvent_t t_prof_start[KVC_KERNEL_COUNT];

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) { hipEvent_t e = g_prof_pool.back(); g_prof_pool.pop_back(); return e; }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void prof_harvest_locked() {
  for (ProfRec& r : g_prof_open) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) { g_prof_ms[r.kind] += ms; g_prof_n[r.kind] += 1; }
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_open.clear();
}

}  // namespace

namespace kvc {
// records msg as the calling thread's last error (kvc_last_error) and returns s
kvc_status report_error(kvc_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace kvc

namespace kvc {
void prof_begin(int kind, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  hipEvent_t e = prof_event();
  if (!e || hipEventRecord(e, s) != hipSuccess) return;
  t_prof_start[kind] = e;
}
void prof_end(int kind, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || !t_prof_start[kind]) return;
  hipEvent_t e = prof_event();
  if (!e || hipEventRecord(e, s) != hipSuccess) { t_prof_start[kind] = nullptr; return; }
  g_prof_open.push_back({kind, t_prof_start[kind], e});
  t_prof_start[kind] = nullptr;
  if (g_prof_open.size() > 4096) prof_harvest_locked();
}
}  // namespace kvc

namespace {

template <typename F>
hipError_t timed(int kind, hipStream_t s, F&& f) {
  prof_begin(kind, s);
  hipError_t e = f();
  prof_end(kind, s);
  return e;
}

// ---------------------------------------------------------------- validation

kvc_status check_policy(const kvc_tensor_policy& t, const char* name, int head_dim) {
  if (!(t.bits == 2 || t.bits == 4 || t.bits == 8)) return fail(KVC_ERR_INVALID_ARG, "%s.bits must be 2, 4 or 8", name);
  if (t.axis > 1) return fail(KVC_ERR_INVALID_ARG, "%s.axis must be 0 or 1", name);
  if (t.hadamard > 1) return fail(KVC_ERR_INVALID_ARG, "%s.hadamard must be 0 or 1", name);
  if (!pow2(t.group)) return fail(KVC_ERR_INVALID_ARG, "%s.group must be a power of two", name);
  if (t.axis == 0 && (t.group < 8 || t.group > head_dim))
    return fail(KVC_ERR_INVALID_ARG, "%s.group must be in [8, head_dim] for per-token groups", name);
  if (t.axis == 1 && (t.group < 16 || t.group > 256))
    return fail(KVC_ERR_INVALID_ARG, "%s.group must be in [16, 256] for per-channel groups", name);
  if (t.delta != 0 && (!pow2(t.delta) || t.delta < 2 || t.delta > 32768))
    return fail(KVC_ERR_INVALID_ARG, "%s.delta must be 0 or a power of two in [2, 32768]", name);
  return KVC_OK;
}

kvc_status check_gpu_support(const kvc_tensor_policy& t, const char* name) {
  if (!t.hadamard)
    return fail(KVC_ERR_UNSUPPORTED, "%s: the GPU kernels always apply the randomized Hadamard transform", name);
  if (t.axis == 0 && t.group < 16)
    return fail(KVC_ERR_UNSUPPORTED, "%s: per-token groups smaller than 16 are not implemented on the GPU", name);
  if (t.axis == 1 && !(t.group == 32 || t.group == 64))
    return fail(KVC_ERR_UNSUPPORTED, "%s: per-channel groups other than 32 or 64 are not implemented on the GPU", name);
  return KVC_OK;
}

kvc_status check_ptr(const void* p, size_t align, const char* name) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "%s is NULL", name);
  if (((uintptr_t)p) % align) return fail(KVC_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, align);
  return KVC_OK;
}

void fill_common(const kvc_plan_s* p, CallDesc& c) {
  std::memset(&c, 0, sizeof(c));
  c.layers = p->cfg.layers;
  c.heads = p->cfg.kv_heads;
  c.dtype = p->cfg.dtype;
  c.pol[0] = p->pol[0];
  c.pol[1] = p->pol[1];
  std::memcpy(c.signs, p->signs, sizeof(c.signs));
  std::memcpy(c.stages, p->cfg.lossless, 4);
  c.chunk_bytes = p->cfg.chunk_bytes;
  c.chunk_shift = (c.chunk_bytes & (c.chunk_bytes - 1)) ? -1 : __builtin_ctz(c.chunk_bytes);
  c.seed = p->cfg.sign_seed;
}

kvc_status device_status(uint32_t bits) {
  if (bits & kStMismatch) return fail(KVC_ERR_PLAN_MISMATCH, "stream header does not match the plan or token count");
  if (bits & kStCorrupt) return fail(KVC_ERR_CORRUPT_STREAM, "stream failed validation on the device");
  if (bits & kStBadBlock) return fail(KVC_ERR_INVALID_ARG, "block table entry out of range");
  if (bits & kStRange) return fail(KVC_ERR_RANGE, "a quantization parameter is not a finite fp16 value (or an input value is infinite or NaN)");
  if (bits & kStStall) return fail(KVC_ERR_HIP, "single-pass placement: a wait ran out or a chunk size disagreed");
  return KVC_OK;
}

kvc_status sync_and_read(Control* d_ctl, hipStream_t s, Control& h) {
  hipError_t e = hipMemcpyAsync(&h, d_ctl, 16, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(status)");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return KVC_OK;
}

// Requests of a paged call, laid out one after another.
struct PagedJob {
  std::vector<ReqDesc> reqs;
  int64_t chunks = 0, pieces = 0, codes_area = 0, params_area = 0, max_total = 0;
  int64_t tiles[2] = {0, 0};
};

// The request area's bytes (descriptors and tile -> request tables) of a
// paged call with R > 1, uploaded in one copy; sets the call's table
// pointers (into the workspace at `d_area`) and shifts.
std::vector<uint8_t> request_area(const PagedJob& j, uint8_t* d_area, CallDesc& c) {
  const int64_t R = (int64_t)j.reqs.size();
  std::vector<uint8_t> bytes((size_t)req_area(R), 0);
  std::memcpy(bytes.data(), j.reqs.data(), (size_t)R * sizeof(ReqDesc));
  for (int w = 0; w < 2; ++w) {
    int sh = 0;
    while (((j.tiles[w] + (int64_t(1) << sh) - 1) >> sh) > kReqTableMax) ++sh;
    const int64_t n = (j.tiles[w] + (int64_t(1) << sh) - 1) >> sh;      // entries 0..n
    int32_t* tab = (int32_t*)(bytes.data() + req_table_off(R)) + w * (kReqTableMax + 1);
    int64_t r = 0;
    for (int64_t i = 0; i <= n; ++i) {
      const int64_t t = i << sh;
      while (r + 1 < R && j.reqs[(size_t)r + 1].tile_begin[w] <= t) ++r;
      tab[i] = (int32_t)r;
    }
    c.req_tab[w] = (const int32_t*)(d_area + req_table_off(R)) + w * (kReqTableMax + 1);
    c.req_shift[w] = sh;
  }
  return bytes;
}

PagedJob paged_job(const kvc_plan_s* p, const int32_t* lens, int R, bool encode) {
  PagedJob j;
  j.reqs.resize(R);
  int64_t fixed = 0;
  for (int r = 0; r < R; ++r) {
    ReqDesc& rq = j.reqs[r];
    request_layout(p, lens[r], rq);
    rq.row = r;
    rq.chunk_begin = j.chunks;
    j.chunks += rq.nchunks[0] + rq.nchunks[1];
    for (int w = 0; w < 2; ++w) {
      rq.tile_begin[w] = j.tiles[w];
      j.tiles[w] += tiles_of(p->pol[w], p->cfg.layers, lens[r], p->cfg.kv_heads, true);
      rq.codes_off[w] = j.codes_area;
      j.codes_area += a256(rq.codes_bytes[w]);
      if (encode) {
        rq.params_ws_off[w] = j.params_area;
        j.params_area += a256(rq.params_bytes[w]);
      }
    }
    rq.piece_begin = j.pieces;
    if (encode) j.pieces += cdiv(rq.params_bytes[0], 65536) + cdiv(rq.params_bytes[1], 65536);
    rq.raw_base = j.max_total;
    rq.fixed_before = fixed;
    if (encode) {
      // the fused encoders write the codes where the request's stream keeps
      // them when every chunk so far is raw (positions in the output buffer)
      rq.codes_off[0] = rq.raw_base + rq.payload_off;
      rq.codes_off[1] = rq.codes_off[0] + a16(rq.codes_bytes[0]);
    }
    fixed += rq.payload_off;
    j.max_total += rq.max_stream;
  }
  // encode: the staging area of the stage engine's chunks uses the same offsets
  if (encode) j.codes_area = a256(j.max_total);
  return j;
}

// Upload the slab tables and width map of a mixed dense call into the
// workspace (a few KiB, host to device on the call's stream; the source
// buffer may be reused once hipMemcpyAsync returns).
kvc_status upload_slabs(const kvc_plan_s* p, int T, uint8_t* d_area, hipStream_t s, CallDesc& c, SlabTables& tb) {
  try {
    tb = slab_tables(p, T);
  } catch (const std::bad_alloc&) {
    return fail(KVC_ERR_NO_MEMORY, "slab table allocation failed");
  }
  const hipError_t e = hipMemcpyAsync(d_area, tb.bytes.data(), tb.bytes.size(), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(slab tables)");
  c.mixed = 1;
  c.slabs = (const SlabDesc*)d_area;
  c.width_map = d_area + tb.map_off;
  return KVC_OK;
}

// The fused encode (or reconstruct) launches of one tensor: one launch for a
// uniform plan; for a mixed plan one per width present over that width's
// slabs, and the 16-bit slabs copied as they are.
hipError_t fused_all(const kvc_plan_s* p, const CallDesc& c, const SlabTables& tb, int which, bool encode,
                     hipStream_t s) {
  if (!c.mixed) return encode ? launch_encode_fused(c, which, s) : launch_decode_fused(c, which, s);
  static const int kW[4] = {2, 4, 8, 16};
  const int T = c.one.T;
  for (int k = 0; k < 4; ++k) {
    const int n = tb.count[which][k];
    if (n == 0) continue;
    CallDesc cb = c;
    cb.slabs = c.slabs + tb.first[which][k];
    cb.nslabs = n;
    hipError_t e;
    if (kW[k] == 16) {
      e = launch_slab_copy(cb, which, encode, s);
    } else {
      cb.pol[which].bits = kW[k];
      const TensorPol& pol = p->pol[which];
      cb.tiles[which] = pol.axis == 0 ? (int64_t)n * cdiv(T, 32) : (int64_t)n * cdiv(T, 64);
      e = encode ? launch_encode_fused(cb, which, s) : launch_decode_fused(cb, which, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// ====================================================================== ABI

extern "C" {

const char* kvc_status_string(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID_ARG: return "invalid argument";
    case KVC_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVC_ERR_NO_MEMORY: return "out of host memory";
    case KVC_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case KVC_ERR_CORRUPT_STREAM: return "corrupt stream";
    case KVC_ERR_PLAN_MISMATCH: return "stream does not match the plan";
    case KVC_ERR_RANGE: return "quantization parameter out of fp16 range";
    case KVC_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kvc_last_error(void) { return g_last_error.c_str(); }

kvc_status kvc_plan(const kvc_config* cfg, kvc_plan_t* out) {
  if (!cfg || !out) return fail(KVC_ERR_INVALID_ARG, "cfg and out must be non-NULL");
  *out = nullptr;
  if (cfg->struct_size != sizeof(kvc_config))
    return fail(KVC_ERR_INVALID_ARG, "struct_size %u != sizeof(kvc_config) %zu", cfg->struct_size, sizeof(kvc_config));
  if (cfg->layers < 1 || cfg->layers > 4096) return fail(KVC_ERR_INVALID_ARG, "layers must be in [1, 4096]");
  if (cfg->max_tokens < 0 || cfg->max_tokens > (1 << 26)) return fail(KVC_ERR_INVALID_ARG, "max_tokens must be in [0, 2^26]");
  if (cfg->kv_heads < 1 || cfg->kv_heads > 1024) return fail(KVC_ERR_INVALID_ARG, "kv_heads must be in [1, 1024]");
  if (!pow2(cfg->head_dim) || cfg->head_dim < 16 || cfg->head_dim > 256)
    return fail(KVC_ERR_INVALID_ARG, "head_dim must be a power of two in [16, 256]");
  if (cfg->dtype != KVC_F16 && cfg->dtype != KVC_BF16) return fail(KVC_ERR_INVALID_ARG, "dtype must be KVC_F16 or KVC_BF16");
  kvc_status st;
  if ((st = check_policy(cfg->k, "k", cfg->head_dim)) != KVC_OK) return st;
  if ((st = check_policy(cfg->v, "v", cfg->head_dim)) != KVC_OK) return st;
  if (cfg->chunk_bytes < 4096 || cfg->chunk_bytes > 65536 || cfg->chunk_bytes % 4096)
    return fail(KVC_ERR_INVALID_ARG, "chunk_bytes must be a multiple of 4096 in [4096, 65536]");
  bool rze = false;
  for (int i = 0; i < 4 && cfg->lossless[i]; ++i) {
    const int s = cfg->lossless[i];
    if (s < KVC_TUPL2_1 || s > KVC_RZE_8) return fail(KVC_ERR_INVALID_ARG, "lossless[%d] = %d is not a stage id", i, s);
    if (rze) return fail(KVC_ERR_UNSUPPORTED, "zero elimination must be the last lossless stage");
    if (s >= KVC_RZE_1) rze = true;
  }
  if (cfg->page_tokens < 0) return fail(KVC_ERR_INVALID_ARG, "page_tokens must be >= 0");
  if (cfg->head_dim != kHeadDim) return fail(KVC_ERR_UNSUPPORTED, "the GPU kernels implement head_dim 128 only");
  if ((st = check_gpu_support(cfg->k, "k")) != KVC_OK) return st;
  if ((st = check_gpu_support(cfg->v, "v")) != KVC_OK) return st;

  kvc_plan_s* p = new (std::nothrow) kvc_plan_s;
  if (!p) return fail(KVC_ERR_NO_MEMORY, "plan allocation failed");
  p->cfg = *cfg;
  const kvc_tensor_policy* tp[2] = {&cfg->k, &cfg->v};
  for (int w = 0; w < 2; ++w) {
    p->pol[w].bits = tp[w]->bits;
    p->pol[w].axis = tp[w]->axis;
    p->pol[w].group = tp[w]->group;
    p->pol[w].hadamard = tp[w]->hadamard;
    p->pol[w].c = tp[w]->hadamard ? (float)(1.0 / std::sqrt((double)cfg->head_dim)) : 1.0f;
    p->pol[w].delta = tp[w]->delta;
  }
  std::memset(p->signs, 0, sizeof(p->signs));
  uint64_t st64 = cfg->sign_seed;
  for (int i = 0; i < kHeadDim; ++i)
    if (splitmix_next(st64) >> 63) p->signs[i >> 5] |= 1u << (i & 31);
  *out = p;
  return KVC_OK;
}

kvc_status kvc_plan_mixed(const kvc_config* cfg, const uint8_t* h_bits, kvc_plan_t* out) {
  if (!h_bits || !out) return fail(KVC_ERR_INVALID_ARG, "h_bits and out must be non-NULL");
  kvc_status st = kvc_plan(cfg, out);
  if (st != KVC_OK) return st;
  kvc_plan_s* p = *out;
  if (cfg->page_tokens != 0) {
    kvc_plan_destroy(p);
    *out = nullptr;
    return fail(KVC_ERR_UNSUPPORTED, "mixed-precision plans are dense only (page_tokens must be 0)");
  }
  const int64_t LH = (int64_t)cfg->layers * cfg->kv_heads;
  try {
    p->widths.assign(h_bits, h_bits + 2 * LH);
  } catch (const std::bad_alloc&) {
    kvc_plan_destroy(p);
    *out = nullptr;
    return fail(KVC_ERR_NO_MEMORY, "plan allocation failed");
  }
  for (int64_t i = 0; i < 2 * LH; ++i) {
    uint8_t& b = p->widths[i];
    if (b == 0) b = (uint8_t)p->pol[i < LH ? 0 : 1].bits;
    if (!(b == 2 || b == 4 || b == 8 || b == 16)) {
      const int given = h_bits[i];
      kvc_plan_destroy(p);
      *out = nullptr;
      return fail(KVC_ERR_INVALID_ARG, "h_bits[%lld] = %d: widths must be 0, 2, 4, 8 or 16", (long long)i, given);
    }
  }
  p->mixed = true;
  return KVC_OK;
}

kvc_status kvc_plan_destroy(kvc_plan_t plan) {
  delete plan;
  return KVC_OK;
}

kvc_status kvc_plan_sizes(kvc_plan_t p, int64_t tokens, size_t* max_stream_bytes, size_t* workspace_bytes) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "plan is NULL");
  if (tokens < 0 || tokens > p->cfg.max_tokens) return fail(KVC_ERR_INVALID_ARG, "tokens must be in [0, max_tokens]");
  ReqDesc rq;
  request_layout(p, (int)tokens, rq);
  const int64_t codes_area = a256(rq.codes_bytes[0]) + a256(rq.codes_bytes[1]);
  const WsLayout w = ws_layout(rq.nchunks[0] + rq.nchunks[1], codes_area, 0, 1, slab_area(p), delta_area(p, tokens));
  if (max_stream_bytes) *max_stream_bytes = (size_t)rq.max_stream;
  if (workspace_bytes) *workspace_bytes = (size_t)w.total;
  return KVC_OK;
}

kvc_status kvc_plan_sizes_paged(kvc_plan_t p, const int32_t* lens, int32_t R, size_t* max_total, size_t* ws_bytes) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "plan is NULL");
  if (R < 0 || (R > 0 && !lens)) return fail(KVC_ERR_INVALID_ARG, "bad request list");
  for (int r = 0; r < R; ++r)
    if (lens[r] < 0 || lens[r] > (1 << 26)) return fail(KVC_ERR_INVALID_ARG, "seq_lens[%d] out of range", r);
  const PagedJob je = paged_job(p, lens, R, true);
  const PagedJob jd = paged_job(p, lens, R, false);
  const WsLayout we = ws_layout(je.chunks, je.codes_area, je.params_area, R);
  const WsLayout wd = ws_layout(jd.chunks, jd.codes_area, jd.params_area, R);
  if (max_total) *max_total = (size_t)je.max_total;
  if (ws_bytes) *ws_bytes = (size_t)std::max(we.total, wd.total);
  return KVC_OK;
}

kvc_status kvc_encode(kvc_plan_t p, const void* d_k, const void* d_v, int32_t tokens, void* d_out,
                      size_t out_capacity, void* d_ws, size_t ws_bytes, size_t* h_out_bytes, void* stream) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "plan is NULL");
  if (tokens < 0 || tokens > p->cfg.max_tokens) return fail(KVC_ERR_INVALID_ARG, "tokens must be in [0, max_tokens]");
  kvc_status st;
  if (tokens > 0) {
    if ((st = check_ptr(d_k, 16, "d_k")) != KVC_OK) return st;
    if ((st = check_ptr(d_v, 16, "d_v")) != KVC_OK) return st;
  }
  if ((st = check_ptr(d_out, 16, "d_out")) != KVC_OK) return st;
  if ((st = check_ptr(d_ws, 256, "d_ws")) != KVC_OK) return st;
  CallDesc c;
  fill_common(p, c);
  c.R = 1;
  request_layout(p, tokens, c.one);
  const int64_t codes_area = a256(c.one.codes_bytes[0]) + a256(c.one.codes_bytes[1]);
  // The fused kernels write the codes where a stream whose chunks are all raw
  // keeps them (K codes at the payload start, V codes 16-byte aligned after
  // them); compressed chunks and raw chunks that must move go through the
  // workspace codes area, which uses the same offsets.
  c.one.codes_off[1] = a16(c.one.codes_bytes[0]);
  int64_t delta_k = 0;
  const WsLayout w =
      ws_layout(c.one.nchunks[0] + c.one.nchunks[1], codes_area, 0, 1, slab_area(p), delta_area(p, tokens, &delta_k));
  if ((int64_t)out_capacity < c.one.max_stream)
    return fail(KVC_ERR_BUFFER_TOO_SMALL, "out_capacity %zu < %lld", out_capacity, (long long)c.one.max_stream);
  if ((int64_t)ws_bytes < w.total) return fail(KVC_ERR_BUFFER_TOO_SMALL, "ws_bytes %zu < %lld", ws_bytes, (long long)w.total);
  uint8_t* ws = (uint8_t*)d_ws;
  c.in_kv[0] = d_k;
  c.in_kv[1] = d_v;
  c.codes = (uint8_t*)d_out + c.one.payload_off;
  c.codes_out = ws + w.codes;
  c.stream = (uint8_t*)d_out;
  c.chunk_sizes = (uint32_t*)(ws + w.sizes);
  c.chunk_counts = (uint32_t*)(ws + w.counts);
  c.chunk_offs = (uint64_t*)(ws + w.offs);
  c.ctl = (Control*)(ws + w.ctl);
  c.total_chunks = c.one.nchunks[0] + c.one.nchunks[1];
  c.place = 1;
  c.place_flags = (uint32_t*)(ws + w.flags);
  c.scan_state = (uint64_t*)(ws + w.scan);
  for (int k = 0; k < 2; ++k) c.tiles[k] = tiles_of(p->pol[k], c.layers, tokens, c.heads, false);
  c.nnz_pipe = lossless_pipe(p->cfg.lossless);
  for (int k = 0; k < 2; ++k) c.nnz_sec[k] = (c.nnz_pipe && fused_count_ok(p->pol[k], tokens, p->cfg.chunk_bytes)) ? 1 : 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  SlabTables tb;
  if (p->mixed) {
    if ((st = upload_slabs(p, tokens, ws + w.slabs, s, c, tb)) != KVC_OK) return st;
    c.nnz_sec[0] = c.nnz_sec[1] = 0;
  }
  if ((e = timed(KVC_KERNEL_AUX, s, [&] { return launch_reset(c, s); })) != hipSuccess) return hip_fail(e, "reset");
  // token delta: the fused encoders read the transformed copy in the workspace
  for (int k = 0; k < 2; ++k) {
    if (!p->pol[k].delta || tokens == 0) continue;
    uint8_t* y = ws + w.delta + (k ? delta_k : 0);
    const void* x = c.in_kv[k];
    if ((e = timed(KVC_KERNEL_DELTA, s, [&] { return launch_delta(c, k, tokens, true, x, y, s); })) != hipSuccess)
      return hip_fail(e, "delta");
    c.in_kv[k] = y;
  }
  // values first: on the 70B shapes the value encoder measured 2-4 % faster
  // when it does not follow the key encoder, the key encoder 1 % slower when
  // it follows the value encoder, the whole step about 0.5-1.5 % faster
  if ((e = timed(KVC_KERNEL_ENCODE_V, s, [&] { return fused_all(p, c, tb, 1, true, s); })) != hipSuccess) return hip_fail(e, "encode V");
  if ((e = timed(KVC_KERNEL_ENCODE_K, s, [&] { return fused_all(p, c, tb, 0, true, s); })) != hipSuccess) return hip_fail(e, "encode K");
  // every chunk counted by the fused kernels and encoded by the placement:
  // the scan turns the counts into sizes itself
  c.counts_to_sizes = (c.nnz_pipe && c.nnz_sec[0] && c.nnz_sec[1] && all_word_parallel(c)) ? 1 : 0;
  if (!c.counts_to_sizes)
    if ((e = timed(KVC_KERNEL_LOSSLESS_ENC, s, [&] { return launch_lossless_encode(c, s); })) != hipSuccess) return hip_fail(e, "lossless");
  if ((e = timed(KVC_KERNEL_SCAN, s, [&] { return launch_scan(c, false, s); })) != hipSuccess) return hip_fail(e, "scan");
  if ((e = timed(KVC_KERNEL_COMPACT, s, [&] { return launch_place(c, s); })) != hipSuccess) return hip_fail(e, "place");
  if (h_out_bytes) {
    Control h;
    if ((st = sync_and_read(c.ctl, s, h)) != KVC_OK) return st;
    *h_out_bytes = (size_t)h.total;
    return device_status(h.status);
  }
  return KVC_OK;
}

kvc_status kvc_decode(kvc_plan_t p, const void* d_in, size_t in_bytes, int32_t tokens, void* d_k, void* d_v,
                      void* d_ws, size_t ws_bytes, void* stream) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "plan is NULL");
  if (tokens < 0 || tokens > p->cfg.max_tokens) return fail(KVC_ERR_INVALID_ARG, "tokens must be in [0, max_tokens]");
  kvc_status st;
  if ((st = check_ptr(d_in, 16, "d_in")) != KVC_OK) return st;
  if (tokens > 0) {
    if ((st = check_ptr(d_k, 16, "d_k")) != KVC_OK) return st;
    if ((st = check_ptr(d_v, 16, "d_v")) != KVC_OK) return st;
  }
  if ((st = check_ptr(d_ws, 256, "d_ws")) != KVC_OK) return st;
  CallDesc c;
  fill_common(p, c);
  c.R = 1;
  request_layout(p, tokens, c.one);
  if ((int64_t)in_bytes < c.one.payload_off)
    return fail(KVC_ERR_CORRUPT_STREAM, "in_bytes %zu is shorter than the stream's fixed sections (%lld)", in_bytes,
                (long long)c.one.payload_off);
  const int64_t codes_area = a256(c.one.codes_bytes[0]) + a256(c.one.codes_bytes[1]);
  c.one.codes_off[1] = a256(c.one.codes_bytes[0]);
  const WsLayout w = ws_layout(c.one.nchunks[0] + c.one.nchunks[1], codes_area, 0, 1, slab_area(p));
  if ((int64_t)ws_bytes < w.total) return fail(KVC_ERR_BUFFER_TOO_SMALL, "ws_bytes %zu < %lld", ws_bytes, (long long)w.total);
  uint8_t* ws = (uint8_t*)d_ws;
  c.out_kv[0] = d_k;
  c.out_kv[1] = d_v;
  c.codes = ws + w.codes;
  c.codes_out = c.codes;
  for (int k = 0; k < 2; ++k) c.direct[k] = tiles_within_chunks(p->pol[k], tokens, p->cfg.chunk_bytes) ? 1 : 0;
  // 2-bit per-token codes: the reconstruct kernel decodes compressed chunks of
  // TUPL8_1 -> BIT_8 -> RZE_2 itself (four tiles share one 4 KiB transpose block)
  for (int k = 0; k < 2; ++k)
    c.mirror[k] = (c.direct[k] && !p->mixed && lossless_pipe(p->cfg.lossless) == 1 && p->pol[k].axis == 0 &&
                   p->pol[k].bits == 2 && p->cfg.chunk_bytes % 4096 == 0) ? 1 : 0;
  c.stream = (uint8_t*)const_cast<void*>(d_in);
  c.stream_bytes = in_bytes;
  c.chunk_sizes = (uint32_t*)(ws + w.sizes);
  c.chunk_offs = (uint64_t*)(ws + w.offs);
  c.ctl = (Control*)(ws + w.ctl);
  c.total_chunks = c.one.nchunks[0] + c.one.nchunks[1];
  c.scan_state = (uint64_t*)(ws + w.scan);
  for (int k = 0; k < 2; ++k) c.tiles[k] = tiles_of(p->pol[k], c.layers, tokens, c.heads, false);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  SlabTables tb;
  if (p->mixed) {
    if ((st = upload_slabs(p, tokens, ws + w.slabs, s, c, tb)) != KVC_OK) return st;
    c.direct[0] = c.direct[1] = 0;
  }
  // small calls (a layer at a time, say): one launch for the whole front
  const bool small = c.total_chunks > 0 && c.total_chunks <= kFrontChunks;
  if (small) {
    if ((e = timed(KVC_KERNEL_AUX, s, [&] { return launch_dec_front_small(c, s); })) != hipSuccess) return hip_fail(e, "front");
  } else {
    c.validate_in_reset = 1;                         // one launch clears the status and checks the header
    if ((e = timed(KVC_KERNEL_AUX, s, [&] { return launch_reset(c, s); })) != hipSuccess) return hip_fail(e, "reset");
    if ((e = timed(KVC_KERNEL_SCAN, s, [&] { return launch_scan(c, true, s); })) != hipSuccess) return hip_fail(e, "scan");
  }
  if ((e = timed(KVC_KERNEL_LOSSLESS_DEC, s, [&] { return launch_lossless_decode(c, small, s); })) != hipSuccess) return hip_fail(e, "lossless");
  if ((e = timed(KVC_KERNEL_DECODE_K, s, [&] { return fused_all(p, c, tb, 0, false, s); })) != hipSuccess) return hip_fail(e, "decode K");
  if ((e = timed(KVC_KERNEL_DECODE_V, s, [&] { return fused_all(p, c, tb, 1, false, s); })) != hipSuccess) return hip_fail(e, "decode V");
  for (int k = 0; k < 2; ++k) {
    if (!p->pol[k].delta || tokens == 0) continue;
    void* x = c.out_kv[k];
    if ((e = timed(KVC_KERNEL_DELTA, s, [&] { return launch_delta(c, k, tokens, false, x, x, s); })) != hipSuccess)
      return hip_fail(e, "delta");
  }
  return KVC_OK;
}

static kvc_status paged_common(kvc_plan_t p, int64_t num_blocks, const int32_t* d_bt, int32_t maxb,
                               const int32_t* lens, int32_t R) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "plan is NULL");
  if (p->cfg.page_tokens < 1) return fail(KVC_ERR_INVALID_ARG, "plan was built without page_tokens");
  if (p->mixed) return fail(KVC_ERR_UNSUPPORTED, "paged calls do not take mixed-precision plans");
  if (p->pol[0].delta || p->pol[1].delta) return fail(KVC_ERR_UNSUPPORTED, "the token delta runs on dense calls only");
  if (p->pol[0].axis != 0 || p->pol[1].axis != 0)
    return fail(KVC_ERR_UNSUPPORTED, "paged calls implement per-token policies only");
  if (((int64_t)p->cfg.page_tokens * p->cfg.kv_heads) % 32)
    return fail(KVC_ERR_UNSUPPORTED, "page_tokens * kv_heads must be a multiple of 32");
  if (R < 1 || !lens) return fail(KVC_ERR_INVALID_ARG, "need at least one request");
  if (num_blocks < 0 || maxb < 1) return fail(KVC_ERR_INVALID_ARG, "bad pool or block table shape");
  kvc_status st;
  if ((st = check_ptr(d_bt, 4, "d_block_table")) != KVC_OK) return st;
  for (int r = 0; r < R; ++r) {
    if (lens[r] < 0 || lens[r] > (1 << 26)) return fail(KVC_ERR_INVALID_ARG, "seq_lens[%d] out of range", r);
    if (cdiv(lens[r], p->cfg.page_tokens) > maxb)
      return fail(KVC_ERR_INVALID_ARG, "seq_lens[%d] needs more than max_blocks_per_req pages", r);
  }
  return KVC_OK;
}

kvc_status kvc_encode_paged(kvc_plan_t p, const void* d_k_pool, const void* d_v_pool, int64_t num_blocks,
                            const int32_t* d_bt, int32_t maxb, const int32_t* lens, int32_t R, void* d_out,
                            size_t out_capacity, uint64_t* d_req_offsets, void* d_ws, size_t ws_bytes,
                            size_t* h_out_bytes, void* stream) {
  kvc_status st = paged_common(p, num_blocks, d_bt, maxb, lens, R);
  if (st != KVC_OK) return st;
  if ((st = check_ptr(d_k_pool, 16, "d_k_pool")) != KVC_OK) return st;
  if ((st = check_ptr(d_v_pool, 16, "d_v_pool")) != KVC_OK) return st;
  if ((st = check_ptr(d_out, 16, "d_out")) != KVC_OK) return st;
  if ((st = check_ptr(d_req_offsets, 8, "d_req_offsets")) != KVC_OK) return st;
  if ((st = check_ptr(d_ws, 256, "d_ws")) != KVC_OK) return st;
  PagedJob j = paged_job(p, lens, R, true);
  const WsLayout w = ws_layout(j.chunks, j.codes_area, j.params_area, R);
  if ((int64_t)out_capacity < j.max_total) return fail(KVC_ERR_BUFFER_TOO_SMALL, "out_capacity too small");
  if ((int64_t)ws_bytes < w.total) return fail(KVC_ERR_BUFFER_TOO_SMALL, "ws_bytes too small");
  CallDesc c;
  fill_common(p, c);
  uint8_t* ws = (uint8_t*)d_ws;
  c.R = R;
  c.one = j.reqs[0];
  c.reqs = (const ReqDesc*)(ws + w.reqs);
  c.page_tokens = p->cfg.page_tokens;
  c.num_blocks = num_blocks;
  c.block_table = d_bt;
  c.max_blocks = maxb;
  c.in_kv[0] = d_k_pool;
  c.in_kv[1] = d_v_pool;
  c.codes = (uint8_t*)d_out;
  c.codes_out = ws + w.codes;
  c.place_flags = (uint32_t*)(ws + w.flags);
  c.params_ws = ws + w.params;
  c.stream = (uint8_t*)d_out;
  c.req_offsets_out = d_req_offsets;
  c.chunk_sizes = (uint32_t*)(ws + w.sizes);
  c.chunk_offs = (uint64_t*)(ws + w.offs);
  c.ctl = (Control*)(ws + w.ctl);
  c.total_chunks = j.chunks;
  c.total_pieces = j.pieces;
  c.tiles[0] = j.tiles[0];
  c.tiles[1] = j.tiles[1];
  c.place = 2;                   // chunks move in place from their all-raw positions
  c.scan_state = (uint64_t*)(ws + w.scan);
  // the fused encoders count the non-zero RZE words of each chunk, so the
  // size pass reads only counters
  c.chunk_counts = (uint32_t*)(ws + w.counts);
  c.nnz_pipe = lossless_pipe(p->cfg.lossless);
  for (int k = 0; k < 2; ++k) c.nnz_sec[k] = paged_count_ok(p->pol[k], c.nnz_pipe, p->cfg.kv_heads, lens, R) ? 1 : 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (R > 1) {
    // pageable source: the copy has taken the bytes when it returns
    const std::vector<uint8_t> area = request_area(j, ws + w.reqs, c);
    e = hipMemcpyAsync(ws + w.reqs, area.data(), area.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(requests)");
  }
  if ((e = timed(KVC_KERNEL_AUX, s, [&] { return launch_reset(c, s); })) != hipSuccess) return hip_fail(e, "reset");
  if ((e = timed(KVC_KERNEL_ENCODE_K, s, [&] { return launch_encode_fused(c, 0, s); })) != hipSuccess) return hip_fail(e, "encode K");
  if ((e = timed(KVC_KERNEL_ENCODE_V, s, [&] { return launch_encode_fused(c, 1, s); })) != hipSuccess) return hip_fail(e, "encode V");
  if ((e = timed(KVC_KERNEL_LOSSLESS_ENC, s, [&] { return launch_lossless_encode(c, s); })) != hipSuccess) return hip_fail(e, "lossless");
  if ((e = timed(KVC_KERNEL_SCAN, s, [&] { return launch_scan(c, false, s); })) != hipSuccess) return hip_fail(e, "scan");
  // the placement first: the tables, headers and parameter sections that the
  // compaction writes at the final request offsets may cover codes of earlier
  // requests that are still to move
  if ((e = timed(KVC_KERNEL_COMPACT, s, [&] { return launch_place(c, s); })) != hipSuccess) return hip_fail(e, "place");
  if ((e = timed(KVC_KERNEL_COMPACT, s, [&] { return launch_compact(c, s); })) != hipSuccess) return hip_fail(e, "compact");
  if (h_out_bytes) {
    Control h;
    if ((st = sync_and_read(c.ctl, s, h)) != KVC_OK) return st;
    *h_out_bytes = (size_t)h.total;
    return device_status(h.status);
  }
  return KVC_OK;
}

kvc_status kvc_decode_paged(kvc_plan_t p, const void* d_in, size_t in_bytes, const uint64_t* d_req_offsets,
                            const int32_t* lens, int32_t R, void* d_k_pool, void* d_v_pool, int64_t num_blocks,
                            const int32_t* d_bt, int32_t maxb, void* d_ws, size_t ws_bytes, void* stream) {
  kvc_status st = paged_common(p, num_blocks, d_bt, maxb, lens, R);
  if (st != KVC_OK) return st;
  if ((st = check_ptr(d_in, 16, "d_in")) != KVC_OK) return st;
  if ((st = check_ptr(d_req_offsets, 8, "d_req_offsets")) != KVC_OK) return st;
  if ((st = check_ptr(d_k_pool, 16, "d_k_pool")) != KVC_OK) return st;
  if ((st = check_ptr(d_v_pool, 16, "d_v_pool")) != KVC_OK) return st;
  if ((st = check_ptr(d_ws, 256, "d_ws")) != KVC_OK) return st;
  PagedJob j = paged_job(p, lens, R, false);
  const WsLayout w = ws_layout(j.chunks, j.codes_area, j.params_area, R);
  if ((int64_t)ws_bytes < w.total) return fail(KVC_ERR_BUFFER_TOO_SMALL, "ws_bytes too small");
  CallDesc c;
  fill_common(p, c);
  uint8_t* ws = (uint8_t*)d_ws;
  c.R = R;
  c.one = j.reqs[0];
  c.reqs = (const ReqDesc*)(ws + w.reqs);
  c.page_tokens = p->cfg.page_tokens;
  c.num_blocks = num_blocks;
  c.block_table = d_bt;
  c.max_blocks = maxb;
  c.out_kv[0] = d_k_pool;
  c.out_kv[1] = d_v_pool;
  c.codes = ws + w.codes;
  c.codes_out = c.codes;
  c.stream = (uint8_t*)const_cast<void*>(d_in);
  c.stream_bytes = in_bytes;
  c.req_offsets = d_req_offsets;
  c.chunk_sizes = (uint32_t*)(ws + w.sizes);
  c.chunk_offs = (uint64_t*)(ws + w.offs);
  c.ctl = (Control*)(ws + w.ctl);
  c.total_chunks = j.chunks;
  c.tiles[0] = j.tiles[0];
  c.tiles[1] = j.tiles[1];
  c.scan_state = (uint64_t*)(ws + w.scan);
  // raw chunks are read from the stream by the reconstruct kernels
  c.direct[0] = c.direct[1] = 1;
  c.straddle = 1;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (R > 1) {
    const std::vector<uint8_t> area = request_area(j, ws + w.reqs, c);
    e = hipMemcpyAsync(ws + w.reqs, area.data(), area.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(requests)");
  }
  if ((e = timed(KVC_KERNEL_AUX, s, [&] { return launch_reset(c, s); })) != hipSuccess) return hip_fail(e, "reset");
  if ((e = timed(KVC_KERNEL_AUX, s, [&] { return launch_validate(c, s); })) != hipSuccess) return hip_fail(e, "validate");
  if ((e = timed(KVC_KERNEL_SCAN, s, [&] { return launch_scan(c, true, s); })) != hipSuccess) return hip_fail(e, "scan");
  if ((e = timed(KVC_KERNEL_LOSSLESS_DEC, s, [&] { return launch_lossless_decode(c, false, s); })) != hipSuccess) return hip_fail(e, "lossless");
  if ((e = timed(KVC_KERNEL_DECODE_K, s, [&] { return launch_decode_fused(c, 0, s); })) != hipSuccess) return hip_fail(e, "decode K");
  if ((e = timed(KVC_KERNEL_DECODE_V, s, [&] { return launch_decode_fused(c, 1, s); })) != hipSuccess) return hip_fail(e, "decode V");
  return KVC_OK;
}

// ---------------------------------------------------------------- no-allocation encode

}  // extern "C"

// Workspace of kvc_encode_noalloc.  Every device the library runs this entry
// point on holds its own copy until the process ends.  In host code the name
// is only a stand-in for the device symbol: kernels and copies get the
// per-device address that hipGetSymbolAddress returns, never this name.
static __device__ __align__(256) uint8_t scratch[KVC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's copy of `scratch`, looked up once per
// device with that device current.
kvc_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(KVC_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || ((uintptr_t)ptr) % 256) return fail(KVC_ERR_HIP, "scratch symbol address is NULL or misaligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVC_OK;
}
}  // namespace

extern "C" {

kvc_status kvc_encode_noalloc(kvc_plan_t p, const void* d_k, const void* d_v, int32_t tokens, void* d_out,
                              size_t out_capacity, size_t* h_out_bytes, void* stream) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "plan is NULL");
  if (p->mixed)
    return fail(KVC_ERR_UNSUPPORTED, "kvc_encode_noalloc: mixed-precision plans upload slab tables from the host; "
                                     "use kvc_encode");
  if (tokens < 0 || tokens > p->cfg.max_tokens) return fail(KVC_ERR_INVALID_ARG, "tokens must be in [0, max_tokens]");
  size_t ms = 0, need = 0;
  kvc_status st = kvc_plan_sizes(p, tokens, &ms, &need);
  if (st != KVC_OK) return st;
  if (need > (size_t)KVC_NOALLOC_SCRATCH_BYTES)
    return fail(KVC_ERR_BUFFER_TOO_SMALL,
                "kvc_encode_noalloc: this call needs %zu bytes of workspace, more than the library's fixed %zu-byte "
                "scratch; use kvc_encode with a workspace", need, (size_t)KVC_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != KVC_OK) return st;
  return kvc_encode(p, d_k, d_v, tokens, d_out, out_capacity, ws, (size_t)KVC_NOALLOC_SCRATCH_BYTES, h_out_bytes,
                    stream);
}

kvc_status kvc_query_status(kvc_plan_t p, const void* d_ws, void* stream) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "plan is NULL");
  kvc_status st = check_ptr(d_ws, 256, "d_ws");
  if (st != KVC_OK) return st;
  Control h;
  Control* ctl = (Control*)const_cast<void*>(d_ws);
  if ((st = sync_and_read(ctl, (hipStream_t)stream, h)) != KVC_OK) return st;
  CallDesc c;
  std::memset(&c, 0, sizeof(c));
  c.ctl = ctl;
  hipError_t e = launch_reset(c, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reset");
  return device_status(h.status);
}

kvc_status kvc_probe_bandwidth(const void* d_src, void* d_dst, int64_t items, int reads, int writes, int flags,
                               uint32_t* d_sink, void* stream) {
  if (items < 0) return fail(KVC_ERR_INVALID_ARG, "items must be >= 0");
  if (flags & ~(KVC_PROBE_NT_LOADS | KVC_PROBE_SHORT_WAVES)) return fail(KVC_ERR_INVALID_ARG, "unknown probe flags %d", flags);
  const int pair = (reads < 0 || reads > 4 || writes < 0 || writes > 4) ? -1 : reads * 16 + writes;
  if (pair != 0x10 && pair != 0x01 && pair != 0x11 && pair != 0x21 && pair != 0x41 && pair != 0x14)
    return fail(KVC_ERR_UNSUPPORTED, "no probe for %d reads : %d writes", reads, writes);
  if ((reads && !d_src) || (writes && !d_dst) || (!writes && !d_sink))
    return fail(KVC_ERR_INVALID_ARG, "a buffer the probe touches is NULL");
  const hipError_t e = launch_probe(d_src, d_dst, items, reads, writes, flags, d_sink, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "probe");
  return KVC_OK;
}

kvc_status kvc_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return KVC_OK;
}

kvc_status kvc_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_harvest_locked();
  for (int k = 0; k < KVC_KERNEL_COUNT; ++k) { g_prof_ms[k] = 0; g_prof_n[k] = 0; }
  return KVC_OK;
}

kvc_status kvc_profile_query(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= KVC_KERNEL_COUNT) return fail(KVC_ERR_INVALID_ARG, "bad kernel kind");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_harvest_locked();
  if (total_ms) *total_ms = g_prof_ms[kind];
  if (launches) *launches = g_prof_n[kind];
  return KVC_OK;
}

}  // extern "C"
