// Bandwidth reference for the measurements: a streaming kernel that reads
// and writes HBM in a fixed ratio with 16-byte buffer accesses and
// non-temporal 16-byte stores, so the fused kernels' throughput can be set
// against what the memory system gives a kernel with their read:write mix
// and no arithmetic.  Two switches: non-temporal loads (the fused kernels
// load with the default policy, except the per-token encoder's LDS DMA and
// the per-channel encoder's tiles), and one unit per wave (a grid of
// short-lived waves instead of a capped grid that loops).
#include "kvc_internal.h"

namespace kvc {

typedef int probe_i4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t probe_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// A wave takes units of 64 U items.  Item reads R 16-byte lines and writes W
// lines; instruction (u, r) of a wave reads 64 consecutive lines (1 KiB), so
// every access is a whole contiguous kilobyte, with U R loads in flight per
// lane.  The lines written hold the XOR of the item's reads (the item index
// when R = 0); with W = 0 one word is written only if the XOR of everything
// read is a value the inputs never produce, which keeps the reads.
template <int R, int W, int U, int LP>
__global__ __launch_bounds__(256) void k_probe(const uint8_t* src, uint8_t* dst, int64_t items, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  for (int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); unit * 64 * U < items; unit += waves) {
    const int64_t base = unit * 64 * U;
    const int64_t n = min((int64_t)(64 * U), items - base);
    probe_i4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = probe_i4{(int)(base + 64 * u + lane), 0, 0, 0};
    if constexpr (R > 0) {
      const __amdgpu_buffer_rsrc_t rs = probe_rsrc(src + base * R * 16, (uint32_t)(n * R * 16));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r)
          acc[u] ^= __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(((u * R + r) * 64 + lane) * 16), 0, LP);
    }
    if constexpr (W > 0) {
      const __amdgpu_buffer_rsrc_t ws = probe_rsrc(dst + base * W * 16, (uint32_t)(n * W * 16));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < W; ++k)
          __builtin_amdgcn_raw_buffer_store_b128(acc[u], ws, (int)(((u * W + k) * 64 + lane) * 16), 0, 2);
    } else {
      probe_i4 t = acc[0];
#pragma unroll
      for (int u = 1; u < U; ++u) t ^= acc[u];
      if (t.x == 0x7fffffff && t.y == -1 && t.z == 0x13579bdf && t.w == 0x2468ace0) sink[0] = 1u;
    }
  }
}

hipError_t launch_probe(const void* src, void* dst, int64_t items, int reads, int writes, int flags,
                        uint32_t* sink, hipStream_t s) {
  constexpr int U = 4;
  // a block is 4 waves of 64 U items each; short waves: one unit per wave
  const int64_t blocks = (items + 1024 * U - 1) / (1024 * U);
  const int64_t cap = (flags & 2) ? (int64_t)INT32_MAX : 256 * 32;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(blocks, cap));
  const uint8_t* a = (const uint8_t*)src;
  uint8_t* b = (uint8_t*)dst;
#define KVC_PROBE(RR, WW)                                                                    \
  if (reads == RR && writes == WW) {                                                         \
    if (flags & 1) k_probe<RR, WW, U, 2><<<grid, 256, 0, s>>>(a, b, items, sink);            \
    else k_probe<RR, WW, U, 0><<<grid, 256, 0, s>>>(a, b, items, sink);                      \
    return hipGetLastError();                                                                \
  }
  KVC_PROBE(1, 0) KVC_PROBE(0, 1) KVC_PROBE(1, 1) KVC_PROBE(2, 1) KVC_PROBE(4, 1) KVC_PROBE(1, 4)
#undef KVC_PROBE
  return hipErrorInvalidValue;
}

}  // namespace kvc
