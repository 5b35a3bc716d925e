// wq_probe.hip -- measurement aid, not part of the product: a plain streaming
// read of a device buffer.
//
// Decode-sized products are bound by the bytes they move (exllama bandwidth
// discussion, GPTQ paper quote and turboderp's reply), so the fastest a GEMV
// launch over B weight bytes can run is the time one launch needs just to read
// B bytes.  This kernel measures that: it reads the buffer once, with 128-bit
// non-temporal buffer loads (the weight stream's own load form), and does no
// arithmetic besides folding the words into one register so the loads stay.
//
// Each workgroup (256 threads) reads one contiguous chunk, U loads of 16 bytes
// per lane in flight per step; the caller chooses the workgroup count and U,
// so a sweep of both gives the best a single launch achieves for that size.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wq_probe.h"
#include "wq_decode.hpp"

namespace {

using wq::make_rsrc;
using wq::rsrc_t;
using wq::u32x4;

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* base, uint64_t bytes, uint32_t chunk,
                                                          uint32_t* sink) {
  const uint64_t start = (uint64_t)blockIdx.x * chunk;
  if (start >= bytes) return;
  const uint64_t left = bytes - start;
  const uint32_t len = left < chunk ? (uint32_t)left : chunk;
  // loads past `len` return zero without touching memory
  const rsrc_t r = make_rsrc(base + start, len);
  constexpr uint32_t kStep = 256u * 16u * U;  // bytes per workgroup step
  const uint32_t lane_off = threadIdx.x * 16u;
  uint32_t acc = 0;
  for (uint32_t off = 0; off < len; off += kStep) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off + (uint32_t)u * 4096u, off, wq::kNontemporal);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // keeps the loads alive; every writer stores the same value to one word
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

template <int U>
void launch(const void* buf, uint64_t bytes, int wgs, uint32_t* sink, hipStream_t s) {
  constexpr uint64_t step = 256u * 16u * U;
  uint64_t chunk = (bytes + wgs - 1) / wgs;
  chunk = (chunk + step - 1) / step * step;
  const unsigned grid = (unsigned)((bytes + chunk - 1) / chunk);
  hipLaunchKernelGGL(stream_read_kernel<U>, dim3(grid), dim3(256), 0, s, (const uint8_t*)buf, bytes,
                     (uint32_t)chunk, sink);
}

}  // namespace

extern "C" int wq_probe_stream_read(const void* buf, size_t bytes, int workgroups, int loads_in_flight,
                                    uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || workgroups <= 0 || workgroups > (1 << 20)) return 1;
  if ((bytes + workgroups - 1) / workgroups >= ((uint64_t)1 << 30)) return 2;  // chunk offsets stay 32-bit
  hipStream_t s = (hipStream_t)stream;
  switch (loads_in_flight) {
    case 2: launch<2>(buf, bytes, workgroups, sink, s); break;
    case 4: launch<4>(buf, bytes, workgroups, sink, s); break;
    case 8: launch<8>(buf, bytes, workgroups, sink, s); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
