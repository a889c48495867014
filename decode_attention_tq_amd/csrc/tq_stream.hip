// Streaming-read reference kernel (measurement helper, not a step of the
// method): reads a device buffer once, as fast as plain 16-byte loads allow,
// so that the decode's packed-cache read rate can be set against the rate this
// part actually reaches on a pure read stream.
//
// Each workgroup reads a contiguous slice of the buffer; inside the slice the
// 256 lanes read consecutive 16-byte pieces (4 KiB per workgroup per pass),
// kUnroll passes in flight before their values are folded, with the
// non-temporal cache policy the decode uses for its streams. Every word read
// is XOR-folded into one word per workgroup, so no load is dead.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kUnroll = 8;
constexpr int kStreamAuxNT = 2;   // non-temporal, as the decode's streamed reads

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const char* src, uint64_t n16,
                                                                       uint32_t* sink) {
  // this workgroup's slice [lo, hi) in 16-byte pieces
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t lo = per * blockIdx.x;
  const uint64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0u;
  if (lo < hi) {
    // (slices are below 2^32 bytes: the buffer resource covers this slice only)
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src + lo * 16, (uint32_t)((hi - lo) * 16));
    const uint32_t n = (uint32_t)(hi - lo);
    for (uint32_t base = 0; base < n; base += kStreamThreads * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        // pieces past the slice read zeros (range-checked buffer loads)
        const uint32_t i = base + u * kStreamThreads + threadIdx.x;
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, i * 16u, 0, kStreamAuxNT);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  // fold the workgroup's words (wave by wave through LDS)
  __shared__ uint32_t part[kStreamThreads / 64];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0u;
#pragma unroll
    for (int w = 0; w < kStreamThreads / 64; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kStreamThreads), 0, stream,
                     (const char*)src, (uint64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace tq
