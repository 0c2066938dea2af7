// k_probe.hip — a plain streaming read of device memory.  It does nothing
// but read every byte once with non-temporal 128-bit loads, so its bandwidth
// is the practical ceiling that the weight-streaming kernels are measured
// against (the nominal HBM peak is not reachable by any kernel).
#include "gq_device.h"
#include "gq_launch.h"

namespace gq {

constexpr int kProbeUnroll = 4;          // 16-byte loads in flight per lane
// Non-temporal cache policy: each line is read once, whole, by one load, and
// streaming it past the caches measured 3-8 % faster than the default policy
// (the GEMV, whose lanes read parts of lines through several loads, loses up
// to 1.6x with it, so it keeps the default).
constexpr int kStreamPolicy = 2;

// Workgroup w XORs the 32-bit words of the 16-byte units it reads (units
// w*256 + t, stepping by the grid's width) into out[w].  Loads past the end
// of the buffer return zero (buffer range check), so every lane runs the
// same count of unrolled rounds and issues all its loads before using any.
__global__ void __launch_bounds__(256) k_stream_read(const void* __restrict__ buf, uint32_t bytes,
                                                     uint32_t* __restrict__ out) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, bytes);
  const uint32_t step = gridDim.x * 256u * 16u;
  const uint32_t rounds = (bytes + step * kProbeUnroll - 1) / (step * kProbeUnroll);
  uint32_t off = (blockIdx.x * 256u + threadIdx.x) * 16u;
  uint32_t acc = 0;
  for (uint32_t k = 0; k < rounds; k++) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; u++)
      v[u] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + u * step), 0, kStreamPolicy));
#pragma unroll
    for (int u = 0; u < kProbeUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    off += kProbeUnroll * step;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_stream_read, dim3(GQ_PROBE_OUT_WORDS), dim3(256), 0, st, buf,
                     (uint32_t)bytes, out);
  return hipGetLastError();
}

}  // namespace gq
