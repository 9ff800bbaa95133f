// Measurement kernel of libvqd (gfx950): a plain streaming read of device
// buffers.  It computes nothing of the method.  Its launch period over a
// layer's index bytes is the floor that the lookup kernels' own periods are
// compared with: the same bytes per launch, read with the lookup kernels'
// load width, cache policy and launch shape, and nothing else.
#include <hip/hip_runtime.h>

#include "vq_internal.h"

namespace vqd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufferWord3 = 0x00020000;
constexpr int kNontemporal = 2;

// Workgroup (x, m) reads bytes [32 KiB x, 32 KiB (x + 1)) of buffer m; wave
// w of it reads the four 1 KiB chunks at 4 KiB w, lane l the 16 bytes at
// 16 l of each, all four requested before the first is used.  Offsets past
// the buffer's end load zeros without a memory access.  Each wave stores
// the XOR of what it read, so no load can be dropped.
__global__ void __launch_bounds__(RD_W * 64) stream_read_kernel(const ReadArgs a) {
  const int m = blockIdx.y;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.buf[m]), (short)0, (int)a.bytes[m], kBufferWord3);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t base = ((uint32_t)blockIdx.x * RD_W + (uint32_t)wave) * (RD_NCH * 1024u) +
                        (uint32_t)lane * 16u;
  u32x4 v[RD_NCH];
#pragma unroll
  for (int c = 0; c < RD_NCH; ++c)
    v[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, base + c * 1024u, 0,
                                                                           kNontemporal));
  uint32_t h = 0u;
#pragma unroll
  for (int c = 0; c < RD_NCH; ++c) h ^= v[c][0] ^ v[c][1] ^ v[c][2] ^ v[c][3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) h ^= __shfl_xor(h, o);
  if (lane == 0) a.sink[((size_t)m * gridDim.x + blockIdx.x) * RD_W + wave] = h;
}

}  // namespace

int launch_stream_read(const ReadArgs &a, int grid_x, void *stream) {
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid_x, a.count), dim3(RD_W * 64), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace vqd
