// Measurement probes (not part of the FFN path): the attainable MFMA rate and
// HBM read bandwidth of the GPU they run on, so that a benchmark can state its
// kernels' fractions of what this chip actually sustains beside the published
// peaks.
//
//  - mfma: every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on 16
//    independent accumulators (no loads, no LDS), one 256-thread workgroup per
//    CU slot of the grid; FLOPs = waves * iters * 16 * 32*32*16*2.
//  - copy: the same stream read and written to a second buffer; bytes =
//    twice the buffer size.
//  - read: a grid-strided stream of 16-byte loads over a buffer (each
//    workgroup takes 32 KB runs), each lane folding what it read into one
//    word that is stored once (so the loads are not dead); bytes = the buffer
//    size. The loads use the non-temporal policy of the kernels that stream
//    data read once (the decode weights): 7.1-7.3 TB/s here against 6.0-6.2
//    TB/s with the default policy.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

__global__ __launch_bounds__(256, 1) void probe_mfma_kernel(int iters, float* out) {
  f32x16 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x16{};
  const float seed = static_cast<float>(threadIdx.x & 7) * 0.001f;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(seed + 0.25f * i);
    b[i] = static_cast<__bf16>(1.0f - seed);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[i][threadIdx.x & 15];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src,
                                                         int64_t n16, uint32_t* out) {
  // each workgroup reads U consecutive 4 KB runs per step (U * 4 KB
  // contiguous), then moves on by the whole grid's span
  constexpr int U = 8;
  uint32_t acc = 0;
  const int64_t span = static_cast<int64_t>(gridDim.x) * blockDim.x * U;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x * U + threadIdx.x;
  for (; i + (U - 1) * static_cast<int64_t>(blockDim.x) < n16; i += span) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld16_stream(src + i + u * blockDim.x);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (int u = 0; u < U; ++u) {  // the tail of the last span
    const int64_t j = i + static_cast<int64_t>(u) * blockDim.x;
    if (j < n16) {
      const u32x4 v = ld16_stream(src + j);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

// dst = src, 16 bytes per access, each workgroup moving U consecutive 4 KB
// runs per step (the read + write pattern of the normalisation and combine
// kernels)
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t n16) {
  constexpr int U = 4;
  const int64_t span = static_cast<int64_t>(gridDim.x) * blockDim.x * U;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x * U + threadIdx.x; i < n16;
       i += span) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + static_cast<int64_t>(u) * blockDim.x;
      if (j < n16) v[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + static_cast<int64_t>(u) * blockDim.x;
      if (j < n16) dst[j] = v[u];
    }
  }
}

}  // namespace

void launch_probe_copy(const void* src, void* dst, int64_t bytes, int workgroups, hipStream_t s) {
  probe_copy_kernel<<<workgroups, 256, 0, s>>>(static_cast<const u32x4*>(src),
                                               static_cast<u32x4*>(dst), bytes / 16);
}

void launch_probe_mfma(int workgroups, int iters, float* out, hipStream_t s) {
  probe_mfma_kernel<<<workgroups, 256, 0, s>>>(iters, out);
}

void launch_probe_read(const void* src, int64_t bytes, int workgroups, uint32_t* out,
                       hipStream_t s) {
  probe_read_kernel<<<workgroups, 256, 0, s>>>(static_cast<const u32x4*>(src), bytes / 16, out);
}

}  // namespace mf
