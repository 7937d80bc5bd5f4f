// fp32 tensor-parallel shard of the gated MLP ("推理计算流梳理", 实际 MLP 计算策略;
// 列并行 / 行并行): H = SiLU(X Wg_s^T) * (X Wu_s^T), P = H Wd_s^T, all in fp32 FMA.
// Used for fp32 inputs (small, latency-bound shapes); bf16 shards use the
// MFMA grouped GEMM with a single group.
//
// 16x16 threads per 16x16 output tile; 16-deep K slices of both operands are
// staged through LDS. Every index is bounds-checked, so any sizes work.
#include "common.h"
#include "launch.h"

namespace mf {

template <bool GATED>
__global__ __launch_bounds__(256) void dense_f32_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ w0,
                                                        const float* __restrict__ w1,
                                                        float* __restrict__ out, int64_t M,
                                                        int K, int N) {
  __shared__ float xs[16][17];
  __shared__ float ws0[16][17];
  __shared__ float ws1[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t row = static_cast<int64_t>(blockIdx.y) * 16 + ty;
  const int col = blockIdx.x * 16 + tx;
  const int wrow = blockIdx.x * 16 + ty;  // weight row (output feature) staged by this thread
  float a0 = 0.f, a1 = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int k = k0 + tx;
    xs[ty][tx] = (row < M && k < K) ? x[row * K + k] : 0.f;
    ws0[ty][tx] = (wrow < N && k < K) ? w0[static_cast<int64_t>(wrow) * K + k] : 0.f;
    if (GATED) ws1[ty][tx] = (wrow < N && k < K) ? w1[static_cast<int64_t>(wrow) * K + k] : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      a0 = fmaf(xs[ty][kk], ws0[tx][kk], a0);
      if (GATED) a1 = fmaf(xs[ty][kk], ws1[tx][kk], a1);
    }
    __syncthreads();
  }
  if (row < M && col < N) out[row * N + col] = GATED ? siluf_(a0) * a1 : a0;
}

void launch_dense_f32(const float* x, const float* w_gate, const float* w_up, const float* w_down,
                      int64_t T, int d, int fs, float* h, float* partial, hipStream_t s) {
  const unsigned gy = static_cast<unsigned>((T + 15) / 16);
  dense_f32_kernel<true><<<dim3((fs + 15) / 16, gy), 256, 0, s>>>(x, w_gate, w_up, h, T, d, fs);
  dense_f32_kernel<false><<<dim3((d + 15) / 16, gy), 256, 0, s>>>(h, w_down, nullptr, partial, T,
                                                                  fs, d);
}

}  // namespace mf
