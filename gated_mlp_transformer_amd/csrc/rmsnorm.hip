// RMSNorm over the hidden dimension: y = gamma * x / sqrt(mean(x^2) + eps).
// ("推理计算流梳理", Norm&Residual, RMSNorm equation.)
//
// One wavefront per row, four rows per 256-thread workgroup. Each lane holds
// its 16-byte slices of the row in registers, so the row is read from HBM
// once and written once (HBM-bound: 2 * d * sizeof(T) bytes per row).
#include "common.h"
#include "launch.h"

namespace mf {

template <typename T, int MAXV>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* x, const T* __restrict__ gamma,
                                                      T* y, int64_t rows, int d, float eps) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (row >= rows) return;
  const int nvec = d / EPV;
  const char* xr = reinterpret_cast<const char*>(x + row * d);
  char* yr = reinterpret_cast<char*>(y + row * d);
  const char* gr = reinterpret_cast<const char*>(gamma);

  u32x4 v[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int vi = lane + i * kWave;
    if (vi < nvec) {
      v[i] = ld16(xr + static_cast<size_t>(vi) * 16);
      if constexpr (sizeof(T) == 2) {
        float f[8];
        unpack_bf16x8(v[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = __uint_as_float(v[i][e]);
          ss = fmaf(f, f, ss);
        }
      }
    }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);

#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int vi = lane + i * kWave;
    if (vi < nvec) {
      const u32x4 g = ld16(gr + static_cast<size_t>(vi) * 16);
      u32x4 o;
      if constexpr (sizeof(T) == 2) {
        float f[8], gf[8], res[8];
        unpack_bf16x8(v[i], f);
        unpack_bf16x8(g, gf);
#pragma unroll
        for (int e = 0; e < 8; ++e) res[e] = gf[e] * (f[e] * r);
        o = pack_bf16x8(res);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = __float_as_uint(__uint_as_float(g[e]) * (__uint_as_float(v[i][e]) * r));
      }
      st16(yr + static_cast<size_t>(vi) * 16, o);
    }
  }
}

void launch_rmsnorm(const void* x, const void* gamma, void* y, int64_t T, int d,
                    float eps, bool bf16, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((T + 3) / 4));
  if (bf16)
    rmsnorm_kernel<bf16_t, 16><<<grid, 256, 0, s>>>(
        static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(gamma),
        static_cast<bf16_t*>(y), T, d, eps);
  else
    rmsnorm_kernel<float, 16><<<grid, 256, 0, s>>>(
        static_cast<const float*>(x), static_cast<const float*>(gamma),
        static_cast<float*>(y), T, d, eps);
}

}  // namespace mf
