// RMSNorm over the hidden dimension: y = gamma * x / sqrt(mean(x^2) + eps).
// ("推理计算流梳理", Norm&Residual, RMSNorm equation.)
//
// One wavefront per row at a time, four per 256-thread workgroup, striding
// over the rows; each lane holds its 16-byte slices of the row in registers
// (the next row's are loaded while the current one is reduced and written),
// so a row is read from HBM once and written once (HBM-bound: 2 * d *
// sizeof(T) bytes per row).
#include "common.h"
#include "launch.h"

namespace mf {

template <typename T, int MAXV>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* x, const T* __restrict__ gamma,
                                                      T* y, int64_t rows, int d, float eps) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  const int lane = threadIdx.x % kWave;
  const int nvec = d / EPV;
  const char* gr = reinterpret_cast<const char*>(gamma);
  // Grid-strided rows: the next row's loads are issued before the current row
  // is reduced and written, so every wave keeps a row in flight.
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  auto load = [&](u32x4 (&v)[MAXV], int64_t r) {
    const char* xr = reinterpret_cast<const char*>(x + r * d);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int vi = lane + i * kWave;
      if (vi < nvec) v[i] = ld16(xr + static_cast<size_t>(vi) * 16);
    }
  };
  // gamma is the same for every row: held in registers for the wave's rows
  u32x4 g[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int vi = lane + i * kWave;
    if (vi < nvec) g[i] = ld16(gr + static_cast<size_t>(vi) * 16);
  }
  u32x4 cur[MAXV], nxt[MAXV];
  if (row < rows) load(cur, row);
  for (; row < rows; row += stride) {
    if (row + stride < rows) load(nxt, row + stride);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int vi = lane + i * kWave;
      if (vi < nvec) {
        if constexpr (sizeof(T) == 2) {
          float f[8];
          unpack_bf16x8(cur[i], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float f = __uint_as_float(cur[i][e]);
            ss = fmaf(f, f, ss);
          }
        }
      }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
    char* yr = reinterpret_cast<char*>(y + row * d);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int vi = lane + i * kWave;
      if (vi < nvec) {
        u32x4 o;
        if constexpr (sizeof(T) == 2) {
          float f[8], gf[8], res[8];
          unpack_bf16x8(cur[i], f);
          unpack_bf16x8(g[i], gf);
#pragma unroll
          for (int e = 0; e < 8; ++e) res[e] = gf[e] * (f[e] * r);
          o = pack_bf16x8(res);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = __float_as_uint(__uint_as_float(g[i][e]) * (__uint_as_float(cur[i][e]) * r));
        }
        st16(yr + static_cast<size_t>(vi) * 16, o);
      }
    }
#pragma unroll
    for (int i = 0; i < MAXV; ++i) cur[i] = nxt[i];
  }
}

// Rows that fill a whole number of 16-byte vectors per lane (d a multiple of
// 64 * 16 / sizeof(T)): no per-lane predicates (they compile to branches
// around every load and store), no register prefetch of the next row, so the
// kernel stays small and many waves per SIMD keep the loads in flight; one
// row per wave at a time, gamma re-read from cache per row.
template <typename T, int NV>
__global__ __launch_bounds__(256) void rmsnorm_full_kernel(const T* x, const T* __restrict__ gamma,
                                                           T* y, int64_t rows, int d, float eps) {
  const int lane = threadIdx.x % kWave;
  const char* gr = reinterpret_cast<const char*>(gamma) + lane * 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave; row < rows;
       row += stride) {
    const char* xr = reinterpret_cast<const char*>(x + row * d) + lane * 16;
    u32x4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = ld16(xr + i * kWave * 16);
    // sum of squares; the pairs are unpacked here by two ALU instructions the
    // compiler cannot merge with the output pass's unpacking, so that no
    // unpacked copy of the row stays in registers between the passes
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float lo, hi;
          asm("v_lshlrev_b32 %0, 16, %2\n\tv_and_b32 %1, 0xffff0000, %2"
              : "=&v"(lo), "=&v"(hi)
              : "v"(v[i][e]));
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = __uint_as_float(v[i][e]);
          ss = fmaf(f, f, ss);
        }
      }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
    char* yr = reinterpret_cast<char*>(y + row * d) + lane * 16;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const u32x4 g = ld16(gr + i * kWave * 16);
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
      st16(yr + i * kWave * 16, o);
    }
  }
}

namespace {

template <typename T>
bool launch_full(const void* x, const void* gamma, void* y, int64_t rows, int d, float eps,
                 hipStream_t s) {
  const int per_lane = d * static_cast<int>(sizeof(T)) / (16 * kWave);  // vectors per lane
  if (d * static_cast<int>(sizeof(T)) % (16 * kWave) != 0) return false;
  int64_t blocks = (rows + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  const dim3 grid(static_cast<unsigned>(blocks < 1 ? 1 : blocks));
  auto* xp = static_cast<const T*>(x);
  auto* gp = static_cast<const T*>(gamma);
  auto* yp = static_cast<T*>(y);
  switch (per_lane) {
    case 1: rmsnorm_full_kernel<T, 1><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps); return true;
    case 2: rmsnorm_full_kernel<T, 2><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps); return true;
    case 4: rmsnorm_full_kernel<T, 4><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps); return true;
    case 8: rmsnorm_full_kernel<T, 8><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps); return true;
    case 16: rmsnorm_full_kernel<T, 16><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps); return true;
    case 32:  // f32 rows of 8192
      if constexpr (sizeof(T) == 4) {
        rmsnorm_full_kernel<T, 32><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps);
        return true;
      }
      return false;
    default: return false;
  }
}

}  // namespace

void launch_rmsnorm(const void* x, const void* gamma, void* y, int64_t T, int d,
                    float eps, bool bf16, hipStream_t s) {
  if (bf16 ? launch_full<bf16_t>(x, gamma, y, T, d, eps, s)
           : launch_full<float>(x, gamma, y, T, d, eps, s))
    return;
  // about two rows per wave: enough waves to fill the chip, each with a row in flight
  int64_t blocks = (T + 7) / 8;
  if (blocks > 2048) blocks = 2048;
  const dim3 grid(static_cast<unsigned>(blocks < 1 ? 1 : blocks));
  // registers for one row per lane: 8 x 16 bytes cover d <= 4096 (bf16) /
  // 2048 (f32); 16 cover bf16 rows up to 8192 and 32 the f32 ones
  const bool small = d * (bf16 ? 2 : 4) <= 8 * 16 * kWave;
  if (bf16) {
    auto* xp = static_cast<const bf16_t*>(x);
    auto* gp = static_cast<const bf16_t*>(gamma);
    auto* yp = static_cast<bf16_t*>(y);
    if (small) rmsnorm_kernel<bf16_t, 8><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps);
    else rmsnorm_kernel<bf16_t, 16><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps);
  } else {
    auto* xp = static_cast<const float*>(x);
    auto* gp = static_cast<const float*>(gamma);
    auto* yp = static_cast<float*>(y);
    if (small) rmsnorm_kernel<float, 8><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps);
    else if (d * 4 <= 16 * 16 * kWave) rmsnorm_kernel<float, 16><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps);
    else rmsnorm_kernel<float, 32><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps);
  }
}

}  // namespace mf
