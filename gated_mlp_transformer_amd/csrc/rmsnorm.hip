// RMSNorm over the hidden dimension: y = gamma * x / sqrt(mean(x^2) + eps).
// ("推理计算流梳理", Norm&Residual, RMSNorm equation.)
//
// One wavefront per row at a time, four per 256-thread workgroup, striding
// over the rows; each lane holds its 16-byte slices of the row in registers
// (the next row's are loaded while the current one is reduced and written),
// so a row is read from HBM once and written once (HBM-bound: 2 * d *
// sizeof(T) bytes per row).
//
// The bf16 kernels can also emit the row's per-token fp8 activations for the
// block-fp8 prefill variant in the same pass: the bf16 output values are cut
// into groups of 128 channels (16 lanes' 16-byte slices of one vector index,
// i.e. one DPP row), the group scale is s = max(amax, 1e-4) / 448 and each
// code is the E4M3FN value nearest to y / s (ties to even), in fp32 with IEEE
// division -- the quantiser's rule applied to the bf16 values it would read.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row_umax(uint32_t v) {
  // lanes outside the source row receive 0, the identity of the unsigned max
  const uint32_t o = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
  return v > o ? v : o;
}

template <bool HI>
__device__ __forceinline__ uint32_t fp8_encode2(float a, float b, float s, uint32_t old) {
  a = fminf(fmaxf(a / s, -448.0f), 448.0f);
  b = fminf(fmaxf(b / s, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), HI));
}

// fp8 codes of the eight bf16 values in o (this lane's slice of a 128-channel
// group held by the lane's 16-lane DPP row) to q8 (8 bytes); the lane at the
// start of the row writes the group scale to *scale.
__device__ __forceinline__ void quant_group_store(const u32x4& o, int lane, uint8_t* q8,
                                                  float* scale) {
  float f[8];
  unpack_bf16x8(o, f);
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  uint32_t mb = __float_as_uint(m);  // non-negative floats order as unsigned integers
  mb = dpp_row_umax<0xB1>(mb);   // quad_perm [1,0,3,2]
  mb = dpp_row_umax<0x4E>(mb);   // quad_perm [2,3,0,1]
  mb = dpp_row_umax<0x141>(mb);  // row_half_mirror
  mb = dpp_row_umax<0x140>(mb);  // row_mirror: every lane of the row has its max
  const float sc = fmaxf(__uint_as_float(mb), 1e-4f) / 448.0f;
  u32x2 out;
  out[0] = fp8_encode2<false>(f[0], f[1], sc, 0u);
  out[0] = fp8_encode2<true>(f[2], f[3], sc, out[0]);
  out[1] = fp8_encode2<false>(f[4], f[5], sc, 0u);
  out[1] = fp8_encode2<true>(f[6], f[7], sc, out[1]);
  *reinterpret_cast<u32x2*>(q8) = out;
  if ((lane & 15) == 0) *scale = sc;
}

}  // namespace

template <typename T, int MAXV>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* x, const T* __restrict__ gamma,
                                                      T* y, int64_t rows, int d, float eps,
                                                      uint8_t* __restrict__ q,
                                                      float* __restrict__ qs) {
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
          if (q != nullptr)  // whole 16-lane rows take this branch together (d % 128 == 0)
            quant_group_store(o, lane, q + row * d + static_cast<int64_t>(vi) * 8,
                              qs + row * (d / 128) + vi / 16);
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
// row per wave at a time, gamma re-read from cache per row. For few rows
// (GPRE: latency, not bandwidth, decides) gamma's loads are issued with the
// row's, so that they are not a second round trip after the sum; for many
// rows they come after it, which keeps the kernel at fewer registers (more
// waves per SIMD, more row loads in flight).
// QUANT (bf16 only) adds the fp8 codes of the output; it is a separate
// instantiation because the encode path's registers would otherwise cost the
// plain kernel waves per SIMD (101 against 61 VGPRs at d = 4096).
template <typename T, int NV, bool GPRE, bool QUANT>
__global__ __launch_bounds__(256) void rmsnorm_full_kernel(const T* x, const T* __restrict__ gamma,
                                                           T* y, int64_t rows, int d, float eps,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ qs) {
  const int lane = threadIdx.x % kWave;
  const char* gr = reinterpret_cast<const char*>(gamma) + lane * 16;
  const int wpg = blockDim.x / kWave;  // one row per wave: 4 per workgroup, or 1 for few rows
  const int64_t stride = static_cast<int64_t>(gridDim.x) * wpg;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * wpg + threadIdx.x / kWave; row < rows;
       row += stride) {
    const char* xr = reinterpret_cast<const char*>(x + row * d) + lane * 16;
    u32x4 v[NV], gv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = ld16(xr + i * kWave * 16);
    if constexpr (GPRE) {
#pragma unroll
      for (int i = 0; i < NV; ++i) gv[i] = ld16(gr + i * kWave * 16);
    }
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
      const u32x4 g = GPRE ? gv[i] : ld16(gr + i * kWave * 16);
      u32x4 o;
      if constexpr (sizeof(T) == 2) {
        // pair by pair (no unpacked copy of the slice): 61 VGPRs at d = 4096,
        // eight waves per SIMD, every row of the 8192-row prefill resident at
        // once (with the slice unpacked, 67 VGPRs left a second round of 1024)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pack_bf16x2(__uint_as_float(g[e] << 16) * (__uint_as_float(v[i][e] << 16) * r),
                             __uint_as_float(g[e] & 0xFFFF0000u) *
                                 (__uint_as_float(v[i][e] & 0xFFFF0000u) * r));
        if constexpr (QUANT) {
          const int vi = lane + i * kWave;
          quant_group_store(o, lane, q + row * d + static_cast<int64_t>(vi) * 8,
                            qs + row * (d / 128) + vi / 16);
        }
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

template <typename T, bool QUANT>
bool launch_full_q(const void* x, const void* gamma, void* y, int64_t rows, int d, float eps,
                   uint8_t* q, float* qs, hipStream_t s) {
  const int per_lane = d * static_cast<int>(sizeof(T)) / (16 * kWave);  // vectors per lane
  if (d * static_cast<int>(sizeof(T)) % (16 * kWave) != 0) return false;
  int64_t blocks = (rows + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  const dim3 grid(static_cast<unsigned>(blocks < 1 ? 1 : blocks));
  auto* xp = static_cast<const T*>(x);
  auto* gp = static_cast<const T*>(gamma);
  auto* yp = static_cast<T*>(y);
  if (rows <= 1024) {  // few rows: gamma with the row (one round trip)
    // up to 256 rows: one row per 64-thread workgroup, spread over as many CUs
    const bool spread = rows <= 256;
    const dim3 g1 = spread ? dim3(static_cast<unsigned>(rows < 1 ? 1 : rows)) : grid;
    const int nt = spread ? kWave : 256;
    switch (per_lane) {
      case 1: rmsnorm_full_kernel<T, 1, true, QUANT><<<g1, nt, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs); return true;
      case 2: rmsnorm_full_kernel<T, 2, true, QUANT><<<g1, nt, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs); return true;
      case 4: rmsnorm_full_kernel<T, 4, true, QUANT><<<g1, nt, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs); return true;
      case 8: rmsnorm_full_kernel<T, 8, true, QUANT><<<g1, nt, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs); return true;
      default: break;  // wider rows: the kernels below
    }
  }
  switch (per_lane) {
    case 1: rmsnorm_full_kernel<T, 1, false, QUANT><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs); return true;
    case 2: rmsnorm_full_kernel<T, 2, false, QUANT><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs); return true;
    case 4: rmsnorm_full_kernel<T, 4, false, QUANT><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs); return true;
    case 8: rmsnorm_full_kernel<T, 8, false, QUANT><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs); return true;
    case 16: rmsnorm_full_kernel<T, 16, false, QUANT><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs); return true;
    case 32:  // f32 rows of 8192
      if constexpr (sizeof(T) == 4) {
        rmsnorm_full_kernel<T, 32, false, QUANT><<<grid, 256, 0, s>>>(xp, gp, yp, rows, d, eps, q, qs);
        return true;
      }
      return false;
    default: return false;
  }
}

template <typename T>
bool launch_full(const void* x, const void* gamma, void* y, int64_t rows, int d, float eps,
                 uint8_t* q, float* qs, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (q != nullptr) return launch_full_q<T, true>(x, gamma, y, rows, d, eps, q, qs, s);
  }
  return launch_full_q<T, false>(x, gamma, y, rows, d, eps, nullptr, nullptr, s);
}

}  // namespace

void launch_rmsnorm(const void* x, const void* gamma, void* y, int64_t T, int d,
                    float eps, bool bf16, hipStream_t s, uint8_t* q, float* qs) {
  if (bf16 ? launch_full<bf16_t>(x, gamma, y, T, d, eps, q, qs, s)
           : launch_full<float>(x, gamma, y, T, d, eps, nullptr, nullptr, s))
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
    if (small) rmsnorm_kernel<bf16_t, 8><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps, q, qs);
    else rmsnorm_kernel<bf16_t, 16><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps, q, qs);
  } else {
    auto* xp = static_cast<const float*>(x);
    auto* gp = static_cast<const float*>(gamma);
    auto* yp = static_cast<float*>(y);
    if (small)
      rmsnorm_kernel<float, 8><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps, nullptr, nullptr);
    else if (d * 4 <= 16 * 16 * kWave)
      rmsnorm_kernel<float, 16><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps, nullptr, nullptr);
    else
      rmsnorm_kernel<float, 32><<<grid, 256, 0, s>>>(xp, gp, yp, T, d, eps, nullptr, nullptr);
  }
}

}  // namespace mf
