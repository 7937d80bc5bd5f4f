// Weighted un-permute ("推理计算流梳理", EP 路径: expert outputs summed with the
// router weights back at the token's source; "「赤兔」Chitu ... MoE":
// token_unpermutation):
//   out[t] = sum_{j : inv_pos[t,j] valid} w[t,j] * y_perm[inv_pos[t,j]]  (+ residual[t])
// The optional residual is the Pre-Norm block's skip connection
// ("推理计算流梳理", Norm&Residual: the layer output is the residual stream plus
// the FFN of its normalised copy), added after the weighted sum.
//
// out may be the residual buffer itself: each element of the residual is read
// by the thread that then writes the same element of out, so neither pointer
// is declared restrict.
//
// A gather, not a scatter: one 256-thread workgroup per token reads at most k
// rows of y_perm with 16-byte loads and sums them in fp32 in slot order, so the
// result is deterministic and needs no atomics. HBM-bound: the bytes are the k
// rows read plus the output row written.
#include "common.h"
#include "launch.h"

namespace mf {

template <bool OUT_F32>
__device__ __forceinline__ void store_out(float (&acc)[8], const void* residual, void* out,
                                          int64_t t, int d, int v) {
  if (residual != nullptr) {
    if constexpr (OUT_F32) {
      const float* rr = static_cast<const float*>(residual) + t * d + static_cast<int64_t>(v) * 8;
      const u32x4 r0 = ld16(rr), r1 = ld16(rr + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += __uint_as_float(r0[e]);
        acc[4 + e] += __uint_as_float(r1[e]);
      }
    } else {
      float rf[8];
      unpack_bf16x8(
          ld16(static_cast<const bf16_t*>(residual) + t * d + static_cast<int64_t>(v) * 8), rf);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += rf[e];
    }
  }
  if constexpr (OUT_F32) {
    float* o = static_cast<float*>(out) + t * d + static_cast<int64_t>(v) * 8;
    st16(o, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                  __float_as_uint(acc[3])});
    st16(o + 4, u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]),
                      __float_as_uint(acc[7])});
  } else {
    bf16_t* o = static_cast<bf16_t*>(out) + t * d + static_cast<int64_t>(v) * 8;
    st16(o, pack_bf16x8(acc));
  }
}

template <bool OUT_F32, bool PAIR>
__global__ __launch_bounds__(256) void combine_kernel(const bf16_t* __restrict__ y,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ w, int k, int d,
                                                      int64_t max_rows, const void* residual,
                                                      void* out) {
  const int64_t t = blockIdx.x;
  int64_t pos[8];
  float wt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pos[j] = -1;
    wt[j] = 0.f;
    if (j < k) {
      const int64_t p = inv_pos[t * k + j];
      if (p >= 0 && p < max_rows) {
        pos[j] = p;
        wt[j] = w[t * k + j];
      }
    }
  }
  const int nvec = d / 8;
  if constexpr (!PAIR) {
    for (int v = threadIdx.x; v < nvec; v += 256) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      u32x4 rows[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (pos[j] >= 0) rows[j] = ld16(y + pos[j] * d + static_cast<int64_t>(v) * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (pos[j] >= 0) {
          float f[8];
          unpack_bf16x8(rows[j], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(wt[j], f[e], acc[e]);
        }
      }
      store_out<OUT_F32>(acc, residual, out, t, d, v);
    }
    return;
  }
  // PAIR (few tokens: latency decides): two 16-byte vectors per thread per
  // pass (d = 4096: the whole row in one pass), every row load of the pass
  // issued before the first FMA. Many tokens keep one vector per pass, whose
  // fewer registers leave more waves per SIMD with loads in flight.
  for (int v0 = threadIdx.x; v0 < nvec; v0 += 512) {
    const int v1 = v0 + 256;
    const bool has1 = v1 < nvec;
    float acc[2][8];
    u32x4 rows[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (pos[j] >= 0) {
        rows[0][j] = ld16(y + pos[j] * d + static_cast<int64_t>(v0) * 8);
        if (has1) rows[1][j] = ld16(y + pos[j] * d + static_cast<int64_t>(v1) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (pos[j] >= 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (u == 1 && !has1) break;
          float f[8];
          unpack_bf16x8(rows[u][j], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[u][e] = fmaf(wt[j], f[e], acc[u][e]);
        }
      }
    }
    store_out<OUT_F32>(acc[0], residual, out, t, d, v0);
    if (has1) store_out<OUT_F32>(acc[1], residual, out, t, d, v1);
  }
}

void launch_combine(const void* y_perm, const int32_t* inv_pos, const float* w, int64_t T, int k,
                    int d, int64_t max_rows, const void* residual, void* out, bool out_f32,
                    hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(T));
  const bf16_t* y = static_cast<const bf16_t*>(y_perm);
  const bool pair = T <= 1024;
  if (out_f32) {
    if (pair) combine_kernel<true, true><<<grid, 256, 0, s>>>(y, inv_pos, w, k, d, max_rows, residual, out);
    else combine_kernel<true, false><<<grid, 256, 0, s>>>(y, inv_pos, w, k, d, max_rows, residual, out);
  } else {
    if (pair) combine_kernel<false, true><<<grid, 256, 0, s>>>(y, inv_pos, w, k, d, max_rows, residual, out);
    else combine_kernel<false, false><<<grid, 256, 0, s>>>(y, inv_pos, w, k, d, max_rows, residual, out);
  }
}

}  // namespace mf
