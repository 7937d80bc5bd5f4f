// Per-token fp8 activation quantisation for the block-fp8 prefill variant
// ("「赤兔」Chitu 框架深度解读（七）：MoE", 专家计算实现: prefill experts run as FP8
// GEMMs; 量化支持: block fp8). Each row is cut into groups of 128 consecutive
// channels; a group's scale is s = max(amax, 1e-4) / 448 and each element's
// code is the E4M3FN value nearest to x / s (ties to even), both computed in
// fp32 with IEEE division.
//
// Sixteen lanes hold one group (eight bf16 values each, one 16-byte load); a
// wave covers four groups of a row per pass. The group maximum is a DPP max
// within the 16-lane row (non-negative floats compare as unsigned integers).
// HBM-bound: 2 bytes read and 1 + 4/128 bytes written per element. An optional
// device row count bounds the rows (the grouped layout's live rows, known
// only on the device); the grid is strided over the (row, group-quad) tasks.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row_max(uint32_t v) {
  // lanes outside the source row receive 0, the identity of the unsigned max
  const uint32_t o = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
  return v > o ? v : o;
}

// code of fl32(x / s), saturated to +-448 before the conversion; HI selects
// the upper 16 bits of the result word
template <bool HI>
__device__ __forceinline__ uint32_t encode2(float a, float b, float s, uint32_t old) {
  a = fminf(fmaxf(a / s, -448.0f), 448.0f);
  b = fminf(fmaxf(b / s, -448.0f), 448.0f);
  return static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), HI));
}

}  // namespace

__global__ __launch_bounds__(256) void quantize_rows_kernel(const bf16_t* __restrict__ x,
                                                            int64_t rows,
                                                            const int32_t* __restrict__ row_count,
                                                            int K, uint8_t* __restrict__ q,
                                                            float* __restrict__ scales) {
  const int lane = threadIdx.x % kWave;
  const int ngroups = K / 128;
  const int quads = (ngroups + 3) / 4;
  int64_t live = rows;  // rows past *row_count (when given) are left alone
  if (row_count != nullptr) live = min(max(static_cast<int64_t>(*row_count), int64_t(0)), rows);
  const int64_t tasks = live * quads;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t task = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave; task < tasks;
       task += stride) {
    const int64_t r = task / quads;
    const int g = static_cast<int>(task - r * quads) * 4 + lane / 16;
    if (g >= ngroups) continue;  // whole 16-lane rows skip together
    const int64_t e0 = r * K + static_cast<int64_t>(g) * 128 + (lane % 16) * 8;
    const u32x4 v = ld16(x + e0);
    float f[8];
    unpack_bf16x8(v, f);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    uint32_t mb = __float_as_uint(m);
    mb = dpp_row_max<0xB1>(mb);   // quad_perm [1,0,3,2]
    mb = dpp_row_max<0x4E>(mb);   // quad_perm [2,3,0,1]
    mb = dpp_row_max<0x141>(mb);  // row_half_mirror
    mb = dpp_row_max<0x140>(mb);  // row_mirror: every lane of the row has its max
    const float s = fmaxf(__uint_as_float(mb), 1e-4f) / 448.0f;
    u32x2 out;
    out[0] = encode2<false>(f[0], f[1], s, 0u);
    out[0] = encode2<true>(f[2], f[3], s, out[0]);
    out[1] = encode2<false>(f[4], f[5], s, 0u);
    out[1] = encode2<true>(f[6], f[7], s, out[1]);
    *reinterpret_cast<u32x2*>(q + e0) = out;
    if (lane % 16 == 0) scales[r * ngroups + g] = s;
  }
}

void launch_quantize_rows(const void* x, int64_t rows, const int32_t* row_count, int K, void* q,
                          float* scales, hipStream_t s) {
  const int64_t quads = (K / 128 + 3) / 4;
  const int64_t tasks = rows * quads;
  if (tasks == 0) return;
  int64_t blocks = (tasks + 3) / 4;  // four waves (tasks) per workgroup
  if (blocks > 8192) blocks = 8192;  // grid-strided beyond
  quantize_rows_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(
      static_cast<const bf16_t*>(x), rows, row_count, K, static_cast<uint8_t*>(q), scales);
}

}  // namespace mf
