// Device helpers shared by the gfx950 kernels: vector types, bf16/fp8
// conversions, MFMA wrappers, wave reductions and launch-time constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mf {

typedef uint16_t bf16_t;  // bf16 storage (bit pattern)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

// ---- conversions --------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, h);
}

// Two fp32 -> packed bf16x2 (low half = a), round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Unpack 8 bf16 held in a 16-byte vector into fp32.
__device__ __forceinline__ void unpack_bf16x8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float* f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return r;
}

// Four E4M3FN codes (one dword) -> four bf16 (two dwords), exactly: every
// E4M3FN value, subnormals included, is representable in bf16. Uses the
// gfx950 conversion with a unit scale.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t q) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, true);
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// ---- MFMA ---------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16].
// Lane l supplies A[l%16][8*(l/16)+v] and B[8*(l/16)+v][l%16] (v = 0..7) and
// holds D[4*(l/16)+r][l%16] (r = 0..3).

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- wave reductions ----------------------------------------------------

// Wave-wide sum, uniform result. DPP lane moves (register speed): two quad
// permutations and the two mirrors give every lane its 16-lane row's sum;
// row_bcast15 adds row 0 into row 1 and row 2 into row 3, row_bcast31 adds
// lane 31 into rows 2 and 3, so lane 63 ends with the sum of all 64 lanes.
// Rows outside a step's row mask receive 0 (the DPP "old" value). The order
// of the additions is fixed, so the result is deterministic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF,
                                                    false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_f32<0x140, 0xF>(v);  // row_mirror
  v += dpp_f32<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  v += dpp_f32<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ---- math ----------------------------------------------------------------

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float siluf_(float a) { return a / (1.0f + expf(-a)); }

// ---- global memory -------------------------------------------------------

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// 16 bytes of data that is read once (weights streamed through a kernel):
// a non-temporal load. On this chip 16-byte streaming reads of a 4 GiB buffer
// reach 7.1-7.3 TB/s with the non-temporal policy against 6.0-6.2 TB/s with
// the default one (one to four workgroups per CU, 8 or 16 loads in flight).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Buffer resource over [p, p + 2^31) for raw buffer loads: p must be the same
// for every lane of the wave (it is read from the first lane), offsets are
// bytes from p.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* p) {
  const uint64_t u = static_cast<uint64_t>(reinterpret_cast<uintptr_t>(p));
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  // 0x00020000: 32-bit data format, as raw buffer loads of dwords need
  return __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), 0x7fffffff, 0x00020000);
}

// 16 bytes at byte offset off of the buffer (default cache policy)
__device__ __forceinline__ u32x4 ld16_buf(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

}  // namespace mf
