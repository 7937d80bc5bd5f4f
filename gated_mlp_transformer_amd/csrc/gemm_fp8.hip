// Grouped GEMMs with block-scaled fp8 (E4M3FN) expert weights and bf16
// activations ("「赤兔」Chitu 框架深度解读（七）：MoE", quantisation support:
// block fp8 experts; "推理计算流梳理", EP 路径 and 实际 MLP 计算策略).
//
//   gate/up:  H[rows of e] = SiLU(A Wg_e^T) * (A Wu_e^T)
//   down:     Y[rows of e] = H Wd_e^T
// with W[n, k] = code[n, k] * scale[n/128, k/128].
//
// Shaped for decode, where an expert holds a handful of rows and the kernel
// streams weights from HBM once: one workgroup per (expert, 256 output
// columns), each wave 64 columns as four 16-row weight sub-tiles (eight for
// gate + up). The weight sub-tile is the MFMA's first operand; the expert's
// rows (up to 16 per pass, zero-padded) are the second. Every lane loads 32
// weight bytes of a 128-deep slab per sub-tile (row l%16, bytes 32(l/16) +
// 0..31), from weights packed so that each of its two 16-byte loads is one
// contiguous 1 KB across the wave; the contraction index is permuted
// identically on both operands (lane group g, MFMA c, element v <-> k =
// 32g + 8c + v), which leaves the dot products unchanged. Codes are converted
// to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 with a unit scale), each slab is
// accumulated on MFMA in fp32 from zero, and
// the slab sum is scaled by its block's fp32 scale into the running fp32 sum.
// The next slab's loads are issued before the current slab is consumed.
// Experts with more than 16 rows are processed 16 rows at a time (the weights
// are re-read per pass; decode shapes need one pass).
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int NTW = 256;  // output columns per workgroup
constexpr int SLAB = 128; // K depth per scale block

struct Fp8Params {
  const char* a;           // [max_rows, K] bf16
  const uint8_t* b0;       // packed fp8 weights (gate, or down), see pack.hip
  const uint8_t* b1;       // packed fp8 weights (up; gated only)
  const float* s0;         // [groups, N/128, K/128]
  const float* s1;
  char* c;                 // [max_rows, N] bf16
  const int32_t* offsets;  // [groups+1]
  int e_count;
  int max_rows;
  int K, N;
};

template <int R>
struct SlabRegs {
  u32x4 b[R][2];
  u32x4 a[4];
};

}  // namespace

template <bool GATED>
__global__ __launch_bounds__(256) void gemm_fp8_kernel(Fp8Params p) {
  constexpr int R = GATED ? 8 : 4;  // 16-row weight sub-tiles per wave
  const int ntw = p.N / NTW;
  const int e = blockIdx.x / ntw;
  const int nt = blockIdx.x - e * ntw;
  const int beg = clampi(p.offsets[e], 0, p.max_rows);
  const int end = clampi(p.offsets[e + 1], beg, p.max_rows);
  if (end <= beg) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0w = nt * NTW + wave * 64;
  const int kslabs = p.K / SLAB;
  const int64_t K = p.K;

  // Packed fp8 weights: 16-row x 128-column blocks of 2 KB, [half][lane][16 B];
  // lane l's two 16-byte loads of a block are row l%16, bytes 32(l/16) + 0..31
  // of the block's 128-byte slab, each load one contiguous 1 KB across lanes.
  const int kblocks = p.K / SLAB;
  const uint8_t* wp[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const uint8_t* base = (GATED && q >= 4) ? p.b1 : p.b0;
    const int nb = (n0w >> 4) + (q & 3);
    wp[q] = base + ((static_cast<int64_t>(e) * (p.N / 16) + nb) * kblocks) * 2048 +
            lane * 16;
  }
  const int64_t sbase = (static_cast<int64_t>(e) * (p.N / SLAB) + n0w / SLAB) * kslabs;
  const float* sp0 = p.s0 + sbase;
  const float* sp1 = GATED ? p.s1 + sbase : nullptr;

  for (int m0 = beg; m0 < end; m0 += 16) {
    const int rows_valid = min(16, end - m0);
    const bool arow_ok = lr < rows_valid;
    const char* ap = p.a + static_cast<int64_t>(m0 + (arow_ok ? lr : 0)) * K * 2 + 64 * lg;

    f32x4 acc[R];
#pragma unroll
    for (int q = 0; q < R; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    SlabRegs<R> cur, nxt;
    auto load = [&](SlabRegs<R>& s, int kb) {
      const int64_t kofs = static_cast<int64_t>(kb) * SLAB;
      const int64_t bofs = static_cast<int64_t>(kb) * 2048;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        s.b[q][0] = ld16(wp[q] + bofs);
        s.b[q][1] = ld16(wp[q] + bofs + 1024);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        s.a[c] = arow_ok ? ld16(ap + kofs * 2 + 16 * c) : u32x4{0u, 0u, 0u, 0u};
    };

    load(cur, 0);
    for (int kb = 0; kb < kslabs; ++kb) {
      if (kb + 1 < kslabs) load(nxt, kb + 1);
      const float sc0 = sp0[kb];
      const float sc1 = GATED ? sp1[kb] : 0.f;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4& w = cur.b[q][c >> 1];
          const u32x2 lo = fp8x4_to_bf16x4(w[(c & 1) * 2]);
          const u32x2 hi = fp8x4_to_bf16x4(w[(c & 1) * 2 + 1]);
          sa = mfma16x16x32(u32x4{lo[0], lo[1], hi[0], hi[1]}, cur.a[c], sa);
        }
        const float sc = (GATED && q >= 4) ? sc1 : sc0;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[q][r] = fmaf(sc, sa[r], acc[q][r]);
      }
      cur = nxt;
    }

    // lane holds output columns 4*lg..4*lg+3 of sub-tile q for row lr.
    if (arow_ok) {
      const int64_t grow = m0 + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0w + 16 * q + 4 * lg;
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          h[r] = GATED ? siluf_(acc[q][r]) * acc[q + (GATED ? 4 : 0)][r] : acc[q][r];
        *reinterpret_cast<u32x2*>(p.c + (grow * p.N + col) * 2) =
            u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
      }
    }
  }
}

void launch_gemm_gateup_fp8(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                            int K, int N, const void* w_gate, const void* w_up,
                            const float* s_gate, const float* s_up, void* h, hipStream_t s) {
  Fp8Params p{static_cast<const char*>(a), static_cast<const uint8_t*>(w_gate),
              static_cast<const uint8_t*>(w_up), s_gate, s_up, static_cast<char*>(h), offsets,
              e_count, static_cast<int>(max_rows), K, N};
  gemm_fp8_kernel<true><<<dim3(static_cast<unsigned>(e_count * (N / NTW))), 256, 0, s>>>(p);
}

void launch_gemm_down_fp8(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                          int K, int N, const void* w_down, const float* s_down, void* y,
                          hipStream_t s) {
  Fp8Params p{static_cast<const char*>(a), static_cast<const uint8_t*>(w_down), nullptr, s_down,
              nullptr, static_cast<char*>(y), offsets, e_count, static_cast<int>(max_rows), K, N};
  gemm_fp8_kernel<false><<<dim3(static_cast<unsigned>(e_count * (N / NTW))), 256, 0, s>>>(p);
}

}  // namespace mf
