// Grouped GEMMs with block-scaled fp8 (E4M3FN) expert weights and bf16
// activations ("「赤兔」Chitu 框架深度解读（七）：MoE", quantisation support:
// block fp8 experts; "推理计算流梳理", EP 路径 and 实际 MLP 计算策略).
//
//   gate/up:  H[rows of e] = SiLU(A Wg_e^T) * (A Wu_e^T)
//   down:     Y[rows of e] = H Wd_e^T
// with W[n, k] = code[n, k] * scale[n/128, k/128].
//
// Shaped for decode, where an expert holds a handful of rows and the kernel
// streams weights from HBM once. A work item is one expert against NTW output
// columns (256 for gate/up, 512 for down); each wave owns a quarter of them as
// eight 16-row weight sub-tiles (four gate + four up, or eight down), so that
// a wave's weight loads per 128-deep slab (16 KB) dwarf its A loads (4 KB). The weight sub-tile is the MFMA's first operand; the expert's
// rows (up to 16 per pass, zero-padded) are the second. Every lane loads 32
// weight bytes of a 128-deep slab per sub-tile (row l%16, bytes 32(l/16) +
// 0..31), from weights packed so that each of its two 16-byte loads is one
// contiguous 1 KB across the wave; the contraction index is permuted
// identically on both operands (lane group g, MFMA c, element v <-> k =
// 32g + 8c + v), which leaves the dot products unchanged. Codes are converted
// to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 with a unit scale), each slab is
// accumulated on MFMA in fp32 from zero, and
// the slab sum is scaled by its block's fp32 scale into the running fp32 sum.
// The next slab's loads are issued before the current slab is consumed; the
// block scales of a pass are loaded once, one slab per lane, so that inside
// the slab loop the only memory accesses are the weight and A loads and the
// in-order load counter waits for exactly the slab being consumed.
// Experts with more than 16 rows are processed 16 rows at a time (the weights
// are re-read per pass; decode shapes need one pass).
//
// Schedule. Items of experts without rows do not exist. An expert's rows are
// [offsets[e], offsets[e+1]) of the contiguous layout, or in the masked
// layout the first counts[e] rows of its fixed block [e*cap, (e+1)*cap). The grid is persistent
// (one workgroup per CU) and workgroup b takes items b, b + G, b + 2G, ...:
// with equal items, a few hundred of them over G workgroups leave the last
// round nearly full, where one workgroup per item would leave a partial
// round of whole workgroups idle. Each workgroup derives the item list from
// the device-side offsets (an LDS prefix sum over experts), so no host sync is
// needed.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int R = 8;      // 16-row weight sub-tiles per wave
constexpr int SLAB = 128; // K depth per scale block
constexpr int MAX_GROUPS = 256;

struct Fp8Params {
  const char* a;           // [max_rows, K] bf16, or [a_src_rows, K] when a_rows is set
  const int32_t* a_rows;   // nullptr, or [max_rows]: row r of A is row a_rows[r] of `a`
  int a_src_rows;          // (clamped to [0, a_src_rows))
  const uint8_t* b0;       // packed fp8 weights (gate, or down), see pack.hip
  const uint8_t* b1;       // packed fp8 weights (up; gated only)
  const float* s0;         // [groups, N/128, K/128]
  const float* s1;
  char* c;                 // [max_rows, N] bf16
  const int32_t* offsets;  // [groups+1]
  int e_count;
  int max_rows;
  int K, N;
  const int32_t* counts;   // masked layout (offsets unused): expert e owns rows
  int cap;                 // [e*cap, e*cap + min(counts[e], cap)); nullptr: offsets
};

template <int R>
struct SlabRegs {
  u32x4 b[R][2];
  u32x4 a[4];
};

}  // namespace

template <bool GATED, bool ODD>
__global__ __launch_bounds__(256) void gemm_fp8_kernel(Fp8Params p) {
  constexpr int NTW = GATED ? 256 : 512;  // output columns per work item
  constexpr int QH = GATED ? R / 2 : R;   // sub-tiles per weight matrix per wave
  __shared__ int s_item0[MAX_GROUPS + 1];
  __shared__ int s_beg[MAX_GROUPS];
  __shared__ int s_end[MAX_GROUPS];
  const int tid = threadIdx.x;
  const int ntw = (p.N + NTW - 1) / NTW;  // items per active expert (the last may be partial)

  // ---- device-side item list: prefix over experts of ntw items per active expert
  int items = 0;
  if (tid < p.e_count) {
    int beg, end;
    if (p.counts != nullptr) {  // masked layout: fixed blocks of cap rows
      beg = clampi(tid * p.cap, 0, p.max_rows);
      end = clampi(beg + clampi(p.counts[tid], 0, p.cap), beg, p.max_rows);
    } else {
      beg = clampi(p.offsets[tid], 0, p.max_rows);
      end = clampi(p.offsets[tid + 1], beg, p.max_rows);
    }
    s_beg[tid] = beg;
    s_end[tid] = end;
    items = end > beg ? ntw : 0;
  }
  s_item0[tid + 1] = items;  // inclusive scan below, shifted by one
  if (tid == 0) s_item0[0] = 0;
  __syncthreads();
  for (int off = 1; off < p.e_count; off <<= 1) {  // entries 0 .. e_count are read
    const int v = tid >= off ? s_item0[tid + 1 - off] : 0;
    __syncthreads();
    s_item0[tid + 1] += v;
    __syncthreads();
  }
  const int total_items = s_item0[p.e_count];

  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lr = lane & 15, lg = lane >> 4;
  const int kslabs = p.K / SLAB;
  const int64_t K = p.K;

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    // expert e: the last with s_item0[e] <= item (it owns the item)
    int lo = 0, hi = p.e_count - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_item0[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int nt = item - s_item0[e];
    const int beg = s_beg[e], end = s_end[e];
    const int n0w = nt * NTW + wave * (16 * QH);
    // N is a multiple of 16 * QH, so a wave's columns are all in range or all
    // past N; a wave past N has nothing to do for this item (there is no
    // workgroup barrier inside the item loop).
    if (n0w >= p.N) continue;

    // Packed fp8 weights: 16-row x 128-column blocks of 2 KB, [half][lane][16 B],
    // slab-major ([slab][group][row block]); lane l's two 16-byte loads of a
    // block are row l%16, bytes 32(l/16) + 0..31 of the block's 128-byte slab,
    // each load one contiguous 1 KB across lanes.
    const int64_t slab_stride = static_cast<int64_t>(p.e_count) * (p.N / 16) * 2048;
    const uint8_t* wp[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const uint8_t* base = (GATED && q >= QH) ? p.b1 : p.b0;
      const int nb = (n0w >> 4) + (q % QH);
      wp[q] = base + (static_cast<int64_t>(e) * (p.N / 16) + nb) * 2048 + lane * 16;
    }
    const int64_t sbase = (static_cast<int64_t>(e) * (p.N / SLAB) + n0w / SLAB) * kslabs;
    const float* sp0 = p.s0 + sbase;
    const float* sp1 = GATED ? p.s1 + sbase : nullptr;

    for (int m0 = beg; m0 < end; m0 += 16) {
      const int rows_valid = min(16, end - m0);
      const bool arow_ok = lr < rows_valid;
      // rows past the valid ones re-read row m0: an output row depends on its
      // own A row only, and those rows are never stored
      int arow = m0 + (arow_ok ? lr : 0);
      if (p.a_rows != nullptr) arow = clampi(p.a_rows[arow], 0, p.a_src_rows - 1);
      const char* ap = p.a + static_cast<int64_t>(arow) * K * 2 + 64 * lg;

      f32x4 acc[R];
#pragma unroll
      for (int q = 0; q < R; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

      auto load = [&](SlabRegs<R>& s, int kb) {
        const int64_t kofs = static_cast<int64_t>(kb) * SLAB;
        const int64_t bofs = static_cast<int64_t>(kb) * slab_stride;
#pragma unroll
        for (int q = 0; q < R; ++q) {  // each weight byte is read once: streamed
          s.b[q][0] = ld16_stream(wp[q] + bofs);
          s.b[q][1] = ld16_stream(wp[q] + bofs + 1024);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) s.a[c] = ld16(ap + kofs * 2 + 16 * c);
      };
      // Block scales of a chunk of up to 64 slabs: lane l holds slab kc + l's,
      // read in the loop with a uniform lane index, so the slab loop issues no
      // memory access besides the weight and A loads (one in-order counter
      // covers all vector loads: a later scale load would hold every
      // prefetched slab ahead of it)
      float scl0 = 0.f, scl1 = 0.f;
      auto compute = [&](const SlabRegs<R>& cur, int j) {
        const float sc0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scl0), j));
        const float sc1 = GATED ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scl1), j))
                                : 0.f;
#pragma unroll
        for (int q = 0; q < R; ++q) {
          f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const u32x4& w = cur.b[q][c >> 1];
            const u32x2 lo2 = fp8x4_to_bf16x4(w[(c & 1) * 2]);
            const u32x2 hi2 = fp8x4_to_bf16x4(w[(c & 1) * 2 + 1]);
            sa = mfma16x16x32(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, cur.a[c], sa);
          }
          const float sc = (GATED && q >= QH) ? sc1 : sc0;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[q][r] = fmaf(sc, sa[r], acc[q][r]);
        }
      };

      // Two register sets in turn; the next slab's loads are issued before
      // the current slab is consumed. The last two slabs of a chunk are
      // peeled (with ODD, for an odd slab count, a separate kernel: the branch
      // raised the even case from 252 to 308 VGPRs, one wave per SIMD), so
      // every wait inside the loop is static.
      // (A scheduling barrier after each group of loads keeps the compiler
      // from sinking them below the MFMAs they are meant to run under.)
      SlabRegs<R> r0, r1;
      for (int kc = 0; kc < kslabs; kc += 64) {
        const int nks = min(64, kslabs - kc);
        if (lane < nks) {
          scl0 = sp0[kc + lane];
          if (GATED) scl1 = sp1[kc + lane];
        }
        load(r0, kc);
        __builtin_amdgcn_sched_barrier(0);
        int j = 0;
        for (; j + 2 < nks; j += 2) {
          load(r1, kc + j + 1);
          __builtin_amdgcn_sched_barrier(0);
          compute(r0, j);
          load(r0, kc + j + 2);
          __builtin_amdgcn_sched_barrier(0);
          compute(r1, j + 1);
        }
        if (!ODD || j + 1 < nks) {
          load(r1, kc + j + 1);
          __builtin_amdgcn_sched_barrier(0);
          compute(r0, j);
          compute(r1, j + 1);
        } else {  // an odd slab count (K % 256 == 128): one slab left
          compute(r0, j);
        }
      }

      // lane holds output columns 4*lg..4*lg+3 of sub-tile q for row lr.
      if (arow_ok) {
        const int64_t grow = m0 + lr;
#pragma unroll
        for (int q = 0; q < QH; ++q) {
          const int col = n0w + 16 * q + 4 * lg;
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            h[r] = GATED ? siluf_(acc[q][r]) * acc[q + (GATED ? QH : 0)][r] : acc[q][r];
          *reinterpret_cast<u32x2*>(p.c + (grow * p.N + col) * 2) =
              u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        }
      }
    }
  }
}

namespace {

// One persistent workgroup per CU, but no more than there can be items.
unsigned fp8_grid(int e_count, int N, int ntw, int num_cus) {
  const int64_t ub = static_cast<int64_t>(e_count) * ((N + ntw - 1) / ntw);
  const int64_t g = ub < num_cus ? ub : num_cus;
  return static_cast<unsigned>(g < 1 ? 1 : g);
}

}  // namespace

void launch_gemm_gateup_fp8(const void* a, const int32_t* a_rows, int64_t a_src_rows,
                            const int32_t* offsets, int e_count, int64_t max_rows, int K, int N,
                            const void* w_gate, const void* w_up, const float* s_gate,
                            const float* s_up, void* h, int num_cus, hipStream_t s,
                            const int32_t* counts, int cap) {
  Fp8Params p{static_cast<const char*>(a), a_rows, static_cast<int>(a_src_rows),
              static_cast<const uint8_t*>(w_gate),
              static_cast<const uint8_t*>(w_up), s_gate, s_up, static_cast<char*>(h), offsets,
              e_count, static_cast<int>(max_rows), K, N, counts, cap};
  const dim3 grid(fp8_grid(e_count, N, 256, num_cus));
  if ((K / SLAB) % 2) gemm_fp8_kernel<true, true><<<grid, 256, 0, s>>>(p);
  else gemm_fp8_kernel<true, false><<<grid, 256, 0, s>>>(p);
}

void launch_gemm_down_fp8(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                          int K, int N, const void* w_down, const float* s_down, void* y,
                          int num_cus, hipStream_t s, const int32_t* counts, int cap) {
  Fp8Params p{static_cast<const char*>(a), nullptr, 0, static_cast<const uint8_t*>(w_down), nullptr, s_down,
              nullptr, static_cast<char*>(y), offsets, e_count, static_cast<int>(max_rows), K, N,
              counts, cap};
  const dim3 grid(fp8_grid(e_count, N, 512, num_cus));
  if ((K / SLAB) % 2) gemm_fp8_kernel<false, true><<<grid, 256, 0, s>>>(p);
  else gemm_fp8_kernel<false, false><<<grid, 256, 0, s>>>(p);
}

}  // namespace mf
