// Grouped bf16 GEMMs of the expert MLPs on MFMA ("推理计算流梳理", EP 路径: one
// rank runs its experts as a grouped GEMM; 实际 MLP 计算策略: the gated MLP).
//
//   gate/up:  H[rows of e] = SiLU(A W_gate_e^T) * (A W_up_e^T)   (fused epilogue)
//   down:     Y[rows of e] = H W_down_e^T                         (bf16 or f32 out)
//
// A is [rows, K] and every weight is [N, K] (K-contiguous), so both operands
// stream K-contiguous 16-byte chunks: C = A B^T.
//
// Tiling. A workgroup (256 threads, 4 waves in 2x2) computes a 128-row tile.
// Its B tile is 256 weight rows: 128 gate + 128 up rows (128 output columns,
// gate and up side by side so the SiLU product is local) or 256 down rows
// (256 output columns). Each wave owns 64 rows x 8 sixteen-wide B sub-tiles:
// 32 v_mfma_f32_16x16x32_bf16 accumulators (128 fp32 per lane). The weight
// fragment is the MFMA's first operand, so each lane ends up holding four
// consecutive output columns of one row (8- or 16-byte stores).
//
// K loop: BK = 64 per stage, two LDS stages (48 KB each) with a 16-byte-chunk
// XOR swizzle (chunk ^ row%8) that keeps both the coalesced row writes and the
// MFMA fragment reads free of bank conflicts. The next stage's global loads
// are in flight while the current stage feeds the MFMAs.
//
// Schedule. Group boundaries come from the device-side offsets, so no host
// sync is needed: each workgroup turns offsets into per-group m-tile counts
// and their prefix sum in LDS. Tiles are numbered group-major, then n-tile,
// then m-tile, so the m-tiles that share one weight tile are consecutive.
// The grid is persistent; workgroup b (dispatched round-robin to XCD b % 8)
// takes tile it*G + (b%8)*(G/8) + b/8 in round it, so each XCD works on a
// contiguous run of tiles and weight tiles are reused from its own L2.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int BM = 128;
constexpr int BK = 64;
constexpr int BROWS = 256;
constexpr int A_BYTES = BM * BK * 2;
constexpr int B_BYTES = BROWS * BK * 2;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int MAX_GROUPS = 256;

struct GemmParams {
  const char* a;           // [max_rows, K] bf16
  const char* b0;          // [groups, N, K] bf16 (gate, or down)
  const char* b1;          // [groups, N, K] bf16 (up; gated only)
  char* c;                 // [max_rows, N] bf16 or f32
  const int32_t* offsets;  // [groups+1] or nullptr (one group of max_rows rows)
  int e_count;
  int max_rows;
  int K, N;
};

__device__ __forceinline__ int swz(int r, int chunk) { return r * (BK * 2) + ((chunk ^ (r & 7)) << 4); }

}  // namespace

template <bool GATED, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmParams p) {
  constexpr int BN_OUT = GATED ? 128 : 256;
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE_BYTES];
  __shared__ int s_tile0[MAX_GROUPS + 1];
  __shared__ int s_beg[MAX_GROUPS];
  __shared__ int s_end[MAX_GROUPS];

  const int tid = threadIdx.x;
  const int NT = p.N / BN_OUT;

  // ---- device-side schedule ---------------------------------------------
  int mt = 0;
  if (tid < p.e_count) {
    int beg = 0, end = p.max_rows;
    if (p.offsets != nullptr) {
      beg = clampi(p.offsets[tid], 0, p.max_rows);
      end = clampi(p.offsets[tid + 1], beg, p.max_rows);
    }
    s_beg[tid] = beg;
    s_end[tid] = end;
    mt = (end - beg + BM - 1) / BM;
  }
  s_tile0[tid + 1] = mt;  // inclusive scan below, shifted by one
  if (tid == 0) s_tile0[0] = 0;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? s_tile0[tid + 1 - off] : 0;
    __syncthreads();
    s_tile0[tid + 1] += v;
    __syncthreads();
  }
  const int total_tiles = s_tile0[p.e_count] * NT;

  const int wave = tid / kWave, lane = tid % kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lg = lane >> 4;
  const int ld_c = tid & 7;    // 16-byte chunk this thread moves
  const int ld_r = tid >> 3;   // first row this thread moves (then +32, +64, ...)
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nk = p.K / BK;
  const int64_t Kb = static_cast<int64_t>(p.K) * 2;

  for (int it = 0;; it += G) {
    const int L = it + xcd * (G >> 3) + slot;
    if (L >= total_tiles) break;

    // group e: the last with s_tile0[e] * NT <= L
    int lo = 0, hi = p.e_count - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tile0[mid] * NT <= L) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int mt_e = s_tile0[e + 1] - s_tile0[e];
    const int rem = L - s_tile0[e] * NT;
    const int ni = rem / mt_e, mi = rem - ni * mt_e;
    const int row0 = s_beg[e] + mi * BM;
    const int rows_valid = min(BM, s_end[e] - row0);
    const int n0 = ni * BN_OUT;

    // ---- per-thread global pointers ---------------------------------------
    const char* ap[4];
    bool av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ld_r + 32 * i;
      av[i] = r < rows_valid;
      ap[i] = p.a + static_cast<int64_t>(row0 + (av[i] ? r : 0)) * Kb + ld_c * 16;
    }
    const char* bp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = ld_r + 32 * i;
      if (GATED) {
        const char* base = i < 4 ? p.b0 : p.b1;
        const int rr = i < 4 ? r : r - 128;
        bp[i] = base + (static_cast<int64_t>(e) * p.N + n0 + rr) * Kb + ld_c * 16;
      } else {
        bp[i] = p.b0 + (static_cast<int64_t>(e) * p.N + n0 + r) * Kb + ld_c * 16;
      }
    }

    u32x4 ra[4], rb[8];
    auto gload = [&](int k0) {
      const int64_t kb = static_cast<int64_t>(k0) * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = av[i] ? ld16(ap[i] + kb) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) rb[i] = ld16(bp[i] + kb);
    };
    auto sstore = [&](int stage) {
      char* A = lds + stage * STAGE_BYTES;
      char* B = A + A_BYTES;
#pragma unroll
      for (int i = 0; i < 4; ++i) st16(A + swz(ld_r + 32 * i, ld_c), ra[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) st16(B + swz(ld_r + 32 * i, ld_c), rb[i]);
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int stage) {
      const char* A = lds + stage * STAGE_BYTES;
      const char* B = A + A_BYTES;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int chunk = kc * 4 + lg;
        u32x4 af[4], bf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = ld16(A + swz(wm * 64 + i * 16 + lr, chunk));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int br = GATED ? (j < 4 ? wn * 64 + j * 16 : 128 + wn * 64 + (j - 4) * 16)
                               : wn * 128 + j * 16;
          bf[j] = ld16(B + swz(br + lr, chunk));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = mfma16x16x32(bf[j], af[i], acc[i][j]);
      }
    };

    __syncthreads();  // the previous tile's LDS reads are done
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) gload((kt + 1) * BK);
      compute(kt & 1);
      if (kt + 1 < nk) sstore((kt + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue: lane holds columns 4*lg..4*lg+3 of row lr per sub-tile --
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 64 + i * 16 + lr;
      if (m >= rows_valid) continue;
      const int64_t grow = row0 + m;
      if constexpr (GATED) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn * 64 + j * 16 + 4 * lg;
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = siluf_(acc[i][j][r]) * acc[i][j + 4][r];
          *reinterpret_cast<u32x2*>(p.c + (grow * p.N + col) * 2) =
              u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = n0 + wn * 128 + j * 16 + 4 * lg;
          if constexpr (OUT_F32) {
            st16(p.c + (grow * p.N + col) * 4,
                 u32x4{__float_as_uint(acc[i][j][0]), __float_as_uint(acc[i][j][1]),
                       __float_as_uint(acc[i][j][2]), __float_as_uint(acc[i][j][3])});
          } else {
            *reinterpret_cast<u32x2*>(p.c + (grow * p.N + col) * 2) =
                u32x2{pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                      pack_bf16x2(acc[i][j][2], acc[i][j][3])};
          }
        }
      }
    }
  }
}

namespace {

int persistent_grid(int64_t max_rows, int e_count, int nt, int num_cus) {
  const int64_t ub = ((max_rows + BM - 1) / BM + e_count) * static_cast<int64_t>(nt);
  int64_t g = ub < num_cus ? ub : num_cus;
  g = (g + 7) & ~int64_t(7);
  return static_cast<int>(g < 8 ? 8 : g);
}

}  // namespace

void launch_gemm_gateup_bf16(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                             int K, int N, const void* w_gate, const void* w_up, void* h,
                             int num_cus, hipStream_t s) {
  GemmParams p{static_cast<const char*>(a), static_cast<const char*>(w_gate),
               static_cast<const char*>(w_up), static_cast<char*>(h), offsets, e_count,
               static_cast<int>(max_rows), K, N};
  const int grid = persistent_grid(max_rows, e_count, N / 128, num_cus);
  gemm_bf16_kernel<true, false><<<grid, 256, 0, s>>>(p);
}

void launch_gemm_down_bf16(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                           int K, int N, const void* w_down, void* y, bool out_f32, int num_cus,
                           hipStream_t s) {
  GemmParams p{static_cast<const char*>(a), static_cast<const char*>(w_down), nullptr,
               static_cast<char*>(y), offsets, e_count, static_cast<int>(max_rows), K, N};
  const int grid = persistent_grid(max_rows, e_count, N / 256, num_cus);
  if (out_f32)
    gemm_bf16_kernel<false, true><<<grid, 256, 0, s>>>(p);
  else
    gemm_bf16_kernel<false, false><<<grid, 256, 0, s>>>(p);
}

}  // namespace mf
