// Grouped bf16 GEMMs of the expert MLPs on MFMA ("推理计算流梳理", EP 路径: one
// rank runs its experts as a grouped GEMM; 实际 MLP 计算策略: the gated MLP).
//
//   gate/up:  H[rows of e] = SiLU(A W_gate_e^T) * (A W_up_e^T)   (fused epilogue)
//   down:     Y[rows of e] = H W_down_e^T                         (bf16 or f32 out)
//
// A is [rows, K] row-major; weights arrive packed (pack.hip): every 32-row x
// 16-column fragment of v_mfma_f32_32x32x16_bf16's weight operand is one
// contiguous 1 KB block, so a wavefront loads a fragment with one fully
// coalesced 16-byte-per-lane load, straight into registers.
//
// Tiling. A workgroup (256 threads, 4 waves) computes a 128-row tile against
// 256 weight rows: 128 gate + 128 up rows (128 output columns, gate and up
// side by side so the SiLU product stays in registers) or 256 down rows
// (256 output columns). Each wave owns 64 weight rows (two 32-row fragments)
// for all 128 tile rows (four 32-row sub-tiles): eight 32x32 accumulators
// (128 fp32 per lane, kept in AGPRs, accumulated in place).
//
// Operand paths. A wave's weight fragments are private to it and come straight
// from global memory. The A tile is shared by the four waves and goes through
// LDS (two 16 KB buffers, 16-byte-chunk XOR swizzle chunk ^ row%8: the
// coalesced row writes and the 32-row fragment reads are both conflict-free).
//
// Pipeline. BK = 64 per stage (four MFMA k-steps). Weights and A are loaded
// three stages ahead; four register slots rotate through a K loop unrolled by
// four, so every slot index is a compile-time constant and the compiler's
// vmcnt waits cover exactly the stage consumed. A tail tile (an expert's last,
// with fewer than 128 rows) runs a K loop instantiated for its live 32-row
// sub-tiles only, skipping the MFMAs and LDS reads of the empty ones.
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
constexpr int A_BYTES = BM * BK * 2;
constexpr int MAX_GROUPS = 256;
constexpr int PREF = 3;        // stages of loads in flight
constexpr int SLOTS = PREF + 1;
constexpr int FRAG = 1024;     // bytes of one packed 32x16 weight fragment

typedef __attribute__((ext_vector_type(16))) float f32x16;

struct GemmParams {
  const char* a;           // [max_rows, K] bf16
  const char* b0;          // packed weights (gate, or down): [groups][nb][K/16] fragments
  const char* b1;          // packed weights (up; gated only)
  char* c;                 // [max_rows, ldc] bf16 or f32 (per K split, see c_split)
  const int32_t* offsets;  // [groups+1] or nullptr (one group of max_rows rows)
  int e_count;
  int max_rows;
  int K;                   // row length of A and of the weights (elements)
  int nb;                  // 32-row weight blocks per group (packed)
  int n_valid;             // weight rows that exist: blocks past them are clamped on
                           // load and output columns >= n_valid are not stored
  int ldc;                 // row stride of C (elements)
  int kc;                  // K range of one split: split y covers [y*kc, (y+1)*kc)
  int64_t c_split;         // elements between the C blocks of consecutive splits
};

__device__ __forceinline__ int swz(int r, int chunk) { return r * (BK * 2) + ((chunk ^ (r & 7)) << 4); }

__device__ __forceinline__ f32x16 mfma32(const u32x4& w, const u32x4& a, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                 __builtin_bit_cast(bf16x8, a), c, 0, 0, 0);
}

}  // namespace

// K loop of one tile for NM live 32-row sub-tiles (1..4). Branch-free: the
// prefetch stage index is clamped (the last steps re-load the final stage),
// so the compiler's vmcnt waits track exactly the slot being consumed.
template <int NM>
__device__ __forceinline__ void k_loop(f32x16 (&acc)[4][2], const char* const (&ap)[4],
                                       const char* const (&bp)[2], char (&lds)[2][A_BYTES],
                                       int nk, int ld_r, int ld_c, int lane) {
  u32x4 areg[SLOTS][4];
  u32x4 breg[SLOTS][8];  // [fragment column jn * 4 + k-step s]
  const int lr = lane & 31, lg = lane >> 5;
  auto issue = [&](u32x4 (&ar)[4], u32x4 (&br)[8], int kt) {
    const int64_t ka = static_cast<int64_t>(kt) * (BK * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = ld16(ap[i] + ka);
    const int64_t kb = static_cast<int64_t>(kt) * (4 * FRAG);
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int s = 0; s < 4; ++s) br[jn * 4 + s] = ld16(bp[jn] + kb + s * FRAG);
  };
  auto write_a = [&](const u32x4 (&ar)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(&lds[buf][swz(ld_r + 32 * i, ld_c)], ar[i]);
  };
  // k-step s reads A chunk 2s + lane/32 of each live sub-tile's rows; the next
  // k-step's fragments are read before this k-step's MFMAs are issued.
  auto compute = [&](const u32x4 (&br)[8], int buf) {
    u32x4 af[2][NM];
#pragma unroll
    for (int i = 0; i < NM; ++i) af[0][i] = ld16(&lds[buf][swz(i * 32 + lr, lg)]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) {
#pragma unroll
        for (int i = 0; i < NM; ++i)
          af[(s + 1) & 1][i] = ld16(&lds[buf][swz(i * 32 + lr, 2 * (s + 1) + lg)]);
      }
#pragma unroll
      for (int i = 0; i < NM; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) acc[i][jn] = mfma32(br[jn * 4 + s], af[s & 1][i], acc[i][jn]);
    }
  };

#pragma unroll
  for (int s = 0; s < PREF; ++s) issue(areg[s], breg[s], s < nk ? s : nk - 1);
  write_a(areg[0], 0);
  __syncthreads();
#define MF_GEMM_STEP(S)                                                                      \
  {                                                                                          \
    const int t_ = kt + (S);                                                                 \
    issue(areg[((S) + PREF) % SLOTS], breg[((S) + PREF) % SLOTS], min(t_ + PREF, nk - 1));    \
    compute(breg[(S)], (S) & 1);                                                             \
    write_a(areg[((S) + 1) % SLOTS], ((S) + 1) & 1);                                         \
    __syncthreads();                                                                         \
  }
  for (int kt = 0; kt < nk; kt += SLOTS) {
    MF_GEMM_STEP(0)
    MF_GEMM_STEP(1)
    MF_GEMM_STEP(2)
    MF_GEMM_STEP(3)
  }
#undef MF_GEMM_STEP
}

template <bool GATED, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmParams p) {
  constexpr int BN_OUT = GATED ? 128 : 256;
  __shared__ __attribute__((aligned(16))) char lds[2][A_BYTES];
  __shared__ int s_tile0[MAX_GROUPS + 1];
  __shared__ int s_beg[MAX_GROUPS];
  __shared__ int s_end[MAX_GROUPS];

  const int tid = threadIdx.x;
  // n-tiles per group: the packed row blocks cover the weight rows
  const int NT = (p.nb * 32 + BN_OUT - 1) / BN_OUT;

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

  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lr = lane & 31, lg = lane >> 5;
  const int ld_c = tid & 7;    // A: 16-byte chunk this thread moves
  const int ld_r = tid >> 3;   // A: first row this thread moves (then +32, +64, +96)
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nk = p.kc / BK;
  const int kblocks = p.K / 16;  // packed fragments per 32-row block
  const int64_t Kb = static_cast<int64_t>(p.K) * 2;
  const int64_t kofs_a = static_cast<int64_t>(blockIdx.y) * p.kc * 2;  // bytes into each A row
  const int64_t kofs_b = static_cast<int64_t>(blockIdx.y) * (p.kc / 16) * FRAG;
  char* const cbase = p.c + static_cast<int64_t>(blockIdx.y) * p.c_split * (OUT_F32 ? 4 : 2);

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
    // A rows past the tile's valid rows re-read row0 (row m of the result
    // depends on row m of A only, and those rows are never stored).
    const char* ap[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ld_r + 32 * i;
      ap[i] = p.a + static_cast<int64_t>(row0 + (r < rows_valid ? r : 0)) * Kb + kofs_a + ld_c * 16;
    }
    const char* bp[2];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const char* base = (GATED && jn == 1) ? p.b1 : p.b0;
      const int row = GATED ? n0 + wave * 32 : n0 + wave * 64 + jn * 32;
      const int blk = min(row >> 5, p.nb - 1);
      bp[jn] = base + ((static_cast<int64_t>(e) * p.nb + blk) * kblocks) * FRAG + kofs_b +
               lane * 16;
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) acc[i][jn] = f32x16{};

    __syncthreads();  // the previous tile's LDS reads are done
    const int nm = (rows_valid + 31) >> 5;  // live 32-row sub-tiles
    if (nm <= 1)
      k_loop<1>(acc, ap, bp, lds, nk, ld_r, ld_c, lane);
    else if (nm == 2)
      k_loop<2>(acc, ap, bp, lds, nk, ld_r, ld_c, lane);
    else if (nm == 3)
      k_loop<3>(acc, ap, bp, lds, nk, ld_r, ld_c, lane);
    else
      k_loop<4>(acc, ap, bp, lds, nk, ld_r, ld_c, lane);

    // ---- epilogue ----------------------------------------------------------
    // Lane l holds, for row lr of sub-tile i, output columns
    // 8q + 4(l/32) + 0..3 (q = 0..3) of each 32-column fragment column jn.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = i * 32 + lr;
      if (m >= rows_valid) continue;
      const int64_t grow = row0 + m;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (GATED) {
          const int col = n0 + wave * 32 + 8 * q + 4 * lg;
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = siluf_(acc[i][0][4 * q + r]) * acc[i][1][4 * q + r];
          *reinterpret_cast<u32x2*>(cbase + (grow * p.ldc + col) * 2) =
              u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        } else {
#pragma unroll
          for (int jn = 0; jn < 2; ++jn) {
            const int col = n0 + wave * 64 + jn * 32 + 8 * q + 4 * lg;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[i][jn][4 * q + r];
            if (col >= p.n_valid) continue;
            if (col + 4 > p.n_valid) {  // ragged last column group: element stores
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                if (col + r >= p.n_valid) break;
                if constexpr (OUT_F32)
                  reinterpret_cast<float*>(cbase)[grow * p.ldc + col + r] = v[r];
                else
                  reinterpret_cast<bf16_t*>(cbase)[grow * p.ldc + col + r] = f32_to_bf16(v[r]);
              }
              continue;
            }
            if constexpr (OUT_F32) {
              st16(cbase + (grow * p.ldc + col) * 4,
                   u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                         __float_as_uint(v[3])});
            } else {
              *reinterpret_cast<u32x2*>(cbase + (grow * p.ldc + col) * 2) =
                  u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
          }
        }
      }
    }
  }
}

namespace {

// Persistent grid: at most one workgroup per CU, a multiple of 8 (the XCD
// count), and no more than an upper bound on the tiles. With offsets each
// group can add one partial m-tile; a single dense group (offsets == nullptr)
// has exactly ceil(rows / BM) m-tiles.
int persistent_grid(int64_t max_rows, int e_count, bool dense, int nt, int num_cus) {
  const int64_t mtiles = (max_rows + BM - 1) / BM + (dense ? 0 : e_count);
  const int64_t ub = mtiles * static_cast<int64_t>(nt);
  int64_t g = ub < num_cus ? ub : num_cus;
  g = (g + 7) & ~int64_t(7);
  if (g > num_cus) g = num_cus & ~7;
  return static_cast<int>(g < 8 ? 8 : g);
}

}  // namespace

void launch_gemm_gateup_bf16(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                             int K, int N, const void* w_gate, const void* w_up, void* h,
                             int num_cus, hipStream_t s) {
  GemmParams p{static_cast<const char*>(a), static_cast<const char*>(w_gate),
               static_cast<const char*>(w_up), static_cast<char*>(h), offsets, e_count,
               static_cast<int>(max_rows), K, N / 32, N, N, K, 0};
  const int grid = persistent_grid(max_rows, e_count, offsets == nullptr, N / 128, num_cus);
  gemm_bf16_kernel<true, false><<<grid, 256, 0, s>>>(p);
}

void launch_gemm_down_bf16(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                           int K, int N, const void* w_down, void* y, bool out_f32, int num_cus,
                           hipStream_t s) {
  GemmParams p{static_cast<const char*>(a), static_cast<const char*>(w_down), nullptr,
               static_cast<char*>(y), offsets, e_count, static_cast<int>(max_rows), K, N / 32,
               N, N, K, 0};
  const int grid = persistent_grid(max_rows, e_count, offsets == nullptr, N / 256, num_cus);
  if (out_f32)
    gemm_bf16_kernel<false, true><<<grid, 256, 0, s>>>(p);
  else
    gemm_bf16_kernel<false, false><<<grid, 256, 0, s>>>(p);
}

void launch_gemm_nt_f32_splitk(const void* a, int64_t rows, int K, const void* b, int n_valid,
                               int splits, float* c_partials, int num_cus, hipStream_t s) {
  // One group of `rows` rows against n_valid (<= 256) packed weight rows, K
  // split in `splits` equal ranges; split y writes its fp32 partial product to
  // c_partials[y][rows][n_valid].
  GemmParams p{static_cast<const char*>(a), static_cast<const char*>(b), nullptr,
               reinterpret_cast<char*>(c_partials), nullptr, 1, static_cast<int>(rows), K,
               (n_valid + 31) / 32, n_valid, n_valid, K / splits,
               rows * static_cast<int64_t>(n_valid)};
  // splits x tiles workgroups: size x so that all of them fit in one round
  int gx = persistent_grid(rows, 1, true, 1, num_cus / splits);
  gemm_bf16_kernel<false, true><<<dim3(gx, splits), 256, 0, s>>>(p);
}

}  // namespace mf
