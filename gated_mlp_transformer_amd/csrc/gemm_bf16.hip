// Grouped bf16 GEMMs of the expert MLPs on MFMA ("推理计算流梳理", EP 路径: one
// rank runs its experts as a grouped GEMM; 实际 MLP 计算策略: the gated MLP).
//
//   gate/up:  H[rows of e] = SiLU(A W_gate_e^T) * (A W_up_e^T)   (fused epilogue)
//   down:     Y[rows of e] = H W_down_e^T                         (bf16 or f32 out)
//
// A is [rows, K] and every weight is [N, K] (K-contiguous): C = A B^T.
//
// Tiling. A workgroup (256 threads, 4 waves) computes a 128-row tile against
// 256 weight rows: 128 gate + 128 up rows (128 output columns, gate and up
// side by side so the SiLU product stays in registers) or 256 down rows
// (256 output columns). The four waves split the weight rows: each wave owns
// 64 of them (four 16-row sub-tiles) for all 128 tile rows (eight 16-row
// sub-tiles), i.e. 32 v_mfma_f32_16x16x32_bf16 accumulators (128 fp32/lane).
//
// Operand paths. A wave's weight rows are private to it, and a K-contiguous
// row already has the MFMA fragment layout (lane l: row l%16, 8 consecutive k
// at 8*(l/16)), so weights stream from global memory straight into fragment
// registers with 16-byte loads and never touch LDS. The A tile is shared by
// the four waves and goes through LDS (two 16 KB buffers, 16-byte-chunk XOR
// swizzle chunk ^ row%8: conflict-free row writes and fragment reads).
//
// Pipeline. BK = 64 per stage. Weight fragments are loaded three stages
// ahead and A two stages ahead of its LDS write; four register slots rotate
// through a K loop unrolled by four, so every slot index is a compile-time
// constant and the compiler's vmcnt waits cover exactly the stage consumed. A tail tile (an expert's last, with
// fewer than 128 rows) runs a K loop instantiated for its live 32-row pairs of
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

struct GemmParams {
  const char* a;           // [max_rows, K] bf16
  const char* b0;          // [groups, N, K] bf16 (gate, or down)
  const char* b1;          // [groups, N, K] bf16 (up; gated only)
  char* c;                 // [max_rows, ldc] bf16 or f32 (per K split, see c_split)
  const int32_t* offsets;  // [groups+1] or nullptr (one group of max_rows rows)
  int e_count;
  int max_rows;
  int K;                   // row length of A and B (elements)
  int N;                   // weight rows per group, a multiple of the tile width
  int n_valid;             // weight rows that exist: rows >= n_valid are clamped on load
                           // and their output columns are not stored
  int ldc;                 // row stride of C (elements)
  int kc;                  // K range of one split: split y covers [y*kc, (y+1)*kc)
  int64_t c_split;         // elements between the C blocks of consecutive splits
};

__device__ __forceinline__ int swz(int r, int chunk) { return r * (BK * 2) + ((chunk ^ (r & 7)) << 4); }

}  // namespace

// The K loop of one tile for NM live 16-row sub-tiles (NM even, 2..8). It is
// branch-free: the prefetch stage index is clamped (the last steps re-load
// the final stage instead of skipping), so the compiler's vmcnt waits track
// exactly the slot being consumed.
template <int NM>
__device__ __forceinline__ void k_loop(f32x4 (&acc)[8][4], const char* const (&ap)[4],
                                       const char* const (&bp)[4], char (&lds)[2][A_BYTES],
                                       int nk, int ld_r, int ld_c, int lr, int lg) {
  u32x4 areg[SLOTS][4];
  u32x4 breg[SLOTS][8];
  auto issue_a = [&](u32x4 (&ar)[4], int kt) {
    const int64_t kb = static_cast<int64_t>(kt) * (BK * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = ld16(ap[i] + kb);
  };
  auto issue_b = [&](u32x4 (&br)[8], int kt) {
    const int64_t kb = static_cast<int64_t>(kt) * (BK * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      br[2 * j] = ld16(bp[j] + kb);
      br[2 * j + 1] = ld16(bp[j] + kb + 64);
    }
  };
  auto write_a = [&](const u32x4 (&ar)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(&lds[buf][swz(ld_r + 32 * i, ld_c)], ar[i]);
  };
  // The MFMAs of one stage walk the (k-chunk c, sub-tile i) fragments in
  // order; LDS reads run one pair of fragments ahead of the MFMAs that use
  // them, and scheduling barriers keep the compiler from sinking the reads
  // next to their uses (with one wave per SIMD nothing else would hide the
  // LDS latency).
  auto compute = [&](const u32x4 (&br)[8], int buf) {
    constexpr int NF = 2 * NM;  // fragments per stage: (c, i) = (f / NM, f % NM)
    auto frag = [&](int f) {
      return ld16(&lds[buf][swz((f % NM) * 16 + lr, (f / NM) * 4 + lg)]);
    };
    u32x4 af[4];
    af[0] = frag(0);
    af[1] = frag(1);
#pragma unroll
    for (int f = 0; f < NF; f += 2) {
      if (f + 2 < NF) {
        af[(f + 2) & 3] = frag(f + 2);
        af[(f + 3) & 3] = frag(f + 3);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int i = (f + q) % NM, c = (f + q) / NM;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(br[2 * j + c], af[(f + q) & 3], acc[i][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Stage t lives in slot t % 4. B runs three stages ahead (issued right
  // after the MFMAs free its slot), A two stages ahead of its LDS write.
#pragma unroll
  for (int s = 0; s < PREF; ++s) issue_b(breg[s], s < nk ? s : nk - 1);
  issue_a(areg[0], 0);
  issue_a(areg[1], 1 < nk ? 1 : nk - 1);
  write_a(areg[0], 0);
  __syncthreads();
#define MF_GEMM_STEP(S)                                                                      \
  {                                                                                          \
    const int t_ = kt + (S);                                                                 \
    issue_a(areg[((S) + 2) % SLOTS], min(t_ + 2, nk - 1));                                   \
    compute(breg[(S)], (S) & 1);                                                             \
    issue_b(breg[((S) + PREF) % SLOTS], min(t_ + PREF, nk - 1));                             \
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

  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lr = lane & 15, lg = lane >> 4;
  const int ld_c = tid & 7;    // A: 16-byte chunk this thread moves
  const int ld_r = tid >> 3;   // A: first row this thread moves (then +32, +64, +96)
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nk = p.kc / BK;
  const int64_t Kb = static_cast<int64_t>(p.K) * 2;
  const int64_t kofs = static_cast<int64_t>(blockIdx.y) * p.kc * 2;  // bytes into each row
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
    // A rows past the tile's valid rows re-read row0 (any in-range row would
    // do: row m of the result depends on row m of A only, and those rows are
    // never stored).
    const char* ap[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ld_r + 32 * i;
      ap[i] = p.a + static_cast<int64_t>(row0 + (r < rows_valid ? r : 0)) * Kb + kofs + ld_c * 16;
    }
    const char* bp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int row;
      const char* base;
      if (GATED) {
        base = j < 2 ? p.b0 : p.b1;
        row = n0 + wave * 32 + (j & 1) * 16 + lr;
      } else {
        base = p.b0;
        row = n0 + wave * 64 + j * 16 + lr;
      }
      row = row < p.n_valid ? row : p.n_valid - 1;
      bp[j] = base + (static_cast<int64_t>(e) * p.N + row) * Kb + kofs + lg * 16;
    }

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // the previous tile's LDS reads are done
    // live 16-row sub-tiles, rounded up to a pair
    const int nm = ((rows_valid + 31) >> 5) << 1;
    if (nm <= 2)
      k_loop<2>(acc, ap, bp, lds, nk, ld_r, ld_c, lr, lg);
    else if (nm <= 4)
      k_loop<4>(acc, ap, bp, lds, nk, ld_r, ld_c, lr, lg);
    else if (nm <= 6)
      k_loop<6>(acc, ap, bp, lds, nk, ld_r, ld_c, lr, lg);
    else
      k_loop<8>(acc, ap, bp, lds, nk, ld_r, ld_c, lr, lg);

    // ---- epilogue: lane holds columns 4*lg..4*lg+3 of row lr per sub-tile --
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = i * 16 + lr;
      if (m >= rows_valid) continue;
      const int64_t grow = row0 + m;
      if constexpr (GATED) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wave * 32 + j * 16 + 4 * lg;
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = siluf_(acc[i][j][r]) * acc[i][j + 2][r];
          *reinterpret_cast<u32x2*>(cbase + (grow * p.ldc + col) * 2) =
              u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wave * 64 + j * 16 + 4 * lg;
          if (col >= p.n_valid) continue;
          if (col + 4 > p.n_valid) {  // ragged last column group: element stores
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (col + r >= p.n_valid) break;
              if constexpr (OUT_F32)
                reinterpret_cast<float*>(cbase)[grow * p.ldc + col + r] = acc[i][j][r];
              else
                reinterpret_cast<bf16_t*>(cbase)[grow * p.ldc + col + r] = f32_to_bf16(acc[i][j][r]);
            }
            continue;
          }
          if constexpr (OUT_F32) {
            st16(cbase + (grow * p.ldc + col) * 4,
                 u32x4{__float_as_uint(acc[i][j][0]), __float_as_uint(acc[i][j][1]),
                       __float_as_uint(acc[i][j][2]), __float_as_uint(acc[i][j][3])});
          } else {
            *reinterpret_cast<u32x2*>(cbase + (grow * p.ldc + col) * 2) =
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
               static_cast<int>(max_rows), K, N, N, N, K, 0};
  const int grid = persistent_grid(max_rows, e_count, N / 128, num_cus);
  gemm_bf16_kernel<true, false><<<grid, 256, 0, s>>>(p);
}

void launch_gemm_down_bf16(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                           int K, int N, const void* w_down, void* y, bool out_f32, int num_cus,
                           hipStream_t s) {
  GemmParams p{static_cast<const char*>(a), static_cast<const char*>(w_down), nullptr,
               static_cast<char*>(y), offsets, e_count, static_cast<int>(max_rows), K, N, N, N,
               K, 0};
  const int grid = persistent_grid(max_rows, e_count, N / 256, num_cus);
  if (out_f32)
    gemm_bf16_kernel<false, true><<<grid, 256, 0, s>>>(p);
  else
    gemm_bf16_kernel<false, false><<<grid, 256, 0, s>>>(p);
}

void launch_gemm_nt_f32_splitk(const void* a, int64_t rows, int K, const void* b, int n_valid,
                               int splits, float* c_partials, int num_cus, hipStream_t s) {
  // One group of `rows` rows against n_valid (<= 256) weight rows, K split in
  // `splits` equal ranges; split y writes its fp32 partial product to
  // c_partials[y][rows][n_valid].
  GemmParams p{static_cast<const char*>(a), static_cast<const char*>(b), nullptr,
               reinterpret_cast<char*>(c_partials), nullptr, 1, static_cast<int>(rows), K, 256,
               n_valid, n_valid, K / splits, rows * static_cast<int64_t>(n_valid)};
  const int gx = persistent_grid(rows, 1, 1, num_cus);
  gemm_bf16_kernel<false, true><<<dim3(gx, splits), 256, 0, s>>>(p);
}

}  // namespace mf
