// Grouped GEMMs with block-scaled fp8 (E4M3FN) expert weights and bf16
// activations, tiled for experts that hold many rows (prefill): the weights
// are read once per 128-row tile instead of once per 16 rows as in the
// decode kernels ("「赤兔」Chitu 框架深度解读（七）：MoE", quantisation support:
// block fp8 experts; "推理计算流梳理", EP 路径 and 实际 MLP 计算策略).
//
//   gate/up:  H[rows of e] = SiLU(A Wg_e^T) * (A Wu_e^T)   (bf16 out)
//   down:     Y[rows of e] = A Wd_e^T                       (bf16 out)
// with W[n, k] = code[n, k] * scale[n/128, k/128], A bf16.
//
// The arithmetic is the decode kernels': codes are converted to bf16 exactly
// (every E4M3FN value is a bf16 value), each 128-deep block is summed from
// zero on the bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulation), and
// the block sum is added into the fp32 result times the block's scale. The
// weight fragment is the MFMA's first operand (32 weight rows), the
// activation rows the second.
//
// Tiling. A workgroup (4 waves) computes up to 128 rows (4 sub-tiles of 32)
// against 256 weight rows (128 gate + 128 up, or 256 down); each wave owns 64
// weight rows (two 32-row fragments) for all the tile's rows: block partials
// in AGPRs, running fp32 sums in VGPRs. One pipeline stage is one 128-deep
// block: A (bf16, optionally gathered by row_index) is loaded one stage ahead
// and staged in LDS (two buffers of 128 rows x 256 bytes, 16-byte chunks
// XOR-swizzled by row); the weight codes come straight from global memory
// into registers one stage ahead (two register sets in turn), 32 bytes of a
// 64-deep half per lane from the two 16-row blocks of the packed fp8 layout
// (pack.hip, slab-major). A lane holds weight bytes k = 64s + 32g + (0..31)
// of half s (g = lane / 32); MFMA step (s, j) takes k = 64s + 32g + 8j + v,
// v = 0..7, from both operands: the contraction order is permuted
// identically on both sides, which leaves the dot products unchanged. A
// step's eight codes are converted once per stage and reused by the tile's
// four sub-tiles. A tile's weight scales for the whole contraction are put
// in LDS at its start.
//
// Schedule. As the other grouped GEMMs: each expert's rows split into
// near-equal chunks of at most 4 sub-tiles, tiles numbered expert / n-tile /
// chunk, persistent grid with XCD-contiguous round-robin.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int ROWW = 256;   // bytes of one bf16 A row per stage (a 128-deep block)
constexpr int W8_MAX_SLABS = 128;  // K <= 16384
constexpr int MAXG = 256;
constexpr int WSLOTS = 2;   // weight register slots: one stage in flight
constexpr int BLK8 = 2048;  // bytes of one packed 16 x 128 fp8 block
constexpr int MT = 4;       // 32-row sub-tiles per tile

typedef __attribute__((ext_vector_type(16))) float f32x16;

struct W8Params {
  const char* a;           // bf16 [max_rows, K], or [a_src_rows, K] with a_rows
  const int32_t* a_rows;   // nullptr or [max_rows]: GEMM row r reads row a_rows[r]
  int a_src_rows;
  const uint8_t* b0;       // packed fp8 weights (gate, or down)
  const uint8_t* b1;       // packed fp8 weights (up; gated only)
  const float* s0;         // weight scales [groups, N/128, K/128]
  const float* s1;
  char* c;                 // [max_rows, N] bf16
  const int32_t* offsets;  // [groups+1]
  int e_count;
  int max_rows;
  int K;
  int N;
};

// chunk c (16 bytes, 0..15) of stage row r sits at chunk c ^ (r & 15): the 32
// rows of a fragment read (one logical chunk) land on distinct chunks of
// every 16 consecutive rows, so each group of 8 lanes hits distinct banks
__device__ __forceinline__ int swzw(int r, int c) { return r * ROWW + ((c ^ (r & 15)) << 4); }

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& w, const u32x4& a, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                 __builtin_bit_cast(bf16x8, a), c, 0, 0, 0);
}

// bf16 weights of step j (0..3) of a half: codes 8j .. 8j+7 of the lane's 32
// bytes, held as two 16-byte registers lo (bytes 0..15) and hi (16..31)
__device__ __forceinline__ u32x4 codes_to_bf16(const u32x4& lo, const u32x4& hi, int j) {
  const u32x4& src = (j >> 1) ? hi : lo;
  const u32x2 a = fp8x4_to_bf16x4(src[2 * (j & 1)]);
  const u32x2 b = fp8x4_to_bf16x4(src[2 * (j & 1) + 1]);
  return u32x4{a[0], a[1], b[0], b[1]};
}

}  // namespace

// K loop of one tile for NM live 32-row sub-tiles. Stage t: issue A(t+1) and
// the weights of t+1; for each of the eight 16-deep steps convert the two
// fragments' codes and run two MFMAs per live sub-tile into the block
// partials; add the partials into the result with the block's weight scales;
// write A(t+1) to the other LDS buffer; barrier. The two-stage loop body has
// no branches (an odd slab count takes a one-stage tail, in a separate kernel
// so that the even case keeps its register allocation), so every wait inside
// the loop is static.
template <int NM, bool GATED, bool ODD>
__device__ __forceinline__ void w8_k_loop(f32x16 (&acc)[MT][2], const char* abase,
                                          const int (&arow)[2 * MT], int64_t Kb,
                                          const uint8_t* const (&bp)[2], const float* s_sw,
                                          char (&lds)[2][MT * 32 * ROWW], int nk, int64_t sstride,
                                          int ld_r, int ld_c, int lane) {
  constexpr int NA = 2 * MT;  // A loads (16 bytes) per thread per stage: 128 rows x 16 chunks / 256
  u32x4 areg[NA];
  u32x4 breg[WSLOTS][8];      // [jn][half s][16-byte part h]
  const int lr = lane & 31, hh = lane >> 5;
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      areg[i] = ld16(abase + static_cast<int64_t>(arow[i]) * Kb + static_cast<int64_t>(kt) * ROWW);
  };
  // weights with the non-temporal cache policy: measured faster in both fp8
  // tiled kernels (8192-token prefill gate/up 338 -> 316 us with fp8
  // activations, 647 -> 595 us with bf16 ones); the bf16 grouped GEMM's
  // weight loads were slower with it (393 -> 402 us) and keep the default
  auto load_b = [&](u32x4 (&br)[8], int kt) {
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          br[jn * 4 + s * 2 + h] =
              ld16_stream(bp[jn] + static_cast<int64_t>(kt) * sstride + s * 512 + h * 1024);
  };
  auto write_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) st16(&lds[buf][swzw(ld_r + 16 * i, ld_c)], areg[i]);
  };
  auto stage = [&](const u32x4 (&br)[8], int buf, int kt, int kt_next, u32x4 (&b_dst)[8],
                   int kt_b) {
    load_a(kt_next);
    load_b(b_dst, kt_b);
    const float sw0 = s_sw[kt], sw1 = s_sw[nk + kt];
    f32x16 part[NM][2];
#pragma unroll
    for (int i = 0; i < NM; ++i) part[i][0] = part[i][1] = f32x16{};
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 w0 = codes_to_bf16(br[s * 2], br[s * 2 + 1], j);
        const u32x4 w1 = codes_to_bf16(br[4 + s * 2], br[4 + s * 2 + 1], j);
        // activation elements k = 64s + 32hh + 8j .. +8: bytes 128s + 64hh + 16j
        const int chunk = 8 * s + 4 * hh + j;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          const u32x4 a = ld16(&lds[buf][swzw(i * 32 + lr, chunk)]);
          part[i][0] = mfma_bf16(w0, a, part[i][0]);
          part[i][1] = mfma_bf16(w1, a, part[i][1]);
        }
      }
#pragma unroll
    for (int i = 0; i < NM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[i][0][v] = fmaf(part[i][0][v], sw0, acc[i][0][v]);
        acc[i][1][v] = fmaf(part[i][1][v], sw1, acc[i][1][v]);
      }
    write_a(buf ^ 1);
  };

  load_a(0);
#pragma unroll
  for (int s = 0; s < WSLOTS - 1; ++s) load_b(breg[s], s < nk ? s : nk - 1);
  write_a(0);
  __syncthreads();
#define MF_W8_STEP(S)                                                                      \
  {                                                                                        \
    const int t_ = kt + (S);                                                               \
    stage(breg[(S)], (S) & 1, t_, min(t_ + 1, nk - 1), breg[((S) + WSLOTS - 1) % WSLOTS],  \
          min(t_ + WSLOTS - 1, nk - 1));                                                   \
    __syncthreads();                                                                       \
  }
  int kt = 0;
  for (; ODD ? kt + WSLOTS <= nk : kt < nk; kt += WSLOTS) {
    MF_W8_STEP(0)
    MF_W8_STEP(1)
  }
  if constexpr (ODD) MF_W8_STEP(0)  // an odd slab count: the last slab
#undef MF_W8_STEP
}

template <bool GATED, bool ODD>
__global__ __launch_bounds__(256, 1) void gemm_w8_kernel(W8Params p) {
  constexpr int BN_OUT = GATED ? 128 : 256;
  __shared__ __attribute__((aligned(16))) char lds[2][MT * 32 * ROWW];
  __shared__ float s_sw[4][2 * W8_MAX_SLABS];  // per wave: weight scales of its two fragments
  __shared__ int s_tile0[MAXG + 1];
  __shared__ int s_beg[MAXG];
  __shared__ int s_end[MAXG];

  const int tid = threadIdx.x;
  // n-tiles of 256 weight rows (gated: 128 gate + 128 up; N % 128 == 0); the
  // down GEMM's last n-tile may hold only 128 valid rows
  const int NT = GATED ? p.N / 128 : (p.N + 255) / 256;
  const int KB = p.K / 128;
  const int NB16 = p.N / 16;
  const int NB128 = p.N / 128;

  // device-side schedule: expert e's ceil(rows/32) sub-tiles in ceil(sub/MT)
  // near-equal chunks; tiles numbered expert / n-tile / chunk
  int ntile = 0;
  if (tid < p.e_count) {
    const int beg = clampi(p.offsets[tid], 0, p.max_rows);
    const int end = clampi(p.offsets[tid + 1], beg, p.max_rows);
    s_beg[tid] = beg;
    s_end[tid] = end;
    ntile = ((((end - beg + 31) >> 5) + MT - 1) / MT) * NT;
  }
  s_tile0[tid + 1] = ntile;
  if (tid == 0) s_tile0[0] = 0;
  __syncthreads();
  for (int off = 1; off < p.e_count; off <<= 1) {  // entries 0 .. e_count are read
    const int v = tid >= off ? s_tile0[tid + 1 - off] : 0;
    __syncthreads();
    s_tile0[tid + 1] += v;
    __syncthreads();
  }
  const int total_tiles = s_tile0[p.e_count];

  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lr = lane & 31, hh = lane >> 5, lg = hh;
  const int ld_c = tid & 15;   // A: 16-byte chunk this thread moves
  const int ld_r = tid >> 4;   // A: first row (then +16, +32, ...)
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nk = KB;
  const int64_t Kb = static_cast<int64_t>(p.K) * 2;  // bytes per A row

  // Split tail (as in the bf16 grouped GEMM): a last round of tiles that is
  // at most half full runs each of its tiles as two units with half of the
  // tile's sub-tiles each, over the whole contraction.
  const int full_t = (total_tiles / G) * G;
  const int tail_t = total_tiles - full_t;
  const bool split = tail_t > 0 && 2 * tail_t <= G;
  const int total_units = split ? full_t + 2 * tail_t : total_tiles;

  for (int it = 0;; it += G) {
    const int U = it + xcd * (G >> 3) + slot;
    if (U >= total_units) break;
    // tile L; for a split tail tile, its first (half 0) or second row half
    int L = U, half = -1;
    if (split && U >= full_t) {
      L = full_t + ((U - full_t) >> 1);
      half = (U - full_t) & 1;
    }
    int lo = 0, hi = p.e_count - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tile0[mid] <= L) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int t = L - s_tile0[e];
    const int sub_e = (s_end[e] - s_beg[e] + 31) >> 5;
    const int nch = (sub_e + MT - 1) / MT;
    const int ni = t / nch, mi = t - ni * nch;  // n-tile major, chunk minor
    const int q = sub_e / nch, r = sub_e - q * nch;
    const int zc = mi * q + min(mi, r);   // first sub-tile of the chunk
    const int nmc = q + (mi < r ? 1 : 0); // sub-tiles in the chunk
    // a split tail tile: the first ceil(nmc/2) sub-tiles, or the rest
    const int z0 = half > 0 ? zc + (nmc + 1) / 2 : zc;
    const int nm = half < 0 ? nmc : (half == 0 ? (nmc + 1) / 2 : nmc / 2);
    if (nm == 0) continue;  // the second half of a one-sub-tile chunk
    const int row0 = s_beg[e] + z0 * 32;
    const int rows_valid = min(nm * 32, s_end[e] - row0);
    const int n0 = ni * BN_OUT;

    // A rows past the tile's valid rows re-read row0 (never stored)
    int arow[2 * MT];
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      const int m = ld_r + 16 * i;
      int ar = row0 + (m < rows_valid ? m : 0);
      if (p.a_rows != nullptr) ar = clampi(p.a_rows[ar], 0, p.a_src_rows - 1);
      arow[i] = ar;
    }
    const char* abase = p.a + ld_c * 16;
    // packed weights are slab-major: one 128-deep slab of every block of every
    // group, then the next slab
    const int64_t sstride = static_cast<int64_t>(p.e_count) * NB16 * BLK8;
    const uint8_t* bp[2];
    const float* wsp[2];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const uint8_t* base = (GATED && jn == 1) ? p.b1 : p.b0;
      const float* sbase = (GATED && jn == 1) ? p.s1 : p.s0;
      const int frow = GATED ? n0 + wave * 32 : n0 + wave * 64 + jn * 32;  // fragment's first row
      const int blk = min((frow + lr) >> 4, NB16 - 1);
      bp[jn] = base + (static_cast<int64_t>(e) * NB16 + blk) * BLK8 + (lr & 15) * 16 + hh * 256;
      wsp[jn] = sbase + (static_cast<int64_t>(e) * NB128 + min(frow >> 7, NB128 - 1)) * KB;
    }

    f32x16 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) acc[i][jn] = f32x16{};

    __syncthreads();  // the previous tile's LDS reads are done
    // this wave's weight scales for the whole contraction, [fragment][slab]
    // (read back by this wave only, in order)
    for (int j = lane; j < KB; j += kWave) {
      s_sw[wave][j] = wsp[0][j];
      s_sw[wave][KB + j] = wsp[1][j];
    }
    switch (nm) {
      case 1: w8_k_loop<1, GATED, ODD>(acc, abase, arow, Kb, bp, s_sw[wave], lds, nk, sstride, ld_r, ld_c, lane); break;
      case 2: w8_k_loop<2, GATED, ODD>(acc, abase, arow, Kb, bp, s_sw[wave], lds, nk, sstride, ld_r, ld_c, lane); break;
      case 3: w8_k_loop<3, GATED, ODD>(acc, abase, arow, Kb, bp, s_sw[wave], lds, nk, sstride, ld_r, ld_c, lane); break;
      default: w8_k_loop<4, GATED, ODD>(acc, abase, arow, Kb, bp, s_sw[wave], lds, nk, sstride, ld_r, ld_c, lane); break;
    }

    // epilogue: lane l holds, for token row lr of sub-tile i, output columns
    // 8q + 4(l/32) + 0..3 (q = 0..3) of each 32-column fragment
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = i * 32 + lr;
      if (m >= rows_valid) continue;
      const int64_t grow = row0 + m;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        if constexpr (GATED) {
          const int col = n0 + wave * 32 + 8 * qq + 4 * lg;
          float h[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            h[rr] = siluf_(acc[i][0][4 * qq + rr]) * acc[i][1][4 * qq + rr];
          *reinterpret_cast<u32x2*>(p.c + (grow * p.N + col) * 2) =
              u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        } else {
#pragma unroll
          for (int jn = 0; jn < 2; ++jn) {
            const int col = n0 + wave * 64 + jn * 32 + 8 * qq + 4 * lg;
            if (col >= p.N) continue;  // past a partial last n-tile
            *reinterpret_cast<u32x2*>(p.c + (grow * p.N + col) * 2) =
                u32x2{pack_bf16x2(acc[i][jn][4 * qq], acc[i][jn][4 * qq + 1]),
                      pack_bf16x2(acc[i][jn][4 * qq + 2], acc[i][jn][4 * qq + 3])};
          }
        }
      }
    }
  }
}

namespace {

int w8_grid(int64_t max_rows, int e_count, int nt, int num_cus) {
  const int64_t mtiles = (max_rows + MT * 32 - 1) / (MT * 32) + e_count;
  const int64_t ub = mtiles * static_cast<int64_t>(nt);
  int64_t g = ub < num_cus ? ub : num_cus;
  g = (g + 7) & ~int64_t(7);
  if (g > num_cus) g = num_cus & ~7;
  return static_cast<int>(g < 8 ? 8 : g);
}

}  // namespace

bool w8_prefers_tiles(int64_t max_rows, int e_count, int K) {
  // tiles once an expert can hold more rows than one 16-row pass of the
  // decode kernels, with the contraction the scale table holds
  return max_rows >= 32 * static_cast<int64_t>(e_count) && K <= 128 * W8_MAX_SLABS;
}

void launch_gemm_gateup_w8(const void* a, const int32_t* a_rows, int64_t a_src_rows,
                           const int32_t* offsets, int e_count, int64_t max_rows, int K, int N,
                           const void* w_gate, const void* w_up, const float* s_gate,
                           const float* s_up, void* h, int num_cus, hipStream_t s) {
  W8Params p{static_cast<const char*>(a), a_rows, static_cast<int>(a_src_rows),
             static_cast<const uint8_t*>(w_gate), static_cast<const uint8_t*>(w_up), s_gate, s_up,
             static_cast<char*>(h), offsets, e_count, static_cast<int>(max_rows), K, N};
  const int grid = w8_grid(max_rows, e_count, N / 128, num_cus);
  if ((K / 128) % 2) gemm_w8_kernel<true, true><<<grid, 256, 0, s>>>(p);
  else gemm_w8_kernel<true, false><<<grid, 256, 0, s>>>(p);
}

void launch_gemm_down_w8(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                         int K, int N, const void* w_down, const float* s_down, void* y,
                         int num_cus, hipStream_t s) {
  W8Params p{static_cast<const char*>(a), nullptr, 0, static_cast<const uint8_t*>(w_down),
             nullptr, s_down, nullptr, static_cast<char*>(y), offsets, e_count,
             static_cast<int>(max_rows), K, N};
  const int grid = w8_grid(max_rows, e_count, (N + 255) / 256, num_cus);
  if ((K / 128) % 2) gemm_w8_kernel<false, true><<<grid, 256, 0, s>>>(p);
  else gemm_w8_kernel<false, false><<<grid, 256, 0, s>>>(p);
}

}  // namespace mf
