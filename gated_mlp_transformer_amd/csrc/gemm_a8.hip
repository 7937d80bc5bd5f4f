// Grouped GEMMs with fp8 activations and block-fp8 weights on the gfx950 fp8
// MFMA: the block-fp8 prefill variant ("「赤兔」Chitu 框架深度解读（七）：MoE",
// 专家计算实现: prefill experts run as FP8 GEMMs on tokens laid out contiguously by
// expert; 量化支持: block fp8; "推理计算流梳理", EP 路径 and 实际 MLP 计算策略).
//
//   gate/up:  H[rows of e] = SiLU(A Wg_e^T) * (A Wu_e^T)   (bf16 out)
//   down:     Y[rows of e] = A Wd_e^T                       (bf16 out)
// with A[t, k] = code[t, k] * a_scale[t, k/128]   (per-token 1x128 groups)
//      W[n, k] = code[n, k] * w_scale[n/128, k/128]
//
// Both scales change every 128 channels of the contraction, and the
// activation scale differs per token, so each 128-deep block is accumulated
// from zero on MFMA (two v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0
// scales: exact fp8 products, fp32 sums) and then added into the fp32 result
// with one FMA per element by a_scale(token) * w_scale. The weight fragment is
// the MFMA's first operand (32 weight rows), the activation rows the second,
// so a lane holds one token of the result and that token's scale is one value
// per lane.
//
// Tiling. A workgroup (4 waves) computes up to 128 rows (MT = 4 sub-tiles of
// 32) against 256 weight rows (128 gate + 128 up, or 256 down); each wave owns
// 64 weight rows (two 32-row fragments) for all the tile's rows, with 8 fp32
// accumulators in VGPRs (the per-block partial sums sit in AGPRs). 128 rows
// is what the register file holds next to the partials; a 256-row x 128
// weight-row layout with the waves in 2 x 2 (half the weight bytes per FLOP)
// was measured slower.
// One pipeline stage is one 128-deep block. A (fp8, optionally gathered by
// row_index) is loaded one stage ahead and staged in LDS (two buffers, rows of
// 128 bytes, 16-byte chunks XOR-swizzled by row); weight fragments come
// straight from global memory into registers three stages ahead (a ring of
// four slots). The activation scales travel with the A rows into LDS; the
// weight scales of a tile's whole contraction are put in LDS at the tile's
// start. The fp8 weights use the same packed order as the decode kernels
// (16-row x 128-column blocks, slab-major, pack.hip); a lane gathers its 32
// bytes of a 32-row fragment from the two 16-row blocks.
//
// Schedule. As the bf16 grouped GEMM: each expert's rows split into
// near-equal chunks of at most MT 32-row sub-tiles, tiles numbered expert /
// n-tile / chunk (the chunks sharing a weight n-tile consecutive), persistent
// grid with XCD-contiguous round-robin.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int ROW8 = 128;   // bytes of one A row per stage (a 128-deep block)
constexpr int A8_MAX_SLABS = 128;  // K <= 16384 (checked by the entry points)
constexpr int MAXG = 256;
constexpr int WSLOTS = 4;   // weight register slots: three stages in flight
constexpr int BLK8 = 2048;  // bytes of one packed 16 x 128 fp8 block

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

struct A8Params {
  const uint8_t* a;        // fp8 codes [max_rows, K], or [a_src_rows, K] with a_rows
  const float* as;         // activation scales, same rows, [.., K/128]
  const int32_t* a_rows;   // nullptr or [max_rows]: GEMM row r reads row a_rows[r]
  int a_src_rows;
  const uint8_t* b0;       // packed fp8 weights (gate, or down)
  const uint8_t* b1;       // packed fp8 weights (up; gated only)
  const float* s0;         // weight scales [groups, N/128, K/128]
  const float* s1;
  char* c;                 // [max_rows, ldc] bf16
  const int32_t* offsets;  // [groups+1]
  int e_count;
  int max_rows;
  int K;                   // contraction length
  int N;                   // weight rows per matrix
  int ldc;
};

// chunk c (16 bytes) of stage row r sits at chunk c ^ (r & 7)
__device__ __forceinline__ int swz8(int r, int c) { return r * ROW8 + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& w, const i32x8& a, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, a, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join(const u32x4& lo, const u32x4& hi) {
  return i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
               static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
               static_cast<int>(hi[2]), static_cast<int>(hi[3])};
}

}  // namespace

// K loop of one tile for NM live 32-row sub-tiles. Stage t: issue A(t+1) with
// the activation scales of the rows this thread moves, and the weights of
// t+3; for each sub-tile read its two 64-deep fragments from LDS, run two
// MFMAs per weight fragment from zero and add the block into the result with
// the block's scales (activation scale from LDS beside the A rows, weight
// scale from the tile's LDS table); write A(t+1) and its scales to the other
// LDS buffer; barrier. Every scale is consumed together with the data it
// travels with, so the one in-order load counter never holds a weight
// prefetch back for a scale, and the four-stage loop body has no branches
// (a two-stage tail takes nk % 4 == 2; with ODD, for an odd slab count, a
// tail of one or three stages, in a separate kernel so that the common even
// case keeps its register allocation), so every wait inside the loop is
// static.
template <int MT, int NM, bool GATED, bool ODD>
__device__ __forceinline__ void a8_k_loop(f32x16 (&acc)[MT][2], const uint8_t* const (&ap)[MT],
                                          const float* const (&aspr)[MT],
                                          const uint8_t* const (&bp)[2], const float* s_sw,
                                          char (&lds)[2][MT * 32 * ROW8],
                                          float (&s_sa)[2][MT * 32], int nk, int64_t sstride,
                                          int ld_r, int ld_c, int lane) {
  constexpr int NA = MT;    // A loads (16 bytes) per thread per stage: BM rows x 8 chunks / 256
  u32x4 areg[NA];
  float ascl[NA];           // activation scales of the rows this thread moves
  u32x4 breg[WSLOTS][8];    // [jn][step s][half h]
  const int lr = lane & 31, hh = lane >> 5;
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NA; ++i) areg[i] = ld16(ap[i] + static_cast<int64_t>(kt) * ROW8);
#pragma unroll
    for (int i = 0; i < NA; ++i) ascl[i] = aspr[i][kt];
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
    for (int i = 0; i < NA; ++i) st16(&lds[buf][swz8(ld_r + 32 * i, ld_c)], areg[i]);
    // the eight threads of a row store the same value
#pragma unroll
    for (int i = 0; i < NA; ++i) s_sa[buf][ld_r + 32 * i] = ascl[i];
  };
  auto stage = [&](const u32x4 (&br)[8], int buf, int kt, int kt_next, u32x4 (&b_dst)[8],
                   int kt_b) {
    load_a(kt_next);
    load_b(b_dst, kt_b);
    const float sw0 = s_sw[kt], sw1 = s_sw[nk + kt];
    const i32x8 w00 = join(br[0], br[1]), w01 = join(br[2], br[3]);
    const i32x8 w10 = join(br[4], br[5]), w11 = join(br[6], br[7]);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int r = i * 32 + lr;
      const i32x8 a0 = join(ld16(&lds[buf][swz8(r, 2 * hh)]), ld16(&lds[buf][swz8(r, 2 * hh + 1)]));
      const i32x8 a1 =
          join(ld16(&lds[buf][swz8(r, 4 + 2 * hh)]), ld16(&lds[buf][swz8(r, 4 + 2 * hh + 1)]));
      f32x16 p0 = mfma_fp8(w00, a0, f32x16{});
      f32x16 p1 = mfma_fp8(w10, a0, f32x16{});
      p0 = mfma_fp8(w01, a1, p0);
      p1 = mfma_fp8(w11, a1, p1);
      const float sa = s_sa[buf][r];
      const float c0 = sa * sw0;
      const float c1 = sa * sw1;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[i][0][v] = fmaf(p0[v], c0, acc[i][0][v]);
        acc[i][1][v] = fmaf(p1[v], c1, acc[i][1][v]);
      }
    }
    write_a(buf ^ 1);
  };

  load_a(0);
#pragma unroll
  for (int s = 0; s < WSLOTS - 1; ++s) load_b(breg[s], s < nk ? s : nk - 1);
  write_a(0);
  __syncthreads();
#define MF_A8_STEP(S)                                                                      \
  {                                                                                        \
    const int t_ = kt + (S);                                                               \
    stage(breg[(S)], (S) & 1, t_, min(t_ + 1, nk - 1), breg[((S) + WSLOTS - 1) % WSLOTS],  \
          min(t_ + WSLOTS - 1, nk - 1));                                                   \
    __syncthreads();                                                                       \
  }
  int kt = 0;
  for (; kt + WSLOTS <= nk; kt += WSLOTS) {
    MF_A8_STEP(0)
    MF_A8_STEP(1)
    MF_A8_STEP(2)
    MF_A8_STEP(3)
  }
  // the last nk % 4 stages, in the slots and buffers the four-stage body
  // would have used
  if constexpr (!ODD) {
    if (kt < nk) {  // nk is even: two stages left
      MF_A8_STEP(0)
      MF_A8_STEP(1)
    }
  } else {
    if (kt < nk) MF_A8_STEP(0)
    if (kt + 1 < nk) MF_A8_STEP(1)
    if (kt + 2 < nk) MF_A8_STEP(2)
  }
#undef MF_A8_STEP
}

template <int MT, bool GATED, bool ODD>
__global__ __launch_bounds__(256, 1) void gemm_a8_kernel(A8Params p) {
  constexpr int BN_OUT = GATED ? 128 : 256;
  __shared__ __attribute__((aligned(16))) char lds[2][MT * 32 * ROW8];
  __shared__ float s_sa[2][MT * 32];           // activation scales of the staged A rows
  __shared__ float s_sw[4][2 * A8_MAX_SLABS];  // per wave: weight scales of its two fragments
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
  const int ld_c = tid & 7;    // A: 16-byte chunk this thread moves
  const int ld_r = tid >> 3;   // A: first row (then +32, +64, ...)
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nk = KB;
  const int64_t Kb = p.K;      // bytes per A row

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
    auto src_row = [&](int m) {
      int arow = row0 + (m < rows_valid ? m : 0);
      if (p.a_rows != nullptr) arow = clampi(p.a_rows[arow], 0, p.a_src_rows - 1);
      return arow;
    };
    const uint8_t* ap[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
      ap[i] = p.a + static_cast<int64_t>(src_row(ld_r + 32 * i)) * Kb + ld_c * 16;
    const float* aspr[MT];  // activation scale rows of the A rows this thread moves
#pragma unroll
    for (int i = 0; i < MT; ++i) aspr[i] = p.as + static_cast<int64_t>(src_row(ld_r + 32 * i)) * KB;
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
    static_assert(MT == 4, "one tile height");
    {
      switch (nm) {
        case 1: a8_k_loop<MT, 1, GATED, ODD>(acc, ap, aspr, bp, s_sw[wave], lds, s_sa, nk, sstride, ld_r, ld_c, lane); break;
        case 2: a8_k_loop<MT, 2, GATED, ODD>(acc, ap, aspr, bp, s_sw[wave], lds, s_sa, nk, sstride, ld_r, ld_c, lane); break;
        case 3: a8_k_loop<MT, 3, GATED, ODD>(acc, ap, aspr, bp, s_sw[wave], lds, s_sa, nk, sstride, ld_r, ld_c, lane); break;
        default: a8_k_loop<MT, 4, GATED, ODD>(acc, ap, aspr, bp, s_sw[wave], lds, s_sa, nk, sstride, ld_r, ld_c, lane); break;
      }
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
          *reinterpret_cast<u32x2*>(p.c + (grow * p.ldc + col) * 2) =
              u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        } else {
#pragma unroll
          for (int jn = 0; jn < 2; ++jn) {
            const int col = n0 + wave * 64 + jn * 32 + 8 * qq + 4 * lg;
            if (col >= p.N) continue;  // past a partial last n-tile
            *reinterpret_cast<u32x2*>(p.c + (grow * p.ldc + col) * 2) =
                u32x2{pack_bf16x2(acc[i][jn][4 * qq], acc[i][jn][4 * qq + 1]),
                      pack_bf16x2(acc[i][jn][4 * qq + 2], acc[i][jn][4 * qq + 3])};
          }
        }
      }
    }
  }
}

namespace {

constexpr int MT_A8 = 4;  // 128-row tiles (see the tiling note above)

int a8_grid(int64_t max_rows, int e_count, int nt, int num_cus) {
  const int64_t mtiles = (max_rows + MT_A8 * 32 - 1) / (MT_A8 * 32) + e_count;
  const int64_t ub = mtiles * static_cast<int64_t>(nt);
  int64_t g = ub < num_cus ? ub : num_cus;
  g = (g + 7) & ~int64_t(7);
  if (g > num_cus) g = num_cus & ~7;
  return static_cast<int>(g < 8 ? 8 : g);
}

}  // namespace

void launch_gemm_gateup_a8(const void* a, const float* a_scale, const int32_t* a_rows,
                           int64_t a_src_rows, const int32_t* offsets, int e_count,
                           int64_t max_rows, int K, int N, const void* w_gate, const void* w_up,
                           const float* s_gate, const float* s_up, void* h, int num_cus,
                           hipStream_t s) {
  A8Params p{static_cast<const uint8_t*>(a), a_scale, a_rows, static_cast<int>(a_src_rows),
             static_cast<const uint8_t*>(w_gate), static_cast<const uint8_t*>(w_up), s_gate, s_up,
             static_cast<char*>(h), offsets, e_count, static_cast<int>(max_rows), K, N, N};
  const int grid = a8_grid(max_rows, e_count, N / 128, num_cus);
  if ((K / 128) % 2) gemm_a8_kernel<MT_A8, true, true><<<grid, 256, 0, s>>>(p);
  else gemm_a8_kernel<MT_A8, true, false><<<grid, 256, 0, s>>>(p);
}

void launch_gemm_down_a8(const void* a, const float* a_scale, const int32_t* offsets,
                         int e_count, int64_t max_rows, int K, int N, const void* w_down,
                         const float* s_down, void* y, int num_cus, hipStream_t s) {
  A8Params p{static_cast<const uint8_t*>(a), a_scale, nullptr, 0,
             static_cast<const uint8_t*>(w_down), nullptr, s_down, nullptr,
             static_cast<char*>(y), offsets, e_count, static_cast<int>(max_rows), K, N, N};
  const int grid = a8_grid(max_rows, e_count, (N + 255) / 256, num_cus);
  if ((K / 128) % 2) gemm_a8_kernel<MT_A8, false, true><<<grid, 256, 0, s>>>(p);
  else gemm_a8_kernel<MT_A8, false, false><<<grid, 256, 0, s>>>(p);
}

}  // namespace mf
