// Weight packing: [groups, N, K] row-major ([out, in]) weights rearranged into
// the order in which the MFMA GEMMs consume them, so that every operand
// fragment a wavefront loads is one contiguous, fully coalesced 1 KB block.
//
// bf16: 32-row x 16-column fragments of v_mfma_f32_32x32x16_bf16's weight
//   operand, 1 KB each, row-block major then k-block:
//     dst[g][nb][kb][l][v] = W[g][32 nb + l % 32][16 kb + 8 (l / 32) + v]
//   (l = lane 0..63, v = 0..7); rows >= N are zero.
// fp8 (E4M3 codes): 16-row x 128-column blocks, 2 KB each, split in two 1 KB
//   halves so that each half is one 16-byte-per-lane load, 128-column slab
//   major (then group, then row block):
//     dst[kb][g][nb][h][l][b] = W[g][16 nb + l % 16][128 kb + 32 (l / 16) + 16 h + b]
//   (h = 0, 1; b = 0..15); rows >= N are zero. The fp8 GEMMs stream every
//   block of a slab before the next slab, so with the slab outermost the
//   workgroups running at one time read one contiguous window of HBM rather
//   than thousands of 2 KB streams 64 KB apart (6.5 vs 5.1 TB/s in a
//   load-only probe of the decode pattern).
//
// A pure permutation (plus zero padding): one thread moves one 16-byte chunk.
//
// The source may also be given [groups, K, N] ([in, out], the Y = X W
// orientation of the pages' gated-MLP formula): the packed result is the same
// as for its transpose. Then a chunk's 8 (bf16) or 16 (fp8) elements lie N
// apart in the source and are gathered one by one; neighbouring lanes take
// neighbouring rows, i.e. neighbouring source addresses.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

struct PackGeom {
  int rows_blk;   // rows per block (32 bf16, 16 fp8)
  int cols_blk;   // columns (elements) per block (16 bf16, 128 fp8)
  int esize;      // bytes per element
};

__host__ __device__ inline PackGeom geom(bool fp8) {
  return fp8 ? PackGeom{16, 128, 1} : PackGeom{32, 16, 2};
}

}  // namespace

size_t packed_bytes(int64_t groups, int N, int K, bool fp8) {
  const PackGeom g = geom(fp8);
  const int64_t nb = (N + g.rows_blk - 1) / g.rows_blk;
  return static_cast<size_t>(groups) * nb * g.rows_blk * K * g.esize;
}

template <bool FP8, bool KN>
__global__ __launch_bounds__(256) void pack_kernel(const char* __restrict__ src, char* __restrict__ dst,
                                                   int64_t groups, int N, int K) {
  const PackGeom g = geom(FP8);
  const int64_t nb = (N + g.rows_blk - 1) / g.rows_blk;
  const int kbs = K / g.cols_blk;
  const int64_t chunks = groups * nb * kbs * (FP8 ? 128 : 64);  // 16-byte chunks of dst
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    // dst chunk c -> (group, row block, k block, [half,] lane)
    int64_t q = c;
    int lane, half = 0, kb;
    int64_t rb, grp;
    if (FP8) {  // [kb][g][nb][h][l]
      lane = static_cast<int>(q % 64);
      q /= 64;
      half = static_cast<int>(q % 2);
      q /= 2;
      rb = q % nb;
      q /= nb;
      grp = q % groups;
      kb = static_cast<int>(q / groups);
    } else {    // [g][nb][kb][l]
      lane = static_cast<int>(q % 64);
      q /= 64;
      kb = static_cast<int>(q % kbs);
      q /= kbs;
      rb = q % nb;
      grp = q / nb;
    }
    int64_t row;
    int64_t col;
    if (FP8) {
      row = rb * 16 + (lane % 16);
      col = static_cast<int64_t>(kb) * 128 + 32 * (lane / 16) + 16 * half;
    } else {
      row = rb * 32 + (lane % 32);
      col = static_cast<int64_t>(kb) * 16 + 8 * (lane / 32);
    }
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < N) {
      if constexpr (!KN) {
        v = ld16(src + ((grp * N + row) * K + col) * g.esize);
      } else {
        // element col + i of row `row`: src[grp][col + i][row]
        const int64_t base = (grp * K + col) * N + row;
        if constexpr (FP8) {
          const uint8_t* s8 = reinterpret_cast<const uint8_t*>(src);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            v[i / 4] |= static_cast<uint32_t>(s8[base + static_cast<int64_t>(i) * N]) << (8 * (i % 4));
        } else {
          const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            v[i / 2] |= static_cast<uint32_t>(s16[base + static_cast<int64_t>(i) * N]) << (16 * (i % 2));
        }
      }
    }
    st16(dst + c * 16, v);
  }
}

void launch_pack(const void* src, void* dst, int64_t groups, int N, int K, bool fp8, bool kn,
                 hipStream_t s) {
  const PackGeom g = geom(fp8);
  const int64_t nb = (N + g.rows_blk - 1) / g.rows_blk;
  const int64_t chunks = groups * nb * (K / g.cols_blk) * (fp8 ? 128 : 64);
  int64_t grid = (chunks + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  const dim3 gr(static_cast<unsigned>(grid));
  const char* sp = static_cast<const char*>(src);
  char* dp = static_cast<char*>(dst);
  if (fp8) {
    if (kn) pack_kernel<true, true><<<gr, 256, 0, s>>>(sp, dp, groups, N, K);
    else pack_kernel<true, false><<<gr, 256, 0, s>>>(sp, dp, groups, N, K);
  } else {
    if (kn) pack_kernel<false, true><<<gr, 256, 0, s>>>(sp, dp, groups, N, K);
    else pack_kernel<false, false><<<gr, 256, 0, s>>>(sp, dp, groups, N, K);
  }
}

}  // namespace mf
