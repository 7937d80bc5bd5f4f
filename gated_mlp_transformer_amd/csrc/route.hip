// Sigmoid-with-bias top-8 router ("推理计算流梳理", 专家并行 / MoE Router 过程):
//   z = x W_r^T, s = sigmoid(z), I = Top8(s + b), w_i = s_i / sum_{j in I} s_j.
//
// Two kernels:
//  1. logits: z = x W_r^T on the bf16 MFMA GEMM core (128-token tiles against
//     all E <= 256 router rows, fp32 accumulation). The d-long contraction is
//     split into `splits` equal ranges so that about 256 workgroups run even
//     for a few thousand tokens; split y writes its fp32 partial logits to
//     workspace[y][T][E]. Splitting K instead of E keeps every workgroup's
//     W_r traffic at 1/splits of the router weight.
//  2. select: one wavefront per token sums the partials in split order (fixed
//     order: deterministic), applies the sigmoid and the bias, and picks the
//     top 8 by eight rounds of a wave-wide arg-max on (key descending, id
//     ascending); the ids are emitted ascending with w = s / sum(s).
//     A round takes the wave-wide maximum of the keys (mapped to
//     order-preserving unsigned integers) with DPP max steps at register
//     speed, then the lowest expert id that holds it as a second DPP
//     maximum (of 256 - id over the lanes' candidates equal to the key
//     maximum; a lane holds experts lane + 64c). Only that candidate is
//     retired, so equal keys are taken in ascending id order over the rounds.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int kTargetWGs = 256;   // one workgroup per CU of an MI355X
constexpr int kTokTile = 128;     // token rows per logits tile
constexpr int kMaxSplits = 16;

// Unsigned integer with the same order as the float (finite values and
// infinities; 0 is below every such value).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// v from the lane CTRL names; lanes in rows outside ROW_MASK receive 0, the
// identity of an unsigned max (so the move folds into the max instruction)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or0(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}

// Wave-wide maximum, uniform. After the two quad permutations and the two
// mirrors every lane holds its 16-lane row's maximum; row_bcast15 folds row 0
// into row 1 and row 2 into row 3, row_bcast31 folds lane 31 into row 3, so
// lane 63 holds the maximum of all 64 lanes.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_or0<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_or0<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_or0<0x141, 0xF>(v));  // row_half_mirror
  v = max(v, dpp_or0<0x140, 0xF>(v));  // row_mirror
  v = max(v, dpp_or0<0x142, 0xA>(v));  // row_bcast15 into rows 1 and 3
  v = max(v, dpp_or0<0x143, 0xC>(v));  // row_bcast31 into rows 2 and 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

}  // namespace

int route_splits(int64_t T, int d) {
  const int64_t tiles = (T + kTokTile - 1) / kTokTile;
  int ks = 1;  // each split's K range must stay a multiple of 256
  while ((d / 256) % (ks * 2) == 0 && tiles * ks * 2 <= kTargetWGs && ks * 2 <= kMaxSplits) ks *= 2;
  return ks;
}

size_t route_workspace_bytes(int64_t T, int d, int E) {
  return static_cast<size_t>(route_splits(T, d)) * static_cast<size_t>(T) * E * sizeof(float);
}

template <int SPLITS>
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ zp,
                                                           const float* __restrict__ bias,
                                                           int64_t T, int E,
                                                           int32_t* __restrict__ idx_out,
                                                           float* __restrict__ w_out) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (t >= T) return;
  const int64_t split_stride = T * E;
  // All partial logits are loaded before any is added (independent loads in
  // flight together), then summed in split order. The loads are
  // unconditional (experts past E re-read expert E-1 and are masked below):
  // a load under a per-lane condition would become a branch with its own wait.
  float part[SPLITS][4];
#pragma unroll
  for (int y = 0; y < SPLITS; ++y)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = min(lane + 64 * c, E - 1);
      part[y][c] = zp[y * split_stride + t * E + e];
    }
  // candidates of this lane: experts lane + 64c, the key s + b mapped to an
  // order-preserving unsigned integer; experts past E and retired winners
  // hold 0, below every valid key
  float sc[4];
  uint32_t key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    float z = 0.f;
#pragma unroll
    for (int y = 0; y < SPLITS; ++y) z += part[y][c];
    sc[c] = sigmoidf_(z);
    key[c] = e < E ? order_key(sc[c] + bias[min(e, E - 1)]) : 0u;
  }
  // Eight rounds; a round takes the wave-wide maximum key m, then the lowest
  // expert id holding it as a second wave-wide maximum, of 256 - e over each
  // lane's candidates equal to m (all in VALU/DPP: no ballot chains on the
  // CU's one scalar unit, which all the resident token waves share). The
  // owner lane retires the winner and flags it.
  uint32_t won = 0;  // bit c: expert lane + 64c was selected
#pragma unroll
  for (int round = 0; round < 8; ++round) {
    const uint32_t m = wave_umax(max(max(key[0], key[1]), max(key[2], key[3])));
    uint32_t cand = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      cand = max(cand, key[c] == m ? 256u - static_cast<uint32_t>(lane + 64 * c) : 0u);
    const int e = 256 - static_cast<int>(wave_umax(cand));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool hit = lane + 64 * c == e;  // only the owner lane's slot matches
      key[c] = hit ? 0u : key[c];
      won |= hit ? 1u << c : 0u;
    }
  }
  // The winners in ascending id order (slot c, then lane): rank r goes to
  // lane r of the outputs, and the scores are summed in that order.
  int out_e = 0;
  float out_s = 0.f, sum = 0.f;
  int r = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint64_t mk = __builtin_amdgcn_ballot_w64((won >> c) & 1u);
    while (mk) {
      const int l = __builtin_ctzll(mk);
      mk &= mk - 1;
      const float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[c]), l));
      if (lane == r) {
        out_e = l + 64 * c;
        out_s = sv;
      }
      sum += sv;
      ++r;
    }
  }
  if (lane < 8) {
    idx_out[t * 8 + lane] = out_e;
    w_out[t * 8 + lane] = out_s / sum;
  }
}

void launch_route(const void* x, const void* w_r, const float* bias, int64_t T, int d, int E,
                  int32_t* idx, float* w, void* workspace, int num_cus, hipStream_t s) {
  const int splits = route_splits(T, d);
  float* zp = static_cast<float*>(workspace);
  launch_gemm_nt_f32_splitk(x, T, d, w_r, E, splits, zp, num_cus, s);
  const dim3 grid(static_cast<unsigned>((T + 3) / 4));
  switch (splits) {  // route_splits returns a power of two <= kMaxSplits
    case 1: route_select_kernel<1><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w); break;
    case 2: route_select_kernel<2><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w); break;
    case 4: route_select_kernel<4><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w); break;
    case 8: route_select_kernel<8><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w); break;
    default: route_select_kernel<kMaxSplits><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w); break;
  }
}

}  // namespace mf
