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
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int kTargetWGs = 256;   // one workgroup per CU of an MI355X
constexpr int kTokTile = 128;     // token rows per logits tile
constexpr int kMaxSplits = 16;

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
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

__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ zp,
                                                           int splits, const float* __restrict__ bias,
                                                           int64_t T, int E,
                                                           int32_t* __restrict__ idx_out,
                                                           float* __restrict__ w_out) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (t >= T) return;
  const int64_t split_stride = T * E;
  // All partial logits are loaded before any is added (independent loads in
  // flight together), then summed in split order.
  float part[kMaxSplits][4];
#pragma unroll
  for (int y = 0; y < kMaxSplits; ++y)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      part[y][c] = (y < splits && e < E) ? zp[y * split_stride + t * E + e] : 0.f;
    }
  float s[4], kv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    float z = 0.f;
#pragma unroll
    for (int y = 0; y < kMaxSplits; ++y) z += part[y][c];
    s[c] = sigmoidf_(z);
    kv[c] = e < E ? s[c] + bias[e] : -__builtin_inff();
  }
  int sel[8];
  float ssel[8];
#pragma unroll
  for (int round = 0; round < 8; ++round) {
    float bk = -__builtin_inff(), bs = 0.f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      if (better(kv[c], e, bk, bi)) {
        bk = kv[c];
        bi = e;
        bs = s[c];
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ok = __shfl_xor(bk, m, kWave);
      const int oi = __shfl_xor(bi, m, kWave);
      const float os = __shfl_xor(bs, m, kWave);
      if (better(ok, oi, bk, bi)) {
        bk = ok;
        bi = oi;
        bs = os;
      }
    }
    sel[round] = bi;
    ssel[round] = bs;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (lane + 64 * c == bi) kv[c] = -__builtin_inff();  // the owner lane retires the winner
  }
  // ids ascending (I is a set), scores carried along
#pragma unroll
  for (int a = 1; a < 8; ++a) {
#pragma unroll
    for (int b = a; b > 0; --b) {
      if (sel[b - 1] > sel[b]) {
        const int ti = sel[b];
        sel[b] = sel[b - 1];
        sel[b - 1] = ti;
        const float ts = ssel[b];
        ssel[b] = ssel[b - 1];
        ssel[b - 1] = ts;
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) sum += ssel[q];
  if (lane < 8) {
    int mine = sel[0];
    float ms = ssel[0];
#pragma unroll
    for (int q = 1; q < 8; ++q)
      if (lane == q) {
        mine = sel[q];
        ms = ssel[q];
      }
    idx_out[t * 8 + lane] = mine;
    w_out[t * 8 + lane] = ms / sum;
  }
}

void launch_route(const void* x, const void* w_r, const float* bias, int64_t T, int d, int E,
                  int32_t* idx, float* w, void* workspace, int num_cus, hipStream_t s) {
  const int splits = route_splits(T, d);
  float* zp = static_cast<float*>(workspace);
  launch_gemm_nt_f32_splitk(x, T, d, w_r, E, splits, zp, num_cus, s);
  route_select_kernel<<<dim3(static_cast<unsigned>((T + 3) / 4)), 256, 0, s>>>(zp, splits, bias,
                                                                               T, E, idx, w);
}

}  // namespace mf
