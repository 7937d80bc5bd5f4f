// Sigmoid-with-bias top-8 router ("推理计算流梳理", 专家并行 / MoE Router 过程):
//   z = x W_r^T, s = sigmoid(z), I = Top8(s + b), w_i = s_i / sum_{j in I} s_j.
//
// One 256-thread workgroup per 16 tokens. The logits tile [16 tokens x 256
// experts] is computed on MFMA (bf16 operands, fp32 accumulation): wave w owns
// experts [64w, 64w+64) as four 16x16 output tiles, so every lane keeps 16
// logits in registers. Both operands are K-contiguous in memory (x rows and
// W_r rows), so MFMA fragments are loaded straight from global memory, 16 bytes
// per lane, without an LDS round trip; the A fragment (tokens) is shared by
// all four waves through the L1. The epilogue writes s and s + b to LDS and
// each wave selects the top 8 of four tokens by eight rounds of a wave-wide
// arg-max on (key descending, id ascending).
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int kTok = 16;       // tokens per workgroup
constexpr int kMaxE = 256;     // experts held by one workgroup
constexpr int kLdsPitch = kMaxE + 4;

struct Frags {
  u32x4 a[2];
  u32x4 b[2][4];
};

__device__ __forceinline__ void load_frags(Frags& f, const char* xrow, const char* const* wrow,
                                           int k0, int g) {
  // k-chunk c covers [k0 + 32c, k0 + 32c + 32); lane group g holds 8 of them.
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const size_t off = static_cast<size_t>(k0 + 32 * c + 8 * g) * 2;
    f.a[c] = ld16(xrow + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[c][j] = ld16(wrow[j] + off);
  }
}

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

}  // namespace

__global__ __launch_bounds__(256) void route_kernel(const bf16_t* __restrict__ x,
                                                    const bf16_t* __restrict__ w_r,
                                                    const float* __restrict__ bias, int64_t T,
                                                    int d, int E, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out) {
  __shared__ float s_lds[kTok][kLdsPitch];
  __shared__ float k_lds[kTok][kLdsPitch];

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTok;

  // A operand: token row (clamped for loads; rows >= T are never written).
  const int64_t trow = t0 + (lane % 16) < T ? t0 + (lane % 16) : T - 1;
  const char* xrow = reinterpret_cast<const char*>(x + trow * d);
  // B operand: W_r rows of this wave's four 16-expert tiles (clamped).
  const char* wrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = wave * 64 + j * 16 + (lane % 16);
    wrow[j] = reinterpret_cast<const char*>(w_r + static_cast<int64_t>(e < E ? e : E - 1) * d);
  }
  const bool wave_active = wave * 64 < E;

  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (wave_active) {
    Frags cur, nxt;
    load_frags(cur, xrow, wrow, 0, g);
    for (int k0 = 0; k0 < d; k0 += 64) {
      if (k0 + 64 < d) load_frags(nxt, xrow, wrow, k0 + 64, g);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16x16x32(cur.a[c], cur.b[c][j], acc[j]);
      cur = nxt;
    }
  }

  // D[token 4*(l/16)+r][expert 64w+16j+l%16]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = wave * 64 + j * 16 + (lane % 16);
    const float be = e < E ? bias[e] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;
      const float s = sigmoidf_(acc[j][r]);
      s_lds[i][e] = s;
      k_lds[i][e] = e < E ? s + be : -__builtin_inff();
    }
  }
  __syncthreads();

  // Top-8 of four tokens per wave.
  for (int ii = 0; ii < 4; ++ii) {
    const int i = wave * 4 + ii;
    const int64_t t = t0 + i;
    if (t >= T) break;
    float kv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) kv[c] = k_lds[i][lane + 64 * c];
    int sel[8];
#pragma unroll
    for (int round = 0; round < 8; ++round) {
      float bk = -__builtin_inff();
      int bi = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        if (better(kv[c], e, bk, bi)) {
          bk = kv[c];
          bi = e;
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ok = __shfl_xor(bk, m, kWave);
        const int oi = __shfl_xor(bi, m, kWave);
        if (better(ok, oi, bk, bi)) {
          bk = ok;
          bi = oi;
        }
      }
      sel[round] = bi;
      // The owner lane retires the winner.
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (lane + 64 * c == bi) kv[c] = -__builtin_inff();
    }
    // ids ascending (I is a set), then w = s / sum s over the set.
#pragma unroll
    for (int a = 1; a < 8; ++a) {
#pragma unroll
      for (int b = a; b > 0; --b) {
        if (sel[b - 1] > sel[b]) {
          const int tmp = sel[b];
          sel[b] = sel[b - 1];
          sel[b - 1] = tmp;
        }
      }
    }
    float sv[8], sum = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      sv[q] = s_lds[i][clampi(sel[q], 0, kMaxE - 1)];
      sum += sv[q];
    }
    if (lane < 8) {
      int mine = sel[0];
      float ms = sv[0];
#pragma unroll
      for (int q = 1; q < 8; ++q)
        if (lane == q) {
          mine = sel[q];
          ms = sv[q];
        }
      idx_out[t * 8 + lane] = mine;
      w_out[t * 8 + lane] = ms / sum;
    }
  }
}

void launch_route(const void* x, const void* w_r, const float* bias, int64_t T, int d, int E,
                  int32_t* idx, float* w, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((T + kTok - 1) / kTok));
  route_kernel<<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(x),
                                    static_cast<const bf16_t*>(w_r), bias, T, d, E, idx, w);
}

}  // namespace mf
