// Sigmoid-with-bias top-8 router ("推理计算流梳理", 专家并行 / MoE Router 过程):
//   z = x W_r^T, s = sigmoid(z), I = Top8(s + b), w_i = s_i / sum_{j in I} s_j.
//
// Two kernels:
//  1. logits: z = x W_r^T with fp32 accumulation, the d-long contraction split
//     into `splits` equal ranges so that about 256 workgroups run; split y
//     writes its fp32 partial logits to workspace[y][T][E].
//     - Many tokens: the bf16 MFMA GEMM core (128-token tiles against all
//       E <= 256 router rows). Splitting K instead of E keeps every
//       workgroup's W_r traffic at 1/splits of the router weight.
//     - Few tokens (decode): one wavefront per 32 tokens x 32 experts x one
//       K range, one 32x32x16 MFMA tile, so that the 2 MB router weight is
//       spread over ~256 workgroups (E/32 expert blocks x K ranges) instead
//       of a handful of 128-token tiles. Each lane loads its token row's
//       64-byte runs (four 16-byte loads per 64-deep step) and, for the same
//       permuted contraction order, the matching 16-byte slots of the packed
//       weight fragments; every load of the K range is in flight before the
//       first MFMA.
//  2. select: sums each token's partials in split order (fixed order:
//     deterministic), applies the sigmoid and the bias, and picks the top 8
//     by eight rounds of an arg-max on (key descending, id ascending); the
//     ids are emitted ascending with w = s / sum(s).
//     - Few tokens: one wavefront per token. Lane l holds experts 4l .. 4l+3,
//       so each split's partials of a token arrive with one 16-byte load per
//       lane (1 KB per wave instruction). A round takes the wave-wide maximum
//       of the keys (mapped to order-preserving unsigned integers) with DPP
//       max steps, then the lowest expert id that holds it as a second DPP
//       maximum (of 256 - id over the lanes' candidates equal to the key
//       maximum). Only that candidate is retired, so equal keys are taken in
//       ascending id order over the rounds. A winner's output slot is its
//       rank among the winners by id (popcounts of per-slot ballots), and the
//       eight scores are summed in that order.
//     - Many tokens: the same rounds with one 16-lane DPP row per token, four
//       tokens per wavefront (route_select_rows_kernel). At these sizes a
//       wave per token was bound by its vector instructions, not by its
//       loads: about 600 per token, mostly wave-wide reduction steps that do
//       one useful compare per lane; a row per token issues about 260.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

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

// sigmoid(z) = 1 / (1 + 2^(-z log2(e))) on the hardware exp2 and reciprocal
// (each within about 1 ulp): about 3e-7 absolute error in s, against the 1e-6
// margin within which two biased scores count as a near tie. An IEEE divide
// and a range-reduced expf cost about 18 instructions per score here, and the
// selection runs 256 of them per token.
__device__ __forceinline__ float sigmoid_hw(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504f));
}

}  // namespace

// Token counts up to this take the few-token logits kernel.
constexpr int64_t kSmallT = 256;

int route_splits(int64_t T, int d) {
  int ks = 1;
  if (T <= kSmallT) {
    // (T/32) x (E/32) x splits workgroups with E up to 256; each split's K
    // range a multiple of 64
    const int64_t tiles = ((T + 31) / 32) * 8;
    while ((d / 64) % (ks * 2) == 0 && tiles * ks * 2 <= kTargetWGs && ks * 2 <= kMaxSplits)
      ks *= 2;
    return ks;
  }
  const int64_t tiles = (T + kTokTile - 1) / kTokTile;
  // each split's K range must stay a multiple of 64 (the GEMM's stage pair)
  while ((d / 64) % (ks * 2) == 0 && tiles * ks * 2 <= kTargetWGs && ks * 2 <= kMaxSplits) ks *= 2;
  return ks;
}

size_t route_workspace_bytes(int64_t T, int d, int E) {
  return static_cast<size_t>(route_splits(T, d)) * static_cast<size_t>(T) * E * sizeof(float);
}

// Few-token logits: one wavefront per (32 tokens, 32 experts, K range z).
// Lane l owns token row t0 + l%32 and lane group g = l/32. For 64-deep step m
// it loads the 64 bytes k0 + 64m + 32g .. +32 of its row; MFMA c of the step
// then takes elements 8c .. 8c+7 of them, i.e. lane group g, element v of
// MFMA c stands for k = k0 + 64m + 32g + 8c + v. The weight operand uses the
// same order: that k lives in packed fragment kb = k / 16 at slot
// (l%32) + 32 ((k / 8) % 2) = (l%32) + 32 (c % 2). The dot products are
// unchanged by the common permutation.
__global__ __launch_bounds__(64) void route_logits_small_kernel(
    const bf16_t* __restrict__ x, const char* __restrict__ w_r, int T, int d, int E, int kc,
    float* __restrict__ zp) {
  constexpr int FRAG = 1024;
  const int lane = threadIdx.x;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32, z = blockIdx.z;
  const int lr = lane & 31, g = lane >> 5;
  const int t = min(t0 + lr, T - 1);  // rows past T re-read row T-1 and are not stored
  const int k0 = z * kc;
  const char* xa = reinterpret_cast<const char*>(x) + (static_cast<int64_t>(t) * d + k0 + 32 * g) * 2;
  // packed weights: fragment (nb, kb) at (nb * d/16 + kb) * 1 KB; slot l' at l' * 16 B
  const int nb = blockIdx.y;
  const char* wb = w_r + (static_cast<int64_t>(nb) * (d / 16) + k0 / 16 + 2 * g) * FRAG + lr * 16;
  f32x16 acc = f32x16{};
  for (int m0 = 0; m0 < kc; m0 += 256) {  // four 64-deep steps in flight at a time
    const int nm = min(4, (kc - m0) / 64);
    u32x4 a[4][4], b[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m < nm) {
        const int mm = m0 / 64 + m;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          a[m][c] = ld16(xa + (64 * mm + 8 * c) * 2);
          b[m][c] = ld16(wb + (4 * mm + c / 2) * static_cast<int64_t>(FRAG) + (c % 2) * 512);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (m < nm)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b[m][c]),
                                                        __builtin_bit_cast(bf16x8, a[m][c]), acc,
                                                        0, 0, 0);
  }
  // lane holds token t0 + lr and experts e0 + 8q + 4g + r (q, r = 0..3)
  if (t0 + lr >= T) return;
  float* zr = zp + (static_cast<int64_t>(z) * T + t0 + lr) * E;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = e0 + 8 * q + 4 * g;
    if ((E & 3) == 0 && e + 3 < E) {
      st16(zr + e, u32x4{__float_as_uint(acc[4 * q]), __float_as_uint(acc[4 * q + 1]),
                         __float_as_uint(acc[4 * q + 2]), __float_as_uint(acc[4 * q + 3])});
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (e + r < E) zr[e + r] = acc[4 * q + r];
    }
  }
}

// Top-8 of one token held by one wavefront: lane l holds experts 4l + c
// (c = 0..3) as order-preserving keys of s + b (0 for experts past E) and
// their scores s. Writes the ids ascending to idx[0..7] and w = s / sum(s) to
// w[0..7]; sc8 is this wave's 8-float LDS staging.
__device__ __forceinline__ void select_top8(uint32_t (&key)[4], const float (&sc)[4], int lane,
                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                            float* sc8) {
  const int eb = 4 * lane;
  // Eight rounds; a round takes the wave-wide maximum key m, then the lowest
  // expert id holding it as a second wave-wide maximum, of 256 - e over each
  // lane's candidates equal to m (all in VALU/DPP: no ballot chains on the
  // CU's one scalar unit, which all the resident waves share). The owner
  // lane retires the winner and flags it.
  uint32_t won = 0;  // bit c: expert 4 lane + c was selected
#pragma unroll
  for (int round = 0; round < 8; ++round) {
    const uint32_t m = wave_umax(max(max(key[0], key[1]), max(key[2], key[3])));
    uint32_t cand = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      cand = max(cand, key[c] == m ? 256u - static_cast<uint32_t>(eb + c) : 0u);
    const int e = 256 - static_cast<int>(wave_umax(cand));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool hit = eb + c == e;  // only the owner lane's slot matches
      key[c] = hit ? 0u : key[c];
      won |= hit ? 1u << c : 0u;
    }
  }
  // Rank of a winner among the winners by id: the winners of the lanes below
  // plus this lane's winners at lower slots.
  const uint64_t below = (1ull << lane) - 1ull;
  int r = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    r += __popcll(__builtin_amdgcn_ballot_w64((won >> c) & 1u) & below);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if ((won >> c) & 1u) {
      idx[r] = eb + c;
      sc8[r] = sc[c];
      ++r;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < 8) {
    float sum = 0.f;  // in ascending id order
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += sc8[i];
    w[lane] = sc8[lane] / sum;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int SPLITS>
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ zp,
                                                           const float* __restrict__ bias,
                                                           int64_t T, int E,
                                                           int32_t* __restrict__ idx_out,
                                                           float* __restrict__ w_out) {
  __shared__ float s_sc[4][8];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  // one token per wave: four per workgroup, or one for few tokens
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + wave;
  if (t >= T) return;
  const int64_t split_stride = T * E;
  // candidates of this lane: experts 4 lane + c
  const int eb = 4 * lane;
  // All partial logits are loaded before any is added (independent loads in
  // flight together), then summed in split order. With E a multiple of 4 each
  // split is one 16-byte load per lane (lanes past E re-read the last four
  // experts and are masked below); otherwise four element loads, clamped the
  // same way. The loads are unconditional: a load under a per-lane condition
  // would become a branch with its own wait.
  float part[SPLITS][4];
  if ((E & 3) == 0) {
    const int ev = min(eb, E - 4);
#pragma unroll
    for (int y = 0; y < SPLITS; ++y) {
      const u32x4 v = ld16(zp + y * split_stride + t * E + ev);
#pragma unroll
      for (int c = 0; c < 4; ++c) part[y][c] = __uint_as_float(v[c]);
    }
  } else {
#pragma unroll
    for (int y = 0; y < SPLITS; ++y)
#pragma unroll
      for (int c = 0; c < 4; ++c) part[y][c] = zp[y * split_stride + t * E + min(eb + c, E - 1)];
  }
  float sc[4];
  uint32_t key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = eb + c;
    float z = 0.f;
#pragma unroll
    for (int y = 0; y < SPLITS; ++y) z += part[y][c];
    sc[c] = sigmoid_hw(z);
    key[c] = e < E ? order_key(sc[c] + bias[min(e, E - 1)]) : 0u;
  }
  select_top8(key, sc, lane, idx_out + t * 8, w_out + t * 8, s_sc[wave]);
}

// Many tokens: four tokens per wavefront, one 16-lane DPP row each (a round's
// maxima stay inside the row: four DPP steps, every lane of the row holds the
// result, no lane read). Lane j of a row holds experts 64q + 4j + c
// (q, c = 0..3), so each split's partials of a token arrive as four 16-byte
// loads per lane, each load instruction covering 256 contiguous bytes of the
// row. A wave per token (the kernel above) spends most of its instructions on
// wave-wide reductions whose steps do one useful compare per lane; here a
// round costs about 90 instructions for four tokens. Same arithmetic and
// order as route_select_kernel: the partials summed in split order, then
// sigmoid, bias, the order-preserving key, ties to the lower id, the eight
// scores summed in ascending id order.
__device__ __forceinline__ uint32_t row_umax(uint32_t v) {
  v = max(v, dpp_or0<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_or0<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_or0<0x141, 0xF>(v));  // row_half_mirror: the 8-lane half
  v = max(v, dpp_or0<0x140, 0xF>(v));  // row_mirror: the 16-lane row
  return v;
}

__device__ __forceinline__ void cex(int& a, int& b) {
  const int lo = min(a, b), hi = max(a, b);
  a = lo;
  b = hi;
}

template <int SPLITS>
__global__ __launch_bounds__(256) void route_select_rows_kernel(const float* __restrict__ zp,
                                                                const float* __restrict__ bias,
                                                                int64_t T, int E,
                                                                int32_t* __restrict__ idx_out,
                                                                float* __restrict__ w_out) {
  __shared__ float s_bias[256];
  __shared__ float s_sc[16][256];  // the scores of the workgroup's 16 tokens
  const int lane = threadIdx.x % kWave;
  const int slot = threadIdx.x / 16;  // token of the workgroup: wave * 4 + row
  const int j = lane & 15;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16 + slot;
  const int64_t t = min(t0, T - 1);  // rows past T redo token T-1 and store nothing
  s_bias[threadIdx.x] = bias[min(static_cast<int>(threadIdx.x), E - 1)];
  __syncthreads();
  const int64_t split_stride = T * E;
  // z summed in split order; the loads of up to eight splits are in flight
  // together (all of them for the split counts the prefill sizes use)
  constexpr int CH = SPLITS < 8 ? SPLITS : 8;
  float z[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
#pragma unroll
  for (int y0 = 0; y0 < SPLITS; y0 += CH) {
    float part[CH][16];
    if ((E & 3) == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ev = min(64 * q + 4 * j, E - 4);  // lanes past E re-read the last four
#pragma unroll
        for (int y = 0; y < CH; ++y) {
          const u32x4 v = ld16(zp + (y0 + y) * split_stride + t * E + ev);
#pragma unroll
          for (int c = 0; c < 4; ++c) part[y][4 * q + c] = __uint_as_float(v[c]);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int y = 0; y < CH; ++y)
            part[y][4 * q + c] =
                zp[(y0 + y) * split_stride + t * E + min(64 * q + 4 * j + c, E - 1)];
    }
#pragma unroll
    for (int y = 0; y < CH; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] += part[y][i];
  }
  float* srow = s_sc[slot];
  uint32_t key[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int eb = 64 * q + 4 * j;
    const f32x4 b4 = *reinterpret_cast<const f32x4*>(s_bias + eb);
    f32x4 s4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s4[c] = sigmoid_hw(z[4 * q + c]);
      key[4 * q + c] = eb + c < E ? order_key(s4[c] + b4[c]) : 0u;
    }
    *reinterpret_cast<f32x4*>(srow + eb) = s4;
  }
  // Eight rounds: the row's maximum key m; the lowest expert id holding it
  // (each lane's lowest slot holding m, slots being in id order within a
  // lane, then the row maximum of 256 - id); the owner lane retires it.
  int win[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint32_t lm = key[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) lm = max(lm, key[i]);
    const uint32_t m = row_umax(lm);
    int lo = 16;
#pragma unroll
    for (int i = 15; i >= 0; --i) lo = key[i] == m ? i : lo;
    const uint32_t cand =
        lo < 16 ? 256u - static_cast<uint32_t>(64 * (lo >> 2) + 4 * j + (lo & 3)) : 0u;
    const int e = 256 - static_cast<int>(row_umax(cand));
    win[r] = e;
    // the winner's slot in its owner lane; 16 or more in every other lane
    const int own = (4 * (e >> 6) + (e & 3)) | ((((e >> 2) & 15) ^ j) << 4);
#pragma unroll
    for (int i = 0; i < 16; ++i) key[i] = own == i ? 0u : key[i];
  }
  // ids ascending (a 19-comparator network on the row-uniform winners)
  cex(win[0], win[2]); cex(win[1], win[3]); cex(win[4], win[6]); cex(win[5], win[7]);
  cex(win[0], win[4]); cex(win[1], win[5]); cex(win[2], win[6]); cex(win[3], win[7]);
  cex(win[0], win[1]); cex(win[2], win[3]); cex(win[4], win[5]); cex(win[6], win[7]);
  cex(win[2], win[4]); cex(win[3], win[5]);
  cex(win[1], win[4]); cex(win[3], win[6]);
  cex(win[1], win[2]); cex(win[3], win[4]); cex(win[5], win[6]);
  // the scores were written by other lanes of this wavefront
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float sum = 0.f;  // in ascending id order
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += srow[win[i]];
  int mine = win[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mine = j == i ? win[i] : mine;
  if (j < 8 && t0 < T) {
    idx_out[t0 * 8 + j] = mine;
    w_out[t0 * 8 + j] = srow[mine] / sum;
  }
}

void launch_route(const void* x, const void* w_r, const float* bias, int64_t T, int d, int E,
                  int32_t* idx, float* w, void* workspace, int num_cus, hipStream_t s) {
  const int splits = route_splits(T, d);
  float* zp = static_cast<float*>(workspace);
  if (T <= kSmallT) {
    const dim3 lg(static_cast<unsigned>((T + 31) / 32), static_cast<unsigned>((E + 31) / 32),
                  static_cast<unsigned>(splits));
    route_logits_small_kernel<<<lg, 64, 0, s>>>(static_cast<const bf16_t*>(x),
                                                static_cast<const char*>(w_r), static_cast<int>(T),
                                                d, E, d / splits, zp);
  } else {
    launch_gemm_nt_f32_splitk(x, T, d, w_r, E, splits, zp, num_cus, s);
  }
  if (T > kSmallT) {  // sixteen tokens per 256-thread workgroup
    const dim3 grid(static_cast<unsigned>((T + 15) / 16));
    switch (splits) {  // route_splits returns a power of two <= kMaxSplits
      case 1: route_select_rows_kernel<1><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w); break;
      case 2: route_select_rows_kernel<2><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w); break;
      case 4: route_select_rows_kernel<4><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w); break;
      case 8: route_select_rows_kernel<8><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w); break;
      default:
        route_select_rows_kernel<kMaxSplits><<<grid, 256, 0, s>>>(zp, bias, T, E, idx, w);
        break;
    }
    return;
  }
  // few tokens: one token per 64-thread workgroup, so that the partial
  // logits are read by as many CUs as there are tokens
  const bool spread = T <= kSmallT;
  const dim3 grid(static_cast<unsigned>(spread ? T : (T + 3) / 4));
  const int nt = spread ? kWave : 256;
  switch (splits) {  // route_splits returns a power of two <= kMaxSplits
    case 1: route_select_kernel<1><<<grid, nt, 0, s>>>(zp, bias, T, E, idx, w); break;
    case 2: route_select_kernel<2><<<grid, nt, 0, s>>>(zp, bias, T, E, idx, w); break;
    case 4: route_select_kernel<4><<<grid, nt, 0, s>>>(zp, bias, T, E, idx, w); break;
    case 8: route_select_kernel<8><<<grid, nt, 0, s>>>(zp, bias, T, E, idx, w); break;
    default: route_select_kernel<kMaxSplits><<<grid, nt, 0, s>>>(zp, bias, T, E, idx, w); break;
  }
}

}  // namespace mf
