// Stable counting sort of routing slots by expert, and the row gather into
// the expert-contiguous layout ("「赤兔」Chitu 框架深度解读（七）：MoE":
// token_permutation; tokens laid out contiguously by expert id).
//
// Deterministic without ordered atomics. Tokens are cut into blocks of 256
// (one 256-thread workgroup, four waves of 64 tokens):
//   1. mask:    each wave builds, per local expert, the 64-bit mask of its
//               tokens routed there (LDS atomicOr: an OR is order-free), and
//               the workgroup writes the masks and the block's count per expert.
//   2. scan:    one workgroup turns the counts into per-(block, expert) bases,
//               the per-expert totals and the exclusive offsets.
//   3. scatter: a slot's row is offsets[e] + base[block][e] + the popcounts of
//               the earlier waves' masks + the popcount of its own wave's mask
//               below its lane, i.e. the number of earlier tokens routed to e.
//   4. gather:  x_perm[r] = x[src_token[r]], 16-byte copies.
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int kBlockTok = 256;
constexpr int kWaves = 4;
constexpr int kMaxLocal = 256;

struct Workspace {
  int32_t* cnt;       // [B][e_count]
  int32_t* base;      // [B][e_count]
  uint64_t* masks;    // [B][4][e_count]
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

Workspace carve(void* ws, int64_t B, int e_count) {
  char* p = static_cast<char*>(ws);
  Workspace w;
  w.cnt = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * B * e_count);
  w.base = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * B * e_count);
  w.masks = reinterpret_cast<uint64_t*>(p);
  return w;
}

}  // namespace

size_t permute_workspace_bytes(int64_t T, int e_count) {
  const int64_t B = (T + kBlockTok - 1) / kBlockTok;
  return 2 * align256(sizeof(int32_t) * B * e_count) +
         align256(sizeof(uint64_t) * B * kWaves * e_count) + 256;
}

__global__ __launch_bounds__(256) void permute_mask_kernel(const int32_t* __restrict__ idx,
                                                           int64_t T, int k, int e_begin,
                                                           int e_count, Workspace ws) {
  __shared__ unsigned long long m[kWaves][kMaxLocal];
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  for (int i = tid; i < kWaves * kMaxLocal; i += 256) (&m[0][0])[i] = 0ull;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlockTok + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j] - e_begin;
      if (e >= 0 && e < e_count) atomicOr(&m[wave][e], 1ull << lane);
    }
  }
  __syncthreads();
  const int64_t b = blockIdx.x;
  for (int e = tid; e < e_count; e += 256) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      c += __popcll(m[w][e]);
      ws.masks[(b * kWaves + w) * e_count + e] = m[w][e];
    }
    ws.cnt[b * e_count + e] = c;
  }
}

__global__ __launch_bounds__(256) void permute_scan_kernel(int64_t B, int e_count, Workspace ws,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int sc[256];
  const int e = threadIdx.x;
  int running = 0;
  if (e < e_count) {
    int64_t b = 0;
    for (; b + 4 <= B; b += 4) {
      int c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) c[u] = ws.cnt[(b + u) * e_count + e];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ws.base[(b + u) * e_count + e] = running;
        running += c[u];
      }
    }
    for (; b < B; ++b) {
      const int c = ws.cnt[b * e_count + e];
      ws.base[b * e_count + e] = running;
      running += c;
    }
    counts[e] = running;
  }
  sc[e] = e < e_count ? running : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 entries
  for (int off = 1; off < 256; off <<= 1) {
    const int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < e_count) offsets[e + 1] = sc[e];
  if (e == 0) offsets[0] = 0;
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int e_begin, int e_count, Workspace ws,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ src_token,
    int32_t* __restrict__ inv_pos) {
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t b = blockIdx.x;
  const int64_t t = b * kBlockTok + tid;
  if (t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j] - e_begin;
    int pos = -1;
    if (e >= 0 && e < e_count) {
      pos = offsets[e] + ws.base[b * e_count + e];
      for (int w = 0; w < wave; ++w) pos += __popcll(ws.masks[(b * kWaves + w) * e_count + e]);
      pos += __popcll(ws.masks[(b * kWaves + wave) * e_count + e] & below);
      src_token[pos] = static_cast<int32_t>(t);
    }
    inv_pos[t * k + j] = pos;
  }
}

// x_perm[r] = x[src_token[r]] for r < min(offsets[e_count], max_rows).
__global__ __launch_bounds__(256) void permute_gather_kernel(
    const char* __restrict__ x, int64_t T, int64_t row_bytes, const int32_t* __restrict__ src_token,
    const int32_t* __restrict__ offsets, int e_count, int64_t max_rows, char* __restrict__ x_perm) {
  int64_t S = offsets[e_count];
  S = S < 0 ? 0 : (S > max_rows ? max_rows : S);
  const int64_t nch = row_bytes / 16;
  const int64_t total = S * nch;
  constexpr int U = 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * U;
  for (int64_t base = (static_cast<int64_t>(blockIdx.x) * blockDim.x) * U + threadIdx.x;
       base < total; base += stride) {
    u32x4 v[U];
    int64_t dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t L = base + static_cast<int64_t>(u) * blockDim.x;
      dst[u] = -1;
      if (L < total) {
        const int64_t r = L / nch, c = L - r * nch;
        int64_t t = src_token[r];
        t = t < 0 ? 0 : (t >= T ? T - 1 : t);
        v[u] = ld16(x + t * row_bytes + c * 16);
        dst[u] = r * row_bytes + c * 16;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst[u] >= 0) st16(x_perm + dst[u], v[u]);
  }
}

void launch_permute(const int32_t* idx, int64_t T, int k, int e_begin, int e_count,
                    const void* x, int64_t row_bytes, void* x_perm, int32_t* counts,
                    int32_t* offsets, int32_t* src_token, int32_t* inv_pos, void* workspace,
                    hipStream_t s) {
  const int64_t B = (T + kBlockTok - 1) / kBlockTok;
  Workspace ws = carve(workspace, B, e_count);
  if (B > 0)
    permute_mask_kernel<<<dim3(static_cast<unsigned>(B)), 256, 0, s>>>(idx, T, k, e_begin,
                                                                       e_count, ws);
  permute_scan_kernel<<<1, 256, 0, s>>>(B, e_count, ws, counts, offsets);
  if (B > 0)
    permute_scatter_kernel<<<dim3(static_cast<unsigned>(B)), 256, 0, s>>>(
        idx, T, k, e_begin, e_count, ws, offsets, src_token, inv_pos);
  if (x != nullptr && B > 0) {
    const int64_t max_rows = T * k;
    const int64_t items = max_rows * (row_bytes / 16);
    int64_t grid = (items + 256 * 4 - 1) / (256 * 4);
    if (grid > 2048) grid = 2048;
    permute_gather_kernel<<<dim3(static_cast<unsigned>(grid)), 256, 0, s>>>(
        static_cast<const char*>(x), T, row_bytes, src_token, offsets, e_count, max_rows,
        static_cast<char*>(x_perm));
  }
}

}  // namespace mf
