// Stable counting sort of routing slots by expert, and the row gather into
// the expert-contiguous layout ("「赤兔」Chitu 框架深度解读（七）：MoE":
// token_permutation; tokens laid out contiguously by expert id).
//
// Deterministic without ordered atomics. Tokens are cut into blocks of 256
// (one 256-thread workgroup, four waves of 64 tokens):
//   1. count:   each workgroup counts its block's slots per local expert (LDS
//               integer atomics: order-free) and writes the counts.
//   2. place:   each workgroup takes, per expert, the sum of the earlier
//               blocks' counts and the total over all blocks (reading the
//               B x e_count counts itself while that table is small, else
//               from a one-workgroup scan pass), the exclusive offsets from
//               an LDS scan of the totals, and per wave and expert the 64-bit
//               mask of its tokens routed there (LDS atomicOr). A slot's row
//               is offsets[e] + (earlier blocks' count) + the popcounts of
//               the earlier waves' masks + the popcount of its own wave's
//               mask below its lane, i.e. the number of earlier tokens routed
//               to e.
//   3. gather:  x_perm[r] = x[src_token[r]], 16-byte copies (only when x is
//               given).
#include <mutex>

#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int kBlockTok = 256;
constexpr int kWaves = 4;
constexpr int kMaxLocal = 256;
// largest count table (blocks x local experts) each workgroup of the place
// pass scans itself; beyond it one workgroup scans it once
constexpr int64_t kSelfScanMax = 16384;

struct Workspace {
  int32_t* cnt;       // [B][e_count] slots per block and expert
  int32_t* base;      // [B][e_count] earlier blocks' slots (scan pass only)
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

Workspace carve(void* ws, int64_t B, int e_count) {
  char* p = static_cast<char*>(ws);
  Workspace w;
  w.cnt = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * B * e_count);
  w.base = reinterpret_cast<int32_t*>(p);
  return w;
}

// inclusive sum over the 256 entries of v (LDS, all 256 threads take part)
__device__ __forceinline__ void block_inclusive_scan(int* v) {
  const int e = threadIdx.x;
  for (int off = 1; off < 256; off <<= 1) {
    const int x = e >= off ? v[e - off] : 0;
    __syncthreads();
    v[e] += x;
    __syncthreads();
  }
}

}  // namespace

size_t permute_workspace_bytes(int64_t T, int e_count) {
  const int64_t B = (T + kBlockTok - 1) / kBlockTok;
  return 2 * align256(sizeof(int32_t) * B * e_count) + 256;
}

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                            int64_t T, int k, int e_begin,
                                                            int e_count, Workspace ws) {
  __shared__ int c[kMaxLocal];
  const int tid = threadIdx.x;
  c[tid] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlockTok + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j] - e_begin;
      if (e >= 0 && e < e_count) atomicAdd(&c[e], 1);
    }
  }
  __syncthreads();
  if (tid < e_count) ws.cnt[blockIdx.x * static_cast<int64_t>(e_count) + tid] = c[tid];
}

// One workgroup: per-(block, expert) bases, per-expert totals and the offsets
// (for count tables too large for every workgroup of the place pass to scan).
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
  block_inclusive_scan(sc);
  if (e < e_count) offsets[e + 1] = sc[e];
  if (e == 0) offsets[0] = 0;
}

// With a single block of tokens (decode) the totals are the block's own
// bitmap popcounts, so the count pass is skipped (ONE_BLOCK: one launch).
template <bool SELF_SCAN, bool ONE_BLOCK = false>
__global__ __launch_bounds__(256) void permute_place_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int e_begin, int e_count, int64_t B,
    Workspace ws, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ src_token, int32_t* __restrict__ inv_pos) {
  __shared__ unsigned long long m[kWaves][kMaxLocal];
  __shared__ int row0[kMaxLocal];  // first row of this block's slots, per expert
  __shared__ int sc[256];
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t b = blockIdx.x;
  for (int i = tid; i < kWaves * kMaxLocal; i += 256) (&m[0][0])[i] = 0ull;
  const int64_t t = b * kBlockTok + tid;
  int ex[8];  // k <= 8; slots past k stay -1 (not local)
  if constexpr (ONE_BLOCK) {  // bitmaps first: they give the totals
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ex[j] = -1;
      if (t < T && j < k) {
        ex[j] = idx[t * k + j] - e_begin;
        if (ex[j] >= 0 && ex[j] < e_count) atomicOr(&m[wave][ex[j]], 1ull << lane);
      }
    }
    __syncthreads();
    int total = 0;
    if (tid < e_count) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) total += __popcll(m[w][tid]);
    }
    sc[tid] = tid < e_count ? total : 0;
    __syncthreads();
    block_inclusive_scan(sc);
    if (tid < e_count) {
      row0[tid] = sc[tid] - total;
      counts[tid] = total;
      offsets[tid + 1] = sc[tid];
    }
    if (tid == 0) offsets[0] = 0;
  } else if constexpr (SELF_SCAN) {
    // per expert (thread e): earlier blocks' slots and the total
    int before = 0, total = 0;
    if (tid < e_count) {
      int64_t q = 0;
      for (; q + 8 <= B; q += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = ws.cnt[(q + u) * e_count + tid];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          before += q + u < b ? c[u] : 0;
          total += c[u];
        }
      }
      for (; q < B; ++q) {
        const int c = ws.cnt[q * e_count + tid];
        before += q < b ? c : 0;
        total += c;
      }
    }
    sc[tid] = tid < e_count ? total : 0;
    __syncthreads();
    block_inclusive_scan(sc);
    if (tid < e_count) {
      row0[tid] = sc[tid] - total + before;
      if (b == 0) {
        counts[tid] = total;
        offsets[tid + 1] = sc[tid];
      }
    }
    if (b == 0 && tid == 0) offsets[0] = 0;
  } else {
    if (tid < e_count) row0[tid] = offsets[tid] + ws.base[b * e_count + tid];
  }
  __syncthreads();
  if constexpr (!ONE_BLOCK) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ex[j] = -1;
      if (t < T && j < k) {
        ex[j] = idx[t * k + j] - e_begin;
        if (ex[j] >= 0 && ex[j] < e_count) atomicOr(&m[wave][ex[j]], 1ull << lane);
      }
    }
    __syncthreads();
  }
  if (t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const int e = ex[j];
    int pos = -1;
    if (e >= 0 && e < e_count) {
      pos = row0[e] + __popcll(m[wave][e] & below);
      for (int w = 0; w < wave; ++w) pos += __popcll(m[w][e]);
      src_token[pos] = static_cast<int32_t>(t);
    }
    inv_pos[t * k + j] = pos;
  }
}

// Masked layout (the decode variant: fixed per-expert capacity, no prefix
// over experts). Local expert e owns rows [e*cap, (e+1)*cap); slot (t, j)
// routed to e goes to row e*cap + rank, rank = the number of earlier tokens
// routed to e (earlier blocks' counts + popcounts of the block's wave masks,
// as in the contiguous placement); a slot whose rank reaches cap is dropped
// (pos -1). counts[e] = min(total, cap). With one block of tokens the totals
// come from the block's own masks and the count pass is skipped.
template <bool ONE_BLOCK>
__global__ __launch_bounds__(256) void dispatch_masked_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int e_begin, int e_count, int cap,
    int64_t B, const int32_t* __restrict__ cnt, int32_t* __restrict__ counts,
    int32_t* __restrict__ row_index, int32_t* __restrict__ pos) {
  __shared__ unsigned long long m[kWaves][kMaxLocal];
  __shared__ int rank0[kMaxLocal];  // earlier blocks' slots, per expert
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t b = blockIdx.x;
  for (int i = tid; i < kWaves * kMaxLocal; i += 256) (&m[0][0])[i] = 0ull;
  __syncthreads();
  const int64_t t = b * kBlockTok + tid;
  int ex[8];  // k <= 8; slots past k stay -1 (not local)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ex[j] = -1;
    if (t < T && j < k) {
      ex[j] = idx[t * k + j] - e_begin;
      if (ex[j] >= 0 && ex[j] < e_count) atomicOr(&m[wave][ex[j]], 1ull << lane);
    }
  }
  __syncthreads();
  if (tid < e_count) {
    int before = 0, total = 0;
    if constexpr (ONE_BLOCK) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) total += __popcll(m[w][tid]);
    } else {
      for (int64_t q = 0; q < B; ++q) {
        const int c = cnt[q * e_count + tid];
        before += q < b ? c : 0;
        total += c;
      }
    }
    rank0[tid] = before;
    if (b == 0) counts[tid] = min(total, cap);
  }
  __syncthreads();
  if (t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const int e = ex[j];
    int p = -1;
    if (e >= 0 && e < e_count) {
      int r = rank0[e] + __popcll(m[wave][e] & below);
      for (int w = 0; w < wave; ++w) r += __popcll(m[w][e]);
      if (r < cap) {
        p = e * cap + r;
        row_index[p] = static_cast<int32_t>(t);
      }
    }
    pos[t * k + j] = p;
  }
}

void launch_dispatch_masked(const int32_t* idx, int64_t T, int k, int e_begin, int e_count,
                            int cap, int32_t* counts, int32_t* row_index, int32_t* pos,
                            void* workspace, hipStream_t s) {
  const int64_t B = (T + kBlockTok - 1) / kBlockTok;
  if (B <= 1) {  // also T == 0: one block writes zero counts
    dispatch_masked_kernel<true><<<1, 256, 0, s>>>(idx, T, k, e_begin, e_count, cap, 1, nullptr,
                                                   counts, row_index, pos);
    return;
  }
  Workspace ws = carve(workspace, B, e_count);
  const dim3 grid(static_cast<unsigned>(B));
  permute_count_kernel<<<grid, 256, 0, s>>>(idx, T, k, e_begin, e_count, ws);
  dispatch_masked_kernel<false><<<grid, 256, 0, s>>>(idx, T, k, e_begin, e_count, cap, B, ws.cnt,
                                                     counts, row_index, pos);
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
  const dim3 grid(static_cast<unsigned>(B));
  if (B == 1) {  // one token block: a single launch
    permute_place_kernel<true, true><<<grid, 256, 0, s>>>(idx, T, k, e_begin, e_count, B, ws,
                                                          counts, offsets, src_token, inv_pos);
  } else if (B > 0 && B * e_count <= kSelfScanMax) {
    permute_count_kernel<<<grid, 256, 0, s>>>(idx, T, k, e_begin, e_count, ws);
    permute_place_kernel<true><<<grid, 256, 0, s>>>(idx, T, k, e_begin, e_count, B, ws, counts,
                                                    offsets, src_token, inv_pos);
  } else {
    // also for T == 0: zero counts and offsets
    if (B > 0) permute_count_kernel<<<grid, 256, 0, s>>>(idx, T, k, e_begin, e_count, ws);
    permute_scan_kernel<<<1, 256, 0, s>>>(B, e_count, ws, counts, offsets);
    if (B > 0)
      permute_place_kernel<false><<<grid, 256, 0, s>>>(idx, T, k, e_begin, e_count, B, ws,
                                                       counts, offsets, src_token, inv_pos);
  }
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

// ---- the allocation-free variant: a static device scratch array -----------
//
// For callers that cannot allocate (code under graph capture, serving loops):
// the count tables live in a file-scope device array instead of a caller
// workspace. Every GPU the library runs on holds its own copy of the array
// until the process ends; its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// handed to kernels. The kernels write every count-table entry they later read
// (nothing must start at zero), so no clearing is needed; calls that overlap
// on one GPU share the array and race.

namespace {

constexpr int kMaxDevices = 256;
__device__ __align__(256) char scratch[kPermuteScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int permute_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return -1;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

}  // namespace mf
