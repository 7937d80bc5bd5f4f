// C ABI of the FFN hot path: argument validation, then kernel launches on the
// caller's stream. Nothing here allocates, synchronises or keeps state.
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "moeffn.h"

namespace {

constexpr int64_t kI32Max = 2147483647LL;

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

int finish() { return hipGetLastError() == hipSuccess ? MF_OK : MF_EHIP; }

hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* mf_version(void) { return "moeffn 0.1.0 (gfx950)"; }

const char* mf_status_string(int status) {
  switch (status) {
    case MF_OK: return "MF_OK";
    case MF_EINVAL: return "MF_EINVAL: invalid argument";
    case MF_EUNSUPPORTED: return "MF_EUNSUPPORTED: valid arguments outside what the kernels implement";
    case MF_EHIP: return "MF_EHIP: HIP runtime error at launch";
    default: return "unknown status";
  }
}

int rmsnorm(const void* x, const void* gamma, void* y, int64_t T, int32_t d, float eps,
            int32_t dtype, void* stream) {
  if (T < 0 || d <= 0 || !(eps >= 0.f) || !isfinite(eps)) return MF_EINVAL;
  if (dtype != MF_BF16 && dtype != MF_F32) return MF_EINVAL;
  if (d % 64 != 0 || d > 8192) return MF_EUNSUPPORTED;
  if (T == 0) return MF_OK;  // zero-size buffers may be NULL
  if (!x || !gamma || !y) return MF_EINVAL;
  if (!a16(x) || !a16(gamma) || !a16(y)) return MF_EUNSUPPORTED;
  if ((T + 3) / 4 > 0xFFFFFFFFLL) return MF_EUNSUPPORTED;
  mf::launch_rmsnorm(x, gamma, y, T, d, eps, dtype == MF_BF16, S(stream));
  return finish();
}

int rmsnorm_quantize_fp8(const void* x, const void* gamma, void* y, void* q, float* scales,
                         int64_t T, int32_t d, float eps, void* stream) {
  if (T < 0 || d <= 0 || !(eps >= 0.f) || !isfinite(eps)) return MF_EINVAL;
  if (d % 128 != 0 || d > 8192) return MF_EUNSUPPORTED;
  if (T == 0) return MF_OK;  // zero-size buffers may be NULL
  if (!x || !gamma || !y || !q || !scales) return MF_EINVAL;
  if (!a16(x) || !a16(gamma) || !a16(y) || reinterpret_cast<uintptr_t>(q) % 8 != 0 ||
      reinterpret_cast<uintptr_t>(scales) % 4 != 0)
    return MF_EUNSUPPORTED;
  if ((T + 3) / 4 > 0xFFFFFFFFLL) return MF_EUNSUPPORTED;
  mf::launch_rmsnorm(x, gamma, y, T, d, eps, true, S(stream), static_cast<uint8_t*>(q), scales);
  return finish();
}

size_t packed_weights_bytes(int64_t groups, int32_t N, int32_t K, int32_t dtype) {
  if (groups < 0 || N <= 0 || K <= 0) return 0;
  if (dtype == MF_BF16 && K % 16 == 0) return mf::packed_bytes(groups, N, K, false);
  if (dtype == MF_FP8_E4M3 && K % 128 == 0) return mf::packed_bytes(groups, N, K, true);
  return 0;
}

int pack_weights(const void* src, void* dst, int64_t groups, int32_t N, int32_t K, int32_t dtype,
                 void* stream) {
  if (groups < 0 || N <= 0 || K <= 0) return MF_EINVAL;
  if (dtype != MF_BF16 && dtype != MF_FP8_E4M3) return MF_EINVAL;
  if ((dtype == MF_BF16 && K % 16 != 0) || (dtype == MF_FP8_E4M3 && K % 128 != 0))
    return MF_EUNSUPPORTED;
  if (groups == 0) return MF_OK;
  if (!src || !dst) return MF_EINVAL;
  if (!a16(src) || !a16(dst)) return MF_EUNSUPPORTED;
  mf::launch_pack(src, dst, groups, N, K, dtype == MF_FP8_E4M3, false, S(stream));
  return finish();
}

int pack_weights_kn(const void* src, void* dst, int64_t groups, int32_t N, int32_t K,
                    int32_t dtype, void* stream) {
  if (groups < 0 || N <= 0 || K <= 0) return MF_EINVAL;
  if (dtype != MF_BF16 && dtype != MF_FP8_E4M3) return MF_EINVAL;
  if ((dtype == MF_BF16 && K % 16 != 0) || (dtype == MF_FP8_E4M3 && K % 128 != 0))
    return MF_EUNSUPPORTED;
  if (groups == 0) return MF_OK;
  if (!src || !dst) return MF_EINVAL;
  if (!a16(dst) || (dtype == MF_BF16 && reinterpret_cast<uintptr_t>(src) % 2 != 0))
    return MF_EUNSUPPORTED;
  mf::launch_pack(src, dst, groups, N, K, dtype == MF_FP8_E4M3, true, S(stream));
  return finish();
}

size_t moe_route_workspace_size(int64_t T, int32_t d, int32_t E) {
  if (T < 0 || d <= 0 || d % 64 != 0 || E < 8 || E > 256 || T > kI32Max / 8) return 0;
  return mf::route_workspace_bytes(T, d, E);
}

int moe_route(const void* x, const void* w_r, const float* bias, int64_t T, int32_t d, int32_t E,
              int32_t k, int32_t* topk_idx, float* topk_w, void* workspace,
              size_t workspace_bytes, void* stream) {
  if (!w_r || !bias || T < 0 || d <= 0) return MF_EINVAL;
  if (k <= 0 || E < k) return MF_EINVAL;
  if (k != 8 || E > 256 || d % 64 != 0) return MF_EUNSUPPORTED;
  if (T > kI32Max / 8) return MF_EUNSUPPORTED;
  if (T == 0) return MF_OK;  // zero-size buffers may be NULL
  if (!x || !topk_idx || !topk_w || !workspace) return MF_EINVAL;
  if (workspace_bytes < mf::route_workspace_bytes(T, d, E)) return MF_EINVAL;
  if (!a16(x) || !a16(w_r) || !a16(workspace)) return MF_EUNSUPPORTED;
  mf::launch_route(x, w_r, bias, T, d, E, topk_idx, topk_w, workspace, num_cus(), S(stream));
  return finish();
}

size_t moe_permute_workspace_size(int64_t T, int32_t k, int32_t e_count) {
  if (T < 0 || k < 1 || k > 8 || e_count < 1 || e_count > 256 || T > kI32Max / 8) return 0;
  return mf::permute_workspace_bytes(T, e_count);
}

int moe_permute(const int32_t* topk_idx, int64_t T, int32_t k, int32_t e_begin, int32_t e_count,
                const void* x, int32_t d, int32_t x_dtype, void* x_perm, int32_t* counts,
                int32_t* offsets, int32_t* src_token, int32_t* inv_pos, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (!counts || !offsets || !workspace) return MF_EINVAL;
  if (T < 0 || k < 1 || e_begin < 0 || e_count < 1) return MF_EINVAL;
  if (T > 0 && (!topk_idx || !src_token || !inv_pos)) return MF_EINVAL;  // NULL only if empty
  if (k > 8 || e_count > 256 || T > kI32Max / 8) return MF_EUNSUPPORTED;
  if (workspace_bytes < mf::permute_workspace_bytes(T, e_count)) return MF_EINVAL;
  if (!a16(workspace)) return MF_EUNSUPPORTED;
  int64_t row_bytes = 0;
  if (x != nullptr && T > 0) {
    if (!x_perm || d <= 0) return MF_EINVAL;
    if (x_dtype != MF_BF16 && x_dtype != MF_F32) return MF_EINVAL;
    row_bytes = static_cast<int64_t>(d) * (x_dtype == MF_BF16 ? 2 : 4);
    if (row_bytes % 16 != 0 || !a16(x) || !a16(x_perm)) return MF_EUNSUPPORTED;
  }
  mf::launch_permute(topk_idx, T, k, e_begin, e_count, T > 0 ? x : nullptr, row_bytes, x_perm,
                     counts, offsets,
                     src_token, inv_pos, workspace, S(stream));
  return finish();
}

int moe_permute_noalloc(const int32_t* topk_idx, int64_t T, int32_t k, int32_t e_begin,
                        int32_t e_count, const void* x, int32_t d, int32_t x_dtype, void* x_perm,
                        int32_t* counts, int32_t* offsets, int32_t* src_token, int32_t* inv_pos,
                        void* stream) {
  // the checks of moe_permute, then the scratch size instead of a workspace
  if (!counts || !offsets) return MF_EINVAL;
  if (T < 0 || k < 1 || e_begin < 0 || e_count < 1) return MF_EINVAL;
  if (T > 0 && (!topk_idx || !src_token || !inv_pos)) return MF_EINVAL;  // NULL only if empty
  if (k > 8 || e_count > 256 || T > kI32Max / 8) return MF_EUNSUPPORTED;
  if (mf::permute_workspace_bytes(T, e_count) > mf::kPermuteScratchBytes) return MF_EUNSUPPORTED;
  int64_t row_bytes = 0;
  if (x != nullptr && T > 0) {
    if (!x_perm || d <= 0) return MF_EINVAL;
    if (x_dtype != MF_BF16 && x_dtype != MF_F32) return MF_EINVAL;
    row_bytes = static_cast<int64_t>(d) * (x_dtype == MF_BF16 ? 2 : 4);
    if (row_bytes % 16 != 0 || !a16(x) || !a16(x_perm)) return MF_EUNSUPPORTED;
  }
  void* ws = nullptr;
  if (mf::permute_scratch(&ws) != 0) return MF_EHIP;
  mf::launch_permute(topk_idx, T, k, e_begin, e_count, T > 0 ? x : nullptr, row_bytes, x_perm,
                     counts, offsets, src_token, inv_pos, ws, S(stream));
  return finish();
}

int moe_dispatch_masked(const int32_t* topk_idx, int64_t T, int32_t k, int32_t e_begin,
                        int32_t e_count, int32_t cap, int32_t* counts, int32_t* row_index,
                        int32_t* pos, void* workspace, size_t workspace_bytes, void* stream) {
  if (!counts || !workspace) return MF_EINVAL;
  if (T < 0 || k < 1 || e_begin < 0 || e_count < 1 || cap < 1) return MF_EINVAL;
  if (T > 0 && (!topk_idx || !row_index || !pos)) return MF_EINVAL;  // NULL only if empty
  if (k > 8 || e_count > 256 || T > kI32Max / 8 ||
      static_cast<int64_t>(e_count) * cap > kI32Max)
    return MF_EUNSUPPORTED;
  if (workspace_bytes < mf::permute_workspace_bytes(T, e_count)) return MF_EINVAL;
  if (!a16(workspace)) return MF_EUNSUPPORTED;
  mf::launch_dispatch_masked(topk_idx, T, k, e_begin, e_count, cap, counts, row_index, pos,
                             workspace, S(stream));
  return finish();
}

namespace {

// Shared validation of the grouped GEMM calls. Returns MF_OK when the launch
// may proceed, a status otherwise (MF_OK with *empty set for max_rows == 0).
int check_grouped(const void* a, const int32_t* offsets, int32_t e_count, int64_t max_rows,
                  int32_t d, int32_t f, int32_t w_dtype, const void* w0, const void* w1,
                  const float* s0, const float* s1, const void* out, bool* empty,
                  const int32_t* row_index = nullptr, int64_t src_rows = 0) {
  *empty = false;
  if (!offsets || !w0 || !w1) return MF_EINVAL;
  if (e_count < 1 || max_rows < 0 || d <= 0 || f <= 0) return MF_EINVAL;
  if (row_index && (src_rows < 1 || src_rows > kI32Max)) return MF_EINVAL;
  if (w_dtype != MF_BF16 && w_dtype != MF_FP8_E4M3) return MF_EINVAL;
  if (w_dtype == MF_FP8_E4M3 && (!s0 || !s1)) return MF_EINVAL;
  if (e_count > 256 || max_rows > kI32Max) return MF_EUNSUPPORTED;
  if (w_dtype == MF_BF16 && (d % 64 != 0 || f % 64 != 0)) return MF_EUNSUPPORTED;
  if (w_dtype == MF_FP8_E4M3 && (d % 128 != 0 || f % 128 != 0)) return MF_EUNSUPPORTED;
  if (max_rows == 0) {  // zero-size buffers may be NULL
    *empty = true;
    return MF_OK;
  }
  if (!a || !out) return MF_EINVAL;
  if (!a16(a) || !a16(w0) || !a16(w1) || !a16(out)) return MF_EUNSUPPORTED;
  return MF_OK;
}

void enqueue_gate_up(const void* x, const int32_t* row_index, int64_t src_rows,
                     const int32_t* offsets, int32_t e_count, int64_t max_rows, int32_t d,
                     int32_t f, const void* w_gate, const void* w_up, int32_t w_dtype,
                     const float* s_gate, const float* s_up, void* h, hipStream_t s,
                     const int32_t* counts = nullptr, int32_t cap = 0) {
  if (w_dtype == MF_BF16)
    mf::launch_gemm_gateup_bf16(x, row_index, src_rows, offsets, e_count, max_rows, d, f, w_gate,
                                w_up, h, num_cus(), s, counts, cap);
  else if (counts == nullptr && mf::w8_prefers_tiles(max_rows, e_count, d))
    mf::launch_gemm_gateup_w8(x, row_index, src_rows, offsets, e_count, max_rows, d, f, w_gate,
                              w_up, s_gate, s_up, h, num_cus(), s);
  else
    mf::launch_gemm_gateup_fp8(x, row_index, src_rows, offsets, e_count, max_rows, d, f, w_gate,
                               w_up, s_gate, s_up, h, num_cus(), s, counts, cap);
}

void enqueue_down(const void* h, const int32_t* offsets, int32_t e_count, int64_t max_rows,
                  int32_t f, int32_t d, const void* w_down, int32_t w_dtype, const float* s_down,
                  void* y, hipStream_t s, const int32_t* counts = nullptr, int32_t cap = 0) {
  if (w_dtype == MF_BF16)
    mf::launch_gemm_down_bf16(h, offsets, e_count, max_rows, f, d, w_down, y, false, num_cus(),
                              s, counts, cap);
  else if (counts == nullptr && mf::w8_prefers_tiles(max_rows, e_count, f))
    mf::launch_gemm_down_w8(h, offsets, e_count, max_rows, f, d, w_down, s_down, y, num_cus(), s);
  else
    mf::launch_gemm_down_fp8(h, offsets, e_count, max_rows, f, d, w_down, s_down, y, num_cus(),
                             s, counts, cap);
}

}  // namespace

int grouped_gate_up(const void* x, const int32_t* row_index, int64_t src_rows,
                    const int32_t* offsets, int32_t e_count, int64_t max_rows, int32_t d,
                    int32_t f, const void* w_gate, const void* w_up, int32_t w_dtype,
                    const float* s_gate, const float* s_up, void* h_out, void* stream) {
  bool empty;
  const int st = check_grouped(x, offsets, e_count, max_rows, d, f, w_dtype, w_gate, w_up,
                               s_gate, s_up, h_out, &empty, row_index, src_rows);
  if (st != MF_OK || empty) return st;
  enqueue_gate_up(x, row_index, src_rows, offsets, e_count, max_rows, d, f, w_gate, w_up,
                  w_dtype, s_gate, s_up, h_out, S(stream));
  return finish();
}

int grouped_down(const void* h, const int32_t* offsets, int32_t e_count, int64_t max_rows,
                 int32_t f, int32_t d, const void* w_down, int32_t w_dtype, const float* s_down,
                 void* y_perm, void* stream) {
  bool empty;
  const int st = check_grouped(h, offsets, e_count, max_rows, d, f, w_dtype, w_down, w_down,
                               s_down, s_down, y_perm, &empty);
  if (st != MF_OK || empty) return st;
  enqueue_down(h, offsets, e_count, max_rows, f, d, w_down, w_dtype, s_down, y_perm, S(stream));
  return finish();
}

int grouped_swiglu(const void* x, const int32_t* row_index, int64_t src_rows,
                   const int32_t* offsets, int32_t e_count, int64_t max_rows, int32_t d,
                   int32_t f, const void* w_gate, const void* w_up, const void* w_down,
                   int32_t w_dtype, const float* s_gate, const float* s_up, const float* s_down,
                   void* h_work, void* y_perm, void* stream) {
  bool empty;
  int st = check_grouped(x, offsets, e_count, max_rows, d, f, w_dtype, w_gate, w_up, s_gate,
                         s_up, h_work, &empty, row_index, src_rows);
  if (st != MF_OK || empty) return st;
  st = check_grouped(h_work, offsets, e_count, max_rows, d, f, w_dtype, w_down, w_down, s_down,
                     s_down, y_perm, &empty);
  if (st != MF_OK) return st;
  const hipStream_t s = S(stream);
  enqueue_gate_up(x, row_index, src_rows, offsets, e_count, max_rows, d, f, w_gate, w_up, w_dtype,
                  s_gate, s_up, h_work, s);
  enqueue_down(h_work, offsets, e_count, max_rows, f, d, w_down, w_dtype, s_down, y_perm, s);
  return finish();
}

int quantize_fp8_rows(const void* x, int64_t rows, const int32_t* row_count, int32_t K, void* q,
                      float* scales, void* stream) {
  if (rows < 0 || K <= 0) return MF_EINVAL;
  if (K % 128 != 0 || rows > kI32Max) return MF_EUNSUPPORTED;
  if (rows == 0) return MF_OK;  // zero-size buffers may be NULL
  if (!x || !q || !scales) return MF_EINVAL;
  if (!a16(x) || reinterpret_cast<uintptr_t>(q) % 8 != 0 ||
      reinterpret_cast<uintptr_t>(scales) % 4 != 0)
    return MF_EUNSUPPORTED;
  mf::launch_quantize_rows(x, rows, row_count, K, q, scales, S(stream));
  return finish();
}

namespace {

int check_a8(const void* a, const float* a_scale, const int32_t* offsets, int32_t e_count,
             int64_t max_rows, int32_t K, int32_t N, const void* w0, const void* w1,
             const float* s0, const float* s1, const void* out, bool* empty,
             const int32_t* row_index = nullptr, int64_t src_rows = 0) {
  *empty = false;
  if (!offsets || !w0 || !w1 || !s0 || !s1) return MF_EINVAL;
  if (e_count < 1 || max_rows < 0 || K <= 0 || N <= 0) return MF_EINVAL;
  if (row_index && (src_rows < 1 || src_rows > kI32Max)) return MF_EINVAL;
  if (e_count > 256 || max_rows > kI32Max) return MF_EUNSUPPORTED;
  if (K % 128 != 0 || N % 128 != 0) return MF_EUNSUPPORTED;
  if (K > 16384) return MF_EUNSUPPORTED;  // weight-scale table of a tile: 128 slabs
  if (max_rows == 0) {  // zero-size buffers may be NULL
    *empty = true;
    return MF_OK;
  }
  if (!a || !a_scale || !out) return MF_EINVAL;
  if (!a16(a) || !a16(w0) || !a16(w1) || !a16(out) ||
      reinterpret_cast<uintptr_t>(a_scale) % 4 != 0)
    return MF_EUNSUPPORTED;
  return MF_OK;
}

}  // namespace

int grouped_gate_up_a8(const void* xq, const float* x_scale, const int32_t* row_index,
                       int64_t src_rows, const int32_t* offsets, int32_t e_count,
                       int64_t max_rows, int32_t d, int32_t f, const void* w_gate,
                       const void* w_up, const float* s_gate, const float* s_up, void* h_out,
                       void* stream) {
  bool empty;
  const int st = check_a8(xq, x_scale, offsets, e_count, max_rows, d, f, w_gate, w_up, s_gate,
                          s_up, h_out, &empty, row_index, src_rows);
  if (st != MF_OK || empty) return st;
  mf::launch_gemm_gateup_a8(xq, x_scale, row_index, src_rows, offsets, e_count, max_rows, d, f,
                            w_gate, w_up, s_gate, s_up, h_out, num_cus(), S(stream));
  return finish();
}

int grouped_down_a8(const void* hq, const float* h_scale, const int32_t* offsets,
                    int32_t e_count, int64_t max_rows, int32_t f, int32_t d, const void* w_down,
                    const float* s_down, void* y_perm, void* stream) {
  bool empty;
  const int st = check_a8(hq, h_scale, offsets, e_count, max_rows, f, d, w_down, w_down, s_down,
                          s_down, y_perm, &empty);
  if (st != MF_OK || empty) return st;
  mf::launch_gemm_down_a8(hq, h_scale, offsets, e_count, max_rows, f, d, w_down, s_down, y_perm,
                          num_cus(), S(stream));
  return finish();
}

int grouped_gate_up_masked(const void* x, const int32_t* row_index, int64_t src_rows,
                           const int32_t* counts, int32_t cap, int32_t e_count, int32_t d,
                           int32_t f, const void* w_gate, const void* w_up, int32_t w_dtype,
                           const float* s_gate, const float* s_up, void* h_out, void* stream) {
  if (!counts || cap < 1) return MF_EINVAL;
  const int64_t max_rows = static_cast<int64_t>(e_count) * cap;
  bool empty;
  // check_grouped needs a non-NULL boundary table: the counts stand in for it
  const int st = check_grouped(x, counts, e_count, max_rows, d, f, w_dtype, w_gate, w_up,
                               s_gate, s_up, h_out, &empty, row_index, src_rows);
  if (st != MF_OK || empty) return st;
  enqueue_gate_up(x, row_index, src_rows, nullptr, e_count, max_rows, d, f, w_gate, w_up,
                  w_dtype, s_gate, s_up, h_out, S(stream), counts, cap);
  return finish();
}

int grouped_down_masked(const void* h, const int32_t* counts, int32_t cap, int32_t e_count,
                        int32_t f, int32_t d, const void* w_down, int32_t w_dtype,
                        const float* s_down, void* y_perm, void* stream) {
  if (!counts || cap < 1) return MF_EINVAL;
  const int64_t max_rows = static_cast<int64_t>(e_count) * cap;
  bool empty;
  const int st = check_grouped(h, counts, e_count, max_rows, d, f, w_dtype, w_down, w_down,
                               s_down, s_down, y_perm, &empty);
  if (st != MF_OK || empty) return st;
  enqueue_down(h, nullptr, e_count, max_rows, f, d, w_down, w_dtype, s_down, y_perm, S(stream),
               counts, cap);
  return finish();
}

int moe_combine(const void* y_perm, const int32_t* inv_pos, const float* topk_w, int64_t T,
                int32_t k, int32_t d, int64_t max_rows, const void* residual, void* out,
                int32_t out_dtype, void* stream) {
  if (T < 0 || k < 1 || d <= 0 || max_rows < 0) return MF_EINVAL;
  if (out_dtype != MF_BF16 && out_dtype != MF_F32) return MF_EINVAL;
  if (k > 8 || d % 64 != 0 || T > 0xFFFFFFFFLL) return MF_EUNSUPPORTED;
  if (T == 0) return MF_OK;  // zero-size buffers may be NULL
  if (!inv_pos || !topk_w || !out || (!y_perm && max_rows > 0)) return MF_EINVAL;
  if (!a16(y_perm) || !a16(out) || !a16(residual)) return MF_EUNSUPPORTED;
  mf::launch_combine(y_perm, inv_pos, topk_w, T, k, d, max_rows, residual, out,
                     out_dtype == MF_F32, S(stream));
  return finish();
}

int tp_shard_mlp(const void* x, const void* w_gate_s, const void* w_up_s, const void* w_down_s,
                 int64_t T, int32_t d, int32_t f_s, int32_t dtype, void* h_work, float* partial,
                 void* stream) {
  if (!w_gate_s || !w_up_s || !w_down_s) return MF_EINVAL;
  if (T < 0 || d <= 0 || f_s <= 0) return MF_EINVAL;
  if (dtype != MF_BF16 && dtype != MF_F32) return MF_EINVAL;
  if (T > kI32Max) return MF_EUNSUPPORTED;
  if (T > 0 && (!x || !h_work || !partial)) return MF_EINVAL;  // NULL only if empty
  if (dtype == MF_BF16) {
    if (d % 64 != 0 || f_s % 64 != 0) return MF_EUNSUPPORTED;
    if (!a16(x) || !a16(w_gate_s) || !a16(w_up_s) || !a16(w_down_s) || !a16(h_work) ||
        !a16(partial))
      return MF_EUNSUPPORTED;
  } else if ((T + 15) / 16 > 65535) {
    return MF_EUNSUPPORTED;
  }
  if (T == 0) return MF_OK;
  const hipStream_t s = S(stream);
  if (dtype == MF_BF16) {
    const int cus = num_cus();
    mf::launch_gemm_gateup_bf16(x, nullptr, 0, nullptr, 1, T, d, f_s, w_gate_s, w_up_s, h_work,
                                cus, s);
    mf::launch_gemm_down_bf16(h_work, nullptr, 1, T, f_s, d, w_down_s, partial, true, cus, s);
  } else {
    mf::launch_dense_f32(static_cast<const float*>(x), static_cast<const float*>(w_gate_s),
                         static_cast<const float*>(w_up_s), static_cast<const float*>(w_down_s),
                         T, d, f_s, static_cast<float*>(h_work), partial, s);
  }
  return finish();
}

int mf_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* out, void* stream) {
  if (workgroups < 1 || iters < 1 || !out) return MF_EINVAL;
  mf::launch_probe_mfma(workgroups, iters, out, S(stream));
  return finish();
}

int mf_probe_hbm_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* out,
                      void* stream) {
  if (!src || !out || bytes < 16 || bytes % 16 != 0 || workgroups < 1) return MF_EINVAL;
  if (!a16(src)) return MF_EUNSUPPORTED;
  mf::launch_probe_read(src, bytes, workgroups, out, S(stream));
  return finish();
}

int mf_probe_hbm_copy(const void* src, void* dst, int64_t bytes, int32_t workgroups,
                      void* stream) {
  if (!src || !dst || bytes < 16 || bytes % 16 != 0 || workgroups < 1) return MF_EINVAL;
  if (!a16(src) || !a16(dst)) return MF_EUNSUPPORTED;
  mf::launch_probe_copy(src, dst, bytes, workgroups, S(stream));
  return finish();
}

}  // extern "C"
