// Internal launchers: one per kernel family. Arguments are validated by the
// C-ABI layer (abi.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mf {

// q / qs (bf16 only, d % 128 == 0, or both nullptr): also the per-token fp8
// codes [T, d] and group scales [T, d/128] of the bf16 output
void launch_rmsnorm(const void* x, const void* gamma, void* y, int64_t T, int d,
                    float eps, bool bf16, hipStream_t s, uint8_t* q = nullptr,
                    float* qs = nullptr);

int route_splits(int64_t T, int d);
size_t route_workspace_bytes(int64_t T, int d, int E);
void launch_route(const void* x, const void* w_r, const float* bias, int64_t T,
                  int d, int E, int32_t* idx, float* w, void* workspace, int num_cus,
                  hipStream_t s);

size_t permute_workspace_bytes(int64_t T, int e_count);
// Size of the static device scratch array of the allocation-free permutation:
// room for the count tables of ceil(T / 256) * e_count <= 65536.
constexpr size_t kPermuteScratchBytes = 2 * 65536 * sizeof(int32_t) + 256;
// Device address of that array on the current device (looked up once per
// device); 0 on success, -1 if the runtime could not provide it.
int permute_scratch(void** ptr);
void launch_permute(const int32_t* idx, int64_t T, int k, int e_begin, int e_count,
                    const void* x, int64_t row_bytes, void* x_perm, int32_t* counts,
                    int32_t* offsets, int32_t* src_token, int32_t* inv_pos,
                    void* workspace, hipStream_t s);

// Masked (fixed-capacity) dispatch: counts [e_count], row_index [e_count*cap],
// pos [T,k] (row e*cap + rank, or -1); workspace as launch_permute's.
void launch_dispatch_masked(const int32_t* idx, int64_t T, int k, int e_begin, int e_count,
                            int cap, int32_t* counts, int32_t* row_index, int32_t* pos,
                            void* workspace, hipStream_t s);

// Weight packing into MFMA fragment order (pack.hip).
size_t packed_bytes(int64_t groups, int N, int K, bool fp8);
// kn: src is [groups, K, N] instead of [groups, N, K]; the output is the same.
void launch_pack(const void* src, void* dst, int64_t groups, int N, int K, bool fp8, bool kn,
                 hipStream_t s);

// bf16 MFMA grouped GEMMs on packed weights. offsets == nullptr means one group
// of max_rows rows. a_rows (optional) makes row r of A the row a_rows[r] of a
// (a_src_rows rows): the permutation's gather fused into the A load.
void launch_gemm_gateup_bf16(const void* a, const int32_t* a_rows, int64_t a_src_rows,
                             const int32_t* offsets, int e_count, int64_t max_rows, int K,
                             int N, const void* w_gate, const void* w_up, void* h, int num_cus,
                             hipStream_t s, const int32_t* counts = nullptr, int cap = 0);
void launch_gemm_down_bf16(const void* a, const int32_t* offsets, int e_count,
                           int64_t max_rows, int K, int N, const void* w_down,
                           void* y, bool out_f32, int num_cus, hipStream_t s,
                           const int32_t* counts = nullptr, int cap = 0);

// C_y = A[:, y*K/splits : (y+1)*K/splits] B[:n_valid, same]^T in fp32 for each K
// split y (one group, bf16 operands). Requires (K / splits) % 64 == 0.
void launch_gemm_nt_f32_splitk(const void* a, int64_t rows, int K, const void* b, int n_valid,
                               int splits, float* c_partials, int num_cus, hipStream_t s);

// fp8-weight (block-scaled) grouped GEMMs.
void launch_gemm_gateup_fp8(const void* a, const int32_t* a_rows, int64_t a_src_rows,
                            const int32_t* offsets, int e_count, int64_t max_rows, int K,
                            int N, const void* w_gate, const void* w_up, const float* s_gate,
                            const float* s_up, void* h, int num_cus, hipStream_t s,
                            const int32_t* counts = nullptr, int cap = 0);
void launch_gemm_down_fp8(const void* a, const int32_t* offsets, int e_count,
                          int64_t max_rows, int K, int N, const void* w_down,
                          const float* s_down, void* y, int num_cus, hipStream_t s,
                          const int32_t* counts = nullptr, int cap = 0);

// fp8-weight grouped GEMMs tiled for many rows per expert (gemm_w8.hip);
// w8_prefers_tiles: whether max_rows over e_count experts and contraction K
// take them instead of the decode kernels above.
bool w8_prefers_tiles(int64_t max_rows, int e_count, int K);
void launch_gemm_gateup_w8(const void* a, const int32_t* a_rows, int64_t a_src_rows,
                           const int32_t* offsets, int e_count, int64_t max_rows, int K, int N,
                           const void* w_gate, const void* w_up, const float* s_gate,
                           const float* s_up, void* h, int num_cus, hipStream_t s);
void launch_gemm_down_w8(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                         int K, int N, const void* w_down, const float* s_down, void* y,
                         int num_cus, hipStream_t s);

// fp8 activations ([rows, K] codes + [rows, K/128] f32 group scales) against
// block-fp8 weights on the fp8 MFMA; bf16 out (gate/up: SiLU(g) * u).
void launch_gemm_gateup_a8(const void* a, const float* a_scale, const int32_t* a_rows,
                           int64_t a_src_rows, const int32_t* offsets, int e_count,
                           int64_t max_rows, int K, int N, const void* w_gate, const void* w_up,
                           const float* s_gate, const float* s_up, void* h, int num_cus,
                           hipStream_t s);
void launch_gemm_down_a8(const void* a, const float* a_scale, const int32_t* offsets,
                         int e_count, int64_t max_rows, int K, int N, const void* w_down,
                         const float* s_down, void* y, int num_cus, hipStream_t s);

// per-token 1x128-group E4M3FN quantisation of bf16 rows
void launch_quantize_rows(const void* x, int64_t rows, const int32_t* row_count, int K, void* q,
                          float* scales, hipStream_t s);

void launch_combine(const void* y_perm, const int32_t* inv_pos, const float* w,
                    int64_t T, int k, int d, int64_t max_rows, const void* residual,
                    void* out, bool out_f32, hipStream_t s);

// fp32 dense shard (FMA, no MFMA).
void launch_dense_f32(const float* x, const float* w_gate, const float* w_up,
                      const float* w_down, int64_t T, int d, int fs, float* h,
                      float* partial, hipStream_t s);

// Measurement probes (probe.hip): out has workgroups * 256 elements.
void launch_probe_mfma(int workgroups, int iters, float* out, hipStream_t s);
void launch_probe_read(const void* src, int64_t bytes, int workgroups, uint32_t* out,
                       hipStream_t s);
void launch_probe_copy(const void* src, void* dst, int64_t bytes, int workgroups, hipStream_t s);

}  // namespace mf
