// Grouped bf16 GEMMs of the expert MLPs on MFMA ("推理计算流梳理", EP 路径: one
// rank runs its experts as a grouped GEMM; 实际 MLP 计算策略: the gated MLP).
//
//   gate/up:  H[rows of e] = SiLU(A W_gate_e^T) * (A W_up_e^T)   (fused epilogue)
//   down:     Y[rows of e] = H W_down_e^T                         (bf16 or f32 out)
//
// A is [rows, K] row-major; weights arrive packed (pack.hip): every 32-row x
// 16-column fragment of v_mfma_f32_32x32x16_bf16's weight operand is one
// contiguous 1 KB block, so a wavefront loads a fragment with one fully
// coalesced 16-byte-per-lane load, straight into registers.
//
// Tiling. A workgroup (256 threads, 4 waves) computes a tile of up to BM = 32*MT
// rows against 256 weight rows: 128 gate + 128 up rows (128 output columns,
// gate and up side by side so the SiLU product stays in registers) or 256 down
// rows (256 output columns). Each wave owns 64 weight rows (two 32-row
// fragments) for all the tile's rows: 2*MT 32x32 accumulators, accumulated in
// place. The grouped GEMMs and the dense TP shard use MT = 4 (128 rows) with
// two workgroups per CU (OCC = 2: 256 registers per wave, two waves per SIMD),
// so that one wave's MFMAs issue while the other waits on its loads. That is
// 1.5 times the bytes per flop of a 256-row tile (MT = 8, the whole AGPR file,
// one workgroup per CU), and measured faster: prefill step 1.6 % (gate/up
// 387 -> 382 us, down 219 -> 213 us), 4096-token TP shard 2.2 % (199 -> 194
// us against 256-row tiles with A by direct-to-LDS loads), two A/B pairs on
// one box each. The router's split-K product uses MT = 4 at one workgroup per
// CU.
//
// Operand paths. A wave's weight fragments are private to it and come straight
// from global memory into registers (buffer loads: the row block's base in a
// buffer resource, 32-bit lane offsets). The A tile is shared by the four waves
// and goes through LDS (four stage buffers; 64-byte rows whose 16-byte chunks
// are XOR-swizzled so that the 32-row fragment reads are bank-conflict free).
// A moves two stages at a time, as whole 128-byte row segments (eight threads
// per row): the L1's outstanding misses bound this kernel's loads (its L1
// waits on L2 data half the time), and a 64-byte access holds a whole 128-byte
// line slot, so half-line A loads cost twice the miss slots of the bytes they
// move. (The two halves of a segment go to two stage buffers that map to the
// same banks, a two-way conflict on those writes; a mapping without it
// measured no faster.)
//
// Pipeline. BK = 32 per stage (two MFMA k-steps). Weight fragments are loaded
// three stages ahead into four register slots that rotate through a K loop
// unrolled by four, so every slot index is a compile-time constant; each
// even stage loads the A pair two stages ahead, the next (odd) stage writes
// it into the pair's two LDS buffers. The loop is branch-free
// (prefetch indices are clamped), so the compiler's vmcnt waits track exactly
// the loads being consumed. Within a stage the instruction order is fixed
// with scheduling groups: the stage's first-k-step fragments are read from
// LDS, then every pair of MFMAs is followed by one second-k-step fragment read
// and one global load, and at odd stages the A pair loaded one stage earlier
// is written to its two LDS buffers between the remaining MFMAs. Spreading the
// loads keeps the address queue from stalling the MFMA issue.
//
// Schedule. Group boundaries come from the device-side offsets (or, in the
// masked layout, from per-group counts within fixed blocks of cap rows), so
// no host sync is needed. Each workgroup computes the schedule itself: group e's
// ceil(rows_e / 32) sub-tiles are split into ceil(sub_e / MT) near-equal
// chunks (so an expert's last chunk is not a sliver), a tile is one chunk
// against one n-tile, and tiles are numbered group-major, then n-tile, then
// chunk, so the chunks that share one weight n-tile are consecutive. A tile
// runs a K loop instantiated for its live sub-tiles only. The grid is
// persistent; workgroup b (dispatched round-robin to XCD b % 8) takes tile
// it*G + (b%8)*(G/8) + b/8 in round it, so each XCD works on a contiguous run
// of tiles at a time and shares weight n-tiles and A chunks through its L2.
// With the chunk minor, a group's run of tiles that straddles two XCDs (or
// two rounds) splits its n-tiles between them, so each weight n-tile is still
// fetched once and only the (smaller) A chunks are fetched twice; with the
// n-tile minor, both sides fetched every n-tile (prefill routing: 1.60 GB of
// L2 misses per gate/up launch against 1.20 GB of algorithmic traffic).
#include "common.h"
#include "launch.h"

namespace mf {

namespace {

constexpr int BK = 32;         // K depth of one pipeline stage: two MFMA k-steps
constexpr int ROWB = BK * 2;   // bytes of one A row of a stage (64)
constexpr int MAX_GROUPS = 256;
constexpr int SLOTS = 4;       // weight register slots
constexpr int PREF = SLOTS - 1;  // weight stages in flight ahead of the one consumed
constexpr int FRAG = 1024;     // bytes of one packed 32x16 weight fragment

typedef __attribute__((ext_vector_type(16))) float f32x16;

struct GemmParams {
  const char* a;           // [max_rows, K] bf16, or [a_src_rows, K] when a_rows is set
  const int32_t* a_rows;   // nullptr, or [max_rows]: row r of the GEMM's A is row a_rows[r]
                           // of `a` (clamped to [0, a_src_rows)): the gather of the
                           // permutation done inside the A load
  int a_src_rows;
  const char* b0;          // packed weights (gate, or down): [groups][nb][K/16] fragments
  const char* b1;          // packed weights (up; gated only)
  char* c;                 // [max_rows, ldc] bf16 or f32 (per K split, see c_split)
  const int32_t* offsets;  // [groups+1] or nullptr (one group of max_rows rows)
  int e_count;
  int max_rows;
  int K;                   // row length of A and of the weights (elements)
  int nb;                  // 32-row weight blocks per group (packed)
  int n_valid;             // weight rows that exist: blocks past them are clamped on
                           // load and output columns >= n_valid are not stored
  int ldc;                 // row stride of C (elements)
  int kc;                  // K range of one split: split y covers [y*kc, (y+1)*kc)
  int64_t c_split;         // elements between the C blocks of consecutive splits
  const int32_t* counts;   // masked layout (offsets unused): group e owns rows
  int cap;                 // [e*cap, e*cap + min(counts[e], cap)); nullptr: offsets
};

// A stage row is 64 bytes (four 16-byte chunks); chunk c of row r sits at
// chunk c ^ f(r) with f(r) = ((r >> 1) ^ (r >> 3)) % 4. A 32-row fragment read
// (one logical chunk of consecutive rows) then hits distinct banks in every
// group of 16 lanes of a 64-bank LDS (rows r and r + 8 no longer collide), and
// in every group of 8 lanes of a 32-bank one; a row write (four chunks of a
// row) is a permutation of the row's chunks, conflict-free either way.
__device__ __forceinline__ int swz(int r, int chunk) {
  return r * ROWB + ((chunk ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4);
}

__device__ __forceinline__ f32x16 mfma32(const u32x4& w, const u32x4& a, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                 __builtin_bit_cast(bf16x8, a), c, 0, 0, 0);
}

}  // namespace

// K loop of one tile for NM live 32-row sub-tiles (1..MT); nk (stages of 32)
// is a multiple of 4, or with TAIL of 2 but not 4 (a separate kernel: a tail
// in the same code made the compiler spill inside the MFMA loop). Branch-free: the
// prefetch stage indices are clamped (the last steps re-load the final stage),
// so the compiler's vmcnt waits track exactly the loads being consumed.
//
// Stage t: (t even) issue the A pair t+2, t+3; issue the weights of t+3; run
// the MFMAs of t; (t odd) write the A pair loaded at stage t-1 into its two
// LDS buffers, then barrier. Thread (ld_r, ld_c) moves 16-byte chunk ld_c of
// the 128-byte pair segment of rows ld_r + 32i, i < NM.
//
// One barrier per stage pair is enough. The pair written at odd stage t goes
// to buffers (t+1)%4 and (t+2)%4. Any wave that has not reached this write is
// at stage t-1 or t, reading buffer (t-1)%4 or t%4, which are different
// buffers. The barrier at the end of stage t-2 ordered the last reads of the
// two target buffers (stages t-3 and t-2) before the write. The barrier at
// the end of stage t makes the written pair visible to stages t+1 and t+2.
// Measured 1 % faster at prefill than a barrier after every stage.
template <int MT, int NM, bool TAIL, bool ROT>
__device__ __forceinline__ void k_loop(f32x16 (&acc)[MT][2], const char* abase,
                                       const int (&arow)[MT], int64_t Kb,
                                       const char* const (&bp)[2],
                                       char (&lds)[4][MT * 32 * ROWB], int nk, int ld_r,
                                       int ld_c, int lane, int rot) {
  // A moves two stages at a time as whole 128-byte row segments (eight
  // threads per row, rows ld_r + 32 i): chunk ld_c & 3 of stage pair member
  // ld_c >> 2. Loaded at even stages, written at the next odd stage into the
  // two LDS buffers of the pair.
  constexpr int NA = NM;
  u32x4 areg[NA];
  u32x4 breg[SLOTS][4];
  const int lr = lane & 31, lg = lane >> 5;
  // ROT: the K loop starts at stage rot (even) and wraps around (the sum is
  // taken in that order)
  auto rotk = [&](int kt) {
    if constexpr (ROT) {
      const int r = kt + rot;
      return r >= nk ? r - nk : r;
    } else {
      return kt;
    }
  };
  auto load_pair = [&](int kt) {  // stages kt and kt + 1 (kt even)
    const int64_t ka = static_cast<int64_t>(rotk(kt)) * ROWB;
#pragma unroll
    for (int i = 0; i < NA; ++i) areg[i] = ld16(abase + static_cast<int64_t>(arow[i]) * Kb + ka);
  };
  auto write_pair = [&](int buf0) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      st16(&lds[(buf0 + (ld_c >> 2)) & 3][swz(ld_r + 32 * i, ld_c & 3)], areg[i]);
  };
  // Weight fragments by buffer loads: the fragment row block's base in a
  // buffer resource (scalar registers, the same for the whole wave) and a
  // 32-bit per-lane offset (a row block spans K/16 fragments of 1 KB), in
  // place of 64-bit per-lane addresses: measured 1-2 % faster (gate/up
  // 432.7 -> 425 us at prefill).
  __amdgpu_buffer_rsrc_t wrs[2];
#pragma unroll
  for (int jn = 0; jn < 2; ++jn) wrs[jn] = wave_rsrc(bp[jn] - lane * 16);
  auto load_b = [&](u32x4 (&br)[4], int kt) {
    const int kb = rotk(kt) * (2 * FRAG);
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int s = 0; s < 2; ++s) br[jn * 2 + s] = ld16_buf(wrs[jn], lane * 16 + kb + s * FRAG);
  };
  // One stage in a fixed instruction order. The k-step 0 fragments of every
  // live sub-tile are read from LDS first; the global loads (the weights of
  // three stages ahead and, at even stages, the A pair two stages ahead) and
  // k-step 1's fragment reads are spread between k-step 0's MFMAs, one load
  // per MFMA pair, so the address queue never backs up into the MFMA issue; at
  // odd stages the pair loaded one stage earlier is written to LDS between
  // k-step 1's MFMAs.
  auto stage = [&](const u32x4 (&br)[4], int buf, bool even, int kt_pair, u32x4 (&b_dst)[4],
                   int kt_b) {
    if (even) load_pair(kt_pair);
    load_b(b_dst, kt_b);
    u32x4 af[2][NM];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < NM; ++i) af[s][i] = ld16(&lds[buf][swz(i * 32 + lr, 2 * s + lg)]);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        acc[i][0] = mfma32(br[s], af[s][i], acc[i][0]);
        acc[i][1] = mfma32(br[2 + s], af[s][i], acc[i][1]);
      }
    if (!even) write_pair((buf + 1) & 3);
    // masks: MFMA 0x008, VMEM read 0x020, DS read 0x100, DS write 0x200
    if (even) {
      constexpr int NLE = NA + 4, LE = NLE > NM ? NLE - NM : 0;
      __builtin_amdgcn_sched_group_barrier(0x020, LE, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NM, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (i < NLE - LE) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NM, 0);
    } else {
      constexpr int NLO = 4, LO = NLO > NM ? NLO - NM : 0;
      __builtin_amdgcn_sched_group_barrier(0x020, LO, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NM, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (i < NLO - LO) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
    }
  };

  // the weights of stages 0..2 and the first A pair, same outstanding order
  // at the loop entry as at its back-edge (A pair, then weights)
  load_pair(0);
#pragma unroll
  for (int s = 0; s < PREF; ++s) load_b(breg[s], s < nk ? s : nk - 1);
  write_pair(0);
  __syncthreads();
#define MF_GEMM_STEP(S)                                                                    \
  {                                                                                        \
    const int t_ = kt + (S);                                                               \
    stage(breg[(S)], (S), ((S) & 1) == 0, min(t_ + 2, nk - 2), breg[((S) + PREF) % SLOTS],  \
          min(t_ + PREF, nk - 1));                                                         \
    if ((S) & 1) __syncthreads();                                                          \
  }
  int kt = 0;
  for (; TAIL ? kt + SLOTS <= nk : kt < nk; kt += SLOTS) {
    MF_GEMM_STEP(0)
    MF_GEMM_STEP(1)
    MF_GEMM_STEP(2)
    MF_GEMM_STEP(3)
  }
  if constexpr (TAIL) {  // nk % 4 == 2: one stage pair left, in slots 0 and 1
    MF_GEMM_STEP(0)
    MF_GEMM_STEP(1)
  }
#undef MF_GEMM_STEP
}

template <int MT, bool GATED, bool OUT_F32, bool TAIL, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_bf16_kernel(GemmParams p) {
  static_assert(MT == 4, "128-row tiles");
  constexpr int BN_OUT = GATED ? 128 : 256;
  __shared__ __attribute__((aligned(16))) char lds[4][MT * 32 * ROWB];  // A stage buffers
  __shared__ int s_tile0[MAX_GROUPS + 1];
  __shared__ int s_beg[MAX_GROUPS];
  __shared__ int s_end[MAX_GROUPS];

  const int tid = threadIdx.x;
  // n-tiles per group: the packed row blocks cover the weight rows
  const int NT = (p.nb * 32 + BN_OUT - 1) / BN_OUT;

  // ---- device-side schedule ---------------------------------------------
  // Group e's rows form sub_e = ceil(rows_e / 32) sub-tiles, split into
  // nch_e = ceil(sub_e / Z) near-equal chunks (the first sub_e % nch_e one
  // sub-tile longer). A tile is one chunk against one n-tile; tiles are
  // numbered group-major, then n-tile, then chunk.
  constexpr int Z = MT;
  int ntile = 0;
  if (tid < p.e_count) {
    int beg = 0, end = p.max_rows;
    if (p.counts != nullptr) {  // masked layout: fixed blocks of cap rows
      beg = clampi(tid * p.cap, 0, p.max_rows);
      end = clampi(beg + clampi(p.counts[tid], 0, p.cap), beg, p.max_rows);
    } else if (p.offsets != nullptr) {
      beg = clampi(p.offsets[tid], 0, p.max_rows);
      end = clampi(p.offsets[tid + 1], beg, p.max_rows);
    }
    s_beg[tid] = beg;
    s_end[tid] = end;
    ntile = ((((end - beg + 31) >> 5) + Z - 1) / Z) * NT;
  }
  s_tile0[tid + 1] = ntile;  // inclusive scan below, shifted by one
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
  const int lr = lane & 31, lg = lane >> 5;
  const int ld_c = tid & 7;    // A: 16-byte chunk of a two-stage (128-byte) row segment
  const int ld_r = tid >> 3;   // A: first row this thread moves (then +32, +64, ...)
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nk = p.kc / BK;
  const int kblocks = p.K / 16;  // packed fragments per 32-row block
  const int64_t Kb = static_cast<int64_t>(p.K) * 2;
  const int64_t kofs_a = static_cast<int64_t>(blockIdx.y) * p.kc * 2;  // bytes into each A row
  const int64_t kofs_b = static_cast<int64_t>(blockIdx.y) * (p.kc / 16) * FRAG;
  char* const cbase = p.c + static_cast<int64_t>(blockIdx.y) * p.c_split * (OUT_F32 ? 4 : 2);

  for (int it = 0;; it += G) {
    const int L = it + xcd * (G >> 3) + slot;
    if (L >= total_tiles) break;

    // group e: the last with s_tile0[e] <= L (it owns tile L)
    int lo = 0, hi = p.e_count - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tile0[mid] <= L) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int t = L - s_tile0[e];
    const int sub_e = (s_end[e] - s_beg[e] + 31) >> 5;
    const int nch = (sub_e + Z - 1) / Z;
    const int ni = t / nch, mi = t - ni * nch;  // n-tile major, chunk minor
    const int q = sub_e / nch, r = sub_e - q * nch;
    const int zc = mi * q + min(mi, r);            // first sub-tile of the chunk
    const int nm = q + (mi < r ? 1 : 0);           // sub-tiles in the chunk
    const int row0 = s_beg[e] + zc * 32;
    const int rows_valid = min(nm * 32, s_end[e] - row0);
    const int n0 = ni * BN_OUT;

    // ---- per-thread global pointers ---------------------------------------
    // A rows past the tile's valid rows re-read row0 (row m of the result
    // depends on row m of A only, and those rows are never stored).
    int arow[MT];  // source rows of the rows ld_r + 32 i this thread moves
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int r = ld_r + 32 * i;
      int ar = row0 + (r < rows_valid ? r : 0);
      if (p.a_rows != nullptr) ar = clampi(p.a_rows[ar], 0, p.a_src_rows - 1);
      arow[i] = ar;
    }
    const char* abase = p.a + kofs_a + ld_c * 16;
    const char* bp[2];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const char* base = (GATED && jn == 1) ? p.b1 : p.b0;
      const int row = GATED ? n0 + wave * 32 : n0 + wave * 64 + jn * 32;
      const int blk = min(row >> 5, p.nb - 1);
      bp[jn] = base + ((static_cast<int64_t>(e) * p.nb + blk) * kblocks) * FRAG + kofs_b +
               lane * 16;
    }

    f32x16 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) acc[i][jn] = f32x16{};

    // The router's split-K product (MT = 4: every workgroup reads the same
    // L2-resident router weight) starts each tile's K loop at a different
    // stage pair, so that concurrent tiles read different K offsets: route
    // stage 48.2 -> 44.2 us at 8192 tokens. The grouped GEMMs keep the common
    // start: there, tiles sharing a weight n-tile or an A chunk read it from
    // the L2 together, and rotated starts measured 12-14 % slower.
    constexpr bool ROT = MT == 4 && OUT_F32 && OCC == 1;  // the router only
    const int rot = ROT ? 2 * ((L * 7) % (nk / 2)) : 0;
    __syncthreads();  // the previous tile's LDS reads are done
    switch (nm) {  // a K loop instantiated for the tile's live sub-tiles
      case 1: k_loop<MT, 1, TAIL, ROT>(acc, abase, arow, Kb, bp, lds, nk, ld_r, ld_c, lane, rot); break;
      case 2: k_loop<MT, 2, TAIL, ROT>(acc, abase, arow, Kb, bp, lds, nk, ld_r, ld_c, lane, rot); break;
      case 3: k_loop<MT, 3, TAIL, ROT>(acc, abase, arow, Kb, bp, lds, nk, ld_r, ld_c, lane, rot); break;
      default: k_loop<MT, 4, TAIL, ROT>(acc, abase, arow, Kb, bp, lds, nk, ld_r, ld_c, lane, rot); break;
    }

    // ---- epilogue ----------------------------------------------------------
    // Lane l holds, for row lr of sub-tile i, output columns
    // 8q + 4(l/32) + 0..3 (q = 0..3) of each 32-column fragment column jn.
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = i * 32 + lr;
      if (m >= rows_valid) continue;
      const int64_t grow = row0 + m;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (GATED) {
          const int col = n0 + wave * 32 + 8 * q + 4 * lg;
          if (col >= p.n_valid) continue;  // n_valid % 32 == 0: whole 4-column groups
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = siluf_(acc[i][0][4 * q + r]) * acc[i][1][4 * q + r];
          *reinterpret_cast<u32x2*>(cbase + (grow * p.ldc + col) * 2) =
              u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        } else {
#pragma unroll
          for (int jn = 0; jn < 2; ++jn) {
            const int col = n0 + wave * 64 + jn * 32 + 8 * q + 4 * lg;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[i][jn][4 * q + r];
            if (col >= p.n_valid) continue;
            if (col + 4 > p.n_valid) {  // ragged last column group: element stores
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                if (col + r >= p.n_valid) break;
                if constexpr (OUT_F32)
                  reinterpret_cast<float*>(cbase)[grow * p.ldc + col + r] = v[r];
                else
                  reinterpret_cast<bf16_t*>(cbase)[grow * p.ldc + col + r] = f32_to_bf16(v[r]);
              }
              continue;
            }
            if constexpr (OUT_F32) {
              st16(cbase + (grow * p.ldc + col) * 4,
                   u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                         __float_as_uint(v[3])});
            } else {
              *reinterpret_cast<u32x2*>(cbase + (grow * p.ldc + col) * 2) =
                  u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
          }
        }
      }
    }
  }
}

namespace {

constexpr int MT_SPLITK = 4;  // 128-row tiles for the router's split-K product
constexpr int MT_PAIR = 4;    // the grouped and dense GEMMs: 128-row tiles, two per CU

// A contraction of K % 128 == 64 (a multiple of 64 but not of the four-stage
// loop body) takes the kernels with the two-stage tail.
bool tail_stages(int kc) { return (kc / BK) % SLOTS != 0; }

// Persistent grid: at most one workgroup per CU, a multiple of 8 (the XCD
// count), and no more than an upper bound on the tiles. With offsets each
// group can add one partial m-tile; a single dense group (offsets == nullptr)
// has exactly ceil(rows / BM) m-tiles.
int persistent_grid(int64_t max_rows, int bm, int e_count, bool dense, int nt, int num_cus) {
  const int64_t mtiles = (max_rows + bm - 1) / bm + (dense ? 0 : e_count);
  const int64_t ub = mtiles * static_cast<int64_t>(nt);
  int64_t g = ub < num_cus ? ub : num_cus;
  g = (g + 7) & ~int64_t(7);
  if (g > num_cus) g = num_cus & ~7;
  return static_cast<int>(g < 8 ? 8 : g);
}

}  // namespace

void launch_gemm_gateup_bf16(const void* a, const int32_t* a_rows, int64_t a_src_rows,
                             const int32_t* offsets, int e_count, int64_t max_rows, int K, int N,
                             const void* w_gate, const void* w_up, void* h, int num_cus,
                             hipStream_t s, const int32_t* counts, int cap) {
  GemmParams p{static_cast<const char*>(a), a_rows, static_cast<int>(a_src_rows),
               static_cast<const char*>(w_gate),
               static_cast<const char*>(w_up), static_cast<char*>(h), offsets, e_count,
               static_cast<int>(max_rows), K, N / 32, N, N, K, 0, counts, cap};
  // 128-row tiles, two workgroups per CU (two waves per SIMD); one dense
  // group (the TP shard) when there are neither offsets nor counts
  const int grid = persistent_grid(max_rows, MT_PAIR * 32, e_count,
                                   offsets == nullptr && counts == nullptr, (N + 127) / 128,
                                   2 * num_cus);
  if (tail_stages(K)) gemm_bf16_kernel<MT_PAIR, true, false, true, 2><<<grid, 256, 0, s>>>(p);
  else gemm_bf16_kernel<MT_PAIR, true, false, false, 2><<<grid, 256, 0, s>>>(p);
}

void launch_gemm_down_bf16(const void* a, const int32_t* offsets, int e_count, int64_t max_rows,
                           int K, int N, const void* w_down, void* y, bool out_f32, int num_cus,
                           hipStream_t s, const int32_t* counts, int cap) {
  GemmParams p{static_cast<const char*>(a), nullptr, 0, static_cast<const char*>(w_down), nullptr,
               static_cast<char*>(y), offsets, e_count, static_cast<int>(max_rows), K, N / 32,
               N, N, K, 0, counts, cap};
  const int grid = persistent_grid(max_rows, MT_PAIR * 32, e_count,
                                   offsets == nullptr && counts == nullptr, (N + 255) / 256,
                                   2 * num_cus);
  const bool tail = tail_stages(K);
  if (out_f32) {  // the TP shard's fp32 partial sum
    if (tail) gemm_bf16_kernel<MT_PAIR, false, true, true, 2><<<grid, 256, 0, s>>>(p);
    else gemm_bf16_kernel<MT_PAIR, false, true, false, 2><<<grid, 256, 0, s>>>(p);
  } else {
    if (tail) gemm_bf16_kernel<MT_PAIR, false, false, true, 2><<<grid, 256, 0, s>>>(p);
    else gemm_bf16_kernel<MT_PAIR, false, false, false, 2><<<grid, 256, 0, s>>>(p);
  }
}

void launch_gemm_nt_f32_splitk(const void* a, int64_t rows, int K, const void* b, int n_valid,
                               int splits, float* c_partials, int num_cus, hipStream_t s) {
  // One group of `rows` rows against n_valid (<= 256) packed weight rows, K
  // split in `splits` equal ranges; split y writes its fp32 partial product to
  // c_partials[y][rows][n_valid].
  GemmParams p{static_cast<const char*>(a), nullptr, 0, static_cast<const char*>(b), nullptr,
               reinterpret_cast<char*>(c_partials), nullptr, 1, static_cast<int>(rows), K,
               (n_valid + 31) / 32, n_valid, n_valid, K / splits,
               rows * static_cast<int64_t>(n_valid)};
  // splits x tiles workgroups: size x so that all of them fit in one round
  int gx = persistent_grid(rows, MT_SPLITK * 32, 1, true, 1, num_cus / splits);
  if (tail_stages(K / splits))
    gemm_bf16_kernel<MT_SPLITK, false, true, true, 1><<<dim3(gx, splits), 256, 0, s>>>(p);
  else
    gemm_bf16_kernel<MT_SPLITK, false, true, false, 1><<<dim3(gx, splits), 256, 0, s>>>(p);
}

}  // namespace mf
