// Grouped GEMM on bf16 MFMA for many rows per segment (prefill).
//
// moonep_experts page, moonep_grouped_gemm: every segment's rows are
// multiplied by the transpose of that segment's [N, K] weight, weights stored
// [G, N, K] with K contiguous; segments with no rows are skipped (module
// docstring). GEMM1 fuses the gate and up projections and applies the
// activation times the per-row route weight in its epilogue (module docstring:
// the route weight is applied to the activation); GEMM2 is the down projection.
//
// Tile: 256 rows x 256 weight rows x 64 K per stage, 4 waves (one per SIMD),
// each wave a 128 x 128 block of v_mfma_f32_32x32x16_bf16 results. For GEMM1
// the 256 weight rows are 128 gate rows and the same 128 up rows, so each
// wave holds gate and up accumulators for the same 128 x 64 outputs. Both
// operands go from HBM straight into LDS with global_load_lds_dwordx4 (no
// staging registers), double buffered (2 x 64 KB), with the 16-byte chunks of
// every row XOR-swizzled by (row & 7) so that the MFMA operand reads are
// bank-conflict free. In a partial row tile the rows
// past the segment end load a valid row of the tile and their results are
// dropped; a wave whose 128 rows are all past the end skips its MFMAs.
#pragma once

#include "common.hpp"

namespace moe {
namespace big {

constexpr int BM = 256;  // rows per tile
constexpr int BN = 256;  // weight rows per tile (GEMM1: 128 gate + 128 up)
constexpr int BK = 64;   // K per stage
constexpr int NT = 256;  // threads
constexpr int GN = 8;    // n-tiles per tile group (L2 locality of concurrently running tiles)

struct Params {
  const uint16_t* A;       // rows [*, K] bf16
  const int32_t* a_perm;   // sorted row -> flat slot, or nullptr when A is already in row order
  int32_t a_div;           // flat slot -> A row divisor (k)
  const uint16_t* B0;      // [G, N, K] (gate or down)
  const uint16_t* B1;      // [G, N, K] (up) for GEMM1
  int32_t N, K;
  const int32_t* tile_seg;
  const int32_t* tile_row0;
  const int32_t* seg_end;  // cumulative end offsets
  const int32_t* status;   // status[2] = number of row tiles
  int32_t mt_cap;          // row tiles the grid covers
  int32_t n_tiles;         // column tiles
  uint16_t* C;             // [rows, N] bf16 output, sorted row order
  const float* row_w;      // GEMM1: route weight per sorted row
  ActParams act;
};

__device__ __forceinline__ int lds_chunk(int row, int chunk) {  // in 16-byte units
  return row * (BK / 8) + (chunk ^ (row & 7));
}

// One wave-wide direct-to-LDS load: 64 lanes x 16 bytes into the 1 KB LDS
// block at lds_block (rows r0..r0+7 of a tile, r0 a multiple of 8). Lane l
// fills the block's 16-byte slot l, i.e. row r0 + l/8, slot l%8, which under
// the swizzle holds global chunk (l%8) ^ (l/8) of that row.
__device__ __forceinline__ void load_block_to_lds(const uint16_t* __restrict__ gbase, uint32_t elem_off,
                                                  u32x4* lds_block) {
  __builtin_amdgcn_global_load_lds(gbase + elem_off, lds_block, 16, 0, 0);
}

template <bool GATED>
__global__ __launch_bounds__(NT, 1) void k_gemm(const Params p) {
  // two stages, each its own LDS object
  __shared__ u32x4 sA0[BM * BK / 8], sA1[BM * BK / 8];
  __shared__ u32x4 sB0[BN * BK / 8], sB1[BN * BK / 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // block -> (row tile, column tile): groups of GN column tiles, row tiles
  // inside a group, column tile fastest; logical ids contiguous per XCD
  const int L = xcd_logical_block(blockIdx.x, gridDim.x);
  const int span = p.mt_cap * GN;
  const int grp = L / span;
  const int r_in = L - grp * span;
  const int mt = r_in / GN;
  const int nt = grp * GN + (r_in - mt * GN);
  if (nt >= p.n_tiles || mt >= p.status[2]) return;

  const int seg = p.tile_seg[mt];
  const int row0 = p.tile_row0[mt];
  const int rows = min(BM, p.seg_end[seg] - row0);
  const int N = p.N, K = p.K;
  const int n0 = nt * (GATED ? BN / 2 : BN);

  // ---- load assignment: wave w fills the 1 KB blocks w*8 .. w*8+7 of the A
  // tile and of the B tile (rows w*64 .. w*64+63). 32-bit element offsets:
  // the host keeps T*H, M*I and N*K below 2^31.
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;
  const uint16_t* __restrict__ Ab = p.A;
  const uint16_t* __restrict__ B0b = p.B0 + (size_t)seg * N * K;
  const uint16_t* __restrict__ B1b = GATED ? p.B1 + (size_t)seg * N * K : B0b;
  uint32_t a_off[8], b_off[8];
  {
    const int first = p.a_perm ? p.a_perm[row0] / p.a_div : row0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave * 64 + i * 8 + lrow;
      int arow = first;
      if (r < rows) arow = p.a_perm ? p.a_perm[row0 + r] / p.a_div : row0 + r;
      a_off[i] = (uint32_t)arow * (uint32_t)K + lchunk * 8;
      const int n = min(n0 + (GATED ? (r & 127) : r), N - 1);
      b_off[i] = (uint32_t)n * (uint32_t)K + lchunk * 8;
    }
  }
  // In GEMM1, rows 0..127 of the B tile are gate rows (waves 0, 1) and rows
  // 128..255 up rows (waves 2, 3).
  const uint16_t* __restrict__ Bw = (GATED && wave >= 2) ? B1b : B0b;

#define MOE_BIG_ISSUE(sA_, sB_, k0)                                          \
  _Pragma("unroll") for (int i = 0; i < 8; ++i) {                            \
    load_block_to_lds(Ab, a_off[i] + (k0), &sA_[(wave * 8 + i) * 64]);       \
    load_block_to_lds(Bw, b_off[i] + (k0), &sB_[(wave * 8 + i) * 64]);       \
  }

  // ---- wave tile
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  const bool active = rows > wm * 128;  // wave has rows of this tile

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#define MOE_BIG_COMPUTE(sA_, sB_)                                                                        \
  if (active) {                                                                                          \
    _Pragma("unroll") for (int ks = 0; ks < BK / 16; ++ks) {                                             \
      const int ch = ks * 2 + lk;                                                                        \
      bf16x8 af[4], bfr[4];                                                                              \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                    \
        const int R = wm * 128 + i * 32 + lr;                                                            \
        af[i] = *(const bf16x8*)&sA_[lds_chunk(R, ch)];                                                  \
      }                                                                                                  \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                    \
        const int R = GATED ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32 + lr) : (wn * 128 + j * 32 + lr); \
        bfr[j] = *(const bf16x8*)&sB_[lds_chunk(R, ch)];                                                 \
      }                                                                                                  \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                      \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                    \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);      \
    }                                                                                                    \
  }

  // vmcnt(0): this wave's direct-to-LDS loads have landed; the barrier then
  // publishes every wave's loads and retires the reads of the other stage.
#define MOE_BIG_SYNC()                               \
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   \
  __syncthreads();

  const int KT = K / BK;
  MOE_BIG_ISSUE(sA0, sB0, 0)
  MOE_BIG_SYNC()
  for (int kt = 0; kt < KT; kt += 2) {
    if (kt + 1 < KT) { MOE_BIG_ISSUE(sA1, sB1, (kt + 1) * BK) }
    MOE_BIG_COMPUTE(sA0, sB0)
    MOE_BIG_SYNC()
    if (kt + 1 >= KT) break;
    if (kt + 2 < KT) { MOE_BIG_ISSUE(sA0, sB0, (kt + 2) * BK) }
    MOE_BIG_COMPUTE(sA1, sB1)
    MOE_BIG_SYNC()
  }
#undef MOE_BIG_ISSUE
#undef MOE_BIG_COMPUTE
#undef MOE_BIG_SYNC

  // ---- epilogue. 32x32 result layout: lane holds column (lane & 31) and, in
  // register r, row 8 (r / 4) + 4 (lane / 32) + (r % 4).
  if (!active) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 128 + i * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
      if (row >= rows) continue;
      uint16_t* crow = p.C + (size_t)(row0 + row) * N;
      if (GATED) {
        const float w = p.row_w[row0 + row];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 64 + j * 32 + lr;
          if (n < N) crow[n] = f32_to_bf16_rne(gated_act(p.act, acc[i][j][r], acc[i][j + 2][r]) * w);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 128 + j * 32 + lr;
          if (n < N) crow[n] = f32_to_bf16_rne(acc[i][j][r]);
        }
      }
    }
  }
}

}  // namespace big
}  // namespace moe
