// Grouped GEMM for the cold segments of a prefill problem: segments with at
// most 32 rows, whose weights are read once for a handful of rows.
//
// Same grouped-GEMM definition as the prefill kernel (moonep_experts page,
// moonep_grouped_gemm; module docstring: empty segments skipped, the route
// weight applied to the activation); only the segments differ: the align
// lists the segments of 1..32 rows apart from the tiled ones, and this
// kernel takes those.
//
// Such a segment is a weight stream: its GEMM1 reads the expert's whole gate
// and up weights for at most 32 rows, so its time is HBM time. Run inside the
// 256-row tile kernel it holds a compute unit for as long as a full tile while
// the unit's matrix cores idle. This kernel is made to run beside that one
// instead, on a second stream: four waves, at most 64 VGPRs each and 9 KB of
// LDS, so that one of its workgroups fits on a compute unit next to a 256-row
// tile workgroup (whose 16 waves leave 64 VGPRs per SIMD and 32 KB of LDS
// free), and the weight streams overlap the tiles' MFMA work. Persistent: one
// workgroup per compute unit, items = (cold segment, column tile), segment
// major so a segment's rows stay in L2 across its column tiles.
//
// Item: up to 32 rows (two 16-row blocks; the second is skipped when the
// segment has at most 16 rows) x 64 outputs. Wave w owns 16 weight rows of
// each of two streams: GEMM1 gate rows c0..c0+15 and the same up rows
// (c0 = 64 nt + 16 w, 16 activation columns), GEMM2 rows c0..c0+15 and
// c0+16..c0+31 (c0 = 128 nt + 32 w). v_mfma_f32_16x16x32_bf16: in a 32-K
// step, lane l holds K values 8 (l / 16)..8 (l / 16)+7 of row l % 16 (A) and of
// weight row l % 16 (B); the result lane holds column l % 16, rows
// 4 (l / 16)..4 (l / 16)+3. The weights go from memory into registers two
// steps ahead (16 lanes read 64 contiguous bytes of each of 16 rows, the next
// step the rest of those 128-byte lines); the rows are staged through LDS 64 K
// at a time (double-buffered), loaded one chunk ahead. With the weights in
// the operand-block layout (PK; the layout is defined beside the tile kernel)
// a step's 16 rows are one contiguous 1 KB block already in operand order,
// lane l's 16 bytes at 16 l: whole lines, consecutive lanes on consecutive
// bytes.
#pragma once

#include "common.hpp"

namespace moe {
namespace cold {

constexpr int NT = 256;       // threads (4 waves)
constexpr int MAX_ROWS = 32;  // rows of the largest cold segment
constexpr int KC = 64;        // K per staged chunk of rows
constexpr int LROW = KC + 8;  // staged row, padded by 16 bytes against bank conflicts

__host__ __device__ constexpr int block_cols(bool gated) { return gated ? 64 : 128; }

struct Params {
  const uint16_t* A;         // rows [*, K] bf16
  const int32_t* a_perm;     // sorted row -> flat slot, or nullptr when A is in sorted row order
  int32_t a_div;             // flat slot -> A row divisor (k)
  const uint16_t* B0;        // [G, N, K] (gate or down)
  const uint16_t* B1;        // [G, N, K] (up) for GEMM1
  int32_t N, K;
  const int32_t* cold_seg;   // cold segment ids, status[4] of them
  const int32_t* seg_end;    // cumulative end offsets
  const int32_t* status;
  int32_t n_tiles;           // column tiles: ceil(N / block_cols)
  uint16_t* C;               // [rows, N] bf16 output, sorted row order (GEMM2 split: [S, rows, N])
  const float* row_w;        // GEMM1: route weight per sorted row, or nullptr
  // GEMM2 when the tiled kernel splits K into ranges with partial outputs
  // (split_k_count over its tiles, as the tiled kernel and the combine
  // compute it): a cold row's result goes to the first, zeros to the others
  int64_t c_split;
  int32_t s_cap, ncu, tiled_cols, tiled_kt;
  ActParams act;
  ExpertParams ep;
};

template <bool GATED, int AK, bool PK>
__global__ __launch_bounds__(NT, 8) void k_cold(const Params p) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][MAX_ROWS * LROW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int N = p.N, K = p.K;
  const int n_items = p.status[4] * p.n_tiles;
  const int nch = K / KC;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int cs = item / p.n_tiles, nt = item - cs * p.n_tiles;
    const int seg = p.cold_seg[cs];
    const int row0 = seg ? p.seg_end[seg - 1] : 0;
    const int rows = p.seg_end[seg] - row0;  // 1 .. MAX_ROWS
    const bool two = rows > 16;

    // this lane's weight rows (rows past N read row N - 1, or the last
    // 16-row block; never stored); a lane's operand of 32-K step s is at
    // b0 + s * SSTEP (and b1 + s * SSTEP)
    const int c0 = GATED ? nt * 64 + wave * 16 : nt * 128 + wave * 32;
    const size_t wbase = (size_t)seg * N * K;
    constexpr int SSTEP = PK ? 512 : 32;
    const uint16_t* b0;
    const uint16_t* b1;
    if constexpr (PK) {
      const size_t brow = (size_t)(K / 32) * 512;  // elements of a 16-row block row
      const int nb0 = min(c0 >> 4, N / 16 - 1), nb1 = min((c0 >> 4) + 1, N / 16 - 1);
      b0 = p.B0 + wbase + nb0 * brow + 8 * lane;
      b1 = (GATED ? p.B1 + wbase + nb0 * brow : p.B0 + wbase + nb1 * brow) + 8 * lane;
    } else {
      b0 = p.B0 + wbase + (size_t)min(c0 + l16, N - 1) * K + 8 * q;
      b1 = (GATED ? p.B1 + wbase + (size_t)min(c0 + l16, N - 1) * K
                  : p.B0 + wbase + (size_t)min(c0 + 16 + l16, N - 1) * K) + 8 * q;
    }
    // this thread's 16-byte piece of a staged chunk (32 rows x 64 K): row
    // tid / 8, K values 8 (tid % 8)..; rows past the segment end read its last
    // row
    const uint16_t* ap;
    {
      const int r = min(tid >> 3, rows - 1);
      const int arow = p.a_perm ? p.a_perm[row0 + r] / p.a_div : row0 + r;
      ap = p.A + (size_t)arow * K + 8 * (tid & 7);
    }
    const int sl = (tid >> 3) * LROW + 8 * (tid & 7);  // its place in a staging buffer
    __syncthreads();  // the last item's reads of the staging buffers are done
    u32x4 ar = *(const u32x4*)ap;
    *(u32x4*)&sa[0][sl] = ar;
    // weights are read once: non-temporal loads (nt), so that the stream
    // leaves the cached panels of the tiled kernel beside it in place
    u32x4 wb[2][2];  // weights of two steps: [step & 1][stream]
    wb[0][0] = __builtin_nontemporal_load((const u32x4*)b0);
    wb[0][1] = __builtin_nontemporal_load((const u32x4*)b1);
    wb[1][0] = __builtin_nontemporal_load((const u32x4*)(b0 + SSTEP));
    wb[1][1] = __builtin_nontemporal_load((const u32x4*)(b1 + SSTEP));
    __syncthreads();

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nch; ++c) {
      const bool more = c + 1 < nch;
      if (more) ar = *(const u32x4*)(ap + (c + 1) * KC);
      const uint16_t* sbuf = sa[c & 1];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int s = 2 * c + j;  // K step (32 values)
        const bf16x8 a0 = *(const bf16x8*)&sbuf[l16 * LROW + 32 * j + 8 * q];
        const bf16x8 bv0 = *(const bf16x8*)&wb[j][0];
        const bf16x8 bv1 = *(const bf16x8*)&wb[j][1];
        acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bv0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bv1, acc[0][1], 0, 0, 0);
        if (two) {
          const bf16x8 a1 = *(const bf16x8*)&sbuf[(16 + l16) * LROW + 32 * j + 8 * q];
          acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bv0, acc[1][0], 0, 0, 0);
          acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bv1, acc[1][1], 0, 0, 0);
        }
        if (s + 2 < 2 * nch) {
          wb[j][0] = __builtin_nontemporal_load((const u32x4*)(b0 + (s + 2) * SSTEP));
          wb[j][1] = __builtin_nontemporal_load((const u32x4*)(b1 + (s + 2) * SSTEP));
        }
      }
      if (more) *(u32x4*)&sa[(c + 1) & 1][sl] = ar;
      __syncthreads();
    }

    // epilogue: GEMM1 act = f(gate * es, up * es) * route weight, GEMM2 down * es
    int nsplit = 1;
    if (!GATED && p.s_cap > 1) nsplit = split_k_count(p.status[2] * p.tiled_cols, p.tiled_kt, p.ncu, p.s_cap);
    const ActParams ap_ = act_for(p.act, p.ep, seg);
    const float es = scale_for(GATED ? p.ep.fc1 : p.ep.fc2, seg);  // fc1 on gate and up, fc2 on down
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if (rb == 1 && !two) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + 4 * q + i;
        if (r >= rows) continue;
        uint16_t* dst = p.C + (size_t)(row0 + r) * N;
        if (GATED) {
          const int col = c0 + l16;
          if (col < N) {
            const float wr = p.row_w ? p.row_w[row0 + r] : 1.f;
            dst[col] = f32_to_bf16_rne(gated_act_k<AK>(ap_, acc[rb][0][i] * es, acc[rb][1][i] * es) * wr);
          }
        } else {
          if (c0 + l16 < N) dst[c0 + l16] = f32_to_bf16_rne(acc[rb][0][i] * es);
          if (c0 + 16 + l16 < N) dst[c0 + 16 + l16] = f32_to_bf16_rne(acc[rb][1][i] * es);
          for (int sp = 1; sp < nsplit; ++sp) {
            if (c0 + l16 < N) dst[sp * p.c_split + c0 + l16] = 0;
            if (c0 + 16 + l16 < N) dst[sp * p.c_split + c0 + 16 + l16] = 0;
          }
        }
      }
    }
  }
}

}  // namespace cold
}  // namespace moe
