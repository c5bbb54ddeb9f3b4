// Grouped GEMM on bf16 MFMA for many rows per segment (prefill).
//
// moonep_experts page, moonep_grouped_gemm: every segment's rows are
// multiplied by the transpose of that segment's [N, K] weight, weights stored
// [G, N, K] with K contiguous; segments with no rows are skipped (module
// docstring). GEMM1 fuses the gate and up projections and applies the
// activation times the per-row route weight in its epilogue (module docstring:
// the route weight is applied to the activation); GEMM2 is the down projection.
//
// Tile: 256 rows x 256 weight rows, 64 K per stage, 8 waves (two per SIMD),
// each wave a 128 x 64 block of v_mfma_f32_32x32x16_bf16 results (128 fp32
// accumulators per lane, so two waves fit a SIMD's registers). For GEMM1 the
// 256 weight rows are 128 gate rows and the same 128 up rows, and each wave
// holds gate and up accumulators for the same 128 x 32 outputs. A wave issues
// in order, so a lone wave whose load, LDS read or barrier stalls leaves its
// SIMD's matrix unit idle; with two waves per SIMD one issues MFMAs while the
// other waits. Both operands go from HBM straight into LDS with
// global_load_lds_dwordx4 (no staging registers) through two 64 KB stages:
// the loads of stage s+1 run under the MFMAs of stage s. Only vmcnt(0)
// reliably orders the completion of direct-to-LDS loads, so a wave waits for
// all of its loads before each stage barrier; 64 K per stage keeps the
// barriers and the load instructions per MFMA few. The 16-byte chunks of
// every row are XOR-swizzled so that the MFMA operand reads are bank-conflict
// free. In a partial row tile, 8-row blocks of A that lie past the segment
// end are not loaded (their rows of the product are garbage and dropped, and
// a row of the product depends on its own A row only), the other rows past
// the end load a valid row of the tile; waves whose 128 rows are all past
// the end skip their MFMAs.
#pragma once

#include "common.hpp"

namespace moe {
namespace big {

constexpr int BM = 256;  // rows per tile
constexpr int BN = 256;  // weight rows per tile (GEMM1: 128 gate + 128 up)
constexpr int BK = 64;   // K per stage
constexpr int NS = 2;    // LDS stages: the loads of stage s+1 run during stage s
constexpr int NT = 512;  // threads (8 waves)
constexpr int STAGE_U4 = BM * BK / 8;  // 16-byte slots per operand per stage (32 KB)
constexpr int KS = BK / 16;            // MFMA k-substeps per stage

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
  int32_t gn;              // column tiles per tile group
  int32_t xcd_remap;       // 1: renumber workgroups so consecutive tiles share an XCD
  int32_t persistent;      // 1: one workgroup per compute unit, looping over lockstep rounds of tiles
  int32_t s_cap;           // GEMM2: at most this many K ranges per tile (1 = no split)
  int32_t ncu;             // compute units of the device (one block each)
  int64_t c_split;         // elements between the partial outputs of consecutive K ranges
  uint16_t* C;             // [rows, N] bf16 output, sorted row order (GEMM2 split: [S, rows, N])
  const float* row_w;      // GEMM1: route weight per sorted row, or nullptr (weight already on the input)
  ActParams act;
  ExpertParams ep;         // per-expert activation parameters and fc1 / fc2 scales
};

// A stage holds 256 rows x 64 K (128 bytes = eight 16-byte chunks per row)
// of A, then the same of B. Chunk c of row r sits in slot c ^ ((r >> 1) & 7):
// ds_read_b128 serves 16 lanes per pass from a 256-byte bank window (two
// rows), and the 16 consecutive rows one MFMA operand read touches fall on 16
// distinct 16-byte banks.
__device__ __forceinline__ int lds_slot(int row, int chunk) {
  return row * (BK / 8) + (chunk ^ ((row >> 1) & 7));
}

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Workgroup barrier without a memory fence. __syncthreads() would make the
// compiler wait for every outstanding direct-to-LDS load (vmcnt(0)), which
// cancels the loads running ahead; instead each wave first waits (vmcnt(N))
// for the stage about to be read, then meets the others here. The "memory"
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N); gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// (7 = no wait) in 6:4, lgkmcnt (15 = no wait) in 11:8.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// MFMA operand reads are inline-asm ds_read_b128: the compiler's wait-count
// pass would otherwise put a vmcnt(0) in front of every LDS read because it
// cannot tell the stage being read from the stages still being filled by
// direct-to-LDS loads. The reads are then completed by an explicit
// lgkmcnt(0) that also names the destination registers, so nothing uses them
// earlier. The reads of one k-substep share an address register; the
// per-fragment row offsets go in the immediate field.
#define MOE_LGKM_WAIT_TIE(a, b)                                                                \
  asm volatile("s_waitcnt lgkmcnt(0)"                                                          \
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]))

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// Epilogue of a wave's 128 x 64 block of 32x32 MFMA results (GEMM1: gate
// results in acc[i][0], up in acc[i][1], for the same 128 x 32 outputs).
// 32x32 result layout: lane holds column (lane & 31) and, in register r, row
// 8 (r / 4) + 4 (lane / 32) + (r % 4) of the 32-row block i. Results go
// through the wave's own 16 KB of LDS (free once every wave has finished its
// operand reads) so that every lane stores 16 contiguous bytes: 128 rows x 32
// columns per pass, rows padded to 40 elements against bank conflicts.
// GEMM1 writes act = f(gate * es, up * es) * route weight; GEMM2 down * es.
// GEMM1's route weights of the block's 128 rows go through the same LDS
// region first (two loads per lane, one wait), so the activation math reads
// four rows' weights with one LDS read instead of waiting on a global load
// per group of rows.
// wrows: rows of the block inside the segment; wrow0: first output row;
// col0: first output column.
template <bool GATED, int AK = 0>
__device__ __forceinline__ void store_block_bf16(const f32x16 (&acc)[4][2], lds_u32x4* smem, int wave, int wrows,
                                                 int wrow0, int col0, int N, uint16_t* __restrict__ Cs,
                                                 const float* row_w, const ActParams& ap, float es) {
  constexpr int LDR = 40;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lk = lane >> 5;
  lds_u16* sc = (lds_u16*)&smem[wave * 1024];
  // row weights after the 128 x LDR staged values (10 KB of the wave's 16 KB)
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  typedef __attribute__((address_space(3))) float lds_float;
  lds_float* wl = (lds_float*)(sc + 128 * LDR);
  if (GATED) {
    const float w0 = (row_w && lane < wrows) ? row_w[wrow0 + lane] : 1.f;
    const float w1 = (row_w && 64 + lane < wrows) ? row_w[wrow0 + 64 + lane] : 1.f;
    wl[lane] = w0;
    wl[64 + lane] = w1;
  }
  const int cc = lane & 3;  // 16-byte chunk of a staged 64-byte row
  const int rr = lane >> 2; // staged row within a group of 16
#pragma unroll
  for (int pass = 0; pass < (GATED ? 1 : 2); ++pass) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int rbase = i * 32 + rq * 8 + lk * 4;  // 4 consecutive rows r = rq*4 + 0..3
        f32x4 w4 = {1.f, 1.f, 1.f, 1.f};
        if (GATED) w4 = *(const lds_f32x4*)&wl[rbase];
#pragma unroll
        for (int r3 = 0; r3 < 4; ++r3) {
          const int r = rq * 4 + r3;
          float v;
          if (GATED) v = gated_act_k<AK>(ap, acc[i][0][r] * es, acc[i][1][r] * es) * w4[r3];
          else v = acc[i][pass][r] * es;
          const __bf16 h = (__bf16)v;
          sc[(rbase + r3) * LDR + lr] = *(const uint16_t*)&h;
        }
      }
    }
    const int c = col0 + pass * 32 + cc * 8;
    if (c < N) {
#pragma unroll 4
      for (int t = 0; t < 8; ++t) {
        const int row = t * 16 + rr;
        if (row < wrows)
          *(u32x4*)(Cs + (size_t)(wrow0 + row) * N + c) = *(const lds_u32x4*)&sc[row * LDR + cc * 8];
      }
    }
  }
}

// Work item -> (row tile, column tile, K range). Items: groups of gn column
// tiles, row tiles inside a group, column tile fastest, K range fastest of
// all (GEMM2 may split K into nsplit ranges when there are too few tiles to
// fill the last round; each range writes its own partial output, summed by
// the combine).
template <class P>
__device__ __forceinline__ void item_tile(const P& p, int item, int mtl, int nsplit, int& mt, int& nt,
                                          int& split) {
  split = item % nsplit;
  const int tl = item / nsplit;
  const int full = p.n_tiles / p.gn;  // groups of exactly gn column tiles
  if (tl < full * mtl * p.gn) {
    const int span = mtl * p.gn;
    const int grp = tl / span;
    const int r_in = tl - grp * span;
    mt = r_in / p.gn;
    nt = grp * p.gn + (r_in - mt * p.gn);
  } else {  // the last, narrower group
    const int gl = p.n_tiles - full * p.gn;
    const int r_in = tl - full * mtl * p.gn;
    mt = r_in / gl;
    nt = full * p.gn + (r_in - mt * gl);
  }
}

template <bool GATED, int AK>
__device__ __forceinline__ void gemm_tile(const Params& p, int mt, int nt, int split, int nsplit,
                                          lds_u32x4* smem) {
  constexpr uint32_t STAGE_BYTES = 2 * STAGE_U4 * 16;
  constexpr uint32_t B_HALF = STAGE_U4 * 16;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA targets go in M0

  const int seg = p.tile_seg[mt];
  const int row0 = p.tile_row0[mt];
  const int rows = min(BM, p.seg_end[seg] - row0);
  const int N = p.N, K = p.K;
  const int n0 = nt * (GATED ? BN / 2 : BN);

  // ---- direct-to-LDS load assignment. One wave instruction fills a 1 KB LDS
  // block = 8 rows of a stage; lane l writes slot l of it, i.e. row l/8, slot
  // l%8, which holds global chunk (l%8) ^ ((row >> 1) & 7). Wave w fills
  // blocks 4w..4w+3 (rows 32w..32w+31) of the A and of the B half.
  // 32-bit byte offsets: the host keeps T*H, M*I and N*K below 2^31 elements.
  // This block's K range: stages [st_lo, st_lo + KT) of K / BK.
  const int st_lo = split * (K / BK) / nsplit;
  const int KT = (split + 1) * (K / BK) / nsplit - st_lo;
  const uint32_t kb0 = (uint32_t)st_lo * BK * 2u;
  const char* __restrict__ Ab = (const char*)p.A;
  const char* __restrict__ B0b = (const char*)(p.B0 + (size_t)seg * N * K);
  const char* __restrict__ B1b = GATED ? (const char*)(p.B1 + (size_t)seg * N * K) : B0b;
  uint32_t a_off[4], b_off[4];
  {
    const int first = p.a_perm ? p.a_perm[row0] / p.a_div : row0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 32 + i * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ ((r >> 1) & 7);
      int arow = first;
      if (r < rows) arow = p.a_perm ? p.a_perm[row0 + r] / p.a_div : row0 + r;
      a_off[i] = ((uint32_t)arow * (uint32_t)K + chunk * 8) * 2u + kb0;
      const int n = min(n0 + (GATED ? (r & 127) : r), N - 1);
      b_off[i] = ((uint32_t)n * (uint32_t)K + chunk * 8) * 2u + kb0;
    }
  }
  // In GEMM1, rows 0..127 of the B half are gate rows (waves 0-3) and rows
  // 128..255 up rows (waves 4-7).
  const char* __restrict__ Bw = (GATED && wave >= 4) ? B1b : B0b;

  // one direct-to-LDS load: q = 0..3 A rows 32w + 8q..; q = 4..7 B rows
#define MOE_BIG_DMA(st, kbytes, q)                                                                           \
  {                                                                                                          \
    const int qq = (q) & 3;                                                                                  \
    if ((q) < 4) {                                                                                           \
      if (wave * 32 + qq * 8 < rows)                                                                         \
        __builtin_amdgcn_global_load_lds(Ab + (a_off[qq] + (kbytes)),                                        \
                                         &smem[(st) * 2 * STAGE_U4 + (wave * 4 + qq) * 64], 16, 0, 0);        \
    } else                                                                                                   \
      __builtin_amdgcn_global_load_lds(Bw + (b_off[qq] + (kbytes)),                                          \
                                       &smem[(st) * 2 * STAGE_U4 + STAGE_U4 + (wave * 4 + qq) * 64], 16, 0, 0); \
  }

  // ---- wave tile: 128 rows x 64 weight rows (GEMM1: 32 gate + the same 32 up)
  const int wm = wave >> 2, wn = wave & 3;
  // Waves 4-7 (rows 128..255) have nothing to do in a tile of at most 128
  // rows (the last tile of a segment); they share their SIMDs with waves 0-3,
  // which then get the matrix units to themselves. They still load and meet
  // the barriers.
  const bool active = rows > wm * 128;
  const int lr = lane & 31, lk = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  uint32_t a_lane[KS], b_lane[KS];  // per k-substep byte address of fragment 0 inside a stage
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    a_lane[ks] = lds0 + 16u * lds_slot(wm * 128 + lr, ks * 2 + lk);
    b_lane[ks] = lds0 + B_HALF + 16u * lds_slot((GATED ? wn * 32 : wn * 64) + lr, ks * 2 + lk);
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 fa[4], fb[2], ga[4], gb[2];
  // One fragment read: q = 0..3 A fragment q (rows +32 q, 4096 bytes apart),
  // q = 4, 5 B fragment q-4 (GEMM1: gate rows 0, up rows +128, i.e. 0 and
  // 16384 bytes; GEMM2: rows +32 (q-4)).
#define MOE_DSR(d, addr, off) asm volatile("ds_read_b128 %0, %1 offset:" #off : "=v"(d) : "v"(addr))
#define MOE_BIG_READ1(dA, dB, st, ks, q)                                 \
  {                                                                      \
    const uint32_t aa = a_lane[ks] + (uint32_t)(st) * STAGE_BYTES;       \
    const uint32_t bb = b_lane[ks] + (uint32_t)(st) * STAGE_BYTES;       \
    switch (q) {                                                         \
      case 0: MOE_DSR(dA[0], aa, 0); break;                              \
      case 1: MOE_DSR(dA[1], aa, 4096); break;                           \
      case 2: MOE_DSR(dA[2], aa, 8192); break;                           \
      case 3: MOE_DSR(dA[3], aa, 12288); break;                          \
      case 4: MOE_DSR(dB[0], bb, 0); break;                              \
      default: if (GATED) MOE_DSR(dB[1], bb, 16384); else MOE_DSR(dB[1], bb, 4096); break; \
    }                                                                    \
  }
  // MFMAs 2k, 2k+1 of an 8-MFMA batch (A fragment k, B fragments 0 and 1)
#define MOE_BIG_MFMA2(dA, dB, k)                                                                    \
  if (ACT_) {                                                                                       \
    acc[k][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dA[k], dB[0], acc[k][0], 0, 0, 0);          \
    acc[k][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dA[k], dB[1], acc[k][1], 0, 0, 0);          \
  }
  // one k-substep: MFMAs on (cA, cB) interleaved with the reads of the next
  // fragments (nA, nB) from stage buffer nst, substep nks, and with four of
  // this wave's loads of the next stage (q0..q0+3 when dma)
#define MOE_BIG_SUBSTEP(cA, cB, nA, nB, nst, nks, rd, dma, q0)                  \
  {                                                                              \
    MOE_LGKM_WAIT_TIE(cA, cB);                                                   \
    _Pragma("unroll") for (int k = 0; k < 4; ++k) {                              \
      if (dma) {                                                                 \
        MOE_BIG_DMA(stn, kl, 2 * k)                                              \
        MOE_BIG_DMA(stn, kl, 2 * k + 1)                                          \
      }                                                                          \
      if (rd) {                                                                  \
        MOE_BIG_READ1(nA, nB, nst, nks, k)                                       \
        if (k < 2) MOE_BIG_READ1(nA, nB, nst, nks, 4 + k)                        \
      }                                                                          \
      MOE_BIG_MFMA2(cA, cB, k)                                                   \
      __builtin_amdgcn_sched_barrier(0);                                         \
    }                                                                            \
  }

  // prologue: stage 0
#pragma unroll
  for (int q = 0; q < 8; ++q) MOE_BIG_DMA(0, 0u, q)
  wait_vmcnt<0>();
  stage_barrier();
#pragma unroll
  for (int q = 0; q < 6; ++q) MOE_BIG_READ1(fa, fb, 0, 0, q)

  // Stage s (buffer st = s & 1): the loads of stage s+1 go into the other
  // buffer, which every wave finished reading before the last barrier; they
  // are issued during the first two k-substeps (one per MFMA pair). Each
  // k-substep's MFMAs run while the next substep's fragments are read. In the
  // last substep, after its first MFMA pair, the wave waits for its loads of
  // stage s+1 (issued two substeps earlier; only vmcnt(0) orders direct-to-LDS
  // loads reliably) and meets the others at the barrier; the reads of
  // (s+1, 0) then go with the remaining MFMA pairs.
  // one stage; LOAD: stage s + 1 exists (its loads are issued here)
#define MOE_BIG_STAGE(LOAD)                                      \
  {                                                              \
    const int stn = st ^ 1;                                      \
    const uint32_t kl = (uint32_t)(s + 1) * BK * 2u;             \
    MOE_BIG_SUBSTEP(fa, fb, ga, gb, st, 1, true, LOAD, 0)        \
    MOE_BIG_SUBSTEP(ga, gb, fa, fb, st, 2, true, false, 0)       \
    MOE_BIG_SUBSTEP(fa, fb, ga, gb, st, 3, true, false, 0)       \
    MOE_LGKM_WAIT_TIE(ga, gb);                                   \
    _Pragma("unroll") for (int k = 0; k < 4; ++k) {              \
      if (LOAD && k >= 1) {                                      \
        MOE_BIG_READ1(fa, fb, stn, 0, 2 * (k - 1))               \
        MOE_BIG_READ1(fa, fb, stn, 0, 2 * (k - 1) + 1)           \
      }                                                          \
      MOE_BIG_MFMA2(ga, gb, k)                                   \
      __builtin_amdgcn_sched_barrier(0);                         \
      if (LOAD && k == 0) {                                      \
        wait_vmcnt<0>();                                         \
        stage_barrier();                                         \
      }                                                          \
    }                                                            \
    st = stn;                                                    \
  }
  // The K loop exists twice, for waves with and without rows (ACT_), and its
  // last stage is peeled, so the loop body has no branches.
#define MOE_BIG_KLOOP                                            \
  {                                                              \
    int st = 0, s = 0;                                           \
    for (; s + 1 < KT; ++s) MOE_BIG_STAGE(true)                  \
    MOE_BIG_STAGE(false)                                         \
  }
  if (active) {
    constexpr bool ACT_ = true;
    MOE_BIG_KLOOP
  } else {
    constexpr bool ACT_ = false;
    MOE_BIG_KLOOP
  }
#undef MOE_BIG_KLOOP
#undef MOE_BIG_STAGE
#undef MOE_BIG_DMA
#undef MOE_DSR
#undef MOE_BIG_READ1
#undef MOE_BIG_MFMA2
#undef MOE_BIG_SUBSTEP
  // every wave has finished its LDS reads: the stage buffers are free for the
  // epilogue's staging
  wait_vmcnt<0>();
  stage_barrier();

  // ---- epilogue
  if (!active) return;
  store_block_bf16<GATED, AK>(acc, smem, wave, min(128, rows - wm * 128), row0 + wm * 128,
                          n0 + (GATED ? wn * 32 : wn * 64), p.N, p.C + (size_t)split * p.c_split,
                          GATED ? p.row_w : nullptr, act_for(p.act, p.ep, seg),
                          scale_for(GATED ? p.ep.fc1 : p.ep.fc2, seg));  // fc1 on gate and up, fc2 on down
}

// Only the device knows the number of row tiles, so the grid covers an upper
// bound and the items are numbered compactly over the live ones.
// One tile per workgroup: blocks past the last item exit, and they are the
// last blocks dispatched (blocks that exit at once, interleaved with live
// ones, have left whole shader engines idle). With xcd_remap (the hardware
// sends workgroup b to XCD b mod 8), each XCD takes a contiguous run of
// items, so tiles that share weight and row panels share an L2.
// Persistent (grid = a multiple of 8 workgroups, one per compute unit): in
// round r, the S = grid / 8 workgroups of XCD x take the S consecutive items
// of block 8 r + x, so each XCD's compute units run one block of tiles at a
// time, in step, and tiles of a block read the same panels of A and B at the
// same K at about the same time.
template <bool GATED, int AK>
__global__ __launch_bounds__(NT, 1) void k_gemm(const Params p) {
  // NS stages of [A 32 KB | B 32 KB]
  __shared__ u32x4 smem_arr[NS * 2 * STAGE_U4];
  lds_u32x4* smem = (lds_u32x4*)smem_arr;
  const int mtl = p.status[2];
  int nsplit = 1;
  if (!GATED && p.s_cap > 1) nsplit = split_k_count(mtl * p.n_tiles, p.K / BK, p.ncu, p.s_cap);
  const int n_live = mtl * p.n_tiles * nsplit;
  int mt, nt, split;
  if (p.persistent) {
    const int S = gridDim.x >> 3, x = blockIdx.x & 7, j = blockIdx.x >> 3;
    for (int r = 0;; ++r) {
      const int item = (r * 8 + x) * S + j;
      if (item >= n_live) break;
      if (r) stage_barrier();  // every wave has read its staged results of the last tile
      item_tile(p, item, mtl, nsplit, mt, nt, split);
      gemm_tile<GATED, AK>(p, mt, nt, split, nsplit, smem);
    }
    return;
  }
  int item = blockIdx.x;
  if (p.xcd_remap) {
    const int per = (n_live + 7) >> 3;
    const int j = blockIdx.x >> 3;
    if (j >= per) return;
    item = (blockIdx.x & 7) * per + j;
  }
  if (item >= n_live) return;
  item_tile(p, item, mtl, nsplit, mt, nt, split);
  gemm_tile<GATED, AK>(p, mt, nt, split, nsplit, smem);
}

}  // namespace big
}  // namespace moe
