// Grouped GEMM on bf16 MFMA for many rows per segment (prefill).
//
// moonep_experts page, moonep_grouped_gemm: every segment's rows are
// multiplied by the transpose of that segment's [N, K] weight, weights stored
// [G, N, K] with K contiguous; segments with no rows are skipped (module
// docstring). GEMM1 fuses the gate and up projections and applies the
// activation times the per-row route weight in its epilogue (module docstring:
// the route weight is applied to the activation); GEMM2 is the down projection.
//
// Tile: 256 rows x 256 weight rows (GEMM1: 128 gate rows and the same 128 up
// rows), 64 K per stage, 16 waves (four per SIMD). Wave w = 4 wm + wn owns
// rows 64 wm..64 wm+63 of the tile and weight rows 64 wn..64 wn+63 (GEMM1:
// gate rows 32 wn.. and the same up rows), a 64 x 64 block of 2 x 2
// v_mfma_f32_32x32x16_bf16 results: 64 accumulator registers, so four waves
// fit a SIMD's registers. The hardware puts wave w on SIMD w mod 4, so each
// SIMD holds the four row blocks of one column block, and in a partial row
// tile (the last of a segment) every SIMD keeps the same share of the MFMAs;
// MFMAs of 32-row fragments past the segment end are skipped.
//
// Loads: both operands go from memory straight into LDS with
// global_load_lds_dwordx4 (1 KB a wave instruction, no staging registers)
// through two 64 KB stages: the loads of stage s+1 run under the MFMAs of
// stage s. Wave w fills rows 16 w..16 w+15 of a stage's A and of its B
// (GEMM1: waves 0-7 gate rows, 8-15 up rows), two 8-row instructions each.
// Sixteen waves rather than eight with 128 x 64 blocks: eight waves read a
// quarter fewer operand bytes from LDS per MFMA, but with two waves per SIMD
// the operand reads and barriers are hidden worse, and the whole kernel
// measured the same or slightly slower. A stage needs 64 KB per 2048 MFMA
// cycles (32 bytes a clock); with the L2 misses of these grouped shapes the
// load path bounds the kernel.
// Weights in the operand-block layout (PK, written once by k_bf16_pack): each
// 16-row x 32-K block of an expert's [N, K] matrix is 1 KB in
// v_mfma_f32_16x16x32_bf16 operand order, so a wave's B instruction copies
// one contiguous block (its 16 rows, half of the stage's K) and the B
// fragments are read from that order instead of the swizzled rows; the
// arithmetic and its order are those of the row layout.
// Only vmcnt(0) reliably orders the completion of these direct-to-LDS
// loads, so a wave waits for all of its loads before each stage barrier. The
// 16-byte chunks of every row are XOR-swizzled so that the MFMA operand
// reads are bank-conflict free. In a partial row tile, 8-row
// blocks of A that lie past the segment end are not loaded (their rows of
// the product are garbage and dropped, and a row of the product depends on
// its own A row only); the other rows past the end load a valid row.
#pragma once

#include "common.hpp"

namespace moe {
namespace big {

constexpr int BM = 256;  // rows per tile
constexpr int BN = 256;  // weight rows per tile (GEMM1: 128 gate + 128 up)
constexpr int BK = 64;   // K per stage
constexpr int NS = 2;    // LDS stages: the loads of stage s+1 run during stage s
constexpr int NW = 16;   // waves
constexpr int NT = NW * 64;
constexpr int KS = BK / 16;  // MFMA k-substeps per stage
constexpr uint32_t STAGE_BYTES = 65536;  // A 32 KB | B 32 KB
constexpr uint32_t B_HALF = 32768;
constexpr int EP_WAVE = NS * (int)STAGE_BYTES / NW;  // epilogue staging bytes per wave (8 KB)

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

// Operand-block layout of a [G, N, K] bf16 weight (N a multiple of 16, K of
// 32): block (g, nb, kb) of 16 rows x 32 K values is 1 KB at byte
// ((g * N / 16 + nb) * K / 32 + kb) * 1024, and its 16-byte piece l (l < 64)
// holds row 16 nb + l % 16, values 32 kb + 8 (l / 16)..+7: the B operand of
// v_mfma_f32_16x16x32_bf16 for those rows and K values, lane by lane. Same
// size as the row layout. In a stage of the tile kernel, B block (w, h) (w =
// 16-row block of the tile, h = K half) lands at B_HALF + (2 w + h) * 1024,
// so a tile row R and 16-byte K chunk c of the stage sit at
// B_HALF + ((R / 16) * 2 + c / 4) * 1024 + (R % 16 + 16 (c % 4)) * 16: rows 32
// apart are 4096 bytes apart, as in the row layout.
__device__ __forceinline__ uint32_t pk_lds_off(int row, int chunk) {
  return (uint32_t)((((row >> 4) * 2 + (chunk >> 2)) * 1024) + ((row & 15) + 16 * (chunk & 3)) * 16);
}

// Writes a [G, N, K] bf16 weight in the operand-block layout (one 16-byte
// piece per thread and step, grid-stride; pieces = G N K / 8).
__global__ __launch_bounds__(256) void k_bf16_pack(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                   int N, int K, long long pieces) {
  const long long nkb = K / 32, nnb = N / 16;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < pieces; i += (long long)gridDim.x * 256) {
    const long long b = i >> 6;
    const int l = (int)(i & 63);
    const long long kb = b % nkb, t = b / nkb;
    const long long nb = t % nnb, g = t / nnb;
    const long long row = g * N + nb * 16 + (l & 15), col = kb * 32 + 8 * (l >> 4);
    *(u32x4*)(dst + i * 8) = *(const u32x4*)(src + row * K + col);
  }
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

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

// Epilogue of a wave's 64 x 64 block (GEMM1: 64 rows x 32 activation
// columns, gate in acc[i][0], up in acc[i][1]). 32x32 result layout: lane
// holds column lane & 31 and, in register r, row 8 (r / 4) + 4 (lane / 32) +
// r % 4 of 32-row block i. Results go through the wave's 8 KB of LDS so that
// every lane stores 16 contiguous bytes.
//  * GEMM2: bf16 of acc * es, 32 rows at a time, rows padded to 72 values;
//    8 lanes write a row's 128 bytes.
//  * GEMM1: bf16 of f(gate * es, up * es) * route weight for all 64 rows,
//    rows padded to 40 values; the rows' route weights are staged after them
//    (one load per lane) and read four rows at a time; 4 lanes write a row's
//    64 bytes.
// nfr: the block's 32-row fragments with rows in the segment (1 or 2).
template <bool GATED, int AK>
__device__ __forceinline__ void store_block(const f32x16 (&acc)[2][2], lds_u8* ws, int lane_in, int nfr, int wrows,
                                            int wrow0, int col0, int N, uint16_t* __restrict__ Cs,
                                            const float* row_w, const ActParams& ap, float es) {
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int lr = lane & 31, lk = lane >> 5;
  if constexpr (!GATED) {
    constexpr int LDR = 72;
    static_assert(32 * LDR * 2 <= EP_WAVE, "GEMM2 staging");
    lds_u16* sh = (lds_u16*)ws;
    const int cc = lane & 7, rr = lane >> 3;
    const bool col_ok = col0 + cc * 8 < N;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i >= nfr) break;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 8 * (r >> 2) + 4 * lk + (r & 3);
          const __bf16 h = (__bf16)(acc[i][j][r] * es);
          sh[rl * LDR + j * 32 + lr] = *(const uint16_t*)&h;
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int rl = t * 8 + rr;
        const u32x4 v = *(const lds_u32x4*)&sh[rl * LDR + cc * 8];
        const int row = 32 * i + rl;
        if (col_ok && row < wrows) *(u32x4*)(Cs + (size_t)(wrow0 + row) * N + col0 + cc * 8) = v;
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    constexpr int LDR = 40;
    static_assert(64 * LDR * 2 + 64 * 4 <= EP_WAVE, "GEMM1 staging");
    lds_u16* sh = (lds_u16*)ws;
    lds_f32* wl = (lds_f32*)(ws + 64 * LDR * 2);
    wl[lane] = (row_w && lane < wrows) ? row_w[wrow0 + lane] : 1.f;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i >= nfr) break;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int rb = 32 * i + 8 * rq + 4 * lk;  // rows rb .. rb + 3
        const f32x4 w4 = *(const lds_f32x4*)&wl[rb];
#pragma unroll
        for (int r3 = 0; r3 < 4; ++r3) {
          const int r = rq * 4 + r3;
          const float v = gated_act_k<AK>(ap, acc[i][0][r] * es, acc[i][1][r] * es) * w4[r3];
          const __bf16 h = (__bf16)v;
          sh[(rb + r3) * LDR + lr] = *(const uint16_t*)&h;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    const int cc = lane & 3, rr = lane >> 2;
    if (col0 + cc * 8 < N) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = t * 16 + rr;
        if (row < wrows)
          *(u32x4*)(Cs + (size_t)(wrow0 + row) * N + col0 + cc * 8) = *(const lds_u32x4*)&sh[row * LDR + cc * 8];
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

template <bool GATED, int AK, bool PK>
__device__ __forceinline__ void gemm_tile(const Params& p, int mt, int nt, int split, int nsplit, lds_u8* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA targets go in M0

  const int seg = p.tile_seg[mt];
  const int row0 = p.tile_row0[mt];
  const int rows = min(BM, p.seg_end[seg] - row0);
  const int N = p.N, K = p.K;
  const int n0 = nt * (GATED ? BN / 2 : BN);

  // ---- loads. Lane l of a wave instruction fills 16-byte slot l of a 1 KB
  // block = 8 rows of the stage: row l / 8, slot l % 8, holding global chunk
  // (l % 8) ^ ((row >> 1) & 7). Block 2 w + q (q = 0, 1) of A and of B.
  // This block's K range: stages [st_lo, st_lo + KT) of K / BK.
  const int st_lo = split * (K / BK) / nsplit;
  const int KT = (split + 1) * (K / BK) / nsplit - st_lo;
  const uint32_t kb0 = (uint32_t)st_lo * BK * 2u;
  const char* __restrict__ Ab = (const char*)p.A;
  const char* __restrict__ B0b = (const char*)(p.B0 + (size_t)seg * N * K);
  const char* __restrict__ B1b = GATED ? (const char*)(p.B1 + (size_t)seg * N * K) : B0b;
  const char* __restrict__ Bw = (GATED && wave >= 8) ? B1b : B0b;
  uint32_t a_off[2], b_off[2];
  {
    const int first = p.a_perm ? p.a_perm[row0] / p.a_div : row0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = wave * 16 + q * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ ((r >> 1) & 7);
      int arow = first;
      if (r < rows) arow = p.a_perm ? p.a_perm[row0 + r] / p.a_div : row0 + r;
      a_off[q] = ((uint32_t)arow * (uint32_t)K + chunk * 8) * 2u + kb0;
      if constexpr (PK) {  // the wave's 16 rows are one block row; instruction q = K half q of the stage
        const int nb = min((n0 >> 4) + (GATED ? (wave & 7) : wave), N / 16 - 1);
        b_off[q] = ((uint32_t)nb * (uint32_t)(K / 32) + 2u * (uint32_t)st_lo + (uint32_t)q) * 1024u + (uint32_t)lane * 16u;
      } else {
        const int n = min(n0 + (GATED ? (r & 127) : r), N - 1);
        b_off[q] = ((uint32_t)n * (uint32_t)K + chunk * 8) * 2u + kb0;
      }
    }
  }
  // 8-row blocks of A past the segment end are not loaded (their rows of the
  // product are dropped); rows past the end inside a loaded block read the
  // segment's first row.
  const bool a_live0 = wave * 16 < rows, a_live1 = wave * 16 + 8 < rows;
#define MOE_W16_DMA(st, kbytes, q)                                                                      \
  {                                                                                                     \
    lds_u8* dst_ = smem + (st) * STAGE_BYTES + (wave * 2 + ((q) & 1)) * 1024;                           \
    if ((q) < 2) {                                                                                      \
      if ((q) == 0 ? a_live0 : a_live1)                                                                 \
        __builtin_amdgcn_global_load_lds(Ab + (a_off[(q) & 1] + (kbytes)), (__attribute__((address_space(3))) void*)dst_, 16, 0, 0); \
    } else {                                                                                            \
      __builtin_amdgcn_global_load_lds(Bw + (b_off[(q) & 1] + (kbytes) * (PK ? 16u : 1u)),              \
                                       (__attribute__((address_space(3))) void*)(dst_ + B_HALF), 16, 0, 0); \
    }                                                                                                   \
  }

  // ---- wave tile
  const int wm = wave >> 2, wn = wave & 3;
  // 32-row fragments of this wave with rows in the segment (MFMAs of the
  // others are skipped)
  const int nfr = min(2, max(0, (rows - wm * 64 + 31) >> 5));
  const int lr = lane & 31, lk = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  uint32_t a_lane[KS], b_lane[KS];  // per k-substep byte address of fragment 0 inside stage 0
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    a_lane[ks] = lds0 + 16u * lds_slot(wm * 64 + lr, ks * 2 + lk);
    b_lane[ks] = lds0 + B_HALF +
                 (PK ? pk_lds_off((GATED ? wn * 32 : wn * 64) + lr, ks * 2 + lk)
                     : 16u * lds_slot((GATED ? wn * 32 : wn * 64) + lr, ks * 2 + lk));
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 fa[2], fb[2], ga[2], gb[2];
  // One fragment read: q = 0, 1 A fragment q (rows +32 q: 4096 bytes); q = 2,
  // 3 B fragment q - 2 (GEMM1: gate rows, then up rows +128 = 16384 bytes;
  // GEMM2: rows +32 = 4096 bytes).
#define MOE_DSR(d, addr, off) asm volatile("ds_read_b128 %0, %1 offset:" #off : "=v"(d) : "v"(addr))
#define MOE_W16_READ1(dA, dB, st, ks, q)                                  \
  {                                                                       \
    const uint32_t aa = a_lane[ks] + (uint32_t)(st) * STAGE_BYTES;        \
    const uint32_t bb = b_lane[ks] + (uint32_t)(st) * STAGE_BYTES;        \
    switch (q) {                                                          \
      case 0: MOE_DSR(dA[0], aa, 0); break;                               \
      case 1: MOE_DSR(dA[1], aa, 4096); break;                            \
      case 2: MOE_DSR(dB[0], bb, 0); break;                               \
      default: if (GATED) MOE_DSR(dB[1], bb, 16384); else MOE_DSR(dB[1], bb, 4096); break; \
    }                                                                     \
  }
#define MOE_W16_WAIT_TIE(a, b) \
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]))
  // MFMA k of a substep: A fragment k / 2 times B fragment k % 2, skipped
  // when the A fragment has no rows in the segment
#define MOE_W16_MFMA(dA, dB, k)                                                                           \
  if (((k) >> 1) < nfr) {                                                                                 \
    acc[(k) >> 1][(k) & 1] =                                                                              \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(dA[(k) >> 1], dB[(k) & 1], acc[(k) >> 1][(k) & 1], 0, 0, 0); \
  }
  // one k-substep: MFMAs on (cA, cB), each followed by one read of the next
  // substep's fragments (nA, nB from stage buffer nst, substep nks)
#define MOE_W16_SUBSTEP(cA, cB, nA, nB, nst, nks)                            \
  {                                                                           \
    MOE_W16_WAIT_TIE(cA, cB);                                                 \
    _Pragma("unroll") for (int k = 0; k < 4; ++k) {                           \
      MOE_W16_READ1(nA, nB, nst, nks, k)                                      \
      MOE_W16_MFMA(cA, cB, k)                                                 \
      __builtin_amdgcn_sched_barrier(0);                                      \
    }                                                                         \
  }

  // prologue: stages 0 and 1 (one into each buffer); stage 0 is read first
#pragma unroll
  for (int q = 0; q < 4; ++q) MOE_W16_DMA(0, 0u, q)
  if (KT > 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) MOE_W16_DMA(1, (uint32_t)(BK * 2), q)
  }
  wait_vmcnt<0>();
  stage_barrier();
#pragma unroll
  for (int q = 0; q < 4; ++q) MOE_W16_READ1(fa, fb, 0, 0, q)

  // Stage s (buffer st = s & 1), with stage s + 1 loading into the other
  // buffer. In the last substep, after the first MFMA, a wave waits for its
  // loads of stage s + 1 and meets the others at the barrier. Past that
  // barrier every wave has read its last fragments of stage s, so the loads
  // of stage s + 2 go into this stage's buffer at once, one with each of the
  // remaining MFMAs, along with the reads of stage s + 1's first fragments:
  // the load path, which bounds the kernel, has work again as soon as a
  // stage's loads are in.
#define MOE_W16_STAGE(LOAD)                                      \
  {                                                              \
    const int stn = st ^ 1;                                      \
    const uint32_t kl2 = (uint32_t)(s + 2) * BK * 2u;            \
    const bool issue2 = LOAD && s + 2 < KT;                      \
    MOE_W16_SUBSTEP(fa, fb, ga, gb, st, 1)                       \
    MOE_W16_SUBSTEP(ga, gb, fa, fb, st, 2)                       \
    MOE_W16_SUBSTEP(fa, fb, ga, gb, st, 3)                       \
    MOE_W16_WAIT_TIE(ga, gb);                                    \
    _Pragma("unroll") for (int k = 0; k < 4; ++k) {              \
      MOE_W16_MFMA(ga, gb, k)                                    \
      __builtin_amdgcn_sched_barrier(0);                         \
      if (LOAD && k == 0) {                                      \
        wait_vmcnt<0>();                                         \
        stage_barrier();                                         \
      }                                                          \
      if (issue2) MOE_W16_DMA(st, kl2, k)                        \
      if (LOAD) MOE_W16_READ1(fa, fb, stn, 0, k)                 \
    }                                                            \
    st = stn;                                                    \
  }
  {
    int st = 0, s = 0;
    for (; s + 1 < KT; ++s) MOE_W16_STAGE(true)
    MOE_W16_STAGE(false)
  }
#undef MOE_W16_STAGE
#undef MOE_W16_SUBSTEP
#undef MOE_W16_MFMA
#undef MOE_W16_WAIT_TIE
#undef MOE_W16_READ1
#undef MOE_DSR
#undef MOE_W16_DMA
  // every wave has finished its LDS reads: the stage buffers are free for the
  // epilogue's staging
  wait_vmcnt<0>();
  stage_barrier();
  if (nfr == 0) return;
  store_block<GATED, AK>(acc, smem + wave * EP_WAVE, lane, nfr, min(64, rows - wm * 64), row0 + wm * 64,
                         n0 + (GATED ? wn * 32 : wn * 64), N, p.C + (size_t)split * p.c_split,
                         GATED ? p.row_w : nullptr, act_for(p.act, p.ep, seg),
                         scale_for(GATED ? p.ep.fc1 : p.ep.fc2, seg));  // fc1 on gate and up, fc2 on down
}

// One tile per workgroup, items numbered compactly over the live tiles (see
// item_tile); the hardware sends workgroup b to XCD b mod 8,
// and each XCD takes a contiguous run of items, so tiles that share weight
// and row panels share an L2. Blocks past the last item exit.
template <bool GATED, int AK, bool PK>
__global__ __launch_bounds__(NT, 1) __attribute__((amdgpu_num_vgpr(96))) void k_gemm(const Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem_arr[NS * STAGE_BYTES];
  const int mtl = p.status[2];
  int nsplit = 1;
  if (!GATED && p.s_cap > 1) nsplit = split_k_count(mtl * p.n_tiles, p.K / BK, p.ncu, p.s_cap);
  const int n_live = mtl * p.n_tiles * nsplit;
  const int per = (n_live + 7) >> 3;
  const int j = blockIdx.x >> 3;
  if (j >= per) return;
  const int item = (blockIdx.x & 7) * per + j;
  if (item >= n_live) return;
  int mt, nt, split;
  item_tile(p, item, mtl, nsplit, mt, nt, split);
  gemm_tile<GATED, AK, PK>(p, mt, nt, split, nsplit, (lds_u8*)smem_arr);
}

}  // namespace big
}  // namespace moe
