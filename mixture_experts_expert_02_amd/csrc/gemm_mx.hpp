// Grouped GEMM with MXFP4 weights and MXFP8 activations for many rows per
// segment (prefill), on the block-scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Same grouped-GEMM definition as the bf16 prefill kernel (moonep_experts
// page, moonep_grouped_gemm; route weight on the activation per the module
// docstring). Weights: e2m1 codes with an e8m0 scale per 32 K values
// (trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase._supports_quant_scheme;
// OCP Microscaling v1.0 reading). Activations: e4m3 codes with an e8m0 scale
// per 32 K values, quantized dynamically (flashinfer_moe_ep page,
// epilogue_from_quant_config), GEMM2's input by GEMM1's epilogue from the
// fp32 activation, with the rule of the MXFP8 decode path.
//
// Tile: 256 rows x 256 weight rows (GEMM1: 128 gate + the same 128 up rows),
// 128 K per stage, 8 waves (two per SIMD), each a 128 x 64 block of 32x32
// results; per 64-K step a wave runs 4 A fragments x 2 B fragments = 8
// MFMAs. A stage holds 32 KB of e4m3 codes (256 rows x 128 bytes), 16 KB of
// e2m1 codes (256 rows x 64 bytes) and a 1 KB scale block for each operand.
// Three stages (150 KB of LDS) let the loads of a stage run two stages ahead
// of its MFMAs: before the stage barrier a wave waits only for the stage
// about to be read (vmcnt = the next-but-one stage's loads still in flight).
// Codes go HBM -> LDS with buffer_load ... lds (16 bytes a lane) through a
// buffer resource over the operand: a lane with nothing to load (rows past
// the segment or past N, K past the end of a row in a half stage) gets an
// offset past the resource's end, which reads zeros without a memory access
// and keeps every wave's load count the same. A rows are XOR-swizzled like
// the bf16 kernel's (16-byte chunk c of row r in slot c ^ ((r >> 1) & 7));
// B rows of 64 bytes put chunk c in slot c ^ ((r >> 2) & 3), so the 16 rows
// one ds_read_b128 pass touches fall on distinct 16-byte banks.
//
// MFMA operand layout (mapped with a probe against a host decoder): the A
// lane (row lane & 31, group q = lane >> 5) holds K values 16q..16q+15 of the
// step in registers 0-3 and 32+16q..32+16q+15 in 4-7; the B lane (column
// lane & 31, group q) holds K values 32q..32q+31, 16 bytes; each lane gives
// the scale of block q of its row or column.
//
// Scale blocks: per row tile (activations) or per expert and column tile
// (weights), and per stage, 1 KB = 256 rows x 4 bytes, a row's 4 blocks of
// the stage in the order (0, 2, 1, 3): the lane of group q reads blocks
// (q, q + 2) as one 16-bit value, whose byte s is the scale of step s (the
// MFMA's scale byte select). k_mx_prep writes the weights' blocks for each
// call and GEMM1's activation blocks from the token rows' scales; GEMM1's
// epilogue writes GEMM2's, since its column tile (128 activation columns) is
// exactly one GEMM2 stage.
//
// Schedule: one workgroup per compute unit, each running a run of tiles with
// the stage stream carried across tile boundaries (see mx_gemm); MFMAs of A
// fragments whose 32 rows lie past the segment are skipped.
#pragma once

#include "common.hpp"
#include "gemm_bf16.hpp"

namespace moe {
namespace mx {

constexpr int BM = 256;                 // rows per tile
constexpr int BN = 256;                 // weight rows per tile (GEMM1: 128 gate + 128 up)
constexpr int BK = 128;                 // K values per stage
constexpr int NS = 3;                   // LDS stages
constexpr int NT = 512;                 // threads (8 waves)
constexpr int A_BYTES = BM * BK;        // e4m3 codes of a stage
constexpr int B_BYTES = BN * BK / 2;    // e2m1 codes of a stage
constexpr int SC_BYTES = 1024;          // scale block of one operand and stage
constexpr int STAGE = A_BYTES + B_BYTES + 2 * SC_BYTES;
constexpr int LOADS = 7;                // load instructions per wave and stage
constexpr uint32_t kNoLoad = 0x80000000u;  // buffer offset past any operand: reads 0

// Packed weights (moe_mx_pack_weights): the kernel's format, made once for a
// set of weights (flashinfer_moe_ep page, process_weights_after_loading: the
// weights are put into the kernel's format before the first forward). For
// each expert, column tile and stage, one PK_STAGE-byte block that is the
// stage's LDS image of the B operand: 256 rows x 64 bytes of e2m1 codes, row
// r's 16-byte chunk c at r * 64 + 16 (c ^ ((r >> 2) & 3)) (GEMM1: rows 0-127
// gate rows n0.., 128-255 the same up rows; codes past N or past K are 0),
// then the 1 KB scale block of those rows (as k_mx_prep makes it). A wave's
// load of 16 rows is then one contiguous 1 KB, whole 128-byte lines, where
// the [E, N, K/2] layout gives 16 rows x 64 bytes. Blocks run column tile
// major, stage minor, expert by expert: GEMM1's experts, then GEMM2's.
constexpr int PK_STAGE = B_BYTES + SC_BYTES;

// position of block b (0..3) of a stage inside a row's 4 scale bytes
__host__ __device__ constexpr int sc_pos(int b) { return ((b & 1) << 1) | (b >> 1); }

__device__ __forceinline__ float sat448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

struct Params {
  const uint8_t* A;        // e4m3 codes, rows of K bytes
  uint32_t a_bytes;        // size of A in bytes
  const int32_t* a_perm;   // sorted row -> flat slot, or nullptr when A is in sorted row order
  int32_t a_div;           // flat slot -> A row divisor (k)
  const uint8_t* A_sc;     // scale blocks [mt_cap][KT]
  const uint8_t* B0;       // e2m1 codes [G, N, K/2] (gate or down)
  const uint8_t* B1;       // (up) for GEMM1
  const uint8_t* B_sc;     // scale blocks [G][n_tiles][KT]
  const uint8_t* Bp;       // packed weights of this GEMM (codes and scale blocks), or nullptr: B0/B1/B_sc
  uint32_t bp_expert;      // bytes of one expert's packed blocks (n_tiles x KT x PK_STAGE)
  int32_t N, K, KT;        // KT = ceil(K / BK); K is a multiple of 64
  const int32_t* tile_seg;
  const int32_t* tile_row0;
  const int32_t* seg_end;
  const int32_t* status;   // status[2] = number of row tiles
  int32_t mt_cap;
  int32_t n_tiles;         // column tiles (GEMM1: ceil(N / 128), GEMM2: ceil(N / 256))
  int32_t gn;              // column tiles per tile group
  int32_t s_cap;           // GEMM2: at most this many K ranges per tile
  int32_t ncu;
  int64_t c_split;         // elements between partial outputs of consecutive K ranges
  uint16_t* C;             // GEMM2: bf16 [rows, N] (split: [S, rows, N])
  uint8_t* Cq;             // GEMM1: e4m3 codes of the activation rows [rows, N]
  uint8_t* Cq_sc;          // GEMM1: their scale blocks [mt_cap][n_tiles] (GEMM2's A_sc)
  const float* row_w;      // GEMM1: route weight per sorted row, or nullptr
  ActParams act;
  ExpertParams ep;
};

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// MXFP8 scale code of a block whose largest magnitude is amax: 2^(e - 8) for
// 2^e <= amax < 2^(e+1), as an e8m0 byte, clamped to [0, 254] (the rule of
// the MXFP8 decode path's epilogue).
__device__ __forceinline__ int mx8_code(float amax) {
  return min(max((int)((__float_as_uint(amax) >> 23) & 0xffu) - 8, 0), 254);
}

// s_waitcnt lgkmcnt(n) (vmcnt and expcnt not waited for); n is a constant
// after unrolling
__device__ __forceinline__ void wait_lgkm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0xc07f); break;
    case 2: __builtin_amdgcn_s_waitcnt(0xc27f); break;
    case 4: __builtin_amdgcn_s_waitcnt(0xc47f); break;
    case 6: __builtin_amdgcn_s_waitcnt(0xc67f); break;
    case 8: __builtin_amdgcn_s_waitcnt(0xc87f); break;
    default: __builtin_amdgcn_s_waitcnt(0xce7f); break;  // 14
  }
}

// One tile's load context for this lane: the tile's place in the problem and
// the per-lane offsets of its loads (see mx_gemm).
struct MxTile {
  int mt, nt, split, seg, row0, rows, KT;
  bool half;                 // the K range ends in a 64-K stage
  uint32_t a_off[4], b_off[2];
  const uint8_t* bbase;      // this wave's weight codes: the expert's gate / up / down rows
  const uint8_t* sc_src;     // this wave's quarter of the scale blocks, first stage of the range
};

// Load assignment. A: wave w fills rows 32w..32w+31, 8 rows x 128 B per
// instruction (lane l: row l / 8, slot l % 8). B: rows 32w..32w+31 of the B
// half, 16 rows x 64 B per instruction (lane l: row l / 4, slot l % 4); in
// GEMM1 waves 0-3 fill the gate rows, 4-7 the up rows. Scales: waves 0-3
// copy a quarter of the stage's A block, 4-7 of its B block.
template <bool GATED>
__device__ __forceinline__ void mx_tile_ctx(const Params& p, int item, int mtl, int nsplit, int wave, int lane_in,
                                            MxTile& t) {
  int lane = lane_in;  // opaque: keeps the per-lane terms from being hoisted out of the tile loop
  asm volatile("" : "+v"(lane));
  big::item_tile(p, item, mtl, nsplit, t.mt, t.nt, t.split);
  t.seg = p.tile_seg[t.mt];
  t.row0 = p.tile_row0[t.mt];
  t.rows = min(BM, p.seg_end[t.seg] - t.row0);
  const int N = p.N, K = p.K;
  const int n0 = t.nt * (GATED ? BN / 2 : BN);
  const int st_lo = t.split * p.KT / nsplit;
  t.KT = (t.split + 1) * p.KT / nsplit - st_lo;
  t.half = (K % BK) != 0 && st_lo + t.KT == p.KT;
  const uint32_t KB2 = (uint32_t)K / 2;
  const int first = p.a_perm ? p.a_perm[t.row0] / p.a_div : t.row0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    int arow = first;
    if (r < t.rows) arow = p.a_perm ? p.a_perm[t.row0 + r] / p.a_div : t.row0 + r;
    t.a_off[i] = r < t.rows ? (uint32_t)arow * (uint32_t)K + (uint32_t)(st_lo * BK + chunk * 16) : kNoLoad;
  }
  if (p.Bp) {
    // packed: this tile's first stage block, rows 32 wave + 16 j .. of it
    const uint32_t blk = (uint32_t)(t.nt * p.KT + st_lo) * PK_STAGE;
#pragma unroll
    for (int j = 0; j < 2; ++j) t.b_off[j] = blk + (uint32_t)((wave * 32 + j * 16) * 64 + lane * 16);
    t.bbase = p.Bp + (size_t)t.seg * p.bp_expert;
    t.sc_src = wave < 4 ? p.A_sc + ((size_t)t.mt * p.KT + st_lo) * SC_BYTES + wave * 256
                        : t.bbase + blk + B_BYTES + (wave - 4) * 256;
    return;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wave * 32 + j * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((r >> 2) & 3);
    const int n = n0 + (GATED ? (r & 127) : r);
    t.b_off[j] = n < N ? (uint32_t)n * KB2 + (uint32_t)(st_lo * (BK / 2) + chunk * 16) : kNoLoad;
  }
  t.bbase = ((GATED && wave >= 4) ? p.B1 : p.B0) + (size_t)t.seg * N * KB2;
  t.sc_src = wave < 4 ? p.A_sc + ((size_t)t.mt * p.KT + st_lo) * SC_BYTES + wave * 256
                      : p.B_sc + (((size_t)t.seg * p.n_tiles + t.nt) * p.KT + st_lo) * SC_BYTES + (wave - 4) * 256;
}

// Epilogue of one tile. Each wave stages its 128 x 64 results (GEMM1: 128
// rows x 32 activation columns) through its own 6400 bytes of one stage
// buffer, 32 rows (one A fragment) at a time.
//  * GEMM2: bf16 of acc * es, rows padded to 72 values; then 8 lanes write a
//    row's 128 bytes, 8 rows per instruction.
//  * GEMM1: act = f(gate * es, up * es) * route weight, quantized as MXFP8
//    for GEMM2 (the wave's 32 columns are one 32-value block of each row).
//    f goes through LDS as fp32, rows padded to 40 floats; then 4 lanes hold
//    8 columns each of a row, reduce the block's largest magnitude across
//    the 4, and write 8 code bytes; the first of them writes the scale byte
//    into GEMM2's scale block.
constexpr int EP_WAVE = STAGE / 8;  // staging bytes per wave
template <bool GATED, int AK>
__device__ __forceinline__ void mx_epilogue(const Params& p, const MxTile& t, const f32x16 (&acc)[4][2],
                                            lds_u8* ebuf, int wave, int lane_in, int nfr) {
  // an opaque copy of the lane index: the per-lane addresses below are then
  // computed here, not hoisted out of the tile loop into registers that
  // would be live through every K loop
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 31, lq = lane >> 5;
  const int N = p.N;
  const int n0 = t.nt * (GATED ? BN / 2 : BN);
  const int wrows = min(128, t.rows - wm * 128);
  const int wrow0 = t.row0 + wm * 128;
  const ActParams ap = act_for(p.act, p.ep, t.seg);
  const float es = scale_for(GATED ? p.ep.fc1 : p.ep.fc2, t.seg);  // fc1 on gate and up, fc2 on down
  if constexpr (!GATED) {
    static_assert(32 * 72 * 2 <= EP_WAVE, "GEMM2 staging");
    constexpr int LDR = 72;
    typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
    lds_u16_t* sh = (lds_u16_t*)(ebuf + wave * EP_WAVE);
    uint16_t* Cs = p.C + (size_t)t.split * p.c_split;
    const int col0 = n0 + wn * 64;
    const int cc = lane & 7, rr = lane >> 3;
    const bool col_ok = col0 + cc * 8 < N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nfr) break;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 8 * (r >> 2) + 4 * lq + (r & 3);
          const __bf16 h = (__bf16)(acc[i][j][r] * es);
          sh[rl * LDR + j * 32 + lr] = *(const uint16_t*)&h;
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int rl = t4 * 8 + rr;
        const u32x4 v = *(const lds_u32x4_t*)&sh[rl * LDR + cc * 8];
        const int row = 32 * i + rl;
        if (col_ok && row < wrows) *(u32x4*)(Cs + (size_t)(wrow0 + row) * N + col0 + cc * 8) = v;
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    static_assert(32 * 40 * 4 <= EP_WAVE, "GEMM1 staging");
    constexpr int LDR = 40;
    lds_f32* sf = (lds_f32*)(ebuf + wave * EP_WAVE);
    const int col = n0 + wn * 32;  // first activation column of the block
    const bool cols_ok = col < N;
    uint8_t* scb = p.Cq_sc + ((size_t)t.mt * p.n_tiles + t.nt) * SC_BYTES + sc_pos(wn);
    const int part = lane & 3;
    // route weights of the lane's 8 rows (rows past the tile read the last
    // row's; their results are not stored)
    float wrow[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) wrow[i][pass] = 1.f;
    if (p.row_w) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int pass = 0; pass < 2; ++pass)
          wrow[i][pass] = p.row_w[wrow0 + min(32 * i + pass * 16 + (lane >> 2), wrows - 1)];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nfr) break;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = 8 * (r >> 2) + 4 * lq + (r & 3);
        sf[rl * LDR + lr] = gated_act_k<AK>(ap, acc[i][0][r] * es, acc[i][1][r] * es);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int rl = pass * 16 + (lane >> 2);
        const int rw = 32 * i + rl;
        float v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = sf[rl * LDR + part * 8 + c] * wrow[i][pass];
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(v[c]));
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        const int code = mx8_code(m);
        const float inv = __uint_as_float((uint32_t)(254 - code) << 23);  // 2^(127 - code)
        uint32_t w2[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          int h4 = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(v[4 * c2] * inv), sat448(v[4 * c2 + 1] * inv), 0, false);
          h4 = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(v[4 * c2 + 2] * inv), sat448(v[4 * c2 + 3] * inv), h4, true);
          w2[c2] = (uint32_t)h4;
        }
        if (rw < wrows) {
          if (cols_ok) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            *(u32x2*)(p.Cq + (size_t)(wrow0 + rw) * N + col + part * 8) = u32x2{w2[0], w2[1]};
          }
          if (part == 0) scb[(size_t)(wm * 128 + rw) * 4] = cols_ok ? (uint8_t)code : (uint8_t)0;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Tiles of a launch, one or more per workgroup. Items are numbered as in the
// bf16 prefill kernel (groups of gn column tiles, row tiles inside a group, K
// ranges fastest); XCD x (the hardware sends workgroup b to XCD b mod 8) owns
// the contiguous run [x per, (x + 1) per) of them, and its S = gridDim / 8
// workgroups take every S-th item of the run, so the tiles an XCD works on at
// any time are neighbours. With a grid of all items each workgroup runs one
// tile; with one workgroup per compute unit each runs its share in turn, and
// the stage stream runs on across tiles: the two loads past a tile's last
// stage fetch the next tile's first two stages, and the last stage's reads of
// "the next stage" are the next tile's first operand reads, so a tile starts
// without waiting for its loads. Its epilogue stages through the buffer of
// the previous tile's last stage, the one buffer no load targets then.
template <bool GATED, int AK>
__device__ __forceinline__ void mx_gemm(const Params& p, lds_u8* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.N;

  const int mtl = p.status[2];
  int nsplit = 1;
  if (!GATED && p.s_cap > 1) nsplit = split_k_count(mtl * p.n_tiles, p.KT, p.ncu, p.s_cap);
  const int n_live = mtl * p.n_tiles * nsplit;
  const int per = (n_live + 7) >> 3;
  const int x = blockIdx.x & 7, S = gridDim.x >> 3;
  const int lo = x * per, hi = min(lo + per, n_live);
  int item = lo + (int)(blockIdx.x >> 3);
  if (item >= hi) return;

  const __amdgpu_buffer_rsrc_t rsA = operand_rsrc(p.A, p.a_bytes);
  // weight codes: one expert's [N, K/2] rows, or its packed blocks; the
  // stride of a stage in them, and in the scale blocks a wave copies
  const uint32_t wbytes = p.Bp ? p.bp_expert : (uint32_t)N * ((uint32_t)p.K / 2);
  const uint32_t b_stage = p.Bp ? (uint32_t)PK_STAGE : (uint32_t)(BK / 2);
  const uint32_t sc_stage = (p.Bp && wave >= 4) ? (uint32_t)PK_STAGE : (uint32_t)SC_BYTES;
  MxTile cur, nxt;
  mx_tile_ctx<GATED>(p, item, mtl, nsplit, wave, lane, cur);
  bool has_next = item + S < hi;
  mx_tile_ctx<GATED>(p, has_next ? item + S : item, mtl, nsplit, wave, lane, nxt);

  // A chunks of the high half of a stage (K 64..127 of it) for this lane's
  // rows: the swizzle makes chunk bit 2 = lane bit 2 for even load
  // instructions and its inverse for odd ones. In a half stage they load
  // zeros, so its second step adds exact zeros (the e4m3 codes 0 times
  // finite e2m1 codes; the scale bytes of both operands are 0 there).
  const uint32_t hi_even = (lane & 4) ? kNoLoad : 0u;
  const uint32_t hi_odd = (lane & 4) ? 0u : kNoLoad;

  // One load instruction of stage U of the stream (U < cur.KT: the current
  // tile's stage U; else the next tile's stage U - cur.KT) into buffer b:
  // q = 0..3 A, 4, 5 B, 6 the scale quarter (lanes 0-15). Every wave issues
  // all seven for every stage; a stage that does not exist reads nothing
  // (offsets past the end) and the scale copy repeats a block of the tile.
#define MOE_MX_DMA(b, U, q)                                                                                    \
  {                                                                                                            \
    const bool in_cur = (U) < cur.KT;                                                                          \
    const int u = in_cur ? (U) : (U) - cur.KT;                                                                 \
    const int ktx = in_cur ? cur.KT : nxt.KT;                                                                  \
    const uint32_t kill = (in_cur || (has_next && u < nxt.KT)) ? 0u : kNoLoad;                                 \
    lds_u8* dst = smem + (b) * STAGE;                                                                          \
    if ((q) < 4) {                                                                                             \
      uint32_t off = ((in_cur ? cur.a_off[(q) & 3] : nxt.a_off[(q) & 3]) + (uint32_t)u * BK) | kill;           \
      if ((in_cur ? cur.half : nxt.half) && u == ktx - 1) off |= ((q) & 1) ? hi_odd : hi_even;                 \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (__attribute__((address_space(3))) void*)(dst + (wave * 32 + (q) * 8) * 128), \
                                               16, off, 0, 0, 0);                                              \
    } else if ((q) < 6) {                                                                                      \
      const __amdgpu_buffer_rsrc_t rsB = operand_rsrc(in_cur ? cur.bbase : nxt.bbase, wbytes);                 \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (__attribute__((address_space(3))) void*)(dst + A_BYTES + (wave * 32 + ((q) - 4) * 16) * 64), \
                                               16, ((in_cur ? cur.b_off[(q) & 1] : nxt.b_off[(q) & 1]) + (uint32_t)u * b_stage) | kill, 0, 0, 0); \
    } else if (lane < 16) {                                                                                    \
      __builtin_amdgcn_global_load_lds((in_cur ? cur.sc_src : nxt.sc_src) + (size_t)min(u, ktx - 1) * sc_stage + lane * 16, \
                                       (__attribute__((address_space(3))) void*)(dst + A_BYTES + B_BYTES + wave * 256), 16, 0, 0); \
    }                                                                                                          \
  }

  // ---- wave tile: 128 rows x 64 weight rows (GEMM1: 32 gate + the same 32 up)
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 31, lq = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // per-lane LDS byte addresses inside a stage: A fragment 0 of step s (two
  // 16-byte halves), B fragment 0 of step s, and the scale pairs
  uint32_t a_rd[2][2], b_rd[2];
  {
    const int ar = wm * 128 + lr;
    const int sw = (ar >> 1) & 7;
    const int br = GATED ? wn * 32 + lr : wn * 64 + lr;
    const int swb = (br >> 2) & 3;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      a_rd[s][0] = lds0 + (uint32_t)(ar * 128 + 16 * ((4 * s + lq) ^ sw));
      a_rd[s][1] = lds0 + (uint32_t)(ar * 128 + 16 * ((4 * s + 2 + lq) ^ sw));
      b_rd[s] = lds0 + (uint32_t)(A_BYTES + br * 64 + 16 * ((2 * s + lq) ^ swb));
    }
  }
  const uint32_t sa_rd = lds0 + (uint32_t)(A_BYTES + B_BYTES + (wm * 128 + lr) * 4 + 2 * lq);
  const uint32_t sb_rd =
      lds0 + (uint32_t)(A_BYTES + B_BYTES + SC_BYTES + (GATED ? wn * 32 + lr : wn * 64 + lr) * 4 + 2 * lq);

  f32x16 acc[4][2];
  // Operands: A fragment k = (lo, hi) 16-byte halves, one set (each
  // fragment is re-read for the next step right after the MFMA pair that
  // used it); B fragments of step 0 (fb) and step 1 (gb); scale pairs of the
  // current stage (sa, sb) and of the next (na, nb).
  i32x4 fal[4], fah[4], fb[2], gb[2];
  uint32_t sa[4], sb[2], na[4], nb[2];

  // Operand reads are inline asm (the compiler's tracking of direct-to-LDS
  // loads would put a vmcnt(0) before every LDS read) completed by explicit
  // lgkmcnt waits: a wave's LDS reads return in order, so before each MFMA
  // pair the wait names how many reads issued after the needed ones may
  // still be in flight. Issue order per stage: A0, B (both), scales (6), A1,
  // A2, A3 for step 0, then A0, B, A1, A2, A3 for step 1 (2 reads per A
  // fragment). A fragments are 32 rows = 4096 bytes apart, B fragment 1 is
  // 128 rows (GEMM1, up) or 32 rows (GEMM2) after fragment 0; scale rows
  // are 4 bytes.
#define MOE_DSR(d, addr, off) asm volatile("ds_read_b128 %0, %1 offset:" #off : "=v"(d) : "v"(addr))
#define MOE_DSR16(d, addr, off) asm volatile("ds_read_u16 %0, %1 offset:" #off : "=v"(d) : "v"(addr))
#define MOE_MX_READ_A(s, k, base)                                              \
  {                                                                            \
    const uint32_t x0 = a_rd[s][0] + (base), x1 = a_rd[s][1] + (base);         \
    switch (k) {                                                               \
      case 0: MOE_DSR(fal[0], x0, 0); MOE_DSR(fah[0], x1, 0); break;           \
      case 1: MOE_DSR(fal[1], x0, 4096); MOE_DSR(fah[1], x1, 4096); break;     \
      case 2: MOE_DSR(fal[2], x0, 8192); MOE_DSR(fah[2], x1, 8192); break;     \
      default: MOE_DSR(fal[3], x0, 12288); MOE_DSR(fah[3], x1, 12288); break;  \
    }                                                                          \
  }
#define MOE_MX_READ_B(d, s, base)                                              \
  {                                                                            \
    const uint32_t x = b_rd[s] + (base);                                       \
    MOE_DSR(d[0], x, 0);                                                       \
    if (GATED) MOE_DSR(d[1], x, 8192);                                         \
    else MOE_DSR(d[1], x, 2048);                                               \
  }
#define MOE_MX_READ_SC(base)                                                   \
  {                                                                            \
    const uint32_t xa = sa_rd + (base), xb = sb_rd + (base);                   \
    MOE_DSR16(na[0], xa, 0);                                                   \
    MOE_DSR16(na[1], xa, 128);                                                 \
    MOE_DSR16(na[2], xa, 256);                                                 \
    MOE_DSR16(na[3], xa, 384);                                                 \
    MOE_DSR16(nb[0], xb, 0);                                                   \
    if (GATED) MOE_DSR16(nb[1], xb, 512);                                      \
    else MOE_DSR16(nb[1], xb, 128);                                            \
  }
  // wait until at most n reads are in flight, then A fragment k may be used
#define MOE_MX_WAIT(n, k)                                                      \
  {                                                                            \
    wait_lgkm(n);                                                              \
    asm volatile("" : "+v"(fal[k]), "+v"(fah[k]));                             \
  }
  // MFMA pair of A fragment k in step S with B fragments bb, skipped when
  // the fragment's 32 rows are all past the segment (nfr = the wave's
  // fragments holding rows). The empty asm reading the two accumulators
  // keeps instruction selection from sinking the pair (which depends on
  // nothing after it) below the next reads.
#define MOE_MX_MFMA2(bb, k, S)                                                                               \
  if ((k) < nfr) {                                                                                           \
    const i32x8 av = __builtin_shufflevector(fal[k], fah[k], 0, 1, 2, 3, 4, 5, 6, 7);                        \
    const i32x8 b0v = __builtin_shufflevector(bb[0], bb[0], 0, 1, 2, 3, -1, -1, -1, -1);                      \
    const i32x8 b1v = __builtin_shufflevector(bb[1], bb[1], 0, 1, 2, 3, -1, -1, -1, -1);                      \
    acc[k][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, b0v, acc[k][0], 0, 4, S, (int)sa[k], S, (int)sb[0]); \
    acc[k][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, b1v, acc[k][1], 0, 4, S, (int)sa[k], S, (int)sb[1]); \
    asm volatile("" : "+v"(acc[k][0]), "+v"(acc[k][1]));                                                     \
  }

  // the operands of step 0 of the stage in buffer b (issue order A0, B,
  // scales, A1, A2, A3: the order the loop's waits count on)
#define MOE_MX_FIRST_READS(b)                                                  \
  {                                                                            \
    const uint32_t fbase = (uint32_t)(b) * STAGE;                              \
    MOE_MX_READ_A(0, 0, fbase)                                                 \
    MOE_MX_READ_B(fb, 0, fbase)                                                \
    MOE_MX_READ_SC(fbase)                                                      \
    MOE_MX_READ_A(0, 1, fbase)                                                 \
    MOE_MX_READ_A(0, 2, fbase)                                                 \
    MOE_MX_READ_A(0, 3, fbase)                                                 \
  }

  // ---- the first tile's stages 0 and 1 (or the next tile's first stage)
  int base = 0;  // buffer of the current tile's stage 0
#pragma unroll
  for (int q = 0; q < LOADS; ++q) MOE_MX_DMA(0, 0, q)
#pragma unroll
  for (int q = 0; q < LOADS; ++q) MOE_MX_DMA(1, 1, q)
  big::wait_vmcnt<LOADS>();
  big::stage_barrier();
  MOE_MX_FIRST_READS(0)

  // Stage s in buffer st. Step 0 runs on fb and the A fragments, with the
  // loads of stream stage s + 2 (into buffer st2, free since the last
  // barrier) and the reads of step 1's operands; step 1 runs on gb: after its
  // first MFMA pair a wave waits for its loads of stage s + 1 and meets the
  // others, and the reads of stage s + 1's step-0 operands and scales follow
  // (at the tile's last stage: the next tile's first operands). The body is
  // the same for every stage, so the wait counts never change.
#define MOE_MX_KLOOP                                                              \
  {                                                                               \
    int st = base, st1 = base == NS - 1 ? 0 : base + 1, st2 = st1 == NS - 1 ? 0 : st1 + 1; \
    for (int s = 0; s < cur.KT; ++s) {                                            \
      const uint32_t sbase = (uint32_t)st * STAGE;                                \
      const uint32_t nbase = (uint32_t)st1 * STAGE;                               \
      _Pragma("unroll") for (int k = 0; k < 4; ++k) {                             \
        if (k == 0) {                                                             \
          MOE_MX_WAIT(6, 0)                                                       \
          asm volatile("" : "+v"(fb[0]), "+v"(fb[1]), "+v"(na[0]), "+v"(na[1]),   \
                       "+v"(na[2]), "+v"(na[3]), "+v"(nb[0]), "+v"(nb[1]));       \
          _Pragma("unroll") for (int t = 0; t < 4; ++t) sa[t] = na[t];            \
          sb[0] = nb[0];                                                          \
          sb[1] = nb[1];                                                          \
        } else {                                                                  \
          MOE_MX_WAIT(8, k)                                                       \
        }                                                                         \
        MOE_MX_MFMA2(fb, k, 0)                                                    \
        MOE_MX_DMA(st2, s + 2, 2 * k)                                             \
        if (k < 3) MOE_MX_DMA(st2, s + 2, 2 * k + 1)                              \
        MOE_MX_READ_A(1, k, sbase)                                                \
        if (k == 0) MOE_MX_READ_B(gb, 1, sbase)                                   \
      }                                                                           \
      _Pragma("unroll") for (int k = 0; k < 4; ++k) {                             \
        if (k == 0) {                                                             \
          MOE_MX_WAIT(6, 0)                                                       \
          asm volatile("" : "+v"(gb[0]), "+v"(gb[1]));                            \
        } else {                                                                  \
          MOE_MX_WAIT(14, k)                                                      \
        }                                                                         \
        MOE_MX_MFMA2(gb, k, 1)                                                    \
        if (k == 0) {                                                             \
          big::wait_vmcnt<LOADS>();                                               \
          big::stage_barrier();                                                   \
        }                                                                         \
        MOE_MX_READ_A(0, k, nbase)                                                \
        if (k == 0) {                                                             \
          MOE_MX_READ_B(fb, 0, nbase)                                             \
          MOE_MX_READ_SC(nbase)                                                   \
        }                                                                         \
      }                                                                           \
      st = st1;                                                                   \
      st1 = st2;                                                                  \
      st2 = (st2 == NS - 1) ? 0 : st2 + 1;                                        \
    }                                                                             \
  }

  for (;;) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // A fragments of this wave with rows in the segment (a partial tile's
    // MFMAs are skipped 32 rows at a time)
    const int nfr = min(4, max(0, (cur.rows - wm * 128 + 31) >> 5));
    MOE_MX_KLOOP
    // Every wave's operand reads of this tile are done once its own are: the
    // buffer of the last stage is free for the epilogue's staging (the
    // loads in flight target the other two). The last stage's reads of the
    // next tile's first operands are dropped (their registers would be live
    // through the epilogue) and made again after it.
    // After the last tile only the loads past its end (which read nothing)
    // are in flight; they land before the epilogue, so no load into LDS
    // outlives the workgroup.
    if (!has_next) big::wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    big::stage_barrier();
    lds_u8* ebuf = smem + ((base + cur.KT - 1) % NS) * STAGE;
    if (nfr > 0) mx_epilogue<GATED, AK>(p, cur, acc, ebuf, wave, lane, nfr);
    if (!has_next) break;
    // the epilogue's buffer takes the next tile's third stage
    big::stage_barrier();
    item += S;
    base = (base + cur.KT) % NS;
    cur = nxt;
    has_next = item + S < hi;
    mx_tile_ctx<GATED>(p, has_next ? item + S : item, mtl, nsplit, wave, lane, nxt);
    MOE_MX_FIRST_READS(base)
  }
#undef MOE_MX_FIRST_READS
#undef MOE_MX_KLOOP
#undef MOE_MX_MFMA2
#undef MOE_MX_WAIT
#undef MOE_MX_READ_SC
#undef MOE_MX_READ_B
#undef MOE_MX_READ_A
#undef MOE_DSR16
#undef MOE_DSR
#undef MOE_MX_DMA
}

template <bool GATED, int AK>
__global__ __launch_bounds__(NT, 1) void k_gemm(const Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem_arr[NS * STAGE];
  mx_gemm<GATED, AK>(p, (lds_u8*)smem_arr);
}

// ---------------------------------------------------------------------------
// Per-call preparation of the scale blocks.
//  * weights: for each expert with rows and each column tile, the 4 scale
//    bytes of each of the tile's 256 weight rows and each stage (GEMM1: rows
//    0-127 gate, 128-255 up; rows past N repeat row N - 1), in the block order
//    (0, 2, 1, 3), 0 past the last block of K;
//  * GEMM1's activations: for each row tile, the same from the scale rows of
//    its A rows (through the permutation), 0 for rows past the segment.
struct PrepParams {
  const uint8_t* Sg;   // e8m0 [E, I, H/32]
  const uint8_t* Su;
  const uint8_t* Sd;   // e8m0 [E, H, I/32]
  uint8_t* WS1;        // [E][NT1][KT1] blocks
  uint8_t* WS2;        // [E][NT2][KT2] blocks
  int32_t E, H, I;
  int32_t NT1, KT1, NT2, KT2;
  const int32_t* counts;
  const uint8_t* xs;   // scale rows of GEMM1's A rows
  int32_t xs_stride;   // bytes per row (a multiple of 16, >= 4 * KT1)
  const int32_t* perm; // sorted row -> flat slot, or nullptr (A rows in sorted order)
  int32_t div;
  const int32_t* tile_seg;
  const int32_t* tile_row0;
  const int32_t* seg_end;
  const int32_t* status;
  int32_t mt_cap;
  uint8_t* SA1;        // [mt_cap][KT1] blocks
};

__device__ __forceinline__ uint32_t order_0213(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  return b0 | (b2 << 8) | (b1 << 16) | (b3 << 24);
}

// LDS bytes k_mx_prep needs: one panel's scale rows (256 rows x K/32 bytes)
__host__ __device__ constexpr int prep_lds_bytes(int kmax) { return 256 * (kmax / 32); }

// Weight panels: the panel's scale rows (contiguous in the [E, N, K/32]
// layout: 128 gate + 128 up rows, or 256 down rows) are copied into LDS with
// coalesced loads, then each stage's 1 KB block is written with coalesced
// 4-byte stores (thread r = row r). Row tiles of GEMM1's activations: thread
// r copies its row's scale bytes (one 4-byte load per stage).
__global__ __launch_bounds__(256) void k_mx_prep(const PrepParams q) {
  extern __shared__ __attribute__((aligned(16))) uint8_t prep_lds[];
  const int r = threadIdx.x;
  int b = blockIdx.x;
  const int n1 = q.E * q.NT1, n2 = q.E * q.NT2;
  if (b < n1 + n2) {
    const bool g1 = b < n1;
    if (!g1) b -= n1;
    const int NTc = g1 ? q.NT1 : q.NT2, KT = g1 ? q.KT1 : q.KT2;
    const int e = b / NTc, nt = b - e * NTc;
    if (q.counts[e] == 0) return;
    const int N = g1 ? q.I : q.H, KB = (g1 ? q.H : q.I) / 32;
    const int n0 = g1 ? nt * 128 : nt * 256;
    const int per = g1 ? 128 : 256;               // rows of one source region
    const int nrows = min(per, N - n0);           // rows of the panel inside N
    for (int part = 0; part < (g1 ? 2 : 1); ++part) {
      const uint8_t* src = (g1 ? (part ? q.Su : q.Sg) : q.Sd) + ((size_t)e * N + n0) * KB;
      uint8_t* dst = prep_lds + part * 128 * KB;
      const int nbytes = nrows * KB;
      if ((((uintptr_t)src | (uintptr_t)nbytes) & 3u) == 0) {
        for (int i = r; i < nbytes / 4; i += 256) ((uint32_t*)dst)[i] = ((const uint32_t*)src)[i];
      } else {
        for (int i = r; i < nbytes; i += 256) dst[i] = src[i];
      }
    }
    __syncthreads();
    // tile row r: rows past N repeat the panel's last row inside N
    const int rr = g1 ? (r & 127) : r;
    const uint8_t* row = prep_lds + ((g1 && r >= 128) ? 128 * KB : 0) + min(rr, nrows - 1) * KB;
    uint8_t* out = (g1 ? q.WS1 : q.WS2) + ((size_t)(e * NTc + nt) * KT) * SC_BYTES + r * 4;
    for (int u = 0; u < KT; ++u) {
      uint32_t v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = 4 * u + t < KB ? row[4 * u + t] : 0u;
      *(uint32_t*)(out + (size_t)u * SC_BYTES) = order_0213(v[0], v[1], v[2], v[3]);
    }
    return;
  }
  const int mt = b - n1 - n2;
  if (mt >= q.mt_cap || mt >= q.status[2]) return;
  const int seg = q.tile_seg[mt], row0 = q.tile_row0[mt];
  const bool live = r < q.seg_end[seg] - row0;
  const int srow = live ? (q.perm ? q.perm[row0 + r] / q.div : row0 + r) : 0;
  const uint8_t* src = q.xs + (size_t)srow * q.xs_stride;
  uint8_t* dst = q.SA1 + (size_t)mt * q.KT1 * SC_BYTES + r * 4;
  for (int u = 0; u < q.KT1; ++u) {
    uint32_t w = 0;
    if (live) {
      const uint32_t x = *(const uint32_t*)(src + 4 * u);
      w = order_0213(x & 0xffu, (x >> 8) & 0xffu, (x >> 16) & 0xffu, x >> 24);
    }
    *(uint32_t*)(dst + (size_t)u * SC_BYTES) = w;
  }
}

// ---------------------------------------------------------------------------
// Packing (moe_mx_pack_weights): one workgroup per packed block (expert,
// column tile, stage; GEMM1's blocks first), thread r writing row r's 64 code
// bytes in the swizzled order and its 4 scale bytes. Made once per set of
// weights, not per call.
struct PackParams {
  const uint8_t* Wg;   // e2m1 codes [E, I, H/2]
  const uint8_t* Wu;
  const uint8_t* Wd;   // [E, H, I/2]
  const uint8_t* Sg;   // e8m0 [E, I, H/32]
  const uint8_t* Su;
  const uint8_t* Sd;   // [E, H, I/32]
  uint8_t* out;
  int32_t E, H, I;
  int32_t NT1, KT1, NT2, KT2;
};

__global__ __launch_bounds__(256) void k_mx_pack(const PackParams q) {
  const int r = threadIdx.x;
  int b = blockIdx.x;
  const int n1 = q.E * q.NT1 * q.KT1;
  const bool g1 = b < n1;
  if (!g1) b -= n1;
  const int NTc = g1 ? q.NT1 : q.NT2, KT = g1 ? q.KT1 : q.KT2;
  const int e = b / (NTc * KT), rem = b - e * (NTc * KT);
  const int nt = rem / KT, u = rem - nt * KT;
  const int N = g1 ? q.I : q.H, K = g1 ? q.H : q.I;
  const int KB2 = K / 2, KB = K / 32;
  const int n = g1 ? nt * 128 + (r & 127) : nt * 256 + r;  // weight row of tile row r
  const uint8_t* W = g1 ? (r < 128 ? q.Wg : q.Wu) : q.Wd;
  const uint8_t* S = g1 ? (r < 128 ? q.Sg : q.Su) : q.Sd;
  uint8_t* blk = q.out + ((size_t)(g1 ? 0 : n1) + ((size_t)e * NTc + nt) * KT + u) * PK_STAGE;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int kb = u * (BK / 2) + c * 16;  // byte of the row
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < N && kb < KB2) v = *(const u32x4*)(W + ((size_t)e * N + n) * KB2 + kb);
    *(u32x4*)(blk + r * 64 + 16 * (c ^ ((r >> 2) & 3))) = v;
  }
  // rows past N repeat row N - 1's scales (their codes are 0), blocks past K are 0
  const uint8_t* srow = S + ((size_t)e * N + min(n, N - 1)) * KB;
  uint32_t sv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) sv[t] = 4 * u + t < KB ? srow[4 * u + t] : 0u;
  *(uint32_t*)(blk + B_BYTES + r * 4) = order_0213(sv[0], sv[1], sv[2], sv[3]);
}

}  // namespace mx
}  // namespace moe
