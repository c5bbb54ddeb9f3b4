// Grouped GEMM for few rows per segment (decode): weights streamed from HBM
// straight into MFMA operand registers; the tile's activation rows are staged
// through LDS in K chunks shared by the workgroup's waves.
//
// Same grouped-GEMM definition as the prefill kernel (moonep_experts page,
// moonep_grouped_gemm; route weight on the activation per the module
// docstring). Weights may be bf16 or MXFP4 (trtllm_mxfp4_moe page,
// TrtLlmMxfp4ExpertsBase._supports_quant_scheme: MXFP4 weights with
// unquantized activations): e2m1 codes with an e8m0 scale per 32 K elements
// (OCP Microscaling v1.0 reading).
//
// Tile: 16 rows. Each wave owns two 16-column weight streams: gate and up of
// the same 16 columns (GEMM1), or two adjacent 16-column groups (GEMM2), so a
// wave moves the same bytes per K step in both GEMMs. 4 waves per workgroup.
// The activations are the MFMA's A operand (row = lane & 15), the weights its
// B operand (column = lane & 15). In K step s (128 values) lane group
// q = lane >> 4 owns the 32-value scale block kb = 4 s + q of the weights: one
// 16-byte load carries a lane's 32 MXFP4 codes, whose single scale comes with
// them; the 16 lanes of a group read 64 contiguous bytes of each of 16 rows.
//
// bf16 weights: four v_mfma_f32_16x16x32_bf16 per step and stream (the K
// order inside a dot product is free as long as A and B agree).
// MXFP4 weights: the codes go to v_mfma_scale_f32_16x16x128_f8f6f4 as they
// are, with their e8m0 scales, so nothing is decoded. Its A operand is e4m3
// with a scale per 32 K values: the activation rows are split beforehand
// (k_quant_rows) into two e4m3 parts per value, hi + lo, which together
// carry every bit of the bf16 value (to within 2^-17 of the block's largest
// value), and the step runs one MFMA per part. Lane group q then holds
// activation K values 16 q..16 q+15 and 64 + 16 q..64 + 16 q + 15 of the step
// (the operand layout of the fp8 A input), and supplies the scales of block q
// for both operands.
//
// MXFP4 scales: the e8m0 bytes of a workgroup's weight rows form one
// contiguous region per stream (64 rows x K/32 bytes for gate and for up, or
// 128 rows for down). The workgroup copies it into LDS once, with coalesced
// 16-byte loads, and lanes read their scale bytes from there; per-step scale
// loads from global memory would touch 16 cache lines for 64 useful bytes.
//
// Pipeline: K is cut into chunks of SPC steps. While chunk c is multiplied
// (A from LDS buffer c & 1, weights from one register set), the weights of
// chunk c + 1 load into the other register set and its activations into
// registers, written to the other LDS buffer after the MFMAs; one LDS-only
// barrier per chunk. The weight loads stay in flight across it.
// Rows of the tile past the segment end hold copies of its last row and are
// never stored (rows of a product are independent).
#pragma once

#include "common.hpp"

namespace moe {
namespace skinny {

constexpr int BM = 16;   // rows per tile
constexpr int NW = 4;    // waves per workgroup
constexpr int NT = NW * 64;

enum WFmt { W_BF16 = 0, W_MXFP4 = 1 };

// output columns covered by one workgroup
__host__ __device__ constexpr int block_cols(bool gated) { return NW * 16 * (gated ? 1 : 2); }

// MXFP4 scale staging: 128 weight rows x K/32 bytes = 4 K bytes of LDS per
// workgroup, copied in 16-byte pieces, spt pieces per thread.
constexpr int kMaxMxfp4K = 16384;
__host__ __device__ constexpr int scale_lds_bytes(int K) { return 4 * K; }
__host__ __device__ constexpr int scale_pieces_per_thread(int K) { return K <= 4096 ? 4 : K <= 8192 ? 8 : 16; }

// Activation rows split for the block-scaled MFMA (MXFP4 weights). Each
// 32-value block of a bf16 row gets the scale 2^s with s = e - 7, where
// 2^e <= the block's largest magnitude < 2^(e+1), so every scaled value v lies
// below 256 in magnitude (e4m3 reaches 448); v is written as two e4m3 values
// hi = rne(v) and lo = rne(v - hi). A bf16 has 8 significant bits and hi
// keeps the top 4, so v - hi needs at most 4 and hi + lo = v exactly while lo
// stays a normal e4m3 (|v| >= 2); below that lo is off by at most half the
// subnormal spacing 2^-9, i.e. 2^-17 of the block's largest value.
// Layout: hi [rows, K] bytes, lo [rows, K] bytes, e8m0 codes s + 127 in rows
// of sc_stride bytes (a multiple of 16 >= K / 32; code 0 past K / 32).
struct QRows {
  uint8_t* hi;
  uint8_t* lo;
  uint8_t* sc;
  int32_t sc_stride;
};

__host__ __device__ constexpr int quant_sc_stride(int K) { return (K / 32 + 15) / 16 * 16; }

struct Params {
  const uint16_t* A;      // rows [*, K] bf16 (bf16 weights)
  QRows Aq;               // the same rows split by k_quant_rows (MXFP4 weights)
  const int32_t* a_perm;  // sorted row -> flat slot, or nullptr
  int32_t a_div;
  const void* B0;         // gate / down: bf16 [G, N, K] or e2m1 codes [G, N, K/2]
  const void* B1;         // up (GEMM1)
  const uint8_t* S0;      // e8m0 scales [G, N, K/32] (MXFP4), 16-byte aligned
  const uint8_t* S1;
  int32_t N, K;
  const int32_t* tile_seg;
  const int32_t* tile_row0;
  const int32_t* seg_end;
  const int32_t* status;  // status[2] = number of row tiles
  int32_t mt_cap;
  int32_t n_tiles;        // ceil(N / block_cols)
  uint16_t* C;            // [rows, N] bf16 output (unused by GEMM1 with MXFP8 activations)
  QRows Cq;               // GEMM1 with MXFP8 activations: the activation rows, quantized
  const float* row_w;     // route weight per sorted row, or nullptr (weight already on the input)
  ActParams act;
  ExpertParams ep;        // per-expert activation parameters and fc1 / fc2 scales
  // MXFP4 codes in the packed layout of the MXFP4 prefill GEMMs (PK kernels):
  // this GEMM's blocks, bp_expert bytes per expert; scales still from S0 / S1
  const uint8_t* Bp;
  uint32_t bp_expert;
};

// The packed MXFP4 layout (written by k_mx_pack, defined with the prefill
// GEMM): per expert, column tile of PK_COLS1 gate + the same up rows (GEMM1)
// or PK_COLS2 down rows (GEMM2), and 128-K stage, one PK_BLOCK-byte block whose
// first bytes hold row r's 64 code bytes at 64 r, 16-byte chunk c at slot
// c ^ ((r >> 2) & 3); codes past N or K are 0.
constexpr int PK_BLOCK = 17408;
constexpr int PK_COLS1 = 128;
constexpr int PK_COLS2 = 256;
constexpr int PK_KSTAGE = 128;

__device__ __forceinline__ float sat448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// Split row r of q from bf16 source row sr (256 threads, one 32-value block
// per thread and step).
// MX8: MXFP8 activations instead (trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase:
// MXFP4 weights with dynamically quantized MXFP8 activations; OCP
// Microscaling v1.0 reading): the block's scale is 2^(e - 8) for
// 2^e <= amax < 2^(e+1) (8 = the largest e4m3 exponent), each scaled value is
// rounded to e4m3 (to nearest, ties to even) after clamping to +-448 (so it
// saturates), and there is no lo part.
template <bool MX8 = false>
__device__ __forceinline__ void quant_row(const uint16_t* __restrict__ src, size_t sr, int r, int K, const QRows& q) {
  const int KB = K / 32;
  for (int b = threadIdx.x; b < q.sc_stride; b += 256) {
    if (b >= KB) {
      q.sc[(size_t)r * q.sc_stride + b] = 0;
      continue;
    }
    const u32x4* in = (const u32x4*)(src + sr * K + 32 * b);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = in[i];
      w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
    }
    uint32_t mx = 0;  // largest magnitude, as bf16 bits
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = max(mx, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
    const int code = min(max((int)((mx >> 7) & 0xffu) - (MX8 ? 8 : 7), 0), 254);
    const float inv = __uint_as_float((uint32_t)(254 - code) << 23);  // 2^(127 - code), normal for code <= 247
    uint32_t hi[8], lo[8];
    if (MX8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v0 = sat448(bf16_bits_to_f32(w[2 * i] & 0xffffu) * inv);
        const float v1 = sat448(bf16_bits_to_f32(w[2 * i] >> 16) * inv);
        const float v2 = sat448(bf16_bits_to_f32(w[2 * i + 1] & 0xffffu) * inv);
        const float v3 = sat448(bf16_bits_to_f32(w[2 * i + 1] >> 16) * inv);
        int h = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
        h = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, h, true);
        hi[i] = (uint32_t)h;
      }
      u32x4* ho = (u32x4*)(q.hi + (size_t)r * K + 32 * b);
      ho[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      ho[1] = u32x4{hi[4], hi[5], hi[6], hi[7]};
      q.sc[(size_t)r * q.sc_stride + b] = (uint8_t)code;
      continue;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v0 = bf16_bits_to_f32(w[2 * i] & 0xffffu) * inv, v1 = bf16_bits_to_f32(w[2 * i] >> 16) * inv;
      const float v2 = bf16_bits_to_f32(w[2 * i + 1] & 0xffffu) * inv, v3 = bf16_bits_to_f32(w[2 * i + 1] >> 16) * inv;
      int h = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
      h = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, h, true);
      const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false), h23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
      int l = __builtin_amdgcn_cvt_pk_fp8_f32(v0 - h01[0], v1 - h01[1], 0, false);
      l = __builtin_amdgcn_cvt_pk_fp8_f32(v2 - h23[0], v3 - h23[1], l, true);
      hi[i] = (uint32_t)h;
      lo[i] = (uint32_t)l;
    }
    u32x4* ho = (u32x4*)(q.hi + (size_t)r * K + 32 * b);
    u32x4* lw = (u32x4*)(q.lo + (size_t)r * K + 32 * b);
    ho[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    ho[1] = u32x4{hi[4], hi[5], hi[6], hi[7]};
    lw[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    lw[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
    q.sc[(size_t)r * q.sc_stride + b] = (uint8_t)code;
  }
}

// One workgroup per row. With perm, output row r is source row perm[r] / div
// (sorted row -> token), for the first status[1] rows (the valid sorted rows;
// the rest are never read).
template <bool MX8>
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ src, int rows, int K, QRows q,
                                                    const int32_t* perm, int div, const int32_t* status) {
  const int r = blockIdx.x;
  if (r >= rows || (perm && r >= status[1])) return;
  quant_row<MX8>(src, perm ? (size_t)(perm[r] / div) : (size_t)r, r, K, q);
}

template <int FMT>
struct Cfg {
  static constexpr int SPC = FMT == W_MXFP4 ? 4 : 1;  // K steps per chunk
  static constexpr int KC = SPC * 128;                // K values per chunk
  // bf16 activations: rows of KC + 8 values (16 B pad)
  static constexpr int LROW = KC + 8;
  static constexpr int PIECES = BM * KC / 8;          // 16-byte pieces of an A chunk
  static constexpr int PPT = PIECES / NT;             // pieces per thread
  static_assert(PIECES % NT == 0, "A chunk must split evenly over the workgroup");
  // split activations: hi and lo rows of KC + 16 bytes, then 16 rows of the
  // chunk's KC / 32 scale bytes (16 B)
  static constexpr int QROW = KC + 16;
  static constexpr int QPPT = BM * KC / 16 / NT;      // 16-byte pieces of hi (and of lo) per thread
  static constexpr int BUF_BYTES = FMT == W_MXFP4 ? 2 * BM * QROW + BM * 16 : BM * LROW * 2;
};

// The weights of one lane for one K step: 32 consecutive K values of row n.
template <int FMT>
struct WChunk {
  u32x4 q[FMT == W_BF16 ? 4 : 1];
};

// Weights of one chunk for both streams of a wave.
template <int FMT>
struct WSet {
  WChunk<FMT> w0[Cfg<FMT>::SPC], w1[Cfg<FMT>::SPC];
};

// Weight loads go through a buffer resource over one segment's weight rows.
// Every load whose bytes lie past its row's end, or past the last chunk, gets
// a VGPR offset past the segment and reads 0 without a memory access; the
// SGPR offset, which carries a chunk's K position, is not relied on for the
// range check. The weights are read once per step, so they carry the
// non-temporal hint (cache policy bit 1, nt): measured, the decode step ran
// 10% faster with it than with the default policy.
constexpr int kAuxNt = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// bf16 MFMA B operand i (8 K values) of a lane's block. A block past the row
// end (!ok) multiplies activations that are zero, and is made zero so that the
// product is exactly 0.
__device__ __forceinline__ bf16x8 w_operand_bf16(const WChunk<W_BF16>& w, int i, bool ok) {
  const uint32_t m = ok ? ~0u : 0u;
  const u32x4 v = w.q[i] & m;
  return *(const bf16x8*)&v;
}

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Block-scaled MFMA, 16 x 16 outputs, K 128: A e4m3 (cbsz 0), B e2m1 (blgp 4,
// the upper half of the B registers unused), one e8m0 code per lane for each.
__device__ __forceinline__ f32x4 mfma_fp8_fp4(const i32x8& a, const i32x8& b, f32x4 acc, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 4, 0, sa, 0, sb);
}

// Barrier that orders LDS accesses only: global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

extern __shared__ __attribute__((aligned(16))) uint8_t skinny_scales[];

// ---------------------------------------------------------------------------
// Single-launch decode step. GEMM1 tiles, GEMM2 tiles and combine rows are
// items of one work queue, taken in that order by the workgroups of one
// persistent launch. Data one workgroup hands to another (GEMM1's activation
// rows for GEMM2, GEMM2's slot rows for the combine) goes out with
// agent-coherent stores, which write through the XCD's own L2, and is read
// with agent-coherent loads, which skip stale L2 copies; a workgroup counts
// itself in only after its stores have completed. Every wait is on items
// with lower queue positions, which were taken by running workgroups that
// never wait on later items, so the waits always end; each is still bounded
// and sets a status flag if it gives up.
struct FusedSync {
  int32_t* queue;     // work-queue position (zero before the launch)
  int32_t* done1;     // [row tiles]: GEMM1 column tiles finished per row tile (zero before)
  int32_t* done2;     // GEMM2 tiles finished (zero before)
  int32_t* status;    // status[3] = 1 when a wait gave up
  int32_t n_tiles1;   // GEMM1 column tiles per row tile
  int32_t spin_limit;
  int32_t batch;      // consecutive items taken from the queue at a time (>= 1)
};

__device__ __forceinline__ void st_coh32(void* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh8(uint8_t* p, uint32_t v) {
  __hip_atomic_store(p, (uint8_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at base + off with the agent-coherence cache policy (sc1, the one
// the compiler gives agent-scope atomic loads), through a buffer resource over
// base so the load stays one instruction.
constexpr int kAuxSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xffffffffu, 0x00020000);
}
__device__ __forceinline__ u32x4 ld_coh128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxSc1);
}

// Control flow around the barriers of the single launch stays uniform
// across the lanes of every wave: wave 0 (a wave-uniform condition) does the
// waiting and the counting on all 64 lanes, and every loaded value that
// decides a branch is made uniform with readfirstlane. A branch on a lane
// condition (thread 0 only) inside the work loop lets the compiler run the
// other lanes of the wave around the loop, barriers included, without it.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Wave 0 waits until *c >= target (or the status flag is set, or the spin
// limit is reached, which sets the flag); the workgroup then meets at an
// LDS-only barrier, so weight loads issued before the wait stay in flight.
__device__ __forceinline__ void wait_count(const int32_t* c, int target, const FusedSync& fs) {
  if (wave_id() == 0) {
    for (int spins = 0;; ++spins) {
      const int cur = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(const_cast<int32_t*>(c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (cur >= target) break;
      const int flag = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(&fs.status[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (flag != 0) break;
      if (spins >= fs.spin_limit) {
        __hip_atomic_store(&fs.status[3], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  lds_barrier();
}

// After a tile's coherent stores: every thread waits for its stores to
// complete, the workgroup meets, and wave 0 counts the tile in (lane 0 adds
// 1, the other lanes 0).
__device__ __forceinline__ void count_in(int32_t* c) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  if (wave_id() == 0)
    __hip_atomic_fetch_add(c, (threadIdx.x & 63) == 0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The bytes b of the 16 lanes of a lane group (16 consecutive columns of one
// row), four at a time: lanes with l16 % 4 == 0 get columns l16 .. l16 + 3.
__device__ __forceinline__ uint32_t gather4(uint32_t b) {
  return (b & 0xffu) | ((uint32_t)__shfl_down((int)b, 1) & 0xffu) << 8 |
         ((uint32_t)__shfl_down((int)b, 2) & 0xffu) << 16 | ((uint32_t)__shfl_down((int)b, 3) & 0xffu) << 24;
}

// 4 x 4 transpose between a lane's four registers and lane bits 2-3: lane
// l of register j receives what lane l' of register j' held, where l' is l
// with bits 2-3 replaced by j and j' is bits 2-3 of l. Two butterfly stages
// (bit 2 with register bit 0, then bit 3 with register bit 1); each moves
// data 4 or 8 lanes within a 16-lane row (DPP row shifts) and selects.
template <int BIT>
__device__ __forceinline__ void quad_swap(u32x4& a, u32x4& b, bool hi) {
  constexpr int SHR = 0x110 + BIT, SHL = 0x100 + BIT;  // DPP row_shr:BIT, row_shl:BIT
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t from_b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b[d], SHR, 0xf, 0xf, false);
    const uint32_t from_a = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a[d], SHL, 0xf, 0xf, false);
    const uint32_t na = hi ? from_b : a[d];
    const uint32_t nb = hi ? b[d] : from_a;
    a[d] = na;
    b[d] = nb;
  }
}
__device__ __forceinline__ void quad_transpose(u32x4 (&r)[4], int lane) {
  const bool b2 = (lane & 4) != 0, b3 = (lane & 8) != 0;
  quad_swap<4>(r[0], r[1], b2);
  quad_swap<4>(r[2], r[3], b2);
  quad_swap<8>(r[0], r[2], b3);
  quad_swap<8>(r[1], r[3], b3);
}

// LDS of one decode tile: two activation buffers, the block maxima
// exchanged by wave pairs.
template <int FMT>
struct TileLds {
  __attribute__((aligned(16))) uint8_t sbuf[2][Cfg<FMT>::BUF_BYTES];
  float half_amax[NW][BM];
};

// One tile: row tile mt, column tile nt.
// SPT: scale pieces per thread (MXFP4; 0 for bf16), scale_pieces_per_thread(K).
// A8: MXFP8 activations (MXFP4 weights): the rows hold one e4m3 part, so each
// step runs one block-scaled MFMA per stream and loads no lo bytes.
// FUSED: a tile of the single-launch decode step (see FusedSync): GEMM1 writes
// the down projection's input rows in the form GEMM2 reads them (bf16 rows,
// or split: hi / lo parts, or MXFP8) with coherent stores and counts its row
// tile in; GEMM2 starts its weight stream, waits for its row tile, reads the
// rows with coherent loads, and writes its slot rows coherently.
// PK: MXFP4 codes from the packed layout (p.Bp): a stream's 16 rows of one
// 128-K step are 1 KB of one block, and lane (l16, q) reads its operand (row
// l16, chunk q) straight from its swizzled slot, so no register transpose.
template <int FMT, bool GATED, int SPT, bool A8, bool FUSED, bool PK = false>
__device__ __forceinline__ void skinny_tile(const Params& p, int mt, int nt, TileLds<FMT>& L,
                                            const FusedSync& fs) {
  static_assert(!PK || FMT == W_MXFP4, "packed codes are MXFP4");
  using C = Cfg<FMT>;
  auto& sbuf = L.sbuf;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (mt >= __builtin_amdgcn_readfirstlane(p.status[2])) return;  // workgroup-uniform, before any barrier
  const int seg = p.tile_seg[mt];
  const int row0 = p.tile_row0[mt];
  const int rows = min(BM, p.seg_end[seg] - row0);
  const int N = p.N, K = p.K;
  const int KB = K / 32;
  const int nch = (K + C::KC - 1) / C::KC;

  // this wave's two weight streams
  const int l16 = lane & 15, q = lane >> 4;
  const int nb = nt * block_cols(GATED) + wave * (GATED ? 16 : 32);
  const bool wave_on = nb < N;  // idle waves still stage A and meet every barrier
  const int c0 = nb + l16, c1 = GATED ? c0 : nb + 16 + l16;
  // weight rows of this segment as buffer resources; lane offsets: row, then
  // block q of the first step (MXFP4: 16 bytes per block, bf16: 64)
  const uint32_t rowbytes = FMT == W_MXFP4 ? K / 2 : 2 * K;
  const uint32_t segbytes = PK ? p.bp_expert : (uint32_t)N * rowbytes;  // range of the buffer resources
  const uint8_t* wb0 = PK ? p.Bp + (size_t)seg * segbytes : (const uint8_t*)p.B0 + (size_t)seg * segbytes;
  const uint8_t* wb1 = PK ? wb0 : (const uint8_t*)(GATED ? p.B1 : p.B0) + (size_t)seg * segbytes;
  const __amdgpu_buffer_rsrc_t rs0 = weight_rsrc(wb0, segbytes);
  const __amdgpu_buffer_rsrc_t rs1 = weight_rsrc(wb1, segbytes);
  const int KT = (K + PK_KSTAGE - 1) / PK_KSTAGE;  // PK: 128-K stages
  constexpr uint32_t BLOCK_BYTES = FMT == W_MXFP4 ? 16 : 64;
  // bf16: lane (l16, q) loads its own blocks. MXFP4: a chunk is 256 bytes of
  // each of a stream's 16 rows, loaded as 4 rows x 256 bytes per instruction,
  // whole 128-byte lines per request: instruction j, lane (l16, q) reads row
  // 4 j + (l16 % 4), 16-byte block 4 (l16 / 4) + q. quad_transpose then
  // exchanges the instruction index with lane bits 2-3, which leaves register
  // u holding, in lane (l16, q), block 4 u + q of row l16: the MFMA operand
  // of step u.
  uint32_t vo0[FMT == W_MXFP4 ? 4 : 1], vo1[FMT == W_MXFP4 ? 4 : 1];
  const int piece = 4 * (l16 >> 2) + q;  // MXFP4: this lane's 16-byte block of a chunk's 256 bytes
  if (PK) {  // vo[u]: step u of chunk 0 = stage u of the column tile's blocks
    constexpr int CT = GATED ? PK_COLS1 : PK_COLS2;
    const int ct = nb / CT, r0 = nb % CT + l16, r1 = (GATED ? PK_COLS1 : 16) + r0;
    const uint32_t lo0 = 64u * r0 + 16u * (q ^ ((r0 >> 2) & 3));
    const uint32_t lo1 = 64u * r1 + 16u * (q ^ ((r1 >> 2) & 3));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      vo0[u] = (uint32_t)(ct * KT + u) * PK_BLOCK + lo0;
      vo1[u] = (uint32_t)(ct * KT + u) * PK_BLOCK + lo1;
    }
  } else if (FMT == W_MXFP4) {
    const int b1 = GATED ? nb : nb + 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vo0[j] = (uint32_t)min(nb + 4 * j + (l16 & 3), N - 1) * rowbytes + 16 * piece;
      vo1[j] = (uint32_t)min(b1 + 4 * j + (l16 & 3), N - 1) * rowbytes + 16 * piece;
    }
  } else {
    vo0[0] = (uint32_t)min(c0, N - 1) * rowbytes + BLOCK_BYTES * q;
    vo1[0] = (uint32_t)min(c1, N - 1) * rowbytes + BLOCK_BYTES * q;
  }

  // MXFP4 scales of the workgroup's rows [n_lo, n_lo + RR) (GEMM1: gate in
  // LDS rows 0..63, up in 64..127), staged in LDS. Pieces past the valid rows
  // re-read the last valid piece; they land in rows no lane looks up.
  constexpr int RR = block_cols(GATED);  // weight rows per region
  const int n_lo = nt * RR;
  const uint8_t* sc0 = nullptr;
  const uint8_t* sc1 = nullptr;
  u32x4 sv[SPT > 0 ? SPT : 1];
  const int npieces = 8 * KB;  // 128 rows x KB bytes / 16
  if (FMT == W_MXFP4) {
    const int reg_pieces = RR * KB / 16;
    const int valid = min(RR, N - n_lo) * KB;  // bytes of a region that hold rows < N
    const size_t gbase = ((size_t)seg * N + n_lo) * KB;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int i = min(tid + NT * j, npieces - 1);
      const int reg = GATED ? (i >= reg_pieces) : 0;
      const int off = min((i - reg * reg_pieces) * 16, valid - 16);
      sv[j] = *(const u32x4*)((reg ? p.S1 : p.S0) + gbase + off);
    }
    sc0 = skinny_scales + (size_t)(min(c0, N - 1) - n_lo) * KB;
    sc1 = skinny_scales + (size_t)((GATED ? RR : 0) + min(c1, N - 1) - n_lo) * KB;
  }

  // This thread's activation pieces. bf16: piece j covers tile row r_j, 8 K
  // values at column 8 * pc of each chunk. Split (MXFP4): pieces of 16 hi
  // bytes and the same 16 lo bytes at column 16 * pc of rows r_j, and threads
  // 0..15 carry the 16 scale bytes of row tid. Rows past the segment end are
  // not loaded but written to LDS as zeros (their results are never stored;
  // decode tiles hold one or two live rows, and loading the other fourteen
  // would spend the compute unit's outstanding-request slots, which the
  // weight stream needs); K past the end is zeroed when written to LDS (the
  // split rows' scale codes there are 0).
  constexpr bool QA = FMT == W_MXFP4;
  constexpr bool COH_A = FUSED && !GATED;  // GEMM2's rows come from GEMM1 tiles of this launch
  constexpr int PPR = QA ? C::KC / 16 : C::KC / 8;  // pieces per row per chunk
  constexpr int NP = QA ? C::QPPT : C::PPT;          // pieces per thread (per array)
  constexpr int VPP = QA ? 16 : 8;                   // K values per piece
  const int pc = tid % PPR;
  size_t a_row[NP];
  int a_lds[NP];
  bool a_live[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int r = (tid + NT * j) / PPR;
    const int rr = min(r, rows - 1);
    a_live[j] = r < rows;
    a_row[j] = (size_t)(p.a_perm ? p.a_perm[row0 + rr] / p.a_div : row0 + rr);
    a_lds[j] = QA ? r * C::QROW + 16 * pc : (r * C::LROW + 8 * pc) * 2;
  }
  size_t s_row = 0;  // split rows: scale row of thread tid < 16
  if (QA) {
    const int rr = min(tid & 15, rows - 1);
    s_row = (size_t)(p.a_perm ? p.a_perm[row0 + rr] / p.a_div : row0 + rr);
  }

  struct ARegs {
    u32x4 v[NP];
    u32x4 l[QA ? NP : 1];
    u32x4 s;
  };
  // GEMM2 of the single launch reads the rows coherently, as offsets from
  // the split rows' base (the host keeps every offset below 2^32)
  const uint8_t* a_base = QA ? p.Aq.hi : (const uint8_t*)p.A;
  const __amdgpu_buffer_rsrc_t a_rs = coh_rsrc(a_base);
  auto ld_a = [&](const void* ptr) -> u32x4 {
    if constexpr (COH_A) return ld_coh128(a_rs, (uint32_t)((const uint8_t*)ptr - a_base));
    else return *(const u32x4*)ptr;
  };
  auto load_a = [&](ARegs& ar, int c) {
    const int kc = min(c * C::KC + VPP * pc, K - VPP);  // clamped: always inside the row
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      ar.v[j] = u32x4{0u, 0u, 0u, 0u};
      if (QA) ar.l[j] = u32x4{0u, 0u, 0u, 0u};
      if (a_live[j]) {
        if (QA) {
          ar.v[j] = ld_a(p.Aq.hi + a_row[j] * K + kc);
          if (!A8) ar.l[j] = ld_a(p.Aq.lo + a_row[j] * K + kc);
        } else {
          ar.v[j] = ld_a(p.A + a_row[j] * K + kc);
        }
      }
    }
    // chunks past the last (the loop below loads two ahead) re-read the last
    // chunk's scale bytes: a row holds exactly 16 * nch of them
    if (QA) ar.s = ld_a(p.Aq.sc + s_row * p.Aq.sc_stride + 16 * min(c, nch - 1));
  };
  auto store_a = [&](const ARegs& ar, int buf, int c) {
    const uint32_t m = c * C::KC + VPP * pc < K ? ~0u : 0u;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      *(u32x4*)&sbuf[buf][a_lds[j]] = ar.v[j] & m;
      if (QA && !A8) *(u32x4*)&sbuf[buf][BM * C::QROW + a_lds[j]] = ar.l[j] & m;
    }
    if (QA && tid < 16) *(u32x4*)&sbuf[buf][2 * BM * C::QROW + 16 * tid] = ar.s;
  };
  // step t = c * SPC + u covers blocks 4 t .. 4 t + 3 (4 BLOCK_BYTES bytes per row)
  // Chunks past the last are loaded too (the loop below has no exits); their
  // offset is moved past the segment, where buffer loads return 0 without a
  // memory access.
  // MXFP4: a lane's 16 bytes of the last chunk that lie past its row end
  // are not read either (their offset is moved past the segment too); the
  // next row's bytes would only meet zero activations.
  auto load_chunk = [&](WSet<FMT>& w, int c) {
    if constexpr (PK) {  // stages past the last (K tail, chunks past the last) read 0 without an access
      const int so = c < nch ? c * C::SPC * PK_BLOCK : 0;
#pragma unroll
      for (int u = 0; u < C::SPC; ++u) {
        const bool in_k = c < nch && c * C::SPC + u < KT;
        w.w0[u].q[0] = __builtin_amdgcn_raw_buffer_load_b128(rs0, in_k ? vo0[u] : segbytes, so, kAuxNt);
        w.w1[u].q[0] = __builtin_amdgcn_raw_buffer_load_b128(rs1, in_k ? vo1[u] : segbytes, so, kAuxNt);
      }
      return;
    }
    // chunks past the last: the VGPR offset itself lies past the segment
    // (the range check covers the VGPR offset, not the SGPR one)
    const bool live = c < nch;
    const int so = live ? c * C::SPC * 4 * BLOCK_BYTES : 0;
    const bool in_row = live && (uint32_t)so + 16u * (FMT == W_MXFP4 ? piece : l16) < rowbytes;
#pragma unroll
    for (int u = 0; u < C::SPC; ++u) {
      if (FMT == W_MXFP4) {  // w.w0[u]: instruction u (rows 4 u + l16 % 4)
        w.w0[u].q[0] = __builtin_amdgcn_raw_buffer_load_b128(rs0, in_row ? vo0[u] : segbytes, so, kAuxNt);
        w.w1[u].q[0] = __builtin_amdgcn_raw_buffer_load_b128(rs1, in_row ? vo1[u] : segbytes, so, kAuxNt);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // 16 bytes past the row end read 0 (w_operand_bf16 zeroes them anyway)
          const uint32_t o = 4 * BLOCK_BYTES * u + 16 * i;
          const bool inr = live && (uint32_t)so + BLOCK_BYTES * q + o < rowbytes;
          w.w0[u].q[i] = __builtin_amdgcn_raw_buffer_load_b128(rs0, inr ? vo0[0] + o : segbytes, so, kAuxNt);
          w.w1[u].q[i] = __builtin_amdgcn_raw_buffer_load_b128(rs1, inr ? vo1[0] + o : segbytes, so, kAuxNt);
        }
      }
    }
  };

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const WSet<FMT>& w, int buf, int c) {
    if (!wave_on) return;
    if constexpr (QA) {
      // the weights of each stream in the MFMA operand layout, one register
      // per step (see quad_transpose)
      u32x4 t0[4] = {w.w0[0].q[0], w.w0[1].q[0], w.w0[2].q[0], w.w0[3].q[0]};
      u32x4 t1[4] = {w.w1[0].q[0], w.w1[1].q[0], w.w1[2].q[0], w.w1[3].q[0]};
      if constexpr (!PK) {  // packed codes arrive in the operand layout
        quad_transpose(t0, lane);
        quad_transpose(t1, lane);
      }
      const uint8_t* hrow = &sbuf[buf][l16 * C::QROW];
      const uint8_t* lrow = hrow + BM * C::QROW;
      const uint8_t* srow = &sbuf[buf][2 * BM * C::QROW + 16 * l16];
#pragma unroll
      for (int u = 0; u < C::SPC; ++u) {
        const int kbc = min(4 * (c * C::SPC + u) + q, KB - 1);
        const u32x4 h0 = *(const u32x4*)(hrow + 128 * u + 16 * q);
        const u32x4 h1 = *(const u32x4*)(hrow + 128 * u + 64 + 16 * q);
        u32x4 l0 = {0u, 0u, 0u, 0u}, l1 = {0u, 0u, 0u, 0u};
        if (!A8) {
          l0 = *(const u32x4*)(lrow + 128 * u + 16 * q);
          l1 = *(const u32x4*)(lrow + 128 * u + 64 + 16 * q);
        }
        const i32x8 ah = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
        const i32x8 al = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
        const int sa = srow[4 * u + q];
        const int sb0 = sc0[kbc], sb1 = sc1[kbc];
        const u32x4 c0w = t0[u];
        const u32x4 c1w = t1[u];
        const i32x8 b0 = {(int)c0w[0], (int)c0w[1], (int)c0w[2], (int)c0w[3], 0, 0, 0, 0};
        const i32x8 b1 = {(int)c1w[0], (int)c1w[1], (int)c1w[2], (int)c1w[3], 0, 0, 0, 0};
        acc0 = mfma_fp8_fp4(ah, b0, acc0, sa, sb0);
        acc1 = mfma_fp8_fp4(ah, b1, acc1, sa, sb1);
        if (!A8) {
          acc0 = mfma_fp8_fp4(al, b0, acc0, sa, sb0);
          acc1 = mfma_fp8_fp4(al, b1, acc1, sa, sb1);
        }
      }
    } else {
      const uint16_t* arow = (const uint16_t*)&sbuf[buf][(l16 * C::LROW + 32 * q) * 2];
#pragma unroll
      for (int u = 0; u < C::SPC; ++u) {
        const int kb = 4 * (c * C::SPC + u) + q;
        const bool ok = kb < KB;
        u32x4 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *(const u32x4*)(arow + 128 * u + 8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 av = *(const bf16x8*)&a[i];
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, w_operand_bf16(w.w0[u], i, ok), acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, w_operand_bf16(w.w1[u], i, ok), acc1, 0, 0, 0);
        }
      }
    }
  };

  WSet<FMT> wx, wy;
  ARegs ar;
  load_chunk(wx, 0);
  // GEMM2 of the single launch: the weight stream has started; now wait for
  // the row tile's activation rows (all GEMM1 column tiles of row tile mt)
  if constexpr (COH_A) wait_count(&fs.done1[mt], fs.n_tiles1, fs);
  load_a(ar, 0);
  if (FMT == W_MXFP4) {
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if (tid + NT * j < npieces) *(u32x4*)(skinny_scales + (size_t)16 * (tid + NT * j)) = sv[j];
  }
  store_a(ar, 0, 0);
  lds_barrier();
  // Chunk c: weights in wx, activations in buffer 0; chunk c + 1: wy, buffer 1.
  // The loop runs whole pairs of chunks and has no exits, so every load in it
  // is unconditional and the compiler keeps exact wait counts: the next chunk
  // stays in flight. A step past the last chunk only meets the barrier.
#define MOE_SKINNY_STEP(wcur, wnext, cc)                    \
  {                                                         \
    load_a(ar, (cc) + 1);                                   \
    load_chunk(wnext, (cc) + 1);                            \
    if ((cc) < nch) compute(wcur, (cc) & 1, cc);            \
    store_a(ar, ((cc) + 1) & 1, (cc) + 1);                  \
    lds_barrier();                                          \
  }
  for (int c = 0; c < nch; c += 2) {
    MOE_SKINNY_STEP(wx, wy, c)
    MOE_SKINNY_STEP(wy, wx, c + 1)
  }
#undef MOE_SKINNY_STEP

  // 16x16 result layout: lane holds column (lane & 15), rows 4 (lane >> 4) + r.
  const ActParams ap = act_for(p.act, p.ep, seg);
  const float es = scale_for(GATED ? p.ep.fc1 : p.ep.fc2, seg);  // fc1 on gate and up, fc2 on down
  if constexpr (GATED && (A8 || (FUSED && QA))) {
    // The down projection's input rows quantized here for the block-scaled
    // MFMA, from the activation (times the route weight), with the same rule
    // as quant_row: MXFP8 from the fp32 value (A8), or the exact hi / lo split
    // of its bf16 rounding (the single launch with bf16 activations). A
    // 32-value block of a row spans the 16 columns of two waves (w, w ^ 1):
    // each wave reduces its magnitude over its 16 lanes, the pair exchanges
    // the two halves through LDS. N is a multiple of 64 here (the host
    // requires I % 64 == 0), so every wave has columns.
    float v[4], m[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = q * 4 + r;
      v[r] = gated_act(ap, acc0[r] * es, acc1[r] * es) * (p.row_w && row < rows ? p.row_w[row0 + row] : 1.f);
      if (!A8) v[r] = bf16_bits_to_f32(f32_to_bf16_rne(v[r]));
      m[r] = fabsf(v[r]);
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) m[r] = fmaxf(m[r], __shfl_xor(m[r], off));
      if (l16 == 0) L.half_amax[wave][row] = m[r];
    }
    lds_barrier();
    const int blk = (nt * block_cols(true) + wave * 16) / 32;
    const int KBo = N / 32;
    const size_t Rq = (size_t)p.Cq.lo - (size_t)p.Cq.hi;  // rows x N bytes between the hi and lo parts
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = q * 4 + r;
      const float amax = fmaxf(m[r], L.half_amax[wave ^ 1][row]);
      const int code = min(max((int)((__float_as_uint(amax) >> 23) & 0xffu) - (A8 ? 8 : 7), 0), 254);
      const float inv = __uint_as_float((uint32_t)(254 - code) << 23);  // 2^(127 - code)
      uint32_t hb, lb = 0;
      if (A8) {
        hb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(v[r] * inv), 0.f, 0, false) & 0xffu;
      } else {
        const float sv0 = v[r] * inv;
        const int h = __builtin_amdgcn_cvt_pk_fp8_f32(sv0, 0.f, 0, false);
        const f32x2 hf = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
        hb = (uint32_t)h & 0xffu;
        lb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sv0 - hf[0], 0.f, 0, false) & 0xffu;
      }
      uint8_t* hi_row = p.Cq.hi + (size_t)(row0 + row) * N;
      uint8_t* sc_row = p.Cq.sc + (size_t)(row0 + row) * p.Cq.sc_stride;
      if (FUSED) {  // four columns per store, agent-coherent
        const uint32_t h4 = gather4(hb), l4 = A8 ? 0u : gather4(lb);
        if (row < rows && (l16 & 3) == 0) {
          st_coh32(hi_row + c0, h4);
          if (!A8) st_coh32(hi_row + Rq + c0, l4);
        }
        if (row < rows && l16 == 0 && (wave & 1) == 0) st_coh8(sc_row + blk, (uint32_t)code);
        if (row < rows && nt == p.n_tiles - 1 && wave == 0 && KBo + l16 < p.Cq.sc_stride) st_coh8(sc_row + KBo + l16, 0u);
      } else if (row < rows) {
        hi_row[c0] = (uint8_t)hb;
        if (!A8) hi_row[Rq + c0] = (uint8_t)lb;
        if (l16 == 0 && (wave & 1) == 0) sc_row[blk] = (uint8_t)code;
        // the row's scale bytes past its last block (up to the 16-byte padded
        // stride) are 0, like the ones quant_row writes: GEMM2 reads them
        if (nt == p.n_tiles - 1 && wave == 0 && KBo + l16 < p.Cq.sc_stride) sc_row[KBo + l16] = 0;
      }
    }
    if (FUSED) count_in(&fs.done1[mt]);
    return;
  }
  if (FUSED) {
    // bf16 rows out, two columns per store, agent-coherent (GEMM1: the bf16
    // activation rows GEMM2 reads; GEMM2: the slot rows the combine reads).
    // N is a multiple of 64, so a wave with columns has all 16 (32) of them.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = q * 4 + r;
      uint32_t b0, b1 = 0;
      if (GATED)
        b0 = f32_to_bf16_rne(gated_act(ap, acc0[r] * es, acc1[r] * es) *
                             (p.row_w && row < rows ? p.row_w[row0 + row] : 1.f));
      else {
        b0 = f32_to_bf16_rne(acc0[r] * es);
        b1 = f32_to_bf16_rne(acc1[r] * es);
      }
      const uint32_t n0 = (uint32_t)__shfl_down((int)b0, 1), n1 = (uint32_t)__shfl_down((int)b1, 1);
      if (wave_on && row < rows && (l16 & 1) == 0) {
        uint16_t* dst = p.C + (size_t)(row0 + row) * N;
        st_coh32(dst + c0, b0 | n0 << 16);
        if (!GATED) st_coh32(dst + c1, b1 | n1 << 16);
      }
    }
    count_in(GATED ? &fs.done1[mt] : fs.done2);
    return;
  }
  if (!wave_on) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = q * 4 + r;
    if (row >= rows) continue;
    uint16_t* dst = p.C + (size_t)(row0 + row) * N;
    if (GATED) {
      if (c0 < N)
        dst[c0] = f32_to_bf16_rne(gated_act(ap, acc0[r] * es, acc1[r] * es) * (p.row_w ? p.row_w[row0 + row] : 1.f));
    } else {
      if (c0 < N) dst[c0] = f32_to_bf16_rne(acc0[r] * es);
      if (c1 < N) dst[c1] = f32_to_bf16_rne(acc1[r] * es);
    }
  }
}

// One tile per workgroup: blockIdx.x = row tile x column tiles + column tile.
template <int FMT, bool GATED, int SPT, bool A8 = false, bool PK = false>
__global__ __launch_bounds__(NT) void k_gemm(const Params p) {
  __shared__ TileLds<FMT> L;
  const int mt = blockIdx.x / p.n_tiles;
  skinny_tile<FMT, GATED, SPT, A8, false, PK>(p, mt, blockIdx.x - mt * p.n_tiles, L, FusedSync{});
}

// The combine of the single launch: token t's slot rows, j ascending in fp32
// (as k_combine), read with agent-coherent loads once every GEMM2 tile is in.
struct FusedCombine {
  const uint16_t* y;        // [rows, H] slot rows, sorted order
  const int32_t* inv_perm;  // [T, k]
  int32_t T, k, H;
  uint16_t* out;            // [T, H]
};

__device__ __forceinline__ void fused_combine_token(const FusedCombine& c, int t) {
  const int32_t* ip = c.inv_perm + (size_t)t * c.k;
  const __amdgpu_buffer_rsrc_t y_rs = coh_rsrc(c.y);
  for (int h = threadIdx.x * 8; h < c.H; h += NT * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < c.k; ++j) {
      const int r = ip[j];
      if (r < 0) continue;
      const u32x4 v = ld_coh128(y_rs, (uint32_t)(((size_t)r * c.H + h) * 2));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_bits_to_f32(v[i] & 0xffffu);
        acc[2 * i + 1] += bf16_bits_to_f32(v[i] >> 16);
      }
    }
    u32x4 o;
    o[0] = pack_bf16x2(acc[0], acc[1]);
    o[1] = pack_bf16x2(acc[2], acc[3]);
    o[2] = pack_bf16x2(acc[4], acc[5]);
    o[3] = pack_bf16x2(acc[6], acc[7]);
    *(u32x4*)(c.out + (size_t)t * c.H + h) = o;
  }
}

// The single-launch decode step after the align prologue: GEMM1 tiles
// (row-tile major), GEMM2 tiles (row-tile major), then one item per token for
// the combine, taken from the work queue.
template <int FMT, int SPT1, int SPT2, bool A8>
__global__ __launch_bounds__(NT) void k_decode_fused(const Params p1, const Params p2, const FusedCombine fc,
                                                     const FusedSync fs) {
  __shared__ TileLds<FMT> L;
  __shared__ int s_item;
  const int mtl = __builtin_amdgcn_readfirstlane(p1.status[2]);
  const int n1 = mtl * p1.n_tiles, n2 = mtl * p2.n_tiles;
  const int total = n1 + n2 + fc.T;
  // Wave 0 takes items from the queue, fs.batch consecutive ones at a time
  // (lane 0 adds the batch, the others 0: lane 0's old value is the first
  // item), and hands them to the other waves through LDS. The next batch is
  // taken while the current one runs, so the atomic's round trip stays off
  // the critical path; it always lies later in queue order than the current
  // one, items run in queue order, and waits only ever point to earlier items.
  const int B = fs.batch;
  auto take = [&]() -> int {
    int v = 0;
    if (wave_id() == 0)
      v = __hip_atomic_fetch_add(fs.queue, (threadIdx.x & 63) == 0 ? B : 0, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    return v;
  };
  auto publish = [&](int v) {
    if (wave_id() == 0) s_item = __builtin_amdgcn_readfirstlane(v);
    lds_barrier();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    lds_barrier();
    return item;
  };
  int first = publish(take());
  // a workgroup takes at most every item once: the bound only guards the loop
  for (int it = 0; it <= total && first < total; ++it) {
    const int next = take();
    for (int item = first; item < min(first + B, total); ++item) {
    if (item < n1) {
      const int mt = item / p1.n_tiles;
      skinny_tile<FMT, true, SPT1, A8, true>(p1, mt, item - mt * p1.n_tiles, L, fs);
    } else if (item < n1 + n2) {
      const int i2 = item - n1, mt = i2 / p2.n_tiles;
      skinny_tile<FMT, false, SPT2, A8, true>(p2, mt, i2 - mt * p2.n_tiles, L, fs);
    } else {
      wait_count(fs.done2, n2, fs);
      fused_combine_token(fc, item - n1 - n2);
    }
    }
    first = publish(next);
  }
}

}  // namespace skinny
}  // namespace moe
