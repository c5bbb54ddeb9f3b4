// Grouped GEMM for few rows per segment (decode): weights streamed from HBM
// straight into MFMA operand registers; the tile's activation rows are staged
// through LDS in K chunks shared by the workgroup's waves.
//
// Same grouped-GEMM definition as the prefill kernel (moonep_experts page,
// moonep_grouped_gemm; route weight on the activation per the module
// docstring). Weights may be bf16 or MXFP4 (trtllm_mxfp4_moe page,
// TrtLlmMxfp4ExpertsBase._supports_quant_scheme: MXFP4 weights with
// unquantized activations): e2m1 codes with an e8m0 scale per 32 K elements
// (OCP Microscaling v1.0 reading). MXFP4 codes are decoded to bf16 in
// registers with v_cvt_scalef32_pk_bf16_fp4; every e2m1 value times a power of
// two in the bf16 range is exact in bf16, so the MFMA sees the exact weights.
//
// Tile: 16 rows. Each wave owns two 16-column weight streams: gate and up of
// the same 16 columns (GEMM1), or two adjacent 16-column groups (GEMM2), so a
// wave moves the same bytes per K step in both GEMMs. 4 waves per workgroup.
// v_mfma_f32_16x16x32_bf16 with the activations as the A operand (row =
// lane & 15) and the weights as the B operand (column = lane & 15). The K
// order inside a dot product is free as long as A and B agree, so in K step s
// (128 values) lane group q = lane >> 4 owns the 32-value scale block
// kb = 4 s + q: one 16-byte load carries a lane's 32 MXFP4 codes, whose single
// scale comes with them, and feeds four MFMAs of 8 K values each; the 16 lanes
// of a group read 64 contiguous bytes of each of 16 weight rows.
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

struct Params {
  const uint16_t* A;      // rows [*, K] bf16
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
  uint16_t* C;
  const float* row_w;
  ActParams act;
};

// e8m0 scale code -> f32 2^(v - 127); 0 -> 2^-127 (subnormal), 255 -> NaN.
// Written as selects so that it stays branch-free.
__device__ __forceinline__ float e8m0_to_f32(uint32_t v) {
  const uint32_t bits = v == 0u ? 0x00400000u : v == 255u ? 0x7fc00000u : v << 23;
  return __uint_as_float(bits);
}

// 8 e2m1 codes (one dword, element 2i in the low nibble of byte i) -> 8 bf16
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

template <int FMT>
struct Cfg {
  static constexpr int SPC = FMT == W_MXFP4 ? 4 : 1;  // K steps per chunk
  static constexpr int KC = SPC * 128;                // K values per chunk
  static constexpr int LROW = KC + 8;                 // LDS row stride (bf16): 16 B pad
  static constexpr int PIECES = BM * KC / 8;          // 16-byte pieces of an A chunk
  static constexpr int PPT = PIECES / NT;             // pieces per thread
  static_assert(PIECES % NT == 0, "A chunk must split evenly over the workgroup");
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

// Raw loads of one lane's K block (no selects here: a value consumed right
// after its load would make the compiler wait for it early). The block index
// is clamped to the row, so every lane issues the same loads; compute()
// neutralises blocks past the row end.
template <int FMT>
__device__ __forceinline__ void load_w(WChunk<FMT>& w, const void* Bm, size_t row, int K, int kb) {
  const int kbc = min(kb, K / 32 - 1);
  if (FMT == W_BF16) {
    const u32x4* src = (const u32x4*)((const uint16_t*)Bm + row * K + (size_t)kbc * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) w.q[i] = src[i];
  } else {
    w.q[0] = *(const u32x4*)((const uint8_t*)Bm + row * (K / 2) + (size_t)kbc * 16);
  }
}

// MFMA B operand i (8 K values) of a lane's block. A block past the row end
// (!ok) multiplies activations that are zero, and is made zero (bf16) or finite
// (MXFP4: scale code 0) so that the product is exactly 0.
template <int FMT>
__device__ __forceinline__ bf16x8 w_operand(const WChunk<FMT>& w, int i, float scale, bool ok) {
  if (FMT == W_BF16) {
    const uint32_t m = ok ? ~0u : 0u;
    const u32x4 v = w.q[i] & m;
    return *(const bf16x8*)&v;
  } else {
    const uint32_t d = i == 0 ? w.q[0][0] : i == 1 ? w.q[0][1] : i == 2 ? w.q[0][2] : w.q[0][3];
    return fp4x8_to_bf16(d, scale);
  }
}

// Barrier that orders LDS accesses only: global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

extern __shared__ __attribute__((aligned(16))) uint8_t skinny_scales[];

// SPT: scale pieces per thread (MXFP4; 0 for bf16), scale_pieces_per_thread(K).
template <int FMT, bool GATED, int SPT>
__global__ __launch_bounds__(NT) void k_gemm(const Params p) {
  using C = Cfg<FMT>;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * C::LROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mt = blockIdx.x / p.n_tiles;
  const int nt = blockIdx.x - mt * p.n_tiles;
  if (mt >= p.status[2]) return;  // workgroup-uniform, before any barrier
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
  const size_t wr0 = (size_t)seg * N + min(c0, N - 1);
  const size_t wr1 = (size_t)seg * N + min(c1, N - 1);
  const void* B1 = GATED ? p.B1 : p.B0;

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

  // This thread's A pieces: piece j covers tile row r_j, 8 K values at column
  // 8 * pc of each chunk. Rows past the segment end re-read the last row (their
  // results are never stored); K past the end is zeroed when written to LDS.
  constexpr int PPR = C::KC / 8;  // pieces per row per chunk
  const int pc = tid % PPR;
  const uint16_t* a_src[C::PPT];
  int a_lds[C::PPT];
#pragma unroll
  for (int j = 0; j < C::PPT; ++j) {
    const int r = (tid + NT * j) / PPR;
    const int rr = min(r, rows - 1);
    const int ar = p.a_perm ? p.a_perm[row0 + rr] / p.a_div : row0 + rr;
    a_src[j] = p.A + (size_t)ar * K + 8 * pc;
    a_lds[j] = r * C::LROW + 8 * pc;
  }

  auto load_a = [&](u32x4 (&ar)[C::PPT], int c) {
    const int kc = min(c * C::KC, K - 8 - 8 * pc);  // clamped: always inside the row
#pragma unroll
    for (int j = 0; j < C::PPT; ++j) ar[j] = *(const u32x4*)(a_src[j] + kc);
  };
  auto store_a = [&](const u32x4 (&ar)[C::PPT], int buf, int c) {
    const uint32_t m = c * C::KC + 8 * pc < K ? ~0u : 0u;
#pragma unroll
    for (int j = 0; j < C::PPT; ++j) *(u32x4*)&sA[buf][a_lds[j]] = ar[j] & m;
  };
  auto load_chunk = [&](WSet<FMT>& w, int c) {
#pragma unroll
    for (int u = 0; u < C::SPC; ++u) {
      const int kb = 4 * (c * C::SPC + u) + q;
      load_w<FMT>(w.w0[u], p.B0, wr0, K, kb);
      load_w<FMT>(w.w1[u], B1, wr1, K, kb);
    }
  };

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const WSet<FMT>& w, int buf, int c) {
    if (!wave_on) return;
    const uint16_t* arow = &sA[buf][l16 * C::LROW + 32 * q];
#pragma unroll
    for (int u = 0; u < C::SPC; ++u) {
      const int kb = 4 * (c * C::SPC + u) + q;
      const bool ok = kb < KB;
      u32x4 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const u32x4*)(arow + 128 * u + 8 * i);
      float s0 = 1.f, s1 = 1.f;
      if (FMT == W_MXFP4) {
        const int kbc = min(kb, KB - 1);
        s0 = e8m0_to_f32(ok ? (uint32_t)sc0[kbc] : 0u);
        s1 = e8m0_to_f32(ok ? (uint32_t)sc1[kbc] : 0u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 av = *(const bf16x8*)&a[i];
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, w_operand<FMT>(w.w0[u], i, s0, ok), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, w_operand<FMT>(w.w1[u], i, s1, ok), acc1, 0, 0, 0);
      }
    }
  };

  WSet<FMT> wx, wy;
  u32x4 ar[C::PPT];
  load_a(ar, 0);
  load_chunk(wx, 0);
  if (FMT == W_MXFP4) {
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if (tid + NT * j < npieces) *(u32x4*)(skinny_scales + (size_t)16 * (tid + NT * j)) = sv[j];
  }
  store_a(ar, 0, 0);
  lds_barrier();
  // Chunk c: weights in wx, activations in buffer 0; chunk c + 1: wy, buffer 1.
  // The loop body has no exits, so every load in it is unconditional and the
  // compiler keeps exact wait counts: the next chunk stays in flight.
  int c = 0;
  for (; c + 2 < nch; c += 2) {
    load_a(ar, c + 1);
    load_chunk(wy, c + 1);
    compute(wx, 0, c);
    store_a(ar, 1, c + 1);
    lds_barrier();
    load_a(ar, c + 2);
    load_chunk(wx, c + 2);
    compute(wy, 1, c + 1);
    store_a(ar, 0, c + 2);
    lds_barrier();
  }
  if (c + 1 < nch) {
    load_a(ar, c + 1);
    load_chunk(wy, c + 1);
    compute(wx, 0, c);
    store_a(ar, 1, c + 1);
    lds_barrier();
    compute(wy, 1, c + 1);
  } else {
    compute(wx, 0, c);
  }

  // 16x16 result layout: lane holds column (lane & 15), rows 4 (lane >> 4) + r.
  if (!wave_on) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = q * 4 + r;
    if (row >= rows) continue;
    uint16_t* dst = p.C + (size_t)(row0 + row) * N;
    if (GATED) {
      if (c0 < N) dst[c0] = f32_to_bf16_rne(gated_act(p.act, acc0[r], acc1[r]) * p.row_w[row0 + row]);
    } else {
      if (c0 < N) dst[c0] = f32_to_bf16_rne(acc0[r]);
      if (c1 < N) dst[c1] = f32_to_bf16_rne(acc1[r]);
    }
  }
}

}  // namespace skinny
}  // namespace moe
