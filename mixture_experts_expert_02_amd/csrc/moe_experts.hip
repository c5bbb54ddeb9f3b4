// Host side of the MoE experts library: argument checks, workspace layout,
// kernel launch sequence. Exports the C ABI declared in include/moe_experts.h.
//
// Launch sequence of a token-major forward, all on the caller's stream, no
// host synchronisation and no device reads on the host:
//   align (1 or 3 kernels) -> GEMM1 (+ activation x route weight) -> GEMM2 -> combine
// The GEMM grids are sized on the host from upper bounds (rows / BM + segments);
// workgroups past the device-side tile count exit at once, so no readback is needed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>

#include "../../include/moe_experts.h"
#include "align.hpp"
#include "combine.hpp"
#include "gemm_bf16.hpp"
#include "gemm_cold.hpp"
#include "gemm_skinny.hpp"
#include "gemm_mx.hpp"
#include "decode_prologue.hpp"
#include "router.hpp"
#include "scale_rows.hpp"

namespace {

constexpr int kMaxExperts = 4096;
constexpr int kFusedMaxRows = 4096;
constexpr int kFusedMaxExperts = 1024;
constexpr size_t kAlign = 256;
constexpr int kMaxSplitK = 4;

// Workspace of moe_experts_forward_noalloc: one array per device, held from
// the library's load until the process ends. Host code never uses its name
// as an address: each device's copy is reached through the pointer that
// hipGetSymbolAddress returns with that device current (scratch_on_device).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address, looked up once per device (no allocation).
int scratch_on_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

size_t up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }
int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

int bits_for(int E) {  // bits needed for keys 0..E
  int b = 0;
  while ((1 << b) <= E) ++b;
  return b;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// MXFP4 weights with MXFP8 activations and more than 32 rows per expert on
// average (token-major entry): the LDS-tiled block-scaled kernels of
// gemm_mx.hpp. MOE_EXPERTS_MX_PREFILL=0 (read at every call) sends these
// problems to the weight-streaming kernels instead (tests compare the two).
bool use_mxbig(const moe_problem& p, long long rows, bool grouped) {
  if (grouped || p.wfmt != MOE_W_MXFP4 || p.a_fmt != MOE_A_MXFP8 || rows <= 32LL * p.E) return false;
  const char* e = std::getenv("MOE_EXPERTS_MX_PREFILL");
  return !(e && std::atoi(e) == 0);
}

// Decode-shaped problems (few rows per weight row) and the other MXFP4
// problems use the weight-streaming kernels; the rest the LDS-tiled MFMA
// kernels.
bool use_skinny(const moe_problem& p, long long rows) {
  return p.wfmt == MOE_W_MXFP4 || rows <= 32LL * p.E;
}

// bf16 prefill problems run their cold segments (at most 32 rows) in the
// cold-segment kernels beside the tiled kernels unless MOE_EXPERTS_COLD=0
// (read at every call; tests compare the two).
bool cold_enabled() {
  const char* e = std::getenv("MOE_EXPERTS_COLD");
  return !(e && std::atoi(e) == 0);
}

struct Plan {
  long long M;   // rows (T*k, or NvS)
  bool skinny;
  int BM;
  int mt_cap;
  int s_cap;     // GEMM2 K ranges the y buffer has room for (token-major big-tile path)
  bool fused_align;
  int chunk, nch;
  // byte offsets
  size_t status, counts, cu, offsets, tile_seg, tile_row0, blkcnt, blkbad, perm, inv_perm, w_sorted, xs, act,
      xq, aq, y, total;
  size_t sync;   // single-launch decode counters: [queue, done2, -, -, done1[mt_cap]] (0 = none)
  int n_sync;
  bool fused;    // the forward runs the single-launch decode step
  // LDS-tiled MXFP4 x MXFP8 kernels: scale blocks of GEMM1's A (sa1) and
  // GEMM2's A (sa2, written by GEMM1), of the weights (ws1, ws2); column
  // tiles and 128-K stages of each GEMM
  bool mxbig;
  size_t sa1, sa2, ws1, ws2;
  int NT1, KT1, NT2, KT2;
  // bf16 prefill: segments of at most moe::cold::MAX_ROWS rows run in the
  // cold-segment kernels beside the tiled ones (cold_seg: their list)
  bool cold;
  size_t cold_seg;
};

int check_problem(const moe_problem* p, bool grouped) {
  if (!p) return MOE_EINVAL;
  if (p->T < 0 || p->H <= 0 || p->I <= 0 || p->E <= 0) return MOE_EINVAL;
  if (!grouped && (p->k <= 0 || p->k > p->E)) return MOE_EINVAL;
  if (p->wfmt != MOE_W_BF16 && p->wfmt != MOE_W_MXFP4) return MOE_EINVAL;
  if (p->act != MOE_ACT_SILU && p->act != MOE_ACT_SWIGLU_OAI && p->act != MOE_ACT_SITU) return MOE_EINVAL;
  if (p->act == MOE_ACT_SWIGLU_OAI) {
    if (!std::isfinite(p->alpha) || !std::isfinite(p->beta) || std::isnan(p->limit)) return MOE_EINVAL;
    if (!(p->limit > 0.f)) return MOE_ENOTSUP;
  }
  if (p->act == MOE_ACT_SITU) {  // the page requires both parameters > 0
    if (!std::isfinite(p->alpha) || !std::isfinite(p->beta)) return MOE_EINVAL;
    if (!(p->alpha > 0.f) || !(p->beta > 0.f)) return MOE_ENOTSUP;
  }
  if (p->weight_on_input != 0 && p->weight_on_input != 1) return MOE_EINVAL;
  if (p->a_fmt != MOE_A_BF16 && p->a_fmt != MOE_A_MXFP8) return MOE_EINVAL;
  if (p->a_fmt == MOE_A_MXFP8 && p->wfmt != MOE_W_MXFP4) return MOE_ENOTSUP;  // block-scaled MFMA path only
  if (p->mx_packed && (p->wfmt != MOE_W_MXFP4 || !aligned16(p->mx_packed))) return MOE_EINVAL;
  if (p->bf16_packed && (p->wfmt != MOE_W_BF16 || !aligned16(p->bf16_packed))) return MOE_EINVAL;
  const void* ep[] = {p->alpha_e, p->beta_e, p->limit_e, p->fc1_alpha, p->fc2_alpha};
  for (const void* q : ep)
    if (((uintptr_t)q & 3u) != 0) return MOE_EINVAL;
  if (p->H % 64 || p->I % 64) return MOE_ENOTSUP;
  if (p->wfmt == MOE_W_MXFP4 && (p->H > moe::skinny::kMaxMxfp4K || p->I > moe::skinny::kMaxMxfp4K))
    return MOE_ENOTSUP;
  if (p->E > kMaxExperts) return MOE_ENOTSUP;
  const long long rows = grouped ? (long long)p->T : (long long)p->T * p->k;
  if (rows > (1LL << 30)) return MOE_ENOTSUP;
  // The kernels address activation rows and one expert's weights with 32-bit
  // byte offsets: T*H and rows*max(H, I) below 2^31 elements, I*H at most 2^30.
  if ((long long)p->T * p->H >= (1LL << 31) || rows * std::max(p->H, p->I) >= (1LL << 31) ||
      (long long)p->I * p->H > (1LL << 30))
    return MOE_ENOTSUP;
  return MOE_OK;
}

// The single-launch decode step is taken only with MOE_EXPERTS_FUSED_DECODE=1
// (read at every call): measured on MI355X it is slower than the separate
// launches (align, GEMM1, activation split, GEMM2, combine), because every
// tile must wait for its write-through hand-over stores before counting in.
bool fused_decode_enabled() {
  const char* e = std::getenv("MOE_EXPERTS_FUSED_DECODE");
  return e && std::atoi(e) == 1;
}

// Items the single-launch decode step's workgroups take from its queue at a
// time: MOE_EXPERTS_FUSED_BATCH=<n> (tuning override, n >= 1); read once.
int fused_batch() {
  static const int v = [] {
    const char* e = std::getenv("MOE_EXPERTS_FUSED_BATCH");
    const int n = e ? std::atoi(e) : 0;
    return n > 0 ? n : 4;
  }();
  return v;
}

// Upper bound on GEMM2's K ranges: MOE_EXPERTS_MAX_SPLIT_K=<n> (n >= 1), read
// at every call (tests use it to pin the split); unset = kMaxSplitK.
int max_split_k() {
  const char* e = std::getenv("MOE_EXPERTS_MAX_SPLIT_K");
  const int n = e ? std::atoi(e) : 0;
  return n > 0 ? std::min(n, kMaxSplitK) : kMaxSplitK;
}

// Workspace layout of problem p. The y buffer comes last and holds s_cap
// partial outputs; with ws_bytes given, s_cap shrinks to what fits, so a
// workspace sized for a larger T (fewer K ranges, more rows) still serves.
size_t quant_bytes(long long R, int K) {
  return (size_t)R * (2ull * K + moe::skinny::quant_sc_stride(K));
}

// Packed MXFP4 x MXFP8 prefill weights: bytes of one expert's GEMM1 blocks
// and of one expert's GEMM2 blocks (gemm_mx.hpp, PK_STAGE).
size_t mx_packed_expert1(const moe_problem& p) {
  return (size_t)ceil_div(p.I, moe::mx::BN / 2) * ceil_div(p.H, moe::mx::BK) * moe::mx::PK_STAGE;
}
size_t mx_packed_expert2(const moe_problem& p) {
  return (size_t)ceil_div(p.H, moe::mx::BN) * ceil_div(p.I, moe::mx::BK) * moe::mx::PK_STAGE;
}

Plan make_plan(const moe_problem& p, bool grouped, size_t ws_bytes = ~(size_t)0) {
  Plan pl{};
  pl.M = grouped ? (long long)p.T : (long long)p.T * p.k;
  pl.mxbig = use_mxbig(p, pl.M, grouped);
  pl.skinny = !pl.mxbig && use_skinny(p, pl.M);
  pl.BM = pl.skinny ? moe::skinny::BM : pl.mxbig ? moe::mx::BM : moe::big::BM;
  if (pl.mxbig) {
    pl.NT1 = ceil_div(p.I, moe::mx::BN / 2);
    pl.KT1 = ceil_div(p.H, moe::mx::BK);
    pl.NT2 = ceil_div(p.H, moe::mx::BN);
    pl.KT2 = ceil_div(p.I, moe::mx::BK);
  }
  pl.mt_cap = ceil_div(pl.M, pl.BM) + (int)std::min<long long>(p.E, pl.M);
  // Splitting GEMM2's K only pays when its tiles fill a few rounds of the
  // compute units at most; with up to 1024 tiles (four rounds of 256 units)
  // room is kept for four partial outputs.
  pl.s_cap = 1;
  if (!grouped && !pl.skinny && (long long)pl.mt_cap * ceil_div(p.H, moe::big::BN) <= 1024)
    pl.s_cap = std::max(1, std::min(max_split_k(), pl.mxbig ? pl.KT2 : p.I / moe::big::BK));
  pl.cold = !pl.skinny && !pl.mxbig && p.wfmt == MOE_W_BF16 && cold_enabled();
  pl.fused_align = !grouped && pl.M <= kFusedMaxRows && p.E <= kFusedMaxExperts;
  if (!grouped && !pl.fused_align) {
    pl.chunk = (int)std::max<long long>(512, (ceil_div(pl.M, 256) + 63) / 64 * 64);
    pl.nch = ceil_div(pl.M, pl.chunk);
  }
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = up(o + bytes);
    return at;
  };
  pl.status = take(32);
  pl.counts = take(4ull * p.E);
  pl.cu = take(4ull * p.E);
  pl.offsets = take(4ull * p.E);
  pl.tile_seg = take(4ull * std::max(pl.mt_cap, 1));
  pl.tile_row0 = take(4ull * std::max(pl.mt_cap, 1));
  if (pl.cold) pl.cold_seg = take(4ull * p.E);
  if (!grouped) {
    if (!pl.fused_align) {
      pl.blkcnt = take(4ull * pl.nch * p.E);
      pl.blkbad = take(4ull * pl.nch);
    }
    pl.perm = take(4ull * pl.M);
    pl.inv_perm = take(4ull * pl.M);
    pl.w_sorted = take(4ull * pl.M);
  }
  // the single-launch decode step: weight-streaming tiles, the one-workgroup
  // align, inputs as given (no weighted copy), K of both GEMMs <= 4096
  const bool fused_ok =
      !grouped && pl.skinny && pl.fused_align && !p.weight_on_input && std::max(p.H, p.I) <= 4096;
  pl.fused = fused_ok && fused_decode_enabled();
  if (fused_ok) {  // reserved whether or not the override turns the single launch off
    pl.n_sync = 4 + pl.mt_cap;
    pl.sync = take(4ull * pl.n_sync);
  }
  if (p.weight_on_input) pl.xs = take(2ull * pl.M * p.H);  // routed rows x * w, sorted order
  if (pl.mxbig) {
    // x rows quantized in token order (the weighted copies in sorted order),
    // GEMM2's input codes in sorted order, the scale blocks
    const size_t blk = moe::mx::SC_BYTES;
    pl.xq = take(quant_bytes(p.weight_on_input ? pl.M : (long long)p.T, p.H));
    pl.sa1 = take(blk * pl.mt_cap * pl.KT1);
    pl.aq = take((size_t)pl.M * p.I);
    pl.sa2 = take(blk * pl.mt_cap * pl.NT1);
    pl.ws1 = take(blk * p.E * pl.NT1 * pl.KT1);
    pl.ws2 = take(blk * p.E * pl.NT2 * pl.KT2);
  } else {
    pl.act = take(2ull * pl.M * p.I);
    if (p.wfmt == MOE_W_MXFP4) {  // activation rows split for the block-scaled MFMA, sorted order
      pl.xq = take(quant_bytes(pl.M, p.H));
      pl.aq = take(quant_bytes(pl.M, p.I));
    }
  }
  if (!grouped) {
    pl.y = o;
    const size_t one = 2ull * pl.M * p.H;
    if (pl.s_cap > 1 && ws_bytes >= pl.y + one && ws_bytes < pl.y + one * pl.s_cap)
      pl.s_cap = (int)((ws_bytes - pl.y) / one);
    take(one * pl.s_cap);
  }
  pl.total = o;
  return pl;
}

template <typename T>
T* at(void* base, size_t off) {
  return (T*)((char*)base + off);
}

// hi and lo bytes, then scale rows, of R split activation rows of K values
moe::skinny::QRows quant_rows_at(void* base, size_t off, long long R, int K) {
  moe::skinny::QRows q;
  q.hi = at<uint8_t>(base, off);
  q.lo = q.hi + (size_t)R * K;
  q.sc = q.lo + (size_t)R * K;
  q.sc_stride = moe::skinny::quant_sc_stride(K);
  return q;
}

// Split R activation rows; with perm, row r comes from source row perm[r] / div
// (the first status[1] rows).
// (mx8: as MXFP8 activations, one e4m3 part per value).
int launch_quant(bool mx8, const void* src, long long R, int K, const moe::skinny::QRows& q, hipStream_t s,
                 const int32_t* perm = nullptr, int div = 1, const int32_t* status = nullptr) {
  if (R <= 0) return MOE_OK;
  if (mx8)
    hipLaunchKernelGGL(moe::skinny::k_quant_rows<true>, dim3((unsigned)R), dim3(256), 0, s, (const uint16_t*)src,
                       (int)R, K, q, perm, div, status);
  else
    hipLaunchKernelGGL(moe::skinny::k_quant_rows<false>, dim3((unsigned)R), dim3(256), 0, s, (const uint16_t*)src,
                       (int)R, K, q, perm, div, status);
  return MOE_OK;
}

moe::ActParams act_params(const moe_problem& p) {
  moe::ActParams a;
  a.kind = p.act;
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.limit = p.limit;
  return a;
}

moe::ExpertParams expert_params(const moe_problem& p) {
  return moe::ExpertParams{p.alpha_e, p.beta_e, p.limit_e, p.fc1_alpha, p.fc2_alpha};
}

// Compute units of the current device, cached per device.
int device_cus(int* n) {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *n = cache[dev];
    return MOE_OK;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return MOE_EHIP;
  if (dev >= 0 && dev < 64) cache[dev] = v;
  *n = v;
  return MOE_OK;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

// A second stream per device for the cold-segment kernels, with the two
// events that fork it from the caller's stream and join it back; created on
// first use with the default priority, kept until the process ends. The
// fork / join calls of one forward are made under the mutex, so forwards
// issued from several host threads do not interleave their event records.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

int side_stream(SideStream** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  SideStream& ss = g_side[dev];
  if (!ss.stream) {
    if (hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) != hipSuccess) return MOE_EHIP;
    if (hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
      return MOE_EHIP;
  }
  *out = &ss;
  return MOE_OK;
}

// ---------------------------------------------------------------- align
int launch_align(const int32_t* ids, const float* w, int M, int E, int BM, const Plan& pl, moe::AlignOut o,
                 void* ws, hipStream_t s) {
  const int nbits = bits_for(E);
  if (pl.fused_align) {
    const size_t lds = (size_t)(7 * E + 16) * 4;
    hipLaunchKernelGGL(moe::k_align_fused, dim3(1), dim3(256), lds, s, ids, w, M, E, nbits, BM, o);
    return launch_status();
  }
  int32_t* blkcnt = at<int32_t>(ws, pl.blkcnt);
  int32_t* blkbad = at<int32_t>(ws, pl.blkbad);
  const int nblk = ceil_div(pl.nch, 4);
  const size_t lds4 = (size_t)4 * E * 4;
  hipLaunchKernelGGL(moe::k_align_count, dim3(nblk), dim3(256), lds4, s, ids, M, E, nbits, pl.chunk, pl.nch,
                     blkcnt, blkbad);
  hipLaunchKernelGGL(moe::k_align_scan, dim3(1), dim3(1024), (size_t)(3 * E + 32) * 4, s, blkcnt,
                     (const int32_t*)blkbad, pl.nch, M, E, BM, o);
  hipLaunchKernelGGL(moe::k_align_scatter, dim3(nblk), dim3(256), lds4, s, ids, w, M, E, nbits, pl.chunk,
                     pl.nch, (const int32_t*)blkcnt, o);
  return launch_status();
}

// Tuning override for the prefill GEMM's tile-group width (column tiles per
// group); read once. MOE_EXPERTS_GROUP_COLS=<n>, n >= 1; unset = built-in choice.
int group_cols_override() {
  static const int v = [] {
    const char* e = std::getenv("MOE_EXPERTS_GROUP_COLS");
    const int n = e ? std::atoi(e) : 0;
    return n > 0 ? n : 0;
  }();
  return v;
}

// Tuning override for the MXFP4 x MXFP8 prefill GEMMs' schedule:
// MOE_EXPERTS_PERSISTENT=0 runs one workgroup per tile instead of one per
// compute unit; read once.
int persistent_override() {
  static const int v = [] {
    const char* e = std::getenv("MOE_EXPERTS_PERSISTENT");
    return e ? (std::atoi(e) != 0 ? 1 : 0) : -1;
  }();
  return v;
}

bool g_attr_done = false;
int set_attrs() {
  if (g_attr_done) return MOE_OK;
  hipError_t e = hipSuccess;
  e = hipFuncSetAttribute((const void*)moe::k_align_count, hipFuncAttributeMaxDynamicSharedMemorySize, 65536);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)moe::k_align_scatter, hipFuncAttributeMaxDynamicSharedMemorySize, 65536);
  // MXFP4 decode GEMM: scale rows staged in dynamic LDS, up to 4 * kMaxMxfp4K bytes
  const void* mx[] = {
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 4>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 8>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 16>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 4>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 8>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 16>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 4, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 8, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 16, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 4, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 8, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 16, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 4, false, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 8, false, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 16, false, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 4, false, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 8, false, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 16, false, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 4, true, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 8, true, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, true, 16, true, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 4, true, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 8, true, true>,
      (const void*)moe::skinny::k_gemm<moe::skinny::W_MXFP4, false, 16, true, true>,
  };
  for (const void* f : mx)
    if (e == hipSuccess)
      e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                              moe::skinny::scale_lds_bytes(moe::skinny::kMaxMxfp4K));
  const void* fused[] = {(const void*)moe::skinny::k_decode_fused<moe::skinny::W_MXFP4, 4, 4, false>,
                         (const void*)moe::skinny::k_decode_fused<moe::skinny::W_MXFP4, 4, 4, true>};
  for (const void* f : fused)
    if (e == hipSuccess)
      e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, moe::skinny::scale_lds_bytes(4096));
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)moe::mx::k_mx_prep, hipFuncAttributeMaxDynamicSharedMemorySize,
                            moe::mx::prep_lds_bytes(moe::skinny::kMaxMxfp4K));
  if (e != hipSuccess) return MOE_EHIP;
  g_attr_done = true;
  return MOE_OK;
}

// ---------------------------------------------------------------- GEMMs
struct GemmIO {
  const void* A;
  const int32_t* a_perm;
  int a_div;
  const void* B0;
  const void* B1;
  const uint8_t* S0;
  const uint8_t* S1;
  int N, K;
  void* C;
  const float* row_w;
  int s_cap;         // GEMM2: K ranges with room in C (1 = C is [rows, N])
  long long c_split; // elements between partial outputs
  moe::skinny::QRows Aq;  // A split for the block-scaled MFMA (MXFP4 weights)
  moe::skinny::QRows Cq;  // GEMM1 with MXFP8 activations: C quantized instead of written as bf16
};

// Weights of the tiled and cold-segment bf16 kernels: the operand-block copy
// (gate, up, down regions of E N K elements each) when the problem has one,
// else the canonical tensors.
template <bool GATED>
void tile_weights(const moe_problem& p, const GemmIO& io, const uint16_t*& b0, const uint16_t*& b1) {
  if (!p.bf16_packed) {
    b0 = (const uint16_t*)io.B0;
    b1 = (const uint16_t*)io.B1;
    return;
  }
  const size_t m = (size_t)p.E * (size_t)p.I * (size_t)p.H;
  const uint16_t* base = (const uint16_t*)p.bf16_packed;
  b0 = GATED ? base : base + 2 * m;
  b1 = GATED ? base + m : nullptr;
}

template <bool GATED, bool PK>
void launch_big_kernel(int act, dim3 g, dim3 b, hipStream_t s, const moe::big::Params& q) {
  if constexpr (!GATED) {
    hipLaunchKernelGGL((moe::big::k_gemm<false, 0, PK>), g, b, 0, s, q);
  } else {  // one instantiation per activation kind
    if (act == MOE_ACT_SWIGLU_OAI) hipLaunchKernelGGL((moe::big::k_gemm<true, 1, PK>), g, b, 0, s, q);
    else if (act == MOE_ACT_SITU) hipLaunchKernelGGL((moe::big::k_gemm<true, 2, PK>), g, b, 0, s, q);
    else hipLaunchKernelGGL((moe::big::k_gemm<true, 0, PK>), g, b, 0, s, q);
  }
}

template <bool GATED, bool PK>
void launch_cold_kernel(int act, dim3 g, dim3 b, hipStream_t s, const moe::cold::Params& q) {
  if constexpr (!GATED) {
    hipLaunchKernelGGL((moe::cold::k_cold<false, 0, PK>), g, b, 0, s, q);
  } else {
    if (act == MOE_ACT_SWIGLU_OAI) hipLaunchKernelGGL((moe::cold::k_cold<true, 1, PK>), g, b, 0, s, q);
    else if (act == MOE_ACT_SITU) hipLaunchKernelGGL((moe::cold::k_cold<true, 2, PK>), g, b, 0, s, q);
    else hipLaunchKernelGGL((moe::cold::k_cold<true, 0, PK>), g, b, 0, s, q);
  }
}

template <bool GATED>
moe::skinny::Params skinny_params(const moe_problem& p, const Plan& pl, const GemmIO& io, void* ws) {
  moe::skinny::Params q;
  q.A = (const uint16_t*)io.A;
  q.Aq = io.Aq;
  q.a_perm = io.a_perm;
  q.a_div = io.a_div;
  q.B0 = io.B0;
  q.B1 = io.B1;
  q.S0 = io.S0;
  q.S1 = io.S1;
  q.N = io.N;
  q.K = io.K;
  q.tile_seg = at<int32_t>(ws, pl.tile_seg);
  q.tile_row0 = at<int32_t>(ws, pl.tile_row0);
  q.seg_end = at<int32_t>(ws, pl.cu);
  q.status = at<int32_t>(ws, pl.status);
  q.mt_cap = pl.mt_cap;
  q.n_tiles = ceil_div(io.N, moe::skinny::block_cols(GATED));
  q.C = (uint16_t*)io.C;
  q.Cq = io.Cq;
  q.row_w = io.row_w;
  q.act = act_params(p);
  q.ep = expert_params(p);
  // packed MXFP4 codes (read by the PK kernels of the separate launches)
  q.Bp = nullptr;
  q.bp_expert = 0;
  if (p.mx_packed && p.wfmt == MOE_W_MXFP4) {
    q.Bp = (const uint8_t*)p.mx_packed + (GATED ? 0 : (size_t)p.E * mx_packed_expert1(p));
    q.bp_expert = (uint32_t)(GATED ? mx_packed_expert1(p) : mx_packed_expert2(p));
  }
  return q;
}

static_assert(moe::skinny::PK_BLOCK == moe::mx::PK_STAGE && moe::skinny::PK_KSTAGE == moe::mx::BK &&
                  moe::skinny::PK_COLS1 == moe::mx::BN / 2 && moe::skinny::PK_COLS2 == moe::mx::BN,
              "the decode kernels read the MXFP4 prefill GEMMs' packed layout");

// MXFP4 decode GEMM: SPT scale pieces per thread, A8 MXFP8 activations, PK packed codes
template <bool GATED, bool A8, bool PK>
void launch_skinny_mx(int spt, dim3 grid, dim3 block, size_t lds, hipStream_t s, const moe::skinny::Params& q) {
  using moe::skinny::k_gemm;
  using moe::skinny::W_MXFP4;
  switch (spt) {
    case 4: hipLaunchKernelGGL((k_gemm<W_MXFP4, GATED, 4, A8, PK>), grid, block, lds, s, q); break;
    case 8: hipLaunchKernelGGL((k_gemm<W_MXFP4, GATED, 8, A8, PK>), grid, block, lds, s, q); break;
    default: hipLaunchKernelGGL((k_gemm<W_MXFP4, GATED, 16, A8, PK>), grid, block, lds, s, q); break;
  }
}

template <bool GATED>
int launch_gemm(const moe_problem& p, const Plan& pl, const GemmIO& io, void* ws, hipStream_t s) {
  const int32_t* tile_seg = at<int32_t>(ws, pl.tile_seg);
  const int32_t* tile_row0 = at<int32_t>(ws, pl.tile_row0);
  const int32_t* cu = at<int32_t>(ws, pl.cu);
  const int32_t* status = at<int32_t>(ws, pl.status);
  if (pl.skinny) {
    const moe::skinny::Params q = skinny_params<GATED>(p, pl, io, ws);
    const dim3 grid((unsigned)pl.mt_cap * q.n_tiles);
    const dim3 block(moe::skinny::NT);
    using moe::skinny::k_gemm;
    using moe::skinny::W_BF16;
    using moe::skinny::W_MXFP4;
    if (p.wfmt == MOE_W_MXFP4) {
      const size_t lds = moe::skinny::scale_lds_bytes(io.K);
      const int spt = moe::skinny::scale_pieces_per_thread(io.K);
      const bool a8 = p.a_fmt == MOE_A_MXFP8;
      if (a8 && q.Bp) launch_skinny_mx<GATED, true, true>(spt, grid, block, lds, s, q);
      else if (a8) launch_skinny_mx<GATED, true, false>(spt, grid, block, lds, s, q);
      else if (q.Bp) launch_skinny_mx<GATED, false, true>(spt, grid, block, lds, s, q);
      else launch_skinny_mx<GATED, false, false>(spt, grid, block, lds, s, q);
    } else {
      hipLaunchKernelGGL((k_gemm<W_BF16, GATED, 0>), grid, block, 0, s, q);
    }
  } else {
    moe::big::Params q;
    q.A = (const uint16_t*)io.A;
    q.a_perm = io.a_perm;
    q.a_div = io.a_div;
    tile_weights<GATED>(p, io, q.B0, q.B1);
    q.N = io.N;
    q.K = io.K;
    q.tile_seg = tile_seg;
    q.tile_row0 = tile_row0;
    q.seg_end = cu;
    q.status = status;
    q.mt_cap = pl.mt_cap;
    q.n_tiles = ceil_div(io.N, GATED ? moe::big::BN / 2 : moe::big::BN);
    q.C = (uint16_t*)io.C;
    q.row_w = io.row_w;
    q.act = act_params(p);
    q.ep = expert_params(p);
    q.gn = std::min(q.n_tiles, group_cols_override() ? group_cols_override() : 2);
    q.s_cap = GATED ? 1 : io.s_cap;
    q.c_split = io.c_split;
    int rc = device_cus(&q.ncu);
    if (rc) return rc;
    long long nblk = (long long)pl.mt_cap * q.n_tiles * q.s_cap;
    nblk = (nblk + 7) / 8 * 8;
    if (nblk > 0x7fffffffLL) return MOE_ENOTSUP;
    const dim3 g((unsigned)nblk), b(moe::big::NT);
    if (p.bf16_packed) launch_big_kernel<GATED, true>(p.act, g, b, s, q);
    else launch_big_kernel<GATED, false>(p.act, g, b, s, q);
  }
  return launch_status();
}

// The cold segments' GEMM (gemm_cold.hpp): one workgroup per compute unit.
template <bool GATED>
int launch_cold(const moe_problem& p, const Plan& pl, const GemmIO& io, void* ws, hipStream_t s) {
  moe::cold::Params q;
  q.A = (const uint16_t*)io.A;
  q.a_perm = io.a_perm;
  q.a_div = io.a_div;
  tile_weights<GATED>(p, io, q.B0, q.B1);
  q.N = io.N;
  q.K = io.K;
  q.cold_seg = at<int32_t>(ws, pl.cold_seg);
  q.seg_end = at<int32_t>(ws, pl.cu);
  q.status = at<int32_t>(ws, pl.status);
  q.n_tiles = ceil_div(io.N, moe::cold::block_cols(GATED));
  q.C = (uint16_t*)io.C;
  q.row_w = io.row_w;
  q.act = act_params(p);
  q.ep = expert_params(p);
  q.c_split = io.c_split;
  q.s_cap = GATED ? 1 : io.s_cap;
  q.tiled_cols = ceil_div(io.N, moe::big::BN);
  q.tiled_kt = io.K / moe::big::BK;
  const int rc = device_cus(&q.ncu);
  if (rc) return rc;
  const dim3 g((unsigned)q.ncu), b(moe::cold::NT);
  if (p.bf16_packed) launch_cold_kernel<GATED, true>(p.act, g, b, s, q);
  else launch_cold_kernel<GATED, false>(p.act, g, b, s, q);
  return launch_status();
}

// GEMM1 then GEMM2 of the tiled segments on s and, with a cold-segment list,
// the cold segments' GEMM1 then GEMM2 on the side stream (forked from s after
// everything before, joined back before what follows), or on s itself when
// side is false. The tiled GEMM1 is issued first, so its workgroups take the
// compute units; the cold kernels' workgroups fit beside them.
int launch_gemms(const moe_problem& p, const Plan& pl, const GemmIO& g1, const GemmIO& g2, void* ws, hipStream_t s,
                 bool side, const std::function<void(int)>& mark) {
  int rc;
  if (!pl.cold) {
    if ((rc = launch_gemm<true>(p, pl, g1, ws, s))) return rc;
    mark(2);
    if ((rc = launch_gemm<false>(p, pl, g2, ws, s))) return rc;
    return MOE_OK;
  }
  if (!side) {
    if ((rc = launch_gemm<true>(p, pl, g1, ws, s)) || (rc = launch_cold<true>(p, pl, g1, ws, s))) return rc;
    mark(2);
    if ((rc = launch_gemm<false>(p, pl, g2, ws, s)) || (rc = launch_cold<false>(p, pl, g2, ws, s))) return rc;
    return MOE_OK;
  }
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* ss = nullptr;
  if ((rc = side_stream(&ss))) return rc;
  if (hipEventRecord(ss->fork, s) != hipSuccess || hipStreamWaitEvent(ss->stream, ss->fork, 0) != hipSuccess)
    return MOE_EHIP;
  if ((rc = launch_gemm<true>(p, pl, g1, ws, s)) || (rc = launch_cold<true>(p, pl, g1, ws, ss->stream))) return rc;
  mark(2);
  if ((rc = launch_gemm<false>(p, pl, g2, ws, s)) || (rc = launch_cold<false>(p, pl, g2, ws, ss->stream))) return rc;
  if (hipEventRecord(ss->join, ss->stream) != hipSuccess || hipStreamWaitEvent(s, ss->join, 0) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

// Workgroups of kernel f (NT threads, dyn bytes of dynamic LDS) that fit on
// the device at once, cached per device, kernel and LDS size.
int resident_blocks(const void* f, size_t dyn, int* n) {
  struct Entry {
    int dev;
    const void* f;
    size_t dyn;
    int n;
  };
  static Entry cache[32];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].dev == dev && cache[i].f == f && cache[i].dyn == dyn) {
      *n = cache[i].n;
      return MOE_OK;
    }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, moe::skinny::NT, dyn) != hipSuccess || per_cu <= 0)
    return MOE_EHIP;
  int rc = device_cus(&cus);
  if (rc) return rc;
  *n = per_cu * cus;
  if (used < 32) cache[used++] = Entry{dev, f, dyn, *n};
  return MOE_OK;
}

// The single-launch decode step after the align prologue: GEMM1 tiles, GEMM2
// tiles and the combine from one work queue (gemm_skinny.hpp,
// k_decode_fused). g1 / g2 as for the separate launches; GEMM1 writes the
// down projection's input in the form GEMM2 reads (bf16 rows, or split for
// the block-scaled MFMA), GEMM2 writes the slot rows y.
int launch_fused_decode(const moe_problem& p, const Plan& pl, const GemmIO& g1, const GemmIO& g2,
                        const int32_t* inv_perm, void* out, void* ws, hipStream_t s) {
  using namespace moe::skinny;
  const Params p1 = skinny_params<true>(p, pl, g1, ws);
  const Params p2 = skinny_params<false>(p, pl, g2, ws);
  const moe::skinny::FusedCombine fc{(const uint16_t*)g2.C, inv_perm, p.T, p.k, p.H, (uint16_t*)out};
  int32_t* sync = at<int32_t>(ws, pl.sync);
  const FusedSync fs{sync, sync + 4, sync + 1, at<int32_t>(ws, pl.status), p1.n_tiles, 1 << 20, fused_batch()};
  const long long items = (long long)pl.mt_cap * (p1.n_tiles + p2.n_tiles) + p.T;
  const bool mx = p.wfmt == MOE_W_MXFP4, mx8 = p.a_fmt == MOE_A_MXFP8;
  const size_t dyn = mx ? (size_t)scale_lds_bytes(std::max(p.H, p.I)) : 0;
  const void* f = mx ? (mx8 ? (const void*)k_decode_fused<W_MXFP4, 4, 4, true>
                            : (const void*)k_decode_fused<W_MXFP4, 4, 4, false>)
                     : (const void*)k_decode_fused<W_BF16, 0, 0, false>;
  int cap = 0;
  int rc = resident_blocks(f, dyn, &cap);
  if (rc) return rc;
  const dim3 grid((unsigned)std::max(1LL, std::min<long long>(items, cap))), block(NT);
  if (mx && mx8)
    hipLaunchKernelGGL((k_decode_fused<W_MXFP4, 4, 4, true>), grid, block, dyn, s, p1, p2, fc, fs);
  else if (mx)
    hipLaunchKernelGGL((k_decode_fused<W_MXFP4, 4, 4, false>), grid, block, dyn, s, p1, p2, fc, fs);
  else
    hipLaunchKernelGGL((k_decode_fused<W_BF16, 0, 0, false>), grid, block, dyn, s, p1, p2, fc, fs);
  return launch_status();
}

// Token-major forward on the LDS-tiled MXFP4 x MXFP8 kernels, after the
// align: x rows quantized (k_quant_rows), scale blocks prepared (k_mx_prep),
// GEMM1 (its epilogue quantizes GEMM2's input), GEMM2, combine.
template <class Mark>
int forward_mx(const moe_problem& p, const Plan& pl, const void* x, const moe::AlignOut& o, const void* wg,
               const void* wu, const void* wd, const uint8_t* sg, const uint8_t* su, const uint8_t* sd, void* out,
               void* ws, hipStream_t s, Mark&& mark) {
  const int M = (int)pl.M;
  const long long R = p.weight_on_input ? pl.M : (long long)p.T;
  const moe::skinny::QRows xq = quant_rows_at(ws, pl.xq, R, p.H);
  if (p.weight_on_input) {  // rows x * w in sorted order, quantized in that order
    hipLaunchKernelGGL(moe::k_scale_rows, dim3((unsigned)pl.M), dim3(256), 0, s, (const uint16_t*)x,
                       (const int32_t*)o.perm, p.k, (const float*)o.w_sorted, (const int32_t*)o.status, M, p.H,
                       at<uint16_t>(ws, pl.xs));
    launch_quant(true, at<void>(ws, pl.xs), R, p.H, xq, s);
  } else {
    launch_quant(true, x, R, p.H, xq, s);
  }
  moe::mx::PrepParams pp;
  pp.Sg = sg;
  pp.Su = su;
  pp.Sd = sd;
  pp.WS1 = at<uint8_t>(ws, pl.ws1);
  pp.WS2 = at<uint8_t>(ws, pl.ws2);
  pp.E = p.E;
  pp.H = p.H;
  pp.I = p.I;
  pp.NT1 = pl.NT1;
  pp.KT1 = pl.KT1;
  pp.NT2 = pl.NT2;
  pp.KT2 = pl.KT2;
  pp.counts = o.counts;
  pp.xs = xq.sc;
  pp.xs_stride = xq.sc_stride;
  pp.perm = p.weight_on_input ? nullptr : o.perm;
  pp.div = p.k;
  pp.tile_seg = o.tile_seg;
  pp.tile_row0 = o.tile_row0;
  pp.seg_end = o.cu;
  pp.status = o.status;
  pp.mt_cap = pl.mt_cap;
  pp.SA1 = at<uint8_t>(ws, pl.sa1);
  if (p.mx_packed) pp.E = 0;  // the packed blocks carry the weights' scale blocks
  const long long nprep = (long long)pp.E * (pl.NT1 + pl.NT2) + pl.mt_cap;
  if (nprep > 0x7fffffffLL) return MOE_ENOTSUP;
  hipLaunchKernelGGL(moe::mx::k_mx_prep, dim3((unsigned)nprep), dim3(256),
                     (size_t)moe::mx::prep_lds_bytes(std::max(p.H, p.I)), s, pp);
  mark(1);

  int ncu = 0;
  int rc = device_cus(&ncu);
  if (rc) return rc;
  moe::mx::Params g{};
  g.A = xq.hi;
  g.a_bytes = (uint32_t)(R * p.H);
  g.a_perm = p.weight_on_input ? nullptr : o.perm;
  g.a_div = p.k;
  g.A_sc = pp.SA1;
  g.B0 = (const uint8_t*)wg;
  g.B1 = (const uint8_t*)wu;
  g.B_sc = pp.WS1;
  g.Bp = (const uint8_t*)p.mx_packed;
  g.bp_expert = (uint32_t)mx_packed_expert1(p);
  g.N = p.I;
  g.K = p.H;
  g.KT = pl.KT1;
  g.tile_seg = o.tile_seg;
  g.tile_row0 = o.tile_row0;
  g.seg_end = o.cu;
  g.status = o.status;
  g.mt_cap = pl.mt_cap;
  g.n_tiles = pl.NT1;
  g.gn = std::min(pl.NT1, group_cols_override() ? group_cols_override() : 2);
  g.s_cap = 1;
  g.ncu = ncu;
  g.Cq = at<uint8_t>(ws, pl.aq);
  g.Cq_sc = at<uint8_t>(ws, pl.sa2);
  g.row_w = p.weight_on_input ? nullptr : o.w_sorted;
  g.act = act_params(p);
  g.ep = expert_params(p);
  // Persistent (the default): one workgroup per compute unit (a tile's
  // 150 KB of LDS leaves room for no second one), each running its XCD's
  // tiles in turn, the next tile's first loads under the current epilogue.
  const bool mx_persist = persistent_override() != 0;
  const long long pgrid = std::max(8, ncu / 8 * 8);
  long long nblk = ((long long)pl.mt_cap * pl.NT1 + 7) / 8 * 8;
  if (mx_persist) nblk = std::min(nblk, pgrid);
  if (nblk > 0x7fffffffLL) return MOE_ENOTSUP;
  if (p.act == MOE_ACT_SWIGLU_OAI)
    hipLaunchKernelGGL((moe::mx::k_gemm<true, 1>), dim3((unsigned)nblk), dim3(moe::mx::NT), 0, s, g);
  else if (p.act == MOE_ACT_SITU)
    hipLaunchKernelGGL((moe::mx::k_gemm<true, 2>), dim3((unsigned)nblk), dim3(moe::mx::NT), 0, s, g);
  else
    hipLaunchKernelGGL((moe::mx::k_gemm<true, 0>), dim3((unsigned)nblk), dim3(moe::mx::NT), 0, s, g);
  if ((rc = launch_status())) return rc;
  mark(2);

  moe::mx::Params g2 = g;
  g2.A = at<uint8_t>(ws, pl.aq);
  g2.a_bytes = (uint32_t)((long long)M * p.I);
  g2.a_perm = nullptr;
  g2.A_sc = g.Cq_sc;
  g2.B0 = (const uint8_t*)wd;
  g2.B1 = nullptr;
  g2.B_sc = at<uint8_t>(ws, pl.ws2);
  g2.Bp = p.mx_packed ? (const uint8_t*)p.mx_packed + (size_t)p.E * mx_packed_expert1(p) : nullptr;
  g2.bp_expert = (uint32_t)mx_packed_expert2(p);
  g2.N = p.H;
  g2.K = p.I;
  g2.KT = pl.KT2;
  g2.n_tiles = pl.NT2;
  g2.gn = std::min(pl.NT2, group_cols_override() ? group_cols_override() : 2);
  g2.s_cap = pl.s_cap;
  g2.c_split = pl.M * p.H;
  g2.C = at<uint16_t>(ws, pl.y);
  g2.Cq = nullptr;
  g2.Cq_sc = nullptr;
  g2.row_w = nullptr;
  nblk = ((long long)pl.mt_cap * pl.NT2 * pl.s_cap + 7) / 8 * 8;
  if (mx_persist) nblk = std::min(nblk, pgrid);
  if (nblk > 0x7fffffffLL) return MOE_ENOTSUP;
  hipLaunchKernelGGL((moe::mx::k_gemm<false, 0>), dim3((unsigned)nblk), dim3(moe::mx::NT), 0, s, g2);
  if ((rc = launch_status())) return rc;
  mark(3);
  moe::SplitSum ss{o.status, pl.NT2, pl.KT2, ncu, pl.s_cap, pl.M * p.H};
  hipLaunchKernelGGL(moe::k_combine, dim3(p.T, ceil_div(p.H, 256 * 8)), dim3(256), 0, s, at<const uint16_t>(ws, pl.y),
                     (const int32_t*)o.inv_perm, p.T, p.k, p.H, ss, (uint16_t*)out);
  mark(4);
  return launch_status();
}

int check_common_ptrs(const moe_problem* p, const void* x, const void* wg, const void* wu, const void* wd,
                      const uint8_t* sg, const uint8_t* su, const uint8_t* sd, const void* out, const void* ws) {
  if (!x || !wg || !wu || !wd || !out || !ws) return MOE_EINVAL;
  if (p->wfmt == MOE_W_MXFP4 && (!sg || !su || !sd)) return MOE_EINVAL;
  if (p->wfmt == MOE_W_MXFP4 && (!aligned16(sg) || !aligned16(su) || !aligned16(sd))) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(wg) || !aligned16(wu) || !aligned16(wd) || !aligned16(out)) return MOE_EINVAL;
  if (((uintptr_t)ws % kAlign) != 0) return MOE_EINVAL;
  return MOE_OK;
}

int forward_impl(const moe_problem* p, const void* x, const int32_t* ids, const float* tw, const void* wg,
                 const void* wu, const void* wd, const uint8_t* sg, const uint8_t* su, const uint8_t* sd,
                 void* out, void* ws, size_t ws_bytes, hipStream_t s, void* const* ev, int n_ev, bool side) {
  int rc = check_problem(p, false);
  if (rc) return rc;
  if (!ids || !tw) return MOE_EINVAL;
  rc = check_common_ptrs(p, x, wg, wu, wd, sg, su, sd, out, ws);
  if (rc) return rc;
  if (n_ev != 0 && (n_ev != 5 || !ev)) return MOE_EINVAL;
  if (p->T == 0) return MOE_OK;
  const Plan pl = make_plan(*p, false, ws_bytes);
  if (ws_bytes < pl.total) return MOE_ENOSPC;
  if ((rc = set_attrs())) return rc;
  auto mark = [&](int i) {
    if (n_ev) (void)hipEventRecord((hipEvent_t)ev[i], s);
  };

  moe::AlignOut o{};
  if (pl.cold) {
    o.cold_seg = at<int32_t>(ws, pl.cold_seg);
    o.cold_max = moe::cold::MAX_ROWS;
  }
  o.counts = at<int32_t>(ws, pl.counts);
  o.cu = at<int32_t>(ws, pl.cu);
  o.offsets = at<int32_t>(ws, pl.offsets);
  o.perm = at<int32_t>(ws, pl.perm);
  o.inv_perm = at<int32_t>(ws, pl.inv_perm);
  o.w_sorted = at<float>(ws, pl.w_sorted);
  o.tile_seg = at<int32_t>(ws, pl.tile_seg);
  o.tile_row0 = at<int32_t>(ws, pl.tile_row0);
  o.status = at<int32_t>(ws, pl.status);
  if (pl.fused) {  // the align prologue zeroes the single launch's counters
    o.sync = at<int32_t>(ws, pl.sync);
    o.n_sync = pl.n_sync;
  }
  const int M = (int)pl.M;

  const bool mx = p->wfmt == MOE_W_MXFP4;
  const bool mx8 = p->a_fmt == MOE_A_MXFP8;
  // MXFP4 with the one-workgroup align: x split in token order in the same
  // launch (GEMM1 reads it through the permutation)
  const bool mx_prologue = mx && pl.fused_align && !p->weight_on_input && !pl.mxbig;
  mark(0);
  if (mx_prologue) {
    const size_t lds = (size_t)(7 * p->E + 16) * 4;
    if (mx8)
      hipLaunchKernelGGL(moe::k_align_fused_quant<true>, dim3((unsigned)p->T + 1), dim3(256), lds, s, ids, tw, M,
                         p->E, bits_for(p->E), pl.BM, o, (const uint16_t*)x, p->T, p->H,
                         quant_rows_at(ws, pl.xq, p->T, p->H));
    else
      hipLaunchKernelGGL(moe::k_align_fused_quant<false>, dim3((unsigned)p->T + 1), dim3(256), lds, s, ids, tw, M,
                         p->E, bits_for(p->E), pl.BM, o, (const uint16_t*)x, p->T, p->H,
                         quant_rows_at(ws, pl.xq, p->T, p->H));
    if ((rc = launch_status())) return rc;
  } else if ((rc = launch_align(ids, tw, M, p->E, pl.BM, pl, o, ws, s))) {
    return rc;
  }

  if (pl.mxbig) return forward_mx(*p, pl, x, o, wg, wu, wd, sg, su, sd, out, ws, s, mark);
  GemmIO g1{x, o.perm, p->k, wg, wu, sg, su, p->I, p->H, at<void>(ws, pl.act), o.w_sorted, 1, 0, {}, {}};
  // MXFP8 activations: GEMM1's epilogue quantizes the activation rows for GEMM2 itself
  if (mx8) g1.Cq = quant_rows_at(ws, pl.aq, pl.M, p->I);
  if (p->weight_on_input) {  // rows x * w in sorted order; no weight in GEMM1's epilogue
    g1.A = at<void>(ws, pl.xs);
    g1.a_perm = nullptr;
    g1.row_w = nullptr;
  }
  if (mx_prologue) {  // x split in token order by the prologue
    g1.Aq = quant_rows_at(ws, pl.xq, p->T, p->H);
  } else if (mx) {  // x split in sorted row order: GEMM1 reads its rows without the permutation
    g1.Aq = quant_rows_at(ws, pl.xq, pl.M, p->H);
    g1.a_perm = nullptr;
  }
  const long long y_split = pl.M * p->H;
  GemmIO g2{at<void>(ws, pl.act), nullptr, 1, wd, nullptr, sd, nullptr, p->H, p->I, at<void>(ws, pl.y), nullptr,
            pl.s_cap, y_split, {}, {}};
  if (mx) g2.Aq = quant_rows_at(ws, pl.aq, pl.M, p->I);
  mark(1);
  if (pl.fused) {  // GEMM1, GEMM2 and the combine in one launch
    if (mx) g1.Cq = g2.Aq;  // GEMM1 writes GEMM2's split (or MXFP8) input rows directly
    rc = launch_fused_decode(*p, pl, g1, g2, o.inv_perm, out, ws, s);
    mark(2);
    mark(3);
    mark(4);
    return rc;
  }
  if (p->weight_on_input)
    hipLaunchKernelGGL(moe::k_scale_rows, dim3((unsigned)pl.M), dim3(256), 0, s, (const uint16_t*)x,
                       (const int32_t*)o.perm, p->k, (const float*)o.w_sorted, (const int32_t*)o.status, M, p->H,
                       at<uint16_t>(ws, pl.xs));
  if (mx && !mx_prologue) {
    if (p->weight_on_input) launch_quant(mx8, g1.A, pl.M, p->H, g1.Aq, s);
    else launch_quant(mx8, x, pl.M, p->H, g1.Aq, s, o.perm, p->k, o.status);
  }
  if (mx) {
    if ((rc = launch_gemm<true>(*p, pl, g1, ws, s))) return rc;
    mark(2);
    if (!mx8) launch_quant(false, g2.A, pl.M, p->I, g2.Aq, s);
    if ((rc = launch_gemm<false>(*p, pl, g2, ws, s))) return rc;
  } else if ((rc = launch_gemms(*p, pl, g1, g2, ws, s, side, mark))) {
    return rc;
  }

  mark(3);
  moe::SplitSum ss{o.status, ceil_div(p->H, moe::big::BN), p->I / moe::big::BK, 1, pl.s_cap, y_split};
  if (pl.s_cap > 1 && (rc = device_cus(&ss.ncu))) return rc;
  hipLaunchKernelGGL(moe::k_combine, dim3(p->T, ceil_div(p->H, 256 * 8)), dim3(256), 0, s, at<const uint16_t>(ws, pl.y),
                     (const int32_t*)o.inv_perm, p->T, p->k, p->H, ss, (uint16_t*)out);
  mark(4);
  return launch_status();
}

}  // namespace

extern "C" {

size_t moe_mx_packed_bytes(const moe_problem* p) {
  if (check_problem(p, true)) return 0;
  if (p->wfmt != MOE_W_MXFP4) return 0;
  return (size_t)p->E * (mx_packed_expert1(*p) + mx_packed_expert2(*p));
}

size_t moe_bf16_packed_bytes(const moe_problem* p) {
  if (check_problem(p, true)) return 0;
  if (p->wfmt != MOE_W_BF16) return 0;
  return (size_t)3 * p->E * (size_t)p->I * (size_t)p->H * 2u;
}

int moe_bf16_pack_weights(const moe_problem* p, const void* w_gate, const void* w_up, const void* w_down,
                          void* packed, size_t packed_bytes, moe_stream_t stream) {
  if (check_problem(p, true)) return MOE_EINVAL;
  if (p->wfmt != MOE_W_BF16) return MOE_EINVAL;
  const void* ptrs[] = {w_gate, w_up, w_down, packed};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return MOE_EINVAL;
  if (packed_bytes < moe_bf16_packed_bytes(p)) return MOE_ENOSPC;
  const size_t m = (size_t)p->E * (size_t)p->I * (size_t)p->H;  // elements of each matrix set
  const long long pieces = (long long)(m / 8);                   // H and I are multiples of 64
  if (pieces == 0) return MOE_OK;
  const unsigned grid = (unsigned)std::min<long long>((pieces + 255) / 256, 65536);
  hipStream_t s = (hipStream_t)stream;
  uint16_t* out = (uint16_t*)packed;
  hipLaunchKernelGGL(moe::big::k_bf16_pack, dim3(grid), dim3(256), 0, s, (const uint16_t*)w_gate, out, p->I, p->H,
                     pieces);
  hipLaunchKernelGGL(moe::big::k_bf16_pack, dim3(grid), dim3(256), 0, s, (const uint16_t*)w_up, out + m, p->I, p->H,
                     pieces);
  hipLaunchKernelGGL(moe::big::k_bf16_pack, dim3(grid), dim3(256), 0, s, (const uint16_t*)w_down, out + 2 * m, p->H,
                     p->I, pieces);
  return launch_status();
}

int moe_mx_pack_weights(const moe_problem* p, const void* w_gate, const void* w_up, const void* w_down,
                        const uint8_t* s_gate, const uint8_t* s_up, const uint8_t* s_down, void* packed,
                        size_t packed_bytes, moe_stream_t stream) {
  if (check_problem(p, true)) return MOE_EINVAL;
  if (p->wfmt != MOE_W_MXFP4) return MOE_EINVAL;
  const void* ptrs[] = {w_gate, w_up, w_down, s_gate, s_up, s_down, packed};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return MOE_EINVAL;
  if (packed_bytes < moe_mx_packed_bytes(p)) return MOE_ENOSPC;
  moe::mx::PackParams q;
  q.Wg = (const uint8_t*)w_gate;
  q.Wu = (const uint8_t*)w_up;
  q.Wd = (const uint8_t*)w_down;
  q.Sg = s_gate;
  q.Su = s_up;
  q.Sd = s_down;
  q.out = (uint8_t*)packed;
  q.E = p->E;
  q.H = p->H;
  q.I = p->I;
  q.NT1 = ceil_div(p->I, moe::mx::BN / 2);
  q.KT1 = ceil_div(p->H, moe::mx::BK);
  q.NT2 = ceil_div(p->H, moe::mx::BN);
  q.KT2 = ceil_div(p->I, moe::mx::BK);
  const long long nblk = (long long)p->E * ((long long)q.NT1 * q.KT1 + (long long)q.NT2 * q.KT2);
  if (nblk > 0x7fffffffLL) return MOE_ENOTSUP;
  if (nblk == 0) return MOE_OK;
  hipLaunchKernelGGL(moe::mx::k_mx_pack, dim3((unsigned)nblk), dim3(256), 0, (hipStream_t)stream, q);
  return launch_status();
}

size_t moe_experts_workspace_bytes(const moe_problem* p) {
  if (check_problem(p, false)) return 0;
  return make_plan(*p, false).total;
}

int moe_experts_workspace_layout(const moe_problem* p, moe_ws_layout* l) {
  if (!l || check_problem(p, false)) return MOE_EINVAL;
  const Plan pl = make_plan(*p, false);
  l->status = pl.status;
  l->counts = pl.counts;
  l->cu_seqlens = pl.cu;
  l->perm = pl.perm;
  l->inv_perm = pl.inv_perm;
  l->w_sorted = pl.w_sorted;
  l->act = pl.act;
  l->y = pl.y;
  l->total = pl.total;
  l->xq = pl.xq;
  l->xq_rows = pl.xq ? (size_t)((pl.fused_align || pl.mxbig) && !p->weight_on_input ? p->T : pl.M) : 0;
  l->aq = pl.aq;
  l->single_launch = pl.fused ? 1 : 0;
  l->mx_tiled = pl.mxbig ? 1 : 0;
  l->aq_sc = pl.mxbig ? pl.sa2 : 0;
  return MOE_OK;
}

int moe_experts_forward(const moe_problem* p, const void* x, const int32_t* topk_ids, const float* topk_weights,
                        const void* w_gate, const void* w_up, const void* w_down, const uint8_t* s_gate,
                        const uint8_t* s_up, const uint8_t* s_down, void* out, void* workspace,
                        size_t workspace_bytes, moe_stream_t stream) {
  return forward_impl(p, x, topk_ids, topk_weights, w_gate, w_up, w_down, s_gate, s_up, s_down, out, workspace,
                      workspace_bytes, (hipStream_t)stream, nullptr, 0, true);
}

int moe_experts_forward_timed(const moe_problem* p, const void* x, const int32_t* topk_ids,
                              const float* topk_weights, const void* w_gate, const void* w_up, const void* w_down,
                              const uint8_t* s_gate, const uint8_t* s_up, const uint8_t* s_down, void* out,
                              void* workspace, size_t workspace_bytes, moe_stream_t stream,
                              void* const* stage_events, int n_events) {
  return forward_impl(p, x, topk_ids, topk_weights, w_gate, w_up, w_down, s_gate, s_up, s_down, out, workspace,
                      workspace_bytes, (hipStream_t)stream, stage_events, n_events, true);
}

int moe_experts_forward_noalloc(const moe_problem* p, const void* x, const int32_t* topk_ids,
                                const float* topk_weights, const void* w_gate, const void* w_up, const void* w_down,
                                const uint8_t* s_gate, const uint8_t* s_up, const uint8_t* s_down, void* out,
                                moe_stream_t stream) {
  const int rc = check_problem(p, false);
  if (rc) return rc;
  if (p->T > 0 && make_plan(*p, false, kScratchBytes).total > kScratchBytes) return MOE_ENOSPC;
  void* ws = nullptr;
  const int r = scratch_on_device(&ws);
  if (r) return r;
  // no second stream here (creating one allocates); the cold kernels follow
  // the tiled ones on the caller's stream
  return forward_impl(p, x, topk_ids, topk_weights, w_gate, w_up, w_down, s_gate, s_up, s_down, out, ws,
                      kScratchBytes, (hipStream_t)stream, nullptr, 0, false);
}

size_t moe_align_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  moe_problem p{};
  p.T = T;
  p.H = 64;
  p.I = 64;
  p.E = E;
  p.k = k;
  if (check_problem(&p, false)) return 0;
  Plan pl = make_plan(p, false);
  // align needs the tables and chunk counters, not perm / act / y
  return pl.perm;
}

int moe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts, int32_t* cu_seqlens,
              int32_t* perm, int32_t* inv_perm, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  moe_problem p{};
  p.T = T;
  p.H = 64;
  p.I = 64;
  p.E = E;
  p.k = k;
  int rc = check_problem(&p, false);
  if (rc) return rc;
  if (!topk_ids || !counts || !cu_seqlens || !perm || !inv_perm || !workspace) return MOE_EINVAL;
  if (((uintptr_t)workspace % kAlign) != 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  const Plan pl = make_plan(p, false);
  if (workspace_bytes < pl.perm) return MOE_ENOSPC;
  if ((rc = set_attrs())) return rc;
  moe::AlignOut o{};
  o.counts = counts;
  o.cu = cu_seqlens;
  o.offsets = at<int32_t>(workspace, pl.offsets);
  o.perm = perm;
  o.inv_perm = inv_perm;
  o.w_sorted = nullptr;
  o.tile_seg = at<int32_t>(workspace, pl.tile_seg);
  o.tile_row0 = at<int32_t>(workspace, pl.tile_row0);
  o.status = at<int32_t>(workspace, pl.status);
  return launch_align(topk_ids, nullptr, (int)pl.M, E, pl.BM, pl, o, workspace, (hipStream_t)stream);
}

size_t moe_experts_grouped_workspace_bytes(const moe_problem* p) {
  if (check_problem(p, true)) return 0;
  return make_plan(*p, true).total;
}

}  // extern "C"

namespace {

int grouped_impl(const moe_problem* p, const void* x_nvs, const int32_t* cu_seqlens, const float* route_w,
                 const void* w_gate, const void* w_up, const void* w_down, const uint8_t* s_gate,
                 const uint8_t* s_up, const uint8_t* s_down, void* out_nvs, void* workspace,
                 size_t workspace_bytes, hipStream_t s, void* const* ev, int n_ev) {
  int rc = check_problem(p, true);
  if (rc) return rc;
  if (!cu_seqlens || !route_w) return MOE_EINVAL;
  rc = check_common_ptrs(p, x_nvs, w_gate, w_up, w_down, s_gate, s_up, s_down, out_nvs, workspace);
  if (rc) return rc;
  if (n_ev != 0 && (n_ev != 5 || !ev)) return MOE_EINVAL;
  if (p->T == 0) return MOE_OK;
  const Plan pl = make_plan(*p, true);
  if (workspace_bytes < pl.total) return MOE_ENOSPC;
  if ((rc = set_attrs())) return rc;
  auto mark = [&](int i) {
    if (n_ev) (void)hipEventRecord((hipEvent_t)ev[i], s);
  };
  void* ws = workspace;
  mark(0);
  moe::AlignOut o{};
  if (pl.cold) {
    o.cold_seg = at<int32_t>(ws, pl.cold_seg);
    o.cold_max = moe::cold::MAX_ROWS;
  }
  o.counts = at<int32_t>(ws, pl.counts);
  o.cu = at<int32_t>(ws, pl.cu);
  o.offsets = at<int32_t>(ws, pl.offsets);
  o.tile_seg = at<int32_t>(ws, pl.tile_seg);
  o.tile_row0 = at<int32_t>(ws, pl.tile_row0);
  o.status = at<int32_t>(ws, pl.status);
  hipLaunchKernelGGL(moe::k_grouped_prep, dim3(1), dim3(1024), (size_t)(3 * p->E + 32) * 4, s, cu_seqlens, p->E,
                     p->T, pl.BM, o);
  if ((rc = launch_status())) return rc;
  const bool mx = p->wfmt == MOE_W_MXFP4;
  const bool mx8 = p->a_fmt == MOE_A_MXFP8;
  GemmIO g1{x_nvs, nullptr, 1, w_gate, w_up, s_gate, s_up, p->I, p->H, at<void>(ws, pl.act), route_w, 1, 0, {}, {}};
  if (mx8) g1.Cq = quant_rows_at(ws, pl.aq, pl.M, p->I);
  if (p->weight_on_input) {
    g1.A = at<void>(ws, pl.xs);
    g1.row_w = nullptr;
    hipLaunchKernelGGL(moe::k_scale_rows, dim3((unsigned)p->T), dim3(256), 0, s, (const uint16_t*)x_nvs,
                       (const int32_t*)nullptr, 1, route_w, (const int32_t*)nullptr, p->T, p->H,
                       at<uint16_t>(ws, pl.xs));
  }
  mark(1);
  if (mx) {
    g1.Aq = quant_rows_at(ws, pl.xq, pl.M, p->H);
    launch_quant(mx8, g1.A, pl.M, p->H, g1.Aq, s);
  }
  GemmIO g2{at<void>(ws, pl.act), nullptr, 1, w_down, nullptr, s_down, nullptr, p->H, p->I, out_nvs, nullptr, 1, 0, {},
            {}};
  if (mx) {
    if ((rc = launch_gemm<true>(*p, pl, g1, ws, s))) return rc;
    mark(2);
    g2.Aq = quant_rows_at(ws, pl.aq, pl.M, p->I);
    if (!mx8) launch_quant(false, g2.A, pl.M, p->I, g2.Aq, s);
    if ((rc = launch_gemm<false>(*p, pl, g2, ws, s))) return rc;
  } else if ((rc = launch_gemms(*p, pl, g1, g2, ws, s, true, mark))) {
    return rc;
  }
  mark(3);
  hipLaunchKernelGGL(moe::k_zero_tail, dim3(p->T), dim3(256), 0, s, (uint16_t*)out_nvs,
                     (const int32_t*)o.status, p->T, p->H);
  mark(4);
  return launch_status();
}

}  // namespace

extern "C" {

int moe_experts_forward_grouped(const moe_problem* p, const void* x_nvs, const int32_t* cu_seqlens,
                                const float* route_w, const void* w_gate, const void* w_up, const void* w_down,
                                const uint8_t* s_gate, const uint8_t* s_up, const uint8_t* s_down, void* out_nvs,
                                void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  return grouped_impl(p, x_nvs, cu_seqlens, route_w, w_gate, w_up, w_down, s_gate, s_up, s_down, out_nvs,
                      workspace, workspace_bytes, (hipStream_t)stream, nullptr, 0);
}

int moe_experts_forward_grouped_timed(const moe_problem* p, const void* x_nvs, const int32_t* cu_seqlens,
                                      const float* route_w, const void* w_gate, const void* w_up,
                                      const void* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                                      const uint8_t* s_down, void* out_nvs, void* workspace,
                                      size_t workspace_bytes, moe_stream_t stream, void* const* stage_events,
                                      int n_events) {
  return grouped_impl(p, x_nvs, cu_seqlens, route_w, w_gate, w_up, w_down, s_gate, s_up, s_down, out_nvs,
                      workspace, workspace_bytes, (hipStream_t)stream, stage_events, n_events);
}

int moe_route(const moe_route_problem* p, const float* logits, const float* bias, int32_t* topk_ids,
              float* topk_weights, moe_stream_t stream) {
  if (!p) return MOE_EINVAL;
  if (p->T < 0 || p->E <= 0 || p->k <= 0) return MOE_EINVAL;
  if (p->method != MOE_ROUTE_RENORMALIZE && p->method != MOE_ROUTE_DEEPSEEK_V3) return MOE_EINVAL;
  if (p->E > moe::kRouteMaxE || p->k > moe::kRouteMaxK) return MOE_ENOTSUP;
  if (p->k > p->E) return MOE_EINVAL;
  const bool ds = p->method == MOE_ROUTE_DEEPSEEK_V3;
  const bool grouped = ds && p->n_group > 1;
  if (ds) {
    if (p->n_group < 0 || !std::isfinite(p->routed_scaling_factor)) return MOE_EINVAL;
    if (grouped && (p->n_group > moe::kRouteMaxGroups || p->E % p->n_group || p->E / p->n_group < 2 ||
                    p->topk_group < 1 || p->topk_group > p->n_group ||
                    (long long)p->k > (long long)p->topk_group * (p->E / p->n_group)))
      return MOE_EINVAL;
  }
  if (!logits || !topk_ids || !topk_weights) return MOE_EINVAL;
  if (((uintptr_t)logits | (uintptr_t)topk_ids | (uintptr_t)topk_weights | (uintptr_t)bias) & 3u) return MOE_EINVAL;
  if (p->T == 0) return MOE_OK;
  moe::RouteParams q;
  q.logits = logits;
  q.bias = ds ? bias : nullptr;
  q.T = p->T;
  q.E = p->E;
  q.k = p->k;
  q.method = ds ? 1 : 0;
  q.n_group = grouped ? p->n_group : 0;
  q.topk_group = grouped ? p->topk_group : 0;
  q.scale = ds ? p->routed_scaling_factor : 1.f;
  q.ids = topk_ids;
  q.w = topk_weights;
  const dim3 grid((unsigned)ceil_div(p->T, 4)), block(256);
  hipStream_t s = (hipStream_t)stream;
  if (p->E <= 64) hipLaunchKernelGGL(moe::k_route<1>, grid, block, 0, s, q);
  else if (p->E <= 128) hipLaunchKernelGGL(moe::k_route<2>, grid, block, 0, s, q);
  else if (p->E <= 256) hipLaunchKernelGGL(moe::k_route<4>, grid, block, 0, s, q);
  else if (p->E <= 512) hipLaunchKernelGGL(moe::k_route<8>, grid, block, 0, s, q);
  else hipLaunchKernelGGL(moe::k_route<16>, grid, block, 0, s, q);
  return launch_status();
}

int moe_device_error(const void* workspace, int32_t* n_bad) {
  if (!workspace || !n_bad) return MOE_EINVAL;
  // status words sit at offset 0 of every workspace layout: [0] bad ids,
  // [3] a single-launch wait gave up
  int32_t st[4] = {0, 0, 0, 0};
  const hipError_t e = hipMemcpy(st, workspace, sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return MOE_EHIP;
  *n_bad = st[0];
  return st[3] ? MOE_ETIMEDOUT : MOE_OK;
}

int moe_check_expert_params(const moe_problem* p, const float* alpha_e, const float* beta_e,
                            const float* limit_e, const float* fc1_alpha, const float* fc2_alpha) {
  if (!p || p->E <= 0) return MOE_EINVAL;
  for (int e = 0; e < p->E; ++e) {
    for (const float* s : {fc1_alpha, fc2_alpha}) {
      if (!s) continue;
      if (!std::isfinite(s[e])) return MOE_EINVAL;
      if (!(s[e] > 0.f)) return MOE_ENOTSUP;
    }
    if (p->act == MOE_ACT_SWIGLU_OAI) {
      if ((alpha_e && !std::isfinite(alpha_e[e])) || (beta_e && !std::isfinite(beta_e[e]))) return MOE_EINVAL;
      if (limit_e && std::isnan(limit_e[e])) return MOE_EINVAL;
      if (limit_e && !(limit_e[e] > 0.f)) return MOE_ENOTSUP;
    } else if (p->act == MOE_ACT_SITU) {
      if ((alpha_e && !std::isfinite(alpha_e[e])) || (beta_e && !std::isfinite(beta_e[e]))) return MOE_EINVAL;
      if ((alpha_e && !(alpha_e[e] > 0.f)) || (beta_e && !(beta_e[e] > 0.f))) return MOE_ENOTSUP;
    }
  }
  return MOE_OK;
}

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "success";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ENOTSUP: return "unsupported problem";
    case MOE_ENOSPC: return "workspace too small";
    case MOE_EHIP: return "HIP error";
    case MOE_ETIMEDOUT: return "a wait on the device gave up";
    default: return "unknown status";
  }
}

}  // extern "C"
