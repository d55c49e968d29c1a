// Key projection with the SimHash codes taken in its epilogue (FAST-AR
// summary, section 2A "Mecanismo": the keys TempCache hashes are the attention
// layer's keys, so they can be hashed where the projection produces them,
// instead of being written out and read back by a separate hash pass).
//
// A workgroup computes the d x 256 (d = 64: d x 128) tile K^T = W_h X^T of
// one head on the 32x32x16 bf16 MFMA (out features as MFMA rows, tokens as
// columns; both operands have D_in contiguous).  Chunks of 32 D_in columns
// move HBM -> LDS with direct-to-LDS loads in MFMA operand order (a lane
// fetches the 16 bytes it will later read as an operand, so every operand
// read is one conflict-free 16-byte LDS load) through a ring of four
// distinct LDS buffers.  The epilogue rounds the tile to bf16 into those
// buffers (64 token rows each, 16-byte chunks permuted by row), stores the keys
// and hashes them against the cache's fragment-ordered hyperplanes, one
// 32-token block per wave, the arithmetic of the hash kernel.
#include "common.hpp"

namespace fastar {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// d = 128: 8 waves on a 256-token tile (each wave 64 features x 64 tokens),
// which brings 24 KiB of operands per 2 MFLOP, within what a CU's load path
// delivers at full MFMA rate; d = 64: 4 waves on 128 tokens.
template <int D>
struct PjCfg {
  static constexpr int kWaves = D == 128 ? 8 : 4;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kTok = D == 128 ? 256 : 128;    // tokens per workgroup
  static constexpr int kFB = D / 32;                    // feature blocks of a head
  static constexpr int kTB = kTok / 32;                 // token blocks
  static constexpr int kWF = 2;                         // waves along features
  static constexpr int kWT = kWaves / kWF;              // waves along tokens
  static constexpr int kFBw = kFB / kWF, kTBw = kTB / kWT;  // blocks per wave
  // A stage is 64 D_in columns (128 bytes) of the head's D weight rows, then
  // of the tile's kTok token rows, row after row in LDS.
  static constexpr int kRows = D + kTok;
  static constexpr int kStage = kRows * 128;
  static constexpr int kInstr = kRows / 8;              // 1 KiB copies per stage
  static constexpr int kPerWave = kInstr / kWaves;      // copies per wave and stage
  static constexpr int kChunks = D / 8;                 // 16-byte chunks of a key row
  static_assert(kInstr % kWaves == 0, "every wave issues the same copies");
  static_assert(kFBw >= 1 && kTBw >= 1, "whole blocks per wave");
  static_assert(2 * 64 * D * 2 <= kStage, "two blocks of 64 epilogue key rows fit a ring buffer");
  static_assert(kTok / 64 <= 4, "the epilogue rows fit the ring buffers");
  // stage rows: 16-byte chunk q of row r sits at chunk q ^ ((r / 2) % 8), so
  // the 16 lanes an LDS read serves at once (16 rows, one chunk) hit
  // distinct banks: row parity picks a 128-byte half of the 256 banks' span,
  // the permutation spreads the 8 rows of each parity over its 8 chunks
  static __device__ __forceinline__ int sw(int r) { return (r >> 1) & 7; }
  // epilogue key rows: chunk c of token row t sits at chunk c ^ (t % kChunks)
  static __device__ __forceinline__ int swz(int t) { return t & (kChunks - 1); }
};

template <int D>
__global__ __launch_bounds__(PjCfg<D>::kThreads, 1) void project_hash_kernel(ProjArgs a) {
  using C = PjCfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t buf0[C::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[C::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t buf2[C::kStage];
  __shared__ uint32_t s_words[C::kTok][9];
  // logical ids run over heads first: an XCD's contiguous range covers all
  // heads of a few token tiles, so each token tile's rows are fetched into one
  // L2 and only the (smaller) key weight is read by every XCD
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int tt = lid / a.H, h = lid - tt * a.H, n0 = tt * C::kTok;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, hf = lane >> 5;
  const int wf = wave % C::kWF, wt = wave / C::kWF;

  // Copy sources.  Copy i of a stage fills stage rows 8i .. 8i+7: lane l
  // fetches 16-byte chunk (l%8) ^ sw(row) of row 8i + l/8 (whole 128-byte
  // lines, 8 per copy) and the copy lands it at chunk l%8.  Rows < D are the
  // head's weight rows, the others tokens (past N: the last token, never
  // stored).  In a last stage of 32 columns (D_in % 64 == 32) chunks 4..7 of
  // a row are refetched from chunks 0..3 instead (read, never used).
  const uint8_t* src[C::kPerWave];
  uint32_t hi_chunk = 0u;  // bit j: copy j fetches a chunk >= 4
#pragma unroll
  for (int j = 0; j < C::kPerWave; ++j) {
    const int r = (wave + j * C::kWaves) * 8 + (lane >> 3);
    const int q = (lane & 7) ^ C::sw(r);
    hi_chunk |= (uint32_t)(q >> 2) << j;
    if (r < D) {
      src[j] = reinterpret_cast<const uint8_t*>(a.w + ((int64_t)h * D + r) * a.sw + q * 8);
    } else {
      const int64_t tok = min(n0 + r - D, a.N - 1);
      src[j] = reinterpret_cast<const uint8_t*>(a.x + tok * a.sx + q * 8);
    }
  }
  const int nk = (a.Din + 63) / 64;
  const bool half_tail = (a.Din & 63) != 0;  // the last stage has 32 columns
  // Copies go through registers: the compiler counts those loads exactly, so
  // a stage's loads can be issued two compute phases before they are written
  // to LDS with no conservative waits in between.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  struct Regs {
    u32x4_t v[C::kPerWave];
  };
  auto load = [&](int stage) __attribute__((always_inline)) {
    const uint32_t tail = (uint32_t)(half_tail && stage == nk - 1);
    Regs R;
#pragma unroll
    for (int j = 0; j < C::kPerWave; ++j) {
      const int back = (int)(((hi_chunk >> j) & tail) << 6);  // branch free
      R.v[j] = *reinterpret_cast<const u32x4_t*>(src[j] + (stage * 128 - back));
    }
    return R;
  };
  auto store = [&](const Regs& R, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < C::kPerWave; ++j)
      *reinterpret_cast<u32x4_t*>(dst + (wave + j * C::kWaves) * 1024 + lane * 16) = R.v[j];
  };

  f32x16_t acc[C::kFBw][C::kTBw];
#pragma unroll
  for (int fb = 0; fb < C::kFBw; ++fb)
#pragma unroll
    for (int tb = 0; tb < C::kTBw; ++tb) acc[fb][tb] = f32x16_t{};

  // Step s: issue the loads of stage s+2 (returned), multiply stage s from
  // cur, write stage s+1 (loaded at step s-1) from Rp into nxt (read at step
  // s-1), then meet the other waves.  The registers travel as values so that
  // they stay in registers; the main loop loads unconditionally so that the
  // count of loads in flight, and so each wait, is exact.
  auto step = [&](const uint8_t* cur, uint8_t* nxt, const Regs& Rp, int s, bool may_load,
                  bool may_store)
      __attribute__((always_inline)) {
    Regs Rn{};
    if (may_load) Rn = load(s + 2);
    const int nks = half_tail && s == nk - 1 ? 2 : 4;  // k-steps of 16 columns
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks >= nks) break;
      const int q = 2 * ks + hf;  // this lane's 8 columns of the k-step
      bf16x8_t A[C::kFBw], B[C::kTBw];
#pragma unroll
      for (int fb = 0; fb < C::kFBw; ++fb) {
        const int r = (wf * C::kFBw + fb) * 32 + m;
        A[fb] = *reinterpret_cast<const bf16x8_t*>(cur + r * 128 + ((q ^ C::sw(r)) << 4));
      }
#pragma unroll
      for (int tb = 0; tb < C::kTBw; ++tb) {
        const int r = D + (wt * C::kTBw + tb) * 32 + m;
        B[tb] = *reinterpret_cast<const bf16x8_t*>(cur + r * 128 + ((q ^ C::sw(r)) << 4));
      }
#pragma unroll
      for (int fb = 0; fb < C::kFBw; ++fb)
#pragma unroll
        for (int tb = 0; tb < C::kTBw; ++tb)
          acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[fb], B[tb], acc[fb][tb], 0, 0, 0);
    }
    if (may_store) store(Rp, nxt);
    __syncthreads();
    return Rn;
  };
  Regs Ra = load(0), Rb{};
  if (nk > 1) Rb = load(1);
  store(Ra, buf0);
  __syncthreads();
  int s = 0;
  for (; s + 3 < nk; s += 2) {  // stages s+2 and s+3 exist
    Ra = step(buf0, buf1, Rb, s, true, true);
    Rb = step(buf1, buf0, Ra, s + 1, true, true);
  }
  // 1 to 3 steps remain
  Ra = step(buf0, buf1, Rb, s, s + 2 < nk, s + 1 < nk);
  if (s + 1 < nk) step(buf1, buf0, Ra, s + 1, false, s + 2 < nk);
  if (s + 2 < nk) step(buf0, buf1, Regs{}, s + 2, false, false);
  __syncthreads();  // the ring is read; it now takes the key rows

  // bf16 keys into token rows: tokens 0..63 in buf0, 64..127 in buf1 (every
  // access below names one of the two buffers, never a choice between them,
  // so the compiler can tell all LDS objects apart in the copy loop above).
  // Register j of lane l: feature 8*(j/4) + 4*(l/32) + j%4 of the block,
  // token l%32: four consecutive features, one 8-byte store.
  auto put_rows = [&](uint8_t* rows, int fb, int tb, int t) __attribute__((always_inline)) {
    uint8_t* row = rows + t * D * 2;  // t: token within the buffer
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int f = (wf * C::kFBw + fb) * 32 + 8 * jg + 4 * hf;
      const uint32_t w0 = f32_to_bf16_bits(acc[fb][tb][4 * jg + 0]) |
                          (f32_to_bf16_bits(acc[fb][tb][4 * jg + 1]) << 16);
      const uint32_t w1 = f32_to_bf16_bits(acc[fb][tb][4 * jg + 2]) |
                          (f32_to_bf16_bits(acc[fb][tb][4 * jg + 3]) << 16);
      *reinterpret_cast<uint2*>(row + (((f >> 3) ^ C::swz(t)) << 4) + (f & 7) * 2) = make_uint2(w0, w1);
    }
  };
#pragma unroll
  for (int fb = 0; fb < C::kFBw; ++fb)
#pragma unroll
    for (int tb = 0; tb < C::kTBw; ++tb) {
      const int blk = wt * C::kTBw + tb;  // wave-uniform; 64 token rows per region
      const int t = (blk & 1) * 32 + m;
      switch (blk >> 1) {
        case 0: put_rows(buf0, fb, tb, t); break;
        case 1: put_rows(buf1, fb, tb, t); break;
        case 2: put_rows(buf2, fb, tb, t); break;
        default: put_rows(buf0 + 64 * D * 2, fb, tb, t); break;
      }
    }
  __syncthreads();

  // the keys, 16 bytes per store
  auto store_rows = [&](const uint8_t* rows, int t0) __attribute__((always_inline)) {
    for (int idx = tid; idx < 64 * C::kChunks; idx += C::kThreads) {
      const int t = idx / C::kChunks, c = idx - t * C::kChunks;
      if (n0 + t0 + t >= a.N) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(rows + t * D * 2 + ((c ^ C::swz(t)) << 4));
      *reinterpret_cast<uint4*>(a.k + (int64_t)h * a.sk_h + (int64_t)(n0 + t0 + t) * a.sk_n + c * 8) = v;
    }
  };
  store_rows(buf0, 0);
  store_rows(buf1, 64);
  if (C::kTok > 128) {
    store_rows(buf2, 128);
    store_rows(buf0 + 64 * D * 2, 192);
  }

  // SimHash of the stored keys: wave w takes tokens 32w .. 32w+31 against
  // every block of 32 hyperplanes (MFMA rows, from the fragment-ordered
  // copy); columns are the wave's tokens, features hf*D/2 + 8*ks .. +7 in
  // k-step ks for both operands (the order the fragments were written in)
  auto hash_rows = [&](const uint8_t* rows, int t) __attribute__((always_inline)) {
    const uint8_t* row = rows + t * D * 2;  // t: token within the buffer
    const bf16x8_t* pf = static_cast<const bf16x8_t*>(a.planes_frag) + lane;
    const int tw = wave * 32 + m;           // token within the tile
    for (int pb = 0; pb < a.Ppad / 32; ++pb) {
      f32x16_t hacc = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8_t pa = pf[(pb * (D / 16) + ks) * 64];
        const int c = hf * (D / 16) + ks;
        const bf16x8_t kb = *reinterpret_cast<const bf16x8_t*>(row + ((c ^ C::swz(t)) << 4));
        hacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, kb, hacc, 0, 0, 0);
      }
      // register j of lane l: plane 8*(j/4) + 4*(l/32) + j%4 of the block,
      // token l%32
      uint32_t bits = 0u;
#pragma unroll
      for (int j = 0; j < 16; ++j) bits |= (hacc[j] > 0.0f ? 1u : 0u) << (8 * (j >> 2) + (j & 3));
      bits <<= 4 * hf;
      const uint32_t word = bits | __shfl_xor(bits, 32);
      if (hf == 0) s_words[tw][pb] = word;
    }
    if (hf == 0)
      for (int pb = a.Ppad / 32; pb < 9; ++pb) s_words[tw][pb] = 0u;
  };
  {
    const int t = (wave & 1) * 32 + m;
    switch (wave >> 1) {  // wave-uniform
      case 0: hash_rows(buf0, t); break;
      case 1: hash_rows(buf1, t); break;
      case 2: hash_rows(buf2, t); break;
      default: hash_rows(buf0 + 64 * D * 2, t); break;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < C::kTok * a.L; idx += C::kThreads) {
    const int t = idx / a.L, tb = idx - t * a.L;
    if (n0 + t >= a.N) continue;
    a.codes[((int64_t)h * a.L + tb) * a.codes_ld + n0 + t] = extract_code(s_words[t], tb * a.b, a.b);
  }
}

template <int D>
hipError_t launch_d(const ProjArgs& a, hipStream_t s) {
  using C = PjCfg<D>;
  const int tiles = (a.N + C::kTok - 1) / C::kTok;
  const int blocks = a.H * tiles;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((project_hash_kernel<D>), dim3(blocks), dim3(C::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_project_hash(const ProjArgs& a, int d, hipStream_t s) {
  if (d == 128) return launch_d<128>(a, s);
  if (d == 64) return launch_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fastar
