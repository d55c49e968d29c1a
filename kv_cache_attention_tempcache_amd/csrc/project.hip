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
  static constexpr int kFrags = 2 * (kFB + kTB);        // 1 KiB fragments per stage
  static constexpr int kStage = kFrags * 1024;
  static constexpr int kPerWave = kFrags / kWaves;      // copies per wave and stage
  static constexpr int kChunks = D / 8;                 // 16-byte chunks of a key row
  static_assert(kFrags % kWaves == 0, "every wave issues the same copies");
  static_assert(kFBw >= 1 && kTBw >= 1, "whole blocks per wave");
  static_assert(64 * D * 2 <= kStage, "64 epilogue key rows fit one ring buffer");
  static_assert(kTok / 64 <= 4, "the epilogue rows fit the four ring buffers");
  // epilogue key rows: chunk c of token row t sits at chunk c ^ (t % kChunks)
  static __device__ __forceinline__ int swz(int t) { return t & (kChunks - 1); }
};

template <int D>
__global__ __launch_bounds__(PjCfg<D>::kThreads, 2) void project_hash_kernel(ProjArgs a) {
  using C = PjCfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t buf0[C::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[C::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t buf2[C::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t buf3[C::kStage];
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

  // Copy sources.  Stage fragment i < 2*kFB: W rows of feature block i/2,
  // k-step i%2; the others: X rows of token block (i - 2*kFB)/2.  Lane l
  // fetches row 32*block + l%32, columns 16*(i%2) + 8*(l/32) .. +7 of the
  // stage's 32; tokens past N fetch the last token (their keys are never
  // stored).
  const uint8_t* src[C::kPerWave];
#pragma unroll
  for (int j = 0; j < C::kPerWave; ++j) {
    const int i = wave + j * C::kWaves;
    const int ks = i & 1;
    if (i < 2 * C::kFB) {
      const int64_t row = (int64_t)h * D + (i >> 1) * 32 + m;
      src[j] = reinterpret_cast<const uint8_t*>(a.w + row * a.sw + ks * 16 + hf * 8);
    } else {
      const int64_t tok = min(n0 + ((i - 2 * C::kFB) >> 1) * 32 + m, a.N - 1);
      src[j] = reinterpret_cast<const uint8_t*>(a.x + tok * a.sx + ks * 16 + hf * 8);
    }
  }
  auto issue = [&](int stage, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < C::kPerWave; ++j)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(src[j] + (int64_t)stage * 64),
                                       (lds_void_t*)(dst + (wave + j * C::kWaves) * 1024), 16, 0, 0);
  };
  // Wait until at most n stages' copies issued by this wave are in flight
  // (every older stage has landed), finish this wave's LDS reads, then meet
  // the other waves.  A plain barrier: __syncthreads() would also wait for
  // the copies that are meant to stay in flight.
  auto wait_barrier = [&](int n) __attribute__((always_inline)) {
    if (n >= 2)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * C::kPerWave) : "memory");
    else if (n == 1)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(C::kPerWave) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  f32x16_t acc[C::kFBw][C::kTBw];
#pragma unroll
  for (int fb = 0; fb < C::kFBw; ++fb)
#pragma unroll
    for (int tb = 0; tb < C::kTBw; ++tb) acc[fb][tb] = f32x16_t{};

  const int nk = a.Din / 32;
  // A ring of four stage buffers: step s reads stage s from cur after issuing
  // the copy of stage s+3 into nxt (the buffer read at step s-1), then waits
  // until stage s+1 has landed, the copies of stages s+2, s+3 staying in
  // flight.
  auto step = [&](const uint8_t* cur, uint8_t* nxt, int s) __attribute__((always_inline)) {
    if (s + 3 < nk) issue(s + 3, nxt);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t A[C::kFBw], B[C::kTBw];
#pragma unroll
      for (int fb = 0; fb < C::kFBw; ++fb)
        A[fb] = *reinterpret_cast<const bf16x8_t*>(cur + (((wf * C::kFBw + fb) * 2 + ks) * 64 + lane) * 16);
#pragma unroll
      for (int tb = 0; tb < C::kTBw; ++tb)
        B[tb] = *reinterpret_cast<const bf16x8_t*>(
            cur + ((2 * C::kFB + (wt * C::kTBw + tb) * 2 + ks) * 64 + lane) * 16);
#pragma unroll
      for (int fb = 0; fb < C::kFBw; ++fb)
#pragma unroll
        for (int tb = 0; tb < C::kTBw; ++tb)
          acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[fb], B[tb], acc[fb][tb], 0, 0, 0);
    }
    wait_barrier(min(nk - 1, s + 3) - (s + 1));
  };
#pragma unroll
  for (int u = 0; u < 3; ++u)
    if (u < nk) issue(u, u == 0 ? buf0 : u == 1 ? buf1 : buf2);
  wait_barrier(min(nk, 3) - 1);
  for (int s = 0; s < nk; s += 4) {
    step(buf0, buf3, s);
    if (s + 1 < nk) step(buf1, buf0, s + 1);
    if (s + 2 < nk) step(buf2, buf1, s + 2);
    if (s + 3 < nk) step(buf3, buf2, s + 3);
  }
  __syncthreads();  // the ring is read; buf0 / buf1 now take the key rows

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
      const int blk = wt * C::kTBw + tb;  // wave-uniform; 64 token rows per buffer
      const int t = (blk & 1) * 32 + m;
      switch (blk >> 1) {
        case 0: put_rows(buf0, fb, tb, t); break;
        case 1: put_rows(buf1, fb, tb, t); break;
        case 2: put_rows(buf2, fb, tb, t); break;
        default: put_rows(buf3, fb, tb, t); break;
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
    store_rows(buf3, 192);
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
      default: hash_rows(buf3, t); break;
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
