// SimHash on gfx950 (FAST-AR summary, section 2A "Mecanismo": the nearest-
// neighbour search runs on locality-sensitive hashes).  Bit j of table t is
// [<r_tj, x> > 0], stored as 1u << j.
//
// bf16 path: the projection is a small GEMM (L*b x d) * (d x rows) on the
// 32x32x16 bf16 MFMA.  A wave owns 32 rows and reads the hyperplane operands
// straight from L2 (a few KiB shared by every wave), with no LDS staging and
// no block barrier between the loads and the MFMAs.  With hyperplanes as the
// MFMA rows, each lane's accumulators hold 16 of the 32 projections of one
// key row, so it packs 16 sign bits locally and one lane exchange with the
// other half-wave completes the 32-bit word, in LSB-first plane order.
//
// f32 path: one thread per (row, table), products and sums in float64.
#include "common.hpp"

namespace fastar {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kHashWaves = 4;

template <int D>
__global__ __launch_bounds__(256) void hash_bf16_kernel(HashArgs a, int tiles_per_head,
                                                        int total_tiles) {
  const int P = a.L * a.b;
  const int Ppad = (P + 31) & ~31;
  const uint16_t* planes = static_cast<const uint16_t*>(a.planes);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, hf = lane >> 5;
  const uint16_t* xbase = static_cast<const uint16_t*>(a.x);

  for (int tile = blockIdx.x * kHashWaves + wave; tile < total_tiles;
       tile += gridDim.x * kHashWaves) {
    const int h = tile / tiles_per_head;
    const int r0 = (tile - h * tiles_per_head) * 32;
    const int nrows = a.rows ? a.n_rows[(int64_t)h * a.n_rows_stride] : a.N;
    if (r0 >= nrows) continue;
    const int r = r0 + m;
    const bool valid = r < nrows;
    int64_t xrow = r;
    if (a.rows) xrow = valid ? a.rows[(int64_t)h * a.rows_ld + r] : 0;
    else if (!valid) xrow = 0;

    // A operand: row m, features hf*D/2 + ks*8 .. +7 for k-step ks (the same
    // feature permutation is applied to the hyperplanes below).
    bf16x8_t A[D / 16];
    const uint16_t* xp = xbase + (int64_t)h * a.sx_h + xrow * a.sx_n + hf * (D / 2);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(xp + ks * 8);
      if (!valid) v = bf16x8_t{};
      A[ks] = v;
    }

    uint32_t words[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) words[k] = 0u;
    // B operands straight from L2: hyperplane pb*32 + m (zero past L*b); the
    // next block's operands are loaded while this block's MFMAs run
    const int npb = Ppad / 32;
    auto load_b = [&](int pb, bf16x8_t (&Bf)[D / 16]) __attribute__((always_inline)) {
      const int prow = pb * 32 + m;
      const uint16_t* pp = planes + (int64_t)(prow < P ? prow : 0) * D + hf * (D / 2);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) Bf[ks] = *reinterpret_cast<const bf16x8_t*>(pp + ks * 8);
      if (pb * 32 + 32 > P) {  // only a last, partial block has padding planes
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          if (prow >= P) Bf[ks] = bf16x8_t{};
      }
    };
    // hyperplanes as MFMA rows, keys as columns: register j of lane l holds
    // plane 8*(j/4) + 4*(l/32) + j%4 of key row l%32
    auto block = [&](int pb, const bf16x8_t (&Bf)[D / 16]) __attribute__((always_inline)) {
      f32x16_t acc = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Bf[ks], A[ks], acc, 0, 0, 0);
      uint32_t bits = 0u;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        bits |= (acc[j] > 0.0f ? 1u : 0u) << (8 * (j >> 2) + (j & 3));
      bits <<= 4 * hf;
      words[pb] = bits | __shfl_xor(bits, 32);  // both halves: the word of row m
    };
    bf16x8_t B0[D / 16], B1[D / 16];
    load_b(0, B0);
#pragma unroll
    for (int pb = 0; pb < 8; pb += 2) {
      if (pb >= npb) break;
      if (pb + 1 < npb) load_b(pb + 1, B1);
      block(pb, B0);
      if (pb + 1 >= npb) break;
      if (pb + 2 < npb) load_b(pb + 2, B0);
      block(pb + 1, B1);
    }

    if (hf == 0 && valid) {
      const int64_t col = a.rows ? xrow : (int64_t)r;
      for (int t = 0; t < a.L; ++t) {
        a.codes[((int64_t)h * a.L + t) * a.codes_ld + a.codes_col0 + col] =
            extract_code(words, t * a.b, a.b);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void hash_f32_kernel(HashArgs a, int64_t total) {
  const float* planes = static_cast<const float*>(a.planes);
  const float* xbase = static_cast<const float*>(a.x);
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(idx % a.L);
    const int64_t rest = idx / a.L;
    const int r = (int)(rest % a.N);
    const int h = (int)(rest / a.N);
    const int nrows = a.rows ? a.n_rows[(int64_t)h * a.n_rows_stride] : a.N;
    if (r >= nrows) continue;
    const int64_t xrow = a.rows ? (int64_t)a.rows[(int64_t)h * a.rows_ld + r] : (int64_t)r;
    const float* xp = xbase + (int64_t)h * a.sx_h + xrow * a.sx_n;
    uint32_t code = 0u;
    for (int j = 0; j < a.b; ++j) {
      const float* rp = planes + ((int64_t)t * a.b + j) * D;
      double acc = 0.0;
      for (int k = 0; k < D; ++k) acc += (double)xp[k] * (double)rp[k];
      if (acc > 0.0) code |= 1u << j;
    }
    a.codes[((int64_t)h * a.L + t) * a.codes_ld + a.codes_col0 + xrow] = code;
  }
}

}  // namespace

hipError_t launch_hash_bf16(const HashArgs& a, hipStream_t s) {
  const int tiles_per_head = (a.N + 31) / 32;
  const int total = a.H * tiles_per_head;
  if (total == 0) return hipSuccess;
  int blocks = (total + kHashWaves - 1) / kHashWaves;
  if (blocks > 4096) blocks = 4096;
  if (a.d == 128)
    hipLaunchKernelGGL(hash_bf16_kernel<128>, dim3(blocks), dim3(256), 0, s, a, tiles_per_head,
                       total);
  else
    hipLaunchKernelGGL(hash_bf16_kernel<64>, dim3(blocks), dim3(256), 0, s, a, tiles_per_head,
                       total);
  return hipGetLastError();
}

hipError_t launch_hash_f32(const HashArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.H * a.N * a.L;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (a.d == 128)
    hipLaunchKernelGGL(hash_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  else
    hipLaunchKernelGGL(hash_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

}  // namespace fastar
