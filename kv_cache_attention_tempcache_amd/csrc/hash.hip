// SimHash on gfx950 (FAST-AR summary, section 2A "Mecanismo": the nearest-
// neighbour search runs on locality-sensitive hashes).  Bit j of table t is
// [<r_tj, x> > 0], stored as 1u << j.
//
// bf16 path: the projection is a small GEMM (L*b x d) * (d x rows) on the
// 32x32x16 bf16 MFMA, hyperplanes as the MFMA rows and key rows as its
// columns.  A workgroup copies the hyperplanes once into LDS, already in MFMA
// operand order (one 1 KiB fragment per 32 planes and k-step, lane-major), so
// the copy is a plain coalesced read and every later operand read is one
// conflict-free 16-byte LDS load; its waves then take 32 key rows at a time.
// The k-steps read features (2*ks + half)*8 .. +7, so the two half-waves load
// adjacent 16 bytes of each row.  Each lane's accumulators hold 16 of the 32
// projections of one key row; it packs 16 sign bits locally and one lane
// exchange with the other half-wave completes the 32-bit word, in LSB-first
// plane order.  Rows past the end and padding planes are read clamped to valid
// memory and never stored.
//
// f32 path: 32 lanes per (row, table), one plane per lane, products and sums
// in float64.
#include "common.hpp"

namespace fastar {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kHashWaves = 8;
constexpr int kHashThreads = kHashWaves * kWave;

template <int D>
__global__ __launch_bounds__(kHashThreads) void hash_bf16_kernel(HashArgs a, int tiles_per_head,
                                                                 int total_tiles) {
  constexpr int KS = D / 16;  // k-steps
  extern __shared__ __attribute__((aligned(16))) bf16x8_t frag[];  // [Ppad/32][KS][64]
  const int P = a.L * a.b;
  const int npb = (P + 31) / 32;
  const uint16_t* planes = static_cast<const uint16_t*>(a.planes);
  const uint16_t* xbase = static_cast<const uint16_t*>(a.x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, hf = lane >> 5;

  // tile -> head, row of this lane, and its source row (clamped into the
  // tile when past the end); `live` is false for a tile wholly past the end
  struct Tile {
    int h, r;
    int64_t xrow;
    bool valid, live;
  };
  auto locate = [&](int tile) __attribute__((always_inline)) {
    Tile t{0, 0, 0, false, false};
    if (tile >= total_tiles) return t;
    t.h = tile / tiles_per_head;
    const int r0 = (tile - t.h * tiles_per_head) * 32;
    const int nrows = a.rows ? a.n_rows[(int64_t)t.h * a.n_rows_stride] : a.N;
    if (r0 >= nrows) return t;
    t.live = true;
    t.r = r0 + m;
    t.valid = t.r < nrows;
    t.xrow = t.valid ? t.r : r0;
    if (a.rows) t.xrow = a.rows[(int64_t)t.h * a.rows_ld + t.xrow];
    return t;
  };
  // k-step ks of this lane: features (2*ks + hf)*8 .. +7 of its row
  auto load_x = [&](const Tile& t, bf16x8_t (&A)[KS]) __attribute__((always_inline)) {
    const uint16_t* xp = xbase + (int64_t)t.h * a.sx_h + t.xrow * a.sx_n + hf * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) A[ks] = *reinterpret_cast<const bf16x8_t*>(xp + ks * 16);
  };

  // the first tile's rows are requested before the hyperplane copy
  int tile = blockIdx.x * kHashWaves + wave;
  const int stride = gridDim.x * kHashWaves;
  Tile cur = locate(tile);
  bf16x8_t A[KS];
  if (cur.live) load_x(cur, A);

  // hyperplanes -> LDS fragments: chunk c (features 8c..8c+7) of plane p is
  // k-step c/2, half c%2 of lane 32*(c%2) + p%32 in block p/32.  Four lanes
  // read 64 contiguous bytes of a plane (their LDS stores then meet at most
  // 4-way bank conflicts, once per workgroup).
  // All of a thread's loads are issued before its first store.
  constexpr int kFill = (FASTAR_MAX_TABLES * FASTAR_MAX_BITS * (D / 8) + kHashThreads - 1) /
                        kHashThreads;
  const int Ppad = npb * 32, n_chunks = Ppad * (D / 8);
  bf16x8_t fv[kFill];
  int fdst[kFill];
#pragma unroll
  for (int i = 0; i < kFill; ++i) {
    const int idx = threadIdx.x + i * kHashThreads;
    fdst[i] = -1;
    if (idx >= n_chunks) continue;
    const int rest = idx >> 2;
    const int p = rest % Ppad, c = 4 * (rest / Ppad) + (idx & 3);
    const int pc = p < P ? p : P - 1;
    fv[i] = *reinterpret_cast<const bf16x8_t*>(planes + (int64_t)pc * D + c * 8);
    fdst[i] = ((p >> 5) * KS + (c >> 1)) * 64 + (c & 1) * 32 + (p & 31);
  }
#pragma unroll
  for (int i = 0; i < kFill; ++i)
    if (fdst[i] >= 0) frag[fdst[i]] = fv[i];
  __syncthreads();

  for (; tile < total_tiles; tile += stride) {
    // the next tile's rows load while this one is projected
    const Tile nxt = locate(tile + stride);
    bf16x8_t An[KS];
    if (nxt.live) load_x(nxt, An);

    if (cur.live) {
      uint32_t words[9];
#pragma unroll
      for (int k = 0; k < 9; ++k) words[k] = 0u;
      // register j of lane l: plane 32*pb + 8*(j/4) + 4*(l/32) + j%4 of key row l%32
#pragma unroll
      for (int pb = 0; pb < 8; ++pb) {
        if (pb >= npb) break;
        const bf16x8_t* fb = frag + pb * KS * 64 + lane;
        f32x16_t acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks * 64], A[ks], acc, 0, 0, 0);
        uint32_t bits = 0u;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          bits |= (acc[j] > 0.0f ? 1u : 0u) << (8 * (j >> 2) + (j & 3));
        bits <<= 4 * hf;
        words[pb] = bits | __shfl_xor(bits, 32);  // both halves: the word of row m
      }
      if (hf == 0 && cur.valid) {
        const int64_t col = a.rows ? cur.xrow : (int64_t)cur.r;
        for (int t = 0; t < a.L; ++t) {
          a.codes[((int64_t)cur.h * a.L + t) * a.codes_ld + a.codes_col0 + col] =
              extract_code(words, t * a.b, a.b);
        }
      }
    }
    cur = nxt;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) A[ks] = An[ks];
  }
}

// 32 lanes per (head, table, row): lane j projects onto plane j of the table
// (a sequential float64 sum over the features, as one thread per row would),
// and a wave ballot packs the bits of the wave's two rows.
template <int D>
__global__ __launch_bounds__(256) void hash_f32_kernel(HashArgs a, int64_t total) {
  const float* planes = static_cast<const float*>(a.planes);
  const float* xbase = static_cast<const float*>(a.x);
  const int j = threadIdx.x & 31;
  // every thread of a block runs the same iterations (the ballot needs the
  // whole wave)
  for (int64_t base = blockIdx.x * (int64_t)blockDim.x; base < total * 32;
       base += (int64_t)gridDim.x * blockDim.x) {
    const int64_t item = (base + threadIdx.x) >> 5;  // (h, t, r), r fastest
    bool valid = item < total;
    int h = 0, t = 0, r = 0;
    int64_t xrow = 0;
    if (valid) {
      r = (int)(item % a.N);
      const int64_t ht = item / a.N;
      t = (int)(ht % a.L);
      h = (int)(ht / a.L);
      const int nrows = a.rows ? a.n_rows[(int64_t)h * a.n_rows_stride] : a.N;
      valid = r < nrows;
      if (valid) xrow = a.rows ? (int64_t)a.rows[(int64_t)h * a.rows_ld + r] : (int64_t)r;
    }
    bool bit = false;
    if (valid && j < a.b) {
      const float* xp = xbase + (int64_t)h * a.sx_h + xrow * a.sx_n;
      const float* rp = planes + ((int64_t)t * a.b + j) * D;
      double acc = 0.0;
      for (int k = 0; k < D; ++k) acc += (double)xp[k] * (double)rp[k];
      bit = acc > 0.0;
    }
    const uint64_t bits = __ballot(bit);
    if (valid && j == 0) {
      const uint32_t code = (uint32_t)(bits >> (threadIdx.x & 32));
      a.codes[((int64_t)h * a.L + t) * a.codes_ld + a.codes_col0 + xrow] = code;
    }
  }
}

}  // namespace

hipError_t launch_hash_bf16(const HashArgs& a, hipStream_t s) {
  if (a.M > 0) return launch_pq(a, true, s);
  const int tiles_per_head = (a.N + 31) / 32;
  const int total = a.H * tiles_per_head;
  const int P = a.L * a.b;
  if (total == 0) return hipSuccess;
  // one pass of 8-wave groups; a larger job loops, two workgroups per CU
  int blocks = (total + kHashWaves - 1) / kHashWaves;
  if (blocks > 512) blocks = 512;
  const size_t lds = (size_t)((P + 31) / 32) * 32 * a.d * sizeof(uint16_t);
  if (a.d == 128)
    hipLaunchKernelGGL(hash_bf16_kernel<128>, dim3(blocks), dim3(kHashThreads), lds, s, a,
                       tiles_per_head, total);
  else
    hipLaunchKernelGGL(hash_bf16_kernel<64>, dim3(blocks), dim3(kHashThreads), lds, s, a,
                       tiles_per_head, total);
  return hipGetLastError();
}

hipError_t launch_hash_f32(const HashArgs& a, hipStream_t s) {
  if (a.M > 0) return launch_pq(a, false, s);
  const int64_t total = (int64_t)a.H * a.N * a.L;  // (head, table, row) items, 32 lanes each
  if (total == 0) return hipSuccess;
  int64_t blocks = (total * 32 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (a.d == 128)
    hipLaunchKernelGGL(hash_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  else
    hipLaunchKernelGGL(hash_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

}  // namespace fastar
