// Product-quantization codes (FAST-AR summary, section 2: the nearest-neighbour
// search uses "LSH or quantization"; this is the quantization).  A table splits
// the d features into M equal slices; slice m takes the index of its nearest
// centroid among K = 2^(b/M) (ties to the lowest index), and the b-bit code
// concatenates the slice indices, slice m at bits [m*b/M, (m+1)*b/M).
//
// bf16 path: nearest in Euclidean distance = largest <x, c> - |c|^2/2, so a
// slice's scores are a small GEMM (centroids x slice features) x (slice
// features x rows) on the 32x32x16 bf16 MFMA, centroids as the MFMA rows.
// For each table the workgroup stages that table's codebooks in LDS in MFMA
// operand order (one 1 KiB fragment per 32 centroids and k-step) beside the
// half squared norms; each wave then takes 32 rows at a time, keeps per lane
// the best (score, index) of the 16 centroids its accumulators hold, and one
// exchange with lane^32 settles each slice.  The k-steps read features
// (2*ks + half)*8 .. +7, so slice m is k-steps [m*d/(16M), (m+1)*d/(16M)).
// Padding centroids (K < 32) score -inf.  Rows past the end are read clamped
// and never stored.
//
// f32 path: one thread per (row, table), squared distances in float64.
#include "common.hpp"

namespace fastar {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kPqWaves = 8;
constexpr int kPqThreads = kPqWaves * kWave;

template <int D, int M>
__global__ __launch_bounds__(kPqThreads) void pq_bf16_kernel(HashArgs a, int tiles_per_head,
                                                             int total_tiles) {
  constexpr int KS = D / 16;        // k-steps of a row
  constexpr int W = D / M;          // features per slice
  constexpr int KSM = W / 16;       // k-steps per slice
  static_assert(W % 16 == 0, "slices of whole k-steps");
  extern __shared__ __attribute__((aligned(16))) bf16x8_t frag[];  // [M][NCB][KSM][64]
  const int bpm = a.b / M;          // bits per slice
  const int K = 1 << bpm;
  const int ncb = (K + 31) / 32, Kpad = ncb * 32;
  float* hn = reinterpret_cast<float*>(frag + (size_t)M * ncb * KSM * 64);  // [M][Kpad]
  const uint16_t* cbooks = static_cast<const uint16_t*>(a.planes);  // [L][M][K][W]
  const uint16_t* xbase = static_cast<const uint16_t*>(a.x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mrow = lane & 31, hf = lane >> 5;

  for (int t = 0; t < a.L; ++t) {
    __syncthreads();  // the previous table's codebooks are no longer read
    const uint16_t* cb_t = cbooks + (size_t)t * M * K * W;
    // fragments: chunk c (features 8c..8c+7 of the slice) of centroid k of
    // slice m is k-step c/2, half c%2 of lane 32*(c%2) + k%32 in block k/32;
    // a thread issues all its loads before its first store
    constexpr int kFill = (256 * D / 8 + kPqThreads - 1) / kPqThreads;
    const int n_chunks = M * Kpad * (W / 8);
    bf16x8_t fv[kFill];
    int fdst[kFill];
#pragma unroll
    for (int i = 0; i < kFill; ++i) {
      const int idx = threadIdx.x + i * kPqThreads;
      fdst[i] = -1;
      if (idx >= n_chunks) continue;
      const int c = idx % (W / 8);
      const int rest = idx / (W / 8);
      const int k = rest % Kpad, m = rest / Kpad;
      fv[i] = bf16x8_t{};
      if (k < K) fv[i] = *reinterpret_cast<const bf16x8_t*>(cb_t + ((size_t)m * K + k) * W + c * 8);
      fdst[i] = ((m * ncb + (k >> 5)) * KSM + (c >> 1)) * 64 + (c & 1) * 32 + (k & 31);
    }
#pragma unroll
    for (int i = 0; i < kFill; ++i)
      if (fdst[i] >= 0) frag[fdst[i]] = fv[i];
    __syncthreads();
    // half squared norms from the staged centroids
    for (int idx = threadIdx.x; idx < M * Kpad; idx += kPqThreads) {
      const int k = idx % Kpad, m = idx / Kpad;
      float h = 3.0e38f;  // padding centroids never win
      if (k < K) {
        float s2 = 0.0f;
        for (int c = 0; c < W / 8; ++c) {
          const bf16x8_t v = frag[((m * ncb + (k >> 5)) * KSM + (c >> 1)) * 64 + (c & 1) * 32 + (k & 31)];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = (float)v[e];
            s2 = __builtin_fmaf(f, f, s2);
          }
        }
        h = 0.5f * s2;
      }
      hn[m * Kpad + k] = h;
    }
    __syncthreads();

    for (int tile = blockIdx.x * kPqWaves + wave; tile < total_tiles;
         tile += gridDim.x * kPqWaves) {
      const int h = tile / tiles_per_head;
      const int r0 = (tile - h * tiles_per_head) * 32;
      const int nrows = a.rows ? a.n_rows[(int64_t)h * a.n_rows_stride] : a.N;
      if (r0 >= nrows) continue;
      const int r = r0 + mrow;
      const bool valid = r < nrows;
      int64_t xrow = valid ? r : r0;
      if (a.rows) xrow = a.rows[(int64_t)h * a.rows_ld + xrow];
      bf16x8_t A[KS];
      const uint16_t* xp = xbase + (int64_t)h * a.sx_h + xrow * a.sx_n + hf * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) A[ks] = *reinterpret_cast<const bf16x8_t*>(xp + ks * 16);

      uint32_t code = 0u;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float best_s = -3.4e38f;
        int best_i = 0x7fffffff;
        for (int cb = 0; cb < ncb; ++cb) {
          const bf16x8_t* fb = frag + (m * ncb + cb) * KSM * 64 + lane;
          f32x16_t acc = {};
#pragma unroll
          for (int ks = 0; ks < KSM; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks * 64], A[m * KSM + ks], acc, 0, 0, 0);
          // register j: centroid cb*32 + 8*(j/4) + 4*hf + j%4 of row mrow
          const float* hb = hn + m * Kpad + cb * 32 + 4 * hf;
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const float4 h4 = *reinterpret_cast<const float4*>(hb + 8 * jg);
            const float hv[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const float s = acc[4 * jg + r4] - hv[r4];
              const int k = cb * 32 + 8 * jg + 4 * hf + r4;
              if (s > best_s || (s == best_s && k < best_i)) {
                best_s = s;
                best_i = k;
              }
            }
          }
        }
        // the other half-wave holds the other 16 centroids of every block
        const float os = __shfl_xor(best_s, 32);
        const int oi = __shfl_xor(best_i, 32);
        if (os > best_s || (os == best_s && oi < best_i)) best_i = oi;
        code |= (uint32_t)best_i << (m * bpm);
      }
      if (hf == 0 && valid) {
        const int64_t col = a.rows ? xrow : (int64_t)r;
        a.codes[((int64_t)h * a.L + t) * a.codes_ld + a.codes_col0 + col] = code;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void pq_f32_kernel(HashArgs a, int64_t total) {
  const float* cbooks = static_cast<const float*>(a.planes);
  const float* xbase = static_cast<const float*>(a.x);
  const int M = a.M, bpm = a.b / a.M, K = 1 << bpm, W = D / a.M;
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
    for (int m = 0; m < M; ++m) {
      double best = 0.0;
      int bi = 0;
      for (int k = 0; k < K; ++k) {
        const float* cp = cbooks + (((int64_t)t * M + m) * K + k) * W;
        double d2 = 0.0;
        for (int f = 0; f < W; ++f) {
          const double df = (double)xp[m * W + f] - (double)cp[f];
          d2 += df * df;
        }
        if (k == 0 || d2 < best) {
          best = d2;
          bi = k;
        }
      }
      code |= (uint32_t)bi << (m * bpm);
    }
    a.codes[((int64_t)h * a.L + t) * a.codes_ld + a.codes_col0 + xrow] = code;
  }
}

template <int D, int M>
hipError_t launch_pq_bf16_m(const HashArgs& a, int tiles_per_head, int total, hipStream_t s) {
  const int K = 1 << (a.b / M);
  const int Kpad = (K + 31) / 32 * 32;
  const size_t lds = (size_t)Kpad * D * 2 + (size_t)M * Kpad * 4;
  auto kern = pq_bf16_kernel<D, M>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  int blocks = (total + kPqWaves - 1) / kPqWaves;
  if (blocks > 512) blocks = 512;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kPqThreads), lds, s, a, tiles_per_head, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pq(const HashArgs& a, bool bf16, hipStream_t s) {
  if (bf16) {
    const int tiles_per_head = (a.N + 31) / 32;
    const int total = a.H * tiles_per_head;
    if (total == 0) return hipSuccess;
    if (a.d == 128) {
      switch (a.M) {
        case 1: return launch_pq_bf16_m<128, 1>(a, tiles_per_head, total, s);
        case 2: return launch_pq_bf16_m<128, 2>(a, tiles_per_head, total, s);
        case 4: return launch_pq_bf16_m<128, 4>(a, tiles_per_head, total, s);
        case 8: return launch_pq_bf16_m<128, 8>(a, tiles_per_head, total, s);
        default: return hipErrorInvalidValue;
      }
    }
    switch (a.M) {
      case 1: return launch_pq_bf16_m<64, 1>(a, tiles_per_head, total, s);
      case 2: return launch_pq_bf16_m<64, 2>(a, tiles_per_head, total, s);
      case 4: return launch_pq_bf16_m<64, 4>(a, tiles_per_head, total, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int64_t total = (int64_t)a.H * a.N * a.L;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (a.d == 128)
    hipLaunchKernelGGL(pq_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  else
    hipLaunchKernelGGL(pq_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

}  // namespace fastar
