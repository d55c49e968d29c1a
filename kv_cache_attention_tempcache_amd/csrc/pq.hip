// Product-quantization codes (FAST-AR summary, section 2: the nearest-neighbour
// search uses "LSH or quantization"; this is the quantization).  A table splits
// the d features into M equal slices; slice m takes the index of its nearest
// centroid among K = 2^(b/M) (ties to the lowest index), and the b-bit code
// concatenates the slice indices, slice m at bits [m*b/M, (m+1)*b/M).
//
// bf16 path: nearest in Euclidean distance = largest <x, c> - |c|^2/2, so a
// slice's scores are a small GEMM (centroids x slice features) x (slice
// features x rows) on the 32x32x16 bf16 MFMA, centroids as the MFMA rows.
// A workgroup serves one table: it stages that table's codebooks in LDS in
// MFMA operand order (one 1 KiB fragment per 32 centroids and k-step) beside
// the negated half squared norms, which seed the accumulators; each wave then
// takes 32 rows of one slice at a time and keeps, per lane, running maxima of
// scores that carry their centroid's position in their lowest mantissa bits
// (one v_max3 per two scores instead of a compare and two selects each), and
// one exchange with lane^32 settles each slice.  The k-steps read features
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
__global__ __launch_bounds__(kPqThreads, 4) void pq_bf16_kernel(HashArgs a, int tiles_per_head,
                                                                int total_tiles) {
  constexpr int W = D / M;          // features per slice
  constexpr int KSM = W / 16;       // k-steps per slice
  constexpr int CPC = W / 8;        // 16-byte chunks per centroid slice
  static_assert(W % 16 == 0, "slices of whole k-steps");
  extern __shared__ __attribute__((aligned(16))) bf16x8_t frag[];  // [M][NCB][KSM][64]
  const int bpm = a.b / M;          // bits per slice
  const int K = 1 << bpm;
  const int ncb = (K + 31) / 32, Kpad = ncb * 32, lkp = __builtin_ctz(Kpad);
  float* nhn = reinterpret_cast<float*>(frag + (size_t)M * ncb * KSM * 64);  // [M][Kpad]
  const uint16_t* cbooks = static_cast<const uint16_t*>(a.planes);  // [L][M][K][W]
  const uint16_t* xbase = static_cast<const uint16_t*>(a.x);
  const int lane = threadIdx.x & 63;
  // (read into a scalar register: the tile arithmetic below is then scalar)
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int mrow = lane & 31, hf = lane >> 5;
  __shared__ uint32_t s_idx[2][kPqWaves][32];  // slice index of each row, per wave

  const int t = blockIdx.y;  // one table per workgroup row of the grid
  // wave w scores slice m = w % M of tile g*TPB + w/M of group g; the M slice
  // indices of a row meet in LDS and the slice-0 wave writes the code
  constexpr int TPB = kPqWaves / M;  // tiles per group
  const int m = wave % M, tsub = wave / M;
  const int n_groups = (total_tiles + TPB - 1) / TPB;
  const int G = gridDim.x;

  // A group's rows are found in two steps whose loads are issued one group
  // apart: the head's row count and (for a row list) the row's index, then
  // the row's features.  Every load is unconditional and reads a valid
  // address (tiles clamped to the last one, list positions to the list; the
  // direct case reads a dummy word), so no load waits for another.
  const bool indirect = a.rows != nullptr;
  const int* cnt_p = indirect ? a.n_rows : reinterpret_cast<const int*>(cbooks);
  const int* row_p = indirect ? a.rows : reinterpret_cast<const int*>(cbooks);
  struct Idx {
    int cnt, row;
  };
  struct Loc {
    int h, r;
    bool live, valid;
    int64_t xrow;
  };
  auto fetch = [&](int g) {
    const int tile = min(g * TPB + tsub, total_tiles - 1);
    const int h = tile / tiles_per_head;
    const int r = (tile - h * tiles_per_head) * 32 + mrow;
    Idx v;
    v.cnt = cnt_p[indirect ? (int64_t)h * a.n_rows_stride : (int64_t)0];
    v.row = row_p[indirect ? (int64_t)h * a.rows_ld + min((int64_t)r, a.rows_ld - 1) : (int64_t)0];
    return v;
  };
  auto locate = [&](int g, const Idx& v) {
    Loc l;
    const int tile = g * TPB + tsub;
    const int tc = min(tile, total_tiles - 1);
    l.h = tc / tiles_per_head;
    const int r0 = (tc - l.h * tiles_per_head) * 32;
    const int nrows = indirect ? __builtin_amdgcn_readfirstlane(v.cnt) : a.N;  // one per head
    l.r = r0 + mrow;
    l.live = g < n_groups && tile < total_tiles && r0 < nrows;
    l.valid = l.live && l.r < nrows;
    l.xrow = l.valid ? (indirect ? (int64_t)v.row : (int64_t)l.r) : 0;  // row 0: any row
    return l;
  };
  auto load_x = [&](const Loc& l, bf16x8_t (&A)[KSM]) {
    const uint16_t* xp = xbase + (int64_t)l.h * a.sx_h + l.xrow * a.sx_n + hf * 8 + m * W;
#pragma unroll
    for (int ks = 0; ks < KSM; ++ks) A[ks] = *reinterpret_cast<const bf16x8_t*>(xp + ks * 16);
  };

  // the first group's rows are on their way while the codebooks are staged
  int g = blockIdx.x;
  Loc cur = locate(g, fetch(g));
  bf16x8_t A[KSM];
  load_x(cur, A);
  Idx inext = fetch(g + G);

  {
    const uint16_t* cb_t = cbooks + (size_t)t * M * K * W;
    // fragments: chunk c (features 8c..8c+7 of the slice) of centroid k of
    // slice m is k-step c/2, half c%2 of lane 32*(c%2) + k%32 in block k/32.
    // A thread issues all its loads (clamped, always valid addresses) before
    // its first store; the CPC lanes that hold one centroid's chunks sum its
    // squared norm with shuffles.  Padding centroids are zero and score -inf.
    constexpr int kFill = (256 * D / 8 + kPqThreads - 1) / kPqThreads;
    const int n_chunks = M * Kpad * CPC;
    bf16x8_t fv[kFill];
#pragma unroll
    for (int i = 0; i < kFill; ++i) {
      const int idx = min((int)threadIdx.x + i * kPqThreads, n_chunks - 1);
      const int c = idx % CPC, rest = idx / CPC;
      const int k = rest & (Kpad - 1), ms = rest >> lkp;
      fv[i] = *reinterpret_cast<const bf16x8_t*>(cb_t + ((size_t)ms * K + min(k, K - 1)) * W + c * 8);
    }
#pragma unroll
    for (int i = 0; i < kFill; ++i) {
      const int raw = (int)threadIdx.x + i * kPqThreads;
      const int idx = min(raw, n_chunks - 1);
      const int c = idx % CPC, rest = idx / CPC;
      const int k = rest & (Kpad - 1), ms = rest >> lkp;
      float s2 = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (float)fv[i][e];
        s2 = __builtin_fmaf(f, f, s2);
      }
#pragma unroll
      for (int o = 1; o < CPC; o <<= 1) s2 += __shfl_xor(s2, o);
      if (raw < n_chunks) {
        const bool pad = k >= K;
        frag[((ms * ncb + (k >> 5)) * KSM + (c >> 1)) * 64 + (c & 1) * 32 + (k & 31)] =
            pad ? bf16x8_t{} : fv[i];
        if (c == 0) nhn[ms * Kpad + k] = pad ? -3.0e38f : -0.5f * s2;
      }
    }
    __syncthreads();
  }

  // a group's codes are stored in the next pass of the loop, after that
  // pass's loads: their waits then never include a store just issued
  bool pend = false;
  int64_t pend_at = 0;
  uint32_t pend_code = 0u;
  for (int buf = 0; g < n_groups; g += G, buf ^= 1) {  // uniform per block
    // next group's rows, and the one after's indices, in flight meanwhile
    const Loc nxt = locate(g + G, inext);
    bf16x8_t An[KSM];
    load_x(nxt, An);
    inext = fetch(g + 2 * G);
    if (pend) a.codes[pend_at] = pend_code;
    if (cur.live) {
      // The accumulators start at -|c|^2/2, so the MFMAs leave the scores.
      // Each register keeps a running maximum over the blocks of its
      // scores with the three lowest mantissa bits replaced by 7 - block,
      // two blocks per v_max3.  Scores that agree above those bits (2^-20
      // of their size, below the fp32 rounding of the dot product) thus go
      // to the lower block, i.e. the lower centroid index, when positive
      // (negative ones order the codes the other way round).
      float bs[16];
      const bf16x8_t* fm = frag + m * ncb * KSM * 64 + lane;
      const float* hm = nhn + m * Kpad + 4 * hf;
      auto scores = [&](int cb) {
        const float* hb = hm + cb * 32;
        f32x16_t acc;
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const float4 h4 = *reinterpret_cast<const float4*>(hb + 8 * jg);
          acc[4 * jg + 0] = h4.x;
          acc[4 * jg + 1] = h4.y;
          acc[4 * jg + 2] = h4.z;
          acc[4 * jg + 3] = h4.w;
        }
        const bf16x8_t* fb = fm + cb * KSM * 64;
#pragma unroll
        for (int ks = 0; ks < KSM; ++ks)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks * 64], A[ks], acc, 0, 0, 0);
        return acc;
      };
      auto coded = [](float v, uint32_t code) {
        return __uint_as_float((__float_as_uint(v) & ~7u) | code);
      };
      // ncb is 1 or even; the first blocks seed the maxima (every maximum
      // is written as fmax(x, fmax(y, z)), which becomes one v_max3)
      constexpr float kFloor = -3.4e38f;
      {
        const f32x16_t s0 = scores(0);
        if (ncb == 1) {
#pragma unroll
          for (int j = 0; j < 16; ++j) bs[j] = coded(s0[j], 7u);
        } else {
          const f32x16_t s1 = scores(1);
#pragma unroll
          for (int j = 0; j < 16; ++j)
            bs[j] = __builtin_fmaxf(kFloor, __builtin_fmaxf(coded(s0[j], 7u), coded(s1[j], 6u)));
        }
      }
      for (int cb = 2; cb < ncb; cb += 2) {
        const f32x16_t s0 = scores(cb), s1 = scores(cb + 1);
        const uint32_t c0 = 7u - (uint32_t)cb, c1 = c0 - 1u;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          bs[j] = __builtin_fmaxf(bs[j], __builtin_fmaxf(coded(s0[j], c0), coded(s1[j], c1)));
      }
      // the 16 registers (equal coded scores share a block, so the lower
      // register is the lower index), then the other half-wave (the other
      // 16 centroids of every block)
      float best_s = bs[0];
      int best_j = 0;
#pragma unroll
      for (int j = 1; j < 16; ++j) {
        const bool up = bs[j] > best_s;
        best_s = up ? bs[j] : best_s;
        best_j = up ? j : best_j;
      }
      int best_i = (7 - (int)(__float_as_uint(best_s) & 7u)) * 32 + 8 * (best_j >> 2) + 4 * hf +
                   (best_j & 3);
      const float os = __shfl_xor(best_s, 32);
      const int oi = __shfl_xor(best_i, 32);
      if (os > best_s || (os == best_s && oi < best_i)) best_i = oi;
      if (hf == 0) s_idx[buf][wave][mrow] = (uint32_t)best_i;
    }
    // one barrier a group: the other buffer is rewritten only after the
    // next barrier, which every reader of this one has passed
    __syncthreads();
    pend = m == 0 && hf == 0 && cur.valid;
    if (pend) {
      pend_code = 0u;
#pragma unroll
      for (int mm = 0; mm < M; ++mm) pend_code |= s_idx[buf][tsub * M + mm][mrow] << (mm * bpm);
      const int64_t col = indirect ? cur.xrow : (int64_t)cur.r;
      pend_at = ((int64_t)cur.h * a.L + t) * a.codes_ld + a.codes_col0 + col;
    }
    cur = nxt;
#pragma unroll
    for (int ks = 0; ks < KSM; ++ks) A[ks] = An[ks];
  }
  if (pend) a.codes[pend_at] = pend_code;
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
  // one round of workgroups (two per CU fit in LDS): each stages its
  // table's codebooks once and loops over groups of tiles
  const int cap = a.L >= 512 ? 1 : 512 / a.L;
  int blocks = (total + kPqWaves / M - 1) / (kPqWaves / M);
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(kern, dim3(blocks, a.L), dim3(kPqThreads), lds, s, a, tiles_per_head, total);
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
