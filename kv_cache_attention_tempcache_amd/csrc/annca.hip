// AnnCA prompt-token selection (FAST-AR summary, section 2B "Mecanismo":
// latent queries and prompt keys share one hashed space; a prompt token is
// kept for a frame iff it shares a bucket with at least one of the frame's
// queries; the rest are pruned for that frame).
//
// One workgroup per (head, frame).  Codes of at most 16 bits (the AnnCA
// tables) use one 2^16-bit LDS bitmap per table: every table's query codes set
// their bits in one pass, every prompt code tests its bit in a second.  A
// workgroup that meets a wider query code falls back to an open-addressing
// set per table.  The kept ids are compacted in ascending order.
#include <algorithm>

#include "common.hpp"

namespace fastar {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBitmapWords = (1 << 16) / 32;  // one bit per 16-bit code

__global__ __launch_bounds__(kSelThreads) void annca_select_kernel(SelectArgs a, int tbits,
                                                                   size_t set_bytes) {
  extern __shared__ __attribute__((aligned(16))) unsigned long long smem[];
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem);                   // [L][kBitmapWords]
  unsigned long long* tab = smem;                                     // fallback set, same bytes
  uint8_t* keep = reinterpret_cast<uint8_t*>(smem) + set_bytes;       // [Np]
  __shared__ int s_scan[kSelWaves];
  __shared__ int s_wide;
  const int TS = 1 << tbits;
  const int hg = blockIdx.x;
  const int h = hg / a.F, g = hg - h * a.F;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = a.L, Nf = a.Nf, Np = a.Np;
  const int64_t q_ld = (int64_t)a.F * Nf;
  const uint32_t* qc0 = a.q_codes + (int64_t)h * L * q_ld + (int64_t)g * Nf;
  const uint32_t* pc0 = a.p_codes + (int64_t)h * L * Np;

  for (int i = tid; i < L * kBitmapWords; i += kSelThreads) bm[i] = 0u;
  for (int j = tid; j < Np; j += kSelThreads) keep[j] = 0;
  if (tid == 0) s_wide = 0;
  __syncthreads();
  // every table's query codes into its bitmap
  for (int idx = tid; idx < L * Nf; idx += kSelThreads) {
    const int t = idx / Nf, i = idx - t * Nf;
    const uint32_t code = qc0[(int64_t)t * q_ld + i];
    if (code >> 16) s_wide = 1;
    else atomicOr(&bm[t * kBitmapWords + (code >> 5)], 1u << (code & 31u));
  }
  __syncthreads();
  if (!s_wide) {
    for (int idx = tid; idx < L * Np; idx += kSelThreads) {
      const int t = idx / Np, j = idx - t * Np;
      const uint32_t code = pc0[(int64_t)t * Np + j];
      if ((code >> 16) == 0u && ((bm[t * kBitmapWords + (code >> 5)] >> (code & 31u)) & 1u))
        keep[j] = 1;
    }
  } else {
    for (int t = 0; t < L; ++t) {
      for (int i = tid; i < TS; i += kSelThreads) tab[i] = 0ull;
      __syncthreads();
      const uint32_t* qc = qc0 + (int64_t)t * q_ld;
      for (int i = tid; i < Nf; i += kSelThreads) {
        const uint32_t code = qc[i];
        const unsigned long long ent = (1ull << 32) | code;
        uint32_t pos = bucket_of(code, tbits);
        while (true) {
          const unsigned long long old = atomicCAS(&tab[pos], 0ull, ent);
          if (old == 0ull || old == ent) break;
          pos = (pos + 1) & (TS - 1);
        }
      }
      __syncthreads();
      const uint32_t* pc = pc0 + (int64_t)t * Np;
      for (int j = tid; j < Np; j += kSelThreads) {
        const uint32_t code = pc[j];
        const unsigned long long ent = (1ull << 32) | code;
        uint32_t pos = bucket_of(code, tbits);
        while (true) {
          const unsigned long long e = tab[pos];
          if (e == 0ull) break;
          if (e == ent) {
            keep[j] = 1;
            break;
          }
          pos = (pos + 1) & (TS - 1);
        }
      }
      __syncthreads();
    }
  }
  __syncthreads();
  // compact the kept ids (each thread owns a contiguous run of prompt ids)
  const int per = (Np + kSelThreads - 1) / kSelThreads;
  const int lo = min(Np, tid * per), hi = min(Np, lo + per);
  int c = 0;
  for (int j = lo; j < hi; ++j) c += (int)keep[j];
  int x = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_scan[w] = x;
  __syncthreads();
  if (w == 0) {
    int sv = lane < kSelWaves ? s_scan[lane] : 0;
#pragma unroll
    for (int o = 1; o < kSelWaves; o <<= 1) {
      const int y = __shfl_up(sv, o, 64);
      if (lane >= o) sv += y;
    }
    if (lane < kSelWaves) s_scan[lane] = sv;
  }
  __syncthreads();
  int pos = (w ? s_scan[w - 1] : 0) + x - c;
  int32_t* out = a.sel_idx + (int64_t)hg * Np;
  for (int j = lo; j < hi; ++j)
    if (keep[j]) out[pos++] = j;
  if (tid == 0) a.sel_count[hg] = s_scan[kSelWaves - 1];
}

}  // namespace

hipError_t launch_annca_select(const SelectArgs& a, hipStream_t s) {
  int tbits = 1;
  while ((1 << tbits) < 2 * a.Nf) ++tbits;
  const size_t set_bytes = std::max((size_t)a.L * kBitmapWords * 4, ((size_t)1 << tbits) * 8);
  const size_t lds = set_bytes + (((size_t)a.Np + 15) & ~(size_t)15);
  hipError_t e = hipFuncSetAttribute((const void*)annca_select_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(annca_select_kernel, dim3(a.H * a.F), dim3(kSelThreads), lds, s, a, tbits,
                     set_bytes);
  return hipGetLastError();
}

}  // namespace fastar
