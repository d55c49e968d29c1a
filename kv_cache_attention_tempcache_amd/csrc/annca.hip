// AnnCA prompt-token selection (FAST-AR summary, section 2B "Mecanismo":
// latent queries and prompt keys share one hashed space; a prompt token is
// kept for a frame iff it shares a bucket with at least one of the frame's
// queries; the rest are pruned for that frame).
//
// One workgroup per (head, frame).  For each table, the frame's query codes go
// into an open-addressing set in LDS; each prompt code is then looked up and
// marks its token kept.  The kept ids are compacted in ascending order.
#include "common.hpp"

namespace fastar {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

__global__ __launch_bounds__(kSelThreads) void annca_select_kernel(SelectArgs a, int tbits) {
  extern __shared__ __attribute__((aligned(16))) unsigned long long tab[];
  const int TS = 1 << tbits;
  uint32_t* keep = reinterpret_cast<uint32_t*>(tab + TS);  // [Np]
  int* s_scan = reinterpret_cast<int*>(keep + a.Np);        // [kSelWaves]
  const int hg = blockIdx.x;
  const int h = hg / a.F, g = hg - h * a.F;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int j = tid; j < a.Np; j += kSelThreads) keep[j] = 0u;
  for (int t = 0; t < a.L; ++t) {
    for (int i = tid; i < TS; i += kSelThreads) tab[i] = 0ull;
    __syncthreads();
    const uint32_t* qc = a.q_codes + ((int64_t)h * a.L + t) * ((int64_t)a.F * a.Nf) + (int64_t)g * a.Nf;
    for (int i = tid; i < a.Nf; i += kSelThreads) {
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
    const uint32_t* pc = a.p_codes + ((int64_t)h * a.L + t) * a.Np;
    for (int j = tid; j < a.Np; j += kSelThreads) {
      const uint32_t code = pc[j];
      const unsigned long long ent = (1ull << 32) | code;
      uint32_t pos = bucket_of(code, tbits);
      while (true) {
        const unsigned long long e = tab[pos];
        if (e == 0ull) break;
        if (e == ent) {
          keep[j] = 1u;
          break;
        }
        pos = (pos + 1) & (TS - 1);
      }
    }
    __syncthreads();
  }
  // compact the kept ids (each thread owns a contiguous run of prompt ids)
  const int per = (a.Np + kSelThreads - 1) / kSelThreads;
  const int lo = min(a.Np, tid * per), hi = min(a.Np, lo + per);
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
  int32_t* out = a.sel_idx + (int64_t)hg * a.Np;
  for (int j = lo; j < hi; ++j)
    if (keep[j]) out[pos++] = j;
  if (tid == 0) a.sel_count[hg] = s_scan[kSelWaves - 1];
}

}  // namespace

hipError_t launch_annca_select(const SelectArgs& a, hipStream_t s) {
  int tbits = 1;
  while ((1 << tbits) < 2 * a.Nf) ++tbits;
  const size_t lds = ((size_t)1 << tbits) * 8 + (size_t)a.Np * 4 + kSelWaves * 4 + 16;
  hipError_t e = hipFuncSetAttribute((const void*)annca_select_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(annca_select_kernel, dim3(a.H * a.F), dim3(kSelThreads), lds, s, a, tbits);
  return hipGetLastError();
}

}  // namespace fastar
