// Bucket index over the live slots, rebuilt after every frame (the candidate
// sets of the next frame's match must reflect merged and inserted slots).
//
// One workgroup per (head, table): LDS atomics give the bucket sizes and each
// slot's position inside its bucket in one pass; an exclusive scan turns the
// sizes into CSR offsets, written out as one coalesced copy; each slot then
// places its (slot, code) entry at its position in an LDS staging array (the
// whole table at once when it fits, else in chunks of positions), which is
// written out coalesced, so the scattered 8-byte stores stay in LDS.  The
// order inside a bucket depends on atomic timing, which does not matter: the
// match reads every entry of a bucket and breaks ties on the slot id.
#include "common.hpp"

namespace fastar {
namespace {

constexpr int kIdxThreads = 1024;
constexpr int kIdxWaves = kIdxThreads / kWave;

// Slots handled per thread: B <= kIdxThreads * kIdxPer.
constexpr int kIdxPer = (FASTAR_MAX_BUDGET + kIdxThreads - 1) / kIdxThreads;

// Dynamic LDS of the kernel: bucket counters, scan partials, then the
// staging array of as many entries as fit.
constexpr int kIdxLds = 150 * 1024;

__device__ __forceinline__ int idx_stage_cap(int NB) { return (kIdxLds - NB * 4 - kIdxWaves * 4) / 8; }

__global__ __launch_bounds__(kIdxThreads) void index_kernel(Dims dm, CacheDev c, int bump_frame) {
  extern __shared__ __attribute__((aligned(16))) uint32_t cnt[];  // [NB], [kIdxWaves], staging
  uint32_t* s_scan = cnt + dm.NB;
  // NB >= 64 is a power of two, so the staging array is 8-byte aligned
  uint2* stage = reinterpret_cast<uint2*>(s_scan + kIdxWaves);
  const int ht = blockIdx.x;
  const int h = ht / dm.L;
  const int n = c.n_live[h];
  const int NB = dm.NB, B = dm.B;
  const int cap = idx_stage_cap(NB);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t* codes = c.codes + (int64_t)ht * B;
  int32_t* off = c.idx_off + (int64_t)ht * (NB + 1);
  uint2* ent = c.idx_ent + (int64_t)ht * B;

  for (int i = tid; i < NB; i += kIdxThreads) cnt[i] = 0u;
  uint32_t code[kIdxPer], pos[kIdxPer];
#pragma unroll
  for (int k = 0; k < kIdxPer; ++k) {
    const int s = tid + k * kIdxThreads;
    code[k] = s < n ? codes[s] : 0u;
  }
  __syncthreads();
  // one atomic pass: bucket sizes and each slot's position inside its bucket
#pragma unroll
  for (int k = 0; k < kIdxPer; ++k) {
    const int s = tid + k * kIdxThreads;
    if (s < n) pos[k] = atomicAdd(&cnt[bucket_of(code[k], dm.nb_bits)], 1u);
  }
  __syncthreads();

  // exclusive scan of cnt: each thread owns a contiguous run of buckets
  const int per = (NB + kIdxThreads - 1) / kIdxThreads;
  const int lo = min(NB, tid * per), hi = min(NB, lo + per);
  uint32_t sum = 0u;
  for (int i = lo; i < hi; ++i) sum += cnt[i];
  uint32_t x = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_scan[w] = x;
  __syncthreads();
  if (w == 0) {
    uint32_t sv = lane < kIdxWaves ? s_scan[lane] : 0u;
#pragma unroll
    for (int o = 1; o < kIdxWaves; o <<= 1) {
      const uint32_t y = __shfl_up(sv, o, 64);
      if (lane >= o) sv += y;
    }
    if (lane < kIdxWaves) s_scan[lane] = sv;
  }
  __syncthreads();
  uint32_t run = (w ? s_scan[w - 1] : 0u) + x - sum;
  for (int i = lo; i < hi; ++i) {
    const uint32_t cc = cnt[i];
    cnt[i] = run;
    run += cc;
  }
  __syncthreads();
  for (int i = tid; i < NB; i += kIdxThreads) off[i] = (int32_t)cnt[i];
  if (tid == 0) off[NB] = n;
  // final positions, then the entries through the staging array
#pragma unroll
  for (int k = 0; k < kIdxPer; ++k) {
    const int s = tid + k * kIdxThreads;
    pos[k] = s < n ? cnt[bucket_of(code[k], dm.nb_bits)] + pos[k] : 0xffffffffu;
  }
  for (int base = 0; base < n; base += cap) {
    const uint32_t len = (uint32_t)min(cap, n - base);
#pragma unroll
    for (int k = 0; k < kIdxPer; ++k) {
      const uint32_t r = pos[k] - (uint32_t)base;  // wraps below the chunk's start
      if (r < len) stage[r] = make_uint2((uint32_t)(tid + k * kIdxThreads), code[k]);
    }
    __syncthreads();
    for (int i = tid; i < (int)len; i += kIdxThreads) ent[base + i] = stage[i];
    __syncthreads();
  }
  if (bump_frame && ht == 0 && tid == 0) *c.frame += 1;
}

}  // namespace

hipError_t launch_index(const Dims& dm, const CacheDev& c, bool bump_frame, hipStream_t s) {
  // at the largest budget (32768 slots, 8192 buckets) the counters take 32 KiB
  // and the staging array holds 15096 entries, so three chunks
  static_assert(kIdxLds - FASTAR_MAX_BUDGET / kSlotsPerBucket * 4 - kIdxWaves * 4 >= 8 * 4096,
                "the staging array holds at least 4096 entries at every budget");
  hipError_t e = hipFuncSetAttribute((const void*)index_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kIdxLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(index_kernel, dim3(dm.H * dm.L), dim3(kIdxThreads), kIdxLds, s, dm, c,
                     bump_frame ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fastar
