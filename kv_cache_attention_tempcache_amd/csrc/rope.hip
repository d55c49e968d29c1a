// Rotated keys of the M-degree attention (LIPAR summary, section 2B
// "Recuperação de Atenção", 1. "Aproximação de Grau-M": a group's exponential
// sum from its m most recent tokens, corrected for the rotary embedding; the
// groups here are the TempCache slots of section 2A).
//
// Region r (r < m) of head h holds, for each live slot s, its key rotated to
// the frame of its (r+1)-th most recent member, R(t_r) k_hat, in bf16, and the
// shift log2(count / m') with m' = min(m, count); rows r >= m' and rows past
// n_live (up to the next multiple of 64, the attention's key tile) get a zero
// key and a -inf shift.  R(t) turns features (2p, 2p+1), p < rope_dims/2, by
// t * base^(-2p/rope_dims).  One 16-lane group per row, each lane 8 (d = 128)
// or 4 (d = 64) consecutive features, so every rotated pair is in one lane.
#include "common.hpp"

namespace fastar {
namespace {

constexpr int kRxGroup = 16;
constexpr int kRxThreads = 256;
constexpr int kRxTile = 64;  // the attention's key tile

template <int D>
__global__ __launch_bounds__(kRxThreads) void rope_expand_kernel(Dims dm, CacheDev c, int m,
                                                                 int rope_dims, float log2_base) {
  constexpr int E = D / kRxGroup;
  static_assert(E % 2 == 0, "rotated pairs stay within a lane");
  const int h = blockIdx.y;
  const int item = blockIdx.x * (kRxThreads / kRxGroup) + threadIdx.x / kRxGroup;
  const int gl = threadIdx.x & (kRxGroup - 1);
  const int n = c.n_live[h];
  const int rows = (n + kRxTile - 1) / kRxTile * kRxTile;  // <= Bp
  if (item >= m * rows) return;
  const int r = item / rows, s = item - r * rows;
  const int64_t orow = ((int64_t)h * dm.R + r) * dm.Bp + s;
  uint16_t* out = static_cast<uint16_t*>(c.rope_k) + orow * D + gl * E;
  int cnt = 0, mm = 0;
  if (s < n) {
    cnt = c.count[(int64_t)h * dm.B + s];
    mm = min(m, cnt);
  }
  uint32_t packed[E / 2];
  if (r < mm) {
    const float t = (float)c.hist[((int64_t)h * dm.B + s) * dm.R + r];
    const uint16_t* kp = static_cast<const uint16_t*>(c.k_mirror) + ((int64_t)h * dm.Bp + s) * D + gl * E;
    uint32_t w[4] = {0u, 0u, 0u, 0u};  // the lane's E bf16 features, two per word
    if constexpr (E == 8) {
      const uint4 raw = *reinterpret_cast<const uint4*>(kp);
      w[0] = raw.x, w[1] = raw.y, w[2] = raw.z, w[3] = raw.w;
    } else {
      const uint2 raw = *reinterpret_cast<const uint2*>(kp);
      w[0] = raw.x, w[1] = raw.y;
    }
#pragma unroll
    for (int q = 0; q < E / 2; ++q) {
      float a = bf16_bits_to_f32(w[q] & 0xffffu), b = bf16_bits_to_f32(w[q] >> 16);
      const int p = (gl * E) / 2 + q;  // pair index within the head
      if (2 * p < rope_dims) {
        const float ang = t * exp2f(-2.0f * (float)p / (float)rope_dims * log2_base);
        float sn, cs;
        sincosf(ang, &sn, &cs);
        const float ra = a * cs - b * sn;
        const float rb = a * sn + b * cs;
        a = ra;
        b = rb;
      }
      packed[q] = f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
    }
  } else {
#pragma unroll
    for (int q = 0; q < E / 2; ++q) packed[q] = 0u;
  }
  if constexpr (E == 8) {
    *reinterpret_cast<uint4*>(out) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  } else {
    *reinterpret_cast<uint2*>(out) = make_uint2(packed[0], packed[1]);
  }
  if (gl == 0)
    c.rope_lb[orow] = r < mm ? __log2f((float)cnt / (float)mm) : -__builtin_huge_valf();
}

}  // namespace

hipError_t launch_rope_expand(const Dims& dm, const CacheDev& c, int m, int rope_dims,
                              float rope_base, hipStream_t s) {
  const int per_block = kRxThreads / kRxGroup;
  const int blocks = (m * dm.Bp + per_block - 1) / per_block;
  const float lb = std::log2(rope_base);
  if (dm.d == 128)
    hipLaunchKernelGGL(rope_expand_kernel<128>, dim3(blocks, dm.H), dim3(kRxThreads), 0, s, dm, c,
                       m, rope_dims, lb);
  else
    hipLaunchKernelGGL(rope_expand_kernel<64>, dim3(blocks, dm.H), dim3(kRxThreads), 0, s, dm, c,
                       m, rope_dims, lb);
  return hipGetLastError();
}

}  // namespace fastar
