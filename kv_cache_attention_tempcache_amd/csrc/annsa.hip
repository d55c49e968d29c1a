// AnnSA over the merged cache (FAST-AR summary, section 2C: the buckets found
// for the cross-attention pruning are reused, and each query attends only to
// the keys of its own bucket(s)).  A query and a slot share a bucket when
// their codes are equal in at least one of L tables; the logit keeps the
// ln(count) shift of the dense step.
//
// The candidates of a query are found through a bucket index of the slots
// (one CSR per table, built by the index kernel over the slots' codes), never
// by comparing all query x slot pairs: the work follows the shared pairs.  A
// group of G lanes owns one query (8 for 2-byte rows, 16 for 4-byte ones), as
// in the match step.  Every table's bucket bounds and first 16 entries load
// up front; the entries whose code equals the query's are listed, each slot
// once, and an online softmax then runs over the list with several slot rows
// in flight.  A query whose list overflows takes a plain second pass instead:
// bucket by bucket, a slot found in table t is dropped if its code of some
// table t' < t equals the query's, and the list is consumed whenever it
// fills.  Both passes take every shared slot exactly once.  Every lane holds
// d/G features of the query, of the running output and of each slot row;
// dot products are summed over the G lanes by DPP moves in binary32.
#include "common.hpp"

#include <cmath>

namespace fastar {
namespace {

constexpr int kCap = 32;   // slots listed before their rows are read
constexpr int kPass = 16;  // bucket entries read per pass of a group

template <int CTRL>
__device__ __forceinline__ float dpp_move_f(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over a query's G lanes (aligned groups of 8 or 16 inside a DPP row);
// each step adds the partner's mirror-image partial sum, so every lane ends
// with the same value.
template <int G>
__device__ __forceinline__ float group_sum_f(float x) {
  static_assert(G == 8 || G == 16, "a query's lanes lie inside one DPP row");
  if constexpr (G == 16) {
    x += dpp_move_f<0x128>(x);  // rotations by 8, 4, 2, 1 within the row
    x += dpp_move_f<0x124>(x);
    x += dpp_move_f<0x122>(x);
    x += dpp_move_f<0x121>(x);
  } else {
    x += dpp_move_f<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_move_f<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp_move_f<0x141>(x);  // row_half_mirror: the other quad
  }
  return x;
}

// E elements of one row as loaded: 2-byte elements as packed pairs, 4-byte
// ones as words; elem() widens element q.
template <typename T, int E>
struct Feats {
  static constexpr int W = sizeof(T) == 2 ? E / 2 : E;
  uint32_t w[W];
};

template <typename T, int E>
__device__ __forceinline__ void load_feats(const T* p, Feats<T, E>& f) {
  constexpr int W = Feats<T, E>::W;
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int c = 0; c < W / 4; ++c) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[c];
      f.w[4 * c] = u.x; f.w[4 * c + 1] = u.y; f.w[4 * c + 2] = u.z; f.w[4 * c + 3] = u.w;
    }
  } else {
    static_assert(W == 2, "row slices are 8 bytes or a multiple of 16");
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    f.w[0] = u.x; f.w[1] = u.y;
  }
}

template <typename T, int E>
__device__ __forceinline__ float elem(const Feats<T, E>& f, int q) {
  if constexpr (sizeof(T) == 2)
    return __uint_as_float((q & 1) ? (f.w[q >> 1] & 0xffff0000u) : (f.w[q >> 1] << 16));
  else
    return __uint_as_float(f.w[q]);
}

template <typename T, int E>
__device__ __forceinline__ void store_feats(T* p, const float (&v)[E]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[E / 2];
#pragma unroll
    for (int k = 0; k < E / 2; ++k)
      w[k] = f32_to_bf16_bits(v[2 * k]) | (f32_to_bf16_bits(v[2 * k + 1]) << 16);
    if constexpr (E % 8 == 0) {
#pragma unroll
      for (int c = 0; c < E / 8; ++c)
        reinterpret_cast<uint4*>(p)[c] = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
    } else {
      *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < E; k += 4)
      *reinterpret_cast<float4*>(p + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  }
}

// c.codes / c.idx_off / c.idx_ent point at the AnnSA slot codes and their
// bucket index; dm.L is the number of AnnSA tables (at most 4).
// G lanes per query; kBatch slot rows in flight together; OCC waves per SIMD;
// kLong: lists expected longer than kCap go straight to the plain pass.
template <typename T, int D, int G, int kBatch, int OCC, bool kLong>
__global__ __launch_bounds__(256, OCC) void annsa_kernel(Dims dm, CacheDev c, AnnsaArgs a) {
  constexpr int E = D / G;
  constexpr int kF = kPass / G;  // entries per lane in a pass
  const int h = blockIdx.y;
  const int i = blockIdx.x * (256 / G) + (threadIdx.x / G);
  const int gl = threadIdx.x & (G - 1);
  if (i >= a.Nq) return;  // all G lanes of a group leave together
  const int L = dm.L, B = dm.B, NB = dm.NB, nb_bits = dm.nb_bits;

  // independent loads first: the query row, its codes, every table's bucket
  // bounds and first kPass entries
  Feats<T, E> qf;
  load_feats<T, E>(static_cast<const T*>(a.q) + (int64_t)h * a.sq_h + (int64_t)i * a.sq_n + gl * E, qf);
  uint32_t qc[4];
  int beg[4], end[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    qc[t] = t < L ? a.q_codes[((int64_t)h * L + t) * a.Nq + i] : 0u;
    beg[t] = end[t] = 0;
    if (t < L) {
      const int32_t* off = c.idx_off + ((int64_t)h * L + t) * (NB + 1) + bucket_of(qc[t], nb_bits);
      beg[t] = off[0];
      end[t] = off[1];
    }
  }
  uint2 first[4][kF];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < kF; ++u) {
      const int p = beg[t] + gl + G * u;
      first[t][u] = (!kLong && t < L && p < end[t]) ? c.idx_ent[((int64_t)h * L + t) * B + p]
                                                    : make_uint2(0u, 0u);
    }
  const float cscale = a.scale * 1.4426950408889634f;  // logits in log2 units
  const T* keys = static_cast<const T*>(c.k_mirror) + (int64_t)h * dm.Bp * D;
  const T* vals = static_cast<const T*>(c.v_mirror) + (int64_t)h * dm.Bp * D;
  const float* lb = c.lb + (int64_t)h * dm.Bp;
  const uint32_t* scodes = c.codes + (int64_t)h * L * B;

  float m = -1e30f, l = 0.0f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.0f;

  // online softmax over list[0..n): the rows of a batch load before any of
  // its arithmetic
  auto consume = [&](const int* list, int n) __attribute__((always_inline)) {
    for (int b0 = 0; b0 < n; b0 += kBatch) {
      // the query is widened per batch instead of being held as E floats
#pragma unroll
      for (int q = 0; q < Feats<T, E>::W; ++q) asm volatile("" : "+v"(qf.w[q]));
      Feats<T, E> kv[kBatch], vv[kBatch];
      float lbs[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int s = list[min(b0 + u, n - 1)];
        load_feats<T, E>(keys + (int64_t)s * D + gl * E, kv[u]);
        load_feats<T, E>(vals + (int64_t)s * D + gl * E, vv[u]);
        lbs[u] = lb[s];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (b0 + u >= n) break;
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) dot = __builtin_fmaf(elem(qf, e), elem(kv[u], e), dot);
        dot = group_sum_f<G>(dot);
        const float z = __builtin_fmaf(dot, cscale, lbs[u]);
        const float mn = fmaxf(m, z);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        const float p = __builtin_amdgcn_exp2f(z - mn);
        l = __builtin_fmaf(l, alpha, p);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(o[e], alpha, p * elem(vv[u], e));
        m = mn;
      }
    }
  };

  // The query's list lives in LDS (every lane of the group writes the same
  // ids, so each lane reads back its own writes).
  __shared__ int s_list[256 / G][kCap];
  int* list = s_list[threadIdx.x / G];
  int n = 0;
  bool full = kLong;
  const int gbase = threadIdx.x & 63 & ~(G - 1);
  constexpr uint32_t gmask = (1u << G) - 1u;
  // lists the matching entries of one pass (kF per lane) of table t, each
  // slot once; a full list stops the listing
  auto list_pass = [&](const uint2 (&e)[kF], int p0, int t) __attribute__((always_inline)) {
    uint32_t mask = 0;
#pragma unroll
    for (int u = 0; u < kF; ++u) {
      const bool ok = p0 + gl + G * u < end[t] && e[u].y == qc[t];
      mask |= ((uint32_t)(__ballot(ok) >> gbase) & gmask) << (G * u);
    }
    while (mask) {
      const int j = __builtin_ctz(mask);
      mask &= mask - 1;
      const int uj = j / G;  // the same in every lane of the group
      int v = (int)e[0].x;
#pragma unroll
      for (int u = 1; u < kF; ++u)
        if (uj == u) v = (int)e[u].x;
      const int sl = __shfl(v, j % G, G);
      bool dup = false;
      for (int k = 0; k < n; ++k) dup |= list[k] == sl;
      if (dup) continue;
      if (n == kCap) {
        full = true;
        break;
      }
      list[n++] = sl;
    }
  };
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (!kLong && t < L) list_pass(first[t], beg[t], t);
  // buckets longer than one pass (rare)
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (kLong || t >= L) break;
    const uint2* ent = c.idx_ent + ((int64_t)h * L + t) * B;
    for (int p0 = beg[t] + kPass; p0 < end[t] && !full; p0 += kPass) {
      uint2 e[kF];
#pragma unroll
      for (int u = 0; u < kF; ++u) {
        const int p = p0 + gl + G * u;
        e[u] = p < end[t] ? ent[p] : make_uint2(0u, 0u);
      }
      list_pass(e, p0, t);
    }
  }
  if (full) {
    // more than kCap shared slots: bucket by bucket, the slot codes of
    // earlier tables decide whether a slot was taken there, and the list is
    // consumed whenever it fills (the code and bucket bounds are read again
    // rather than kept live)
    n = 0;
    for (int t = 0; t < L; ++t) {
      const uint32_t code = a.q_codes[((int64_t)h * L + t) * a.Nq + i];
      const int32_t* off = c.idx_off + ((int64_t)h * L + t) * (NB + 1) + bucket_of(code, nb_bits);
      const int b0 = off[0], b1 = off[1];
      const uint2* ent = c.idx_ent + ((int64_t)h * L + t) * B;
      for (int p0 = b0; p0 < b1; p0 += G) {
        const int p = p0 + gl;
        const uint2 e = p < b1 ? ent[p] : make_uint2(0u, 0u);
        bool ok = p < b1 && e.y == code;
        for (int t2 = 0; t2 < t; ++t2)
          if (ok) ok = scodes[(int64_t)t2 * B + e.x] != a.q_codes[((int64_t)h * L + t2) * a.Nq + i];
        uint32_t mask = (uint32_t)(__ballot(ok) >> gbase) & gmask;
        while (mask) {
          const int j = __builtin_ctz(mask);
          mask &= mask - 1;
          if (n == kCap) {
            consume(list, n);
            n = 0;
          }
          list[n++] = __shfl((int)e.x, j, G);
        }
      }
    }
  }
  if (n) consume(list, n);

  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] *= inv;
  store_feats<T, E>(static_cast<T*>(a.o) + (int64_t)h * a.so_h + (int64_t)i * a.so_n + gl * E, o);
  if (a.lse && gl == 0)
    a.lse[(int64_t)h * a.Nq + i] = l > 0.0f ? (m + __log2f(l)) * 0.6931471805599453f
                                            : -__builtin_huge_valf();
}

}  // namespace

template <typename T, int G, int kBatch, int OCC, bool kLong>
hipError_t launch_annsa_cfg(const Dims& dm, const CacheDev& c, const AnnsaArgs& a, hipStream_t s) {
  const dim3 grid((a.Nq + 256 / G - 1) / (256 / G), dm.H);
  if (dm.d == 128) hipLaunchKernelGGL((annsa_kernel<T, 128, G, kBatch, OCC, kLong>), grid, dim3(256), 0, s, dm, c, a);
  else hipLaunchKernelGGL((annsa_kernel<T, 64, G, kBatch, OCC, kLong>), grid, dim3(256), 0, s, dm, c, a);
  return hipGetLastError();
}

// dm.b: the AnnSA code bits.  Short lists (few random collisions expected:
// L * budget * 2^-b <= 16) take the listing pass with 8 lanes per query and
// one row in flight, so 7 waves of 8 queries fit each SIMD; long lists take
// the plain pass with 16 lanes and four rows in flight, since their time is
// the chain of row loads per query.  4-byte rows take 16 lanes either way.
hipError_t launch_annsa(const Dims& dm, const CacheDev& c, const AnnsaArgs& a, hipStream_t s) {
  if (a.Nq == 0) return hipSuccess;
  const bool long_lists = (double)dm.L * dm.B * std::ldexp(1.0, -dm.b) > 16.0;
  if (dm.elem == 2)
    return long_lists ? launch_annsa_cfg<uint16_t, 16, 4, 4, true>(dm, c, a, s)
                      : launch_annsa_cfg<uint16_t, 8, 1, 7, false>(dm, c, a, s);
  return long_lists ? launch_annsa_cfg<float, 16, 4, 4, true>(dm, c, a, s)
                    : launch_annsa_cfg<float, 16, 2, 5, false>(dm, c, a, s);
}

}  // namespace fastar
