// AnnSA over the merged cache (FAST-AR summary, section 2C: the buckets found
// for the cross-attention pruning are reused, and each query attends only to
// the keys of its own bucket(s)).  A query and a slot share a bucket when
// their codes are equal in at least one of L tables; the logit keeps the
// ln(count) shift of the dense step.
//
// The candidates of a query are found through a bucket index of the slots
// (one CSR per table, built by the index kernel over the slots' codes), never
// by comparing all query x slot pairs: the work follows the shared pairs.  A
// group of 16 lanes owns one query, as in the match step: for every table it
// reads its bucket 16 entries at a time, keeps the entries whose code equals
// the query's and that no earlier table already shares (a slot found in
// table t is dropped if its code of some table t' < t equals the query's),
// and runs an online softmax over the kept slots, several slot rows in flight
// at a time.  Every lane holds d/16 features of the query, of the running
// output and of each slot row; dot products are summed over the 16 lanes by
// DPP row rotations in binary32.
#include "common.hpp"

namespace fastar {
namespace {

constexpr int kGroup = 16;     // lanes per query
constexpr int kMaxList = 8;    // slots listed before their rows are read
constexpr int kBatch = 4;      // slot rows in flight together

template <int R>
__device__ __forceinline__ float row_rotate_f(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x120 + R, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a DPP row; every lane ends with the same value.
__device__ __forceinline__ float group_sum_f(float x) {
  x += row_rotate_f<8>(x);
  x += row_rotate_f<4>(x);
  x += row_rotate_f<2>(x);
  x += row_rotate_f<1>(x);
  return x;
}

template <typename T, int E>
__device__ __forceinline__ void load_feats(const T* p, float (&v)[E]) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (E == 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      v[0] = __uint_as_float(u.x << 16);
      v[1] = __uint_as_float(u.x & 0xffff0000u);
      v[2] = __uint_as_float(u.y << 16);
      v[3] = __uint_as_float(u.y & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < E; k += 4) {
      const float4 f = *reinterpret_cast<const float4*>(p + k);
      v[k] = f.x;
      v[k + 1] = f.y;
      v[k + 2] = f.z;
      v[k + 3] = f.w;
    }
  }
}

template <typename T, int E>
__device__ __forceinline__ void store_feats(T* p, const float (&v)[E]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[E / 2];
#pragma unroll
    for (int k = 0; k < E / 2; ++k)
      w[k] = f32_to_bf16_bits(v[2 * k]) | (f32_to_bf16_bits(v[2 * k + 1]) << 16);
    if constexpr (E == 8) *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    else *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int k = 0; k < E; k += 4)
      *reinterpret_cast<float4*>(p + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  }
}

// c.codes / c.idx_off / c.idx_ent point at the AnnSA slot codes and their
// bucket index; dm.L is the number of AnnSA tables.
template <typename T, int D>
__global__ __launch_bounds__(256) void annsa_kernel(Dims dm, CacheDev c, AnnsaArgs a) {
  constexpr int E = D / kGroup;
  const int h = blockIdx.y;
  const int i = blockIdx.x * (256 / kGroup) + (threadIdx.x / kGroup);
  const int gl = threadIdx.x & (kGroup - 1);
  if (i >= a.Nq) return;  // all 16 lanes of a group leave together
  const int L = dm.L, B = dm.B, NB = dm.NB, nb_bits = dm.nb_bits;

  float qv[E];
  load_feats<T, E>(static_cast<const T*>(a.q) + (int64_t)h * a.sq_h + (int64_t)i * a.sq_n + gl * E, qv);
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
  auto consume = [&](const int (&list)[kMaxList], int n) __attribute__((always_inline)) {
    for (int b0 = 0; b0 < n; b0 += kBatch) {
      float kv[kBatch][E], vv[kBatch][E], lbs[kBatch];
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
        for (int e = 0; e < E; ++e) dot = __builtin_fmaf(qv[e], kv[u][e], dot);
        dot = group_sum_f(dot);
        const float z = __builtin_fmaf(dot, cscale, lbs[u]);
        const float mn = fmaxf(m, z);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        const float p = __builtin_amdgcn_exp2f(z - mn);
        l = __builtin_fmaf(l, alpha, p);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(o[e], alpha, p * vv[u][e]);
        m = mn;
      }
    }
  };

  int list[kMaxList];
  int n = 0;
  const int gbase = threadIdx.x & 63 & ~(kGroup - 1);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t >= L) break;
    const uint2* ent = c.idx_ent + ((int64_t)h * L + t) * B;
    for (int p0 = beg[t]; p0 < end[t]; p0 += kGroup) {
      const int p = p0 + gl;
      const uint2 e = p < end[t] ? ent[p] : make_uint2(0u, 0u);
      bool ok = p < end[t] && e.y == qc[t];
      // a slot sharing an earlier table's bucket was already taken there
#pragma unroll
      for (int t2 = 0; t2 < t; ++t2)
        if (ok) ok = scodes[(int64_t)t2 * B + e.x] != qc[t2];
      uint32_t mask = (uint32_t)(__ballot(ok) >> gbase) & 0xffffu;
      while (mask) {
        const int j = __builtin_ctz(mask);
        mask &= mask - 1;
        if (n == kMaxList) {
          consume(list, n);
          n = 0;
        }
        list[n++] = __shfl((int)e.x, j, kGroup);
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

hipError_t launch_annsa(const Dims& dm, const CacheDev& c, const AnnsaArgs& a, hipStream_t s) {
  if (a.Nq == 0) return hipSuccess;
  const dim3 grid((a.Nq + 15) / 16, dm.H);
  if (dm.elem == 2) {
    if (dm.d == 128) hipLaunchKernelGGL((annsa_kernel<uint16_t, 128>), grid, dim3(256), 0, s, dm, c, a);
    else hipLaunchKernelGGL((annsa_kernel<uint16_t, 64>), grid, dim3(256), 0, s, dm, c, a);
  } else {
    if (dm.d == 128) hipLaunchKernelGGL((annsa_kernel<float, 128>), grid, dim3(256), 0, s, dm, c, a);
    else hipLaunchKernelGGL((annsa_kernel<float, 64>), grid, dim3(256), 0, s, dm, c, a);
  }
  return hipGetLastError();
}

}  // namespace fastar
