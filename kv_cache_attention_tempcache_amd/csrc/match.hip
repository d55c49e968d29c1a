// Top-1 match of a frame's new keys against the cached slot keys (FAST-AR
// summary, section 2A "Mecanismo": find each current-frame token's nearest
// neighbour among earlier frames through LSH, without full attention matrices).
//
// A group of 16 lanes owns one token.  For every table it reads the token's
// bucket from the CSR index of (slot, code) entries, 16 entries at a time,
// keeps the slots whose code equals the token's code (a bucket may hold several
// codes) and that no earlier table listed, and scores each candidate by the
// cosine of the token key and the slot's stored key, a few candidate rows in
// flight at a time.  A list that overflows is scored and restarted, so a slot
// may then be scored twice, which only costs time.  Products and sums are float64, so the decision agrees
// with an exact evaluation except within ~1e-15 of a tie.  Ties go to the
// lowest slot id; the token merges iff its best cosine >= the threshold.
//
// The traffic is a gather of a handful of random 128- or 256-byte slot rows per
// token: there is no reuse between lanes to stage through LDS, so rows go
// straight from L2/HBM into registers with 8- or 16-byte loads per lane.
#include "common.hpp"

namespace fastar {
namespace {

constexpr int kGroup = 16;  // lanes per token
#ifndef FASTAR_MATCH_MAXCAND
#define FASTAR_MATCH_MAXCAND 8
#endif
#ifndef FASTAR_MATCH_BATCH
#define FASTAR_MATCH_BATCH 2
#endif
#ifndef FASTAR_MATCH_OCC
#define FASTAR_MATCH_OCC 5
#endif

template <typename T, int E>
__device__ __forceinline__ void load_row(const T* p, float (&v)[E]) {
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

// Sum over the 16 lanes of a DPP row (a token's lane group): rotations by 8,
// 4, 2, 1 within the row.  Every lane adds the same two partial sums (in
// commuted order), so all 16 end with the identical value.
template <int R>
__device__ __forceinline__ double row_rotate(double x) {
  const int l = __double2loint(x), h = __double2hiint(x);
  const int lo = __builtin_amdgcn_update_dpp(l, l, 0x120 + R, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(h, h, 0x120 + R, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double group_sum(double x) {
  static_assert(kGroup == 16, "a token's lanes are one DPP row");
  x += row_rotate<8>(x);
  x += row_rotate<4>(x);
  x += row_rotate<2>(x);
  x += row_rotate<1>(x);
  return x;
}

// LT: a bound on the number of tables (sizes the per-table registers)
template <typename T, int D, int LT>
__global__ __launch_bounds__(256, FASTAR_MATCH_OCC) void match_kernel(Dims dm, CacheDev c, MatchArgs a) {
  constexpr int E = D / kGroup;
  constexpr int kMaxCand = FASTAR_MATCH_MAXCAND;  // candidates listed before scoring
  constexpr int kBatch = FASTAR_MATCH_BATCH;  // candidate rows in flight together
  const int h = blockIdx.y;
  const int i = blockIdx.x * (256 / kGroup) + (threadIdx.x / kGroup);
  const int gl = threadIdx.x & (kGroup - 1);
  if (i >= a.T) return;  // all 16 lanes of a group leave together
  const int L = dm.L, B = dm.B, NB = dm.NB, nb_bits = dm.nb_bits;

  // All independent loads first: the token's key, its codes, then every
  // table's bucket bounds and first entry, so the dependent chain per token is
  // codes -> bucket bounds -> entries -> candidate keys.
  float xv[E];
  load_row<T, E>(static_cast<const T*>(a.x) + (int64_t)h * a.sx_h + (int64_t)i * a.sx_n + gl * E,
                 xv);
  uint32_t qc[LT];
#pragma unroll
  for (int t = 0; t < LT; ++t)
    qc[t] = t < L ? a.codes[((int64_t)h * L + t) * a.codes_ld + a.codes_col0 + i] : 0u;
  int beg[LT], end[LT];
#pragma unroll
  for (int t = 0; t < LT; ++t) {
    beg[t] = end[t] = 0;
    if (t < L) {
      const int32_t* off = c.idx_off + ((int64_t)h * L + t) * (NB + 1) + bucket_of(qc[t], nb_bits);
      beg[t] = off[0];
      end[t] = off[1];
    }
  }
  // the first 16 entries of every table's bucket, one per lane, all in flight
  // together (buckets hold a few entries; longer ones are read on in the loop)
  uint2 first[LT];
#pragma unroll
  for (int t = 0; t < LT; ++t)
    first[t] = (t < L && beg[t] + gl < end[t])
                   ? c.idx_ent[((int64_t)h * L + t) * B + beg[t] + gl]
                   : make_uint2(0u, 0u);

  double xd[E];
  double nx2 = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    xd[e] = (double)xv[e];
    nx2 = __builtin_fma(xd[e], xd[e], nx2);
  }
  nx2 = group_sum(nx2);

  const T* keys = static_cast<const T*>(c.k_mirror) + (int64_t)h * dm.Bp * D;
  // Candidates are ranked by key = dot*|dot| / |k|^2, an increasing function
  // of the cosine for a fixed token, compared by cross-multiplication (no
  // division or square root per candidate); ties go to the lower slot.  A
  // zero key row scores cosine 0, i.e. key 0/1.
  double bnum = 0.0, bden = 1.0, bdot = 0.0, bnk2 = 0.0;
  int best_s = -1;
  // score candidates cand[0..n): the row loads of a batch are issued before
  // any of its arithmetic, so one memory round trip serves kBatch candidates
  auto score = [&](const int (&cand)[kMaxCand], int n) __attribute__((always_inline)) {
    for (int b0 = 0; b0 < n; b0 += kBatch) {
      float kv[kBatch][E];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        load_row<T, E>(keys + (int64_t)cand[min(b0 + u, n - 1)] * D + gl * E, kv[u]);
      double dot[kBatch], nk2[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        dot[u] = 0.0;
        nk2[u] = 0.0;
#pragma unroll
        for (int q = 0; q < E; ++q) {
          const double k = (double)kv[u][q];
          dot[u] = __builtin_fma(xd[q], k, dot[u]);
          nk2[u] = __builtin_fma(k, k, nk2[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        dot[u] = group_sum(dot[u]);
        nk2[u] = group_sum(nk2[u]);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (b0 + u >= n) break;
        const int s = cand[b0 + u];
        const bool zero = nx2 == 0.0 || nk2[u] == 0.0;
        const double num = zero ? 0.0 : dot[u] * fabs(dot[u]);
        const double den = zero ? 1.0 : nk2[u];
        const double lhs = num * bden, rhs = bnum * den;
        if (best_s < 0 || lhs > rhs || (lhs == rhs && s < best_s)) {
          bnum = num;
          bden = den;
          bdot = zero ? 0.0 : dot[u];
          bnk2 = nk2[u];
          best_s = s;
        }
      }
    }
  };

  // Candidates: entries of the token's bucket in every table whose code equals
  // the token's, each slot once.  The 16 lanes read 16 entries of a bucket at
  // a time; a ballot over the group lists the matching ones.  The candidate
  // list is identical in every lane of the group.
  int cand[kMaxCand];
  int nc = 0;
  const int gbase = threadIdx.x & 63 & ~(kGroup - 1);
#pragma unroll
  for (int t = 0; t < LT; ++t) {
    if (t >= L) break;
    const uint2* ent = c.idx_ent + ((int64_t)h * L + t) * B;
    for (int p0 = beg[t]; p0 < end[t]; p0 += kGroup) {
      const int p = p0 + gl;
      const uint2 e = p < end[t] ? (p0 == beg[t] ? first[t] : ent[p]) : make_uint2(0u, 0u);
      const bool ok = p < end[t] && e.y == qc[t];
      uint32_t mask = (uint32_t)(__ballot(ok) >> gbase) & 0xffffu;
      while (mask) {
        const int j = __builtin_ctz(mask);
        mask &= mask - 1;
        const int s = __shfl((int)e.x, j, kGroup);
        bool dup = false;
        for (int k = 0; k < nc; ++k) dup |= cand[k] == s;
        if (dup) continue;
        if (nc == kMaxCand) {  // rare: a full list is scored and emptied
          score(cand, nc);
          nc = 0;
        }
        cand[nc++] = s;
      }
    }
  }
  score(cand, nc);
  // the winner's cosine, evaluated once
  const double best = (best_s < 0 || nx2 == 0.0 || bnk2 == 0.0)
                          ? 0.0 : bdot / (sqrt(nx2) * sqrt(bnk2));
  if (gl == 0) {
    const int64_t o = (int64_t)h * B + i;
    c.best_slot[o] = best_s;
    c.best_cos[o] = best_s >= 0 ? (float)best : 0.0f;
    const bool merge = best_s >= 0 && best >= (double)a.tau;
    c.dec[o] = merge ? best_s : -1;
    if (merge) {
      // order-independent: the lowest merging token and the group size
      atomicMin(&c.owner[(int64_t)h * B + best_s], i);
      atomicAdd(&c.gsize[(int64_t)h * B + best_s], 1);
    }
  }
}

}  // namespace

template <int LT>
hipError_t launch_match_lt(const Dims& dm, const CacheDev& c, const MatchArgs& a, hipStream_t s) {
  const dim3 grid((a.T + 15) / 16, dm.H);
  if (dm.elem == 2) {
    if (dm.d == 128) hipLaunchKernelGGL((match_kernel<uint16_t, 128, LT>), grid, dim3(256), 0, s, dm, c, a);
    else hipLaunchKernelGGL((match_kernel<uint16_t, 64, LT>), grid, dim3(256), 0, s, dm, c, a);
  } else {
    if (dm.d == 128) hipLaunchKernelGGL((match_kernel<float, 128, LT>), grid, dim3(256), 0, s, dm, c, a);
    else hipLaunchKernelGGL((match_kernel<float, 64, LT>), grid, dim3(256), 0, s, dm, c, a);
  }
  return hipGetLastError();
}

hipError_t launch_match(const Dims& dm, const CacheDev& c, const MatchArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  static_assert(FASTAR_MAX_TABLES_DEV == 8, "table bounds below");
  return dm.L <= 4 ? launch_match_lt<4>(dm, c, a, s) : launch_match_lt<8>(dm, c, a, s);
}

}  // namespace fastar
