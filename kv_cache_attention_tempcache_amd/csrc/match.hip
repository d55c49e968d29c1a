// Top-1 match of a frame's new keys against the cached slot keys (FAST-AR
// summary, section 2A "Mecanismo": find each current-frame token's nearest
// neighbour among earlier frames through LSH, without full attention matrices).
//
// A group of G lanes owns one token (8 for 2-byte keys, 16 for 4-byte ones).
// For every table it reads the token's bucket from the CSR index of
// (slot, code) entries, 16 entries per pass, keeps the slots whose code equals
// the token's code (a bucket may hold several codes) and that no earlier table
// listed, and scores each candidate by the cosine of the token key and the
// slot's stored key.  Products and sums are float64, so the decision agrees
// with an exact evaluation except within ~1e-15 of a tie.  Ties go to the
// lowest slot id; the token merges iff its best cosine >= the threshold.
//
// The traffic is a gather of a handful of random 128- or 256-byte slot rows per
// token: there is no reuse between lanes to stage through LDS, so rows go
// straight from L2/HBM into registers with 16-byte loads.  The kernel is bound
// by the latency of its dependent loads (codes -> bucket bounds -> entries ->
// candidate rows), so what counts is how many tokens are in flight: 8 lanes
// per token and ~70 registers per lane keep 7 waves of 8 tokens on every SIMD
// (16 lanes per token at 5 waves took 1.8x as long at 144k tokens per frame).
#include "common.hpp"

namespace fastar {
namespace {

#ifndef FASTAR_MATCH_MAXCAND
#define FASTAR_MATCH_MAXCAND 8
#endif
#ifndef FASTAR_MATCH_BATCH
#define FASTAR_MATCH_BATCH 1
#endif
#ifndef FASTAR_MATCH_OCC
#define FASTAR_MATCH_OCC 7
#endif
#ifndef FASTAR_MATCH_GROUP_BF16
#define FASTAR_MATCH_GROUP_BF16 8
#endif
#ifndef FASTAR_MATCH_FIRST
#define FASTAR_MATCH_FIRST 16
#endif

// One row slice of E elements per lane, kept as loaded: 2-byte keys as packed
// pairs (E/2 words), 4-byte keys as E words.  elem() widens element q.
template <typename T, int E>
struct RowSlice {
  static constexpr int W = sizeof(T) == 2 ? E / 2 : E;
  uint32_t w[W];
};

template <typename T, int E>
__device__ __forceinline__ void load_row(const T* p, RowSlice<T, E>& r) {
  constexpr int W = RowSlice<T, E>::W;
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int c = 0; c < W / 4; ++c) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[c];
      r.w[4 * c] = u.x;
      r.w[4 * c + 1] = u.y;
      r.w[4 * c + 2] = u.z;
      r.w[4 * c + 3] = u.w;
    }
  } else {
    static_assert(W == 2, "row slices are 8 bytes or a multiple of 16");
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    r.w[0] = u.x;
    r.w[1] = u.y;
  }
}

template <typename T, int E>
__device__ __forceinline__ double elem(const RowSlice<T, E>& r, int q) {
  if constexpr (sizeof(T) == 2)
    return (double)__uint_as_float((q & 1) ? (r.w[q >> 1] & 0xffff0000u) : (r.w[q >> 1] << 16));
  else
    return (double)__uint_as_float(r.w[q]);
}

// A double moved between lanes by a DPP control (both halves alike).
template <int CTRL>
__device__ __forceinline__ double dpp_move(double x) {
  const int l = __double2loint(x), h = __double2hiint(x);
  const int lo = __builtin_amdgcn_update_dpp(l, l, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(h, h, CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// Sum over a token's G lanes (aligned groups of 4, 8 or 16 lanes).  Every
// step pairs each lane with a partner that holds the mirror-image partial sum,
// and a + b == b + a exactly, so all G lanes end with the identical value.
template <int G>
__device__ __forceinline__ double group_sum(double x) {
  static_assert(G == 4 || G == 8 || G == 16, "a token's lanes lie inside one DPP row");
  if constexpr (G == 16) {
    // rotations by 8, 4, 2, 1 within the 16-lane row
    x += dpp_move<0x128>(x);
    x += dpp_move<0x124>(x);
    x += dpp_move<0x122>(x);
    x += dpp_move<0x121>(x);
  } else {
    x += dpp_move<0xB1>(x);                      // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_move<0x4E>(x);                      // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G == 8) x += dpp_move<0x141>(x);  // row_half_mirror: the other quad
  }
  return x;
}

// G: lanes per token; LT: a bound on the number of tables (sizes the
// per-table registers)
template <typename T, int D, int LT, int G>
__global__ __launch_bounds__(256, LT > 4 ? 5 : FASTAR_MATCH_OCC) void match_kernel(Dims dm, CacheDev c, MatchArgs a) {
  constexpr int E = D / G;
  constexpr int kMaxCand = FASTAR_MATCH_MAXCAND;  // candidates listed before scoring
  constexpr int kBatch = FASTAR_MATCH_BATCH;  // candidate rows in flight together
  // entries of a bucket read per pass, kF per lane (the first pass of every
  // table is issued with the other independent loads)
  constexpr int kF = FASTAR_MATCH_FIRST / G > 0 ? FASTAR_MATCH_FIRST / G : 1;
  constexpr int kPass = G * kF;
  static_assert(kPass <= 32, "one pass of a bucket fits a 32-bit mask");
  const int h = blockIdx.y;
  const int i = blockIdx.x * (256 / G) + (threadIdx.x / G);
  const int gl = threadIdx.x & (G - 1);
  if (i >= a.T) return;  // all G lanes of a group leave together
  const int L = dm.L, B = dm.B, NB = dm.NB, nb_bits = dm.nb_bits;

  // All independent loads first: the token's key, its codes, then every
  // table's bucket bounds and first entries, so the dependent chain per token
  // is codes -> bucket bounds -> entries -> candidate keys.
  RowSlice<T, E> xr;
  load_row<T, E>(static_cast<const T*>(a.x) + (int64_t)h * a.sx_h + (int64_t)i * a.sx_n + gl * E,
                 xr);
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
  // the first kPass entries of every table's bucket, kF per lane, all in
  // flight together (buckets hold a few entries; longer ones are read on in
  // the loop)
  uint2 first[LT][kF];
#pragma unroll
  for (int t = 0; t < LT; ++t)
#pragma unroll
    for (int u = 0; u < kF; ++u) {
      const int p = beg[t] + gl + G * u;
      first[t][u] = (t < L && p < end[t]) ? c.idx_ent[((int64_t)h * L + t) * B + p]
                                          : make_uint2(0u, 0u);
    }

  double nx2 = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) nx2 = __builtin_fma(elem(xr, e), elem(xr, e), nx2);
  nx2 = group_sum<G>(nx2);

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
      // the token's key is widened per batch instead of being held as 2E
      // float64 registers across the whole kernel
#pragma unroll
      for (int q = 0; q < RowSlice<T, E>::W; ++q) asm volatile("" : "+v"(xr.w[q]));
      RowSlice<T, E> kv[kBatch];
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
          const double k = elem(kv[u], q);
          dot[u] = __builtin_fma(elem(xr, q), k, dot[u]);
          nk2[u] = __builtin_fma(k, k, nk2[u]);
          // widen a few elements at a time, not all 2E of them at once
          if ((q & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        dot[u] = group_sum<G>(dot[u]);
        nk2[u] = group_sum<G>(nk2[u]);
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
  // the token's, each slot once.  The G lanes read kPass entries of a bucket
  // per pass; ballots over the group list the matching ones.  The candidate
  // list is identical in every lane of the group.  The common case (every
  // match fits the list) scores once, after all tables; a list that fills up
  // sends the token to a plain pass over all buckets that scores whenever its
  // list is full (slots scored twice only cost time: a rescored slot never
  // displaces the best).
  int cand[kMaxCand];
  int nc = 0;
  bool full = false;
  const int gbase = threadIdx.x & 63 & ~(G - 1);
  constexpr uint32_t gmask = (1u << G) - 1u;
  // lists the matching entries of one pass (kF per lane) of table t
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
      const int s = __shfl(v, j % G, G);
      bool dup = false;
      for (int k = 0; k < nc; ++k) dup |= cand[k] == s;
      if (dup) continue;
      if (nc == kMaxCand) {
        full = true;
        break;
      }
      cand[nc++] = s;
    }
  };
#pragma unroll
  for (int t = 0; t < LT; ++t)
    if (t < L) list_pass(first[t], beg[t], t);
  // buckets longer than one pass (rare)
#pragma unroll
  for (int t = 0; t < LT; ++t) {
    if (t >= L) break;
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
  score(cand, nc);
  if (full) {
    // every bucket again, one entry per lane per pass, scoring each full list
    // (the code and bucket bounds are read again rather than kept live)
    nc = 0;
    for (int t = 0; t < L; ++t) {
      const uint32_t code = a.codes[((int64_t)h * L + t) * a.codes_ld + a.codes_col0 + i];
      const int32_t* off = c.idx_off + ((int64_t)h * L + t) * (NB + 1) + bucket_of(code, nb_bits);
      const int b0 = off[0], b1 = off[1];
      const uint2* ent = c.idx_ent + ((int64_t)h * L + t) * B;
      for (int p0 = b0; p0 < b1; p0 += G) {
        const int p = p0 + gl;
        const uint2 e = p < b1 ? ent[p] : make_uint2(0u, 0u);
        const bool ok = p < b1 && e.y == code;
        uint32_t mask = (uint32_t)(__ballot(ok) >> gbase) & gmask;
        while (mask) {
          const int j = __builtin_ctz(mask);
          mask &= mask - 1;
          const int s = __shfl((int)e.x, j, G);
          bool dup = false;
          for (int k = 0; k < nc; ++k) dup |= cand[k] == s;
          if (dup) continue;
          if (nc == kMaxCand) {
            score(cand, nc);
            nc = 0;
          }
          cand[nc++] = s;
        }
      }
    }
    score(cand, nc);
  }
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
  constexpr int Gb = FASTAR_MATCH_GROUP_BF16;  // lanes per token, 2-byte keys
  constexpr int Gf = 16;                       // lanes per token, 4-byte keys
  const int G = dm.elem == 2 ? Gb : Gf;
  const dim3 grid((a.T + 256 / G - 1) / (256 / G), dm.H);
  if (dm.elem == 2) {
    if (dm.d == 128) hipLaunchKernelGGL((match_kernel<uint16_t, 128, LT, Gb>), grid, dim3(256), 0, s, dm, c, a);
    else hipLaunchKernelGGL((match_kernel<uint16_t, 64, LT, Gb>), grid, dim3(256), 0, s, dm, c, a);
  } else {
    if (dm.d == 128) hipLaunchKernelGGL((match_kernel<float, 128, LT, Gf>), grid, dim3(256), 0, s, dm, c, a);
    else hipLaunchKernelGGL((match_kernel<float, 64, LT, Gf>), grid, dim3(256), 0, s, dm, c, a);
  }
  return hipGetLastError();
}

hipError_t launch_match(const Dims& dm, const CacheDev& c, const MatchArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  static_assert(FASTAR_MAX_TABLES_DEV == 8, "table bounds below");
  return dm.L <= 4 ? launch_match_lt<4>(dm, c, a, s) : launch_match_lt<8>(dm, c, a, s);
}

}  // namespace fastar
