// Merge, evict and insert one frame of tokens into the bounded slot store
// (FAST-AR summary, section 2A: merged tokens keep the mean of their values and
// their group size; the cache growth is limited so memory stays constant).
//
// plan_kernel (one workgroup per head) decides everything that needs a view of
// the whole frame:
//   - groups the merging tokens by target slot, tokens ascending: the match
//     step left, per slot, the lowest merging token (the group's leader) and
//     the group size; one block scan gives every leader its group index and
//     member offset and every insert its rank; a leader of a group of several
//     tokens collects the others in token order.  Each group then has exactly
//     one owner in the apply step, so slot state is never updated atomically;
//   - when the inserts exceed the free slots, selects exactly the missing
//     number of slots not merged into in this frame, smallest
//     (last updated frame, slot id) first: an 8-bit radix select on `last`
//     finds the cut-off frame, a block scan breaks the tie on slot id;
//   - gives the inserts the evicted ids, then the never-used ids, ascending.
// apply_kernel: 16 lanes per merge group or insert.  A merge group replays
// m += (x - m) / (count + 1) in binary32, one correctly rounded op at a time,
// token by token, for the key and the value master, then refreshes the
// storage-dtype mirrors.  Integer counters in LDS use atomics only where the
// result does not depend on their order (histograms, bit sets, sums).
#include "common.hpp"

namespace fastar {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;

// Exclusive scan over the block; `total` receives the block sum.  Uses
// s_scan[0..kPlanWaves) and leaves it reusable on return.
template <typename V>
__device__ V block_excl_scan(V v, V* s_scan, V& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  V x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_scan[w] = x;
  __syncthreads();
  if (w == 0) {
    V sv = lane < kPlanWaves ? s_scan[lane] : V(0);
#pragma unroll
    for (int o = 1; o < kPlanWaves; o <<= 1) {
      const V y = __shfl_up(sv, o, 64);
      if (lane >= o) sv += y;
    }
    if (lane < kPlanWaves) s_scan[lane] = sv;
  }
  __syncthreads();
  const V base = w ? s_scan[w - 1] : V(0);
  total = s_scan[kPlanWaves - 1];
  __syncthreads();
  return base + x - v;
}

struct PlanShared {
  uint32_t red_m[2][kPlanWaves];  // per-wave (min, count of min), two buffers
  int red_c[2][kPlanWaves];
  int digit, krem;
  int refused;  // fewer evictable slots than needed: the frame changes nothing
};

// Three counts per token packed in one 64-bit scan: group leaders (bits
// 42..62), members of the groups they lead (bits 21..41), inserts (0..20).
constexpr int kLeadShift = 42, kMemShift = 21;
constexpr uint64_t kField = (1ull << 21) - 1;

#ifndef FASTAR_PLAN_PREFETCH
#define FASTAR_PLAN_PREFETCH 1
#endif
typedef __attribute__((address_space(3))) void plan_lds_t;
typedef __attribute__((address_space(1))) void plan_gbl_t;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Dims dm, CacheDev c, MergeArgs a,
                                                           int stage_keys) {
  extern __shared__ __attribute__((aligned(16))) int32_t sm[];
  const int T = a.T, B = dm.B;
  int32_t* dec_s = sm;                 // [T] merge target of each token, -1 = insert
  int32_t* ins_list = dec_s + T;       // [T] inserting tokens, ascending
  int32_t* ev_list = ins_list + T;     // [T] evicted slots, ascending
  int32_t* lead_s = ev_list + T;       // [T] group size if the token leads its group, else 0
  uint32_t* keys_s = reinterpret_cast<uint32_t*>(lead_s + T);  // [B] eviction keys, if staged
  __shared__ uint64_t s_scan64[kPlanWaves];
  __shared__ int s_scan[kPlanWaves];
  __shared__ int hist[256];
  __shared__ PlanShared ps;

  const int h = blockIdx.x, tid = threadIdx.x;
  const int f = *c.frame;
  const int n_live = c.n_live[h];
  int32_t* owner = c.owner + (int64_t)h * B;
  int32_t* gsize = c.gsize + (int64_t)h * B;
#if FASTAR_PLAN_PREFETCH
  // Eviction is possible only if the frame's tokens can outnumber the free
  // slots.  Then the live slots' last-update frames are copied into LDS
  // (direct-to-LDS loads, 64 slots per wave instruction) while the token
  // passes below run; the slots merged into in this frame are masked out of
  // that copy afterwards, from the tokens' targets.
  const bool prefetch = stage_keys && n_live + T > B;  // block-uniform
  if (prefetch) {
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), ln = tid & 63;
    const int32_t* lastp = c.last + (int64_t)h * B;
    for (int c0 = wv * 64; c0 < n_live; c0 += kPlanThreads)
      if (c0 + ln < n_live)
        __builtin_amdgcn_global_load_lds((plan_gbl_t*)(lastp + c0 + ln),
                                         (plan_lds_t*)(keys_s + c0), 4, 0, 0);
  }
#endif
  // 0. per token (strided over the threads, every load of a thread issued
  //    together): its merge target, and whether it leads the target's group
  //    (the lowest merging token, recorded by the match step) with the group
  //    size, or 0.
  constexpr int kPerT = (FASTAR_MAX_TOKENS_PER_FRAME + kPlanThreads - 1) / kPlanThreads;
  {
    int dv[kPerT], ow[kPerT], gs[kPerT];
#pragma unroll
    for (int k = 0; k < kPerT; ++k) {
      const int i = tid + k * kPlanThreads;
      dv[k] = i < T ? c.dec[(int64_t)h * B + i] : -1;
    }
#pragma unroll
    for (int k = 0; k < kPerT; ++k) {
      const int sx = dv[k] < 0 ? 0 : dv[k];
      ow[k] = owner[sx];
      gs[k] = gsize[sx];
    }
#pragma unroll
    for (int k = 0; k < kPerT; ++k) {
      const int i = tid + k * kPlanThreads;
      if (i >= T) continue;
      dec_s[i] = dv[k];
      lead_s[i] = (dv[k] >= 0 && ow[k] == i) ? gs[k] : 0;
    }
  }
  __syncthreads();

  // 1. per token: leader of a merge group (its group size), or insert.  A
  //    thread's tokens are few (T <= FASTAR_MAX_TOKENS_PER_FRAME): their
  //    leader flags and group sizes stay in registers for the passes below.
  const int per_t = (T + kPlanThreads - 1) / kPlanThreads;
  const int t_lo = min(T, tid * per_t), t_hi = min(T, t_lo + per_t);
  int lead_size[kPerT];  // group size if token t_lo+k leads its group, else 0
  uint64_t mine = 0;
#pragma unroll
  for (int k = 0; k < kPerT; ++k) {
    const int i = t_lo + k;
    lead_size[k] = 0;
    if (i >= t_hi) continue;
    if (dec_s[i] < 0) {
      mine += 1;
    } else {
      lead_size[k] = lead_s[i];
      if (lead_size[k]) mine += (1ull << kLeadShift) | ((uint64_t)lead_size[k] << kMemShift);
    }
  }
  uint64_t tot = 0;
  uint64_t run = block_excl_scan<uint64_t>(mine, s_scan64, tot);
  const int n_groups = (int)(tot >> kLeadShift);
  const int M = (int)((tot >> kMemShift) & kField);
  const int m = (int)(tot & kField);

  // 2. merge groups (members ascending) and the insert list
  int32_t* g_tok = c.group_tok + (int64_t)h * B;
  int32_t* g_slot = c.group_slot + (int64_t)h * B;
  int4* items = c.items + (int64_t)h * B;
#pragma unroll
  for (int k = 0; k < kPerT; ++k) {
    const int i = t_lo + k;
    if (i >= t_hi) continue;
    const int s = dec_s[i];
    if (s < 0) {
      ins_list[(int)(run & kField)] = i;
      run += 1;
      continue;
    }
    if (lead_size[k] == 0) continue;
    const int g = (int)(run >> kLeadShift);
    const int start = (int)((run >> kMemShift) & kField);
    const int size = lead_size[k];
    g_slot[g] = s;
    items[g] = make_int4(s, start, size, i);
    g_tok[start] = i;
    // the other members follow the leader in token order
    for (int j = i + 1, k = 1; k < size && j < T; ++j)
      if (dec_s[j] == s) g_tok[start + k++] = j;
    run += (1ull << kLeadShift) | ((uint64_t)size << kMemShift);
  }

  // 3. eviction, only if the inserts do not fit: exactly `need` slots not
  //    merged into in this frame (owner unset), smallest (last, slot) first
  const int need = max(0, m - (B - n_live));
  if (tid == 0) ps.refused = 0;
  if (need > 0) {
    if (tid == 0) ps.krem = need;
    __syncthreads();
    // Each thread owns a contiguous run [s_lo, s_hi) of the live slots.  Its
    // slots' keys are read once into registers: the last-update frame of a
    // slot not merged into in this frame (every such frame is <= f-1), else
    // ~0u.  All passes below work on these registers.
    constexpr int kPerS = (FASTAR_MAX_BUDGET + kPlanThreads - 1) / kPlanThreads;
    const int per_s = (n_live + kPlanThreads - 1) / kPlanThreads;
    const int s_lo = min(n_live, tid * per_s), s_hi = min(n_live, s_lo + per_s);
    const int32_t* last = c.last + (int64_t)h * B;
    uint32_t key[kPerS];
#if FASTAR_PLAN_PREFETCH
    if (stage_keys) {
      // every wave's copies have landed (prefetch holds: need > 0 implies
      // n_live + T > B); then the slots merged into lose eligibility
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      for (int i = tid; i < T; i += kPlanThreads) {
        const int s = dec_s[i];
        if (s >= 0) keys_s[s] = 0xffffffffu;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPerS; ++k)
        key[k] = s_lo + k < s_hi ? keys_s[s_lo + k] : 0xffffffffu;
    } else
#else
    if (stage_keys) {
      // coalesced: thread tid reads slots tid, tid + 1024, ... into LDS, four
      // slots' loads in flight at a time; then each thread takes its run
      for (int s0 = tid; s0 < n_live; s0 += 4 * kPlanThreads) {
        int32_t ow[4], lv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sx = min(s0 + u * kPlanThreads, n_live - 1);
          ow[u] = owner[sx];
          lv[u] = last[sx];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sx = s0 + u * kPlanThreads;
          if (sx < n_live) keys_s[sx] = ow[u] == kNoOwner ? (uint32_t)lv[u] : 0xffffffffu;
        }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPerS; ++k)
        key[k] = s_lo + k < s_hi ? keys_s[s_lo + k] : 0xffffffffu;
    } else
#endif
    {
#pragma unroll
      for (int k = 0; k < kPerS; ++k) {
        const int sx = min(s_lo + k, B - 1);
        const int32_t ow = owner[sx];
        const int32_t lv = last[sx];
        key[k] = (s_lo + k < s_hi && ow == kNoOwner) ? (uint32_t)lv : 0xffffffffu;
      }
    }
    // The need-th smallest key among the eligible slots (the cut-off frame)
    // and how many slots with exactly that key to evict.  Eviction takes the
    // oldest frames first, and those hold few distinct values: walk them
    // upward, one block-wide (min, count of min) reduction each.  If eight
    // values do not cover `need`, a radix select over the rest finishes.
    uint32_t cut = 0u;
    int take_eq = 0;
    bool found = false;
    {
      int krem = need;
      uint32_t lo = 0u;  // keys below lo are already counted
      for (int step = 0; step < 8 && !found; ++step) {
        uint32_t mv = 0xffffffffu;
#pragma unroll
        for (int k = 0; k < kPerS; ++k)
          if (key[k] >= lo) mv = min(mv, key[k]);
        int cv = 0;
#pragma unroll
        for (int k = 0; k < kPerS; ++k) cv += key[k] == mv && mv != 0xffffffffu;
        // (min, count of min) over the wave, then over the waves
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t m2 = (uint32_t)__shfl_xor((int)mv, o, 64);
          const int c2 = __shfl_xor(cv, o, 64);
          const uint32_t mn = min(mv, m2);
          cv = (mv == mn ? cv : 0) + (m2 == mn ? c2 : 0);
          mv = mn;
        }
        uint32_t* rm = ps.red_m[step & 1];
        int* rc = ps.red_c[step & 1];
        if ((tid & 63) == 0) {
          rm[tid >> 6] = mv;
          rc[tid >> 6] = cv;
        }
        __syncthreads();
        mv = 0xffffffffu;
        cv = 0;
#pragma unroll
        for (int w = 0; w < kPlanWaves; ++w) mv = min(mv, rm[w]);
#pragma unroll
        for (int w = 0; w < kPlanWaves; ++w) cv += rm[w] == mv ? rc[w] : 0;
        if (mv == 0xffffffffu) break;  // fewer eligible slots than needed
        if (cv >= krem) {
          cut = mv;
          take_eq = krem;
          found = true;
        } else {
          krem -= cv;
          lo = mv + 1u;
        }
      }
      if (tid == 0) ps.krem = found ? take_eq : need;
      __syncthreads();
    }
    if (!found) {
    // radix select of the need-th smallest key among the eligible slots,
    // 8 bits at a time from the top (digits above f-1's skipped)
    uint32_t prefix = 0u;
    const uint32_t maxv = (uint32_t)(f - 1);
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (shift > 0 && (maxv >> shift) == 0u) continue;
      for (int q = tid; q < 256; q += kPlanThreads) hist[q] = 0;
      __syncthreads();
      const uint64_t hi_mask = ~((1ull << (shift + 8)) - 1ull);
#pragma unroll
      for (int k = 0; k < kPerS; ++k) {
        const uint32_t lv = key[k];
        if (lv != 0xffffffffu && ((uint64_t)lv & hi_mask) == ((uint64_t)prefix & hi_mask))
          atomicAdd(&hist[(lv >> shift) & 255u], 1);
      }
      __syncthreads();
      // the digit holding the krem-th smallest key: lane l of wave 0 scans
      // bins 4l .. 4l+3, a wave prefix sum gives each lane its base count
      if (tid < 64) {
        const int kr = ps.krem;
        const int h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2],
                  h3 = hist[4 * tid + 3];
        const int tot = h0 + h1 + h2 + h3;
        int incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o, 64);
          if (tid >= o) incl += y;
        }
        const int base = incl - tot;
        if (base < kr && kr <= incl) {
          int cum = base, dg = 4 * tid;
          if (cum + h0 < kr) {
            cum += h0;
            ++dg;
            if (cum + h1 < kr) {
              cum += h1;
              ++dg;
              if (cum + h2 < kr) {
                cum += h2;
                ++dg;
              }
            }
          }
          ps.digit = dg;
          ps.krem = kr - cum;
        }
        if (tid == 63 && incl < kr) {  // fewer eligible slots than needed
          ps.digit = 256;
          ps.krem = kr - incl;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)ps.digit << shift;
      __syncthreads();
    }
    cut = prefix;          // the need-th smallest `last`
    take_eq = ps.krem;     // how many slots with last == cut to evict
    }
    // rank of each slot among the eligible ones with last == cut
    int eq = 0;
#pragma unroll
    for (int k = 0; k < kPerS; ++k) eq += key[k] == cut;
    int eq_total = 0;
    const int eq_base = block_excl_scan<int>(eq, s_scan, eq_total);
    int evc = 0;
    {
      int er = eq_base;
#pragma unroll
      for (int k = 0; k < kPerS; ++k) {
        if (key[k] < cut) ++evc;
        else if (key[k] == cut) evc += (er++ < take_eq);
      }
    }
    int ev_total = 0;
    int ep = block_excl_scan<int>(evc, s_scan, ev_total);
    // With tokens_per_frame <= budget and every live slot's last update
    // before this frame (both checked on the host), the eligible slots always
    // cover `need`.  Otherwise ev_list would be short: refuse the frame.
    if (ev_total < need) {
      if (tid == 0) ps.refused = 1;
    } else {
      // (the tokens the evicted slots held are tallied by the apply step,
      // which reads each slot's count before its insert overwrites it)
      int er = eq_base;
#pragma unroll
      for (int k = 0; k < kPerS; ++k) {
        bool ev = false;
        if (key[k] < cut) ev = true;
        else if (key[k] == cut) ev = (er++ < take_eq);
        if (ev) ev_list[ep++] = s_lo + k;
      }
    }
  }
#if FASTAR_PLAN_PREFETCH
  // no LDS copy may still be in flight when the block ends
  if (prefetch) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
  __syncthreads();

  // 4. reset the per-slot bookkeeping for the next frame (leaders own it)
#pragma unroll
  for (int k = 0; k < kPerT; ++k) {
    const int i = t_lo + k;
    if (i >= t_hi || lead_size[k] == 0) continue;
    const int s = dec_s[i];
    owner[s] = kNoOwner;
    gsize[s] = 0;
  }

  if (ps.refused) {
    if (tid == 0) {
      c.counters[(int64_t)h * kNumCounters + kCntRefused] += 1;
      int32_t* pl = c.plan + (int64_t)h * kPlanStride;
      pl[kPlanGroups] = 0;
      pl[kPlanInserts] = 0;
      pl[kPlanMergeTokens] = 0;
      pl[kPlanEvict] = 0;
    }
    if (a.slot_out != nullptr || a.merged_out != nullptr) {
      for (int i = tid; i < T; i += kPlanThreads) {
        const int64_t o = (int64_t)h * a.out_ld + a.out_col0 + i;
        if (a.slot_out) a.slot_out[o] = -1;
        if (a.merged_out) a.merged_out[o] = 0;
      }
    }
    return;
  }

  // 5. slots for the inserts: evicted ids first, then never-used ids, ascending
  const bool want_out = a.slot_out != nullptr || a.merged_out != nullptr;
  for (int q = tid; q < m; q += kPlanThreads) {
    const int tok = ins_list[q];
    const int slot = q < need ? ev_list[q] : n_live + (q - need);
    // y = -2 marks an insert into an evicted slot (its old count is tallied)
    items[n_groups + q] = make_int4(slot, q < need ? -2 : -1, 1, tok);
    if (want_out) {
      const int64_t o = (int64_t)h * a.out_ld + a.out_col0 + tok;
      if (a.slot_out) a.slot_out[o] = slot;
      if (a.merged_out) a.merged_out[o] = 0;
    }
  }
  if (want_out) {
    for (int i = tid; i < T; i += kPlanThreads) {
      const int dv = dec_s[i];
      if (dv < 0) continue;
      const int64_t o = (int64_t)h * a.out_ld + a.out_col0 + i;
      if (a.slot_out) a.slot_out[o] = dv;
      if (a.merged_out) a.merged_out[o] = 1;
    }
  }
  if (tid == 0) {
    c.n_live[h] = n_live + m - need;
    int64_t* cn = c.counters + (int64_t)h * kNumCounters;
    cn[kCntTokens] += T;
    cn[kCntMerged] += M;
    cn[kCntInserted] += m;
    cn[kCntEvictedSlots] += need;
    int32_t* pl = c.plan + (int64_t)h * kPlanStride;
    pl[kPlanGroups] = n_groups;
    pl[kPlanInserts] = m;
    pl[kPlanMergeTokens] = M;
    pl[kPlanEvict] = need;
  }
}

template <typename T> __device__ __forceinline__ void store_mirror(T* p, float v);
template <> __device__ __forceinline__ void store_mirror<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_mirror<uint16_t>(uint16_t* p, float v) {
  *p = (uint16_t)f32_to_bf16_bits(v);
}

// Vector of E storage elements as floats (E = 4 or 8).
template <typename T, int E>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[E]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[E / 2];
    if constexpr (E == 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      w[0] = u.x; w[1] = u.y;
    }
#pragma unroll
    for (int k = 0; k < E / 2; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < E; k += 4) {
      const float4 f = *reinterpret_cast<const float4*>(p + k);
      v[k] = f.x; v[k + 1] = f.y; v[k + 2] = f.z; v[k + 3] = f.w;
    }
  }
}

template <int E>
__device__ __forceinline__ void load_f32vec(const float* p, float (&v)[E]) {
#pragma unroll
  for (int k = 0; k < E; k += 4) {
    const float4 f = *reinterpret_cast<const float4*>(p + k);
    v[k] = f.x; v[k + 1] = f.y; v[k + 2] = f.z; v[k + 3] = f.w;
  }
}

template <int E>
__device__ __forceinline__ void store_f32vec(float* p, const float (&v)[E]) {
#pragma unroll
  for (int k = 0; k < E; k += 4) *reinterpret_cast<float4*>(p + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
}

constexpr int kApplyGroup = 16;  // lanes per merge group or insert

// E consecutive mirror elements of one row, stored with one vector store.
template <typename T, int E>
__device__ __forceinline__ void store_mirror_vec(T* p, const float (&v)[E]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[E / 2];
#pragma unroll
    for (int k = 0; k < E / 2; ++k)
      w[k] = f32_to_bf16_bits(v[2 * k]) | (f32_to_bf16_bits(v[2 * k + 1]) << 16);
    if constexpr (E == 8) *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    else *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else {
    store_f32vec<E>(reinterpret_cast<float*>(p), v);
  }
}

#ifndef FASTAR_APPLY_OCC
#define FASTAR_APPLY_OCC 6
#endif
#ifndef FASTAR_APPLY_PREFETCH
#define FASTAR_APPLY_PREFETCH 2
#endif
constexpr int kApplyThreads = 512;
constexpr int kApplyItems = kApplyThreads / kApplyGroup;  // 32: one MFMA tile of key rows

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// With bf16 storage the block then refreshes the codes of its merge groups'
// slots: SimHash of the new key mirror rows (kept in LDS) against all L*b
// hyperplanes, one 32-plane block per wave on the 32x32x16 MFMA with
// hyperplanes as rows, the arithmetic of the hash kernel.
template <typename T, int D>
__global__ __launch_bounds__(kApplyThreads, FASTAR_APPLY_OCC) void apply_kernel(Dims dm, CacheDev c, MergeArgs a) {
#pragma clang fp contract(off)
  constexpr int E = D / kApplyGroup;  // features per lane
  constexpr bool kHash = sizeof(T) == 2;
  // new key rows (bf16 bits, rows padded by 16 bytes against bank conflicts),
  // the 32-bit words of sign bits per row and plane block, the rows' slots
  __shared__ __attribute__((aligned(16))) uint16_t s_rows[kHash ? kApplyItems : 1][D + 8];
  __shared__ uint32_t s_words[kApplyItems][9];
  __shared__ int32_t s_slot[kApplyItems];
  const int h = blockIdx.y;
  const int item = threadIdx.x / kApplyGroup;
  const int first = blockIdx.x * kApplyItems;
  const int w = first + item;
  const int gl = threadIdx.x & (kApplyGroup - 1);
  const int B = dm.B, L = dm.L, Bp = dm.Bp;
  const int32_t* pl = c.plan + (int64_t)h * kPlanStride;
  // the item record is read beside the plan summary (w < B keeps it in
  // bounds; records past the frame's items are stale and left unused)
  const int4 it = w < B ? c.items[(int64_t)h * B + w] : make_int4(0, 0, 0, 0);
  const int ng = pl[kPlanGroups], nins = pl[kPlanInserts];
  if (first >= ng + nins) return;  // the whole block is idle
  const int f = *c.frame;
  const T* kin = static_cast<const T*>(a.k) + (int64_t)h * a.sx_h;  // frame base, head h
  const T* vin = static_cast<const T*>(a.v) + (int64_t)h * a.sx_h;
  T* kmir = static_cast<T*>(c.k_mirror);
  T* vmir = static_cast<T*>(c.v_mirror);
  const int e0 = gl * E;

  if (w >= ng + nins) {
    // idle item of a busy block: nothing to update
  } else if (w < ng) {
    const int s = it.x, k0 = it.y, k1 = it.y + it.z, lead = it.w;
    const int64_t row = ((int64_t)h * B + s) * D + e0;
    const int c0 = c.count[(int64_t)h * B + s];
    float km[E], vm[E];
    load_f32vec<E>(c.k_master + row, km);
    load_f32vec<E>(c.v_master + row, vm);
    // The updates run strictly in token order; only the loads run ahead: the
    // leader's inputs load beside the slot state, the other members' ids are
    // read kApplyGroup at a time (one per lane), and the inputs of kPrefetch
    // members are in flight together.
    auto update = [&](const float (&xk)[E], const float (&xv)[E], int n_before) {
#pragma clang fp contract(off)
      const float div = (float)(c0 + n_before + 1);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float dk = xk[e] - km[e];
        const float dv = xv[e] - vm[e];
        const float qk = dk / div;
        const float qv = dv / div;
        km[e] = km[e] + qk;
        vm[e] = vm[e] + qv;
      }
    };
    {
      float xk[E], xv[E];
      load_vec<T, E>(kin + (int64_t)lead * a.sx_n + e0, xk);
      load_vec<T, E>(vin + (int64_t)lead * a.sx_n + e0, xv);
      update(xk, xv, 0);
    }
    constexpr int kPrefetch = FASTAR_APPLY_PREFETCH;
    const int32_t* gt = c.group_tok + (int64_t)h * B;
    for (int b0 = k0 + 1; b0 < k1; b0 += kApplyGroup) {
      const int nb = min(kApplyGroup, k1 - b0);
      const int my_tok = gl < nb ? gt[b0 + gl] : 0;
      for (int j = 0; j < nb; j += kPrefetch) {
        float xk[kPrefetch][E], xv[kPrefetch][E];
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u) {
          const int tok = __shfl(my_tok, min(j + u, nb - 1), kApplyGroup);
          load_vec<T, E>(kin + (int64_t)tok * a.sx_n + e0, xk[u]);
          load_vec<T, E>(vin + (int64_t)tok * a.sx_n + e0, xv[u]);
        }
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u) {
          if (j + u >= nb) break;
          update(xk[u], xv[u], b0 - k0 + j + u);
        }
      }
    }
    store_f32vec<E>(c.k_master + row, km);
    store_f32vec<E>(c.v_master + row, vm);
    const int64_t mrow = ((int64_t)h * Bp + s) * D + e0;
    store_mirror_vec<T, E>(kmir + mrow, km);
    store_mirror_vec<T, E>(vmir + mrow, vm);
    if constexpr (kHash) {
      store_mirror_vec<T, E>(reinterpret_cast<T*>(&s_rows[item][e0]), km);
      if (gl == 0) s_slot[item] = s;
    }
    if (gl == 0) {
      const int cnt = c0 + (k1 - k0);
      c.count[(int64_t)h * B + s] = cnt;
      c.last[(int64_t)h * B + s] = f;
      c.lb[(int64_t)h * Bp + s] = __log2f((float)cnt);
      if (dm.R > 0) {  // this frame's k1 - k0 members become the most recent
        int32_t* hr = c.hist + ((int64_t)h * B + s) * dm.R;
        int32_t old[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) old[i] = i < dm.R ? hr[i] : 0;
        const int g = k1 - k0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i >= dm.R) break;
          int32_t v = f;  // entry i after the shift: old entry i - g, if any
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j == i - g) v = old[j];
          hr[i] = v;
        }
      }
    }
  } else {
    const int s = it.x, tok = it.w;
    const int64_t row = ((int64_t)h * B + s) * D + e0;
    const int64_t mrow = ((int64_t)h * Bp + s) * D + e0;
    const T* kp = kin + (int64_t)tok * a.sx_n + e0;
    const T* vp = vin + (int64_t)tok * a.sx_n + e0;
    float xk[E], xv[E];
    load_vec<T, E>(kp, xk);
    load_vec<T, E>(vp, xv);
    store_f32vec<E>(c.k_master + row, xk);
    store_f32vec<E>(c.v_master + row, xv);
    store_mirror_vec<T, E>(kmir + mrow, xk);  // inputs are storage-exact: copies
    store_mirror_vec<T, E>(vmir + mrow, xv);
    if (gl == 0) {
      if (it.y == -2)  // the evicted group's tokens, an order-free integer sum
        atomicAdd(reinterpret_cast<unsigned long long*>(c.evicted_tokens + h),
                  (unsigned long long)c.count[(int64_t)h * B + s]);
      c.count[(int64_t)h * B + s] = 1;
      c.last[(int64_t)h * B + s] = f;
      c.lb[(int64_t)h * Bp + s] = 0.0f;
    }
    if (gl < dm.R) c.hist[((int64_t)h * B + s) * dm.R + gl] = f;
    if (gl < L)
      c.codes[((int64_t)h * L + gl) * B + s] =
          a.codes[((int64_t)h * L + gl) * a.codes_ld + a.codes_col0 + tok];
  }

  if constexpr (kHash) {
    if (first < ng && dm.M == 0) {  // block-uniform: SimHash codes of merge groups
      __syncthreads();
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      const int m = lane & 31, hf = lane >> 5;
      const int P = L * dm.b;
      uint32_t word = 0u;
      if (wave * 32 < P) {
        // MFMA rows: hyperplane wave*32 + m (zero past L*b), read from the
        // cache's fragment-ordered copy; columns: key row m; features
        // hf*D/2 + ks*8 .. +7 in k-step ks for both
        const bf16x8_t* pf =
            static_cast<const bf16x8_t*>(c.planes_frag) + wave * (D / 16) * 64 + lane;
        f32x16_t acc = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8_t pa = pf[ks * 64];
          const bf16x8_t xb = *reinterpret_cast<const bf16x8_t*>(&s_rows[m][hf * (D / 2) + ks * 8]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, xb, acc, 0, 0, 0);
        }
        // register j of lane l: plane 8*(j/4) + 4*(l/32) + j%4 of key row l%32
        uint32_t bits = 0u;
#pragma unroll
        for (int j = 0; j < 16; ++j) bits |= (acc[j] > 0.0f ? 1u : 0u) << (8 * (j >> 2) + (j & 3));
        bits <<= 4 * hf;
        word = bits | __shfl_xor(bits, 32);
      }
      if (hf == 0) s_words[m][wave] = word;
      if (threadIdx.x < kApplyItems) s_words[threadIdx.x][8] = 0u;
      __syncthreads();
      const int ngb = min(kApplyItems, ng - first);
      for (int idx = threadIdx.x; idx < ngb * L; idx += kApplyThreads) {
        const int r = idx / L, t = idx - r * L;
        c.codes[((int64_t)h * L + t) * B + s_slot[r]] = extract_code(s_words[r], t * dm.b, dm.b);
      }
    }
  }
}

// lb[s] = log2(count[s]) for live slots, -inf for the rest, whose mirror rows
// are zeroed (attention tiles may cover them; they must contribute nothing).
template <typename T, int D>
__global__ __launch_bounds__(256) void finalize_kernel(Dims dm, CacheDev c) {
  const int h = blockIdx.y;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= dm.Bp) return;
  if (s < dm.B && lane == 0) {
    c.owner[(int64_t)h * dm.B + s] = kNoOwner;
    c.gsize[(int64_t)h * dm.B + s] = 0;
  }
  const int n = c.n_live[h];
  if (s < n) {
    if (lane == 0) c.lb[(int64_t)h * dm.Bp + s] = __log2f((float)c.count[(int64_t)h * dm.B + s]);
    return;
  }
  if (lane == 0) c.lb[(int64_t)h * dm.Bp + s] = -__builtin_huge_valf();
  T* kmir = static_cast<T*>(c.k_mirror);
  T* vmir = static_cast<T*>(c.v_mirror);
  for (int e = lane; e < D; e += kWave) {
    kmir[((int64_t)h * dm.Bp + s) * D + e] = T(0);
    vmir[((int64_t)h * dm.Bp + s) * D + e] = T(0);
  }
}

}  // namespace

hipError_t launch_plan(const Dims& dm, const CacheDev& c, const MergeArgs& a, hipStream_t s) {
  // four per-token lists (128 KiB at FASTAR_MAX_TOKENS_PER_FRAME), and the
  // eviction keys of every slot staged in LDS when they fit beside them
  const size_t lists = (size_t)a.T * 4 * 4;
  const size_t keys = (size_t)dm.B * 4;
  const int stage = lists + keys <= 144 * 1024 ? 1 : 0;
  const size_t lds = lists + (stage ? keys : 0);
  if (lds > 64 * 1024) {  // beyond the default dynamic LDS limit of a launch
    hipError_t e = hipFuncSetAttribute((const void*)plan_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(plan_kernel, dim3(dm.H), dim3(kPlanThreads), lds, s, dm, c, a, stage);
  return hipGetLastError();
}

hipError_t launch_apply(const Dims& dm, const CacheDev& c, const MergeArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.T + kApplyItems - 1) / kApplyItems, dm.H), block(kApplyThreads);
  if (dm.elem == 2) {
    if (dm.d == 128) hipLaunchKernelGGL((apply_kernel<uint16_t, 128>), grid, block, 0, s, dm, c, a);
    else hipLaunchKernelGGL((apply_kernel<uint16_t, 64>), grid, block, 0, s, dm, c, a);
    return hipGetLastError();
  }
  if (dm.d == 128) hipLaunchKernelGGL((apply_kernel<float, 128>), grid, block, 0, s, dm, c, a);
  else hipLaunchKernelGGL((apply_kernel<float, 64>), grid, block, 0, s, dm, c, a);
  return hipGetLastError();
}

hipError_t launch_finalize_state(const Dims& dm, const CacheDev& c, hipStream_t s) {
  const dim3 grid((dm.Bp + 3) / 4, dm.H);
  if (dm.elem == 2) {
    if (dm.d == 128) hipLaunchKernelGGL((finalize_kernel<uint16_t, 128>), grid, dim3(256), 0, s, dm, c);
    else hipLaunchKernelGGL((finalize_kernel<uint16_t, 64>), grid, dim3(256), 0, s, dm, c);
  } else {
    if (dm.d == 128) hipLaunchKernelGGL((finalize_kernel<float, 128>), grid, dim3(256), 0, s, dm, c);
    else hipLaunchKernelGGL((finalize_kernel<float, 64>), grid, dim3(256), 0, s, dm, c);
  }
  return hipGetLastError();
}

hipError_t launch_rehash(const Dims& dm, const CacheDev& c, int T, hipStream_t s) {
  HashArgs h{};
  h.x = c.k_mirror;
  h.sx_h = (int64_t)dm.Bp * dm.d;
  h.sx_n = dm.d;
  h.H = dm.H;
  h.N = T;
  h.d = dm.d;
  h.L = dm.L;
  h.b = dm.b;
  h.planes = c.planes;
  h.codes = c.codes;
  h.codes_ld = dm.B;
  h.codes_col0 = 0;
  h.rows = c.group_slot;
  h.rows_ld = dm.B;
  h.n_rows = c.plan + kPlanGroups;
  h.n_rows_stride = kPlanStride;
  h.M = dm.M;
  return dm.elem == 2 ? launch_hash_bf16(h, s) : launch_hash_f32(h, s);
}

}  // namespace fastar
