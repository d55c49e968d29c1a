// Shared definitions of the gfx950 TempCache library: storage types, the
// workspace layout of a cache, and the internal launcher interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fastar.h"

#define FASTAR_MAX_TABLES_DEV FASTAR_MAX_TABLES

namespace fastar {

constexpr int kWave = 64;
constexpr int kSlotPad = 128;  // mirror rows per head are padded to a multiple of this
#ifndef FASTAR_SLOTS_PER_BUCKET
#define FASTAR_SLOTS_PER_BUCKET 4
#endif
// Buckets of the LSH index: about this many budget slots per bucket.  The
// match reads a bucket 16 entries at a time and filters by code, so a few
// slots per bucket cost it nothing while shrinking the index rebuild.
constexpr int kSlotsPerBucket = FASTAR_SLOTS_PER_BUCKET;

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i to XCD
// i % 8).  Renumbering them so that XCD x runs the contiguous range
// [x*q + min(x, r), ...) of logical ids keeps neighbouring tiles, which share
// operands, on one XCD and its L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = bid & 7, k = bid >> 3;
  return x * q + min(x, r) + k;
}

// ---------------------------------------------------------------- bfloat16
// bfloat16 values travel as raw 16-bit patterns.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// binary32 -> bfloat16, round to nearest, ties to even (the format definition:
// keep the upper 16 bits, decide the rounding from the lower 16).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN -> quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Load/store one element of storage type T (float or uint16_t bf16 bits) as float.
template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p) {
  return bf16_bits_to_f32(*p);
}

// Bucket of a code in a table of 2^nb_bits buckets (multiplicative hashing;
// the bucket only narrows the search, equality of codes is checked exactly).
__device__ __forceinline__ uint32_t bucket_of(uint32_t code, int nb_bits) {
  return nb_bits == 0 ? 0u : (code * 0x9E3779B1u) >> (32 - nb_bits);
}

// Code of one table: bits [off, off+b) of the concatenated 32-bit words of
// sign bits (word k holds planes 32k .. 32k+31, LSB first).
__device__ __forceinline__ uint32_t extract_code(const uint32_t (&w)[9], int off, int b) {
  if (b == 0) return 0u;
  const int wi = off >> 5, sh = off & 31;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k == wi) lo = w[k];
    if (k == wi + 1) hi = w[k];
  }
  uint64_t both = ((uint64_t)hi << 32) | lo;
  uint32_t code = (uint32_t)(both >> sh);
  return b == 32 ? code : (code & ((1u << b) - 1u));
}

// ---------------------------------------------------------------- cache layout
// Per-head counters (int64): tokens seen, merged tokens, inserted tokens,
// evicted slots, and frames the planning step refused because fewer slots
// were evictable than the inserts needed (only an inconsistent state can do
// that; the refused frame changes nothing).
enum {
  kCntTokens = 0, kCntMerged = 1, kCntInserted = 2, kCntEvictedSlots = 3, kCntRefused = 4,
  kNumCounters = 5
};
// Per-head plan summary written by the planning kernel of each frame (int32).
enum { kPlanGroups = 0, kPlanInserts = 1, kPlanMergeTokens = 2, kPlanEvict = 3, kPlanStride = 8 };
constexpr int32_t kNoOwner = 0x7fffffff;

struct Dims {
  int H, d, B, L, b;
  int M;         // 0: SimHash codes; M > 0: product-quantization codes, M slices
  int Bp;        // B rounded up to a multiple of kSlotPad (mirror rows per head)
  int elem;      // storage bytes per element (2 or 4)
  int nb_bits;   // log2 of buckets per (head, table)
  int NB;        // buckets per (head, table)
  int Ppad;      // L*b rounded up to a multiple of 32
  int R;         // frames of each slot's most recent members kept (0: none)
};

// Queries per workgroup of the bf16 attention over the cache: 8 waves of 32
// at d = 128, 4 waves of 32 at d = 64.
inline int attn_query_tile(const Dims& dm) { return dm.d == 128 ? 256 : 128; }
// (head, query tile) pairs whose key tiles the attention may split in four
// (the last, partial round of workgroups): at most three quarters of the
// GPU's 256 CUs, and 8 per head for small caches.
inline int attn_split_pairs(const Dims& dm) { return dm.H * 8 < 192 ? dm.H * 8 : 192; }

// Device pointers into one cache's workspace.
struct CacheDev {
  void* planes;        // SimHash: [L][b][d]; PQ: codebooks [L][M][2^(b/M)][d/M]; storage dtype
  void* planes_frag;   // bf16 caches: the hyperplanes as 32x32x16 MFMA A fragments,
                       // [Ppad/32][d/16][64 lanes] x 16 bytes, zero past L*b
  float* k_master;     // [H][B][d]
  float* v_master;     // [H][B][d]
  void* k_mirror;      // [H][Bp][d] storage dtype
  void* v_mirror;      // [H][Bp][d] storage dtype
  float* lb;           // [H][Bp] log2(count) of live slots, -inf elsewhere
  int32_t* count;      // [H][B]
  int32_t* last;       // [H][B]
  uint32_t* codes;     // [H][L][B]
  int32_t* idx_off;    // [H][L][NB+1] CSR offsets of the buckets
  uint2* idx_ent;      // [H][L][B] (slot, code) entries grouped by bucket
  int32_t* n_live;     // [H]
  int64_t* evicted_tokens;  // [H]
  int64_t* counters;   // [H][kNumCounters]
  int32_t* frame;      // [1]
  // Per-slot merge bookkeeping of the frame being processed: the lowest token
  // that merges into the slot (kNoOwner if none) and how many tokens do.  Set
  // by the match step, consumed and reset by the planning step.
  int32_t* owner;      // [H][B]
  int32_t* gsize;      // [H][B]
  // per-frame scratch (a frame has at most B tokens)
  int32_t* best_slot;  // [H][B] top-1 candidate or -1
  float* best_cos;     // [H][B]
  int32_t* dec;        // [H][B] merge target or -1 (insert)
  uint32_t* frame_codes;  // [H][L][B] codes of the frame when hashed here
  int32_t* group_tok;  // [H][B] merging tokens, group by group, ascending within a group
  int32_t* group_slot; // [H][B] slot of each merge group
  int4* items;         // [H][B] the frame's work items of the apply kernel: merge groups
                       // {slot, first member in group_tok, members, leader token},
                       // then inserts {slot, -1, 1, token}, y = -2 when the
                       // slot was evicted in this frame
  int32_t* plan;       // [H][kPlanStride]
  // AnnSA: slot codes under the AnnSA hyperplanes and their bucket index
  uint32_t* annsa_codes;  // [H][4][B]
  int32_t* annsa_off;     // [H][4][NB+1]
  uint2* annsa_ent;       // [H][4][B]
  // R > 0: frames of each slot's R most recent members, most recent first
  // (entries past the slot's count are unspecified), and the rotated keys and
  // log-count shifts of the M-degree attention, region r = member r
  int32_t* hist;          // [H][B][R]
  void* rope_k;           // bf16 [H][R*Bp][d]
  float* rope_lb;         // [H][R*Bp]
  // the shifts of the last attention call divided by its logit scale
  // (scale * log2(e)): [H][Bp], or [H][R*Bp] for the M-degree regions
  float* lbc;
  // partial results of attention workgroups that cover a quarter of a
  // (head, query tile)'s key tiles: unnormalised outputs [P][4][BM][d] fp32
  // and (running max in log2 units, sum) [P][4][BM], P = attn_pairs
  float* attn_part;
  float2* attn_ml;
  int attn_pairs;
};

struct Layout {
  size_t off[40];
  size_t total;
};

// Computes the byte offsets of every CacheDev member for these dimensions.
Layout make_layout(const Dims& dm);
CacheDev carve(void* base, const Dims& dm);

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `stream` and return the launch status.

// SimHash.  Row n of head h is x + h*sx_h + n*sx_n (or row rows[h*rows_ld+n]
// when rows != nullptr, for n < n_rows[h]).  Codes go to
// codes[(h*L + t)*codes_ld + codes_col0 + n] (or column rows[...] when gathering).
struct HashArgs {
  const void* x;
  int64_t sx_h, sx_n;
  int H, N, d, L, b;
  const void* planes;
  uint32_t* codes;
  int64_t codes_ld, codes_col0;
  const int32_t* rows;      // optional gather list
  int64_t rows_ld;
  const int32_t* n_rows;    // per-head row count when gathering (device)
  int n_rows_stride;        // int32 stride between heads in n_rows
  int M;                    // 0: SimHash with planes [L][b][d]; M > 0: product
                            // quantization with codebooks [L][M][2^(b/M)][d/M]
};
hipError_t launch_hash_bf16(const HashArgs& a, hipStream_t s);
hipError_t launch_hash_f32(const HashArgs& a, hipStream_t s);
hipError_t launch_pq(const HashArgs& a, bool bf16, hipStream_t s);

// One frame of matching.
struct MatchArgs {
  const void* x;            // keys of the frame: head h, token i at x + h*sx_h + i*sx_n
  int64_t sx_h, sx_n;
  const uint32_t* codes;    // codes[(h*L + t)*codes_ld + codes_col0 + i]
  int64_t codes_ld, codes_col0;
  int T;
  float tau;
};
hipError_t launch_match(const Dims& dm, const CacheDev& c, const MatchArgs& a, hipStream_t s);

// One frame of planning + applying (merge, evict, insert).
struct MergeArgs {
  const void* k;            // token i of the frame at k + h*sx_h + i*sx_n
  const void* v;
  int64_t sx_h, sx_n;
  const uint32_t* codes;    // as MatchArgs
  int64_t codes_ld, codes_col0;
  int T;
  int32_t* slot_out;        // optional, slot_out[h*out_ld + out_col0 + i]
  uint8_t* merged_out;      // optional
  int64_t out_ld, out_col0;
};
hipError_t launch_plan(const Dims& dm, const CacheDev& c, const MergeArgs& a, hipStream_t s);
hipError_t launch_apply(const Dims& dm, const CacheDev& c, const MergeArgs& a, hipStream_t s);
hipError_t launch_rehash(const Dims& dm, const CacheDev& c, int T, hipStream_t s);
hipError_t launch_index(const Dims& dm, const CacheDev& c, bool bump_frame, hipStream_t s);
// Recompute lb from count/n_live and zero the mirrors of slots >= n_live.
hipError_t launch_finalize_state(const Dims& dm, const CacheDev& c, hipStream_t s);

// Attention of queries over the live slots of a bf16 cache.
struct CacheAttendArgs {
  const void* q;
  int64_t sq_h, sq_n;
  void* o;
  int64_t so_h, so_n;
  float* lse;               // optional [H][Nq]
  int Nq;
  float scale;
  // optional raw tokens attended after the slots with count 1 (no logit
  // shift): key j of head h at xk + h*sx_h + j*sx_n (same for xv), j < n_x
  const void* xk;
  const void* xv;
  int64_t sx_h, sx_n;
  int n_x;
  // n_reg > 0: keys and log2 shifts from c.rope_k / c.rope_lb, n_reg regions
  // of Bp rows per head; region r's row s pairs with the V mirror row s
  int n_reg;
  // set by the launcher: (head, query tile) pairs [0, nfull) run whole, the
  // rest as four workgroups of a quarter of the key tiles each
  int nfull;
};
// The M-degree regions: rotated keys of each live slot's m most recent
// members' frames and their log2(count/m') shifts (-inf past m' or n_live).
hipError_t launch_rope_expand(const Dims& dm, const CacheDev& c, int m, int rope_dims,
                              float rope_base, hipStream_t s);
hipError_t launch_attend_cache_bf16(const Dims& dm, const CacheDev& c, const CacheAttendArgs& a,
                                    hipStream_t s);

// AnnSA over the cache: c.codes / c.idx_off / c.idx_ent and dm.L describe the
// AnnSA slot codes and their bucket index (at most 4 tables).
struct AnnsaArgs {
  const void* q;            // query i of head h at q + h*sq_h + i*sq_n (cfg dtype)
  int64_t sq_h, sq_n;
  const uint32_t* q_codes;  // [H][L][Nq]
  int Nq;
  float scale;
  void* o;
  int64_t so_h, so_n;
  float* lse;               // optional [H][Nq]
};
hipError_t launch_annsa(const Dims& dm, const CacheDev& c, const AnnsaArgs& a, hipStream_t s);

// Attention (TempCache over the live slots, or AnnCA over a per-frame subset).
struct AttendArgs {
  const void* q;
  int64_t sq_h, sq_n;
  const void* k;            // key j of head h at k + h*sk_h + j*sk_n
  const void* v;
  int64_t sk_h, sk_n;
  const int32_t* count;     // optional [H][count_ld] group sizes (ln-count bias)
  int64_t count_ld;
  const int32_t* n_keys;    // per (head, segment) key count (device), or nullptr
  int n_keys_const;         // used when n_keys == nullptr
  const int32_t* sel;       // optional gather list: sel[(h*F + g)*sel_ld + j]
  int64_t sel_ld;
  void* o;
  int64_t so_h, so_n;
  float* lse;               // optional [H][F*Nseg]
  int H, d, Nseg, F;        // F segments (frames) of Nseg queries each
  float scale;              // logit scale
  // f32 only, with F = 1: raw tokens attended after the keys with no logit
  // shift (count 1), as in CacheAttendArgs
  const void* xk;
  const void* xv;
  int64_t sx_h, sx_n;
  int n_x;
  // AnnCA selection inside the attention kernel (bf16, d = 128): query i of
  // head h has code q_codes[(h*sel_L + t)*F*Nseg + i] in table t (codes
  // < 2^16, sel_L <= 4), and a key row j is kept for frame g iff
  // p_codes[(h*sel_L + t)*n_keys_const + j] equals the code of some query of
  // the frame in some table t; sel and n_keys are unused
  const uint32_t* q_codes;
  const uint32_t* p_codes;
  int sel_L;
};
hipError_t launch_attend_bf16(const AttendArgs& a, hipStream_t s);
// Subset attention with the AnnCA selection in its prologue (AttendArgs.q_codes).
hipError_t launch_annca_fused(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_f32(const AttendArgs& a, hipStream_t s);

// Key projection with SimHash codes in its epilogue: k = x W^T for N tokens,
// head h owning rows [h*d, (h+1)*d) of W, rounded to bf16 and stored, then
// hashed under the cache's fragment-ordered hyperplanes.
struct ProjArgs {
  const uint16_t* x;        // token n at x + n*sx (Din bf16)
  int64_t sx;
  const uint16_t* w;        // row r (out feature) at w + r*sw (Din bf16)
  int64_t sw;
  int N, Din, H, L, b, Ppad;
  uint16_t* k;              // (h, n, :) at k + h*sk_h + n*sk_n
  int64_t sk_h, sk_n;
  uint32_t* codes;          // [H][L][codes_ld]
  int64_t codes_ld;
  const void* planes_frag;  // [Ppad/32][d/16][64] x 16 B
};
hipError_t launch_project_hash(const ProjArgs& a, int d, hipStream_t s);

// AnnCA per-frame selection.
struct SelectArgs {
  const uint32_t* q_codes;  // [H][L][F*Nf]
  const uint32_t* p_codes;  // [H][L][Np]
  int Nf, F, Np, H, L;
  int32_t* sel_idx;         // [H][F][Np]
  int32_t* sel_count;       // [H][F]
};
hipError_t launch_annca_select(const SelectArgs& a, hipStream_t s);

}  // namespace fastar
