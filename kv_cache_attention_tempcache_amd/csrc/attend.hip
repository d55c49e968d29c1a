// Attention over the merged cache with the group-size logit shift (FAST-AR
// summary, section 2A, Lemma 5.1: merging identical keys is exact when values
// are averaged and each logit is shifted by its group size), and the same
// kernel over a per-frame subset of prompt keys for AnnCA (section 2B).
//
// bf16 path, per workgroup of 8 waves; each wave owns 32 queries:
//   S^T = K Q^T on the 32x32x16 bf16 MFMA: A = a K tile row block from LDS,
//     B = the wave's queries, held in registers for the whole key loop.  The
//     accumulator gives each lane one query column and 16 key rows, so the
//     running max and sum stay in the lane (plus one exchange with lane^32,
//     a VALU permute).
//   logits in log2 units: t = s * scale * log2(e) + log2(count), computed as
//     (s + log2(count) / (scale * log2(e))) * scale * log2(e): the accumulators
//     start at the divided shift, and each weight is one FMA and one exp2
//     (the shifts are divided once per call by a small kernel).  The running
//     max is refreshed lazily (only when a tile's max exceeds it by more than
//     8), which keeps every weight <= 2^8 and skips most rescales of O.
//   O^T += V^T P^T: B = the probabilities, converted to bf16 in registers in
//     exactly the k-order the accumulator produced them; A = 8 keys of one
//     feature, gathered from row-major V in LDS by transposing LDS reads.
//   K, V (and log2-count) tiles move HBM -> LDS with direct-to-LDS loads into
//     a ring of buffers ahead of the tile in use (slot tiles as buffer loads:
//     scalar tile offset, fixed lane offsets): 128-key tiles in a ring of two
//     for the plain step, 64-key tiles in a ring of four for the others.
//     One wave per SIMD issues them; the other starts its QK^T right after
//     each barrier, so the two run their MFMA and softmax phases offset.
//     In a head's last query tile, waves that hold only padding queries
//     still issue copies and meet the barriers but skip the tile work.
//   Blocks are renumbered so each XCD (blocks are dealt round-robin over the 8
//     XCDs) gets a contiguous range of (head, query tile) and shares its L2.
//   The normalised output tile leaves through LDS as whole rows.  When the
//     grid's last round of workgroups would leave a quarter or more of the
//     CUs idle, its (head, query tile) pairs run as four key-tile quarters
//     each, and a combine kernel merges the quarters' partial results.
// f32 path (small fp32 workloads): sixteen key parts per query (four waves on
// every fourth 16-key tile, four lanes per query inside a tile), fp32 online
// softmax, parts merged by lane exchanges and through LDS.
#include <algorithm>

#include "common.hpp"

namespace fastar {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
// Half of the waves (one per SIMD) issue a tile's copies; the other half
// starts its QK^T right after each barrier, so the two waves of a SIMD run
// their MFMA and softmax phases offset from each other.  The AnnCA launch
// that selects in its prologue attends over a few tiles only, and there all
// waves issue (its start-up copies are then spread over twice the waves).
#ifndef FASTAR_ATTN_IW_DIV
#define FASTAR_ATTN_IW_DIV 2
#endif
#ifndef FASTAR_ATTN_SKIPW
#define FASTAR_ATTN_SKIPW 1
#endif
#ifndef FASTAR_ATTN_IW_DIV_SEL
#define FASTAR_ATTN_IW_DIV_SEL 1
#endif

// The values of lanes l and l ^ 32 in every lane, lower half's first:
// v_permlane32_swap exchanges the two 32-lane halves in the VALU, without the
// LDS round trip of a lane shuffle.
__device__ __forceinline__ void half_pair(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  lo = __int_as_float(r[0]);
  hi = __int_as_float(r[1]);
}

// Logit shifts of a raw-token key tile of 64 rows: 64 zeros, then 64 -inf.
// A tile with r rows left reads its 64 shifts from entry 64 - r on, so rows
// past the chunk get -inf by the same LDS copy that brings slot tiles their
// log2-counts, with no masking in registers.
constexpr int kRawTile = 64;
struct RawShifts {
  float v[2 * kRawTile];
};
constexpr RawShifts make_raw_shifts() {
  RawShifts t{};
  for (int i = 0; i < 2 * kRawTile; ++i) t.v[i] = i < kRawTile ? 0.0f : -__builtin_huge_valf();
  return t;
}
__device__ const RawShifts raw_shifts = make_raw_shifts();


// Sixteen key parts per query: the 16 queries of a block are shared by its 4
// waves, wave p taking key tiles p, p+4, ..., and inside a wave the four lanes
// of a query take one key of every four of the tile; each part keeps its own
// running max, sum and output, merged by lane exchanges and then through LDS.
constexpr int kF32Parts = 4;     // waves per block, one key tile each per round
constexpr int kF32Queries = 16;  // queries per block (lanes qq, qq+16, qq+32, qq+48)
constexpr int kF32Subparts = 64 / kF32Queries;
constexpr int kF32Tile = 16;
template <int D>
constexpr size_t attend_f32_lds_bytes() {
  const size_t tiles = (size_t)kF32Parts * (2 * kF32Tile * D + kF32Tile);
  const size_t parts = (size_t)2 * kF32Queries * (D + 2);
  return 4 * (tiles > parts ? tiles : parts);
}

template <int D, bool GATHER>
__global__ __launch_bounds__(64 * kF32Parts) void attend_f32_kernel(AttendArgs a, int qtiles) {
  constexpr int KT = kF32Tile, P = kF32Parts;
  extern __shared__ __attribute__((aligned(16))) float f32_lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int qq = lane & (kF32Queries - 1), sub = lane / kF32Queries;  // query, key sub-part
  const int part = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  float* Ks = f32_lds + part * (2 * KT * D + KT);
  float* Vs = Ks + KT * D;
  float* lbs = Vs + KT * D;
  const int per_head = a.F * qtiles;
  const int h = blockIdx.x / per_head;
  const int g = (blockIdx.x - h * per_head) / qtiles;
  const int qt = blockIdx.x - h * per_head - g * qtiles;
  const int qi = qt * kF32Queries + qq;
  const bool ok = qi < a.Nseg;
  const int nkeys = a.n_keys ? a.n_keys[h * a.F + g] : a.n_keys_const;
  const float cscale = a.scale * kLog2e;
  const float* qp = static_cast<const float*>(a.q) + (int64_t)h * a.sq_h +
                    (int64_t)(g * a.Nseg + (ok ? qi : 0)) * a.sq_n;
  const float* kbase = static_cast<const float*>(a.k) + (int64_t)h * a.sk_h;
  const float* vbase = static_cast<const float*>(a.v) + (int64_t)h * a.sk_h;
  const int32_t* cnt = a.count ? a.count + (int64_t)h * a.count_ld : nullptr;
  const int32_t* sel = GATHER ? a.sel + (int64_t)(h * a.F + g) * a.sel_ld : nullptr;
  // raw tokens after the keys (count 1): key nkeys + j is row j of xk / xv
  const int ntot = nkeys + a.n_x;
  const float* xkb = a.n_x ? static_cast<const float*>(a.xk) + (int64_t)h * a.sx_h : nullptr;
  const float* xvb = a.n_x ? static_cast<const float*>(a.xv) + (int64_t)h * a.sx_h : nullptr;

  float qv[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = ok ? qp[e] : 0.0f;
    o[e] = 0.0f;
  }
  float mrun = -__builtin_huge_valf(), l = 0.0f;
  const int ntiles = (ntot + KT - 1) / KT;
  for (int t0 = 0; t0 < ntiles; t0 += P) {  // block-uniform
    const int tile = t0 + part;
    const int k0 = tile * KT;
    if (tile < ntiles) {
      // eight elements of K and of V per lane in flight before their stores
      constexpr int kBatch = 8;
      static_assert((KT * D / 64) % kBatch == 0, "tile elements per lane");
#pragma unroll
      for (int i0 = 0; i0 < KT * D / 64; i0 += kBatch) {
        float kx[kBatch], vx[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int idx = lane + 64 * (i0 + u);
          const int r = idx / D, e = idx % D;
          const int key = k0 + r;
          kx[u] = 0.0f;
          vx[u] = 0.0f;
          if (key < nkeys) {
            const int src = GATHER ? sel[key] : key;
            kx[u] = kbase[(int64_t)src * a.sk_n + e];
            vx[u] = vbase[(int64_t)src * a.sk_n + e];
          } else if (key < ntot) {
            kx[u] = xkb[(int64_t)(key - nkeys) * a.sx_n + e];
            vx[u] = xvb[(int64_t)(key - nkeys) * a.sx_n + e];
          }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          Ks[lane + 64 * (i0 + u)] = kx[u];
          Vs[lane + 64 * (i0 + u)] = vx[u];
        }
      }
      if (lane < KT) {
        const int key = k0 + lane;
        float lbv = -__builtin_huge_valf();
        if (key < nkeys) {
          const int src = GATHER ? sel[key] : key;
          lbv = cnt ? log2f((float)cnt[src]) : 0.0f;
        } else if (key < ntot) {
          lbv = 0.0f;
        }
        lbs[lane] = lbv;
      }
    }
    __syncthreads();
    const int nr = tile < ntiles ? min(KT, ntot - k0) : 0;
    // this lane's keys of the tile: sub, sub + 4, sub + 8, sub + 12, scored
    // together with one rescale test.  Tile rows past the last key hold zero
    // rows and a -inf shift, so they add nothing; key `sub` is real whenever
    // sub < nr, which makes the running max finite before any weight.
    static_assert(KT == 4 * kF32Subparts, "four keys per lane and tile");
    if (sub < nr) {
      float t4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4* kr = reinterpret_cast<const float4*>(Ks + (sub + kF32Subparts * j) * D);
        float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int e4 = 0; e4 < D / 4; ++e4) {
          const float4 kv = kr[e4];
          d4[0] = __builtin_fmaf(qv[4 * e4 + 0], kv.x, d4[0]);
          d4[1] = __builtin_fmaf(qv[4 * e4 + 1], kv.y, d4[1]);
          d4[2] = __builtin_fmaf(qv[4 * e4 + 2], kv.z, d4[2]);
          d4[3] = __builtin_fmaf(qv[4 * e4 + 3], kv.w, d4[3]);
        }
        t4[j] = ((d4[0] + d4[1]) + (d4[2] + d4[3])) * cscale + lbs[sub + kF32Subparts * j];
      }
      const float tm = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
      if (tm > mrun) {
        const float alpha = exp2f(mrun - tm);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] *= alpha;
        mrun = tm;
      }
      float p4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p4[j] = exp2f(t4[j] - mrun);
        l += p4[j];
      }
#pragma unroll
      for (int e4 = 0; e4 < D / 4; ++e4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 vv =
              reinterpret_cast<const float4*>(Vs + (sub + kF32Subparts * j) * D)[e4];
          o[4 * e4 + 0] = __builtin_fmaf(p4[j], vv.x, o[4 * e4 + 0]);
          o[4 * e4 + 1] = __builtin_fmaf(p4[j], vv.y, o[4 * e4 + 1]);
          o[4 * e4 + 2] = __builtin_fmaf(p4[j], vv.z, o[4 * e4 + 2]);
          o[4 * e4 + 3] = __builtin_fmaf(p4[j], vv.w, o[4 * e4 + 3]);
        }
      }
    }
    __syncthreads();
  }
  // merge the parts: a part that saw no key (running max -inf) adds nothing.
  // First the four sub-parts of each query inside a wave (lanes qq, qq+16,
  // qq+32, qq+48, by two lane exchanges), then the waves: 2 and 3 hand over to
  // 0 and 1 through LDS, then 1 to 0.
  auto merge_with = [&](float m2, float l2, const float* o2, int o2_stride)
      __attribute__((always_inline)) {
    const float m = fmaxf(mrun, m2);
    if (m == -__builtin_huge_valf()) return;
    const float w1 = exp2f(mrun - m), w2 = exp2f(m2 - m);
    l = l * w1 + l2 * w2;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = o[e] * w1 + o2[e * o2_stride] * w2;
    mrun = m;
  };
#pragma unroll
  for (int x = kF32Queries; x < 64; x <<= 1) {
    float o2[D];
#pragma unroll
    for (int e = 0; e < D; ++e) o2[e] = __shfl_xor(o[e], x);
    const float m2 = __shfl_xor(mrun, x), l2 = __shfl_xor(l, x);
    merge_with(m2, l2, o2, 1);
  }
  constexpr int kRow = D + 2;
  auto hand_over = [&](float* dst) __attribute__((always_inline)) {
    if (sub != 0) return;  // the four sub-part lanes of a query now agree
    dst[qq * kRow] = mrun;
    dst[qq * kRow + 1] = l;
#pragma unroll
    for (int e = 0; e < D; ++e) dst[qq * kRow + 2 + e] = o[e];
  };
  auto absorb = [&](const float* src) __attribute__((always_inline)) {
    merge_with(src[qq * kRow], src[qq * kRow + 1], src + qq * kRow + 2, 1);
  };
  float* R0 = f32_lds;
  float* R1 = f32_lds + kF32Queries * kRow;
  if (part >= 2) hand_over(part == 2 ? R0 : R1);
  __syncthreads();
  if (part < 2) absorb(part == 0 ? R0 : R1);
  __syncthreads();
  if (part == 1) hand_over(R0);
  __syncthreads();
  if (part != 0 || sub != 0) return;
  absorb(R0);
  if (!ok) return;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float* op = static_cast<float*>(a.o) + (int64_t)h * a.so_h + (int64_t)(g * a.Nseg + qi) * a.so_n;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = o[e] * inv;
  if (a.lse)
    a.lse[(int64_t)h * a.F * a.Nseg + (int64_t)g * a.Nseg + qi] =
        l > 0.0f ? (mrun + log2f(l)) * kLn2 : -__builtin_huge_valf();
}

// ---------------------------------------------------------------------------
// Attention over a bf16 cache in its own layout: K and V mirror rows
// [H][Bp][D] and lb = log2(count) per slot with -inf past n_live.  Tiles of BN
// slots are copied HBM -> LDS with direct-to-LDS loads (no registers in
// between), the 16-byte chunks of every K and V row permuted by row so that
// the operand reads below are bank-conflict free.  K rows feed S^T = K Q^T
// directly (a lane reads 8 consecutive features of one key).  For
// O^T += V^T P^T a lane needs 8 keys of one feature: gfx950's transposing LDS
// read (ds_read_b64_tr_b16) gathers them from row-major V, 4 keys per read.
// Slots past n_live inside the last tile have zero rows and lb = -inf, so they
// need no masking.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(1))) void gbl_void_t;

template <int D, int BN, int WAVES, int QB>
struct CCfg {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int BM = WAVES * 32 * QB;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kRowChunks = D / 8;
  static constexpr int kKBytes = BN * D * 2;
  static constexpr int kVBytes = BN * D * 2;
  static constexpr int kBuf = kKBytes + kVBytes + BN * 4;
  static constexpr int kKInstr = kKBytes / 1024;  // wave-wide 1 KiB direct loads per tile
  static_assert(kKBytes % 1024 == 0 && kBuf % 16 == 0, "tile shape");
  static_assert(kKInstr % WAVES == 0, "the copies divide evenly among the waves");
  // LDS chunk permutations (XOR on the 16-byte chunk index of a row).  K: a
  // wave reads one chunk of 32 consecutive rows.  V: a half-wave reads 4
  // chunks (32 features) of 4 consecutive rows, which this spreads over all
  // 64 banks (D = 128: row r's chunks move by 4*(r%4); D = 64, two rows per
  // 256 bytes: by 4*((r/2)%2)).
  static __device__ __forceinline__ int kswz(int row) { return row & (kRowChunks - 1); }
  static __device__ __forceinline__ int vswz(int row) {
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
  }
};

// AnnCA selection by one workgroup of 512 threads for frame g of head h (FAST-AR
// summary, section 2B "Mecanismo": a prompt token is kept for a frame iff it
// shares a bucket with at least one of the frame's queries).  Every code of
// the frame's queries sets a bit of its table's 2^16-bit LDS bitmap; each
// prompt code tests its bit; the kept rows are compacted into `sel` in
// ascending order.  Uses the ring buffers' LDS before any copy is issued:
// bitmaps in `bmb`, keep flags in `kf`.  Returns the kept count
// (block-uniform).
__device__ int annca_select_in_block(const AttendArgs& sa, int h, int g, uint8_t* kf,
                                     uint8_t* bmb, int32_t* sel) {
  constexpr int kThreads = 512, kWaves = kThreads / 64;
  __shared__ int s_cnt[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = sa.sel_L, Np = sa.n_keys_const, Nf = sa.Nseg;
  uint32_t* bm = reinterpret_cast<uint32_t*>(bmb);  // [L][2048]
  for (int i = tid; i < L * 512; i += kThreads) reinterpret_cast<uint4*>(bm)[i] = uint4{0, 0, 0, 0};
  // the frame's codes: table t holds Nf consecutive words per head row.  A
  // thread requests up to kPer codes of every table before its first bitmap
  // update, so the loads are in flight together.
  constexpr int kPer = 4;
  const int64_t nq = (int64_t)sa.F * Nf;
  const uint32_t* qc = sa.q_codes + (int64_t)h * L * nq + (int64_t)g * Nf;
  // the prompt codes of row tid are requested now too (the first pass of the
  // test below uses them)
  const uint32_t* pc = sa.p_codes + (int64_t)h * L * Np;
  uint32_t pc0[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) pc0[t] = t < L && tid < Np ? pc[(int64_t)t * Np + tid] : 0xffffffffu;
  __syncthreads();
  for (int r0 = 0; r0 < Nf; r0 += kPer * kThreads) {
    uint32_t cv[4][kPer];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int r = r0 + u * kThreads + tid;
        cv[t][u] = t < L && r < Nf ? qc[(int64_t)t * nq + r] : 0xffffffffu;
      }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (cv[t][u] < 65536u) atomicOr(&bm[t * 2048 + (cv[t][u] >> 5)], 1u << (cv[t][u] & 31u));
  }
  __syncthreads();
  // prompt codes test their bits
  for (int j = tid; j < Np; j += kThreads) {
    uint32_t code[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      code[t] = j == tid ? pc0[t] : t < L ? pc[(int64_t)t * Np + j] : 0xffffffffu;
    uint32_t hit = 0u;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      hit |= code[t] >> 16 ? 0u : (bm[t * 2048 + (code[t] >> 5)] >> (code[t] & 31u)) & 1u;
    kf[j] = (uint8_t)hit;
  }
  __syncthreads();
  // kept ids in ascending order: each thread a contiguous run, a block scan
  const int per = (Np + kThreads - 1) / kThreads;
  const int lo = min(Np, tid * per), hi = min(Np, lo + per);
  int cnt = 0;
  for (int j = lo; j < hi; ++j) cnt += kf[j];
  int x = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_cnt[wave] = x;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    base += w < wave ? s_cnt[w] : 0;
    total += s_cnt[w];
  }
  int pos = base + x - cnt;
  for (int j = lo; j < hi; ++j)
    if (kf[j]) sel[pos++] = j;
  __syncthreads();
  return total;
}

// One 16-byte-per-lane direct-to-LDS copy through a buffer load: `base` and
// `bytes` describe the rows as a buffer resource (descriptor word 3: raw
// 32-bit data, no swizzle), `soff` is the tile's byte offset (a scalar) and
// `voff` the lane's fixed byte offset inside the tile, so a copy needs no
// vector address arithmetic.
__device__ __forceinline__ void copy16_lds(const uint8_t* base, int bytes, uint32_t voff, int soff,
                                           lds_void_t* dst) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// QB blocks of 32 queries per wave: every K or V fragment read from LDS feeds
// QB MFMAs, which is what keeps the kernel below the LDS bandwidth (one 1 KiB
// operand per 32x32x16 MFMA would need all 128 B/clk of a CU's LDS).
// SUBSET = false: attention over the cache (mirror rows, log2-count bias, the
// live count of each head).  SUBSET = true: every segment (frame) of sa.Nseg
// queries attends over rows of arbitrary [H][N][d] key and value arrays with
// no bias: all sa.n_keys_const rows, or the first n_keys[h][g] rows of the
// segment's gather list sa.sel, staged in LDS at the start.
template <int D, int BN, int WAVES, int QB, int NBUF, bool SUBSET, bool RAW, bool REG,
          bool SEL = false>
__global__ __launch_bounds__(WAVES * 64, QB == 1 ? 2 : 1) void attend_cache_kernel(
    Dims dm, CacheDev c, CacheAttendArgs a, AttendArgs sa, int qtiles) {
  using C = CCfg<D, BN, WAVES, QB>;
  static_assert(NBUF >= 2 && NBUF <= 4, "ring depth");
  static_assert(!SEL || (SUBSET && NBUF == 4 && D == 128), "selection in the kernel");
  extern __shared__ int32_t sel_lds[];  // SUBSET with a gather list
  // A ring of NBUF distinct LDS objects: tile it is read from one while the
  // copies of tiles it+1 .. it+NBUF-1 are in flight into the others.  Distinct
  // objects let the compiler see that the reads never alias the copies in
  // flight.
  __shared__ __attribute__((aligned(16))) uint8_t buf0[C::kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[C::kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t buf2[NBUF >= 3 ? C::kBuf : 16];
  __shared__ __attribute__((aligned(16))) uint8_t buf3[NBUF == 4 ? C::kBuf : 16];
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform by construction: keeps the barrier paths below scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, hf = lane >> 5;
  int h, g, qt;
  // part >= 0: this workgroup attends key-tile quarter `part` of the split
  // pair sp (pair a.nfull + sp); the whole pairs take the first a.nfull
  // workgroup ids, so they are dispatched first, and the quarters fill the
  // last round.  Each range is renumbered for the XCDs on its own.
  int part = -1, sp = 0;
  if constexpr (SUBSET) {
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int per_head = sa.F * qtiles;
    h = lid / per_head;
    g = (lid - h * per_head) / qtiles;
    qt = lid - h * per_head - g * qtiles;
  } else {
    int lid;
    if ((int)blockIdx.x < a.nfull) {
      lid = xcd_remap(blockIdx.x, a.nfull);
    } else {
      const int q4 = xcd_remap(blockIdx.x - a.nfull, gridDim.x - a.nfull);
      sp = q4 >> 2;
      part = q4 & 3;
      lid = a.nfull + sp;
    }
    h = lid / qtiles;
    g = 0;
    qt = lid - h * qtiles;
  }
  // queries, outputs, key/value rows of this block
  const int Np = SUBSET ? sa.n_keys_const : 0;  // rows of the subset arrays
  const float cscale = (SUBSET ? sa.scale : a.scale) * kLog2e;
  const int nq = SUBSET ? sa.Nseg : a.Nq;
  const int64_t sq_n = SUBSET ? sa.sq_n : a.sq_n, so_n = SUBSET ? sa.so_n : a.so_n;
  const uint16_t* qbase =
      SUBSET ? static_cast<const uint16_t*>(sa.q) + (int64_t)h * sa.sq_h + (int64_t)g * sa.Nseg * sa.sq_n
             : static_cast<const uint16_t*>(a.q) + (int64_t)h * a.sq_h;
  // queries of this wave: qi = qt*BM + wave*32*QB + qb*32 + m (requested
  // first, so that their latency overlaps the selection below)
  bf16x8_t Qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qt * C::BM + (wave * QB + qb) * 32 + m;
    const bool qok = qi < nq;
    const uint16_t* qp = qbase + (int64_t)(qok ? qi : 0) * sq_n + hf * (D / 2);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qp + ks * 8);
      if (!qok) v = bf16x8_t{};
      Qf[qb][ks] = v;
    }
  }
  int nkeys_sel = 0;
  if constexpr (SEL) nkeys_sel = annca_select_in_block(sa, h, g, buf1, buf3, sel_lds);
  const int nkeys = SEL      ? nkeys_sel
                    : SUBSET ? (sa.n_keys ? min(max(sa.n_keys[h * sa.F + g], 0), Np) : Np)
                             : c.n_live[h];
  uint16_t* obase =
      SUBSET ? static_cast<uint16_t*>(sa.o) + (int64_t)h * sa.so_h + (int64_t)g * sa.Nseg * sa.so_n
             : static_cast<uint16_t*>(a.o) + (int64_t)h * a.so_h;
  float* lse_row = SUBSET ? (sa.lse ? sa.lse + (int64_t)(h * sa.F + g) * sa.Nseg : nullptr)
                          : (a.lse ? a.lse + (int64_t)h * a.Nq : nullptr);
  // REG: keys (and shifts) from the M-degree regions, r * Bp rows apart
  const uint8_t* kg =
      SUBSET ? static_cast<const uint8_t*>(sa.k) + (int64_t)h * sa.sk_h * 2
      : REG  ? reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(c.rope_k) +
                                                (int64_t)h * dm.R * dm.Bp * D)
             : reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(c.k_mirror) +
                                                (int64_t)h * dm.Bp * D);
  const uint8_t* vg =
      SUBSET ? static_cast<const uint8_t*>(sa.v) + (int64_t)h * sa.sk_h * 2
             : reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(c.v_mirror) +
                                                (int64_t)h * dm.Bp * D);
  const int64_t rs = SUBSET ? sa.sk_n * 2 : C::kRowBytes;  // bytes between key rows
  // slot shifts divided by the logit scale (written by scale_shift_kernel
  // just before this launch), so they can start the QK^T accumulators
  const float* lbg = SUBSET ? nullptr
                     : REG  ? c.lbc + (int64_t)h * dm.R * dm.Bp
                            : c.lbc + (int64_t)h * dm.Bp;
  // RAW: raw tokens (count 1, no logit shift) follow the slots: key tiles
  // ntc .. of the loop read rows of a.xk / a.xv, rows past a.n_x read row 0
  // and are masked by their bias.
  static_assert(!(RAW && SUBSET), "raw tokens follow cache slots only");
  static_assert(!(REG && (RAW || SUBSET)), "regions replace the slots' keys only");
  const int ntc = (nkeys + BN - 1) / BN;
  const int nx = RAW ? a.n_x : 0;
  const uint8_t* xkg = nx ? static_cast<const uint8_t*>(a.xk) + (int64_t)h * a.sx_h * 2 : nullptr;
  const uint8_t* xvg = nx ? static_cast<const uint8_t*>(a.xv) + (int64_t)h * a.sx_h * 2 : nullptr;
  const int64_t xrs = SUBSET ? 0 : a.sx_n * 2;  // bytes between raw rows
  const bool gather = SEL || (SUBSET && sa.sel != nullptr);  // block-uniform
  if (gather && !SEL) {
    const int32_t* sel = sa.sel + (int64_t)(h * sa.F + g) * sa.sel_ld;
    for (int i = tid; i < nkeys; i += C::kThreads) sel_lds[i] = min(max(sel[i], 0), Np - 1);
    __syncthreads();
  }

  // Copy addresses: a wave-uniform tile offset plus per-lane byte offsets that
  // do not change from tile to tile, so issuing a slot tile's copy costs no
  // vector math.
  // The first IW waves issue the copies: wave w copies the 1 KiB chunks w,
  // w + IW, ... of the K and V tiles; LDS position (row, chunk) receives
  // global chunk chunk ^ swz(row).
  // In a subset, a lane's source row is looked up per tile instead (rows past
  // the kept count read row 0 and are masked by their bias).
  constexpr int IW = SEL ? WAVES / FASTAR_ATTN_IW_DIV_SEL : WAVES / FASTAR_ATTN_IW_DIV;  // waves that issue the copies
  constexpr int kPerWave = C::kKInstr / IW;
  const bool iw = wave < IW;  // wave-uniform
  uint32_t koff[kPerWave], voff[kPerWave];
  int rrow[kPerWave];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int off = (wave % IW + j * IW) * 1024 + lane * 16;
    const int row = off / C::kRowBytes;
    const int slot = (off - row * C::kRowBytes) >> 4;
    rrow[j] = row;
    const int rb = SUBSET ? 0 : row * C::kRowBytes;
    koff[j] = (uint32_t)(rb + ((slot ^ C::kswz(row)) << 4));
    voff[j] = (uint32_t)(rb + ((slot ^ C::vswz(row)) << 4));
  }
  // the head's K (and region) rows and V rows, as buffer sizes for the copies
  const int kbytes = SUBSET ? 0 : (REG ? dm.R * dm.Bp : dm.Bp) * C::kRowBytes;
  const int vbytes = SUBSET ? 0 : dm.Bp * C::kRowBytes;
  auto issue = [&](int k0, uint8_t* buf) __attribute__((always_inline)) {
    const bool raw = RAW && k0 >= ntc * BN;  // block-uniform
    // REG: tile k0/BN is tile u of region r; K and shift rows r*Bp + u*BN, V rows u*BN
    int kr = k0, vr = k0;
    if constexpr (REG) {
      const int tr = k0 / BN, r = tr / ntc, u = tr - r * ntc;
      kr = r * dm.Bp + u * BN;
      vr = u * BN;
    }
    const uint8_t* kt = kg + (SUBSET || raw ? 0 : (int64_t)kr * C::kRowBytes);
    const uint8_t* vt = vg + (SUBSET || raw ? 0 : (int64_t)vr * C::kRowBytes);
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      if (!iw) break;
      const int i = wave + j * IW;
      if constexpr (!SUBSET) {
        if (!raw) {  // slot tiles: scalar tile offset, fixed lane offsets
          copy16_lds(kg, kbytes, koff[j], kr * C::kRowBytes, (lds_void_t*)(buf + i * 1024));
          copy16_lds(vg, vbytes, voff[j], vr * C::kRowBytes,
                     (lds_void_t*)(buf + C::kKBytes + i * 1024));
          continue;
        }
      }
      const uint8_t* ks;
      const uint8_t* vs;
      if constexpr (SUBSET) {
        const int key = k0 + rrow[j];
        const int64_t ro = (int64_t)(key < nkeys ? (gather ? sel_lds[key] : key) : 0) * rs;
        ks = kt + ro + koff[j];
        vs = vt + ro + voff[j];
      } else if (raw) {  // koff / voff hold the mirror row offset; swap it for the raw row's
        const int key = k0 - ntc * BN + rrow[j];
        const int64_t ro = (int64_t)(key < nx ? key : 0) * xrs - rrow[j] * C::kRowBytes;
        ks = xkg + ro + koff[j];
        vs = xvg + ro + voff[j];
      } else {
        ks = kt + koff[j];
        vs = vt + voff[j];
      }
      __builtin_amdgcn_global_load_lds((gbl_void_t*)ks, (lds_void_t*)(buf + i * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)vs, (lds_void_t*)(buf + C::kKBytes + i * 1024),
                                       16, 0, 0);
    }
    // the bias row: slots' log2-counts, or for a raw or subset tile zeros up
    // to the last kept row and -inf past it
    static_assert((!RAW && !SUBSET) || BN == kRawTile, "constant shifts cover one 64-row tile");
    const float* lsrc = SUBSET ? nullptr : lbg + kr;
    if (SUBSET || (RAW && raw)) {
      // rows of the chunk, or of the kept subset, in the tile
      const int left = min(max(SUBSET ? nkeys - k0 : nx - (k0 - ntc * BN), 0), BN);
      lsrc = raw_shifts.v + (BN - left);
    }
#pragma unroll
    for (int i = 0; i < (BN + 63) / 64; ++i) {
      if (wave == (IW - 1 - i) % IW && i * 64 + lane < BN)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(lsrc + i * 64 + (uint32_t)lane),
                                         (lds_void_t*)(buf + C::kKBytes + C::kVBytes + i * 256), 4, 0, 0);
    }
  };

  // Transposing V reads: within each 16-lane group, source lane j reads 4
  // features (8 bytes) of key row 4*hf + j/4 at feature 16*(group%2) + 4*(j%4)
  // of a 32-feature block; lane i then holds 4 consecutive keys of feature
  // 16*(group%2) + i.  Offsets per feature block; the key offset of a tile
  // (a multiple of 8 rows) leaves the chunk permutation unchanged.
  uint32_t vtr[D / 32];
  {
    const int j = lane & 15;
    const int row = 4 * hf + (j >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      vtr[db] = (uint32_t)(row * C::kRowBytes + (((col >> 3) ^ C::vswz(row)) << 4) + (col & 7) * 2);
    }
  }
  f32x16_t O[D / 32][QB];
  float mrun[QB], lrun[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrun[qb] = -__builtin_huge_valf();
    lrun[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) O[db][qb] = f32x16_t{};
  }

  // Copies an issuing wave makes per tile: K and V chunks, plus the bias row
  // for the last issuing wave(s).  The others have none in flight, so their
  // waits below pass at once and the barrier orders them after the copies.
  constexpr int kCopies = 2 * C::kKInstr / IW;
  const bool lb_wave = iw && wave >= IW - (BN + 63) / 64;

  // Wait until at most n tiles' copies issued by this wave are in flight
  // (every older tile has landed), finish this wave's LDS reads, then meet
  // the other waves.  A plain barrier, not __syncthreads(): the latter's
  // fence would also wait for the copies that are meant to stay in flight.
  auto wait_barrier = [&](int n) __attribute__((always_inline)) {
    if (lb_wave) {
      if (n >= 2) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * (kCopies + 1)) : "memory");
      else if (n == 1) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kCopies + 1) : "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      if (n >= 2) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * kCopies) : "memory");
      else if (n == 1) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kCopies) : "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };

  // One key tile: read `cur`, issue the copy of tile it+NBUF-1 into `nxt`
  // (the buffer read in the previous step).
  auto compute = [&](const uint8_t* cur) __attribute__((always_inline)) {
    const uint8_t* vt_lds = cur + C::kKBytes;
    const float* lb_lds = reinterpret_cast<const float*>(cur + C::kKBytes + C::kVBytes);

    // The accumulators start at the tile's shifts (already divided by the
    // logit scale): the rows of lane (m, hf) are 8*jg + 4*hf + 0..3 of each
    // 32-key block, so S = K Q^T + shift / scale directly.
    f32x16_t S[BN / 32][QB];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      f32x16_t init;
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const float4 b4 = *reinterpret_cast<const float4*>(lb_lds + kb * 32 + 8 * jg + 4 * hf);
        init[4 * jg + 0] = b4.x;
        init[4 * jg + 1] = b4.y;
        init[4 * jg + 2] = b4.z;
        init[4 * jg + 3] = b4.w;
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[kb][qb] = init;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        const int row = kb * 32 + m;
        const int chunk = hf * (D / 16) + ks;
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
            cur + row * C::kRowBytes + ((chunk ^ C::kswz(row)) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, Qf[qb][ks], S[kb][qb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // the tile's largest logit in log2 units: the scale is positive, so it
      // is the scale times the largest accumulator
      float sx = -__builtin_huge_valf();
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sx = fmaxf(sx, S[kb][qb][r]);
      float mx = sx * cscale;
      {
        float lo, hi;
        half_pair(mx, lo, hi);
        mx = fmaxf(lo, hi);
      }
      const bool need = mx > mrun[qb] + 8.0f;
      if (__ballot(need)) {
        const float mnew = need ? mx : mrun[qb];
        const float alpha = __builtin_amdgcn_exp2f(mrun[qb] - mnew);
        lrun[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) O[db][qb][j] *= alpha;
        mrun[qb] = mnew;
      }
    }
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // A operand: feature db*32 + m, keys kb*32 + kk*16 + {4*hf..4*hf+3}
        // then {8+4*hf..8+4*hf+3}, the key order of the P fragment
        const uint8_t* vrow = vt_lds + (kb * 32 + kk * 16) * C::kRowBytes;
        bf16x8_t pf[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            pf[qb][i] = (__bf16)__builtin_amdgcn_exp2f(
                __builtin_fmaf(S[kb][qb][8 * kk + i], cscale, -mrun[qb]));
          // row sum of the same bf16-rounded weights the MFMA multiplies
          float ls = lrun[qb];
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            const bf16x2_t pp = {pf[qb][i], pf[qb][i + 1]};
            ls = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ls, false);
          }
          lrun[qb] = ls;
          // keep the sum beside the conversions, while the packed weights are
          // still in registers (else it sinks into the next tile and some
          // weights are converted again)
          asm volatile("" : "+v"(lrun[qb]));
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t*)(vrow + vtr[db]));
          const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t*)(vrow + vtr[db] + 8 * C::kRowBytes));
          const bf16x8_t vf = __builtin_bit_cast(
              bf16x8_t, (v8i16_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            O[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb], O[db][qb], 0, 0, 0);
        }
      }
    }
  };
  const int nt_all = REG ? a.n_reg * ntc : ntc + (nx + BN - 1) / BN;
  // key tiles [tb, tb + nt) of this workgroup (a quarter may be empty)
  const int tb = part < 0 ? 0 : part * nt_all / 4;
  const int nt = part < 0 ? nt_all : (part + 1) * nt_all / 4 - tb;
  // A wave whose queries all lie past the last one (the last query tile of a
  // head) still issues its copies and meets every barrier, but skips the
  // MFMA and softmax work, leaving its SIMD to the other wave there.
  const bool wq = FASTAR_ATTN_SKIPW == 0 || qt * C::BM + wave * QB * 32 < nq;  // wave-uniform
  auto step = [&](const uint8_t* cur, uint8_t* nxt, int it, int nt) __attribute__((always_inline)) {
    if (it + NBUF - 1 < nt) issue((tb + it + NBUF - 1) * BN, nxt);
    if (wq) compute(cur);
    // Tile it+1 must have landed; the copies of tiles it+2 .. it+NBUF-1
    // stay in flight.
    wait_barrier(min(nt - 1, it + NBUF - 1) - (it + 1));
  };

  if constexpr (NBUF == 4) {
    // One barrier per two tiles: tiles it, it+1 are read while the copies of
    // it+2, it+3 land; after the barrier (every wave is done with it, it+1)
    // their buffers receive it+4, it+5.  Measured slightly faster than a
    // barrier per tile (0.5-1.3 % in same-process comparisons).
    if (0 < nt) issue(tb * BN, buf0);
    if (1 < nt) issue((tb + 1) * BN, buf1);
    if (2 < nt) issue((tb + 2) * BN, buf2);
    if (3 < nt) issue((tb + 3) * BN, buf3);
    wait_barrier(max(min(nt, 4) - 2, 0));
    for (int it = 0; it < nt; it += 4) {
      if (wq) {
        compute(buf0);
        if (it + 1 < nt) compute(buf1);
      }
      if (it + 2 < nt) {
        wait_barrier(0);
        if (it + 4 < nt) issue((tb + it + 4) * BN, buf0);
        if (it + 5 < nt) issue((tb + it + 5) * BN, buf1);
        if (wq) {
          compute(buf2);
          if (it + 3 < nt) compute(buf3);
        }
        if (it + 4 < nt) {
          wait_barrier(0);
          if (it + 6 < nt) issue((tb + it + 6) * BN, buf2);
          if (it + 7 < nt) issue((tb + it + 7) * BN, buf3);
        }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u)
      if (u < nt) issue((tb + u) * BN, u == 0 ? buf0 : u == 1 ? buf1 : buf2);
    wait_barrier(min(nt, NBUF - 1) - 1);
    for (int it = 0; it < nt; it += NBUF) {
      if (NBUF == 2) {
        step(buf0, buf1, it, nt);
        if (it + 1 < nt) step(buf1, buf0, it + 1, nt);
      } else {
        step(buf0, buf2, it, nt);
        if (it + 1 < nt) step(buf1, buf0, it + 1, nt);
        if (it + 2 < nt) step(buf2, buf1, it + 2, nt);
      }
    }
  }

  if constexpr (!SUBSET) {
    if (part >= 0) {  // block-uniform: a quarter's unnormalised result
      const int64_t base = ((int64_t)sp * 4 + part) * C::BM;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int r = (wave * QB + qb) * 32 + m;
        float llo, lhi;
        half_pair(lrun[qb], llo, lhi);
        const float lt = llo + lhi;
        float* po = c.attn_part + (base + r) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg)
            *reinterpret_cast<float4*>(po + db * 32 + 8 * jg + 4 * hf) =
                make_float4(O[db][qb][4 * jg], O[db][qb][4 * jg + 1], O[db][qb][4 * jg + 2],
                            O[db][qb][4 * jg + 3]);
        if (hf == 0) c.attn_ml[base + r] = make_float2(mrun[qb], lt);
      }
      return;
    }
  }
  // The output tile goes through LDS, so that global stores write whole rows:
  // each wave normalises its 32*QB rows into its own region of the ring (free
  // once every wave has left the key loop), 16-byte chunk c of row r at
  // c ^ (r mod chunks), then stores 16 bytes per lane with a row's chunks in
  // consecutive lanes.
  constexpr int kOChunks = D / 8;              // 16-byte chunks per row
  constexpr int kORow = D * 2;                 // bytes per output row
  constexpr int kOWave = 32 * QB * kORow;
  static_assert(4 * kOWave <= C::kBuf && WAVES <= 8, "four waves' tiles per ring buffer");
  __syncthreads();
  uint8_t* ost = (wave < 4 ? buf0 : buf1) + (wave & 3) * kOWave;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qt * C::BM + (wave * QB + qb) * 32 + m;
    float llo, lhi;
    half_pair(lrun[qb], llo, lhi);
    const float lt = llo + lhi;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int r = qb * 32 + m;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const uint32_t w0 = f32_to_bf16_bits(O[db][qb][4 * jg + 0] * inv) |
                            (f32_to_bf16_bits(O[db][qb][4 * jg + 1] * inv) << 16);
        const uint32_t w1 = f32_to_bf16_bits(O[db][qb][4 * jg + 2] * inv) |
                            (f32_to_bf16_bits(O[db][qb][4 * jg + 3] * inv) << 16);
        const int cs = (db * 4 + jg) ^ (r & (kOChunks - 1));
        *reinterpret_cast<uint2*>(ost + r * kORow + cs * 16 + hf * 8) = make_uint2(w0, w1);
      }
    if (lse_row && hf == 0 && qi < nq)
      lse_row[qi] = lt > 0.0f ? (mrun[qb] + __log2f(lt)) * kLn2 : -__builtin_huge_valf();
  }
  constexpr int kORowsPer = 64 / kOChunks;     // rows per wave-wide store
  const int cc = lane % kOChunks;
#pragma unroll
  for (int i = 0; i < 32 * QB / kORowsPer; ++i) {
    const int r = i * kORowsPer + lane / kOChunks;
    const int qi = qt * C::BM + wave * QB * 32 + r;
    const uint4 v =
        *reinterpret_cast<const uint4*>(ost + r * kORow + ((cc ^ (r & (kOChunks - 1))) << 4));
    if (qi < nq) *reinterpret_cast<uint4*>(obase + (int64_t)qi * so_n + cc * 8) = v;
  }
}

// The four quarters of each split (head, query tile): per query row, the
// parts' running maxima m_p (log2 units) and sums l_p give the common max m
// and weights 2^(m_p - m); o = sum_p 2^(m_p - m) O_p / sum_p 2^(m_p - m) l_p,
// rounded to bf16 like the unsplit epilogue; a part that saw no key weight
// (l_p = 0) adds nothing.  Threads own 4 features of one row.
template <int D>
__global__ __launch_bounds__(256) void attend_combine_kernel(CacheDev c, CacheAttendArgs a,
                                                             int qtiles, int bm) {
  constexpr int kT = D / 4, kRows = 256 / kT;
  const int sp = blockIdx.y;
  const int r = blockIdx.x * kRows + (int)threadIdx.x / kT;
  const int f = ((int)threadIdx.x % kT) * 4;
  if (r >= bm) return;
  const int pair = a.nfull + sp, h = pair / qtiles, qt = pair - h * qtiles;
  const int qi = qt * bm + r;
  if (qi >= a.Nq) return;
  const int64_t base = (int64_t)sp * 4 * bm + r;
  float2 ml[4];
  float mx = -__builtin_huge_valf();
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    ml[p] = c.attn_ml[base + (int64_t)p * bm];
    if (ml[p].y > 0.0f) mx = fmaxf(mx, ml[p].x);
  }
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float l = 0.0f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (!(ml[p].y > 0.0f)) continue;
    const float w = __builtin_amdgcn_exp2f(ml[p].x - mx);
    const float4 o = *reinterpret_cast<const float4*>(c.attn_part + (base + (int64_t)p * bm) * D + f);
    l = __builtin_fmaf(ml[p].y, w, l);
    acc.x = __builtin_fmaf(o.x, w, acc.x);
    acc.y = __builtin_fmaf(o.y, w, acc.y);
    acc.z = __builtin_fmaf(o.z, w, acc.z);
    acc.w = __builtin_fmaf(o.w, w, acc.w);
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const uint32_t w0 = f32_to_bf16_bits(acc.x * inv) | (f32_to_bf16_bits(acc.y * inv) << 16);
  const uint32_t w1 = f32_to_bf16_bits(acc.z * inv) | (f32_to_bf16_bits(acc.w * inv) << 16);
  uint16_t* op = static_cast<uint16_t*>(a.o) + (int64_t)h * a.so_h + (int64_t)qi * a.so_n + f;
  *reinterpret_cast<uint2*>(op) = make_uint2(w0, w1);
  if (a.lse && f == 0)
    a.lse[(int64_t)h * a.Nq + qi] = l > 0.0f ? (mx + __log2f(l)) * kLn2 : -__builtin_huge_valf();
}

// Compute units of the current device (a split pays only when the last round
// of workgroups leaves CUs idle).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// lbc = lb / (scale * log2(e)) over every head's shift rows (-inf stays -inf).
__global__ __launch_bounds__(256) void scale_shift_kernel(const float* __restrict__ src,
                                                          float* __restrict__ dst, int64_t n,
                                                          float cscale) {
  const int64_t n4 = n / 4;
  const float4* s4 = reinterpret_cast<const float4*>(src);
  float4* d4 = reinterpret_cast<float4*>(dst);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float4 v = s4[i];
    d4[i] = make_float4(v.x / cscale, v.y / cscale, v.z / cscale, v.w / cscale);
  }
}

template <int D, int BN, int WAVES, int QB, int NBUF>
hipError_t launch_cache_cfg(const Dims& dm, const CacheDev& c, const CacheAttendArgs& a,
                            hipStream_t s) {
  using C = CCfg<D, BN, WAVES, QB>;
  const int qtiles = (a.Nq + C::BM - 1) / C::BM;
  const int pairs = dm.H * qtiles;
  if (pairs == 0) return hipSuccess;
  // The last round of workgroups: when it would leave a quarter or more of
  // the CUs idle, its r pairs run as 4r workgroups of a quarter of the key
  // tiles each (not for the M-degree regions, whose later tiles can be wholly
  // masked), and a combine kernel merges the quarters.  Caches of at least
  // 1024 slots only.
  const int cus = device_cus();
  const int r = pairs % cus;
  const bool split = a.n_reg == 0 && r > 0 && 4 * r <= 3 * cus && r <= c.attn_pairs &&
                     C::BM == attn_query_tile(dm) && dm.B >= 1024;
  CacheAttendArgs aa = a;
  aa.nfull = split ? pairs - r : pairs;
  const int blocks = split ? pairs - r + 4 * r : pairs;
  {
    // rows per head are a multiple of 128 (Bp), so n is a multiple of 4
    const int64_t n = (int64_t)dm.H * (a.n_reg > 0 ? dm.R : 1) * dm.Bp;
    const int64_t b = std::min<int64_t>((n / 4 + 255) / 256, 2048);
    hipLaunchKernelGGL(scale_shift_kernel, dim3((unsigned)b), dim3(256), 0, s,
                       a.n_reg > 0 ? c.rope_lb : c.lb, c.lbc, n, a.scale * kLog2e);
  }
  if constexpr (BN == kRawTile) {
    if (a.n_reg > 0)
      hipLaunchKernelGGL((attend_cache_kernel<D, BN, WAVES, QB, NBUF, false, false, true>),
                         dim3(blocks), dim3(C::kThreads), 0, s, dm, c, aa, AttendArgs{}, qtiles);
    else if (a.n_x > 0)
      hipLaunchKernelGGL((attend_cache_kernel<D, BN, WAVES, QB, NBUF, false, true, false>),
                         dim3(blocks), dim3(C::kThreads), 0, s, dm, c, aa, AttendArgs{}, qtiles);
    else
      hipLaunchKernelGGL((attend_cache_kernel<D, BN, WAVES, QB, NBUF, false, false, false>),
                         dim3(blocks), dim3(C::kThreads), 0, s, dm, c, aa, AttendArgs{}, qtiles);
  } else {
    // wider key tiles serve the plain step only (the launcher routes the
    // chunk tiles and the regions to 64-key tiles)
    if (a.n_reg > 0 || a.n_x > 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attend_cache_kernel<D, BN, WAVES, QB, NBUF, false, false, false>),
                       dim3(blocks), dim3(C::kThreads), 0, s, dm, c, aa, AttendArgs{}, qtiles);
  }
  if (split) {
    constexpr int kRows = 256 / (D / 4);
    hipLaunchKernelGGL(attend_combine_kernel<D>, dim3((C::BM + kRows - 1) / kRows, r), dim3(256),
                       0, s, c, aa, qtiles, C::BM);
  }
  return hipGetLastError();
}

// Subsets: 8 waves x 32 queries per workgroup per (head, segment); a gather
// list is staged in LDS (4 bytes per prompt row) beside the ring.
template <int D, int NBUF>
hipError_t launch_subset_cfg(const AttendArgs& a, hipStream_t s) {
  using C = CCfg<D, 64, 8, 1>;
  const int qtiles = (a.Nseg + C::BM - 1) / C::BM;
  const int blocks = a.H * a.F * qtiles;
  if (blocks == 0) return hipSuccess;
  const size_t lds = a.sel ? (size_t)a.n_keys_const * 4 : 0;
  auto kern = attend_cache_kernel<D, 64, 8, 1, NBUF, true, false, false>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(C::kThreads), lds, s, Dims{}, CacheDev{}, CacheAttendArgs{},
                     a, qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_annca_fused(const AttendArgs& a, hipStream_t s) {
  using C = CCfg<128, 64, 8, 1>;
  if (a.d != 128) return hipErrorInvalidValue;
  const int qtiles = (a.Nseg + C::BM - 1) / C::BM;
  const int blocks = a.H * a.F * qtiles;
  if (blocks == 0) return hipSuccess;
  const size_t lds = (size_t)a.n_keys_const * 4;
  auto kern = attend_cache_kernel<128, 64, 8, 1, 4, true, false, false, true>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(C::kThreads), lds, s, Dims{}, CacheDev{},
                     CacheAttendArgs{}, a, qtiles);
  return hipGetLastError();
}

hipError_t launch_attend_bf16(const AttendArgs& a, hipStream_t s) {
  if (a.count != nullptr) return hipErrorInvalidValue;  // no count bias on subsets
  // a gather list of up to 4096 prompt rows (16 KiB) fits beside the 4-deep
  // ring; longer lists take the 2-deep one
  const bool deep = a.sel == nullptr || a.n_keys_const <= 4096;
  if (a.d == 128) return deep ? launch_subset_cfg<128, 4>(a, s) : launch_subset_cfg<128, 2>(a, s);
  return deep ? launch_subset_cfg<64, 4>(a, s) : launch_subset_cfg<64, 2>(a, s);
}

// The plain step (slots only) takes 128-key tiles in a ring of two; the
// step with the chunk's raw tokens and the M-degree regions take 64-key
// tiles in a ring of four (their constant shift rows cover 64 keys).  At the
// 14B layer the 128-key tiles measured 1-2 % faster in same-process A/B runs:
// one max exchange, one rescale test and one tile's bookkeeping per 128 keys.
#ifndef FASTAR_PLAIN_BN
#define FASTAR_PLAIN_BN 128
#endif
#ifndef FASTAR_PLAIN_NBUF
#define FASTAR_PLAIN_NBUF 2
#endif
#ifndef FASTAR_CACHE_NBUF
#define FASTAR_CACHE_NBUF 4
#endif
#ifndef FASTAR_CACHE_BN
#define FASTAR_CACHE_BN 64
#endif
#ifndef FASTAR_CACHE_WAVES
#define FASTAR_CACHE_WAVES 8
#endif
#ifndef FASTAR_CACHE_QB
#define FASTAR_CACHE_QB 1
#endif

hipError_t launch_attend_cache_bf16(const Dims& dm, const CacheDev& c, const CacheAttendArgs& a,
                                    hipStream_t s) {
  constexpr int BN = FASTAR_CACHE_BN, W = FASTAR_CACHE_WAVES, QB = FASTAR_CACHE_QB;
  if (dm.d == 128 && a.n_reg == 0 && a.n_x == 0)
    return launch_cache_cfg<128, FASTAR_PLAIN_BN, W, QB, FASTAR_PLAIN_NBUF>(dm, c, a, s);
  if (dm.d == 128) return launch_cache_cfg<128, BN, W, QB, FASTAR_CACHE_NBUF>(dm, c, a, s);
  return launch_cache_cfg<64, 64, 4, 1, FASTAR_CACHE_NBUF>(dm, c, a, s);
}

template <int D, bool GATHER>
hipError_t launch_attend_f32_cfg(const AttendArgs& a, int qtiles, int blocks, hipStream_t s) {
  constexpr size_t lds = attend_f32_lds_bytes<D>();
  auto kern = attend_f32_kernel<D, GATHER>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * kF32Parts), lds, s, a, qtiles);
  return hipGetLastError();
}

hipError_t launch_attend_f32(const AttendArgs& a, hipStream_t s) {
  const int qtiles = (a.Nseg + kF32Queries - 1) / kF32Queries;
  const int blocks = a.H * a.F * qtiles;
  if (blocks == 0) return hipSuccess;
  const bool gather = a.sel != nullptr;
  if (a.d == 128)
    return gather ? launch_attend_f32_cfg<128, true>(a, qtiles, blocks, s)
                  : launch_attend_f32_cfg<128, false>(a, qtiles, blocks, s);
  return gather ? launch_attend_f32_cfg<64, true>(a, qtiles, blocks, s)
                : launch_attend_f32_cfg<64, false>(a, qtiles, blocks, s);
}

}  // namespace fastar
