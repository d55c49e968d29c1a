// Attention over the merged cache with the group-size logit shift (FAST-AR
// summary, section 2A, Lemma 5.1: merging identical keys is exact when values
// are averaged and each logit is shifted by its group size), and the same
// kernel over a per-frame subset of prompt keys for AnnCA (section 2B).
//
// bf16 path, per workgroup of 8 waves; each wave owns 32 queries:
//   S^T = K Q^T on the 32x32x16 bf16 MFMA: A = a K tile row block from LDS,
//     B = the wave's queries, held in registers for the whole key loop.  The
//     accumulator gives each lane one query column and 16 key rows, so the
//     running max and sum stay in the lane (plus one exchange with lane^32).
//   logits in log2 units: t = s * scale * log2(e) + log2(count).  The running
//     max is refreshed lazily (only when a tile's max exceeds it by more than
//     8), which keeps every weight <= 2^8 and skips most rescales of O.
//   O^T += V^T P^T: B = the probabilities, converted to bf16 in registers in
//     exactly the k-order the accumulator produced them; A = 8 keys of one
//     feature, gathered from row-major V in LDS by transposing LDS reads.
//   K, V (and log2-count) tiles of 64 keys move HBM -> LDS with direct-to-LDS
//     loads into a ring of buffers, several tiles ahead of the one in use.
//   Blocks are renumbered so each XCD (blocks are dealt round-robin over the 8
//     XCDs) gets a contiguous range of (head, query tile) and shares its L2.
// f32 path (small fp32 workloads): one thread per query, fp32 online softmax.
#include "common.hpp"

namespace fastar {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

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


template <int D, bool GATHER>
__global__ __launch_bounds__(64) void attend_f32_kernel(AttendArgs a, int qtiles) {
  constexpr int KT = 32;
  __shared__ float Ks[KT][D];
  __shared__ float Vs[KT][D];
  __shared__ float lbs[KT];
  const int per_head = a.F * qtiles;
  const int h = blockIdx.x / per_head;
  const int g = (blockIdx.x - h * per_head) / qtiles;
  const int qt = blockIdx.x - h * per_head - g * qtiles;
  const int tid = threadIdx.x;
  const int qi = qt * 64 + tid;
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
  for (int k0 = 0; k0 < ntot; k0 += KT) {
    for (int idx = tid; idx < KT * D; idx += 64) {
      const int r = idx / D, e = idx % D;
      const int key = k0 + r;
      float kx = 0.0f, vx = 0.0f;
      if (key < nkeys) {
        const int src = GATHER ? sel[key] : key;
        kx = kbase[(int64_t)src * a.sk_n + e];
        vx = vbase[(int64_t)src * a.sk_n + e];
      } else if (key < ntot) {
        kx = xkb[(int64_t)(key - nkeys) * a.sx_n + e];
        vx = xvb[(int64_t)(key - nkeys) * a.sx_n + e];
      }
      Ks[r][e] = kx;
      Vs[r][e] = vx;
    }
    if (tid < KT) {
      const int key = k0 + tid;
      float lbv = -__builtin_huge_valf();
      if (key < nkeys) {
        const int src = GATHER ? sel[key] : key;
        lbv = cnt ? log2f((float)cnt[src]) : 0.0f;
      } else if (key < ntot) {
        lbv = 0.0f;
      }
      lbs[tid] = lbv;
    }
    __syncthreads();
    const int nr = min(KT, ntot - k0);
    for (int r = 0; r < nr; ++r) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = __builtin_fmaf(qv[e], Ks[r][e], dot);
      const float t = dot * cscale + lbs[r];
      if (t > mrun) {
        const float alpha = exp2f(mrun - t);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] *= alpha;
        mrun = t;
      }
      const float p = exp2f(t - mrun);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = __builtin_fmaf(p, Vs[r][e], o[e]);
    }
    __syncthreads();
  }
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
  static_assert(kKInstr % WAVES == 0, "every wave issues the same number of copies");
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

// QB blocks of 32 queries per wave: every K or V fragment read from LDS feeds
// QB MFMAs, which is what keeps the kernel below the LDS bandwidth (one 1 KiB
// operand per 32x32x16 MFMA would need all 128 B/clk of a CU's LDS).
// SUBSET = false: attention over the cache (mirror rows, log2-count bias, the
// live count of each head).  SUBSET = true: every segment (frame) of sa.Nseg
// queries attends over rows of arbitrary [H][N][d] key and value arrays with
// no bias: all sa.n_keys_const rows, or the first n_keys[h][g] rows of the
// segment's gather list sa.sel, staged in LDS at the start.
template <int D, int BN, int WAVES, int QB, int NBUF, bool SUBSET, bool RAW, bool REG>
__global__ __launch_bounds__(WAVES * 64, QB == 1 ? 2 : 1) void attend_cache_kernel(
    Dims dm, CacheDev c, CacheAttendArgs a, AttendArgs sa, int qtiles) {
  using C = CCfg<D, BN, WAVES, QB>;
  static_assert(NBUF >= 2 && NBUF <= 4, "ring depth");
  extern __shared__ int32_t sel_lds[];  // SUBSET with a gather list
  // A ring of NBUF distinct LDS objects: tile it is read from one while the
  // copies of tiles it+1 .. it+NBUF-1 are in flight into the others.  Distinct
  // objects let the compiler see that the reads never alias the copies in
  // flight.
  __shared__ __attribute__((aligned(16))) uint8_t buf0[C::kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[C::kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t buf2[NBUF >= 3 ? C::kBuf : 16];
  __shared__ __attribute__((aligned(16))) uint8_t buf3[NBUF == 4 ? C::kBuf : 16];
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform by construction: keeps the barrier paths below scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, hf = lane >> 5;
  int h, g, qt;
  if constexpr (SUBSET) {
    const int per_head = sa.F * qtiles;
    h = lid / per_head;
    g = (lid - h * per_head) / qtiles;
    qt = lid - h * per_head - g * qtiles;
  } else {
    h = lid / qtiles;
    g = 0;
    qt = lid - h * qtiles;
  }
  // queries, outputs, key/value rows of this block
  const int Np = SUBSET ? sa.n_keys_const : 0;  // rows of the subset arrays
  const int nkeys = SUBSET ? (sa.n_keys ? min(max(sa.n_keys[h * sa.F + g], 0), Np) : Np)
                           : c.n_live[h];
  const float cscale = (SUBSET ? sa.scale : a.scale) * kLog2e;
  const int nq = SUBSET ? sa.Nseg : a.Nq;
  const int64_t sq_n = SUBSET ? sa.sq_n : a.sq_n, so_n = SUBSET ? sa.so_n : a.so_n;
  const uint16_t* qbase =
      SUBSET ? static_cast<const uint16_t*>(sa.q) + (int64_t)h * sa.sq_h + (int64_t)g * sa.Nseg * sa.sq_n
             : static_cast<const uint16_t*>(a.q) + (int64_t)h * a.sq_h;
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
  const float* lbg = SUBSET ? nullptr
                     : REG  ? c.rope_lb + (int64_t)h * dm.R * dm.Bp
                            : c.lb + (int64_t)h * dm.Bp;
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
  const bool gather = SUBSET && sa.sel != nullptr;  // block-uniform
  if (gather) {
    const int32_t* sel = sa.sel + (int64_t)(h * sa.F + g) * sa.sel_ld;
    for (int i = tid; i < nkeys; i += C::kThreads) sel_lds[i] = min(max(sel[i], 0), Np - 1);
    __syncthreads();
  }

  // Copy addresses: a wave-uniform tile base plus per-lane byte offsets that
  // do not change from tile to tile, so issuing a copy costs no vector math.
  // Wave w copies the 1 KiB chunks w, w + WAVES, ... of the K and V tiles; LDS
  // position (row, chunk) receives global chunk chunk ^ swz(row).
  // In a subset, a lane's source row is looked up per tile instead (rows past
  // the kept count read row 0 and are masked by their bias).
  constexpr int kPerWave = C::kKInstr / WAVES;
  uint32_t koff[kPerWave], voff[kPerWave];
  int rrow[kPerWave];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int off = (wave + j * WAVES) * 1024 + lane * 16;
    const int row = off / C::kRowBytes;
    const int slot = (off - row * C::kRowBytes) >> 4;
    rrow[j] = row;
    const int rb = SUBSET ? 0 : row * C::kRowBytes;
    koff[j] = (uint32_t)(rb + ((slot ^ C::kswz(row)) << 4));
    voff[j] = (uint32_t)(rb + ((slot ^ C::vswz(row)) << 4));
  }
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
      const int i = wave + j * WAVES;
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
      if (wave == (WAVES - 1 - i) % WAVES && i * 64 + lane < BN)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(lsrc + i * 64 + (uint32_t)lane),
                                         (lds_void_t*)(buf + C::kKBytes + C::kVBytes + i * 256), 4, 0, 0);
    }
  };

  // queries of this wave: qi = qt*BM + wave*32*QB + qb*32 + m
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

  // Copies this wave issues per tile: K and V chunks, plus the bias row for
  // the last wave(s).
  constexpr int kCopies = 2 * C::kKInstr / WAVES;
  const bool lb_wave = wave >= WAVES - (BN + 63) / 64;

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
  auto step = [&](const uint8_t* cur, uint8_t* nxt, int it, int nt) __attribute__((always_inline)) {
    const uint8_t* vt_lds = cur + C::kKBytes;
    const float* lb_lds = reinterpret_cast<const float*>(cur + C::kKBytes + C::kVBytes);
    if (it + NBUF - 1 < nt) issue((it + NBUF - 1) * BN, nxt);

    f32x16_t S[BN / 32][QB];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[kb][qb] = f32x16_t{};
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
    float4 lbr[BN / 32][4];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        lbr[kb][jg] = *reinterpret_cast<const float4*>(lb_lds + kb * 32 + 8 * jg + 4 * hf);
      }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -__builtin_huge_valf();
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const float bb[4] = {lbr[kb][jg].x, lbr[kb][jg].y, lbr[kb][jg].z, lbr[kb][jg].w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float t = __builtin_fmaf(S[kb][qb][4 * jg + r], cscale, bb[r]);
            S[kb][qb][4 * jg + r] = t;
            mx = fmaxf(mx, t);
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
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
        bf16x8_t pf[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            pf[qb][i] = (__bf16)__builtin_amdgcn_exp2f(S[kb][qb][8 * kk + i] - mrun[qb]);
          // row sum of the same bf16-rounded weights the MFMA multiplies
          float ls = lrun[qb];
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            const bf16x2_t pp = {pf[qb][i], pf[qb][i + 1]};
            ls = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ls, false);
          }
          lrun[qb] = ls;
        }
        // A operand: feature db*32 + m, keys kb*32 + kk*16 + {4*hf..4*hf+3}
        // then {8+4*hf..8+4*hf+3}, the key order of the P fragment
        const uint8_t* vrow = vt_lds + (kb * 32 + kk * 16) * C::kRowBytes;
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
    // Tile it+1 must have landed; the copies of tiles it+2 .. it+NBUF-1
    // stay in flight.
    wait_barrier(min(nt - 1, it + NBUF - 1) - (it + 1));
  };

  const int nt = REG ? a.n_reg * ntc : ntc + (nx + BN - 1) / BN;
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u)
    if (u < nt) issue(u * BN, u == 0 ? buf0 : u == 1 ? buf1 : u == 2 ? buf2 : buf3);
  wait_barrier(min(nt, NBUF - 1) - 1);
  for (int it = 0; it < nt; it += NBUF) {
    if (NBUF == 2) {
      step(buf0, buf1, it, nt);
      if (it + 1 < nt) step(buf1, buf0, it + 1, nt);
    } else if (NBUF == 3) {
      step(buf0, buf2, it, nt);
      if (it + 1 < nt) step(buf1, buf0, it + 1, nt);
      if (it + 2 < nt) step(buf2, buf1, it + 2, nt);
    } else {
      step(buf0, buf3, it, nt);
      if (it + 1 < nt) step(buf1, buf0, it + 1, nt);
      if (it + 2 < nt) step(buf2, buf1, it + 2, nt);
      if (it + 3 < nt) step(buf3, buf2, it + 3, nt);
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qt * C::BM + (wave * QB + qb) * 32 + m;
    const float lt = lrun[qb] + __shfl_xor(lrun[qb], 32);
    if (qi >= nq) continue;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    uint16_t* op = obase + (int64_t)qi * so_n;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const uint32_t w0 = f32_to_bf16_bits(O[db][qb][4 * jg + 0] * inv) |
                            (f32_to_bf16_bits(O[db][qb][4 * jg + 1] * inv) << 16);
        const uint32_t w1 = f32_to_bf16_bits(O[db][qb][4 * jg + 2] * inv) |
                            (f32_to_bf16_bits(O[db][qb][4 * jg + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + db * 32 + 8 * jg + 4 * hf) = make_uint2(w0, w1);
      }
    if (lse_row && hf == 0)
      lse_row[qi] = lt > 0.0f ? (mrun[qb] + __log2f(lt)) * kLn2 : -__builtin_huge_valf();
  }
}

template <int D, int BN, int WAVES, int QB, int NBUF>
hipError_t launch_cache_cfg(const Dims& dm, const CacheDev& c, const CacheAttendArgs& a,
                            hipStream_t s) {
  using C = CCfg<D, BN, WAVES, QB>;
  const int qtiles = (a.Nq + C::BM - 1) / C::BM;
  const int blocks = dm.H * qtiles;
  if (blocks == 0) return hipSuccess;
  if (a.n_reg > 0)
    hipLaunchKernelGGL((attend_cache_kernel<D, BN, WAVES, QB, NBUF, false, false, true>),
                       dim3(blocks), dim3(C::kThreads), 0, s, dm, c, a, AttendArgs{}, qtiles);
  else if (a.n_x > 0)
    hipLaunchKernelGGL((attend_cache_kernel<D, BN, WAVES, QB, NBUF, false, true, false>),
                       dim3(blocks), dim3(C::kThreads), 0, s, dm, c, a, AttendArgs{}, qtiles);
  else
    hipLaunchKernelGGL((attend_cache_kernel<D, BN, WAVES, QB, NBUF, false, false, false>),
                       dim3(blocks), dim3(C::kThreads), 0, s, dm, c, a, AttendArgs{}, qtiles);
  return hipGetLastError();
}

// Subsets: 8 waves x 32 queries per workgroup per (head, segment); a gather
// list is staged in LDS (up to 4 bytes per prompt row) beside a 2-deep ring.
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

hipError_t launch_attend_bf16(const AttendArgs& a, hipStream_t s) {
  if (a.count != nullptr) return hipErrorInvalidValue;  // no count bias on subsets
  if (a.d == 128) return a.sel ? launch_subset_cfg<128, 2>(a, s) : launch_subset_cfg<128, 4>(a, s);
  return a.sel ? launch_subset_cfg<64, 2>(a, s) : launch_subset_cfg<64, 4>(a, s);
}

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
  if (dm.d == 128) return launch_cache_cfg<128, BN, W, QB, FASTAR_CACHE_NBUF>(dm, c, a, s);
  return launch_cache_cfg<64, 64, 4, 1, FASTAR_CACHE_NBUF>(dm, c, a, s);
}

hipError_t launch_attend_f32(const AttendArgs& a, hipStream_t s) {
  const int qtiles = (a.Nseg + 63) / 64;
  const int blocks = a.H * a.F * qtiles;
  if (blocks == 0) return hipSuccess;
  const bool gather = a.sel != nullptr;
  if (a.d == 128) {
    if (gather) hipLaunchKernelGGL((attend_f32_kernel<128, true>), dim3(blocks), dim3(64), 0, s, a, qtiles);
    else hipLaunchKernelGGL((attend_f32_kernel<128, false>), dim3(blocks), dim3(64), 0, s, a, qtiles);
  } else {
    if (gather) hipLaunchKernelGGL((attend_f32_kernel<64, true>), dim3(blocks), dim3(64), 0, s, a, qtiles);
    else hipLaunchKernelGGL((attend_f32_kernel<64, false>), dim3(blocks), dim3(64), 0, s, a, qtiles);
  }
  return hipGetLastError();
}

}  // namespace fastar
