// Host side of the C ABI declared in fastar.h: argument validation, the
// workspace layout of a cache, and the launch sequence of one chunk step.
// Nothing here allocates device memory; every launch goes on the caller's
// stream and nothing synchronises except create, stats, export and import.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"
#include "fastar.h"

using namespace fastar;

struct fastar_cache_s {
  fastar_config cfg;
  Dims dm;
  CacheDev dev;
  Layout lay;
  void* ws;
  size_t ws_bytes;
  int device;
  // every change of the slot state bumps `version`; the AnnSA index is valid
  // for the version it was built at, with annsa_L tables
  uint64_t version = 0;
  uint64_t annsa_version = ~0ull;
  int annsa_L = 0;
  int annsa_b = 0;  // bits of those codes
};

namespace {

thread_local std::string g_err;

fastar_status fail(fastar_status st, const std::string& msg) {
  g_err = msg;
  return st;
}
fastar_status ok() {
  g_err.clear();
  return FASTAR_OK;
}

#define FASTAR_HIP(expr)                                                              \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(FASTAR_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define FASTAR_REQUIRE(cond, msg) \
  do {                            \
    if (!(cond)) return fail(FASTAR_ERR_INVALID_ARGUMENT, msg); \
  } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_bytes(fastar_dtype dt) { return dt == FASTAR_BF16 ? 2 : 4; }

bool valid_dtype(fastar_dtype dt) { return dt == FASTAR_F32 || dt == FASTAR_BF16; }

fastar_status make_dims(const fastar_config* cfg, Dims* dm) {
  FASTAR_REQUIRE(cfg != nullptr, "config is NULL");
  FASTAR_REQUIRE(cfg->num_heads >= 1, "num_heads must be >= 1");
  FASTAR_REQUIRE(cfg->head_dim == 64 || cfg->head_dim == 128, "head_dim must be 64 or 128");
  FASTAR_REQUIRE(cfg->budget_slots >= 1 && cfg->budget_slots <= FASTAR_MAX_BUDGET,
                 "budget_slots out of range");
  FASTAR_REQUIRE(cfg->num_tables >= 1 && cfg->num_tables <= FASTAR_MAX_TABLES,
                 "num_tables out of range");
  FASTAR_REQUIRE(cfg->num_bits >= 0 && cfg->num_bits <= FASTAR_MAX_BITS, "num_bits out of range");
  FASTAR_REQUIRE(std::isfinite(cfg->cos_threshold), "cos_threshold must be finite");
  FASTAR_REQUIRE(valid_dtype(cfg->dtype), "unknown dtype");
  const int M = cfg->pq_subspaces;
  FASTAR_REQUIRE(M == 0 || M == 1 || M == 2 || M == 4 || (M == 8 && cfg->head_dim == 128),
                 "pq_subspaces must be 0 (SimHash) or 1, 2, 4 (8 with head_dim 128)");
  FASTAR_REQUIRE(M == 0 || (cfg->num_bits % M == 0 && cfg->num_bits / M >= 1 &&
                            cfg->num_bits / M <= 8),
                 "product quantization needs num_bits = pq_subspaces x (1..8)");
  FASTAR_REQUIRE(cfg->rope_members >= 0 && cfg->rope_members <= 4, "rope_members must be 0..4");
  dm->H = cfg->num_heads;
  dm->d = cfg->head_dim;
  dm->B = cfg->budget_slots;
  dm->L = cfg->num_tables;
  dm->b = cfg->num_bits;
  dm->elem = elem_bytes(cfg->dtype);
  dm->M = M;
  int nb = 6;  // at least 64 buckets
  while ((1 << nb) * kSlotsPerBucket < dm->B) ++nb;
  dm->nb_bits = nb;
  dm->NB = 1 << nb;
  dm->Ppad = M ? 0 : (dm->L * dm->b + 31) & ~31;  // SimHash planes of the fused re-hash
  dm->Bp = (dm->B + kSlotPad - 1) / kSlotPad * kSlotPad;
  dm->R = cfg->rope_members;
  return FASTAR_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Elements of the hyperplanes ([L][b][d]) or PQ codebooks ([L][M][2^(b/M)][d/M]).
size_t plane_elems(const Dims& dm) {
  if (dm.L * dm.b == 0) return (size_t)dm.d;
  if (dm.M) return (size_t)dm.L * ((size_t)1 << (dm.b / dm.M)) * dm.d;
  return (size_t)dm.L * dm.b * dm.d;
}

enum Region {
  kPlanes, kPlanesFrag, kKMaster, kVMaster, kKMirror, kVMirror, kLb, kCount, kLast, kHist, kCodes,
  kIdxOff, kIdxSlot, kNLive, kEvicted, kCounters, kOwner, kGsize, kFrame, kStateEnd = kFrame,
  kBestSlot, kBestCos, kDec, kFrameCodes, kGroupTok, kGroupSlot, kItems,
  kPlan, kAnnsaCodes, kAnnsaOff, kAnnsaEnt, kRopeK, kRopeLb, kLbc, kAttnPart, kAttnMl,
  kNumRegions
};
static_assert(kNumRegions + 1 <= (int)(sizeof(Layout::off) / sizeof(size_t)),
              "Layout::off holds every region's offset and the total");

fastar_status check_device_gfx950(int* device) {
  FASTAR_HIP(hipGetDevice(device));
  hipDeviceProp_t prop;
  FASTAR_HIP(hipGetDeviceProperties(&prop, *device));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(FASTAR_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName +
                                            ", this library is built for gfx950");
  return FASTAR_OK;
}

__global__ void zero_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Zero [ptr, ptr+bytes) with a kernel (bytes and ptr are 256-byte aligned).
hipError_t zero_bytes(void* ptr, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<uint4*>(ptr), n16);
  return hipGetLastError();
}

fastar_status check_handle(fastar_cache_t c) {
  if (c == nullptr) return fail(FASTAR_ERR_INVALID_ARGUMENT, "cache handle is NULL");
  return FASTAR_OK;
}

}  // namespace

namespace fastar {

Layout make_layout(const Dims& dm) {
  Layout L{};
  const size_t H = dm.H, B = dm.B, d = dm.d, Lt = dm.L, e = dm.elem;
  size_t sizes[kNumRegions] = {};
  sizes[kPlanes] = plane_elems(dm) * e;
  sizes[kPlanesFrag] = e == 2 ? (size_t)dm.Ppad * d * 2 : 0;
  sizes[kKMaster] = H * B * d * 4;
  sizes[kVMaster] = H * B * d * 4;
  const size_t Bp = dm.Bp;
  sizes[kKMirror] = H * Bp * d * e;
  sizes[kVMirror] = H * Bp * d * e;
  sizes[kLb] = H * Bp * 4;
  sizes[kCount] = H * B * 4;
  sizes[kLast] = H * B * 4;
  sizes[kHist] = H * B * (size_t)dm.R * 4;
  sizes[kCodes] = H * Lt * B * 4;
  sizes[kIdxOff] = H * Lt * ((size_t)dm.NB + 1) * 4;
  sizes[kIdxSlot] = H * Lt * B * 8;
  sizes[kNLive] = H * 4;
  sizes[kEvicted] = H * 8;
  sizes[kCounters] = H * kNumCounters * 8;
  sizes[kOwner] = H * B * 4;
  sizes[kGsize] = H * B * 4;
  sizes[kFrame] = 4;
  sizes[kBestSlot] = H * B * 4;
  sizes[kBestCos] = H * B * 4;
  sizes[kDec] = H * B * 4;
  sizes[kFrameCodes] = H * Lt * B * 4;
  sizes[kGroupTok] = H * B * 4;
  sizes[kGroupSlot] = H * B * 4;
  sizes[kItems] = H * B * 16;
  sizes[kPlan] = H * kPlanStride * 4;
  sizes[kAnnsaCodes] = H * 4 * B * 4;
  sizes[kAnnsaOff] = H * 4 * ((size_t)dm.NB + 1) * 4;
  sizes[kAnnsaEnt] = H * 4 * B * 8;
  sizes[kRopeK] = e == 2 ? H * (size_t)dm.R * Bp * d * 2 : 0;
  sizes[kRopeLb] = e == 2 ? H * (size_t)dm.R * Bp * 4 : 0;
  sizes[kLbc] = e == 2 ? H * (size_t)std::max(dm.R, 1) * Bp * 4 : 0;
  // partial results of split attention workgroups (bf16 caches): the tail of
  // at most attn_split_pairs (head, query tile) pairs, four quarters each
  const size_t P = e == 2 ? (size_t)attn_split_pairs(dm) : 0, bm = attn_query_tile(dm);
  sizes[kAttnPart] = P * 4 * bm * d * 4;
  sizes[kAttnMl] = P * 4 * bm * 8;
  size_t off = 0;
  for (int r = 0; r < kNumRegions; ++r) {
    L.off[r] = off;
    off = align256(off + sizes[r]);
  }
  L.off[kNumRegions] = off;
  L.total = off;
  return L;
}

CacheDev carve(void* base, const Dims& dm) {
  const Layout L = make_layout(dm);
  uint8_t* b = static_cast<uint8_t*>(base);
  CacheDev c{};
  c.planes = b + L.off[kPlanes];
  c.planes_frag = b + L.off[kPlanesFrag];
  c.k_master = reinterpret_cast<float*>(b + L.off[kKMaster]);
  c.v_master = reinterpret_cast<float*>(b + L.off[kVMaster]);
  c.k_mirror = b + L.off[kKMirror];
  c.v_mirror = b + L.off[kVMirror];
  c.lb = reinterpret_cast<float*>(b + L.off[kLb]);
  c.count = reinterpret_cast<int32_t*>(b + L.off[kCount]);
  c.last = reinterpret_cast<int32_t*>(b + L.off[kLast]);
  c.hist = reinterpret_cast<int32_t*>(b + L.off[kHist]);
  c.codes = reinterpret_cast<uint32_t*>(b + L.off[kCodes]);
  c.idx_off = reinterpret_cast<int32_t*>(b + L.off[kIdxOff]);
  c.idx_ent = reinterpret_cast<uint2*>(b + L.off[kIdxSlot]);
  c.n_live = reinterpret_cast<int32_t*>(b + L.off[kNLive]);
  c.evicted_tokens = reinterpret_cast<int64_t*>(b + L.off[kEvicted]);
  c.counters = reinterpret_cast<int64_t*>(b + L.off[kCounters]);
  c.frame = reinterpret_cast<int32_t*>(b + L.off[kFrame]);
  c.owner = reinterpret_cast<int32_t*>(b + L.off[kOwner]);
  c.gsize = reinterpret_cast<int32_t*>(b + L.off[kGsize]);
  c.best_slot = reinterpret_cast<int32_t*>(b + L.off[kBestSlot]);
  c.best_cos = reinterpret_cast<float*>(b + L.off[kBestCos]);
  c.dec = reinterpret_cast<int32_t*>(b + L.off[kDec]);
  c.frame_codes = reinterpret_cast<uint32_t*>(b + L.off[kFrameCodes]);
  c.group_tok = reinterpret_cast<int32_t*>(b + L.off[kGroupTok]);
  c.group_slot = reinterpret_cast<int32_t*>(b + L.off[kGroupSlot]);
  c.items = reinterpret_cast<int4*>(b + L.off[kItems]);
  c.plan = reinterpret_cast<int32_t*>(b + L.off[kPlan]);
  c.annsa_codes = reinterpret_cast<uint32_t*>(b + L.off[kAnnsaCodes]);
  c.annsa_off = reinterpret_cast<int32_t*>(b + L.off[kAnnsaOff]);
  c.annsa_ent = reinterpret_cast<uint2*>(b + L.off[kAnnsaEnt]);
  c.rope_k = b + L.off[kRopeK];
  c.rope_lb = reinterpret_cast<float*>(b + L.off[kRopeLb]);
  c.lbc = reinterpret_cast<float*>(b + L.off[kLbc]);
  c.attn_part = reinterpret_cast<float*>(b + L.off[kAttnPart]);
  c.attn_ml = reinterpret_cast<float2*>(b + L.off[kAttnMl]);
  c.attn_pairs = dm.elem == 2 ? attn_split_pairs(dm) : 0;
  return c;
}

}  // namespace fastar

extern "C" {

const char* fastar_last_error(void) { return g_err.c_str(); }

fastar_status fastar_cache_workspace_bytes(const fastar_config* cfg, size_t* bytes) {
  Dims dm;
  fastar_status st = make_dims(cfg, &dm);
  if (st != FASTAR_OK) return st;
  FASTAR_REQUIRE(bytes != nullptr, "bytes is NULL");
  *bytes = make_layout(dm).total;
  return ok();
}

fastar_status fastar_cache_create(const fastar_config* cfg, const void* planes_host,
                                  void* workspace_dev, size_t workspace_bytes, void* stream,
                                  fastar_cache_t* out) {
  Dims dm;
  fastar_status st = make_dims(cfg, &dm);
  if (st != FASTAR_OK) return st;
  FASTAR_REQUIRE(out != nullptr, "out is NULL");
  FASTAR_REQUIRE(workspace_dev != nullptr, "workspace is NULL");
  FASTAR_REQUIRE(aligned(workspace_dev, 256), "workspace must be 256-byte aligned");
  FASTAR_REQUIRE(planes_host != nullptr || dm.L * dm.b == 0, "planes_host is NULL");
  const Layout lay = make_layout(dm);
  if (workspace_bytes < lay.total)
    return fail(FASTAR_ERR_WORKSPACE_TOO_SMALL,
                "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                    std::to_string(lay.total));
  int device = 0;
  st = check_device_gfx950(&device);
  if (st != FASTAR_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  CacheDev dev = carve(workspace_dev, dm);
  FASTAR_HIP(zero_bytes(workspace_dev, lay.off[kStateEnd + 1], s));
  const size_t plane_bytes = dm.L * dm.b > 0 ? plane_elems(dm) * dm.elem : 0;
  if (plane_bytes) FASTAR_HIP(hipMemcpyAsync(dev.planes, planes_host, plane_bytes,
                                             hipMemcpyHostToDevice, s));
  // bf16: the re-hash of merged keys reads the hyperplanes as MFMA A operands;
  // fragment (block pb, k-step ks), lane l holds plane 32*pb + l%32, features
  // (l/32)*d/2 + 8*ks .. +7, so each operand load is one contiguous 1 KiB read
  std::vector<uint16_t> frag;
  if (dm.elem == 2 && dm.Ppad > 0) {
    const uint16_t* ph = static_cast<const uint16_t*>(planes_host);
    const int KS = dm.d / 16, P = dm.L * dm.b;
    frag.assign((size_t)dm.Ppad * dm.d, 0);
    for (int pb = 0; pb < dm.Ppad / 32; ++pb)
      for (int ks = 0; ks < KS; ++ks)
        for (int l = 0; l < 64; ++l) {
          const int p = pb * 32 + (l & 31);
          if (p >= P) continue;
          const int f0 = (l >> 5) * (dm.d / 2) + ks * 8;
          for (int e = 0; e < 8; ++e)
            frag[(((size_t)pb * KS + ks) * 64 + l) * 8 + e] = ph[(size_t)p * dm.d + f0 + e];
        }
    FASTAR_HIP(hipMemcpyAsync(dev.planes_frag, frag.data(), frag.size() * 2,
                              hipMemcpyHostToDevice, s));
  }
  FASTAR_HIP(launch_finalize_state(dm, dev, s));
  FASTAR_HIP(hipStreamSynchronize(s));
  fastar_cache_s* c = new fastar_cache_s;
  c->cfg = *cfg;
  c->dm = dm;
  c->dev = dev;
  c->lay = lay;
  c->ws = workspace_dev;
  c->ws_bytes = workspace_bytes;
  c->device = device;
  *out = c;
  return ok();
}

fastar_status fastar_cache_destroy(fastar_cache_t cache) {
  delete cache;
  return ok();
}

fastar_status fastar_cache_reset(fastar_cache_t c, void* stream) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  ++c->version;
  uint8_t* b = static_cast<uint8_t*>(c->ws);
  const size_t lo = c->lay.off[kKMaster], hi = c->lay.off[kStateEnd + 1];
  FASTAR_HIP(zero_bytes(b + lo, hi - lo, static_cast<hipStream_t>(stream)));
  FASTAR_HIP(launch_finalize_state(c->dm, c->dev, static_cast<hipStream_t>(stream)));
  return ok();
}

fastar_status fastar_cache_planes(fastar_cache_t c, const void** planes_dev) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  FASTAR_REQUIRE(planes_dev != nullptr, "planes_dev is NULL");
  *planes_dev = c->dev.planes;
  return ok();
}

fastar_status fastar_hash(const void* x_dev, fastar_dtype dtype, int32_t H, int32_t N, int32_t d,
                          int64_t stride_h, int64_t stride_n, const void* planes_dev, int32_t L,
                          int32_t b, uint32_t* codes_dev, void* stream) {
  FASTAR_REQUIRE(valid_dtype(dtype), "unknown dtype");
  FASTAR_REQUIRE(H >= 0 && N >= 0, "H and N must be >= 0");
  FASTAR_REQUIRE(d == 64 || d == 128, "d must be 64 or 128");
  FASTAR_REQUIRE(L >= 1 && L <= FASTAR_MAX_TABLES, "L out of range");
  FASTAR_REQUIRE(b >= 0 && b <= FASTAR_MAX_BITS, "b out of range");
  if ((int64_t)H * N == 0) return ok();
  FASTAR_REQUIRE(x_dev && codes_dev, "NULL pointer");
  FASTAR_REQUIRE(planes_dev != nullptr || b == 0, "planes_dev is NULL");
  const int vec = dtype == FASTAR_BF16 ? 8 : 4;
  FASTAR_REQUIRE(aligned(x_dev, 16) && aligned(planes_dev, 16) && aligned(codes_dev, 4),
                 "x and planes must be 16-byte aligned");
  FASTAR_REQUIRE(stride_h % vec == 0 && stride_n % vec == 0 && stride_n >= d,
                 "strides must be multiples of 16 bytes and rows must not overlap");
  HashArgs a{};
  a.x = x_dev;
  a.sx_h = stride_h;
  a.sx_n = stride_n;
  a.H = H;
  a.N = N;
  a.d = d;
  a.L = L;
  a.b = b;
  a.planes = planes_dev;
  a.codes = codes_dev;
  a.codes_ld = N;
  a.codes_col0 = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  FASTAR_HIP(dtype == FASTAR_BF16 ? launch_hash_bf16(a, s) : launch_hash_f32(a, s));
  return ok();
}

fastar_status fastar_pq_codes(const void* x_dev, fastar_dtype dtype, int32_t H, int32_t N, int32_t d,
                              int64_t stride_h, int64_t stride_n, const void* codebooks_dev,
                              int32_t L, int32_t M, int32_t b, uint32_t* codes_dev, void* stream) {
  FASTAR_REQUIRE(valid_dtype(dtype), "unknown dtype");
  FASTAR_REQUIRE(H >= 0 && N >= 0, "H and N must be >= 0");
  FASTAR_REQUIRE(d == 64 || d == 128, "d must be 64 or 128");
  FASTAR_REQUIRE(L >= 1 && L <= FASTAR_MAX_TABLES, "L out of range");
  FASTAR_REQUIRE(M == 1 || M == 2 || M == 4 || (M == 8 && d == 128),
                 "M must be 1, 2, 4 (8 with d = 128)");
  FASTAR_REQUIRE(b % M == 0 && b / M >= 1 && b / M <= 8, "b must be M x (1..8)");
  if ((int64_t)H * N == 0) return ok();
  FASTAR_REQUIRE(x_dev && codes_dev, "NULL pointer");
  FASTAR_REQUIRE(codebooks_dev != nullptr, "codebooks_dev is NULL");
  const int vec = dtype == FASTAR_BF16 ? 8 : 4;
  FASTAR_REQUIRE(aligned(x_dev, 16) && aligned(codebooks_dev, 16) && aligned(codes_dev, 4),
                 "x and codebooks must be 16-byte aligned");
  FASTAR_REQUIRE(stride_h % vec == 0 && stride_n % vec == 0 && stride_n >= d,
                 "strides must be multiples of 16 bytes and rows must not overlap");
  HashArgs a{};
  a.x = x_dev;
  a.sx_h = stride_h;
  a.sx_n = stride_n;
  a.H = H;
  a.N = N;
  a.d = d;
  a.L = L;
  a.b = b;
  a.planes = codebooks_dev;
  a.M = M;
  a.codes = codes_dev;
  a.codes_ld = N;
  a.codes_col0 = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  FASTAR_HIP(dtype == FASTAR_BF16 ? launch_hash_bf16(a, s) : launch_hash_f32(a, s));
  return ok();
}

fastar_status fastar_match_merge(fastar_cache_t c, const void* k_dev, const void* v_dev,
                                 int64_t stride_h, int64_t stride_n, const uint32_t* codes_dev,
                                 int32_t tokens_per_frame, int32_t num_frames,
                                 int32_t* slot_out_dev, uint8_t* merged_out_dev, void* stream) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  const Dims& dm = c->dm;
  const int T = tokens_per_frame, F = num_frames;
  FASTAR_REQUIRE(T >= 1 && F >= 1, "tokens_per_frame and num_frames must be >= 1");
  if (T > dm.B || T > FASTAR_MAX_TOKENS_PER_FRAME)
    return fail(FASTAR_ERR_CAPACITY, "tokens_per_frame " + std::to_string(T) +
                                         " exceeds the budget or the per-frame limit");
  FASTAR_REQUIRE(k_dev && v_dev, "k or v is NULL");
  const int vec = dm.elem == 2 ? 8 : 4;
  FASTAR_REQUIRE(aligned(k_dev, 16) && aligned(v_dev, 16), "k and v must be 16-byte aligned");
  FASTAR_REQUIRE(stride_h % vec == 0 && stride_n % vec == 0 && stride_n >= dm.d,
                 "strides must be multiples of 16 bytes and rows must not overlap");
  FASTAR_REQUIRE(codes_dev == nullptr || aligned(codes_dev, 4), "codes misaligned");
  // every check passed: from here on the slot state changes
  ++c->version;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const CacheDev& dev = c->dev;
  const int64_t N = (int64_t)T * F;
  // Without caller codes, the new keys are hashed into frame_codes ([H][L][B])
  // ahead of their frames, as many frames per launch as fit in B columns: the
  // codes of new keys do not depend on the cache state.
  const int hash_group = std::max(1, dm.B / T);
  for (int f = 0; f < F; ++f) {
    const int64_t tok0 = (int64_t)f * T;
    const uint8_t* kf = static_cast<const uint8_t*>(k_dev) + tok0 * stride_n * dm.elem;
    const uint8_t* vf = static_cast<const uint8_t*>(v_dev) + tok0 * stride_n * dm.elem;
    const uint32_t* codes = codes_dev;
    int64_t codes_ld = N, codes_col0 = tok0;
    if (codes == nullptr) {
      const int g = f % hash_group;  // position of this frame in its hash group
      if (g == 0) {
        HashArgs ha{};
        ha.x = kf;
        ha.sx_h = stride_h;
        ha.sx_n = stride_n;
        ha.H = dm.H;
        ha.N = T * std::min(hash_group, F - f);
        ha.d = dm.d;
        ha.L = dm.L;
        ha.b = dm.b;
        ha.planes = dev.planes;
        ha.M = dm.M;
        ha.codes = dev.frame_codes;
        ha.codes_ld = dm.B;
        ha.codes_col0 = 0;
        FASTAR_HIP(dm.elem == 2 ? launch_hash_bf16(ha, s) : launch_hash_f32(ha, s));
      }
      codes = dev.frame_codes;
      codes_ld = dm.B;
      codes_col0 = (int64_t)g * T;
    }
    MatchArgs ma{kf, stride_h, stride_n, codes, codes_ld, codes_col0, T, c->cfg.cos_threshold};
    FASTAR_HIP(launch_match(dm, dev, ma, s));
    MergeArgs ga{kf, vf, stride_h, stride_n, codes, codes_ld, codes_col0, T,
                 slot_out_dev, merged_out_dev, N, tok0};
    FASTAR_HIP(launch_plan(dm, dev, ga, s));
    FASTAR_HIP(launch_apply(dm, dev, ga, s));
    // bf16 storage: the apply kernel already refreshed the merged slots' codes
    if (dm.elem != 2 || dm.M > 0) FASTAR_HIP(launch_rehash(dm, dev, T, s));
    FASTAR_HIP(launch_index(dm, dev, true, s));
  }
  return ok();
}

fastar_status fastar_cache_hash_slots(fastar_cache_t c, const void* planes_dev, int32_t L,
                                      int32_t b, uint32_t* codes_dev, int64_t codes_ld,
                                      void* stream) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  const Dims& dm = c->dm;
  FASTAR_REQUIRE(L >= 1 && L <= 4, "AnnSA takes 1 to 4 tables");
  FASTAR_REQUIRE(b >= 0 && b <= FASTAR_MAX_BITS, "b out of range");
  FASTAR_REQUIRE(planes_dev != nullptr || b == 0, "planes_dev is NULL");
  FASTAR_REQUIRE(aligned(planes_dev, 16), "planes must be 16-byte aligned");
  FASTAR_REQUIRE(codes_dev == nullptr || (codes_ld >= dm.B && aligned(codes_dev, 4)),
                 "codes_dev misaligned or codes_ld < budget");
  hipStream_t s = static_cast<hipStream_t>(stream);
  HashArgs a{};
  a.x = c->dev.k_mirror;
  a.sx_h = (int64_t)dm.Bp * dm.d;
  a.sx_n = dm.d;
  a.H = dm.H;
  a.N = dm.B;
  a.d = dm.d;
  a.L = L;
  a.b = b;
  a.planes = planes_dev;
  a.codes = c->dev.annsa_codes;
  a.codes_ld = dm.B;
  a.codes_col0 = 0;
  FASTAR_HIP(dm.elem == 2 ? launch_hash_bf16(a, s) : launch_hash_f32(a, s));
  // the bucket index of those codes, by the cache's own index kernel
  Dims da = dm;
  da.L = L;
  CacheDev ca = c->dev;
  ca.codes = c->dev.annsa_codes;
  ca.idx_off = c->dev.annsa_off;
  ca.idx_ent = c->dev.annsa_ent;
  FASTAR_HIP(launch_index(da, ca, false, s));
  if (codes_dev)
    FASTAR_HIP(hipMemcpy2DAsync(codes_dev, (size_t)codes_ld * 4, c->dev.annsa_codes,
                                (size_t)dm.B * 4, (size_t)dm.B * 4, (size_t)dm.H * L,
                                hipMemcpyDeviceToDevice, s));
  c->annsa_version = c->version;
  c->annsa_L = L;
  c->annsa_b = b;
  return ok();
}

fastar_status fastar_annsa_attend(fastar_cache_t c, const void* q_dev, int64_t stride_h,
                                  int64_t stride_n, int32_t Nq, const uint32_t* q_codes_dev,
                                  int32_t L, float scale, void* o_dev, int64_t o_stride_h,
                                  int64_t o_stride_n, float* lse_dev, void* stream) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  const Dims& dm = c->dm;
  FASTAR_REQUIRE(c->annsa_version == c->version && c->annsa_L == L,
                 "call fastar_cache_hash_slots with these L tables after the last change of "
                 "the cache");
  FASTAR_REQUIRE(Nq >= 0, "Nq must be >= 0");
  if (Nq == 0) return ok();
  FASTAR_REQUIRE(q_dev && o_dev && q_codes_dev, "NULL pointer");
  FASTAR_REQUIRE(std::isfinite(scale) && scale >= 0.0f,
                 "scale must be finite and >= 0 (0 selects 1/sqrt(d))");
  const int vec = dm.elem == 2 ? 8 : 4;
  FASTAR_REQUIRE(aligned(q_dev, 16) && aligned(o_dev, 16), "q and o must be 16-byte aligned");
  FASTAR_REQUIRE(stride_h % vec == 0 && stride_n % vec == 0 && stride_n >= dm.d,
                 "q strides must be multiples of 16 bytes");
  FASTAR_REQUIRE(o_stride_h % vec == 0 && o_stride_n % vec == 0 && o_stride_n >= dm.d,
                 "o strides must be multiples of 16 bytes");
  FASTAR_REQUIRE(aligned(q_codes_dev, 4), "q_codes misaligned");
  FASTAR_REQUIRE(lse_dev == nullptr || aligned(lse_dev, 4), "lse misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  AnnsaArgs a{q_dev, stride_h, stride_n, q_codes_dev, Nq,
              scale == 0.0f ? 1.0f / std::sqrt((float)dm.d) : scale, o_dev, o_stride_h,
              o_stride_n, lse_dev};
  Dims da = dm;
  da.L = L;
  da.b = c->annsa_b;
  CacheDev ca = c->dev;
  ca.codes = c->dev.annsa_codes;
  ca.idx_off = c->dev.annsa_off;
  ca.idx_ent = c->dev.annsa_ent;
  FASTAR_HIP(launch_annsa(da, ca, a, s));
  return ok();
}

// Attention over the live slots, optionally followed by n_new raw tokens
// (count 1) in the same softmax.
static fastar_status attend_impl(fastar_cache_t c, const void* q_dev, int64_t stride_h, int64_t stride_n,
                          int32_t Nq, const void* k_new, const void* v_new, int64_t kv_stride_h,
                          int64_t kv_stride_n, int32_t n_new, float scale, void* o_dev,
                          int64_t o_stride_h, int64_t o_stride_n, float* lse_dev, void* stream) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  const Dims& dm = c->dm;
  FASTAR_REQUIRE(Nq >= 0, "Nq must be >= 0");
  FASTAR_REQUIRE(n_new >= 0, "n_new must be >= 0");
  if (Nq == 0) return ok();
  FASTAR_REQUIRE(q_dev && o_dev, "q or o is NULL");
  FASTAR_REQUIRE(std::isfinite(scale) && scale >= 0.0f,
                 "scale must be finite and >= 0 (0 selects 1/sqrt(d))");
  const int vec = dm.elem == 2 ? 8 : 4;
  FASTAR_REQUIRE(aligned(q_dev, 16) && aligned(o_dev, 16), "q and o must be 16-byte aligned");
  FASTAR_REQUIRE(stride_h % vec == 0 && stride_n % vec == 0 && stride_n >= dm.d,
                 "q strides must be multiples of 16 bytes");
  FASTAR_REQUIRE(o_stride_h % vec == 0 && o_stride_n % vec == 0 && o_stride_n >= dm.d,
                 "o strides must be multiples of 16 bytes");
  FASTAR_REQUIRE(lse_dev == nullptr || aligned(lse_dev, 4), "lse misaligned");
  if (n_new > 0) {
    FASTAR_REQUIRE(k_new && v_new, "k_new or v_new is NULL");
    FASTAR_REQUIRE(aligned(k_new, 16) && aligned(v_new, 16), "k_new and v_new must be 16-byte aligned");
    FASTAR_REQUIRE(kv_stride_h % vec == 0 && kv_stride_n % vec == 0 && kv_stride_n >= dm.d &&
                       kv_stride_h >= 0,
                   "k_new / v_new strides must be multiples of 16 bytes");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float sc = scale == 0.0f ? 1.0f / std::sqrt((float)dm.d) : scale;
  if (dm.elem == 2) {
    CacheAttendArgs ca{q_dev, stride_h, stride_n, o_dev, o_stride_h, o_stride_n, lse_dev, Nq, sc};
    if (n_new > 0) {
      ca.xk = k_new;
      ca.xv = v_new;
      ca.sx_h = kv_stride_h;
      ca.sx_n = kv_stride_n;
      ca.n_x = n_new;
    }
    FASTAR_HIP(launch_attend_cache_bf16(dm, c->dev, ca, s));
    return ok();
  }
  AttendArgs a{};
  a.q = q_dev;
  a.sq_h = stride_h;
  a.sq_n = stride_n;
  a.k = c->dev.k_mirror;
  a.v = c->dev.v_mirror;
  a.sk_h = (int64_t)dm.Bp * dm.d;
  a.sk_n = dm.d;
  a.count = c->dev.count;
  a.count_ld = dm.B;
  a.n_keys = c->dev.n_live;
  a.n_keys_const = 0;
  a.sel = nullptr;
  a.sel_ld = 0;
  a.o = o_dev;
  a.so_h = o_stride_h;
  a.so_n = o_stride_n;
  a.lse = lse_dev;
  a.H = dm.H;
  a.d = dm.d;
  a.Nseg = Nq;
  a.F = 1;
  a.scale = sc;
  if (n_new > 0) {
    a.xk = k_new;
    a.xv = v_new;
    a.sx_h = kv_stride_h;
    a.sx_n = kv_stride_n;
    a.n_x = n_new;
  }
  FASTAR_HIP(launch_attend_f32(a, s));
  return ok();
}

fastar_status fastar_project_keys(fastar_cache_t c, const void* x_dev, int64_t x_stride,
                                  int32_t n_tok, int32_t d_in, const void* w_dev, int64_t w_stride,
                                  void* k_out_dev, int64_t k_stride_h, int64_t k_stride_n,
                                  uint32_t* codes_dev, int64_t codes_ld, void* stream) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  const Dims& dm = c->dm;
  if (dm.elem != 2 || dm.M != 0)
    return fail(FASTAR_ERR_UNSUPPORTED, "fastar_project_keys needs a bf16 cache with SimHash codes");
  FASTAR_REQUIRE(n_tok >= 0, "n_tok must be >= 0");
  FASTAR_REQUIRE(d_in > 0 && d_in % 32 == 0, "d_in must be a positive multiple of 32");
  if (n_tok == 0) return ok();
  FASTAR_REQUIRE(x_dev && w_dev && k_out_dev && codes_dev, "NULL pointer");
  FASTAR_REQUIRE(aligned(x_dev, 16) && aligned(w_dev, 16) && aligned(k_out_dev, 16) &&
                     aligned(codes_dev, 4),
                 "x, w and k_out must be 16-byte aligned, codes 4-byte aligned");
  FASTAR_REQUIRE(x_stride % 8 == 0 && x_stride >= d_in && w_stride % 8 == 0 && w_stride >= d_in,
                 "x and w row strides must be multiples of 16 bytes and >= d_in");
  FASTAR_REQUIRE(k_stride_h % 8 == 0 && k_stride_n % 8 == 0 && k_stride_n >= dm.d,
                 "k_out strides must be multiples of 16 bytes");
  FASTAR_REQUIRE(codes_ld >= n_tok, "codes_ld must be >= n_tok");
  ProjArgs a{};
  a.x = static_cast<const uint16_t*>(x_dev);
  a.sx = x_stride;
  a.w = static_cast<const uint16_t*>(w_dev);
  a.sw = w_stride;
  a.N = n_tok;
  a.Din = d_in;
  a.H = dm.H;
  a.L = dm.L;
  a.b = dm.b;
  a.Ppad = dm.Ppad;
  a.k = static_cast<uint16_t*>(k_out_dev);
  a.sk_h = k_stride_h;
  a.sk_n = k_stride_n;
  a.codes = codes_dev;
  a.codes_ld = codes_ld;
  a.planes_frag = c->dev.planes_frag;
  FASTAR_HIP(launch_project_hash(a, dm.d, static_cast<hipStream_t>(stream)));
  return ok();
}

fastar_status fastar_attend(fastar_cache_t c, const void* q_dev, int64_t stride_h,
                            int64_t stride_n, int32_t Nq, float scale, void* o_dev,
                            int64_t o_stride_h, int64_t o_stride_n, float* lse_dev, void* stream) {
  return attend_impl(c, q_dev, stride_h, stride_n, Nq, nullptr, nullptr, 0, 0, 0, scale, o_dev,
                     o_stride_h, o_stride_n, lse_dev, stream);
}

fastar_status fastar_attend_with_chunk(fastar_cache_t c, const void* q_dev, int64_t stride_h,
                                       int64_t stride_n, int32_t Nq, const void* k_new_dev,
                                       const void* v_new_dev, int64_t kv_stride_h,
                                       int64_t kv_stride_n, int32_t n_new, float scale, void* o_dev,
                                       int64_t o_stride_h, int64_t o_stride_n, float* lse_dev,
                                       void* stream) {
  return attend_impl(c, q_dev, stride_h, stride_n, Nq, k_new_dev, v_new_dev, kv_stride_h,
                     kv_stride_n, n_new, scale, o_dev, o_stride_h, o_stride_n, lse_dev, stream);
}

fastar_status fastar_attend_rope(fastar_cache_t c, const void* q_dev, int64_t stride_h,
                                 int64_t stride_n, int32_t Nq, int32_t m, int32_t rope_dims,
                                 float rope_base, float scale, void* o_dev, int64_t o_stride_h,
                                 int64_t o_stride_n, float* lse_dev, void* stream) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  const Dims& dm = c->dm;
  if (dm.elem != 2 || dm.R == 0)
    return fail(FASTAR_ERR_UNSUPPORTED, "fastar_attend_rope needs a bf16 cache with rope_members > 0");
  FASTAR_REQUIRE(m >= 1 && m <= dm.R, "m must be in 1..rope_members");
  FASTAR_REQUIRE(rope_dims >= 0 && rope_dims <= dm.d && rope_dims % 2 == 0,
                 "rope_dims must be even and in [0, d]");
  FASTAR_REQUIRE(std::isfinite(rope_base) && rope_base > 0.0f, "rope_base must be > 0");
  FASTAR_REQUIRE(Nq >= 0, "Nq must be >= 0");
  if (Nq == 0) return ok();
  FASTAR_REQUIRE(q_dev && o_dev, "q or o is NULL");
  FASTAR_REQUIRE(std::isfinite(scale) && scale >= 0.0f,
                 "scale must be finite and >= 0 (0 selects 1/sqrt(d))");
  FASTAR_REQUIRE(aligned(q_dev, 16) && aligned(o_dev, 16), "q and o must be 16-byte aligned");
  FASTAR_REQUIRE(stride_h % 8 == 0 && stride_n % 8 == 0 && stride_n >= dm.d,
                 "q strides must be multiples of 16 bytes");
  FASTAR_REQUIRE(o_stride_h % 8 == 0 && o_stride_n % 8 == 0 && o_stride_n >= dm.d,
                 "o strides must be multiples of 16 bytes");
  FASTAR_REQUIRE(lse_dev == nullptr || aligned(lse_dev, 4), "lse misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float sc = scale == 0.0f ? 1.0f / std::sqrt((float)dm.d) : scale;
  FASTAR_HIP(launch_rope_expand(dm, c->dev, m, rope_dims, rope_base, s));
  CacheAttendArgs ca{q_dev, stride_h, stride_n, o_dev, o_stride_h, o_stride_n, lse_dev, Nq, sc};
  ca.n_reg = m;
  FASTAR_HIP(launch_attend_cache_bf16(dm, c->dev, ca, s));
  return ok();
}

fastar_status fastar_cache_stats(fastar_cache_t c, void* stream, fastar_stats* out) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  FASTAR_REQUIRE(out != nullptr, "out is NULL");
  const Dims& dm = c->dm;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t lo = c->lay.off[kNLive], hi = c->lay.off[kStateEnd + 1];
  std::string buf(hi - lo, '\0');
  FASTAR_HIP(hipMemcpyAsync(&buf[0], static_cast<uint8_t*>(c->ws) + lo, hi - lo,
                            hipMemcpyDeviceToHost, s));
  FASTAR_HIP(hipStreamSynchronize(s));
  const uint8_t* base = reinterpret_cast<const uint8_t*>(buf.data());
  const int32_t* n_live = reinterpret_cast<const int32_t*>(base);
  const int64_t* ev = reinterpret_cast<const int64_t*>(base + (c->lay.off[kEvicted] - lo));
  const int64_t* cn = reinterpret_cast<const int64_t*>(base + (c->lay.off[kCounters] - lo));
  const int32_t* fr = reinterpret_cast<const int32_t*>(base + (c->lay.off[kFrame] - lo));
  fastar_stats r{};
  r.frame = *fr;
  for (int h = 0; h < dm.H; ++h) {
    r.live_slots += n_live[h];
    if (n_live[h] > r.max_live) r.max_live = n_live[h];
    r.evicted_tokens += ev[h];
    r.tokens_seen += cn[h * kNumCounters + kCntTokens];
    r.merged_tokens += cn[h * kNumCounters + kCntMerged];
    r.inserted_tokens += cn[h * kNumCounters + kCntInserted];
    r.evicted_slots += cn[h * kNumCounters + kCntEvictedSlots];
    r.refused_frames += (int32_t)cn[h * kNumCounters + kCntRefused];
  }
  *out = r;
  return ok();
}

fastar_status fastar_cache_export(fastar_cache_t c, void* stream, fastar_cache_state* out) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  FASTAR_REQUIRE(out != nullptr, "out is NULL");
  const Dims& dm = c->dm;
  const CacheDev& d = c->dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t HBd = (size_t)dm.H * dm.B * dm.d, HB = (size_t)dm.H * dm.B;
  auto cp = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
    return dst ? hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s) : hipSuccess;
  };
  FASTAR_HIP(cp(out->k_master, d.k_master, HBd * 4));
  FASTAR_HIP(cp(out->v_master, d.v_master, HBd * 4));
  const size_t row = (size_t)dm.d * dm.elem;
  if (out->k_mirror)
    FASTAR_HIP(hipMemcpy2DAsync(out->k_mirror, (size_t)dm.B * row, d.k_mirror, (size_t)dm.Bp * row,
                                (size_t)dm.B * row, dm.H, hipMemcpyDeviceToHost, s));
  if (out->v_mirror)
    FASTAR_HIP(hipMemcpy2DAsync(out->v_mirror, (size_t)dm.B * row, d.v_mirror, (size_t)dm.Bp * row,
                                (size_t)dm.B * row, dm.H, hipMemcpyDeviceToHost, s));
  FASTAR_HIP(cp(out->count, d.count, HB * 4));
  FASTAR_HIP(cp(out->last, d.last, HB * 4));
  FASTAR_HIP(cp(out->codes, d.codes, HB * dm.L * 4));
  FASTAR_HIP(cp(out->n_live, d.n_live, (size_t)dm.H * 4));
  FASTAR_HIP(cp(out->evicted_tokens, d.evicted_tokens, (size_t)dm.H * 8));
  if (dm.R > 0) FASTAR_HIP(cp(out->member_frames, d.hist, HB * dm.R * 4));
  int32_t frame = 0;
  FASTAR_HIP(hipMemcpyAsync(&frame, d.frame, 4, hipMemcpyDeviceToHost, s));
  FASTAR_HIP(hipStreamSynchronize(s));
  out->frame = frame;
  return ok();
}

fastar_status fastar_cache_import(fastar_cache_t c, const fastar_cache_state* in, void* stream) {
  fastar_status st = check_handle(c);
  if (st != FASTAR_OK) return st;
  FASTAR_REQUIRE(in != nullptr, "in is NULL");
  FASTAR_REQUIRE(in->frame >= -1 && in->frame < INT32_MAX,
                 "frame out of range (-1 keeps the current frame counter)");
  const Dims& dm = c->dm;
  const CacheDev& d = c->dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t HBd = (size_t)dm.H * dm.B * dm.d, HB = (size_t)dm.H * dm.B;
  // The merge step relies on every live slot holding at least one token and
  // having been updated before the current frame (so eviction always finds
  // room).  Check that on the state as it will be after the import: members
  // not given are read back from the device first.
  std::vector<int32_t> n_live(dm.H), count(HB), last(HB);
  int32_t frame = (int32_t)in->frame;
  if (!in->n_live) FASTAR_HIP(hipMemcpyAsync(n_live.data(), d.n_live, (size_t)dm.H * 4,
                                             hipMemcpyDeviceToHost, s));
  if (!in->count) FASTAR_HIP(hipMemcpyAsync(count.data(), d.count, HB * 4, hipMemcpyDeviceToHost, s));
  if (!in->last) FASTAR_HIP(hipMemcpyAsync(last.data(), d.last, HB * 4, hipMemcpyDeviceToHost, s));
  if (in->frame < 0) FASTAR_HIP(hipMemcpyAsync(&frame, d.frame, 4, hipMemcpyDeviceToHost, s));
  FASTAR_HIP(hipStreamSynchronize(s));
  if (in->n_live) std::memcpy(n_live.data(), in->n_live, (size_t)dm.H * 4);
  if (in->count) std::memcpy(count.data(), in->count, HB * 4);
  if (in->last) std::memcpy(last.data(), in->last, HB * 4);
  for (int h = 0; h < dm.H; ++h) {
    FASTAR_REQUIRE(n_live[h] >= 0 && n_live[h] <= dm.B,
                   "n_live[" + std::to_string(h) + "] out of range");
    for (int sl = 0; sl < n_live[h]; ++sl) {
      const size_t i = (size_t)h * dm.B + sl;
      FASTAR_REQUIRE(count[i] >= 1, "live slot " + std::to_string(sl) + " of head " +
                                        std::to_string(h) + " has count < 1");
      FASTAR_REQUIRE(last[i] >= 0 && last[i] < frame,
                     "live slot " + std::to_string(sl) + " of head " + std::to_string(h) +
                         " has a last-update frame outside [0, frame)");
    }
  }
  // every check passed: from here on the slot state changes
  ++c->version;
  auto cp = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
    return src ? hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, s) : hipSuccess;
  };
  FASTAR_HIP(cp(d.k_master, in->k_master, HBd * 4));
  FASTAR_HIP(cp(d.v_master, in->v_master, HBd * 4));
  const size_t row = (size_t)dm.d * dm.elem;
  if (in->k_mirror)
    FASTAR_HIP(hipMemcpy2DAsync(d.k_mirror, (size_t)dm.Bp * row, in->k_mirror, (size_t)dm.B * row,
                                (size_t)dm.B * row, dm.H, hipMemcpyHostToDevice, s));
  if (in->v_mirror)
    FASTAR_HIP(hipMemcpy2DAsync(d.v_mirror, (size_t)dm.Bp * row, in->v_mirror, (size_t)dm.B * row,
                                (size_t)dm.B * row, dm.H, hipMemcpyHostToDevice, s));
  FASTAR_HIP(cp(d.count, in->count, HB * 4));
  FASTAR_HIP(cp(d.last, in->last, HB * 4));
  FASTAR_HIP(cp(d.codes, in->codes, HB * dm.L * 4));
  FASTAR_HIP(cp(d.n_live, in->n_live, (size_t)dm.H * 4));
  FASTAR_HIP(cp(d.evicted_tokens, in->evicted_tokens, (size_t)dm.H * 8));
  if (dm.R > 0) FASTAR_HIP(cp(d.hist, in->member_frames, HB * dm.R * 4));
  if (in->frame >= 0) FASTAR_HIP(hipMemcpyAsync(d.frame, &frame, 4, hipMemcpyHostToDevice, s));
  FASTAR_HIP(launch_finalize_state(dm, d, s));
  FASTAR_HIP(launch_index(dm, d, false, s));
  FASTAR_HIP(hipStreamSynchronize(s));
  return ok();
}

fastar_status fastar_annca_select(const uint32_t* q_codes_dev, int32_t Nf, int32_t F,
                                  const uint32_t* p_codes_dev, int32_t Np, int32_t H, int32_t L,
                                  int32_t* sel_idx_dev, int32_t* sel_count_dev, void* stream) {
  FASTAR_REQUIRE(H >= 1 && F >= 1 && L >= 1 && L <= FASTAR_MAX_TABLES, "H, F, L out of range");
  FASTAR_REQUIRE(Nf >= 1 && Nf <= FASTAR_MAX_ANNCA_QUERIES_PER_FRAME, "Nf out of range");
  FASTAR_REQUIRE(Np >= 1 && Np <= FASTAR_MAX_ANNCA_PROMPT, "Np out of range");
  FASTAR_REQUIRE(q_codes_dev && p_codes_dev && sel_idx_dev && sel_count_dev, "NULL pointer");
  SelectArgs a{q_codes_dev, p_codes_dev, Nf, F, Np, H, L, sel_idx_dev, sel_count_dev};
  FASTAR_HIP(launch_annca_select(a, static_cast<hipStream_t>(stream)));
  return ok();
}

fastar_status fastar_attend_subset(const void* q_dev, int64_t q_stride_h, int64_t q_stride_n,
                                   const void* k_dev, const void* v_dev, int64_t kv_stride_h,
                                   int64_t kv_stride_n, const int32_t* sel_idx_dev,
                                   const int32_t* sel_count_dev, int32_t Nf, int32_t F, int32_t Np,
                                   int32_t H, int32_t d, fastar_dtype dtype, float scale,
                                   void* o_dev, int64_t o_stride_h, int64_t o_stride_n,
                                   void* stream) {
  FASTAR_REQUIRE(valid_dtype(dtype), "unknown dtype");
  FASTAR_REQUIRE(d == 64 || d == 128, "d must be 64 or 128");
  FASTAR_REQUIRE(H >= 1 && F >= 1 && Nf >= 0 && Np >= 0, "sizes out of range");
  FASTAR_REQUIRE((sel_idx_dev == nullptr) == (sel_count_dev == nullptr),
                 "sel_idx and sel_count must both be given or both be NULL");
  FASTAR_REQUIRE(std::isfinite(scale) && scale >= 0.0f,
                 "scale must be finite and >= 0 (0 selects 1/sqrt(d))");
  if (Nf == 0) return ok();
  FASTAR_REQUIRE(q_dev && k_dev && v_dev && o_dev, "NULL pointer");
  const int vec = dtype == FASTAR_BF16 ? 8 : 4;
  FASTAR_REQUIRE(aligned(q_dev, 16) && aligned(k_dev, 16) && aligned(v_dev, 16) &&
                     aligned(o_dev, 16),
                 "q, k, v, o must be 16-byte aligned");
  FASTAR_REQUIRE(q_stride_h % vec == 0 && q_stride_n % vec == 0 && kv_stride_h % vec == 0 &&
                     kv_stride_n % vec == 0 && o_stride_h % vec == 0 && o_stride_n % vec == 0,
                 "strides must be multiples of 16 bytes");
  AttendArgs a{};
  a.q = q_dev;
  a.sq_h = q_stride_h;
  a.sq_n = q_stride_n;
  a.k = k_dev;
  a.v = v_dev;
  a.sk_h = kv_stride_h;
  a.sk_n = kv_stride_n;
  a.count = nullptr;
  a.count_ld = 0;
  a.n_keys = sel_count_dev;
  a.n_keys_const = Np;
  a.sel = sel_idx_dev;
  a.sel_ld = Np;
  a.o = o_dev;
  a.so_h = o_stride_h;
  a.so_n = o_stride_n;
  a.lse = nullptr;
  a.H = H;
  a.d = d;
  a.Nseg = Nf;
  a.F = F;
  a.scale = scale == 0.0f ? 1.0f / std::sqrt((float)d) : scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  FASTAR_HIP(dtype == FASTAR_BF16 ? launch_attend_bf16(a, s) : launch_attend_f32(a, s));
  return ok();
}

fastar_status fastar_annca_attend(const void* q_dev, int64_t q_stride_h, int64_t q_stride_n,
                                  const void* q_planes_dev, int32_t L, int32_t b,
                                  uint32_t* q_codes_dev, const uint32_t* p_codes_dev,
                                  const void* k_dev, const void* v_dev,
                                  int64_t kv_stride_h, int64_t kv_stride_n, int32_t Nf, int32_t F,
                                  int32_t Np, int32_t H, int32_t d, float scale, void* o_dev,
                                  int64_t o_stride_h, int64_t o_stride_n, void* stream) {
  FASTAR_REQUIRE(d == 128, "the fused AnnCA step needs d = 128");
  FASTAR_REQUIRE(H >= 1 && F >= 1, "H and F must be >= 1");
  FASTAR_REQUIRE(L >= 1 && L <= 4 && b >= 0 && b <= 16, "the fused AnnCA step takes 1..4 tables "
                                                         "of 0..16 bits");
  FASTAR_REQUIRE(Nf >= 0 && Nf <= FASTAR_MAX_ANNCA_QUERIES_PER_FRAME, "Nf out of range");
  FASTAR_REQUIRE(Np >= 1 && Np <= 4096, "the fused AnnCA step takes 1..4096 prompt tokens");
  FASTAR_REQUIRE(std::isfinite(scale) && scale >= 0.0f,
                 "scale must be finite and >= 0 (0 selects 1/sqrt(d))");
  if (Nf == 0) return ok();
  FASTAR_REQUIRE(q_dev && k_dev && v_dev && o_dev && q_codes_dev && p_codes_dev, "NULL pointer");
  FASTAR_REQUIRE(q_planes_dev != nullptr || b == 0, "q_planes is NULL");
  FASTAR_REQUIRE(aligned(q_dev, 16) && aligned(k_dev, 16) && aligned(v_dev, 16) &&
                     aligned(o_dev, 16) && aligned(q_planes_dev, 16) &&
                     aligned(q_codes_dev, 4) && aligned(p_codes_dev, 4),
                 "q, k, v, o and the hyperplanes must be 16-byte aligned, codes 4-byte aligned");
  FASTAR_REQUIRE(q_stride_h % 8 == 0 && q_stride_n % 8 == 0 && kv_stride_h % 8 == 0 &&
                     kv_stride_n % 8 == 0 && o_stride_h % 8 == 0 && o_stride_n % 8 == 0 &&
                     q_stride_n >= d && kv_stride_n >= d && o_stride_n >= d,
                 "strides must be multiples of 16 bytes");
  AttendArgs a{};
  a.q = q_dev;
  a.sq_h = q_stride_h;
  a.sq_n = q_stride_n;
  a.k = k_dev;
  a.v = v_dev;
  a.sk_h = kv_stride_h;
  a.sk_n = kv_stride_n;
  a.n_keys_const = Np;
  a.o = o_dev;
  a.so_h = o_stride_h;
  a.so_n = o_stride_n;
  a.H = H;
  a.d = d;
  a.Nseg = Nf;
  a.F = F;
  a.scale = scale == 0.0f ? 1.0f / std::sqrt((float)d) : scale;
  a.q_codes = q_codes_dev;
  a.p_codes = p_codes_dev;
  a.sel_L = L;
  // the queries' codes, as fastar_hash computes them, then selection and
  // attention in one launch
  HashArgs ha{};
  ha.x = q_dev;
  ha.sx_h = q_stride_h;
  ha.sx_n = q_stride_n;
  ha.H = H;
  ha.N = F * Nf;
  ha.d = d;
  ha.L = L;
  ha.b = b;
  ha.planes = q_planes_dev;
  ha.codes = q_codes_dev;
  ha.codes_ld = (int64_t)F * Nf;
  ha.codes_col0 = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  FASTAR_HIP(launch_hash_bf16(ha, s));
  FASTAR_HIP(launch_annca_fused(a, s));
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// AnnCA without allocation.  The per-frame selection (kept prompt ids and
// their count per head and frame) lives in this file-scope device array
// instead of caller buffers.  Each GPU holds its own copy until the process
// ends; host code uses only the address hipGetSymbolAddress gives for the
// current device, never the array's name.
static __device__ __align__(256) int32_t scratch[FASTAR_ANNCA_STATIC_MAX_SELECTED +
                                                  FASTAR_ANNCA_STATIC_MAX_SEGMENTS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device.
fastar_status scratch_for_current_device(int32_t** out) {
  int dev = 0;
  FASTAR_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FASTAR_ERR_UNSUPPORTED, "device index beyond the library's table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    FASTAR_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return fail(FASTAR_ERR_HIP, "hipGetSymbolAddress gave a NULL address");
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FASTAR_OK;
}

}  // namespace

extern "C" {

fastar_status fastar_annca_attend_static(const void* q_dev, int64_t q_stride_h, int64_t q_stride_n,
                                         const uint32_t* q_codes_dev, const void* k_dev,
                                         const void* v_dev, int64_t kv_stride_h,
                                         int64_t kv_stride_n, const uint32_t* p_codes_dev,
                                         int32_t Nf, int32_t F, int32_t Np, int32_t H, int32_t d,
                                         int32_t L, fastar_dtype dtype, float scale, void* o_dev,
                                         int64_t o_stride_h, int64_t o_stride_n, void* stream) {
  FASTAR_REQUIRE(valid_dtype(dtype), "unknown dtype");
  FASTAR_REQUIRE(d == 64 || d == 128, "d must be 64 or 128");
  FASTAR_REQUIRE(H >= 1 && F >= 1 && L >= 1 && L <= FASTAR_MAX_TABLES, "H, F, L out of range");
  FASTAR_REQUIRE(Nf >= 1 && Nf <= FASTAR_MAX_ANNCA_QUERIES_PER_FRAME, "Nf out of range");
  FASTAR_REQUIRE(Np >= 1 && Np <= FASTAR_MAX_ANNCA_PROMPT, "Np out of range");
  FASTAR_REQUIRE(std::isfinite(scale) && scale >= 0.0f,
                 "scale must be finite and >= 0 (0 selects 1/sqrt(d))");
  if ((int64_t)H * F > FASTAR_ANNCA_STATIC_MAX_SEGMENTS ||
      (int64_t)H * F * Np > FASTAR_ANNCA_STATIC_MAX_SELECTED)
    return fail(FASTAR_ERR_CAPACITY,
                "H*F = " + std::to_string((int64_t)H * F) + " and H*F*Np = " +
                    std::to_string((int64_t)H * F * Np) + " must stay within " +
                    std::to_string(FASTAR_ANNCA_STATIC_MAX_SEGMENTS) + " and " +
                    std::to_string(FASTAR_ANNCA_STATIC_MAX_SELECTED));
  FASTAR_REQUIRE(q_dev && q_codes_dev && k_dev && v_dev && p_codes_dev && o_dev, "NULL pointer");
  const int vec = dtype == FASTAR_BF16 ? 8 : 4;
  FASTAR_REQUIRE(aligned(q_dev, 16) && aligned(k_dev, 16) && aligned(v_dev, 16) &&
                     aligned(o_dev, 16) && aligned(q_codes_dev, 4) && aligned(p_codes_dev, 4),
                 "q, k, v, o must be 16-byte aligned, codes 4-byte aligned");
  FASTAR_REQUIRE(q_stride_h % vec == 0 && q_stride_n % vec == 0 && kv_stride_h % vec == 0 &&
                     kv_stride_n % vec == 0 && o_stride_h % vec == 0 && o_stride_n % vec == 0,
                 "strides must be multiples of 16 bytes");
  int32_t* sp = nullptr;
  fastar_status st = scratch_for_current_device(&sp);
  if (st != FASTAR_OK) return st;
  int32_t* sel_idx = sp;                                    // [H][F][Np]
  int32_t* sel_count = sp + FASTAR_ANNCA_STATIC_MAX_SELECTED;  // [H][F]
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the select kernel writes every (head, frame) count and the first `count`
  // ids of each list, which is all the attention reads: nothing needs clearing
  SelectArgs sa{q_codes_dev, p_codes_dev, Nf, F, Np, H, L, sel_idx, sel_count};
  FASTAR_HIP(launch_annca_select(sa, s));
  AttendArgs a{};
  a.q = q_dev;
  a.sq_h = q_stride_h;
  a.sq_n = q_stride_n;
  a.k = k_dev;
  a.v = v_dev;
  a.sk_h = kv_stride_h;
  a.sk_n = kv_stride_n;
  a.count = nullptr;
  a.count_ld = 0;
  a.n_keys = sel_count;
  a.n_keys_const = Np;
  a.sel = sel_idx;
  a.sel_ld = Np;
  a.o = o_dev;
  a.so_h = o_stride_h;
  a.so_n = o_stride_n;
  a.lse = nullptr;
  a.H = H;
  a.d = d;
  a.Nseg = Nf;
  a.F = F;
  a.scale = scale == 0.0f ? 1.0f / std::sqrt((float)d) : scale;
  FASTAR_HIP(dtype == FASTAR_BF16 ? launch_attend_bf16(a, s) : launch_attend_f32(a, s));
  return ok();
}

}  // extern "C"
