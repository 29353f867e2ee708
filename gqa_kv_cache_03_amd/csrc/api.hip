// Host side of the C ABI: argument checks, launch planning and the launches (decode
// and merge; for the GQLA absorbed path also the query fold).
//
// Every argument check runs before any HIP call, so invalid calls return a status
// without touching the device. The library allocates nothing: split partials go to
// the caller's workspace, or, for the no-allocation entry point, to a fixed device
// array that the code object brings. The only state it keeps is a per-device cache of
// the CU count (a read-only device property) and of that array's device address.

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/gqa_decode.h"
#include "../../include/gqla_absorb.h"
#include "gqa_internal.h"

namespace {

using gqa::DecodeParams;

constexpr int kMaxRows = 1024;        // packed rows per KV group (H/G * q_len)
constexpr int kLatentWidth = 512;     // d_c of the GQLA latent (the kernel's head width)
constexpr int kSplitBlockRows = 128;  // rows per block when a group needs several
constexpr int kMaxMappedHeads = 256;  // query heads a head -> group map may cover
constexpr int kTargetSlots = 8192;   // split-kernel workgroup slots the VALU heuristic aims for
constexpr size_t kWsAlign = 256;
constexpr int kMfmaTile = 32;        // keys per tile of the persistent MFMA schedule
constexpr int kDefaultCUs = 256;     // MI355X, used when no device can be queried
constexpr int kWgsPerCu = 2;         // persistent workgroups per CU (fewer if fewer fit)
constexpr double kMfmaMinCacheBytes = 16.0 * (1 << 20);  // K+V capacity from which bf16 R < 4 uses MFMA
constexpr int kMaxDevices = 64;

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int ilog2(int x) { int s = 0; while ((1 << s) < x) ++s; return s; }

// Compute units of the current device (cached per device; MI355X value without one).
int device_cus() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  const int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Scratch of the no-allocation entry point: a file-scope device array, so the code
// object's loader places one copy on every GPU the library runs on, held until the
// process ends. In host code `scratch` only names the symbol; its device address comes
// from hipGetSymbolAddress, once per device, and only that address is handed to
// kernels.
constexpr size_t kScratchBytes = GQA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// This device's copy of `scratch` (looked up on the first call on a device; nullptr
// on failure, with the HIP error cleared).
void* device_scratch() {
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* ptr = cache[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  cache[dev].store(ptr, std::memory_order_release);
  return ptr;
}

struct Plan {
  gqa_plan pub;
  bool paged;
  int page_shift;
  int row_block;
  size_t ws_o_bytes;
  size_t ws_lse_bytes;
};

// latent: the attention of the GQLA absorbed path -- one KV head (G = 1) of width
// d_h = 512 that is both K and V, on the matrix cores only.
int make_plan(int B, int H, int G, int d_h, int q_len, const gqa_decode_opts* opts, bool paged,
              bool query_device, Plan* out, bool latent = false) {
  if (!opts || opts->struct_size < sizeof(gqa_decode_opts)) return GQA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || G <= 0 || d_h <= 0 || q_len <= 0) return GQA_ERR_INVALID_ARGUMENT;
  // grouping variants: a call-time head -> KV head map and a per-(token, head) active
  // mask (matrix-core path only)
  const bool head_map = opts->head_group != nullptr;
  const bool variant = head_map || opts->head_active != nullptr;
  if (G > H || (!head_map && H % G != 0)) return GQA_ERR_INVALID_ARGUMENT;
  if (opts->reserved0 != 0) return GQA_ERR_INVALID_ARGUMENT;
  if (opts->max_group_heads < 0 || opts->max_group_heads > H) return GQA_ERR_INVALID_ARGUMENT;
  if (head_map && !aligned(opts->head_group, 4)) return GQA_ERR_INVALID_ARGUMENT;
  if (opts->dtype != GQA_DTYPE_F32 && opts->dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  if (variant && (opts->dtype != GQA_DTYPE_BF16 || opts->policy == GQA_POLICY_VALU || H > kMaxMappedHeads))
    return GQA_ERR_UNSUPPORTED;
  if (latent ? d_h != kLatentWidth : (d_h != 64 && d_h != 128)) return GQA_ERR_UNSUPPORTED;
  if (latent && (variant || opts->dtype != GQA_DTYPE_BF16 || opts->policy == GQA_POLICY_VALU))
    return GQA_ERR_UNSUPPORTED;
  if (opts->causal != 0 && opts->causal != 1) return GQA_ERR_INVALID_ARGUMENT;
  if (opts->num_splits < 0 || opts->chunk_tokens < 0) return GQA_ERR_INVALID_ARGUMENT;
  if (opts->policy < GQA_POLICY_AUTO || opts->policy > GQA_POLICY_MFMA) return GQA_ERR_INVALID_ARGUMENT;

  // packed rows per KV group: H/G heads x q_len tokens, or the largest group a head
  // map may form
  const int hpg = head_map ? (opts->max_group_heads > 0 ? opts->max_group_heads : H) : H / G;
  const long long R = (long long)hpg * q_len;
  if (R > kMaxRows) return GQA_ERR_UNSUPPORTED;
  if ((long long)B * q_len * H > INT32_MAX / 256) return GQA_ERR_UNSUPPORTED;
  if (B > 65535) return GQA_ERR_UNSUPPORTED;

  Plan p{};
  p.paged = paged;
  int capacity;
  if (paged) {
    const int P = opts->page_size;
    if (P < 16 || P > 256 || (P & (P - 1)) != 0) return GQA_ERR_INVALID_ARGUMENT;
    if (opts->max_blocks_per_seq <= 0 || opts->num_pages <= 0) return GQA_ERR_INVALID_ARGUMENT;
    if ((long long)opts->max_blocks_per_seq * P > INT32_MAX / 2) return GQA_ERR_UNSUPPORTED;
    capacity = opts->max_blocks_per_seq * P;
    p.page_shift = ilog2(P);
  } else {
    if (opts->cache_capacity <= 0) return GQA_ERR_INVALID_ARGUMENT;
    capacity = opts->cache_capacity;
  }
  if (capacity < q_len) return GQA_ERR_INVALID_ARGUMENT;

  int policy = opts->policy;
  if (policy == GQA_POLICY_AUTO) {
    // bf16 runs on the matrix cores from R = 4, and below that too once the cache is
    // large enough (the persistent kernel then streams 10-33% faster than the vector
    // kernel, whose one launch without a merge wins only on small caches)
    const double cache_bytes = 4.0 * B * G * (double)capacity * d_h;
    policy = (opts->dtype == GQA_DTYPE_BF16 && (R >= 4 || variant || latent || cache_bytes >= kMfmaMinCacheBytes))
                 ? GQA_POLICY_MFMA
                 : GQA_POLICY_VALU;
  }
  if (policy == GQA_POLICY_MFMA && opts->dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;

  gqa_plan& pub = p.pub;
  pub.policy = policy;
  pub.rows = (int)R;
  pub.capacity = capacity;
  pub.block_threads = 256;

  if (policy == GQA_POLICY_MFMA) {
    // Persistent balanced schedule: the (sequence, group, row block) segments, cut
    // into 32-key tiles and laid end to end, are shared equally by every workgroup the
    // device holds at once; num_splits > 0 forces the workgroup count instead. A group
    // with more packed rows than one workgroup holds is split into equal row blocks,
    // each a segment that reads the group's K/V (at that size the step is bound by the
    // matrix cores, not by the extra reads).
    // Such a group is cut into blocks of at most 128 rows
    // (for the 64/128-wide kernels): their variant leaves room for two workgroups per
    // CU, which measured faster than half as many 256-row blocks. Each block reads the
    // group's K/V once more, but the blocks of a group are neighbours in the schedule
    // and stream the same tiles at about the same time, and their kernel loads with the
    // default cache policy, so L2 serves most of the repeats (four blocks of 512 rows:
    // 1.06x the single-read bytes from HBM).
    int block_rows = gqa::mfma_max_rows(d_h);
    if (R > block_rows && d_h != kLatentWidth) block_rows = kSplitBlockRows;
    const int n_rb = (int)((R + block_rows - 1) / block_rows);
    const int rb_rows = n_rb == 1 ? (int)R : (int)(((R + n_rb - 1) / n_rb + 15) / 16 * 16);
    const long long max_tiles = (long long)B * G * n_rb * ((capacity + kMfmaTile - 1) / kMfmaTile);
    if (max_tiles > INT32_MAX / 2) return GQA_ERR_UNSUPPORTED;
    const gqa::MfmaVariant v = gqa::mfma_variant_for_rows(rb_rows, d_h, paged, query_device);
    int nwg = opts->num_splits;
    if (nwg == 0) {
      // two per CU measured fastest; fewer when the variant's registers or LDS allow
      // only one
      const int per_cu = (v.wgs_per_cu > 0 && v.wgs_per_cu < kWgsPerCu) ? v.wgs_per_cu : kWgsPerCu;
      nwg = (query_device ? device_cus() : kDefaultCUs) * per_cu;
    }
    if (nwg > (1 << 20)) return GQA_ERR_UNSUPPORTED;
    pub.schedule = 1;
    pub.row_blocks = n_rb;
    p.row_block = rb_rows;
    pub.tile_tokens = kMfmaTile;
    pub.chunk_tokens = 0;
    pub.max_splits = 2;
    pub.workgroups = nwg;
    pub.grid[0] = nwg;
    pub.grid[1] = 1;
    pub.grid[2] = 1;
    pub.lds_bytes = v.lds_bytes;
    const size_t prow = (size_t)nwg * 2 * (size_t)rb_rows;
    p.ws_o_bytes = round_up(prow * d_h * sizeof(float), kWsAlign);
    p.ws_lse_bytes = round_up(prow * sizeof(float), kWsAlign);
    pub.workspace_bytes = p.ws_o_bytes + p.ws_lse_bytes + round_up(((size_t)B + 1) * sizeof(int32_t), kWsAlign);
    *out = p;
    return GQA_OK;
  }

  // split-K grid over (split, group x row block, sequence): the VALU policy
  const int row_block = R >= 8 ? 8 : (R >= 4 ? 4 : (R >= 2 ? 2 : 1));
  const int n_rb = (int)((R + row_block - 1) / row_block);
  const int tile = gqa::valu_tile_tokens(opts->dtype, d_h);
  if ((long long)G * n_rb > 65535) return GQA_ERR_UNSUPPORTED;

  const long long cap_tiles = ((long long)capacity + tile - 1) / tile * tile;
  long long chunk;
  if (opts->chunk_tokens > 0) {
    chunk = ((long long)opts->chunk_tokens + tile - 1) / tile * tile;
  } else if (opts->num_splits > 0) {
    const long long per = ((long long)capacity + opts->num_splits - 1) / opts->num_splits;
    chunk = (per + tile - 1) / tile * tile;
  } else {
    // Enough workgroup slots to balance ragged lengths, but each split long enough
    // that its fp32 partials stay small next to its KV bytes.
    const long long units = (long long)B * G * n_rb;
    const long long par = (long long)capacity * units / kTargetSlots;
    long long lo = 4LL * tile;
    if (16 * R > lo) lo = 16 * R;
    chunk = par > lo ? par : lo;
    chunk = (chunk + tile - 1) / tile * tile;
  }
  if (chunk > cap_tiles) chunk = cap_tiles;
  if (chunk < tile) chunk = tile;
  const long long splits = ((long long)capacity + chunk - 1) / chunk;
  if (splits > INT32_MAX / 2) return GQA_ERR_UNSUPPORTED;

  pub.schedule = 0;
  pub.row_blocks = n_rb;
  pub.tile_tokens = tile;
  pub.chunk_tokens = (int)chunk;
  pub.max_splits = (int)splits;
  pub.workgroups = (int)(splits * G * n_rb * B > INT32_MAX ? INT32_MAX : splits * G * n_rb * B);
  pub.grid[0] = (int)splits;
  pub.grid[1] = G * n_rb;
  pub.grid[2] = B;
  pub.lds_bytes = gqa::valu_lds_bytes(opts->dtype, d_h, row_block);
  p.row_block = row_block;
  if (splits > 1) {
    const size_t rows = (size_t)B * q_len * H * (size_t)splits;
    p.ws_o_bytes = round_up(rows * d_h * sizeof(float), kWsAlign);
    p.ws_lse_bytes = round_up(rows * sizeof(float), kWsAlign);
    pub.workspace_bytes = p.ws_o_bytes + p.ws_lse_bytes;
  }
  *out = p;
  return GQA_OK;
}

// Sizes, schedule and scale of a planned launch (pointers are set by the caller).
void fill_params(DecodeParams& dp, const Plan& p, const gqa_decode_opts* opts, int B, int H, int G, int q_len,
                 float scale) {
  const gqa_plan& pl = p.pub;
  dp.B = B;
  dp.H = H;
  dp.G = G;
  dp.q_len = q_len;
  dp.hpg = H / G;
  dp.R = pl.rows;
  dp.capacity = pl.capacity;
  dp.page_shift = p.paged ? p.page_shift : 0;
  dp.max_blocks = p.paged ? opts->max_blocks_per_seq : 0;
  dp.num_pages = p.paged ? opts->num_pages : 0;
  dp.chunk = pl.chunk_tokens;
  dp.max_splits = pl.max_splits;
  dp.causal = opts->causal;
  dp.row_block = p.row_block;
  dp.n_row_blocks = pl.row_blocks;
  dp.nwg = pl.workgroups;
  dp.qk_scale_log2 = scale * 1.4426950408889634f;
}

// Split partials at the start of `ws`: ws_o, then ws_lse, then the persistent
// schedule's per-sequence prefix sums.
void set_workspace(DecodeParams& dp, const Plan& p, void* ws_base) {
  unsigned char* ws = static_cast<unsigned char*>(ws_base);
  dp.ws_o = reinterpret_cast<float*>(ws);
  dp.ws_lse = reinterpret_cast<float*>(ws + p.ws_o_bytes);
  dp.ws_prefix = reinterpret_cast<int32_t*>(ws + p.ws_o_bytes + p.ws_lse_bytes);
}

// Shared by gqa_decode (k_new == v_new == nullptr) and gqa_decode_append.
// use_scratch: the no-allocation entry point -- the plan's partials go to this
// device's `scratch` instead of opts->workspace (which is not read).
int decode_impl(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                const void* v_cache, const int32_t* seq_lens, const int32_t* block_table, void* out,
                int B, int H, int G, int d_h, int q_len, float scale, void* stream,
                const gqa_decode_opts* opts, bool use_scratch = false) {
  if (!q || !k_cache || !v_cache || !seq_lens || !out || !opts) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(seq_lens, 4) || (block_table && !aligned(block_table, 4)))
    return GQA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARGUMENT;
  if (opts->struct_size >= sizeof(gqa_decode_opts) && !block_table && opts->page_size != 0)
    return GQA_ERR_INVALID_ARGUMENT;
  const bool paged = block_table != nullptr;
  Plan p;
  int st = make_plan(B, H, G, d_h, q_len, opts, paged, /*query_device=*/false, &p);
  if (st != GQA_OK) return st;
  // the device-free plan has the most workgroups the device plan can have on MI355X,
  // so an oversize plan is refused here, before any HIP call
  if (use_scratch && p.pub.workspace_bytes > kScratchBytes) return GQA_ERR_SCRATCH;
  st = make_plan(B, H, G, d_h, q_len, opts, paged, /*query_device=*/true, &p);
  if (st != GQA_OK) return st;
  const gqa_plan& pl = p.pub;
  void* workspace = opts->workspace;
  if (use_scratch) {
    if (pl.workspace_bytes > kScratchBytes) return GQA_ERR_SCRATCH;
    workspace = nullptr;
    if (pl.workspace_bytes > 0 && (workspace = device_scratch()) == nullptr) return GQA_ERR_HIP;
  } else if (pl.workspace_bytes > 0) {
    if (!workspace || !aligned(workspace, kWsAlign) || opts->workspace_bytes < pl.workspace_bytes)
      return GQA_ERR_WORKSPACE;
  }

  DecodeParams dp{};
  fill_params(dp, p, opts, B, H, G, q_len, scale);
  dp.q = q;
  dp.k = k_cache;
  dp.v = v_cache;
  dp.k_new = k_new;
  dp.v_new = v_new;
  dp.seq_lens = seq_lens;
  dp.table = block_table;
  dp.out = out;
  if (pl.workspace_bytes > 0) set_workspace(dp, p, workspace);
  dp.hpg = opts->head_group ? 1 : H / G;  // unused with a head map (groups are counted)
  dp.head_group = opts->head_group;
  dp.head_active = opts->head_active;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(opts->profile_events));
  const dim3 grid(pl.grid[0], pl.grid[1], pl.grid[2]);
  // the persistent merge fills a head map's unmapped rows itself; the split-K path
  // launches the fill on its own
  if (opts->head_group && pl.policy != GQA_POLICY_MFMA && gqa::launch_fill_unmapped(dp, d_h, s) != hipSuccess)
    return GQA_ERR_HIP;
  if (k_new && pl.policy != GQA_POLICY_MFMA) {
    // the vector-ALU kernel reads every key from the cache: write the new rows first
    if (gqa::launch_append(dp, opts->dtype == GQA_DTYPE_BF16 ? 2 : 4, d_h, p.paged, s) != hipSuccess)
      return GQA_ERR_HIP;
  }
  // the profile events ride on the launches: [0]/[1] take the decode kernel's own begin
  // and end times, [2] the merge kernel's end
  hipError_t e = (pl.policy == GQA_POLICY_MFMA)
                     ? gqa::launch_decode_mfma(dp, opts->dtype, d_h, p.paged, grid, s, ev[0], ev[1])
                     : gqa::launch_decode_valu(dp, opts->dtype, d_h, p.paged, grid, s, ev[0], ev[1]);
  if (e != hipSuccess) return GQA_ERR_HIP;
  if (pl.policy == GQA_POLICY_MFMA) {
    e = gqa::launch_merge_persistent(dp, d_h, s, nullptr, ev[2]);
    if (e != hipSuccess) return GQA_ERR_HIP;
  } else if (pl.max_splits > 1) {
    e = gqa::launch_merge(dp, opts->dtype, d_h, s, nullptr, ev[2]);
    if (e != hipSuccess) return GQA_ERR_HIP;
  } else if (ev[2] && hipEventRecord(ev[2], s) != hipSuccess) {
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

// ---- GQLA, absorbed execution ----

struct LatentPlan {
  Plan attn;           // the latent attention: G = 1, head width d_c, rows H * q_len
  size_t q_lat_bytes;  // absorbed queries, bf16 [B q_len H, d_c]
  size_t u_bytes;      // weighted latents, fp32 [B q_len H, d_c]
  size_t total;        // the whole workspace: q_lat, u, then the attention's partials
};

int make_latent_plan(int B, int H, int G, int d_h, int d_c, int q_len, const gqa_decode_opts* opts,
                     bool paged, bool query_device, LatentPlan* out) {
  if (!opts || opts->struct_size < sizeof(gqa_decode_opts)) return GQA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || G <= 0 || d_h <= 0 || d_c <= 0 || q_len <= 0) return GQA_ERR_INVALID_ARGUMENT;
  if (G > H || H % G != 0) return GQA_ERR_INVALID_ARGUMENT;
  if (opts->dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  if ((d_h != 64 && d_h != 128) || d_c != kLatentWidth) return GQA_ERR_UNSUPPORTED;
  LatentPlan lp{};
  const int st = make_plan(B, H, 1, d_c, q_len, opts, paged, query_device, &lp.attn, /*latent=*/true);
  if (st != GQA_OK) return st;
  const size_t rows = (size_t)B * q_len * H;
  lp.q_lat_bytes = round_up(rows * d_c * 2, kWsAlign);
  lp.u_bytes = round_up(rows * d_c * sizeof(float), kWsAlign);
  lp.total = lp.q_lat_bytes + lp.u_bytes + lp.attn.pub.workspace_bytes;
  *out = lp;
  return GQA_OK;
}

// c_new: the append's new latents [B, q_len, d_c] (nullptr: no append).
int latent_impl(const void* q, const void* c_new, const void* latent, const void* w_uk, const void* w_uv,
                const int32_t* seq_lens, const int32_t* block_table, void* out, int B, int H, int G, int d_h,
                int d_c, int q_len, float scale, void* stream, const gqa_decode_opts* opts) {
  if (!q || !latent || !w_uk || !w_uv || !seq_lens || !out || !opts) return GQA_ERR_INVALID_ARGUMENT;
  if (c_new && !aligned(c_new, 16)) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(latent, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16) ||
      !aligned(out, 16) || !aligned(seq_lens, 4) || (block_table && !aligned(block_table, 4)))
    return GQA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARGUMENT;
  if (opts->struct_size >= sizeof(gqa_decode_opts) && !block_table && opts->page_size != 0)
    return GQA_ERR_INVALID_ARGUMENT;
  const bool paged = block_table != nullptr;
  LatentPlan lp;
  int st = make_latent_plan(B, H, G, d_h, d_c, q_len, opts, paged, /*query_device=*/false, &lp);
  if (st != GQA_OK) return st;
  st = make_latent_plan(B, H, G, d_h, d_c, q_len, opts, paged, /*query_device=*/true, &lp);
  if (st != GQA_OK) return st;
  if (!opts->workspace || !aligned(opts->workspace, kWsAlign) || opts->workspace_bytes < lp.total)
    return GQA_ERR_WORKSPACE;
  unsigned char* ws = static_cast<unsigned char*>(opts->workspace);

  gqa::LatentProjParams pp{};
  pp.q = q;
  pp.w_uk = w_uk;
  pp.q_lat = ws;
  pp.B = B;
  pp.H = H;
  pp.G = G;
  pp.q_len = q_len;
  pp.d_h = d_h;
  pp.d_c = d_c;

  // the attention over the latent: every query head (rows H * q_len) reads the one
  // latent head, as K and as V, and leaves its weighted latent u in fp32
  const Plan& p = lp.attn;
  const gqa_plan& pl = p.pub;
  DecodeParams dp{};
  fill_params(dp, p, opts, B, H, 1, q_len, scale);
  dp.q = pp.q_lat;
  dp.k = latent;
  dp.v = latent;
  // the append: the new tokens' latents are read from c_new and written to the cache by
  // the kernel that attends over them (the latent is one tensor, so both pointers)
  dp.k_new = c_new;
  dp.v_new = c_new;
  dp.seq_lens = seq_lens;
  dp.table = block_table;
  dp.out = ws + lp.q_lat_bytes;
  dp.out_f32 = 1;
  // the merge applies each row's W_UV and writes `out`
  dp.w_uv = w_uv;
  dp.proj_out = out;
  dp.proj_dh = d_h;
  dp.proj_groups = G;
  set_workspace(dp, p, ws + lp.q_lat_bytes + lp.u_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(opts->profile_events));
  if (gqa::launch_latent_absorb_q(pp, s) != hipSuccess) return GQA_ERR_HIP;
  const dim3 grid(pl.grid[0], pl.grid[1], pl.grid[2]);
  if (gqa::launch_decode_mfma(dp, GQA_DTYPE_BF16, d_c, paged, grid, s, ev[0], ev[1]) != hipSuccess)
    return GQA_ERR_HIP;
  if (gqa::launch_merge_persistent(dp, d_c, s, nullptr, ev[2]) != hipSuccess) return GQA_ERR_HIP;
  return GQA_OK;
}

}  // namespace

extern "C" {

void gqa_decode_opts_init(gqa_decode_opts* opts) {
  if (!opts) return;
  std::memset(opts, 0, sizeof(*opts));
  opts->struct_size = sizeof(gqa_decode_opts);
  opts->dtype = GQA_DTYPE_BF16;
  opts->causal = 1;
  opts->policy = GQA_POLICY_AUTO;
}

int gqa_abi_version(void) { return GQA_ABI_VERSION; }

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case GQA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case GQA_ERR_HIP: return "HIP runtime error";
    case GQA_ERR_SCRATCH:
      return "the plan needs more split partials than the no-allocation entry point's scratch holds";
    default: return "unknown status";
  }
}

int gqa_decode_plan(int B, int H, int G, int d_h, int q_len, const gqa_decode_opts* opts,
                    gqa_plan* plan) {
  if (!plan || !opts) return GQA_ERR_INVALID_ARGUMENT;
  const bool paged = opts->struct_size >= sizeof(gqa_decode_opts) && opts->page_size > 0;
  Plan p;
  int st = make_plan(B, H, G, d_h, q_len, opts, paged, /*query_device=*/false, &p);
  if (st != GQA_OK) return st;
  // arguments are valid: the device may now be asked how many workgroups it holds
  st = make_plan(B, H, G, d_h, q_len, opts, paged, /*query_device=*/true, &p);
  if (st != GQA_OK) return st;
  *plan = p.pub;
  return GQA_OK;
}

int gqa_decode_workspace_size(int B, int H, int G, int d_h, int q_len, const gqa_decode_opts* opts,
                              size_t* bytes) {
  if (!bytes) return GQA_ERR_INVALID_ARGUMENT;
  gqa_plan plan;
  const int st = gqa_decode_plan(B, H, G, d_h, q_len, opts, &plan);
  if (st != GQA_OK) return st;
  *bytes = plan.workspace_bytes;
  return GQA_OK;
}

int gqa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
               const int32_t* block_table, void* out, int B, int H, int G, int d_h, int q_len,
               float scale, void* stream, const gqa_decode_opts* opts) {
  return decode_impl(q, nullptr, nullptr, k_cache, v_cache, seq_lens, block_table, out, B, H, G, d_h,
                     q_len, scale, stream, opts);
}

int gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                       const int32_t* block_table, void* out, int B, int H, int G, int d_h, int q_len,
                       float scale, void* stream, const gqa_decode_opts* opts) {
  return decode_impl(q, nullptr, nullptr, k_cache, v_cache, seq_lens, block_table, out, B, H, G, d_h,
                     q_len, scale, stream, opts, /*use_scratch=*/true);
}

int gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* seq_lens, const int32_t* block_table, void* out, int B, int H,
                      int G, int d_h, int q_len, float scale, void* stream,
                      const gqa_decode_opts* opts) {
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return GQA_ERR_INVALID_ARGUMENT;
  return decode_impl(q, k_new, v_new, k_cache, v_cache, seq_lens, block_table, out, B, H, G, d_h, q_len,
                     scale, stream, opts);
}

int gqa_decode_check_inputs(const int32_t* seq_lens, const int32_t* block_table, int B, int q_len, void* stream,
                            const gqa_decode_opts* opts, int32_t* report) {
  if (!seq_lens || !report || !opts || opts->struct_size < sizeof(gqa_decode_opts)) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned(seq_lens, 4) || !aligned(report, 4) || (block_table && !aligned(block_table, 4)))
    return GQA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || q_len <= 0) return GQA_ERR_INVALID_ARGUMENT;
  gqa::CheckParams cp{};
  cp.seq_lens = seq_lens;
  cp.table = block_table;
  cp.report = report;
  cp.B = B;
  cp.q_len = q_len;
  if (block_table) {
    const int P = opts->page_size;
    if (P < 16 || P > 256 || (P & (P - 1)) != 0) return GQA_ERR_INVALID_ARGUMENT;
    if (opts->max_blocks_per_seq <= 0 || opts->num_pages <= 0) return GQA_ERR_INVALID_ARGUMENT;
    if ((long long)opts->max_blocks_per_seq * P > INT32_MAX / 2) return GQA_ERR_UNSUPPORTED;
    if ((long long)B * opts->max_blocks_per_seq > INT32_MAX) return GQA_ERR_UNSUPPORTED;
    cp.page_size = P;
    cp.max_blocks = opts->max_blocks_per_seq;
    cp.num_pages = opts->num_pages;
    cp.capacity = opts->max_blocks_per_seq * P;
  } else {
    if (opts->page_size != 0 || opts->cache_capacity <= 0) return GQA_ERR_INVALID_ARGUMENT;
    cp.capacity = opts->cache_capacity;
  }
  if (gqa::launch_check_inputs(cp, static_cast<hipStream_t>(stream)) != hipSuccess) return GQA_ERR_HIP;
  return GQA_OK;
}

int gqla_absorb_plan(int B, int H, int G, int d_h, int d_c, int q_len, const gqa_decode_opts* opts,
                     gqa_plan* plan) {
  if (!plan || !opts) return GQA_ERR_INVALID_ARGUMENT;
  const bool paged = opts->struct_size >= sizeof(gqa_decode_opts) && opts->page_size > 0;
  LatentPlan lp;
  int st = make_latent_plan(B, H, G, d_h, d_c, q_len, opts, paged, /*query_device=*/false, &lp);
  if (st != GQA_OK) return st;
  st = make_latent_plan(B, H, G, d_h, d_c, q_len, opts, paged, /*query_device=*/true, &lp);
  if (st != GQA_OK) return st;
  *plan = lp.attn.pub;
  plan->workspace_bytes = lp.total;
  return GQA_OK;
}

int gqla_absorb_workspace_size(int B, int H, int G, int d_h, int d_c, int q_len, const gqa_decode_opts* opts,
                               size_t* bytes) {
  if (!bytes) return GQA_ERR_INVALID_ARGUMENT;
  gqa_plan plan;
  const int st = gqla_absorb_plan(B, H, G, d_h, d_c, q_len, opts, &plan);
  if (st != GQA_OK) return st;
  *bytes = plan.workspace_bytes;
  return GQA_OK;
}

int gqla_absorb_decode(const void* q, const void* latent_cache, const void* w_uk, const void* w_uv,
                       const int32_t* seq_lens, const int32_t* block_table, void* out, int B, int H, int G,
                       int d_h, int d_c, int q_len, float scale, void* stream, const gqa_decode_opts* opts) {
  return latent_impl(q, nullptr, latent_cache, w_uk, w_uv, seq_lens, block_table, out, B, H, G, d_h, d_c, q_len,
                     scale, stream, opts);
}

int gqla_absorb_decode_append(const void* q, const void* c_new, const void* w_uk, const void* w_uv,
                              void* latent_cache, const int32_t* seq_lens, const int32_t* block_table, void* out,
                              int B, int H, int G, int d_h, int d_c, int q_len, float scale, void* stream,
                              const gqa_decode_opts* opts) {
  if (!c_new) return GQA_ERR_INVALID_ARGUMENT;
  return latent_impl(q, c_new, latent_cache, w_uk, w_uv, seq_lens, block_table, out, B, H, G, d_h, d_c, q_len,
                     scale, stream, opts);
}

}  // extern "C"
