// GQA decode on CDNA4 matrix cores (bf16 in, fp32 accumulate), as a balanced
// persistent split-K pass.
//
// What is computed: for the H/G query heads of KV group g (the aiwiki GQA listing's
// repeat_interleave grouping; the llms.blog page, "Grouped-Query Attention" >
// "Mathematical Formulation": the group's K/V head is broadcast to its H/G query
// heads) and the q_len new tokens, softmax(scale * Q K^T + mask) V over the cached
// keys (llms.blog, "Multi-Query Attention" > "Mathematical Formulation").
//
// Work split. The cached keys of all (sequence b, group g) pairs -- "segments" -- are
// cut into tiles of 32 keys and laid end to end (b-major, then g). Exactly as many
// workgroups run as the chip holds at once (two per CU), and each takes an equal
// contiguous run of that tile sequence, so every workgroup streams the same number of
// bytes whatever the length mix. A segment that starts and ends inside one workgroup
// is finished there and written straight to `out`; a segment cut by a workgroup
// boundary leaves a normalised partial (O, log-sum-exp) in the workspace -- at most
// two per workgroup, its first and last segment -- and the LSE merge kernel combines
// them (flash-decoding split-K over context, with splits sized by work, not by length).
//
// Per workgroup: the group's R = (H/G) * q_len query rows are packed into 16-row MFMA
// tiles held in registers (a group of more than 256 rows is split into row blocks of
// at most 128, each a segment of its own). K/V rows stream from HBM exactly once per
// row block (the aiwiki note after the listing: the cache is read once, not copied per
// head) through an LDS ring (two stages; three at d_h = 64) filled by direct
// global->LDS loads (16 bytes per lane; nontemporal unless the group is split into row
// blocks, whose repeated reads L2 then serves); the ring keeps running across segment
// boundaries.
// Every packed row consumes each staged tile, i.e. the H/G-fold broadcast happens in
// registers, never in memory.
//
// Options handled here as well: the cache append (the new tokens' rows come from
// k_new / v_new and are copied into the cache from LDS), a call-time head -> KV head
// map (non-uniform groups) and a per-(token, head) active mask. D = 512 is the GQLA
// latent of the absorbed execution: one KV head that is both K and V, staged once (its
// append reads the new latents from k_new and writes the one cache).
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, A 16x32 / B 32x16 / C 16x16):
//   S^T = K Q^T with K as the A operand (rows = keys) and Q^T as B (columns = query
//   rows): the C layout leaves lane l with the scores of query row l%16 for keys
//   4*(l/16)+i -- the B-operand layout of P^T, so nothing is shuffled between products.
//   O^T = V^T P^T: A = V^T (one transposed LDS read per 4 keys x column), B = P^T in
//   bf16, C = O^T with lane l holding output row l%16, so softmax rescales are per lane.
// The four waves of a workgroup share each tile and split the rows (NRW) and the
// output columns (NCW); every wave computes the scores it needs itself, except at
// D = 512, where the waves of a row slice split the scores' reduction over d and add
// their parts through LDS.

#include "mfma_common.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
// LDS ring depth and the number of tiles issued ahead of the one being consumed
// (< kStages). Measured on MI355X with two workgroups per CU: one tile ahead (32 KiB
// of K/V in flight per CU) streams faster than two or three, on every workload
// shape here at d_h = 128, so the ring is a double buffer there (d_h = 64: see MfmaCfg).
constexpr int kStages = 2;
constexpr int kAhead = 1;

template <int D, int NRW, int NCW, int RTW>
struct MfmaCfg {
  static constexpr int T = kTile;
  // A d_h = 64 tile is half the bytes: its ring keeps two tiles ahead in three stages,
  // the same 32 KiB in flight per CU (measured 20-24% faster than one tile ahead).
  static constexpr int NS = D == 64 ? 3 : kStages;
  static constexpr int AHEAD = D == 64 ? 2 : kAhead;
  static_assert(AHEAD >= 1 && AHEAD < NS, "a tile is refilled only after every wave has consumed it");
  static constexpr int KB = T / 16;           // 16-key blocks per tile
  static constexpr int CC = D / 32;           // k-steps of QK^T
  static constexpr int CB = D / 16;           // 16-column output blocks
  static constexpr int CBW = CB / NCW;        // output blocks per wave
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  // D = 512 is the GQLA latent: one staged tile is both K and V
  static constexpr bool SHARED = D == 512;
  static constexpr int TENSOR_BYTES = T * ROW_BYTES;
  static constexpr int STAGE_BYTES = (SHARED ? 1 : 2) * TENSOR_BYTES;
  static constexpr int LOADS = T * CPR / kThreads;  // 16-B loads per thread per tensor
  static constexpr int RPL = kThreads / CPR;        // tile rows covered by one such load
  static constexpr int LD = (SHARED ? 1 : 2) * LOADS;  // per thread per stage (K and V)
  // rows after which the staging swizzles repeat
  static constexpr int SWZ_ROWS = SHARED ? 16 : CPR;
  // distinct lane offsets of the staging loads (a load covers RPL rows)
  static constexpr int KP = RPL % SWZ_ROWS == 0 ? 1 : SWZ_ROWS / RPL;
  // The latent's 512-wide scores: the waves that share a row slice split the QK^T
  // reduction over d (each reads a quarter or half of the K tile instead of all of it)
  // and add their partial scores through LDS, instead of each repeating all of it.
  static constexpr bool SPLIT_S = SHARED && NCW > 1;
  static constexpr int CCW = SPLIT_S ? CC / NCW : CC;      // QK^T k-steps per wave
  static constexpr int XCH_BYTES = SPLIT_S ? 4 * 64 * RTW * KB * 16 : 0;  // partial scores
  static constexpr int RING_BYTES = NS * STAGE_BYTES;
  static constexpr int LDS_BYTES = RING_BYTES + XCH_BYTES;
  static_assert(NRW * NCW == 4, "four waves per workgroup");
  static_assert(KB == 2, "one 32-deep PV product per tile");
  static_assert(LOADS >= 1 && (T * CPR) % kThreads == 0, "stage load split");
  static_assert(CB % NCW == 0, "column split");
  static_assert(RPL % SWZ_ROWS == 0 || SWZ_ROWS % RPL == 0, "swizzle period and rows per load");
  static_assert(!SPLIT_S || CC % NCW == 0, "QK^T split");
};

// Position in the flattened tile sequence: segment (b, g, rb) -- row block rb of KV
// group g of sequence b -- tile t of n, sequence length L. Set per segment for the
// staging: fast = the number of leading tiles the plain staging path takes (tiles
// wholly before the end that hold no new token), and base = the byte offset of the
// segment's row 0 in a contiguous cache.
struct Cursor {
  int b, g, rb, t, n, L;
  int fast;
  uint64_t base;
};

// REREAD: the group's rows are split into row blocks, so every K/V tile is staged once
// per block. The blocks of a group are neighbours in the schedule and stream the same
// tiles at about the same time; the default cache policy then lets L2 serve the
// repeats. A single block keeps nontemporal loads (its tiles are never read again).
// The two policies are two kernels (decode_mfma_kernel, decode_mfma_reread_kernel
// below), so neither carries a branch for the other.
template <int D, int NRW, int NCW, int RTW, bool PAGED, bool REREAD>
__device__ __forceinline__ void decode_mfma_body(DecodeParams p) {
  using C = MfmaCfg<D, NRW, NCW, RTW>;
  constexpr int kPolicy = REREAD ? 0 : kNontemporal;
  constexpr int T = C::T, NS = C::NS, AHEAD = C::AHEAD, KB = C::KB, CBW = C::CBW;
  constexpr int CPR = C::CPR, LOADS = C::LOADS, LD = C::LD, ROW_BYTES = C::ROW_BYTES;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cw = wave % NCW;
  const int rw = wave / NCW;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int w = blockIdx.x;

  // ---- 1. this workgroup's share of the flattened tile sequence ----
  // A KV group's R packed rows form n_row_blocks blocks of at most row_block rows (one
  // block unless R exceeds what a workgroup's registers hold); each block is a segment
  // of its own that reads the group's K/V. The first wave of workgroup 0 publishes the
  // per-sequence prefix sums for the merge kernel.
  const ScheduleStart ss = schedule_start(p, T, w, w == 0 && wave == 0);
  const int lo = ss.lo, count = ss.count;
  const int b_start = ss.b, pre_start = ss.pre, L_start = ss.L;
  if (count <= 0 || b_start < 0) return;

  Cursor issue;
  issue.b = b_start;
  issue.L = L_start;
  issue.n = (issue.L + T - 1) / T;
  {
    const int seg = (lo - pre_start) / issue.n;
    issue.g = seg / p.n_row_blocks;
    issue.rb = seg - issue.g * p.n_row_blocks;
    issue.t = (lo - pre_start) - seg * issue.n;
  }
  const unsigned char* __restrict__ kn = static_cast<const unsigned char*>(p.k_new);
  const unsigned char* __restrict__ vn = static_cast<const unsigned char*>(p.v_new);
  auto seg_setup = [&](Cursor& c) {
    int fast = c.L / T;
    // with the append, tile t holds a new token (position >= L - q_len) iff
    // t >= (L - q_len) / T (any t when L - q_len < T)
    if (kn != nullptr) fast = min(fast, (c.L - p.q_len) / T);
    c.fast = fast;
    c.base = ((uint64_t)c.b * p.G + c.g) * (uint64_t)p.capacity * ROW_BYTES;
  };
  seg_setup(issue);
  Cursor cons = issue;

  auto advance = [&](Cursor& c) {
    if (++c.t == c.n) {
      c.t = 0;
      if (++c.rb == p.n_row_blocks) {
        c.rb = 0;
        if (++c.g == p.G) {
          c.g = 0;
          ++c.b;
          if (c.b < p.B) {
            c.L = clamp_len(load_uniform_i32(p.seq_lens, c.b), p.capacity);
            c.n = (c.L + T - 1) / T;
          }
        }
      }
      if (c.b < p.B) seg_setup(c);
    }
  };

  const unsigned char* __restrict__ kg = static_cast<const unsigned char*>(p.k);
  const unsigned char* __restrict__ vg = static_cast<const unsigned char*>(p.v);
  const int pshift = p.page_shift;
  const int pmask = (1 << pshift) - 1;

  // ---- 2. staging: tile f of this workgroup goes to ring stage f % NS ----
  // Cache append (k_new set): positions new0 = L - q_len .. L - 1 are the new tokens,
  // read from k_new / v_new [B, q_len, G, D] instead of the cache (which does not
  // hold them yet); copy_new_rows writes them into the cache once they are in LDS.
  auto tile_has_new = [&](const Cursor& c) { return kn != nullptr && c.t * T + T > c.L - p.q_len; };

  auto cache_row = [&](const Cursor& c, const int* pg, int row, int j) -> size_t {
    if constexpr (PAGED) {
      return (((size_t)pg[row >> 4] * p.G + c.g) * (size_t)(pmask + 1) + (j & pmask)) * ROW_BYTES;
    } else {
      return (((size_t)c.b * p.G + c.g) * (size_t)p.capacity + j) * ROW_BYTES;
    }
  };
  auto tile_pages = [&](const Cursor& c, int* pg) {
    if constexpr (PAGED) {
      const int32_t* trow = p.table + (size_t)c.b * p.max_blocks;
      const int t0 = c.t * T;
#pragma unroll
      for (int gi = 0; gi < T / 16; ++gi) {
        int page = load_uniform_i32(trow, min(t0 + gi * 16, c.L - 1) >> pshift);
        pg[gi] = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
      }
    }
  };

  // Lane-constant part of a staging load: load n of this lane covers tile row
  // n * RPL + rl, 16-byte chunk pch, and fetches global chunk pch ^ swizzle(row). The
  // swizzles repeat every SWZ_ROWS rows, so load n uses offset n % KP of this lane
  // (one offset when a load spans whole periods).
  const int rl = tid / CPR;
  const int pch = tid % CPR;
  uint32_t koff[C::KP], voff[C::KP];
#pragma unroll
  for (int kp = 0; kp < C::KP; ++kp) {
    const int row = kp * C::RPL + rl;
    koff[kp] = (uint32_t)(rl * ROW_BYTES + ((pch ^ swz_k<CPR, C::SHARED>(row)) << 4));
    voff[kp] = (uint32_t)(rl * ROW_BYTES + ((pch ^ swz_v<CPR, C::SHARED>(row)) << 4));
  }

  // Block-table entries of the next tile to issue, one per 16 rows (pages hold at
  // least 16 rows), loaded one pipeline step early so that the scalar loads' latency
  // overlaps the current tile's work instead of delaying the next tile's loads.
  int pf[T / 16] = {};
  auto prefetch_pages = [&](const Cursor& c) {
    if constexpr (PAGED) {
      if (c.b < p.B) {
        const int32_t* trow = p.table + (size_t)c.b * p.max_blocks;
        const int t0 = c.t * T;
#pragma unroll
        for (int gi = 0; gi < T / 16; ++gi) pf[gi] = load_uniform_i32(trow, min(t0 + gi * 16, c.L - 1) >> pshift);
      }
    }
  };
  auto issue_tile = [&](const Cursor& c, int f) {
    unsigned char* st = smem + (f % NS) * C::STAGE_BYTES;
    const int t0 = c.t * T;
    const int end = c.L;
    const int new0 = end - p.q_len;
    const bool has_new = tile_has_new(c);
    // A full tile (no row past the end, no new token) whose loads each stay within one
    // page: a scalar base per load plus the lane-constant offsets.
    if (c.t < c.fast && (!PAGED || (1 << pshift) >= C::RPL)) {
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int j0 = t0 + n * C::RPL;  // first row of this load
        size_t rb;
        if constexpr (PAGED) {
          int page = pf[(n * C::RPL) >> 4];
          page = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
          rb = (((size_t)page * p.G + c.g) * (size_t)(pmask + 1) + (j0 & pmask)) * ROW_BYTES;
        } else {
          rb = c.base + (uint64_t)(uint32_t)j0 * ROW_BYTES;
        }
        const int lds_off = n * kThreads * 16 + wave * 1024;  // this wave's 64 x 16 B slots
        load16_to_lds<kPolicy>(kg + rb + koff[n % C::KP], st + lds_off);
        if constexpr (!C::SHARED)
          load16_to_lds<kPolicy>(vg + rb + voff[n % C::KP], st + C::TENSOR_BYTES + lds_off);
      }
      return;
    }
    int pg[T / 16] = {};
    tile_pages(c, pg);
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int qi = n * kThreads + tid;
      const int row = qi / CPR, pch = qi % CPR;
      const int j = min(t0 + row, end - 1);  // past the end: re-read the last row (masked)
      const size_t rb = cache_row(c, pg, row, j);
      const unsigned char* ksrc = kg + rb;
      const unsigned char* vsrc = vg + rb;
      if (has_new) {
        asm volatile("");  // keep this a branch: only tiles holding new tokens pay for it
        if (j >= new0) {
          const size_t nb = (((size_t)c.b * p.q_len + (j - new0)) * p.G + c.g) * ROW_BYTES;
          ksrc = kn + nb;
          vsrc = vn + nb;
        }
      }
      const int lds_off = n * kThreads * 16 + wave * 1024;  // this wave's 64 x 16 B slots
      load16_to_lds<kPolicy>(ksrc + ((pch ^ swz_k<CPR, C::SHARED>(row)) << 4), st + lds_off);
      if constexpr (!C::SHARED)
        load16_to_lds<kPolicy>(vsrc + ((pch ^ swz_v<CPR, C::SHARED>(row)) << 4), st + C::TENSOR_BYTES + lds_off);
    }
  };

  // Writes the new tokens' rows of staged tile f (already in LDS: every lane reads
  // back the chunks its own loads placed) into the cache. Called right after the
  // tile's wait, which its own loads have passed (later tiles may still be loading).
  auto copy_new_rows = [&](const Cursor& c, int f) {
    // every row block of a group stages the same tile; the first one writes it (the
    // latent is one tensor: its new rows go to the one cache)
    if (!tile_has_new(c) || c.rb != 0) return;
    const unsigned char* st = smem + (f % NS) * C::STAGE_BYTES;
    const int t0 = c.t * T;
    const int new0 = c.L - p.q_len;
    unsigned char* kc = static_cast<unsigned char*>(const_cast<void*>(p.k));
    [[maybe_unused]] unsigned char* vc = static_cast<unsigned char*>(const_cast<void*>(p.v));
    int pg[T / 16] = {};
    tile_pages(c, pg);
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int qi = n * kThreads + tid;
      const int row = qi / CPR, pch = qi % CPR;
      const int j = t0 + row;
      if (j >= new0 && j < c.L) {  // a new token's row (not a re-read past the end)
        const int slot = n * kThreads * 16 + wave * 1024 + lane * 16;
        const u32x4 kv = *reinterpret_cast<const u32x4*>(st + slot);
        const size_t rb = cache_row(c, pg, row, j);
        *reinterpret_cast<u32x4*>(kc + rb + ((pch ^ swz_k<CPR, C::SHARED>(row)) << 4)) = kv;
        if constexpr (!C::SHARED) {
          const u32x4 vv = *reinterpret_cast<const u32x4*>(st + C::TENSOR_BYTES + slot);
          *reinterpret_cast<u32x4*>(vc + rb + ((pch ^ swz_v<CPR, C::SHARED>(row)) << 4)) = vv;
        }
      }
    }
  };

  // ---- 3. per-segment state ----
  // query fragments: k-steps cc0 .. cc0 + CCW - 1 of QK^T (all of them unless split)
  constexpr int CCW = C::CCW;
  const int cc0 = C::SPLIT_S ? cw * CCW : 0;
  bf16x8 qf[RTW][CCW];
  float m_run[RTW], l_run[RTW];
  f32x4 o[RTW][CBW];
  float neg_m[RTW];  // -m_run (0 while m_run = -inf)
  int lim_k[RTW];    // the row's last visible key, less this lane's key offset g4 * 4
  int lim_min = 0;
  // query (token, head) of this lane's packed row in each row tile of the current
  // segment (-1: a padding row), and whether that pair is active
  int row_t[RTW], row_h[RTW];
  bool row_on[RTW];

  auto begin_segment = [&](const Cursor& c) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      m_run[rt] = kNegInf;
      neg_m[rt] = 0.f;
      l_run[rt] = 0.f;
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) o[rt][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // padding rows take the last token's limit (their results are discarded)
      const int t = row_t[rt] >= 0 ? row_t[rt] : p.q_len - 1;
      lim_k[rt] = (p.causal ? (c.L - p.q_len + t) : (c.L - 1)) - g4 * 4;
    }
    lim_min = p.causal ? (c.L - p.q_len) : (c.L - 1);
  };

  // |scale| log2(e), kept away from 0 so that a masked -inf logit stays -inf; with a
  // zero scale every visible exponent is then within 1e-20 of 0 and every weight
  // rounds to exactly 1, as it should
  const float qk_c = fmaxf(fabsf(p.qk_scale_log2), 1e-30f);
  const unsigned q_sign = p.qk_scale_log2 < 0.f ? 0x80008000u : 0u;  // negative scale: flip q

  // Packed rows of a segment: row r of KV group g is query token t = r / n_g of the
  // group's (r % n_g)-th query head, n_g heads in ascending order. Contiguous groups
  // (no head map): n_g = H/G, heads g*n_g ... A head map (non-uniform groups) is read
  // with one ballot per 64 heads; a lane then finds its head as the k-th set bit.
  auto map_rows = [&](const Cursor& c) {
    int n_g = p.hpg;
    unsigned long long gm[4] = {0ull, 0ull, 0ull, 0ull};
    if (p.head_group) {
      n_g = 0;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const int h = ch * 64 + lane;
        const bool in = h < p.H && p.head_group[h] == c.g;
        gm[ch] = __builtin_amdgcn_ballot_w64(in);
        n_g += __builtin_popcountll(gm[ch]);
      }
    }
    const int R_g = n_g * p.q_len;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int r_local = (rw * RTW + rt) * 16 + l16;
      const int r = c.rb * p.row_block + r_local;
      row_t[rt] = -1;
      row_h[rt] = 0;
      if (r_local < p.row_block && r < R_g) {
        const int t = r / n_g;
        const int k = r - t * n_g;
        int h = c.g * n_g + k;
        if (p.head_group) {
          int before = 0;
          h = 0;
#pragma unroll
          for (int ch = 0; ch < 4; ++ch) {
            const int cnt = __builtin_popcountll(gm[ch]);
            if (k >= before && k < before + cnt) {
              // position of set bit (k - before) of gm[ch], by binary search on
              // prefix popcounts
              const int want = k - before;
              int pos = 0;
#pragma unroll
              for (int step = 32; step >= 1; step >>= 1) {
                const unsigned long long below = (1ull << (pos + step)) - 1ull;
                if (__builtin_popcountll(gm[ch] & below) <= want) pos += step;
              }
              h = ch * 64 + pos;
            }
            before += cnt;
          }
        }
        row_t[rt] = t;
        row_h[rt] = h;
      }
      row_on[rt] = row_t[rt] >= 0 &&
                   (p.head_active == nullptr ||
                    p.head_active[((size_t)c.b * p.q_len + row_t[rt]) * p.H + row_h[rt]] != 0);
    }
  };

  // packed query rows of segment (b, g, rb), as B operands of S^T = K Q^T
  auto load_q = [&](const Cursor& c) {
    map_rows(c);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      if (row_t[rt] >= 0) {
        const int t = row_t[rt];
        const int h = row_h[rt];
        const __bf16* qrow = static_cast<const __bf16*>(p.q) + ((size_t)(c.b * p.q_len + t) * p.H + h) * D;
#pragma unroll
        for (int cc = 0; cc < CCW; ++cc) {
          const u32x4 bits = *reinterpret_cast<const u32x4*>(qrow + (cc0 + cc) * 32 + g4 * 8) ^ q_sign;
          qf[rt][cc] = __builtin_bit_cast(bf16x8, bits);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < CCW; ++cc) qf[rt][cc] = bf16x8{};
      }
    }
  };

  // ---- 4. consume one staged tile: S^T = K Q^T, online softmax, O^T += V^T P^T ----
  // Every LDS read address of a tile is one of the lane constants below (for ring
  // stage 0) plus the stage's byte offset, one add per address per tile.
  constexpr int HI = 16 * ROW_BYTES;  // 16 rows on (the staging swizzles repeat every 16 rows)
  // QK^T A operands: key rows l16 and l16 + 16, chunk (cc0 + cc) * 4 + g4
  unsigned k_lane[CCW];
#pragma unroll
  for (int cc = 0; cc < CCW; ++cc)
    k_lane[cc] = lds_addr(smem + l16 * ROW_BYTES + ((((cc0 + cc) * 4 + g4) ^ swz_k<CPR, C::SHARED>(l16)) << 4));
  // O^T += V^T P^T over this wave's output columns. k-slots 8 * g4 + e are keys
  // 4 * g4 + e of block 0 (e < 4), then of block 1 (e >= 4); a V^T fragment (4 keys of
  // one column per lane) is one transposed LDS read: lane p of a 16-lane group points
  // at key row g4 * 4 + p / 4, columns c0 + 4 (p % 4) .. +3 of column block cb (the
  // second half of the k-slots: the same columns 16 rows further on). In the latent
  // the V tile is the K tile.
  unsigned v_lane[CBW];
#pragma unroll
  for (int cb = 0; cb < CBW; ++cb) {
    const int r = g4 * 4 + (l16 >> 2);
    const int c = (cw * CBW + cb) * 16 + ((l16 & 3) << 2);
    v_lane[cb] = lds_addr(smem + (C::SHARED ? 0 : C::TENSOR_BYTES) + r * ROW_BYTES +
                          ((((c >> 3) ^ swz_v<CPR, C::SHARED>(r)) << 4) | ((c & 7) << 1)));
  }

  // so: the stage's byte offset. masked: some key of the tile lies past a row's last
  // visible key (only the last tile or two of a segment), so those logits are set to
  // -inf first.
  auto consume = [&](const unsigned so, const int tile0, const bool masked) {
    // The two waves that share a SIMD (one per workgroup) alternate between matrix
    // products and softmax; a wave issuing products and their operand reads runs at a
    // raised issue priority (s_setprio 1), so the matrix cores are fed first while the
    // other wave's softmax fills the gaps (2-4% faster at R = 128 and 512, neutral below).
    __builtin_amdgcn_s_setprio(1);
    f32x4 s[RTW][KB];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[rt][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K fragments in groups of up to four k-steps, one LDS round trip per group
    constexpr int KG = CCW >= 4 ? 4 : CCW;
    static_assert((KG == 2 || KG == 4) && CCW % KG == 0, "K read groups");
#pragma unroll
    for (int c0 = 0; c0 < CCW; c0 += KG) {
      u32x4 kf[KG][KB];
      unsigned ka[KG];
#pragma unroll
      for (int i = 0; i < KG; ++i) ka[i] = k_lane[c0 + i] + so;
      lds_read_b128_rows<KG, HI>(ka, kf);
#pragma unroll
      for (int i = 0; i < KG; ++i)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt)
            s[rt][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[i][kb]),
                                                                qf[rt][c0 + i], s[rt][kb], 0, 0, 0);
    }
    if constexpr (C::SPLIT_S) {
      // Every wave of the row slice now holds the partial scores of its share of d,
      // laid out identically; sum them through the exchange area. The barrier waits
      // for LDS only: the ring's loads stay in flight. The exchange area is rewritten
      // only after the next tile's ring barrier, when every wave has read it.
      f32x4* xs = reinterpret_cast<f32x4*>(smem + C::RING_BYTES);
      constexpr int NV = RTW * KB;  // 16-byte vectors per lane
      // [wave][vector][lane]: each 16-byte store and load of a wave is contiguous
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) xs[(wave * NV + rt * KB + kb) * 64 + lane] = s[rt][kb];
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt((15 << 0) | (7 << 4) | (3 << 14));  // lgkmcnt(0) only
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int o = 1; o < NCW; ++o) {
        const int other = rw * NCW + (cw + o) % NCW;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) s[rt][kb] += xs[(other * NV + rt * KB + kb) * 64 + lane];
      }
    }

    // With separate K and V tiles, every V^T fragment is read right after the QK^T
    // products are issued, so that the reads' latency passes while the matrix cores
    // work; the scheduling barriers keep the products above the reads and the softmax
    // below them. (The latent's wider rows would need twice the registers; it reads
    // each pair of blocks just before its product.)
    constexpr bool EARLY_V = !C::SHARED;
    bf16x4 vlo[EARLY_V ? CBW : 1], vhi[EARLY_V ? CBW : 1];
    if constexpr (EARLY_V) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (CBW >= 4) {
        static_assert(CBW % 4 == 0, "V^T read groups");
#pragma unroll
        for (int c0 = 0; c0 < CBW; c0 += 4) {
          const unsigned va[4] = {v_lane[c0] + so, v_lane[c0 + 1] + so, v_lane[c0 + 2] + so, v_lane[c0 + 3] + so};
          u32x2 vf[4][2];
          lds_read_tr16_x8<HI>(va, vf);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vlo[c0 + i] = __builtin_bit_cast(bf16x4, vf[i][0]);
            vhi[c0 + i] = __builtin_bit_cast(bf16x4, vf[i][1]);
          }
        }
      } else if constexpr (CBW == 2) {
        lds_read_tr16_x4<HI>(v_lane[0] + so, v_lane[1] + so, vlo[0], vhi[0], vlo[1], vhi[1]);
      } else {
        lds_read_tr16_x2<HI>(v_lane[0] + so, vlo[0], vhi[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);

    // Online softmax (base 2). Logits are s * c with c = |scale| log2(e) > 0 (a
    // negative scale was moved into the query's sign), so the row max is taken on the
    // raw products and p = exp2(fma(s, c, -m)) costs one FMA per score. A row's
    // reference max m only moves when a tile max exceeds it by more than
    // 2^kRescaleLog2; until then p <= 2^kRescaleLog2 and O and l keep their scale, so
    // most tiles skip the rescale (numerator and denominator share m). Each lane first
    // checks its own scores; only when one of them crosses that line anywhere in the
    // wave are the row maxima formed across lanes. P is rounded to bf16 for the PV
    // product and the denominator sums those rounded weights (dot2 with (1, 1)), so the
    // normalised weights sum to one.
    bf16x2 pk[RTW][KB][2];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      if (masked) {
        // a real (uniform) branch: without the empty volatile statement the compiler
        // turns the block into a compare and select per score on every tile
        asm volatile("");
        const int d = lim_k[rt] - tile0;  // key kb * 16 + g4 * 4 + i is visible iff kb * 16 + i <= d
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb * 16 + i > d) s[rt][kb][i] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[rt][kb][i]);
      // -inf + c = -inf: a first finite max grows
      if (__builtin_amdgcn_ballot_w64(mx * qk_c > m_run[rt] + kRescaleLog2)) {
        mx = wave_max_across_groups(mx) * qk_c;
        const bool grow = mx > m_run[rt] + kRescaleLog2;
        const float m_new = grow ? mx : m_run[rt];
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[rt] - m_new) : 1.f;
        l_run[rt] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CBW; ++cb) o[rt][cb] *= alpha;
        m_run[rt] = m_new;
        neg_m[rt] = (m_new == kNegInf) ? 0.f : -m_new;
      }
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x2 e = {(__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][kb][2 * h], qk_c, neg_m[rt])),
                            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][kb][2 * h + 1], qk_c, neg_m[rt]))};
          pk[rt][kb][h] = e;
          sum = __builtin_amdgcn_fdot2_f32_bf16(e, kOnes2, sum, false);
        }
      l_run[rt] += sum;
    }

    bf16x8 pb[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const bf16x4 lo4 = __builtin_shufflevector(pk[rt][0][0], pk[rt][0][1], 0, 1, 2, 3);
      const bf16x4 hi4 = __builtin_shufflevector(pk[rt][1][0], pk[rt][1][1], 0, 1, 2, 3);
      pb[rt] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    auto pv = [&](int cb, bf16x4 lo4, bf16x4 hi4) {
      const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
        o[rt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rt], o[rt][cb], 0, 0, 0);
    };
    if constexpr (EARLY_V) {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) pv(cb, vlo[cb], vhi[cb]);
      __builtin_amdgcn_s_setprio(0);
    } else if constexpr (CBW % 2 == 0) {
#pragma unroll
      for (int cb = 0; cb < CBW; cb += 2) {
        bf16x4 l0, h0, l1, h1;
        lds_read_tr16_x4<HI>(v_lane[cb] + so, v_lane[cb + 1] + so, l0, h0, l1, h1);
        pv(cb, l0, h0);
        pv(cb + 1, l1, h1);
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) {
        bf16x4 l0, h0;
        lds_read_tr16_x2<HI>(v_lane[cb] + so, l0, h0);
        pv(cb, l0, h0);
      }
    }
  };

  // ---- 5. finish a segment: final output, or a partial for the merge ----
  // slot 0: the workgroup's first segment; slot 1: its last one (when different).
  auto finish_segment = [&](const Cursor& c, bool complete, int slot) {
    const size_t rows_per_b = (size_t)p.q_len * p.H;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      // an inactive (token, head) pair writes zeros (and an empty partial)
      const float l = wave_sum_across_groups(l_run[rt]);
      const bool live = l > 0.f && row_on[rt];
      const float inv = live ? 1.f / l : 0.f;
      const float lse = live ? m_run[rt] + __log2f(l) : kNegInf;
      const int r_local = (rw * RTW + rt) * 16 + l16;
      if (row_t[rt] >= 0) {
        const int t = row_t[rt];
        const int h = row_h[rt];
        const size_t orow = (size_t)c.b * rows_per_b + (size_t)t * p.H + h;
        const size_t prow = ((size_t)w * 2 + slot) * p.row_block + r_local;
#pragma unroll
        for (int cb = 0; cb < CBW; ++cb) {
          const int col = (cw * CBW + cb) * 16 + g4 * 4;
          const f32x4 val = o[rt][cb] * inv;
          if (complete && p.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + orow * D + col) = val;
          } else if (complete) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = (__bf16)val[i];
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + orow * D + col) = ov;
          } else {
            *reinterpret_cast<f32x4*>(p.ws_o + prow * D + col) = val;
          }
        }
        if (!complete && cw == 0 && g4 == 0) p.ws_lse[prow] = lse;
      }
    }
  };

  // ---- 6. the pipeline ----
  // prologue: tiles 0 .. AHEAD-1 in flight, then the first segment's queries; one
  // full wait covers both, so no wait for the query registers is left in the loop.
  {
    Cursor c = issue;
    prefetch_pages(c);
#pragma unroll
    for (int f = 0; f < AHEAD; ++f) {
      if (f < count) {
        issue_tile(c, f);
        advance(c);
        prefetch_pages(c);
      }
    }
    issue = c;
  }
  asm volatile("" ::: "memory");
  load_q(cons);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((7 << 4));  // vmcnt(0) expcnt(7) lgkmcnt(0)
  asm volatile("" ::: "memory");

  bool first_segment = true;  // the segment being consumed contains tile lo
  bool seg_from_start = cons.t == 0;
  begin_segment(cons);
  for (int f = 0; f < count; ++f) {
    const bool new_segment = f > 0 && cons.t == 0;
    if (new_segment) {
      // A segment switch: the previous segment's stores and this segment's query
      // loads share the vector-memory counter with the ring's loads and may complete
      // out of order with them, so wait for everything once (rare: at most a few
      // switches per workgroup).
      load_q(cons);
      asm volatile("" ::: "memory");
      wait_vm_and_sync<0>();
      begin_segment(cons);
      seg_from_start = true;
    } else {
      wait_tiles<LD, AHEAD - 1>(count - 1 - f);  // tiles issued after this one: min(AHEAD - 1, .)
    }
    // new tokens' rows of this tile go to the cache before the next tile is issued,
    // so their LDS read-back needs no wait beyond the tile's own
    copy_new_rows(cons, f);
    // the stage refilled next was last read at step f + AHEAD - NS <= f - 1, which
    // every wave has finished (the barrier above)
    if (f + AHEAD < count) {
      issue_tile(issue, f + AHEAD);
      advance(issue);
      prefetch_pages(issue);
    }
    const int tile0 = cons.t * T;
    const bool masked = tile0 + T - 1 > lim_min;
    consume((unsigned)((f % NS) * C::STAGE_BYTES), tile0, masked);
    const bool seg_end = cons.t == cons.n - 1;
    if (seg_end || f == count - 1) {
      const bool complete = seg_from_start && seg_end;
      finish_segment(cons, complete, first_segment ? 0 : 1);
      first_segment = false;
    }
    advance(cons);
  }
}

template <int D, int NRW, int NCW, int RTW, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeParams p) {
  decode_mfma_body<D, NRW, NCW, RTW, PAGED, false>(p);
}

template <int D, int NRW, int NCW, int RTW, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_mfma_reread_kernel(DecodeParams p) {
  decode_mfma_body<D, NRW, NCW, RTW, PAGED, true>(p);
}

// The layouts a group split into row blocks runs on (blocks of at most 128 rows, or 32
// in the latent), which alone get the re-reading kernel.
template <int D, int NRW, int NCW, int RTW>
constexpr bool kRowBlockLayout = D == 512 ? (NRW == 2 && NCW == 2) : (NRW == 4 && RTW == 2);

template <int D, int NRW, int NCW, int RTW>
hipError_t launch_variant(const DecodeParams& p, bool paged, dim3 grid, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
  static_assert(kThreads == 256, "launch_timed launches 256 threads");
  if constexpr (kRowBlockLayout<D, NRW, NCW, RTW>) {
    if (p.n_row_blocks > 1) {
      if (paged)
        launch_timed(decode_mfma_reread_kernel<D, NRW, NCW, RTW, true>, grid, stream, start, stop, p);
      else
        launch_timed(decode_mfma_reread_kernel<D, NRW, NCW, RTW, false>, grid, stream, start, stop, p);
      return hipGetLastError();
    }
  }
  if (paged)
    launch_timed(decode_mfma_kernel<D, NRW, NCW, RTW, true>, grid, stream, start, stop, p);
  else
    launch_timed(decode_mfma_kernel<D, NRW, NCW, RTW, false>, grid, stream, start, stop, p);
  return hipGetLastError();
}

template <int D, int NRW, int NCW, int RTW>
int variant_occupancy(bool paged) {
  int n = 0;
  const hipError_t e =
      paged ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<D, NRW, NCW, RTW, true>, kThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<D, NRW, NCW, RTW, false>, kThreads, 0);
  return e == hipSuccess ? n : 0;
}

// Wave layouts by packed row count R: X(max R, row slices, column slices, row tiles
// per wave). Every wave of a workgroup reads the whole tile.
#define GQA_MFMA_VARIANTS(X) \
  X(16, 1, 4, 1)             \
  X(32, 2, 2, 1)             \
  X(64, 4, 1, 1)             \
  X(128, 4, 1, 2)            \
  X(256, 4, 1, 4)

// The 512-wide latent (K = V, staged once): up to 32 rows per workgroup, the query
// fragments alone taking 64 registers per row tile.
#define GQA_MFMA_LATENT_VARIANTS(X) \
  X(16, 1, 4, 1)                    \
  X(32, 2, 2, 1)

template <int D>
hipError_t launch_for_rows(const DecodeParams& p, bool paged, dim3 grid, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop) {
#define X(ROWS, NRW, NCW, RTW) \
  if (p.row_block <= ROWS) return launch_variant<D, NRW, NCW, RTW>(p, paged, grid, stream, start, stop);
  if constexpr (D == 512) {
    GQA_MFMA_LATENT_VARIANTS(X)
  } else {
    GQA_MFMA_VARIANTS(X)
  }
#undef X
  return hipErrorInvalidValue;
}

template <int D>
MfmaVariant variant_for(int R, bool paged, bool query_device) {
#define X(ROWS, NRW, NCW, RTW)                                                                      \
  if (R <= ROWS)                                                                                     \
    return MfmaVariant{ROWS, kTile, MfmaCfg<D, NRW, NCW, RTW>::LDS_BYTES,                            \
                       query_device ? variant_occupancy<D, NRW, NCW, RTW>(paged) : 0};
  if constexpr (D == 512) {
    GQA_MFMA_LATENT_VARIANTS(X)
  } else {
    GQA_MFMA_VARIANTS(X)
  }
#undef X
  return MfmaVariant{0, kTile, 0, 0};
}

}  // namespace

MfmaVariant mfma_variant_for_rows(int R, int d_h, bool paged, bool query_device) {
  if (d_h == 512) return variant_for<512>(R, paged, query_device);
  return d_h == 64 ? variant_for<64>(R, paged, query_device) : variant_for<128>(R, paged, query_device);
}

int mfma_max_rows(int d_h) { return d_h == 512 ? 32 : 256; }

hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int d_h, bool paged, dim3 grid,
                              hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  (void)dtype;  // bf16 only (checked by the planner)
  if (d_h == 512) return launch_for_rows<512>(p, paged, grid, stream, start, stop);
  if (d_h == 64) return launch_for_rows<64>(p, paged, grid, stream, start, stop);
  return launch_for_rows<128>(p, paged, grid, stream, start, stop);
}

}  // namespace gqa
