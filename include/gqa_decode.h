/*
 * gqa_decode.h -- C ABI of the MI355X (gfx950) grouped-query-attention decode library.
 *
 * One call computes one attention layer's decode step for a batch of sequences:
 * for every sequence b, new query token t and query head h,
 *
 *     out[b,t,h,:] = sum_j softmax_j( scale * <q[b,t,h,:], K[b,g(h),j,:]> ) * V[b,g(h),j,:]
 *
 * over the cache positions j the token may see, with g(h) = h / (H/G).
 *
 * Sources (page title, section):
 *  - "Grouped-Query Attention (GQA) and Multi-Query Attention (MQA): Mathematical
 *    Foundations ..." (llms.blog), "Multi-Query Attention (MQA)" > "Mathematical
 *    Formulation": logits = einsum(bhnk,bmk->bhnm), weights = softmax(logits + mask),
 *    O = einsum(bhnm,bmv->bhnv); "Grouped-Query Attention (GQA)" > "Mathematical
 *    Formulation": each group's key/value head is broadcast to its H/G query heads,
 *    cache shape [b, G, m, d_k]; "PagedAttention": fixed-size token blocks.
 *  - "Grouped-Query Attention" (aiwiki), the PyTorch listing: repeat_interleave of the
 *    KV heads (contiguous head groups) and scaled_dot_product_attention with is_causal;
 *    the note after it: the kernel derives the KV head from the query head and reads
 *    the cache once instead of copying it. "Interaction with the cache": a page is
 *    shared by the h/g query heads of its group.
 *
 * Conventions shared by every entry point:
 *  - Return value: a gqa_status (0 = success). Nothing is thrown or aborted across
 *    the ABI. Every argument check runs on the host before any HIP call.
 *  - Device arrays are row-major, contiguous, 16-byte aligned, owned by the caller.
 *  - The library never allocates memory; the only state it keeps between calls is a
 *    per-device cache of the compute-unit count and of the device address of the
 *    no-allocation entry point's scratch array (GQA_NOALLOC_SCRATCH_BYTES, which the
 *    code object's loader places on each GPU the library runs on, held until the
 *    process ends).
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* the library is built with hidden visibility; these are its exported symbols */
#pragma GCC visibility push(default)

#define GQA_ABI_VERSION 1

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARGUMENT = 1, /* a NULL/misaligned pointer, a bad size, H % G != 0 ... */
  GQA_ERR_UNSUPPORTED = 2,      /* valid but not compiled: d_h not 64/128, R > 1024, ... */
  GQA_ERR_WORKSPACE = 3,        /* the plan needs split-K scratch the caller did not give */
  GQA_ERR_HIP = 4,              /* a HIP launch or event call failed */
  GQA_ERR_SCRATCH = 5           /* gqa_decode_noalloc: the plan's partials exceed
                                   GQA_NOALLOC_SCRATCH_BYTES */
} gqa_status;

/* Size of the fixed per-device scratch behind gqa_decode_noalloc (65 MiB): the split
 * partials of up to 512 persistent workgroups x 128 packed rows at d_h = 128. */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)65 << 20)

typedef enum gqa_dtype { GQA_DTYPE_F32 = 0, GQA_DTYPE_BF16 = 1 } gqa_dtype;

/* Inner-product policy. AUTO: bf16 groups of R >= 4 packed query rows run QK^T and PV
 * on MFMA (the packed rows make them dense contractions), and so do bf16 groups of
 * fewer rows once the cache (B * G * capacity * d_h K and V elements) holds 16 MiB or
 * more; fp32, and small bf16 caches below R = 4, run on the vector ALUs. The other
 * values force one policy (tests, measurement). */
typedef enum gqa_policy { GQA_POLICY_AUTO = 0, GQA_POLICY_VALU = 1, GQA_POLICY_MFMA = 2 } gqa_policy;

typedef struct gqa_decode_opts {
  uint32_t struct_size;       /* = sizeof(gqa_decode_opts); smaller values are rejected */
  int32_t  dtype;             /* gqa_dtype of q, k_cache, v_cache and out */
  int32_t  causal;            /* 1: token t of q_len sees keys 0 .. L-q_len+t; 0: all L keys */
  int32_t  cache_capacity;    /* contiguous: token stride m of [B,G,m,d_h]; ignored if paged */
  int32_t  page_size;         /* paged: tokens per page, a power of two in [16, 256] */
  int32_t  max_blocks_per_seq;/* paged: row stride of block_table */
  int32_t  num_pages;         /* paged: pages in the pool (entries are clamped to it) */
  int32_t  num_splits;        /* 0: library choice. MFMA policy: number of persistent
                                 workgroups sharing the work; VALU policy: at most this
                                 many context splits per sequence */
  int32_t  chunk_tokens;      /* VALU policy only: 0 or tokens per context split
                                 (rounded up to the kernel's tile) */
  int32_t  policy;            /* gqa_policy */
  void*    workspace;         /* device scratch for split partials (caller-owned) */
  size_t   workspace_bytes;
  void*    profile_events[3]; /* optional hipEvent_t, created by the caller with timing
                                 on. The launches stamp them (hipExtLaunchKernel): [0] and
                                 [1] with the decode kernel's own begin and end times, so
                                 their elapsed time is that kernel's execution alone; [2]
                                 with the end of the merge kernel (recorded on `stream`
                                 after the decode kernel when no merge runs). Any may be
                                 NULL. */
  /* Grouping variants (matrix-core policy, bf16, H <= 256; NULL/0 = plain GQA):
   *  head_group   device int32 [H]: the KV head (in [0, G)) each query head reads, for
   *               a non-uniform allocation of query heads to KV heads decided at call
   *               time (key-norm driven KDGQA/DGQA, "Beyond Uniform Query
   *               Distribution: Key-Driven Grouped Query Attention", Figure 1). H % G
   *               need not be 0 then; a KV head may serve any number of query heads.
   *  max_group_heads  with head_group: an upper bound on the query heads of any one
   *               KV head (0: H); it sizes the packed tile. A larger group is an error
   *               the host cannot see (the map lives on the device): the (token, head)
   *               rows that do not fit the packed tile (row t * n_g + k of a group of
   *               n_g heads, k-th head in ascending order, at or beyond the tile's
   *               rows) are written as NaN, and so are the rows of any head whose
   *               entry lies outside [0, G). `out` is always fully overwritten.
   *  head_active  device uint8 [B, q_len, H]: 0 marks a (token, head) pair that a
   *               router left inactive (Grouped Query Experts: k query heads per token
   *               and group); its output row is 0. Every K/V byte is still read: the
   *               variant cuts query rows, not cache traffic. */
  const int32_t* head_group;
  int32_t  max_group_heads;
  int32_t  reserved0;          /* 0 */
  const uint8_t* head_active;
} gqa_decode_opts;

/* What the library will launch for a shape (no device work; with a GPU present the
 * persistent schedule's workgroup count comes from the device). */
typedef struct gqa_plan {
  int32_t policy;             /* GQA_POLICY_VALU or GQA_POLICY_MFMA */
  int32_t schedule;           /* 0: split-K grid (splits, G*row_blocks, B);
                                 1: persistent balanced workgroups (grid[0] of them) */
  int32_t rows;               /* R = (H/G) * q_len query rows per KV group */
  int32_t row_blocks;         /* split-K grid: workgroups that share one (b, g, split)
                                 along rows; persistent: row blocks per KV group (a
                                 group of more than 256 packed rows is split into equal
                                 blocks of at most 128, each reading the group's K/V;
                                 the 512-wide latent: blocks of at most 32) */
  int32_t tile_tokens;        /* keys staged per pipeline step */
  int32_t chunk_tokens;       /* split-K grid: keys per context split; else 0 */
  int32_t max_splits;         /* split-K grid: ceil(capacity / chunk_tokens);
                                 persistent: partial slots per workgroup (2) */
  int32_t workgroups;         /* workgroups launched by the decode kernel */
  int32_t capacity;           /* tokens addressable per sequence */
  int32_t grid[3];            /* decode kernel grid */
  int32_t block_threads;
  int32_t lds_bytes;
  size_t  workspace_bytes;    /* 0 when no partial results are needed */
} gqa_plan;

/* Fill *opts with defaults: struct_size set, bf16, causal, library-chosen splits, AUTO. */
void gqa_decode_opts_init(gqa_decode_opts* opts);

/*
 * gqa_decode -- one decode step of grouped-query attention (asynchronous on `stream`).
 *
 *   q            [B, q_len, H, d_h]  queries of the q_len new tokens (dtype)
 *   k_cache      contiguous: [B, G, cache_capacity, d_h]
 *                paged (block_table != NULL): pool [num_pages, G, page_size, d_h]
 *   v_cache      same layout as k_cache
 *   seq_lens     int32 [B]: visible keys of sequence b, counting the q_len new tokens,
 *                whose K/V the caller has already written. Precondition (not checked,
 *                it lives on the device): q_len <= seq_lens[b] <= capacity. Values
 *                outside are clamped to [1, capacity]; the result is then unspecified.
 *   block_table  NULL for a contiguous cache, else int32 [B, max_blocks_per_seq]:
 *                entry k is the pool page holding tokens [k*P, (k+1)*P) of sequence b.
 *                Only entries below ceil(seq_lens[b]/P) are read.
 *   out          [B, q_len, H, d_h] (dtype); fully overwritten, must not alias inputs.
 *                bf16 results are rounded to nearest-even from fp32.
 *   B, H, G      batch, query heads, KV heads: 1 <= G <= H, H % G == 0
 *   d_h          head dimension: 64 or 128
 *   q_len        new tokens per sequence (>= 1)
 *   scale        logit scale, applied as given (1/sqrt(d_h) is the SDPA default)
 *   stream       hipStream_t (NULL = default stream)
 *   opts         required; see gqa_decode_opts
 *
 * Errors: INVALID_ARGUMENT for NULL or misaligned pointers, non-positive sizes,
 * H % G != 0, non-finite scale, a bad opts struct or paged geometry; UNSUPPORTED for
 * d_h not in {64,128}, an unknown dtype, R = (H/G)*q_len > 1024, a forced MFMA
 * policy with fp32 or sizes whose tile counts overflow int32; WORKSPACE when the
 * plan needs workspace (gqa_decode_workspace_size) and it is NULL, too small or not
 * 256-byte aligned; HIP when a launch or event record fails.
 */
int gqa_decode(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* seq_lens, const int32_t* block_table, void* out,
               int B, int H, int G, int d_h, int q_len, float scale,
               void* stream, const gqa_decode_opts* opts);

/*
 * gqa_decode_append -- the same decode step, fused with writing the q_len new tokens'
 * keys and values into the cache (asynchronous on `stream`). Each step of
 * autoregressive decoding appends its tokens' K/V to the cache and then attends over
 * the whole cache: the cache traffic that bounds decoding ("The KV-Cache Bandwidth
 * Wall", llms.blog GQA/MQA page); paged caches keep those rows in fixed-size blocks
 * ("PagedAttention", same page).
 *
 *   k_new, v_new [B, q_len, G, d_h] (dtype): K and V of the new tokens, row t of
 *                sequence b being cache position seq_lens[b] - q_len + t.
 *   k_cache, v_cache  written at those positions (contiguous: [b, g, pos]; paged:
 *                page block_table[b][pos / P], slot pos % P, which the caller has
 *                allocated), read everywhere else; no other cache byte is written.
 *   Everything else is as for gqa_decode, whose result this equals when called on
 *   the cache after the append.
 *
 * k_new and v_new must be 16-byte aligned and must not alias the cache or out. On
 * the matrix-core path the new rows are read straight from k_new/v_new and copied
 * into the cache by the kernel that attends over them (one launch plus the merge);
 * on the vector-ALU path a copy kernel runs first. Errors are those of gqa_decode
 * plus INVALID_ARGUMENT for NULL or misaligned k_new / v_new.
 */
int gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                      void* out, int B, int H, int G, int d_h, int q_len, float scale,
                      void* stream, const gqa_decode_opts* opts);

/*
 * gqa_decode_noalloc -- gqa_decode without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Arguments, layouts and results are those of gqa_decode;
 * opts->workspace and opts->workspace_bytes are not read. The split partials go to a
 * fixed array of GQA_NOALLOC_SCRATCH_BYTES per GPU, owned by the library: the call
 * itself allocates nothing and launches the same kernels as gqa_decode.
 *
 * Limit: plans whose workspace (gqa_decode_workspace_size) exceeds
 * GQA_NOALLOC_SCRATCH_BYTES return GQA_ERR_SCRATCH before any HIP call; that covers up
 * to 128 packed rows per KV group at d_h = 128 (256 at d_h = 64) with the default
 * workgroup count. Every call on one GPU shares that GPU's array and leaves it holding
 * its partials: calls that overlap in time on one GPU (two streams, two host threads)
 * race and must be serialised by the caller. Nothing in the array needs clearing
 * between calls: each call writes every partial it reads. Errors are those of
 * gqa_decode, with GQA_ERR_SCRATCH in place of GQA_ERR_WORKSPACE, and GQA_ERR_HIP if
 * the array's device address cannot be obtained.
 */
int gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int32_t* block_table, void* out,
                       int B, int H, int G, int d_h, int q_len, float scale,
                       void* stream, const gqa_decode_opts* opts);

/*
 * gqa_decode_check_inputs -- checks on the device the preconditions that gqa_decode,
 * gqa_decode_noalloc, gqa_decode_append and gqla_absorb_decode document for data in
 * device memory but do not verify: q_len <= seq_lens[b] <= capacity for every b, and,
 * with a block table, every entry a step reads (entry k of row b for
 * k < ceil(seq_lens[b] / page_size)) in [0, num_pages). A paged cache is reached
 * through that table ("PagedAttention", llms.blog GQA/MQA page), so a stray entry is
 * the caller mistake that would make a decode kernel read memory it does not own. For
 * debugging: call it with the seq_lens, block_table, B, q_len and opts of a decode call
 * (capacity or page geometry are read from opts, as there).
 *
 *   report  device int32[4], 4-byte aligned, written by the call: [0] sequences with a
 *           bad length, [1] bad table entries among those read (a row whose length is
 *           bad is checked up to the length clamped to [1, capacity], as the kernels
 *           clamp it), [2] the first bad sequence, [3] the first bad entry as
 *           b * max_blocks_per_seq + k; INT32_MAX in [2] and [3] when there is none.
 *
 * Asynchronous on `stream`; read report after synchronising. Allocates nothing and
 * clears report itself (a kernel, not a memset, so it can be captured in a graph).
 * Errors: INVALID_ARGUMENT for NULL or misaligned seq_lens / block_table / report,
 * B <= 0, q_len <= 0, a bad opts struct or paged geometry (as gqa_decode);
 * UNSUPPORTED when B * max_blocks_per_seq exceeds INT32_MAX; HIP when a launch fails.
 */
int gqa_decode_check_inputs(const int32_t* seq_lens, const int32_t* block_table, int B, int q_len,
                            void* stream, const gqa_decode_opts* opts, int32_t* report);

/* The plan gqa_decode would use for these sizes (validation included). */
int gqa_decode_plan(int B, int H, int G, int d_h, int q_len,
                    const gqa_decode_opts* opts, gqa_plan* plan);

/* Workspace bytes gqa_decode needs for these sizes (0 if none). */
int gqa_decode_workspace_size(int B, int H, int G, int d_h, int q_len,
                              const gqa_decode_opts* opts, size_t* bytes);

const char* gqa_status_string(int status);
int gqa_abi_version(void);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif
#endif /* GQA_DECODE_H */
