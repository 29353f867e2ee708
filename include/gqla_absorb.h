/*
 * gqla_absorb.h -- C ABI of the absorbed (MQA) execution of a Group-Query Latent
 * Attention (GQLA) decode step, in the same library as gqa_decode.h.
 *
 * Source: the thelatestinai page for paper 2604.07766, the GQLA abstract. Each group g
 * of H/G query heads shares one pair of up-projections, W_UK[g] and W_UV[g], each
 * d_h x d_c. Every cached token keeps one joint latent vector c_j of d_c numbers,
 * shared by all groups. The group's key and value for token j are W_UK[g] c_j and
 * W_UV[g] c_j: the expanded, per-group cache that plain GQA execution (gqa_decode)
 * reads. The same weights also run as MQA with the projections absorbed, which is
 * what this entry point computes. For every sequence b, new token t and query head h
 * with group g = h / (H/G):
 *
 *     q_lat   = W_UK[g]^T q[b,t,h,:]                      (d_c numbers)
 *     u       = sum_j softmax_j( scale * <q_lat, c_j> ) c_j  (over the visible j)
 *     out[b,t,h,:] = W_UV[g] u
 *
 * This equals gqa_decode over the expanded cache up to rounding. That cache holds
 * 2 G d_h numbers per token; the latent holds d_c.
 *
 * Conventions are those of gqa_decode.h: a gqa_status return, every check on the host
 * before any HIP call, caller-owned 16-byte-aligned row-major device arrays, and no
 * allocation.
 */
#ifndef GQLA_ABSORB_H
#define GQLA_ABSORB_H

#include "gqa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

#pragma GCC visibility push(default)

/*
 * gqla_absorb_decode -- one decode step of a GQLA layer in its absorbed form
 * (asynchronous on `stream`).
 *
 *   q            bf16 [B, q_len, H, d_h]  queries of the q_len new tokens
 *   latent_cache bf16, contiguous: [B, cache_capacity, d_c]; paged (block_table !=
 *                NULL): pool [num_pages, page_size, d_c], one latent row per token
 *   w_uk, w_uv   bf16 [G, d_h, d_c]: the groups' up-projections (row i of w_uk[g]
 *                maps a latent to component i of the group's key)
 *   seq_lens     int32 [B]: visible tokens of sequence b, counting the q_len new ones,
 *                whose latents the caller has already written. Same precondition and
 *                clamping as gqa_decode.
 *   block_table  as for gqa_decode, over latent pages
 *   out          bf16 [B, q_len, H, d_h]; fully overwritten, must not alias inputs
 *   B, H, G      batch, query heads, groups: 1 <= G <= H, H % G == 0
 *   d_h          64 or 128;  d_c  the latent width: 512
 *   q_len, scale, stream   as for gqa_decode
 *   opts         required: dtype must be GQA_DTYPE_BF16. causal, cache_capacity,
 *                page_size, max_blocks_per_seq, num_pages, num_splits (persistent
 *                workgroups), policy (AUTO or MFMA), workspace and workspace_bytes
 *                mean what they mean for gqa_decode. profile_events time the latent
 *                attention kernel and its merge. head_group and head_active must be
 *                NULL.
 *
 * The workspace (gqla_absorb_workspace_size, always > 0) holds the absorbed queries
 * (bf16), the weighted latents (fp32) and the attention kernel's split partials. Three
 * launches: fold the queries, attend over the latent (the matrix-core decode kernel with
 * one KV head that serves as both K and V), then merge the partials and project each
 * row up through its group's W_UV.
 *
 * Errors: INVALID_ARGUMENT for NULL or misaligned pointers, non-positive sizes,
 * H % G != 0, non-finite scale, a bad opts struct or paged geometry; UNSUPPORTED for
 * a dtype other than bf16, d_h not in {64,128}, d_c != 512, a head map or mask, the
 * vector-ALU policy, H * q_len > 1024 or sizes whose tile counts overflow int32;
 * WORKSPACE when the workspace is NULL, too small or not 256-byte aligned; HIP when a
 * launch fails.
 */
int gqla_absorb_decode(const void* q, const void* latent_cache, const void* w_uk, const void* w_uv,
                       const int32_t* seq_lens, const int32_t* block_table, void* out,
                       int B, int H, int G, int d_h, int d_c, int q_len, float scale,
                       void* stream, const gqa_decode_opts* opts);

/*
 * gqla_absorb_decode_append -- the same absorbed decode step, fused with writing the
 * q_len new tokens' latents into the latent cache (asynchronous on `stream`). Every
 * cached token keeps one joint latent vector (the GQLA abstract), so a decode step adds
 * one latent row per new token, and then attends over the whole cache.
 *
 *   c_new        bf16 [B, q_len, d_c]: the new tokens' latents, row t of sequence b
 *                being cache position seq_lens[b] - q_len + t.
 *   latent_cache written at those positions (contiguous: [b, pos]; paged: page
 *                block_table[b][pos / P], slot pos % P, which the caller has allocated),
 *                read everywhere else; no other cache byte is written.
 *   Everything else is as for gqla_absorb_decode, whose result this equals when called
 *   on the cache after the append.
 *
 * The new rows are read straight from c_new by the latent attention kernel, which also
 * copies them into the cache from LDS: the launches are those of gqla_absorb_decode.
 * c_new must be 16-byte aligned and must not alias the cache or out. Errors are those
 * of gqla_absorb_decode plus INVALID_ARGUMENT for a NULL or misaligned c_new.
 */
int gqla_absorb_decode_append(const void* q, const void* c_new, const void* w_uk, const void* w_uv,
                              void* latent_cache, const int32_t* seq_lens, const int32_t* block_table,
                              void* out, int B, int H, int G, int d_h, int d_c, int q_len, float scale,
                              void* stream, const gqa_decode_opts* opts);

/* The plan of the latent attention kernel gqla_absorb_decode would launch (rows =
 * H * q_len: every query head reads the one latent), with workspace_bytes covering the
 * whole call. Set opts->page_size > 0 for a paged latent. */
int gqla_absorb_plan(int B, int H, int G, int d_h, int d_c, int q_len,
                     const gqa_decode_opts* opts, gqa_plan* plan);

/* Workspace bytes gqla_absorb_decode needs for these sizes. */
int gqla_absorb_workspace_size(int B, int H, int G, int d_h, int d_c, int q_len,
                               const gqa_decode_opts* opts, size_t* bytes);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif
#endif /* GQLA_ABSORB_H */
