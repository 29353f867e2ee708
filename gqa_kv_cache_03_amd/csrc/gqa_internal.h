// Internal declarations shared by the host planner and the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Everything a decode kernel needs; passed by value as the kernel argument.
struct DecodeParams {
  const void* q;           // [B, q_len, H, D]
  const void* k;           // contiguous [B, G, cap, D] or paged [pages, G, P, D]
  const void* v;
  const void* k_new;       // append: new tokens' K [B, q_len, G, D] (nullptr: none)
  const void* v_new;       // append: new tokens' V
  const int32_t* seq_lens; // [B]
  const int32_t* table;    // [B, max_blocks] or nullptr
  const int32_t* head_group;   // [H] KV head of each query head, or nullptr: h / hpg
  const uint8_t* head_active;  // [B, q_len, H]: 0 = (token, head) inactive (output 0), or nullptr
  void* out;               // [B, q_len, H, D]
  // split partials (normalised O, log2-domain log-sum-exp):
  //   split-K grid (VALU): ws_o [B, q_len, H, max_splits, D], ws_lse [B, q_len, H, max_splits]
  //   persistent (MFMA):   ws_o [nwg, 2, R, D], ws_lse [nwg, 2, R], ws_prefix [B + 1]
  float* ws_o;
  float* ws_lse;
  int32_t* ws_prefix;      // tiles before sequence b's segments (persistent schedule)
  int B, H, G, q_len;
  int hpg;                 // H / G
  int R;                   // hpg * q_len packed rows per group
  int capacity;            // tokens addressable per sequence
  int page_shift;          // log2(page size) when paged
  int max_blocks;          // block table row stride
  int num_pages;
  int chunk;               // tokens per split (multiple of the kernel tile)
  int max_splits;
  int causal;
  int row_block;           // rows per workgroup along grid.y (VALU policy)
  int n_row_blocks;
  int nwg;                 // persistent workgroups (MFMA policy)
  float qk_scale_log2;     // scale * log2(e): logits in base-2 units
  int out_f32;             // write `out` as float32 instead of the input dtype (latent path)
  // GQLA absorbed execution (D = 512 merge only; w_uv null otherwise): `out` holds the
  // weighted latents u, and the merge also writes proj_out = W_UV[group] u, bf16
  // [B, q_len, H, proj_dh], with H / proj_groups query heads per group
  const void* w_uv;        // [proj_groups, proj_dh, 512] bf16
  void* proj_out;
  int proj_dh;
  int proj_groups;
};

// Row r of the packed group tile is query token t = r / hpg of head g*hpg + r % hpg.

// Launch `kernel` with the decode parameter block on `stream`. With a start or stop
// event the launch stamps them with the kernel's own begin and end times
// (hipExtLaunchKernel); without, it is a plain launch (also inside graph capture).
template <typename K>
inline void launch_timed(K kernel, dim3 grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                         const DecodeParams& p) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, start, stop, 0, p);
  else
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, p);
}

// Launchers (defined next to their kernels). Return hipSuccess or the launch error.
// `start` / `stop` (may be null) are caller-created events that the launch itself
// stamps with the kernel's own begin and end times (hipExtLaunchKernel), so the
// elapsed time between them is that kernel's execution, free of queue gaps.
hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int d_h, bool paged,
                              dim3 grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int d_h, bool paged,
                              dim3 grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
hipError_t launch_merge(const DecodeParams& p, int dtype, int d_h, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop);
hipError_t launch_merge_persistent(const DecodeParams& p, int d_h, hipStream_t stream, hipEvent_t start,
                                   hipEvent_t stop);
// With a head -> KV head map: NaN into the (token, head) rows of `out` that no packed
// group tile holds (oversize groups, map entries outside [0, G)); bf16 only.
hipError_t launch_fill_unmapped(const DecodeParams& p, int d_h, hipStream_t stream);
// Writes k_new / v_new into the cache rows of the new tokens (vector-ALU path).
hipError_t launch_append(const DecodeParams& p, int elem_bytes, int d_h, bool paged, hipStream_t stream);

// GQLA latent path: the query fold before the latent attention (the up-projection
// after it runs inside the merge).
struct LatentProjParams {
  const void* q;        // [rows, d_h] bf16, rows = B * q_len * H (row = (b q_len + t) H + h)
  const void* w_uk;     // [G, d_h, d_c] bf16
  void* q_lat;          // [rows, d_c] bf16: q folded through its group's W_UK
  int B, H, G, q_len, d_h, d_c;
};
hipError_t launch_latent_absorb_q(const LatentProjParams& p, hipStream_t stream);

// Device-side check of the decode calls' device-resident preconditions (check.hip).
struct CheckParams {
  const int32_t* seq_lens;  // [B]
  const int32_t* table;     // [B, max_blocks] or nullptr
  int32_t* report;          // [4]: bad lengths, bad entries, first bad sequence, first bad entry
  int B, q_len, capacity, page_size, max_blocks, num_pages;
};
hipError_t launch_check_inputs(const CheckParams& p, hipStream_t stream);

// Geometry of the MFMA kernel variants, chosen by packed row count R.
struct MfmaVariant {
  int max_rows;      // R this variant serves (multiple of 16)
  int tile;          // keys per pipeline step
  int lds_bytes;     // LDS per workgroup
  int wgs_per_cu;    // resident workgroups per CU (0 when not queried / no device)
};
MfmaVariant mfma_variant_for_rows(int R, int d_h, bool paged, bool query_device);
// Most packed rows one MFMA workgroup holds at this head width (d_h 512: the latent).
int mfma_max_rows(int d_h);
int valu_tile_tokens(int dtype, int d_h);
int valu_lds_bytes(int dtype, int d_h, int row_block);

}  // namespace gqa
