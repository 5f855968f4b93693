// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "poem_device.hpp"

namespace poem {

constexpr int kMaxHeadsQ = 128;  // query heads the selector accepts (tau travels in kernel arguments)

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* row_ptr;    // sparse only
  const int32_t* block_idx;  // sparse only
  void* out;
  float* lse;                // nullable
  int32_t hq, hkv, group;
  int32_t out_f32;
  int32_t total_q;
  float scale_log2;          // softmax scale * log2(e)
  // sparse persistent schedule (queue == nullptr: one workgroup per row)
  int32_t* queue;            // queue head, reset by the schedule kernel
  int32_t* order;            // [num_rows] rows by retained count, descending
  int32_t num_rows;          // hq * total_tiles
  int32_t shared;            // sparse: every head reads the list of its GQA group's first head
  SeqTable seqs;
};

// The device scratch of poem_sparse_prefill_noalloc on the current device (looked up
// once per device): 256 bytes of queue head, then POEM_NOALLOC_MAX_ROWS int32 of row order.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// in_dtype: 0 bf16, 1 fp32.
hipError_t launch_attention(const AttnParams& p, int in_dtype, int head_dim, int block, bool sparse,
                            hipStream_t stream);

// Selector modes: the output-relative score (ranking by mean I, cut on the triangle
// bound) and the mass-only baseline (ranking by mean m, cut on omitted mass).
constexpr int kSelectOutputRelative = 0;
constexpr int kSelectMass = 1;
constexpr int kSelectPractical = 2;  // practical POEM: mass preselection, log rerank, pooled mass

struct SelectParams {
  const void* q;
  const void* k;
  const void* v;
  int32_t hq, hkv, group;
  int32_t S;                 // sampled rows per tile
  int32_t col_tiles;         // 32-column tiles per (KV head, tile)
  int32_t n_sink, n_local;
  int32_t max_vis;
  int32_t mode;              // kSelectOutputRelative, kSelectMass or kSelectPractical
  float prac_w, prac_rho;    // practical POEM: deviation weight, preselected mass fraction
  // column layout of the per-(KV head, tile) records. Per-head lists: column
  // f = hg * S + j (row j of head g G + hg), cols_rec = 32 * col_tiles, one tile per
  // wave. Group-shared lists (group_mode): column j is row j of head g G + j mod G,
  // cols_rec = S and a wave holds tiles_per_wave = 32 / S tiles.
  int32_t group_mode;
  int32_t cols_rec;
  int32_t tiles_per_wave;
  int32_t p2_chunk_blocks, p2_chunks;  // pass 2 grid: blocks per chunk, chunks per tile group (set at launch)
  float scale_log2;
  float tau[kMaxHeadsQ];     // per query head, passed by value
  // workspace regions
  float* row_stats;          // [hkv][total_tiles][cols_rec][2 D + 4]: M2, l, L_rest / l, pad, o, R / l
  float* blk_stats;          // per (KV head, gtile, visible block): I[cols_rec] then m[cols_rec]
  int32_t* counts;           // [hq * total_tiles]
  int32_t* slots;            // [hq * vis_per_head] retained ids at slot offsets
  // bf16 inputs: V for pass 2 as fp16, each (key block, KV head) scaled by a power of
  // two vscale so that its largest |v| lies in [2^14, 2^15); same layout as V
  uint16_t* v16;             // [total_k][hkv][D]
  float* vscale;             // [hkv][total_kb]
  int32_t total_kb;          // key blocks over all sequences
  // outputs
  int32_t* row_ptr;
  int32_t* block_idx;
  float* tile_scores;        // nullable
  float* tile_mass;          // nullable
  float* row_bound;          // nullable
  SeqTable seqs;
};

hipError_t launch_select(const SelectParams& p, int in_dtype, int head_dim, int block, hipStream_t stream);

}  // namespace poem
