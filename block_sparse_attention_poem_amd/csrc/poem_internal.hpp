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
  int32_t n_sink, n_local;
  int32_t max_vis;
  int32_t mode;              // kSelectOutputRelative, kSelectMass or kSelectPractical
  float prac_w, prac_rho;    // practical POEM: deviation weight, preselected mass fraction
  // column layout of the per-(KV head, tile) records. Per-head lists: column
  // f = hg * S + j (row j of head g G + hg), cols_rec = G S, the tiles of a sweep
  // workgroup's group laid end to end over its waves' 32-column tiles. Group-shared
  // lists (group_mode): column j is row j of head g G + j mod G, cols_rec = S and a
  // wave holds tiles_per_wave = 32 / S tiles.
  int32_t group_mode;
  int32_t cols_rec;
  int32_t tiles_per_wave;
  int32_t tile_group;                  // tiles per sweep workgroup (set at launch)
  int32_t sweep_items;                 // tile groups (set at launch)
  int32_t p1_chunk_blocks, p1_chunks;  // pass 1 grid: blocks per chunk, chunks per tile group
  int32_t p2_chunk_blocks, p2_chunks;  // pass 2 grid (set at launch)
  float scale_log2;
  float tau[kMaxHeadsQ];     // per query head, passed by value
  // workspace regions
  float* row_stats;          // [hkv][total_tiles][cols_rec][2 D + 4]: M2, l, L_rest / l, pad, o, R / l
  float* p1_part;            // pass 1 in chunks: [hkv][total_tiles][cols_rec][p1_chunks - 1][D + 4]
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

// Selector sweeps, host side. A sweep workgroup walks the visible blocks of a tile
// group (TG consecutive tiles of one sequence and KV head): eight waves for bf16 inputs,
// four for fp32, of 32 columns each. Per-head lists: the group's cols = G S columns per
// tile, laid end to end over the waves (a wave's 32 columns may span two tiles), so
// TG = floor(32 waves / cols) tiles and at most cols - 1 columns of the workgroup are
// idle. Group-shared lists: each wave holds tiles_per_wave tiles of S columns.
inline int sel_tile_group(bool bf16, int cols, bool group_mode, int tiles_per_wave) {
  const int waves = bf16 ? 8 : 4;
  if (group_mode) return waves * tiles_per_wave;
  return 32 * waves / cols > 1 ? 32 * waves / cols : 1;
}

// A long group's blocks can be split into chunks of whole blocks, one workgroup each,
// so that few long groups do not leave most CUs idle behind the longest: the largest
// power-of-two chunk of kSweepMaxChunk .. kSweepMinChunk blocks that gives at least
// `target` non-empty workgroups, then doubled while a group would need more than
// max_chunks chunks.
constexpr int kSweepMaxChunk = 1024;
constexpr int kSweepMinChunk = 1;
constexpr int64_t kPass1Workgroups = 1024;
constexpr int64_t kPass2Workgroups = 1024;
struct SweepChunks {
  int blocks, chunks;
};
inline SweepChunks sweep_chunks(const SeqTable& st, int hkv, int TG, int max_chunks, int64_t target) {
  int max_nblk = 1;
  for (int s = 0; s < st.num_seqs; ++s)
    if (st.n_tiles[s] > 0 && st.diag0[s] + st.n_tiles[s] > max_nblk) max_nblk = st.diag0[s] + st.n_tiles[s];
  auto nonempty = [&](int C) {
    int64_t n = 0;
    for (int s = 0; s < st.num_seqs; ++s)
      for (int t0 = 0; t0 < st.n_tiles[s]; t0 += TG) {
        const int t1 = t0 + TG < st.n_tiles[s] ? t0 + TG : st.n_tiles[s];
        n += (st.diag0[s] + t1 + C - 1) / C;
      }
    return n * hkv;
  };
  int C = kSweepMaxChunk;
  while (C > kSweepMinChunk && nonempty(C) < target) C >>= 1;
  while ((max_nblk + C - 1) / C > max_chunks) C <<= 1;
  return {C, (max_nblk + C - 1) / C};
}
constexpr int kPass1MaxChunks = 8;  // bounds pass 1's partial records (workspace)

}  // namespace poem
