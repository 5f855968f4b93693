// libpoem C ABI: argument validation, geometry, workspace layout and launches.
// Every check runs on the host before anything is enqueued; nothing here allocates
// device memory, copies host data to the device or synchronises the host.
#include <algorithm>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "poem.h"
#include "poem_internal.hpp"

namespace {

thread_local std::string g_error;

poem_status fail(poem_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

poem_status ok() {
  g_error.clear();
  return POEM_OK;
}

struct Geometry {
  poem::SeqTable st;
  int64_t total_q = 0, total_k = 0;
  int64_t num_tiles = 0;
  int64_t vis_per_head = 0;
  int64_t max_vis = 0;
  int64_t capacity = 0;
  float scale = 0.f;
};

poem_status build_geometry(const poem_problem* p, Geometry& g) {
  if (p == nullptr) return fail(POEM_ERR_INVALID_ARG, "problem is NULL");
  if (p->num_seqs < 1) return fail(POEM_ERR_INVALID_ARG, "num_seqs must be >= 1 (got %d)", p->num_seqs);
  if (p->num_seqs > POEM_MAX_SEQS)
    return fail(POEM_ERR_UNSUPPORTED, "num_seqs %d exceeds POEM_MAX_SEQS (%d)", p->num_seqs, POEM_MAX_SEQS);
  if (p->seqlens_q_host == nullptr || p->seqlens_k_host == nullptr)
    return fail(POEM_ERR_INVALID_ARG, "seqlens_q_host / seqlens_k_host is NULL");
  if (p->num_heads_q < 1 || p->num_heads_kv < 1)
    return fail(POEM_ERR_INVALID_ARG, "num_heads_q and num_heads_kv must be >= 1 (got %d, %d)", p->num_heads_q,
                p->num_heads_kv);
  if (p->num_heads_q % p->num_heads_kv != 0)
    return fail(POEM_ERR_INVALID_ARG, "num_heads_q (%d) is not a multiple of num_heads_kv (%d)", p->num_heads_q,
                p->num_heads_kv);
  if (p->head_dim <= 0) return fail(POEM_ERR_INVALID_ARG, "head_dim must be positive (got %d)", p->head_dim);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(POEM_ERR_UNSUPPORTED, "head_dim %d is not built (64 or 128)", p->head_dim);
  if (p->block_size <= 0) return fail(POEM_ERR_INVALID_ARG, "block_size must be positive (got %d)", p->block_size);
  if (p->block_size != 64 && p->block_size != 128)
    return fail(POEM_ERR_UNSUPPORTED, "block_size %d is not built (64 or 128)", p->block_size);
  if (!isfinite(p->softmax_scale)) return fail(POEM_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (p->in_dtype != POEM_BF16 && p->in_dtype != POEM_FP32)
    return fail(POEM_ERR_INVALID_ARG, "in_dtype %d is not a poem_dtype", p->in_dtype);

  const int B = p->block_size;
  memset(&g.st, 0, sizeof g.st);
  g.st.num_seqs = p->num_seqs;
  g.st.block = B;
  int64_t qs = 0, ks = 0, tiles = 0, vis = 0, maxv = 0;
  for (int s = 0; s < p->num_seqs; ++s) {
    const int64_t nq = p->seqlens_q_host[s], nk = p->seqlens_k_host[s];
    if (nq < 0 || nk < 0) return fail(POEM_ERR_INVALID_ARG, "sequence %d: negative length (N_q=%lld, N_k=%lld)", s,
                                      (long long)nq, (long long)nk);
    if (nk < nq)
      return fail(POEM_ERR_INVALID_ARG, "sequence %d: N_k (%lld) < N_q (%lld)", s, (long long)nk, (long long)nq);
    if ((nk - nq) % B != 0)
      return fail(POEM_ERR_INVALID_ARG, "sequence %d: N_k - N_q (%lld) is not a multiple of block_size %d", s,
                  (long long)(nk - nq), B);
    const int64_t nt = (nq + B - 1) / B;
    const int64_t d0 = (nk - nq) / B;
    g.st.q_start[s] = (int32_t)qs;
    g.st.k_start[s] = (int32_t)ks;
    g.st.n_q[s] = (int32_t)nq;
    g.st.n_k[s] = (int32_t)nk;
    g.st.n_tiles[s] = (int32_t)nt;
    g.st.tile_start[s] = (int32_t)tiles;
    g.st.diag0[s] = (int32_t)d0;
    g.st.vis_start[s] = vis;
    vis += nt * (d0 + 1) + nt * (nt - 1) / 2;
    if (nt > 0) maxv = maxv > d0 + nt ? maxv : d0 + nt;
    qs += nq;
    ks += nk;
    tiles += nt;
    if (qs > INT32_MAX || ks > INT32_MAX) return fail(POEM_ERR_UNSUPPORTED, "total tokens exceed 2^31 - 1");
  }
  g.st.total_tiles = (int32_t)tiles;
  g.st.vis_per_head = vis;
  g.total_q = qs;
  g.total_k = ks;
  g.num_tiles = tiles;
  g.vis_per_head = vis;
  g.max_vis = maxv;
  g.capacity = vis * p->num_heads_q;
  if (g.capacity > INT32_MAX)
    return fail(POEM_ERR_UNSUPPORTED, "CSR capacity %lld exceeds int32 offsets", (long long)g.capacity);
  if (tiles * (int64_t)p->num_heads_q > INT32_MAX) return fail(POEM_ERR_UNSUPPORTED, "too many (head, tile) rows");
  g.scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf((float)p->head_dim);
  return POEM_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SelLayout {
  size_t row_stats = 0, p1_part = 0, blk_stats = 0, counts = 0, slots = 0, v16 = 0, vscale = 0, total = 0;
  poem::SweepChunks p1 = {0, 1};  // pass 1 chunks
};

// key blocks over all sequences (ceil(N_k / B) each)
int64_t total_key_blocks(const Geometry& g) {
  int64_t n = 0;
  for (int s = 0; s < g.st.num_seqs; ++s) n += g.st.diag0[s] + g.st.n_tiles[s];
  return n;
}

// Record columns per (KV head, tile): per-head lists hold the G heads' S rows; a
// group-shared list has S columns.
int record_columns(const poem_problem* p, int S, bool group_mode) {
  const int G = p->num_heads_q / p->num_heads_kv;
  return group_mode ? S : G * S;
}

SelLayout sel_layout(const poem_problem* p, const Geometry& g, int S, bool group_mode) {
  SelLayout L;
  const int cols = record_columns(p, S, group_mode);
  size_t off = 0;
  L.row_stats = off;
  off += align256(sizeof(float) * (size_t)p->num_heads_kv * g.num_tiles * cols * (2 * p->head_dim + 4));
  {  // pass 1 in chunks: partial records of the chunks after the first
    const int TG = poem::sel_tile_group(p->in_dtype == POEM_BF16, cols, group_mode, group_mode ? 32 / S : 1);
    L.p1 = poem::sweep_chunks(g.st, p->num_heads_kv, TG, poem::kPass1MaxChunks, poem::kPass1Workgroups);
    L.p1_part = off;
    off += align256(sizeof(float) * (size_t)p->num_heads_kv * g.num_tiles * cols * (L.p1.chunks - 1) *
                    (p->head_dim + 4));
  }
  L.blk_stats = off;
  off += align256(sizeof(float) * (size_t)p->num_heads_kv * g.vis_per_head * cols * 2);
  L.counts = off;
  off += align256(sizeof(int32_t) * (size_t)p->num_heads_q * g.num_tiles);
  L.slots = off;
  off += align256(sizeof(int32_t) * (size_t)p->num_heads_q * g.vis_per_head);
  if (p->in_dtype == POEM_BF16) {  // fp16 V and its block scales for pass 2
    L.v16 = off;
    off += align256(sizeof(uint16_t) * (size_t)g.total_k * p->num_heads_kv * p->head_dim);
    L.vscale = off;
    off += align256(sizeof(float) * (size_t)p->num_heads_kv * total_key_blocks(g));
  }
  L.total = off;
  return L;
}

poem_status check_rows(const poem_problem* p, int32_t S, bool group_mode) {
  if (S < 1) return fail(POEM_ERR_INVALID_ARG, "rows_per_tile must be >= 1 (got %d)", S);
  if (S > POEM_MAX_ROWS_PER_TILE)
    return fail(POEM_ERR_UNSUPPORTED, "rows_per_tile %d exceeds POEM_MAX_ROWS_PER_TILE (%d)", S, POEM_MAX_ROWS_PER_TILE);
  const int G = p->num_heads_q / p->num_heads_kv;
  if (!group_mode && (int64_t)G * S > 128)
    return fail(POEM_ERR_UNSUPPORTED, "group size x rows_per_tile = %d exceeds 128 selector columns", G * S);
  return POEM_OK;
}

poem_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(POEM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int64_t poem_num_tiles(const poem_problem* problem) {
  Geometry g;
  poem_status s = build_geometry(problem, g);
  if (s != POEM_OK) return s;
  ok();
  return g.num_tiles;
}

int64_t poem_csr_capacity(const poem_problem* problem) {
  Geometry g;
  poem_status s = build_geometry(problem, g);
  if (s != POEM_OK) return s;
  ok();
  return g.capacity;
}

int64_t poem_max_visible_blocks(const poem_problem* problem) {
  Geometry g;
  poem_status s = build_geometry(problem, g);
  if (s != POEM_OK) return s;
  ok();
  return g.max_vis;
}

int64_t poem_select_workspace_bytes(const poem_problem* problem, int32_t rows_per_tile) {
  Geometry g;
  poem_status s = build_geometry(problem, g);
  if (s != POEM_OK) return s;
  s = check_rows(problem, rows_per_tile, true);
  if (s != POEM_OK) return s;
  ok();
  // enough for every selector entry point the problem allows
  const int G = problem->num_heads_q / problem->num_heads_kv;
  size_t bytes = sel_layout(problem, g, rows_per_tile, true).total;
  if ((int64_t)G * rows_per_tile <= 128) bytes = std::max(bytes, sel_layout(problem, g, rows_per_tile, false).total);
  return (int64_t)bytes;
}

static poem_status select_impl(int mode, bool group_mode, float prac_w, float prac_rho, const poem_problem* problem, const void* q, const void* k, const void* v,
                               const float* tau_host, int32_t n_sink_blocks, int32_t n_local_blocks,
                               int32_t rows_per_tile, int32_t* row_ptr, int32_t* block_idx,
                               int64_t block_idx_capacity, float* tile_scores, float* tile_mass, float* row_bound,
                               void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  poem_status s = build_geometry(problem, g);
  if (s != POEM_OK) return s;
  s = check_rows(problem, rows_per_tile, group_mode);
  if (s != POEM_OK) return s;
  if (q == nullptr || k == nullptr || v == nullptr) return fail(POEM_ERR_INVALID_ARG, "q, k or v is NULL");
  if (row_ptr == nullptr || block_idx == nullptr) return fail(POEM_ERR_INVALID_ARG, "row_ptr or block_idx is NULL");
  if (tau_host == nullptr) return fail(POEM_ERR_INVALID_ARG, "tau_host is NULL");
  if (problem->num_heads_q > poem::kMaxHeadsQ)
    return fail(POEM_ERR_UNSUPPORTED, "num_heads_q %d exceeds %d for the selector", problem->num_heads_q,
                poem::kMaxHeadsQ);
  for (int h = 0; h < problem->num_heads_q; ++h)
    if (!(tau_host[h] >= 0.f) || !isfinite(tau_host[h]))
      return fail(POEM_ERR_INVALID_ARG, "tau_host[%d] must be finite and >= 0", h);
  if (n_sink_blocks < 0) return fail(POEM_ERR_INVALID_ARG, "n_sink_blocks must be >= 0 (got %d)", n_sink_blocks);
  if (n_local_blocks < 1)
    return fail(POEM_ERR_INVALID_ARG, "n_local_blocks must be >= 1 (it counts the diagonal block; got %d)",
                n_local_blocks);
  if (g.max_vis > POEM_MAX_VISIBLE_BLOCKS)
    return fail(POEM_ERR_UNSUPPORTED, "a tile sees %lld blocks, above POEM_MAX_VISIBLE_BLOCKS (%d)",
                (long long)g.max_vis, POEM_MAX_VISIBLE_BLOCKS);
  if (block_idx_capacity < g.capacity)
    return fail(POEM_ERR_CAPACITY, "block_idx capacity %lld < required %lld", (long long)block_idx_capacity,
                (long long)g.capacity);
  const int cols = record_columns(problem, rows_per_tile, group_mode);
  const SelLayout L = sel_layout(problem, g, rows_per_tile, group_mode);
  if (workspace == nullptr) return fail(POEM_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < L.total)
    return fail(POEM_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
  if (((uintptr_t)workspace & 255) != 0) return fail(POEM_ERR_WORKSPACE, "workspace is not 256-byte aligned");

  poem::SelectParams sp;
  memset(&sp, 0, sizeof sp);
  sp.q = q;
  sp.k = k;
  sp.v = v;
  sp.hq = problem->num_heads_q;
  sp.hkv = problem->num_heads_kv;
  sp.group = problem->num_heads_q / problem->num_heads_kv;
  sp.S = rows_per_tile;
  sp.group_mode = group_mode ? 1 : 0;
  sp.cols_rec = cols;
  sp.tiles_per_wave = group_mode ? 32 / rows_per_tile : 1;
  sp.n_sink = n_sink_blocks;
  sp.n_local = n_local_blocks;
  sp.max_vis = (int32_t)g.max_vis;
  sp.mode = mode;
  sp.prac_w = prac_w;
  sp.prac_rho = prac_rho;
  sp.scale_log2 = g.scale * poem::kLog2e;
  for (int h = 0; h < problem->num_heads_q; ++h) sp.tau[h] = tau_host[h];
  char* ws = static_cast<char*>(workspace);
  sp.row_stats = reinterpret_cast<float*>(ws + L.row_stats);
  sp.p1_part = reinterpret_cast<float*>(ws + L.p1_part);
  sp.p1_chunk_blocks = L.p1.blocks;
  sp.p1_chunks = L.p1.chunks;
  sp.blk_stats = reinterpret_cast<float*>(ws + L.blk_stats);
  sp.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  sp.slots = reinterpret_cast<int32_t*>(ws + L.slots);
  if (problem->in_dtype == POEM_BF16) {
    sp.v16 = reinterpret_cast<uint16_t*>(ws + L.v16);
    sp.vscale = reinterpret_cast<float*>(ws + L.vscale);
  }
  sp.total_kb = (int32_t)total_key_blocks(g);
  sp.row_ptr = row_ptr;
  sp.block_idx = block_idx;
  sp.tile_scores = tile_scores;
  sp.tile_mass = tile_mass;
  sp.row_bound = row_bound;
  sp.seqs = g.st;
  return hip_status(poem::launch_select(sp, problem->in_dtype, problem->head_dim, problem->block_size,
                                        static_cast<hipStream_t>(stream)),
                    "poem_select launch");
}

poem_status poem_select(const poem_problem* problem, const void* q, const void* k, const void* v,
                        const float* tau_host, int32_t n_sink_blocks, int32_t n_local_blocks, int32_t rows_per_tile,
                        int32_t* row_ptr, int32_t* block_idx, int64_t block_idx_capacity, float* tile_scores,
                        float* tile_mass, float* row_bound, void* workspace, size_t workspace_bytes, void* stream) {
  return select_impl(poem::kSelectOutputRelative, false, 0.f, 1.f, problem, q, k, v, tau_host, n_sink_blocks, n_local_blocks,
                     rows_per_tile, row_ptr, block_idx, block_idx_capacity, tile_scores, tile_mass, row_bound,
                     workspace, workspace_bytes, stream);
}

poem_status poem_select_group(const poem_problem* problem, const void* q, const void* k, const void* v,
                              const float* tau_host, int32_t n_sink_blocks, int32_t n_local_blocks,
                              int32_t rows_per_tile, int32_t* row_ptr, int32_t* block_idx,
                              int64_t block_idx_capacity, float* tile_scores, float* tile_mass, float* row_bound,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return select_impl(poem::kSelectOutputRelative, true, 0.f, 1.f, problem, q, k, v, tau_host, n_sink_blocks, n_local_blocks,
                     rows_per_tile, row_ptr, block_idx, block_idx_capacity, tile_scores, tile_mass, row_bound,
                     workspace, workspace_bytes, stream);
}

poem_status poem_select_practical(const poem_problem* problem, const void* q, const void* k, const void* v,
                                  const float* eps_host, int32_t n_sink_blocks, int32_t n_local_blocks,
                                  int32_t rows_per_tile, float weight, float presel_fraction, int32_t* row_ptr,
                                  int32_t* block_idx, int64_t block_idx_capacity, float* tile_scores,
                                  float* tile_mass, float* row_bound, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (!isfinite(weight)) return fail(POEM_ERR_INVALID_ARG, "weight must be finite");
  if (!(presel_fraction > 0.f && presel_fraction <= 1.f))
    return fail(POEM_ERR_INVALID_ARG, "presel_fraction must be in (0, 1] (got %g)", (double)presel_fraction);
  return select_impl(poem::kSelectPractical, false, weight, presel_fraction, problem, q, k, v, eps_host,
                     n_sink_blocks, n_local_blocks, rows_per_tile, row_ptr, block_idx, block_idx_capacity,
                     tile_scores, tile_mass, row_bound, workspace, workspace_bytes, stream);
}

poem_status poem_select_mass(const poem_problem* problem, const void* q, const void* k, const void* v,
                             const float* eps_host, int32_t n_sink_blocks, int32_t n_local_blocks,
                             int32_t rows_per_tile, int32_t* row_ptr, int32_t* block_idx,
                             int64_t block_idx_capacity, float* tile_scores, float* tile_mass, float* row_bound,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return select_impl(poem::kSelectMass, false, 0.f, 1.f, problem, q, k, v, eps_host, n_sink_blocks, n_local_blocks, rows_per_tile,
                     row_ptr, block_idx, block_idx_capacity, tile_scores, tile_mass, row_bound, workspace,
                     workspace_bytes, stream);
}

static size_t sparse_ws_bytes(const poem_problem* p, const Geometry& g) {
  return 256 + align256(sizeof(int32_t) * (size_t)p->num_heads_q * g.num_tiles);
}

static poem_status attention(const poem_problem* problem, const void* q, const void* k, const void* v,
                             const int32_t* row_ptr, const int32_t* block_idx, void* out, int32_t out_dtype,
                             float* lse, void* workspace, size_t workspace_bytes, void* stream, bool sparse,
                             bool shared) {
  Geometry g;
  poem_status s = build_geometry(problem, g);
  if (s != POEM_OK) return s;
  if (workspace != nullptr) {
    const size_t need = sparse ? sparse_ws_bytes(problem, g) : (size_t)POEM_DENSE_WORKSPACE_BYTES;
    if (workspace_bytes < need)
      return fail(POEM_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (((uintptr_t)workspace & 255) != 0) return fail(POEM_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  if (q == nullptr || k == nullptr || v == nullptr) return fail(POEM_ERR_INVALID_ARG, "q, k or v is NULL");
  if (out == nullptr) return fail(POEM_ERR_INVALID_ARG, "out is NULL");
  if (sparse && (row_ptr == nullptr || block_idx == nullptr))
    return fail(POEM_ERR_INVALID_ARG, "row_ptr or block_idx is NULL");
  if (out_dtype != POEM_BF16 && out_dtype != POEM_FP32)
    return fail(POEM_ERR_INVALID_ARG, "out_dtype %d is not a poem_dtype", out_dtype);
  poem::AttnParams ap;
  memset(&ap, 0, sizeof ap);
  ap.q = q;
  ap.k = k;
  ap.v = v;
  ap.row_ptr = row_ptr;
  ap.block_idx = block_idx;
  ap.out = out;
  ap.lse = lse;
  ap.hq = problem->num_heads_q;
  ap.hkv = problem->num_heads_kv;
  ap.group = problem->num_heads_q / problem->num_heads_kv;
  ap.out_f32 = out_dtype == POEM_FP32 ? 1 : 0;
  ap.total_q = (int32_t)g.total_q;
  ap.scale_log2 = g.scale * poem::kLog2e;
  ap.num_rows = (int32_t)(problem->num_heads_q * g.num_tiles);
  ap.shared = shared ? 1 : 0;
  if (workspace != nullptr) {
    ap.queue = static_cast<int32_t*>(workspace);
    if (sparse) ap.order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + 256);
  }
  ap.seqs = g.st;
  return hip_status(poem::launch_attention(ap, problem->in_dtype, problem->head_dim, problem->block_size, sparse,
                                           static_cast<hipStream_t>(stream)),
                    !sparse ? "poem_dense_prefill launch"
                            : (shared ? "poem_sparse_prefill_group launch" : "poem_sparse_prefill launch"));
}

int64_t poem_sparse_workspace_bytes(const poem_problem* problem) {
  Geometry g;
  poem_status s = build_geometry(problem, g);
  if (s != POEM_OK) return s;
  ok();
  return (int64_t)sparse_ws_bytes(problem, g);
}

poem_status poem_sparse_prefill(const poem_problem* problem, const void* q, const void* k, const void* v,
                                const int32_t* row_ptr, const int32_t* block_idx, void* out, int32_t out_dtype,
                                float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return attention(problem, q, k, v, row_ptr, block_idx, out, out_dtype, lse, workspace, workspace_bytes, stream,
                   true, false);
}

poem_status poem_sparse_prefill_group(const poem_problem* problem, const void* q, const void* k, const void* v,
                                      const int32_t* row_ptr, const int32_t* block_idx, void* out,
                                      int32_t out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return attention(problem, q, k, v, row_ptr, block_idx, out, out_dtype, lse, workspace, workspace_bytes, stream,
                   true, true);
}

poem_status poem_sparse_prefill_noalloc(const poem_problem* problem, const void* q, const void* k, const void* v,
                                        const int32_t* row_ptr, const int32_t* block_idx, void* out,
                                        int32_t out_dtype, float* lse, void* stream) {
  Geometry g;
  poem_status s = build_geometry(problem, g);
  if (s != POEM_OK) return s;
  const int64_t rows = (int64_t)problem->num_heads_q * g.num_tiles;
  if (rows > POEM_NOALLOC_MAX_ROWS)
    return fail(POEM_ERR_UNSUPPORTED, "num_heads_q * num_tiles = %lld exceeds POEM_NOALLOC_MAX_ROWS (%d)",
                (long long)rows, POEM_NOALLOC_MAX_ROWS);
  if (q == nullptr || k == nullptr || v == nullptr) return fail(POEM_ERR_INVALID_ARG, "q, k or v is NULL");
  if (out == nullptr) return fail(POEM_ERR_INVALID_ARG, "out is NULL");
  if (row_ptr == nullptr || block_idx == nullptr) return fail(POEM_ERR_INVALID_ARG, "row_ptr or block_idx is NULL");
  if (out_dtype != POEM_BF16 && out_dtype != POEM_FP32)
    return fail(POEM_ERR_INVALID_ARG, "out_dtype %d is not a poem_dtype", out_dtype);
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  s = hip_status(poem::noalloc_scratch(&scratch, &scratch_bytes), "poem_sparse_prefill_noalloc scratch lookup");
  if (s != POEM_OK) return s;
  if (sparse_ws_bytes(problem, g) > scratch_bytes)  // implied by the row limit above
    return fail(POEM_ERR_UNSUPPORTED, "schedule needs %zu bytes, the scratch holds %zu", sparse_ws_bytes(problem, g),
                scratch_bytes);
  return attention(problem, q, k, v, row_ptr, block_idx, out, out_dtype, lse, scratch, scratch_bytes, stream, true,
                   false);
}

poem_status poem_dense_prefill(const poem_problem* problem, const void* q, const void* k, const void* v, void* out,
                               int32_t out_dtype, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return attention(problem, q, k, v, nullptr, nullptr, out, out_dtype, lse, workspace, workspace_bytes, stream, false,
                   false);
}

const char* poem_last_error(void) { return g_error.c_str(); }

const char* poem_version(void) { return "libpoem 0.1.0 (gfx950)"; }

}  // extern "C"
