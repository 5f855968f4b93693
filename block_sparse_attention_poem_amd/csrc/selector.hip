// Output-relative block selector for gfx950 (POEM note, Section 4.1 and Equation (4)).
//
// Columns. For a KV head g and query tile t, the selector's query columns are the
// sampled rows of the G query heads that share g (BFLA Section 3.3): column
// f = hg * S + j is row r_j of head g*G + hg. The G S columns of consecutive tiles are
// laid end to end over a workgroup's waves, 32 to a wave, so one K/V fetch serves every
// head of the group and at most G S - 1 of a workgroup's columns are idle (none when
// G S divides 256: Llama-3-8B shapes, G = 4 and S = 8, put one tile on each wave).
//
// Pass 1 (sel_sweep_kernel<..., false>): per column, the dense softmax statistics
//   over all visible keys (c = scale * log2 e): the final running max M2 of c s_j,
//   l = sum_j 2^(c s_j - M2) and o = sum_j 2^(c s_j - M2) v_j / l. Block 0's sums are
//   kept apart while they are formed, and the record also holds R / l and L_rest / l,
//   with R = sum_j w_j v_j and L_rest = sum_j w_j over the keys after block 0.
// Pass 2 (sel_sweep_kernel<..., true>): per column and visible block b, with the
//   same weights w_j = 2^(c s_j - M2): L_b = sum_{j in b} w_j, U_b = sum_{j in b} w_j v_j,
//   then m_b = L_b / l and I_b = ||U_b - L_b o|| / l (= ||u_b - m_b o||; a cross-lane
//   sum of squares). For block 0 the vector is formed as (U_0 L_rest - L_0 R) / l, the
//   same quantity since l = L_0 + L_rest and l o = U_0 + R: with a sink in block 0
//   holding nearly all of a row's mass (1 - m_0 of a few 1e-4 at 128K tokens), U_0 and
//   L_0 o agree to 1 - m_0 and their difference would lose that factor of fp32's
//   precision; L_0 R and U_0 L_rest differ by L_0 L_rest (v_0 - v_rest), which does not.
// Both passes stream the visible K/V blocks through the same LDS stages as the
// attention kernel; a workgroup of eight waves (bf16) holds several tiles of one KV
// head (one CU each: two waves per SIMD), so each fetch is shared by up to 256 columns
// and the direct loads per MFMA are half those of four-wave workgroups (measured: the
// selector's two passes run 6% faster at 128K). When the tile groups are too few to
// fill the chip with long ones among them (short sequences; chunks of a few thousand
// queries against long prefixes), each group's blocks are split into chunks of whole
// blocks, one workgroup per chunk, run chunk-major so that the workgroups of one XCD
// read the same key range; pass 1's chunks leave partial sums at their own exponent
// references that sel_merge_kernel combines (see there).
//
// Precision of P V (bf16 inputs). Pass 1 takes one bf16 P for o, R, l and L_rest: the
// row's maximum key weighs exactly 1, the rounding of the other weights averages out
// over every visible key, and o is the exact mean under the rounded weights. Pass 2
// needs more: with bf16 weights (2^-9 relative rounding), a block whose mass sits on a
// few keys would carry up to 2^-9 relative error in I_b. It runs P V on fp16 instead
// (2^-11): v16_kernel first writes V as fp16, each (key block, KV head) scaled by a
// power of two s_b that puts its largest |v| in [2^14, 2^15) (exact for bf16 values,
// whose 8-bit significands fit fp16's 11, down to s_b |v| = 2^-14); the weights are
// formed as 2^14 w_j, at most 2^14, so fp16 keeps 11 bits of them down to w_j = 2^-28.
// U_b - L_b o is formed with L_b the sum of the same fp16 weights, so I_b sees each
// weight's rounding once, as a perturbation of the weight; m_b = L_b / l comes from that
// sum too (at most 2^-12 relative per weight). Only a block other than block 0 that
// holds nearly all of a row's mass would lose digits to the cancellation above.
//
// Threshold (sel_threshold_kernel): per (query head, tile), the tile score is the
// mean of I over the sampled rows; candidates (visible, not mandatory) are sorted
// by (score ascending, id descending) with an LDS bitonic sort; the cut is the
// first prefix whose per-row bound sum I / (1 - sum m), maximised over rows,
// exceeds tau (prefix sums in fp64). The kept ids are compacted in ascending order.
// CSR: an exclusive scan of the per-row counts and a scatter.
#include "poem_internal.hpp"

namespace poem {

// Sweep workgroup: eight waves for bf16; fp32 stages need more than the 256 VGPRs two
// waves per SIMD leave, so fp32 keeps four waves (one per SIMD).
template <typename T> constexpr int sel_threads() { return sizeof(T) == 2 ? 512 : 256; }
template <bool B> struct BoolTag { static constexpr bool value = B; };
constexpr int kMaxSeqBlocks = 4096;  // key blocks a tile may see (POEM_MAX_VISIBLE_BLOCKS)
// Per-column record of pass 1: M2, l, L_rest / l, pad, o[D], R / l [D], where R and
// L_rest sum w_j v_j and w_j over the keys after block 0 (output-relative selectors;
// pass 2 forms block 0's I from them, see the file header).
template <int D> constexpr int kRecordFloats = 2 * D + 4;
// fp16 P V of pass 2: weights carry 2^14 (log2 and inverse)
constexpr float kP16Log2 = 14.f;
constexpr float kP16Inv = 1.f / 16384.f;

// MASS: the mass-only selector needs neither o nor U_b, so both passes skip P V and
// stage K alone.
template <typename T, int D, int BLK, bool PASS2, bool MASS>
__global__ __launch_bounds__(sel_threads<T>()) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, 2)))
void sel_sweep_kernel(SelectParams p) {
  constexpr int kSelWaves = sel_threads<T>() / 64;
  using St = Stage<T, D, sel_threads<T>()>;
  constexpr int SUBS = BLK / kStageKeys;
  constexpr bool SPLIT = sizeof(T) == 2;
  // bf16 pass 1 of the output-relative selectors runs the pipelined sweep below; pass 2
  // (which also holds o for its per-block norms), the mass-only passes and fp32 run
  // the plain double-buffered sweep
  constexpr bool PIPE = St::ASYNC && !MASS && !PASS2;
  // bf16 pass 2 of the output-relative selectors: P V on fp16 (see the file header)
  constexpr bool F16PV = St::ASYNC && PASS2 && !MASS;
  // pass 1 of the output-relative selectors keeps block 0's sums apart from the rest
  // (see the file header)
  constexpr bool SPLIT0 = !MASS && !PASS2;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int jcol = lane & 31, g2 = lane >> 5;
  const int TPW = p.tiles_per_wave;
  const int TG = p.tile_group;  // tiles per workgroup (sel_tile_group)

  const int gk = blockIdx.x % p.hkv;
  // the tile group's visible blocks in chunks of whole blocks, one chunk per workgroup.
  // The grid runs chunk 0 of every group (longest groups first), then chunk 1, ...: the
  // workgroups resident together on an XCD (one KV head each) then read the same range
  // of key blocks, which its L2 serves once. Pass 2's chunks are independent (a block's
  // I and m need only pass 1's record); pass 1's chunks leave partial sums that
  // sel_merge_kernel combines.
  const int n_chunks = PASS2 ? p.p2_chunks : p.p1_chunks;
  const int chunk_blocks = PASS2 ? p.p2_chunk_blocks : p.p1_chunk_blocks;
  const int chunk = (int)(blockIdx.x / p.hkv) / p.sweep_items;
  const int rank = (int)(blockIdx.x / p.hkv) % p.sweep_items;
  int seq, tile0;
  rank_to_item(p.seqs, TG, rank, seq, tile0);
  if (seq < 0) return;
  const int n_q = p.seqs.n_q[seq], n_k = p.seqs.n_k[seq], n_tiles = p.seqs.n_tiles[seq];
  const int diag0 = p.seqs.diag0[seq];
  const int t_last = min(tile0 + TG - 1, n_tiles - 1);
  const int nblk_wg = diag0 + t_last + 1;
  const int blk_lo = chunk * chunk_blocks;  // this workgroup's blocks: blk_lo .. blk_hi - 1
  const int blk_hi = min(nblk_wg, blk_lo + chunk_blocks);
  if (blk_lo >= blk_hi) return;

  // this lane's column: tile t, record column col, row jr of the tile's sample taken
  // from query head gk * G + hg
  int t, col, jr, hg, tw0, tw1;
  bool in_range;
  if (p.group_mode) {
    tw0 = tile0 + wave * TPW;
    tw1 = min(tw0 + TPW - 1, n_tiles - 1);
    t = tw0 + jcol / p.S;
    jr = col = jcol % p.S;
    hg = jr % p.group;
    in_range = jcol < TPW * p.S && t < n_tiles;
  } else {
    // the group's tiles end to end: flattened column F = (t - tile0) C + col, 32 per wave
    const int C = p.cols_rec;
    const int F = 32 * wave + jcol;
    const int F_end = TG * C;  // columns of the workgroup's tiles
    t = tile0 + F / C;
    col = F % C;
    hg = col / p.S;
    jr = col % p.S;
    in_range = F < F_end && t < n_tiles;
    tw0 = tile0 + (32 * wave) / C;
    tw1 = min(tile0 + min(32 * wave + 31, F_end - 1) / C, n_tiles - 1);
  }
  const bool wave_on = tw0 < n_tiles && (p.group_mode || 32 * wave < TG * p.cols_rec);
  const int diag = diag0 + t;
  const int n_rows_t = in_range ? min(BLK, n_q - t * BLK) : 1;
  const int s_t = min(p.S, n_rows_t);
  const bool col_on = in_range && jr < s_t;
  const int h = gk * p.group + (col_on ? hg : 0);
  const int r_local = col_on ? ((jr + 1) * n_rows_t + s_t - 1) / s_t - 1 : 0;
  const int tile_pos0 = (n_k - n_q) + t * BLK;
  const int my_pos = tile_pos0 + r_local;
  // key range the wave's rows see: its first tile's first row .. its last tile's last row
  const int wave_pos_min = wave_on ? (n_k - n_q) + tw0 * BLK : 0;
  const int wave_pos_max = wave_on ? (n_k - n_q) + min((tw1 + 1) * BLK, n_q) - 1 : -1;
  const int gtile = p.seqs.tile_start[seq] + (in_range ? t : 0);

  const int64_t qrow = (int64_t)p.seqs.q_start[seq] + t * BLK + r_local;
  QFrag<T, D> qf;
  qf.load(reinterpret_cast<const T*>(p.q) + (qrow * p.hq + h) * D, col_on, g2);

  const int64_t row_stride = (int64_t)p.hkv * D;
  const T* kbase = reinterpret_cast<const T*>(p.k) + ((int64_t)p.seqs.k_start[seq] * p.hkv + gk) * D;
  const T* vsrc;
  if constexpr (F16PV) vsrc = reinterpret_cast<const T*>(p.v16);
  else vsrc = reinterpret_cast<const T*>(p.v);
  const T* vbase = vsrc + ((int64_t)p.seqs.k_start[seq] * p.hkv + gk) * D;
  // fp16 V: the scale of each key block of this sequence and KV head (read-only here,
  // so the reads go through the scalar cache)
  using cfloat = const __attribute__((address_space(4))) float;
  cfloat* vsc = nullptr;
  if constexpr (F16PV) vsc = (cfloat*)p.vscale + (int64_t)gk * p.total_kb + kblocks_before(p.seqs, seq);
  // per column: M2, l, L_rest / l, a pad word, then o and R / l (16-byte aligned); see
  // kRecordFloats
  float* rs_col = p.row_stats + (((int64_t)gk * p.seqs.total_tiles + gtile) * p.cols_rec + (in_range ? col : 0)) *
                                    kRecordFloats<D>;
  const float c = p.scale_log2;

  f32x16 O[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) O[dt] = f32x16{};
  // pass 1: running max and sum; pass 2: M2, l, dense output o, block weight sum
  float m_run = -INFINITY, l_run = 0.f;
  float m_ref = 0.f;                 // bf16 pass 1: final exponent reference
  float u0_ref = 0.f, l0_run = 0.f;  // bf16 pass 1: block 0's reference and weight sum
  float m2 = 0.f, inv_l = 0.f, mloc = 0.f, lrest = 0.f;
  float lt = 0.f;  // fp16 P V: the block's sum of the fp16 weights
  f32x16 Od[D / 32];
  if constexpr (PASS2) {
    if (col_on) {
      m2 = rs_col[0];
      inv_l = 1.f / rs_col[1];
      lrest = rs_col[2];
    }
  }
  // a D-vector of the column's record (at float offset `at`) in the accumulator layout
  auto load_vec = [&](f32x16 (&o)[D / 32], int at) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 v4 = {0.f, 0.f, 0.f, 0.f};
        if (col_on) v4 = *reinterpret_cast<const f32x4*>(rs_col + at + 32 * dt + 8 * a + 4 * g2);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[dt][4 * a + e] = v4[e];
      }
  };
  // pass 2 holds o, except that it holds R / l while it forms block 0
  if constexpr (PASS2 && !MASS && !PIPE) load_vec(Od, blk_lo == 0 ? 4 + D : 4);
  // per (KV head, tile, visible block): I of the record's columns, then m of them, so
  // a wave's per-block results are one coalesced store each per tile
  float* blk_I = nullptr;
  const int64_t bstride = 2 * (int64_t)p.cols_rec;
  if constexpr (PASS2) {
    if (in_range)
      blk_I = p.blk_stats + ((int64_t)gk * p.seqs.vis_per_head + vis_offset(p.seqs, seq, t)) * bstride + col;
  }

  // fp16 passes: the V scale of every key block of the sweep, staged in LDS, so the reads
  // inside the loop wait on LDS alone (a scalar load there makes the wait drain the LDS
  // fragment reads in flight as well); the sweep's first barrier publishes it
  __shared__ float vsc_sh[F16PV ? kMaxSeqBlocks : 1];
  if constexpr (F16PV) {
    for (int i = blk_lo + tid; i < blk_hi; i += sel_threads<T>()) vsc_sh[i] = vsc[i];
  }
  wait_vmem_all();
  const int total = (blk_hi - blk_lo) * SUBS;  // stages of this workgroup
  const int it_base = blk_lo * SUBS;
  auto stage_key0 = [](int it) { return (it / SUBS) * BLK + (it % SUBS) * kStageKeys; };
  // pass 2: I and m of one block from its weight sum and U (O), for the pair's column
  // fp16 P V: the weights and U carry 2^14 and U also the block's V scale s_b;
  // U - L o is formed at that scale, with L the sum of the same fp16 weights (which
  // also gives m_b = L / l)
  // For block 0, o holds R / l and U - L o is formed as
  // U L_rest / l - L R / l: the same vector (o = (U + R) / l, l = L + L_rest), without
  // the cancellation between U and L o when block 0 holds nearly all of the mass.
  auto finalize_block = [&](int blk, const f32x16 (&o)[D / 32]) {
    float mt, lo_coef, i_scale = inv_l;
    if constexpr (F16PV) {
      const float sb = vsc_sh[blk];
      const float ltt = half_sum(lt);
      lo_coef = ltt * sb;
      i_scale = inv_l * kP16Inv / sb;
      mt = ltt * kP16Inv;
    } else {
      mt = half_sum(mloc);
      lo_coef = mt;
    }
    float ss = 0.f;
    if constexpr (!MASS) {
      auto norm = [&](auto block0_tag) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float u = decltype(block0_tag)::value ? O[dt][r] * lrest : O[dt][r];
            const float dv = __builtin_fmaf(-lo_coef, o[dt][r], u);
            ss = __builtin_fmaf(dv, dv, ss);
          }
      };
      if (blk == 0) norm(BoolTag<true>{});
      else norm(BoolTag<false>{});
      ss = half_sum(ss);
    }
    if (col_on && g2 == 0) {
      float* dst = blk_I + (int64_t)blk * bstride;
      if constexpr (!MASS) dst[0] = __builtin_sqrtf(ss) * i_scale;
      dst[p.cols_rec] = mt * inv_l;
    }
  };
  if constexpr (PIPE) {
    // Software pipeline over stages, as in the attention kernel: K and V in separate
    // double buffers, V one stage behind K. Step j: the QK^T MFMAs of stage j next to
    // the exponentials (and sums) of stage j-1; then the P V MFMAs of stage j-1 next
    // to the bf16 packs of its following key step and stage j's running max. Every
    // wave computes every stage of the workgroup: a stage whose keys all lie above the
    // wave's rows is fully masked, so its weights are exactly zero (such stages are the
    // last few of the wave).
    __shared__ __attribute__((aligned(16))) char kb0[St::TENSOR];
    __shared__ __attribute__((aligned(16))) char kb1[St::TENSOR];
    __shared__ __attribute__((aligned(16))) char vb0[St::TENSOR];
    __shared__ __attribute__((aligned(16))) char vb1[St::TENSOR];
    constexpr int NQK = 2 * (D / 16);  // QK^T MFMAs per stage
    constexpr int NDT = D / 32;        // d tiles of O
    constexpr int NPV = 4 * NDT;       // P V MFMAs per stage (V fragment, key step)
    constexpr int EPM = 32 / NQK;      // exponentials per QK MFMA
    constexpr int XPM = 32 / NPV;      // max candidates per V fragment (pass 1)
    const typename St::LaneOffsets lofs = St::lane_offsets(row_stride, tid);
    float m_use = 0.f;  // pass 1: exponent reference of the stage being exponentiated
    const typename St::KOffsets ko = St::k_offsets(lane);
    auto kfrag = [&](const char* kbuf, int i) {  // K operand of QK MFMA i
      return St::k_frag(kbuf, ko, i & 1, i >> 1);
    };
    auto mask = [&](f32x16 (&S)[2], int key0) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + acc_key(kt, r, g2) > my_pos) S[kt][r] = -INFINITY;
    };
    auto finish_max = [&](float mx) {  // pass 1: running max of a stage, rare rescale
      mx = half_max(mx);
      const float m_new = fmaxf(m_run, mx * c);
      const float m_next = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_next);
      m_run = m_new;
      m_use = m_next;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) O[dt] *= alpha;
        l_run *= alpha;
      }
    };
    f32x16 Sp[2] = {f32x16{}, f32x16{}};
    auto skey = [&](int i) { return stage_key0(it_base + i); };  // first key of the chunk's stage i
    {
      St::load_k(kbase, row_stride, skey(0), n_k, tid, kb0, lofs);
      wait_vmem_all();
      __syncthreads();
      St::load_k(kbase, row_stride, skey(min(1, total - 1)), n_k, tid, kb1, lofs);
      St::load_v(vbase, row_stride, skey(0), n_k, tid, vb0, lofs);
      if (total > 0) {
        Sp[0] = St::qk_tile(kb0, qf, 0, lane);
        Sp[1] = St::qk_tile(kb0, qf, 1, lane);
        if (skey(0) + kStageKeys - 1 > wave_pos_min) mask(Sp, skey(0));
        if constexpr (!PASS2) {
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 32; ++e) mx = fmaxf(mx, Sp[e >> 4][e & 15]);
          finish_max(mx);
        }
      }
      wait_vmem_all();
      __syncthreads();
    }
    // step it (1 <= it <= total): with MORE (it < total) the QK of stage it, then the
    // softmax and P V of stage it - 1; the last step (it = total) has P V alone
    auto step = [&](auto more_tag, int it, const char* kcur, char* knext, const char* vprev, char* vcur) {
      constexpr bool MORE = decltype(more_tag)::value;
      const int key0 = MORE ? skey(it) : 0;
      if constexpr (MORE) {
        St::load_k(kbase, row_stride, skey(min(it + 1, total - 1)), n_k, tid, knext, lofs);
        St::load_v(vbase, row_stride, key0, n_k, tid, vcur, lofs);
      }
      f32x16 Sn[2] = {f32x16{}, f32x16{}};
      float mx = -INFINITY;
      // QK phase
      bf16x8 ka[3];
      if constexpr (MORE) {
        ka[0] = kfrag(kcur, 0);
        ka[1] = kfrag(kcur, 1);
      }
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        if constexpr (MORE) {
          Sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % 3], qf.q[i >> 1], Sn[i & 1], 0, 0, 0);
          if (i + 2 < NQK) ka[(i + 2) % 3] = kfrag(kcur, i + 2);
        }
#pragma unroll
        for (int u = 0; u < EPM; ++u) {
          const int e = i * EPM + u;
          Sp[e >> 4][e & 15] = __builtin_amdgcn_exp2f(__builtin_fmaf(Sp[e >> 4][e & 15], c, -m_use));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const int pst = it - 1;  // the stage whose P V this step runs
      // PV phase: O += V^T P with the packs one key step ahead (one bf16 P: see the
      // file header); l adds the same bf16 weights, two per dot instruction, so o is
      // their exact weighted mean
      __builtin_amdgcn_s_setprio(1);
      bf16x8 ph[2], unused;
      p_step<false>(Sp, 0, ph[0], unused);
      float rs = row_sum_bf16(ph[0], 0.f);
      bf16x8 va[3];  // V fragments read two MFMAs ahead of their use
      va[0] = St::v_frag(vprev, 0, 0, lane);
      va[1] = St::v_frag(vprev, 1 % NDT, 1 / NDT, lane);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int dt = i % NDT, st = i / NDT;
        if (i + 2 < NPV) va[(i + 2) % 3] = St::v_frag(vprev, (i + 2) % NDT, (i + 2) / NDT, lane);
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 3], ph[st & 1], O[dt], 0, 0, 0);
        if (dt == 0 && st + 1 < 4) {
          p_step<false>(Sp, st + 1, ph[(st + 1) & 1], unused);
          rs = row_sum_bf16(ph[(st + 1) & 1], rs);
        }
        if constexpr (MORE) {
#pragma unroll
          for (int u = 0; u < XPM; ++u) {
            const int e = i * XPM + u;
            mx = fmaxf(mx, Sn[e >> 4][e & 15]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      l_run += rs;
      if (it_base + pst == SUBS - 1) {
        // block 0 is complete: its sums U_0 (in the record's o slot) and L_0 are kept
        // apart, at the reference they were formed with, and O and l restart for the
        // blocks after it
        u0_ref = m_use;
        l0_run = l_run;
        l_run = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 u = {O[dt][4 * a], O[dt][4 * a + 1], O[dt][4 * a + 2], O[dt][4 * a + 3]};
            if (col_on) *reinterpret_cast<f32x4*>(rs_col + 4 + 32 * dt + 8 * a + 4 * g2) = u;
          }
          O[dt] = f32x16{};
        }
      }
      if constexpr (MORE) {
        if (key0 + kStageKeys - 1 > wave_pos_min) {
          mask(Sn, key0);
          mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 32; ++e) mx = fmaxf(mx, Sn[e >> 4][e & 15]);
        }
        finish_max(mx);
        Sp[0] = Sn[0];
        Sp[1] = Sn[1];
        wait_vmem_all();
        __syncthreads();
      }
    };
    int it = 1;
    for (; it + 1 < total; it += 2) {
      step(BoolTag<true>{}, it, kb1, kb0, vb0, vb1);
      step(BoolTag<true>{}, it + 1, kb0, kb1, vb1, vb0);
    }
    if (it < total) {
      step(BoolTag<true>{}, it, kb1, kb0, vb0, vb1);
      ++it;
    }
    // it == total: the P V of the last stage, whose V sits in vb[(total - 1) & 1]
    if (total > 0) step(BoolTag<false>{}, it, nullptr, nullptr, ((total - 1) & 1) ? vb1 : vb0, nullptr);
    m_ref = m_use;
  } else {
  __shared__ __attribute__((aligned(16))) char buf0[St::BYTES];
  __shared__ __attribute__((aligned(16))) char buf1[St::BYTES];
  const typename St::KOffsets ko = St::k_offsets(lane);
  // pass 2 stage for bf16 (see its call below); MASKED: the stage reaches past a row
  // MASKED: the stage reaches past a row; FIRST: it opens a block, so its first P V
  // MFMA of each d tile starts from zero instead of O
  auto pass2_stage = [&](auto masked_tag, auto first_tag, const char* cur, int key0) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    if constexpr (F16PV) {
      constexpr int ST = D / 16;   // d steps of one QK^T tile
      constexpr int NDT = D / 32;  // d tiles of O
      auto kfrag = [&](int kt, int st) { return St::k_frag(cur, ko, kt, st); };
      const float wbias = kP16Log2 - m2;  // weights 2^14 w_j, at most 2^14 (fp16 range)
      auto weight = [&](float s, int kt, int r) {
        if (MASKED && key0 + acc_key(kt, r, g2) > my_pos) return 0.f;
        return __builtin_amdgcn_exp2f(__builtin_fmaf(s, c, wbias));
      };
      const char* vt = cur + St::TENSOR;
      f32x16 S0 = {}, S1 = {};
      bf16x8 ka[3];
      ka[0] = kfrag(0, 0);
      ka[1] = kfrag(0, 1);
#pragma unroll
      for (int i = 0; i < ST; ++i) {  // key tile 0
        S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % 3], qf.q[i], S0, 0, 0, 0);
        ka[(i + 2) % 3] = kfrag((i + 2) / ST, (i + 2) % ST);
        __builtin_amdgcn_sched_barrier(0);
      }
      f32x16 Sp[2];
      f16x8 ph[4];
#pragma unroll
      for (int i = 0; i < ST; ++i) {  // key tile 1, next to the weights of key tile 0
        S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[(ST + i) % 3], qf.q[i], S1, 0, 0, 0);
        if (i + 2 < ST) ka[(ST + i + 2) % 3] = kfrag(1, i + 2);
#pragma unroll
        for (int u = 0; u < 16 / ST; ++u) {
          const int r = i * (16 / ST) + u;
          S0[r] = weight(S0[r], 0, r);
        }
        if (i == ST - 1) {
          Sp[0] = S0;
          ph[0] = p_step_f16(Sp, 0);
          ph[1] = p_step_f16(Sp, 1);
          lt = row_sum_f16(ph[1], row_sum_f16(ph[0], lt));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // P V over key steps 0 and 1, next to the weights and packs of key tile 1
      bf16x8 va[3];  // V fragments read two MFMAs ahead of their use
      va[0] = St::v_frag(vt, 0, 0, lane);
      va[1] = St::v_frag(vt, 1 % NDT, 1 / NDT, lane);
#pragma unroll
      for (int i = 0; i < 2 * NDT; ++i) {
        const int dt = i % NDT, st = i / NDT;
        va[(i + 2) % 3] = St::v_frag(vt, (i + 2) % NDT, (i + 2) / NDT, lane);
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, va[i % 3]), ph[st],
                                                       (FIRST && st == 0) ? f32x16{} : O[dt], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 16 / (2 * NDT); ++u) {
          const int r = i * (16 / (2 * NDT)) + u;
          S1[r] = weight(S1[r], 1, r);
        }
        if (i == 2 * NDT - 1) {
          Sp[1] = S1;
          ph[2] = p_step_f16(Sp, 2);
          ph[3] = p_step_f16(Sp, 3);
          lt = row_sum_f16(ph[3], row_sum_f16(ph[2], lt));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 2 * NDT; i < 4 * NDT; ++i) {  // key steps 2 and 3
        const int dt = i % NDT, st = i / NDT;
        if (i + 2 < 4 * NDT) va[(i + 2) % 3] = St::v_frag(vt, (i + 2) % NDT, (i + 2) / NDT, lane);
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, va[i % 3]), ph[st], O[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto key0_of = [&](int i) { return stage_key0(it_base + i); };
  sweep<St, MASS>(total, key0_of, kbase, vbase, row_stride, n_k, tid, buf0, buf1, [&](int i, const char* cur) {
    const int it = it_base + i;
    const int blk = it / SUBS, sub = it % SUBS;
    const int key0 = stage_key0(it);
    if (PASS2 && sub == 0) {
      if constexpr (!F16PV) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) O[dt] = f32x16{};
      }
      mloc = 0.f;
      lt = 0.f;
    }
    if constexpr (F16PV) {
      // pass 2, bf16: one stage with its work overlapped inside the wave. The QK^T MFMAs
      // of key tile 1 run next to the weights of key tile 0; the first half of the fp16
      // P V next to the weights and packs of key tile 1; fragments are read ahead. A
      // block's first stage always runs when the block is finalised (its keys start at
      // or below the tile's first row), so it is the one that starts U from zero.
      if (key0 <= wave_pos_max) {
        const bool masked = key0 + kStageKeys - 1 > wave_pos_min;
        if (sub == 0) {
          if (masked) pass2_stage(BoolTag<true>{}, BoolTag<true>{}, cur, key0);
          else pass2_stage(BoolTag<false>{}, BoolTag<true>{}, cur, key0);
        } else {
          if (masked) pass2_stage(BoolTag<true>{}, BoolTag<false>{}, cur, key0);
          else pass2_stage(BoolTag<false>{}, BoolTag<false>{}, cur, key0);
        }
      }
    } else if (key0 <= wave_pos_max) {
      f32x16 S[2];
      S[0] = St::qk_tile(cur, qf, 0, lane);
      S[1] = St::qk_tile(cur, qf, 1, lane);
      const bool need_mask = key0 + kStageKeys - 1 > wave_pos_min;
      if constexpr (!PASS2) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float s = (need_mask && key0 + acc_key(kt, r, g2) > my_pos) ? -INFINITY : S[kt][r];
            S[kt][r] = s;
            mx = fmaxf(mx, s);
          }
        mx = half_max(mx);
        const float m_new = fmaxf(m_run, mx * c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float e = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kt][r], c, -m_use));
            S[kt][r] = e;
            rs += e;
          }
        l_run = l_run * alpha + rs;
        m_run = m_new;
        if (!MASS && __any(alpha != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) O[dt] *= alpha;
        }
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float e = (need_mask && key0 + acc_key(kt, r, g2) > my_pos)
                          ? 0.f
                          : __builtin_amdgcn_exp2f(__builtin_fmaf(S[kt][r], c, -m2));
            S[kt][r] = e;
            mloc += e;
          }
      }
      if constexpr (!MASS) St::template pv<SPLIT>(cur, S, O, lane);
      if constexpr (SPLIT0) {
        if (it == SUBS - 1) {
          // block 0 is complete (every wave computes it): its sums U_0 (in the record's
          // o slot) and L_0 are kept apart, at the reference they were formed with, and
          // O and l restart for the blocks after it, as in the pipelined sweep
          u0_ref = (m_run == -INFINITY) ? 0.f : m_run;
          l0_run = l_run;
          l_run = 0.f;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const f32x4 u = {O[dt][4 * a], O[dt][4 * a + 1], O[dt][4 * a + 2], O[dt][4 * a + 3]};
              if (col_on) *reinterpret_cast<f32x4*>(rs_col + 4 + 32 * dt + 8 * a + 4 * g2) = u;
            }
            O[dt] = f32x16{};
          }
        }
      }
    }
    if constexpr (PASS2) {
      // lanes l and l ^ 32 hold the same column, so the pair takes the branch together
      if (sub == SUBS - 1 && in_range && blk <= diag) finalize_block(blk, Od);
      if constexpr (!MASS) {
        if (sub == SUBS - 1 && blk == 0) load_vec(Od, 4);  // o for the other blocks
      }
    }
  });
  // the reference O and l were last formed at
  if constexpr (!PASS2) m_ref = (m_run == -INFINITY) ? 0.f : m_run;
  }

  if (!PASS2 && SPLIT0 && n_chunks > 1) {
    // one chunk of the group's blocks: raw sums at this chunk's own reference m_ref, for
    // sel_merge_kernel. Chunk 0 leaves in the record M2 <- m_ref, l <- L_rest of its
    // blocks after block 0, then u0_ref and L_0, with U_0 already in the o slot and R in
    // the R / l slot; a later chunk leaves (m_ref, or -inf when it saw no key, its weight
    // sum, U) in its partial record.
    const float l_c = half_sum(l_run);
    const float l0 = half_sum(l0_run);
    if (col_on) {
      float* vdst;
      if (chunk == 0) {
        if (g2 == 0) {
          rs_col[0] = m_ref;
          rs_col[1] = l_c;
          rs_col[2] = u0_ref;
          rs_col[3] = l0;
        }
        vdst = rs_col + 4 + D;
      } else {
        float* part = p.p1_part + ((((int64_t)gk * p.seqs.total_tiles + gtile) * p.cols_rec + col) * (n_chunks - 1) +
                                   (chunk - 1)) * (D + 4);
        if (g2 == 0) {
          part[0] = l_c > 0.f ? m_ref : -INFINITY;
          part[1] = l_c;
        }
        vdst = part + 4;
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 u = {O[dt][4 * a], O[dt][4 * a + 1], O[dt][4 * a + 2], O[dt][4 * a + 3]};
          *reinterpret_cast<f32x4*>(vdst + 32 * dt + 8 * a + 4 * g2) = u;
        }
    }
  } else if constexpr (!PASS2 && SPLIT0) {
    // O and l hold R and L_rest (the blocks after block 0) at reference m_ref; U_0 (in the
    // record) and L_0 were formed at reference u0_ref <= m_ref
    const float f0 = __builtin_amdgcn_exp2f(u0_ref - m_ref);
    const float l_rest = half_sum(l_run);
    const float l_all = half_sum(l0_run) * f0 + l_rest;
    const float r_coef = 1.f / l_all;  // R -> R / l
    const float u_coef = f0 / l_all;   // U_0 -> U_0 / l
    wait_vmem_all();  // this lane's U_0 stores have landed
    if (col_on) {
      if (g2 == 0) {
        rs_col[0] = m_ref;
        rs_col[1] = l_all;
        rs_col[2] = l_rest / l_all;
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float* po = rs_col + 4 + 32 * dt + 8 * a + 4 * g2;
          const f32x4 u = *reinterpret_cast<const f32x4*>(po);
          const f32x4 rn = {O[dt][4 * a] * r_coef, O[dt][4 * a + 1] * r_coef, O[dt][4 * a + 2] * r_coef,
                            O[dt][4 * a + 3] * r_coef};
          const f32x4 o = {__builtin_fmaf(u[0], u_coef, rn[0]), __builtin_fmaf(u[1], u_coef, rn[1]),
                           __builtin_fmaf(u[2], u_coef, rn[2]), __builtin_fmaf(u[3], u_coef, rn[3])};
          *reinterpret_cast<f32x4*>(po) = o;
          *reinterpret_cast<f32x4*>(po + D) = rn;
        }
    }
  } else if (!PASS2 && n_chunks > 1) {
    // mass-only, one chunk: the chunk's raw weight sum at its own reference, in the
    // layout of the split sweep's chunks with L_0 = 0 (chunk 0's record: reference, L,
    // u0_ref = the reference, L_0; a later chunk's partial record: reference or -inf, L)
    const float l_c = half_sum(l_run);
    if (col_on) {
      float* vdst;
      if (chunk == 0) {
        if (g2 == 0) {
          rs_col[0] = m_ref;
          rs_col[1] = l_c;
          rs_col[2] = m_ref;
          rs_col[3] = 0.f;
        }
        if constexpr (!MASS) {
#pragma unroll
          for (int e = 0; e < D / 32 * 4; ++e)
            *reinterpret_cast<f32x4*>(rs_col + 4 + 32 * (e / 4) + 8 * (e % 4) + 4 * g2) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        vdst = rs_col + 4 + D;
      } else {
        float* part = p.p1_part + ((((int64_t)gk * p.seqs.total_tiles + gtile) * p.cols_rec + col) * (n_chunks - 1) +
                                   (chunk - 1)) * (D + 4);
        if (g2 == 0) {
          part[0] = l_c > 0.f ? m_ref : -INFINITY;
          part[1] = l_c;
        }
        vdst = part + 4;
      }
      if constexpr (!MASS) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 u = {O[dt][4 * a], O[dt][4 * a + 1], O[dt][4 * a + 2], O[dt][4 * a + 3]};
            *reinterpret_cast<f32x4*>(vdst + 32 * dt + 8 * a + 4 * g2) = u;
          }
      }
    }
  } else if constexpr (!PASS2) {
    const float l_tot = half_sum(l_run);
    if (col_on) {
      const float inv = 1.f / l_tot;
      if (g2 == 0) {
        rs_col[0] = m_run;
        rs_col[1] = l_tot;
      }
      if constexpr (!MASS) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            f32x4 o = {O[dt][4 * a] * inv, O[dt][4 * a + 1] * inv, O[dt][4 * a + 2] * inv, O[dt][4 * a + 3] * inv};
            *reinterpret_cast<f32x4*>(rs_col + 4 + 32 * dt + 8 * a + 4 * g2) = o;
          }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Threshold, ranking and compaction: one workgroup per (query head, tile).
//
// The G query heads of one (KV head, tile) read disjoint S-float slices of the same
// per-block records. The grid puts those G workgroups on one XCD (workgroup ids are
// dealt round-robin over the XCDs) and next to each other in time, so one L2 fetch
// of a record line serves the whole group. STAGED: a head's per-row values are read
// once, coalesced, into LDS and both walks of the discard order run on LDS; without
// it (tiles too long for LDS) the walks gather the rows from the workspace.
// ---------------------------------------------------------------------------

constexpr int kThrThreads = 256;
constexpr int kThrWaves = kThrThreads / 64;
constexpr int kMaxVis = kMaxSeqBlocks;
constexpr int kStageVis = 1024;   // STAGED: visible blocks per tile
constexpr int kStageVals = 8192;  // STAGED: visible blocks x sampled rows
constexpr int kXcds = 8;

// Exclusive prefix over the workgroup, in thread order, of N pairs of doubles (each
// thread's A[r], D[r] are replaced by the sums over lower threads). sh: 2 * N *
// kThrWaves doubles.
constexpr int kRowChunk = 8;
template <int N>
__device__ __forceinline__ void block_excl_scan_vec(double (&A)[N], double (&D)[N], double* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double ia[N], id[N];
#pragma unroll
  for (int r = 0; r < N; ++r) { ia[r] = A[r]; id[r] = D[r]; }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
    for (int r = 0; r < N; ++r) {
      const double ta = __shfl_up(ia[r], o), td = __shfl_up(id[r], o);
      if (lane >= o) { ia[r] += ta; id[r] += td; }
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int r = 0; r < N; ++r) {
      sh[(2 * r) * kThrWaves + wave] = ia[r];
      sh[(2 * r + 1) * kThrWaves + wave] = id[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < N; ++r) {
    double xa = __shfl_up(ia[r], 1), xd = __shfl_up(id[r], 1);
    if (lane == 0) { xa = 0.0; xd = 0.0; }
    double oa = 0.0, od = 0.0;
    for (int w = 0; w < wave; ++w) { oa += sh[(2 * r) * kThrWaves + w]; od += sh[(2 * r + 1) * kThrWaves + w]; }
    A[r] = oa + xa;
    D[r] = od + xd;
  }
  __syncthreads();
}

__device__ __forceinline__ int block_min_int(int v, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  int r = sh[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = min(r, sh[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)x, m), hi = __shfl_xor((uint32_t)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Ascending bitonic sort of 256 * E keys held in blocked order (thread tid holds
// positions tid * E .. tid * E + E - 1). Partners in the same thread are swapped in
// registers, partners in the same wave by shuffles, and only the stages whose
// partners sit in other waves go through LDS (sh: 256 * E keys).
template <int E>
__device__ __forceinline__ void sort_blocked(uint64_t (&x)[E], uint64_t* sh) {
  constexpr int N = kThrThreads * E;
  const int tid = threadIdx.x, lane = tid & 63;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int ep = e ^ j;
          if (ep > e) {
            const bool up = ((tid * E + e) & k) == 0;
            const uint64_t a = x[e], b = x[ep];
            if ((a > b) == up) { x[e] = b; x[ep] = a; }
          }
        }
      } else if (j < 64 * E) {
        const int lj = j / E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint64_t o = shfl_xor_u64(x[e], lj);
          const bool up = ((tid * E + e) & k) == 0;
          const bool keep_min = ((lane & lj) == 0) == up;
          x[e] = keep_min ? (x[e] < o ? x[e] : o) : (x[e] < o ? o : x[e]);
        }
      } else {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) sh[tid * E + e] = x[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = tid * E + e;
          const uint64_t o = sh[i ^ j];
          const bool keep_min = ((i & j) == 0) == ((i & k) == 0);
          x[e] = keep_min ? (x[e] < o ? x[e] : o) : (x[e] < o ? o : x[e]);
        }
      }
    }
  }
}

// Sampled rows i0 .. i0 + nr - 1 (nr <= kRowChunk, i0 a multiple of kRowChunk) of visible
// block b, from the LDS copy (st) or the workspace (glob). A staged record holds a
// block's S rows side by side, so with S a multiple of 4 they are read as 16-byte
// vectors: one 32-bit read per row, with the lanes of a wave on records S floats
// apart, would put the whole wave on a few LDS banks. Entries r >= nr are not set.
template <bool STAGED>
__device__ __forceinline__ void block_rows(const float* st, const float* glob, int64_t bstride, int S, int b, int i0,
                                           int nr, float (&v)[kRowChunk]) {
  if (STAGED && S % 4 == 0) {
    const float* rec = st + b * S + i0;  // 16-byte aligned: st is, and b * S + i0 is a multiple of 4
#pragma unroll
    for (int r = 0; r < kRowChunk; r += 4)
      if (r < nr) {  // rows up to r + 3 < S stay inside the record
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(rec + r);
        v[r] = q4[0];
        v[r + 1] = q4[1];
        v[r + 2] = q4[2];
        v[r + 3] = q4[3];
      }
  } else {
#pragma unroll
    for (int r = 0; r < kRowChunk; ++r)
      if (r < nr) v[r] = STAGED ? st[b * S + i0 + r] : glob[(int64_t)b * bstride + i0 + r];
  }
}

// One (query head, tile) of the threshold kernel after staging: scores, sort, cut,
// row bounds and compaction, with E = padded candidates / 256 keys per thread.
struct ThrTile {
  int h0, nh;  // the list is written for query heads h0 .. h0 + nh - 1 (nh = G when shared)
  int gtile, S, s_t, n_vis, diag;
  int64_t slot, bstride;
  const float* Ib;  // the rows' slice of the per-block records (global)
  const float* Mb;
  int tau_group;    // 0: every row uses tau[h0]; G: row i uses tau[h0 + i % G]
};

// MODE kSelectOutputRelative: key = mean_i I_ib, bound = max_i A_i(k) / (1 - Delta_i(k));
// MODE kSelectMass: key = mean_i m_ib, bound = max_i Delta_i(k).
template <int MODE, bool STAGED, int E>
__device__ __forceinline__ void threshold_tile(const SelectParams& p, const ThrTile& w, const float* st_I,
                                               const float* st_m, uint64_t* sh, uint8_t* keep, double* shd,
                                               int* shi) {
  constexpr bool POEM = MODE == kSelectOutputRelative;
  const int tid = threadIdx.x;
  const int T = p.seqs.total_tiles;
  const int S = w.S, s_t = w.s_t, n_vis = w.n_vis, diag = w.diag;
  auto rows_I = [&](int b, int i0, int nr, float (&v)[kRowChunk]) {
    block_rows<STAGED>(st_I, w.Ib, w.bstride, S, b, i0, nr, v);
  };
  auto rows_m = [&](int b, int i0, int nr, float (&v)[kRowChunk]) {
    block_rows<STAGED>(st_m, w.Mb, w.bstride, S, b, i0, nr, v);
  };
  auto mandatory = [&](int b) { return b < p.n_sink || b > diag - p.n_local; };
  const float inv_s = 1.f / (float)s_t;
  const int64_t head_stride = (int64_t)T * p.max_vis;  // score rows of consecutive heads
  const int64_t diag_row = ((int64_t)w.h0 * T + w.gtile) * p.max_vis;
  auto tau_of = [&](int i) { return p.tau[w.h0 + (w.tau_group ? i % w.tau_group : 0)]; };

  // scores of blocks e * 256 + tid as sort keys (score bits, ~id); the sort does not
  // care where a key starts
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int b = e * kThrThreads + tid;
    x[e] = ~0ull;
    if (b < n_vis) {
      float si = 0.f, sm = 0.f;
      for (int i0 = 0; i0 < s_t; i0 += kRowChunk) {
        const int nr = min(kRowChunk, s_t - i0);
        float vi[kRowChunk], vm[kRowChunk];
        if constexpr (POEM) rows_I(b, i0, nr, vi);
        rows_m(b, i0, nr, vm);
#pragma unroll
        for (int r = 0; r < kRowChunk; ++r)
          if (r < nr) {
            if constexpr (POEM) si += vi[r];
            sm += vm[r];
          }
      }
      const float mass = sm * inv_s;
      const float score = POEM ? si * inv_s : mass;
      for (int hh = 0; hh < w.nh; ++hh) {
        if (p.tile_scores) p.tile_scores[diag_row + hh * head_stride + b] = score;
        if (p.tile_mass) p.tile_mass[diag_row + hh * head_stride + b] = mass;
      }
      if (!mandatory(b)) x[e] = ((uint64_t)__float_as_uint(score) << 32) | (uint64_t)(0xffffffffu - (uint32_t)b);
    }
  }
  for (int hh = 0; hh < w.nh; ++hh)
    for (int b = n_vis + tid; b < p.max_vis; b += kThrThreads) {
      if (p.tile_scores) p.tile_scores[diag_row + hh * head_stride + b] = -1.f;
      if (p.tile_mass) p.tile_mass[diag_row + hh * head_stride + b] = -1.f;
    }
  sort_blocked<E>(x, sh);  // ascending: the discard order

  // |{b < n_sink} U {diag - n_local < b <= diag}| inside 0 .. diag
  const int sink_hi = min(p.n_sink, n_vis);
  const int loc_lo = max(0, diag - p.n_local + 1);
  const int n_mand = sink_hi + (n_vis - loc_lo) - max(0, sink_hi - loc_lo);
  const int n_cand = n_vis - n_mand;
  int ids[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ids[e] = (int)(0xffffffffu - (uint32_t)(x[e] & 0xffffffffull));
  auto bound_of = [&](double a, double dl) -> double {
    if constexpr (POEM) return (1.0 - dl > 0.0) ? a / (1.0 - dl) : INFINITY;
    else return dl;
  };
  // bound > t without the division: A / (1 - Delta) > t  <=>  A > t (1 - Delta) when
  // 1 - Delta > 0 (otherwise the bound is infinite). The two forms can differ only
  // when the bound lies within an fp64 rounding of t.
  auto exceeds = [&](double a, double dl, double t) -> bool {
    if constexpr (POEM) return !(1.0 - dl > 0.0) || a > t * (1.0 - dl);
    else return dl > t;
  };

  // Prefix sums over the discard order, kRowChunk sampled rows at a time: each thread
  // sums its E consecutive positions, a vector scan gives each thread its exclusive
  // prefixes, and the first prefix length whose per-row bound exceeds tau is a block
  // minimum. With `limit` = the cut, the same walk yields the per-row bound at the cut.
  // KEEP (one chunk holds every row): the find walk also keeps each position's per-row
  // bounds, so the bounds at the cut need no second walk.
  float kept_b[E][kRowChunk];
  const bool keep_bounds = p.row_bound != nullptr;  // the bounds at the cut are an optional output
  auto walk = [&](auto keep_tag, int i0, int nr, int limit, bool find, int& local_fail, float* rb_out) {
    constexpr bool KEEP = decltype(keep_tag)::value;
    double A[kRowChunk], Dl[kRowChunk];
#pragma unroll
    for (int r = 0; r < kRowChunk; ++r) A[r] = Dl[r] = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (tid * E + e < limit) {
        float vi[kRowChunk], vm[kRowChunk];
        if constexpr (POEM) rows_I(ids[e], i0, nr, vi);
        rows_m(ids[e], i0, nr, vm);
#pragma unroll
        for (int r = 0; r < kRowChunk; ++r)
          if (r < nr) {
            if constexpr (POEM) A[r] += (double)vi[r];
            Dl[r] += (double)vm[r];
          }
      }
    }
    block_excl_scan_vec<kRowChunk>(A, Dl, shd);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int k = tid * E + e;
      if (k < limit) {
        bool over = false;
        float vi[kRowChunk], vm[kRowChunk];
        if constexpr (POEM) rows_I(ids[e], i0, nr, vi);
        rows_m(ids[e], i0, nr, vm);
#pragma unroll
        for (int r = 0; r < kRowChunk; ++r)
          if (r < nr) {
            if constexpr (POEM) A[r] += (double)vi[r];
            Dl[r] += (double)vm[r];
            if (find) over |= exceeds(A[r], Dl[r], (double)tau_of(i0 + r));
            if constexpr (KEEP)
              if (keep_bounds) kept_b[e][r] = (float)bound_of(A[r], Dl[r]);
            if (!find && k == limit - 1) rb_out[i0 + r] = (float)bound_of(A[r], Dl[r]);
          }
        if (find && over && local_fail == INT_MAX) local_fail = k + 1;
      }
    }
  };
  int k_fail = n_cand + 1;
  const bool one_chunk = s_t <= kRowChunk;
  if (one_chunk) {
    int local_fail = INT_MAX;
    walk(BoolTag<true>{}, 0, s_t, n_cand, true, local_fail, nullptr);
    k_fail = min(k_fail, block_min_int(local_fail, shi));
  } else {
    for (int i0 = 0; i0 < s_t; i0 += kRowChunk) {
      int local_fail = INT_MAX;
      walk(BoolTag<false>{}, i0, min(kRowChunk, s_t - i0), n_cand, true, local_fail, nullptr);
      k_fail = min(k_fail, block_min_int(local_fail, shi));
    }
  }
  const int k_star = k_fail - 1;

  if (p.row_bound) {
    float* rb = p.row_bound + ((int64_t)w.h0 * T + w.gtile) * S;
    if (one_chunk) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (k_star > 0 && tid * E + e == k_star - 1)
#pragma unroll
          for (int r = 0; r < kRowChunk; ++r)
            if (r < s_t) rb[r] = kept_b[e][r];
    } else {
      for (int i0 = 0; i0 < s_t; i0 += kRowChunk) {
        int unused = INT_MAX;
        walk(BoolTag<false>{}, i0, min(kRowChunk, s_t - i0), k_star, false, unused, rb);
      }
    }
    for (int i = tid; i < S; i += kThrThreads)
      if (i >= s_t) rb[i] = -1.f;
      else if (k_star == 0) rb[i] = 0.f;
    if (w.nh > 1) {  // the same rows' bounds under every head of the group
      __syncthreads();
      for (int hh = 1; hh < w.nh; ++hh)
        for (int i = tid; i < S; i += kThrThreads) rb[(int64_t)hh * T * S + i] = rb[i];
    }
  }

  // retained set, compacted in ascending id order
  for (int b = tid; b < n_vis; b += kThrThreads) keep[b] = 1;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (tid * E + e < k_star) keep[ids[e]] = 0;
  __syncthreads();
  const int E2 = (n_vis + kThrThreads - 1) / kThrThreads;
  int cnt = 0;
  for (int e = 0; e < E2; ++e) {
    const int b = tid * E2 + e;
    if (b < n_vis) cnt += keep[b];
  }
  int total;
  int off = block_excl_scan_int(cnt, total, shi);
  int32_t* out = p.slots + w.slot;
  for (int e = 0; e < E2; ++e) {
    const int b = tid * E2 + e;
    if (b < n_vis && keep[b]) out[off++] = b;
  }
  if (tid < w.nh) p.counts[(w.h0 + tid) * T + w.gtile] = total;
}

template <int V> struct IntTag { static constexpr int value = V; };

// float -> uint32 whose unsigned order is the float order (-inf lowest)
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix over the workgroup of one double per position, positions held in
// blocked order (E per thread): x[e] becomes the sum over positions <= tid * E + e.
// Returns the total.
template <int E>
__device__ __forceinline__ double blocked_inclusive_scan(double (&x)[E], double* shd, double* total_sh) {
  double run = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) { run += x[e]; x[e] = run; }
  double a[1] = {run}, d[1] = {0.0};
  block_excl_scan_vec<1>(a, d, shd);  // a: this thread's exclusive offset
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] += a[0];
  if (threadIdx.x == kThrThreads - 1) *total_sh = x[E - 1];  // the last position holds the total
  __syncthreads();
  const double total = *total_sh;
  __syncthreads();
  return total;
}

// Practical POEM for one (query head, tile): pooled estimates, a mass preselection,
// a rerank by log mbar + w log(Ibar / mbar), and blocks kept in that order until the
// pooled retained mass reaches (1 - eps) of the pooled total (POEM note Equation (6)
// and its selection procedure). Two register sorts and two fp64 prefix scans.
template <bool STAGED, int E>
__device__ __forceinline__ void practical_tile(const SelectParams& p, const ThrTile& w, const float* st_I,
                                               const float* st_m, float* bar_I, float* bar_m, uint64_t* sh,
                                               uint8_t* keep, double* shd, int* shi) {
  __shared__ double sums[2];
  const int tid = threadIdx.x;
  const int T = p.seqs.total_tiles;
  const int S = w.S, s_t = w.s_t, n_vis = w.n_vis, diag = w.diag;
  auto mandatory = [&](int b) { return b < p.n_sink || b > diag - p.n_local; };
  const float inv_s = 1.f / (float)s_t;
  const float wt = p.prac_w;
  const int64_t diag_row = ((int64_t)w.h0 * T + w.gtile) * p.max_vis;
  // natural-log rerank key of a block (-inf without mass, or without deviation if w != 0)
  auto rerank_key = [&](float mb, float ib) {
    constexpr float kLn2f = 0.6931471805599453f;
    float key = -INFINITY;
    if (mb > 0.f) {
      key = __builtin_amdgcn_logf(mb) * kLn2f;
      if (wt != 0.f) key = ib > 0.f ? key + wt * (__builtin_amdgcn_logf(ib / mb) * kLn2f) : -INFINITY;
    }
    return key;
  };

  // pooled estimates and keys by mass (descending, ids ascending among equal masses)
  uint64_t x[E];
  double tot_all = 0.0, tot_mand = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int b = tid * E + e;
    x[e] = ~0ull;
    if (b < n_vis) {
      float si = 0.f, sm = 0.f;
      for (int i0 = 0; i0 < s_t; i0 += kRowChunk) {
        const int nr = min(kRowChunk, s_t - i0);
        float vi[kRowChunk], vm[kRowChunk];
        block_rows<STAGED>(st_I, w.Ib, w.bstride, S, b, i0, nr, vi);
        block_rows<STAGED>(st_m, w.Mb, w.bstride, S, b, i0, nr, vm);
#pragma unroll
        for (int r = 0; r < kRowChunk; ++r)
          if (r < nr) {
            si += vi[r];
            sm += vm[r];
          }
      }
      const float mb = sm * inv_s, ib = si * inv_s;
      bar_I[b] = ib;
      bar_m[b] = mb;
      if (p.tile_scores) p.tile_scores[diag_row + b] = rerank_key(mb, ib);
      if (p.tile_mass) p.tile_mass[diag_row + b] = mb;
      tot_all += (double)mb;
      if (mandatory(b)) tot_mand += (double)mb;
      else x[e] = ((uint64_t)(0xffffffffu - __float_as_uint(mb)) << 32) | (uint64_t)(uint32_t)b;
    }
  }
  for (int b = n_vis + tid; b < p.max_vis; b += kThrThreads) {
    if (p.tile_scores) p.tile_scores[diag_row + b] = -1.f;
    if (p.tile_mass) p.tile_mass[diag_row + b] = -1.f;
  }
  {
    double a[1] = {tot_all}, d[1] = {tot_mand};
    block_excl_scan_vec<1>(a, d, shd);
    if (tid == kThrThreads - 1) {
      sums[0] = a[0] + tot_all;
      sums[1] = d[0] + tot_mand;
    }
    __syncthreads();
    tot_all = sums[0];
    tot_mand = sums[1];
    __syncthreads();
  }
  sort_blocked<E>(x, sh);

  // preselection: the shortest prefix of the mass order reaching rho of the candidates' mass
  auto id_of = [](uint64_t key) { return (int)(uint32_t)(key & 0xffffffffull); };
  double c[E];
#pragma unroll
  for (int e = 0; e < E; ++e) c[e] = x[e] == ~0ull ? 0.0 : (double)bar_m[id_of(x[e])];
  const double cand_mass = blocked_inclusive_scan<E>(c, shd, &sums[0]);
  const double need = (double)p.prac_rho * cand_mass;
  int first_reach = INT_MAX;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (x[e] != ~0ull && c[e] >= need && first_reach == INT_MAX) first_reach = tid * E + e;
  const int reach = block_min_int(first_reach, shi);
  const int n_pre = need <= 0.0 ? 0 : (reach == INT_MAX ? INT_MAX : reach + 1);

  // rerank the preselected blocks: key descending, ids ascending among equal keys
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (x[e] != ~0ull && tid * E + e < n_pre) {
      const int b = id_of(x[e]);
      x[e] = ((uint64_t)(~ordered_bits(rerank_key(bar_m[b], bar_I[b]))) << 32) | (uint64_t)(uint32_t)b;
    } else {
      x[e] = ~0ull;
    }
  }
  sort_blocked<E>(x, sh);

  // keep in that order while the pooled retained mass is below (1 - eps) of the total
  const double target = (1.0 - (double)p.tau[w.h0]) * tot_all;
  double incl[E];
#pragma unroll
  for (int e = 0; e < E; ++e) c[e] = incl[e] = x[e] == ~0ull ? 0.0 : (double)bar_m[id_of(x[e])];
  blocked_inclusive_scan<E>(incl, shd, &sums[0]);
  for (int b = tid; b < n_vis; b += kThrThreads) keep[b] = mandatory(b) ? 1 : 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double before = tot_mand + (incl[e] - c[e]);  // retained mass ahead of this position
    if (x[e] != ~0ull && before < target) keep[id_of(x[e])] = 1;
  }
  __syncthreads();

  if (p.row_bound) {  // per-row omitted mass of the final discard set
    float* rb = p.row_bound + ((int64_t)w.h0 * T + w.gtile) * S;
    for (int i0 = 0; i0 < s_t; i0 += kRowChunk) {
      double a[kRowChunk], d[kRowChunk], mine[kRowChunk];
#pragma unroll
      for (int r = 0; r < kRowChunk; ++r) a[r] = d[r] = 0.0;
      const int nr = min(kRowChunk, s_t - i0);
      for (int b = tid; b < n_vis; b += kThrThreads)
        if (!keep[b]) {
          float vm[kRowChunk];
          block_rows<STAGED>(st_m, w.Mb, w.bstride, S, b, i0, nr, vm);
#pragma unroll
          for (int r = 0; r < kRowChunk; ++r)
            if (r < nr) a[r] += (double)vm[r];
        }
#pragma unroll
      for (int r = 0; r < kRowChunk; ++r) mine[r] = a[r];
      block_excl_scan_vec<kRowChunk>(a, d, shd);
      if (tid == kThrThreads - 1)
        for (int r = 0; r < kRowChunk && i0 + r < s_t; ++r) rb[i0 + r] = (float)(a[r] + mine[r]);
      __syncthreads();
    }
    for (int i = s_t + tid; i < S; i += kThrThreads) rb[i] = -1.f;
  }

  // retained set, compacted in ascending id order
  const int E2 = (n_vis + kThrThreads - 1) / kThrThreads;
  int cnt = 0;
  for (int e = 0; e < E2; ++e) {
    const int b = tid * E2 + e;
    if (b < n_vis) cnt += keep[b];
  }
  int total;
  int off = block_excl_scan_int(cnt, total, shi);
  int32_t* out = p.slots + w.slot;
  for (int e = 0; e < E2; ++e) {
    const int b = tid * E2 + e;
    if (b < n_vis && keep[b]) out[off++] = b;
  }
  if (tid == 0) p.counts[w.h0 * T + w.gtile] = total;
}

// SMALL (staged only): the launch for tiles of at most kStageVis / 2 visible blocks,
// whose LDS is half the size, so twice as many workgroups share a CU; each launch
// skips the tiles of the other.
template <int MODE, bool STAGED, bool SMALL = false>
__global__ __launch_bounds__(kThrThreads) void sel_threshold_kernel(SelectParams p) {
  constexpr bool NEED_I = MODE != kSelectMass;  // the mass-only ranking reads m alone
  constexpr bool PRAC = MODE == kSelectPractical;
  static_assert(STAGED || !SMALL, "the small launch is staged");
  constexpr int VIS = SMALL ? kStageVis / 2 : kStageVis;     // staged blocks per tile
  constexpr int VALS = SMALL ? kStageVals / 2 : kStageVals;  // staged blocks x sampled rows
  constexpr int NK = STAGED ? VIS : kMaxVis;
  __shared__ uint64_t sh[NK];
  __shared__ uint8_t keep[NK];
  __shared__ __attribute__((aligned(16))) float st_I[STAGED && NEED_I ? VALS : 1];
  __shared__ float bar_I[PRAC ? NK : 1], bar_m[PRAC ? NK : 1];  // practical: pooled estimates
  __shared__ __attribute__((aligned(16))) float st_m[STAGED ? VALS : 1];
  __shared__ double shd[2 * kRowChunk * kThrWaves];
  __shared__ int shi[kThrWaves];
  const int tid = threadIdx.x;
  const int T = p.seqs.total_tiles;
  const int G = p.group_mode ? 1 : p.group;  // workgroups per (KV head, tile)
  const int xcd = blockIdx.x % kXcds, rest = blockIdx.x / kXcds;
  const int hg = rest % G;
  const int unit = (rest / G) * kXcds + xcd;  // gtile * hkv + KV head
  if (unit >= T * p.hkv) return;
  ThrTile w;
  w.gtile = unit / p.hkv;
  const int gk = unit % p.hkv;
  w.h0 = gk * p.group + hg;
  w.nh = p.group_mode ? p.group : 1;
  w.tau_group = p.group_mode ? p.group : 0;
  const int seq = find_seq(p.seqs, w.gtile);
  const int t = w.gtile - p.seqs.tile_start[seq];
  const int B = p.seqs.block;
  w.diag = p.seqs.diag0[seq] + t;
  w.n_vis = w.diag + 1;
  if constexpr (STAGED) {
    if ((w.n_vis <= kStageVis / 2 && w.n_vis * p.S <= kStageVals / 2) != SMALL) return;  // the other launch's tile
  }
  const int n_rows_t = min(B, p.seqs.n_q[seq] - t * B);
  w.S = p.S;
  w.s_t = min(p.S, n_rows_t);
  w.slot = (int64_t)w.h0 * p.seqs.vis_per_head + vis_offset(p.seqs, seq, t);
  const int cols = p.cols_rec;
  w.bstride = 2 * cols;  // floats per visible block
  // per-head lists: row i of head hg is column hg * S + i of the KV head's tile
  // record; shared lists: row i is column i
  w.Ib = p.blk_stats + ((int64_t)gk * p.seqs.vis_per_head + vis_offset(p.seqs, seq, t)) * w.bstride +
         (p.group_mode ? 0 : hg * w.S);
  w.Mb = w.Ib + cols;

  if constexpr (STAGED) {
    // the head's s_t values of I (not for the mass-only ranking) and m per visible block, read with every
    // load of a batch in flight before the first LDS store
    if (w.S % 4 == 0 && w.s_t % 4 == 0) {
      // 16-byte pieces: four rows of a block are adjacent in the record and in LDS
      const int q_per_blk = w.s_t / 4;
      const int per_tensor = w.n_vis * q_per_blk;
      const int total = NEED_I ? 2 * per_tensor : per_tensor;
      constexpr int BATCH = 8;
      for (int base = 0; base < total; base += BATCH * kThrThreads) {
        f32x4 val[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int idx = base + u * kThrThreads + tid;
          if (idx < total) {
            const bool is_m = !NEED_I || idx >= per_tensor;
            const int r = is_m && NEED_I ? idx - per_tensor : idx;
            const int b = r / q_per_blk, i = 4 * (r % q_per_blk);
            val[u] = *reinterpret_cast<const f32x4*>((is_m ? w.Mb : w.Ib) + (int64_t)b * w.bstride + i);
          }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int idx = base + u * kThrThreads + tid;
          if (idx < total) {
            const bool is_m = !NEED_I || idx >= per_tensor;
            const int r = is_m && NEED_I ? idx - per_tensor : idx;
            const int b = r / q_per_blk, i = 4 * (r % q_per_blk);
            *reinterpret_cast<f32x4*>((is_m ? st_m : st_I) + b * w.S + i) = val[u];
          }
        }
      }
    } else {
      const int per_tensor = w.n_vis * w.s_t;
      const int total = NEED_I ? 2 * per_tensor : per_tensor;
      constexpr int BATCH = 16;
      for (int base = 0; base < total; base += BATCH * kThrThreads) {
        float val[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int idx = base + u * kThrThreads + tid;
          val[u] = 0.f;
          if (idx < total) {
            const bool is_m = !NEED_I || idx >= per_tensor;
            const int r = is_m && NEED_I ? idx - per_tensor : idx;
            const int b = r / w.s_t, i = r % w.s_t;
            val[u] = (is_m ? w.Mb : w.Ib)[(int64_t)b * w.bstride + i];
          }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int idx = base + u * kThrThreads + tid;
          if (idx < total) {
            const bool is_m = !NEED_I || idx >= per_tensor;
            const int r = is_m && NEED_I ? idx - per_tensor : idx;
            const int b = r / w.s_t, i = r % w.s_t;
            (is_m ? st_m : st_I)[b * w.S + i] = val[u];
          }
        }
      }
    }
    __syncthreads();
  }
  int n_pad = kThrThreads;
  while (n_pad < w.n_vis) n_pad <<= 1;
  auto run = [&](auto e_tag) {
    constexpr int E = decltype(e_tag)::value;
    if constexpr (PRAC) practical_tile<STAGED, E>(p, w, st_I, st_m, bar_I, bar_m, sh, keep, shd, shi);
    else threshold_tile<MODE, STAGED, E>(p, w, st_I, st_m, sh, keep, shd, shi);
  };
  // keys per thread; staged tiles hold at most VIS blocks
  constexpr int EMAX = STAGED ? VIS / kThrThreads : kMaxVis / kThrThreads;
  switch (n_pad / kThrThreads) {
    case 1: run(IntTag<1>{}); break;
    case 2: if constexpr (EMAX >= 2) run(IntTag<2>{}); break;
    case 4: if constexpr (EMAX >= 4) run(IntTag<4>{}); break;
    case 8: if constexpr (EMAX >= 8) run(IntTag<8>{}); break;
    default: if constexpr (EMAX >= 16) run(IntTag<16>{}); break;
  }
}

// Exclusive scan of the per-row counts into row_ptr (one workgroup).
__global__ __launch_bounds__(1024) void csr_scan_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ row_ptr,
                                                      int rows) {
  // chunks of 1024 x 8 rows: each thread loads its 8 consecutive counts at once
  // (16-byte loads; counts sits 256-byte aligned in the workspace), one block scan per
  // chunk, a running carry between chunks, and independent stores (row_ptr is only
  // 4-byte aligned)
  constexpr int kPer = 8;
  __shared__ int sh[16];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < rows; base += 1024 * kPer) {
    const int r0 = base + tid * kPer;
    int c[kPer];
    if (r0 + kPer <= rows) {
#pragma unroll
      for (int q = 0; q < kPer / 4; ++q) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(counts + r0 + 4 * q);
#pragma unroll
        for (int j = 0; j < 4; ++j) c[4 * q + j] = (int)a[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) c[j] = r0 + j < rows ? counts[r0 + j] : 0;
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) s += c[j];
    int total;
    int off = carry + block_excl_scan_int(s, total, sh);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (r0 + j < rows) row_ptr[r0 + j] = off;
      off += c[j];
    }
    carry += total;
  }
  if (tid == 0) row_ptr[rows] = carry;
}

// Copy each row's ids from its slot to its CSR position.
__global__ __launch_bounds__(64) void csr_scatter_kernel(SelectParams p) {
  const int T = p.seqs.total_tiles;
  // heads of one tile are adjacent in the grid: they read the same workspace lines
  const int gtile = blockIdx.x / p.hq, h = blockIdx.x % p.hq;
  const int R = h * T + gtile;  // CSR row
  const int seq = find_seq(p.seqs, gtile);
  const int t = gtile - p.seqs.tile_start[seq];
  const int hs = p.group_mode ? (h / p.group) * p.group : h;  // a shared list lives in its first head's slot
  const int32_t* src = p.slots + (int64_t)hs * p.seqs.vis_per_head + vis_offset(p.seqs, seq, t);
  const int n = p.counts[R];
  int32_t* dst = p.block_idx + p.row_ptr[R];
  for (int i = threadIdx.x; i < n; i += 64) dst[i] = src[i];
}

// fp16 copy of V for pass 2 (bf16 inputs): one workgroup per (key block, KV head),
// KV head fastest. s_b = 2^(15 - e) with e the binary exponent of the block's largest
// |v| (|v| = f 2^e, f in [0.5, 1)), clamped to normal floats; a block that holds
// non-finite values keeps s_b = 1. Rows past the sequence end are not written (pass 2
// reads them as zeros).
constexpr int kV16Threads = 256;
template <int D, int BLK>
__global__ __launch_bounds__(kV16Threads) void v16_kernel(SelectParams p) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  constexpr int PER = BLK * CH / kV16Threads;
  static_assert(PER * kV16Threads == BLK * CH, "block must split evenly");
  __shared__ uint32_t red[kV16Threads / 64];
  const int tid = threadIdx.x;
  const int g = blockIdx.x % p.hkv, kb = blockIdx.x / p.hkv;
  int seq = 0, base = 0;
  while (seq + 1 < p.seqs.num_seqs && kb >= base + p.seqs.diag0[seq] + p.seqs.n_tiles[seq]) {
    base += p.seqs.diag0[seq] + p.seqs.n_tiles[seq];
    ++seq;
  }
  const int row0 = (kb - base) * BLK;
  const int rows = min(BLK, p.seqs.n_k[seq] - row0);
  const int64_t first = ((int64_t)p.seqs.k_start[seq] + row0) * p.hkv + g;  // row 0 of the block, in rows of D
  const uint16_t* src = reinterpret_cast<const uint16_t*>(p.v);
  u32x4 w[PER];
  uint32_t amax = 0;  // largest |v| as bf16 bits (ordered like the values)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * kV16Threads, r = c / CH, ch = c % CH;
    w[i] = u32x4{0u, 0u, 0u, 0u};
    if (r < rows) w[i] = *reinterpret_cast<const u32x4*>(src + (first + (int64_t)r * p.hkv) * D + ch * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = max(amax, max(w[i][e] & 0x7FFFu, (w[i][e] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int i = 1; i < kV16Threads / 64; ++i) amax = max(amax, red[i]);
  // biased exponent E of the largest |v|: |v| in [2^(E-127), 2^(E-126)), so e = E - 126
  const int E = (int)(amax >> 7);
  // s_b = 2^(15 - e) = 2^(141 - E); an all-zero block keeps s_b = 1, so the rescale of
  // pass 1's accumulator between neighbouring blocks stays within the fp32 range
  const int k = (E >= 255 || amax == 0) ? 0 : min(141 - E, 127);
  const float sb = __builtin_bit_cast(float, (uint32_t)(k + 127) << 23);
  uint16_t* dst = p.v16;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * kV16Threads, r = c / CH, ch = c % CH;
    if (r < rows) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 ab = {bf16_lo_to_f32(w[i][e]) * sb, bf16_hi_to_f32(w[i][e]) * sb};
        o[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(ab, f16x2));
      }
      *reinterpret_cast<u32x4*>(dst + (first + (int64_t)r * p.hkv) * D + ch * 8) = o;
    }
  }
  if (tid == 0) p.vscale[(int64_t)g * p.total_kb + kb] = sb;
}

// Pass 1 in chunks: 16 lanes per record column combine the chunks' sums into the
// record pass 2 reads. With M2 the largest chunk reference and f_k = 2^(m_k - M2):
// L_rest = sum_k l_k f_k and R = sum_k U_k f_k over every chunk's blocks after block 0,
// l = L_0 2^(u0_ref - M2) + L_rest, o = (U_0 2^(u0_ref - M2) + R) / l: the sums of the
// unsplit sweep, each chunk's rescaled once to the common reference. The mass-only
// sweeps, which do not split off block 0, leave L_0 = 0 and hold no vectors.
template <int D>
__global__ __launch_bounds__(256) void sel_merge_kernel(SelectParams p) {
  constexpr int kLanes = 16;  // lanes per record column: four columns per wave
  const int T = p.seqs.total_tiles;
  // (KV head * T + gtile) * cols_rec + col
  const int64_t rec = ((int64_t)blockIdx.x * 256 + threadIdx.x) / kLanes;
  const int l16 = threadIdx.x % kLanes;
  if (rec >= (int64_t)p.hkv * T * p.cols_rec) return;
  const int col = (int)(rec % p.cols_rec);
  const int gtile = (int)((rec / p.cols_rec) % T);
  const int seq = find_seq(p.seqs, gtile);
  const int t = gtile - p.seqs.tile_start[seq];
  const int B = p.seqs.block;
  const int s_t = min(p.S, min(B, p.seqs.n_q[seq] - t * B));
  const bool on = p.group_mode ? col < s_t : (col / p.S < p.group && col % p.S < s_t);
  if (!on) return;  // a column pass 1 did not write
  const int TG = p.tile_group;
  const int t_last = min((t / TG) * TG + TG - 1, p.seqs.n_tiles[seq] - 1);
  const int nblk = p.seqs.diag0[seq] + t_last + 1;
  const int nch = (nblk + p.p1_chunk_blocks - 1) / p.p1_chunk_blocks;  // chunks the group ran
  float* r = p.row_stats + rec * kRecordFloats<D>;
  const float* part = p.p1_part + rec * (int64_t)(p.p1_chunks - 1) * (D + 4);
  const float m0 = r[0], l0rest = r[1], u0_ref = r[2], L0 = r[3];
  // every chunk's (reference, weight sum), loaded together; unrolled so f stays in registers
  float mk[kPass1MaxChunks], lk[kPass1MaxChunks], f[kPass1MaxChunks];
#pragma unroll
  for (int k = 1; k < kPass1MaxChunks; ++k) {
    mk[k] = k < nch ? part[(k - 1) * (D + 4)] : -INFINITY;
    lk[k] = k < nch ? part[(k - 1) * (D + 4) + 1] : 0.f;
  }
  float M2 = m0;
#pragma unroll
  for (int k = 1; k < kPass1MaxChunks; ++k) M2 = fmaxf(M2, mk[k]);
  f[0] = __builtin_amdgcn_exp2f(m0 - M2);
  float l_rest = l0rest * f[0];
#pragma unroll
  for (int k = 1; k < kPass1MaxChunks; ++k) {
    f[k] = lk[k] > 0.f ? __builtin_amdgcn_exp2f(mk[k] - M2) : 0.f;
    l_rest += lk[k] * f[k];
  }
  const float fu = __builtin_amdgcn_exp2f(u0_ref - M2);
  const float l_all = L0 * fu + l_rest;
  const float r_coef = 1.f / l_all, u_coef = fu / l_all;
  const int dv = p.mode == kSelectMass ? 0 : D;
  for (int d = l16; d < dv; d += kLanes) {
    float R = r[4 + D + d] * f[0];
#pragma unroll
    for (int k = 1; k < kPass1MaxChunks; ++k)
      if (k < nch) R += part[(k - 1) * (D + 4) + 4 + d] * f[k];
    const float rn = R * r_coef;
    r[4 + d] = __builtin_fmaf(r[4 + d], u_coef, rn);
    r[4 + D + d] = rn;
  }
  if (l16 == 0) {  // after the column's lanes have read them (they run in one wave)
    r[0] = M2;
    r[1] = l_all;
    r[2] = l_rest / l_all;
  }
}

template <typename T, int D, int BLK>
static hipError_t launch_sel(const SelectParams& p, hipStream_t s) {
  constexpr int kSelWaves = sel_threads<T>() / 64;
  constexpr int kSelThreads = sel_threads<T>();
  const int TG = sel_tile_group(sizeof(T) == 2, p.cols_rec, p.group_mode, p.tiles_per_wave);
  int items = 0;
  for (int i = 0; i < p.seqs.num_seqs; ++i) items += (p.seqs.n_tiles[i] + TG - 1) / TG;
  const int64_t rows = (int64_t)p.hq * p.seqs.total_tiles;
  if (rows == 0) {
    hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, s, p.counts, p.row_ptr, 0);
    return hipGetLastError();
  }
  const bool mass = p.mode == kSelectMass;
  SelectParams pp = p;
  pp.tile_group = TG;
  pp.sweep_items = items;
  // pass 1 runs in the chunks the workspace was sized for, pass 2 in chunks of its own
  // choosing
  const SweepChunks c2 = sweep_chunks(p.seqs, p.hkv, TG, kMaxSeqBlocks, kPass2Workgroups);
  pp.p2_chunk_blocks = c2.blocks;
  pp.p2_chunks = c2.chunks;
  const unsigned grid1 = (unsigned)((int64_t)items * p.hkv * pp.p1_chunks);
  const unsigned grid2 = (unsigned)((int64_t)items * p.hkv * pp.p2_chunks);
  const int64_t recs = (int64_t)p.hkv * p.seqs.total_tiles * p.cols_rec;
  const dim3 merge_grid((unsigned)((recs + 15) / 16));
  if (mass) {
    hipLaunchKernelGGL((sel_sweep_kernel<T, D, BLK, false, true>), dim3(grid1), dim3(kSelThreads), 0, s, pp);
    if (pp.p1_chunks > 1) hipLaunchKernelGGL(sel_merge_kernel<D>, merge_grid, dim3(256), 0, s, pp);
    hipLaunchKernelGGL((sel_sweep_kernel<T, D, BLK, true, true>), dim3(grid2), dim3(kSelThreads), 0, s, pp);
  } else {
    hipLaunchKernelGGL((sel_sweep_kernel<T, D, BLK, false, false>), dim3(grid1), dim3(kSelThreads), 0, s, pp);
    if (pp.p1_chunks > 1) hipLaunchKernelGGL(sel_merge_kernel<D>, merge_grid, dim3(256), 0, s, pp);
    if (sizeof(T) == 2 && p.total_kb > 0)  // the fp16 copy of V that pass 2 reads (bf16 inputs)
      hipLaunchKernelGGL((v16_kernel<D, BLK>), dim3((unsigned)((int64_t)p.total_kb * p.hkv)), dim3(kV16Threads), 0, s,
                         p);
    hipLaunchKernelGGL((sel_sweep_kernel<T, D, BLK, true, false>), dim3(grid2), dim3(kSelThreads), 0, s, pp);
  }
  // threshold grid: (KV-head unit, head in group) with the unit's XCD kept fixed
  const int64_t units = (int64_t)p.seqs.total_tiles * p.hkv;
  const unsigned tgrid = (unsigned)(((units + kXcds - 1) / kXcds) * kXcds * (p.group_mode ? 1 : p.group));
  const bool staged = p.max_vis <= kStageVis && (int64_t)p.max_vis * p.S <= kStageVals;
  // staged: the tiles of at most half the staging size in a launch of their own with half
  // the LDS (twice the workgroups per CU), then the others
  auto thr = [&](auto mode_tag) {
    constexpr int M = decltype(mode_tag)::value;
    if (staged) {
      hipLaunchKernelGGL((sel_threshold_kernel<M, true, true>), dim3(tgrid), dim3(kThrThreads), 0, s, p);
      hipLaunchKernelGGL((sel_threshold_kernel<M, true, false>), dim3(tgrid), dim3(kThrThreads), 0, s, p);
    } else {
      hipLaunchKernelGGL((sel_threshold_kernel<M, false>), dim3(tgrid), dim3(kThrThreads), 0, s, p);
    }
  };
  if (mass) thr(IntTag<kSelectMass>{});
  else if (p.mode == kSelectPractical) thr(IntTag<kSelectPractical>{});
  else thr(IntTag<kSelectOutputRelative>{});
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, s, p.counts, p.row_ptr, (int)rows);
  hipLaunchKernelGGL(csr_scatter_kernel, dim3((unsigned)rows), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_sel_b(const SelectParams& p, int block, hipStream_t s) {
  return block == 64 ? launch_sel<T, D, 64>(p, s) : launch_sel<T, D, 128>(p, s);
}

template <typename T>
static hipError_t launch_sel_d(const SelectParams& p, int d, int block, hipStream_t s) {
  return d == 64 ? launch_sel_b<T, 64>(p, block, s) : launch_sel_b<T, 128>(p, block, s);
}

hipError_t launch_select(const SelectParams& p, int in_dtype, int head_dim, int block, hipStream_t stream) {
  return in_dtype == 0 ? launch_sel_d<uint16_t>(p, head_dim, block, stream)
                       : launch_sel_d<float>(p, head_dim, block, stream);
}

}  // namespace poem
