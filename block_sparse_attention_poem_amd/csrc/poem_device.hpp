// Device building blocks shared by the attention and selector sweeps (gfx950).
//
// A "sweep" walks key blocks of one sequence/KV head in 64-key stages. Each stage
// is staged global -> registers -> LDS by the whole workgroup (K row-major, V
// transposed so that PV operands are 16-byte LDS reads), double-buffered with one
// barrier per stage. Every wave owns 32 query columns and runs 32x32 MFMAs:
//   S^T[key][col]  = K[key][:] . Q[col][:]        (A = K from LDS, B = Q in registers)
//   O^T[d][col]   += V^T[d][key] . P^T[key][col]   (A = V^T from LDS, B = P in registers)
// Computing the transposes keeps every per-column quantity (max, sum, scale) in one
// lane pair (l, l^32), and lets the fp32 scores become PV operands without shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poem {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxSeqs = 64;
constexpr int kStageKeys = 64;  // keys per LDS stage
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Per-sequence geometry, passed by value in kernel arguments (no device tables).
struct SeqTable {
  int32_t num_seqs;
  int32_t total_tiles;
  int32_t block;        // B
  int32_t q_start[kMaxSeqs];   // first packed query row
  int32_t k_start[kMaxSeqs];   // first packed key row
  int32_t n_q[kMaxSeqs];
  int32_t n_k[kMaxSeqs];
  int32_t n_tiles[kMaxSeqs];
  int32_t tile_start[kMaxSeqs];  // first global tile
  int32_t diag0[kMaxSeqs];       // (N_k - N_q) / B
  int64_t vis_start[kMaxSeqs];   // per head: visible (tile, block) pairs of earlier sequences
  int64_t vis_per_head;          // per head: all visible (tile, block) pairs
};

// Visible (tile, block) pairs before tile t of sequence s, per head.
__host__ __device__ __forceinline__ int64_t vis_offset(const SeqTable& st, int s, int t) {
  const int64_t d0 = st.diag0[s];
  return st.vis_start[s] + (int64_t)t * (d0 + 1) + (int64_t)t * (t - 1) / 2;
}

// Items of TG consecutive tiles per sequence, ranked by the diagonal block of their
// first tile, descending (ties: lower sequence first). Longest work goes first.
// Returns the sequence and the first tile of the rank-th item.
__host__ __device__ __forceinline__ void rank_to_item(const SeqTable& st, int TG, int rank, int& seq, int& tile0) {
  auto items = [&](int s) { return (st.n_tiles[s] + TG - 1) / TG; };
  auto count_ge = [&](int x) {  // items whose key >= x
    int c = 0;
    for (int s = 0; s < st.num_seqs; ++s) {
      int n = items(s);
      int need = x - st.diag0[s];  // key = diag0 + TG * i >= x  <=>  i >= ceil(need / TG)
      int first = need <= 0 ? 0 : (need + TG - 1) / TG;
      c += first >= n ? 0 : n - first;
    }
    return c;
  };
  int lo = 0, hi = 0;
  for (int s = 0; s < st.num_seqs; ++s) {
    int n = items(s);
    if (n > 0) hi = max(hi, st.diag0[s] + TG * (n - 1));
  }
  // largest x in [0, hi] with count_ge(x) > rank
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (count_ge(mid) > rank) lo = mid; else hi = mid - 1;
  }
  int r = rank - count_ge(lo + 1);
  seq = -1;
  tile0 = 0;
  for (int s = 0; s < st.num_seqs; ++s) {
    int n = items(s);
    int off = lo - st.diag0[s];
    if (n > 0 && off >= 0 && off % TG == 0 && off / TG < n) {
      if (r == 0) { seq = s; tile0 = off; return; }
      --r;
    }
  }
}

// Sequence holding global tile gtile.
__host__ __device__ __forceinline__ int find_seq(const SeqTable& st, int gtile) {
  int s = 0;
  while (s + 1 < st.num_seqs && st.tile_start[s + 1] <= gtile) ++s;
  return s;
}

// Exclusive prefix sum over the workgroup in thread order; total receives the sum.
// sh holds one int per wave.
__device__ __forceinline__ int block_excl_scan_int(int a, int& total, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ia = a;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int ta = __shfl_up(ia, o);
    if (lane >= o) ia += ta;
  }
  if (lane == 63) sh[wave] = ia;
  __syncthreads();
  int off = 0;
  total = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wave) off += sh[w];
    total += sh[w];
  }
  __syncthreads();
  return off + ia - a;
}

// Key position inside a 16-key group of the transposed-V LDS rows: bits 2 and 3 of
// the key swapped. It places the keys a lane group holds in one PV k-step next to
// each other, so each PV operand is one contiguous LDS read.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <typename T> struct ElemTraits;
template <> struct ElemTraits<uint16_t> { static constexpr int bytes = 2; };
template <> struct ElemTraits<float> { static constexpr int bytes = 4; };

// LDS stage geometry for element type T and head dim D with NT threads.
template <typename T, int D, int NT>
struct Stage {
  static constexpr int EB = ElemTraits<T>::bytes;
  static constexpr int K_STRIDE = D * EB + 16;              // bytes per K row (16-byte pad)
  static constexpr int V_STRIDE = kStageKeys * EB + 16;     // bytes per V^T row
  static constexpr int K_BYTES = kStageKeys * K_STRIDE;
  static constexpr int V_BYTES = D * V_STRIDE;
  static constexpr int BYTES = K_BYTES + V_BYTES;
  static constexpr int CH_PER_ROW = D * EB / 16;            // 16-byte chunks per key row
  static constexpr int K_CHUNKS = kStageKeys * CH_PER_ROW;
  static constexpr int K_ITERS = (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_UNITS = (kStageKeys / 4) * CH_PER_ROW;  // 4 keys x 16 bytes
  static constexpr int V_ITERS = (V_UNITS + NT - 1) / NT;

  struct Regs {
    u32x4 k[K_ITERS];
    u32x4 v[V_ITERS][4];
  };

  // Global -> registers for keys [key0, key0 + 64) of one KV head (K and V bases point
  // at key 0 of the sequence for that head). Keys at or past n_valid read as zero.
  // row_stride is the element stride between consecutive keys.
  static __device__ __forceinline__ void load(Regs& r, const T* __restrict__ kbase, const T* __restrict__ vbase,
                                              int64_t row_stride, int key0, int n_valid, int tid) {
    const char* b = reinterpret_cast<const char*>(kbase);
    const char* bv = reinterpret_cast<const char*>(vbase);
#pragma unroll
    for (int i = 0; i < K_ITERS; ++i) {
      int c = tid + i * NT;
      r.k[i] = u32x4{0, 0, 0, 0};
      if (c < K_CHUNKS) {
        int key = c / CH_PER_ROW, ch = c % CH_PER_ROW;
        if (key0 + key < n_valid)
          r.k[i] = *reinterpret_cast<const u32x4*>(b + ((int64_t)(key0 + key) * row_stride) * EB + ch * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < V_ITERS; ++i) {
      int u = tid + i * NT;
#pragma unroll
      for (int j = 0; j < 4; ++j) r.v[i][j] = u32x4{0, 0, 0, 0};
      if (u < V_UNITS) {
        const int kq = u % (kStageKeys / 4), ch = u / (kStageKeys / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int key = key0 + 4 * kq + j;
          if (key < n_valid)
            r.v[i][j] = *reinterpret_cast<const u32x4*>(bv + ((int64_t)key * row_stride) * EB + ch * 16);
        }
      }
    }
  }

  // Registers -> LDS stage. K rows as they are; V transposed to V^T[d][vt_pos(key)].
  static __device__ __forceinline__ void store(const Regs& r, char* lds, int tid) {
#pragma unroll
    for (int i = 0; i < K_ITERS; ++i) {
      int c = tid + i * NT;
      if (c < K_CHUNKS) {
        int key = c / CH_PER_ROW, ch = c % CH_PER_ROW;
        *reinterpret_cast<u32x4*>(lds + key * K_STRIDE + ch * 16) = r.k[i];
      }
    }
    char* vt = lds + K_BYTES;
#pragma unroll
    for (int i = 0; i < V_ITERS; ++i) {
      int u = tid + i * NT;
      if (u < V_UNITS) {
        // consecutive lanes take consecutive key quads of one d-chunk, so the 16 lanes
        // that write one V^T row together cover its 128 bytes without bank conflicts
        const int kq = u % (kStageKeys / 4), ch = u / (kStageKeys / 4);
        const int pos = vt_pos(4 * kq);  // keys 4kq .. 4kq+3 stay contiguous
        if constexpr (EB == 2) {
          // 4 keys x 8 d (bf16) -> 8 rows of V^T, 4 keys (8 bytes) each
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            uint32_t a0 = r.v[i][0][c], a1 = r.v[i][1][c], a2 = r.v[i][2][c], a3 = r.v[i][3][c];
            u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
            u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
            int d = ch * 8 + 2 * c;
            *reinterpret_cast<u32x2*>(vt + d * V_STRIDE + pos * 2) = lo;
            *reinterpret_cast<u32x2*>(vt + (d + 1) * V_STRIDE + pos * 2) = hi;
          }
        } else {
          // 4 keys x 4 d (fp32) -> 4 rows of V^T, 4 keys (16 bytes) each
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x4 w = {r.v[i][0][c], r.v[i][1][c], r.v[i][2][c], r.v[i][3][c]};
            int d = ch * 4 + c;
            *reinterpret_cast<u32x4*>(vt + d * V_STRIDE + pos * 4) = w;
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA fragments. Lane l: column j = l % 32, lane group g = l / 32.
// 32x32 accumulator register r holds row 8*(r/4) + 4*g + r%4 of column j.
// ---------------------------------------------------------------------------

// Q (B operand of S^T = K Q^T) for 32 columns. bf16: 16-d steps, lane group g
// holds d = 16s + 8g .. +7. fp32: 2-d steps, lane group g holds d = (D/2) g + s.
template <typename T, int D> struct QFrag;
template <int D> struct QFrag<uint16_t, D> {
  static constexpr int STEPS = D / 16;
  bf16x8 q[STEPS];
  __device__ __forceinline__ void load(const uint16_t* row, bool valid, int g) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      u32x4 w = {0, 0, 0, 0};
      if (valid) w = *reinterpret_cast<const u32x4*>(row + 16 * s + 8 * g);
      q[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
};
template <int D> struct QFrag<float, D> {
  static constexpr int STEPS = D / 2;
  float q[STEPS];
  __device__ __forceinline__ void load(const float* row, bool valid, int g) {
#pragma unroll
    for (int s4 = 0; s4 < STEPS / 4; ++s4) {
      f32x4 w = {0.f, 0.f, 0.f, 0.f};
      if (valid) w = *reinterpret_cast<const f32x4*>(row + (D / 2) * g + 4 * s4);
      q[4 * s4 + 0] = w[0]; q[4 * s4 + 1] = w[1]; q[4 * s4 + 2] = w[2]; q[4 * s4 + 3] = w[3];
    }
  }
};

// S^T for one 32-key tile kt of the LDS stage: acc = K[32kt + i][:] . Q[:][j].
template <typename T, int D, int K_STRIDE>
__device__ __forceinline__ f32x16 qk_tile(const char* klds, const QFrag<T, D>& qf, int kt, int lane) {
  f32x16 acc = {};
  const int i = lane & 31, g = lane >> 5;
  const char* rowp = klds + (32 * kt + i) * K_STRIDE;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int s = 0; s < QFrag<T, D>::STEPS; ++s) {
      bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(rowp + (16 * s + 8 * g) * 2));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.q[s], acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int s4 = 0; s4 < D / 8; ++s4) {
      f32x4 a = *reinterpret_cast<const f32x4*>(rowp + ((D / 2) * g + 4 * s4) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf.q[4 * s4 + e], acc, 0, 0, 0);
    }
  }
  return acc;
}

// Key (0..63 inside the stage) of accumulator register r of key tile kt for lane group g.
__device__ __forceinline__ int acc_key(int kt, int r, int g) {
  return 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
}

// bf16 pack of two floats, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// O^T[dt] += V^T[32dt + i][keys] . P^T[keys][j] over the 64 keys of the stage.
// p holds the probabilities in the S^T accumulator layout (two key tiles).
// SPLIT (bf16 only) adds a second MFMA with the bf16 rounding residual of P.
template <typename T, int D, int V_STRIDE, bool SPLIT>
__device__ __forceinline__ void pv_stage(const char* vt, const f32x16 (&p)[2], f32x16* O, int lane) {
  const int i = lane & 31, g = lane >> 5;
  if constexpr (sizeof(T) == 2) {
    bf16x8 ph[4], pl[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kt = s >> 1, r0 = 8 * (s & 1);
      u32x4 w, wl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = p[kt][r0 + 2 * e], b = p[kt][r0 + 2 * e + 1];
        w[e] = pack_bf16(a, b);
        if constexpr (SPLIT) wl[e] = pack_bf16(a - bf16_lo_to_f32(w[e]), b - bf16_hi_to_f32(w[e]));
      }
      ph[s] = __builtin_bit_cast(bf16x8, w);
      if constexpr (SPLIT) pl[s] = __builtin_bit_cast(bf16x8, wl);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const char* rowp = vt + (32 * dt + i) * V_STRIDE;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(rowp + (16 * s + 8 * g) * 2));
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ph[s], O[dt], 0, 0, 0);
        if constexpr (SPLIT) O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pl[s], O[dt], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const char* rowp = vt + (32 * dt + i) * V_STRIDE;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          // registers r = 4*q4 .. 4*q4+3 sit at positions 32kt + 8g + r + 8*(r>>3)
          const int r0 = 4 * q4;
          f32x4 a = *reinterpret_cast<const f32x4*>(rowp + (32 * kt + 8 * g + r0 + 8 * (r0 >> 3)) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            O[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], p[kt][r0 + e], O[dt], 0, 0, 0);
        }
      }
    }
  }
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32); }

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima). Issued once after the
// per-column loads that precede a sweep: otherwise those loads stay "pending" at the
// loop header on some path and every iteration waits for its own K/V prefetch too.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace poem
