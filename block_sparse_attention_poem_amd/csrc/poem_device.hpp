// Device building blocks shared by the attention and selector sweeps (gfx950).
//
// A "sweep" walks key blocks of one sequence/KV head in 64-key stages, double-
// buffered in LDS with one barrier per stage. Every wave owns 32 query columns and
// runs 32x32 MFMAs:
//   S^T[key][col]  = K[key][:] . Q[col][:]        (A = K from LDS, B = Q in registers)
//   O^T[d][col]   += V^T[d][key] . P^T[key][col]   (A = V^T from LDS, B = P in registers)
// Computing the transposes keeps every per-column quantity (max, sum, scale) in one
// lane pair (l, l^32), and lets the fp32 scores become PV operands without shuffles.
//
// bf16 stages are filled by direct global->LDS loads (no registers, no LDS stores)
// into unpadded row-major K and V whose 16-byte chunks are XOR-swizzled per row; the
// PV operand V^T is read with the transposing LDS load. fp32 stages go through
// registers and store V transposed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poem {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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

// Key blocks of the sequences before s (a sequence has diag0 + n_tiles of them).
__host__ __device__ __forceinline__ int kblocks_before(const SeqTable& st, int s) {
  int n = 0;
  for (int i = 0; i < s; ++i) n += st.diag0[i] + st.n_tiles[i];
  return n;
}

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


template <typename T> struct ElemTraits;
template <> struct ElemTraits<uint16_t> { static constexpr int bytes = 2; };
template <> struct ElemTraits<float> { static constexpr int bytes = 4; };

typedef __attribute__((address_space(3))) char lds_char;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Q fragments (B operand of S^T = K Q^T) for 32 columns. Lane l: column j = l % 32,
// lane group g = l / 32. bf16: 16-d steps, lane group g holds d = 16s + 8g .. +7.
// fp32: 2-d steps, lane group g holds d = (D/2) g + s.
// 32x32 accumulator register r holds row 8*(r/4) + 4*g + r%4 of column j.
// ---------------------------------------------------------------------------
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

// Key (0..63 inside the stage) of accumulator register r of key tile kt for lane group g.
__device__ __forceinline__ int acc_key(int kt, int r, int g) {
  return 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
}

// bf16 pack of two floats, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// acc + the sum of the eight bf16 values of p (four v_dot2 with (1, 1); products exact).
// The pairs are taken with shufflevector: bit-casting 32-bit words of the packed
// vector to bf16x2 made the compiler feed the first word to all four dot products.
__device__ __forceinline__ float row_sum_bf16(const bf16x8& p, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
  return acc;
}
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// P operand of one 16-key PV step s (bf16): registers 8(s&1) .. +7 of key tile s/2.
// Lane group g then holds keys 16s + 4g + 0..3 (elements 0..3) and 16s + 8 + 4g + 0..3
// (elements 4..7). With SPLIT the bf16 rounding residual is packed into lo.
template <bool SPLIT>
__device__ __forceinline__ void p_step(const f32x16 (&p)[2], int s, bf16x8& hi, bf16x8& lo) {
  const int kt = s >> 1, r0 = 8 * (s & 1);
  u32x4 w, wl;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = p[kt][r0 + 2 * e], b = p[kt][r0 + 2 * e + 1];
    w[e] = pack_bf16(a, b);
    if constexpr (SPLIT) wl[e] = pack_bf16(a - bf16_lo_to_f32(w[e]), b - bf16_hi_to_f32(w[e]));
  }
  hi = __builtin_bit_cast(bf16x8, w);
  if constexpr (SPLIT) lo = __builtin_bit_cast(bf16x8, wl);
}

// One 16-key step of fp32 weights as fp16 (round to nearest even), in the operand
// layout of p_step.
__device__ __forceinline__ f16x8 p_step_f16(const f32x16 (&p)[2], int s) {
  const int kt = s >> 1, r0 = 8 * (s & 1);
  f16x8 h;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2 ab = {p[kt][r0 + 2 * e], p[kt][r0 + 2 * e + 1]};
    const f16x2 w = __builtin_convertvector(ab, f16x2);
    h[2 * e] = w[0];
    h[2 * e + 1] = w[1];
  }
  return h;
}

// Sum of the eight fp16 weights of a packed step, added to acc in fp32.
__device__ __forceinline__ float row_sum_f16(const f16x8& p, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
}

// ---------------------------------------------------------------------------
// bf16 stage: 64 keys of K then 64 keys of V, each row-major [key][D] (no padding).
// Chunk c (16 bytes) of row r sits at chunk position c ^ swizzle(r): the K swizzle
// spreads the 16 rows that 16 lanes read together for QK over all banks; the V
// swizzle does the same for the 4 rows x 4 chunks one transposing read touches per
// 32 lanes. Rows past the sequence end read as zeros (their scores are masked).
// ---------------------------------------------------------------------------
template <int D, int NT>
struct StageB16 {
  static constexpr int ROW = D * 2;
  static constexpr int CH = D / 8;  // 16-byte chunks per row
  static constexpr int TENSOR = kStageKeys * ROW;
  static constexpr int BYTES = 2 * TENSOR;
  static constexpr int WAVES = NT / 64;
  static constexpr int INSTR = TENSOR / 1024;  // 1 KB per wave-wide direct load
  static_assert(INSTR % WAVES == 0, "stage must split evenly over the waves");
  struct Regs {};

  static __device__ __forceinline__ int kswz(int r) { return r & (CH - 1); }
  static __device__ __forceinline__ int vswz(int r) {
    return CH >= 16 ? (2 * (r & 3) + 8 * (r & 1)) : (2 * (r & 3));
  }

  // Buffer descriptors start at the stage's first key and cover only the valid keys,
  // so rows past the sequence end load as zeros; the per-lane offsets do not depend
  // on the stage and all stage-dependent addressing stays in scalar registers.
  // Per-lane byte offsets of the direct loads. One wave-wide load covers RPI whole
  // rows: lane l takes chunk l % CH of row RPI * blk + l / CH. Every swizzle above only
  // sees the low bits of the row, which the wave's first row (a multiple of RPI) leaves
  // to the lane's own l / CH, plus, for K when RPI < CH, a part that depends on blk.
  // When that part is the same for all of a wave's loads (RPI * WAVES a multiple of CH)
  // the whole per-lane offset is fixed for the sweep and each load adds only a scalar.
  static constexpr uint32_t RPI = 1024 / ROW;
  static_assert(RPI % 4 == 0 && RPI <= CH, "row groups must keep the swizzle bits lane-local");
  static constexpr bool K_FIXED = (RPI * WAVES) % CH == 0;
  struct LaneOffsets {
    uint32_t k, v;
  };
  static __device__ __forceinline__ uint32_t lane_off(uint32_t row_bytes, uint32_t lane, uint32_t r0, bool is_v) {
    const uint32_t lr = lane / CH, pos = lane % CH;
    const uint32_t sw = is_v ? (uint32_t)vswz(lr) : ((r0 & (CH - 1)) | lr);
    return lr * row_bytes + ((pos ^ sw) << 4);
  }
  static __device__ __forceinline__ LaneOffsets lane_offsets(int64_t row_stride, int tid) {
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = (uint32_t)tid & 63u;
    const uint32_t row_bytes = (uint32_t)(row_stride * 2);
    return {lane_off(row_bytes, lane, RPI * wave, false), lane_off(row_bytes, lane, 0, true)};
  }

  template <bool IS_V>
  static __device__ __forceinline__ void load_one(const uint16_t* __restrict__ base_ptr, int64_t row_stride,
                                                  int key0, int n_valid, int tid, char* dst,
                                                  const LaneOffsets& lo) {
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lane = (uint32_t)tid & 63u;
    const uint32_t row_bytes = (uint32_t)(row_stride * 2);
    // Valid rows of the stage, clamped to [0, kStageKeys] with scalar instructions: the
    // empty statement between the two clamps keeps them from fusing into a vector med3.
    // Uniform by construction; the "s" constraint keeps the value in a scalar register.
    int rows = n_valid - key0;
    rows = rows < kStageKeys ? rows : kStageKeys;
    __asm__("" : "+s"(rows));
    rows = rows > 0 ? rows : 0;
    const int records = rows * (int)row_bytes;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(base_ptr) + (int64_t)key0 * row_stride * 2), (short)0, records,
        0x00020000);
#pragma unroll
    for (int j = 0; j < INSTR / WAVES; ++j) {
      const uint32_t blk = j * WAVES + wave;
      const uint32_t r0 = RPI * blk;  // uniform
      uint32_t off;
      if constexpr (IS_V) off = lo.v;
      else if constexpr (K_FIXED) off = lo.k;
      else off = lane_off(row_bytes, lane, r0, false);
      // the row group's byte offset goes in the scalar offset (it counts toward the
      // range check like the lane's vector offset), so no vector add per load
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_char*)(dst + blk * 1024), 16, (int)off,
                                               (int)(r0 * row_bytes), 0, 0);
    }
  }
  static __device__ __forceinline__ void load_k(const uint16_t* kbase, int64_t row_stride, int key0, int n_valid,
                                                int tid, char* kbuf, const LaneOffsets& lo) {
    load_one<false>(kbase, row_stride, key0, n_valid, tid, kbuf, lo);
  }
  static __device__ __forceinline__ void load_v(const uint16_t* vbase, int64_t row_stride, int key0, int n_valid,
                                                int tid, char* vbuf, const LaneOffsets& lo) {
    load_one<true>(vbase, row_stride, key0, n_valid, tid, vbuf, lo);
  }
  static __device__ __forceinline__ void load_k(const uint16_t* kbase, int64_t row_stride, int key0, int n_valid,
                                                int tid, char* kbuf) {
    load_k(kbase, row_stride, key0, n_valid, tid, kbuf, lane_offsets(row_stride, tid));
  }
  static __device__ __forceinline__ void load_v(const uint16_t* vbase, int64_t row_stride, int key0, int n_valid,
                                                int tid, char* vbuf) {
    load_v(vbase, row_stride, key0, n_valid, tid, vbuf, lane_offsets(row_stride, tid));
  }
  // both tensors of a stage into one buffer: K, then V at +TENSOR
  static __device__ __forceinline__ void load(Regs&, const uint16_t* __restrict__ kbase,
                                              const uint16_t* __restrict__ vbase, int64_t row_stride, int key0,
                                              int n_valid, int tid, char* lds) {
    load_k(kbase, row_stride, key0, n_valid, tid, lds);
    load_v(vbase, row_stride, key0, n_valid, tid, lds + TENSOR);
  }
  static __device__ __forceinline__ void store(const Regs&, char*, int) {}
  // the direct loads write LDS asynchronously: wait for this wave's before the barrier
  static constexpr bool ASYNC = true;

  // Per-lane byte offsets of the QK^T K operands within a K buffer, one per d step s:
  // row lane % 32, chunk (2s + lane / 32) ^ swizzle. Key tile kt adds 32 rows, which
  // leaves the swizzle unchanged. The empty statements make the offsets opaque, so the
  // compiler keeps them whole and folds each buffer's fixed LDS address into the
  // read's immediate offset instead of re-adding it every stage.
  struct KOffsets {
    uint32_t o[D / 16];
  };
  static __device__ __forceinline__ KOffsets k_offsets(int lane) {
    KOffsets ko;
    const int r = lane & 31, g = (lane >> 5) & 1;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      ko.o[st] = (uint32_t)(r * ROW + (((2 * st + g) ^ kswz(r)) << 4));
      __asm__ volatile("" : "+v"(ko.o[st]));
    }
    return ko;
  }
  static __device__ __forceinline__ bf16x8 k_frag(const char* kbuf, const KOffsets& ko, int kt, int st) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kbuf + 32 * kt * ROW + ko.o[st]));
  }

  // S^T for 32-key tile kt: acc = K[32kt + i][:] . Q[:][j]
  static __device__ __forceinline__ f32x16 qk_tile(const char* lds, const QFrag<uint16_t, D>& qf, int kt, int lane) {
    f32x16 acc = {};
    const int r = 32 * kt + (lane & 31), g = lane >> 5;
    const char* rowp = lds + r * ROW;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 a =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(rowp + ((2 * s + g) ^ kswz(r)) * 16));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.q[s], acc, 0, 0, 0);
    }
    return acc;
  }

  // V^T operand of d-tile dt, key step s: lane l gets d = 32dt + l%32 and the keys its
  // lane group's P elements hold (16s + 4g + 0..3, then 16s + 8 + 4g + 0..3). In each
  // group of 16 lanes the transposing read hands lane i element (i & 3) of the 8 bytes
  // addressed by lane 4e + (i >> 2), as its element e; so lane 4e + k addresses key
  // base + e, d = 16-column base + 4k.
  static __device__ __forceinline__ bf16x8 v_frag(const char* vt, int dt, int s, int lane) {
    const int q = lane >> 4, i = lane & 15, g = q >> 1;
    const int d = 32 * dt + 16 * (q & 1) + 4 * (i & 3);
    const int c = d >> 3, half = (d >> 2) & 1;
    const int r0 = 16 * s + 4 * g + (i >> 2), r1 = r0 + 8;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4i16 __attribute__((address_space(3)))*)(vt + r0 * ROW + (c ^ vswz(r0)) * 16 + half * 8));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4i16 __attribute__((address_space(3)))*)(vt + r1 * ROW + (c ^ vswz(r1)) * 16 + half * 8));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, ab);
  }

  // O^T[dt] += V^T . P^T with P already packed to bf16 (one operand per 16-key step).
  static __device__ __forceinline__ void pv_packed(const char* vbuf, const bf16x8 (&P)[4], f32x16* O, int lane) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(vbuf, dt, s, lane), P[s], O[dt], 0, 0, 0);
  }

  // O^T[dt] += V^T . P^T over the stage's 64 keys, one 16-key step at a time.
  template <bool SPLIT>
  static __device__ __forceinline__ void pv(const char* lds, const f32x16 (&p)[2], f32x16* O, int lane) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 ph, pl;
      p_step<SPLIT>(p, s, ph, pl);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8 a = v_frag(lds + TENSOR, dt, s, lane);
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ph, O[dt], 0, 0, 0);
        if constexpr (SPLIT) O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pl, O[dt], 0, 0, 0);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// fp32 stage: registers -> LDS. K row-major with a 16-byte pad per row; V stored
// transposed, V^T[d][vt_pos(key)], where vt_pos swaps bits 2 and 3 of the key so
// the keys a lane group holds in one PV step sit together.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D, int NT>
struct StageF32 {
  static constexpr int EB = 4;
  static constexpr int K_STRIDE = D * EB + 16;
  static constexpr int V_STRIDE = kStageKeys * EB + 16;
  static constexpr int K_BYTES = kStageKeys * K_STRIDE;
  static constexpr int V_BYTES = D * V_STRIDE;
  static constexpr int BYTES = K_BYTES + V_BYTES;
  static constexpr int CH_PER_ROW = D * EB / 16;
  static constexpr int K_CHUNKS = kStageKeys * CH_PER_ROW;
  static constexpr int K_ITERS = (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_UNITS = (kStageKeys / 4) * CH_PER_ROW;  // 4 keys x 16 bytes
  static constexpr int V_ITERS = (V_UNITS + NT - 1) / NT;
  static constexpr bool ASYNC = false;
  struct KOffsets {};  // the fp32 stage reads its K operands through qk_tile only
  static __device__ __forceinline__ KOffsets k_offsets(int) { return {}; }

  struct Regs {
    u32x4 k[K_ITERS];
    u32x4 v[V_ITERS][4];
  };

  static __device__ __forceinline__ void load(Regs& r, const float* __restrict__ kbase, const float* __restrict__ vbase,
                                              int64_t row_stride, int key0, int n_valid, int tid, char*) {
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

  // consecutive lanes take consecutive key quads of one d-chunk, so the 16 lanes
  // that write one V^T row together cover it without bank conflicts
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
        const int kq = u % (kStageKeys / 4), ch = u / (kStageKeys / 4);
        const int pos = vt_pos(4 * kq);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4 w = {r.v[i][0][c], r.v[i][1][c], r.v[i][2][c], r.v[i][3][c]};
          *reinterpret_cast<u32x4*>(vt + (ch * 4 + c) * V_STRIDE + pos * 4) = w;
        }
      }
    }
  }

  static __device__ __forceinline__ f32x16 qk_tile(const char* lds, const QFrag<float, D>& qf, int kt, int lane) {
    f32x16 acc = {};
    const int i = lane & 31, g = lane >> 5;
    const char* rowp = lds + (32 * kt + i) * K_STRIDE;
#pragma unroll
    for (int s4 = 0; s4 < D / 8; ++s4) {
      f32x4 a = *reinterpret_cast<const f32x4*>(rowp + ((D / 2) * g + 4 * s4) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf.q[4 * s4 + e], acc, 0, 0, 0);
    }
    return acc;
  }

  template <bool SPLIT>
  static __device__ __forceinline__ void pv(const char* lds, const f32x16 (&p)[2], f32x16* O, int lane) {
    const int i = lane & 31, g = lane >> 5;
    const char* vt = lds + K_BYTES;
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
};

template <typename T, int D, int NT> struct StageSel;
template <int D, int NT> struct StageSel<uint16_t, D, NT> { using type = StageB16<D, NT>; };
template <int D, int NT> struct StageSel<float, D, NT> { using type = StageF32<D, NT>; };
template <typename T, int D, int NT> using Stage = typename StageSel<T, D, NT>::type;

// Lanes l and l ^ 32 hold the two halves of one accumulator column. half_sum and
// half_max combine them with one v_permlane32_swap (a VALU lane swap between the wave's
// halves) instead of an LDS permute and its wait. With a = b = x the swap leaves
// a = x[l & 31] and b = x[(l & 31) + 32] in every lane, so both halves get the same
// result. The leading s_nop gives the two wait states the swap needs after a VALU
// write of its operands (the compiler does not see inside the statement).
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float half_sum(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}
__device__ __forceinline__ float half_max(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}

// Workgroup barrier that does not drain global loads (__syncthreads waits for every
// outstanding load, including direct loads into LDS still meant to be in flight).
// Each wave has already waited, with an explicit s_waitcnt vmcnt, for the direct loads
// the other waves will read after the barrier. Waiting for its own LDS reads first
// keeps a buffer from being refilled under a pending read, and the memory clobber
// keeps the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima). Issued once after the
// per-column loads that precede a sweep: otherwise those loads stay "pending" at the
// loop header on some path and every iteration waits for its own K/V prefetch too.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Double-buffered sweep over `total` stages. Stage it lives in buf0 for even it and
// in buf1 for odd it (two distinct LDS objects, so the compiler sees that reading one
// never waits on the loads filling the other). body(it, lds) computes on stage it
// while stage it+1 is being fetched; one barrier per stage.
// With KONLY (a consumer that never reads V) bf16 stages load K alone.
template <typename St, bool KONLY = false, typename T, typename KeyFn, typename Body>
__device__ __forceinline__ void sweep(int total, KeyFn key0_of, const T* kbase, const T* vbase, int64_t row_stride,
                                      int n_valid, int tid, char* buf0, char* buf1, Body&& body) {
  typename St::Regs regs;
  auto fetch = [&](int it, char* dst) {
    if constexpr (KONLY && St::ASYNC) St::load_k(kbase, row_stride, key0_of(it), n_valid, tid, dst);
    else St::load(regs, kbase, vbase, row_stride, key0_of(it), n_valid, tid, dst);
  };
  if (total > 0) {
    fetch(0, buf0);
    St::store(regs, buf0, tid);
  }
  wait_vmem_all();
  __syncthreads();
  auto one = [&](int it, char* cur, char* nxt) {
    const bool more = it + 1 < total;
    if (more) fetch(it + 1, nxt);
    body(it, static_cast<const char*>(cur));
    if (more) St::store(regs, nxt, tid);
    if constexpr (St::ASYNC) wait_vmem_all();
    __syncthreads();
  };
  for (int it = 0; it < total; it += 2) {
    one(it, buf0, buf1);
    if (it + 1 < total) one(it + 1, buf1, buf0);
  }
}

}  // namespace poem
