// Block-sparse (and dense) causal prefill attention for gfx950.
//
// One workgroup computes one (query head, query tile): B rows, 32 per wave, over
// the key blocks the tile retains (sparse: its CSR row; dense: 0 .. diagonal), the
// retained-block attention of the POEM note (Section 4.1). K/V of each 64-key
// stage are loaded into LDS once and shared by the tile's waves; the loop visits
// only listed blocks, as BFLA's support-restricted kernel does (Section 3.4).
// Online softmax runs in the log2 domain in fp32; QK^T and PV run on bf16 (or
// fp32) MFMAs with fp32 accumulation. Only the diagonal block is masked. bf16 tiles
// take the first stage's row max as the exponent reference for all stages and fall
// back to the exact running max when later weights outgrow it (see attn_tile).
//
// Work order. Sparse rows: a persistent kernel pulls rows from a queue that a schedule
// kernel sorts one KV head after another, by sequence and then by retained count (or,
// without a workspace, one workgroup per row in the static order below); lists shared
// by a GQA group run two heads per workgroup (attn_sparse_pair_kernel). Dense tiles: a persistent kernel
// walks one KV head after another, longest tile first, pulling from a queue when the
// caller gives a workspace. Static order: workgroups ranked by the tile's diagonal
// block, longest first, with the KV head as the fastest-varying index of the
// workgroup id, so with 8 KV heads and the round-robin dispatch over the 8 XCDs every
// XCD streams one KV head's K/V through its own L2.
#include <mutex>

#include "poem.h"
#include "poem_internal.hpp"

namespace poem {

// Scratch of poem_sparse_prefill_noalloc: the queue head (first 256 bytes) and the row
// order of the persistent sparse schedule, in a device array the library owns. Host
// code never passes `scratch` itself to a kernel (on the host the name stands for a
// host-side shadow, not a device address): it uses the per-device address that
// hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kNoAllocScratchBytes = 256 + sizeof(int32_t) * (size_t)POEM_NOALLOC_MAX_ROWS;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy (the device is current)
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255) != 0) return hipErrorInvalidValue;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  *bytes = kNoAllocScratchBytes;
  return hipSuccess;
}

// Two waves per SIMD (two workgroups per CU) when the LDS stages allow it: the MFMA
// work of one wave overlaps the softmax of the other.
template <typename T, int D>
constexpr int attn_waves_per_eu() { return (sizeof(T) == 4 && D == 128) ? 1 : 2; }

// HEADS: query heads per workgroup (2: two heads of one GQA group walk one list, and
// each K/V stage is loaded once for both)
template <typename T, int D, int BLK, int HEADS = 1>
struct AttnCfg {
  static constexpr int WAVES_PER_HEAD = BLK / 32;
  static constexpr int WAVES = HEADS * WAVES_PER_HEAD;
  static constexpr int NT = WAVES * 64;
  using St = Stage<T, D, NT>;
  static constexpr int SUBS = BLK / kStageKeys;
  // bf16: K and V each double-buffered in four separate LDS arrays (a pipelined sweep);
  // fp32: two stage buffers (K and transposed V together)
  static constexpr int KBUF = St::ASYNC ? St::BYTES / 2 : St::BYTES;
  static constexpr int VBUF = St::ASYNC ? St::BYTES / 2 : 16;
  static constexpr int KBUF3 = St::ASYNC ? St::BYTES / 2 : 16;  // bf16: a third K buffer
  // direct loads one wave issues for one tensor of a stage (bf16)
  static constexpr int LOADS = St::ASYNC ? (St::BYTES / 2 / 1024) / WAVES : 0;
};

#define POEM_ATTN_LDS(T, D, BLK)                                              \
  __shared__ __attribute__((aligned(16))) char kb0[AttnCfg<T, D, BLK>::KBUF];  \
  __shared__ __attribute__((aligned(16))) char kb1[AttnCfg<T, D, BLK>::KBUF];  \
  __shared__ __attribute__((aligned(16))) char kb2[AttnCfg<T, D, BLK>::KBUF3]; \
  __shared__ __attribute__((aligned(16))) char vb0[AttnCfg<T, D, BLK>::VBUF];  \
  __shared__ __attribute__((aligned(16))) char vb1[AttnCfg<T, D, BLK>::VBUF];

// Largest per-lane sum of one stage's weights the lazy reference accepts (see attn_tile).
constexpr float kLazyCap = 4294967296.0f;  // 2^32

// One (query head h, tile t of sequence seq): the whole workgroup, B rows. Sparse: the
// list of h, or with p.shared that of h's GQA group's first head.
//
// Exponent reference (bf16): the tile is first computed with the first stage's row max
// as the reference for every stage (no per-stage max or rescale), so later weights may
// exceed 1. A stage whose per-lane weight sum exceeds kLazyCap, or is not finite, marks
// the tile; a tile marked by any wave is computed again with the exact running max. The
// rule depends only on the tile's data, so every schedule gives the same bits, and on
// accepted tiles the weights stay below 2^32, far inside the range of the bf16 weights
// and fp32 sums.
template <typename T, int D, int BLK, bool SPARSE, int HEADS = 1>
__device__ __forceinline__ void attn_tile(const AttnParams& p, int h0, int seq, int t, char* kb0, char* kb1,
                                          char* kb2, char* vb0, char* vb1) {
  using C = AttnCfg<T, D, BLK, HEADS>;
  using St = typename C::St;
  constexpr int SUBS = C::SUBS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the head and the CSR row below are too
  const int jcol = lane & 31, g2 = lane >> 5;
  const int hw = wave % C::WAVES_PER_HEAD;    // the wave's 32 rows within its head's tile
  const int h = h0 + wave / C::WAVES_PER_HEAD;  // its query head
  const int gk = h / p.group;
  const int n_q = p.seqs.n_q[seq], n_k = p.seqs.n_k[seq];
  const int diag = p.seqs.diag0[seq] + t;
  const int row0 = t * BLK;
  const int n_rows = min(BLK, n_q - row0);
  const int pos0 = (n_k - n_q) + row0;  // absolute position of the tile's first row
  const int wrow = 32 * hw + jcol;
  const bool row_ok = wrow < n_rows;
  const int my_pos = pos0 + wrow;
  const int wave_pos_min = pos0 + 32 * hw, wave_pos_max = wave_pos_min + 31;

  const int64_t qrow = (int64_t)p.seqs.q_start[seq] + row0 + wrow;
  QFrag<T, D> qf;
  qf.load(reinterpret_cast<const T*>(p.q) + (qrow * p.hq + h) * D, row_ok, g2);
  wait_vmem_all();

  const int64_t row_stride = (int64_t)p.hkv * D;
  const T* kbase = reinterpret_cast<const T*>(p.k) + ((int64_t)p.seqs.k_start[seq] * p.hkv + gk) * D;
  const T* vbase = reinterpret_cast<const T*>(p.v) + ((int64_t)p.seqs.k_start[seq] * p.hkv + gk) * D;

  // block list
  // The CSR is read-only for the whole launch, so its reads go through the scalar cache
  // (constant address space): a vector load here would make each stage's first wait
  // drain the K/V prefetch along with it.
  using cint = const __attribute__((address_space(4))) int32_t;
  cint* ids = nullptr;
  int nblk;
  if constexpr (SPARSE) {
    const int hl = p.shared ? (h / p.group) * p.group : h;  // the head whose list is walked
    const int64_t r = (int64_t)hl * p.seqs.total_tiles + p.seqs.tile_start[seq] + t;
    cint* rp = (cint*)p.row_ptr;
    const int a = rp[r], b = rp[r + 1];
    ids = (cint*)p.block_idx + a;
    int n = b - a;
    // rows are ascending: keep the ids in [0, diag]
    int lo = 0, hi = n;  // first index with id >= 0
    while (lo < hi) { int mid = (lo + hi) >> 1; if (ids[mid] < 0) lo = mid + 1; else hi = mid; }
    int first = lo;
    hi = n;  // first index with id > diag
    while (lo < hi) { int mid = (lo + hi) >> 1; if (ids[mid] <= diag) lo = mid + 1; else hi = mid; }
    ids += first;
    nblk = lo - first;
  } else {
    nblk = diag + 1;
  }
  auto stage_key0 = [&](int it) {
    const int blk = SPARSE ? ids[it / SUBS] : it / SUBS;
    return blk * BLK + (it % SUBS) * kStageKeys;
  };

  const int total = nblk * SUBS;
  f32x16 O[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) O[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;

  // causal mask of one stage's scores: only stages that reach past a row need it
  auto mask = [&](f32x16 (&S)[2], int key0) {
    if (key0 + kStageKeys - 1 > wave_pos_min) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + acc_key(kt, r, g2) > my_pos) S[kt][r] = -INFINITY;
    }
  };
  // Online softmax in two parts, so that only the running max precedes the rescale
  // branch. update(): new running max m; when some column's max grew (rare once the
  // sink is seen) the accumulated O and row sums are rescaled. exps(): the scores
  // become weights 2^(c s - m) and are added to the row sums.
  float m_use = 0.f;
  bool ovf = false;  // a stage's weights outgrew the lazy reference
  auto update = [&](const f32x16 (&S)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kt][r]);
    mx = half_max(mx);
    const float m_new = fmaxf(m_run, mx * c);
    m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) O[dt] *= alpha;
      l_run *= alpha;
    }
  };
  auto exps = [&](f32x16 (&S)[2]) {
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        S[kt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kt][r], c, -m_use));
        rs += S[kt][r];
      }
    l_run += rs;
  };

  if constexpr (St::ASYNC) {
    // Software pipeline over stages. V has two buffers and lags K by one stage: step j
    // reads K(j) and V(j-1) while V(j) and K(j+2) load. K has three buffers, so K, needed
    // first in a step, has two steps of lead (sparse rows mostly miss L2; with the same
    // pipeline the dense tiles ran 0.3% faster than with one step of K lead). The step
    // is laid out by hand in short chunks fenced off from the scheduler:
    //   QK phase : each QK^T MFMA of stage j with the next-but-one K fragment read and
    //              the exponentials (and bf16 packs) of key steps 0-1 of stage j-1;
    //   mask     : only on stages that reach past a row;
    //   PV phase : each P V MFMA of stage j-1 with the next-but-one V fragment read, the
    //              first half also with the exponentials of key steps 2-3.
    // The reference is the first stage's max (see above); a rejected tile is computed
    // again one stage at a time with the exact running max.
    constexpr int NQK = 2 * (D / 16);  // QK^T MFMAs per stage (2 key tiles x d steps)
    constexpr int NDT = D / 32;        // d tiles of O
    constexpr int NPV = 4 * NDT;       // P V MFMAs per stage (4 key steps x d tiles)
    constexpr int EPQ = 16 / NQK;      // exponentials per QK MFMA (key steps 0-1)
    constexpr int EPV = 16 / (NPV / 2);  // per P V MFMA of the first half (key steps 2-3)
    // key step 2's pack is complete after PV MFMA NPV/4 - 1, step 3's after NPV/2 - 1,
    // ahead of their first use at MFMAs 2 NDT = NPV/2 and 3 NDT
    static_assert(16 % NQK == 0 && 16 % (NPV / 2) == 0, "exponential split");
    // The row sums add the bf16 weights the P V MFMAs use (two per dot instruction), so
    // numerator and denominator see the same rounding.
    f32x16 Sp[2];
    const typename St::KOffsets ko = St::k_offsets(lane);
    auto kfrag = [&](const char* kbuf, int i) {  // K operand of QK MFMA i
      return St::k_frag(kbuf, ko, i & 1, i >> 1);
    };
    auto finish_max = [&](float mx) {  // running max of the stage, rare rescale
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
    const typename St::LaneOffsets lo = St::lane_offsets(row_stride, tid);
    // s_waitcnt vmcnt(LOADS): every direct load but this wave's newest K stage has landed
    constexpr int kWait = C::LOADS | 0x0F70;
    static_assert(C::LOADS < 16, "vmcnt field");
    // A K load past the row's last stage still issues its instructions (the waits count
    // them), but with no valid keys: its buffer descriptor covers no bytes, so the loads
    // write zeros without a memory access and the row's last waits do not sit on them.
    auto first = [&]() {
      // the waits count this wave's loads in issue order, which the fences keep
      St::load_k(kbase, row_stride, stage_key0(0), n_k, tid, kb0, lo);
      __builtin_amdgcn_sched_barrier(0);
      St::load_k(kbase, row_stride, stage_key0(min(1, total - 1)), total > 1 ? n_k : 0, tid, kb1, lo);
      __builtin_amdgcn_s_waitcnt(kWait);
      lds_barrier();
      St::load_v(vbase, row_stride, stage_key0(0), n_k, tid, vb0, lo);
      __builtin_amdgcn_sched_barrier(0);
      St::load_k(kbase, row_stride, stage_key0(min(2, total - 1)), total > 2 ? n_k : 0, tid, kb2, lo);
      Sp[0] = St::qk_tile(kb0, qf, 0, lane);
      Sp[1] = St::qk_tile(kb0, qf, 1, lane);
      mask(Sp, stage_key0(0));
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 32; ++e) mx = fmaxf(mx, Sp[e >> 4][e & 15]);
      finish_max(mx);
      __builtin_amdgcn_s_waitcnt(kWait);
      lds_barrier();
    };
    auto step = [&](int it, const char* kcur, char* knext, const char* vprev, char* vcur) {
      const int key0 = stage_key0(it);
      // V(it) first, then K(it + 2): the wait below leaves only the K loads in flight
      St::load_v(vbase, row_stride, key0, n_k, tid, vcur, lo);
      __builtin_amdgcn_sched_barrier(0);
      St::load_k(kbase, row_stride, stage_key0(min(it + 2, total - 1)), it + 2 < total ? n_k : 0, tid, knext, lo);
      // QK phase at raised wave priority (s_setprio): its issue slots go ahead of the PV
      // phase of the other wave on the SIMD (measured at 128K: -1.8% for the sparse
      // kernel against raising the PV phase instead)
      __builtin_amdgcn_s_setprio(1);
      f32x16 Sn[2] = {f32x16{}, f32x16{}};
      bf16x8 P[4];
      bf16x8 ka[3];
      ka[0] = kfrag(kcur, 0);
      ka[1] = kfrag(kcur, 1);
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        Sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % 3], qf.q[i >> 1], Sn[i & 1], 0, 0, 0);
        if (i + 2 < NQK) ka[(i + 2) % 3] = kfrag(kcur, i + 2);
        // key steps 0 and 1 of stage j-1 here, steps 2 and 3 next to the first half of the
        // PV MFMAs, which do not use them yet (measured at 128K against all four here:
        // sparse -0.45%, dense -1.5%, the same bits)
#pragma unroll
        for (int u = 0; u < EPQ; ++u) {
          const int e = i * EPQ + u;
          Sp[e >> 4][e & 15] = __builtin_amdgcn_exp2f(__builtin_fmaf(Sp[e >> 4][e & 15], c, -m_use));
          if ((e & 7) == 7) {
            bf16x8 unused;
            p_step<false>(Sp, e >> 3, P[e >> 3], unused);
            rs = row_sum_bf16(P[e >> 3], rs);
            // keep the sum in this chunk (an empty statement, no code); left free, the
            // compiler sinks it past the mask branch (slower, measured at 128K)
            __asm__ volatile("" : "+v"(rs));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // PV phase
      __builtin_amdgcn_s_setprio(0);
      bf16x8 va[3];
      va[0] = St::v_frag(vprev, 0, 0, lane);
      va[1] = St::v_frag(vprev, 1 % NDT, 1 / NDT, lane);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int dt = i % NDT, st = i / NDT;
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 3], P[st], O[dt], 0, 0, 0);
        if (i + 2 < NPV) va[(i + 2) % 3] = St::v_frag(vprev, (i + 2) % NDT, (i + 2) / NDT, lane);
        if (i < NPV / 2) {  // exponentials, packs and sums of key steps 2 and 3
#pragma unroll
          for (int u = 0; u < EPV; ++u) {
            const int e = 16 + i * EPV + u;
            Sp[e >> 4][e & 15] = __builtin_amdgcn_exp2f(__builtin_fmaf(Sp[e >> 4][e & 15], c, -m_use));
            if ((e & 7) == 7) {
              bf16x8 unused;
              p_step<false>(Sp, e >> 3, P[e >> 3], unused);
              rs = row_sum_bf16(P[e >> 3], rs);
              __asm__ volatile("" : "+v"(rs));
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run += rs;
      ovf |= !(rs <= kLazyCap);
      if (key0 + kStageKeys - 1 > wave_pos_min) mask(Sn, key0);
      Sp[0] = Sn[0];
      Sp[1] = Sn[1];
      __builtin_amdgcn_s_waitcnt(kWait);
      lds_barrier();
    };
    if (total > 0) {
      first();
      // stage it: K in kb[it % 3], V in vb[it % 2]. Six unconditional steps per trip
      // keep every buffer a distinct LDS object in each step, so the compiler sees that
      // reading K(it) never waits on the K(it + 1) load still in flight (a conditional
      // step would merge the two); the last stages take the buffers picked at run time.
      int it = 1;
      for (; it + 5 < total; it += 6) {
        step(it, kb1, kb0, vb0, vb1);
        step(it + 1, kb2, kb1, vb1, vb0);
        step(it + 2, kb0, kb2, vb0, vb1);
        step(it + 3, kb1, kb0, vb1, vb0);
        step(it + 4, kb2, kb1, vb0, vb1);
        step(it + 5, kb0, kb2, vb1, vb0);
      }
      for (; it < total; ++it) {
        const int r3 = it % 3;
        char* kc = r3 == 0 ? kb0 : (r3 == 1 ? kb1 : kb2);
        char* kn = r3 == 0 ? kb2 : (r3 == 1 ? kb0 : kb1);
        step(it, kc, kn, (it & 1) ? vb0 : vb1, (it & 1) ? vb1 : vb0);
      }
      bf16x8 P[4], unused;
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) Sp[e >> 4][e & 15] = __builtin_amdgcn_exp2f(__builtin_fmaf(Sp[e >> 4][e & 15], c, -m_use));
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        p_step<false>(Sp, s4, P[s4], unused);
        rs = row_sum_bf16(P[s4], rs);
      }
      l_run += rs;
      ovf |= !(rs <= kLazyCap);
      St::pv_packed(((total - 1) & 1) ? vb1 : vb0, P, O, lane);
      // the last K prefetches (empty ones past the row's end) may still be in flight:
      // they land before this workgroup's LDS can be reused
      wait_vmem_all();
    }
    // Did any wave mark the tile? Each wave writes its own word of the third K buffer,
    // free once every wave has passed the barrier after its loads landed (the next user
    // of those words, a persistent kernel's queue slot, writes them after a barrier).
    lds_barrier();
    int* flags = reinterpret_cast<int*>(kb2);
    const int mine = __any(ovf) ? 1 : 0;
    if (lane == 0) flags[wave] = mine;
    lds_barrier();
    // The decision is per query head (its own waves' marks), so a tile's bits do not
    // depend on the other head sharing the workgroup; every wave takes part in the
    // redo's loads and barriers.
    int redo = 0, redo_any = 0;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) {
      redo_any |= flags[w];
      if (w / C::WAVES_PER_HEAD == wave / C::WAVES_PER_HEAD) redo |= flags[w];
    }
    if (__builtin_amdgcn_readfirstlane(redo_any) != 0) {
      // the exact running max, one stage at a time in the first K and V buffers (rare)
      const bool mine_redo = HEADS == 1 || __builtin_amdgcn_readfirstlane(redo) != 0;
      if (mine_redo) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x16{};
        m_run = -INFINITY;
        l_run = 0.f;
        m_use = 0.f;
      }
      for (int it = 0; it < total; ++it) {
        const int key0 = stage_key0(it);
        St::load_k(kbase, row_stride, key0, n_k, tid, kb0, lo);
        St::load_v(vbase, row_stride, key0, n_k, tid, vb0, lo);
        wait_vmem_all();
        lds_barrier();
        if (mine_redo) {
          f32x16 S[2];
          S[0] = St::qk_tile(kb0, qf, 0, lane);
          S[1] = St::qk_tile(kb0, qf, 1, lane);
          mask(S, key0);
          update(S);
          bf16x8 P[4], unused;
          float rs = 0.f;
#pragma unroll
          for (int e = 0; e < 32; ++e)
            S[e >> 4][e & 15] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e >> 4][e & 15], c, -m_use));
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            p_step<false>(S, s4, P[s4], unused);
            rs = row_sum_bf16(P[s4], rs);
          }
          l_run += rs;
          St::pv_packed(vb0, P, O, lane);
        }
        lds_barrier();  // every wave is done with the buffers before the next stage loads
      }
    }
  } else {
    sweep<St>(total, stage_key0, kbase, vbase, row_stride, n_k, tid, kb0, kb1, [&](int it, const char* cur) {
      const int key0 = stage_key0(it);
      if (key0 > wave_pos_max) return;  // every key of the stage is above this wave's rows
      f32x16 S[2];
      S[0] = St::qk_tile(cur, qf, 0, lane);
      S[1] = St::qk_tile(cur, qf, 1, lane);
      mask(S, key0);
      update(S);
      exps(S);
      St::template pv<false>(cur, S, O, lane);
    });
  }

  const float l_tot = half_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    // a per-lane base pointer (the lane's half of each 8-column group) with the d tile
    // and column group as constant offsets, which fold into the stores' immediate
    // offsets; offsets kept as values of their own would be loop-invariant in the
    // persistent kernels, hoisted out of the row loop and spilled
    const int64_t e0 = (qrow * p.hq + h) * D + 4 * g2;
    if (p.out_f32) {
      float* orow = reinterpret_cast<float*>(p.out) + e0;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 o = {O[dt][4 * a] * inv, O[dt][4 * a + 1] * inv, O[dt][4 * a + 2] * inv,
                           O[dt][4 * a + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * a) = o;
        }
    } else {
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + e0;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const u32x2 w = {pack_bf16(O[dt][4 * a] * inv, O[dt][4 * a + 1] * inv),
                           pack_bf16(O[dt][4 * a + 2] * inv, O[dt][4 * a + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a) = w;
        }
    }
    // the weights are 2^(c s - m_use); with the lazy reference m_use stays at the first
    // stage's max (0 if that stage was masked) while later stages add weight
    if (p.lse != nullptr && g2 == 0)
      p.lse[(int64_t)h * p.total_q + qrow] = l_tot > 0.f ? (m_use + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Static schedule (sparse rows without a workspace): one workgroup per (head, tile),
// ranked by the tile's diagonal block (longest first) with the KV head as the
// fastest-varying index (see the file header).
template <typename T, int D, int BLK, bool SPARSE>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<T, D>(), 2)))
void attn_fwd_kernel(AttnParams p) {
  POEM_ATTN_LDS(T, D, BLK)
  const int bid = blockIdx.x;
  const int gk = bid % p.hkv;
  const int rest = bid / p.hkv;
  const int hg = rest % p.group;
  const int rank = rest / p.group;
  int seq, t;
  rank_to_item(p.seqs, 1, rank, seq, t);
  if (seq < 0) return;
  attn_tile<T, D, BLK, SPARSE>(p, gk * p.group + hg, seq, t, kb0, kb1, kb2, vb0, vb1);
}

// Persistent schedule for dense rows: one workgroup per resident slot walks the tiles
// in a fixed order, one KV head after another (its K/V stays in the memory-side cache)
// and, within a KV head, longest first with the G query heads of a tile adjacent.
// With a queue (p.queue) each slot pulls its next tile from it; without one, round k
// of the order goes to the slots forward on even rounds and backward on odd ones, so
// each slot pairs long tiles with short ones. The queue adapts to slots that run
// faster or slower than others (at 128K: 2.8% faster than the fixed interleave, 3.8%
// faster than one workgroup per tile).
__global__ void dense_queue_reset_kernel(int32_t* queue) { *queue = 0; }

template <typename T, int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<T, D>(), 2)))
void attn_dense_persistent_kernel(AttnParams p) {
  POEM_ATTN_LDS(T, D, BLK)
  // the queue slot borrows kb2, which no wave reads between tiles
  int* item_sh = reinterpret_cast<int*>(kb2);
  const int total = p.num_rows;
  const int per_kv = total / p.hkv;
  const int S = gridDim.x;
  for (int round = 0;; ++round) {
    int bid;
    if (p.queue != nullptr) {
      // every wave's direct loads of the previous tile have landed (attn_tile ends
      // with them drained); the barrier orders them before the slot is written
      __syncthreads();
      if (threadIdx.x == 0) *item_sh = atomicAdd(p.queue, 1);
      __syncthreads();
      bid = __builtin_amdgcn_readfirstlane(*item_sh);  // uniform by construction
      __syncthreads();
      if (bid >= total) break;
    } else {
      const int base = round * S;
      if (base >= total) break;
      bid = base + ((round & 1) ? S - 1 - (int)blockIdx.x : (int)blockIdx.x);
      if (bid >= total) continue;
      // every wave is done with the previous tile's buffers before they are refilled
      __syncthreads();
    }
    const int gk = bid / per_kv;
    const int rest = bid % per_kv;
    const int hg = rest % p.group;
    const int rank = rest / p.group;
    int seq, t;
    rank_to_item(p.seqs, 1, rank, seq, t);
    if (seq < 0) continue;
    attn_tile<T, D, BLK, false>(p, gk * p.group + hg, seq, t, kb0, kb1, kb2, vb0, vb1);
  }
}

// Persistent schedule for sparse rows, whose lengths vary from a few blocks to
// thousands: one workgroup per resident slot pulls CSR rows from a queue that the
// schedule kernel ordered by retained count, longest first. Rows are independent,
// so the results do not depend on which workgroup takes which row.
template <typename T, int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<T, D>(), 2)))
void attn_sparse_persistent_kernel(AttnParams p) {
  POEM_ATTN_LDS(T, D, BLK)
  // the queue slot borrows kb2, which no wave reads between rows (bf16: this keeps the
  // workgroup's LDS at 80 KB, two workgroups per CU)
  int* item_sh = reinterpret_cast<int*>(kb2);
  const int n_tiles = p.seqs.total_tiles;
  for (;;) {
    // every wave's direct loads of the previous row have landed (attn_tile ends with
    // them drained); the barrier orders them before the slot is written
    __syncthreads();
    if (threadIdx.x == 0) *item_sh = atomicAdd(p.queue, 1);
    __syncthreads();
    // uniform by construction; readfirstlane lets the row's CSR and block ids load
    // through the scalar cache (vector loads here would each drain the K/V prefetch)
    const int item = __builtin_amdgcn_readfirstlane(*item_sh);
    __syncthreads();
    if (item >= p.num_rows) break;
    const int r = p.order[item];
    const int h = r / n_tiles, gtile = r % n_tiles;
    const int seq = find_seq(p.seqs, gtile);
    attn_tile<T, D, BLK, true>(p, h, seq, gtile - p.seqs.tile_start[seq], kb0, kb1, kb2, vb0, vb1);
  }
}

// Group-shared lists (bf16, G even): one workgroup of eight waves per (KV head, tile,
// pair of the group's query heads), both heads walking the group's one list, so each
// K/V stage is loaded into LDS once for the two heads' rows (the heads of a BFLA group
// share one selection, Section 3.3, and with it the blocks each stage reads). Items
// come from a queue over (KV head, tile) units that the schedule kernel sorted by list
// length, longest first, each unit followed by its G / 2 pairs.
template <typename T, int D, int BLK>
__global__ __launch_bounds__(BLK * 4) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_sparse_pair_kernel(AttnParams p) {
  POEM_ATTN_LDS(T, D, BLK)
  int* item_sh = reinterpret_cast<int*>(kb2);  // as in the kernel above
  const int n_tiles = p.seqs.total_tiles;
  const int pairs = p.group / 2;
  const int n_items = p.hkv * n_tiles * pairs;
  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0) *item_sh = atomicAdd(p.queue, 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(*item_sh);
    __syncthreads();
    if (item >= n_items) break;
    const int r = p.order[item / pairs];  // the unit's first-head row, g G T + gtile
    const int gtile = r % n_tiles;
    const int h0 = r / n_tiles + 2 * (item % pairs);
    const int seq = find_seq(p.seqs, gtile);
    attn_tile<T, D, BLK, true, 2>(p, h0, seq, gtile - p.seqs.tile_start[seq], kb0, kb1, kb2, vb0, vb1);
  }
}

// Orders the CSR rows of each KV head by sequence, longest sequence first, and within
// a sequence by retained count, descending (a counting sort in LDS; one workgroup per
// KV head, whose rows h*T .. are contiguous), KV heads one after another, and resets
// the queue head (group_stride: rows from one KV head's first row to the next one's;
// rows_per_group of them are ordered). Pulling rows in this order keeps the running
// workgroups on one KV head's K/V of one sequence at a time (64 MiB at 128K tokens),
// which the 256 MiB memory-side cache can hold while the rows re-read it (measured on
// four chunked sequences of 16K-128K keys: 9.51 -> 9.38 ms against the count order
// alone). shared_tiles > 0 (shared lists): row i of a KV head's block takes the count
// of its group's first-head row, i mod shared_tiles. Counts are clamped to the bins
// each sequence gets (4097 / sequences), for ordering only.
constexpr int kSchedThreads = 1024;
constexpr int kSchedBins = 4097;  // counts are clamped to 4096 for ordering only
__global__ __launch_bounds__(kSchedThreads) void sparse_schedule_kernel(const int32_t* __restrict__ row_ptr,
                                                                       int rows_per_group, int group_stride,
                                                                       int shared_tiles,
                                                                       int32_t* __restrict__ order_all,
                                                                       int32_t* __restrict__ queue, SeqTable seqs) {
  __shared__ int hist[kSchedBins];
  __shared__ int sh[16];
  __shared__ int seq_rank[kMaxSeqs];  // position of each sequence, longest N_k first
  const int tid = threadIdx.x;
  const int first = blockIdx.x * group_stride;  // the KV head's first row
  const int rows = rows_per_group;
  int32_t* order = order_all + blockIdx.x * rows_per_group;
  const int nseq = seqs.num_seqs;
  const int per_seq = kSchedBins / nseq;  // count bins of one sequence
  for (int i = tid; i < kSchedBins; i += kSchedThreads) hist[i] = 0;
  if (tid < nseq) {
    int rk = 0;
    for (int s = 0; s < nseq; ++s)
      rk += (seqs.n_k[s] > seqs.n_k[tid] || (seqs.n_k[s] == seqs.n_k[tid] && s < tid)) ? 1 : 0;
    seq_rank[tid] = rk;
  }
  __syncthreads();
  auto bin = [&](int i) {
    const int local = shared_tiles > 0 ? i % shared_tiles : i;
    const int r = first + local;
    const int c = min(max(row_ptr[r + 1] - row_ptr[r], 0), per_seq - 1);
    const int sq = nseq > 1 ? seq_rank[find_seq(seqs, local % seqs.total_tiles)] : 0;
    return sq * per_seq + (per_seq - 1 - c);  // longest first
  };
  for (int r = tid; r < rows; r += kSchedThreads) atomicAdd(&hist[bin(r)], 1);
  __syncthreads();
  constexpr int PER = (kSchedBins + kSchedThreads - 1) / kSchedThreads;
  int local = 0;
  for (int e = 0; e < PER; ++e) {
    const int i = tid * PER + e;
    if (i < kSchedBins) local += hist[i];
  }
  int total;
  int off = block_excl_scan_int(local, total, sh);
  __syncthreads();
  for (int e = 0; e < PER; ++e) {
    const int i = tid * PER + e;
    if (i < kSchedBins) {
      const int c = hist[i];
      hist[i] = off;
      off += c;
    }
  }
  __syncthreads();
  for (int r = tid; r < rows; r += kSchedThreads) order[atomicAdd(&hist[bin(r)], 1)] = first + r;
  if (blockIdx.x == 0 && tid == 0) *queue = 0;
}

// Group-shared lists with G even (bf16): (KV head, tile) units ordered by the first
// head's count, two heads of the group per workgroup.
template <typename T, int D, int BLK>
static hipError_t launch_pairs(const AttnParams& p, int64_t rows, hipStream_t stream) {
  hipLaunchKernelGGL(sparse_schedule_kernel, dim3(p.hkv), dim3(kSchedThreads), 0, stream, p.row_ptr,
                     p.seqs.total_tiles, p.num_rows / p.hkv, 0, p.order, p.queue, p.seqs);
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_sparse_pair_kernel<T, D, BLK>, BLK * 4, 0);
  if (e != hipSuccess) return e;
  const int64_t items = rows / 2;
  const int64_t slots = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
  hipLaunchKernelGGL((attn_sparse_pair_kernel<T, D, BLK>), dim3((unsigned)(slots < items ? slots : items)),
                     dim3(BLK * 4), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D, int BLK, bool SPARSE>
static hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.seqs.total_tiles * p.hq;
  if (grid == 0) return hipSuccess;
  if constexpr (SPARSE && sizeof(T) == 2) {
    if (p.queue != nullptr && p.shared && p.group % 2 == 0)
      return launch_pairs<T, D, BLK>(p, grid, stream);
  }
  if (SPARSE && p.queue != nullptr) {
    hipLaunchKernelGGL(sparse_schedule_kernel, dim3(p.hkv), dim3(kSchedThreads), 0, stream, p.row_ptr,
                       p.num_rows / p.hkv, p.num_rows / p.hkv, p.shared ? p.seqs.total_tiles : 0, p.order, p.queue,
                       p.seqs);
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_sparse_persistent_kernel<T, D, BLK>, BLK * 2, 0);
    if (e != hipSuccess) return e;
    const int64_t slots = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    hipLaunchKernelGGL((attn_sparse_persistent_kernel<T, D, BLK>), dim3((unsigned)(slots < grid ? slots : grid)),
                       dim3(BLK * 2), 0, stream, p);
    return hipGetLastError();
  }
  if constexpr (!SPARSE) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_dense_persistent_kernel<T, D, BLK>, BLK * 2, 0);
    if (e != hipSuccess) return e;
    const int64_t slots = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    if (p.queue != nullptr) hipLaunchKernelGGL(dense_queue_reset_kernel, dim3(1), dim3(1), 0, stream, p.queue);
    hipLaunchKernelGGL((attn_dense_persistent_kernel<T, D, BLK>), dim3((unsigned)(slots < grid ? slots : grid)),
                       dim3(BLK * 2), 0, stream, p);
    return hipGetLastError();
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, BLK, SPARSE>), dim3((unsigned)grid), dim3(BLK * 2), 0, stream, p);
    return hipGetLastError();
  }
}

template <typename T, int D, int BLK>
static hipError_t launch_mode(const AttnParams& p, bool sparse, hipStream_t s) {
  return sparse ? launch_one<T, D, BLK, true>(p, s) : launch_one<T, D, BLK, false>(p, s);
}

template <typename T, int D>
static hipError_t launch_block(const AttnParams& p, int block, bool sparse, hipStream_t s) {
  return block == 64 ? launch_mode<T, D, 64>(p, sparse, s) : launch_mode<T, D, 128>(p, sparse, s);
}

template <typename T>
static hipError_t launch_dim(const AttnParams& p, int d, int block, bool sparse, hipStream_t s) {
  return d == 64 ? launch_block<T, 64>(p, block, sparse, s) : launch_block<T, 128>(p, block, sparse, s);
}

hipError_t launch_attention(const AttnParams& p, int in_dtype, int head_dim, int block, bool sparse,
                            hipStream_t stream) {
  return in_dtype == 0 ? launch_dim<uint16_t>(p, head_dim, block, sparse, stream)
                       : launch_dim<float>(p, head_dim, block, sparse, stream);
}

}  // namespace poem
