// Shared tile machinery of the attention kernels (gfx950): LDS staging by DMA,
// the 32x32x16 bf16 MFMA layouts, the fixed-maximum and online softmax tiles.
#pragma once
// Frame-aligned window-sparse attention forward kernel for gfx950 (CDNA4).
//
// Method: "HeyGen x Google Cloud: Bringing Avatar IV to TPUs".
//   * section "Deleting the mask" (Fig. 3): tiles are whole 16-token granules
//     that divide the frame span, so a query block's key granules are either
//     all visible (reference frame + window) or skipped. The reference frame's
//     granules are simply the first granules of the same single pass: no mask
//     predicate, no padding, no second pass, no merge.
//   * section "Unchaining softmax" (Fig. 4): for eligible items the softmax
//     maximum of row i is fixed in advance to M_i = scale*(<q_i,mu> + ||q_i||*kvis)
//     where kvis bounds ||k_j - mu|| over every key the row sees (the head's
//     largest centred key norm, or the largest over the visible frames), so
//     M_i >= every visible logit by Cauchy-Schwarz and the key loop has no
//     running maximum and no accumulator rescale; the row sum stays a per-lane
//     partial and is reduced across lanes once, at the end. Items whose bound
//     is too loose run the online softmax in the same kernel (one branch per
//     (batch, head, query frame), uniform over the workgroup).
//   * section "Proving pixels unchanged": P is rounded to bf16 and PV runs on
//     the bf16 matrix cores with fp32 accumulation.
//
// Work decomposition: a work item is one query block of 16*gq rows of one (batch,
// head, frame), the last block of a frame whatever rows are left (a multiple of 16);
// a workgroup runs one item at a time (the attention kernel keeps its workgroups
// resident and hands them items from a queue). WAVES waves each own QT 32-row query
// tiles; a tile with 16 real rows holds 16 repeats that are computed but never
// stored, and a wave with no real row only helps move the keys. All waves stream the
// same key granules through LDS.
//
// MFMA orientation (v_mfma_f32_32x32x16_bf16, wave64; 32x32x16 runs at twice
// the rate of 16x16x32 on this chip):
//   S^T[key][q] = K[key][:] . Q[q][:]        A = K from LDS, B = Q in registers;
//     accumulator lane l holds query l%32 and MFMA rows 8*(i/4) + 4*(l/32) + i%4
//     (i = 0..15), so all 16 scores of a lane belong to one query row. MFMA
//     row rho is fed the key pi(rho) = 16*(m/2) + 8*g + 4*(m%2) + i for
//     rho = 8m + 4g + i, which makes register i of lane group g hold key
//     16*(i/8) + 8*g + i%8: the 8 keys of each PV half are contiguous.
//   O^T[e][q] += V^T[e][key] . P^T[key][q]   B = P^T straight from the score
//     registers (regs 8h..8h+7 = keys 16h + 8g + 0..7), A = V^T rows read as one
//     16-byte LDS load per lane; the O accumulator lane again holds one query
//     row, so the online rescale and the final 1/l are per-lane scalars.
//
// Staging: the memory-bound prologue (sfa_norms) writes V^T [b][h][d][S] into
// the workspace (LDS transpose reads run at well under half the rate of plain
// 16-byte reads on gfx950). K rows and V^T granules then go from HBM straight into LDS by
// DMA (buffer_load_dwordx4 ... lds: no registers, no VALU), in NBUF rotating 64-key
// stages. 16-byte chunks are XOR-swizzled through the DMA source address
// so the operand reads are free of bank conflicts:
//   K   [key][d]            : chunk ^= key % 16 (16 lanes read 16 rows);
//   V^T [granule][d][16 keys]: half ^= (d / 8) % 2 (16 lanes read 16 rows of 32 B).
#include "sfa_internal.h"

namespace {

using sfa::FwdParams;
using sfa::Item;
using sfa::KeyRanges;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// (1.0, 1.0) in bf16: dot2 with it adds the two halves of a packed pair
constexpr bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};

constexpr int kStageKeys = 64;  // keys per LDS stage (4 granules, 2 tiles of 32)

// Online softmax keeps a stale running maximum until a tile's maximum exceeds it by
// more than kLazy (log2 units). P then stays below 2^kLazy, which bf16 and the fp32
// sums hold with unchanged relative precision: with fewer than 2^24 keys per row,
// l < 2^88 and |O| < 2^88 * max|v|, far below 2^127 for any bf16 v up to 2^38. A large
// kLazy makes rescales rare when the scores are wide.
constexpr float kLazy = 64.0f;

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Wait until at most N of this wave's vector-memory operations (the LDS DMAs
// of younger stages) are still in flight.
template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, int WAVES, int QT, int NBUF>
struct Attn {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int KS = D / 16;             // 16-dim k-steps of QK^T
  static constexpr int DT = D / 32;             // 32-dim tiles of O^T
  static constexpr int CH = D / 8;              // 16-byte chunks per key row
  static constexpr int ROWB = 2 * D;            // bytes per key row
  static constexpr int KPR = 256 / ROWB;        // key rows per 256-byte bank sweep
  static constexpr int STAGE_B = kStageKeys * ROWB;          // bytes per tensor per stage
  static constexpr int DMA_KEYS = 1024 / ROWB;               // K keys per DMA instruction
  static constexpr int DMA_N = 2 * STAGE_B / 1024;           // K + V instructions per stage
  static constexpr int VG_B = D * 32;                        // bytes of one V^T granule
  static constexpr int DMA_VG = VG_B / 1024;                 // DMA instructions per V^T granule
  static constexpr int LDS_BYTES = NBUF * 2 * STAGE_B;       // NBUF stages of K and V
  // LDS layout: K stage buffers [0, NBUF*STAGE_B), V^T stage buffers after them.
  // Lane offsets of V^T reads include VBASE so every operand read is a base
  // register plus an immediate below 64 KB.
  static constexpr int VBASE = NBUF * STAGE_B;
  static_assert(DMA_N % WAVES == 0, "DMA instructions split evenly over waves");

  static constexpr int DMA_W = DMA_N / WAVES;                // DMA instructions per wave
  static constexpr int LPR = 64 / DMA_KEYS;                  // lanes per key row

  __device__ static inline int k_phys(int key, int c) { return c ^ ((key / KPR) % CH); }
  __device__ static inline int vt_half(int d, int half) { return half ^ ((d >> 3) & 1); }
  // key fed to S^T MFMA row rho (see the header)
  __device__ static inline int key_of_row(int rho) {
    const int m = rho >> 3, gg = (rho >> 2) & 1, i = rho & 3;
    return 16 * (m >> 1) + 8 * gg + 4 * (m & 1) + i;
  }

  __device__ static inline int granule_key(const KeyRanges& r, int gi) {
    const int t = gi * 16;
    return t < r.r0_end ? t : r.r1_begin + (t - r.r0_end);
  }

  // Per-lane constants of the hot loop, computed once per item so that every
  // LDS read in the loop is base register + immediate and every DMA is a
  // uniform base + one lane offset.
  static constexpr int KW = DMA_N / 2 / WAVES;  // K DMA slots per wave per stage
  static constexpr int VW = DMA_N / 2 / WAVES;  // V^T DMA slots per wave per stage
  static_assert(KW * WAVES * 2 == DMA_N, "K and V DMA slots split evenly over waves");

  // Per-lane constants of the hot loop, computed once per item so that every
  // LDS read in the loop is base register + immediate and every DMA is a
  // uniform (SGPR) base plus one precomputed lane offset.
  struct Lane {
    uint32_t kofs[KS];       // K operand byte offset inside a stage, per 16-dim k-step
    uint32_t vofs[DT];       // VBASE + V^T operand offset inside a granule, per 32-dim tile
    uint32_t kdma[KW];       // K DMA source offset from the stage's first key row
    uint32_t vdma[VW];       // V^T DMA source offset from the stage's first key column
  };

  // Wave-uniform per item: which keys / granules each DMA slot of this wave moves.
  struct Slots {
    int kkey0[KW];           // first stage key of K slot i (DMA_KEYS keys per slot)
    int vgr[VW];             // stage granule of V^T slot j
    int kdst[KW];            // LDS byte offset of K slot i inside a stage buffer
    int vdst[VW];            // LDS byte offset of V^T slot j inside a stage buffer
  };

  // Key source of one item: granule gi starts at token 16*gi before the seam
  // (the end of the first key range) and 16*gi + shift after it.
  struct Src {
    const char* k;           // K row of token 0 of this (b, h)
    const char* v;           // V^T column of token 0 of this (b, h)
    int64_t kss2;            // K row stride in bytes
    int n0;                  // first granule past the seam
    int shift;               // token shift of granules at or past the seam
  };

  __device__ static inline void lane_setup(Lane& L, Slots& W, int64_t kss, int S) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int krow = key_of_row(l32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) L.kofs[ks] = krow * ROWB + k_phys(krow, 2 * ks + g) * 16;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + l32;
      L.vofs[dt] = VBASE + d * 32 + vt_half(d, g) * 16;
    }
#pragma unroll
    for (int i = 0; i < KW; ++i) {  // K rows: lane -> (key, physical chunk)
      const int key0 = (wave * KW + i) * DMA_KEYS;
      const int key = key0 + lane / LPR;
      const int c = k_phys(key, lane % LPR);
      W.kkey0[i] = key0;
      W.kdst[i] = key0 * ROWB;
      L.kdma[i] = uint32_t((key * kss + c * 8) * 2);
    }
#pragma unroll
    for (int j = 0; j < VW; ++j) {  // V^T granule quarter: lane -> (d, physical half)
      const int m = wave * VW + j;
      const int gr = m / DMA_VG, qd = m % DMA_VG;
      const int d = 32 * qd + lane / 2;
      W.vgr[j] = gr;
      W.vdst[j] = VBASE + gr * VG_B + qd * 1024;
      L.vdma[j] = uint32_t((int64_t(d) * S + 16 * gr + 8 * vt_half(d, lane & 1)) * 2);
    }
  }

  // 16 bytes per lane from base + off into LDS at dst + 16 * lane, through a raw buffer
  // resource (base in SGPRs, no range limit, 32-bit data format; off in one VGPR, below
  // 2^32 by the host's size checks). A buffer load, unlike the global form, leaves the
  // compiler's LDS read waits exact: while a global-segment LDS DMA is outstanding it
  // widens every wait on an LDS read to "all of them".
  __device__ static inline void dma16(const char* base, uint32_t off, char* dst) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, -1, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)dst, 16, off, 0, 0, 0);
  }

  // DMA the first `ng` granules of stage s into LDS buffer `buf` (a constant
  // after unrolling).
  __device__ static inline void issue_stage(char* lds, int buf, const Lane& L, const Slots& W,
                                            const Src& X, int s, int ng) {
    const int g0 = 4 * s;
    const char* kst = X.k + int64_t(16 * g0) * X.kss2;
    const char* vst = X.v + int64_t(16 * g0) * 2;
    char* lb = lds + buf * STAGE_B;  // + VBASE for V^T (inside vdst)
    if (g0 >= X.n0 || g0 + ng <= X.n0) {  // one side of the seam: a single base per tensor
      if (g0 >= X.n0) {
        kst += int64_t(X.shift) * X.kss2;
        vst += int64_t(X.shift) * 2;
      }
#pragma unroll
      for (int i = 0; i < KW; ++i)
        if (W.kkey0[i] < 16 * ng) dma16(kst, L.kdma[i], lb + W.kdst[i]);
#pragma unroll
      for (int j = 0; j < VW; ++j)
        if (W.vgr[j] < ng) dma16(vst, L.vdma[j], lb + W.vdst[j]);
    } else {                              // the stage straddles the seam
#pragma unroll
      for (int i = 0; i < KW; ++i) {
        const int gr = W.kkey0[i] / 16;
        if (gr >= ng) continue;
        const int sh = g0 + gr >= X.n0 ? X.shift : 0;
        dma16(kst + int64_t(sh) * X.kss2, L.kdma[i], lb + W.kdst[i]);
      }
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        if (W.vgr[j] >= ng) continue;
        const int sh = g0 + W.vgr[j] >= X.n0 ? X.shift : 0;
        dma16(vst + int64_t(sh) * 2, L.vdma[j], lb + W.vdst[j]);
      }
    }
  }

  // One 32-key tile (HALF: only its first 16 keys exist) for all QT query tiles.
  // kl / vl: LDS byte offsets of the tile's first K and V rows.
  template <bool HALF, bool ONLINE, int NT>
  __device__ static inline void tile(const char* lds, const Lane& L, int kl, int vl,
                                     const bf16x8 (&qf)[NT][KS], f32x16 (&o)[NT][DT],
                                     float (&mrow)[NT], float (&lsum)[NT], float cexp) {
    // S^T = K . Q^T
    f32x16 s[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[t][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + kl + L.kofs[ks]);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t][ks], s[t], 0, 0, 0);
    }
    // softmax numerators: 16 (8 for HALF) scores of one query row per lane
    constexpr int NV = HALF ? 8 : 16;
    uint32_t pk[NT][NV / 2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (ONLINE) {
        float mx = s[t][0];
#pragma unroll
        for (int i = 1; i < NV; ++i) mx = fmaxf(mx, s[t][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * cexp;
        // lazy rescale: keep the stale maximum while the tile stays within 2^kLazy
        // of it (exact up to rounding: numerator and denominator share the shift)
        const bool grow = mx > mrow[t] + kLazy;
        if (__ballot(grow) != 0) {
          const float mnew = fmaxf(mrow[t], mx);
          const float alpha = __builtin_amdgcn_exp2f(mrow[t] - mnew);
          lsum[t] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
          mrow[t] = mnew;
        }
      }
      const float m = mrow[t];
#pragma unroll
      for (int i = 0; i < NV / 2; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t][2 * i], cexp, -m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t][2 * i + 1], cexp, -m));
        pk[t][i] = pack_bf16x2(p0, p1);
        // row sum of the bf16 weights that PV uses: p0 + p1 in one dot2
        lsum[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[t][i]),
                                                   kOnes, lsum[t], false);
      }
    }
    // O^T += V^T . P^T, two 16-key halves (granules 2*tile and 2*tile + 1)
#pragma unroll
    for (int h = 0; h < (HALF ? 1 : 2); ++h) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + vl + h * VG_B + L.vofs[dt]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 b = __builtin_bit_cast(
              bf16x8, make_uint4(pk[t][4 * h], pk[t][4 * h + 1], pk[t][4 * h + 2],
                                 pk[t][4 * h + 3]));
          o[t][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[t][dt], 0, 0, 0);
        }
      }
    }
  }

  // ---- software-pipelined fixed-maximum stage for two query tiles per wave ----
  // Within a 32-key tile the MFMA work of one query tile overlaps the softmax
  // VALU work of the other:  QK(q0) | QK(q1) + softmax(q0) + V^T loads |
  // PV(q0) + softmax(q1) + next K loads | PV(q1). sched_group_barrier pins the
  // interleave (1 MFMA : 1 LDS read : 6 VALU), which matches 8 MFMAs (256
  // cycles) with one query tile's softmax (48 VALU).
  struct KFrag {
    bf16x8 a[KS];
  };
  struct VFrag {
    bf16x8 a[2][DT];
  };

  __device__ static inline void load_k(KFrag& f, const char* lds, const Lane& L, int kl) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) f.a[ks] = *reinterpret_cast<const bf16x8*>(lds + kl + L.kofs[ks]);
  }
  __device__ static inline void load_v(VFrag& f, const char* lds, const Lane& L, int vl) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        f.a[h][dt] = *reinterpret_cast<const bf16x8*>(lds + vl + h * VG_B + L.vofs[dt]);
  }
  __device__ static inline f32x16 qk(const KFrag& f, const bf16x8 (&q)[KS]) {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks], q[ks], s, 0, 0, 0);
    return s;
  }
  __device__ static inline void softmax_fixed(const f32x16& s, float m, float& l, uint32_t (&pk)[8],
                                              float cexp) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[2 * i], cexp, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[2 * i + 1], cexp, -m));
      pk[i] = pack_bf16x2(p0, p1);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), kOnes, l, false);
    }
  }
  __device__ static inline void pv(const VFrag& f, const uint32_t (&pk)[8], f32x16 (&o)[DT]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, make_uint4(pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[h][dt], b, o[dt], 0, 0, 0);
    }
  }
  // 8 MFMAs, 8 LDS reads and 48 VALU ops in lock step
  __device__ static inline void interleave_8() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
    }
  }

  // One pipelined region: its 16 operand reads first (the other wave of the
  // SIMD runs its MFMAs meanwhile), then 16 MFMAs with 3 VALU ops behind each
  // (one 32x32x16 MFMA hides about four plain VALU ops or two exponentials
  // when two waves share the SIMD).
  __device__ static inline void interleave_16() {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i == 0) __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    }
  }

  // Region with V^T one region ahead: the 8 K reads of QK(j+1) first, then the 16 MFMAs
  // with 3 VALU ops behind each, and the 8 reads of the next tile's V^T operand placed
  // after the PV MFMAs that consume the same registers.
  __device__ static inline void interleave_kv() {
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // DS read: K
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i >= 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read: V^T
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    }
  }

  // Both 32-key tiles of one stage (K at kl, V^T at vl), QT == 2, fixed maximum.
  __device__ static inline void stage2_fixed(const char* lds, const Lane& L, int kl, int vl,
                                             const bf16x8 (&qf)[2][KS], f32x16 (&o)[2][DT],
                                             const float (&mrow)[2], float (&lsum)[2],
                                             float cexp) {
    KFrag kf;
    VFrag vf;
    uint32_t p0[8], p1[8];
    load_k(kf, lds, L, kl);
    f32x16 s0 = qk(kf, qf[0]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      __builtin_amdgcn_sched_barrier(0);
      // A: QK(q1) + softmax(q0) + V^T loads of this tile
      f32x16 s1 = qk(kf, qf[1]);
      softmax_fixed(s0, mrow[0], lsum[0], p0, cexp);
      load_v(vf, lds, L, vl + tt * 2 * VG_B);
      interleave_8();
      __builtin_amdgcn_sched_barrier(0);
      // B: PV(q0) + softmax(q1) + K loads of the next tile
      pv(vf, p0, o[0]);
      softmax_fixed(s1, mrow[1], lsum[1], p1, cexp);
      if (tt == 0) {
        load_k(kf, lds, L, kl + 32 * ROWB);
        interleave_8();
      }
      __builtin_amdgcn_sched_barrier(0);
      // C: PV(q1), then QK(q0) of the next tile
      pv(vf, p1, o[1]);
      if (tt == 0) s0 = qk(kf, qf[0]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Streams all visible key granules of the item once for NT of the wave's
  // query tiles (t0 .. t0 + NT - 1).
  template <bool ONLINE, int NT>
  __device__ static void run(const FwdParams& p, const Item& it, char* lds, int t0) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const KeyRanges r = it.half < 0 ? sfa::key_ranges(it.f, p.F, p.T, p.w)
                                    : sfa::half_key_ranges(it.f, it.half, p.F, p.T, p.w);
    const int ngran = (r.r0_end + (r.r1_end - r.r1_begin)) / 16;
    const char* kb = reinterpret_cast<const char*>(p.k + it.b * p.ksb + it.h * p.ksh);
    const char* vtb =
        reinterpret_cast<const char*>(p.vt + (int64_t(it.b) * p.H + it.h) * D * p.S);

    const int rows = min(p.gq * 16, p.T - it.qb * p.gq * 16);  // real rows of this item
    const int row0 = it.f * p.T + it.qb * p.gq * 16;
    const int64_t rowstat = (int64_t(it.b) * p.H + it.h) * p.S;
    const float kmax = p.kvis[(int64_t(it.b) * p.H + it.h) * (p.F + 1) + it.f];
    // a wave whose query tiles hold no real row only helps with the DMA (wave-uniform)
    const bool active = __builtin_amdgcn_readfirstlane((wave * QT + t0) * 32) < rows;

    Lane L;
    Slots W;
    lane_setup(L, W, p.kss, p.S);
    Src X;
    X.k = kb;
    X.v = vtb;
    X.kss2 = p.kss * 2;
    X.n0 = r.r0_end / 16;
    X.shift = r.r1_begin - r.r0_end;

    bf16x8 qf[NT][KS];
    float mrow[NT], lsum[NT];
    f32x16 o[NT][DT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int lr = min((wave * QT + t0 + t) * 32 + l32, rows - 1);  // repeats past the end
      const int row = row0 + lr;
      const uint16_t* qp = p.q + it.b * p.qsb + int64_t(row) * p.qss + it.h * p.qsh + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[t][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 16 * ks));
      mrow[t] = ONLINE ? -__builtin_inff()
                       : (p.qmu[rowstat + row] + p.qn[rowstat + row] * kmax) * p.c;
      lsum[t] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][dt][i] = 0.f;
    }

    const int nfull = ngran / 4;
    const int rem = ngran - nfull * 4;
    const int nst = nfull + (rem > 0 ? 1 : 0);
    if constexpr (!ONLINE && NT == 1 && (NBUF == 3 || NBUF == 4)) {
      // Tile-level software pipeline over the N = 2*nfull full 32-key tiles:
      //   region j:  QK(j+1) + PV(j-1)  (16 MFMAs)  ||  softmax(j)  (48 VALU)
      // Region j reads K(j+1) for its own QK and V^T(j) for the PV of region j+1,
      // so the V^T reads have a whole region to land. Stage s (tiles 2s, 2s+1)
      // sits in buffer s % NBUF; barrier B_s, just before the region that first
      // reads stage s, waits for its DMA and then launches the DMA of stage
      // s + NBUF - 2 into the buffer of stage s - 2, whose last read (V^T of tile
      // 2s - 3, in region 2s - 3) was consumed by the PV of region 2s - 2, before B_s.
      // So NBUF - 2 stages are in flight while one is read.
      constexpr int AH = NBUF - 2;
      // wait for stage sn's DMA: with AH == 2 the next stage's (DMA_W per wave when it is
      // a full stage) may stay in flight
      auto wait_stage = [&](int sn) {
        if (AH == 2 && sn + 1 < nfull)
          wait_vm<(AH - 1) * DMA_W>();
        else
          wait_vm<0>();
      };
      const int N = 2 * nfull;
      f32x16(&oo)[DT] = o[0];
      if (N > 0) {
        issue_stage(lds, 0, L, W, X, 0, 4);
        wait_vm<0>();
        __syncthreads();
#pragma unroll
        for (int a = 1; a <= AH; ++a)
          if (a < nst) issue_stage(lds, a, L, W, X, a, a < nfull ? 4 : rem);
      }
      if (N > 0 && !active) {
        // no real row: the same DMA issues and barriers as the regions below, no compute
        for (int j = 1; j < N - 1; j += 2) {
          const int sn = (j + 1) / 2;
          wait_stage(sn);
          __syncthreads();
          if (sn + AH < nst)
            issue_stage(lds, (sn + AH) % NBUF, L, W, X, sn + AH, sn + AH < nfull ? 4 : rem);
        }
      } else if (N > 0) {
        KFrag kf;
        VFrag vf;
        uint32_t pprev[8], pcur[8];
        load_k(kf, lds, L, 0);
        f32x16 scur = qk(kf, qf[0]);
        // region 0: QK(1) + softmax(0)
        __builtin_amdgcn_sched_barrier(0);
        load_k(kf, lds, L, 32 * ROWB);
        f32x16 snext = qk(kf, qf[0]);
        load_v(vf, lds, L, 0);  // V^T(0), used by PV(0) in region 1
        softmax_fixed(scur, mrow[0], lsum[0], pprev, p.c);
        scur = snext;
        __builtin_amdgcn_sched_barrier(0);
        // steady regions j = 1 .. N-2, unrolled over the 2*NBUF-tile period of (buffer, half)
        for (int j0 = 1; j0 < N - 1; j0 += 2 * NBUF) {
#pragma unroll
          for (int u = 0; u < 2 * NBUF; ++u) {
            const int j = j0 + u;
            if (j >= N - 1) break;
            if ((u & 1) == 0) {  // j odd: tile j+1 opens stage (j+1)/2
              const int sn = (j + 1) / 2;
              wait_stage(sn);
              __syncthreads();
              if (sn + AH < nst)
                issue_stage(lds, (sn + AH) % NBUF, L, W, X, sn + AH, sn + AH < nfull ? 4 : rem);
            }
            // tile j+1 = 1 + u + 1 and tile j = 1 + u (mod 2*NBUF)
            const int bn = ((u + 2) / 2) % NBUF, tn = (u + 2) & 1;
            const int bc = ((u + 1) / 2) % NBUF, tc = (u + 1) & 1;
            __builtin_amdgcn_sched_barrier(0);
            load_k(kf, lds, L, bn * STAGE_B + tn * 32 * ROWB);
            snext = qk(kf, qf[0]);
            pv(vf, pprev, oo);                                 // V^T(j-1), read last region
            load_v(vf, lds, L, bc * STAGE_B + tc * 2 * VG_B);  // V^T(j) for the next region
            softmax_fixed(scur, mrow[0], lsum[0], pcur, p.c);
            interleave_kv();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; ++i) pprev[i] = pcur[i];
            scur = snext;
          }
        }
        // region N-1: PV(N-2) + softmax(N-1); then PV(N-1)
        {
          const int jm = N - 2;  // tiles N-2 and N-1 are the two halves of stage nfull-1
          const int b = ((jm / 2) % NBUF);
          pv(vf, pprev, oo);     // V^T(N-2), read in region N-2
          softmax_fixed(scur, mrow[0], lsum[0], pcur, p.c);
          load_v(vf, lds, L, b * STAGE_B + 2 * VG_B);
          pv(vf, pcur, oo);
        }
      } else if (nst > 0) {
        issue_stage(lds, 0, L, W, X, 0, rem);
      }
      if (rem > 0) {
        wait_vm<0>();
        __syncthreads();
        const int kl = (nfull % NBUF) * STAGE_B;
        if (!active) {
        } else if (rem >= 2) {
          tile<false, ONLINE, NT>(lds, L, kl, kl, qf, o, mrow, lsum, p.c);
        } else {
          tile<true, ONLINE, NT>(lds, L, kl, kl, qf, o, mrow, lsum, p.c);
        }
        if (active && rem == 3)
          tile<true, ONLINE, NT>(lds, L, kl + 32 * ROWB, kl + 2 * VG_B, qf, o, mrow, lsum, p.c);
      }
    } else {
    // Stages of 64 keys; NBUF of them in flight. Iteration s waits for stage s
    // (only the DMAs of younger stages may still be outstanding), crosses one
    // barrier (stage s visible to all waves, stage s-1's buffer free), refills
    // that buffer with stage s + NBUF - 1 and computes stage s. The 1..3
    // granule tail stage is computed after the loop.
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j)
      if (j < nst) issue_stage(lds, j, L, W, X, j, j < nfull ? 4 : rem);

    for (int s0 = 0; s0 < nfull; s0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int s = s0 + u;
        if (s >= nfull) break;
        if (s + NBUF - 2 < nfull)
          wait_vm<(NBUF - 2) * DMA_W>();
        else
          wait_vm<0>();
        __syncthreads();
        const int sn = s + NBUF - 1;
        if (sn < nst)
          issue_stage(lds, (u + NBUF - 1) % NBUF, L, W, X, sn, sn < nfull ? 4 : rem);
        if (active) {
          const int kl = u * STAGE_B;  // K and V^T stage offsets
          if constexpr (!ONLINE && NT == 2) {
            stage2_fixed(lds, L, kl, kl, qf, o, mrow, lsum, p.c);
          } else {
            tile<false, ONLINE, NT>(lds, L, kl, kl, qf, o, mrow, lsum, p.c);
            tile<false, ONLINE, NT>(lds, L, kl + 32 * ROWB, kl + 2 * VG_B, qf, o, mrow, lsum,
                                    p.c);
          }
        }
      }
    }
    if (rem > 0) {
      wait_vm<0>();
      __syncthreads();
      if (active) {
        const int kl = (nfull % NBUF) * STAGE_B;
        const int vl = kl;
        if (rem >= 2)
          tile<false, ONLINE, NT>(lds, L, kl, vl, qf, o, mrow, lsum, p.c);
        else
          tile<true, ONLINE, NT>(lds, L, kl, vl, qf, o, mrow, lsum, p.c);
        if (rem == 3)
          tile<true, ONLINE, NT>(lds, L, kl + 32 * ROWB, vl + 2 * VG_B, qf, o, mrow, lsum, p.c);
      }
    }

    }

    if (it.half >= 0) {  // a key half (the plan splits 8-wave items only: NT == 1)
      if constexpr (NT == 1 && QT == 1) merge_halves(p, it, o[0], lsum[0], mrow[0], rows, row0);
      return;
    }

    // epilogue: the two lane halves hold the two key halves of every row
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float l = lsum[t] + __shfl_xor(lsum[t], 32, 64);
      const float inv = 1.0f / l;
      const int lr = (wave * QT + t0 + t) * 32 + l32;
      if (lr < rows) {
        uint16_t* op = p.o + it.b * p.osb + int64_t(row0 + lr) * p.oss + it.h * p.osh + 4 * g;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            uint2 w;
            w.x = pack_bf16x2(o[t][dt][4 * m] * inv, o[t][dt][4 * m + 1] * inv);
            w.y = pack_bf16x2(o[t][dt][4 * m + 2] * inv, o[t][dt][4 * m + 3] * inv);
            *reinterpret_cast<uint2*>(op + 32 * dt + 8 * m) = w;
          }
      }
    }
  }

  // Epilogue of one key half of a split item. The half leaves its partial output O
  // (not normalised), row sum l and the maximum m they are relative to in the
  // workspace, then counts itself in; the half that comes second reads the other's
  // partial and writes O = (O_0 s_0 + O_1 s_1) / (l_0 s_0 + l_1 s_1) with
  // s_h = 2^(m_h - max(m_0, m_1)) (s_h = 1 for a shared fixed maximum), always in half
  // order, so the result does not depend on which half finished first. The halves may
  // run on different XCDs, whose L2 caches are not coherent with each other: the partial
  // goes out with device-scope (write-through) stores, every one of them acknowledged
  // before the count, and the second half reads it with device-scope loads. A device-scope
  // fence would do the same by writing back and invalidating the whole L2 of the XCD,
  // which costs its other workgroups their cached K and V^T. The second half clears the
  // count for the next launch.
  __device__ static void merge_halves(const FwdParams& p, const Item& it, const f32x16 (&o)[DT],
                                      float lpart, float m, int rows, int row0) {
    constexpr int PF = sfa::part_floats(D);
    constexpr int WF = DT * 16 * 64;  // floats of one wave's O
    constexpr int OL = 8 * WF;        // l of 256 rows, then m
    __shared__ int split_seen;
    // thread index re-read here (an empty asm the compiler cannot see through), so that
    // these lane addresses are not hoisted out of the item loop, where they would stay
    // live across the key loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    const float l = lpart + __shfl_xor(lpart, 32, 64);
    const int slot = ((it.split * p.B + it.b) * p.H + it.h) * p.nqb + it.qb;
    float* mine = p.part + (int64_t(slot) * 2 + it.half) * PF;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __hip_atomic_store(&mine[wave * WF + (dt * 16 + i) * 64 + lane], o[dt][i],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int row = wave * 32 + l32;
    if (g == 0) {
      __hip_atomic_store(&mine[OL + row], l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&mine[OL + 256 + row], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vm<0>();  // every store of this wave acknowledged
    __syncthreads();
    if (tid == 0) split_seen = atomicAdd(&p.split_cnt[slot], 1);
    __syncthreads();
    const int first = split_seen == 0;
    __syncthreads();
    if (first) return;
    if (tid == 0) atomicExch(&p.split_cnt[slot], 0);
    float* other = p.part + (int64_t(slot) * 2 + (1 - it.half)) * PF;
    const float lo = __hip_atomic_load(&other[OL + row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float mo = __hip_atomic_load(&other[OL + 256 + row], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    const bool h0 = it.half == 0;
    const float m0 = h0 ? m : mo, m1 = h0 ? mo : m;
    const float l0 = h0 ? l : lo, l1 = h0 ? lo : l;
    const float mm = fmaxf(m0, m1);
    const float s0 = __builtin_amdgcn_exp2f(m0 - mm), s1 = __builtin_amdgcn_exp2f(m1 - mm);
    const float inv = 1.0f / (l0 * s0 + l1 * s1);
    if (row >= rows) return;
    uint16_t* op = p.o + it.b * p.osb + int64_t(row0 + row) * p.oss + it.h * p.osh + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = 4 * q4 + u;
          const float a = o[dt][i];
          const float b = __hip_atomic_load(&other[wave * WF + (dt * 16 + i) * 64 + lane],
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          y[u] = ((h0 ? a : b) * s0 + (h0 ? b : a) * s1) * inv;
        }
        uint2 wv;
        wv.x = pack_bf16x2(y[0], y[1]);
        wv.y = pack_bf16x2(y[2], y[3]);
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * q4) = wv;
      }
  }

  // Fixed maximum: every query tile of the wave in one pass over the keys.
  __device__ static void run_fixed(const FwdParams& p, const Item& it, char* lds) {
    run<false, QT>(p, it, lds, 0);
  }

  // Online softmax rescales the accumulators with VALU work, so it holds one
  // query tile at a time (QT passes over the keys).
  __device__ static void run_online(const FwdParams& p, const Item& it, char* lds) {
#pragma unroll
    for (int t0 = 0; t0 < QT; ++t0) {
      if (t0 > 0) __syncthreads();  // the next pass refills the LDS stages
      run<true, 1>(p, it, lds, t0);
    }
  }
};


}  // namespace
