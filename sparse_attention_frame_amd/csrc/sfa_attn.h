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
// Staging: the memory-bound prologue (sfa_norms) copies K and V into the workspace in
// the byte order of the LDS stages (sfa_internal.h: K as [granule][16-byte chunk][16 keys],
// V transposed as [granule][d][16 keys] with the halves of odd 8-row groups swapped, since
// LDS transpose reads run at well under half the rate of plain 16-byte reads on gfx950).
// Granules then go from HBM straight into LDS by DMA (buffer_load_dwordx4 ... lds: no
// registers, no VALU), 1 KB of contiguous bytes per request, in NBUF rotating 64-key stages;
// 16 lanes reading one operand hit 16 distinct 16-byte bank groups.
#include "sfa_gfx950.h"

namespace {

using sfa::FwdParams;
using sfa::Item;
using sfa::KeyRanges;

// (1.0, 1.0) in bf16: dot2 with it adds the two halves of a packed pair
constexpr bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};


// Online softmax keeps a stale running maximum until a tile's maximum exceeds it by
// more than kLazy (log2 units). P then stays below 2^kLazy, which bf16 and the fp32
// sums hold with unchanged relative precision: with fewer than 2^24 keys per row,
// l < 2^88 and |O| < 2^88 * max|v|, far below 2^127 for any bf16 v up to 2^38. A large
// kLazy makes rescales rare when the scores are wide.
constexpr float kLazy = 64.0f;

// The larger of a lane's value and that of lane ^ 32 (the other key half of the same
// query row): one v_permlane32_swap, no LDS round trip.
__device__ inline float max_xor32(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, uint32_t(r[0])), __builtin_bit_cast(float, uint32_t(r[1])));
}


template <int D, int WAVES, int QT, int NBUF>
struct Attn {
  static constexpr int kThreads = WAVES * 64;
  // The fixed-maximum path with two query tiles per wave runs every stage, the partial
  // last one included, through one code shape (masked tail): with 64 query rows a wave's
  // accumulators, Q and scores fill its 256 registers, and a separate tail would make
  // the compiler spill them.
  static constexpr bool kMaskTail = QT == 2;
  static constexpr int KS = D / 16;             // 16-dim k-steps of QK^T
  static constexpr int DT = D / 32;             // 32-dim tiles of O^T
  // LDS stages copy the staged HBM layouts (sfa_internal.h) granule by granule:
  //   K   [granule][16-byte chunk c][16 keys]: the operand of k-step ks for a lane is its
  //        key's row, chunk 2ks + g, at a fixed lane offset + 512 * ks;
  //   V^T [granule][d][16 keys], 16-byte halves swizzled by (d / 8) % 2.
  // 16 lanes reading one chunk of 16 keys, or one half of 16 V^T rows, hit 16 distinct
  // 16-byte bank groups.
  static constexpr int GB = sfa::staged_granule_bytes(D);   // bytes of one staged granule
  // keys per LDS stage: 64 (4 granules, 2 tiles of 32); 96 with 12 waves, so that a
  // stage's DMA requests split evenly over the waves
  static constexpr int SK = WAVES == 12 ? 96 : 64;
  static constexpr int GPS = SK / 16;                        // granules per stage
  static constexpr int TPS = SK / 32;                        // 32-key tiles per stage
  static constexpr int STAGE_B = GPS * GB;                   // bytes per tensor per stage
  static constexpr int DMA_G = GB / 1024;                    // DMA requests per granule
  static constexpr int DMA_N = 2 * GPS * DMA_G;              // K + V requests per stage
  static constexpr int LDS_BYTES = NBUF * 2 * STAGE_B;       // NBUF stages of K and V
  // LDS layout: K stage buffers [0, NBUF*STAGE_B), V^T stage buffers after them.
  // Lane offsets of V^T reads include VBASE so every operand read is a base
  // register plus an immediate below 64 KB.
  static constexpr int VBASE = NBUF * STAGE_B;
  static_assert(DMA_N % WAVES == 0, "DMA requests split evenly over waves");

  static constexpr int DMA_W = DMA_N / WAVES;                // DMA requests per wave

  __device__ static inline int vt_half(int d, int half) { return half ^ ((d >> 3) & 1); }
  // key fed to S^T MFMA row rho (see the header)
  __device__ static inline int key_of_row(int rho) {
    const int m = rho >> 3, gg = (rho >> 2) & 1, i = rho & 3;
    return 16 * (m >> 1) + 8 * gg + 4 * (m & 1) + i;
  }

  // Per-lane constants of the hot loop: with the staged layouts every LDS read in the
  // loop is one of these registers plus an immediate, and every DMA request moves
  // 16 bytes per lane at lane * 16 from a uniform (SGPR) source address.
  struct Lane {
    uint32_t kofs;           // K operand byte offset of k-step 0 in a stage's first tile
    uint32_t vofs;           // VBASE + V^T operand offset inside a granule, 32-dim tile 0
                             // (tile dt adds dt * 1024, the second 16-key half adds GB)
    uint32_t dma;            // lane * 16: a lane's bytes in every DMA request
  };

  // Wave-uniform per kernel: the DMA requests of this wave inside a stage. Request
  // m = wave * DMA_W + i copies 1 KB: tensor m / (DMA_N / 2) (0 K, 1 V), stage granule
  // (m % (DMA_N / 2)) / DMA_G, kilobyte (m % DMA_G) of that granule.
  struct Slots {
    int gi[DMA_W];           // stage granule of request i
    int src[DMA_W];          // byte offset of request i inside its granule (kilobyte * 1024)
    int dst[DMA_W];          // LDS byte offset of request i inside a stage buffer
    bool v[DMA_W];           // request i copies V (else K)
  };

  // Key source of one item: granule gi of the item starts at token 16*gi before the
  // seam (the end of the first key range) and 16*gi + shift after it.
  struct Src {
    const char* k;           // staged K of this (b, h)
    const char* v;           // staged V of this (b, h)
    int n0;                  // first granule past the seam
    int gshift;              // granule shift of granules at or past the seam
  };

  __device__ static inline void lane_setup(Lane& L, Slots& W) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int krow = key_of_row(l32);
    L.kofs = (krow >> 4) * GB + g * 256 + (krow & 15) * 16;
    L.vofs = VBASE + l32 * 32 + vt_half(l32, g) * 16;
    L.dma = lane * 16;
#pragma unroll
    for (int i = 0; i < DMA_W; ++i) {
      const int m = wave * DMA_W + i;
      const int r = m % (DMA_N / 2);
      W.v[i] = m >= DMA_N / 2;
      W.gi[i] = r / DMA_G;
      W.src[i] = (r % DMA_G) * 1024;
      W.dst[i] = (W.v[i] ? VBASE : 0) + W.gi[i] * GB + (r % DMA_G) * 1024;
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
  // after unrolling): every request copies one contiguous kilobyte of a staged granule.
  // With fill, the stage's other granules receive a copy of its last one (finite
  // operands for a tile whose second granule is masked).
  __device__ static inline void issue_stage(char* lds, int buf, const Lane& L, const Slots& W,
                                            const Src& X, int s, int ng, bool fill = false) {
    char* lb = lds + buf * STAGE_B;  // + VBASE for V^T (inside dst)
#pragma unroll
    for (int i = 0; i < DMA_W; ++i) {
      if (W.gi[i] >= ng && !fill) continue;
      const int gr = GPS * s + min(W.gi[i], ng - 1);   // granule of the item
      const int gs = gr >= X.n0 ? gr + X.gshift : gr;  // granule of the (b, h) sequence
      dma16((W.v[i] ? X.v : X.k) + int64_t(gs) * GB + W.src[i], L.dma, lb + W.dst[i]);
    }
  }

  // One 32-key tile (HALF: only its first 16 keys exist) for the wave's NT query tiles.
  // kl / vl: LDS byte offsets of the tile's first K and V^T granules.
  // hi_valid (full tiles only): false when the tile's second granule holds no visible
  // key (the last stage of an item with an odd granule count, where the DMA has copied a
  // visible granule in its place so every operand is finite); its 16 weights are then
  // exp2(-inf) = 0 and add nothing to O or l.
  template <bool HALF, bool ONLINE, int NT>
  __device__ static inline void tile(const char* lds, const Lane& L, int kl, int vl,
                                     const bf16x8 (&qf)[NT][KS], f32x16 (&o)[NT][DT],
                                     float (&mrow)[NT], float (&lsum)[NT], float cexp,
                                     bool hi_valid = true) {
    // S^T = K . Q^T
    f32x16 s[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[t][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + kl + L.kofs + 512 * ks);
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
        mx = max_xor32(mx) * cexp;
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
      const float mh = hi_valid ? m : __builtin_inff();  // subtrahend of the second granule
#pragma unroll
      for (int i = 0; i < NV / 2; ++i) {
        const float mi = i < 4 ? m : mh;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t][2 * i], cexp, -mi));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t][2 * i + 1], cexp, -mi));
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
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + vl + h * GB + dt * 1024 + L.vofs);
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

  // ---- pieces of the software-pipelined fixed-maximum loop (one query tile per wave) ----
  struct KFrag {
    bf16x8 a[KS];
  };
  struct VFrag {
    bf16x8 a[2][DT];
  };

  __device__ static inline void load_k(KFrag& f, const char* lds, const Lane& L, int kl) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      f.a[ks] = *reinterpret_cast<const bf16x8*>(lds + kl + L.kofs + 512 * ks);
  }
  __device__ static inline void load_v(VFrag& f, const char* lds, const Lane& L, int vl) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        f.a[h][dt] = *reinterpret_cast<const bf16x8*>(lds + vl + h * GB + dt * 1024 + L.vofs);
  }
  __device__ static inline f32x16 qk(const KFrag& f, const bf16x8 (&q)[KS]) {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks], q[ks], s, 0, 0, 0);
    return s;
  }
  // Numerators and their row sum, which two accumulators split (even and odd pairs) so
  // that the chain of dependent dot2 operations is half as long.
  __device__ static inline void softmax_fixed(const f32x16& s, float m, float& l, float& l2,
                                              uint32_t (&pk)[8], float cexp) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[2 * i], cexp, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[2 * i + 1], cexp, -m));
      pk[i] = pack_bf16x2(p0, p1);
      float& acc = (i & 1) ? l2 : l;
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), kOnes, acc, false);
    }
  }
  // Online numerators of one tile for the pipelined loop. The running maximum is lazy per
  // row and branch-free: a row whose tile maximum exceeds it by more than kLazy takes the
  // tile maximum, the others keep theirs (alpha = exp2(0) = 1). The row sum is rescaled
  // here; the returned alpha rescales the row's O once the PV of the previous tile, which
  // is still relative to the old maximum, has been added.
  __device__ static inline float softmax_online(const f32x16& s, float& m, float& l, float& l2,
                                                uint32_t (&pk)[8], float cexp) {
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = max_xor32(mx) * cexp;
    const float mnew = mx > m + kLazy ? mx : m;
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    l *= alpha;
    l2 *= alpha;
    softmax_fixed(s, m, l, l2, pk, cexp);
    return alpha;
  }
  __device__ static inline void rescale(f32x16 (&o)[DT], float alpha) {
    if (__ballot(alpha != 1.0f) != 0) {  // rare: a row moved its maximum
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
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
  // Region with V^T one region ahead: the 8 K reads of QK(j+1) first, then the 16 MFMAs
  // with VALU ops behind each (3 on the fixed-maximum path, 4 on the online one), and the
  // 8 reads of the next tile's V^T operand placed after the PV MFMAs that consume the same
  // registers.
  template <int VALU>
  __device__ static inline void interleave_kv() {
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // DS read: K
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i >= 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read: V^T
      __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);  // VALU
    }
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
    const int64_t bh_elems = (int64_t(it.b) * p.H + it.h) * p.S * D;  // staged (b, h) start

    const int rows = min(p.gq * 16, p.T - it.qb * p.gq * 16);  // real rows of this item
    const int row0 = it.f * p.T + it.qb * p.gq * 16;
    const int64_t rowstat = (int64_t(it.b) * p.H + it.h) * p.S;
    const float kmax = p.kvis[(int64_t(it.b) * p.H + it.h) * (p.F + 1) + it.f];
    // a wave whose query tiles hold no real row only helps with the DMA (wave-uniform);
    // a second tile without real rows is computed on repeated rows and never stored
    const bool active = __builtin_amdgcn_readfirstlane((wave * QT + t0) * 32) < rows;

    Lane L;
    Slots W;
    lane_setup(L, W);
    Src X;
    X.k = reinterpret_cast<const char*>(p.kst + bh_elems);
    X.v = reinterpret_cast<const char*>(p.vst + bh_elems);
    X.n0 = r.r0_end / 16;
    X.gshift = (r.r1_begin - r.r0_end) / 16;

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

    const int nfull = ngran / GPS;
    const int rem = ngran - nfull * GPS;
    const int nst = nfull + (rem > 0 ? 1 : 0);
    if constexpr (NT == 1 && TPS == 2 && (NBUF == 3 || NBUF == 4)) {
      // Tile-level software pipeline over the N = 2*nfull full 32-key tiles:
      //   region j:  QK(j+1) + PV(j-1)  (16 MFMAs)  ||  softmax(j)  (48 VALU; some 30
      //   more with the online maximum, whose O rescale, if any row moved its maximum,
      //   follows the region's PV)
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
          if (a < nst) issue_stage(lds, a, L, W, X, a, a < nfull ? GPS : rem);
      }
      if (N > 0 && !active) {
        // no real row: the same DMA issues and barriers as the regions below, no compute
        for (int j = 1; j < N - 1; j += 2) {
          const int sn = (j + 1) / 2;
          wait_stage(sn);
          __syncthreads();
          if (sn + AH < nst)
            issue_stage(lds, (sn + AH) % NBUF, L, W, X, sn + AH, sn + AH < nfull ? GPS : rem);
        }
      } else if (N > 0) {
        KFrag kf;
        VFrag vf;
        uint32_t pprev[8], pcur[8];
        float l2 = 0.f;  // second row-sum accumulator
        load_k(kf, lds, L, 0);
        f32x16 scur = qk(kf, qf[0]);
        // region 0: QK(1) + softmax(0)
        __builtin_amdgcn_sched_barrier(0);
        load_k(kf, lds, L, 2 * GB);
        f32x16 snext = qk(kf, qf[0]);
        load_v(vf, lds, L, 0);  // V^T(0), used by PV(0) in region 1
        if constexpr (ONLINE)
          softmax_online(scur, mrow[0], lsum[0], l2, pprev, p.c);  // O is still zero
        else
          softmax_fixed(scur, mrow[0], lsum[0], l2, pprev, p.c);
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
                issue_stage(lds, (sn + AH) % NBUF, L, W, X, sn + AH, sn + AH < nfull ? GPS : rem);
            }
            // tile j+1 = 1 + u + 1 and tile j = 1 + u (mod 2*NBUF)
            const int bn = ((u + 2) / 2) % NBUF, tn = (u + 2) & 1;
            const int bc = ((u + 1) / 2) % NBUF, tc = (u + 1) & 1;
            __builtin_amdgcn_sched_barrier(0);
            load_k(kf, lds, L, bn * STAGE_B + tn * 2 * GB);
            snext = qk(kf, qf[0]);
            pv(vf, pprev, oo);                                 // V^T(j-1), read last region
            load_v(vf, lds, L, bc * STAGE_B + tc * 2 * GB);  // V^T(j) for the next region
            if constexpr (ONLINE) {
              const float alpha = softmax_online(scur, mrow[0], lsum[0], l2, pcur, p.c);
              interleave_kv<4>();
              __builtin_amdgcn_sched_barrier(0);
              rescale(oo, alpha);
            } else {
              softmax_fixed(scur, mrow[0], lsum[0], l2, pcur, p.c);
              interleave_kv<3>();
            }
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
          if constexpr (ONLINE)
            rescale(oo, softmax_online(scur, mrow[0], lsum[0], l2, pcur, p.c));
          else
            softmax_fixed(scur, mrow[0], lsum[0], l2, pcur, p.c);
          load_v(vf, lds, L, b * STAGE_B + 2 * GB);
          pv(vf, pcur, oo);
        }
        lsum[0] += l2;
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
          tile<true, ONLINE, NT>(lds, L, kl + 2 * GB, kl + 2 * GB, qf, o, mrow, lsum, p.c);
      }
    } else if constexpr (kMaskTail && !ONLINE) {
      static_assert(GPS == 4, "the masked stage loop takes two tiles per stage");
    // Stages of 64 keys, NBUF - 1 of them in flight, one code shape for every stage: the
    // last stage of an item whose granule count is not a multiple of 4 is filled with
    // copies of its last granule and computed as whole tiles, the copies' weights masked
    // to zero or the tile skipped. Iteration s waits for stage s (the younger stages'
    // DMAs may stay in flight), crosses one barrier (stage s visible to all waves, the
    // buffer of stage s - 1 free), refills that buffer with stage s + NBUF - 1 and
    // computes stage s; unrolled over the NBUF buffers so that every LDS offset is an
    // immediate.
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j)
      if (j < nst) issue_stage(lds, j, L, W, X, j, j < nfull ? GPS : rem, true);
    for (int s0 = 0; s0 < nst; s0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int s = s0 + u;
        if (s >= nst) break;
        if (s + NBUF - 2 < nst)
          wait_vm<(NBUF - 2) * DMA_W>();
        else
          wait_vm<0>();
        __syncthreads();
        const int sn = s + NBUF - 1;
        if (sn < nst)
          issue_stage(lds, (u + NBUF - 1) % NBUF, L, W, X, sn, sn < nfull ? GPS : rem, true);
        if (active) {
          const int kl = u * STAGE_B;          // K and V^T stage offsets
          const int ng = s < nfull ? GPS : rem;  // visible granules of this stage (GPS == 4)
          tile<false, false, NT>(lds, L, kl, kl, qf, o, mrow, lsum, p.c, ng >= 2);
          if (ng >= 3)
            tile<false, false, NT>(lds, L, kl + 2 * GB, kl + 2 * GB, qf, o, mrow, lsum, p.c,
                                   ng == 4);
        }
      }
    }
    } else {
    // Stages of 64 keys (the last one holds the 1..3 granules left, if any), NBUF - 1 of
    // them in flight. Iteration s waits for stage s (only the DMAs of younger full
    // stages may still be outstanding), crosses one barrier (stage s visible to all
    // waves, the buffer of stage s - 1 free), refills that buffer with stage
    // s + NBUF - 1 and computes stage s; unrolled over the NBUF buffers so that every
    // LDS offset is an immediate. The partial last stage is computed after the loop.
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j)
      if (j < nst) issue_stage(lds, j, L, W, X, j, j < nfull ? GPS : rem);

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
          issue_stage(lds, (u + NBUF - 1) % NBUF, L, W, X, sn, sn < nfull ? GPS : rem);
        if (active) {
          const int kl = u * STAGE_B;  // K and V^T stage offsets
#pragma unroll
          for (int tt = 0; tt < TPS; ++tt)
            tile<false, ONLINE, NT>(lds, L, kl + tt * 2 * GB, kl + tt * 2 * GB, qf, o, mrow,
                                    lsum, p.c);
        }
      }
    }
    if (rem > 0) {  // the 1..GPS-1 granules of the last stage, in buffer nfull % NBUF
      wait_vm<0>();
      __syncthreads();
      if (active) {
        // one copy per buffer, so that the LDS offsets stay immediates
#pragma unroll
        for (int u = 0; u < NBUF; ++u)
          if (u == nfull % NBUF) {
            const int kl = u * STAGE_B;
#pragma unroll
            for (int tt = 0; tt < TPS; ++tt) {
              const int tl = kl + tt * 2 * GB;
              if (2 * tt + 2 <= rem)
                tile<false, ONLINE, NT>(lds, L, tl, tl, qf, o, mrow, lsum, p.c);
              else if (2 * tt + 1 == rem)
                tile<true, ONLINE, NT>(lds, L, tl, tl, qf, o, mrow, lsum, p.c);
            }
          }
      }
    }

    }

    if (it.half >= 0) {  // a key half (the plan splits the items of 8 or 12 waves only)
      if constexpr (WAVES >= 8) merge_halves<NT>(p, it, o, lsum, mrow, rows, row0, t0);
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
  template <int NT>
  __device__ static void merge_halves(const FwdParams& p, const Item& it,
                                      const f32x16 (&o)[NT][DT], const float (&lpart)[NT],
                                      const float (&m)[NT], int rows, int row0, int t0) {
    constexpr int PF = sfa::part_floats(D);
    constexpr int WF = DT * 16 * 64;                   // floats of one 32-row tile's O
    constexpr int OL = sfa::kPartRows / 32 * WF;       // l of kPartRows rows, then m
    __shared__ int split_seen;
    // thread index re-read here (an empty asm the compiler cannot see through), so that
    // these lane addresses are not hoisted out of the item loop, where they would stay
    // live across the key loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    const int slot = ((it.split * p.B + it.b) * p.H + it.h) * p.nqb + it.qb;
    const int cnt = slot * sfa::kSplitPasses + t0;  // one counter per pass over the keys
    float* mine = p.part + (int64_t(slot) * 2 + it.half) * PF;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tile = wave * QT + t0 + t;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          __hip_atomic_store(&mine[tile * WF + (dt * 16 + i) * 64 + lane], o[t][dt][i],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float l = lpart[t] + __shfl_xor(lpart[t], 32, 64);
      if (g == 0) {
        __hip_atomic_store(&mine[OL + tile * 32 + l32], l, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&mine[OL + sfa::kPartRows + tile * 32 + l32], m[t],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    wait_vm<0>();  // every store of this wave acknowledged
    __syncthreads();
    if (tid == 0) split_seen = atomicAdd(&p.split_cnt[cnt], 1);
    __syncthreads();
    const int first = split_seen == 0;
    __syncthreads();
    if (first) return;
    if (tid == 0) atomicExch(&p.split_cnt[cnt], 0);
    const float* other = p.part + (int64_t(slot) * 2 + (1 - it.half)) * PF;
    const bool h0 = it.half == 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tile = wave * QT + t0 + t;
      const int row = tile * 32 + l32;
      const float l = lpart[t] + __shfl_xor(lpart[t], 32, 64);
      const float lo = __hip_atomic_load(&other[OL + row], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      const float mo = __hip_atomic_load(&other[OL + sfa::kPartRows + row], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      const float m0 = h0 ? m[t] : mo, m1 = h0 ? mo : m[t];
      const float l0 = h0 ? l : lo, l1 = h0 ? lo : l;
      const float mm = fmaxf(m0, m1);
      const float s0 = __builtin_amdgcn_exp2f(m0 - mm), s1 = __builtin_amdgcn_exp2f(m1 - mm);
      const float inv = 1.0f / (l0 * s0 + l1 * s1);
      if (row >= rows) continue;
      uint16_t* op = p.o + it.b * p.osb + int64_t(row0 + row) * p.oss + it.h * p.osh + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float y[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * q4 + u;
            const float a = o[t][dt][i];
            const float b = __hip_atomic_load(&other[tile * WF + (dt * 16 + i) * 64 + lane],
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            y[u] = ((h0 ? a : b) * s0 + (h0 ? b : a) * s1) * inv;
          }
          uint2 wv;
          wv.x = pack_bf16x2(y[0], y[1]);
          wv.y = pack_bf16x2(y[2], y[3]);
          *reinterpret_cast<uint2*>(op + 32 * dt + 8 * q4) = wv;
        }
    }
  }

  // Fixed maximum: every query tile of the wave in one pass over the keys.
  __device__ static void run_fixed(const FwdParams& p, const Item& it, char* lds) {
    run<false, QT>(p, it, lds, 0);
  }

  // Online softmax rescales the accumulators with VALU work, so it holds one query
  // tile at a time in vector registers (QT passes over the keys).
  __device__ static void run_online(const FwdParams& p, const Item& it, char* lds) {
#pragma unroll
    for (int t0 = 0; t0 < QT; ++t0) {
      if (t0 > 0) __syncthreads();  // the next pass refills the LDS stages
      run<true, 1>(p, it, lds, t0);
    }
  }
};


}  // namespace
