// Frame-aligned window-sparse attention forward kernel for gfx950 (CDNA4).
//
// Method: "HeyGen x Google Cloud: Bringing Avatar IV to TPUs".
//   * section "Deleting the mask" (Fig. 3): tiles are whole 16-token granules
//     that divide the frame span, so a query block's key granules are either
//     all visible (reference frame + window) or skipped. The reference frame's
//     granules are simply the first granules of the same single pass: no mask
//     predicate, no padding, no second pass, no merge.
//   * section "Unchaining softmax" (Fig. 4): for eligible heads the softmax
//     maximum of row i is fixed in advance to M_i = scale*(<q_i,mu> + ||q_i||*kmax)
//     (>= every logit of the head by Cauchy-Schwarz), so the key loop has no
//     running maximum and no accumulator rescale; the row sum stays a per-lane
//     partial and is reduced across lanes once, at the end. Heads that are not
//     eligible run the online softmax in the same kernel (one branch, uniform
//     over the workgroup).
//   * section "Proving pixels unchanged": P is rounded to bf16 and PV runs on
//     the bf16 matrix cores with fp32 accumulation.
//
// Work decomposition: one workgroup = one work item = one query block of
// 16*gq rows (gq | T/16) of one (batch, head, frame). WAVES waves each own QT
// 32-row query tiles; when gq is odd the last tile holds 16 real rows and 16
// repeats that are computed but never stored. All waves stream the same key
// granules through LDS.
//
// MFMA orientation (v_mfma_f32_32x32x16_bf16, wave64; 32x32x16 runs at twice
// the rate of 16x16x32 on this chip):
//   S^T[key][q] = K[key][:] . Q[q][:]        A = K from LDS, B = Q in registers;
//     the accumulator lane l holds query l%32 and keys 8*(i/4) + 4*(l/32) + i%4
//     (i = 0..15), so all 16 scores of a lane belong to one query row;
//   O^T[e][q] += V^T[e][key] . P^T[key][q]   B = P^T straight from the score
//     registers (regs 8h..8h+7 are the keys of half h of the 32-key tile),
//     A = V^T gathered by LDS transpose reads; the O accumulator lane again
//     holds one query row, so the online rescale and the final 1/l are
//     per-lane scalars.
//
// Staging: K and V tiles go from HBM straight into LDS by DMA
// (global_load_lds_dwordx4; no registers, no VALU), double-buffered per 64-key
// stage. Rows keep their natural [key][dim] layout; 16-byte chunks are
// XOR-swizzled by key (through the DMA source address) so that the MFMA
// operand reads are free of bank conflicts:
//   K: lane l reads 16 bytes of key l%32 -> chunk ^= key % 16;
//   V: ds_read_b64_tr_b16 -- in each 16-lane group lane r supplies the address
//      of 4 dims of key kb + r/4 and receives dim d0 + r of keys kb..kb+3 --
//      reads 4 keys x 32 bytes at once -> chunk ^= 2 * (key % 4).
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

constexpr int kStageKeys = 64;  // keys per LDS stage (4 granules, 2 tiles of 32)

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, int WAVES, int QT>
struct Attn {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int KS = D / 16;             // 16-dim k-steps of QK^T
  static constexpr int DT = D / 32;             // 32-dim tiles of O^T
  static constexpr int CH = D / 8;              // 16-byte chunks per key row
  static constexpr int ROWB = 2 * D;            // bytes per key row
  static constexpr int KPR = 256 / ROWB;        // key rows per 256-byte bank sweep
  static constexpr int STAGE_B = kStageKeys * ROWB;          // bytes per tensor per stage
  static constexpr int DMA_KEYS = 1024 / ROWB;               // keys per DMA instruction
  static constexpr int DMA_N = 2 * STAGE_B / 1024;           // K + V instructions per stage
  static constexpr int LDS_BYTES = 2 * 2 * STAGE_B;          // double-buffered K and V
  static_assert(DMA_N % WAVES == 0, "DMA instructions split evenly over waves");

  __device__ static inline int k_phys(int key, int c) { return c ^ ((key / KPR) % CH); }
  __device__ static inline int v_phys(int key, int c) { return c ^ (2 * (key & 3)); }

  __device__ static inline int granule_key(const KeyRanges& r, int gi) {
    const int t = gi * 16;
    return t < r.r0_end ? t : r.r1_begin + (t - r.r0_end);
  }

  // DMA `nkeys` keys (a multiple of 16) of one stage into LDS buffer `buf`.
  __device__ static inline void issue_stage(char* lds, int buf, const uint16_t* kb,
                                            const uint16_t* vb, int64_t kss, int64_t vss,
                                            const KeyRanges& r, int g0, int nkeys) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lpr = 64 / DMA_KEYS;  // lanes per key row (16-byte chunks)
#pragma unroll
    for (int n = wave; n < DMA_N; n += WAVES) {
      const bool is_v = n >= DMA_N / 2;
      const int key0 = (is_v ? n - DMA_N / 2 : n) * DMA_KEYS;
      if (key0 >= nkeys) continue;
      const int key = key0 + lane / lpr;
      const int pc = lane % lpr;
      const int c = is_v ? v_phys(key, pc) : k_phys(key, pc);
      const int tok = granule_key(r, g0 + key / 16) + (key & 15);
      const uint16_t* src = (is_v ? vb + int64_t(tok) * vss : kb + int64_t(tok) * kss) + c * 8;
      char* dst = lds + (buf * 2 + (is_v ? 1 : 0)) * STAGE_B + key0 * ROWB;
      __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)dst, 16, 0, 0);
    }
  }

  // One 32-key tile (HALF: only its first 16 keys exist) for all QT query tiles.
  template <bool HALF, bool ONLINE>
  __device__ static inline void tile(const char* kl, const char* vl,
                                     const bf16x8 (&qf)[QT][KS], f32x16 (&o)[QT][DT],
                                     float (&mrow)[QT], float (&lsum)[QT], float cexp,
                                     bool active) {
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    if (!active) return;
    // S^T = K . Q^T
    f32x16 s[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[t][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int key = l32;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + key * ROWB +
                                                         k_phys(key, 2 * ks + g) * 16);
#pragma unroll
      for (int t = 0; t < QT; ++t)
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t][ks], s[t], 0, 0, 0);
    }
    // softmax numerators: 16 (8 for HALF) scores of one query row per lane
    constexpr int NV = HALF ? 8 : 16;
    uint32_t pk[QT][NV / 2];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (ONLINE) {
        float mx = s[t][0];
#pragma unroll
        for (int i = 1; i < NV; ++i) mx = fmaxf(mx, s[t][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * cexp;
        // lazy rescale: keep the stale maximum while the tile stays within 2^8 of
        // it (exact up to rounding: numerator and denominator share the shift)
        const bool grow = mx > mrow[t] + 8.0f;
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
      float pv[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(fmaf(s[t][i], cexp, -m));
        lsum[t] += pv[i];
      }
#pragma unroll
      for (int i = 0; i < NV / 2; ++i) pk[t][i] = pack_bf16x2(pv[2 * i], pv[2 * i + 1]);
    }
    // O^T += V^T . P^T, two 16-key halves
    const int r = lane & 15;           // row this lane supplies to the transpose read
    const int d0 = ((lane >> 4) & 1) * 16;
#pragma unroll
    for (int h = 0; h < (HALF ? 1 : 2); ++h) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        i16x4 part[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int key = 16 * h + 8 * u + 4 * g + (r >> 2);
          const int d = 32 * dt + d0 + 4 * (r & 3);
          const char* addr = vl + key * ROWB + v_phys(key, d >> 3) * 16 + (d & 7) * 2;
          part[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_ptr)(lds_void_ptr)const_cast<char*>(addr));
        }
        const uint2 p0 = __builtin_bit_cast(uint2, part[0]);
        const uint2 p1 = __builtin_bit_cast(uint2, part[1]);
        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(p0.x, p0.y, p1.x, p1.y));
#pragma unroll
        for (int t = 0; t < QT; ++t) {
          const bf16x8 b = __builtin_bit_cast(
              bf16x8, make_uint4(pk[t][4 * h], pk[t][4 * h + 1], pk[t][4 * h + 2],
                                 pk[t][4 * h + 3]));
          o[t][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[t][dt], 0, 0, 0);
        }
      }
    }
  }

  template <bool ONLINE>
  __device__ static void run(const FwdParams& p, const Item& it, char* lds) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const KeyRanges r = sfa::key_ranges(it.f, p.F, p.T, p.w);
    const int ngran = (r.r0_end + (r.r1_end - r.r1_begin)) / 16;
    const uint16_t* kb = p.k + it.b * p.ksb + it.h * p.ksh;
    const uint16_t* vb = p.v + it.b * p.vsb + it.h * p.vsh;

    const int rows = p.gq * 16;                 // real rows of this item
    const int row0 = it.f * p.T + it.qb * rows;
    const int64_t rowstat = (int64_t(it.b) * p.H + it.h) * p.S;
    const float kmax = p.kmax[it.b * p.H + it.h];
    // query tiles of this wave; a wave whose tiles hold no real row skips the math
    const bool active = wave * QT * 32 < rows;

    bf16x8 qf[QT][KS];
    float mrow[QT], lsum[QT];
    f32x16 o[QT][DT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int lr = min((wave * QT + t) * 32 + l32, rows - 1);  // repeats past the end
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
    issue_stage(lds, 0, kb, vb, p.kss, p.vss, r, 0, (nfull > 0 ? 4 : rem) * 16);
    wait_dma();
    __syncthreads();

    for (int s = 0; s < nfull; ++s) {
      const int buf = s & 1;
      if (s + 1 < nfull || rem > 0)
        issue_stage(lds, buf ^ 1, kb, vb, p.kss, p.vss, r, (s + 1) * 4,
                    (s + 1 < nfull ? 4 : rem) * 16);
      const char* kl = lds + (buf * 2) * STAGE_B;
      const char* vl = kl + STAGE_B;
      tile<false, ONLINE>(kl, vl, qf, o, mrow, lsum, p.c, active);
      tile<false, ONLINE>(kl + 32 * ROWB, vl + 32 * ROWB, qf, o, mrow, lsum, p.c, active);
      wait_dma();
      __syncthreads();
    }
    if (rem > 0) {
      const int buf = nfull & 1;
      const char* kl = lds + (buf * 2) * STAGE_B;
      const char* vl = kl + STAGE_B;
      if (rem >= 2)
        tile<false, ONLINE>(kl, vl, qf, o, mrow, lsum, p.c, active);
      else
        tile<true, ONLINE>(kl, vl, qf, o, mrow, lsum, p.c, active);
      if (rem == 3)
        tile<true, ONLINE>(kl + 32 * ROWB, vl + 32 * ROWB, qf, o, mrow, lsum, p.c, active);
    }

    // epilogue: the two lane halves hold the two key halves of every row
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const float l = lsum[t] + __shfl_xor(lsum[t], 32, 64);
      const float inv = 1.0f / l;
      const int lr = (wave * QT + t) * 32 + l32;
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
};

template <int D, int WAVES, int QT>
__global__ __launch_bounds__(WAVES * 64, 1) void fwd_kernel(FwdParams p) {
  using A = Attn<D, WAVES, QT>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const Item it = sfa::decode_item(blockIdx.x, p.frame_order, p.B, p.H, p.nqb, p.items);
  if (p.elig[it.b * p.H + it.h])
    A::template run<false>(p, it, lds);
  else
    A::template run<true>(p, it, lds);
}

template <int D, int WAVES, int QT>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  using A = Attn<D, WAVES, QT>;
  auto kern = fwd_kernel<D, WAVES, QT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, A::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.items), dim3(A::kThreads), A::LDS_BYTES, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t sfa_launch_fwd(const sfa::FwdParams& p, int head_dim, int waves, hipStream_t stream) {
  if (p.items <= 0) return hipSuccess;
  if (head_dim == 128)
    return waves == 4 ? launch<128, 4, 2>(p, stream) : launch<128, 8, 1>(p, stream);
  return waves == 4 ? launch<64, 4, 2>(p, stream) : launch<64, 8, 1>(p, stream);
}
