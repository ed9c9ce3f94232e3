// Frame-aligned window-sparse attention forward kernel for gfx950 (CDNA4).
//
// Method: "HeyGen x Google Cloud: Bringing Avatar IV to TPUs".
//   * section "Deleting the mask" (Fig. 3): tiles are whole 16-token granules
//     that divide the frame span, so a query block's key granules are either
//     all visible (reference frame + window) or skipped. The reference frame's
//     granules are just the first granules of the same single pass: no mask
//     predicate, no padding, no second pass, no merge.
//   * section "Unchaining softmax" (Fig. 4): for eligible heads the softmax
//     maximum of row i is fixed in advance to M_i = scale*(<q_i,mu> + ||q_i||*kmax)
//     (>= every logit of the head by Cauchy-Schwarz), so the key loop has no
//     running maximum and no accumulator rescale; the row sum is kept as
//     per-lane partials and reduced across lanes once, at the end. Heads that
//     are not eligible run the online softmax in the same kernel (one branch,
//     uniform over the workgroup).
//   * section "Proving pixels unchanged": P is rounded to bf16 and PV runs on
//     the bf16 matrix cores with fp32 accumulation.
//
// Work decomposition (one workgroup = one work item = one query block of
// 16*gq rows of one (batch, head, frame)): 4 waves, each owning up to four
// 16-row sub-tiles; all waves stream the same key granules through LDS.
//
// MFMA orientation (v_mfma_f32_16x16x32_bf16, wave64):
//   S^T[key][q] = K[key][:] . Q[q][:]      A = K from LDS, B = Q in registers
//     -> accumulator lane l holds query l%16 and keys 4*(l/16)+i (i = 0..3),
//        so each lane's scores belong to one query row;
//   O^T[e][q] += V^T[e][key] . P^T[key][q] A = V^T from LDS, B = P^T straight
//     from the score registers (two 16-key score tiles -> 8 bf16 per lane);
//     the O accumulator lane again holds one query row (query l%16, dims
//     4*(l/16)+i), so the online rescale and the final 1/l are per-lane scalars.
// An odd trailing 16-key granule uses v_mfma_f32_16x16x16_bf16 for PV.
//
// LDS (double-buffered, 64 keys per stage):
//   K: [granule][key][16-byte column chunk], chunk index XOR-swizzled by key
//      so the 16 keys read by one MFMA operand hit distinct banks;
//   V: transposed while staging, per 32-key chunk [g][dim][8 keys] where
//      lane group g holds keys {4g..4g+3, 16+4g..16+4g+3} -- exactly the key
//      slots of the P^T operand -- so each PV A-operand is one 16-byte read.
#include "sfa_internal.h"

namespace {

using sfa::FwdParams;
using sfa::Item;
using sfa::KeyRanges;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = sfa::kFwdWaves;
constexpr int kSub = sfa::kFwdSub;
constexpr int kThreads = kWaves * 64;
constexpr int kStageGr = 4;  // key granules per LDS stage (64 keys)

template <int D>
struct Cfg {
  static constexpr int DC = D / 32;       // 32-wide d chunks of the QK^T contraction
  static constexpr int DT = D / 16;       // 16-wide d tiles of the PV output
  static constexpr int CH = D / 8;        // 16-byte chunks per key row
  static constexpr int KPR = 256 / (2 * D);  // key rows per 256 bytes (bank sweep)
  // LDS sizes in 16-byte units
  static constexpr int K_STAGE = kStageGr * 16 * CH;
  static constexpr int V_CHUNK = 4 * D;   // [g][dim]
  static constexpr int V_STAGE = 2 * V_CHUNK;
  static constexpr int LDS_UNITS = 2 * (K_STAGE + V_STAGE);
  static constexpr int K_LOADS = K_STAGE / kThreads;  // 16-byte K loads per thread per stage
  static constexpr int V_JOBS = 2 * 4 * (D / 4);      // (chunk, g, 4-dim group)
};

__device__ inline int k_swz(int key, int c, int CH, int KPR) { return c ^ ((key / KPR) % CH); }
__device__ inline int v_slot(int d) { return d ^ ((d >> 4) & 3); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

template <int D>
struct Kernel {
  using C = Cfg<D>;

  // global -> register staging of one 64-key stage
  struct Stage {
    uint4 k[C::K_LOADS];
    uint2 v[8];
  };

  __device__ static inline int granule_key(const KeyRanges& r, int gi) {
    const int t = gi * 16;
    return t < r.r0_end ? t : r.r1_begin + (t - r.r0_end);
  }

  template <bool FULL>
  __device__ static inline void load_stage(Stage& st, const FwdParams& p, const uint16_t* kb,
                                           const uint16_t* vb, const KeyRanges& r, int g0,
                                           int ng) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int idx = tid + kThreads * i;
      const int gr = idx / (16 * C::CH);
      const int rem = idx - gr * 16 * C::CH;
      const int key = rem / C::CH;
      const int c = rem - key * C::CH;
      if (FULL || gr < ng) {
        const int tok = granule_key(r, g0 + gr) + key;
        st.k[i] = *reinterpret_cast<const uint4*>(kb + int64_t(tok) * p.kss + c * 8);
      } else {
        st.k[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < C::V_JOBS) {
      const int cc = tid / D;
      const int g = (tid / (D / 4)) & 3;
      const int dq = tid % (D / 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gr = 2 * cc + (j >> 2);
        if (FULL || gr < ng) {
          const int tok = granule_key(r, g0 + gr) + 4 * g + (j & 3);
          st.v[j] = *reinterpret_cast<const uint2*>(vb + int64_t(tok) * p.vss + dq * 4);
        } else {
          st.v[j] = make_uint2(0, 0);
        }
      }
    }
  }

  __device__ static inline void store_stage(const Stage& st, uint4* lds_k, uint4* lds_v) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int idx = tid + kThreads * i;
      const int gr = idx / (16 * C::CH);
      const int rem = idx - gr * 16 * C::CH;
      const int key = rem / C::CH;
      const int c = rem - key * C::CH;
      lds_k[(gr * 16 + key) * C::CH + k_swz(key, c, C::CH, C::KPR)] = st.k[i];
    }
    if (tid < C::V_JOBS) {
      const int cc = tid / D;
      const int g = (tid / (D / 4)) & 3;
      const int dq = tid % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t a = (e >> 1) ? st.v[2 * q].y : st.v[2 * q].x;
          const uint32_t b = (e >> 1) ? st.v[2 * q + 1].y : st.v[2 * q + 1].x;
          w[q] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        lds_v[cc * C::V_CHUNK + g * D + v_slot(4 * dq + e)] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  // One 32-key chunk (NK = 2 granules) or a trailing 16-key granule (NK = 1).
  template <int NK, bool ONLINE, int NT>
  __device__ static inline void chunk(const uint4* lds_k, const uint4* lds_v,
                                      const bf16x8 (&qf)[NT][C::DC], f32x4 (&o)[NT][C::DT],
                                      float (&mrow)[NT], float (&lsum)[NT], float cexp) {
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15;
    const int g = lane >> 4;
    f32x4 s[NT][NK];
#pragma unroll
    for (int kg = 0; kg < NK; ++kg) {
#pragma unroll
      for (int t = 0; t < NT; ++t) s[t][kg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) {
        const uint4 raw = lds_k[(kg * 16 + l16) * C::CH + k_swz(l16, 4 * dc + g, C::CH, C::KPR)];
        const bf16x8 a = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          s[t][kg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[t][dc], s[t][kg], 0, 0, 0);
      }
    }
    // softmax numerators; lane holds 4*NK scores of its query row per sub-tile
    uint32_t pk[NT][2 * NK];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float m = mrow[t];
      if (ONLINE) {
        float mx = s[t][0][0];
#pragma unroll
        for (int kg = 0; kg < NK; ++kg)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[t][kg][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m, mx * cexp);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        lsum[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) o[t][dt] *= alpha;
        mrow[t] = mnew;
        m = mnew;
      }
      float pv[4 * NK];
#pragma unroll
      for (int kg = 0; kg < NK; ++kg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(s[t][kg][i], cexp, -m));
          pv[kg * 4 + i] = pe;
          lsum[t] += pe;
        }
#pragma unroll
      for (int i = 0; i < 2 * NK; ++i) pk[t][i] = pack_bf16x2(pv[2 * i], pv[2 * i + 1]);
    }
    // O^T += V^T . P^T
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const uint4 raw = lds_v[g * D + v_slot(16 * dt + l16)];
      if constexpr (NK == 2) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint4 bp = make_uint4(pk[t][0], pk[t][1], pk[t][2], pk[t][3]);
          o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bp),
                                                            o[t][dt], 0, 0, 0);
        }
      } else {
        const i16x4 a = __builtin_bit_cast(i16x4, make_uint2(raw.x, raw.y));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const i16x4 bp = __builtin_bit_cast(i16x4, make_uint2(pk[t][0], pk[t][1]));
          o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bp, o[t][dt], 0, 0, 0);
        }
      }
    }
  }

  // Streams every visible key granule of the item once for NT sub-tiles
  // (t0 .. t0+NT-1) of each wave's query rows.
  template <bool ONLINE, int NT>
  __device__ static void run_pass(const FwdParams& p, const Item& it, uint4* lds, int t0) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int g = lane >> 4;

    const KeyRanges r = sfa::key_ranges(it.f, p.F, p.T, p.w);
    const int ngran = (r.r0_end + (r.r1_end - r.r1_begin)) / 16;

    const uint16_t* kb = p.k + it.b * p.ksb + it.h * p.ksh;
    const uint16_t* vb = p.v + it.b * p.vsb + it.h * p.vsh;

    // this wave's query granules inside the item (balanced split)
    const int gfirst = (wave * p.gq) / kWaves;
    const int nsub = ((wave + 1) * p.gq) / kWaves - gfirst;
    const int row0 = it.f * p.T + it.qb * p.gq * 16;
    const int64_t rowstat = (int64_t(it.b) * p.H + it.h) * p.S;
    const float kmax = p.kmax[it.b * p.H + it.h];

    bf16x8 qf[NT][C::DC];
    float mrow[NT], lsum[NT];
    f32x4 o[NT][C::DT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // sub-tiles past this wave's share repeat a valid granule; never stored
      const int tt = t0 + t;
      const int gi = nsub > 0 ? gfirst + (tt < nsub ? tt : nsub - 1) : 0;
      const int row = row0 + gi * 16 + l16;
      const uint16_t* qp = p.q + it.b * p.qsb + int64_t(row) * p.qss + it.h * p.qsh + 8 * g;
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc)
        qf[t][dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * dc));
      if (ONLINE) {
        mrow[t] = -__builtin_inff();
      } else {
        mrow[t] = (p.qmu[rowstat + row] + p.qn[rowstat + row] * kmax) * p.c;
      }
      lsum[t] = 0.f;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    uint4* lds_k[2] = {lds, lds + C::K_STAGE};
    uint4* lds_v[2] = {lds + 2 * C::K_STAGE, lds + 2 * C::K_STAGE + C::V_STAGE};

    // full 64-key stages in the main loop, then the 1..3 granule tail once
    const int nfull = ngran / kStageGr;
    const int rem = ngran - nfull * kStageGr;
    Stage st;
    if (nfull > 0)
      load_stage<true>(st, p, kb, vb, r, 0, kStageGr);
    else
      load_stage<false>(st, p, kb, vb, r, 0, rem);
    store_stage(st, lds_k[0], lds_v[0]);
    __syncthreads();

    for (int s = 0; s < nfull; ++s) {
      const int buf = s & 1;
      const int gnext = (s + 1) * kStageGr;
      if (s + 1 < nfull)
        load_stage<true>(st, p, kb, vb, r, gnext, kStageGr);
      else if (rem > 0)
        load_stage<false>(st, p, kb, vb, r, gnext, rem);
      chunk<2, ONLINE, NT>(lds_k[buf], lds_v[buf], qf, o, mrow, lsum, p.c);
      chunk<2, ONLINE, NT>(lds_k[buf] + 32 * C::CH, lds_v[buf] + C::V_CHUNK, qf, o, mrow, lsum,
                           p.c);
      if (s + 1 < nfull || rem > 0) store_stage(st, lds_k[buf ^ 1], lds_v[buf ^ 1]);
      __syncthreads();
    }
    if (rem > 0) {
      const int buf = nfull & 1;
      if (rem >= 2) chunk<2, ONLINE, NT>(lds_k[buf], lds_v[buf], qf, o, mrow, lsum, p.c);
      if (rem == 1) chunk<1, ONLINE, NT>(lds_k[buf], lds_v[buf], qf, o, mrow, lsum, p.c);
      if (rem == 3)
        chunk<1, ONLINE, NT>(lds_k[buf] + 32 * C::CH, lds_v[buf] + C::V_CHUNK, qf, o, mrow, lsum,
                             p.c);
    }

    // epilogue: one cross-lane reduction of the row sums, normalise, store bf16
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float l = lsum[t];
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      const float inv = 1.0f / l;
      if (t0 + t < nsub) {
        const int row = row0 + (gfirst + t0 + t) * 16 + l16;
        uint16_t* op = p.o + it.b * p.osb + int64_t(row) * p.oss + it.h * p.osh + 4 * g;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          uint2 w;
          w.x = pack_bf16x2(o[t][dt][0] * inv, o[t][dt][1] * inv);
          w.y = pack_bf16x2(o[t][dt][2] * inv, o[t][dt][3] * inv);
          *reinterpret_cast<uint2*>(op + 16 * dt) = w;
        }
      }
    }
  }

  // Fixed maximum: all four sub-tiles in one pass over the keys.
  __device__ static void run_fixed(const FwdParams& p, const Item& it, uint4* lds) {
    run_pass<false, kSub>(p, it, lds, 0);
  }

  // Online softmax: the running maximum rescales the accumulators with VALU
  // work, so hold half the sub-tiles at a time (two passes over the keys).
  __device__ static void run_online(const FwdParams& p, const Item& it, uint4* lds) {
    run_pass<true, kSub / 2>(p, it, lds, 0);
    __syncthreads();  // LDS buffers are refilled by the second pass
    run_pass<true, kSub / 2>(p, it, lds, kSub / 2);
  }
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdParams p) {
  __shared__ uint4 lds[Cfg<D>::LDS_UNITS];
  const Item it = sfa::decode_item(blockIdx.x, p.frame_order, p.B, p.H, p.nqb, p.items);
  if (p.elig[it.b * p.H + it.h])
    Kernel<D>::run_fixed(p, it, lds);
  else
    Kernel<D>::run_online(p, it, lds);
}

}  // namespace

hipError_t sfa_launch_fwd(const sfa::FwdParams& p, int head_dim, hipStream_t stream) {
  if (p.items <= 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(fwd_kernel<128>, dim3(p.items), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_kernel<64>, dim3(p.items), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}
