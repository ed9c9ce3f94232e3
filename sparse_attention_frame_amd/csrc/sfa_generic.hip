// Ablation: generic block-sparse attention (not the product path).
//
// "HeyGen x Google Cloud: Bringing Avatar IV to TPUs", section "Deleting the
// mask": the kernel the pages started from tiled the sequence with generic
// block sizes that ignore frame boundaries, so blocks straddling a frame edge
// were partial and needed an element-wise mask predicate, the sequence was
// padded to the block size, and the reference frame ran as a second pass whose
// result was merged afterwards. This file rebuilds that design on the same
// MI355X tile machinery (sfa_attn.h) so the two can be measured side by side:
// 256-row query blocks, 128-key blocks, online softmax, a window pass and a
// reference pass, and a merge through the per-pass log-sum-exp.
#include "sfa_attn.h"

namespace {

template <int D>
struct Generic : Attn<D, 8, 1, 2> {
  using A = Attn<D, 8, 1, 2>;
  using typename A::Lane;
  using typename A::Slots;
  using A::KS;
  using A::DT;
  using A::DMA_W;
  using A::STAGE_B;
  using A::GB;
  using A::dma16;
  using A::lane_setup;

  // DMA of the 64-key stage starting at key0 of one (b, h) from the staged K and V;
  // granules past the end of the sequence are loaded from the last valid granule
  // instead (finite values; those keys are masked).
  __device__ static inline void issue_generic(char* lds, int buf, const Lane& L, const Slots& W,
                                              const char* kbase, const char* vbase, int key0,
                                              int S) {
    const int ng = S >> 4;
    char* lb = lds + buf * STAGE_B;
#pragma unroll
    for (int i = 0; i < DMA_W; ++i) {
      const int gr = (key0 >> 4) + W.gi[i];
      const int gs = gr < ng ? gr : ng - 1;
      dma16((W.v[i] ? vbase : kbase) + int64_t(gs) * GB + W.src[i], L.dma, lb + W.dst[i]);
    }
  }

  // One 32-key tile of the generic kernel for the wave's query tile: online
  // softmax, and for partial blocks the element mask of the frame window.
  template <bool MASKED>
  __device__ static inline void tile_generic(const char* lds, const Lane& L, int kl, int vl,
                                             const bf16x8 (&qf)[KS], f32x16 (&o)[DT], float& m,
                                             float& l, float cexp, int key0, int fi, int pass,
                                             int S, int T, int w) {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + kl + L.kofs + 512 * ks);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
    }
    if (MASKED) {
      const int g = (threadIdx.x >> 5) & 1;
      const int f0 = key0 / T;            // a 32-key tile spans at most 3 frames (T >= 16)
      const int e1 = (f0 + 1) * T, e2 = (f0 + 2) * T;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // branch-free: bitwise combinations and one select per score
        const int key = key0 + 16 * (i >> 3) + 8 * g + (i & 7);
        const int fj = f0 + int(key >= e1) + int(key >= e2);
        const int df = fi - fj;
        const bool win = (fi >= 1) & (fj >= 1) & (df <= w) & (df >= -w);
        const bool ok = (key < S) & (pass == 1 ? (fj == 0) : win);
        s[i] = ok ? s[i] : -__builtin_inff();
      }
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * cexp;
    const bool grow = mx > m + 8.0f;
    if (__ballot(grow) != 0) {
      const float mnew = fmaxf(m, mx);
      // rows that have met no visible key yet (m = -inf) hold l = 0 and o = 0
      const float alpha = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m = mnew;
    }
    // a row that has met no visible key yet keeps m = -inf; its weights are 0
    const float ms = m == -__builtin_inff() ? 0.f : m;
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[2 * i], cexp, -ms));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[2 * i + 1], cexp, -ms));
      pk[i] = pack_bf16x2(p0, p1);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), kOnes, l, false);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, make_uint4(pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + vl + h * GB + dt * 1024 + L.vofs);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[dt], 0, 0, 0);
      }
    }
  }

  // One (pass, b, h, query block) item of the generic kernel: 256 rows (rows past
  // the sequence computed on a repeated row, never stored), its key blocks from
  // the list, two 64-key LDS stages per block, double-buffered.
  __device__ static void run_generic(const sfa::GenericParams& p, int idx, char* lds) {
    const int per_pass = p.B * p.H * p.nqb;
    const int pass = idx / per_pass;
    const int rest = idx - pass * per_pass;
    const int bh = rest / p.nqb, qb = rest - bh * p.nqb;
    const int b = bh / p.H, h = bh - b * p.H;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    const int row = qb * sfa::kGenericBq + wave * 32 + l32;
    const int rowc = min(row, p.S - 1);
    const int fi = rowc / p.T;
    bf16x8 qf[KS];
    const uint16_t* qp = p.q + b * p.qsb + int64_t(rowc) * p.qss + h * p.qsh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 16 * ks));
    float m = -__builtin_inff(), l = 0.f;
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    Lane L;
    Slots W;
    lane_setup(L, W);
    const char* kbase = reinterpret_cast<const char*>(p.kst + int64_t(bh) * D * p.S);
    const char* vbase = reinterpret_cast<const char*>(p.vst + int64_t(bh) * D * p.S);
    const int32_t* lst = p.lists + p.offs[pass * (p.nqb + 1) + qb];
    const int nst = 2 * (p.offs[pass * (p.nqb + 1) + qb + 1] - p.offs[pass * (p.nqb + 1) + qb]);
    if (nst > 0) issue_generic(lds, 0, L, W, kbase, vbase, (lst[0] & 0x3fffffff) * 128, p.S);
    for (int st = 0; st < nst; ++st) {
      wait_vm<0>();
      __syncthreads();
      if (st + 1 < nst)
        issue_generic(lds, (st + 1) & 1, L, W, kbase, vbase,
                      (lst[(st + 1) >> 1] & 0x3fffffff) * 128 + ((st + 1) & 1) * 64, p.S);
      const int e = lst[st >> 1];
      const int key0 = (e & 0x3fffffff) * 128 + (st & 1) * 64;
      const int kl = (st & 1) * STAGE_B;
      if (e >> 30) {
        tile_generic<false>(lds, L, kl, kl, qf, o, m, l, p.c, key0, fi, pass, p.S, p.T, p.w);
        tile_generic<false>(lds, L, kl + 2 * GB, kl + 2 * GB, qf, o, m, l, p.c, key0 + 32, fi,
                            pass, p.S, p.T, p.w);
      } else {
        tile_generic<true>(lds, L, kl, kl, qf, o, m, l, p.c, key0, fi, pass, p.S, p.T, p.w);
        tile_generic<true>(lds, L, kl + 2 * GB, kl + 2 * GB, qf, o, m, l, p.c, key0 + 32, fi,
                           pass, p.S, p.T, p.w);
      }
    }
    const float lt = l + __shfl_xor(l, 32, 64);
    if (row < p.S) {
      const int64_t r = (int64_t(pass) * p.B * p.H + bh) * p.S + row;
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      float* op = p.part + r * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int mq = 0; mq < 4; ++mq)
          *reinterpret_cast<float4*>(op + 32 * dt + 8 * mq) =
              make_float4(o[dt][4 * mq] * inv, o[dt][4 * mq + 1] * inv, o[dt][4 * mq + 2] * inv,
                          o[dt][4 * mq + 3] * inv);
      if (g == 0) p.lse[r] = lt > 0.f ? m + __log2f(lt) : -__builtin_inff();
    }
  }

};

template <int D>
__global__ __launch_bounds__(512, 1) void generic_kernel(sfa::GenericParams p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  Generic<D>::run_generic(p, blockIdx.x, lds);
}

// O = sum over the two passes of 2^(lse_p - lse) * O_p with lse = log2 of the
// summed weights; one thread per 4 output elements.
__global__ __launch_bounds__(256) void merge_kernel(sfa::MergeParams p) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int d4n = p.D / 4;
  const int64_t total = int64_t(p.B) * p.S * p.H * d4n;
  if (idx >= total) return;
  const int d4 = int(idx % d4n);
  int64_t t = idx / d4n;
  const int h = int(t % p.H);
  t /= p.H;
  const int row = int(t % p.S);
  const int b = int(t / p.S);
  const int64_t r0 = (int64_t(b) * p.H + h) * p.S + row;
  const int64_t r1 = (int64_t(p.B + b) * p.H + h) * p.S + row;
  const float l0 = p.lse[r0], l1 = p.lse[r1];
  const float mx = fmaxf(l0, l1);
  const float w0 = l0 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(l0 - mx);
  const float w1 = l1 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(l1 - mx);
  const float inv = 1.0f / (w0 + w1);
  const float4 a = *reinterpret_cast<const float4*>(p.part + r0 * p.D + 4 * d4);
  const float4 c = *reinterpret_cast<const float4*>(p.part + r1 * p.D + 4 * d4);
  uint2 out;
  out.x = pack_bf16x2((w0 * a.x + w1 * c.x) * inv, (w0 * a.y + w1 * c.y) * inv);
  out.y = pack_bf16x2((w0 * a.z + w1 * c.z) * inv, (w0 * a.w + w1 * c.w) * inv);
  *reinterpret_cast<uint2*>(p.o + b * p.osb + int64_t(row) * p.oss + h * p.osh + 4 * d4) = out;
}

}  // namespace

hipError_t sfa_launch_generic(const sfa::GenericParams& p, const sfa::MergeParams& m, int head_dim,
                              hipStream_t stream) {
  if (p.items > 0) {
    const int lds = 2 * 2 * 64 * 2 * head_dim;  // two stages of K and V^T
    auto kern = head_dim == 128 ? generic_kernel<128> : generic_kernel<64>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(p.items), dim3(512), lds, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t total = int64_t(m.B) * m.S * m.H * (m.D / 4);
  if (total > 0)
    hipLaunchKernelGGL(merge_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, stream, m);
  return hipGetLastError();
}
