// Norm array for the Cauchy-Schwarz fixed softmax maximum (gfx950).
//
// "HeyGen x Google Cloud: Bringing Avatar IV to TPUs", section "Unchaining
// softmax" (Fig. 4): a logit is at most ||q|| times the largest key norm;
// centring the keys on their mean tightens the bound without changing the
// softmax; heads whose bound is too loose fall back to the online path.
//
// Three memory-bound passes, all deterministic (fixed summation order, no
// atomics). Blocks stream whole token rows ([H, d] contiguous in the usual
// BSHD layout): thread t owns one 8-element (16-byte) column group of one head.
//   1. ksum   : per 64-token chunk, column sums of k            -> psum
//   2. kmean  : mu = (sum over chunks of psum) / S              -> mu
//   3. stats  : per 16-token granule, max ||k - mu||^2 and max ||q||^2, and per
//               row ||q|| and <q, mu>                           -> pkmax, pqmax, qn, qmu
//   4. final  : per frame the maxima of its granules; per head kmax, qmax,
//               bound = scale * qmax * kmax; per query frame the key-norm
//               maximum its rows use (the head's, or the largest over the
//               frames it sees), its bound and its eligibility flag
//   5. stage  : K and V copied into the granule layouts the attention kernel's LDS
//               stages use (sfa_internal.h): each of its DMA requests then copies
//               1 KB of contiguous bytes, and its QK^T and PV operands are single
//               16-byte LDS reads at a fixed lane offset plus an immediate
#include "sfa_internal.h"

namespace {

using sfa::NormParams;
using sfa::kNormChunk;

constexpr int kThreads = 256;

__device__ inline void unpack8(const uint4& r, float x[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ inline uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Sum over the `lanes` consecutive lanes that share one token row of one head.
template <int LANES>
__device__ inline float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__global__ __launch_bounds__(kThreads) void ksum_kernel(NormParams p) {
  const int chunk = blockIdx.x;
  const int b = blockIdx.y;
  const int cpr = p.D / 8;           // column groups per head
  const int groups = p.H * cpr;
  const int s0 = chunk * kNormChunk;
  const int s1 = min(p.S, s0 + kNormChunk);  // s1 - s0 is a multiple of 16
  for (int cg = threadIdx.x; cg < groups; cg += blockDim.x) {
    const int h = cg / cpr;
    const int e0 = (cg - h * cpr) * 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint16_t* kp = p.k + b * p.ksb + h * p.ksh + e0;
    for (int s = s0; s < s1; s += 4) {
      uint4 raw[4];  // four rows in flight per lane
#pragma unroll
      for (int t = 0; t < 4; ++t) raw[t] = load16(kp + int64_t(s + t) * p.kss);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float x[8];
        unpack8(raw[t], x);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += x[i];
      }
    }
    float* out = p.psum + ((int64_t(chunk) * p.B + b) * p.H + h) * p.D + e0;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = acc[i];
  }
}

// mu = (sum of the chunk partials) / S. One block per (b, h): D columns x P
// parts; part j adds chunks j, j+P, ... in order, then the parts are added in
// a fixed order.
constexpr int kReduceThreads = 1024;

__global__ __launch_bounds__(kReduceThreads) void kmean_kernel(NormParams p) {
  __shared__ float part[kReduceThreads];
  const int bh = blockIdx.x;  // b * H + h
  const int e = threadIdx.x % p.D;
  const int j = threadIdx.x / p.D;
  const int parts = kReduceThreads / p.D;
  const int64_t stride = int64_t(p.B) * p.H * p.D;
  const float* src = p.psum + int64_t(bh) * p.D + e;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int c = j;
  for (; c + 3 * parts < p.nchunk; c += 4 * parts) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += src[(c + u * parts) * stride];
  }
  for (; c < p.nchunk; c += parts) acc[0] += src[c * stride];
  part[threadIdx.x] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (j == 0) {
    float t = 0.f;
    for (int q = 0; q < parts; ++q) t += part[q * p.D + e];
    p.mu[int64_t(bh) * p.D + e] = t / float(p.S);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void stats_kernel(NormParams p) {
  constexpr int CPR = D / 8;  // lanes per (token, head); a power of two <= 16
  const int chunk = blockIdx.x;
  const int b = blockIdx.y;
  const int groups = p.H * CPR;
  const int s0 = chunk * kNormChunk;
  const int s1 = min(p.S, s0 + kNormChunk);
  // groups is a multiple of CPR and the loop stride (a multiple of 64) is too, so
  // the CPR lanes of one head always iterate together (shuffles stay inside the group)
  for (int cgb = 0; cgb < groups; cgb += blockDim.x) {
    const int cg = cgb + threadIdx.x;
    const bool active = cg < groups;
    const int h = active ? cg / CPR : 0;
    const int e0 = (cg % CPR) * 8;
    float mu[8];
    const float* mup = p.mu + (int64_t(b) * p.H + h) * D + e0;
#pragma unroll
    for (int i = 0; i < 8; ++i) mu[i] = active ? mup[i] : 0.f;
    const uint16_t* kp = p.k + b * p.ksb + h * p.ksh + e0;
    const uint16_t* qp = p.q + b * p.qsb + h * p.qsh + e0;
    float kmax2 = 0.f, qmax2 = 0.f;
    for (int sb = s0; sb < s1; sb += 4) {  // s1 - s0 is a multiple of 16
      uint4 kr[4], qr[4];  // four rows of k and q in flight per lane
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        kr[t] = active ? load16(kp + int64_t(sb + t) * p.kss) : make_uint4(0, 0, 0, 0);
        qr[t] = active ? load16(qp + int64_t(sb + t) * p.qss) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int s = sb + t;
        float kx[8], qx[8];
        unpack8(kr[t], kx);
        unpack8(qr[t], qx);
        float kc = 0.f, qq = 0.f, qm = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float dk = kx[i] - mu[i];
          kc = fmaf(dk, dk, kc);
          qq = fmaf(qx[i], qx[i], qq);
          qm = fmaf(qx[i], mu[i], qm);
        }
        kc = group_sum<CPR>(kc);
        qq = group_sum<CPR>(qq);
        qm = group_sum<CPR>(qm);
        kmax2 = fmaxf(kmax2, kc);
        qmax2 = fmaxf(qmax2, qq);
        if (active && (cg % CPR) == 0) {
          const int64_t row = (int64_t(b) * p.H + h) * p.S + s;
          p.qn[row] = sqrtf(qq);
          p.qmu[row] = qm;
          if ((s & 15) == 15) {  // last token of a granule (S and s0 are multiples of 16)
            const int64_t at = (int64_t(b) * p.H + h) * (p.S >> 4) + (s >> 4);
            p.pkmax[at] = kmax2;
            p.pqmax[at] = qmax2;
          }
        }
        if ((s & 15) == 15) kmax2 = qmax2 = 0.f;
      }
    }
  }
}

// Per (b, h), one block: the squared-norm maxima of every frame (its granules
// in order), the head maxima kmax and qmax and the head bound; then per query
// frame g the key-norm maximum kvis[g] its rows use, its bound and its flag:
//   bound_mode 0: kvis[g] = kmax, bound[g] = scale * qmax * kmax;
//   bound_mode 1: kvis[g] = max over the frames g sees (reference frame and the
//                 video frames within the window) of the frame's key maximum,
//                 bound[g] = scale * (max ||q|| over frame g) * kvis[g].
// The head flag is set when every query frame of the head is eligible.
__global__ __launch_bounds__(256) void final_kernel(NormParams p) {
  // squared norms are >= 0, so their float bit patterns order like the values
  // and an integer max is exact (and independent of the order of updates)
  __shared__ int kf2i[sfa::kMaxFrameSlots], qf2i[sfa::kMaxFrameSlots];
  __shared__ float k2s[256], q2s[256];
  const int bh = blockIdx.x;
  if (bh == 0 && threadIdx.x < sfa::kQueueWords) p.queue[threadIdx.x] = 0;
  // the split items' counters: block bh clears its share
  for (int i = bh * 256 + threadIdx.x; i < p.nsplit_cnt; i += gridDim.x * 256) p.split_cnt[i] = 0;
  const int nf = p.F + 1;
  const int gpf = p.T / 16;  // granules per frame
  const int ngran = p.S / 16;
  for (int f = threadIdx.x; f < nf; f += 256) kf2i[f] = qf2i[f] = 0;
  __syncthreads();
  const float* pk = p.pkmax + int64_t(bh) * ngran;
  const float* pq = p.pqmax + int64_t(bh) * ngran;
  for (int g = threadIdx.x; g < ngran; g += 256) {
    const int f = g / gpf;
    atomicMax(&kf2i[f], __float_as_int(pk[g]));
    atomicMax(&qf2i[f], __float_as_int(pq[g]));
  }
  __syncthreads();
  auto kf2 = [&](int f) { return __int_as_float(kf2i[f]); };
  auto qf2 = [&](int f) { return __int_as_float(qf2i[f]); };
  float k2 = 0.f, q2 = 0.f;
  for (int f = threadIdx.x; f < nf; f += 256) {
    k2 = fmaxf(k2, kf2(f));
    q2 = fmaxf(q2, qf2(f));
  }
  k2s[threadIdx.x] = k2;
  q2s[threadIdx.x] = q2;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (int(threadIdx.x) < w) {
      k2s[threadIdx.x] = fmaxf(k2s[threadIdx.x], k2s[threadIdx.x + w]);
      q2s[threadIdx.x] = fmaxf(q2s[threadIdx.x], q2s[threadIdx.x + w]);
    }
    __syncthreads();
  }
  const float kmax = sqrtf(k2s[0]);
  const float qmax = sqrtf(q2s[0]);
  const float hbound = p.scale * qmax * kmax;
  const bool limit_ok = p.bound_limit >= 0.f;
  int all = 1;
  for (int g = threadIdx.x; g < nf; g += 256) {
    float kv = kmax, fb = hbound;
    if (p.bound_mode == 1) {
      float m2 = kf2(0);  // the reference frame is visible to every query frame
      if (g > 0) {
        const int lo = max(1, g - p.w), hi = min(p.F, g + p.w);
        for (int f = lo; f <= hi; ++f) m2 = fmaxf(m2, kf2(f));
      }
      kv = sqrtf(m2);
      fb = p.scale * sqrtf(qf2(g)) * kv;
    }
    const uint8_t e = (limit_ok && fb <= p.bound_limit) ? 1 : 0;
    const int64_t at = int64_t(bh) * nf + g;
    p.kvis[at] = kv;
    p.fbound[at] = fb;
    p.felig[at] = e;
    all &= e;
  }
  all = __syncthreads_and(all);
  if (threadIdx.x == 0) {
    p.kmax[bh] = kmax;
    p.qmax[bh] = qmax;
    p.bound[bh] = hbound;
    p.elig[bh] = all ? 1 : 0;
  }
}

// K and V staged for the attention kernel (layouts in sfa_internal.h): one block per
// 64 tokens of one (b, h). The rows go through LDS so that both the row reads and the
// staged writes move whole 16-byte pieces of contiguous memory.
template <int D>
__global__ __launch_bounds__(256) void stage_kernel(NormParams p) {
  constexpr int CHUNK = 64;
  constexpr int PITCH = D + 8;  // elements; a 16-byte column of 16 rows hits 16 bank groups
  constexpr int CH = D / 8;     // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t tk[CHUNK * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t tv[CHUNK * PITCH];
  const int s0 = blockIdx.x * CHUNK;
  const int bh = blockIdx.y;
  const int b = bh / p.H, h = bh - b * p.H;
  const int n = min(CHUNK, p.S - s0);  // a multiple of 16
  const uint16_t* ksrc = p.k + b * p.ksb + h * p.ksh;
  const uint16_t* vsrc = p.v + b * p.vsb + h * p.vsh;
  for (int idx = threadIdx.x; idx < CHUNK * CH; idx += 256) {
    const int tok = idx / CH, c = idx % CH;
    if (tok < n) {
      *reinterpret_cast<uint4*>(&tk[tok * PITCH + 8 * c]) =
          *reinterpret_cast<const uint4*>(ksrc + int64_t(s0 + tok) * p.kss + 8 * c);
      *reinterpret_cast<uint4*>(&tv[tok * PITCH + 8 * c]) =
          *reinterpret_cast<const uint4*>(vsrc + int64_t(s0 + tok) * p.vss + 8 * c);
    }
  }
  __syncthreads();
  // the chunk's granules are contiguous in both staged tensors
  const int64_t base = (int64_t(bh) * p.S + s0) * D;  // elements
  uint4* kd = reinterpret_cast<uint4*>(p.kst + base);
  uint4* vd = reinterpret_cast<uint4*>(p.vst + base);
  const int units = n * CH;  // 16-byte pieces of the chunk in each staged tensor
  for (int u = threadIdx.x; u < units; u += 256) {
    // K piece u = (granule * CH + c) * 16 + key: row 16 * granule + key, elements 8c..8c+7
    const int gk = u / (CH * 16), ck = (u / 16) % CH, key = u % 16;
    kd[u] = *reinterpret_cast<const uint4*>(&tk[(16 * gk + key) * PITCH + 8 * ck]);
    // V piece u = (granule * D + e) * 2 + physical half: 8 keys of column e
    const int gv = u / (2 * D), e = (u / 2) % D, hp = u % 2;
    const int k0 = 16 * gv + 8 * (hp ^ ((e >> 3) & 1));
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = uint32_t(tv[(k0 + 2 * j) * PITCH + e]) |
             (uint32_t(tv[(k0 + 2 * j + 1) * PITCH + e]) << 16);
    vd[u] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t sfa_launch_norms(const sfa::NormParams& p, hipStream_t stream) {
  const dim3 grid(p.nchunk, p.B);
  // one lane per (head, 8 columns), rounded up to whole waves (no idle lanes at
  // H * d / 8 = 192, the 12-head layers), at most kThreads
  const int groups = p.H * (p.D / 8);
  const dim3 block(groups < kThreads ? (groups + 63) / 64 * 64 : kThreads);
  hipLaunchKernelGGL(ksum_kernel, grid, block, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kmean_kernel, dim3(p.B * p.H), dim3(kReduceThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.D == 128)
    hipLaunchKernelGGL(stats_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(stats_kernel<64>, grid, block, 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(final_kernel, dim3(p.B * p.H), dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return sfa_launch_stage(p, stream);
}

hipError_t sfa_launch_stage(const sfa::NormParams& p, hipStream_t stream) {
  const dim3 sgrid((p.S + 63) / 64, p.B * p.H);
  if (p.D == 128)
    hipLaunchKernelGGL(stage_kernel<128>, sgrid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(stage_kernel<64>, sgrid, dim3(256), 0, stream, p);
  return hipGetLastError();
}
