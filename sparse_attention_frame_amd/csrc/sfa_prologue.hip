// Fused attention prologue (gfx950): RMSNorm, q/k/v projection, rotary
// embedding and head packing in one MFMA kernel that writes straight into the
// layout the attention reads.
//
// "HeyGen x Google Cloud: Bringing Avatar IV to TPUs", section "Layout as ABI"
// (Fig. 5): the chain normalisation -> rotary -> projection -> head packing is
// fused into one kernel whose output buffer is the consumer's input buffer.
//
// RMSNorm folds into the projection: rms(x) * gamma . W = rstd * x . (gamma W),
// so the weights are pre-multiplied by gamma once (sfa_prologue_fold, bf16) and
// the kernel scales each token's outputs by its inverse RMS (rstd_kernel, a
// memory-bound pre-pass). The contraction runs as D[feature][token] =
// W'[feature][:] . x[token][:] on v_mfma_f32_32x32x16_bf16 with W' as the A
// operand and x as the B operand, so the accumulator lane holds one token and
// 16 features; a head's rotation pairs (e, e + d/2) then sit in the same lane
// and the same register of two accumulator tiles, and the rotation, the row
// scale and the bf16 store into q, k or v [b][s][h][e] need no data exchange.
#include "sfa_attn.h"

namespace {

using sfa::ProParams;

// ---- inverse RMS per token: one wave per row of C elements ----
__global__ __launch_bounds__(256) void rstd_kernel(ProParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // b * S + s
  if (row >= int64_t(p.B) * p.S) return;
  const int b = int(row / p.S), s = int(row - int64_t(b) * p.S);
  const uint16_t* xr = p.x + b * p.xsb + int64_t(s) * p.xss;
  float acc = 0.f;
  for (int c = 8 * lane; c < p.C; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(wv[i] << 16), hi = __uint_as_float(wv[i] & 0xffff0000u);
      acc = fmaf(lo, lo, acc);
      acc = fmaf(hi, hi, acc);
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (lane == 0) p.rstd[row] = 1.0f / sqrtf(acc / float(p.C) + p.eps);
}

// ---- W' = bf16(gamma[c] * W[n][c]) ----
__global__ __launch_bounds__(256) void fold_kernel(const uint16_t* w, const uint16_t* gamma,
                                                   uint16_t* out, int rows, int cols) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;  // pair index
  const int64_t n = int64_t(rows) * cols / 2;
  if (i >= n) return;
  const int c = int((2 * i) % cols);
  const uint32_t wv = reinterpret_cast<const uint32_t*>(w)[i];
  const uint32_t gv = *reinterpret_cast<const uint32_t*>(gamma + c);
  const float a = __uint_as_float(wv << 16) * __uint_as_float(gv << 16);
  const float b = __uint_as_float(wv & 0xffff0000u) * __uint_as_float(gv & 0xffff0000u);
  reinterpret_cast<uint32_t*>(out)[i] = pack_bf16x2(a, b);
}

// ---- the fused projection ----
// LDS stage (64 KB): A = 256 W' rows x 128 B at [0, 32 KB), B = 256 x rows x
// 128 B at [32 KB, 64 KB); two stages. Row r keeps its 16-byte chunk c at
// position c ^ ((r >> 1) & 7), applied through the DMA source address, so the
// 16 lanes of one operand read hit 16 different bank groups.
constexpr int kStageBytes = 65536;
constexpr int kHalf = 32768;

__device__ inline void dma16(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)lds_dst, 16, 0, 0);
}

template <int D>
__global__ __launch_bounds__(512, 1) void prologue_kernel(ProParams p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave >> 2, wt = wave & 3;   // 128 features x 64 tokens per wave

  // workgroup -> (token tile, feature tile); each run of 8 * ntile_f workgroups
  // gives every XCD the feature tiles of one token tile (its x rows stay in L2)
  const int nf = p.ntile_f;
  const int nblk = nf * p.B * p.ntile_t;
  const int run = 8 * nf;
  int logical = blockIdx.x;
  if (int(blockIdx.x) < (nblk / run) * run) {
    const int c = blockIdx.x / run, r = blockIdx.x - c * run;
    logical = c * run + (r & 7) * nf + (r >> 3);
  }
  const int ttile = logical / nf, ftile = logical - ttile * nf;
  const int b = ttile / p.ntile_t;
  const int tok0 = (ttile - b * p.ntile_t) * sfa::kProTile;
  const int n0 = ftile * sfa::kProTile;

  // DMA slots of this wave: 8 x 1 KB per stage (slots 0-31 W' rows, 32-63 x rows)
  const char* srcb[8];
  uint32_t srco[8];
  int dsto[8];
  const char* wbase = reinterpret_cast<const char*>(p.w) + int64_t(n0) * p.C * 2;
  const char* xbase = reinterpret_cast<const char*>(p.x + b * p.xsb + int64_t(tok0) * p.xss);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int slot = wave * 8 + j;
    const int r = (slot & 31) * 8 + (lane >> 3);        // tile row
    const int c = (lane & 7) ^ ((r >> 1) & 7);          // logical chunk of this lane
    if (slot < 32) {
      srcb[j] = wbase;
      srco[j] = uint32_t(r * p.C * 2 + c * 16);
      dsto[j] = slot * 1024;
    } else {
      const int rr = min(r, p.S - 1 - tok0);             // past the sequence: repeat the last row
      srcb[j] = xbase;
      srco[j] = uint32_t(int64_t(rr) * p.xss * 2 + c * 16);
      dsto[j] = kHalf + (slot - 32) * 1024;
    }
  }
  auto issue = [&](int buf, int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      dma16(srcb[j] + uint64_t(srco[j]) + k0 * 2, lds + buf * kStageBytes + dsto[j]);
  };

  // operand read offsets: row bits 1..3 equal those of l32 for every tile
  const int sw = (l32 >> 1) & 7;
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int x = (((2 * ks + g) ^ sw) * 16);
    aoff[ks] = uint32_t(l32 * 128 + wf * 128 * 128 + x);
    boff[ks] = uint32_t(kHalf + l32 * 128 + wt * 64 * 128 + x);
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[f][t][i] = 0.f;

  const int nst = p.C / sfa::kProKStage;
  issue(0, 0);
  for (int st = 0; st < nst; ++st) {
    wait_vm<0>();
    __syncthreads();
    if (st + 1 < nst) issue((st + 1) & 1, (st + 1) * sfa::kProKStage);
    const char* sb = lds + (st & 1) * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[4], bb[2];
#pragma unroll
      for (int f = 0; f < 4; ++f)
        a[f] = *reinterpret_cast<const bf16x8*>(sb + aoff[ks] + f * 32 * 128);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        bb[t] = *reinterpret_cast<const bf16x8*>(sb + boff[ks] + t * 32 * 128);
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f], bb[t], acc[f][t], 0, 0, 0);
    }
  }

  // epilogue: row scale, rotation of q and k, bf16 store into [b][s][h][e]
  const int HD = p.H * D;
  const int which = n0 / HD;                  // 0 q, 1 k, 2 v (tiles never straddle)
  const int nw = n0 + 128 * wf - which * HD;  // first feature of this wave inside its tensor
  uint16_t* ob = p.out[which];
  const int64_t osb = p.osb[which], oss = p.oss[which], osh = p.osh[which];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = tok0 + 64 * wt + 32 * t + l32;
    const int tc = min(tok, p.S - 1);
    const float rs = p.rstd[int64_t(b) * p.S + tc];
    float y[4][16];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int i = 0; i < 16; ++i) y[f][i] = acc[f][t][i] * rs;
    if (which < 2) {
      // pairs: D = 128: tiles (0, 2), (1, 3); D = 64: tiles (0, 1), (2, 3)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int fa = D == 128 ? pr : 2 * pr;
        const int fb = D == 128 ? pr + 2 : 2 * pr + 1;
        const int jb = D == 128 ? 32 * pr : 0;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int j0 = jb + 8 * qd + 4 * g;
          const float4 c4 = *reinterpret_cast<const float4*>(p.cosv + int64_t(tc) * (D / 2) + j0);
          const float4 s4 = *reinterpret_cast<const float4*>(p.sinv + int64_t(tc) * (D / 2) + j0);
          const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float av = y[fa][4 * qd + u], bv = y[fb][4 * qd + u];
            y[fa][4 * qd + u] = av * cv[u] - bv * sv[u];
            y[fb][4 * qd + u] = av * sv[u] + bv * cv[u];
          }
        }
      }
    }
    if (tok < p.S) {
      uint16_t* orow = ob + b * osb + int64_t(tok) * oss;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int feat = nw + 32 * f;             // first feature of tile f
        const int h = feat / D, e0 = feat - h * D;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          uint2 w2;
          w2.x = pack_bf16x2(y[f][4 * qd], y[f][4 * qd + 1]);
          w2.y = pack_bf16x2(y[f][4 * qd + 2], y[f][4 * qd + 3]);
          *reinterpret_cast<uint2*>(orow + h * osh + e0 + 8 * qd + 4 * g) = w2;
        }
      }
    }
  }
}

}  // namespace

hipError_t sfa_launch_fold(const uint16_t* w, const uint16_t* gamma, uint16_t* out, int rows,
                           int cols, hipStream_t stream) {
  const int64_t pairs = int64_t(rows) * cols / 2;
  if (pairs > 0)
    hipLaunchKernelGGL(fold_kernel, dim3(unsigned((pairs + 255) / 256)), dim3(256), 0, stream, w,
                       gamma, out, rows, cols);
  return hipGetLastError();
}

hipError_t sfa_launch_prologue(const sfa::ProParams& p, hipStream_t stream) {
  const int64_t rows = int64_t(p.B) * p.S;
  hipLaunchKernelGGL(rstd_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto kern = p.d == 128 ? prologue_kernel<128> : prologue_kernel<64>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStageBytes);
  if (e != hipSuccess) return e;
  const int blocks = p.ntile_f * p.B * p.ntile_t;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(512), 2 * kStageBytes, stream, p);
  return hipGetLastError();
}
