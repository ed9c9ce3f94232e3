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
// the kernel scales each token's outputs by its inverse RMS, which it sums up
// from the x operands it already holds. The contraction runs as D[feature][token] =
// W'[feature][:] . x[token][:] on v_mfma_f32_32x32x16_bf16 with W' as the A
// operand and x as the B operand, so the accumulator lane holds one token and
// 16 features; a head's rotation pairs (e, e + d/2) then sit in the same lane
// and the same register of two accumulator tiles, and the rotation, the row
// scale and the bf16 store into q, k or v [b][s][h][e] need no data exchange.
#include "sfa_gfx950.h"

namespace {

using sfa::ProParams;

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
// A workgroup computes a 256-feature x 256-token tile; each wave owns 128
// features x (512 / WAVES) tokens, so every 16-byte LDS operand read of W'
// feeds 16 / WAVES MFMAs and every read of x feeds four. LDS stage (64 KB):
// A = 256 W' rows x 128 B at [0, 32 KB), B = 256 x rows x 128 B at
// [32 KB, 64 KB); two stages. Row r keeps its 16-byte chunk c at position
// c ^ ((r >> 1) & 7), applied through the DMA source address, so the 16 lanes
// of one operand read hit 16 bank groups. The token's sum of squares comes from
// the same B operand registers (dot2 of each bf16 pair with itself), so the
// norm needs no pass of its own.
constexpr int kStageBytes = 65536;
constexpr int kHalf = 32768;

// Wait for every LDS read of this wave (vmcnt and expcnt left at their maxima).
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier for LDS reads and writes by instructions only: each wave retires its
// own LDS operations, then meets the others; the empty asm statements keep the compiler
// from moving memory accesses across it. A fence (as in __syncthreads) would also wait for
// every store and LDS DMA still in flight (one in-order counter covers both); here each
// wave waits beforehand for exactly the DMA it needs (wait_vm).
__device__ inline void barrier_lds() {
  wait_lgkm0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline void dma16(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)lds_dst, 16, 0, 0);
}

// Workgroup -> (feature tile, token tile). Workgroups go to the 8 XCDs round
// robin, so XCD x runs workgroups x, x + 8, ...; each XCD takes a contiguous
// share of a grouped order that walks 6 token tiles x 6 feature tiles at a
// time, so the ~32 workgroups an XCD runs at once share their W' and x slices
// through its L2 (12 slices fetched per 36 tiles instead of 2 per tile).
__device__ inline void tile_of(int bid, int nf, int T, int* ftile, int* ttile) {
  constexpr int G = 6, FG = 6;
  const int nblk = nf * T;
  const int per = nblk / 8, rem = nblk - 8 * (nblk / 8);
  const int x = bid & 7, i = bid >> 3;
  const int j = x * per + min(x, rem) + i;
  const int tg = j / (G * nf);
  const int gt = min(G, T - tg * G);
  const int r = j - tg * G * nf;
  const int fg = r / (gt * FG);
  const int rr = r - fg * gt * FG;
  *ttile = tg * G + rr % gt;
  *ftile = fg * FG + rr / gt;
}

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void prologue_kernel(ProParams p) {
  constexpr int WPH = WAVES / 2;        // waves per 128-feature half
  constexpr int TT = 8 / WPH;           // 32-token tiles per wave
  constexpr int SL = 64 / WAVES;        // 1 KB DMA requests per wave per stage
  constexpr int NST = 8;                // output stores per wave per 32-token tile
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave / WPH, wt = wave % WPH;
  // DMA: the first half of the waves fetches the 256 W' rows, the second the 256 x rows
  const bool is_w = wave < WPH;
  char* const dst0 = lds + (is_w ? 0 : kHalf) + wt * SL * 1024;
  const int nst = p.C / sfa::kProKStage;
  const int ntiles = p.ntile_f * p.B * p.ntile_t;
  const int HD = p.H * D;

  // This wave's DMA source for tile tl: a base and one 32-bit offset per request.
  struct Src {
    const char* base;
    uint32_t off[SL];
  };
  auto source = [&](int tl, Src& s) {
    int ftile, ttile;
    tile_of(tl, p.ntile_f, p.B * p.ntile_t, &ftile, &ttile);
    const int b = ttile / p.ntile_t;
    const int tok0 = (ttile - b * p.ntile_t) * sfa::kProTile;
    const int n0 = ftile * sfa::kProTile;
    s.base = is_w ? reinterpret_cast<const char*>(p.w) + int64_t(n0) * p.C * 2
                  : reinterpret_cast<const char*>(p.x + b * p.xsb + int64_t(tok0) * p.xss);
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      const int r = (wt * SL + j) * 8 + (lane >> 3);                  // tile row
      const int c = (lane & 7) ^ ((r >> 1) & 7);                      // logical chunk of this lane
      const int rr = is_w ? r : min(r, p.S - 1 - tok0);               // past S: repeat the last row
      s.off[j] = uint32_t(int64_t(rr) * (is_w ? p.C : p.xss) * 2 + c * 16);
    }
  };
  auto issue = [&](const Src& s, int st, int buf) {
    char* d = dst0 + buf * kStageBytes;
    const int koff = st * sfa::kProKStage * 2;
#pragma unroll
    for (int j = 0; j < SL; ++j) dma16(s.base + uint64_t(s.off[j]) + koff, d + j * 1024);
  };

  // operand read offsets: row bits 1..3 equal those of l32 for every tile
  const int sw = (l32 >> 1) & 7;
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int x = (((2 * ks + g) ^ sw) * 16);
    aoff[ks] = uint32_t(l32 * 128 + wf * 128 * 128 + x);
    boff[ks] = uint32_t(kHalf + l32 * 128 + wt * TT * 32 * 128 + x);
  }
  struct Frags {
    bf16x8 a[4], b[TT];
  };

  // Persistent: the grid is a multiple of 8 workgroups, so every tile a workgroup takes
  // keeps its XCD (tile & 7 == blockIdx.x & 7) and each XCD walks its share of the
  // grouped order 32 tiles at a time. Tiles overlap: stage 0 of the next tile is fetched
  // into the buffer the last-but-one stage frees, while the last stage is computed, and
  // the tile's output stores are issued after that fetch and before the fetch of stage 1,
  // so the next tile waits for its stage 0 only, never for the stores.
  int par = 0;         // stage st of the current tile sits in buffer (st + par) & 1
  bool have0 = false;  // stage 0 of the current tile was fetched by the previous one
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    int ftile, ttile;
    tile_of(tile, p.ntile_f, p.B * p.ntile_t, &ftile, &ttile);
    const int b = ttile / p.ntile_t;
    const int tok0 = (ttile - b * p.ntile_t) * sfa::kProTile;
    const int n0 = ftile * sfa::kProTile;
    const int next = tile + gridDim.x;
    Src cur;
    source(tile, cur);

    auto load = [&](Frags& f, int st, int ks) {
      const char* sb = lds + ((st + par) & 1) * kStageBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(sb + aoff[ks] + i * 4096);
#pragma unroll
      for (int i = 0; i < TT; ++i) f.b[i] = *reinterpret_cast<const bf16x8*>(sb + boff[ks] + i * 4096);
    };

    f32x16 acc[4][TT];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[f][t][i] = 0.f;
    float ss[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) ss[t] = 0.f;

    auto mma = [&](const Frags& f) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const auto v = __builtin_bit_cast(uint4, f.b[t]);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2 h = __builtin_bit_cast(bf16x2, u[i]);
          ss[t] = __builtin_amdgcn_fdot2_f32_bf16(h, h, ss[t], false);
        }
        asm volatile("" : "+v"(ss[t]));   // keep the sums here, beside their operands
      }
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int t = 0; t < TT; ++t)
          acc[fi][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[fi], f.b[t], acc[fi][t], 0, 0, 0);
    };

    // Stages 0 and 1 in flight; wait for stage 0 only. What may still be outstanding
    // behind it: the stage 1 fetch and, when stage 0 came from the previous tile, that
    // tile's TT * NST output stores (issued between the two fetches).
    if (!have0) issue(cur, 0, par & 1);
    if (nst > 1) issue(cur, 1, (1 + par) & 1);
    if (have0) {
      if (nst > 1) wait_vm<TT * NST + SL>(); else wait_vm<TT * NST>();
    } else {
      if (nst > 1) wait_vm<SL>(); else wait_vm<0>();
    }
    barrier_lds();
    have0 = false;
    // K loop: the DMA of stage st + 2 starts once every wave has read stage st, and the
    // first operands of stage st + 1 load under the last MFMAs of stage st. Each MFMA
    // group runs while the operands of the next one load. The explicit lgkmcnt(0) before
    // each load batch retires the batch issued one group earlier (long landed by then), so
    // the compiler sees no LDS read pending when the MFMAs use it and does not wait for
    // the batch just issued; the sched_barrier fences keep the scheduler from moving
    // loads next to their first use.
    Frags fr[2];
    load(fr[0], 0, 0);
    auto step = [&](Frags& nxt, int st, int ks, Frags& now) {
      wait_lgkm0();
      __builtin_amdgcn_sched_barrier(0);
      load(nxt, st, ks);
      __builtin_amdgcn_sched_barrier(0);
      mma(now);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int st = 0; st < nst; ++st) {
      step(fr[1], st, 1, fr[0]);
      step(fr[0], st, 2, fr[1]);
      step(fr[1], st, 3, fr[0]);
      if (st + 1 < nst) {
        wait_vm<0>();          // stage st + 1 has landed (this wave's part) ...
        barrier_lds();       // ... everybody's, and everybody has read stage st
        if (st + 2 < nst) {
          issue(cur, st + 2, (st + 2 + par) & 1);
        } else if (next < ntiles) {
          // the buffer of stage st = nst - 2 is free: the next tile's stage 0 goes there
          Src nx;
          source(next, nx);
          issue(nx, 0, (st + par) & 1);
          have0 = true;
        }
      }
      // unconditional (after the last stage it reads a stale buffer and is unused), so
      // both paths into the next iteration leave the same loads in flight
      step(fr[0], st + 1, 0, fr[1]);
    }

    // epilogue: row scale, rotation of q and k, bf16 store into [b][s][h][e] through LDS.
    // The lane index is re-read per tile (an empty asm the compiler cannot see through) so
    // that the epilogue's lane-dependent addresses are not hoisted out of the tile loop,
    // where they would stay live across the K loop and push it past 256 registers.
    int lane_t = lane;
    asm volatile("" : "+v"(lane_t));
    const int l32 = lane_t & 31, g = lane_t >> 5;
    // inverse RMS of the tokens of this lane: the two lane halves hold alternate chunks
    float rs[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float tot = ss[t] + __shfl_xor(ss[t], 32, 64);
      rs[t] = 1.0f / sqrtf(tot / float(p.C) + p.eps);
    }
    const int which = n0 / HD;                  // 0 q, 1 k, 2 v (tiles never straddle)
    const int nw = n0 + 128 * wf - which * HD;  // first feature of this wave inside its tensor
    uint16_t* ob = p.out[which];
    const int64_t osb = p.osb[which], oss = p.oss[which], osh = p.osh[which];
    // the last stage's buffer is free once every wave has passed this barrier (the other
    // one may hold the next tile's stage 0); each wave stages one 32-token tile at a time,
    // 32 tokens x 256 B, so the global stores are whole rows
    barrier_lds();
    char* stg = lds + ((nst - 1 + par) & 1) * kStageBytes + wave * (32 * 256);
    // Token tile t: scaled and rotated values -> bf16 staging rows -> whole-row stores.
    // Tile t + 1 is computed (its cos / sin loads waited for) before tile t's stores are
    // issued, so no wait in the epilogue waits for a store: one in-order counter covers
    // loads, stores and the LDS DMA, and the stores drain under the next tile's K loop.
    auto compute = [&](int t, float (&y)[4][16]) {
      const int tc = min(tok0 + wt * TT * 32 + 32 * t + l32, p.S - 1);
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) y[f][i] = acc[f][t][i] * rs[t];
      if (which < 2) {
        // pairs: D = 128: tiles (0, 2), (1, 3); D = 64: tiles (0, 1), (2, 3)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const int fa = D == 128 ? pr : 2 * pr;
          const int fb = D == 128 ? pr + 2 : 2 * pr + 1;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int j0 = (D == 128 ? 32 * pr : 0) + 8 * qd + 4 * g;
            const float4 c4 = *reinterpret_cast<const float4*>(p.cosv + int64_t(tc) * (D / 2) + j0);
            const float4 s4 = *reinterpret_cast<const float4*>(p.sinv + int64_t(tc) * (D / 2) + j0);
            const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float av = y[fa][4 * qd + u], bv = y[fb][4 * qd + u];
              y[fa][4 * qd + u] = fmaf(av, cv[u], -(bv * sv[u]));  // rounding fixed in the source
              y[fb][4 * qd + u] = fmaf(av, sv[u], bv * cv[u]);
            }
          }
        }
      }
    };
    // bf16 into this wave's staging rows: [token][128 features] (256 B per token), the
    // 16-byte chunk index XOR-swizzled by token % 16
    auto stage = [&](const float (&y)[4][16]) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          uint2 w2;
          w2.x = pack_bf16x2(y[f][4 * qd], y[f][4 * qd + 1]);
          w2.y = pack_bf16x2(y[f][4 * qd + 2], y[f][4 * qd + 3]);
          *reinterpret_cast<uint2*>(stg + l32 * 256 + (((4 * f + qd) ^ (l32 & 15)) * 16) + 8 * g) = w2;
        }
    };
    // write back whole rows: 16 lanes cover one token's 256 contiguous bytes (one head of
    // 128, or two of 64), 4 tokens per instruction. Every store is issued (the fetch waits
    // at the top of the tile loop count them): a token past S rewrites token S - 1, whose
    // x row, norm, cos / sin and hence output bytes it repeats exactly.
    auto flush = [&](int t) {
#pragma unroll
      for (int i = 0; i < NST; ++i) {
        const int r = 4 * i + (lane_t >> 4), c = lane_t & 15;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 256 + ((c ^ (r & 15)) * 16));
        const int tok = min(tok0 + wt * TT * 32 + 32 * t + r, p.S - 1);
        const int feat = nw + 8 * c;
        const int h = feat / D, e = feat - h * D;
        *reinterpret_cast<uint4*>(ob + b * osb + int64_t(tok) * oss + h * osh + e) = v;
      }
    };
    float y[4][16];
    compute(0, y);
    stage(y);
#pragma unroll
    for (int t = 1; t < TT; ++t) {
      compute(t, y);
      flush(t - 1);
      stage(y);
    }
    flush(TT - 1);
    // every wave has read its staging rows back before the next tile's stage 1 fetch
    // reuses the buffer
    barrier_lds();
    par = (nst + par) & 1;
  }
}

}  // namespace

// Compute units of the current device, cached per device (256 if the query fails).
static int pro_cu_count() {
  static int n[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (n[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 8)
      c = 256;
    n[dev] = c;
  }
  return n[dev];
}

hipError_t sfa_launch_fold(const uint16_t* w, const uint16_t* gamma, uint16_t* out, int rows,
                           int cols, hipStream_t stream) {
  const int64_t pairs = int64_t(rows) * cols / 2;
  if (pairs > 0)
    hipLaunchKernelGGL(fold_kernel, dim3(unsigned((pairs + 255) / 256)), dim3(256), 0, stream, w,
                       gamma, out, rows, cols);
  return hipGetLastError();
}

hipError_t sfa_launch_prologue(const sfa::ProParams& p, hipStream_t stream) {
  hipError_t e;
  // 8 waves (two per SIMD, 242 registers): measured faster than 4 waves of 128 x 128
  // (which needs all 512 registers and spills in the epilogue)
  constexpr int waves = 8;
  auto kern = p.d == 128 ? prologue_kernel<128, waves> : prologue_kernel<64, waves>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStageBytes);
  if (e != hipSuccess) return e;
  // persistent: one workgroup per compute unit (the two stages take 128 KB of LDS), a
  // multiple of 8 so that each workgroup's tiles stay on its XCD
  const int tiles = p.ntile_f * p.B * p.ntile_t;
  const int cus = pro_cu_count() & ~7;
  const int blocks = tiles < cus ? tiles : cus;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(waves * 64), 2 * kStageBytes, stream, p);
  return hipGetLastError();
}
