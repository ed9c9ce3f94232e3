// Matrix-core microbenchmarks for gfx950 (declared in sfa_probe.h): the measured
// v_mfma_f32_32x32x16_bf16 peak and the ceiling of the attention tile loop when its
// operands already sit in LDS. Nothing here is part of the attention library; the
// benchmark links it to report how far the attention kernel is from these ceilings.
#include <hip/hip_runtime.h>

#include "sfa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMaxGroups = 1024;
constexpr int kMaxThreads = 512;
constexpr int kLdsBytes = 65536;     // four 16 KB slots: 32 keys of K, then 32 keys of V^T
constexpr bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline void record_clock(long long* tim, long long r0, long long c0) {
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  const long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    tim[2 * blockIdx.x] = r1 - r0;
    tim[2 * blockIdx.x + 1] = c1 - c0;
  }
}

// Four independent accumulator chains per wave, 16 MFMAs per iteration.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void chain_kernel(float* sink, long long* tim,
                                                               int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)0.5f;
  }
  f32x16 acc[4];
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  const long long c0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  record_clock(tim, r0, c0);
  float r = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 16; ++i) r += acc[j][i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// The attention tile loop for d = 128 with NT 32-row query tiles per wave: per 32-key
// tile, S^T = K Q^T (8 k-steps, key operand from LDS), P = exp2(S c - m) packed to bf16
// with its row sum, O^T += V^T P^T (2 key halves x 4 d-tiles, V^T operand from LDS). The
// LDS slot rotates over four 16 KB slots so the operand reads are not hoisted. The LDS
// offsets follow the staged granule layouts of the attention kernel: key lanes read 16
// distinct 16-byte bank groups.
template <int WAVES, int NT, bool SOFTMAX>
__global__ __launch_bounds__(WAVES * 64, 1) void tile_kernel(float* sink, long long* tim,
                                                              int iters, float c) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += blockDim.x)
    reinterpret_cast<uint32_t*>(lds)[i] = 0x3c003c00u ^ (i & 0x003f003f);
  __syncthreads();
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  bf16x8 q[NT][8];
  for (int t = 0; t < NT; ++t)
    for (int ks = 0; ks < 8; ++ks)
      for (int i = 0; i < 8; ++i) q[t][ks][i] = (__bf16)(0.01f * (lane + i + ks + t));
  f32x16 o[NT][4];
  for (int t = 0; t < NT; ++t)
    for (int d = 0; d < 4; ++d)
      for (int i = 0; i < 16; ++i) o[t][d][i] = 0.f;
  float m[NT], l[NT];
  for (int t = 0; t < NT; ++t) {
    m[t] = 1.f + t;
    l[t] = 0.f;
  }
  const uint32_t kbase = (l32 >> 4) * 4096 + g * 256 + (l32 & 15) * 16;
  const uint32_t vbase = 8192 + l32 * 32 + ((g ^ ((l32 >> 3) & 1)) * 16);
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  const long long c0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    const uint32_t slot = (it & 3) * 16384;
    f32x16 s[NT];
    for (int t = 0; t < NT; ++t)
      for (int i = 0; i < 16; ++i) s[t][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + slot + kbase + 512 * ks);
#pragma unroll
      for (int t = 0; t < NT; ++t) s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[t][ks], s[t], 0, 0, 0);
    }
    uint32_t p[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (SOFTMAX) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t][2 * i], c, -m[t]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t][2 * i + 1], c, -m[t]));
          p[t][i] = pack_bf16x2(p0, p1);
          l[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[t][i]), kOnes, l[t], false);
        } else {
          p[t][i] = __builtin_bit_cast(uint32_t, s[t][2 * i]);
        }
      }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + slot + vbase + h * 4096 + dt * 1024);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 b = __builtin_bit_cast(
              bf16x8, make_uint4(p[t][4 * h], p[t][4 * h + 1], p[t][4 * h + 2], p[t][4 * h + 3]));
          o[t][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[t][dt], 0, 0, 0);
        }
      }
  }
  record_clock(tim, r0, c0);
  float r = 0.f;
  for (int t = 0; t < NT; ++t) {
    r += l[t];
    for (int d = 0; d < 4; ++d)
      for (int i = 0; i < 16; ++i) r += o[t][d][i];
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

int cu_count(int dev) {
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return c;
}

template <typename K, typename... Args>
hipError_t launch(K kern, int grid, int threads, int lds, hipStream_t s, Args... args) {
  if (lds > 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, s, args...);
  return hipGetLastError();
}

hipError_t dispatch(int kind, int waves, int grid, int iters, float* sink, long long* tim,
                    hipStream_t s) {
  const int th = waves * 64;
  if (kind == SFA_PROBE_MFMA_CHAIN)
    return waves == 8 ? launch(chain_kernel<8>, grid, th, 0, s, sink, tim, iters)
                      : launch(chain_kernel<4>, grid, th, 0, s, sink, tim, iters);
  const float c = 0.18f;
  if (kind == SFA_PROBE_TILE_LOOP)
    return waves == 8 ? launch(tile_kernel<8, 1, true>, grid, th, kLdsBytes, s, sink, tim, iters, c)
                      : launch(tile_kernel<4, 1, true>, grid, th, kLdsBytes, s, sink, tim, iters, c);
  if (kind == SFA_PROBE_TILE_LOOP64)
    return waves == 8 ? launch(tile_kernel<8, 2, true>, grid, th, kLdsBytes, s, sink, tim, iters, c)
                      : launch(tile_kernel<4, 2, true>, grid, th, kLdsBytes, s, sink, tim, iters, c);
  return waves == 8 ? launch(tile_kernel<8, 1, false>, grid, th, kLdsBytes, s, sink, tim, iters, c)
                    : launch(tile_kernel<4, 1, false>, grid, th, kLdsBytes, s, sink, tim, iters, c);
}

}  // namespace

extern "C" size_t sfa_probe_scratch_bytes(void) {
  return size_t(kMaxGroups) * kMaxThreads * sizeof(float) + size_t(kMaxGroups) * 2 * sizeof(long long);
}

extern "C" int sfa_probe_run(int32_t kind, int32_t waves, int32_t iters, void* scratch,
                             size_t scratch_bytes, void* stream, sfa_probe_result* result) {
  if (kind < SFA_PROBE_MFMA_CHAIN || kind > SFA_PROBE_TILE_NOEXP) return -1;
  if ((waves != 4 && waves != 8) || iters < 1 || !result || !scratch) return -1;
  if (scratch_bytes < sfa_probe_scratch_bytes()) return -1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -3;
  const int grid = cu_count(dev);
  int wall_khz = 0;
  if (grid < 1 || grid > kMaxGroups ||
      hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
      wall_khz <= 0)
    return -3;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* sink = static_cast<float*>(scratch);
  long long* tim = reinterpret_cast<long long*>(static_cast<char*>(scratch) +
                                                size_t(kMaxGroups) * kMaxThreads * sizeof(float));
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  // a short launch first brings the clock up
  if (e == hipSuccess) e = dispatch(kind, waves, grid, iters / 8 + 1, sink, tim, s);
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) e = dispatch(kind, waves, grid, iters, sink, tim, s);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  long long h[2 * kMaxGroups];
  if (e == hipSuccess) e = hipMemcpy(h, tim, sizeof(long long) * 2 * grid, hipMemcpyDeviceToHost);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return -3;
  double wall = 0, cyc = 0;
  for (int i = 0; i < grid; ++i) {
    wall += double(h[2 * i]);
    cyc += double(h[2 * i + 1]);
  }
  const int per_iter = kind == SFA_PROBE_TILE_LOOP64 ? 32 : 16;   // MFMAs per wave per iteration
  const double mfma = double(grid) * waves * per_iter * iters;
  result->ms = ms;
  result->tflops = mfma * 32768.0 / (double(ms) * 1e-3) / 1e12;
  result->clock_ghz = wall > 0 ? cyc / wall * double(wall_khz) * 1e-6 : 0.0;
  const double simds = double(grid) * 4;
  result->mfma_busy = result->clock_ghz > 0
                          ? (mfma / simds) * 32.0 / (double(ms) * 1e-3 * result->clock_ghz * 1e9)
                          : 0.0;
  return 0;
}
