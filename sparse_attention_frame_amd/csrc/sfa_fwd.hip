// The attention kernel (product path) and its launcher; the tile machinery and
// the method description are in sfa_attn.h.
#include "sfa_attn.h"

namespace {

// Persistent workgroups (at most one per CU). Item index i belongs to XCD i % 8
// (the order decode_item is built for); the workgroups of XCD x (blockIdx % 8 ==
// x: workgroups are handed to the XCDs round robin) take x, x + 8, ... from
// their XCD's counter, largest items first, and once it runs dry take items
// from the other XCDs' counters, so no XCD idles while another still has work.
// Every attempt advances one counter, so the loop ends after at most eight
// failed attempts. The last workgroup to run dry sets the counters back to zero
// for the next launch.
template <int D, int WAVES, int QT, int NBUF>
__global__ __launch_bounds__(WAVES * 64, 1) void fwd_kernel(FwdParams p) {
  using A = Attn<D, WAVES, QT, NBUF>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int next_item;
  const int x = blockIdx.x & 7;
  int q = 0;  // queues found empty so far, in the order x, x + 1, ...
  for (;;) {
    if (threadIdx.x == 0) {
      int idx = -1;
      while (q < 8) {
        const int xq = (x + q) & 7;
        const int c = atomicAdd(&p.queue[xq], 1);
        const int cand = xq + 8 * c;
        if (cand < p.items) {
          idx = cand;
          break;
        }
        ++q;
      }
      next_item = idx;
    }
    __syncthreads();  // also: every wave is done with the previous item's LDS stages
    const int idx = next_item;
    __syncthreads();
    if (idx < 0) break;
    const Item it = sfa::decode_item(idx, p.frame_order, p.B, p.H, p.nqb, p.items);
    if (p.felig[(int64_t(it.b) * p.H + it.h) * (p.F + 1) + it.f])
      A::run_fixed(p, it, lds);
    else
      A::run_online(p, it, lds);
  }
  if (threadIdx.x == 0 && atomicAdd(&p.queue[8], 1) == int(gridDim.x) - 1) {
#pragma unroll
    for (int i = 0; i < 9; ++i) atomicExch(&p.queue[i], 0);
  }
}

int cu_count() {
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

template <int D, int WAVES, int QT, int NBUF>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  using A = Attn<D, WAVES, QT, NBUF>;
  auto kern = fwd_kernel<D, WAVES, QT, NBUF>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, A::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int grid = p.items < cu_count() ? p.items : cu_count();
  hipLaunchKernelGGL(kern, dim3(grid), dim3(A::kThreads), A::LDS_BYTES, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t sfa_launch_fwd(const sfa::FwdParams& p, int head_dim, int waves, int qt, int stages,
                          hipStream_t stream) {
  if (p.items <= 0) return hipSuccess;
  if (waves == 12) {  // 96-key stages: at most three fit in LDS
    if (head_dim == 128) return stages == 2 ? launch<128, 12, 1, 2>(p, stream)
                                            : launch<128, 12, 1, 3>(p, stream);
    return stages == 2 ? launch<64, 12, 1, 2>(p, stream) : launch<64, 12, 1, 3>(p, stream);
  }
  if (head_dim == 128) {
    if (waves == 4) {
      if (stages == 2) return launch<128, 4, 2, 2>(p, stream);
      if (stages == 3) return launch<128, 4, 2, 3>(p, stream);
      return launch<128, 4, 2, 4>(p, stream);
    }
    if (qt == 2) {
      if (stages == 2) return launch<128, 8, 2, 2>(p, stream);
      if (stages == 3) return launch<128, 8, 2, 3>(p, stream);
      return launch<128, 8, 2, 4>(p, stream);
    }
    if (stages == 2) return launch<128, 8, 1, 2>(p, stream);
    if (stages == 3) return launch<128, 8, 1, 3>(p, stream);
    return launch<128, 8, 1, 4>(p, stream);
  }
  if (waves == 4) {
    if (stages == 2) return launch<64, 4, 2, 2>(p, stream);
    if (stages == 3) return launch<64, 4, 2, 3>(p, stream);
    return launch<64, 4, 2, 4>(p, stream);
  }
  if (qt == 2) {
    if (stages == 2) return launch<64, 8, 2, 2>(p, stream);
    if (stages == 3) return launch<64, 8, 2, 3>(p, stream);
    return launch<64, 8, 2, 4>(p, stream);
  }
  if (stages == 2) return launch<64, 8, 1, 2>(p, stream);
  if (stages == 3) return launch<64, 8, 1, 3>(p, stream);
  return launch<64, 8, 1, 4>(p, stream);
}
