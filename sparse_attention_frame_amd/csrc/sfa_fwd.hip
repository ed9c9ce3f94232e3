// The attention kernel (product path) and its launcher; the tile machinery and
// the method description are in sfa_attn.h.
#include "sfa_attn.h"

namespace {

template <int D, int WAVES, int QT, int NBUF>
__global__ __launch_bounds__(WAVES * 64, 1) void fwd_kernel(FwdParams p) {
  using A = Attn<D, WAVES, QT, NBUF>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const Item it = sfa::decode_item(blockIdx.x, p.frame_order, p.B, p.H, p.nqb, p.items);
  if (p.felig[(int64_t(it.b) * p.H + it.h) * (p.F + 1) + it.f])
    A::run_fixed(p, it, lds);
  else
    A::run_online(p, it, lds);
}

template <int D, int WAVES, int QT, int NBUF>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  using A = Attn<D, WAVES, QT, NBUF>;
  auto kern = fwd_kernel<D, WAVES, QT, NBUF>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, A::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.items), dim3(A::kThreads), A::LDS_BYTES, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t sfa_launch_fwd(const sfa::FwdParams& p, int head_dim, int waves, int stages,
                          hipStream_t stream) {
  if (p.items <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (waves == 4) {
      if (stages == 2) return launch<128, 4, 2, 2>(p, stream);
      if (stages == 3) return launch<128, 4, 2, 3>(p, stream);
      return launch<128, 4, 2, 4>(p, stream);
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
  if (stages == 2) return launch<64, 8, 1, 2>(p, stream);
  if (stages == 3) return launch<64, 8, 1, 3>(p, stream);
  return launch<64, 8, 1, 4>(p, stream);
}

