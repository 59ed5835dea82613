// Combine: y[t] = sum over token t's kept slots j (in j order) of w[t,j] * y_perm[dest[t,j]].
//
// Method: y = sum_{i in K(x)} g_i(x) E_i(x) (kwkr.cn page on sparse activation, section 2.1),
// which the page's section 3.2 code computes as a weighted scatter-add of the expert outputs
// back onto their tokens. Here each token gathers its own k rows instead, so no atomics are
// needed and the sum order is fixed: float32 accumulation in j order, one final rounding.
// Dropped slots (dest = -1) contribute exactly zero (the page's section 2.3 and 6.1). With a
// shared expert (lpnh.cn page, "Mixture of Experts（MoE）原理与工程落地全指南",
// section 2.3) each token's sum starts from its output.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

// Each thread produces 8 consecutive outputs of one token.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const float* __restrict__ y_shared,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ w, int T, int d, int k, int R,
                                                      void* __restrict__ y) {
  const int groups = d >> 3;
  const long long items = static_cast<long long>(T) * groups;
  for (long long it = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; it < items;
       it += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int t = static_cast<int>(it / groups);
    const int c = static_cast<int>(it - static_cast<long long>(t) * groups) * 8;
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    if (y_shared != nullptr) {
      const floatx4* sh = reinterpret_cast<const floatx4*>(y_shared + static_cast<size_t>(t) * d + c);
      acc0 = sh[0];
      acc1 = sh[1];
    }
    for (int j = 0; j < k; ++j) {
      const int r = dest[static_cast<size_t>(t) * k + j];
      if (r < 0 || r >= R) continue;   // dropped (or out-of-range) slot: contributes zero
      const float wj = w[static_cast<size_t>(t) * k + j];
      const floatx4* src = reinterpret_cast<const floatx4*>(y_perm + static_cast<size_t>(r) * d + c);
      const floatx4 v0 = src[0], v1 = src[1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc0[q] = fmaf(wj, v0[q], acc0[q]);
        acc1[q] = fmaf(wj, v1[q], acc1[q]);
      }
    }
    if (BF16) {
      u32x4 o;
      o[0] = pack_bf16x2(acc0[0], acc0[1]);
      o[1] = pack_bf16x2(acc0[2], acc0[3]);
      o[2] = pack_bf16x2(acc1[0], acc1[1]);
      o[3] = pack_bf16x2(acc1[2], acc1[3]);
      *reinterpret_cast<u32x4*>(static_cast<u16*>(y) + static_cast<size_t>(t) * d + c) = o;
    } else {
      floatx4* dst = reinterpret_cast<floatx4*>(static_cast<float*>(y) + static_cast<size_t>(t) * d + c);
      dst[0] = acc0;
      dst[1] = acc1;
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const float* y_shared, const int32_t* dest,
                          const float* w, int T, int d, int k, int R, int bf16, void* y, hipStream_t stream) {
  const long long items = static_cast<long long>(T) * (d / 8);
  long long blocks = (items + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, y_perm,
                       y_shared, dest, w, T, d, k, R, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, y_perm,
                       y_shared, dest, w, T, d, k, R, y);
  return hipGetLastError();
}

}  // namespace moe
