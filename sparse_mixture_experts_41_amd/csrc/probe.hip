// Peak probes: what this chip sustains, measured next to the published peaks against which the
// layer's kernels are judged. Neither kernel is part of the layer.
//   probe_copy_kernel: a plain device copy in 16-byte vectors (HBM read + write bandwidth).
//   probe_mfma_kernel: independent v_mfma_f32_16x16x32_bf16 chains on register operands (the
//                      matrix-core rate the grouped GEMM's inner loop issues), no memory traffic.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

// Workgroup b copies the 16-byte vectors [b per, min((b + 1) per, n)), every lane keeping 4
// non-temporal loads in flight (contiguous chunks per workgroup measured 5.3-5.8 TB/s on
// MI355X against 4.0-5.0 TB/s for a grid-stride loop; non-temporal access adds about 5%).
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         size_t n, size_t per) {
  const size_t b = static_cast<size_t>(blockIdx.x) * per;
  const size_t e = b + per < n ? b + per : n;
  size_t i = b + threadIdx.x;
  for (; i + 3 * 256 < e; i += 4 * 256) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i), v1 = __builtin_nontemporal_load(src + i + 256);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 512), v3 = __builtin_nontemporal_load(src + i + 768);
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + 256);
    __builtin_nontemporal_store(v2, dst + i + 512);
    __builtin_nontemporal_store(v3, dst + i + 768);
  }
  for (; i < e; i += 256) dst[i] = src[i];
}

constexpr int kProbeChains = 16;

// Each wave runs kProbeChains independent accumulator chains of `iters` MFMAs each. The
// operands are fixed per lane, bf16 values spread over +-0.125 from a hash of the lane and
// workgroup (data-dependent power is part of what the probe measures). One float per thread
// goes to `out` so that no chain is dead code.
__global__ __launch_bounds__(256) void probe_mfma_kernel(float* __restrict__ out, int iters) {
  const uint32_t id = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t h = (id * 8u + static_cast<uint32_t>(i)) * 0x9E3779B9u;
    h ^= h >> 15;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    a[i] = static_cast<__bf16>((static_cast<float>(h & 0xffffu) / 65536.0f - 0.5f) * 0.25f);
    b[i] = static_cast<__bf16>((static_cast<float>(h >> 16) / 65536.0f - 0.5f) * 0.25f);
  }
  floatx4 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[id] = s;
}

}  // namespace

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 16;
  const size_t grid = n / 1024 < 16384 ? (n + 1023) / 1024 : 16384;       // at least one vector each
  const size_t per = ((n + grid - 1) / grid + 1023) / 1024 * 1024;          // whole 4 x 256-vector rounds
  hipLaunchKernelGGL(probe_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n, per);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(float* out, int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(workgroups), dim3(256), 0, stream, out, iters);
  return hipGetLastError();
}

int probe_mfma_chains() { return kProbeChains; }

}  // namespace moe
