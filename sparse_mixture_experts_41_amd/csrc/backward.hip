// Backward pass of the MoE layer: the gradients of sum(dy * y) + lam * L.
//
// What carries gradient (kwkr.cn page on sparse activation, sections 2.2, 2.3 and 3.3): the
// routing decisions (top-k, capacity, the capacity policy) and f are discrete and fixed; the
// weights w and the balance term's P are continuous. A dropped slot has no expert-path
// gradient (its output was masked to zero), but its probability stays in the token's
// renormalisation denominator, so it still moves the router.
//
// Steps (per expert e, over its kept rows r, token t = perm[r], slot weight w_r):
//   router  dw_tj = <dy_t, o_r>; dp from w = p_e / S (S = the token's k final experts) and
//           lam * E f_e / T; ds = p (dp - <p, dp>); dz = ds / tau              (bwd_router)
//   GEMMs   dA = (w_r dy_t W2_e) * act'(a_r); dXp = dA W1_e                    (expert_gemm.hip)
//           dW2_e = sum_r (w_r dy_t)^T h_r;  dW1_e = sum_r dA_r^T x_t          (wgrad mode)
//   biases  db2_e = sum_r w_r dy_t; db1_e = sum_r dA_r                       (segment_rowsum)
//   router  dW_g = dz^T x; db_g = sum_t dz_t                                   (dwg_*, colsum)
//   input   dx_t = sum_j dXp[dest_tj] + dz_t W_g                               (dx_kernel)
// Every operand of the MFMA products is K-contiguous: the weights are transposed once per
// call, and the weight-gradient products read each expert's rows as columns of transposed,
// zero-padded copies (rows_to_cols). Every sum has a fixed order: no float atomics.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

template <bool BF16>
__device__ __forceinline__ void load8(const void* p, size_t i, float v[8]) {
  if constexpr (BF16) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const u16*>(p) + i);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[2 * u] = __uint_as_float(q[u] << 16);
      v[2 * u + 1] = __uint_as_float(q[u] & 0xFFFF0000u);
    }
  } else {
    const floatx4 a = *reinterpret_cast<const floatx4*>(static_cast<const float*>(p) + i);
    const floatx4 b = *reinterpret_cast<const floatx4*>(static_cast<const float*>(p) + i + 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = a[u];
      v[4 + u] = b[u];
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// One wave per token. dw_tj = <dy_t, o_r> over d in a fixed order (lane-strided 8-element
// chunks, then an xor butterfly); wrow[r] = w_tj; the router gradient dz_t, one expert per
// lane, from the float32 softmax of the token's scores.
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_router_kernel(BwdRouterArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = lane_id();
  const int k = a.k, E = a.E, d = a.d;
  int dst[kMaxK], fin[kMaxK];
  float part[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    dst[j] = -1;
    fin[j] = -1;
    part[j] = 0.0f;
    if (j < k) {
      const size_t sj = static_cast<size_t>(t) * k + j;
      dst[j] = a.dest[sj];
      const int c = a.cand != nullptr ? a.cand[sj] : -1;
      fin[j] = c >= 0 ? c : a.idx[sj];
    }
  }
  for (int c0 = lane * 8; c0 < d; c0 += kWave * 8) {
    float g[8];
    load8<BF16>(a.dy, static_cast<size_t>(t) * d + c0, g);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k && dst[j] >= 0) {
        float o[8];
        load8<false>(a.y_perm, static_cast<size_t>(dst[j]) * d + c0, o);
        if (a.y_perm2 != nullptr) {
          float o2[8];
          load8<false>(a.y_perm2, static_cast<size_t>(dst[j]) * d + c0, o2);
#pragma unroll
          for (int u = 0; u < 8; ++u) o[u] += o2[u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) part[j] = fmaf(g[u], o[u], part[j]);
      }
    }
  }
  float dw[kMaxK], w[kMaxK];
  float corr = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    dw[j] = 0.0f;
    w[j] = 0.0f;
    if (j < k) {
      dw[j] = wave_sum(part[j]);             // 0 for a dropped slot
      w[j] = a.w[static_cast<size_t>(t) * k + j];
      corr = fmaf(dw[j], w[j], corr);
      if (lane == 0 && dst[j] >= 0) a.wrow[dst[j]] = w[j];
    }
  }
  // softmax of the scores, one expert per lane
  const bool live = lane < E;
  const float s = live ? a.s[static_cast<size_t>(t) * E + lane] : -INFINITY;
  const float m = wave_max(s);
  const float ex = live ? expf(s - m) : 0.0f;
  const float p = ex / wave_sum(ex);
  float dpw = 0.0f;                          // the renormalisation part of dp at this expert
  bool mine = false;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k && fin[j] == lane) {
      dpw = dw[j] - corr;
      mine = true;
    }
  const float S = wave_sum(mine ? p : 0.0f);
  float dp = mine ? dpw / S : 0.0f;
  if (live) dp += a.lam_E_over_T * a.f[lane];
  const float pdp = wave_sum(live ? p * dp : 0.0f);
  if (live) a.dz[static_cast<size_t>(t) * E + lane] = p * (dp - pdp) / a.tau;
}

// dst[b][c][r] = src[b][r][c] for [B][Rn][Cn] matrices (Rn, Cn multiples of 8); 64 x 64 tiles
// through LDS, 4 elements per access (edge tiles guarded).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int Rn,
                                                        int Cn) {
  __shared__ T tile[64][64 + 4];
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const T* s = src + static_cast<size_t>(b) * Rn * Cn;
  T* o = dst + static_cast<size_t>(b) * Rn * Cn;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty + 16 * i;
    if (r0 + r < Rn && c0 + 4 * tx < Cn) {   // Cn % 4 == 0: four columns together
      const T* p = s + static_cast<size_t>(r0 + r) * Cn + c0 + 4 * tx;
#pragma unroll
      for (int u = 0; u < 4; ++u) tile[r][4 * tx + u] = p[u];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = ty + 16 * i;
    if (c0 + c < Cn && r0 + 4 * tx < Rn) {   // Rn % 4 == 0
      T* p = o + static_cast<size_t>(c0 + c) * Rn + r0 + 4 * tx;
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = tile[4 * tx + u][c];
    }
  }
}

// Expert-sorted rows -> zero-padded columns: for expert e and i < K_e (kept[e] rounded up to
// kWgradK), dst[n][koff[e] + i] = scale[r] * src[row(r)][n] with r = offsets[e] + i while
// i < kept[e] (row(r) = rows[r] when gathering, else r; no scale when null), 0 past it.
// Tiles of 32 padded positions x 64 columns; tile j belongs to the expert whose padded range
// holds position 32 j; tiles past the last expert exit.
template <typename T>
__global__ __launch_bounds__(256) void rows_to_cols_kernel(RowsToColsArgs a) {
  __shared__ float tile[32][64 + 1];
  __shared__ int s_e;
  const int pos0 = blockIdx.y * 32, c0 = blockIdx.x * 64;
  if (threadIdx.x == 0) {
    int found = -1;
    for (int e = 0; e < a.E; ++e) {
      const int kp = (a.kept[e] + kWgradK - 1) / kWgradK * kWgradK;
      if (kp > 0 && pos0 >= a.koff[e] && pos0 < a.koff[e] + kp) found = e;
    }
    s_e = found;
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int i0 = pos0 - a.koff[e];
  const int n_rows = a.kept[e];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const T* __restrict__ src = static_cast<const T*>(a.src);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int ii = ty + 4 * q;
    float v = 0.0f;
    if (i0 + ii < n_rows && c0 + tx < a.ncol) {
      const int r = a.offsets[e] + i0 + ii;
      const int sr = a.rows != nullptr ? a.rows[r] : r;
      if constexpr (sizeof(T) == 2)
        v = bf16_to_f32(src[static_cast<size_t>(sr) * a.ncol + c0 + tx]);
      else
        v = src[static_cast<size_t>(sr) * a.ncol + c0 + tx];
      if (a.scale != nullptr) v *= a.scale[r];
    }
    tile[ii][tx] = v;
  }
  __syncthreads();
  T* __restrict__ dst = static_cast<T*>(a.dst);
  // 64 destination rows of 32 positions each: 32 threads per row, 8 rows per pass
  const int lr = threadIdx.x >> 5, lp = threadIdx.x & 31;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int c = lr + 8 * q;
    if (c0 + c >= a.ncol) continue;
    const float v = tile[lp][c];
    T out;
    if constexpr (sizeof(T) == 2)
      out = f32_to_bf16(v);
    else
      out = v;
    dst[static_cast<size_t>(c0 + c) * a.ld + pos0 + lp] = out;
  }
}

// db[e][m] = sum of src[m][koff[e] .. koff[e] + K_e) (the padding is zero), 0 for an expert
// without rows. One wave per (m, e): lane-strided float sums in a fixed order, xor butterfly.
template <typename T>
__global__ __launch_bounds__(256) void segment_rowsum_kernel(const T* __restrict__ src, const int32_t* __restrict__ kept,
                                                            const int32_t* __restrict__ koff, int M, int ld,
                                                            float* __restrict__ db) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int e = blockIdx.y;
  if (m >= M) return;
  const int lane = lane_id();
  const int kp = (kept[e] + kWgradK - 1) / kWgradK * kWgradK;
  const T* row = src + static_cast<size_t>(m) * ld + (kp > 0 ? koff[e] : 0);
  float acc = 0.0f;
  for (int i = lane; i < kp; i += kWave) {
    if constexpr (sizeof(T) == 2)
      acc += bf16_to_f32(row[i]);
    else
      acc += row[i];
  }
  acc = wave_sum(acc);
  if (lane == 0) db[static_cast<size_t>(e) * M + m] = acc;
}

// out[e] = 0 ([M*N] floats) for every expert without kept rows (the weight-gradient products
// skip them).
__global__ __launch_bounds__(256) void zero_empty_kernel(float* __restrict__ out, const int32_t* __restrict__ kept,
                                                         size_t per_expert) {
  const int e = blockIdx.y;
  if (kept[e] != 0) return;
  float* o = out + static_cast<size_t>(e) * per_expert;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < per_expert;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    o[i] = 0.0f;
}

// dW_g partials: part[s][e][n] = sum over tokens t of chunk s (ascending) of dz[t][e] x[t][n].
// One thread per column n; dz rows are uniform over the workgroup.
template <bool BF16>
__global__ __launch_bounds__(256) void dwg_partial_kernel(const void* __restrict__ x, const float* __restrict__ dz,
                                                          int T, int d, int E, int chunk, float* __restrict__ part) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int s = blockIdx.y;
  const int t0 = s * chunk, t1 = min(T, t0 + chunk);
  float acc[kMaxE];
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) acc[e] = 0.0f;
  if (n < d) {
    for (int t = t0; t < t1; ++t) {
      const float xv = BF16 ? bf16_to_f32(static_cast<const u16*>(x)[static_cast<size_t>(t) * d + n])
                            : static_cast<const float*>(x)[static_cast<size_t>(t) * d + n];
      const float* zr = dz + static_cast<size_t>(t) * E;
#pragma unroll
      for (int e = 0; e < kMaxE; ++e)
        if (e < E) acc[e] = fmaf(zr[e], xv, acc[e]);
    }
#pragma unroll
    for (int e = 0; e < kMaxE; ++e)
      if (e < E) part[(static_cast<size_t>(s) * E + e) * d + n] = acc[e];
  }
}

// dWg[e][n] = sum over s (ascending) of part[s][e][n].
__global__ __launch_bounds__(256) void dwg_reduce_kernel(const float* __restrict__ part, int S, size_t En,
                                                         float* __restrict__ dWg) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= En) return;
  float acc = 0.0f;
  for (int s = 0; s < S; ++s) acc += part[static_cast<size_t>(s) * En + i];
  dWg[i] = acc;
}

// dx[t][n] = sum_j (dXp + dXp2)[dest_tj][n] (kept slots, j order) + sum_e dz[t][e] W_g[e][n].
// Workgroup = 16 tokens x 256 columns, one column per thread; the thread's W_g column is read
// once for the 16 tokens.
template <bool BF16>
__global__ __launch_bounds__(256) void dx_kernel(DxArgs a) {
  const int n = blockIdx.y * 256 + threadIdx.x;
  const int t0 = blockIdx.x * kGroupTokens;
  if (n >= a.d) return;
  const int E = a.E, k = a.k, d = a.d;
  float wg[kMaxE];
#pragma unroll
  for (int e = 0; e < kMaxE; ++e)
    wg[e] = e < E ? (BF16 ? bf16_to_f32(static_cast<const u16*>(a.Wg)[static_cast<size_t>(e) * d + n])
                          : static_cast<const float*>(a.Wg)[static_cast<size_t>(e) * d + n])
                  : 0.0f;
  for (int t = t0; t < min(a.T, t0 + kGroupTokens); ++t) {
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = a.dest[static_cast<size_t>(t) * k + j];
      if (r < 0) continue;
      float v = a.dXp[static_cast<size_t>(r) * d + n];
      if (a.dXp2 != nullptr) v += a.dXp2[static_cast<size_t>(r) * d + n];
      acc += v;
    }
    const float* zr = a.dz + static_cast<size_t>(t) * E;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e)
      if (e < E) acc = fmaf(zr[e], wg[e], acc);
    if (BF16)
      static_cast<u16*>(a.dx)[static_cast<size_t>(t) * d + n] = f32_to_bf16(acc);
    else
      static_cast<float*>(a.dx)[static_cast<size_t>(t) * d + n] = acc;
  }
}

// koff[e] = sum over e' < e of kept[e'] rounded up to kWgradK; koff[E] = the total.
__global__ void wgrad_offsets_kernel(const int32_t* __restrict__ kept, int E, int32_t* __restrict__ koff) {
  if (threadIdx.x != 0) return;
  int run = 0;
  for (int e = 0; e < E; ++e) {
    koff[e] = run;
    run += (kept[e] + kWgradK - 1) / kWgradK * kWgradK;
  }
  koff[E] = run;
}

}  // namespace

hipError_t launch_bwd_router(const BwdRouterArgs& a, int bf16, hipStream_t stream) {
  const dim3 grid((a.T + 3) / 4);
  if (bf16)
    hipLaunchKernelGGL(bwd_router_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_router_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int B, int Rn, int Cn, int bf16, hipStream_t stream) {
  const dim3 grid((Cn + 63) / 64, (Rn + 63) / 64, B);
  if (bf16)
    hipLaunchKernelGGL(transpose_kernel<u16>, grid, dim3(256), 0, stream, static_cast<const u16*>(src),
                       static_cast<u16*>(dst), Rn, Cn);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(src),
                       static_cast<float*>(dst), Rn, Cn);
  return hipGetLastError();
}

hipError_t launch_rows_to_cols(const RowsToColsArgs& a, int bf16, hipStream_t stream) {
  const dim3 grid((a.ncol + 63) / 64, a.ld / 32);
  if (bf16)
    hipLaunchKernelGGL(rows_to_cols_kernel<u16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(rows_to_cols_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_segment_rowsum(const void* src, const int32_t* kept, const int32_t* koff, int E, int M, int ld,
                                 int bf16, float* db, hipStream_t stream) {
  const dim3 grid((M + 3) / 4, E);
  if (bf16)
    hipLaunchKernelGGL(segment_rowsum_kernel<u16>, grid, dim3(256), 0, stream, static_cast<const u16*>(src), kept,
                       koff, M, ld, db);
  else
    hipLaunchKernelGGL(segment_rowsum_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(src),
                       kept, koff, M, ld, db);
  return hipGetLastError();
}

hipError_t launch_zero_empty(float* out, const int32_t* kept, int E, size_t per_expert, hipStream_t stream) {
  size_t blocks = (per_expert + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_empty_kernel, dim3(static_cast<unsigned>(blocks), E), dim3(256), 0, stream, out, kept,
                     per_expert);
  return hipGetLastError();
}

int dwg_slices(int T, int d) {
  const int cols = (d + 255) / 256;
  int s = (1024 + cols - 1) / cols;          // aim at >= 1024 workgroups
  const int max_s = (T + 15) / 16;           // at least 16 tokens per slice
  s = s < max_s ? s : max_s;
  return s < 1 ? 1 : (s > 64 ? 64 : s);
}

hipError_t launch_dwg(const void* x, const float* dz, int T, int d, int E, int bf16, float* part, float* dWg,
                      hipStream_t stream) {
  const int S = dwg_slices(T, d);
  const int chunk = (T + S - 1) / S;
  const dim3 grid((d + 255) / 256, S);
  if (bf16)
    hipLaunchKernelGGL(dwg_partial_kernel<true>, grid, dim3(256), 0, stream, x, dz, T, d, E, chunk, part);
  else
    hipLaunchKernelGGL(dwg_partial_kernel<false>, grid, dim3(256), 0, stream, x, dz, T, d, E, chunk, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t En = static_cast<size_t>(E) * d;
  hipLaunchKernelGGL(dwg_reduce_kernel, dim3(static_cast<unsigned>((En + 255) / 256)), dim3(256), 0, stream, part, S,
                     En, dWg);
  return hipGetLastError();
}

hipError_t launch_dx(const DxArgs& a, int bf16, hipStream_t stream) {
  const dim3 grid((a.T + kGroupTokens - 1) / kGroupTokens, (a.d + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(dx_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(dx_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_wgrad_offsets(const int32_t* kept, int E, int32_t* koff, hipStream_t stream) {
  hipLaunchKernelGGL(wgrad_offsets_kernel, dim3(1), dim3(64), 0, stream, kept, E, koff);
  return hipGetLastError();
}

}  // namespace moe
