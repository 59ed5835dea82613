// Router: logits, scores, softmax, top-k, renormalised weights, per-block probability sums
// and per-block expert histograms, in one kernel.
//
// Method: the gate p_i = softmax(x W_g)_i, top-k selection on the logits rather than the
// probabilities, and the second normalisation of the k chosen probabilities (kwkr.cn page on
// sparse activation, section 2.1); Gumbel noise added before a temperature-scaled softmax
// ("Mixture of Experts (MoE) 原理与工程落地全指南", lpnh.cn, section 2.2); softmax and top-k fused
// in one kernel (kwkr.cn page, section 5.3).
//
// Layout: one wave per block of 64 tokens, 4 waves per workgroup. For bfloat16 the logits come
// from v_mfma_f32_16x16x32_bf16 (x rows as the A operand, W_g rows as the B operand, both
// K-contiguous, float32 accumulation); x is read exactly once from HBM. The 64 x E logit tile
// goes through LDS so that each lane then owns one token row for softmax and top-k.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

// Per-token epilogue. `row` is this lane's LDS row holding the float32 logits z[0..E) (bias
// already added). Writes logits/scores/top-k, leaves p[0..E) in `row` (zeros for tokens past T)
// and returns the bitmask of chosen experts.
__device__ __forceinline__ uint64_t token_epilogue(float* row, int t, bool valid, int E, int k, float tau,
                                                   int gumbel, uint32_t key0, uint32_t key1,
                                                   float* __restrict__ logits, float* __restrict__ scores,
                                                   int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  if (!valid) {
    for (int e = 0; e < E; ++e) row[e] = 0.0f;
    return 0ull;
  }
  const size_t zoff = static_cast<size_t>(t) * E;
  for (int e = 0; e < E; ++e) {
    const float z = row[e];
    logits[zoff + e] = z;
    float s = z;
    if (gumbel) s = s + gumbel_noise(static_cast<uint32_t>(t), static_cast<uint32_t>(e), key0, key1);
    if (tau != 1.0f) s = s / tau;
    row[e] = s;
    if (scores) scores[zoff + e] = s;
  }
  // top-k on the scores: strict '>' keeps the lowest index among equal values (and -0 == +0)
  uint64_t sel = 0ull;
  int idx[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    idx[j] = 0;
    if (j < k) {
      int best = -1;
      float bv = 0.0f;
      for (int e = 0; e < E; ++e) {
        if ((sel >> e) & 1ull) continue;
        const float v = row[e];
        if (best < 0 || v > bv) {
          best = e;
          bv = v;
        }
      }
      idx[j] = best;
      sel |= 1ull << best;
    }
  }
  // softmax of the scores (float32; the max is the first chosen score)
  const float m = row[idx[0]];
  float sum = 0.0f;
  for (int e = 0; e < E; ++e) {
    const float ex = expf(row[e] - m);
    row[e] = ex;
    sum += ex;
  }
  for (int e = 0; e < E; ++e) row[e] = row[e] / sum;
  float psel = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) psel += row[idx[j]];
  const size_t koff = static_cast<size_t>(t) * k;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      idx_out[koff + j] = idx[j];
      w_out[koff + j] = row[idx[j]] / psel;
    }
  }
  return sel;
}

// After the epilogue: column sums of p over the wave's 64 rows (fixed order) and the
// block histogram of chosen experts.
__device__ __forceinline__ void block_partials(const float* rows, int ldr, uint64_t sel, int blk, int E,
                                               float* __restrict__ probsum_part, int32_t* __restrict__ hist) {
  const int lane = lane_id();
  if (lane < E) {
    float s = 0.0f;
    for (int r = 0; r < kBlockTokens; ++r) s += rows[r * ldr + lane];
    probsum_part[static_cast<size_t>(blk) * E + lane] = s;
  }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    if (lane == e) hist[static_cast<size_t>(blk) * E + e] = __popcll(b);
  }
}

template <int NT>
__global__ __launch_bounds__(256) void router_bf16_kernel(RouterArgs a) {
  constexpr int EP = 16 * NT;
  constexpr int LDR = EP + 1;
  __shared__ float zs[4][kBlockTokens * LDR];
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int nblk = (a.T + kBlockTokens - 1) / kBlockTokens;
  const int blk = blockIdx.x * 4 + wave;
  const bool active = blk < nblk;
  const int tok0 = blk * kBlockTokens;
  const u16* __restrict__ x = static_cast<const u16*>(a.x);
  const u16* __restrict__ Wg = static_cast<const u16*>(a.Wg);
  const int d = a.d, E = a.E;
  float* rows = zs[wave];

  if (active) {
    const int r16 = lane & 15, g = lane >> 4;
    floatx4 acc[4][NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    const u16* ap[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      int t = tok0 + mt * 16 + r16;
      t = t < a.T ? t : a.T - 1;
      ap[mt] = x + static_cast<size_t>(t) * d + 16 * g;
    }
    const u16* bp[NT];
    bool bvalid[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = nt * 16 + r16;
      bvalid[nt] = e < E;
      bp[nt] = Wg + static_cast<size_t>(bvalid[nt] ? e : 0) * d + 16 * g;
    }
    // K chunks of 64: lane group g covers k in [kc + 16g, kc + 16g + 16) as two 8-element
    // pieces; MFMA step i uses piece i of both operands, so A and B agree on the k order.
    for (int kc = 0; kc < d; kc += 64) {
      bf16x8 av[4][2], bv[NT][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        av[mt][0] = *reinterpret_cast<const bf16x8*>(ap[mt] + kc);
        av[mt][1] = *reinterpret_cast<const bf16x8*>(ap[mt] + kc + 8);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (bvalid[nt]) {
          bv[nt][0] = *reinterpret_cast<const bf16x8*>(bp[nt] + kc);
          bv[nt][1] = *reinterpret_cast<const bf16x8*>(bp[nt] + kc + 8);
        } else {
          bv[nt][0] = bf16x8{};
          bv[nt][1] = bf16x8{};
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt][i], bv[nt][i], acc[mt][nt], 0, 0, 0);
    }
    // C layout of the 16x16 tile: lane holds column (lane & 15), rows 4*(lane>>4) + i.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + r16;
      const float bias = (a.bg != nullptr && col < E) ? a.bg[col] : 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) rows[(mt * 16 + 4 * g + i) * LDR + col] = acc[mt][nt][i] + bias;
    }
  }
  __syncthreads();
  uint64_t sel = 0ull;
  if (active) {
    const int t = tok0 + lane;
    sel = token_epilogue(rows + lane * LDR, t, t < a.T, E, a.k, a.tau, a.gumbel, a.key0, a.key1, a.logits,
                         a.scores, a.idx, a.w);
  }
  __syncthreads();
  if (active) block_partials(rows, LDR, sel, blk, E, a.probsum_part, a.hist);
}

// float32 storage: plain FMA dot products, one lane per token (small sizes only).
__global__ __launch_bounds__(256) void router_f32_kernel(RouterArgs a) {
  constexpr int LDR = kMaxE + 1;
  __shared__ float zs[4][kBlockTokens * LDR];
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int nblk = (a.T + kBlockTokens - 1) / kBlockTokens;
  const int blk = blockIdx.x * 4 + wave;
  const bool active = blk < nblk;
  const int t = blk * kBlockTokens + lane;
  const bool valid = active && t < a.T;
  const float* __restrict__ x = static_cast<const float*>(a.x);
  const float* __restrict__ Wg = static_cast<const float*>(a.Wg);
  float* rows = zs[wave];
  float* row = rows + lane * LDR;
  if (valid) {
    const float* xr = x + static_cast<size_t>(t) * a.d;
    for (int e = 0; e < a.E; ++e) {
      const float* wr = Wg + static_cast<size_t>(e) * a.d;
      float s = 0.0f;
      for (int c = 0; c < a.d; ++c) s = fmaf(xr[c], wr[c], s);
      row[e] = s + (a.bg != nullptr ? a.bg[e] : 0.0f);
    }
  }
  __syncthreads();
  uint64_t sel = 0ull;
  if (active)
    sel = token_epilogue(row, t, valid, a.E, a.k, a.tau, a.gumbel, a.key0, a.key1, a.logits, a.scores, a.idx, a.w);
  __syncthreads();
  if (active) block_partials(rows, LDR, sel, blk, a.E, a.probsum_part, a.hist);
}

__global__ __launch_bounds__(64) void histogram_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                       int32_t* __restrict__ hist) {
  const int lane = lane_id();
  const int blk = blockIdx.x;
  const int t = blk * kBlockTokens + lane;
  uint64_t sel = 0ull;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = idx[static_cast<size_t>(t) * k + j];
      if (e >= 0 && e < E) sel |= 1ull << e;
    }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    if (lane == e) hist[static_cast<size_t>(blk) * E + e] = __popcll(b);
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t stream) {
  const int nblk = (a.T + kBlockTokens - 1) / kBlockTokens;
  const dim3 grid((nblk + 3) / 4), block(256);
  if (!a.bf16) {
    hipLaunchKernelGGL(router_f32_kernel, grid, block, 0, stream, a);
  } else if (a.E <= 16) {
    hipLaunchKernelGGL(router_bf16_kernel<1>, grid, block, 0, stream, a);
  } else if (a.E <= 32) {
    hipLaunchKernelGGL(router_bf16_kernel<2>, grid, block, 0, stream, a);
  } else if (a.E <= 48) {
    hipLaunchKernelGGL(router_bf16_kernel<3>, grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL(router_bf16_kernel<4>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_histogram(const int32_t* idx, int T, int E, int k, int32_t* hist, hipStream_t stream) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(histogram_kernel, dim3(nblk), dim3(64), 0, stream, idx, T, E, k, hist);
  return hipGetLastError();
}

}  // namespace moe
