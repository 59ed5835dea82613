// Router: logits, scores, softmax, top-k, renormalised weights, per-block probability sums
// and per-block expert histograms, in one kernel.
//
// Method: the gate p_i = softmax(x W_g)_i, top-k selection on the logits rather than the
// probabilities, and the second normalisation of the k chosen probabilities (kwkr.cn page on
// sparse activation, section 2.1); Gumbel noise added before a temperature-scaled softmax
// ("Mixture of Experts (MoE) 原理与工程落地全指南", lpnh.cn, section 2.2); softmax and top-k fused
// in one kernel (kwkr.cn page, section 5.3).
//
// Layout (bfloat16): kernel A computes the logits with MFMAs over (token block, K slice)
// workgroups, enough of them to fill the chip even for a few hundred tokens, reading x once;
// kernel B takes one wave per block of 64 tokens, sums the K-slice partials in a fixed order and
// runs softmax and top-k with one lane per token row (the row lives in LDS).
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

// Epilogue of one block of up to 64 tokens held by one wave. `rows` (LDS, row pitch ldr) holds
// the float32 logits z (bias added) of tokens t0 .. t0+nt-1. Writes the logits and scores
// (coalesced, from LDS), then per token (one lane each) the top-k indices and weights; leaves
// p in `rows` (zero rows past nt) and returns this lane's bitmask of chosen experts.
__device__ uint64_t block_epilogue(float* rows, int ldr, int t0, int nt, int E, int k, float tau, int gumbel,
                                   uint32_t key0, uint32_t key1, float* __restrict__ logits,
                                   float* __restrict__ scores, int32_t* __restrict__ idx_out,
                                   float* __restrict__ w_out) {
  const int lane = lane_id();
  const size_t base = static_cast<size_t>(t0) * E;
  for (int i = lane; i < nt * E; i += kWave) logits[base + i] = rows[(i / E) * ldr + i % E];
  float* row = rows + lane * ldr;
  const bool valid = lane < nt;
  if (valid && (gumbel || tau != 1.0f)) {
    const int t = t0 + lane;
    for (int e = 0; e < E; ++e) {
      float s = row[e];
      if (gumbel) s = s + gumbel_noise(static_cast<uint32_t>(t), static_cast<uint32_t>(e), key0, key1);
      if (tau != 1.0f) s = s / tau;
      row[e] = s;
    }
  }
  __syncthreads();
  if (scores)
    for (int i = lane; i < nt * E; i += kWave) scores[base + i] = rows[(i / E) * ldr + i % E];
  __syncthreads();
  if (!valid) {
    for (int e = 0; e < E; ++e) row[e] = 0.0f;
    return 0ull;
  }
  // top-k on the scores: strict '>' keeps the lowest index among equal values (and -0 == +0);
  // branch-free scans so the LDS reads of a row pipeline
  uint64_t sel = 0ull;
  int idx[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    idx[j] = 0;
    if (j < k) {
      int best = -1;
      float bv = 0.0f;
#pragma unroll 8
      for (int e = 0; e < E; ++e) {
        const float v = row[e];
        const bool take = !((sel >> e) & 1ull) && (best < 0 || v > bv);
        best = take ? e : best;
        bv = take ? v : bv;
      }
      idx[j] = best;
      sel |= 1ull << best;
    }
  }
  // softmax of the scores (float32; the max is the first chosen score)
  const float m = row[idx[0]];
  float sum = 0.0f;
#pragma unroll 8
  for (int e = 0; e < E; ++e) {
    const float ex = expf(row[e] - m);
    row[e] = ex;
    sum += ex;
  }
#pragma unroll 8
  for (int e = 0; e < E; ++e) row[e] = row[e] / sum;
  float psel = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) psel += row[idx[j]];
  const size_t koff = static_cast<size_t>(t0 + lane) * k;
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
#pragma unroll 16
    for (int r = 0; r < kBlockTokens; ++r) s += rows[r * ldr + lane];
    probsum_part[static_cast<size_t>(blk) * E + lane] = s;
  }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    if (lane == e) hist[static_cast<size_t>(blk) * E + e] = __popcll(b);
  }
}

// bf16 logits, kernel A: workgroup = TB = 16*MT tokens x one slice of K (blockIdx.y of KS).
// The slice is cut into 64-wide chunks dealt round-robin to the 4 waves; each wave accumulates
// MT x NT tiles of v_mfma_f32_16x16x32_bf16 (x rows as A, W_g rows as B, both K-contiguous),
// then the four wave partials are added in LDS in wave order and written to zpart[ks][t][e].
template <int MT, int NT>
__global__ __launch_bounds__(256) void router_logits_kernel(RouterArgs a, int KS, float* __restrict__ zpart) {
  constexpr int TB = 16 * MT, EP = 16 * NT, LDR = EP + 1;
  __shared__ float red[4][TB * LDR];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int tok0 = blockIdx.x * TB, ks = blockIdx.y;
  const int d = a.d, E = a.E, T = a.T;
  const int nchunk = d / 64;
  const int c0 = ks * nchunk / KS, c1 = (ks + 1) * nchunk / KS;
  const u16* __restrict__ x = static_cast<const u16*>(a.x);
  const u16* __restrict__ Wg = static_cast<const u16*>(a.Wg);
  const int r16 = lane & 15, g = lane >> 4;
  floatx4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  const u16* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int t = min(tok0 + mt * 16 + r16, T - 1);
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
  // chunk c covers k in [64c, 64c + 64): lane group g takes k 64c + 16g + [0, 16) as two
  // 8-element pieces, and MFMA step i uses piece i of both operands (same k order on A and B)
#pragma unroll 2
  for (int c = c0 + wave; c < c1; c += 4) {
    const int kc = c * 64;
    bf16x8 av[MT][2], bv[NT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      av[mt][0] = *reinterpret_cast<const bf16x8*>(ap[mt] + kc);
      av[mt][1] = *reinterpret_cast<const bf16x8*>(ap[mt] + kc + 8);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bv[nt][0] = bvalid[nt] ? *reinterpret_cast<const bf16x8*>(bp[nt] + kc) : bf16x8{};
      bv[nt][1] = bvalid[nt] ? *reinterpret_cast<const bf16x8*>(bp[nt] + kc + 8) : bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt][i], bv[nt][i], acc[mt][nt], 0, 0, 0);
  }
  // C layout of the 16x16 tile: lane holds column (lane & 15), rows 4*(lane>>4) + i.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][(mt * 16 + 4 * g + i) * LDR + nt * 16 + r16] = acc[mt][nt][i];
  __syncthreads();
  for (int o = threadIdx.x; o < TB * E; o += 256) {
    const int row = o / E, col = o - row * E;
    const int t = tok0 + row;
    if (t < T) {
      const int l = row * LDR + col;
      zpart[(static_cast<size_t>(ks) * T + t) * E + col] = ((red[0][l] + red[1][l]) + red[2][l]) + red[3][l];
    }
  }
}

// Kernel B: one workgroup per 64-token block. All 256 threads add up the block's KS slice
// partials (contiguous [64, E] tiles; slice order) plus b_g into LDS, many loads in flight;
// wave 0 then runs the epilogue with one lane per token.
__global__ __launch_bounds__(256) void router_epilogue_kernel(RouterArgs a, int KS, const float* __restrict__ zpart) {
  constexpr int LDR = kMaxE + 1;
  __shared__ float rows[kBlockTokens * LDR];
  const int blk = blockIdx.x;
  const int t0 = blk * kBlockTokens;
  const int nt = min(kBlockTokens, a.T - t0);
  const int E = a.E;
  const size_t base = static_cast<size_t>(t0) * E, slice = static_cast<size_t>(a.T) * E;
  const int n = nt * E;                      // <= 64 * 64: at most 16 elements per thread
  constexpr int PER = kBlockTokens * kMaxE / 256;
  float z[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + 256 * j;
    z[j] = i < n ? zpart[base + i] : 0.0f;
  }
  for (int ks = 1; ks < KS; ++ks) {           // one round of independent loads per slice
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = threadIdx.x + 256 * j;
      v[j] = i < n ? zpart[ks * slice + base + i] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) z[j] += v[j];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < n) {
      const int e = i % E;
      rows[(i / E) * LDR + e] = z[j] + (a.bg != nullptr ? a.bg[e] : 0.0f);
    }
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  const uint64_t sel = block_epilogue(rows, LDR, t0, nt, E, a.k, a.tau, a.gumbel, a.key0, a.key1, a.logits, a.scores,
                                      a.idx, a.w);
  __syncthreads();
  block_partials(rows, LDR, sel, blk, E, a.probsum_part, a.hist);
}

// float32 storage: plain FMA dot products, one lane per token (small sizes only).
__global__ __launch_bounds__(64) void router_f32_kernel(RouterArgs a) {
  constexpr int LDR = kMaxE + 1;
  __shared__ float rows[kBlockTokens * LDR];
  const int lane = lane_id();
  const int blk = blockIdx.x;
  const int t0 = blk * kBlockTokens;
  const int nt = min(kBlockTokens, a.T - t0);
  const float* __restrict__ x = static_cast<const float*>(a.x);
  const float* __restrict__ Wg = static_cast<const float*>(a.Wg);
  if (lane < nt) {
    const float* xr = x + static_cast<size_t>(t0 + lane) * a.d;
    for (int e = 0; e < a.E; ++e) {
      const float* wr = Wg + static_cast<size_t>(e) * a.d;
      float s = 0.0f;
      for (int c = 0; c < a.d; ++c) s = fmaf(xr[c], wr[c], s);
      rows[lane * LDR + e] = s + (a.bg != nullptr ? a.bg[e] : 0.0f);
    }
  }
  __syncthreads();
  const uint64_t sel = block_epilogue(rows, LDR, t0, nt, a.E, a.k, a.tau, a.gumbel, a.key0, a.key1, a.logits,
                                      a.scores, a.idx, a.w);
  __syncthreads();
  block_partials(rows, LDR, sel, blk, a.E, a.probsum_part, a.hist);
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

RouterPlan router_plan(int T, int d, int E) {
  (void)E;
  RouterPlan p;
  p.mt = 1;
  const int blocks = (T + 16 * p.mt - 1) / (16 * p.mt);
  const int nchunk = d / 64;
  int ks = (1024 + blocks - 1) / blocks;                 // aim at >= 1024 workgroups
  ks = ks < nchunk / 4 ? ks : nchunk / 4;                // >= 4 chunks (one per wave) per slice
  p.ks = ks < 1 ? 1 : (ks > 8 ? 8 : ks);
  return p;
}

template <int MT>
void launch_logits(const RouterArgs& a, int KS, float* zpart, hipStream_t stream) {
  const dim3 grid((a.T + 16 * MT - 1) / (16 * MT), KS), block(256);
  const int nt = (a.E + 15) / 16;
  if (nt == 1)
    hipLaunchKernelGGL((router_logits_kernel<MT, 1>), grid, block, 0, stream, a, KS, zpart);
  else if (nt == 2)
    hipLaunchKernelGGL((router_logits_kernel<MT, 2>), grid, block, 0, stream, a, KS, zpart);
  else if (nt == 3)
    hipLaunchKernelGGL((router_logits_kernel<MT, 3>), grid, block, 0, stream, a, KS, zpart);
  else
    hipLaunchKernelGGL((router_logits_kernel<MT, 4>), grid, block, 0, stream, a, KS, zpart);
}

hipError_t launch_router(const RouterArgs& a, float* zpart, hipStream_t stream) {
  const dim3 grid((a.T + kBlockTokens - 1) / kBlockTokens), block(kWave);
  if (!a.bf16) {
    hipLaunchKernelGGL(router_f32_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
  }
  const RouterPlan p = router_plan(a.T, a.d, a.E);
  launch_logits<1>(a, p.ks, zpart, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(router_epilogue_kernel, grid, dim3(256), 0, stream, a, p.ks, zpart);
  return hipGetLastError();
}

hipError_t launch_histogram(const int32_t* idx, int T, int E, int k, int32_t* hist, hipStream_t stream) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(histogram_kernel, dim3(nblk), dim3(64), 0, stream, idx, T, E, k, hist);
  return hipGetLastError();
}

}  // namespace moe
