// Dispatch: expert counts, capacity truncation, the stable permutation and the row gather.
//
// Method (kwkr.cn page on sparse activation, sections 2.3 and 3.2): every token's k choices
// become k slots in token order; slots are grouped by expert in a stable order (ascending
// token index), counted per expert, and each expert keeps only the first C = ceil(c k T / E)
// of its slots; the rest are dropped and contribute nothing. The page's version sorts the
// slots; here the same order comes from a counting sort that needs no sort at all:
//   per-group histograms (16 tokens per group, written by the router or by the histogram
//   kernel) -> a one-workgroup scan giving, for every (group, expert), the number of earlier
//   slots of that expert -> a slot's rank among its expert's slots is that base plus the
//   number of lower lanes of its 16-lane group that chose the same expert (wave ballot).
// A token never picks an expert twice, so ranks are unique and the result is bit-exact.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kScanThreads = 1024;

__device__ __forceinline__ int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Fixed-order column sums of part [ng,E]: thread group g sums a contiguous run of rows in
// ascending order, then the group sums are added by a pairwise tree over g (a fixed order).
// Needs all kScanThreads threads of the workgroup; `lds` holds kScanThreads floats.
__device__ void blocked_colsum(const float* __restrict__ part, int ng, int E, float* __restrict__ out, float* lds) {
  const int E2 = pow2_at_least(E);
  const int G = kScanThreads / E2;
  const int chunk = (ng + G - 1) / G;
  const int e = threadIdx.x % E2, g = threadIdx.x / E2;
  float s = 0.0f;
  if (e < E) {
    const int b0 = g * chunk, b1 = min(ng, b0 + chunk);
    int b = b0;
    for (; b + 8 <= b1; b += 8) {            // eight independent loads in flight, added in order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[static_cast<size_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < b1; ++b) s += part[static_cast<size_t>(b) * E + e];
  }
  lds[threadIdx.x] = s;
  __syncthreads();
  for (int h = G >> 1; h > 0; h >>= 1) {     // G is a power of two
    if (g < h) lds[threadIdx.x] += lds[threadIdx.x + h * E2];
    __syncthreads();
  }
  if (g == 0 && e < E) out[e] = lds[e];
  __syncthreads();
}

__global__ __launch_bounds__(kScanThreads) void colsum_kernel(const float* __restrict__ part, int ng, int E,
                                                              float* __restrict__ out) {
  __shared__ float lds[kScanThreads];
  blocked_colsum(part, ng, E, out, lds);
}

// f_e = counts_e / (k T) and P_e = colsum_e / T, each rounded once from float64, one expert
// per lane of wave 0; L = E * sum_e f_e P_e accumulated in float64 in expert order by lane 0.
// `prod` is LDS scratch of kMaxE doubles. Called by all threads of the workgroup.
__device__ void write_stats(const int32_t* counts, const float* colsum, int E, int k, int T, float* f, float* P,
                            float* L, double* prod) {
  const int e = threadIdx.x;
  if (e < E) {
    const double kT = static_cast<double>(k) * static_cast<double>(T);
    const float fe = static_cast<float>(static_cast<double>(counts[e]) / kT);
    const float pe = static_cast<float>(static_cast<double>(colsum[e]) / static_cast<double>(T));
    f[e] = fe;
    P[e] = pe;
    prod[e] = static_cast<double>(fe) * static_cast<double>(pe);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int ee = 0; ee < E; ++ee) acc += prod[ee];
    L[0] = static_cast<float>(static_cast<double>(E) * acc);
  }
}

// Counts, capacity truncation, expert offsets and the per-(group, expert) base ranks, plus the
// balance statistics when the probability partials are given. One workgroup.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(ScanArgs a) {
  __shared__ int ilds[kScanThreads];
  __shared__ float flds[kScanThreads];
  __shared__ int tot[kMaxE];
  __shared__ float csum[kMaxE];
  __shared__ double prod[kMaxE];
  const int E = a.E, ng = a.ng;
  const int E2 = pow2_at_least(E);
  const int G = kScanThreads / E2;
  const int chunk = (ng + G - 1) / G;
  const int e = threadIdx.x % E2, g = threadIdx.x / E2;
  const int b0 = g * chunk, b1 = min(ng, b0 + chunk);
  int s = 0;
  if (e < E) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {            // eight independent loads in flight, added in order
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = a.hist[static_cast<size_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < b1; ++b) s += a.hist[static_cast<size_t>(b) * E + e];
  }
  ilds[threadIdx.x] = s;
  __syncthreads();
  for (int off = 1; off < G; off <<= 1) {    // inclusive scan over the thread groups
    const int v = g >= off ? ilds[threadIdx.x - off * E2] : 0;
    __syncthreads();
    ilds[threadIdx.x] += v;
    __syncthreads();
  }
  if (e < E) {
    const int pre = ilds[threadIdx.x] - s;
    if (g == G - 1) tot[e] = pre + s;
    int run = pre;
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = a.hist[static_cast<size_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a.blockbase[static_cast<size_t>(b + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; b < b1; ++b) {
      a.blockbase[static_cast<size_t>(b) * E + e] = run;
      run += a.hist[static_cast<size_t>(b) * E + e];
    }
  }
  __syncthreads();
  if (threadIdx.x < kWave) {                 // wave 0: one expert per lane, exclusive scan of kept
    const int ee = threadIdx.x;
    const int c = ee < E ? tot[ee] : 0;
    const int kp = c < a.C ? c : a.C;
    int incl = kp;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int n = __shfl_up(incl, off);
      if (ee >= off) incl += n;
    }
    if (ee < E) {
      a.counts[ee] = c;
      a.kept[ee] = kp;
      a.offsets[ee] = incl - kp;
    }
  }
  if (a.probsum_part != nullptr) {
    blocked_colsum(a.probsum_part, ng, E, csum, flds);   // contains __syncthreads
    if (threadIdx.x < E) a.colsum[threadIdx.x] = csum[threadIdx.x];
    write_stats(tot, csum, E, a.k, a.T, a.f, a.P, a.L, prod);
  }
}

__global__ __launch_bounds__(64) void stats_kernel(const int32_t* __restrict__ counts, const float* __restrict__ colsum,
                                                   int E, int k, int T, float* f, float* P, float* L) {
  __shared__ double prod[kMaxE];
  write_stats(counts, colsum, E, k, T, f, P, L, prod);
}

// One wave per 64 tokens: stable ranks by wave ballot within each 16-token group, capacity
// test, dest and perm.
__global__ __launch_bounds__(64) void permute_kernel(const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ blockbase,
                                                    const int32_t* __restrict__ offsets, int T, int E, int k,
                                                    int C, int32_t* __restrict__ dest,
                                                    int32_t* __restrict__ perm) {
  __shared__ uint64_t emask[kMaxE];
  const int lane = lane_id();
  const int blk = blockIdx.x;
  const int t = blk * kBlockTokens + lane;
  const bool valid = t < T;
  int ch[kMaxK];
  uint64_t sel = 0ull;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ch[j] = 0;
    if (valid && j < k) {
      ch[j] = idx[static_cast<size_t>(t) * k + j];
      if (ch[j] >= 0 && ch[j] < E) sel |= 1ull << ch[j];   // out-of-range choices are dropped
    }
  }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    if (lane == 0) emask[e] = b;
  }
  __syncthreads();
  if (!valid) return;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint64_t gmask = 0xFFFFull << (lane & ~(kGroupTokens - 1));   // this lane's 16-lane group
  const int grp = t / kGroupTokens;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      const int e = ch[j];
      if (e < 0 || e >= E) {
        dest[static_cast<size_t>(t) * k + j] = -1;
        continue;
      }
      const int r = blockbase[static_cast<size_t>(grp) * E + e] + __popcll(emask[e] & below & gmask);
      int dst = -1;
      if (r < C) {
        dst = offsets[e] + r;
        perm[dst] = t;
      }
      dest[static_cast<size_t>(t) * k + j] = dst;
    }
  }
}

// x_perm[r] = x[perm[r]] for r < sum(kept), 16-byte vectors; one row per workgroup iteration.
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ x, const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ kept,
                                                     const int32_t* __restrict__ offsets, int E, int R, int row_bytes,
                                                     uint8_t* __restrict__ x_perm) {
  const int total = offsets[E - 1] + kept[E - 1];
  const int nvec = row_bytes >> 4;
  for (int r = blockIdx.x; r < total && r < R; r += gridDim.x) {
    const int src = perm[r];
    const u32x4* s = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(src) * row_bytes);
    u32x4* d = reinterpret_cast<u32x4*>(x_perm + static_cast<size_t>(r) * row_bytes);
    for (int v = threadIdx.x; v < nvec; v += blockDim.x) d[v] = s[v];
  }
}

}  // namespace

hipError_t launch_colsum(const float* part, int ng, int E, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(colsum_kernel, dim3(1), dim3(kScanThreads), 0, stream, part, ng, E, out);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_stats(const int32_t* counts, const float* colsum, int E, int k, int T, float* f, float* P,
                        float* L, hipStream_t stream) {
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(64), 0, stream, counts, colsum, E, k, T, f, P, L);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, const int32_t* blockbase, const int32_t* offsets, int T, int E,
                          int k, int C, int32_t* dest, int32_t* perm, hipStream_t stream) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(permute_kernel, dim3(nblk), dim3(64), 0, stream, idx, blockbase, offsets, T, E, k, C, dest,
                     perm);
  return hipGetLastError();
}

hipError_t launch_gather(const void* x, const int32_t* perm, const int32_t* kept, const int32_t* offsets, int E,
                         int R, int row_bytes, void* x_perm, hipStream_t stream) {
  const int grid = R < 8192 ? R : 8192;
  hipLaunchKernelGGL(gather_kernel, dim3(grid > 0 ? grid : 1), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(x), perm, kept, offsets, E, R, row_bytes,
                     static_cast<uint8_t*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
