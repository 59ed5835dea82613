// Dispatch: expert counts, capacity truncation, the stable permutation and the row gather.
//
// Method (kwkr.cn page on sparse activation, sections 2.3 and 3.2): every token's k choices
// become k slots in token order; slots are grouped by expert in a stable order (ascending
// token index), counted per expert, and each expert keeps only the first C = ceil(c k T / E)
// of its slots; the rest are dropped and contribute nothing. The page's version sorts the
// slots; here the same order comes from a counting sort that needs no sort at all:
//   per-group histograms (kGroupTokens = 16 tokens per group, written by the router or by the
//   histogram kernel) -> a scan giving, for every (group, expert), the number of earlier
//   slots of that expert (one workgroup; for many groups two levels: one wave per chunk of
//   kScanChunk groups writes the bases within its chunk and the chunk's totals, then one
//   workgroup scans the chunk totals) ->
//   a slot's rank among its expert's slots is its group's base plus the number of lower lanes
//   of its 16-lane group that chose the same expert (wave ballot). Under token-order dropping,
//   a batch of at most one 64-token block per scan wave is ranked by the one-level scan
//   kernel's own waves after its last barrier (one launch fewer).
// A token never picks an expert twice, so ranks are unique and the result is bit-exact.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanChunk = 16;               // groups per chunk of the two-level scan

// The bases buffer of a scan, scan_bases_ints(ng, E) 4-byte entries, nc = ceil(ng / kScanChunk):
//   [0, ng E)            group bases: slots of the expert in earlier groups of the same chunk
//   [ng E, +nc E)        chunk bases: slots of the expert in earlier chunks
//   [+nc E)              slots per (chunk, expert); [+nc E) float probability sums per
//                        (chunk, expert); [+nc) float entropy sums per chunk
// The base of (group, expert) is its group base plus its chunk's base (group_base).
struct ScanRegion {
  int32_t* gbase;
  int32_t* cbase;
  int32_t* ctot;
  float* cps;
  float* cent;
  int nc;
};

__host__ __device__ inline ScanRegion scan_region(int32_t* bb, int ng, int E) {
  ScanRegion r;
  r.nc = (ng + kScanChunk - 1) / kScanChunk;
  const size_t ge = static_cast<size_t>(ng) * E, ce = static_cast<size_t>(r.nc) * E;
  r.gbase = bb;
  r.cbase = bb + ge;
  r.ctot = bb + ge + ce;
  r.cps = reinterpret_cast<float*>(bb + ge + 2 * ce);
  r.cent = reinterpret_cast<float*>(bb + ge + 3 * ce);
  return r;
}

__device__ __forceinline__ int group_base(const int32_t* __restrict__ bb, int ng, int E, int grp, int e) {
  return bb[static_cast<size_t>(grp) * E + e] +
         bb[static_cast<size_t>(ng) * E + static_cast<size_t>(grp / kScanChunk) * E + e];
}

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

// Load statistics of the batch from the expert counts (before capacity) and the sum of the
// tokens' routing entropies (lpnh.cn page, "Mixture of Experts（MoE）原理与工程落地全指南",
// sections 2.4 and 3.6; mhpn.cn
// page on MoE architecture, section 3.1), in float64, rounded once to float32:
//   out[0] = sum_e u_e^2 with u_e = counts_e / T
//   out[1] = 0.5 Q50(u) + 0.3 Q90(u) + 0.2 Q99(u), Qq by linear interpolation between the
//            order statistics at position (E - 1) q
//   out[2] = sum_e (counts_e - mean counts)^2
//   out[3] = population standard deviation of u
//   out[4] = ent_sum / T (mean routing entropy)
// Called by every thread of the workgroup; `srt` is LDS scratch of kMaxE doubles.
__device__ void write_route_stats(const int* tot, int E, int T, float ent_sum, float* out, double* srt) {
  const int e = threadIdx.x;
  if (e < E) {                               // rank sort of the counts (ties by index)
    const int c = tot[e];
    int rank = 0;
    for (int j = 0; j < E; ++j) {
      const int cj = tot[j];
      rank += (cj < c || (cj == c && j < e)) ? 1 : 0;
    }
    srt[rank] = static_cast<double>(c) / static_cast<double>(T);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double dT = static_cast<double>(T), dE = static_cast<double>(E);
    double sq = 0.0, csum = 0.0, usum = 0.0;
    for (int j = 0; j < E; ++j) {
      const double u = static_cast<double>(tot[j]) / dT;
      sq += u * u;
      csum += static_cast<double>(tot[j]);
      usum += u;
    }
    const double cmean = csum / dE, umean = usum / dE;
    double var = 0.0, uvar = 0.0;
    for (int j = 0; j < E; ++j) {
      const double dc = static_cast<double>(tot[j]) - cmean;
      const double du = static_cast<double>(tot[j]) / dT - umean;
      var += dc * dc;
      uvar += du * du;
    }
    auto quantile = [&](double q) {
      const double h = (dE - 1.0) * q;
      const int lo = static_cast<int>(floor(h));
      const int hi = lo + 1 < E ? lo + 1 : E - 1;
      return srt[lo] + (h - static_cast<double>(lo)) * (srt[hi] - srt[lo]);
    };
    out[0] = static_cast<float>(sq);
    out[1] = static_cast<float>(0.5 * quantile(0.5) + 0.3 * quantile(0.9) + 0.2 * quantile(0.99));
    out[2] = static_cast<float>(var);
    out[3] = static_cast<float>(sqrt(uvar / dE));
    out[4] = static_cast<float>(static_cast<double>(ent_sum) / dT);
  }
}

// First level of the scan: wave c takes the groups [c kScanChunk, +kScanChunk), lane e expert
// e. All of the lane's histogram entries (and probability partials, entropy partials) are
// loaded before any is used; the group bases within the chunk are the running sums in
// ascending group order, and the chunk's float sums add the groups in that order too. hist may
// be null (probability sums only), as may psum and ent.
__global__ __launch_bounds__(kWave) void scan_chunks_kernel(const int32_t* __restrict__ hist,
                                                            const float* __restrict__ psum,
                                                            const float* __restrict__ ent, int ng, int E,
                                                            int32_t* __restrict__ bb) {
  const ScanRegion r = scan_region(bb, ng, E);
  const int c = blockIdx.x, lane = threadIdx.x;
  const int g0 = c * kScanChunk, n = min(kScanChunk, ng - g0);
  if (lane < E) {
    // unconditional loads at clamped rows, issued back to back; rows past n are not used
    int h[kScanChunk];
    float p[kScanChunk];
    if (hist != nullptr) {
#pragma unroll
      for (int u = 0; u < kScanChunk; ++u) h[u] = hist[static_cast<size_t>(g0 + min(u, n - 1)) * E + lane];
    }
    if (psum != nullptr) {
#pragma unroll
      for (int u = 0; u < kScanChunk; ++u) p[u] = psum[static_cast<size_t>(g0 + min(u, n - 1)) * E + lane];
    }
    if (hist != nullptr) {
      int run = 0;
#pragma unroll
      for (int u = 0; u < kScanChunk; ++u)
        if (u < n) {
          r.gbase[static_cast<size_t>(g0 + u) * E + lane] = run;
          run += h[u];
        }
      r.ctot[static_cast<size_t>(c) * E + lane] = run;
    }
    if (psum != nullptr) {
      float s = 0.0f;
#pragma unroll
      for (int u = 0; u < kScanChunk; ++u)
        if (u < n) s += p[u];
      r.cps[static_cast<size_t>(c) * E + lane] = s;
    }
  }
  if (ent != nullptr && lane == 0) {
    float q[kScanChunk];
#pragma unroll
    for (int u = 0; u < kScanChunk; ++u) q[u] = ent[g0 + min(u, n - 1)];
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kScanChunk; ++u)
      if (u < n) s += q[u];
    r.cent[c] = s;
  }
}

// Counts, capacity truncation, expert offsets and the per-(group, expert) base ranks, plus the
// balance statistics when the probability partials are given. One workgroup: thread (g, e)
// takes expert e over the contiguous run of `chunk` groups of thread group g. With R > 0
// (chunk <= R <= kScanRegs, R a power of two, chosen by the launcher) all of a thread's R
// histogram entries and probability partials are loaded at once into registers: the kernel
// then makes one round trip to memory, where the general path (R = 0) makes one per batch of
// 8 and per pass (histogram, bases, probability partials). Both paths add every float in the
// same order (a thread's run in ascending groups, then a pairwise tree over the thread
// groups), so the statistics do not depend on the path.
constexpr int kScanRegs = 16;

// One wave's 64-token block of the stable permutation (defined below with the drop policies).
template <bool RANDOM>
__device__ void permute_block(const int32_t* __restrict__ idx, const int32_t* __restrict__ blockbase,
                              const int32_t* __restrict__ offsets, int T, int E, int k, int C,
                              const uint64_t* __restrict__ thresh, uint32_t key0, uint32_t key1,
                              int32_t* __restrict__ dest, int32_t* __restrict__ perm, int blk);

template <int R>
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
  const bool stats = a.probsum_part != nullptr && !a.bases_only;   // uniform
  constexpr bool in_regs = R > 0;
  constexpr int NR = R > 0 ? R : 1;
  int v[NR];
  int s = 0;
  float ps = 0.0f;
  if (in_regs && ng > 0) {
    // unconditional loads at clamped (in-bounds) positions, issued back to back; entries past
    // the thread's run or past E are zeroed afterwards
    float p[NR];
    const int ec = e < E ? e : E - 1;
#pragma unroll
    for (int u = 0; u < NR; ++u) v[u] = a.hist[static_cast<size_t>(min(b0 + u, ng - 1)) * E + ec];
    if (stats) {
#pragma unroll
      for (int u = 0; u < NR; ++u) p[u] = a.probsum_part[static_cast<size_t>(min(b0 + u, ng - 1)) * E + ec];
    }
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      v[u] = (e < E && b0 + u < b1) ? v[u] : 0;
      s += v[u];
    }
    if (stats) {
#pragma unroll
      for (int u = 0; u < NR; ++u)
        if (e < E && b0 + u < b1) ps += p[u];
    }
  } else if (!in_regs && e < E) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {            // eight independent loads in flight, added in order
      int w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = a.hist[static_cast<size_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += w[u];
    }
    for (; b < b1; ++b) s += a.hist[static_cast<size_t>(b) * E + e];
  }
  ilds[threadIdx.x] = s;
  if (in_regs && stats) flds[threadIdx.x] = ps;
  __syncthreads();
  for (int off = 1; off < G; off <<= 1) {    // inclusive scan over the thread groups
    const int x = g >= off ? ilds[threadIdx.x - off * E2] : 0;
    __syncthreads();
    ilds[threadIdx.x] += x;
    __syncthreads();
  }
  if (in_regs && stats) {                    // column sums: pairwise tree over the thread groups
    for (int h = G >> 1; h > 0; h >>= 1) {   // G is a power of two
      if (g < h) flds[threadIdx.x] += flds[threadIdx.x + h * E2];
      __syncthreads();
    }
    if (g == 0 && e < E) csum[e] = flds[e];
  }
  if (e < E) {
    const int pre = ilds[threadIdx.x] - s;
    if (g == G - 1) tot[e] = pre + s;
    int run = pre;
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < NR; ++u)
        if (b0 + u < b1) {
          a.blockbase[static_cast<size_t>(b0 + u) * E + e] = run;
          run += v[u];
        }
    } else {
      int b = b0;
      for (; b + 8 <= b1; b += 8) {
        int w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) w[u] = a.hist[static_cast<size_t>(b + u) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          a.blockbase[static_cast<size_t>(b + u) * E + e] = run;
          run += w[u];
        }
      }
      for (; b < b1; ++b) {
        a.blockbase[static_cast<size_t>(b) * E + e] = run;
        run += a.hist[static_cast<size_t>(b) * E + e];
      }
    }
  }
  for (int i = threadIdx.x; i < a.zero_n; i += kScanThreads) a.zero_bases[i] = 0;
  __syncthreads();
  if (a.bases_only) return;                  // uniform over the workgroup
  if (threadIdx.x < kWave) {                 // wave 0: one expert per lane, exclusive scan of kept
    const int ee = threadIdx.x;
    const int c = ee < E ? tot[ee] : 0;
    const int base = (a.base_kept != nullptr && ee < E) ? a.base_kept[ee] : 0;
    const int room = a.C - base;
    const int kp = base + (c < room ? c : room);
    int incl = kp;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int n = __shfl_up(incl, off);
      if (ee >= off) incl += n;
    }
    if (ee < E) {
      if (a.counts != nullptr) a.counts[ee] = c;
      a.kept[ee] = kp;
      a.offsets[ee] = incl - kp;
    }
  }
  if (stats) {
    if (!in_regs) blocked_colsum(a.probsum_part, ng, E, csum, flds);   // contains __syncthreads
    if (threadIdx.x < E) a.colsum[threadIdx.x] = csum[threadIdx.x];
    write_stats(tot, csum, E, a.k, a.T, a.f, a.P, a.L, prod);
  }
  if (a.route_stats != nullptr) {
    __syncthreads();                         // prod is reused below
    blocked_colsum(a.ent_part, ng, 1, csum, flds);
    write_route_stats(tot, E, a.T, csum[0], a.route_stats, prod);
  }
  if (a.perm_idx != nullptr) {               // uniform: the token-order permutation, fused
    // the bases and offsets this workgroup wrote are visible to all its waves past the barrier
    __syncthreads();
    const int nblk = (a.T + kBlockTokens - 1) / kBlockTokens;
    for (int blk = threadIdx.x / kWave; blk < nblk; blk += kScanThreads / kWave)
      permute_block<false>(a.perm_idx, a.blockbase, a.offsets, a.T, E, a.k, a.C, nullptr, 0u, 0u, a.perm_dest,
                           a.perm_out, blk);
  }
}

__global__ __launch_bounds__(64) void stats_kernel(const int32_t* __restrict__ counts, const float* __restrict__ colsum,
                                                   int E, int k, int T, float* f, float* P, float* L) {
  __shared__ double prod[kMaxE];
  write_stats(counts, colsum, E, k, T, f, P, L, prod);
}

// Key of slot (token t, expert e) under random capacity dropping: the slot's priority in the
// high word, the token in the low word, so keys are unique within an expert and order by
// (priority, token).
__device__ __forceinline__ uint64_t drop_key(int t, int e, uint32_t key0, uint32_t key1) {
  return (static_cast<uint64_t>(drop_priority(static_cast<uint32_t>(t), static_cast<uint32_t>(e), key0, key1)) << 32) |
         static_cast<uint32_t>(t);
}

// Whether slot (t, e) survives random dropping: thresh[e] is the largest kept key, all ones
// when the expert is within capacity (no priority needed then).
__device__ __forceinline__ bool kept_at_random(int t, int e, const uint64_t* __restrict__ thresh, uint32_t key0,
                                               uint32_t key1) {
  const uint64_t th = thresh[e];
  return th == ~0ull || drop_key(t, e, key0, key1) <= th;
}

// One wave per 64 tokens: stable ranks by wave ballot within each 16-token group, capacity
// test, dest and perm. RANDOM: only the slots kept by random dropping take part, ranked in
// token order among themselves (blockbase counts kept slots only). Every lane of the wave runs
// the ballots and shuffles; lane e keeps the block's mask of the lanes that chose expert e, and
// each lane fetches the masks of its own experts from those lanes.
template <bool RANDOM>
__device__ void permute_block(const int32_t* __restrict__ idx, const int32_t* __restrict__ blockbase,
                              const int32_t* __restrict__ offsets, int T, int E, int k, int C,
                              const uint64_t* __restrict__ thresh, uint32_t key0, uint32_t key1,
                              int32_t* __restrict__ dest, int32_t* __restrict__ perm, int blk) {
  const int lane = lane_id();
  const int t = blk * kBlockTokens + lane;
  const bool valid = t < T;
  int ch[kMaxK];
  uint64_t sel = 0ull;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ch[j] = -1;
    if (valid && j < k) {
      const int e = idx[static_cast<size_t>(t) * k + j];
      if (e >= 0 && e < E && (!RANDOM || kept_at_random(t, e, thresh, key0, key1))) {
        ch[j] = e;                                           // out-of-range or dropped: -1
        sel |= 1ull << e;
      }
    }
  }
  uint64_t mine = 0ull;
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    if (lane == e) mine = b;
  }
  uint64_t emask[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) emask[j] = __shfl(mine, ch[j] >= 0 ? ch[j] : 0);
  if (!valid) return;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint64_t gmask = 0xFFFFull << (lane & ~(kGroupTokens - 1));   // this lane's 16-lane group
  const int grp = t / kGroupTokens, ng = (T + kGroupTokens - 1) / kGroupTokens;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      const int e = ch[j];
      if (e < 0) {
        dest[static_cast<size_t>(t) * k + j] = -1;
        continue;
      }
      const int r = group_base(blockbase, ng, E, grp, e) + __popcll(emask[j] & below & gmask);
      int dst = -1;
      if (r < C) {
        dst = offsets[e] + r;
        perm[dst] = t;
      }
      dest[static_cast<size_t>(t) * k + j] = dst;
    }
  }
}

template <bool RANDOM>
__global__ __launch_bounds__(64) void permute_kernel(const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ blockbase,
                                                    const int32_t* __restrict__ offsets, int T, int E, int k,
                                                    int C, const uint64_t* __restrict__ thresh, uint32_t key0,
                                                    uint32_t key1, int32_t* __restrict__ dest,
                                                    int32_t* __restrict__ perm) {
  permute_block<RANDOM>(idx, blockbase, offsets, T, E, k, C, thresh, key0, key1, dest, perm, blockIdx.x);
}

// Random dropping, selection: one workgroup per expert finds the C-th smallest key among the
// expert's slots by radix selection over the 64-bit key, eight bits per pass, most significant
// first (a pass histograms the next digit of the slots that match the digits fixed so far, then
// fixes the digit whose bin holds the wanted rank). When the wanted bin holds a single slot, one
// more pass reads that slot's key. Experts within capacity keep everything: all ones.
__global__ __launch_bounds__(kScanThreads) void select_random_kernel(const int32_t* __restrict__ idx,
                                                                     const int32_t* __restrict__ counts, int T,
                                                                     int k, int C, uint32_t key0, uint32_t key1,
                                                                     uint64_t* __restrict__ thresh) {
  __shared__ int bins[256];
  __shared__ int pick_digit, pick_need, pick_count;
  __shared__ uint64_t found;
  const int e = blockIdx.x;
  if (counts[e] <= C) {
    if (threadIdx.x == 0) thresh[e] = ~0ull;
    return;
  }
  uint64_t prefix = 0ull;                    // the digits fixed so far, in place
  int need = C;                              // wanted rank (1-based) among the matching slots
  int shift = 64;
  bool unique = false;
  while (shift > 0) {
    shift -= 8;
    for (int i = threadIdx.x; i < 256; i += blockDim.x) bins[i] = 0;
    __syncthreads();
    const int hs = shift + 8;                // bits at and above hs are fixed (none when 64)
    for (int t = threadIdx.x; t < T; t += blockDim.x) {
      bool mine = false;
      for (int j = 0; j < k; ++j) mine |= idx[static_cast<size_t>(t) * k + j] == e;
      if (!mine) continue;
      const uint64_t key = drop_key(t, e, key0, key1);
      if (hs < 64 && (key >> hs) != (prefix >> hs)) continue;
      atomicAdd(&bins[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {               // wave 0: four bins per lane, prefix over lanes
      const int l = threadIdx.x;
      int b4[4], loc = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        b4[u] = bins[4 * l + u];
        loc += b4[u];
      }
      int incl = loc;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int n = __shfl_up(incl, off);
        if (l >= off) incl += n;
      }
      int run = incl - loc;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (run < need && run + b4[u] >= need) {
          pick_digit = 4 * l + u;
          pick_need = need - run;
          pick_count = b4[u];
        }
        run += b4[u];
      }
    }
    __syncthreads();
    prefix |= static_cast<uint64_t>(pick_digit) << shift;
    need = pick_need;
    const int cnt = pick_count;
    __syncthreads();                         // pick_* and bins are rewritten by the next pass
    if (cnt == 1 && shift > 0) {
      unique = true;
      break;
    }
  }
  if (unique) {                              // the one slot that matches the fixed digits
    for (int t = threadIdx.x; t < T; t += blockDim.x) {
      bool mine = false;
      for (int j = 0; j < k; ++j) mine |= idx[static_cast<size_t>(t) * k + j] == e;
      if (!mine) continue;
      const uint64_t key = drop_key(t, e, key0, key1);
      if ((key >> shift) == (prefix >> shift)) found = key;
    }
    __syncthreads();
    if (threadIdx.x == 0) thresh[e] = found;
  } else if (threadIdx.x == 0) {
    thresh[e] = prefix;
  }
}

// Random dropping: per-group histogram of the surviving slots. One wave per 64 tokens.
__global__ __launch_bounds__(64) void kept_histogram_kernel(const int32_t* __restrict__ idx,
                                                            const uint64_t* __restrict__ thresh, int T, int E, int k,
                                                            uint32_t key0, uint32_t key1,
                                                            int32_t* __restrict__ hist) {
  constexpr int NG = kBlockTokens / kGroupTokens;
  const int lane = lane_id();
  const int t = blockIdx.x * kBlockTokens + lane;
  const int ng = (T + kGroupTokens - 1) / kGroupTokens;
  const int grp0 = blockIdx.x * NG;
  uint64_t sel = 0ull;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = idx[static_cast<size_t>(t) * k + j];
      if (e >= 0 && e < E && kept_at_random(t, e, thresh, key0, key1)) sel |= 1ull << e;
    }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    if (lane < NG && grp0 + lane < ng)
      hist[static_cast<size_t>(grp0 + lane) * E + e] = __popcll((b >> (kGroupTokens * lane)) & 0xFFFFull);
  }
}

// Rerouting, first half. One wave per 64 tokens. Pass-1 rank of each slot as in the token-order
// dispatch; a token's slots past capacity take, in j order, its next-ranked experts
// idx_next[t, 0], idx_next[t, 1], ...: cand[t, j] = that expert, or -1 (kept in pass 1, or no
// next expert). A token's candidates go to distinct experts, so per-group ballots rank them in
// slot order; hist2 is their per-group histogram.
__global__ __launch_bounds__(64) void reroute_rank_kernel(const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ idx_next,
                                                          const int32_t* __restrict__ blockbase1, int T, int E,
                                                          int k, int C, int32_t* __restrict__ cand,
                                                          int32_t* __restrict__ hist2) {
  constexpr int NG = kBlockTokens / kGroupTokens;
  __shared__ uint64_t emask[kMaxE];
  const int lane = lane_id();
  const int t = blockIdx.x * kBlockTokens + lane;
  const bool valid = t < T;
  const int ng = (T + kGroupTokens - 1) / kGroupTokens;
  const int grp0 = blockIdx.x * NG;
  int ch[kMaxK];
  uint64_t sel = 0ull;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ch[j] = -1;
    if (valid && j < k) {
      const int e = idx[static_cast<size_t>(t) * k + j];
      if (e >= 0 && e < E) {
        ch[j] = e;
        sel |= 1ull << e;
      }
    }
  }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    if (lane == 0) emask[e] = b;
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  const uint64_t gmask = 0xFFFFull << (lane & ~(kGroupTokens - 1));
  const int grp = t / kGroupTokens;
  uint64_t csel = 0ull;
  int m = 0;                                 // the token's dropped slots so far
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (valid && j < k) {
      const int e = ch[j];
      int c = -1;
      if (e >= 0) {
        const int r = group_base(blockbase1, ng, E, grp, e) + __popcll(emask[e] & below & gmask);
        if (r >= C) {
          const int e2 = idx_next[static_cast<size_t>(t) * k + m];
          ++m;
          if (e2 >= 0 && e2 < E) {
            c = e2;
            csel |= 1ull << e2;
          }
        }
      }
      cand[static_cast<size_t>(t) * k + j] = c;
    }
  }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((csel >> e) & 1ull));
    if (lane < NG && grp0 + lane < ng)
      hist2[static_cast<size_t>(grp0 + lane) * E + e] = __popcll((b >> (kGroupTokens * lane)) & 0xFFFFull);
  }
}

// Rerouting, second half. One wave per 64 tokens. Slots kept in pass 1 take row offsets[e] +
// rank1 (the first kept1[e] rows of the segment); candidates take offsets[e2] + kept1[e2] +
// rank2 while rank2 < C - kept1[e2], else are dropped. A token with a candidate gets its weights
// renormalised over the experts its slots end at, from the float32 scores s:
// w_j = exp(s_j - m) / sum_j' exp(s_j' - m), m the largest of those scores (equal to the ratio of
// the softmax probabilities, whose common denominator cancels).
__global__ __launch_bounds__(64) void permute_reroute_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cand, const int32_t* __restrict__ blockbase1,
    const int32_t* __restrict__ blockbase2, const int32_t* __restrict__ kept1, const int32_t* __restrict__ offsets,
    const float* __restrict__ s, int T, int E, int k, int C, int32_t* __restrict__ dest, int32_t* __restrict__ perm,
    float* __restrict__ w) {
  __shared__ uint64_t emask[kMaxE], emask2[kMaxE];
  const int lane = lane_id();
  const int t = blockIdx.x * kBlockTokens + lane;
  const bool valid = t < T;
  int ch[kMaxK], cd[kMaxK];
  uint64_t sel = 0ull, csel = 0ull;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ch[j] = -1;
    cd[j] = -1;
    if (valid && j < k) {
      const int e = idx[static_cast<size_t>(t) * k + j];
      if (e >= 0 && e < E) {
        ch[j] = e;
        sel |= 1ull << e;
      }
      const int c = cand[static_cast<size_t>(t) * k + j];
      if (c >= 0 && c < E) {
        cd[j] = c;
        csel |= 1ull << c;
      }
    }
  }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    const uint64_t b2 = __ballot(static_cast<int>((csel >> e) & 1ull));
    if (lane == 0) {
      emask[e] = b;
      emask2[e] = b2;
    }
  }
  __syncthreads();
  if (!valid) return;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint64_t gmask = 0xFFFFull << (lane & ~(kGroupTokens - 1));
  const int grp = t / kGroupTokens, ng = (T + kGroupTokens - 1) / kGroupTokens;
  bool moved = false;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      int dst = -1;
      if (cd[j] >= 0) {
        const int e2 = cd[j];
        moved = true;
        const int r2 = group_base(blockbase2, ng, E, grp, e2) + __popcll(emask2[e2] & below & gmask);
        const int k1 = kept1[e2];
        if (r2 < C - k1) dst = offsets[e2] + k1 + r2;
      } else if (ch[j] >= 0) {
        const int e = ch[j];
        const int r = group_base(blockbase1, ng, E, grp, e) + __popcll(emask[e] & below & gmask);
        if (r < C) dst = offsets[e] + r;
      }
      if (dst >= 0) perm[dst] = t;
      dest[static_cast<size_t>(t) * k + j] = dst;
    }
  }
  if (!moved) return;
  const float* srow = s + static_cast<size_t>(t) * E;
  float sv[kMaxK];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    sv[j] = 0.0f;
    if (j < k) {
      const int e = cd[j] >= 0 ? cd[j] : ch[j];
      sv[j] = e >= 0 ? srow[e] : -INFINITY;
      m = fmaxf(m, sv[j]);
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      sv[j] = expf(sv[j] - m);
      sum += sv[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) w[static_cast<size_t>(t) * k + j] = sv[j] / sum;
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

// Whether a scan over ng groups takes two levels: when one workgroup's threads would hold more
// than kScanRegs groups each (more than 1024 groups for 16 experts, 256 for 64). There the
// single workgroup makes one round trip to memory per batch of 8 groups and per pass, which
// costs more than a second launch (measured on MI355X: 4096 groups of 16 experts 22.6 ->
// 16.9 us, 1024 groups of 64 experts 20.7 -> 16.1 us; at 256 groups of 8 experts the second
// launch made it 10 -> 17 us). With one level the scan writes absolute group bases and zero
// chunk bases.
static int scan_run(int ng, int E) {         // groups per thread of the one-workgroup scan
  int e2 = 1;
  while (e2 < E) e2 <<= 1;
  const int G = kScanThreads / e2;
  return (ng + G - 1) / G;
}

static bool scan_two_level(int ng, int E) { return scan_run(ng, E) > kScanRegs; }

// scan_kernel with the smallest R that holds a thread's run (0: the general path).
static hipError_t launch_scan_kernel(const ScanArgs& a, hipStream_t stream) {
  const int run = scan_run(a.ng, a.E);
  const dim3 g(1), b(kScanThreads);
  if (run <= 1)
    hipLaunchKernelGGL(scan_kernel<1>, g, b, 0, stream, a);
  else if (run <= 2)
    hipLaunchKernelGGL(scan_kernel<2>, g, b, 0, stream, a);
  else if (run <= 4)
    hipLaunchKernelGGL(scan_kernel<4>, g, b, 0, stream, a);
  else if (run <= 8)
    hipLaunchKernelGGL(scan_kernel<8>, g, b, 0, stream, a);
  else if (run <= kScanRegs)
    hipLaunchKernelGGL(scan_kernel<kScanRegs>, g, b, 0, stream, a);
  else
    hipLaunchKernelGGL(scan_kernel<0>, g, b, 0, stream, a);
  return hipGetLastError();
}

size_t scan_bases_ints(int ng, int E) {
  const size_t nc = (static_cast<size_t>(ng) + kScanChunk - 1) / kScanChunk;
  return static_cast<size_t>(ng) * E + 3 * nc * E + nc;
}

// The same two-level order as the scan's probability sums: per chunk, then over the chunks.
hipError_t launch_colsum(const float* part, int ng, int E, int32_t* bases, float* out, hipStream_t stream) {
  if (!scan_two_level(ng, E)) {
    hipLaunchKernelGGL(colsum_kernel, dim3(1), dim3(kScanThreads), 0, stream, part, ng, E, out);
    return hipGetLastError();
  }
  const ScanRegion r = scan_region(bases, ng, E);
  hipLaunchKernelGGL(scan_chunks_kernel, dim3(r.nc), dim3(kWave), 0, stream, nullptr, part, nullptr, ng, E, bases);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(colsum_kernel, dim3(1), dim3(kScanThreads), 0, stream, r.cps, r.nc, E, out);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
  const ScanRegion r = scan_region(a.blockbase, a.ng, a.E);
  if (!scan_two_level(a.ng, a.E)) {
    ScanArgs b = a;
    b.zero_bases = r.cbase;
    b.zero_n = r.nc * a.E;
    return launch_scan_kernel(b, stream);
  }
  const bool stats = a.probsum_part != nullptr && !a.bases_only;
  hipLaunchKernelGGL(scan_chunks_kernel, dim3(r.nc), dim3(kWave), 0, stream, a.hist,
                     stats ? a.probsum_part : nullptr, a.route_stats != nullptr ? a.ent_part : nullptr, a.ng, a.E,
                     a.blockbase);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // second level: the same scan over the chunk totals, its bases the chunk bases
  ScanArgs b = a;
  b.zero_bases = nullptr;
  b.zero_n = 0;
  b.perm_idx = nullptr;
  b.hist = r.ctot;
  b.ng = r.nc;
  b.blockbase = r.cbase;
  b.probsum_part = stats ? r.cps : nullptr;
  b.ent_part = a.route_stats != nullptr ? r.cent : nullptr;
  return launch_scan_kernel(b, stream);
}

hipError_t launch_stats(const int32_t* counts, const float* colsum, int E, int k, int T, float* f, float* P,
                        float* L, hipStream_t stream) {
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(64), 0, stream, counts, colsum, E, k, T, f, P, L);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, const int32_t* blockbase, const int32_t* offsets, int T, int E,
                          int k, int C, int32_t* dest, int32_t* perm, hipStream_t stream) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(permute_kernel<false>, dim3(nblk), dim3(64), 0, stream, idx, blockbase, offsets, T, E, k, C,
                     nullptr, 0u, 0u, dest, perm);
  return hipGetLastError();
}

// The token-order permutation runs in the scan kernel itself when the scan takes one level and
// the tokens are at most one 64-token block per wave of it (kScanThreads / 64 blocks): one launch
// and one launch gap fewer on decode-sized batches.
static bool scan_fuses_permute(const ScanArgs& a) {
  return !a.bases_only && !scan_two_level(a.ng, a.E) &&
         (a.T + kBlockTokens - 1) / kBlockTokens <= kScanThreads / kWave;
}

hipError_t launch_scan_permute(const ScanArgs& a, const int32_t* idx, int32_t* dest, int32_t* perm,
                               hipStream_t stream) {
  if (scan_fuses_permute(a)) {
    ScanArgs b = a;
    b.perm_idx = idx;
    b.perm_dest = dest;
    b.perm_out = perm;
    return launch_scan(b, stream);
  }
  hipError_t err = launch_scan(a, stream);
  if (err != hipSuccess) return err;
  return launch_permute(idx, a.blockbase, a.offsets, a.T, a.E, a.k, a.C, dest, perm, stream);
}

hipError_t launch_select_random(const int32_t* idx, const int32_t* counts, int T, int E, int k, int C, uint32_t key0,
                                uint32_t key1, uint64_t* thresh, hipStream_t stream) {
  hipLaunchKernelGGL(select_random_kernel, dim3(E), dim3(kScanThreads), 0, stream, idx, counts, T, k, C, key0, key1,
                     thresh);
  return hipGetLastError();
}

hipError_t launch_histogram_kept(const int32_t* idx, const uint64_t* thresh, int T, int E, int k, uint32_t key0,
                                 uint32_t key1, int32_t* hist, hipStream_t stream) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(kept_histogram_kernel, dim3(nblk), dim3(64), 0, stream, idx, thresh, T, E, k, key0, key1, hist);
  return hipGetLastError();
}

hipError_t launch_permute_kept(const int32_t* idx, const uint64_t* thresh, const int32_t* blockbase,
                               const int32_t* offsets, int T, int E, int k, uint32_t key0, uint32_t key1,
                               int32_t* dest, int32_t* perm, hipStream_t stream) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(permute_kernel<true>, dim3(nblk), dim3(64), 0, stream, idx, blockbase, offsets, T, E, k, T,
                     thresh, key0, key1, dest, perm);
  return hipGetLastError();
}

hipError_t launch_reroute_rank(const int32_t* idx, const int32_t* idx_next, const int32_t* blockbase1, int T, int E,
                               int k, int C, int32_t* cand, int32_t* hist2, hipStream_t stream) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(reroute_rank_kernel, dim3(nblk), dim3(64), 0, stream, idx, idx_next, blockbase1, T, E, k, C,
                     cand, hist2);
  return hipGetLastError();
}

hipError_t launch_permute_reroute(const int32_t* idx, const int32_t* cand, const int32_t* blockbase1,
                                  const int32_t* blockbase2, const int32_t* kept1, const int32_t* offsets,
                                  const float* s, int T, int E, int k, int C, int32_t* dest, int32_t* perm, float* w,
                                  hipStream_t stream) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(permute_reroute_kernel, dim3(nblk), dim3(64), 0, stream, idx, cand, blockbase1, blockbase2,
                     kept1, offsets, s, T, E, k, C, dest, perm, w);
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
