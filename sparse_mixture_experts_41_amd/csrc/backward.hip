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
//   router  dW_g = dz^T x; db_g = sum_t dz_t                                   (dwg_*)
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

// 16-byte vectors of a storage element type: 8 bf16 or 4 floats.
template <typename T>
struct Vec {
  static constexpr int N = 16 / static_cast<int>(sizeof(T));
  static constexpr int PAD = 4 / static_cast<int>(sizeof(T));   // one dword: odd row strides in dwords
};

// 16 bytes into LDS at a 4-byte aligned address (the padded tiles are not 16-byte aligned).
__device__ __forceinline__ void lds_store16(void* p, const u32x4& q) {
  uint32_t* d = static_cast<uint32_t*>(p);
#pragma unroll
  for (int u = 0; u < 4; ++u) d[u] = q[u];
}

__device__ __forceinline__ float to_f32(u16 v) { return bf16_to_f32(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ void from_f32(float v, u16& o) { o = f32_to_bf16(v); }
__device__ __forceinline__ void from_f32(float v, float& o) { o = v; }

// dst[b][c][r] = src[b][r][c] for [B][Rn][Cn] matrices (Rn, Cn multiples of the vector width):
// 64 x 64 tiles through LDS; 16-byte global loads and stores (a store packs one column's
// vector of rows from LDS). The tile rows are 64 elements plus one dword, an odd number of
// dwords, so the column gathers of a wave fall in distinct banks.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int Rn,
                                                        int Cn) {
  constexpr int V = Vec<T>::N, CH = 64 / V, P = 64 + Vec<T>::PAD;
  __shared__ __attribute__((aligned(16))) T tile[64 * P];
  const int b = blockIdx.z;
  // diagonal order: the workgroups running together read different source column blocks and
  // write different destination row blocks, instead of striding one of them by a power of two
  const int gx = gridDim.x, gy = gridDim.y;
  const int lin = blockIdx.y * gx + blockIdx.x;
  const int by = lin % gy, bx = (lin / gy + by) % gx;
  const int r0 = by * 64, c0 = bx * 64;
  const T* s = src + static_cast<size_t>(b) * Rn * Cn;
  T* o = dst + static_cast<size_t>(b) * Rn * Cn;
  for (int ch = threadIdx.x; ch < 64 * CH; ch += 256) {
    const int r = ch / CH, cc = ch % CH;
    if (r0 + r < Rn && c0 + V * cc < Cn)
      lds_store16(&tile[r * P + V * cc],
                  *reinterpret_cast<const u32x4*>(s + static_cast<size_t>(r0 + r) * Cn + c0 + V * cc));
  }
  __syncthreads();
  for (int ch = threadIdx.x; ch < 64 * CH; ch += 256) {
    const int c = ch / CH, rc = ch % CH;
    if (c0 + c < Cn && r0 + V * rc < Rn) {
      T v[V];
#pragma unroll
      for (int u = 0; u < V; ++u) v[u] = tile[(V * rc + u) * P + c];
      *reinterpret_cast<u32x4*>(o + static_cast<size_t>(c0 + c) * Rn + r0 + V * rc) =
          *reinterpret_cast<const u32x4*>(v);
    }
  }
}

// Expert-sorted rows -> zero-padded columns: for expert e and i < K_e (kept[e] rounded up to
// kWgradK), dst[n][koff[e] + i] = scale[r] * src[row(r)][n] with r = offsets[e] + i while
// i < kept[e] (row(r) = rows[r] when gathering, else r; no scale when null), 0 past it.
// With src_tiled the source row i of expert e is row i mod 256 of K-step-tiled panel
// (row tiles of the experts before e) + i / 256. With dst_tiled, dst[n][p] sits at row n mod 256
// of block p / 32 of panel n / 256 (ld / 32 blocks of 256 x 32 per panel).
// Tiles of 32 padded positions x 16 vectors of columns (128 bf16 or 64 floats); tile j
// belongs to the expert whose padded range holds position 32 j; tiles past the last expert
// exit. 16-byte loads of source rows; 16-byte stores of destination rows gathered from LDS.
template <typename T>
__global__ __launch_bounds__(256) void rows_to_cols_kernel(RowsToColsArgs a) {
  constexpr int V = Vec<T>::N, TC = 16 * V, P = TC + Vec<T>::PAD, PC = 32 / V;
  __shared__ __attribute__((aligned(16))) T tile[32 * P];
  __shared__ int s_e, s_mbase;
  const int pos0 = blockIdx.y * 32, c0 = blockIdx.x * TC;
  if (threadIdx.x < 64) {   // wave 0, lane l = expert l (E <= 64): the expert whose K range holds pos0
    const int l = threadIdx.x;
    const int kept = l < a.E ? a.kept[l] : 0;
    const int kp = (kept + kWgradK - 1) / kWgradK * kWgradK;
    const int ko = l < a.E ? a.koff[l] : 0;
    const int own = (kept + 255) / 256;      // row tiles of expert l
    int mb = own;                            // ... of experts 0..l
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(mb, o, 64);
      if (l >= o) mb += t;
    }
    // the K ranges are disjoint: at most one lane matches
    const unsigned long long hit = __ballot(l < a.E && kp > 0 && pos0 >= ko && pos0 < ko + kp);
    const int found = hit ? static_cast<int>(__builtin_ctzll(hit)) : -1;
    const int base = __shfl(mb - own, found < 0 ? 0 : found, 64);
    if (l == 0) {
      s_e = found;
      s_mbase = found < 0 ? 0 : base;
    }
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int i0 = pos0 - a.koff[e];
  const int n_rows = a.kept[e];
  const T* __restrict__ src = static_cast<const T*>(a.src);
  for (int ch = threadIdx.x; ch < 32 * 16; ch += 256) {
    const int ii = ch / 16, cc = ch % 16;
    u32x4 q = {0u, 0u, 0u, 0u};
    if (i0 + ii < n_rows && c0 + V * cc < a.ncol) {
      const int r = a.offsets[e] + i0 + ii;
      if (a.src_tiled) {
        const int i = i0 + ii, c = c0 + V * cc;
        const size_t blk = static_cast<size_t>(s_mbase + i / 256) * (a.ncol / 32) + c / 32;
        q = *reinterpret_cast<const u32x4*>(src + (blk * 256 + i % 256) * 32 + c % 32);
      } else {
        const int sr = a.rows != nullptr ? a.rows[r] : r;
        q = *reinterpret_cast<const u32x4*>(src + static_cast<size_t>(sr) * a.ncol + c0 + V * cc);
      }
      if (a.scale != nullptr) {
        const float sc = a.scale[r];
        T* v = reinterpret_cast<T*>(&q);
#pragma unroll
        for (int u = 0; u < V; ++u) from_f32(to_f32(v[u]) * sc, v[u]);
      }
    }
    lds_store16(&tile[ii * P + V * cc], q);
  }
  __syncthreads();
  T* __restrict__ dst = static_cast<T*>(a.dst);
  for (int ch = threadIdx.x; ch < TC * PC; ch += 256) {
    const int c = ch / PC, pc = ch % PC;
    if (c0 + c >= a.ncol) continue;
    T v[V];
#pragma unroll
    for (int u = 0; u < V; ++u) v[u] = tile[(V * pc + u) * P + c];
    const int n = c0 + c;
    const size_t o = a.dst_tiled ? (static_cast<size_t>(n / 256) * (a.ld / 32) + pos0 / 32) * (256 * 32) +
                                       static_cast<size_t>(n % 256) * 32 + V * pc
                                 : static_cast<size_t>(n) * a.ld + pos0 + V * pc;
    *reinterpret_cast<u32x4*>(dst + o) = *reinterpret_cast<const u32x4*>(v);
  }
}

// db[e][m] = sum of src[m][koff[e] .. koff[e] + K_e) (the padding is zero), 0 for an expert
// without rows. One wave per (m, e): lane-strided 16-byte vectors summed in a fixed order,
// then an xor butterfly.
template <typename T>
__global__ __launch_bounds__(256) void segment_rowsum_kernel(const T* __restrict__ src, const int32_t* __restrict__ kept,
                                                            const int32_t* __restrict__ koff, int M, int ld, int tiled,
                                                            float* __restrict__ db) {
  constexpr int V = Vec<T>::N;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int e = blockIdx.y;
  if (m >= M) return;
  const int lane = lane_id();
  const int kp = (kept[e] + kWgradK - 1) / kWgradK * kWgradK;   // a multiple of V
  const int k0 = kp > 0 ? koff[e] : 0;
  const T* row = src + static_cast<size_t>(m) * ld + k0;
  float acc = 0.0f;
  for (int i = lane * V; i < kp; i += kWave * V) {
    // tiled: position k0 + i of row m is element (m mod 256, (k0 + i) mod 32) of block
    // (k0 + i) / 32 of panel m / 256; a vector of V never crosses a block (k0, i multiples of V)
    const T* p = tiled ? src + (static_cast<size_t>(m / 256) * (ld / 32) + (k0 + i) / 32) * (256 * 32) +
                             static_cast<size_t>(m % 256) * 32 + (k0 + i) % 32
                       : row + i;
    const u32x4 q = *reinterpret_cast<const u32x4*>(p);
    const T* v = reinterpret_cast<const T*>(&q);
#pragma unroll
    for (int u = 0; u < V; ++u) acc += to_f32(v[u]);
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
// EB = E rounded up to 8, 16, 32 or 64; each thread owns EB experts x 64/EB consecutive
// columns (64 accumulators), so a token costs one vector load of x and 64 FMAs; the chunk's
// dz rows are staged in LDS 64 tokens at a time and read as 16-byte broadcasts. The blocks
// of column block 0 also write the chunk's dz column sums (bpart, for db_g).
template <bool BF16, int EB>
__global__ __launch_bounds__(256) void dwg_partial_kernel(const void* __restrict__ x, const float* __restrict__ dz,
                                                          int T, int d, int E, int chunk, float* __restrict__ part,
                                                          float* __restrict__ bpart) {
  constexpr int CPT = 64 / EB, TB = 64;
  __shared__ __attribute__((aligned(16))) float zs[TB][EB];
  const int n0 = (blockIdx.x * 256 + threadIdx.x) * CPT;
  const int s = blockIdx.y;
  const int t0 = s * chunk, t1 = min(T, t0 + chunk);
  if (bpart != nullptr && blockIdx.x == 0 && threadIdx.x < E) {
    float b = 0.0f;
    for (int t = t0; t < t1; ++t) b += dz[static_cast<size_t>(t) * E + threadIdx.x];
    bpart[static_cast<size_t>(s) * E + threadIdx.x] = b;
  }
  float acc[EB][CPT];
#pragma unroll
  for (int e = 0; e < EB; ++e)
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[e][c] = 0.0f;
  const bool live = n0 < d;
  for (int tb = t0; tb < t1; tb += TB) {
    __syncthreads();
    for (int i = threadIdx.x; i < TB * EB; i += 256) {
      const int tt = i / EB, e = i % EB;
      zs[tt][e] = (tb + tt < t1 && e < E) ? dz[static_cast<size_t>(tb + tt) * E + e] : 0.0f;
    }
    __syncthreads();
    const int nt = min(TB, t1 - tb);
    if (!live) continue;
#pragma unroll 8
    for (int tt = 0; tt < nt; ++tt) {
      float xv[CPT];
      const size_t o = static_cast<size_t>(tb + tt) * d + n0;
      if constexpr (BF16) {
        typedef u16 raw_t __attribute__((ext_vector_type(CPT)));
        const raw_t q = *reinterpret_cast<const raw_t*>(static_cast<const u16*>(x) + o);
#pragma unroll
        for (int c = 0; c < CPT; ++c) xv[c] = bf16_to_f32(q[c]);
      } else {
        typedef float raw_t __attribute__((ext_vector_type(CPT)));
        const raw_t q = *reinterpret_cast<const raw_t*>(static_cast<const float*>(x) + o);
#pragma unroll
        for (int c = 0; c < CPT; ++c) xv[c] = q[c];
      }
#pragma unroll
      for (int e4 = 0; e4 < EB; e4 += 4) {
        const floatx4 z = *reinterpret_cast<const floatx4*>(&zs[tt][e4]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < CPT; ++c) acc[e4 + u][c] = fmaf(z[u], xv[c], acc[e4 + u][c]);
      }
    }
  }
  if (!live) return;
#pragma unroll
  for (int e = 0; e < EB; ++e)
    if (e < E)
#pragma unroll
      for (int c = 0; c < CPT; ++c) part[(static_cast<size_t>(s) * E + e) * d + n0 + c] = acc[e][c];
}

// dWg[e][n] = sum over s of part[s][e][n]; dbg[e] likewise from bpart [S][E]. Workgroup = 64
// outputs x 4 waves: wave g sums slices g, g + 4, g + 8, ... in ascending order, then the four
// wave sums are added in wave order (a fixed order either way).
__global__ __launch_bounds__(256) void dwg_reduce_kernel(const float* __restrict__ part, int S, size_t En,
                                                         float* __restrict__ dWg, const float* __restrict__ bpart,
                                                         int E, float* __restrict__ dbg) {
  __shared__ float red[4][64];
  const int g = threadIdx.x >> 6, l = threadIdx.x & 63;
  const size_t i = static_cast<size_t>(blockIdx.x) * 64 + l;
  float acc = 0.0f, b = 0.0f;
  const bool bias = dbg != nullptr && blockIdx.x == 0 && l < E;
  for (int s = g; s < S; s += 4) {
    if (i < En) acc += part[static_cast<size_t>(s) * En + i];
    if (bias) b += bpart[static_cast<size_t>(s) * E + l];
  }
  red[g][l] = acc;
  __syncthreads();
  if (g == 0 && i < En) dWg[i] = ((red[0][l] + red[1][l]) + red[2][l]) + red[3][l];
  __syncthreads();
  if (blockIdx.x == 0) {
    red[g][l] = b;
    __syncthreads();
    if (g == 0 && bias) dbg[l] = ((red[0][l] + red[1][l]) + red[2][l]) + red[3][l];
  }
}

// dx[t][n] = sum_j dXp[dest_tj][n] (kept slots, j order) + sum_e dz[t][e] W_g[e][n]
// (experts in order). Workgroup = 16 tokens x 512 columns; each thread owns 2 adjacent
// columns of the 16 tokens (32 accumulators, few enough registers for four waves per SIMD):
// 8-byte loads of dXp rows, all 16 of a slot issued together (a dropped slot reads row 0 and
// adds nothing); W_g columns read 16 experts at a time and used for the 16 tokens; dz rows and
// dest from LDS.
template <bool BF16>
__global__ __launch_bounds__(256) void dx_kernel(DxArgs a) {
  constexpr int TT = kGroupTokens;
  __shared__ float zs[TT][kMaxE];
  __shared__ int ds[TT][kMaxK];
  const int t0 = blockIdx.x * TT;
  const int n0 = (blockIdx.y * 256 + threadIdx.x) * 2;
  const int E = a.E, k = a.k, d = a.d;
  const int nt = min(TT, a.T - t0);
  {
    float zv[TT * kMaxE / 256];
#pragma unroll
    for (int q = 0; q < TT * kMaxE / 256; ++q) {
      const int i = threadIdx.x + 256 * q, tt = i / kMaxE, e = i % kMaxE;
      zv[q] = (tt < nt && e < E) ? a.dz[static_cast<size_t>(t0 + tt) * E + e] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < TT * kMaxE / 256; ++q) {
      const int i = threadIdx.x + 256 * q;
      zs[i / kMaxE][i % kMaxE] = zv[q];
    }
  }
  if (threadIdx.x < TT * kMaxK) {
    const int tt = threadIdx.x / kMaxK, j = threadIdx.x % kMaxK;
    ds[tt][j] = (tt < nt && j < k) ? a.dest[static_cast<size_t>(t0 + tt) * k + j] : -1;
  }
  __syncthreads();
  if (n0 >= d) return;
  float2 acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[tt] = float2{0.0f, 0.0f};
  for (int j = 0; j < k; ++j) {
    float2 v[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int r = ds[tt][j];
      v[tt] = *reinterpret_cast<const float2*>(a.dXp + static_cast<size_t>(r < 0 ? 0 : r) * d + n0);
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      if (ds[tt][j] >= 0) {
        acc[tt].x += v[tt].x;
        acc[tt].y += v[tt].y;
      }
  }
  for (int e0 = 0; e0 < E; e0 += 16) {
    float2 wg[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      wg[e] = float2{0.0f, 0.0f};
      if (e0 + e < E) {
        const size_t o = static_cast<size_t>(e0 + e) * d + n0;
        if constexpr (BF16) {
          const uint32_t q = *reinterpret_cast<const uint32_t*>(static_cast<const u16*>(a.Wg) + o);
          wg[e] = float2{__uint_as_float(q << 16), __uint_as_float(q & 0xFFFF0000u)};
        } else {
          wg[e] = *reinterpret_cast<const float2*>(static_cast<const float*>(a.Wg) + o);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float z = zs[tt][e0 + e];
        acc[tt].x = fmaf(z, wg[e].x, acc[tt].x);
        acc[tt].y = fmaf(z, wg[e].y, acc[tt].y);
      }
  }
  // unrolled with a guard: a loop bounded by nt would index acc at run time and move it to
  // scratch memory
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    if (tt >= nt) continue;
    const size_t o = static_cast<size_t>(t0 + tt) * d + n0;
    if constexpr (BF16) {
      *reinterpret_cast<uint32_t*>(static_cast<u16*>(a.dx) + o) =
          static_cast<uint32_t>(f32_to_bf16(acc[tt].x)) | (static_cast<uint32_t>(f32_to_bf16(acc[tt].y)) << 16);
    } else {
      *reinterpret_cast<float2*>(static_cast<float*>(a.dx) + o) = acc[tt];
    }
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
  const int tc = bf16 ? 128 : 64;
  const dim3 grid((a.ncol + tc - 1) / tc, a.ld / 32);
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
                       koff, M, ld, wgrad_tiled(bf16) ? 1 : 0, db);
  else
    hipLaunchKernelGGL(segment_rowsum_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(src),
                       kept, koff, M, ld, wgrad_tiled(bf16) ? 1 : 0, db);
  return hipGetLastError();
}

hipError_t launch_zero_empty(float* out, const int32_t* kept, int E, size_t per_expert, hipStream_t stream) {
  size_t blocks = (per_expert + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_empty_kernel, dim3(static_cast<unsigned>(blocks), E), dim3(256), 0, stream, out, kept,
                     per_expert);
  return hipGetLastError();
}

static int dwg_block_cols(int E) {
  const int EB = E <= 8 ? 8 : (E <= 16 ? 16 : (E <= 32 ? 32 : 64));
  return 256 * (64 / EB);
}

int dwg_slices(int T, int d, int E) {
  const int cols = (d + dwg_block_cols(E) - 1) / dwg_block_cols(E);
  int s = (2048 + cols - 1) / cols;          // aim at >= 2048 workgroups (8 per CU)
  // each slice writes (and the reduction reads) an E x d float32 partial while reading
  // (T/S) x d of x: with many experts, keep that traffic near x's own (S <= T / (2E)), as long
  // as about 256 workgroups remain
  const int by_traffic = T / (2 * E), by_width = (256 + cols - 1) / cols;
  const int cap = by_traffic > by_width ? by_traffic : by_width;
  s = s < cap ? s : cap;
  const int max_s = (T + 15) / 16;           // at least 16 tokens per slice
  s = s < max_s ? s : max_s;
  return s < 1 ? 1 : (s > 512 ? 512 : s);
}

hipError_t launch_dwg(const void* x, const float* dz, int T, int d, int E, int bf16, float* part, float* dWg,
                      float* dbg, hipStream_t stream) {
  const int S = dwg_slices(T, d, E);
  const int chunk = (T + S - 1) / S;
  const size_t En = static_cast<size_t>(E) * d;
  float* bpart = dbg != nullptr ? part + static_cast<size_t>(S) * En : nullptr;
  const int EB = E <= 8 ? 8 : (E <= 16 ? 16 : (E <= 32 ? 32 : 64));
  const dim3 grid((d + dwg_block_cols(E) - 1) / dwg_block_cols(E), S);
#define MOE_DWG(B, EBV)                                                                                       \
  hipLaunchKernelGGL((dwg_partial_kernel<B, EBV>), grid, dim3(256), 0, stream, x, dz, T, d, E, chunk, part, \
                     bpart)
  if (bf16) {
    if (EB == 8) MOE_DWG(true, 8); else if (EB == 16) MOE_DWG(true, 16);
    else if (EB == 32) MOE_DWG(true, 32); else MOE_DWG(true, 64);
  } else {
    if (EB == 8) MOE_DWG(false, 8); else if (EB == 16) MOE_DWG(false, 16);
    else if (EB == 32) MOE_DWG(false, 32); else MOE_DWG(false, 64);
  }
#undef MOE_DWG
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dwg_reduce_kernel, dim3(static_cast<unsigned>((En + 63) / 64)), dim3(256), 0, stream, part, S,
                     En, dWg, bpart, E, dbg);
  return hipGetLastError();
}

hipError_t launch_dx(const DxArgs& a, int bf16, hipStream_t stream) {
  const dim3 grid((a.T + kGroupTokens - 1) / kGroupTokens, (a.d + 511) / 512);
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
