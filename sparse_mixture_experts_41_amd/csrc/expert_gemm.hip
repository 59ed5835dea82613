// Expert FFN: grouped GEMMs over the expert-sorted rows.
//
// Method: every expert is Linear(d -> d_ffn) -> GELU -> Linear(d_ffn -> d) (kwkr.cn page on
// sparse activation, section 3.1; intelliparadigm.com page "MoE模型：动态计算架构解析与实践指南",
// section 2.1) and runs only on its own contiguous segment of the expert-sorted rows
// (kwkr.cn page, section 3.2). The page loops over experts on the host; here one launch covers
// every expert (its section 3.2 notes that dozens of experts need a fused kernel): each
// workgroup decodes its (expert, row tile, column tile) from the per-expert kept counts on the
// device, so the host never learns the counts and nothing synchronises.
//
// Both operands are K-contiguous (rows of x_perm / H, and nn.Linear [out, in] weight rows),
// which is the natural operand layout of the gfx950 bf16 MFMAs.
//   grouped_gemm_bf16: v_mfma_f32_32x32x16_bf16, LDS-staged tiles; the compute path.
//   grouped_gemv_bf16: at most 16 rows per expert (decode-sized batches): no LDS, the weight
//                      rows stream from HBM straight into v_mfma_f32_16x16x32_bf16 operands.
//   grouped_gemm_f32:  float32 storage, plain FMA (small sizes only).
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

struct GemmArgs {
  const void* A;          // [R,K] expert-sorted rows
  const void* B;          // [E,N,K] weights
  const void* bias;       // [E,N] or null (dtype)
  void* out;              // [R,N]
  const int32_t* kept;    // [E]
  const int32_t* offsets; // [E]
  int E, N, K;
  int R, C;               // rows of A/out and the capacity: segments outside them are skipped
};

enum { kEpiGelu = 0, kEpiLinear = 1 };

// Rows of expert e's segment; a segment that does not fit [0, R) or exceeds C counts as empty.
__device__ __forceinline__ int segment_rows(const GemmArgs& g, int e) {
  const int m = g.kept[e], o = g.offsets[e];
  return (m > 0 && m <= g.C && o >= 0 && o <= g.R - m) ? m : 0;
}

// Tile t -> (expert, row tile, column tile); column tiles outer, row tiles inner so that the
// workgroups sharing one weight panel are adjacent. Returns false past the last tile.
__device__ __forceinline__ bool decode_tile(int tile, const GemmArgs& g, int BM, int tiles_n, int& e, int& mt,
                                            int& nt) {
  for (int ee = 0; ee < g.E; ++ee) {
    const int tm = (segment_rows(g, ee) + BM - 1) / BM;
    const int cnt = tm * tiles_n;
    if (tile < cnt) {
      e = ee;
      nt = tile / tm;
      mt = tile - nt * tm;
      return true;
    }
    tile -= cnt;
  }
  return false;
}

__device__ __forceinline__ float load_bias(const void* bias, size_t i, bool bf16) {
  if (bias == nullptr) return 0.0f;
  return bf16 ? bf16_to_f32(static_cast<const u16*>(bias)[i]) : static_cast<const float*>(bias)[i];
}

// ---------------------------------------------------------------------------------------
// bf16 grouped GEMM: 128x128 tile, K step 64, 4 waves in a 2x2 grid of 64x64 wave tiles,
// each wave 2x2 MFMA 32x32x16 tiles. LDS rows padded by 16 bytes against bank conflicts;
// the next K step's global loads are in flight while the current one is multiplied.
constexpr int GBM = 128, GBN = 128, GBK = 64, GLDK = GBK + 8;

template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) u16 As[GBM * GLDK];
  __shared__ __attribute__((aligned(16))) u16 Bs[GBN * GLDK];
  const int tiles_n = (g.N + GBN - 1) / GBN;
  int e, mt, nt;
  if (!decode_tile(blockIdx.x, g, GBM, tiles_n, e, mt, nt)) return;
  const int m_e = segment_rows(g, e);
  const int row0 = g.offsets[e];
  const int m0 = mt * GBM, n0 = nt * GBN;
  const int N = g.N, K = g.K;
  const u16* __restrict__ A = static_cast<const u16*>(g.A);
  const u16* __restrict__ B = static_cast<const u16*>(g.B) + static_cast<size_t>(e) * N * K;
  const int tid = threadIdx.x;

  // global -> register staging: 4 x 16 B of A and of B per thread per K step
  const u16* ap[4];
  const u16* bp[4];
  bool av_ok[4], bv_ok[4];
  int soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, kc = (c & 7) * 8;
    av_ok[i] = (m0 + r) < m_e;
    bv_ok[i] = (n0 + r) < N;
    ap[i] = A + static_cast<size_t>(row0 + (av_ok[i] ? m0 + r : 0)) * K + kc;
    bp[i] = B + static_cast<size_t>(bv_ok[i] ? n0 + r : 0) * K + kc;
    soff[i] = r * GLDK + kc;
  }
  u32x4 ra[4], rb[4];
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = av_ok[i] ? *reinterpret_cast<const u32x4*>(ap[i]) : zero;
    rb[i] = bv_ok[i] ? *reinterpret_cast<const u32x4*>(bp[i]) : zero;
  }

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lk = 8 * (lane >> 5);
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  for (int k0 = 0; k0 < K; k0 += GBK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(As + soff[i]) = ra[i];
      *reinterpret_cast<u32x4*>(Bs + soff[i]) = rb[i];
    }
    __syncthreads();
    if (k0 + GBK < K) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = av_ok[i] ? *reinterpret_cast<const u32x4*>(ap[i] + k0 + GBK) : zero;
        rb[i] = bv_ok[i] ? *reinterpret_cast<const u32x4*>(bp[i] + k0 + GBK) : zero;
      }
    }
#pragma unroll
    for (int kk = 0; kk < GBK / 16; ++kk) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 32 + l32) * GLDK + kk * 16 + lk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + j * 32 + l32) * GLDK + kk * 16 + lk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // C layout of the 32x32 tile: lane holds column (lane & 31), rows 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = n0 + wn * 64 + j * 32 + l32;
    if (c >= N) continue;
    const float bias = load_bias(g.bias, static_cast<size_t>(e) * N + c, true);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r < m_e) {
          const size_t o = static_cast<size_t>(row0 + r) * N + c;
          const float val = acc[i][j][v] + bias;
          if (EPI == kEpiGelu)
            static_cast<u16*>(g.out)[o] = f32_to_bf16(gelu_erf(val));
          else
            static_cast<float*>(g.out)[o] = val;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// bf16 grouped GEMV-like kernel for experts with at most 16 rows. Workgroup = one expert x 64
// output columns; wave = 16 columns over the full K. Each lane group (16 lanes) reads 32
// contiguous bytes of a weight row per K step of 64, so a row is read in 128-byte runs.
template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemv_bf16_kernel(GemmArgs g) {
  const int nblk_n = g.N / 64;
  const int e = blockIdx.x / nblk_n, nb = blockIdx.x - e * nblk_n;
  const int m_e = segment_rows(g, e);
  if (m_e == 0) return;
  const int row0 = g.offsets[e];
  const int N = g.N, K = g.K;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int n = nb * 64 + wave * 16 + r16;
  const bool arow = r16 < m_e;
  const u16* __restrict__ ap = static_cast<const u16*>(g.A) + static_cast<size_t>(row0 + (arow ? r16 : 0)) * K + 16 * grp;
  const u16* __restrict__ bp = static_cast<const u16*>(g.B) + (static_cast<size_t>(e) * N + n) * K + 16 * grp;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int kc = 0; kc < K; kc += 64) {
    bf16x8 a0 = bf16x8{}, a1 = bf16x8{};
    if (arow) {
      a0 = *reinterpret_cast<const bf16x8*>(ap + kc);
      a1 = *reinterpret_cast<const bf16x8*>(ap + kc + 8);
    }
    const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(bp + kc);
    const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(bp + kc + 8);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc, 0, 0, 0);
  }
  const float bias = load_bias(g.bias, static_cast<size_t>(e) * N + n, true);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;
    if (r < m_e) {
      const size_t o = static_cast<size_t>(row0 + r) * N + n;
      const float val = acc[i] + bias;
      if (EPI == kEpiGelu)
        static_cast<u16*>(g.out)[o] = f32_to_bf16(gelu_erf(val));
      else
        static_cast<float*>(g.out)[o] = val;
    }
  }
}

// ---------------------------------------------------------------------------------------
// float32 grouped GEMM: 16x16 tiles through LDS, sequential K order, FMA.
constexpr int FBM = 16;

template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[16][17];
  __shared__ float Bs[16][17];
  const int tiles_n = (g.N + 15) / 16;
  int e, mt, nt;
  if (!decode_tile(blockIdx.x, g, FBM, tiles_n, e, mt, nt)) return;
  const int m_e = segment_rows(g, e);
  const int row0 = g.offsets[e];
  const int m0 = mt * 16, n0 = nt * 16;
  const int N = g.N, K = g.K;
  const float* __restrict__ A = static_cast<const float*>(g.A);
  const float* __restrict__ B = static_cast<const float*>(g.B) + static_cast<size_t>(e) * N * K;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    As[ty][tx] = (m0 + ty < m_e && k0 + tx < K) ? A[static_cast<size_t>(row0 + m0 + ty) * K + k0 + tx] : 0.0f;
    Bs[ty][tx] = (n0 + ty < N && k0 + tx < K) ? B[static_cast<size_t>(n0 + ty) * K + k0 + tx] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(As[ty][kk], Bs[tx][kk], acc);
    __syncthreads();
  }
  const int r = m0 + ty, c = n0 + tx;
  if (r < m_e && c < N) {
    const float val = acc + load_bias(g.bias, static_cast<size_t>(e) * N + c, false);
    static_cast<float*>(g.out)[static_cast<size_t>(row0 + r) * N + c] = (EPI == kEpiGelu) ? gelu_erf(val) : val;
  }
}

int tile_grid(int R, int E, int C, int BM, int N, int BN) {
  const long long by_rows = (R + BM - 1) / BM + E;
  const long long by_cap = static_cast<long long>(E) * ((C + BM - 1) / BM);
  const long long tm = by_rows < by_cap ? by_rows : by_cap;
  return static_cast<int>(tm * ((N + BN - 1) / BN));
}

}  // namespace

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream, hipEvent_t ev_mid) {
  GemmArgs g1{a.x_perm, a.W1, a.b1, a.H, a.kept, a.offsets, a.E, a.d_ffn, a.d, a.R, a.C};
  GemmArgs g2{a.H, a.W2, a.b2, a.y_perm, a.kept, a.offsets, a.E, a.d, a.d_ffn, a.R, a.C};
  hipError_t err;
  if (!a.bf16) {
    const int grid1 = tile_grid(a.R, a.E, a.C, FBM, a.d_ffn, 16);
    const int grid2 = tile_grid(a.R, a.E, a.C, FBM, a.d, 16);
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<kEpiGelu>, dim3(grid1), dim3(256), 0, stream, g1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev_mid && (err = hipEventRecord(ev_mid, stream)) != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<kEpiLinear>, dim3(grid2), dim3(256), 0, stream, g2);
    return hipGetLastError();
  }
  if (a.C <= 16) {
    hipLaunchKernelGGL(grouped_gemv_bf16_kernel<kEpiGelu>, dim3(a.E * (a.d_ffn / 64)), dim3(256), 0, stream, g1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev_mid && (err = hipEventRecord(ev_mid, stream)) != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemv_bf16_kernel<kEpiLinear>, dim3(a.E * (a.d / 64)), dim3(256), 0, stream, g2);
    return hipGetLastError();
  }
  const int grid1 = tile_grid(a.R, a.E, a.C, GBM, a.d_ffn, GBN);
  const int grid2 = tile_grid(a.R, a.E, a.C, GBM, a.d, GBN);
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<kEpiGelu>, dim3(grid1), dim3(256), 0, stream, g1);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev_mid && (err = hipEventRecord(ev_mid, stream)) != hipSuccess) return err;
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<kEpiLinear>, dim3(grid2), dim3(256), 0, stream, g2);
  return hipGetLastError();
}

}  // namespace moe
