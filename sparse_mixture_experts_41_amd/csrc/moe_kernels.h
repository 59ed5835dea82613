// Host-side launchers of the MoE kernels. Internal to the library; the public ABI is moe.h.
// Each launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Router noise added to the logits before the temperature: none, Gumbel, or Gaussian.
enum { kNoiseNone = 0, kNoiseGumbel = 1, kNoiseGaussian = 2 };

struct RouterArgs {
  const void* x;          // [T,d] dtype
  const void* Wg;         // [E,d] dtype
  const float* bg;        // [E] or null
  int T, d, E, k;
  int bf16;               // 1 = bfloat16 storage, 0 = float32
  float tau;
  int noise;              // kNoiseNone, kNoiseGumbel or kNoiseGaussian
  float noise_std;        // Gaussian noise only
  uint32_t key0, key1;
  float* logits;          // [T,E]
  float* scores;          // [T,E] or null
  int32_t* idx;           // [T,k]
  float* w;               // [T,k]
  float* probsum_part;    // [ng,E], ng = ceil(T/16) token groups
  int32_t* hist;          // [ng,E]
  int ng;
  float* ent_part;        // [ng] or null: per-group sums of the token entropies -sum_e p ln p
  int32_t* idx_next;      // [T,k] or null: the (k+1)-th ... (2k)-th ranked experts (-1 past E)
};
// K slices of the bf16 router (1 = one fused kernel); zpart needs slices * T * E floats when
// slices > 1 (unused otherwise and for float32).
int router_slices(int T, int d, int E);
hipError_t launch_router(const RouterArgs& a, float* zpart, hipStream_t stream);

// Per-group expert histogram of top-k indices ([ng,E], 16 tokens per group).
hipError_t launch_histogram(const int32_t* idx, int T, int E, int k, int32_t* hist, hipStream_t stream);

// Column sums of part [ng,E] in the order of the scan's probability sums; `bases` is a scan
// bases buffer of scan_bases_ints(ng, E) entries, used as scratch.
hipError_t launch_colsum(const float* part, int ng, int E, int32_t* bases, float* out, hipStream_t stream);
// 4-byte entries of a scan's bases buffer (group bases, then the chunk level of the scan).
size_t scan_bases_ints(int ng, int E);

struct ScanArgs {
  const int32_t* hist;    // [ng,E]
  int ng, E, k, T;
  int C;
  int32_t* counts;        // [E]
  int32_t* kept;          // [E]
  int32_t* offsets;       // [E]
  int32_t* blockbase;     // [scan_bases_ints(ng,E)] bases buffer: earlier slots of each expert before each group
  // optional statistics (all null or all set)
  const float* probsum_part;  // [ng,E]
  float* colsum;          // [E]
  float* f;               // [E]
  float* P;               // [E]
  float* L;               // [1]
  // second pass of a capacity policy: base_kept [E] slots already kept per expert, so the
  // capacity left is C - base_kept; kept = base_kept + min(new, C - base_kept); counts may be null
  const int32_t* base_kept;
  int bases_only;         // 1: write blockbase only (counts, kept, offsets, statistics untouched)
  // routing statistics (both null or both set): ent_part [ng] -> route_stats [MOE_ROUTE_STATS]
  const float* ent_part;
  float* route_stats;
  // set by launch_scan: zero_n entries at zero_bases are cleared (the chunk bases of a
  // one-level scan)
  int32_t* zero_bases;
  int zero_n;
  // set by launch_scan_permute when the token-order permutation runs in the scan kernel:
  // slots idx [T,k] -> dest [T,k], perm (as launch_permute with C and the bases above)
  const int32_t* perm_idx;
  int32_t* perm_dest;
  int32_t* perm_out;
};
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);
// launch_scan, then the token-order permutation (launch_permute with a.C), fused into the scan
// kernel where the batch is small enough.
hipError_t launch_scan_permute(const ScanArgs& a, const int32_t* idx, int32_t* dest, int32_t* perm,
                               hipStream_t stream);

// Random capacity dropping: thresh[e] = the largest kept key (priority << 32 | token) of expert
// e (all ones when within capacity); a slot is kept iff its key <= thresh[its expert].
hipError_t launch_select_random(const int32_t* idx, const int32_t* counts, int T, int E, int k, int C, uint32_t key0,
                                uint32_t key1, uint64_t* thresh, hipStream_t stream);
// Per-group histogram of the kept slots (keys <= thresh).
hipError_t launch_histogram_kept(const int32_t* idx, const uint64_t* thresh, int T, int E, int k, uint32_t key0,
                                 uint32_t key1, int32_t* hist, hipStream_t stream);
// permute for random dropping: only kept slots get rows, ranked by token order among them.
hipError_t launch_permute_kept(const int32_t* idx, const uint64_t* thresh, const int32_t* blockbase,
                               const int32_t* offsets, int T, int E, int k, uint32_t key0, uint32_t key1,
                               int32_t* dest, int32_t* perm, hipStream_t stream);
// Rerouting, first half: pass-1 ranks from blockbase1; the token's dropped slots take its next
// experts idx_next [T,k] in j order -> cand [T,k] (-1 = none) and their group histogram hist2.
hipError_t launch_reroute_rank(const int32_t* idx, const int32_t* idx_next, const int32_t* blockbase1, int T, int E,
                               int k, int C, int32_t* cand, int32_t* hist2, hipStream_t stream);
// Rerouting, second half: final dest and perm (pass-1 rows, then pass-2 rows of each expert),
// and the weights of tokens with a moved slot renormalised over their final experts from the
// scores s [T,E].
hipError_t launch_permute_reroute(const int32_t* idx, const int32_t* cand, const int32_t* blockbase1,
                                  const int32_t* blockbase2, const int32_t* kept1, const int32_t* offsets,
                                  const float* s, int T, int E, int k, int C, int32_t* dest, int32_t* perm, float* w,
                                  hipStream_t stream);

hipError_t launch_permute(const int32_t* idx, const int32_t* blockbase, const int32_t* offsets,
                          int T, int E, int k, int C, int32_t* dest, int32_t* perm, hipStream_t stream);

hipError_t launch_gather(const void* x, const int32_t* perm, const int32_t* kept, const int32_t* offsets,
                         int E, int R, int row_bytes, void* x_perm, hipStream_t stream);

// Expert activation: GeLU (the default) or SiLU.
enum { kActGelu = 0, kActSilu = 1 };

struct FfnArgs {
  const void* x_perm;     // [R,d] (unused when rows is set)
  const void* x;          // [T,d] token rows, read through `rows` (bf16 MFMA path only)
  const int32_t* rows;    // [R] or null: x row of expert-sorted row r (perm); see ffn_gathers
  int T;
  const int32_t* kept;    // [E]
  const int32_t* offsets; // [E]
  const void* W1;         // [E,d_ffn,d]
  const void* b1;         // [E,d_ffn] or null
  const void* W2;         // [E,d,d_ffn]
  const void* b2;         // [E,d] or null
  void* H;                // ffn_h_rows(R, E, C, bf16) x d_ffn: row-major, or tiled panels (ffn_h_tiled)
  float* y_perm;          // [R,d]
  float* side;            // tail_side_floats(R, E, C, d) floats when ffn_splits() > 1: GEMM2's split-tail parts
  int E, d, d_ffn, R, C;
  int bf16;
  int act;                // kActGelu or kActSilu
  void* pre;              // [R,d_ffn] or null: GEMM1 also stores its pre-activation (training)
  int w_packed;           // 1: W1 and W2 in the packed panels of launch_pack_weights (bf16, d and
                          // d_ffn multiples of 256)
};
// Whether GEMM1 can read the token rows of x through the permutation instead of a gathered
// copy: the bf16 GEMV path (C <= 16), and the bf16 MFMA path with x addressable by 32-bit
// buffer offsets.
bool ffn_gathers(const FfnArgs& a);
// Most K parts a tile of the last, partial round of GEMM2 is split into (1 = no tail split):
// kTailMaxParts on the bf16 MFMA path, 1 elsewhere. Part 0 writes y_perm, the other parts
// write `side`, and a fixup kernel adds them to y_perm in part order, so y_perm alone is the
// GEMM2 result.
int ffn_splits(const FfnArgs& a);
// Floats of the side buffer of a tail-split product (255 dense 256 x 256 tiles).
size_t tail_side_floats(int R, int E, int C, int N);
// Whether the hidden layer H between the two expert GEMMs is kept in K-step-tiled panels (the
// bf16 MFMA path): the rows of each (expert, 256-row tile) form one panel of d_ffn/32 contiguous
// 16 KB blocks of 256 rows x 32 columns, panels in the order of the experts' row tiles. Rows past
// an expert's segment inside its last panel are never written.
bool ffn_h_tiled(int bf16, int C);
// Rows to allocate for H (and the shared expert's H, with R = T, E = 1, C = T).
size_t ffn_h_rows(int R, int E, int C, int bf16);
// GEMM1 (+bias, GeLU) then GEMM2 (+bias). `ev_mid` (nullable) is recorded between them.
hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream, hipEvent_t ev_mid);
// W [E][rows][cols] row-major bf16 -> W_packed, the same bytes as K-step-tiled panels: panel
// e rows/256 + p is rows [256 p, 256 p + 256) of expert e as cols/32 contiguous blocks of 256
// rows x 32 columns (64-byte rows). rows a multiple of 256, cols of 32.
hipError_t launch_pack_weights(const void* W, void* W_packed, int64_t E, int64_t rows, int64_t cols,
                               hipStream_t stream);
// The shared expert: one dense FFN over the T token rows of x (no routing):
// H = act(x W1ᵀ + b1) [T, d_ffn], y = H W2ᵀ + b2 [T, d] float.
struct SharedFfnArgs {
  const void* x;          // [T,d]
  const void* W1;         // [d_ffn,d]
  const void* b1;         // [d_ffn] or null
  const void* W2;         // [d,d_ffn]
  const void* b2;         // [d] or null
  void* H;                // ffn_h_rows(T, 1, T, bf16) x d_ffn: row-major, or tiled panels (ffn_h_tiled)
  float* y;               // [T,d]
  int T, d, d_ffn;
  int bf16, act;
};
hipError_t launch_shared_ffn(const SharedFfnArgs& a, hipStream_t stream);

// y_shared
// (nullable, [T,d] float): the shared expert's output, where each token's sum starts.
hipError_t launch_combine(const float* y_perm, const float* y_shared, const int32_t* dest,
                          const float* w, int T, int d, int k, int R, int bf16, void* y, hipStream_t stream);

hipError_t launch_stats(const int32_t* counts, const float* colsum, int E, int k, int T, float* f, float* P,
                        float* L, hipStream_t stream);

// ---------------------------------------------------------------------------------------
// Backward pass.
constexpr int kWgradK = 32;   // rows of a weight-gradient product are padded to this granule

// Whether the backward products need the weights transposed (W2T, W1T): off the bf16 MFMA path.
// On it they read W2 and W1 as given, N-contiguous, through LDS transpose reads.
bool bwd_weights_transposed(int bf16, int C);

// dA[r] = (A_row(r) W2_e) * wrow[r] * act'(pre[r]) over each expert's segment rows, where
// A_row(r) = A[rows[r]] (rows set: the bf16 MFMA path reads dy through the permutation) or A[r]
// (an expert-sorted copy). W2 [E, d, d_ffn] as given; W2T [E, d_ffn, d] is W2 transposed, read
// (and needed) only when bwd_weights_transposed(). pre: [R, d_ffn] dtype. dA: like H, in the
// K-step-tiled panels of ffn_h_tiled() on the MFMA path (ffn_h_rows rows), else [R, d_ffn].
struct BwdDactArgs {
  const void* A;
  const int32_t* rows;
  int a_rows;
  const void* W2;
  const void* W2T;
  const float* wrow;
  const void* pre;
  void* dA;
  const int32_t* kept;
  const int32_t* offsets;
  int E, d, d_ffn, R, C, bf16, act;
};
hipError_t launch_bwd_dact(const BwdDactArgs& a, hipStream_t stream);

// dXp[r] = dA[r] W1_e (float, [R, d]); W1 [E, d_ffn, d] as given, W1T [E, d, d_ffn] its transpose
// (read only when bwd_weights_transposed()). With bwd_dx_splits() > 1 the last round's tiles are
// tail-split through `side` (tail_side_floats(R, E, C, d)).
struct BwdDxArgs {
  const void* dA;
  const void* W1;
  const void* W1T;
  float* dXp;
  float* side;
  const int32_t* kept;
  const int32_t* offsets;
  int E, d, d_ffn, R, C, bf16;
};
int bwd_dx_splits(int R, int E, int C, int d, int d_ffn, int bf16);
hipError_t launch_bwd_dx(const BwdDxArgs& a, hipStream_t stream);

// out[e] = A[:, koff[e] : +K_e] B[:, koff[e] : +K_e]^T (float [E, M, N]) with K_e = kept[e]
// rounded up to kWgradK; A [M, ld] and B [N, ld] dtype hold each expert's rows as columns, zero
// past kept[e]. Experts with kept[e] = 0 are not written. With wgrad_tiled() the [rows, ld]
// operands are K-step-tiled: panel p (rows 256 p .. 256 p + 255) is ld/32 contiguous blocks of
// 256 rows x 32 positions (64-byte rows), wgrad_rows(rows) rows allocated.
struct WgradArgs {
  const void* A;
  const void* B;
  float* out;
  const int32_t* kept;
  const int32_t* koff;
  int E, M, N, ld, C, bf16;
};
bool wgrad_tiled(int bf16);
size_t wgrad_rows(int rows, int bf16);
hipError_t launch_wgrad(const WgradArgs& a, hipStream_t stream);

// koff[e] = sum over e' < e of kept[e'] rounded up to kWgradK; koff[E] = the total.
hipError_t launch_wgrad_offsets(const int32_t* kept, int E, int32_t* koff, hipStream_t stream);

// Router backward, one wave per token: wrow[r] = w of the slot at row r; dz [T,E] = the
// gradient of sum(dy * y) + lam * L with respect to the logits.
struct BwdRouterArgs {
  const void* dy;         // [T,d] dtype
  const float* y_perm;    // [R,d] expert outputs (GEMM2 result)
  const int32_t* dest;    // [T,k]
  const int32_t* idx;     // [T,k] the router's choices
  const int32_t* cand;    // [T,k] or null: rerouted experts (-1: the slot stays at idx)
  const float* w;         // [T,k] combine weights
  const float* s;         // [T,E] scores (or logits when they are the scores)
  const float* f;         // [E]
  float lam_E_over_T;     // lam * E / T
  float tau;
  int T, d, E, k;
  float* wrow;            // [R]
  float* dz;              // [T,E]
};
hipError_t launch_bwd_router(const BwdRouterArgs& a, int bf16, hipStream_t stream);

// dst[b] = src[b] transposed, [B][Rn][Cn] -> [B][Cn][Rn] (Rn, Cn multiples of 4).
hipError_t launch_transpose(const void* src, void* dst, int B, int Rn, int Cn, int bf16, hipStream_t stream);

// Expert-sorted rows to zero-padded columns (see WgradArgs): dst [ncol, ld] with
// dst[n][koff[e] + i] = scale[r] * src[rows ? rows[r] : r][n], r = offsets[e] + i, i < kept[e];
// zero for kept[e] <= i < K_e. ld is a multiple of kWgradK at least sum_e K_e.
struct RowsToColsArgs {
  const void* src;
  const int32_t* rows;    // or null
  const float* scale;     // [R] or null
  const int32_t* kept;
  const int32_t* offsets;
  const int32_t* koff;
  int E, ncol, ld;
  void* dst;
  int src_tiled;          // src is in the K-step-tiled panels of ffn_h_tiled (rows unused)
  int dst_tiled;          // dst is in the K-step-tiled layout of wgrad_tiled (ncol rows)
};
hipError_t launch_rows_to_cols(const RowsToColsArgs& a, int bf16, hipStream_t stream);

// db[e][m] = sum_i src[m][koff[e] + i] over expert e's padded columns (float [E, M]); src in
// the layout of wgrad_tiled(bf16).
hipError_t launch_segment_rowsum(const void* src, const int32_t* kept, const int32_t* koff, int E, int M, int ld,
                                 int bf16, float* db, hipStream_t stream);

// out[e] = 0 (per_expert floats) for every expert e with kept[e] = 0.
hipError_t launch_zero_empty(float* out, const int32_t* kept, int E, size_t per_expert, hipStream_t stream);

// dWg = dz^T x (float [E,d]) and dbg = column sums of dz (float [E], nullable) through part
// [dwg_slices(T,d,E) * (E*d + E)] partial sums.
int dwg_slices(int T, int d, int E);
hipError_t launch_dwg(const void* x, const float* dz, int T, int d, int E, int bf16, float* part, float* dWg,
                      float* dbg, hipStream_t stream);

// dx[t] = sum_j dXp[dest_tj] + dz_t W_g (dtype [T,d]).
struct DxArgs {
  const float* dXp;
  const int32_t* dest;
  const float* dz;
  const void* Wg;
  int T, d, E, k;
  void* dx;
};
hipError_t launch_dx(const DxArgs& a, int bf16, hipStream_t stream);

// Peak probes (csrc/probe.hip): a plain device copy of `bytes` (a multiple of 16), and
// `workgroups` x 256 threads of independent bf16 MFMA chains (probe_mfma_chains() per wave).
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_probe_mfma(float* out, int workgroups, int iters, hipStream_t stream);
int probe_mfma_chains();

}  // namespace moe
