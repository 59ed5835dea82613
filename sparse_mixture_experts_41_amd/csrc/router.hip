// Router: logits, scores, softmax, top-k, renormalised weights, per-group probability sums
// and per-group expert histograms, in one kernel.
//
// Method: the gate p_i = softmax(x W_g)_i, top-k selection on the logits rather than the
// probabilities, and the second normalisation of the k chosen probabilities (kwkr.cn page on
// sparse activation, section 2.1); Gumbel noise added before a temperature-scaled softmax
// ("Mixture of Experts (MoE) 原理与工程落地全指南", lpnh.cn, section 2.2); softmax and top-k fused
// with the gate product in one kernel (kwkr.cn page, section 5.3).
//
// Layout (bfloat16): one workgroup per 16 tokens computes their logits over all of d with
// MFMAs, reading each x row once, adds the four wave partials in a fixed order, and runs
// softmax and top-k with four lanes per token row (the row lives in LDS). With fewer than 256
// groups of 16 tokens, d is cut into K slices instead: slice partials go to a workspace and a
// second kernel adds them in slice order before the same epilogue. With many groups and a
// small W_g, a persistent streaming kernel instead gives each wave whole groups and keeps W_g
// in LDS (router_stream_kernel). Partial statistics (column sums of p, expert histograms) are
// written per group of 16 tokens.
#include <type_traits>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ float router_noise(int kind, float std, uint32_t t, uint32_t e, uint32_t k0,
                                              uint32_t k1) {
  return kind == kNoiseGumbel ? gumbel_noise(t, e, k0, k1) : gaussian_noise(t, e, k0, k1, std);
}

// Epilogue of up to BT tokens held by one wave (BT = 16 or 64). `rows` (LDS, BT rows of pitch
// ldr) holds the float32 logits z (bias added) of tokens t0 .. t0+nt-1. Writes the logits and
// scores (coalesced, from LDS), then per token (one lane each) the top-k indices and weights;
// leaves p in `rows` (zero rows past nt) and returns this lane's bitmask of chosen experts.
template <int BT>
__device__ uint64_t group_epilogue(float* rows, int ldr, int t0, int nt, int E, int k, float tau, int noise,
                                   float noise_std, uint32_t key0, uint32_t key1, float* __restrict__ logits,
                                   float* __restrict__ scores, int32_t* __restrict__ idx_out,
                                   float* __restrict__ w_out, int32_t* __restrict__ next_out, float& entropy) {
  const int lane = lane_id();
  const size_t base = static_cast<size_t>(t0) * E;
  for (int i = lane; i < nt * E; i += kWave) logits[base + i] = rows[(i / E) * ldr + i % E];
  const bool valid = lane < nt;                    // nt <= BT
  entropy = 0.0f;
  float* row = rows + (lane < BT ? lane : 0) * ldr;
  if (valid && (noise != kNoiseNone || tau != 1.0f)) {
    const int t = t0 + lane;
    for (int e = 0; e < E; ++e) {
      float s = row[e];
      if (noise != kNoiseNone)
        s = s + router_noise(noise, noise_std, static_cast<uint32_t>(t), static_cast<uint32_t>(e), key0, key1);
      if (tau != 1.0f) s = s / tau;
      row[e] = s;
    }
  }
  __syncthreads();
  if (scores)
    for (int i = lane; i < nt * E; i += kWave) scores[base + i] = rows[(i / E) * ldr + i % E];
  __syncthreads();
  if (!valid) {
    if (lane < BT)
      for (int e = 0; e < E; ++e) row[e] = 0.0f;
    return 0ull;
  }
  // top-k on the scores: strict '>' keeps the lowest index among equal values (and -0 == +0);
  // branch-free scans so the LDS reads of a row pipeline. With next_out, up to k more
  // selections give the next-ranked experts (for rerouting).
  const int jmax = next_out != nullptr ? min(2 * k, E) : k;
  uint64_t sel = 0ull, used = 0ull;
  int idx[2 * kMaxK];
#pragma unroll
  for (int j = 0; j < 2 * kMaxK; ++j) {
    idx[j] = -1;
    if (j < jmax) {
      int best = -1;
      float bv = 0.0f;
#pragma unroll 8
      for (int e = 0; e < E; ++e) {
        const float v = row[e];
        const bool take = !((used >> e) & 1ull) && (best < 0 || v > bv);
        best = take ? e : best;
        bv = take ? v : bv;
      }
      idx[j] = best;
      used |= 1ull << best;
      if (j < k) sel |= 1ull << best;
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
  float h = 0.0f;
#pragma unroll 8
  for (int e = 0; e < E; ++e) {
    const float pe = row[e] / sum;
    row[e] = pe;
    h -= pe > 0.0f ? pe * logf(pe) : 0.0f;
  }
  entropy = h;
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
      if (next_out != nullptr) next_out[koff + j] = idx[k + j];
    }
  }
  return sel;
}

// After the epilogue: for each 16-token group g of the wave's BT rows, the column sums of p
// over the group's rows (ascending order) and the group's histogram of chosen experts.
// Group indices at or past ng are not written.
template <int BT>
__device__ __forceinline__ void group_partials(const float* rows, int ldr, uint64_t sel, int grp0, int ng, int E,
                                               float* __restrict__ probsum_part, int32_t* __restrict__ hist) {
  constexpr int NG = BT / kGroupTokens;
  const int lane = lane_id();
  if (lane < E) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (grp0 + g >= ng) break;
      float s = 0.0f;
#pragma unroll
      for (int r = 0; r < kGroupTokens; ++r) s += rows[(g * kGroupTokens + r) * ldr + lane];
      probsum_part[static_cast<size_t>(grp0 + g) * E + lane] = s;
    }
  }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    if (lane < NG && grp0 + lane < ng)
      hist[static_cast<size_t>(grp0 + lane) * E + e] = __popcll((b >> (kGroupTokens * lane)) & 0xFFFFull);
  }
}

// Epilogue of the 16 tokens of one group held by one wave, four lanes per token: lane
// 4 t + q handles experts [q EQ, (q+1) EQ) of token t (EQ = ceil(E/4)). Same results as
// group_epilogue: top-k on the scores with the lowest index kept among equal values, softmax
// in float32 (its max is the first chosen score), weights renormalised over the k chosen.
// Cross-lane steps are xor butterflies within each group of four lanes, so all four lanes of a
// token hold identical values. Leaves p in `rows` (zero rows past nt); lane 4 t returns token
// t's bitmask of chosen experts, the other lanes 0.
// The synchronisation of the epilogue's LDS row buffer: the workgroup barrier when the
// workgroup's waves share the rows, or only a compiler fence when one wave owns them (a
// wave's LDS accesses are processed in order, so its lanes see each other's earlier writes).
template <bool WAVE>
__device__ __forceinline__ void rows_sync() {
  if constexpr (WAVE) {
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  } else {
    __syncthreads();
  }
}

template <bool WAVE>
__device__ __forceinline__ uint64_t quad_epilogue(float* rows, int ldr, int t0, int nt, int E, int k, float tau, int noise,
                                  float noise_std, uint32_t key0, uint32_t key1, float* __restrict__ logits,
                                  float* __restrict__ scores, int32_t* __restrict__ idx_out,
                                  float* __restrict__ w_out, int32_t* __restrict__ next_out, bool want_entropy,
                                  float& entropy) {
  // the per-expert loops unrolled by 4 so that their LDS reads pipeline; not in the streaming
  // kernel (WAVE), whose in-flight operand loads leave no registers for it
  constexpr int UNR = WAVE ? 1 : 4;
  const int lane = lane_id();
  const size_t base = static_cast<size_t>(t0) * E;
  for (int r = 0; r < nt; ++r)               // E <= 64: one coalesced row per step
    if (lane < E) logits[base + static_cast<size_t>(r) * E + lane] = rows[r * ldr + lane];
  const int tl = lane >> 2, q = lane & 3;
  const int EQ = (E + 3) >> 2;
  const int e0 = q * EQ, e1 = min(E, e0 + EQ);
  float* row = rows + tl * ldr;
  const bool valid = tl < nt;
  if (valid && (noise != kNoiseNone || tau != 1.0f)) {
    const int t = t0 + tl;
#pragma unroll UNR
    for (int e = e0; e < e1; ++e) {
      float s = row[e];
      if (noise != kNoiseNone)
        s = s + router_noise(noise, noise_std, static_cast<uint32_t>(t), static_cast<uint32_t>(e), key0, key1);
      if (tau != 1.0f) s = s / tau;
      row[e] = s;
    }
  }
  rows_sync<WAVE>();
  if (scores)
    for (int r = 0; r < nt; ++r)
      if (lane < E) scores[base + static_cast<size_t>(r) * E + lane] = rows[r * ldr + lane];
  rows_sync<WAVE>();
  entropy = 0.0f;
  if (!valid) {
    for (int e = e0; e < e1; ++e) row[e] = 0.0f;
    return 0ull;
  }
  // selections in score order: the first k are the choices; with next_out, up to k more (the
  // next-ranked experts, for rerouting)
  const int jmax = next_out != nullptr ? min(2 * k, E) : k;
  uint64_t sel = 0ull, used = 0ull;
  int idx[2 * kMaxK];
#pragma unroll
  for (int j = 0; j < 2 * kMaxK; ++j) {
    idx[j] = -1;
    if (j < jmax) {
      int best = -1;
      float bv = 0.0f;
#pragma unroll UNR
      for (int e = e0; e < e1; ++e) {
        const float v = row[e];
        const bool take = !((used >> e) & 1ull) && (best < 0 || v > bv);
        best = take ? e : best;
        bv = take ? v : bv;
      }
#pragma unroll
      for (int m = 1; m <= 2; m <<= 1) {   // the lower lane of each pair holds the lower experts
        const int ob = __shfl_xor(best, m);
        const float ov = __shfl_xor(bv, m);
        const bool other_lower = (lane & m) != 0;   // the partner's experts come first
        const bool take = ob >= 0 && (best < 0 || ov > bv || (ov == bv && other_lower));
        best = take ? ob : best;
        bv = take ? ov : bv;
      }
      idx[j] = best;
      used |= 1ull << best;
      if (j < k) sel |= 1ull << best;
    }
  }
  const float mx = row[idx[0]];
  float sum = 0.0f;
#pragma unroll UNR
  for (int e = e0; e < e1; ++e) {
    const float ex = __expf(row[e] - mx);
    row[e] = ex;
    sum += ex;
  }
  sum += __shfl_xor(sum, 1);
  sum += __shfl_xor(sum, 2);
  const float inv = 1.0f / sum;
  float h = 0.0f;                            // -sum p ln p over this lane's experts (0 ln 0 = 0)
#pragma unroll UNR
  for (int e = e0; e < e1; ++e) {
    const float pe = row[e] * inv;
    row[e] = pe;
    if (want_entropy) h -= pe > 0.0f ? pe * __logf(pe) : 0.0f;
  }
  if (want_entropy) {
    h += __shfl_xor(h, 1);
    h += __shfl_xor(h, 2);
  }
  entropy = h;
  rows_sync<WAVE>();
  float psel = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) psel += row[idx[j]];
  if (q == 0) {
    const size_t koff = static_cast<size_t>(t0 + tl) * k;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        idx_out[koff + j] = idx[j];
        w_out[koff + j] = row[idx[j]] / psel;
        if (next_out != nullptr) next_out[koff + j] = idx[k + j];
      }
    }
  }
  return q == 0 ? sel : 0ull;
}

// One wave per 16-token group `grp`: epilogue (four lanes per token) and the group partials.
// `rows` holds the group's logits with b_g added; rows past nt_tok are ignored. WAVE: the
// calling wave owns `rows` and its scratch (no workgroup barrier).
template <bool WAVE = false>
__device__ __forceinline__ void group_finish(const RouterArgs& a, float* rows, int LDE, int t0, int nt_tok, int grp) {
  const int lane = lane_id();
  const int E = a.E;
  float ent;
  const uint64_t sel = quad_epilogue<WAVE>(rows, LDE, t0, nt_tok, E, a.k, a.tau, a.noise, a.noise_std, a.key0,
                                           a.key1, a.logits, a.scores, a.idx, a.w, a.idx_next,
                                           a.ent_part != nullptr, ent);
  rows_sync<WAVE>();
  if (a.ent_part != nullptr) {               // the group's entropy sum, tokens in order
    __shared__ float ents[kWaves][kGroupTokens];
    float* en = ents[threadIdx.x >> 6];
    if ((lane & 3) == 0) en[lane >> 2] = ent;   // zero for tokens past nt_tok
    rows_sync<WAVE>();
    if (lane == 0) {
      float sum = 0.0f;
#pragma unroll
      for (int t = 0; t < kGroupTokens; ++t) sum += en[t];
      a.ent_part[grp] = sum;
    }
  }
  // group partials: column sums of p over the 16 rows (ascending), and the histogram, whose bits
  // come from lane 4 t of each token (the popcount of the whole ballot)
  const size_t gofs = static_cast<size_t>(grp) * E;
  if (lane < E) {
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < kGroupTokens; ++r) ps += rows[r * LDE + lane];
    a.probsum_part[gofs + lane] = ps;
  }
  // each token's mask (held by lane 4 t) to LDS, then lane e counts expert e over the tokens
  __shared__ uint64_t masks[kWaves][kGroupTokens];
  uint64_t* mk = masks[threadIdx.x >> 6];
  if ((lane & 3) == 0) mk[lane >> 2] = sel;   // zero for tokens past nt_tok
  rows_sync<WAVE>();
  if (lane < E) {
    int c = 0;
#pragma unroll
    for (int t = 0; t < kGroupTokens; ++t) c += static_cast<int>((mk[t] >> lane) & 1ull);
    a.hist[gofs + lane] = c;
  }
}

// bf16 router: one workgroup per MT groups of 16 tokens over all of d (or over one K slice,
// SPLIT). The chunks of 64 along d are dealt round-robin to the WV waves; each wave issues the
// loads of NB chunks before their MFMAs and accumulates MT x NT tiles of
// v_mfma_f32_16x16x32_bf16 (x rows as A, W_g rows as B, both K-contiguous). The wave partials
// are added in LDS in wave order, the bias is added, and wave w runs the epilogue of group w.
// MT = 4 cuts the W_g traffic per token by four when E is large. WV = 8 (when the grid is at
// most one workgroup per CU) keeps twice the loads in flight per CU.
template <int NT, int NB, int MT, bool SPLIT, int WV = kWaves>
__global__ __launch_bounds__(kWave * WV) void router_bf16_kernel(RouterArgs a, float* __restrict__ zpart) {
  static_assert(MT <= kWaves && (WV == 4 || WV == 8), "group_finish's scratch is indexed by wave < kWaves");
  constexpr int TB = kGroupTokens * MT;
  constexpr int LDR = 16 * NT + 1, LDE = kMaxE + 1;
  constexpr int NTH = kWave * WV;
  __shared__ float red[WV][TB * LDR];
  __shared__ float rows[TB * LDE];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int t0 = blockIdx.x * TB;
  const int nt_tok = min(TB, a.T - t0);
  const int d = a.d, E = a.E;
  // K slice blockIdx.y of gridDim.y: chunks [cb, ce) of 64
  const int nchunk_all = d / 64, ks = blockIdx.y, KS = gridDim.y;
  const int cb = ks * nchunk_all / KS, ce = (ks + 1) * nchunk_all / KS;
  const int nchunk = ce - cb;
  const u16* __restrict__ x = static_cast<const u16*>(a.x) + static_cast<size_t>(cb) * 64;
  const u16* __restrict__ Wg = static_cast<const u16*>(a.Wg) + static_cast<size_t>(cb) * 64;
  const int r16 = lane & 15, g = lane >> 4;
  // rows past the last token re-read the last token; they only feed rows that are not kept
  const u16* ap[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) ap[m] = x + static_cast<size_t>(t0 + min(m * 16 + r16, nt_tok - 1)) * d + 16 * g;
  const u16* bp[NT];
  bool bvalid[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int e = n * 16 + r16;
    bvalid[n] = e < E;
    bp[n] = Wg + static_cast<size_t>(bvalid[n] ? e : 0) * d + 16 * g;
  }
  floatx4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = floatx4{0.f, 0.f, 0.f, 0.f};
  // chunk c covers k in [64c, 64c + 64): lane group g takes k 64c + 16g + [0, 16) as two
  // 8-element pieces, and MFMA step h uses piece h of both operands (same k order on A and B)
  for (int c0 = wave; c0 < nchunk; c0 += WV * NB) {
    bf16x8 av[NB][MT][2], bv[NB][NT][2];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int kc = (c0 + WV * i) * 64;
      if (c0 + WV * i < nchunk) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          av[i][m][0] = *reinterpret_cast<const bf16x8*>(ap[m] + kc);
          av[i][m][1] = *reinterpret_cast<const bf16x8*>(ap[m] + kc + 8);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          bv[i][n][0] = bvalid[n] ? *reinterpret_cast<const bf16x8*>(bp[n] + kc) : bf16x8{};
          bv[i][n][1] = bvalid[n] ? *reinterpret_cast<const bf16x8*>(bp[n] + kc + 8) : bf16x8{};
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (c0 + WV * i < nchunk) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int n = 0; n < NT; ++n)
              acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i][m][h], bv[i][n][h], acc[m][n], 0, 0, 0);
      }
    }
  }
  // C layout of the 16x16 tile: lane holds column (lane & 15), rows 4*(lane>>4) + i.
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][(m * 16 + 4 * g + i) * LDR + n * 16 + r16] = acc[m][n][i];
  __syncthreads();
  // the wave partials of element l, added in wave order
  auto wave_sum = [&](int l) {
    float z = red[0][l];
#pragma unroll
    for (int w = 1; w < WV; ++w) z += red[w][l];
    return z;
  };
  if (SPLIT) {   // slice partial sums to zpart[ks][t][e]; router_finish_kernel does the rest
    for (int o = threadIdx.x; o < nt_tok * E; o += NTH) {
      const int row = o / E, col = o - row * E;
      zpart[(static_cast<size_t>(ks) * a.T + t0 + row) * E + col] = wave_sum(row * LDR + col);
    }
    return;
  }
  for (int o = threadIdx.x; o < TB * E; o += NTH) {
    const int row = o / E, col = o - row * E;
    rows[row * LDE + col] = wave_sum(row * LDR + col) + (a.bg != nullptr ? a.bg[col] : 0.0f);
  }
  __syncthreads();
  // wave w finishes group w; waves without a group leave (the remaining barriers count the rest)
  const int nt_w = min(kGroupTokens, nt_tok - wave * kGroupTokens);
  if (wave >= MT || nt_w <= 0) return;
  group_finish(a, rows + wave * kGroupTokens * LDE, LDE, t0 + wave * kGroupTokens, nt_w, blockIdx.x * MT + wave);
}

// Streaming bf16 router for many token groups. A persistent grid in which each wave owns whole
// 16-token groups over all of d (wave slot s of S takes groups s, s + S, ...), so waves never
// wait for one another. W_g is staged in LDS once per workgroup (E rows, row pitch 2d + 16
// bytes, which spreads the 16 rows of a fragment read over the banks) and supplies every
// group's B fragments, so only x streams from HBM. A wave's loads come in batches of NB chunks
// of 64 along d, double-buffered: the next batch (the next group's first, after a group's
// last) is issued before the current one is multiplied, which keeps the next group's rows in
// flight during this group's epilogue. A lane's two 16-byte pieces of a chunk are k offsets
// 8 g and 32 + 8 g (its lane group g): each load instruction reads 64 contiguous bytes of
// each of 16 rows, and A and B use the same k order. Rows past the last token re-read the
// last token; they only feed rows that are not kept. Wave slot s takes a group's batches in
// the order s, s + 1, ... (mod the batches per group), so that the waves running at one time
// read different column ranges of their rows (rows d * 2 bytes apart): 76 -> 70 us on 65536
// tokens of d = 2048 against every wave starting at column 0.
constexpr int kStreamWg = 68 * 1024;     // W_g bytes in LDS (two workgroups per CU)

template <int NT, int NB, int WCAP>
__global__ __launch_bounds__(256) void router_stream_kernel(RouterArgs a) {
  constexpr int LDE = 16 * NT + 1;
  __shared__ __attribute__((aligned(16))) char wlds[WCAP];
  __shared__ float rows_all[kWaves][kGroupTokens * LDE];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int d = a.d, E = a.E, T = a.T;
  const int ng = (T + kGroupTokens - 1) / kGroupTokens;
  const int pitch = 2 * d + 16;
  const int nchunk = d / 64;
  const int nbat = (nchunk + NB - 1) / NB;          // batches per group
  const int S = gridDim.x * kWaves;
  const int slot = blockIdx.x * kWaves + wave;
  const int r16 = lane & 15, g = lane >> 4;
  const u16* __restrict__ x = static_cast<const u16*>(a.x);
  // the wave's batch q: group slot + (q / nbat) S, chunks [NB (q % nbat), ...); loads past the
  // wave's last batch re-read it (the count of loads in flight stays the same every step)
  const int my_groups = slot < ng ? (ng - 1 - slot) / S + 1 : 0;
  const int nq = my_groups * nbat;
  bf16x8 av[2][NB][2];
  // buffers are chosen by compile-time constants (a runtime index would put av in scratch)
  auto issue = [&](int q, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int qq = q < nq ? q : nq - 1;
    const int grp = slot + (qq / nbat) * S, b = (qq % nbat + slot) % nbat;
    const int t = min(grp * kGroupTokens + r16, T - 1);
    const u16* row = x + static_cast<size_t>(t) * d + 8 * g;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = min(b * NB + i, nchunk - 1);
      av[buf][i][0] = *reinterpret_cast<const bf16x8*>(row + c * 64);
      av[buf][i][1] = *reinterpret_cast<const bf16x8*>(row + c * 64 + 32);
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (nq > 0) issue(0, B0{});
  // stage W_g: 16-byte pieces, row e at e * pitch, eight loads in flight per thread
  {
    const int per_row = d / 8, n = E * per_row;
    const u16* __restrict__ Wg = static_cast<const u16*>(a.Wg);
    for (int i0 = threadIdx.x; i0 < n; i0 += 8 * 256) {
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + 256 * j;
        if (i < n) {
          const int e = i / per_row, c = i - e * per_row;
          v[j] = *reinterpret_cast<const u32x4*>(Wg + static_cast<size_t>(e) * d + c * 8);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + 256 * j;
        if (i < n) {
          const int e = i / per_row, c = i - e * per_row;
          *reinterpret_cast<u32x4*>(wlds + e * pitch + c * 16) = v[j];
        }
      }
    }
  }
  __syncthreads();
  if (nq == 0) return;
  // B fragment of tile n: row e = 16 n + r16 (zero past E), k offset 8 g (+ 32) in the chunk
  int boff[NT];
  bool bvalid[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int e = 16 * n + r16;
    bvalid[n] = e < E;
    boff[n] = (bvalid[n] ? e : 0) * pitch + 16 * g;
  }
  float* rows = rows_all[wave];
  floatx4 acc[NT];
  auto step = [&](int q, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int p = q % nbat, b = (p + slot) % nbat;   // position p in the group, batch b of d
    if (p == 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = b * NB + i;
      if (c < nchunk) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const bf16x8 bv = bvalid[n] ? *reinterpret_cast<const bf16x8*>(wlds + boff[n] + c * 128 + 64 * h)
                                        : bf16x8{};
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[buf][i][h], bv, acc[n], 0, 0, 0);
          }
      }
    }
    if (p == nbat - 1) {                     // the group's logits are complete: epilogue
      const int grp = slot + (q / nbat) * S;
      const int t0 = grp * kGroupTokens;
      // C layout of a 16x16 tile: lane holds column r16, rows 4 g + i
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 16 * n + r16;
          if (e < E) rows[(4 * g + i) * LDE + e] = acc[n][i] + (a.bg != nullptr ? a.bg[e] : 0.0f);
        }
      group_finish<true>(a, rows, LDE, t0, min(kGroupTokens, T - t0), grp);
    }
  };
  int q = 0;
  for (; q + 1 < nq; q += 2) {
    issue(q + 1, B1{});
    step(q, B0{});
    issue(q + 2, B0{});
    step(q + 1, B1{});
  }
  if (q < nq) {
    issue(q + 1, B1{});                      // keeps the loads in flight uniform; unused
    step(q, B0{});
  }
}

// Sums the KS slice partials of one 16-token group in slice order (all 256 threads, every load
// in flight at once), adds b_g, and runs the group epilogue on wave 0.
constexpr int kMaxSlices = 16;
__global__ __launch_bounds__(256) void router_finish_kernel(RouterArgs a, int KS, const float* __restrict__ zpart) {
  constexpr int LDE = kMaxE + 1;
  constexpr int PER = kGroupTokens * kMaxE / 256;   // <= 4 elements per thread
  __shared__ float rows[kGroupTokens * LDE];
  const int t0 = blockIdx.x * kGroupTokens;
  const int nt_tok = min(kGroupTokens, a.T - t0);
  const int E = a.E, n = nt_tok * E;
  const size_t base = static_cast<size_t>(t0) * E, slice = static_cast<size_t>(a.T) * E;
  // every slice's loads in flight at once (KS <= kMaxSlices), then added in slice order
  float v[kMaxSlices][PER];
#pragma unroll
  for (int ks = 0; ks < kMaxSlices; ++ks)
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = threadIdx.x + 256 * j;
      v[ks][j] = (ks < KS && i < n) ? zpart[ks * slice + base + i] : 0.0f;
    }
  float z[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    z[j] = v[0][j];
#pragma unroll
    for (int ks = 1; ks < kMaxSlices; ++ks)
      if (ks < KS) z[j] += v[ks][j];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < n) {
      const int e = i % E;
      rows[(i / E) * LDE + e] = z[j] + (a.bg != nullptr ? a.bg[e] : 0.0f);
    }
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;   // the remaining barriers count wave 0 only
  group_finish(a, rows, LDE, t0, nt_tok, blockIdx.x);
}

// float32 storage: plain FMA dot products, one lane per token, 64 tokens per workgroup
// (small sizes only).
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
  float ent;
  const uint64_t sel = group_epilogue<kBlockTokens>(rows, LDR, t0, nt, a.E, a.k, a.tau, a.noise, a.noise_std, a.key0,
                                                    a.key1, a.logits, a.scores, a.idx, a.w, a.idx_next, ent);
  __syncthreads();
  const int grp0 = blk * (kBlockTokens / kGroupTokens);
  group_partials<kBlockTokens>(rows, LDR, sel, grp0, a.ng, a.E, a.probsum_part, a.hist);
  if (a.ent_part != nullptr) {               // per-group entropy sums, tokens in order
    __shared__ float ents[kBlockTokens];
    ents[lane] = ent;                         // zero past nt
    __syncthreads();
    if (lane < kBlockTokens / kGroupTokens && grp0 + lane < a.ng) {
      float sum = 0.0f;
      for (int t = 0; t < kGroupTokens; ++t) sum += ents[lane * kGroupTokens + t];
      a.ent_part[grp0 + lane] = sum;
    }
  }
}

// Per-group expert histogram of given top-k indices: one wave per 64 tokens, four groups.
__global__ __launch_bounds__(64) void histogram_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                       int32_t* __restrict__ hist) {
  constexpr int NG = kBlockTokens / kGroupTokens;
  const int lane = lane_id();
  const int blk = blockIdx.x;
  const int t = blk * kBlockTokens + lane;
  const int ng = (T + kGroupTokens - 1) / kGroupTokens;
  const int grp0 = blk * NG;
  uint64_t sel = 0ull;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = idx[static_cast<size_t>(t) * k + j];
      if (e >= 0 && e < E) sel |= 1ull << e;
    }
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(static_cast<int>((sel >> e) & 1ull));
    if (lane < NG && grp0 + lane < ng)
      hist[static_cast<size_t>(grp0 + lane) * E + e] = __popcll((b >> (kGroupTokens * lane)) & 0xFFFFull);
  }
}

}  // namespace

int router_slices(int T, int d, int E) {
  (void)E;
  const int ng = (T + kGroupTokens - 1) / kGroupTokens;
  if (ng >= 256) return 1;                   // enough groups to fill the chip: one fused kernel
  int ks = (512 + ng - 1) / ng;              // aim at >= 512 workgroups
  const int cap = d / 64 / 4;                // >= 4 chunks (one per wave) per slice
  ks = ks < cap ? ks : cap;
  return ks < 1 ? 1 : (ks > kMaxSlices ? kMaxSlices : ks);
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// The bytes of W_g in LDS with the streaming router's padded row pitch.
static size_t stream_wg_bytes(const RouterArgs& a) { return static_cast<size_t>(a.E) * (2 * a.d + 16); }

template <int NT>
static hipError_t launch_router_bf16(const RouterArgs& a, float* zpart, hipStream_t stream) {
  // keep about 8 chunks' worth of operand registers per lane: 2 (x) + 2 NT (W_g) per chunk
  constexpr int NB = NT == 1 ? 8 : (NT == 2 ? 4 : 2);
  const int ng = (a.T + kGroupTokens - 1) / kGroupTokens;
  const int KS = router_slices(a.T, a.d, a.E);
  const int cus = device_cus();
  // W_g up to 68 KB (two workgroups per CU): measured 93 -> 79 us on 65536 tokens, d = 2048,
  // E = 16. With one workgroup per CU (W_g up to 132 KB) it measured no faster than the
  // per-group kernel below (16384 tokens, d = 1024, E = 64: 43 vs 46 us), so it is not used.
  if (KS == 1 && ng >= 4 * cus && stream_wg_bytes(a) <= static_cast<size_t>(kStreamWg)) {
    const int grid = min(2 * cus, (ng + kWaves - 1) / kWaves);
    hipLaunchKernelGGL((router_stream_kernel<NT, 8, kStreamWg>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (KS == 1) {
    // at most one workgroup per CU: 8 waves each, twice the loads in flight per CU
    if constexpr (NT >= 3) {
      if (ng >= 4 * 256) {                   // large E and enough tokens: 64 tokens per workgroup
        const int grid = (ng + 3) / 4;
        if (grid <= cus)
          hipLaunchKernelGGL((router_bf16_kernel<NT, 2, 4, false, 8>), dim3(grid), dim3(8 * kWave), 0, stream, a,
                             nullptr);
        else
          hipLaunchKernelGGL((router_bf16_kernel<NT, 2, 4, false>), dim3(grid), dim3(256), 0, stream, a, nullptr);
        return hipGetLastError();
      }
    }
    if (ng <= cus)
      hipLaunchKernelGGL((router_bf16_kernel<NT, NB, 1, false, 8>), dim3(ng), dim3(8 * kWave), 0, stream, a, nullptr);
    else
      hipLaunchKernelGGL((router_bf16_kernel<NT, NB, 1, false>), dim3(ng), dim3(256), 0, stream, a, nullptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((router_bf16_kernel<NT, NB, 1, true>), dim3(ng, KS), dim3(256), 0, stream, a, zpart);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(router_finish_kernel, dim3(ng), dim3(256), 0, stream, a, KS, zpart);
  return hipGetLastError();
}

hipError_t launch_router(const RouterArgs& a, float* zpart, hipStream_t stream) {
  if (!a.bf16) {
    const dim3 grid((a.T + kBlockTokens - 1) / kBlockTokens), block(kWave);
    hipLaunchKernelGGL(router_f32_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
  }
  switch ((a.E + 15) / 16) {
    case 1: return launch_router_bf16<1>(a, zpart, stream);
    case 2: return launch_router_bf16<2>(a, zpart, stream);
    case 3: return launch_router_bf16<3>(a, zpart, stream);
    default: return launch_router_bf16<4>(a, zpart, stream);
  }
}

hipError_t launch_histogram(const int32_t* idx, int T, int E, int k, int32_t* hist, hipStream_t stream) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(histogram_kernel, dim3(nblk), dim3(64), 0, stream, idx, T, E, k, hist);
  return hipGetLastError();
}

}  // namespace moe
