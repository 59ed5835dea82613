// C ABI of the MoE layer: argument validation, workspace carving and stage orchestration.
// Every check happens before the first HIP call, so an invalid call enqueues nothing.
#include "../../include/moe.h"
#include "../../include/moe_probe.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>

#include "moe_kernels.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

struct Derived {
  int T, d, E, k, dff;
  int64_t C;
  int R;       // rows of the expert-sorted buffers: min(k*T, E*C)
  int ng;      // 16-token routing groups
  bool bf16;
  size_t esize;
  float tau;
  int noise;        // moe::kNoiseNone / kNoiseGumbel / kNoiseGaussian
  float noise_std;  // Gaussian only
  int act;          // moe::kActGelu / kActSilu
  int dffs;         // shared expert hidden width, 0 = none
  int policy;       // MOE_DROP_*
  bool stats;       // routing statistics requested
  bool train;       // the workspace also holds what moe_backward needs, and its scratch
  bool packed = false;   // W1 and W2 come packed by moe_pack_expert_weights
  uint32_t key0, key1;
};

struct Layout {
  size_t probsum, hist, blockbase, colsum, zpart, logits, scores, idx, w, offsets, dest, perm, x_perm, H, y_perm,
      side, Hs, ys, ent, idx_next, cand, hist2, blockbase2, kept1, thresh,
      // training: saved by moe_forward_train, then moe_backward's scratch
      pre, kept_s, f_s, koff, wrow, dz, dA, dXp, W2T, W1T, dOT, HT, dAT, XT, dwg, dyp, total;
  int ld;   // row pitch of the transposed, padded activations
};

// C = ceil(c*k*T/E) for the exact value of the double c = m * 2^sh (m a 53-bit integer).
int64_t capacity_exact(int64_t T, int64_t E, int64_t k, double c) {
  int q = 0;
  const double fr = std::frexp(c, &q);                     // c = fr * 2^q, fr in [0.5, 1)
  const uint64_t m = static_cast<uint64_t>(std::ldexp(fr, 53));
  const int sh = q - 53;
  const unsigned __int128 num = static_cast<unsigned __int128>(m) * static_cast<uint64_t>(k * T);
  if (sh >= 0) {                                           // c >= 2^53: far beyond any token count
    return INT64_MAX;
  }
  if (-sh > 100) return 1;                                 // c*k*T/E < 2^84 / 2^100 < 1, and > 0
  const unsigned __int128 den = static_cast<unsigned __int128>(E) << (-sh);
  const unsigned __int128 C = (num + den - 1) / den;
  return C > static_cast<unsigned __int128>(INT64_MAX) ? INT64_MAX : static_cast<int64_t>(C);
}

moe_status check_config(const moe_config* cfg, Derived* D) {
  if (cfg == nullptr) return fail(MOE_EINVAL, "cfg is NULL");
  const int64_t T = cfg->T, d = cfg->d, E = cfg->E, k = cfg->k, dff = cfg->d_ffn;
  if (T < 1 || d < 1 || E < 1 || k < 1 || dff < 1) return fail(MOE_EINVAL, "T, d, E, k and d_ffn must be >= 1");
  if (k > E) return fail(MOE_EINVAL, "k must not exceed E");
  if (!(cfg->capacity_factor > 0.0) || !std::isfinite(cfg->capacity_factor))
    return fail(MOE_EINVAL, "capacity_factor must be finite and > 0");
  if (!(cfg->temperature > 0.0f) || !std::isfinite(cfg->temperature))
    return fail(MOE_EINVAL, "temperature must be finite and > 0");
  if (cfg->gumbel != 0 && cfg->gumbel != 1) return fail(MOE_EINVAL, "gumbel must be 0 or 1");
  if (cfg->dtype != MOE_F32 && cfg->dtype != MOE_BF16) return fail(MOE_EINVAL, "unknown dtype");
  if (cfg->reserved != 0) return fail(MOE_EINVAL, "reserved must be 0");
  if (T > (int64_t(1) << 31) || T * k >= (int64_t(1) << 31)) return fail(MOE_EINVAL, "k*T must be below 2^31");
  if (E > 64) return fail(MOE_EUNSUPPORTED, "at most 64 experts");
  if (k > 8) return fail(MOE_EUNSUPPORTED, "at most k = 8");
  if (d > 65536 || dff > 65536) return fail(MOE_EUNSUPPORTED, "d and d_ffn are limited to 65536");
  if (cfg->capacity_factor > 1048576.0) return fail(MOE_EUNSUPPORTED, "capacity_factor above 2^20");
  const bool bf16 = cfg->dtype == MOE_BF16;
  if (bf16) {
    if (d % 64 != 0 || dff % 64 != 0) return fail(MOE_EUNSUPPORTED, "bf16 needs d and d_ffn multiples of 64");
  } else {
    if (d % 8 != 0 || dff % 8 != 0) return fail(MOE_EUNSUPPORTED, "float32 needs d and d_ffn multiples of 8");
    if (T > 65536 || d > 4096 || dff > 16384)
      return fail(MOE_EUNSUPPORTED, "float32 is a correctness path: T <= 65536, d <= 4096, d_ffn <= 16384");
  }
  D->T = static_cast<int>(T);
  D->d = static_cast<int>(d);
  D->E = static_cast<int>(E);
  D->k = static_cast<int>(k);
  D->dff = static_cast<int>(dff);
  D->C = capacity_exact(T, E, k, cfg->capacity_factor);
  const int64_t ecap = D->C >= T ? E * T : E * D->C;        // an expert never gets more than T slots
  const int64_t R = (k * T < ecap) ? k * T : ecap;
  D->R = static_cast<int>(R);
  D->ng = static_cast<int>((T + 15) / 16);
  D->bf16 = bf16;
  D->esize = bf16 ? 2 : 4;
  D->tau = cfg->temperature;
  D->noise = cfg->gumbel ? moe::kNoiseGumbel : moe::kNoiseNone;
  D->noise_std = 0.0f;
  D->act = moe::kActGelu;
  D->dffs = 0;
  D->policy = MOE_DROP_TOKEN_ORDER;
  D->stats = false;
  D->train = false;
  D->packed = false;
  D->key0 = static_cast<uint32_t>(cfg->seed & 0xffffffffull);
  D->key1 = static_cast<uint32_t>(cfg->seed >> 32);
  return MOE_OK;
}

// Forward variants on top of a checked configuration.
moe_status check_variant(const moe_variant* v, Derived* D) {
  if (v == nullptr) return MOE_OK;
  if (v->activation != MOE_ACT_GELU && v->activation != MOE_ACT_SILU) return fail(MOE_EINVAL, "unknown activation");
  if (!(v->noise_std >= 0.0f) || !std::isfinite(v->noise_std))
    return fail(MOE_EINVAL, "noise_std must be finite and >= 0");
  if (v->noise_std > 0.0f && D->noise == moe::kNoiseGumbel)
    return fail(MOE_EINVAL, "Gaussian noise (noise_std > 0) needs gumbel = 0");
  if (v->shared_d_ffn < 0) return fail(MOE_EINVAL, "shared_d_ffn must be >= 0");
  if (v->shared_d_ffn > 65536) return fail(MOE_EUNSUPPORTED, "shared_d_ffn is limited to 65536");
  if (v->shared_d_ffn > 0) {
    if (D->bf16 && v->shared_d_ffn % 64 != 0) return fail(MOE_EUNSUPPORTED, "bf16 needs shared_d_ffn % 64 == 0");
    if (!D->bf16 && (v->shared_d_ffn % 8 != 0 || v->shared_d_ffn > 16384))
      return fail(MOE_EUNSUPPORTED, "float32 needs shared_d_ffn a multiple of 8, at most 16384");
  }
  D->act = v->activation == MOE_ACT_SILU ? moe::kActSilu : moe::kActGelu;
  if (v->noise_std > 0.0f) {
    D->noise = moe::kNoiseGaussian;
    D->noise_std = v->noise_std;
  }
  D->dffs = static_cast<int>(v->shared_d_ffn);
  if (v->drop_policy != MOE_DROP_TOKEN_ORDER && v->drop_policy != MOE_DROP_RANDOM && v->drop_policy != MOE_DROP_REROUTE)
    return fail(MOE_EINVAL, "unknown drop_policy");
  if (v->weight_layout != MOE_WEIGHTS_LINEAR && v->weight_layout != MOE_WEIGHTS_PACKED)
    return fail(MOE_EINVAL, "unknown weight_layout");
  if (v->weight_layout == MOE_WEIGHTS_PACKED) {
    if (!D->bf16) return fail(MOE_EUNSUPPORTED, "packed weights need the bf16 dtype");
    if (D->d % 256 != 0 || D->dff % 256 != 0)
      return fail(MOE_EUNSUPPORTED, "packed weights need d and d_ffn multiples of 256");
    D->packed = true;
  }
  if (v->route_stats != nullptr && (reinterpret_cast<uintptr_t>(v->route_stats) & 3u) != 0)
    return fail(MOE_EINVAL, "route_stats is not 4-byte aligned");
  D->policy = v->drop_policy;
  D->stats = v->route_stats != nullptr;
  return MOE_OK;
}

int clamp_c(const Derived& D) { return static_cast<int>(D.C < D.T ? D.C : D.T); }

// Whether the backward's first product reads dy through the permutation (every path but the
// bf16 MFMA path with dy beyond 32-bit buffer offsets, which gathers dy into a copy first).
bool bwd_gathers(const Derived& D) {
  return !D.bf16 || clamp_c(D) <= 16 || static_cast<long long>(D.T) * D.d * 2 < (1ll << 31);
}

Layout layout_of(const Derived& D) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~static_cast<size_t>(255);
    return o;
  };
  const size_t T = D.T, E = D.E, k = D.k, ng = D.ng, R = D.R;
  L.probsum = take(ng * E * 4);
  L.hist = take(ng * E * 4);
  L.blockbase = take(moe::scan_bases_ints(static_cast<int>(ng), static_cast<int>(E)) * 4);
  L.colsum = take(E * 4);
  const int ks = D.bf16 ? moe::router_slices(D.T, D.d, D.E) : 1;
  L.zpart = take(ks > 1 ? static_cast<size_t>(ks) * T * E * 4 : 0);
  L.logits = take(T * E * 4);
  L.scores = take(T * E * 4);
  L.idx = take(T * k * 4);
  L.w = take(T * k * 4);
  L.offsets = take(E * 4);
  L.dest = take(T * k * 4);
  L.perm = take(R * 4);
  L.x_perm = take(R * static_cast<size_t>(D.d) * D.esize);
  L.H = take(moe::ffn_h_rows(static_cast<int>(R), static_cast<int>(E), clamp_c(D), D.bf16) * D.dff * D.esize);
  L.y_perm = take(R * static_cast<size_t>(D.d) * 4);
  L.side = take(D.bf16 && clamp_c(D) > 16 ? moe::tail_side_floats(D.R, D.E, clamp_c(D), D.d) * 4 : 0);
  L.Hs = take(D.dffs > 0 ? moe::ffn_h_rows(static_cast<int>(T), 1, static_cast<int>(T), D.bf16) * D.dffs * D.esize : 0);
  L.ys = take(D.dffs > 0 ? T * static_cast<size_t>(D.d) * 4 : 0);
  const bool random = D.policy == MOE_DROP_RANDOM, reroute = D.policy == MOE_DROP_REROUTE;
  L.ent = take(D.stats ? ng * 4 : 0);
  L.idx_next = take(reroute ? T * k * 4 : 0);
  L.cand = take(reroute ? T * k * 4 : 0);
  L.hist2 = take(random || reroute ? ng * E * 4 : 0);
  L.blockbase2 = take(random || reroute ? moe::scan_bases_ints(static_cast<int>(ng), static_cast<int>(E)) * 4 : 0);
  L.kept1 = take(reroute ? E * 4 : 0);
  L.thresh = take(random ? E * 8 : 0);
  const size_t d = D.d, dff = D.dff, es = D.esize;
  const bool tr = D.train;
  const int64_t ld = (static_cast<int64_t>(R) + static_cast<int64_t>(moe::kWgradK - 1) * D.E + moe::kWgradK - 1) /
                     moe::kWgradK * moe::kWgradK;
  L.ld = tr ? static_cast<int>(ld) : 0;
  const size_t ldz = tr ? static_cast<size_t>(ld) : 0;
  L.pre = take(tr ? R * dff * es : 0);
  L.kept_s = take(tr ? E * 4 : 0);
  L.f_s = take(tr ? E * 4 : 0);
  L.koff = take(tr ? (E + 1) * 4 : 0);
  L.wrow = take(tr ? R * 4 : 0);
  L.dz = take(tr ? T * E * 4 : 0);
  L.dA = take(tr ? moe::ffn_h_rows(static_cast<int>(R), static_cast<int>(E), clamp_c(D), D.bf16) * dff * es : 0);
  L.dXp = take(tr ? R * d * 4 : 0);
  const bool wt = tr && moe::bwd_weights_transposed(D.bf16, clamp_c(D));
  L.W2T = take(wt ? E * d * dff * es : 0);
  L.W1T = take(wt ? E * d * dff * es : 0);
  L.dOT = take(moe::wgrad_rows(static_cast<int>(d), D.bf16) * ldz * es);
  L.HT = take(moe::wgrad_rows(static_cast<int>(dff), D.bf16) * ldz * es);
  L.dAT = take(moe::wgrad_rows(static_cast<int>(dff), D.bf16) * ldz * es);
  L.XT = take(moe::wgrad_rows(static_cast<int>(d), D.bf16) * ldz * es);
  L.dwg = take(tr ? static_cast<size_t>(moe::dwg_slices(D.T, D.d, D.E)) * (E * d + E) * 4 : 0);
  L.dyp = take(tr && !bwd_gathers(D) ? R * d * es : 0);
  L.total = off;
  return L;
}

moe_status need(const void* p, size_t align, const char* name, bool nullable = false) {
  if (p == nullptr) {
    if (nullable) return MOE_OK;
    return fail(MOE_EINVAL, std::string(name) + " is NULL");
  }
  if ((reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0)
    return fail(MOE_EINVAL, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return MOE_OK;
}

moe_status need_ws(const Derived& D, const void* ws, size_t ws_bytes, Layout* L) {
  *L = layout_of(D);
  if (ws_bytes < L->total)
    return fail(MOE_EWORKSPACE, "workspace needs " + std::to_string(L->total) + " bytes, got " + std::to_string(ws_bytes));
  return need(ws, 256, "ws");
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_EHIP, std::string(where) + ": " + hipGetErrorString(e));
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

#define MOE_CHECK(expr)                 \
  do {                                  \
    const moe_status s_ = (expr);       \
    if (s_ != MOE_OK) return s_;        \
  } while (0)

#define MOE_HIP(expr, where)                             \
  do {                                                   \
    const hipError_t e_ = (expr);                        \
    if (e_ != hipSuccess) return hip_fail(e_, where);    \
  } while (0)

// The allocation-free forward's workspace: one file-scope device array, which every GPU the
// library runs on holds until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: its device address on each GPU is looked up once, with that GPU current,
// and only that address is ever handed to kernels.
__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices) return fail(MOE_EUNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MOE_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

moe::RouterArgs router_args(const Derived& D, const void* x, const void* Wg, const float* bg, float* logits,
                            float* scores, int32_t* idx, float* w, float* probsum, int32_t* hist) {
  moe::RouterArgs a{};
  a.x = x;
  a.Wg = Wg;
  a.bg = bg;
  a.T = D.T;
  a.d = D.d;
  a.E = D.E;
  a.k = D.k;
  a.bf16 = D.bf16 ? 1 : 0;
  a.tau = D.tau;
  a.noise = D.noise;
  a.noise_std = D.noise_std;
  a.key0 = D.key0;
  a.key1 = D.key1;
  a.logits = logits;
  a.scores = scores;
  a.idx = idx;
  a.w = w;
  a.probsum_part = probsum;
  a.hist = hist;
  a.ng = D.ng;
  return a;
}

}  // namespace

extern "C" {

int64_t moe_capacity(const moe_config* cfg) {
  Derived D;
  if (check_config(cfg, &D) != MOE_OK) return -1;
  return D.C;
}

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  Derived D;
  MOE_CHECK(check_config(cfg, &D));
  if (bytes == nullptr) return fail(MOE_EINVAL, "bytes is NULL");
  *bytes = layout_of(D).total;
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* Wg, const float* bg, float* logits,
                     float* scores, int32_t* topk_idx, float* topk_w, float* prob_colsum, void* ws, size_t ws_bytes,
                     moe_stream_t stream) {
  Derived D;
  Layout L;
  MOE_CHECK(check_config(cfg, &D));
  MOE_CHECK(need(x, 16, "x"));
  MOE_CHECK(need(Wg, 16, "Wg"));
  MOE_CHECK(need(bg, 4, "bg", true));
  MOE_CHECK(need(logits, 4, "logits"));
  MOE_CHECK(need(scores, 4, "scores", true));
  MOE_CHECK(need(topk_idx, 4, "topk_idx"));
  MOE_CHECK(need(topk_w, 4, "topk_w"));
  MOE_CHECK(need(prob_colsum, 4, "prob_colsum"));
  MOE_CHECK(need_ws(D, ws, ws_bytes, &L));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const moe::RouterArgs a = router_args(D, x, Wg, bg, logits, scores, topk_idx, topk_w, at<float>(ws, L.probsum),
                                        at<int32_t>(ws, L.hist));
  MOE_HIP(moe::launch_router(a, at<float>(ws, L.zpart), st), "router");
  MOE_HIP(moe::launch_colsum(at<float>(ws, L.probsum), D.ng, D.E, at<int32_t>(ws, L.blockbase), prob_colsum, st),
          "colsum");
  return MOE_OK;
}

moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, const void* x, int32_t* counts,
                        int32_t* kept, int32_t* offsets, int32_t* dest, int32_t* perm, void* x_perm, void* ws,
                        size_t ws_bytes, moe_stream_t stream) {
  Derived D;
  Layout L;
  MOE_CHECK(check_config(cfg, &D));
  MOE_CHECK(need(topk_idx, 4, "topk_idx"));
  MOE_CHECK(need(x, 16, "x"));
  MOE_CHECK(need(counts, 4, "counts"));
  MOE_CHECK(need(kept, 4, "kept"));
  MOE_CHECK(need(offsets, 4, "offsets"));
  MOE_CHECK(need(dest, 4, "dest"));
  MOE_CHECK(need(perm, 4, "perm"));
  MOE_CHECK(need(x_perm, 16, "x_perm"));
  MOE_CHECK(need_ws(D, ws, ws_bytes, &L));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int32_t* hist = at<int32_t>(ws, L.hist);
  int32_t* blockbase = at<int32_t>(ws, L.blockbase);
  MOE_HIP(moe::launch_histogram(topk_idx, D.T, D.E, D.k, hist, st), "histogram");
  moe::ScanArgs s{};
  s.hist = hist;
  s.ng = D.ng;
  s.E = D.E;
  s.k = D.k;
  s.T = D.T;
  s.C = static_cast<int>(D.C < D.T ? D.C : D.T);
  s.counts = counts;
  s.kept = kept;
  s.offsets = offsets;
  s.blockbase = blockbase;
  MOE_HIP(moe::launch_scan_permute(s, topk_idx, dest, perm, st), "scan + permute");
  MOE_HIP(moe::launch_gather(x, perm, kept, offsets, D.E, D.R, static_cast<int>(D.d * D.esize), x_perm, st),
          "gather");
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* kept, const int32_t* offsets,
                          const void* W1, const void* b1, const void* W2, const void* b2, float* y_perm, void* ws,
                          size_t ws_bytes, moe_stream_t stream) {
  Derived D;
  Layout L;
  MOE_CHECK(check_config(cfg, &D));
  MOE_CHECK(need(x_perm, 16, "x_perm"));
  MOE_CHECK(need(kept, 4, "kept"));
  MOE_CHECK(need(offsets, 4, "offsets"));
  MOE_CHECK(need(W1, 16, "W1"));
  MOE_CHECK(need(b1, D.esize, "b1", true));
  MOE_CHECK(need(W2, 16, "W2"));
  MOE_CHECK(need(b2, D.esize, "b2", true));
  MOE_CHECK(need(y_perm, 16, "y_perm"));
  MOE_CHECK(need_ws(D, ws, ws_bytes, &L));
  moe::FfnArgs a{};
  a.x_perm = x_perm;
  a.kept = kept;
  a.offsets = offsets;
  a.W1 = W1;
  a.b1 = b1;
  a.W2 = W2;
  a.b2 = b2;
  a.H = at<void>(ws, L.H);
  a.y_perm = y_perm;
  a.E = D.E;
  a.d = D.d;
  a.d_ffn = D.dff;
  a.R = D.R;
  a.C = static_cast<int>(D.C < D.T ? D.C : D.T);
  a.bf16 = D.bf16 ? 1 : 0;
  a.side = at<float>(ws, L.side);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  MOE_HIP(moe::launch_expert_ffn(a, st, nullptr), "expert_ffn");
  return MOE_OK;
}

moe_status moe_combine(const moe_config* cfg, const float* y_perm, const int32_t* dest, const float* topk_w,
                       const int32_t* counts, const float* prob_colsum, void* y, float* f, float* P, float* L,
                       void* ws, size_t ws_bytes, moe_stream_t stream) {
  Derived D;
  Layout Lw;
  MOE_CHECK(check_config(cfg, &D));
  MOE_CHECK(need(y_perm, 16, "y_perm"));
  MOE_CHECK(need(dest, 4, "dest"));
  MOE_CHECK(need(topk_w, 4, "topk_w"));
  MOE_CHECK(need(y, 16, "y"));
  const bool stats = f != nullptr || P != nullptr || L != nullptr;
  if (stats) {
    MOE_CHECK(need(f, 4, "f"));
    MOE_CHECK(need(P, 4, "P"));
    MOE_CHECK(need(L, 4, "L"));
    MOE_CHECK(need(counts, 4, "counts"));
    MOE_CHECK(need(prob_colsum, 4, "prob_colsum"));
  }
  MOE_CHECK(need_ws(D, ws, ws_bytes, &Lw));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  MOE_HIP(moe::launch_combine(y_perm, nullptr, dest, topk_w, D.T, D.d, D.k, D.R, D.bf16 ? 1 : 0, y, st),
          "combine");
  if (stats) MOE_HIP(moe::launch_stats(counts, prob_colsum, D.E, D.k, D.T, f, P, L, st), "stats");
  return MOE_OK;
}

namespace {

moe_status forward_impl(const moe_config* cfg, const moe_variant* variant, const void* x, const void* Wg,
                        const float* bg, const void* W1, const void* b1, const void* W2, const void* b2, void* y,
                        float* f, float* P, float* L, int32_t* counts, int32_t* kept, const moe_forward_aux* aux,
                        void* ws, size_t ws_bytes, moe_stream_t stream, bool train = false) {
  Derived D;
  Layout Lw;
  MOE_CHECK(check_config(cfg, &D));
  MOE_CHECK(check_variant(variant, &D));
  D.train = train;
  if (train && D.dffs > 0) return fail(MOE_EUNSUPPORTED, "the backward pass does not cover a shared expert");
  if (train && D.packed) return fail(MOE_EUNSUPPORTED, "training takes the row-major weights");
  if (D.dffs > 0) {
    MOE_CHECK(need(variant->W1s, 16, "W1s"));
    MOE_CHECK(need(variant->b1s, D.esize, "b1s", true));
    MOE_CHECK(need(variant->W2s, 16, "W2s"));
    MOE_CHECK(need(variant->b2s, D.esize, "b2s", true));
  }
  MOE_CHECK(need(x, 16, "x"));
  MOE_CHECK(need(Wg, 16, "Wg"));
  MOE_CHECK(need(bg, 4, "bg", true));
  MOE_CHECK(need(W1, 16, "W1"));
  MOE_CHECK(need(b1, D.esize, "b1", true));
  MOE_CHECK(need(W2, 16, "W2"));
  MOE_CHECK(need(b2, D.esize, "b2", true));
  MOE_CHECK(need(y, 16, "y"));
  MOE_CHECK(need(f, 4, "f"));
  MOE_CHECK(need(P, 4, "P"));
  MOE_CHECK(need(L, 4, "L"));
  MOE_CHECK(need(counts, 4, "counts"));
  MOE_CHECK(need(kept, 4, "kept"));
  moe_forward_aux none{};
  const moe_forward_aux& ax = aux != nullptr ? *aux : none;
  MOE_CHECK(need(ax.logits, 4, "aux.logits", true));
  MOE_CHECK(need(ax.scores, 4, "aux.scores", true));
  MOE_CHECK(need(ax.topk_idx, 4, "aux.topk_idx", true));
  MOE_CHECK(need(ax.topk_w, 4, "aux.topk_w", true));
  MOE_CHECK(need(ax.offsets, 4, "aux.offsets", true));
  MOE_CHECK(need(ax.dest, 4, "aux.dest", true));
  MOE_CHECK(need(ax.perm, 4, "aux.perm", true));
  MOE_CHECK(need(ax.prob_colsum, 4, "aux.prob_colsum", true));
  if (ax.stage_events != nullptr)
    for (int i = 0; i <= MOE_FORWARD_STAGES; ++i)
      if (ax.stage_events[i] == nullptr) return fail(MOE_EINVAL, "aux.stage_events has a NULL event");
  MOE_CHECK(need_ws(D, ws, ws_bytes, &Lw));

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t* ev = reinterpret_cast<hipEvent_t*>(ax.stage_events);
  // training keeps the routing in the workspace for the backward (aux gets copies at the end)
  const bool own = !train;
  float* logits = (own && ax.logits) ? ax.logits : at<float>(ws, Lw.logits);
  const bool has_scores = D.noise != moe::kNoiseNone || D.tau != 1.0f;
  float* scores = (own && ax.scores) ? ax.scores : (has_scores ? at<float>(ws, Lw.scores) : nullptr);
  int32_t* idx = (own && ax.topk_idx) ? ax.topk_idx : at<int32_t>(ws, Lw.idx);
  float* w = (own && ax.topk_w) ? ax.topk_w : at<float>(ws, Lw.w);
  int32_t* offsets = (own && ax.offsets) ? ax.offsets : at<int32_t>(ws, Lw.offsets);
  int32_t* dest = (own && ax.dest) ? ax.dest : at<int32_t>(ws, Lw.dest);
  int32_t* perm = (own && ax.perm) ? ax.perm : at<int32_t>(ws, Lw.perm);
  int32_t* const kept_user = kept;
  float* const f_user = f;
  if (train) {                               // the backward reads kept and f from the workspace
    kept = at<int32_t>(ws, Lw.kept_s);
    f = at<float>(ws, Lw.f_s);
  }
  float* colsum = ax.prob_colsum ? ax.prob_colsum : at<float>(ws, Lw.colsum);
  float* probsum = at<float>(ws, Lw.probsum);
  int32_t* hist = at<int32_t>(ws, Lw.hist);
  int32_t* blockbase = at<int32_t>(ws, Lw.blockbase);
  void* x_perm = at<void>(ws, Lw.x_perm);
  float* y_perm = at<float>(ws, Lw.y_perm);
  const int C = static_cast<int>(D.C < D.T ? D.C : D.T);

  if (ev) MOE_HIP(hipEventRecord(ev[0], st), "event");
  const bool reroute = D.policy == MOE_DROP_REROUTE;
  float* ent = D.stats ? at<float>(ws, Lw.ent) : nullptr;
  int32_t* idx_next = reroute ? at<int32_t>(ws, Lw.idx_next) : nullptr;
  int32_t* kept1 = reroute ? at<int32_t>(ws, Lw.kept1) : kept;
  // 1-2. router: logits, scores, softmax, top-k, weights, block partials (and the next-ranked
  // experts for rerouting, the entropy partials for the statistics)
  moe::RouterArgs ra = router_args(D, x, Wg, bg, logits, scores, idx, w, probsum, hist);
  ra.ent_part = ent;
  ra.idx_next = idx_next;
  MOE_HIP(moe::launch_router(ra, at<float>(ws, Lw.zpart), st), "router");
  if (ev) MOE_HIP(hipEventRecord(ev[1], st), "event");
  // 3a. counts, capacity, offsets, block bases; f, P, L
  moe::ScanArgs s{};
  s.hist = hist;
  s.ng = D.ng;
  s.E = D.E;
  s.k = D.k;
  s.T = D.T;
  s.C = C;
  s.counts = counts;
  s.kept = kept1;
  s.offsets = offsets;
  s.blockbase = blockbase;
  s.probsum_part = probsum;
  s.colsum = colsum;
  s.f = f;
  s.P = P;
  s.L = L;
  s.ent_part = ent;
  s.route_stats = D.stats ? variant->route_stats : nullptr;
  // token order: the permutation follows the scan directly (in the scan kernel itself for small
  // batches); the other policies need their second pass first
  const bool token_order = D.policy != MOE_DROP_RANDOM && !reroute;
  if (token_order)
    MOE_HIP(moe::launch_scan_permute(s, idx, dest, perm, st), "scan + permute");
  else
    MOE_HIP(moe::launch_scan(s, st), "scan");
  if (ev) MOE_HIP(hipEventRecord(ev[2], st), "event");
  // 3a'. capacity policies: the rows the surviving slots take (second scan over them)
  int32_t* hist2 = at<int32_t>(ws, Lw.hist2);
  int32_t* blockbase2 = at<int32_t>(ws, Lw.blockbase2);
  moe::ScanArgs s2{};
  s2.hist = hist2;
  s2.ng = D.ng;
  s2.E = D.E;
  s2.k = D.k;
  s2.T = D.T;
  s2.C = C;
  s2.blockbase = blockbase2;
  if (D.policy == MOE_DROP_RANDOM) {
    uint64_t* thresh = at<uint64_t>(ws, Lw.thresh);
    MOE_HIP(moe::launch_select_random(idx, counts, D.T, D.E, D.k, C, D.key0, D.key1, thresh, st), "select_random");
    MOE_HIP(moe::launch_histogram_kept(idx, thresh, D.T, D.E, D.k, D.key0, D.key1, hist2, st), "histogram_kept");
    s2.bases_only = 1;
    MOE_HIP(moe::launch_scan(s2, st), "scan_kept");
  } else if (reroute) {
    int32_t* cand = at<int32_t>(ws, Lw.cand);
    MOE_HIP(moe::launch_reroute_rank(idx, idx_next, blockbase, D.T, D.E, D.k, C, cand, hist2, st), "reroute_rank");
    s2.base_kept = kept1;
    s2.kept = kept;
    s2.offsets = offsets;
    MOE_HIP(moe::launch_scan(s2, st), "scan_reroute");
  }
  // 3b. stable permutation with the drop mask, then the row gather (unless GEMM1 reads the
  // token rows through the permutation itself)
  moe::FfnArgs fa{};
  fa.x = x;
  fa.T = D.T;
  fa.rows = nullptr;
  if (D.policy == MOE_DROP_RANDOM) {
    MOE_HIP(moe::launch_permute_kept(idx, at<uint64_t>(ws, Lw.thresh), blockbase2, offsets, D.T, D.E, D.k, D.key0,
                                     D.key1, dest, perm, st),
            "permute_kept");
  } else if (reroute) {
    MOE_HIP(moe::launch_permute_reroute(idx, at<int32_t>(ws, Lw.cand), blockbase, blockbase2, kept1, offsets,
                                        scores != nullptr ? scores : logits, D.T, D.E, D.k, C, dest, perm, w, st),
            "permute_reroute");
  }
  // 4. experts
  fa.x_perm = x_perm;
  fa.kept = kept;
  fa.offsets = offsets;
  fa.W1 = W1;
  fa.b1 = b1;
  fa.W2 = W2;
  fa.b2 = b2;
  fa.H = at<void>(ws, Lw.H);
  fa.y_perm = y_perm;
  fa.E = D.E;
  fa.d = D.d;
  fa.d_ffn = D.dff;
  fa.R = D.R;
  fa.C = C;
  fa.bf16 = D.bf16 ? 1 : 0;
  fa.side = at<float>(ws, Lw.side);
  fa.act = D.act;
  fa.w_packed = D.packed ? 1 : 0;
  fa.pre = train ? at<void>(ws, Lw.pre) : nullptr;
  if (moe::ffn_gathers(fa))
    fa.rows = perm;   // GEMM1 reads the token rows of x through the permutation
  else
    MOE_HIP(moe::launch_gather(x, perm, kept, offsets, D.E, D.R, static_cast<int>(D.d * D.esize), x_perm, st),
            "gather");
  if (ev) MOE_HIP(hipEventRecord(ev[3], st), "event");
  MOE_HIP(moe::launch_expert_ffn(fa, st, ev ? ev[4] : nullptr), "expert_ffn");
  // 4b. the shared expert on every token (timed with the second expert GEMM)
  float* y_shared = nullptr;
  if (D.dffs > 0) {
    moe::SharedFfnArgs sa{};
    sa.x = x;
    sa.W1 = variant->W1s;
    sa.b1 = variant->b1s;
    sa.W2 = variant->W2s;
    sa.b2 = variant->b2s;
    sa.H = at<void>(ws, Lw.Hs);
    sa.y = y_shared = at<float>(ws, Lw.ys);
    sa.T = D.T;
    sa.d = D.d;
    sa.d_ffn = D.dffs;
    sa.bf16 = D.bf16 ? 1 : 0;
    sa.act = D.act;
    MOE_HIP(moe::launch_shared_ffn(sa, st), "shared_ffn");
  }
  if (ev) MOE_HIP(hipEventRecord(ev[5], st), "event");
  // 5. combine (each token's float32 sum starts from the shared expert's output, if any; the
  // K parts of GEMM2's split tail tiles were already added by tail_fixup_kernel)
  MOE_HIP(moe::launch_combine(y_perm, y_shared, dest, w, D.T, D.d, D.k, D.R, D.bf16 ? 1 : 0, y, st),
          "combine");
  if (ev) MOE_HIP(hipEventRecord(ev[6], st), "event");
  if (train) {
    const size_t T = D.T, E = D.E, k = D.k;
    auto copy = [&](void* dst, const void* src, size_t bytes) {
      return dst != nullptr ? hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st) : hipSuccess;
    };
    MOE_HIP(copy(kept_user, kept, E * 4), "copy");
    MOE_HIP(copy(f_user, f, E * 4), "copy");
    MOE_HIP(copy(ax.logits, logits, T * E * 4), "copy");
    MOE_HIP(copy(ax.scores, scores != nullptr ? scores : logits, T * E * 4), "copy");
    MOE_HIP(copy(ax.topk_idx, idx, T * k * 4), "copy");
    MOE_HIP(copy(ax.topk_w, w, T * k * 4), "copy");
    MOE_HIP(copy(ax.offsets, offsets, E * 4), "copy");
    MOE_HIP(copy(ax.dest, dest, T * k * 4), "copy");
    MOE_HIP(copy(ax.perm, perm, static_cast<size_t>(D.R) * 4), "copy");
  }
  return MOE_OK;
}

}  // namespace

moe_status moe_forward(const moe_config* cfg, const void* x, const void* Wg, const float* bg, const void* W1,
                       const void* b1, const void* W2, const void* b2, void* y, float* f, float* P, float* L,
                       int32_t* counts, int32_t* kept, const moe_forward_aux* aux, void* ws, size_t ws_bytes,
                       moe_stream_t stream) {
  return forward_impl(cfg, nullptr, x, Wg, bg, W1, b1, W2, b2, y, f, P, L, counts, kept, aux, ws, ws_bytes, stream);
}

moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const void* Wg, const float* bg,
                               const void* W1, const void* b1, const void* W2, const void* b2, void* y, float* f,
                               float* P, float* L, int32_t* counts, int32_t* kept, const moe_forward_aux* aux,
                               moe_stream_t stream) {
  Derived D;
  MOE_CHECK(check_config(cfg, &D));
  const size_t need_bytes = layout_of(D).total;
  if (need_bytes > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_EUNSUPPORTED, "this configuration needs " + std::to_string(need_bytes) +
                                      " bytes of workspace; the static scratch of moe_forward_noalloc holds " +
                                      std::to_string(static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES)));
  void* ws = nullptr;
  MOE_CHECK(scratch_of_current_device(&ws));
  return forward_impl(cfg, nullptr, x, Wg, bg, W1, b1, W2, b2, y, f, P, L, counts, kept, aux, ws,
                      MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_forward_ex(const moe_config* cfg, const moe_variant* variant, const void* x, const void* Wg,
                          const float* bg, const void* W1, const void* b1, const void* W2, const void* b2, void* y,
                          float* f, float* P, float* L, int32_t* counts, int32_t* kept, const moe_forward_aux* aux,
                          void* ws, size_t ws_bytes, moe_stream_t stream) {
  return forward_impl(cfg, variant, x, Wg, bg, W1, b1, W2, b2, y, f, P, L, counts, kept, aux, ws, ws_bytes, stream);
}

moe_status moe_pack_expert_weights(int64_t E, int64_t rows, int64_t cols, const void* W, void* W_packed,
                                   moe_stream_t stream) {
  if (E < 1 || rows < 1 || cols < 1) return fail(MOE_EINVAL, "E, rows and cols must be >= 1");
  if (E > (int64_t{1} << 20) || rows > (int64_t{1} << 20) || cols > (int64_t{1} << 20) ||
      E * rows > (int64_t{1} << 40) / cols)
    return fail(MOE_EINVAL, "E*rows*cols must be below 2^40");
  if (rows % 256 != 0) return fail(MOE_EUNSUPPORTED, "rows must be a multiple of 256");
  if (cols % 32 != 0) return fail(MOE_EUNSUPPORTED, "cols must be a multiple of 32");
  MOE_CHECK(need(W, 16, "W"));
  MOE_CHECK(need(W_packed, 16, "W_packed"));
  const uintptr_t a = reinterpret_cast<uintptr_t>(W), b = reinterpret_cast<uintptr_t>(W_packed);
  const uintptr_t n = static_cast<uintptr_t>(E * rows * cols * 2);
  if (a < b + n && b < a + n) return fail(MOE_EINVAL, "W and W_packed overlap");
  MOE_HIP(moe::launch_pack_weights(W, W_packed, E, rows, cols, reinterpret_cast<hipStream_t>(stream)), "pack");
  return MOE_OK;
}

moe_status moe_probe_copy(const void* src, void* dst, size_t bytes, moe_stream_t stream) {
  if (bytes < 16 || bytes % 16 != 0) return fail(MOE_EINVAL, "bytes must be a positive multiple of 16");
  MOE_CHECK(need(src, 16, "src"));
  MOE_CHECK(need(dst, 16, "dst"));
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return fail(MOE_EINVAL, "src and dst overlap");
  MOE_HIP(moe::launch_probe_copy(src, dst, bytes, reinterpret_cast<hipStream_t>(stream)), "probe_copy");
  return MOE_OK;
}

moe_status moe_probe_mfma(float* out, int64_t workgroups, int64_t iters, moe_stream_t stream) {
  static_assert(MOE_PROBE_CHAINS == 16, "the header's chain count");
  if (moe::probe_mfma_chains() != MOE_PROBE_CHAINS) return fail(MOE_EINVAL, "probe chain count mismatch");
  if (workgroups < 1 || workgroups > (int64_t{1} << 20)) return fail(MOE_EINVAL, "workgroups must be in [1, 2^20]");
  if (iters < 1 || iters > (int64_t{1} << 24)) return fail(MOE_EINVAL, "iters must be in [1, 2^24]");
  MOE_CHECK(need(out, 4, "out"));
  MOE_HIP(moe::launch_probe_mfma(out, static_cast<int>(workgroups), static_cast<int>(iters),
                                 reinterpret_cast<hipStream_t>(stream)),
          "probe_mfma");
  return MOE_OK;
}

moe_status moe_workspace_size_ex(const moe_config* cfg, const moe_variant* variant, size_t* bytes) {
  Derived D;
  MOE_CHECK(check_config(cfg, &D));
  MOE_CHECK(check_variant(variant, &D));
  if (bytes == nullptr) return fail(MOE_EINVAL, "bytes is NULL");
  *bytes = layout_of(D).total;
  return MOE_OK;
}

moe_status moe_workspace_size_train(const moe_config* cfg, const moe_variant* variant, size_t* bytes) {
  Derived D;
  MOE_CHECK(check_config(cfg, &D));
  MOE_CHECK(check_variant(variant, &D));
  if (D.dffs > 0) return fail(MOE_EUNSUPPORTED, "the backward pass does not cover a shared expert");
  if (D.packed) return fail(MOE_EUNSUPPORTED, "training takes the row-major weights");
  if (bytes == nullptr) return fail(MOE_EINVAL, "bytes is NULL");
  D.train = true;
  *bytes = layout_of(D).total;
  return MOE_OK;
}

moe_status moe_forward_train(const moe_config* cfg, const moe_variant* variant, const void* x, const void* Wg,
                             const float* bg, const void* W1, const void* b1, const void* W2, const void* b2, void* y,
                             float* f, float* P, float* L, int32_t* counts, int32_t* kept,
                             const moe_forward_aux* aux, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return forward_impl(cfg, variant, x, Wg, bg, W1, b1, W2, b2, y, f, P, L, counts, kept, aux, ws, ws_bytes, stream,
                      true);
}

moe_status moe_backward(const moe_config* cfg, const moe_variant* variant, const void* x, const void* Wg,
                        const void* W1, const void* W2, const void* dy, float lam, void* dx, float* dWg, float* dbg,
                        float* dW1, float* db1, float* dW2, float* db2, const moe_backward_aux* aux, void* ws,
                        size_t ws_bytes, moe_stream_t stream) {
  Derived D;
  Layout Lw;
  MOE_CHECK(check_config(cfg, &D));
  MOE_CHECK(check_variant(variant, &D));
  if (D.dffs > 0) return fail(MOE_EUNSUPPORTED, "the backward pass does not cover a shared expert");
  if (D.packed) return fail(MOE_EUNSUPPORTED, "training takes the row-major weights");
  if (!std::isfinite(lam)) return fail(MOE_EINVAL, "lam must be finite");
  D.train = true;
  MOE_CHECK(need(x, 16, "x"));
  MOE_CHECK(need(Wg, 16, "Wg"));
  MOE_CHECK(need(W1, 16, "W1"));
  MOE_CHECK(need(W2, 16, "W2"));
  MOE_CHECK(need(dy, 16, "dy"));
  MOE_CHECK(need(dx, 16, "dx"));
  MOE_CHECK(need(dWg, 4, "dWg"));
  MOE_CHECK(need(dbg, 4, "dbg", true));
  MOE_CHECK(need(dW1, 4, "dW1"));
  MOE_CHECK(need(db1, 4, "db1", true));
  MOE_CHECK(need(dW2, 4, "dW2"));
  MOE_CHECK(need(db2, 4, "db2", true));
  moe_backward_aux none{};
  const moe_backward_aux& ax = aux != nullptr ? *aux : none;
  if (ax.stage_events != nullptr)
    for (int i = 0; i <= MOE_BACKWARD_STAGES; ++i)
      if (ax.stage_events[i] == nullptr) return fail(MOE_EINVAL, "aux.stage_events has a NULL event");
  MOE_CHECK(need(ax.dz, 4, "aux.dz", true));
  MOE_CHECK(need_ws(D, ws, ws_bytes, &Lw));

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t* ev = reinterpret_cast<hipEvent_t*>(ax.stage_events);
  const int bf = D.bf16 ? 1 : 0;
  const int C = clamp_c(D);
  const int E = D.E, T = D.T, d = D.d, dff = D.dff, R = D.R;
  const bool has_scores = D.noise != moe::kNoiseNone || D.tau != 1.0f;
  const int32_t* kept = at<int32_t>(ws, Lw.kept_s);
  const int32_t* offsets = at<int32_t>(ws, Lw.offsets);
  const int32_t* perm = at<int32_t>(ws, Lw.perm);
  const int32_t* dest = at<int32_t>(ws, Lw.dest);
  int32_t* koff = at<int32_t>(ws, Lw.koff);
  float* wrow = at<float>(ws, Lw.wrow);
  float* dz = ax.dz != nullptr ? ax.dz : at<float>(ws, Lw.dz);
  void* dA = at<void>(ws, Lw.dA);
  float* dXp = at<float>(ws, Lw.dXp);

  if (ev) MOE_HIP(hipEventRecord(ev[0], st), "event");
  // 1. router backward: dw, the softmax backward and the balance term -> dz; row weights
  moe::BwdRouterArgs ra{};
  ra.dy = dy;
  ra.y_perm = at<float>(ws, Lw.y_perm);
  ra.dest = dest;
  ra.idx = at<int32_t>(ws, Lw.idx);
  ra.cand = D.policy == MOE_DROP_REROUTE ? at<int32_t>(ws, Lw.cand) : nullptr;
  ra.w = at<float>(ws, Lw.w);
  ra.s = has_scores ? at<float>(ws, Lw.scores) : at<float>(ws, Lw.logits);
  ra.f = at<float>(ws, Lw.f_s);
  ra.lam_E_over_T = static_cast<float>(static_cast<double>(lam) * E / T);
  ra.tau = D.tau;
  ra.T = T;
  ra.d = d;
  ra.E = E;
  ra.k = D.k;
  ra.wrow = wrow;
  ra.dz = dz;
  MOE_HIP(moe::launch_bwd_router(ra, bf, st), "bwd_router");
  MOE_HIP(moe::launch_wgrad_offsets(kept, E, koff, st), "wgrad_offsets");
  if (ev) MOE_HIP(hipEventRecord(ev[1], st), "event");
  // 2. off the bf16 MFMA path, the weights transposed: W2 [E,d,dff] -> W2T [E,dff,d] and
  // W1 [E,dff,d] -> W1T [E,d,dff] (the MFMA path reads them as given)
  void* W2T = nullptr;
  void* W1T = nullptr;
  if (moe::bwd_weights_transposed(bf, C)) {
    W2T = at<void>(ws, Lw.W2T);
    W1T = at<void>(ws, Lw.W1T);
    MOE_HIP(moe::launch_transpose(W2, W2T, E, d, dff, bf, st), "transpose W2");
    MOE_HIP(moe::launch_transpose(W1, W1T, E, dff, d, bf, st), "transpose W1");
  }
  if (ev) MOE_HIP(hipEventRecord(ev[2], st), "event");
  // 3. dA = (w dy W2) * act'(a); dXp = dA W1
  moe::BwdDactArgs da{};
  const bool gathers = bwd_gathers(D);
  if (gathers) {
    da.A = dy;
    da.rows = perm;
    da.a_rows = T;
  } else {
    void* dyp = at<void>(ws, Lw.dyp);
    MOE_HIP(moe::launch_gather(dy, perm, kept, offsets, E, R, static_cast<int>(d * D.esize), dyp, st), "gather dy");
    da.A = dyp;
  }
  da.W2 = W2;
  da.W2T = W2T;
  da.wrow = wrow;
  da.pre = at<void>(ws, Lw.pre);
  da.dA = dA;
  da.kept = kept;
  da.offsets = offsets;
  da.E = E;
  da.d = d;
  da.d_ffn = dff;
  da.R = R;
  da.C = C;
  da.bf16 = bf;
  da.act = D.act;
  MOE_HIP(moe::launch_bwd_dact(da, st), "bwd_dact");
  if (ev) MOE_HIP(hipEventRecord(ev[3], st), "event");
  moe::BwdDxArgs dxa{dA, W1, W1T, dXp, bf && C > 16 ? at<float>(ws, Lw.side) : nullptr, kept, offsets, E, d, dff, R, C, bf};
  MOE_HIP(moe::launch_bwd_dx(dxa, st), "bwd_dx");
  if (ev) MOE_HIP(hipEventRecord(ev[4], st), "event");
  // 4. weight gradients: each expert's rows as zero-padded columns, then per-expert products
  const int ld = Lw.ld;
  void* dOT = at<void>(ws, Lw.dOT);
  void* HT = at<void>(ws, Lw.HT);
  void* dAT = at<void>(ws, Lw.dAT);
  void* XT = at<void>(ws, Lw.XT);
  moe::RowsToColsArgs rc{};
  rc.kept = kept;
  rc.offsets = offsets;
  rc.koff = koff;
  rc.E = E;
  rc.ld = ld;
  rc.dst_tiled = moe::wgrad_tiled(bf) ? 1 : 0;
  rc.src = dy, rc.rows = perm, rc.scale = wrow, rc.ncol = d, rc.dst = dOT;
  MOE_HIP(moe::launch_rows_to_cols(rc, bf, st), "rows_to_cols dO");
  rc.src = at<void>(ws, Lw.H), rc.rows = nullptr, rc.scale = nullptr, rc.ncol = dff, rc.dst = HT;
  rc.src_tiled = moe::ffn_h_tiled(bf, C) ? 1 : 0;
  MOE_HIP(moe::launch_rows_to_cols(rc, bf, st), "rows_to_cols H");
  rc.src = dA, rc.rows = nullptr, rc.scale = nullptr, rc.ncol = dff, rc.dst = dAT;   // tiled like H
  MOE_HIP(moe::launch_rows_to_cols(rc, bf, st), "rows_to_cols dA");
  rc.src_tiled = 0;
  rc.src = x, rc.rows = perm, rc.scale = nullptr, rc.ncol = d, rc.dst = XT;
  MOE_HIP(moe::launch_rows_to_cols(rc, bf, st), "rows_to_cols X");
  if (ev) MOE_HIP(hipEventRecord(ev[5], st), "event");
  moe::WgradArgs wa{dOT, HT, dW2, kept, koff, E, d, dff, ld, C, bf};
  MOE_HIP(moe::launch_wgrad(wa, st), "wgrad W2");
  MOE_HIP(moe::launch_zero_empty(dW2, kept, E, static_cast<size_t>(d) * dff, st), "zero W2");
  if (ev) MOE_HIP(hipEventRecord(ev[6], st), "event");
  moe::WgradArgs wb{dAT, XT, dW1, kept, koff, E, dff, d, ld, C, bf};
  MOE_HIP(moe::launch_wgrad(wb, st), "wgrad W1");
  MOE_HIP(moe::launch_zero_empty(dW1, kept, E, static_cast<size_t>(d) * dff, st), "zero W1");
  if (ev) MOE_HIP(hipEventRecord(ev[7], st), "event");
  if (db2 != nullptr) MOE_HIP(moe::launch_segment_rowsum(dOT, kept, koff, E, d, ld, bf, db2, st), "db2");
  if (db1 != nullptr) MOE_HIP(moe::launch_segment_rowsum(dAT, kept, koff, E, dff, ld, bf, db1, st), "db1");
  // 5. router weights and the input gradient
  MOE_HIP(moe::launch_dwg(x, dz, T, d, E, bf, at<float>(ws, Lw.dwg), dWg, dbg, st), "dWg");
  moe::DxArgs xa{dXp, dest, dz, Wg, T, d, E, D.k, dx};
  MOE_HIP(moe::launch_dx(xa, bf, st), "dx");
  if (ev) MOE_HIP(hipEventRecord(ev[8], st), "event");
  return MOE_OK;
}

float moe_temperature_at(int64_t step, float tau0, float tau_min, float rate) {
  const double t = static_cast<double>(tau0) - static_cast<double>(rate) * static_cast<double>(step);
  return static_cast<float>(t > static_cast<double>(tau_min) ? t : static_cast<double>(tau_min));
}

const char* moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: configuration not supported";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
  }
  return "unknown moe_status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
