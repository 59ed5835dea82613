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
#include <type_traits>

#include "moe_common.h"
#include "moe_kernels.h"
#include "tile_plan.h"

namespace moe {

namespace {

struct GemmArgs {
  const void* A;          // [R,K] expert-sorted rows, or [a_rows,K] rows picked by `rows`
  const void* B;          // [E,N,K] weights
  const void* bias;       // [E,N] or null (dtype)
  void* out;              // [R,N]
  const int32_t* kept;    // [E]
  const int32_t* offsets; // [E]
  int E, N, K;
  int R, C;               // rows of A/out and the capacity: segments outside them are skipped
  int splits;             // > 1: the tiles of the last, partial round of 256 are split along K into at
                          // most this many parts (linear epilogue only); see tile_plan.h
  void* out2;             // float side buffer of those parts past the first: dense 256 x 256 tiles
  const int32_t* rows;    // [R] or null: A row of expert-sorted row r is rows[r] (fused gather)
  int a_rows;             // rows of A when `rows` is set (a_rows * K * 2 < 2^31)
  int dense;              // 1: one expert (E = 1) over all R rows; kept and offsets are unused
  // -- training --
  void* pre;              // [R,N] or null: an activation epilogue also stores its input (dtype)
  const float* row_scale; // [R]: activation-gradient epilogues multiply row r by row_scale[r]
  const void* act_in;     // [R,N] dtype: the activation's input at the output positions
  int lda, ldb;           // row pitches of A and B in elements (0: K)
  // wgrad = 1: group e is a dense product over K = kept[e] rounded up to kWgradK, starting at
  // column koff[e] of A [M, lda] and B [N, ldb] (columns past kept[e] hold zeros); its
  // output is the e-th [M, N] block of out. Groups with kept[e] = 0 write nothing.
  int wgrad;
  int M;
  const int32_t* koff;    // [E]
  // K-step-tiled panels (bf16 MFMA path): the rows of each (expert, 256-row tile) form one panel
  // of K/32 contiguous 16 KB blocks, block s holding the panel's 256 rows x columns [32 s, 32 s +
  // 32) in 64-byte rows; panel p = the tile's index in the tile order of all experts' row tiles.
  // A load of one such block covers whole 128-byte lines, where a row-major tile row gives a half.
  // The activation epilogues of the bf16 MFMA kernel always write out in this layout (N = its
  // columns); a_tiled says that A is in it (K = its columns). In the weight-gradient mode A and
  // B are [M, ld] / [N, ld] in the layout of wgrad_tiled (a_tiled, b_tiled): panel = row tile,
  // ld / 32 blocks per panel, and expert e's K steps start at block koff[e] / 32. Outside that
// mode, b_tiled says that B holds packed weights: panel e N/256 + t is rows [256 t, 256 t + 256)
// of expert e's [N, K] matrix (N a multiple of 256), as pack_weights_kernel writes them.
  int a_tiled;
  int b_tiled;
};

// GEMM1 (activation, bf16 or dtype out), GEMM2 (float out), and the backward's
// activation-gradient epilogue: out = acc * row_scale[r] * act'(act_in[r, n]) (dtype out).
enum { kEpiGelu = 0, kEpiLinear = 1, kEpiSilu = 2, kEpiGeluGrad = 3, kEpiSiluGrad = 4 };

constexpr bool is_grad_epi(int epi) { return epi == kEpiGeluGrad || epi == kEpiSiluGrad; }

// The activation of an expert's hidden layer, for results rounded to bf16.
template <int EPI>
__device__ __forceinline__ float activation_bf16(float v) {
  return EPI == kEpiGelu ? gelu_bf16_path(v) : silu_bf16_path(v);
}

template <int EPI>
__device__ __forceinline__ float activation_grad(float v) {
  return EPI == kEpiGeluGrad ? gelu_grad_exact(v) : silu_grad_exact(v);
}

// The derivative for results rounded to bf16 (hardware exp2 and reciprocal).
template <int EPI>
__device__ __forceinline__ float activation_grad_bf16(float v) {
  return EPI == kEpiGeluGrad ? gelu_grad_bf16_path(v) : silu_grad_bf16_path(v);
}

// Rows of expert e's segment; a segment that does not fit [0, R) or exceeds C counts as empty.
// In wgrad mode every group with kept rows has M output rows.
__device__ __forceinline__ int segment_rows(const GemmArgs& g, int e) {
  if (g.wgrad) return (g.kept[e] > 0 && g.kept[e] <= g.C) ? g.M : 0;
  if (g.dense) return e == 0 ? g.R : 0;
  const int m = g.kept[e], o = g.offsets[e];
  return (m > 0 && m <= g.C && o >= 0 && o <= g.R - m) ? m : 0;
}

// Tile t -> (expert, row tile, column tile); column tiles outer, row tiles inner so that the
// workgroups sharing one weight panel are adjacent. Returns false past the last tile.
// `mbase` = row tiles of the experts before e (the panel index of row tile mt is mbase + mt).
__device__ __forceinline__ bool decode_tile(int tile, const GemmArgs& g, int BM, int tiles_n, int& e, int& mt,
                                            int& nt, int& mbase) {
  mbase = 0;
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
    mbase += tm;
  }
  return false;
}

__device__ __forceinline__ float load_bias(const void* bias, size_t i, bool bf16) {
  if (bias == nullptr) return 0.0f;
  return bf16 ? bf16_to_f32(static_cast<const u16*>(bias)[i]) : static_cast<const float*>(bias)[i];
}

// The same tile order for the bf16 kernel without a dependent scalar load per expert: lane l of
// every wave loads expert l's segment (E <= 64), and prefix sums over the wave give each
// expert's first tile and first row tile. A tile's expert is then the first lane whose
// inclusive tile count exceeds it.
struct TileScan {
  int rows;       // segment rows of expert `lane` (0 past E)
  int tm;         // its row tiles
  int cnt_incl;   // tiles of experts 0..lane
  int tm_incl;    // row tiles of experts 0..lane
  int total;      // all tiles (uniform)
  int kept;       // kept[lane] (0 past E or for one dense group)
  int off;        // offsets[lane], or koff[lane] in the weight-gradient mode (0 past E or dense)
};

__device__ __forceinline__ int wave_scan_incl(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ TileScan scan_tiles(const GemmArgs& g, int BM, int tiles_n) {
  const int lane = threadIdx.x & 63;
  TileScan s;
  const bool per_expert = lane < g.E && !g.dense;
  s.kept = per_expert ? g.kept[lane] : 0;
  s.off = per_expert ? (g.wgrad ? g.koff[lane] : g.offsets[lane]) : 0;
  s.rows = lane < g.E ? segment_rows(g, lane) : 0;
  s.tm = (s.rows + BM - 1) / BM;
  s.cnt_incl = wave_scan_incl(s.tm * tiles_n);
  s.tm_incl = wave_scan_incl(s.tm);
  s.total = __builtin_amdgcn_readlane(s.cnt_incl, 63);
  return s;
}

// Tile t < total -> (e, mt, nt, mbase) and e's segment rows. Experts come in order, each
// expert's tiles in the order of plan::tile_in_expert (blocks of 4 column tiles, row tiles outer
// and column tiles inner within a block).
__device__ __forceinline__ void locate_tile(const TileScan& s, int tile, int tiles_n, int& e, int& mt, int& nt,
                                            int& mbase, int& m_e) {
  const unsigned long long past = __ballot(s.cnt_incl > tile);
  e = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(past)));
  const int tm = __builtin_amdgcn_readlane(s.tm, e);
  const int t = tile - (__builtin_amdgcn_readlane(s.cnt_incl, e) - tm * tiles_n);
  plan::tile_in_expert(t, tm, tiles_n, mt, nt);
  mbase = __builtin_amdgcn_readlane(s.tm_incl, e) - tm;
  m_e = __builtin_amdgcn_readlane(s.rows, e);
}

// Tile order, placement over the XCDs and the K split of the last, partial round: tile_plan.h.
constexpr int kTailMaxParts = plan::kMaxParts;
constexpr size_t kTailTile = 256 * 256;            // floats per side-buffer tile

// Workgroups of a launch over at most n_max tiles (max_parts > 1: with the tail split).
int plan_grid(int n_max, int max_parts) { return plan::grid_bound(n_max, max_parts); }

// s_waitcnt with only vmcnt limited (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over [base, base + bytes): stride 0, dword 3 = 0x00020000 (32-bit data
// format, the gfx9 raw-buffer setting); offsets at or past `bytes` read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, 0x00020000);
}

// One 16-byte buffer -> LDS load per lane (buffer_load_dwordx4 ... lds): lane i reads
// base + voff_i and writes bytes [16 i, 16 i + 16) of the wave's 1 KB block at `lds` (which
// must be the same for every lane; it goes to M0).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 at LDS address p (8-byte aligned).
__device__ __forceinline__ v4i16 ds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(const_cast<char*>(p)));
}

// Slot of logical 16-byte chunk c of tile row r (64-byte rows) in LDS: c ^ chunk_swizzle(r).
// The fragment reads of one instruction cover 16 consecutive rows at one logical chunk (lane
// group lg reads chunk lg). Measured with SQ_LDS_BANK_CONFLICT, a swizzle on (r / 4) mod 4
// doubles the LDS cycles of these reads, and (r / 2) mod 4 makes them conflict-free.
__device__ __forceinline__ int chunk_swizzle(int r) { return (r >> 1) & 3; }

// Chunk swizzle of the N-contiguous B tile's k-row kr: even, so chunk pairs stay together, and
// distinct over the 8 rows {u, 8 + u} (u < 4) that one half-wave of a transpose read covers.
__device__ __forceinline__ int bnm_swizzle(int kr) { return 2 * ((kr & 3) | (((kr >> 3) & 1) << 2)); }

// acc += A_blk B_blk^T on one 16x16x32 bf16 block, operands given B first (so acc holds the
// transposed block), with acc tied to its AGPRs; FIRST starts from zero (srcC = 0).
template <bool FIRST>
__device__ __forceinline__ void mfma_16x16x32(floatx4& acc, const bf16x8& b, const bf16x8& a) {
  if constexpr (FIRST)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(b), "v"(a));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}

// load_lds16 written as inline asm, for kernels that read LDS with ds_read_b64_tr_b16: the
// compiler makes every such read wait for all buffer -> LDS loads in flight (vmcnt(0)), which
// would drain the operand prefetch on every fragment read. Issued as asm, the loads are
// invisible to that rule; the kernel orders them itself, as it does for the builtin's loads
// (vmcnt waits before the barrier that publishes a stage). The resource is built by hand in
// the layout buffer_rsrc gives (stride 0, num_records = bytes, dword 3 = 0x00020000); base,
// bytes and the LDS target must be wave-uniform.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load_lds16_asm(const char* base, int bytes, uint32_t voff, void* lds) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const i32x4 rsrc = {__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b))),
                      __builtin_amdgcn_readfirstlane(static_cast<int>((b >> 32) & 0xffff)),
                      __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
  const int m0 = __builtin_amdgcn_readfirstlane(
      static_cast<int>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)(lds))));
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(m0)
               : "memory", "m0");
}

// Workgroup barrier without the LDS-read wait that __syncthreads adds: the callers order
// their own LDS traffic (vmcnt waits for the direct loads, register dependences for reads).
__device__ __forceinline__ void barrier_no_lds_wait() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------------------
// bf16 grouped GEMM C[r, n] = sum_k A[r, k] B_e[n, k] over each expert's row segment.
// 256 x 256 workgroup tile, 4 waves in a 2x2 grid of 128 x 128 wave tiles, each an 8x8 grid of
// v_mfma_f32_16x16x32_bf16 blocks (256 accumulators per lane); a forward tile with at most 128
// segment rows runs WIDE instead, the 4 waves side by side over rows 0..127 (128 x 64 each). The 16x16x32 form moves a quarter
// of the accumulator data per flop that 32x32x16 does and runs at a higher clock under load.
// The MFMAs are written as inline asm with each accumulator tied to one AGPR quad (destination
// = srcC): left to itself the compiler shuffles these 64 accumulators between register files.
// Operand tiles go from global
// memory straight into LDS (buffer_load_dwordx4 ... lds: 64 lanes fill one contiguous 1 KB
// block; per-lane offsets are fixed, the K step moves the resource base in scalar registers)
// through a ring of NS K-steps of BK; the 16-byte chunks of each row are XOR-swizzled
// (chunk_swizzle) so that the 16-byte fragment reads run without bank conflicts.
// The workgroup barrier opens each K step s: after it, step s+1 is complete in LDS (its
// fragments are read during step s's MFMAs) and the buffer of step s-1 is free for step
// s+NS-1, so NS-3 steps of loads stay in flight while waiting.
// Loads past the last K step re-read the last step into buffers nobody reads again, which keeps
// the number of loads in flight the same in every iteration.
// Rows past the segment (or past N) are loaded from the last valid row: they only feed output
// rows (columns) that are never stored.
// BNM: B is N-contiguous, [E][K][N] (the layout of the forward weights seen from the backward's
// products). Each K step's B tile is then 32 k-rows of 256 columns (512-byte rows, two whole rows
// per 1 KB wave load), its 16-byte chunks XOR-swizzled by bnm_swizzle(k), and the fragments come
// from ds_read_b64_tr_b16: in each 16-lane group, lane 4u + q names 4 consecutive elements of row
// u of a 4 x 16 block and lane i receives column i of the block (one element from each of the
// 4 rows), so two such reads give a lane the 8 consecutive k of its column that the MFMA takes.
// Columns past N read neighbouring data or zeros and feed only outputs that are never stored.
// PAIR = 1 (row-major A, not tiled) or 2 (row-major B): that operand is staged by K-step pairs.
// Each of its rows' 128 bytes of steps 2q and 2q+1 are one LDS row of pair buffer q mod 3 (three
// 32 KB buffers), so a 1 KB wave load covers 8 rows x 128 bytes, whole lines, where a one-step
// stage takes 16 half lines; the 16-byte chunks of a 128-byte row are swizzled by row mod 8
// (conflict-free for the fragment reads, measured). The other operand keeps its NS-step ring
// after the pair buffers (96 + 64 KB of LDS). Step s issues that operand's loads of step s+3
// and, when s is even, the paired operand's loads of pair s/2 + 2, so every step's wait is
// vmcnt <= 12.
template <int EPI, int BK, int NS, bool BNM = false, int PAIR = 0>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(GemmArgs g) {
  constexpr int BM = 256, BN = 256;
  constexpr int CPR = BK / 8;                // 16-byte chunks per tile row
  constexpr int RPI = 64 / CPR;              // tile rows per 1 KB wave load
  constexpr int ROWB = BK * 2;               // bytes per tile row
  constexpr int TILE = BM * ROWB;            // bytes of the A (or B) tile of one K step
  constexpr int STAGE = 2 * TILE;
  constexpr int LOADS = BM / RPI / 4;        // 1 KB loads per wave per operand per K step
  constexpr int PER_STAGE = 2 * LOADS;       // vm operations per thread per K step
  constexpr bool AP = PAIR == 1, BP = PAIR == 2;
  constexpr int PAIRB = 2 * ROWB;            // paired: bytes of a row of a K-step pair
  constexpr int APAIR = BM * PAIRB;          // paired: bytes of a pair buffer
  constexpr int NPA = 3;                     // paired: pair buffers
  constexpr int RING = NPA * APAIR;          // paired: start of the other operand's ring
  constexpr int SMEM = PAIR ? RING + NS * TILE : NS * STAGE;
  static_assert(NS >= 3 && SMEM <= 160 * 1024, "LDS ring");
  static_assert(!PAIR || NS == 4, "the pair schedule assumes loads three steps ahead");
  static_assert(!(BP && BNM), "N-major B has its own staging");
  static_assert(BK == 32, "one v_mfma_f32_16x16x32_bf16 K step per K step");
  static_assert(PER_STAGE == 8, "one operand load per 16-row MFMA block");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tiles_n = (g.N + BN - 1) / BN;
  const TileScan scan = scan_tiles(g, BM, tiles_n);
  plan::Unit unit;
  if (!plan::unit_of(blockIdx.x, scan.total, g.K / BK, EPI == kEpiLinear && !g.wgrad ? g.splits : 1, unit)) return;
  // uniform by construction; said so, so that the buffer resources stay in scalar registers
  const int tile = __builtin_amdgcn_readfirstlane(unit.tile);
  const int kpart = __builtin_amdgcn_readfirstlane(unit.kpart);
  const int parts = __builtin_amdgcn_readfirstlane(unit.parts);
  const int side_slot = __builtin_amdgcn_readfirstlane(unit.side);
  int e, mt, nt, mbase, m_e;
  locate_tile(scan, tile, tiles_n, e, mt, nt, mbase, m_e);
  const int panel = __builtin_amdgcn_readfirstlane(mbase + mt);   // K-step-tiled layouts
  mt = __builtin_amdgcn_readfirstlane(mt);
  nt = __builtin_amdgcn_readfirstlane(nt);
  const int row0 = (g.dense || g.wgrad) ? 0 : __builtin_amdgcn_readlane(scan.off, e);
  const int m0 = mt * BM, n0 = nt * BN;
  const int N = g.N;
  const int lda = g.lda ? g.lda : g.K, ldb = g.ldb ? g.ldb : g.K;
  const int K = g.wgrad ? (__builtin_amdgcn_readlane(scan.kept, e) + kWgradK - 1) / kWgradK * kWgradK : g.K;
  const size_t kofs = g.wgrad ? static_cast<size_t>(__builtin_amdgcn_readlane(scan.off, e)) : 0;
  int kf, kl;
  plan::part_range(K / BK, kpart, parts, kf, kl);   // pair-aligned: K / BK is even here
  const int k_first = __builtin_amdgcn_readfirstlane(kf);
  const int k_last = __builtin_amdgcn_readfirstlane(kl);
  const int nk = k_last - k_first;           // K steps of this part
  const bool gathered = g.rows != nullptr;
  const bool a_tiled = g.a_tiled != 0;
  const bool b_tiled = !BNM && g.b_tiled != 0;
  // tiled operands: panel index, blocks per panel and the first block of this tile's K range
  const size_t a_blk0 = g.wgrad ? (static_cast<size_t>(mt) * (lda / BK) + kofs / BK)
                                : static_cast<size_t>(panel) * (g.K / BK);
  const char* Ab = a_tiled ? static_cast<const char*>(g.A) + (a_blk0 + k_first) * TILE
                           : reinterpret_cast<const char*>(static_cast<const u16*>(g.A) + kofs +
                                                           (gathered ? 0 : static_cast<size_t>(row0 + m0) * lda)) +
                                 static_cast<size_t>(k_first) * ROWB;
  const char* Bb = BNM ? reinterpret_cast<const char*>(static_cast<const u16*>(g.B) +
                                                      (static_cast<size_t>(e) * g.K + static_cast<size_t>(k_first) * BK) * N + n0)
                  : b_tiled ? static_cast<const char*>(g.B) + ((g.wgrad ? static_cast<size_t>(nt)
                                                           : static_cast<size_t>(e) * tiles_n + nt) * (ldb / BK) +
                                                  kofs / BK + k_first) * TILE
                      : reinterpret_cast<const char*>(static_cast<const u16*>(g.B) + kofs +
                                                      (g.wgrad ? static_cast<size_t>(n0) * ldb
                                                               : (static_cast<size_t>(e) * N + n0) * ldb)) +
                            static_cast<size_t>(k_first) * ROWB;
  const size_t out_base = g.wgrad ? static_cast<size_t>(e) * g.M * N : 0;   // elements
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets stay scalar

  // direct loads: wave w fills 1 KB blocks w, w+4, ... of each operand tile
  const int lrow = lane / CPR, lslot = lane % CPR;
  uint32_t aoff[AP ? 8 : LOADS], boff[BP ? 8 : LOADS];
  const int a_last = m_e - 1 - m0, b_last = N - 1 - n0;
  if constexpr (AP) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // wave w's A load j of a pair: 1 KB block w + 4 j = rows 8 (w + 4 j) .. +7 of the pair buffer;
      // lane l fills slot l mod 8 of row l / 8 with logical chunk (slot ^ row mod 8)
      const int r = 8 * (wave + 4 * j) + (lane >> 3), c = (lane & 7) ^ (r & 7);
      const int ra = r < a_last ? r : a_last;
      const uint32_t arow = gathered ? static_cast<uint32_t>(g.rows[row0 + m0 + ra]) : static_cast<uint32_t>(ra);
      aoff[j] = static_cast<uint32_t>((arow * lda + c * 8) * 2);
    }
  }
  if constexpr (BP) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {   // as for A above, over B's rows
      const int r = 8 * (wave + 4 * j) + (lane >> 3), c = (lane & 7) ^ (r & 7);
      const uint32_t rb = static_cast<uint32_t>(r < b_last ? r : b_last);
      boff[j] = (rb * ldb + c * 8) * 2;
    }
  }
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int r = (wave + 4 * i) * RPI + lrow;
    const int c = lslot ^ chunk_swizzle(r);
    const int ra = r < a_last ? r : a_last;
    if constexpr (!AP) {
      const uint32_t arow = gathered ? static_cast<uint32_t>(g.rows[row0 + m0 + ra]) : static_cast<uint32_t>(ra);
      aoff[i] = a_tiled ? static_cast<uint32_t>(ra * ROWB + c * 16) : static_cast<uint32_t>((arow * lda + c * 8) * 2);
    }
    if constexpr (BNM) {
      const int kr = 2 * (wave + 4 * i) + (lane >> 5);     // k-row of the step's B tile
      boff[i] = static_cast<uint32_t>(kr * N * 2 + (((lane & 31) ^ bnm_swizzle(kr)) * 16));
    } else if constexpr (!BP) {
      const uint32_t rb = static_cast<uint32_t>(r < b_last ? r : b_last);
      boff[i] = b_tiled ? rb * ROWB + c * 16 : (rb * ldb + c * 8) * 2;
    }
  }
  // the clamped offsets stay below 256 rows of the pitch past the B resource base and below
  // the tile's (or, gathered, all of A's) rows past the A base; anything beyond reads as zero
  const int span = BNM ? (BK * N - n0) * 2 : b_tiled ? TILE : BM * ldb * 2;
  const int span_a = a_tiled ? TILE : gathered ? g.a_rows * lda * 2 : BM * lda * 2;
  const size_t b_step = BNM ? static_cast<size_t>(BK) * N * 2 : b_tiled ? TILE : ROWB;   // bytes per K step of B
  // LDS start of step st's A and B tiles (of its pair's buffer for the paired operand)
  auto a_stage = [&](int st) {
    return AP ? ((st >> 1) % NPA) * APAIR : BP ? RING + (st % NS) * TILE : (st % NS) * STAGE;
  };
  auto b_stage = [&](int st) {
    return BP ? ((st >> 1) % NPA) * APAIR : AP ? RING + (st % NS) * TILE : (st % NS) * STAGE + TILE;
  };
  auto load = [&](const char* base, int bytes, uint32_t voff, char* lds) {
    if constexpr (BNM)
      load_lds16_asm(base, bytes, voff, lds);
    else
      load_lds16(buffer_rsrc(base, bytes), voff, lds);
  };
  // load q (0..7) of K step min(st, nk-1): A blocks 0..3, then B blocks (not the paired operand)
  auto issue1 = [&](int st, int q) {
    const uint32_t ks = static_cast<uint32_t>(st < nk ? st : nk - 1);
    if (!AP && q < LOADS)
      load(Ab + ks * (a_tiled ? TILE : ROWB), span_a, aoff[q], smem + a_stage(st) + wave * 1024 + q * 4096);
    else if (!BP && q >= LOADS)
      load(Bb + ks * b_step, span, boff[q - LOADS], smem + b_stage(st) + wave * 1024 + (q - LOADS) * 4096);
  };
  // paired operand: load j (0..7) of pair min(pq, last pair) into buffer pq mod 3
  auto issue_pair = [&](int pq, int j) {
    const int last = (nk - 1) >> 1;
    const uint32_t qq = static_cast<uint32_t>(pq < last ? pq : last);
    char* dst = smem + (pq % NPA) * APAIR + (wave + 4 * j) * 1024;
    if constexpr (AP)
      load(Ab + qq * PAIRB, span_a, aoff[j], dst);
    else
      load(Bb + qq * PAIRB, span, boff[j], dst);
  };

  // fragment addressing: lane (l16, lg) reads row (wave-tile row + 16 i + l16), 16-byte chunk lg
  // of the step's 64 bytes: the 8 K values an operand lane holds in v_mfma_f32_16x16x32_bf16
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lg = lane >> 4;
  const int slot = (lg ^ chunk_swizzle(l16)) * 16;   // rows 16 i + l16: same swizzle as row l16
  // Wave tiles: a 2 x 2 grid of 128 x 128 (rows wm*128.., columns wn*128..), or, on a WIDE tile
  // (at most 128 segment rows), rows 0..127 and columns wave*64.. for every wave, so that all
  // four SIMDs multiply where the 2 x 2 grid would leave the lower two waves without rows.
  auto wave_rows = [&](auto wide) { return decltype(wide)::value ? 0 : wm * 128; };
  auto wave_cols = [&](auto wide) { return decltype(wide)::value ? wave * 64 : wn * 128; };
  // BNM transpose reads: lane (group lg, 4u + q) reads k-rows 8 lg + 4 h + u of block j at the
  // 8 bytes of columns wn*128 + 16 j + 4 q; the swizzle depends on u and lg only (not on h)
  const int tr_u = (lane & 15) >> 2, tr_q = lane & 3;
  const int tr_sw = bnm_swizzle(8 * lg + tr_u);
  const int b_tr = (8 * lg + tr_u) * 512 + (16 * wn + (tr_q >> 1)) * 16 + 8 * (tr_q & 1);
  floatx4 acc[8][8];

  // Epilogue. The MFMAs take the B fragment as their first operand, so block (i, j) holds the
  // transposed 16x16 result: lane (l16, lg) has tile row wm*128 + 16 i + l16 at columns
  // wn*128 + 16 j + 4 lg + (0..3), four consecutive outputs of one row. Bias and GeLU are
  // applied in registers; each 32x128 row block (MFMA rows 2 ib, 2 ib + 1) then goes through the wave's own
  // LDS region (8-byte bf16 or 16-byte float pieces) and back out as whole rows: 16 lanes
  // (bf16) or 32 lanes (float) store each row's 256 or 512 contiguous bytes, so every store
  // covers whole cache lines. N is a multiple of 64, so each 16-byte piece lies wholly inside
  // or outside [0, N). Only the NI row blocks the wave multiplied can hold segment rows.
  auto epilogue = [&](auto ni_const, auto bias_const, auto pre_const, auto wide_const) {
    constexpr int NI = decltype(ni_const)::value;
    constexpr bool BIAS = decltype(bias_const)::value;
    constexpr bool PRE = decltype(pre_const)::value;       // also store the activation's input
    constexpr bool WIDE = decltype(wide_const)::value;
    constexpr int WC = WIDE ? 64 : 128;                    // columns of the wave tile
    constexpr int NJ = WC / 16;                            // its 16-column MFMA blocks
    const int rbase = wave_rows(wide_const), cbase = wave_cols(wide_const);
    constexpr int OB = EPI == kEpiLinear ? 4 : 2;         // output bytes per element
    constexpr int PITCH = 128 * OB + 16;                   // bytes per staged row (padded)
    constexpr int CPRW = WC * OB / 16;                     // 16-byte pieces per row
    constexpr int RPW = 64 / CPRW;                         // rows per wave store
    static_assert((EPI == kEpiLinear ? 4 : 8) * 32 * PITCH <= NS * STAGE, "epilogue staging fits the operand ring");
    static_assert(4 * 32768 <= NS * STAGE, "the gradient epilogue's act_in blocks fit the operand ring");
    char* st = smem + wave * 32 * PITCH;
    char* st2 = smem + (4 + wave) * 32 * PITCH;            // staged inputs of the activation
    // the tile's output block and its row pitch: the output (part 0) or a side-buffer tile
    const bool side = EPI == kEpiLinear && kpart > 0;
    char* outb = side ? static_cast<char*>(g.out2) + static_cast<size_t>(side_slot) * kTailTile * 4
                      : static_cast<char*>(g.out) + (out_base + static_cast<size_t>(row0 + m0) * N + n0) * OB;
    const size_t pitch = side ? 256 : static_cast<size_t>(N);
    __syncthreads();                                       // every wave is done with the ring
    // whole-row pieces of the wave's row block: LDS <-> global, 16 bytes per lane (float outputs,
    // read once by the next kernel, go out as non-temporal stores)
    auto rows_out = [&](const char* stage, char* base, size_t bpitch, int i) {
#pragma unroll
      for (int it = 0; it < 32 / RPW; ++it) {
        const int rr = it * RPW + lane / CPRW, pc = lane % CPRW;
        const int rl = rbase + i * 32 + rr;
        const int cl = cbase + pc * (16 / OB);
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + rr * PITCH + pc * 16);
        if (m0 + rl < m_e && n0 + cl < N) {
          u32x4* dst = reinterpret_cast<u32x4*>(base + (static_cast<size_t>(rl) * bpitch + cl) * OB);
          if constexpr (EPI == kEpiLinear)
            __builtin_nontemporal_store(v, dst);
          else
            *dst = v;
        }
      }
    };
    // the same block into K-step-tiled panel `panel` of out: its 4 column chunks of 32 go to
    // blocks (n0 + wn*128)/32 + j, 32 rows x 64 bytes each, two 1 KB stores per chunk. Lane
    // (row rr, piece pc) with rr running fastest: 8 consecutive lanes read 8 staged rows, whose
    // pitch puts them on distinct banks. The stores are non-temporal: H is read back only by the
    // next kernel, and as ordinary stores its dirty lines were still being written back while
    // that kernel ran (GEMM2 -8% on the switch-style layer, GEMM1 -2% on the long-tail one).
    auto rows_out_tiled = [&](const char* stage, int i) {
      char* pbase = static_cast<char*>(g.out) + static_cast<size_t>(panel) * (N / BK) * TILE;
#pragma unroll
      for (int it = 0; it < WC / 16; ++it) {
        const int j = it >> 1, rr = 16 * (it & 1) + (lane & 15), pc = lane >> 4;
        const int rl = rbase + i * 32 + rr;                // row within the tile = row of the panel
        const int cb = n0 + cbase + 32 * j;                // first column of the chunk
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + rr * PITCH + (32 * j + 8 * pc) * OB);
        if (m0 + rl < m_e && cb < N)
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(pbase + static_cast<size_t>(cb / BK) * TILE +
                                                                  rl * ROWB + pc * 16));
      }
    };
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int rl = 16 * h + l16;                      // row within the 32-row block
          const int cl = j * 16 + 4 * lg;                   // column within the wave tile
          float o[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)   // one addition either way: GeLU then needs no canonicalisation
            o[u] = acc[2 * i + h][j][u] +
                   (BIAS ? load_bias(g.bias, static_cast<size_t>(e) * N + min(n0 + cbase + cl + u, N - 1), true)
                         : 0.0f);
          char* dst = st + rl * PITCH + cl * OB;
          if constexpr (EPI != kEpiLinear) {
            bf16x4 pk;
#pragma unroll
            for (int u = 0; u < 4; ++u) pk[u] = static_cast<__bf16>(activation_bf16<EPI>(o[u]));
            *reinterpret_cast<bf16x4*>(dst) = pk;
            if constexpr (PRE) {
              bf16x4 pv;
#pragma unroll
              for (int u = 0; u < 4; ++u) pv[u] = static_cast<__bf16>(o[u]);
              *reinterpret_cast<bf16x4*>(st2 + rl * PITCH + cl * OB) = pv;
            }
          } else {
            *reinterpret_cast<floatx4*>(dst) = floatx4{o[0], o[1], o[2], o[3]};
          }
        }
      // the wave reads back only what it wrote itself: LDS keeps one wave's accesses in order
      if constexpr (EPI != kEpiLinear)
        rows_out_tiled(st, i);
      else
        rows_out(st, outb, pitch, i);
      if constexpr (PRE && EPI != kEpiLinear)
        rows_out(st2, static_cast<char*>(g.pre) + (static_cast<size_t>(row0 + m0) * N + n0) * OB, N, i);
      __builtin_amdgcn_sched_barrier(0);   // one row block at a time: bounded register use
    }
  };

  // Activation-gradient epilogue: out = acc * row_scale[r] * act'(act_in[r, n]), bf16. Each
  // wave's act_in block (NI row blocks of 32 x 128 bf16) goes straight into the free operand
  // ring with buffer -> LDS loads, all issued at once (32 KB per wave, 8 KB per row block,
  // rows of 256 bytes whose 16-byte pieces are XOR-swizzled by row so that the fragment-order
  // reads spread over the banks). Each lane then overwrites its own inputs with its outputs in
  // place, and the block goes out as whole rows. Rows past the segment read as zero (the
  // resource ends at the last valid row) and are never stored.
  auto grad_epilogue = [&](auto ni_const) {
    constexpr int NI = decltype(ni_const)::value;
    char* region = smem + wave * 32768;
    __syncthreads();                                       // every wave is done with the ring
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rb = m0 + wm * 128 + i * 32;              // first tile row of the block
      // uniform by construction; said so, so that the buffer resource stays in scalar registers
      const int valid_rows = __builtin_amdgcn_readfirstlane(max(0, min(32, m_e - rb)));
      const char* base = static_cast<const char*>(g.act_in) +
                         (static_cast<size_t>(row0 + rb) * N + n0 + wn * 128) * 2;
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, valid_rows * N * 2);
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int rr = 4 * it + lane / 16, pp = lane % 16;
        const uint32_t off = static_cast<uint32_t>(rr * N * 2 + ((pp ^ (rr % 16)) * 16));
        load_lds16(rs, off, region + i * 8192 + it * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // this block's loads are older than every later block's 8 (the stores issued since are
      // younger still, so the wait can only be stricter than needed)
      if (i == 0) wait_vmcnt<(NI > 1 ? 8 * (NI - 1) : 0)>();
      else if (i == 1) wait_vmcnt<(NI > 2 ? 8 * (NI - 2) : 0)>();
      else if (i == 2) wait_vmcnt<(NI > 3 ? 8 : 0)>();
      else wait_vmcnt<0>();
      char* blk = region + i * 8192;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rl = 16 * h + l16;                        // row within the block; rl % 16 = l16
        const int r = min(m0 + wm * 128 + i * 32 + rl, m_e - 1);
        const float scale = g.row_scale[row0 + r];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // columns 16 j + 4 lg .. + 3: 16-byte piece 2 j + lg / 2, half lg % 2
          char* pa = blk + rl * 256 + (((2 * j + (lg >> 1)) ^ l16) * 16) + 8 * (lg & 1);
          const bf16x4 a = *reinterpret_cast<const bf16x4*>(pa);
          bf16x4 pk;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            pk[u] = static_cast<__bf16>(acc[2 * i + h][j][u] * scale *
                                        activation_grad_bf16<EPI>(static_cast<float>(a[u])));
          *reinterpret_cast<bf16x4*>(pa) = pk;
        }
      }
      // out (dA) goes to K-step-tiled panel `panel`, as H does: chunk j (32 columns) of the
      // block is 32 rows x 64 bytes at block (n0 + wn*128)/32 + j, two 1 KB stores per chunk;
      // 16 lanes with one piece read 16 rows whose swizzle spreads them over the banks
      char* pbase = static_cast<char*>(g.out) + static_cast<size_t>(panel) * (N / BK) * TILE;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int j = it >> 1, rr = 16 * (it & 1) + (lane & 15), pc = lane >> 4;
        const int rl = wm * 128 + i * 32 + rr;             // row within the tile = row of the panel
        const int cb = n0 + wn * 128 + 32 * j;
        const u32x4 v = *reinterpret_cast<const u32x4*>(blk + rr * 256 + (((4 * j + pc) ^ (rr % 16)) * 16));
        if (m0 + rl < m_e && cb < N)
          *reinterpret_cast<u32x4*>(pbase + static_cast<size_t>(cb / BK) * TILE + rl * ROWB + pc * 16) = v;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const bool add_bias = kpart == 0 && g.bias != nullptr;

  // The wave multiplies only the 32-row blocks of its 128 rows that hold segment rows (2 or 4
  // of them; rows past the segment are never stored). Every wave still issues its share of
  // the loads and takes every barrier.
  auto mainloop = [&](auto ni_const, auto wide_const) {
    constexpr int NI = decltype(ni_const)::value;
    constexpr int NR = 2 * NI;                         // 16-row MFMA blocks multiplied
    constexpr bool WIDE = decltype(wide_const)::value;
    constexpr int NJ = WIDE ? 4 : 8;                   // 16-column MFMA blocks of the wave tile
    const int rbase = wave_rows(wide_const), cbase = wave_cols(wide_const);
    const int a_frag = (rbase + l16) * ROWB + slot;
    const int a_frag_ap = (rbase + l16) * PAIRB;       // paired A: row of the pair buffer; swizzle l16 mod 8
    const int b_frag_bp = (cbase + l16) * PAIRB;       // paired B
    const int b_frag = (cbase + l16) * ROWB + slot;
    // A fragments single-buffered (row i's next one is read once row i's MFMAs are issued), B
    // fragments double-buffered by step parity (the next ones are read during rows 0..NJ/2-1)
    bf16x8 fa[8], fb[2][8];
    auto rd_a = [&](int st, int i) {
      if constexpr (AP)
        fa[i] = *reinterpret_cast<const bf16x8*>(smem + a_stage(st) + a_frag_ap + i * 16 * PAIRB +
                                                 (((4 * (st & 1) + lg) ^ (l16 & 7)) * 16));
      else
        fa[i] = *reinterpret_cast<const bf16x8*>(smem + a_stage(st) + a_frag + i * 16 * ROWB);
    };
    auto rd_b = [&](int st, int f, int j) {
      if constexpr (BNM) {
        const char* p = smem + b_stage(st) + b_tr + (((2 * j) ^ tr_sw) * 16);
        const v4i16 lo = ds_read_tr16(p), hi = ds_read_tr16(p + 4 * 512);
        fb[f][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else if constexpr (BP) {
        fb[f][j] = *reinterpret_cast<const bf16x8*>(smem + b_stage(st) + b_frag_bp + j * 16 * PAIRB +
                                                    (((4 * (st & 1) + lg) ^ (l16 & 7)) * 16));
      } else {
        fb[f][j] = *reinterpret_cast<const bf16x8*>(smem + b_stage(st) + b_frag + j * 16 * ROWB);
      }
    };
    // K step s: barrier, then per 16-row block i one operand load of step s+NS-1, the block's 8
    // MFMAs on fragments of step s, and reads of step s+1's fragments. FIRST: srcC = 0.
    auto step = [&](int s, auto f_const, auto first_const) {
      constexpr int F = decltype(f_const)::value;
      constexpr bool FIRST = decltype(first_const)::value;
      // this thread's loads of step s+1 have landed (paired: the loads issued after the other
      // operand's of step s+1 are the pair's of (s-2)/2 + 2 when s is even, then step s-1's: 12
      // either way)
      wait_vmcnt<PAIR ? 12 : (NS - 3) * PER_STAGE>();
      // Everyone's have, and step s-1's buffer is free: every wave consumed its reads of step
      // s-1 (issued during step s-2) in the MFMAs it ran before arriving here. Paired: pair
      // (s-2)/2's buffer is free at an even step s, which refills it with pair s/2 + 2.
      barrier_no_lds_wait();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (PAIR) {
          if (i < 4) {
            issue1(s + NS - 1, AP ? LOADS + i : i);
          } else if (F == 0) {
            issue_pair((s >> 1) + 2, 2 * (i - 4));
            issue_pair((s >> 1) + 2, 2 * (i - 4) + 1);
          }
        } else {
          issue1(s + NS - 1, i);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (i < NR) mfma_16x16x32<FIRST>(acc[i][j], fb[F][j], fa[i]);
          if (NR > 0 && i < NJ / 2 && (j == 1 || j == 3)) rd_b(s + 1, F ^ 1, 2 * i + (j == 3));
        }
        if (i < NR) rd_a(s + 1, i);         // past the last step this reads unused data
      }
    };
    if constexpr (PAIR) {
      // the loop's pattern for steps -4..-1: pair 0, other 0, other 1 and pair 1, other 2
      constexpr int Q0 = AP ? LOADS : 0;     // the other operand's loads
#pragma unroll
      for (int j = 0; j < 8; ++j) issue_pair(0, j);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int q = Q0; q < Q0 + LOADS; ++q) issue1(st, q);
#pragma unroll
      for (int j = 0; j < 8; ++j) issue_pair(1, j);
#pragma unroll
      for (int q = Q0; q < Q0 + LOADS; ++q) issue1(2, q);
      wait_vmcnt<16>();                      // pair 0 and the other operand's step 0 have landed
    } else {
#pragma unroll
      for (int st = 0; st < NS - 1; ++st)
#pragma unroll
        for (int q = 0; q < PER_STAGE; ++q) issue1(st, q);
      wait_vmcnt<(NS - 2) * PER_STAGE>();
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < NR) rd_a(0, i);
      if (NR > 0 && i < NJ) rd_b(0, 0, i);
    }
    using F0 = std::integral_constant<int, 0>;
    using F1 = std::integral_constant<int, 1>;
    step(0, F0{}, std::true_type{});                    // nk >= 1: K is at least one step
    int s = 1;
    for (; s + 1 < nk; s += 2) {
      step(s, F1{}, std::false_type{});
      step(s + 1, F0{}, std::false_type{});
    }
    if (s < nk) step(s, F1{}, std::false_type{});
    // the asm MFMAs are invisible to the hazard checks: wait out the last ones' latency, then
    // pin every later read of the accumulators behind that wait
    asm volatile("s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) asm volatile("" : "+a"(acc[i][j]));
    wait_vmcnt<0>();     // the trailing re-loads must land before the workgroup's LDS is released
    if constexpr (is_grad_epi(EPI)) {
      grad_epilogue(ni_const);
      return;
    }
    if constexpr (EPI == kEpiGelu || EPI == kEpiSilu) {
      if (g.pre != nullptr) {
        if (add_bias)
          epilogue(ni_const, std::true_type{}, std::true_type{}, wide_const);
        else
          epilogue(ni_const, std::false_type{}, std::true_type{}, wide_const);
        return;
      }
    }
    if (add_bias)
      epilogue(ni_const, std::true_type{}, std::false_type{}, wide_const);
    else
      epilogue(ni_const, std::false_type{}, std::false_type{}, wide_const);
  };
  // A tile with at most 128 segment rows runs WIDE (the forward products only: not the N-major
  // B operand, the gradient epilogues or the weight-gradient mode). Uniform per workgroup.
  if constexpr (!BNM && !is_grad_epi(EPI)) {
    if (!g.wgrad && m_e - m0 <= 128) {
      if (m_e - m0 > 64)
        mainloop(std::integral_constant<int, 4>{}, std::true_type{});
      else
        mainloop(std::integral_constant<int, 2>{}, std::true_type{});
      return;
    }
  }
  const int valid = m_e - m0 - wm * 128;     // segment rows in this wave's 128 rows
  if (valid > 64)
    mainloop(std::integral_constant<int, 4>{}, std::false_type{});
  else if (valid > 0)
    mainloop(std::integral_constant<int, 2>{}, std::false_type{});
  else
    mainloop(std::integral_constant<int, 0>{}, std::false_type{});
}

// ---------------------------------------------------------------------------------------
// bf16 grouped GEMV-like kernel for experts with at most 16 rows (decode-sized batches): the
// weights are streamed from HBM exactly once, straight into v_mfma_f32_16x16x32_bf16 operands.
// Workgroup = one expert x GV_COLS output columns (two 16-column tiles); its 4 waves split K
// into 4 contiguous ranges of 64-element chunks, so each wave's chain of dependent loads is a
// quarter of the row and four times as many workgroups share the stream. Within a chunk, lane
// group g (16 lanes) takes elements [16 g, 16 g + 16) of its row as two 8-element pieces, and
// MFMA step i takes piece i of both operands (the k order of A and B agrees); each load
// instruction covers 16 rows x 64 bytes. A wave issues the loads of GV_BATCH chunks before their
// MFMAs. The four partial tiles are added in wave order through LDS (a fixed order), and wave 0
// applies the epilogue. Rows past the expert's segment are read from its last row: they only
// feed output rows that are never stored.
constexpr int GV_COLS = 32, GV_BATCH = 4;

template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemv_bf16_kernel(GemmArgs g) {
  __shared__ floatx4 part[kWaves][2][kWave];
  const int nblk_n = (g.N + GV_COLS - 1) / GV_COLS;
  const int e = blockIdx.x / nblk_n, nb = blockIdx.x - e * nblk_n;
  const int m_e = segment_rows(g, e);
  if (m_e == 0) return;
  const int row0 = g.dense ? 0 : g.offsets[e];
  const int N = g.N, K = g.K;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int nbase = nb * GV_COLS;
  const int ar = row0 + (r16 < m_e ? r16 : m_e - 1);
  const u16* __restrict__ ap = static_cast<const u16*>(g.A) +
                               static_cast<size_t>(g.rows != nullptr ? g.rows[ar] : ar) * K + 16 * grp;
  // a lane's 16 elements of row n at K offset kc + 16 grp lie at bp + kc * kstep: in row-major
  // weights, and in packed ones, where those 16 sit in one 64-byte row of K block kc/32 + grp/2
  const u16* bp[2];
  const int kstep = g.b_tiled ? 256 : 1;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = min(nbase + t * 16 + r16, N - 1);
    bp[t] = static_cast<const u16*>(g.B) +
            (g.b_tiled ? ((static_cast<size_t>(e) * (N / 256) + n / 256) * (K / 32) + (grp >> 1)) * 8192 +
                             (n % 256) * 32 + 16 * (grp & 1)
                       : (static_cast<size_t>(e) * N + n) * K + 16 * grp);
  }
  // this wave's chunks of 64: [c0, c1)
  const int nch = K / 64;
  const int c0 = nch * wave / kWaves, c1 = nch * (wave + 1) / kWaves;
  floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  int c = c0;
  for (; c + GV_BATCH <= c1; c += GV_BATCH) {
    bf16x8 a[GV_BATCH][2], b[GV_BATCH][2][2];
#pragma unroll
    for (int i = 0; i < GV_BATCH; ++i) {
      const size_t kc = static_cast<size_t>(c + i) * 64;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        b[i][t][0] = *reinterpret_cast<const bf16x8*>(bp[t] + kc * kstep);
        b[i][t][1] = *reinterpret_cast<const bf16x8*>(bp[t] + kc * kstep + 8);
      }
      a[i][0] = *reinterpret_cast<const bf16x8*>(ap + kc);
      a[i][1] = *reinterpret_cast<const bf16x8*>(ap + kc + 8);
    }
#pragma unroll
    for (int i = 0; i < GV_BATCH; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][0], b[i][t][0], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][1], b[i][t][1], acc[t], 0, 0, 0);
      }
  }
  if (c < c1) {                              // the last 1..GV_BATCH-1 chunks, loads all issued first
    bf16x8 a[GV_BATCH - 1][2], b[GV_BATCH - 1][2][2];
#pragma unroll
    for (int i = 0; i < GV_BATCH - 1; ++i) {
      if (c + i < c1) {
        const size_t kc = static_cast<size_t>(c + i) * 64;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          b[i][t][0] = *reinterpret_cast<const bf16x8*>(bp[t] + kc * kstep);
          b[i][t][1] = *reinterpret_cast<const bf16x8*>(bp[t] + kc * kstep + 8);
        }
        a[i][0] = *reinterpret_cast<const bf16x8*>(ap + kc);
        a[i][1] = *reinterpret_cast<const bf16x8*>(ap + kc + 8);
      }
    }
#pragma unroll
    for (int i = 0; i < GV_BATCH - 1; ++i)
      if (c + i < c1)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][0], b[i][t][0], acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][1], b[i][t][1], acc[t], 0, 0, 0);
        }
  }
  part[wave][0][lane] = acc[0];
  part[wave][1][lane] = acc[1];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < 2; ++t) {              // partial sums added in wave order
    floatx4 v = part[0][t][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const floatx4 o = part[w][t][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += o[i];
    }
    acc[t] = v;
  }
  // C layout of the 16x16 tile: lane holds column (lane & 15), rows 4*(lane>>4) + i.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = nbase + t * 16 + r16;
    if (n >= N) continue;
    const float bias = load_bias(g.bias, static_cast<size_t>(e) * N + n, true);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * grp + i;
      if (r < m_e) {
        const size_t o = static_cast<size_t>(row0 + r) * N + n;
        const float val = acc[t][i] + bias;
        if constexpr (is_grad_epi(EPI)) {
          const float a = bf16_to_f32(static_cast<const u16*>(g.act_in)[o]);
          static_cast<u16*>(g.out)[o] = f32_to_bf16(val * g.row_scale[row0 + r] * activation_grad_bf16<EPI>(a));
        } else if constexpr (EPI != kEpiLinear) {
          static_cast<u16*>(g.out)[o] = f32_to_bf16(activation_bf16<EPI>(val));
          if (g.pre != nullptr) static_cast<u16*>(g.pre)[o] = f32_to_bf16(val);
        } else {
          static_cast<float*>(g.out)[o] = val;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Weight packing: W [E][rows][cols] row-major bf16 -> the K-step-tiled panels the expert GEMMs
// read as B (b_tiled): panel e rows/256 + p holds rows [256 p, 256 p + 256) of expert e as
// cols/32 contiguous blocks of 256 rows x 32 columns (64-byte rows). Thread i moves 16-byte
// piece i of the packed array, so the stores are contiguous; the loads take 64 contiguous bytes
// of each of 16 rows per wave. rows is a multiple of 256 and cols of 32.
__global__ __launch_bounds__(256) void pack_weights_kernel(const u16* __restrict__ W, u16* __restrict__ Wp,
                                                           int cols, size_t pieces) {
  const int nkb = cols / 32;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < pieces;
       i += static_cast<size_t>(gridDim.x) * 256) {
    const int q = static_cast<int>(i & 3);                 // 16-byte piece of a 64-byte row
    const int r = static_cast<int>((i >> 2) & 255);        // row within the panel
    const size_t blk = i >> 10;                            // panel * nkb + block
    const size_t panel = blk / nkb;
    const int kb = static_cast<int>(blk - panel * nkb);
    const size_t src = (panel * 256 + r) * cols + kb * 32 + q * 8;   // panel*256 = e rows + 256 p
    *reinterpret_cast<u32x4*>(Wp + i * 8) = *reinterpret_cast<const u32x4*>(W + src);
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
  int mbase;
  if (!decode_tile(blockIdx.x, g, FBM, tiles_n, e, mt, nt, mbase)) return;
  const int m_e = segment_rows(g, e);
  const int row0 = (g.dense || g.wgrad) ? 0 : g.offsets[e];
  const int m0 = mt * 16, n0 = nt * 16;
  const int N = g.N;
  const int lda = g.lda ? g.lda : g.K, ldb = g.ldb ? g.ldb : g.K;
  const int K = g.wgrad ? (g.kept[e] + kWgradK - 1) / kWgradK * kWgradK : g.K;
  const size_t kofs = g.wgrad ? static_cast<size_t>(g.koff[e]) : 0;
  const float* __restrict__ A = static_cast<const float*>(g.A) + kofs;
  const float* __restrict__ B =
      static_cast<const float*>(g.B) + kofs + (g.wgrad ? 0 : static_cast<size_t>(e) * N * ldb);
  const int32_t* rows = g.rows;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int ar = m0 + ty < m_e ? (rows != nullptr ? rows[row0 + m0 + ty] : row0 + m0 + ty) : 0;
  float acc = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    As[ty][tx] = (m0 + ty < m_e && k0 + tx < K) ? A[static_cast<size_t>(ar) * lda + k0 + tx] : 0.0f;
    Bs[ty][tx] = (n0 + ty < N && k0 + tx < K) ? B[static_cast<size_t>(n0 + ty) * ldb + k0 + tx] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(As[ty][kk], Bs[tx][kk], acc);
    __syncthreads();
  }
  const int r = m0 + ty, c = n0 + tx;
  if (r < m_e && c < N) {
    const size_t o = (g.wgrad ? static_cast<size_t>(e) * g.M * N : 0) + static_cast<size_t>(row0 + r) * N + c;
    const float val = acc + load_bias(g.bias, static_cast<size_t>(e) * N + c, false);
    float* out = static_cast<float*>(g.out);
    if constexpr (is_grad_epi(EPI)) {
      out[o] = val * g.row_scale[row0 + r] * activation_grad<EPI>(static_cast<const float*>(g.act_in)[o]);
    } else {
      out[o] = EPI == kEpiGelu ? gelu_erf(val) : (EPI == kEpiSilu ? silu_exact(val) : val);
      if (EPI != kEpiLinear && g.pre != nullptr) static_cast<float*>(g.pre)[o] = val;
    }
  }
}

// Adds the side-buffer parts of the split tail tiles to the output, parts 1, 2, ... in that
// order after part 0 (already in the output). A work unit is kFixupRows rows of one split
// tile (plan::split_tile); the fixed grid strides over the units so that the whole chip
// shares the traffic, and each thread issues the loads of all parts before it adds.
constexpr int kFixupRows = 8;
constexpr int kFixupGrid = 1024;
__global__ __launch_bounds__(256) void tail_fixup_kernel(GemmArgs g) {
  constexpr int BM = 256, BN = 256, BK = 32, SLABS = BM / kFixupRows, RPP = 256 / (BN / 4);
  const int tiles_n = (g.N + BN - 1) / BN;
  const TileScan scan = scan_tiles(g, BM, tiles_n);
  const int nk_total = g.K / BK;
  const int n_split = plan::split_tiles(scan.total, nk_total, g.splits);
  const int N = g.N;
  float* out = static_cast<float*>(g.out);
  const int c = (threadIdx.x % (BN / 4)) * 4;
  for (int u = blockIdx.x; u < n_split * SLABS; u += gridDim.x) {
    const int slab = u % SLABS;
    int tile, P, side0;
    plan::split_tile(u / SLABS, scan.total, nk_total, g.splits, tile, P, side0);
    int e, mt, nt, mbase, m_e;
    locate_tile(scan, tile, tiles_n, e, mt, nt, mbase, m_e);
    const int row0 = g.dense ? 0 : __builtin_amdgcn_readlane(scan.off, e);
    const int m0 = mt * BM, n0 = nt * BN;
    const float* side = static_cast<const float*>(g.out2) + static_cast<size_t>(side0) * kTailTile;
#pragma unroll
    for (int j = 0; j < kFixupRows / RPP; ++j) {
      const int r = slab * kFixupRows + j * RPP + static_cast<int>(threadIdx.x) / (BN / 4);
      if (m0 + r >= m_e || n0 + c >= N) continue;
      floatx4 w[kTailMaxParts - 1];
#pragma unroll
      for (int p = 1; p < kTailMaxParts; ++p)
        if (p < P)
          w[p - 1] = __builtin_nontemporal_load(
              reinterpret_cast<const floatx4*>(side + (p - 1) * kTailTile + r * BN + c));
      floatx4* o = reinterpret_cast<floatx4*>(out + static_cast<size_t>(row0 + m0 + r) * N + n0 + c);
      floatx4 v = *o;
#pragma unroll
      for (int p = 1; p < kTailMaxParts; ++p)
        if (p < P) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] += w[p - 1][q];
        }
      *o = v;
    }
  }
}

int tile_grid(int R, int E, int C, int BM, int N, int BN) {
  const long long by_rows = (R + BM - 1) / BM + E;
  const long long by_cap = static_cast<long long>(E) * ((C + BM - 1) / BM);
  const long long tm = by_rows < by_cap ? by_rows : by_cap;
  return static_cast<int>(tm * ((N + BN - 1) / BN));
}

}  // namespace

bool ffn_gathers(const FfnArgs& a) {
  // the GEMV (C <= 16) forms 64-bit row addresses; the MFMA kernel's buffer offsets are 32-bit
  return a.bf16 && (a.C <= 16 || static_cast<long long>(a.T) * a.d * 2 < (1ll << 31));
}

int ffn_splits(const FfnArgs& a) { return (a.bf16 && a.C > 16) ? kTailMaxParts : 1; }

size_t tail_side_floats(int R, int E, int C, int N) {
  // a split tail writes L (P - 1) side tiles: fewer than kSideSlots, and at most
  // (kMaxParts - 1) per tile of the launch
  const long long by_tiles = static_cast<long long>(kTailMaxParts - 1) * tile_grid(R, E, C, 256, N, 256);
  return static_cast<size_t>(by_tiles < plan::kSideSlots ? by_tiles : plan::kSideSlots) * kTailTile;
}

bool ffn_h_tiled(int bf16, int C) { return bf16 && C > 16; }

size_t ffn_h_rows(int R, int E, int C, int bf16) {
  // at most R/256 + E row tiles: every expert's last one may be partial
  return ffn_h_tiled(bf16, C) ? (static_cast<size_t>(R) / 256 + E) * 256 : static_cast<size_t>(R);
}

template <int ACT>
static hipError_t launch_ffn(const GemmArgs& g1, const GemmArgs& g2, bool bf16, int C, int R, int E, int N1, int N2,
                             hipStream_t stream, hipEvent_t ev_mid) {
  hipError_t err;
  if (!bf16) {
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<ACT>, dim3(tile_grid(R, E, C, FBM, N1, 16)), dim3(256), 0, stream, g1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev_mid && (err = hipEventRecord(ev_mid, stream)) != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<kEpiLinear>, dim3(tile_grid(R, E, C, FBM, N2, 16)), dim3(256), 0,
                       stream, g2);
    return hipGetLastError();
  }
  if (C <= 16) {
    hipLaunchKernelGGL(grouped_gemv_bf16_kernel<ACT>, dim3(E * ((N1 + GV_COLS - 1) / GV_COLS)), dim3(256), 0, stream,
                       g1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev_mid && (err = hipEventRecord(ev_mid, stream)) != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemv_bf16_kernel<kEpiLinear>, dim3(E * ((N2 + GV_COLS - 1) / GV_COLS)), dim3(256), 0,
                       stream, g2);
    return hipGetLastError();
  }
  const int grid1 = plan_grid(tile_grid(R, E, C, 256, N1, 256), 1);
  const int grid2 = plan_grid(tile_grid(R, E, C, 256, N2, 256), g2.splits);
  // GEMM1's A (the token rows, gathered or a plain copy) is row-major: pair staging for it.
  // GEMM2's A (H) is K-step-tiled; its B (W2) is pair-staged when row-major, and packed weights
  // are K-step-tiled like H
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<ACT, 32, 4, false, 1>), dim3(grid1), dim3(256), 0, stream, g1);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev_mid && (err = hipEventRecord(ev_mid, stream)) != hipSuccess) return err;
  if (g2.a_tiled && g2.b_tiled)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<kEpiLinear, 32, 4>), dim3(grid2), dim3(256), 0, stream, g2);
  else if (g2.a_tiled)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<kEpiLinear, 32, 4, false, 2>), dim3(grid2), dim3(256), 0, stream, g2);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<kEpiLinear, 32, 4>), dim3(grid2), dim3(256), 0, stream, g2);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (g2.splits > 1) hipLaunchKernelGGL(tail_fixup_kernel, dim3(kFixupGrid), dim3(256), 0, stream, g2);
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream, hipEvent_t ev_mid) {
  GemmArgs g1{a.x_perm, a.W1, a.b1, a.H, a.kept, a.offsets, a.E, a.d_ffn, a.d, a.R, a.C, 1, nullptr, nullptr, 0, 0};
  g1.pre = a.pre;
  GemmArgs g2{a.H, a.W2, a.b2, a.y_perm, a.kept, a.offsets, a.E, a.d, a.d_ffn, a.R, a.C, ffn_splits(a), a.side,
              nullptr, 0, 0};
  if (ffn_h_tiled(a.bf16, a.C)) g2.a_tiled = 1;   // GEMM1 runs the MFMA kernel: H is tiled
  g1.b_tiled = g2.b_tiled = a.w_packed;          // bf16 only, d and d_ffn multiples of 256
  if (a.bf16 && a.rows != nullptr) {   // GEMM1 (or the GEMV) reads the token rows of x directly
    g1.A = a.x;
    g1.rows = a.rows;
    g1.a_rows = a.T;
  }
  return a.act == kActSilu ? launch_ffn<kEpiSilu>(g1, g2, a.bf16, a.C, a.R, a.E, a.d_ffn, a.d, stream, ev_mid)
                           : launch_ffn<kEpiGelu>(g1, g2, a.bf16, a.C, a.R, a.E, a.d_ffn, a.d, stream, ev_mid);
}

hipError_t launch_shared_ffn(const SharedFfnArgs& a, hipStream_t stream) {
  // one dense expert over the T token rows in order: E = 1, no split of K
  GemmArgs g1{a.x, a.W1, a.b1, a.H, nullptr, nullptr, 1, a.d_ffn, a.d, a.T, a.T, 1, nullptr, nullptr, 0, 1};
  GemmArgs g2{a.H, a.W2, a.b2, a.y, nullptr, nullptr, 1, a.d, a.d_ffn, a.T, a.T, 1, nullptr, nullptr, 0, 1};
  if (ffn_h_tiled(a.bf16, a.T)) g2.a_tiled = 1;
  return a.act == kActSilu ? launch_ffn<kEpiSilu>(g1, g2, a.bf16, a.T, a.T, 1, a.d_ffn, a.d, stream, nullptr)
                           : launch_ffn<kEpiGelu>(g1, g2, a.bf16, a.T, a.T, 1, a.d_ffn, a.d, stream, nullptr);
}

hipError_t launch_pack_weights(const void* W, void* W_packed, int64_t E, int64_t rows, int64_t cols,
                               hipStream_t stream) {
  const size_t pieces = static_cast<size_t>(E) * rows * cols / 8;
  const size_t blocks = (pieces + 255) / 256;
  const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const u16*>(W),
                     static_cast<u16*>(W_packed), static_cast<int>(cols), pieces);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Backward products (the weights already transposed, so every operand is K-contiguous).
// bnm: on the bf16 MFMA path B is N-contiguous ([E][K][N]); elsewhere B is always [E][N][K].
template <int EPI>
static hipError_t launch_rows_gemm(const GemmArgs& g, bool bf16, int C, hipStream_t stream, bool bnm = false) {
  if (!bf16) {
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<EPI>, dim3(tile_grid(g.R, g.E, C, FBM, g.N, 16)), dim3(256), 0,
                       stream, g);
  } else if (C <= 16) {
    hipLaunchKernelGGL(grouped_gemv_bf16_kernel<EPI>, dim3(g.E * ((g.N + GV_COLS - 1) / GV_COLS)), dim3(256), 0,
                       stream, g);
  } else {
    const int grid = plan_grid(tile_grid(g.R, g.E, C, 256, g.N, 256), EPI == kEpiLinear ? g.splits : 1);
    // (pair staging of row-major A measured 1-2% slower on the dA product, whose B takes the
    // transpose reads: one-step stages here)
    if (bnm)
      hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EPI, 32, 4, true>), dim3(grid), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EPI, 32, 4>), dim3(grid), dim3(256), 0, stream, g);
    if (EPI == kEpiLinear && g.splits > 1) {
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL(tail_fixup_kernel, dim3(kFixupGrid), dim3(256), 0, stream, g);
    }
  }
  return hipGetLastError();
}

bool bwd_weights_transposed(int bf16, int C) { return !(bf16 && C > 16); }

bool wgrad_tiled(int bf16) { return bf16 != 0; }   // the bf16 weight gradients run the MFMA kernel

size_t wgrad_rows(int rows, int bf16) {
  return wgrad_tiled(bf16) ? (static_cast<size_t>(rows) + 255) / 256 * 256 : static_cast<size_t>(rows);
}

hipError_t launch_bwd_dact(const BwdDactArgs& a, hipStream_t stream) {
  const bool bnm = !bwd_weights_transposed(a.bf16, a.C);
  GemmArgs g{};
  g.A = a.A;
  g.rows = a.rows;
  g.a_rows = a.a_rows;
  g.B = bnm ? a.W2 : a.W2T;
  g.out = a.dA;
  g.kept = a.kept;
  g.offsets = a.offsets;
  g.E = a.E;
  g.N = a.d_ffn;
  g.K = a.d;
  g.R = a.R;
  g.C = a.C;
  g.splits = 1;
  g.row_scale = a.wrow;
  g.act_in = a.pre;
  return a.act == kActSilu ? launch_rows_gemm<kEpiSiluGrad>(g, a.bf16, a.C, stream, bnm)
                           : launch_rows_gemm<kEpiGeluGrad>(g, a.bf16, a.C, stream, bnm);
}

int bwd_dx_splits(int R, int E, int C, int d, int d_ffn, int bf16) {
  (void)R, (void)E, (void)d, (void)d_ffn;
  return (bf16 && C > 16) ? kTailMaxParts : 1;
}

hipError_t launch_bwd_dx(const BwdDxArgs& a, hipStream_t stream) {
  const bool bnm = !bwd_weights_transposed(a.bf16, a.C);
  GemmArgs g{};
  g.A = a.dA;
  g.B = bnm ? a.W1 : a.W1T;
  g.out = a.dXp;
  g.out2 = a.side;
  g.kept = a.kept;
  g.offsets = a.offsets;
  g.E = a.E;
  g.N = a.d;
  g.K = a.d_ffn;
  g.R = a.R;
  g.C = a.C;
  g.splits = bwd_dx_splits(a.R, a.E, a.C, a.d, a.d_ffn, a.bf16);
  g.a_tiled = ffn_h_tiled(a.bf16, a.C) ? 1 : 0;   // dA comes from the MFMA kernel's gradient epilogue
  return launch_rows_gemm<kEpiLinear>(g, a.bf16, a.C, stream, bnm);
}

hipError_t launch_wgrad(const WgradArgs& a, hipStream_t stream) {
  GemmArgs g{};
  g.A = a.A;
  g.B = a.B;
  g.out = a.out;
  g.kept = a.kept;
  g.koff = a.koff;
  g.E = a.E;
  g.M = a.M;
  g.N = a.N;
  g.K = kWgradK;
  g.lda = a.ld;
  g.ldb = a.ld;
  g.R = a.M;
  g.C = a.C;
  g.splits = 1;
  g.wgrad = 1;
  g.a_tiled = g.b_tiled = wgrad_tiled(a.bf16) ? 1 : 0;
  if (!a.bf16) {
    const int grid = a.E * ((a.M + 15) / 16) * ((a.N + 15) / 16);
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<kEpiLinear>, dim3(grid), dim3(256), 0, stream, g);
  } else {
    const int grid = plan_grid(a.E * ((a.M + 255) / 256) * ((a.N + 255) / 256), 1);
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<kEpiLinear, 32, 4>), dim3(grid), dim3(256), 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace moe
