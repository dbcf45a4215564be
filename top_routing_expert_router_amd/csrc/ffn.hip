// Grouped SwiGLU expert FFN over aligned rows, on gfx950 bf16 MFMA.
//
// "Route-Block Membership Selects Packed-AWQ Arithmetic", "The boundary that
// mattered": the expert path is the fused first projection W13, the activation,
// and the routed second projection W2, applied to padded expert blocks.  The
// FFN form is SwiGLU: act = silu(h W1^T) * (h W3^T), y = act W2^T, with W13 rows
// 0..I-1 = W1 (gate) and I..2I-1 = W3 (up).
//
// Unlike the packed kernel studied on that page, no row's arithmetic depends on
// the block it lands in: there is no split-K and no schedule class; every output
// element is one MFMA chain over K in ascending 16-wide steps ("Why
// temperature=0 Still Gives Different Answers: Batch Invariance", tier 2: one
// tile configuration, no atomic split-K).  Rows are independent, so permuting
// routes inside or across blocks leaves each row's bits unchanged.
//
// Kernel shape (bf16 / fp8-weight path):
//   persistent: one workgroup per CU claims 256-row x 256-weight-row tiles (per-XCD
//   counters, or a static stride without a workspace); K step 64, 4 waves of
//   128 x 128, v_mfma_f32_32x32x16_bf16 with weights as the MFMA "A" operand, so
//   each lane ends with 4 consecutive output columns of one row (8-byte stores);
//   two LDS stages of (256 x 64) bf16 for each operand, 16-byte chunks XOR-swizzled
//   by (row >> 1) & 7 so the fragment reads are free of bank conflicts;
//   global -> LDS copies by buffer loads with an LDS destination (the A-row gather,
//   route -> token row of h, folded into their offsets), one barrier per K step,
//   fragments read two 16-wide steps ahead of the MFMAs;
//   W13 tiles hold 128 gate rows and the matching 128 up rows, so SwiGLU is a
//   register-local epilogue; W2 writes each row straight to its route's y row;
//   M tiles are 256-row slices of one expert's padded segment (a fixed constant,
//   decoupled from B), run in full, half or quarter mode by their valid rows; W2
//   has micro tiles (run_tile_micro) for its small last m-tiles; workgroups map
//   to XCDs so each XCD walks a contiguous run of (n-tile group, m-tile) pairs and
//   shares weight tiles in its L2.
// fp8 weights: E4M3FN codes are loaded into registers three MFMA steps ahead, decoded
// with the hardware converter, multiplied by their 128x128 block's bf16 scale in
// fp32 and rounded to bf16 into LDS, spread over the MFMAs of the next half stage.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;  // BN: the W13 tile (128 gate + 128 up rows)
constexpr int kThreads = 256;
// n-tiles per raster group: 2 with bf16 weights; 8 with fp8 weights, whose stages take
// longer (the decode) and whose workgroups then share each expert's activation rows across
// more n-tiles (DeepSeek-V3 shape: W2 4.53 -> 4.37 ms; the bf16 shapes measured no faster
// or slower with wider groups)
template <bool FP8>
constexpr int group_n() { return FP8 ? 8 : 2; }
// buffer resource word 3 for raw (untyped, stride 0) buffer loads on gfx9-family parts
constexpr int kBufferFlags = 0x00020000;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct FfnArgs {
  const void* x;          // W13: h [T, H];  W2: act [rows, I]
  const int32_t* sorted;  // routed: sorted_route_ids; identity: nullptr
  const int32_t* offsets; // routed: expert_offsets [N + 1]
  const void* w;          // W13: [E, 2I, H];  W2: [E, H, I]
  const __bf16* wscale;   // fp8 block scales or nullptr
  void* out;              // W13: act [rows, I];  W2: y [*, H]
  int T, H, I, N, k;
  int sentinel;           // T*k: padding row marker; any id outside [0, T*k) is treated as padding
  int rows;               // rows of the act buffer (P_max routed, T identity): no row index reaches it
  int mtiles;             // M-tile bound used for the grid
  int ntiles;
  int32_t* work;          // nullable: 8 zeroed per-XCD tile counters (dynamic schedule)
  int dest_is_row;        // W2: 1 = y row p (expert choice: sorted holds token ids), 0 = y row sorted[p]
  int micro;              // W2, bf16 weights, K % 256 == 0, one to four rounds of tiles: small last
                          // m-tiles run as micro tiles, after all full-height tiles
  void* w13_out;          // W13 only, nullable: [rows, 2I] gate then up projection, act dtype
  uint64_t* clk;          // nullable: per workgroup, shader-clock and real-time counters at its
                          // start and its end (4 words at 4 * blockIdx.x)
};

// The core-cycle counter (clock64: it counts at whatever clock the shader runs at) and the
// constant-rate wall-clock counter (wall_clock64, hipDeviceAttributeWallClockRate) now, into
// p[0], p[1]: their ratio over a workgroup's life is the clock it ran at.  Counter reads and
// a vector store, outside any K loop.
__device__ __forceinline__ void clock_stamp(uint64_t* p) {
  const uint64_t t = (uint64_t)clock64();
  const uint64_t r = (uint64_t)wall_clock64();
  p[0] = t;
  p[1] = r;
}

// LDS tile layout: row-major 128-byte rows of 8 16-byte chunks, chunk index XORed
// with (row >> 1) & 7.  A ds_read_b128 serves 16 lanes per cycle from 64 banks;
// the 32x32 fragment reads put 16 consecutive rows at one logical chunk in those
// 16 lanes, and this XOR spreads them over all 64 banks (rows r and r+1 differ in
// the bank half, rows 2m.. in the chunk).
__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * (BK * 2) + (swz_chunk(row, chunk) << 4); }
// Micro tiles: 128-deep stages, rows of 256 B (16 chunks); chunk index XORed with
// row & 15, so the 16 consecutive rows a 16-lane group reads at one logical chunk
// land in 16 different chunks, i.e. all 64 banks.
__device__ __forceinline__ int swzn_chunk(int row, int chunk) { return chunk ^ (row & 15); }
__device__ __forceinline__ int swzn(int row, int chunk) { return row * (BK * 4) + (swzn_chunk(row, chunk) << 4); }

// Tile table, built once per workgroup in LDS: beg[e] = first padded row of expert
// e (beg[N] = end of the last).  Each expert's padded segment is cut into
// ceil(len / BM) m-tiles; m-slots are numbered in expert order, big0[e] = m-slots of
// the experts before e (big0[N] = all of them), so an expert's m-tiles stay together
// and share its weight tiles in L2.  Micro-tile kernels: a last m-tile of at most BM / 2
// rows is "small": it runs as micro tiles of up to 64 of its rows and a quarter (64
// rows) of the weight n-tile, so it takes four m-slots (up to 64 rows) or eight (65 to
// 128 rows: row half j / 4, weight quarter j % 4), numbered after all other m-tiles
// (sm0[e] = small m-slots before e), so within each raster group the short tiles come
// last and fill the end of the schedule instead of pushing full tiles into an extra
// round.  Identity rows: one expert, rows [0, T).
constexpr int kMaxExperts = 256;
constexpr int kEpiWaveBytes = 32 * (64 * 2 + 16);
constexpr int kMicroB = 16384;  // micro tiles: byte offset of the weight rows in a stage buffer

template <bool MICRO>
__device__ void build_tile_table(const FfnArgs& a, int* beg, int* big0, int* sm0) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int b[4], nb[4], ns[4];
    int sb = 0, ss = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = lane * 4 + i;
      const bool ok = ee < a.N;
      b[i] = !ok ? 0 : (a.sorted == nullptr ? 0 : a.offsets[ee]);
      const int end = !ok ? 0 : (a.sorted == nullptr ? a.T : a.offsets[ee + 1]);
      const int len = end - b[i];
      const int nf = ok ? ceil_div(len, BM) : 0;
      const int last = len - (nf - 1) * BM;  // rows of the last m-tile (nf > 0)
      const bool small = MICRO && nf > 0 && last <= BM / 2;
      nb[i] = small ? nf - 1 : nf;
      ns[i] = small ? (last > BM / 4 ? 8 : 4) : 0;
      sb += nb[i];
      ss += ns[i];
    }
    const int ib = wave_incl_scan_i32(sb);
    const int is = MICRO ? wave_incl_scan_i32(ss) : 0;
    int pb = ib - sb, ps = is - ss;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = lane * 4 + i;
      if (ee < a.N) {
        beg[ee] = b[i];
        big0[ee] = pb;
        if (MICRO) sm0[ee] = ps;
      }
      pb += nb[i];
      ps += ns[i];
    }
    if (lane == kWave - 1) {
      beg[a.N] = a.sorted == nullptr ? a.T : a.offsets[a.N];
      big0[a.N] = ib;
      if (MICRO) sm0[a.N] = is;
    }
  }
  __syncthreads();
}

// A pointer that is the same in every lane, made scalar: a 64-bit product may be
// computed on the vector unit, and a buffer resource built from it must be scalar.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void*)(((uint64_t)hi << 32) | lo);
}

// Buffer resources of a tile's operands, built from scalar values where they are used
// (a resource carried from tile to tile can end up in VGPRs, and every copy then
// becomes a waterfall loop).  A: all of h (W13, gathered rows) or the tile's own act
// rows (W2, contiguous from p0).  B: expert e's weights.
template <int MODE>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t act_rsrc(const __bf16* X, int T, int K, int p0, int p1) {
  p0 = __builtin_amdgcn_readfirstlane(p0);
  p1 = __builtin_amdgcn_readfirstlane(p1);
  if constexpr (MODE == 0)
    return __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, (int)((unsigned)T * K * 2u), kBufferFlags);
  else
    return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(X + (long)p0 * K), (short)0,
                                             (int)((unsigned)(p1 - p0) * K * 2u), kBufferFlags);
}
template <bool FP8>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const void* w, int e, int WR, int K) {
  const long ex = __builtin_amdgcn_readfirstlane(e);
  if constexpr (!FP8)
    return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr((const __bf16*)w + ex * WR * K), (short)0,
                                             (int)((unsigned)WR * K * 2u), kBufferFlags);
  else
    return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr((const uint8_t*)w + ex * WR * K), (short)0,
                                             (int)((unsigned)WR * K), kBufferFlags);
}

// One output tile: expert e, padded rows [p0, p1), weight n-tile nt; sub = -1, or the
// quarter (sub & 3) of the n-tile's weight rows a micro tile covers.
struct Tile {
  int e, p0, p1, nt, sub;
};

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))


// Barrier that publishes LDS written by global->LDS DMA.  The DMA is counted by
// vmcnt, so every wave waits for its own DMA *before* the barrier; only then are all
// waves' rows in LDS when any wave passes it.  s_waitcnt imm 0x70 = vmcnt(0) expcnt(7)
// lgkmcnt(0).  (The workgroup fence of __syncthreads() would wait for all of them too: it
// counts LDS copies as LDS writes.)
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0x70);
  __syncthreads();
}

// fp8 weights: the same, except that the newest BJ + 2 vector loads (the next stage's
// weight codes and block scales, into registers) may still be in flight.  vmcnt(10):
// imm 0x7A = vmcnt(10) expcnt(7) lgkmcnt(0).
__device__ __forceinline__ void fp8_barrier() {
  __builtin_amdgcn_s_waitcnt(0x7A);
  __syncthreads();
}

// Barrier after this wave's LDS reads have completed (lgkmcnt(0): imm 0xC07F), so no
// wave's later DMA can overwrite what a read still needs.  The workgroup fence of
// __syncthreads() also makes it wait for the copies in flight (the next tile's first
// stage, issued a few steps earlier); a bare barrier here measured no faster.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __syncthreads();
}

// MODE 0: W13 + SwiGLU -> act.  MODE 1: W2 -> y rows.
//
// Three tile modes over the same 256-row weight tile (W13: 128 gate and the matching
// 128 up rows), by the m-tile's valid rows R:
//  - full (R > 128): waves 2 x 2, each 128 rows x 128 weight rows;
//  - half (64 < R <= 128, as the last tile of an expert often is): all 4 waves on the
//    same 128 rows, each with 64 weight rows -- half the MFMAs of a full tile;
//  - quarter (R <= 64): all 4 waves on the same 64 rows, each with 64 weight rows.
// An output element's K order is the same in every mode (one MFMA chain over K in
// ascending 16-wide steps), so the mode changes no output bit.
// MICRO (W2, bf16 weights only): small last m-tiles run as micro tiles; see
// run_tile_micro.  A kernel of its own, so the others keep their register allocation.
// W13OUT (W13 only): the epilogue also stores the gate and up projections, each rounded
// from its fp32 accumulator, to a.w13_out (the pre-activation surface); an instantiation
// of its own, so the kernel the layer runs is unchanged.
template <int MODE, bool FP8, bool MICRO, bool W13OUT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void ffn_gemm_bf16(FfnArgs a) {
  static_assert(!MICRO || (MODE == 1 && !FP8), "micro tiles: W2 with bf16 weights only");
  static_assert(!W13OUT || MODE == 0, "the pre-activation surface is the W13 GEMM's");
  static_assert(BN / 32 + 2 == 10, "fp8_barrier leaves BJ + 2 loads in flight");
  constexpr int TBN = BN;           // weight rows per tile
  constexpr int BJ = TBN / 32;      // weight-row DMA instructions (8 rows each) per wave and stage
  // Two stages, each its own array so the compiler can see that the tile being
  // filled by DMA never aliases the tile being read.
  __shared__ __attribute__((aligned(16))) char sA0[BM * BK * 2];
  __shared__ __attribute__((aligned(16))) char sB0[TBN * BK * 2];
  __shared__ __attribute__((aligned(16))) char sA1[BM * BK * 2];
  __shared__ __attribute__((aligned(16))) char sB1[TBN * BK * 2];
  __shared__ int t_beg[kMaxExperts + 1], t_big0[kMaxExperts + 1], t_sm0[MICRO ? kMaxExperts + 1 : 1];
  // each wave's epilogue staging area: 32 rows x up to 64 output columns (bf16), rows
  // padded by 16 bytes so that the staging writes and the row reads spread over the banks
  __shared__ __attribute__((aligned(16))) char s_epi[4 * kEpiWaveBytes];

  // ---- persistent work.  Tiles in logical order: groups of kGroupN n-tiles, all
  // m-tiles of a group before the next group.  Hardware deals workgroups to the 8
  // XCDs round-robin; XCD x owns the contiguous run [x, x+1) * ceil(G / 8) of that
  // order, so the ~32 workgroups of an XCD work on neighbouring tiles at any time.
  // Static schedule: the workgroup in slot s takes tiles s, s + slots, ... of the run.
  // Dynamic schedule (a.work): workgroups claim the run's tiles in order from the
  // XCD's counter -- a workgroup claims its next tile when it starts the current
  // one, so tiles of unequal cost (full and half) balance across the XCD.
  if (a.clk != nullptr && threadIdx.x == 0) clock_stamp(a.clk + 4 * blockIdx.x);
  build_tile_table<MICRO>(a, t_beg, t_big0, t_sm0);
  // values read from the table are the same in every lane; readfirstlane makes them
  // scalar, so the buffer resources built from them stay in SGPRs
  constexpr bool kMicro = MICRO;
  const int total_big = __builtin_amdgcn_readfirstlane(t_big0[a.N]);
  const int total_m = kMicro ? total_big + __builtin_amdgcn_readfirstlane(t_sm0[a.N]) : total_big;
  const int G = total_m * a.ntiles;
  const int per_xcd = ceil_div(G, 8);
  const int slots = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  const int run0 = xcd * per_xcd;
  const int lid_end = min(G, run0 + per_xcd);
  const bool dyn = a.work != nullptr;
  __shared__ int sh_claim;
  int lid = run0 + (blockIdx.x >> 3);
  if (dyn) {
    if (threadIdx.x == 0) sh_claim = atomicAdd(a.work + xcd, 1);
    __syncthreads();
    lid = run0 + __builtin_amdgcn_readfirstlane(sh_claim);
  }
  if (lid >= lid_end) {
    if (a.clk != nullptr && threadIdx.x == 0) clock_stamp(a.clk + 4 * blockIdx.x + 2);
    return;
  }
  auto decode = [&](int l, Tile& t) {
    constexpr int kGroupN = group_n<FP8>();
    const int group = l / (kGroupN * total_m);
    const int gn0 = group * kGroupN;
    const int gsize = min(kGroupN, a.ntiles - gn0);
    const int idx = l - group * kGroupN * total_m;
    const int m = idx / gsize;
    t.nt = gn0 + idx % gsize;
    const bool big = !kMicro || m < total_big;
    const int* pre = big ? t_big0 : t_sm0;
    const int mm = big ? m : m - total_big;
    int lo = 0, hi = a.N;  // last expert e with pre[e] <= mm (experts without such slots are skipped)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= mm) lo = mid; else hi = mid;
    }
    t.e = __builtin_amdgcn_readfirstlane(lo);
    const int j = mm - pre[lo], len = t_beg[lo + 1] - t_beg[lo], nf = ceil_div(len, BM);
    // a big slot is m-tile j; a small slot j is row half j / 4 and weight quarter j % 4 of
    // the last m-tile
    t.sub = __builtin_amdgcn_readfirstlane(!big && kMicro ? j : -1);
    const int mrow = big ? j * BM : (nf - 1) * BM + (j >> 2) * (BM / 4);
    t.p0 = __builtin_amdgcn_readfirstlane(t_beg[lo] + mrow);
    t.p1 = __builtin_amdgcn_readfirstlane(min(min(t_beg[lo + 1], t.p0 + (big ? BM : BM / 4)), a.rows));
  };
  // tile mode: the activation rows it covers, 256 (full), 128 (half) or 64 (quarter);
  // micro tiles (64 weight rows, 128-deep stages, up to 64 rows): 65
  auto tile_rows = [&](const Tile& t) {
    const int r = __builtin_amdgcn_readfirstlane(t.p1 - t.p0);
    const int rows = r <= BM / 4 ? BM / 4 : (r <= BM / 2 ? BM / 2 : BM);
    return kMicro && __builtin_amdgcn_readfirstlane(t.sub) >= 0 ? BM / 4 + 1 : rows;
  };
  Tile cur;
  decode(lid, cur);

  const int K = MODE == 0 ? a.H : a.I;
  const int WR = MODE == 0 ? 2 * a.I : a.H;  // weight rows per expert
  // The wave index is uniform: made scalar, every per-wave LDS destination of a copy is an
  // SGPR sum (M0 set by scalar code, no VALU -> SGPR moves between the MFMAs), and the
  // kernels keep all their state in registers (no spills).
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- global -> LDS copy plan.  8 rows (1 KB) per DMA instruction; lane L lands
  // in physical 16-byte chunk L % 8 of its row, so it fetches the logical chunk that
  // the swizzle puts there (the swizzle is an involution in the chunk index).
  // Activation rows: wave w fills rows [64 w, 64 w + 64) of a full tile (8
  // instructions), [32 w, 32 w + 32) of a half tile (4), [16 w, 16 w + 16) of a quarter
  // tile (2).  Weight rows: wave w fills rows [64 w, 64 w + 64) in every mode.
  const int drow = lane >> 3;                    // row within the 8-row group
  auto arow_of = [&](int rows, int j) { return wave * (rows / 4) + j * 8 + drow; };
  auto brow_of = [&](int j) { return wave * (TBN / 4) + j * 8 + drow; };
  // The copies are buffer loads with LDS destination: a buffer resource per operand
  // (base address + byte size, out-of-range reads return zeros) and a 32-bit byte
  // offset per lane.  The resources are rebuilt from the tile's (scalar) fields where
  // they are used rather than carried from tile to tile, so they stay in SGPRs (a
  // carried resource can end up in VGPRs, and every copy then becomes a waterfall loop).
  const __bf16* X = (const __bf16*)a.x;
  uint32_t aoff[8];                              // byte offset of each of the lane's A rows
  uint32_t boff[8];                              // byte offset of each of the lane's weight rows
  // prefetch (bf16 W2, fp8 W13): byte offset of activation row 64 wave + lane (or none), and
  // that row's route id (W13)
  uint32_t poff = 0x80000000u;
  int prid = 0;
  auto weight_row = [&](int n0, int j) {  // j = tile row
    const int r = MODE == 0 ? (j < TBN / 2 ? n0 + j : a.I + n0 + (j - TBN / 2)) : n0 + j;
    return (MODE == 1 && r >= a.H) ? -1 : r;
  };
  // ---- fp8 weights: register staging with decode + scale (rows rb + 32 i); boff[i]
  // is then the byte offset of row rb + 32 i, chunk (tid & 7), or past the end of the
  // expert's codes for a row beyond the weights (the load returns zeros)
  const int chunk = tid & 7, rb = tid >> 3;
  long srow_lo = 0, srow_hi = 0;
  // Buffers, offsets and weight rows of tile t.  A: all of h (MODE 0, gathered
  // rows) or the tile's own act rows (MODE 1, contiguous from p0).  B: expert e.
  // Rows outside the tile or padding rows read a harmless valid row (token 0, or a
  // row of the tile's own act block); their results are never stored (rows never
  // interact in the product).  W13 gathers token rows: the eight route ids are loaded
  // unconditionally (index clamped into the tile), so the loads are in flight together.
  // W2 reads the tile's act rows in order and needs no route id.
  int rid[8];
  auto setup_ids = [&](const Tile& t) {
    const int rows = tile_rows(t);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      rid[j] = (MODE == 0 && a.sorted != nullptr) ? a.sorted[min(t.p0 + arow_of(rows, j), t.p1 - 1)] : 0;
    if constexpr (MODE == 0 && FP8)
      prid = a.sorted != nullptr ? a.sorted[min(t.p0 + wave * 64 + lane, t.p1 - 1)] : 0;
  };
  // activation-row offsets of tile t (W13: from the route ids setup_ids loaded)
  auto setup_a = [&](const Tile& t) {
    const int rows = tile_rows(t);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ar = arow_of(rows, j);
      const int p = t.p0 + ar;
      unsigned row = 0;
      if (p < t.p1) {
        if (MODE == 1) row = p - t.p0;
        else if (a.sorted == nullptr) row = p;
        else if ((unsigned)rid[j] < (unsigned)a.sentinel) row = rid[j] / a.k;
      }
      aoff[j] = (row * (unsigned)K + swz_chunk(ar, lane & 7) * 8) * 2u;
    }
    if constexpr (MODE == 1 || FP8) {
      // one lane per activation row of the tile; lanes past its rows, and padding rows,
      // fetch nothing (an offset beyond the buffer's size)
      const int pr = wave * 64 + lane;
      const int p = t.p0 + pr;
      poff = 0x80000000u;
      if (pr < rows && p < t.p1) {
        if (MODE == 1) poff = (unsigned)pr * (unsigned)K * 2u;
        else if (a.sorted == nullptr) poff = (unsigned)p * (unsigned)K * 2u;
        else if ((unsigned)prid < (unsigned)a.sentinel) poff = (unsigned)(prid / a.k) * (unsigned)K * 2u;
      }
    }
  };
  // weight-row offsets of tile t (fp8: and its scale rows)
  auto setup_b = [&](const Tile& t) {
    const int n0 = MODE == 0 ? t.nt * (TBN / 2) : t.nt * TBN;
    if constexpr (!FP8) {
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        const int r = weight_row(n0, brow_of(j));
        boff[j] = ((unsigned)(r < 0 ? 0 : r) * (unsigned)K + swz_chunk(brow_of(j), lane & 7) * 8) * 2u;
      }
    } else {
#pragma unroll
      for (int i = 0; i < BJ; ++i) {
        const int r = weight_row(n0, rb + 32 * i);
        boff[i] = r < 0 ? 0x80000000u : (unsigned)r * (unsigned)K + chunk * 8;
      }
      const int kb = K / 128;
      const int rhi = MODE == 0 ? a.I + n0 : n0 + 128;
      srow_lo = ((long)t.e * (WR / 128) + n0 / 128) * kb;
      srow_hi = ((long)t.e * (WR / 128) + min(rhi, WR - 1) / 128) * kb;
    }
  };
  auto setup = [&](const Tile& t) {
    const int rows = tile_rows(t);
    if (kMicro && (rows & 1)) {
      // micro (W2): activation rows [16 wave, +16) of the tile's 64 and weight rows [16 wave,
      // +16) of its quarter, each in 4 DMAs of 4 rows.  Lane L lands in physical chunk L % 16
      // of row L / 16 of its group and fetches the logical chunk stored there.  Rows past the
      // tile read its first row (never stored); weight rows past H read row 0 (a column past H
      // is never stored either).
      const int pc = lane & 15, gr = lane >> 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wave * 16 + j * 4 + gr;
        const unsigned row = t.p0 + r < t.p1 ? (unsigned)r : 0u;
        aoff[j] = (row * (unsigned)K + swzn_chunk(r, pc) * 8) * 2u;
        const int wr = t.nt * TBN + (t.sub & 3) * (TBN / 4) + r;
        boff[j] = ((unsigned)(wr < a.H ? wr : 0) * (unsigned)K + swzn_chunk(r, pc) * 8) * 2u;
      }
      return;
    }
    setup_ids(t);
    setup_a(t);
    setup_b(t);
  };
  u32x2 bq[BJ];
  // block scales of the staged codes, as raw bf16 bits: converted where the decode uses
  // them, so that no conversion (and no wait for the load) lands in the step that
  // issues the loads -- vmcnt counts in order, so waiting for a scale would also wait
  // for the codes issued just before it
  uint32_t sc_lo = 0x3F80u, sc_hi = 0x3F80u;

  // part 0: the activation-row DMAs (AJ of them); part 1: the weight-row DMAs
  // (bf16) or the weight-code loads into registers (fp8).
  auto issue_part = [&](auto rows_tag, const Tile& t, char* sA, char* sB, int k0, int part) {
    constexpr int AJ = decltype(rows_tag)::value / 32;
    const __amdgpu_buffer_rsrc_t rsrcA = act_rsrc<MODE>(X, a.T, K, t.p0, t.p1);
    const __amdgpu_buffer_rsrc_t rsrcB = weight_rsrc<FP8>(a.w, t.e, WR, K);
    if (part == 0) {
#pragma unroll
      for (int j = 0; j < AJ; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrcA, LDS_PTR(sA + (wave * AJ + j) * 1024), 16, aoff[j], k0 * 2, 0, 0);
    } else if constexpr (!FP8) {
#pragma unroll
      for (int j = 0; j < BJ; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrcB, LDS_PTR(sB + (wave * BJ + j) * 1024), 16, boff[j], k0 * 2, 0, 0);
    } else {
      // fp8 codes: part 1 all rows and both scales; 2: rows i < BJ / 2 and their scale;
      // 3: the other rows and theirs
#pragma unroll
      for (int i = 0; i < BJ; ++i)
        if (part == 1 || (part == 2) == (i < BJ / 2)) bq[i] = __builtin_amdgcn_raw_buffer_load_b64(rsrcB, boff[i], k0, 0);
      if (part != 3) sc_lo = reinterpret_cast<const uint16_t*>(a.wscale)[srow_lo + k0 / 128];
      if (part != 2) sc_hi = reinterpret_cast<const uint16_t*>(a.wscale)[srow_hi + k0 / 128];
    }
  };
  auto issue_loads = [&](auto rows_tag, const Tile& t, char* sA, char* sB, int k0) {
    issue_part(rows_tag, t, sA, sB, k0, 0);
    issue_part(rows_tag, t, sA, sB, k0, 1);
  };
  // micro tiles: one 128-deep stage (K columns [k0, k0 + 128)) into the 32 KB buffer dst:
  // the 64 activation rows at byte 0, the 64 weight rows at 16 KB; 4 + 4 DMAs of 1 KB per
  // wave
  auto issue_micro = [&](const Tile& t, char* dst, int k0) {
    const __amdgpu_buffer_rsrc_t rsrcA = act_rsrc<MODE>(X, a.T, K, t.p0, t.p1);
    const __amdgpu_buffer_rsrc_t rsrcB = weight_rsrc<FP8>(a.w, t.e, WR, K);
    const uint32_t base = lds_addr(dst) + wave * 4 * 1024;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_copy16(rsrcA, base + j * 1024, aoff[j], k0 * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_copy16(rsrcB, base + kMicroB + j * 1024, boff[j], k0 * 2);
  };
  // the next tile's first copies (its stage 0 or 1), in its own mode (outside any
  // scheduled region); a micro tile issues its own first stages
  auto issue_loads_for = [&](const Tile& t, char* sA, char* sB, int stage) {
    const int rows = tile_rows(t);
    if constexpr (kMicro) {
      if (rows & 1) return;
    }
    auto go = [&](auto rows_tag) { issue_loads(rows_tag, t, sA, sB, stage * BK); };
    if (rows == BM / 4)
      go(std::integral_constant<int, BM / 4>{});
    else if (rows == BM / 2)
      go(std::integral_constant<int, BM / 2>{});
    else
      go(std::integral_constant<int, BM>{});
  };
  // fp8 only: decode the staged codes, scale, round to bf16 and write the B tile
  // (part 0: rows rb + 32 i for i < BJ / 2; part 1: the rest; -1: all)
  auto store_fp8 = [&](char* sB, int part = -1) {
    if constexpr (FP8) {
#pragma unroll
      for (int i = 0; i < BJ; ++i) {
        if ((part == 0 && i >= BJ / 2) || (part == 1 && i < BJ / 2)) continue;
        const u32x2 q = bq[i];
        const float s = __uint_as_float((i < 4 ? sc_lo : sc_hi) << 16);  // bf16 -> fp32, exact
        const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[0], false);
        const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[0], true);
        const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[1], false);
        const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[1], true);
        // both products rounded to bf16 by one paired conversion (round to nearest even,
        // as a scalar cast would), low half first
        auto pack = [&](float lo, float hi) {
          return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo * s, hi * s}, bf16x2));
        };
        *reinterpret_cast<u32x4*>(sB + swz(rb + 32 * i, chunk)) =
            u32x4{pack(f0[0], f0[1]), pack(f1[0], f1[1]), pack(f2[0], f2[1]), pack(f3[0], f3[1])};
      }
    }
  };

  // ---- wave sub-tiles.  Full: rows [wm*128, +128), weight sub-tiles brf[0..3]
  // (W13: gate 0, 1 and up 2, 3).  Half: rows [0, 128), quarter: rows [0, 64); weight
  // sub-tiles brh[0..1] (W13: gate 0, up 1).
  const int wm = wave & 1, wn = wave >> 1;
  int brf[4], brh[2];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
    brf[ns] = MODE == 0 ? (ns < 2 ? wn * 64 + ns * 32 : TBN / 2 + wn * 64 + (ns - 2) * 32) : wn * 128 + ns * 32;
#pragma unroll
  for (int ns = 0; ns < 2; ++ns) brh[ns] = MODE == 0 ? ns * (TBN / 2) + wave * 32 : wave * 64 + ns * 32;
  const int khalf = lane >> 5;

  f32x16 acc[4][4];
  bf16x8 fw[4][4], fx[4][4];
  int next_lid = 0;

  // ---- one tile, in the mode of its rows R, from its first stage's barrier to its
  // epilogue.  The next tile's first two stages are copied during this tile's tail and
  // epilogue.
  auto run_tile = [&](auto rows_tag, const Tile& t, bool& more, Tile& nxt) {
    constexpr int R = decltype(rows_tag)::value;
    constexpr int NS = R == BM ? 4 : 2;        // weight sub-tiles per wave
    constexpr int MSUB = R == BM / 4 ? 2 : 4;  // 32-row activation sub-tiles per wave
    constexpr int AJ = R / 32;                 // activation DMAs per wave and stage
    const int* br = R == BM ? brf : brh;
    const int arow0 = R == BM ? wm * 128 : 0;
    // fragment addresses are computed per tile from an opaque copy of the lane
    // index: hoisted out of the tile loop, both modes' addresses would stay live
    // together and spill
    int l32 = lane & 31;
    asm volatile("" : "+v"(l32));

    // Fragments of one 16-wide K step: NS weight sub-tiles and 4 activation sub-tiles.
    auto load_frags = [&](const char* sA, const char* sB, int kk, bf16x8* wf, bf16x8* xf) {
      const int ch = kk * 2 + khalf;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) wf[ns] = *reinterpret_cast<const bf16x8*>(sB + swz(br[ns] + l32, ch));
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms) xf[ms] = *reinterpret_cast<const bf16x8*>(sA + swz(arow0 + ms * 32 + l32, ch));
    };
    // first: the tile's first K step, which starts every accumulator from zero
    auto mfma_step = [&](const bf16x8* wf, const bf16x8* xf, bool first) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms)
          acc[ns][ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ns], xf[ms], first ? f32x16{} : acc[ns][ms], 0, 0, 0);
    };
    // Software pipeline over fragments.  Four register sets hold the fragments of
    // the four 16-wide steps of a 64-deep stage.  Every block of MF MFMAs runs with
    // the RD reads of a later step spread between them, so LDS latency hides behind
    // the matrix core:
    //   [MFMA s.0 | read s.2] [MFMA s.1 | read s.3] barrier, DMA(stage s+2)
    //   [MFMA s.2 | read (s+1).0] [MFMA s.3 | read (s+1).1]
    // The reads of stage s+1 can start before its half-way barrier because that
    // barrier of stage s already waited for stage s+1's DMA.
    constexpr int MF = MSUB * NS, RD = NS + MSUB;
    auto step = [&](int mset, const char* sA, const char* sB, int kk, int lset, bool first = false) {
      load_frags(sA, sB, kk, fw[lset], fx[lset]);
      mfma_step(fw[mset], fx[mset], first);
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                           // MFMA
        if ((i * RD) / MF != ((i + 1) * RD) / MF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // The same, with the global loads of a later stage spread between the MFMAs
    // (a burst of them would stall the wave at issue while the matrix core idles).
    auto step_dma = [&](int mset, const char* sA, const char* sB, int kk, int lset, char* dA, char* dB, int k0,
                        int part) {
      load_frags(sA, sB, kk, fw[lset], fx[lset]);
      issue_part(rows_tag, t, dA, dB, k0, part);
      mfma_step(fw[mset], fx[mset], false);
      const int VM = part == 0 ? AJ : BJ;
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                           // MFMA
        if ((i * RD) / MF != ((i + 1) * RD) / MF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        if ((i * VM) / MF != ((i + 1) * VM) / MF) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // global load
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // fp8: the first two steps of a half.  dpart 0: the activation DMAs of the stage being
    // filled, the decode of the first half of its codes, then the next stage's codes of
    // that half (and their scale) at k0 = kcodes; dpart 1: the same for the second half.
    // Each half's registers are reloaded as soon as they are decoded, so the loads have
    // three steps to arrive.
    auto step_f8 = [&](int mset, const char* sA, const char* sB, int kk, int lset, char* dA, char* dB, int k0,
                       int dpart, int kcodes) {
      load_frags(sA, sB, kk, fw[lset], fx[lset]);
      if (dpart == 0) issue_part(rows_tag, t, dA, dB, k0, 0);
      store_fp8(dB, dpart);
      issue_part(rows_tag, t, dA, dB, kcodes, 2 + dpart);
      mfma_step(fw[mset], fx[mset], false);
      const int VM = dpart == 0 ? AJ + BJ / 2 + 1 : BJ / 2 + 1;
      constexpr int DW = BJ / 2;      // LDS writes of the decode
      constexpr int VA = 16 * DW / MF + 1;  // its VALU work per MFMA (about 16 per row)
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                           // MFMA
        if ((i * RD) / MF != ((i + 1) * RD) / MF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, VA, 0);                          // VALU (decode)
        if ((i * DW) / MF != ((i + 1) * DW) / MF) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
        if ((i * VM) / MF != ((i + 1) * VM) / MF) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // global load
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // Stage s of the K loop lives in buffer s & 1.  The DMA of stage s+2 is issued
    // right after the barrier that ends the reads of stage s, spread over the next
    // two steps.  K is a multiple of 128, so the stage count is even.  The loop is
    // rotated so that its head is a barrier (which waits for all LDS reads anyway),
    // its body is one basic block (so the scheduling barriers hold), and the last
    // two stages are peeled off: no copy is issued past the end of K.
    const int KT = K / BK;
    dma_barrier();
    int claim = 0;  // dynamic schedule: this workgroup's next tile, claimed now
    if (dyn && threadIdx.x == 0) claim = atomicAdd(a.work + xcd, 1);
    load_frags(sA0, sB0, 0, fw[0], fx[0]);
    load_frags(sA0, sB0, 1, fw[1], fx[1]);
    __builtin_amdgcn_sched_barrier(0);
    step(0, sA0, sB0, 2, 2, true);
    step(1, sA0, sB0, 3, 3);
    if constexpr (FP8) {
      // fp8 weights.  The codes of a stage are loaded into registers one half-stage
      // before they are decoded, and the decode (convert, scale, round, LDS write) of
      // stage s+1 is spread over the MFMAs of the first two steps of the half that frees
      // its buffer; the barrier then waits for all copies but the newest code loads.
      store_fp8(sB1);  // stage 1 (its codes were staged with the tile's first copies)
      issue_part(rows_tag, t, sA0, sB0, min(2, KT - 1) * BK, 1);
      // W13 also touches the token rows of the stage after next, as W2 with bf16 weights
      // does below (the loads after the next stage's codes: each head then leaves 11 loads
      // in flight).  fp8 W2 measured no faster with it.
      auto prefetch8 = [&](int k0) {
        return __builtin_amdgcn_raw_buffer_load_b32(act_rsrc<MODE>(X, a.T, K, t.p0, t.p1), poff, k0 * 2, 0);
      };
      auto head8 = [&](int pf) {
        if constexpr (MODE == 0) {
          __builtin_amdgcn_s_waitcnt(0x7B);  // vmcnt(11) expcnt(7) lgkmcnt(0)
          __syncthreads();
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("" ::"v"(pf));  // the previous prefetch has arrived: its register is free
        } else {
          fp8_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      int pf0 = 0, pf1 = 0;
      for (int kt = 0; kt < KT - 2; kt += 2) {
        head8(pf0);
        step_f8(2, sA1, sB1, 0, 0, sA0, sB0, (kt + 2) * BK, 0, (kt + 3) * BK);
        step_f8(3, sA1, sB1, 1, 1, sA0, sB0, (kt + 2) * BK, 1, (kt + 3) * BK);
        if constexpr (MODE == 0) pf0 = prefetch8((kt + 3) * BK);
        step(0, sA1, sB1, 2, 2);
        step(1, sA1, sB1, 3, 3);
        head8(pf1);
        step_f8(2, sA0, sB0, 0, 0, sA1, sB1, (kt + 3) * BK, 0, min(kt + 4, KT - 1) * BK);
        step_f8(3, sA0, sB0, 1, 1, sA1, sB1, (kt + 3) * BK, 1, min(kt + 4, KT - 1) * BK);
        if constexpr (MODE == 0) pf1 = prefetch8(min(kt + 4, KT - 1) * BK);
        step(0, sA0, sB0, 2, 2);
        step(1, sA0, sB0, 3, 3);
      }
      asm volatile("" ::"v"(pf0), "v"(pf1));
      // stage KT-1 is in buffer 1 (decoded above); the last code loads fetched nothing needed
      if (dyn && threadIdx.x == 0) sh_claim = claim;
      dma_barrier();
    } else {
      // W2 also touches the activation rows of the stage after next: one 4-byte load per
      // row (lane) brings that row's 128-byte line into L2, so the stage's copies, issued
      // one stage later, find it there instead of going to memory.  The loads land in
      // registers nobody reads; each stage head then waits for all loads but the newest
      // (the prefetch issued after the copies it needs), as a bare barrier, since the
      // workgroup fence of __syncthreads() would wait for the prefetch too.  With bf16
      // weights, W13's gathered token rows and the weight rows measured slower with the same.
      auto prefetch = [&](int k0) {
        return __builtin_amdgcn_raw_buffer_load_b32(act_rsrc<MODE>(X, a.T, K, t.p0, t.p1), poff, k0 * 2, 0);
      };
      auto head = [&](int pf) {
        if constexpr (MODE == 1) {
          __builtin_amdgcn_s_waitcnt(0x71);  // vmcnt(1) expcnt(7) lgkmcnt(0)
          bare_barrier();
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("" ::"v"(pf));  // the previous prefetch has arrived: its register is free
        } else {
          dma_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      int pf0 = 0, pf1 = 0;
      for (int kt = 0; kt < KT - 2; kt += 2) {
        head(pf0);
        step_dma(2, sA1, sB1, 0, 0, sA0, sB0, (kt + 2) * BK, 0);
        step_dma(3, sA1, sB1, 1, 1, sA0, sB0, (kt + 2) * BK, 1);
        if constexpr (MODE == 1) pf0 = prefetch((kt + 3) * BK);
        step(0, sA1, sB1, 2, 2);
        step(1, sA1, sB1, 3, 3);
        head(pf1);
        step_dma(2, sA0, sB0, 0, 0, sA1, sB1, (kt + 3) * BK, 0);
        step_dma(3, sA0, sB0, 1, 1, sA1, sB1, (kt + 3) * BK, 1);
        if constexpr (MODE == 1) pf1 = prefetch(min(kt + 4, KT - 1) * BK);
        step(0, sA0, sB0, 2, 2);
        step(1, sA0, sB0, 3, 3);
      }
      asm volatile("" ::"v"(pf0), "v"(pf1));
      // stages KT-2 (fragments 2, 3 in registers) and KT-1 (buffer 1)
      if (dyn && threadIdx.x == 0) sh_claim = claim;
      dma_barrier();
    }
    // buffer 0 is free: the next tile's stage 0 goes there now
    const int nlid = dyn ? run0 + __builtin_amdgcn_readfirstlane(sh_claim) : lid + slots;
    next_lid = nlid;
    more = nlid < lid_end;
    // The next tile's stage 0 goes to buffer 0 (free now).
    if (more) {
      decode(nlid, nxt);
      setup(nxt);
      issue_loads_for(nxt, sA0, sB0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    step(2, sA1, sB1, 0, 0);
    step(3, sA1, sB1, 1, 1);
    step(0, sA1, sB1, 2, 2);
    step(1, sA1, sB1, 3, 3);
    // every wave has read buffer 1: the next tile's stage 1 goes there
    if (more) {
      lds_barrier();
      store_fp8(sB0);
      issue_loads_for(nxt, sA1, sB1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(fw[2], fx[2], false);
    mfma_step(fw[3], fx[3], false);
    // route ids of this lane's four output rows, all in flight together
    int erid[4];
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms)
      erid[ms] = a.sorted != nullptr ? a.sorted[min(t.p0 + arow0 + ms * 32 + l32, t.p1 - 1)] : 0;

    // ---- epilogue.  Lane holds row (lane & 31) of each 32-row sub-tile and, per
    // register group g, the 4 consecutive columns 8 g + 4 (lane >> 5) + [0, 4) of a
    // weight sub-tile (W2: output columns; W13: act columns of a gate sub-tile, its
    // up partner NS/2 sub-tiles later).
    const int n0 = MODE == 0 ? t.nt * (TBN / 2) : t.nt * TBN;
    if constexpr (MODE == 0 && W13OUT) {
      // the pre-activation surface too: stored straight from the registers
      __bf16* act = (__bf16*)a.out;
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms) {
        const int p = t.p0 + arow0 + ms * 32 + l32;
        bool ok = p < t.p1;
        if (ok && a.sorted != nullptr) ok = (unsigned)erid[ms] < (unsigned)a.sentinel;
        if (!ok) continue;
#pragma unroll
        for (int ns = 0; ns < NS / 2; ++ns) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = n0 + br[ns] + g * 8 + khalf * 4;
            bf16x4 o, og, ou;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float gt = acc[ns][ms][g * 4 + q], up = acc[ns + NS / 2][ms][g * 4 + q];
              o[q] = (__bf16)(silu_fast(gt) * up);
              og[q] = (__bf16)gt;
              ou[q] = (__bf16)up;
            }
            *reinterpret_cast<bf16x4*>(act + (long)p * a.I + col) = o;
            __bf16* w13o = (__bf16*)a.w13_out + (long)p * 2 * a.I;
            *reinterpret_cast<bf16x4*>(w13o + col) = og;
            *reinterpret_cast<bf16x4*>(w13o + a.I + col) = ou;
          }
        }
      }
    } else {
      // The wave's output columns are contiguous: W13 the act columns of its gate
      // sub-tiles, W2 its weight sub-tiles.  Per 32-row sub-tile they go out in chunks of
      // up to 64 columns through the wave's LDS area: staged in the accumulator layout,
      // read back by row, and stored 16 B per lane with a row's chunk in consecutive lanes
      // (whole 128-byte lines) -- instead of 8 B into 32 different rows per store.  Only
      // this wave touches its area, and its LDS operations complete in order.
      constexpr int SUBS = MODE == 0 ? NS / 2 : NS;  // 32-column sub-tiles of the wave
      constexpr int CWS = SUBS >= 2 ? 2 : 1;          // of them per chunk
      constexpr int CW = CWS * 32;                    // chunk width, columns
      constexpr int RB = CW * 2 + 16;                 // staged row pitch, bytes
      constexpr int LPR = CW / 8;                     // lanes per row on the way out
      constexpr int RPI = kWave / LPR;                // rows per store
      static_assert(32 * RB <= kEpiWaveBytes, "epilogue staging area");
      char* stg = s_epi + wave * kEpiWaveBytes;
      __bf16* outp = (__bf16*)a.out;
      const long ld = MODE == 0 ? a.I : a.H;
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms) {
#pragma unroll
        for (int c = 0; c < SUBS / CWS; ++c) {
          const int col0 = n0 + br[c * CWS];
          // W2: a chunk past H (the last n-tile when H % 256 == 128) is staged but not stored
          const bool cols_ok = MODE == 0 || col0 < a.H;
#pragma unroll
          for (int nl = 0; nl < CWS; ++nl) {
            const int ns = c * CWS + nl;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              bf16x4 o;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                if constexpr (MODE == 0)
                  o[q] = (__bf16)(silu_fast(acc[ns][ms][g * 4 + q]) * acc[ns + NS / 2][ms][g * 4 + q]);
                else
                  o[q] = (__bf16)acc[ns][ms][g * 4 + q];
              }
              *reinterpret_cast<bf16x4*>(stg + l32 * RB + (nl * 32 + g * 8 + khalf * 4) * 2) = o;
            }
          }
          if constexpr (FP8 && MODE == 1) {
            // fp8 W2: one LDS round trip pair per store (reading ahead, as below, takes
            // registers that its K loop then spills)
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {
              const int rr = i * RPI + lane / LPR, c16 = lane % LPR;
              const int eid = __shfl(erid[ms], rr, kWave);  // lane rr holds row rr's route id
              const int p = t.p0 + arow0 + ms * 32 + rr;
              bool ok = cols_ok && p < t.p1;
              int dest = p;
              if (a.sorted != nullptr) {
                ok = ok && (unsigned)eid < (unsigned)a.sentinel;
                if (!a.dest_is_row) dest = eid;
              }
              const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rr * RB + c16 * 16);
              if (ok) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(outp + (long)dest * ld + col0 + c16 * 8));
            }
          } else {
            // the chunk's route ids and staged rows are all read before the first store,
            // so their LDS round trips overlap instead of one pair per store.  The stores
            // are non-temporal: this kernel never reads its output, and the output lines
            // then displace less of the operand tiles the XCD's workgroups share in L2
            constexpr int NR = 32 / RPI;
            const int c16 = lane % LPR;
            int eid[NR];
            u32x4 v[NR];
#pragma unroll
            for (int i = 0; i < NR; ++i) {
              const int rr = i * RPI + lane / LPR;
              eid[i] = __shfl(erid[ms], rr, kWave);  // lane rr holds row rr's route id
              v[i] = *reinterpret_cast<const u32x4*>(stg + rr * RB + c16 * 16);
            }
#pragma unroll
            for (int i = 0; i < NR; ++i) {
              const int rr = i * RPI + lane / LPR;
              const int p = t.p0 + arow0 + ms * 32 + rr;
              bool ok = cols_ok && p < t.p1;
              int dest = p;
              if (a.sorted != nullptr) {
                ok = ok && (unsigned)eid[i] < (unsigned)a.sentinel;
                if (MODE == 1 && !a.dest_is_row) dest = eid[i];
              }
              if (ok) __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4*>(outp + (long)dest * ld + col0 + c16 * 8));
            }
          }
        }
      }
    }
  };

  // ---- a micro tile (W2, bf16 weights): up to 64 activation rows x one quarter (64 rows)
  // of the weight n-tile, in 128-deep stages (32 KB: activation rows, then weight rows).
  // A small m-tile's K loop is latency-bound: with two stages its copies had one stage of
  // compute to arrive.  A micro tile's stages rotate through all four LDS arrays (stage s
  // in buffer s % 4), so the copies of three stages are in flight while one is multiplied;
  // and a small m-tile becomes four or eight micro tiles, spread over as many CUs.  Wave w
  // computes the 32 x 32 output block (activation rows 32 (w & 1), weight rows 32 (w >> 1)).
  // Same K order per output element as every other mode (one MFMA chain over K in
  // ascending 16-wide steps): no bit changes.
  auto run_tile_micro = [&](const Tile& t, bool& more, Tile& nxt) {
    constexpr int KS = 2 * BK;  // stage depth
    int l32 = lane & 31;
    asm volatile("" : "+v"(l32));
    const int arow = (wave & 1) * 32 + l32, wrow = (wave >> 1) * 32 + l32;
    const int KT = K / KS;  // even, >= 2: K is a multiple of 256 for micro tiles
    // every wave is done with the LDS of the previous tile: its last stage's fragment reads
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    bare_barrier();
    int claim = 0;
    if (dyn && threadIdx.x == 0) claim = atomicAdd(a.work + xcd, 1);
    issue_micro(t, sA0, 0);
    issue_micro(t, sB0, KS);
    if (KT > 2) issue_micro(t, sA1, 2 * KS);
    acc[0][0] = f32x16{};
    // Stage s from buffer cur: its head waits for this wave's copies of stage s (the 8
    // copies of each later stage already issued may stay in flight) and for its own LDS
    // reads, then the barrier; the copies of stage s + 3 then go to buffer fill, the
    // buffer of stage s - 1, which every wave has finished reading.
    auto stage = [&](int s, const char* cur, char* fill) {
      if (s + 2 < KT)
        __builtin_amdgcn_s_waitcnt(0x4070);  // vmcnt(16) expcnt(7) lgkmcnt(0)
      else if (s + 1 < KT)
        __builtin_amdgcn_s_waitcnt(0x78);    // vmcnt(8)
      else
        __builtin_amdgcn_s_waitcnt(0x70);    // vmcnt(0)
      bare_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (s + 3 < KT) issue_micro(t, fill, (s + 3) * KS);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 wf[8], xf[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int ch = kk * 2 + khalf;
        wf[kk] = *reinterpret_cast<const bf16x8*>(cur + kMicroB + swzn(wrow, ch));
        xf[kk] = *reinterpret_cast<const bf16x8*>(cur + swzn(arow, ch));
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk], xf[kk], acc[0][0], 0, 0, 0);
      // all 16 fragment reads first, then the MFMAs (each waits only for its own two)
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int s0 = 0; s0 < KT; s0 += 4) {
      stage(s0, sA0, sB1);
      stage(s0 + 1, sB0, sA0);
      if (s0 + 2 < KT) {
        stage(s0 + 2, sA1, sB0);
        stage(s0 + 3, sB1, sA1);
      }
    }
    // every wave has read its last stage: the next tile's first two stages (a full-height
    // tile's; a micro tile issues its own) may go to the buffers now
    if (dyn && threadIdx.x == 0) sh_claim = claim;
    __syncthreads();
    const int nlid = dyn ? run0 + __builtin_amdgcn_readfirstlane(sh_claim) : lid + slots;
    next_lid = nlid;
    more = nlid < lid_end;
    if (more) {
      decode(nlid, nxt);
      setup(nxt);
      issue_loads_for(nxt, sA0, sB0, 0);
      issue_loads_for(nxt, sA1, sB1, 1);
    }
    // epilogue: lane holds activation row (lane & 31) of the wave's block and, per register
    // group g, weight rows (output columns) 8 g + 4 (lane >> 5) + [0, 4) of its 32
    const int p = t.p0 + arow;
    const int erid = a.sorted != nullptr ? a.sorted[min(p, t.p1 - 1)] : 0;
    __bf16* y = (__bf16*)a.out;
    const int cbase = t.nt * TBN + (t.sub & 3) * (TBN / 4) + (wave >> 1) * 32;
    bool ok = p < t.p1 && cbase < a.H;
    int dest = p;
    if (a.sorted != nullptr) {
      ok = ok && (unsigned)erid < (unsigned)a.sentinel;
      if (!a.dest_is_row) dest = erid;
    }
    if (ok) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = (__bf16)acc[0][0][g * 4 + q];
        *reinterpret_cast<bf16x4*>(y + (long)dest * a.H + cbase + g * 8 + khalf * 4) = o;
      }
    }
  };

  setup(cur);
  issue_loads_for(cur, sA0, sB0, 0);
  store_fp8(sB0);
  issue_loads_for(cur, sA1, sB1, 1);
  while (true) {
    bool more = false;
    Tile nxt = cur;
    const int rows = tile_rows(cur);
    if constexpr (kMicro) {
      if (rows & 1) {
        run_tile_micro(cur, more, nxt);
        if (!more) break;
        cur = nxt;
        lid = next_lid;
        continue;
      }
    }
    if (rows == BM / 4)
      run_tile(std::integral_constant<int, BM / 4>{}, cur, more, nxt);
    else if (rows == BM / 2)
      run_tile(std::integral_constant<int, BM / 2>{}, cur, more, nxt);
    else
      run_tile(std::integral_constant<int, BM>{}, cur, more, nxt);
    if (!more) break;
    cur = nxt;
    lid = next_lid;
  }
  if (a.clk != nullptr && threadIdx.x == 0) clock_stamp(a.clk + 4 * blockIdx.x + 2);
}

// ---------------------------------------------------------------- fp32 path
// One thread per (row, output column); fmaf over K in ascending order.

__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int N, int p) {
  int lo = 0, hi = N;  // offsets[lo] <= p < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn_w13_f32(FfnArgs a, int rows) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)rows * a.I) return;
  const int p = (int)(i / a.I), col = (int)(i % a.I);
  int e = 0;
  const float* x;
  if (a.sorted == nullptr) {
    x = (const float*)a.x + (long)p * a.H;
  } else {
    if (p >= a.offsets[a.N]) return;
    const int r = a.sorted[p];
    if ((unsigned)r >= (unsigned)a.sentinel) return;
    e = expert_of_row(a.offsets, a.N, p);
    x = (const float*)a.x + (long)(r / a.k) * a.H;
  }
  const float* w1 = (const float*)a.w + ((long)e * 2 * a.I + col) * a.H;
  const float* w3 = w1 + (long)a.I * a.H;
  float u = 0.f, v = 0.f;
  for (int kk = 0; kk < a.H; ++kk) {
    u = fmaf(x[kk], w1[kk], u);
    v = fmaf(x[kk], w3[kk], v);
  }
  ((float*)a.out)[(long)p * a.I + col] = silu_f32(u) * v;
  if (a.w13_out != nullptr) {  // the pre-activation surface
    float* w13o = (float*)a.w13_out + (long)p * 2 * a.I;
    w13o[col] = u;
    w13o[a.I + col] = v;
  }
}

__global__ __launch_bounds__(256) void ffn_w2_f32(FfnArgs a, int rows) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)rows * a.H) return;
  const int p = (int)(i / a.H), col = (int)(i % a.H);
  int e = 0, dest = p;
  if (a.sorted != nullptr) {
    if (p >= a.offsets[a.N]) return;
    const int r = a.sorted[p];
    if ((unsigned)r >= (unsigned)a.sentinel) return;
    if (!a.dest_is_row) dest = r;
    e = expert_of_row(a.offsets, a.N, p);
  }
  const float* x = (const float*)a.x + (long)p * a.I;
  const float* w = (const float*)a.w + ((long)e * a.H + col) * a.I;
  float acc = 0.f;
  for (int kk = 0; kk < a.I; ++kk) acc = fmaf(x[kk], w[kk], acc);
  ((float*)a.out)[(long)dest * a.H + col] = acc;
}

int mtile_bound(const moe_config& c, bool identity) {
  if (identity) return ceil_div(c.T, BM);
  if (expert_choice(c)) return c.N * ceil_div(ec_segment(c), BM);
  const long p_max = (long)c.T * c.k + (long)c.N * (c.B - 1);
  return (int)((p_max + (long)c.N * (BM - 1)) / BM);
}

// Persistent launch: one workgroup per CU (the kernel's LDS allows no more), at most
// as many as there can be tiles, a multiple of the 8 XCDs.
template <int MODE, bool FP8, bool MICRO = false, bool W13OUT = false>
hipError_t launch_gemm(FfnArgs a, hipStream_t s) {
  int cus = 0;
  hipError_t err = current_device_cus(&cus);
  if (err != hipSuccess) return err;
  const int G = a.mtiles * a.ntiles;
  if (G == 0) return hipSuccess;  // no rows (an expert-choice capacity of 0)
  const int grid = ceil_div(min(G, max(cus, 8)), 8) * 8;
  if (grid > MOE_CLOCK_SLOTS) a.clk = nullptr;  // more workgroups than stamp slots: none
  ffn_gemm_bf16<MODE, FP8, MICRO, W13OUT><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

namespace {

FfnArgs base_args(const moe_config& c, const int32_t* sorted_ids, const int32_t* offsets, bool identity) {
  FfnArgs a{};
  a.sorted = identity ? nullptr : sorted_ids;
  a.offsets = identity ? nullptr : offsets;
  a.T = c.T;
  a.H = c.H;
  a.I = c.I;
  a.N = identity ? 1 : c.N;
  a.k = c.k;
  a.sentinel = c.T * c.k;
  a.mtiles = mtile_bound(c, identity);
  a.rows = identity ? c.T : c.T * c.k + c.N * (c.B - 1);
  if (!identity && expert_choice(c)) {  // rows hold token ids; y is written by padded row
    a.k = 1;
    a.sentinel = c.T;
    a.rows = c.N * ec_segment(c);
    a.dest_is_row = 1;
  }
  return a;
}

}  // namespace

hipError_t launch_gate_up(const moe_config& c, const void* h, const int32_t* sorted_ids, const int32_t* offsets,
                          const void* w13, const void* w13_scale, void* act, void* w13_out, bool identity,
                          hipStream_t s, int32_t* work, uint64_t* clk) {
  FfnArgs a = base_args(c, sorted_ids, offsets, identity);
  a.work = work;
  a.clk = clk;
  a.x = h;
  a.w = w13;
  a.wscale = (const __bf16*)w13_scale;
  a.out = act;
  a.w13_out = w13_out;
  if (c.expert_dtype == MOE_F32) {
    const long n = (long)a.rows * c.I;
    if (n == 0) return hipSuccess;
    ffn_w13_f32<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(a, a.rows);
    return hipGetLastError();
  }
  a.ntiles = c.I / (BN / 2);
  if (w13_out != nullptr)
    return c.expert_dtype == MOE_FP8_E4M3 ? launch_gemm<0, true, false, true>(a, s)
                                          : launch_gemm<0, false, false, true>(a, s);
  return c.expert_dtype == MOE_FP8_E4M3 ? launch_gemm<0, true>(a, s) : launch_gemm<0, false>(a, s);
}

hipError_t launch_down(const moe_config& c, const void* act, const int32_t* sorted_ids, const int32_t* offsets,
                       const void* w2, const void* w2_scale, void* y, bool identity, hipStream_t s,
                       int32_t* work, uint64_t* clk) {
  FfnArgs a = base_args(c, sorted_ids, offsets, identity);
  a.work = work;
  a.clk = clk;
  a.x = act;
  a.w = w2;
  a.wscale = (const __bf16*)w2_scale;
  a.out = y;
  if (c.expert_dtype == MOE_F32) {
    const long n = (long)a.rows * c.H;
    if (n == 0) return hipSuccess;
    ffn_w2_f32<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(a, a.rows);
    return hipGetLastError();
  }
  a.ntiles = ceil_div(c.H, 256);
  // Micro tiles need 128-deep stages in pairs (K a multiple of 256).  They pay where the
  // tiles make one to four rounds over the CUs: the short tiles, last in the order, then
  // fill the final round (fewer tiles: the longest tile sets the time anyway; more: the
  // last round is a small part, and keeping an expert's m-tiles together saves weight
  // re-reads).  Each expert's last m-tile may take eight m-slots instead of one.
  int cus = 0;
  hipError_t err = current_device_cus(&cus);
  if (err != hipSuccess) return err;
  const long tiles = (long)a.mtiles * a.ntiles;
  a.micro = c.expert_dtype == MOE_BF16 && c.I % 256 == 0 && tiles > cus && tiles <= 4L * cus;
  if (a.micro) {
    a.mtiles += 7 * a.N;
    return launch_gemm<1, false, true>(a, s);
  }
  return c.expert_dtype == MOE_FP8_E4M3 ? launch_gemm<1, true>(a, s) : launch_gemm<1, false>(a, s);
}

hipError_t launch_expert_ffn(const moe_config& c, const void* h, const int32_t* sorted_ids, const int32_t* offsets,
                             const void* w13, const void* w2, const void* w13_scale, const void* w2_scale, void* act,
                             void* w13_out, void* y, bool identity, hipStream_t s, int32_t* work) {
  hipError_t err = launch_gate_up(c, h, sorted_ids, offsets, w13, w13_scale, act, w13_out, identity, s, work);
  if (err != hipSuccess) return err;
  return launch_down(c, act, sorted_ids, offsets, w2, w2_scale, y, identity, s,
                     work ? work + kGemmWorkWords : nullptr);
}

}  // namespace moe
