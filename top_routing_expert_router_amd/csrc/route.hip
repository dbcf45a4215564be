// Router: projection h . W_g^T to one fp32 logit per expert, then top-k with the
// lowest-index tie rule, renormalised softmax gates and the router margin.
//
// "Mixture-of-Experts Routing at Inference Time", "How sparse routing works" and
// "Worked example: a top-k router": W_g projects h to N logits; softmax; keep the
// top k; renormalise their gates.  "Mixture-of-experts routing & LLM
// repeatability": top-k is fixed by the scores and the tie rule; the margin is
// the gap between the k-th and (k+1)-th scores.
//
// Batch invariance ("Why temperature=0 Still Gives Different Answers: Batch
// Invariance", "How do I make LLM inference reproducible?", tier 2): each logit
// is reduced in a fixed order that depends only on H and on N's kernel (up to 64
// experts: 64-wide K chunks dealt to eight waves round-robin, each wave in ascending
// chunk order, then the eight wave partials added in wave order; more than 64: one
// MFMA chain over K in ascending 32-wide steps).  Nothing depends on T or on the
// other tokens.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRouterTokens = 16;   // tokens per MFMA column block (a workgroup takes TB blocks)
constexpr int kRouterWaves = 8;     // waves per workgroup; wave w takes K chunks w, w+8, ...
constexpr int kRouterThreads = kRouterWaves * 64;
constexpr int kChunkK = 64;         // K per chunk: lane group q = lane / 16 holds k in [16 q, 16 q + 16)

// chunks in flight per wave: a CU's whole share of h for 16 experts, four for up to 64
template <int NSUB>
struct RouterUnroll {
  static_assert(NSUB >= 1 && NSUB <= 4, "the 16-token router takes up to 64 experts");
  static constexpr int value = NSUB <= 1 ? 8 : 4;
};

typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x8_t __attribute__((ext_vector_type(8)));
// buffer resource word 3 for raw (untyped, stride 0) buffer loads on gfx9-family parts
constexpr int kRawBufferFlags = 0x00020000;

// 32 bytes at byte offset off + soff of a raw buffer, as 16 bf16 (two 16-byte loads)
__device__ __forceinline__ bf16x16 load32(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, soff, 0);
  return __builtin_bit_cast(bf16x16, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Top-k, gates and margin of one token from its N logits (global or LDS), by one
// aligned group of L = topk_lanes(N) lanes; a wave ranks 64 / L tokens at once.
// Lane g of the group holds experts g + L i, i < P.  k+1 rounds of a group max over
// (value, -index) keys give the ranked ids and the (k+1)-th logit for the margin.
// Gate weight_j = exp(l_j - l_0) (0 for a NaN logit); divided by the sum over the
// k chosen in rank order, or by the sum over all N experts without renormalisation.
// Replay ("Mixture-of-experts routing & LLM repeatability", router replay paragraph):
// with recorded ids the experts are those ids in their recorded order, ids are not
// written, and weight_j = exp(l_{id_j} - m), m the largest recorded logit (an id
// outside [0, N) weighs 0); the margin is still this run's.  Replaying a run's own
// ids gives its gates bit for bit (same values, same order, m = l_0).
// Expert-choice scores (scores != null; "Mixture-of-experts routing & LLM repeatability",
// paragraph on expert-choice routing): every expert's softmax value exp(l_e - l_0) / sum
// over all N, written to scores[t, :] instead of ids, gates and margin -- the same
// operations, so a token's top-k scores equal its gates with renormalize = 0 bit for bit.
// P = experts per lane actually used (ceil(N / L), at most kTopkPerLane): slots past it
// hold no expert, so they are left out at compile time (topk_one picks P); the result is
// the same for every P that covers N.
// L, P and the mode (plain, replay, scores) are compile-time: each kernel then holds only
// the code of its own case.  A kernel that carried every case was ~50 KB of code, and the
// first pass of each CU through it (every launch, after the expert GEMMs have filled the
// instruction caches) cost about 2 us of the Mixtral-shape router's 13.
enum : int { kTopkPlain = 0, kTopkReplay = 1, kTopkScores = 2 };
__host__ __device__ constexpr int topk_mode(const int32_t* replay, const float* scores) {
  return scores != nullptr ? kTopkScores : (replay != nullptr ? kTopkReplay : kTopkPlain);
}
// smallest of 1, 2, 4, 8 that is at least v (v <= 8)
constexpr int topk_slots(int v) { return v <= 1 ? 1 : (v <= 2 ? 2 : (v <= 4 ? 4 : 8)); }

template <int P, int L, int MODE, typename RowPtr>
__device__ __forceinline__ void topk_one_p(RowPtr row, int t, int N, int k, int renormalize,
                                           int32_t* __restrict__ ids, float* __restrict__ gates,
                                           float* __restrict__ margin, const int32_t* __restrict__ replay,
                                           float* __restrict__ scores) {
  static_assert(P >= 1 && P <= kTopkPerLane, "experts per lane");
  static_assert(L == 8 || L == 16 || L == 32, "lanes per token");
  const int lane = threadIdx.x & 63;
  const int g = lane & (L - 1), base = lane - g;
  float lv[P];
  uint64_t key[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = g + L * i;
    lv[i] = e < N ? row[e] : 0.f;
    key[i] = e < N ? rank_key(lv[i], e) : 0ull;
  }
  if constexpr (MODE == kTopkScores) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < P; ++i) best = key[i] > best ? key[i] : best;
    best = group_max_u64(best, L);
    const int e0 = (int)(0xFFFFFFFFu - (uint32_t)best);
    const int owner = e0 & (L - 1), slot = e0 / L;
    float mine = lv[0];
#pragma unroll
    for (int i = 1; i < P; ++i) mine = slot == i ? lv[i] : mine;
    const float l0 = __shfl(mine, base + owner, kWave);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = g + L * i;
      if (e < N && lv[i] == lv[i]) z += expf(lv[i] - l0);
    }
    const float sum = group_sum_f32(z, L);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = g + L * i;
      if (e < N) scores[(size_t)t * N + e] = (lv[i] == lv[i] ? expf(lv[i] - l0) : 0.f) / sum;
    }
    return;
  }
  const int rounds = k < N ? k + 1 : k;
  float sl[9];
  int sid[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    sl[j] = 0.f;
    sid[j] = 0;
    if (j < rounds) {
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < P; ++i) best = key[i] > best ? key[i] : best;
      best = group_max_u64(best, L);
      const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
      const int owner = e & (L - 1), slot = e / L;
      float mine = lv[0];
#pragma unroll
      for (int i = 1; i < P; ++i) mine = slot == i ? lv[i] : mine;
      sl[j] = __shfl(mine, base + owner, kWave);
      sid[j] = e;
      if (g == owner) {
#pragma unroll
        for (int i = 0; i < P; ++i)
          if (i == slot) key[i] = 0ull;
      }
    }
  }
  const float l0 = sl[0];
  float w[8];
  float s = 0.f;
  if constexpr (MODE != kTopkReplay) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w[j] = 0.f;
      if (j < k) {
        w[j] = (sl[j] != sl[j]) ? 0.f : expf(sl[j] - l0);
        s += w[j];
      }
    }
  } else {
    float rl[8];
    float m = -__builtin_inff();
    int rid[8];  // all recorded ids in flight together (index clamped into the token's k)
#pragma unroll
    for (int j = 0; j < 8; ++j) rid[j] = replay[(size_t)t * k + min(j, k - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rl[j] = __builtin_nanf("");
      if (j < k) {
        const int id = rid[j];
        if ((unsigned)id < (unsigned)N) rl[j] = row[id];
        m = rl[j] > m ? rl[j] : m;  // NaN never wins
      }
    }
    const float ref = renormalize ? m : l0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w[j] = 0.f;
      if (j < k) {
        w[j] = (rl[j] != rl[j]) ? 0.f : expf(rl[j] - ref);
        s += w[j];
      }
    }
  }
  if (!renormalize) {
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = g + L * i;
      if (e < N && lv[i] == lv[i]) z += expf(lv[i] - l0);
    }
    s = group_sum_f32(z, L);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k && g == j) {
      if constexpr (MODE != kTopkReplay) ids[(size_t)t * k + j] = sid[j];
      gates[(size_t)t * k + j] = w[j] / s;
    }
  }
  if (margin && g == 0) {
    float m = __builtin_inff();
#pragma unroll
    for (int j = 1; j < 9; ++j)
      if (j == k && k < N) m = sl[j - 1] - sl[j];
    margin[t] = m;
  }
}

// P = the smallest of 1, 2, 4, 8 that covers N; the caller's N lies where that choice is
// one of [PMIN, PMAX], so only those are compiled.
template <int L, int PMIN, int PMAX, int MODE, typename RowPtr>
__device__ __forceinline__ void topk_one(RowPtr row, int t, int N, int k, int renormalize,
                                         int32_t* __restrict__ ids, float* __restrict__ gates,
                                         float* __restrict__ margin, const int32_t* __restrict__ replay,
                                         float* __restrict__ scores) {
  static_assert(PMIN <= PMAX && PMAX <= kTopkPerLane, "slot window");
  const int per = ceil_div(N, L);  // uniform
  if constexpr (PMIN <= 1 && 1 < PMAX)
    if (per <= 1) return topk_one_p<1, L, MODE>(row, t, N, k, renormalize, ids, gates, margin, replay, scores);
  if constexpr (PMIN <= 2 && 2 < PMAX)
    if (per <= 2) return topk_one_p<2, L, MODE>(row, t, N, k, renormalize, ids, gates, margin, replay, scores);
  if constexpr (PMIN <= 4 && 4 < PMAX)
    if (per <= 4) return topk_one_p<4, L, MODE>(row, t, N, k, renormalize, ids, gates, margin, replay, scores);
  topk_one_p<PMAX, L, MODE>(row, t, N, k, renormalize, ids, gates, margin, replay, scores);
}

// bf16 router on MFMA 16x16x32, with top-k fused: D[expert][token] = sum_k W_g[expert][k] h[token][k].
// Per 64-wide K chunk each lane loads 32 contiguous bytes of its token row (a whole
// 128-byte line per row and instruction) and of its expert row, and issues two MFMAs
// (the first and second 8 elements of its 16).  Wave w accumulates chunks w, w+4, ...
// in ascending order; the eight wave partials are added in wave order; nothing depends
// on T or on the other tokens.
template <int NSUB, int TB, int MODE, int P>
__global__ __launch_bounds__(kRouterThreads) void router_bf16(const __bf16* __restrict__ h, const __bf16* __restrict__ wg,
                                                   const float* __restrict__ bias, float* __restrict__ logits,
                                                   int32_t* __restrict__ ids, float* __restrict__ gates,
                                                   float* __restrict__ margin, int T, int H, int N, int k,
                                                   int renormalize, const int32_t* __restrict__ replay,
                                                   float* __restrict__ scores) {
  constexpr int NP = NSUB * 16, TW = TB * kRouterTokens;
  __shared__ float part[kRouterWaves][NP][TW];
  __shared__ float lg[TW][NP + 1];
  // the wave index made scalar: the chunk offsets of the buffer loads below are then
  // scalar operands (a vector one turns every load into a waterfall loop)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * TW;
  const int col = lane & 15, kq = (lane >> 4) * 16;
  // Buffer loads: token columns past T and expert rows past N (the padding of the last
  // 16-expert block) start at the buffer's end, so they read zeros without a memory
  // request (bounds-checked loads never fault); their accumulator entries are never
  // written out.
  const uint32_t hbytes = (uint32_t)T * H * 2u, wbytes = (uint32_t)N * H * 2u;  // T H < 2^31
  const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc((void*)h, (short)0, (int)hbytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void*)wg, (short)0, (int)wbytes, kRawBufferFlags);
  uint32_t hoff[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int t = t0 + b * 16 + col;
    hoff[b] = t < T ? ((uint32_t)t * H + kq) * 2u : hbytes;
  }
  uint32_t woff[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) woff[s] = s * 16 + col < N ? ((uint32_t)(s * 16 + col) * H + kq) * 2u : wbytes;
  const int nchunks = H / kChunkK;

  f32x4 acc[NSUB][TB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[s][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int kUnroll = RouterUnroll<NSUB>::value;
  auto mfma2 = [&](f32x4& acc, const bf16x16& wv, const bf16x16& hv) {
    const bf16x8 hlo = __builtin_shufflevector(hv, hv, 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 hhi = __builtin_shufflevector(hv, hv, 8, 9, 10, 11, 12, 13, 14, 15);
    const bf16x8 wlo = __builtin_shufflevector(wv, wv, 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 whi = __builtin_shufflevector(wv, wv, 8, 9, 10, 11, 12, 13, 14, 15);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wlo, hlo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi, hhi, acc, 0, 0, 0);
  };
  const bf16x16 zero16 = bf16x16{};
  for (int c0 = wave; c0 < nchunks; c0 += kRouterWaves * kUnroll) {
    // Every load of this round is issued before the first MFMA.  A chunk slot past
    // the end of H (which slots exist depends on H only) re-reads the last chunk
    // and has its activations replaced by zeros, adding exact zeros to the sums.
    bf16x16 hv[kUnroll][TB];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = min(c0 + u * kRouterWaves, nchunks - 1);
#pragma unroll
      for (int b = 0; b < TB; ++b) hv[u][b] = load32(hrs, hoff[b], c * kChunkK * 2);
    }
    bf16x16 wv[kUnroll][NSUB];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = min(c0 + u * kRouterWaves, nchunks - 1);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) wv[u][s] = load32(wrs, woff[s], c * kChunkK * 2);
    }
    // without this barrier the compiler moves each weight load next to the MFMAs that
    // use it and waits for it there, one load in flight per wave
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool in = c0 + u * kRouterWaves < nchunks;
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int b = 0; b < TB; ++b) mfma2(acc[s][b], wv[u][s], in ? hv[u][b] : zero16);
    }
  }
  // lane holds token column (lane & 15), expert rows 4*(lane>>4) + r
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave][s * 16 + (lane >> 4) * 4 + r][b * 16 + col] = acc[s][b][r];
  __syncthreads();
  // this thread's biases for its entries, all loads in flight together (index clamped)
  constexpr int kPer = (NP * TW + kRouterThreads - 1) / kRouterThreads;
  float bv[kPer];
  if (bias) {
#pragma unroll
    for (int m = 0; m < kPer; ++m) bv[m] = bias[min(((int)threadIdx.x + m * kRouterThreads) / TW, N - 1)];
  }
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int i = threadIdx.x + m * kRouterThreads;
    const int e = i / TW, t = i % TW;
    if (i >= NP * TW || e >= N) continue;
    float v = part[0][e][t];
#pragma unroll
    for (int w = 1; w < kRouterWaves; ++w) v += part[w][e][t];
    if (bias) v += bv[m];
    lg[t][e] = v;
    if (logits && t0 + t < T) logits[(size_t)(t0 + t) * N + e] = v;  // nullable: no logits out
  }
  __syncthreads();
  // fused top-k: one group of L lanes per token, 64 / L tokens per wave.  The launch
  // takes NSUB = ceil(N / 16) <= 4, so L = topk_lanes(N) = 8, and P = topk_slots(ceil(N /
  // 8)) (the launch picks the kernel).
  constexpr int L = 8;
  constexpr int per_wave = kWave / L;
  for (int t = wave * per_wave + lane / L; t < TW; t += kRouterWaves * per_wave)
    if (t0 + t < T) topk_one_p<P, L, MODE>(&lg[t][0], t0 + t, N, k, renormalize, ids, gates, margin, replay, scores);
}

// bf16 router for more than 64 experts, top-k fused: the K chunks stream through an LDS
// ring.  A workgroup of 8 waves takes TW tokens; each 64-wide K chunk of all NP (padded)
// expert rows of W_g and of the TW token rows is copied global -> LDS as one stage of RS
// rows (NP + TW rounded up to 64: 128-byte rows, 16-byte chunks XORed with (row >> 1) & 7),
// S stages in the ring, so the copies of S - 1 chunks are in flight while one is multiplied.
// Wave w owns expert blocks [w EPW, (w + 1) EPW) of 16 for all TW tokens: its logits are
// one 16x16x32 MFMA chain over K in ascending 32-wide steps (W_g rows as the A operand),
// then the bias is added.  No partial sums cross waves, and nothing depends on T or TW.
// The copies are inline assembly and the stage heads bare barriers with the ring's own
// waits (the compiler's wait-count pass cannot tell the stages apart).  Expert rows past
// N, token rows past T and the padding rows start at their buffer's end: zeros, no fetch.
template <int NP, int TW, int S, int MODE>
__global__ __launch_bounds__(512) void router_ring(const __bf16* __restrict__ h, const __bf16* __restrict__ wg,
                                                   const float* __restrict__ bias, float* __restrict__ logits,
                                                   int32_t* __restrict__ ids, float* __restrict__ gates,
                                                   float* __restrict__ margin, int T, int H, int N, int k,
                                                   int renormalize, const int32_t* __restrict__ replay,
                                                   float* __restrict__ scores) {
  constexpr int NW = 8;
  constexpr int RS = (NP + TW + 63) / 64 * 64;  // rows per stage
  constexpr int SB = RS * 128;                   // bytes per stage
  constexpr int IPW = RS / 64;                   // copies (8 rows each) per wave and stage
  constexpr int EB = NP / 16, TB = TW / 16;      // 16-row expert blocks, 16-token blocks
  constexpr int EPW = EB / NW;                   // expert blocks per wave
  static_assert(EPW >= 1 && EB % NW == 0 && TW % 16 == 0 && S >= 3, "tile shape");
  static_assert(S * SB >= TW * (NP + 1) * 4, "the logit rows reuse the ring");
  static_assert(S - 2 <= 3, "head waits below cover up to three later stages");
  __shared__ __attribute__((aligned(16))) char ring[S * SB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TW;
  const uint32_t hbytes = (uint32_t)T * H * 2u, wbytes = (uint32_t)N * H * 2u;  // T H < 2^31
  const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc((void*)h, (short)0, (int)hbytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void*)wg, (short)0, (int)wbytes, kRawBufferFlags);
  // copy plan: copy i of wave w moves rows [8 (w IPW + i), +8); lane L lands in physical
  // chunk L % 8 of row 8 (w IPW + i) + L / 8 and fetches the logical chunk stored there.
  // A copy's 8 rows are all expert rows or all token (or padding) rows: NP and TW are
  // multiples of 16.
  uint32_t voff[IPW];
  bool wrow[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int g = wave * IPW + i;              // copy group, uniform
    const int r = g * 8 + (lane >> 3);
    const int lchunk = (lane & 7) ^ ((r >> 1) & 7);
    wrow[i] = g * 8 < NP;
    if (wrow[i]) {
      voff[i] = r < N ? ((uint32_t)r * H + lchunk * 8) * 2u : wbytes;
    } else {
      const int t = t0 + r - NP;
      voff[i] = (r < NP + TW && t < T) ? ((uint32_t)t * H + lchunk * 8) * 2u : hbytes;
    }
  }
  const uint32_t ring0 = lds_addr(ring);
  auto issue = [&](int c, int b) {
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      lds_copy16(wrow[i] ? wrs : hrs, ring0 + b * SB + (wave * IPW + i) * 1024, voff[i], c * 128);
  };
  const int nchunks = H / 64;
  f32x4 acc[EPW][TB];
#pragma unroll
  for (int eb = 0; eb < EPW; ++eb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[eb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this wave's biases (index clamped into [0, N)), loaded before the loop
  float bv[EPW][4];
#pragma unroll
  for (int eb = 0; eb < EPW; ++eb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      bv[eb][r] = bias ? bias[min((wave * EPW + eb) * 16 + 4 * (lane >> 4) + r, N - 1)] : 0.f;
  auto swz = [](int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); };
  const int l16 = lane & 15, q = lane >> 4;
  for (int c = 0; c < S - 1 && c < nchunks; ++c) issue(c, c);
  for (int c = 0; c < nchunks; ++c) {
    // head: this wave's copies of chunk c have landed (those of the later chunks already
    // issued may be in flight) and its reads of chunk c - 1 are done; then the barrier,
    // and chunk c + S - 1 goes to the buffer of chunk c - 1
    const int later = min(S - 2, nchunks - 1 - c);
    if (later >= 3)
      __builtin_amdgcn_s_waitcnt((3 * IPW & 15) | ((3 * IPW >> 4) << 14) | 0x70);
    else if (later == 2)
      __builtin_amdgcn_s_waitcnt((2 * IPW & 15) | ((2 * IPW >> 4) << 14) | 0x70);
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt((IPW & 15) | ((IPW >> 4) << 14) | 0x70);
    else
      __builtin_amdgcn_s_waitcnt(0x70);
    bare_barrier();
    if (c + S - 1 < nchunks) issue(c + S - 1, (c + S - 1) % S);
    const char* st = ring + (c % S) * SB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {  // 32-wide K steps: lane group q holds k in [32 s + 8 q, +8)
      bf16x8 wf[EPW], tf[TB];
#pragma unroll
      for (int eb = 0; eb < EPW; ++eb)
        wf[eb] = *reinterpret_cast<const bf16x8*>(st + swz((wave * EPW + eb) * 16 + l16, 4 * s + q));
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) tf[tb] = *reinterpret_cast<const bf16x8*>(st + swz(NP + tb * 16 + l16, 4 * s + q));
#pragma unroll
      for (int eb = 0; eb < EPW; ++eb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[eb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[eb], tf[tb], acc[eb][tb], 0, 0, 0);
    }
  }
  // logits of the TW tokens, [TW][NP + 1] floats over the ring: lane holds token l16 of
  // each token block and experts 4 q + r of each of its expert blocks
  __syncthreads();
  float* lg = reinterpret_cast<float*>(ring);
#pragma unroll
  for (int eb = 0; eb < EPW; ++eb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = (wave * EPW + eb) * 16 + 4 * q + r;
        float v = acc[eb][tb][r];
        if (bias && e < N) v += bv[eb][r];
        lg[(tb * 16 + l16) * (NP + 1) + e] = v;
      }
  __syncthreads();
  if (logits) {  // nullable: no logits out
    for (int i = tid; i < TW * N; i += NW * 64) {
      const int t = i / N, e = i - t * N;
      if (t0 + t < T) logits[(size_t)(t0 + t) * N + e] = lg[t * (NP + 1) + e];
    }
  }
  // one group of L lanes per token, 64 / L tokens per wave: N in (64, NP] with NP = 128 or
  // 256 gives L = topk_lanes(N) = NP / 8 and 5 to 8 experts per lane
  constexpr int L = NP / 8;
  static_assert(NP == 128 || NP == 256, "lanes per token below");
  constexpr int per_wave = kWave / L;
  for (int t = wave * per_wave + lane / L; t < TW; t += NW * per_wave)
    if (t0 + t < T)
      topk_one_p<8, L, MODE>(lg + t * (NP + 1), t0 + t, N, k, renormalize, ids, gates, margin, replay, scores);
}

// fp32 projection: one thread per (token, expert), fmaf over H in ascending order.
__global__ __launch_bounds__(256) void router_logits_f32(const float* __restrict__ h, const float* __restrict__ wg,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int T, int H, int N) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)T * N) return;
  const int t = (int)(i / N), e = (int)(i % N);
  const float* x = h + (size_t)t * H;
  const float* w = wg + (size_t)e * H;
  float acc = 0.f;
  for (int kk = 0; kk < H; ++kk) acc = fmaf(x[kk], w[kk], acc);
  if (bias) acc += bias[e];
  logits[i] = acc;
}

// Standalone top-k over stored logits (fp32 path and routing from given logits):
// 256 threads, one group of L = topk_lanes(N) lanes per token, 256 / L tokens per
// workgroup.  L = 8 covers 1 to 64 experts (1 to 8 per lane); 16 and 32 take 65 to 128
// and 129 to 256 experts, 5 to 8 per lane.
template <int L, int MODE>
__global__ __launch_bounds__(256) void topk_gates(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                   float* __restrict__ gates, float* __restrict__ margin,
                                                   int T, int N, int k, int renormalize,
                                                   const int32_t* __restrict__ replay, float* __restrict__ scores) {
  const int t = blockIdx.x * (256 / L) + threadIdx.x / L;
  if (t >= T) return;
  topk_one<L, L == 8 ? 1 : 8, 8, MODE>(logits + (size_t)t * N, t, N, k, renormalize, ids, gates, margin, replay,
                                       scores);
}

template <int NSUB, int MODE>
hipError_t launch_router_bf16(const moe_config& c, const void* h, const void* wg, const float* bias, float* logits,
                              int32_t* ids, float* gates, float* margin, hipStream_t s, const int32_t* replay,
                              float* scores) {
  constexpr int TB = 1;
  constexpr int L = 8;
  // the slots per lane for N in (16 (NSUB - 1), 16 NSUB]: two choices for NSUB = 1, one above
  constexpr int PMIN = topk_slots((16 * (NSUB - 1) + L) / L), PMAX = topk_slots((16 * NSUB + L - 1) / L);
  static_assert(PMIN == PMAX || (NSUB == 1 && PMIN == 1 && PMAX == 2), "slot choices");
  dim3 grid(ceil_div(c.T, TB * kRouterTokens));
  if (PMIN != PMAX && topk_slots(ceil_div(c.N, L)) == PMIN)
    router_bf16<NSUB, TB, MODE, PMIN><<<grid, kRouterThreads, 0, s>>>((const __bf16*)h, (const __bf16*)wg, bias, logits,
                                                                     ids, gates, margin, c.T, c.H, c.N, c.k,
                                                                     c.renormalize, replay, scores);
  else
    router_bf16<NSUB, TB, MODE, PMAX><<<grid, kRouterThreads, 0, s>>>((const __bf16*)h, (const __bf16*)wg, bias, logits,
                                                                     ids, gates, margin, c.T, c.H, c.N, c.k,
                                                                     c.renormalize, replay, scores);
  return hipGetLastError();
}
template <int NSUB>
hipError_t launch_router_bf16(const moe_config& c, const void* h, const void* wg, const float* bias, float* logits,
                              int32_t* ids, float* gates, float* margin, hipStream_t s, const int32_t* replay,
                              float* scores) {
  switch (topk_mode(replay, scores)) {
    case kTopkScores:
      return launch_router_bf16<NSUB, kTopkScores>(c, h, wg, bias, logits, ids, gates, margin, s, replay, scores);
    case kTopkReplay:
      return launch_router_bf16<NSUB, kTopkReplay>(c, h, wg, bias, logits, ids, gates, margin, s, replay, scores);
    default:
      return launch_router_bf16<NSUB, kTopkPlain>(c, h, wg, bias, logits, ids, gates, margin, s, replay, scores);
  }
}

template <int NP, int MODE>
hipError_t launch_router_ring(const moe_config& c, const void* h, const void* wg, const float* bias, float* logits,
                              int32_t* ids, float* gates, float* margin, hipStream_t s, const int32_t* replay,
                              float* scores) {
  int cus = 0;
  hipError_t err = current_device_cus(&cus);
  if (err != hipSuccess) return err;
  // 256 experts: 64 tokens per workgroup when that still gives every CU a workgroup, else
  // 32; stages of 40 KB, three in the ring.  128 experts: 32 tokens, stages of 24 KB, five.
  if constexpr (NP == 256) {
    if (ceil_div(c.T, 64) >= cus) {
      router_ring<256, 64, 3, MODE><<<ceil_div(c.T, 64), 512, 0, s>>>((const __bf16*)h, (const __bf16*)wg, bias, logits,
                                                                       ids, gates, margin, c.T, c.H, c.N, c.k,
                                                                       c.renormalize, replay, scores);
      return hipGetLastError();
    }
    router_ring<256, 32, 3, MODE><<<ceil_div(c.T, 32), 512, 0, s>>>((const __bf16*)h, (const __bf16*)wg, bias, logits,
                                                                     ids, gates, margin, c.T, c.H, c.N, c.k,
                                                                     c.renormalize, replay, scores);
  } else {
    router_ring<128, 32, 5, MODE><<<ceil_div(c.T, 32), 512, 0, s>>>((const __bf16*)h, (const __bf16*)wg, bias, logits,
                                                                     ids, gates, margin, c.T, c.H, c.N, c.k,
                                                                     c.renormalize, replay, scores);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const moe_config& c, const void* h, const void* w_gate, const float* bias, float* logits,
                         int32_t* ids, float* gates, float* margin, hipStream_t s, const int32_t* replay,
                         float* scores) {
  if (c.act_dtype == MOE_F32) {
    const long n = (long)c.T * c.N;
    router_logits_f32<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>((const float*)h, (const float*)w_gate, bias,
                                                                        logits, c.T, c.H, c.N);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_topk(c, logits, ids, gates, margin, s, replay, scores);
  }
  // more than 64 experts: every workgroup reads all of W_g, so it streams through an LDS
  // ring shared by the waves, 32 or 64 tokens per workgroup (Qwen shape: 32.8 -> 23.7 us
  // against the 16-token kernel with two column blocks; DeepSeek shape: 123 -> 120.5 us
  // against a register-staged kernel)
  if (c.N > 64) {
    auto ring = [&](auto np) {
      constexpr int NP = decltype(np)::value;
      switch (topk_mode(replay, scores)) {
        case kTopkScores:
          return launch_router_ring<NP, kTopkScores>(c, h, w_gate, bias, logits, ids, gates, margin, s, replay, scores);
        case kTopkReplay:
          return launch_router_ring<NP, kTopkReplay>(c, h, w_gate, bias, logits, ids, gates, margin, s, replay, scores);
        default:
          return launch_router_ring<NP, kTopkPlain>(c, h, w_gate, bias, logits, ids, gates, margin, s, replay, scores);
      }
    };
    return c.N > 128 ? ring(std::integral_constant<int, 256>{}) : ring(std::integral_constant<int, 128>{});
  }
  switch (ceil_div(c.N, 16)) {  // N <= 64 here: the 16-token kernel
    case 1: return launch_router_bf16<1>(c, h, w_gate, bias, logits, ids, gates, margin, s, replay, scores);
    case 2: return launch_router_bf16<2>(c, h, w_gate, bias, logits, ids, gates, margin, s, replay, scores);
    case 3: return launch_router_bf16<3>(c, h, w_gate, bias, logits, ids, gates, margin, s, replay, scores);
    default: return launch_router_bf16<4>(c, h, w_gate, bias, logits, ids, gates, margin, s, replay, scores);
  }
}

hipError_t launch_topk(const moe_config& c, const float* logits, int32_t* ids, float* gates, float* margin,
                       hipStream_t s, const int32_t* replay, float* scores) {
  const int L = topk_lanes(c.N);
  dim3 grid(ceil_div(c.T, 256 / L));
  auto go = [&](auto lanes, auto mode) {
    topk_gates<decltype(lanes)::value, decltype(mode)::value><<<grid, 256, 0, s>>>(logits, ids, gates, margin, c.T, c.N,
                                                                                 c.k, c.renormalize, replay, scores);
  };
  auto by_mode = [&](auto lanes) {
    switch (topk_mode(replay, scores)) {
      case kTopkScores: go(lanes, std::integral_constant<int, kTopkScores>{}); break;
      case kTopkReplay: go(lanes, std::integral_constant<int, kTopkReplay>{}); break;
      default: go(lanes, std::integral_constant<int, kTopkPlain>{}); break;
    }
  };
  if (L == 8)
    by_mode(std::integral_constant<int, 8>{});
  else if (L == 16)
    by_mode(std::integral_constant<int, 16>{});
  else
    by_mode(std::integral_constant<int, 32>{});
  return hipGetLastError();
}

}  // namespace moe
