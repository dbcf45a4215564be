// Expert-choice routing: each expert takes its C highest-scoring tokens.
//
// "Mixture-of-experts routing & LLM repeatability", paragraph on expert-choice routing:
// the assignment is turned around, and each expert takes its highest-scoring tokens out
// of the whole batch.  "Mixture-of-Experts Routing at Inference Time", "Integration: where
// routing lives in a serving stack", paragraph on expert-choice routing: each expert picks
// up to its capacity, so none overflows, and a token may be picked by no expert.
//
// Selection (ec_select, one 1024-thread workgroup per expert):
//  - every token's score for the expert becomes a 32-bit order key (float_order_key: a
//    larger score has a larger key, NaN the smallest), held in registers: thread i holds
//    tokens i, i + 1024, ...;
//  - a radix select over the key's four bytes, high to low, finds the C-th largest key:
//    per byte, a 256-bin count of the tokens still matching the chosen prefix (a wave
//    adds each bin once, from a ballot peer mask), then one wave finds the bin where the
//    running count from the top reaches the picks still needed.  Counting is order-free;
//  - tokens above that key are picked; of the tokens equal to it, the lowest token
//    indices fill the remaining picks.  Both the tie rank and the output position are
//    prefix counts in token order (ballots within a wave, waves added in order), so
//    the picks come out in ascending token order with no atomic deciding anything.
// Alignment (ec_align_*): every expert has exactly C picks, so its segment is the fixed
// row range [e * Cp, e * Cp + C) of whole B-row blocks, Cp = ceil(C / B) * B, with the
// sentinel T after the picks; only the token ids and the per-token pick counts vary.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// The float whose float_order_key is k (k = 0: NaN).
__device__ __forceinline__ float key_value(uint32_t k) {
  if (k == 0u) return __builtin_nanf("");
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Exclusive prefix count of `flag` over the workgroup in thread order; `total` gets the
// workgroup's count.  Called by every thread; `wave_tot` is kSelWaves ints of LDS.
__device__ __forceinline__ int block_prefix(bool flag, int* wave_tot, int& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint64_t bal = __ballot(flag);
  if (lane == 0) wave_tot[wave] = __popcll(bal);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int c = wave_tot[w];
    before += w < wave ? c : 0;
    total += c;
  }
  __syncthreads();
  return before + __popcll(bal & ((1ull << lane) - 1ull));
}

// J: key slots per thread (tokens tid + 1024 j, j < J); J * 1024 >= T.
template <int J>
__global__ __launch_bounds__(kSelThreads) void ec_select(const float* __restrict__ scores, int T, int N, int C,
                                                         int32_t* __restrict__ tokens, int32_t* __restrict__ slot,
                                                         float* __restrict__ margin) {
  __shared__ int hist[256];
  __shared__ int wave_tot[kSelWaves];
  __shared__ uint32_t wave_max[kSelWaves];
  __shared__ int sh_digit, sh_above, sh_eq;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint64_t lower = (1ull << lane) - 1ull;

  // all J loads in flight together: the index is clamped rather than the load guarded
  // (a guarded load gets its own branch and a wait of its own)
  uint32_t key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int t = tid + j * kSelThreads;
    const float v = scores[(size_t)min(t, T - 1) * N + e];
    key[j] = float_order_key(v) & (t < T ? 0xFFFFFFFFu : 0u);  // a mask, not a select: the
                                                               // compiler sinks a load used on one side only
  }

  if (C == 0) {  // nothing to pick
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int t = tid + j * kSelThreads;
      if (t < T) slot[(size_t)t * N + e] = -1;
    }
    if (margin && tid == 0) margin[e] = __builtin_inff();
    return;
  }

  // ---- radix select of the C-th largest key
  uint32_t prefix = 0;
  int rem = C;  // picks still to be found among the keys matching the prefix
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int t = tid + j * kSelThreads;
      const bool match = t < T && (pass == 0 || (key[j] >> (shift + 8)) == prefix);
      const int d = match ? (int)((key[j] >> shift) & 255u) : 256;
      const uint64_t peers = peer_mask(d);
      if (match && (peers & lower) == 0) atomicAdd(&hist[d], __popcll(peers));
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds the bins 255 - 4l, ..., 252 - 4l (descending digits)
      int c[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[255 - 4 * lane - i];
        sum += c[i];
      }
      int above = wave_incl_scan_i32(sum) - sum;  // keys in higher bins than this lane's first
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < rem && rem <= above + c[i]) {  // exactly one bin of the workgroup
          sh_digit = 255 - 4 * lane - i;
          sh_above = above;
          sh_eq = c[i];
        }
        above += c[i];
      }
    }
    __syncthreads();
    prefix = (prefix << 8) | (uint32_t)sh_digit;
    rem -= sh_above;
  }
  const uint32_t thr = prefix;  // the C-th largest key
  const int ties_at_thr = sh_eq;  // tokens whose key equals thr (rem of them are picked)

  // ---- margin: the C-th score minus the (C+1)-th
  if (C < T) {
    uint32_t next = thr;  // a tie at the cut: the (C+1)-th has the same key
    if (rem == ties_at_thr) {  // every tie was picked: the largest key below thr
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int t = tid + j * kSelThreads;
        if (t < T && key[j] < thr) m = key[j] > m ? key[j] : m;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t x = (uint32_t)__shfl_xor((int)m, o, kWave);
        m = x > m ? x : m;
      }
      if (lane == 0) wave_max[wave] = m;
      __syncthreads();
      next = 0;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) next = wave_max[w] > next ? wave_max[w] : next;
    }
    if (margin && tid == 0) margin[e] = key_value(thr) - key_value(next);
  } else if (margin && tid == 0) {
    margin[e] = __builtin_inff();
  }

  // ---- picks in token order
  int ties_before = 0, picks_before = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j * kSelThreads >= T) break;  // uniform
    const int t = tid + j * kSelThreads;
    const bool valid = t < T;
    const bool tie = valid && key[j] == thr;
    int tot;
    const int tie_rank = ties_before + block_prefix(tie, wave_tot, tot);
    ties_before += tot;
    const bool pick = valid && (key[j] > thr || (tie && tie_rank < rem));
    const int pos = picks_before + block_prefix(pick, wave_tot, tot);
    picks_before += tot;
    if (pick && pos < C) tokens[(size_t)e * C + pos] = t;  // pos < C holds by construction
    if (valid) slot[(size_t)t * N + e] = pick ? pos : -1;
  }
}

template <int J>
hipError_t launch_select_j(const moe_config& c, int C, const float* scores, int32_t* tokens, int32_t* slot,
                           float* margin, hipStream_t s) {
  ec_select<J><<<c.N, kSelThreads, 0, s>>>(scores, c.T, c.N, C, tokens, slot, margin);
  return hipGetLastError();
}

// Offsets, padded row count, the fixed statistics, the GEMM work counters; clears the
// two per-token counters that ec_align_rows adds to.  One workgroup.
__global__ __launch_bounds__(256) void ec_align_init(int N, int C, int Cp, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ num_padded, int32_t* __restrict__ stats,
                                                     int32_t* __restrict__ zero, int nzero) {
  for (int e = threadIdx.x; e <= N; e += blockDim.x) offsets[e] = e * Cp;
  for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0;
  if (stats) {
    for (int e = threadIdx.x; e < N; e += blockDim.x) stats[e] = C;
    if (threadIdx.x == 0) {
      int32_t* x = stats + N;
      x[MOE_STAT_KEPT] = N * C;
      x[MOE_STAT_DROPPED] = 0;
      x[MOE_STAT_INVALID] = 0;
      x[MOE_STAT_CAPACITY] = C;
      x[MOE_STAT_MAX_LOAD] = C;
      x[MOE_STAT_MIN_LOAD] = C;
      x[MOE_STAT_NUM_PADDED] = N * Cp;
      x[MOE_STAT_REROUTED] = 0;
      x[MOE_STAT_UNPICKED] = 0;
      x[MOE_STAT_MAX_PICKS] = 0;
    }
  }
  if (threadIdx.x == 0) num_padded[0] = N * Cp;
}

// Thread i: padded row i (token id or sentinel, and the block's expert at a block's first
// row) and token i's pick count (integer sums and maxima: the order of the atomics cannot
// change them).
__global__ __launch_bounds__(256) void ec_align_rows(const int32_t* __restrict__ tokens,
                                                     const int32_t* __restrict__ slot, int T, int N, int C, int Cp,
                                                     int B, int32_t* __restrict__ sorted_ids,
                                                     int32_t* __restrict__ block_expert, int32_t* __restrict__ stats) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int P = N * Cp;
  if (i < P) {
    const int e = i / Cp, c = i - e * Cp;
    sorted_ids[i] = c < C ? tokens[(size_t)e * C + c] : T;
    if (c % B == 0) block_expert[i / B] = e;
  }
  if (stats == nullptr) return;
  int picks = 0;
  const bool tok = i < T;
  if (tok) {
    const int32_t* row = slot + (size_t)i * N;
    if ((N & 3) == 0 && ((uintptr_t)slot & 15) == 0) {
      for (int x = 0; x < N; x += 4) {
        const int4 v = *reinterpret_cast<const int4*>(row + x);
        picks += (v.x >= 0) + (v.y >= 0) + (v.z >= 0) + (v.w >= 0);
      }
    } else {
      for (int x = 0; x < N; ++x) picks += row[x] >= 0;
    }
  }
  const int unpicked = __popcll(__ballot(tok && picks == 0));
  int m = picks;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0 && blockIdx.x * blockDim.x + (int)threadIdx.x < T) {
    if (unpicked) atomicAdd(stats + N + MOE_STAT_UNPICKED, unpicked);
    atomicMax(stats + N + MOE_STAT_MAX_PICKS, m);
  }
}

}  // namespace

hipError_t launch_ec_select(const moe_config& c, const float* scores, int32_t* tokens, int32_t* slot, float* margin,
                            hipStream_t s) {
  const int C = ec_capacity(c);
  const int J = ceil_div(c.T, kSelThreads);
  if (J <= 1) return launch_select_j<1>(c, C, scores, tokens, slot, margin, s);
  if (J <= 2) return launch_select_j<2>(c, C, scores, tokens, slot, margin, s);
  if (J <= 4) return launch_select_j<4>(c, C, scores, tokens, slot, margin, s);
  if (J <= 8) return launch_select_j<8>(c, C, scores, tokens, slot, margin, s);
  if (J <= 16) return launch_select_j<16>(c, C, scores, tokens, slot, margin, s);
  if (J <= 32) return launch_select_j<32>(c, C, scores, tokens, slot, margin, s);
  return launch_select_j<64>(c, C, scores, tokens, slot, margin, s);  // T <= 65536
}

hipError_t launch_ec_align(const moe_config& c, const int32_t* tokens, const int32_t* slot, int32_t* sorted_ids,
                           int32_t* block_expert, int32_t* offsets, int32_t* num_padded, int32_t* stats,
                           hipStream_t s, int32_t* zero, int nzero) {
  const int C = ec_capacity(c), Cp = ec_segment(c);
  ec_align_init<<<1, 256, 0, s>>>(c.N, C, Cp, offsets, num_padded, stats, zero, nzero);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n = max(c.N * Cp, c.T);
  ec_align_rows<<<ceil_div(n, 256), 256, 0, s>>>(tokens, slot, c.T, c.N, C, Cp, c.B, sorted_ids, block_expert, stats);
  return hipGetLastError();
}

}  // namespace moe
