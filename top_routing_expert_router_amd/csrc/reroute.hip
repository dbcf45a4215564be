// Capacity with the reroute overflow policy.
//
// "Mixture-of-Experts Routing at Inference Time", "The hard part", Figure 2: a
// token routed to an expert that is at capacity is either dropped or rerouted --
// sent to its second-choice expert -- and the mitigation paragraph after the
// routing-stats probe: change the overflow policy from drop to reroute.
//
// Policy (rounds; the config's reroute_depth is the number of rounds):
//  1. the drop policy fills capacity in ascending route id (a route runs its expert
//     iff fewer than cap earlier routes chose that expert);
//  2. per round, every token with an overflowed route offers its lowest such route
//     one new candidate: the next expert in the token's ranking of its logits
//     (value descending, lower index first, NaN last, -0 == +0) that is not among
//     its recorded ids and was not offered before.  Requests to an expert are
//     admitted in token order while it has room left.  An admitted route runs the
//     candidate with its original gate.
// Depth 1 is the literal "second choice"; depth N - k walks the whole ranking.
//
// Each token's ranking of all its experts is computed first, spread over the GPU
// (reroute_rank); a round then takes a token's next candidate from it in constant time.
// One workgroup does the rest: the decisions chain through the remaining capacity,
// round after round.  Every position in token or route order is a prefix count --
// ballot peer masks inside a wave, waves added in order -- so no atomic decides an
// order; LDS atomics only add up totals.  The alignment proper then runs on the
// experts the routes ended up with (dropless: every route with an expert runs it).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRThreads = 1024;
constexpr int kRWaves = kRThreads / kWave;

// order[t * N + r] = the expert of rank r in token t's ranking of its logits (value
// descending, lower index first, NaN last, -0 == +0: the order of rank_key).  A group of L
// lanes per token (N rounded up to a power of two, at most 64): the token's keys are staged
// in LDS, and a lane ranks experts l, l + L, ... by counting the keys above each.  Keys are
// distinct (they hold the index), so the ranks are a permutation.
template <int L>
__global__ __launch_bounds__(256) void reroute_rank(const float* __restrict__ logits, int T, int N,
                                                    uint8_t* __restrict__ order) {
  constexpr int TPB = 256 / L;  // tokens per workgroup; TPB * N <= 1024
  __shared__ uint64_t key[1024];
  const long t0 = (long)blockIdx.x * TPB;
  const int nt = (int)min((long)TPB, (long)T - t0);
  for (int i = threadIdx.x; i < nt * N; i += 256) key[i] = rank_key(logits[t0 * N + i], i % N);
  __syncthreads();
  const int g = threadIdx.x / L, l = threadIdx.x % L;
  if (g >= nt) return;
  const uint64_t* kt = key + g * N;
  for (int e = l; e < N; e += L) {
    const uint64_t ke = kt[e];
    int r = 0;
    for (int j = 0; j < N; ++j) r += kt[j] > ke ? 1 : 0;
    order[(t0 + g) * N + r] = (uint8_t)e;
  }
}

// Position of each of this thread's C keys (0..N-1; -1 = none) among the keys before it,
// plus base[key]; afterwards base[key] has grown by the count of that key.  Thread i's key
// c is entry c * NT + i of the run (chunk c of NT entries, in thread order).  Peer masks
// from ballots within a wave; per key, the wave counts of chunk 0, then of chunk 1, ...,
// added in that order: no atomic decides a position.  Called by every thread of the
// NT-thread workgroup; cnt is [C * NT / 64][256] ints of LDS.
template <int NT, int C>
__device__ void chunk_positions(const int (&key)[C], int (&pos)[C], int N, int* base, int (*cnt)[256]) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int i = tid; i < C * NW * N; i += NT) cnt[i / N][i % N] = 0;
  __syncthreads();
  uint64_t peers[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const bool valid = key[c] >= 0;
    peers[c] = peer_mask(valid ? key[c] : 256);
    if (valid && (peers[c] & lt) == 0) cnt[c * NW + wave][key[c]] = __popcll(peers[c]);  // one writer
  }
  __syncthreads();
  for (int e = tid; e < N; e += NT) {
    int acc = base[e];
    for (int w = 0; w < C * NW; ++w) {
      const int x = cnt[w][e];
      cnt[w][e] = acc;
      acc += x;
    }
    base[e] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < C; ++c) pos[c] = key[c] >= 0 ? cnt[c * NW + wave][key[c]] + __popcll(peers[c] & lt) : -1;
  __syncthreads();
}

// Two chunks of tokens (or routes) per step: half the barriers of one chunk at a time.
constexpr int kRChunks = 2;

__global__ __launch_bounds__(kRThreads) void reroute_capacity(const int32_t* __restrict__ ids,
                                                              const uint8_t* __restrict__ order, int T, int N,
                                                              int k, int cap, int depth,
                                                              int32_t* __restrict__ route_expert,
                                                              int32_t* __restrict__ next,
                                                              int32_t* __restrict__ stats) {
  __shared__ int base[256], room[256];
  __shared__ int cnt[kRChunks * kRWaves][256];
  __shared__ int sh_any, sh_kept, sh_rer, sh_invalid, sh_max, sh_min;
  const int tid = threadIdx.x;
  const int R = T * k;
  for (int e = tid; e < N; e += kRThreads) base[e] = 0;
  if (tid == 0) {
    sh_kept = 0;
    sh_rer = 0;
    sh_invalid = 0;
    sh_max = 0;
    sh_min = 0x7fffffff;
  }
  __syncthreads();

  // 1. drop-policy fill in route-id order
  for (int r0 = 0; r0 < R; r0 += kRChunks * kRThreads) {
    int key[kRChunks], pos[kRChunks];
#pragma unroll
    for (int c = 0; c < kRChunks; ++c) {
      const int r = r0 + c * kRThreads + tid;
      const int e = r < R ? ids[r] : -1;
      key[c] = e >= 0 && e < N ? e : -1;
    }
    chunk_positions<kRThreads, kRChunks>(key, pos, N, base, cnt);
#pragma unroll
    for (int c = 0; c < kRChunks; ++c) {
      const int r = r0 + c * kRThreads + tid;
      if (r < R) route_expert[r] = (key[c] >= 0 && (cap < 0 || pos[c] < cap)) ? key[c] : -1;
    }
  }
  // base[e] is now expert e's routed load (before capacity)
  for (int e = tid; e < N; e += kRThreads) {
    room[e] = cap < 0 ? 0 : cap - min(base[e], cap);
    atomicMax(&sh_max, base[e]);
    atomicMin(&sh_min, base[e]);
    if (stats) stats[e] = base[e];
  }
  for (int t = tid; t < T; t += kRThreads) next[t] = 0;  // rank of the next candidate to look at
  __syncthreads();

  // 2. rounds
  for (int round = 0; cap >= 0 && round < depth; ++round) {
    for (int e = tid; e < N; e += kRThreads) base[e] = 0;
    if (tid == 0) sh_any = 0;
    __syncthreads();
    for (int t00 = 0; t00 < T; t00 += kRChunks * kRThreads) {
      int want[kRChunks], route[kRChunks], pos[kRChunks];
#pragma unroll
      for (int c = 0; c < kRChunks; ++c) {
        const int t = t00 + c * kRThreads + tid;
        want[c] = -1;
        route[c] = -1;
        if (t < T) {
          const int32_t* tid_ids = ids + (size_t)t * k;
          for (int j = 0; j < k; ++j) {
            const int e = tid_ids[j];
            if (e >= 0 && e < N && route_expert[t * k + j] < 0) {
              route[c] = t * k + j;
              break;
            }
          }
          if (route[c] >= 0) {
            // the next candidate: the next expert down the token's ranking that is not one
            // of its own (none once the ranking is used up)
            int own[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) own[j] = j < k ? tid_ids[j] : -1;
            const uint8_t* ot = order + (size_t)t * N;
            int r = next[t];
            while (r < N && want[c] < 0) {
              const int e = ot[r++];
              bool mine = false;
#pragma unroll
              for (int j = 0; j < 8; ++j) mine |= own[j] == e;
              if (!mine) want[c] = e;
            }
            next[t] = r;
          }
        }
      }
      chunk_positions<kRThreads, kRChunks>(want, pos, N, base, cnt);
#pragma unroll
      for (int c = 0; c < kRChunks; ++c) {
        if (want[c] >= 0) {
          sh_any = 1;
          if (pos[c] < room[want[c]]) route_expert[route[c]] = want[c];
        }
      }
    }
    __syncthreads();
    // base[e] = requests to e this round; the first room[e] of them were admitted
    for (int e = tid; e < N; e += kRThreads) room[e] -= min(base[e], room[e]);
    const int any = sh_any;
    __syncthreads();
    if (!any) break;
  }

  // 3. totals
  int kept = 0, rer = 0, invalid = 0;
  for (int r = tid; r < R; r += kRThreads) {
    const int e = ids[r], x = route_expert[r];
    invalid += (e < 0 || e >= N) ? 1 : 0;
    kept += x >= 0 ? 1 : 0;
    rer += (x >= 0 && x != e) ? 1 : 0;
  }
  atomicAdd(&sh_kept, kept);
  atomicAdd(&sh_rer, rer);
  atomicAdd(&sh_invalid, invalid);
  __syncthreads();
  if (stats && tid == 0) {
    stats[N + MOE_STAT_KEPT] = sh_kept;
    stats[N + MOE_STAT_DROPPED] = (R - sh_invalid) - sh_kept;
    stats[N + MOE_STAT_INVALID] = sh_invalid;
    stats[N + MOE_STAT_CAPACITY] = cap;
    stats[N + MOE_STAT_MAX_LOAD] = sh_max;
    stats[N + MOE_STAT_MIN_LOAD] = sh_min;
    stats[N + MOE_STAT_REROUTED] = sh_rer;
    stats[N + MOE_STAT_UNPICKED] = 0;  // expert-choice counters
    stats[N + MOE_STAT_MAX_PICKS] = 0;
  }
}

}  // namespace

// the rankings (T x N bytes, with reroute rounds only) and the walk positions (T ints)
static size_t ranking_bytes(const moe_config& c) {
  return c.reroute_depth > 0 ? (((size_t)c.T * c.N + 255) & ~(size_t)255) : 0;
}
size_t reroute_workspace_bytes(const moe_config& c) {
  return ranking_bytes(c) + (((size_t)c.T * 4 + 255) & ~(size_t)255);
}

hipError_t launch_align_reroute(const moe_config& c, const int32_t* ids, const float* logits, int32_t* route_expert,
                                uint8_t* kept, int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                                int32_t* num_padded, int32_t* stats, void* ws, hipStream_t s, int32_t* zero,
                                int nzero) {
  int cap = -1;
  if (!(c.cap_num == 0 && c.cap_den == 0)) {
    const long long cl = ((long long)c.T * c.k * c.cap_num) / ((long long)c.N * c.cap_den);
    cap = cl > 0x7fffffffLL ? 0x7fffffff : (int)cl;
  }
  uint8_t* order = (uint8_t*)ws;
  int32_t* next = (int32_t*)((char*)ws + ranking_bytes(c));
  if (cap >= 0 && c.reroute_depth > 0 && c.T > 0) {
    auto rank = [&](auto lanes) {
      constexpr int L = decltype(lanes)::value;
      reroute_rank<L><<<(c.T + 256 / L - 1) / (256 / L), 256, 0, s>>>(logits, c.T, c.N, order);
    };
    if (c.N <= 2) rank(std::integral_constant<int, 2>{});
    else if (c.N <= 4) rank(std::integral_constant<int, 4>{});
    else if (c.N <= 8) rank(std::integral_constant<int, 8>{});
    else if (c.N <= 16) rank(std::integral_constant<int, 16>{});
    else if (c.N <= 32) rank(std::integral_constant<int, 32>{});
    else rank(std::integral_constant<int, 64>{});
  }
  reroute_capacity<<<1, kRThreads, 0, s>>>(ids, order, c.T, c.N, c.k, cap, c.reroute_depth, route_expert, next,
                                           stats);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // the alignment of the routes as they run: dropless on route_expert
  moe_config d = c;
  d.cap_num = 0;
  d.cap_den = 0;
  return launch_align(d, route_expert, kept, sorted_ids, block_expert, offsets, num_padded, stats,
                      (char*)ws + reroute_workspace_bytes(c), s, zero, nzero, true);
}

}  // namespace moe
