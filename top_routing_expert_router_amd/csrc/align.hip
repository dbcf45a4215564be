// Capacity and alignment: a deterministic stable counting sort of the kept routes
// by (expert id, flattened route id), padded to whole B-row blocks per expert.
//
// "Route-Block Membership Selects Packed-AWQ Arithmetic": routed rows are grouped
// by expert and padded into fixed-size blocks ("The bookkeeping before the matrix
// multiplication"); the stable construction orders valid routes by expert id and
// flattened route id instead of atomic arrival order ("Stable construction
// selected a third trajectory").  "Mixture-of-experts routing & LLM
// repeatability", paragraph on expert capacity: capacity = tokens/experts x
// factor, overflow skips the expert, capacity is filled in order -- here in
// ascending route id.  "Mixture-of-Experts Routing at Inference Time", "Worked
// example" and "The hard part": per-expert load = bincount of the flattened ids;
// dropped = sum of max(load - capacity, 0).
//
// Up to 8192 routes: one workgroup does all three (align_fused).  Else three
// kernels on one stream:
//   hist    : per chunk of kChunk routes, per-expert counts (LDS atomics only count;
//             a count does not depend on the order the increments land in)
//   scan    : one workgroup: per expert, exclusive prefix of the chunk counts (in
//             place), capacity, padded segment sizes, expert offsets, block map, stats
//   scatter : per chunk, each route's position among the routes to its expert is
//             chunk prefix + the count of earlier routes in the chunk with the same
//             expert (ballot peer masks, waves in order) -- no atomic decides a slot.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kChunk = 1024;        // routes per chunk (4 waves x 4 steps x 64 lanes)
constexpr int kThreads = 256;
constexpr int kStepsPerWave = kChunk / (4 * kWave);

__global__ __launch_bounds__(kThreads) void align_hist(const int32_t* __restrict__ ids, int R, int N,
                                                       int32_t* __restrict__ counts) {
  __shared__ int cnt[257];
  for (int i = threadIdx.x; i <= N; i += kThreads) cnt[i] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * kChunk + threadIdx.x;
  int my[kChunk / kThreads];
#pragma unroll
  for (int j = 0; j < kChunk / kThreads; ++j) my[j] = ids[min(r0 + j * kThreads, R - 1)];  // all in flight
#pragma unroll
  for (int j = 0; j < kChunk / kThreads; ++j) {
    const int e = my[j];
    if (r0 + j * kThreads < R) atomicAdd(&cnt[(e >= 0 && e < N) ? e : N], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i <= N; i += kThreads) counts[(size_t)blockIdx.x * (N + 1) + i] = cnt[i];
}

// Per-expert layout from the routed loads, run by every thread of an NT-thread
// workgroup (thread e < N holds expert e's load; thread 0 also the invalid count):
// capacity, padded segment sizes, expert offsets (exclusive scan over experts in
// order), sentinel pads inside each segment, the block -> expert map, the stats, and
// the zeroed words.  Returns expert e's offset; *total_out = padded row count.
// The pads and block entries of each expert are written by a group of G threads, G the
// largest power of two with G N <= NT (at least 1), striding over its rows and blocks:
// with few experts one thread walking each expert's up to B - 1 pads and its blocks was
// most of the one-workgroup alignment's time; with as many experts as threads (G = 1)
// that walk is the fastest.
template <int NT>
__device__ int layout_experts(int load, int invalid, int N, int B, int cap, int n_blocks,
                              int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded,
                              int32_t* __restrict__ stats, int sentinel, int32_t* __restrict__ zero, int nzero,
                              int stats_ready, int* total_out) {
  constexpr int NW = NT / kWave;
  __shared__ int wave_tot[NW];
  __shared__ int red[NW][3];
  __shared__ int seg[2][256 + 1];  // per expert: first row of its segment (seg[0][N] = total), kept rows
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  for (int i = e; i < nzero; i += NT) zero[i] = 0;
  const int kept = e < N ? (cap < 0 ? load : min(load, cap)) : 0;
  const int padded = ceil_div(kept, B) * B;
  // exclusive scan of padded sizes over experts: per wave, then across waves in order
  const int incl = wave_incl_scan_i32(padded);
  if (lane == 63) wave_tot[wave] = incl;
  // per-wave partial stats (kept sum, max load, min load over valid experts)
  int ksum = wave_sum_i32(kept);
  int mx = e < N ? load : 0, mn = e < N ? load : 0x7fffffff;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    mx = max(mx, __shfl_xor(mx, m, kWave));
    mn = min(mn, __shfl_xor(mn, m, kWave));
  }
  if (lane == 0) {
    red[wave][0] = ksum;
    red[wave][1] = mx;
    red[wave][2] = mn;
  }
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < NW; ++w) {
    base += w < wave ? wave_tot[w] : 0;
    total += wave_tot[w];
  }
  const int off = base + incl - padded;
  if (e < N) {
    offsets[e] = off;
    seg[0][e] = off;
    seg[1][e] = kept;
    if (stats && !stats_ready) stats[e] = load;
  }
  if (e == 0) {
    offsets[N] = total;
    *num_padded = total;
    seg[0][N] = total;
  }
  __syncthreads();
  int G = 1;
  while (2 * G * N <= NT) G *= 2;
  for (int x = e / G; x < N; x += NT / G) {
    const int o = seg[0][x], o1 = seg[0][x + 1], kp = seg[1][x], sub = e % G;
    for (int i = o + kp + sub; i < o1; i += G) sorted_ids[i] = sentinel;
    for (int b = o / B + sub; b < o1 / B; b += G) block_expert[b] = x;
  }
  for (int b = total / B + e; b < n_blocks; b += NT) block_expert[b] = -1;
  if (stats && e == 0) {
    int ks = 0, mxx = 0, mnn = 0x7fffffff;
    for (int w = 0; w < NW; ++w) {
      ks += red[w][0];
      mxx = max(mxx, red[w][1]);
      mnn = min(mnn, red[w][2]);
    }
    stats[N + MOE_STAT_NUM_PADDED] = total;
    if (!stats_ready) {  // else the reroute pass wrote the rest (its loads are before capacity)
      stats[N + MOE_STAT_KEPT] = ks;
      stats[N + MOE_STAT_DROPPED] = (sentinel - invalid) - ks;  // valid routes not kept
      stats[N + MOE_STAT_INVALID] = invalid;
      stats[N + MOE_STAT_CAPACITY] = cap;
      stats[N + MOE_STAT_MAX_LOAD] = mxx;
      stats[N + MOE_STAT_MIN_LOAD] = mnn;
      stats[N + MOE_STAT_REROUTED] = 0;
      stats[N + MOE_STAT_UNPICKED] = 0;  // expert-choice counters
      stats[N + MOE_STAT_MAX_PICKS] = 0;
    }
  }
  *total_out = total;
  return off;
}

__global__ __launch_bounds__(kThreads) void align_scan(int32_t* __restrict__ counts, int nchunks, int N, int B,
                                                       int cap, int n_blocks,
                                                       int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
                                                       int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded,
                                                       int32_t* __restrict__ stats, int sentinel,
                                                       int32_t* __restrict__ zero, int nzero, int stats_ready) {
  constexpr int kBatch = 32;  // chunk counts loaded together (clamped index: no branch, no serial waits)
  __shared__ int s_inv[kThreads / kWave];
  const int e = threadIdx.x;
  int load = 0;
  if (e < N) {
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = counts[(size_t)min(c0 + j, nchunks - 1) * (N + 1) + e];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (c0 + j < nchunks) {
          counts[(size_t)(c0 + j) * (N + 1) + e] = load;  // exclusive prefix over chunks, in place
          load += v[j];
        }
      }
    }
  }
  int inv = 0;  // invalid routes: column N, summed over chunks by all threads
  for (int c = e; c < nchunks; c += kThreads) inv += counts[(size_t)c * (N + 1) + N];
  inv = wave_sum_i32(inv);
  if ((e & 63) == 0) s_inv[e >> 6] = inv;
  __syncthreads();
  int invalid = 0;
  for (int w = 0; w < kThreads / kWave; ++w) invalid += s_inv[w];
  int total;
  layout_experts<kThreads>(load, invalid, N, B, cap, n_blocks, sorted_ids, block_expert, offsets, num_padded, stats,
                           sentinel, zero, nzero, stats_ready, &total);
}

// All three steps in one workgroup of kFThreads, for up to kFWaves x kFSteps x 64
// routes.  Wave w takes the w-th of kFWaves equal runs of consecutive routes (a
// multiple of 64, in registers): it counts its run's routes per expert (ballot peer
// masks over KB key bits, into its own LDS row); per expert, an exclusive prefix of
// the waves' counts in wave order gives each wave's first position; the layout
// follows; then each wave walks its run again and places each route at its first
// position plus the routes to the same expert before it in the run -- the positions
// of the three-kernel path.  Keys: expert 0..N-1, N = invalid id, 2^KB - 1 = none.
constexpr int kFThreads = 1024;
constexpr int kFWaves = kFThreads / kWave;
constexpr int kFSteps = 8;  // beyond 8192 routes the three kernels, spread over CUs, are faster

template <int KB>
__global__ __launch_bounds__(kFThreads) void align_fused(const int32_t* __restrict__ ids, int R, int N, int B,
                                                         int cap, int n_blocks, int p_max,
                                                         uint8_t* __restrict__ kept_out,
                                                         int32_t* __restrict__ sorted_ids,
                                                         int32_t* __restrict__ block_expert,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ num_padded,
                                                         int32_t* __restrict__ stats,
                                                         int32_t* __restrict__ zero, int nzero, int stats_ready) {
  constexpr int kNone = (1 << KB) - 1;
  __shared__ int run[kFWaves][257];
  __shared__ int s_off[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int steps = ceil_div(R, kFWaves * kWave);  // <= kFSteps (host-checked)
  const int rw = wave * steps * kWave;             // this wave's first route
  for (int i = lane; i <= N; i += kWave) run[wave][i] = 0;
  int my[kFSteps];  // key of this lane's route at each step
  if (R > 0) {
    // unconditional loads from a clamped index, so all of them are in flight together
#pragma unroll
    for (int j = 0; j < kFSteps; ++j) {
      const int r = rw + j * kWave + lane;
      const bool has = j < steps && r < R;
      const int e = ids[has ? r : R - 1];
      my[j] = has ? ((e >= 0 && e < N) ? e : N) : kNone;
    }
  }
  __builtin_amdgcn_wave_barrier();
  uint64_t peers[kFSteps];  // lanes of the step with the same key, kept for the second walk
#pragma unroll
  for (int j = 0; j < kFSteps; ++j) {
    if (j < steps) {  // uniform
      peers[j] = peer_mask<KB>(my[j]);
      if (my[j] != kNone && (peers[j] & lt) == 0) run[wave][my[j]] += __popcll(peers[j]);  // one writer per key
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  int load = 0, invalid = 0;
  if (tid < N) {
    for (int w = 0; w < kFWaves; ++w) {
      const int c = run[w][tid];
      run[w][tid] = load;  // first position of wave w's routes to expert tid
      load += c;
    }
  }
  if (tid == 0)
    for (int w = 0; w < kFWaves; ++w) invalid += run[w][N];
  int total;
  const int off = layout_experts<kFThreads>(load, invalid, N, B, cap, n_blocks, sorted_ids, block_expert, offsets,
                                            num_padded, stats, R, zero, nzero, stats_ready, &total);
  if (tid < N) s_off[tid] = off;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kFSteps; ++j) {
    if (j < steps) {  // uniform
      const int e = my[j] < N ? my[j] : -1;
      const int pos = e >= 0 ? run[wave][e] + __popcll(peers[j] & lt) : 0;
      __builtin_amdgcn_wave_barrier();
      if (e >= 0 && (peers[j] & lt) == 0) run[wave][e] += __popcll(peers[j]);
      __builtin_amdgcn_wave_barrier();
      const int r = rw + j * kWave + lane;
      const bool keep = e >= 0 && (cap < 0 || pos < cap);
      if (keep) sorted_ids[s_off[e] + pos] = r;
      if (my[j] != kNone) kept_out[r] = keep ? 1 : 0;
    }
  }
  for (int i = total + tid; i < p_max; i += kFThreads) sorted_ids[i] = R;  // sentinel tail
}

template <int KB>
hipError_t launch_fused(const moe_config& c, int R, int cap, int n_blocks, int p_max, const int32_t* ids,
                        uint8_t* kept, int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                        int32_t* num_padded, int32_t* stats, hipStream_t s, int32_t* zero, int nzero,
                        bool stats_ready) {
  align_fused<KB><<<1, kFThreads, 0, s>>>(ids, R, c.N, c.B, cap, n_blocks, p_max, kept, sorted_ids, block_expert,
                                          offsets, num_padded, stats, zero, zero ? nzero : 0, stats_ready ? 1 : 0);
  return hipGetLastError();
}

__global__ __launch_bounds__(kThreads) void align_scatter(const int32_t* __restrict__ ids, int R, int N, int cap,
                                                          const int32_t* __restrict__ chunk_base,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ num_padded, int p_max,
                                                          uint8_t* __restrict__ kept_out,
                                                          int32_t* __restrict__ sorted_ids, int sentinel) {
  __shared__ int run[4][256];
  __shared__ int s_off[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int rw = blockIdx.x * kChunk + wave * (kStepsPerWave * kWave);
  int my[kStepsPerWave];  // this lane's expert ids, loaded together (clamped index)
#pragma unroll
  for (int s = 0; s < kStepsPerWave; ++s) my[s] = ids[min(rw + s * kWave + lane, R - 1)];
  for (int i = threadIdx.x; i < 4 * 256; i += kThreads) (&run[0][0])[i] = 0;
  for (int e = threadIdx.x; e < N; e += kThreads) s_off[e] = offsets[e];
  __syncthreads();
  // pass 1: per-wave counts per expert
#pragma unroll
  for (int s = 0; s < kStepsPerWave; ++s) {
    const int r = rw + s * kWave + lane;
    const int e = r < R ? my[s] : -1;
    const bool valid = e >= 0 && e < N;
    const int key = valid ? e : 256;
    const uint64_t peers = peer_mask(key);
    if (valid && (peers & lt) == 0) run[wave][e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // per-wave starting positions: chunk prefix + counts of earlier waves, in wave order
  for (int e = threadIdx.x; e < N; e += kThreads) {
    int acc = chunk_base[(size_t)blockIdx.x * (N + 1) + e];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = run[w][e];
      run[w][e] = acc;
      acc += c;
    }
  }
  __syncthreads();
  // pass 2: position of each route among all routes to its expert (route-id order)
#pragma unroll
  for (int s = 0; s < kStepsPerWave; ++s) {
    const int r = rw + s * kWave + lane;
    const int e = r < R ? my[s] : -1;
    const bool valid = e >= 0 && e < N;
    const int key = valid ? e : 256;
    const uint64_t peers = peer_mask(key);
    int pos = 0;
    if (valid) pos = run[wave][e] + __popcll(peers & lt);
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers & lt) == 0) run[wave][e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    const bool keep = valid && (cap < 0 || pos < cap);
    if (keep) sorted_ids[s_off[e] + pos] = r;
    if (r < R) kept_out[r] = keep ? 1 : 0;
  }
  // sentinel tail of the padded row list
  const int np = *num_padded;
  for (int i = np + blockIdx.x * kThreads + threadIdx.x; i < p_max; i += gridDim.x * kThreads) sorted_ids[i] = sentinel;
}

}  // namespace

int align_chunk_routes() { return kChunk; }

size_t align_workspace_bytes(const moe_config& c) {
  const long R = (long)c.T * c.k;
  const long nchunks = (R + kChunk - 1) / kChunk;
  return (size_t)(nchunks * (c.N + 1)) * sizeof(int32_t);
}

hipError_t launch_align(const moe_config& c, const int32_t* ids, uint8_t* kept, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* offsets, int32_t* num_padded, int32_t* stats, void* ws,
                        hipStream_t s, int32_t* zero, int nzero, bool stats_ready) {
  const int R = c.T * c.k;
  const int nchunks = ceil_div(R, kChunk);
  const int p_max = R + c.N * (c.B - 1);
  const int n_blocks = ceil_div(p_max, c.B);
  int cap = -1;
  if (!(c.cap_num == 0 && c.cap_den == 0)) {
    const long long cl = ((long long)c.T * c.k * c.cap_num) / ((long long)c.N * c.cap_den);
    cap = cl > 0x7fffffffLL ? 0x7fffffff : (int)cl;
  }
  if (R <= kFWaves * kFSteps * kWave) {
    // key bits: experts 0..N-1, the invalid key N and the none key 2^KB - 1 all distinct
#define MOE_FUSED(KB) \
  launch_fused<KB>(c, R, cap, n_blocks, p_max, ids, kept, sorted_ids, block_expert, offsets, num_padded, stats, s, \
                   zero, nzero, stats_ready)
    const int need = c.N + 2;
    if (need <= 16) return MOE_FUSED(4);
    if (need <= 32) return MOE_FUSED(5);
    if (need <= 64) return MOE_FUSED(6);
    if (need <= 128) return MOE_FUSED(7);
    if (need <= 256) return MOE_FUSED(8);
    return MOE_FUSED(9);
#undef MOE_FUSED
  }
  int32_t* counts = (int32_t*)ws;
  align_hist<<<nchunks, kThreads, 0, s>>>(ids, R, c.N, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  align_scan<<<1, kThreads, 0, s>>>(counts, nchunks, c.N, c.B, cap, n_blocks, sorted_ids, block_expert, offsets,
                                    num_padded, stats, R, zero, zero ? nzero : 0, stats_ready ? 1 : 0);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  align_scatter<<<nchunks, kThreads, 0, s>>>(ids, R, c.N, cap, counts, offsets, num_padded, p_max, kept, sorted_ids, R);
  err = hipGetLastError();
  return err;
}

}  // namespace moe
