// Routing: gate top-k with a fixed tie-break, softmax over the selected
// logits, per-expert histogram, and the deterministic (token, k) -> slot map.
//
// UniEP article, section 1.1 (gate scores, top-k per token) and section 2.2,
// "deterministic token mapping" / Algorithm 1: a stable sort by expert, the
// per-expert counts and prefix-sum base offsets give each pair a unique slot
// without atomic locks.  On one GPU the "ranks" of Algorithm 1 become chunks
// of 64 tokens: the base of chunk c in expert e is the sum of the counts of
// lower chunks for e (exactly the rank-major prefix of the article), and the
// position inside a chunk is the pair's rank among the chunk's pairs routed to
// e, taken with wave ballots in (token, k) order.  No atomic decides a slot.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(64) void chunk_hist_kernel(const int32_t* __restrict__ topk_idx,
                                  const int32_t* __restrict__ chunk_t0, int T, int E, int K,
                                  int32_t* __restrict__ chunk_counts);

// Order-preserving 32-bit image of a finite logit (a larger logit gives a
// larger value, never 0); -0.0 is folded onto +0.0.
__device__ __forceinline__ uint32_t route_ord(float l) {
  uint32_t u = __float_as_uint(l);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float route_ord_logit(uint32_t hi) {
  return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}

// Order-preserving 64-bit key: a larger logit gives a larger key; for equal
// logits the lower expert id gives the larger key.
__device__ __forceinline__ uint64_t route_key(float l, int e) {
  return ((uint64_t)route_ord(l) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float route_key_logit(uint64_t key) {
  return route_ord_logit((uint32_t)(key >> 32));
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// One lane per token (E <= EMAX <= 32, K <= kLaneMaxK): the token's logits sit
// in the lane's registers and each of the K picks scans them, the first
// maximum winning (the lowest expert id among equal logits), so a wave routes
// 64 tokens without cross-lane traffic.  Same keys, picks, order and weight
// arithmetic as the group kernel below, hence the same bits.  A wave's tokens
// are one routing chunk, so it also writes the chunk's expert histogram
// (chunk_counts[c][e], as chunk_hist_kernel does).
constexpr int kLaneMaxK = 8;
static_assert(kChunkTokens == kWave, "one wave of the lane kernel is one routing chunk");
template <int EMAX>
__device__ __forceinline__ void route_lane_token(const float* __restrict__ logits, int t, int E, int K,
                                                 int32_t* __restrict__ topk_idx,
                                                 float* __restrict__ topk_w, int* hist) {
  const float* row = logits + (int64_t)t * E;
  uint32_t key[EMAX];
  if (E == EMAX) {   // whole row: 16-byte loads (rows are 16-byte aligned)
#pragma unroll
    for (int i = 0; i < EMAX / 4; ++i) {
      const float4 v = reinterpret_cast<const float4*>(row)[i];
      key[4 * i] = route_ord(v.x);
      key[4 * i + 1] = route_ord(v.y);
      key[4 * i + 2] = route_ord(v.z);
      key[4 * i + 3] = route_ord(v.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) key[e] = e < E ? route_ord(row[e]) : 0u;   // 0: none
  }
  float l0 = 0.f, zsum = 0.f, pl[kLaneMaxK];
#pragma unroll
  for (int k = 0; k < kLaneMaxK; ++k) {
    if (k < K) {
      uint32_t best = key[0];
      int be = 0;
#pragma unroll
      for (int e = 1; e < EMAX; ++e) {
        if (key[e] > best) {
          best = key[e];
          be = e;
        }
      }
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e == be) key[e] = 0u;   // an expert is picked once
      const float l = route_ord_logit(best);
      if (k == 0) l0 = l;
      zsum += expf(l - l0);
      pl[k] = l;
      topk_idx[(int64_t)t * K + k] = be;
      atomicAdd(&hist[be], 1);
    }
  }
#pragma unroll
  for (int k = 0; k < kLaneMaxK; ++k)
    if (k < K) topk_w[(int64_t)t * K + k] = expf(pl[k] - l0) / zsum;
}

template <int EMAX>
__global__ __launch_bounds__(64) void route_topk_lane_kernel(const float* __restrict__ logits, int T,
                                                             int E, int K, int32_t* __restrict__ topk_idx,
                                                             float* __restrict__ topk_w,
                                                             int32_t* __restrict__ chunk_counts) {
  __shared__ int hist[EMAX];
  const int lane = threadIdx.x, c = blockIdx.x;
  const int t = c * kWave + lane;
  if (lane < EMAX) hist[lane] = 0;
  __syncthreads();
  if (t < T) route_lane_token<EMAX>(logits, t, E, K, topk_idx, topk_w, hist);
  __syncthreads();
  if (lane < E) chunk_counts[(int64_t)c * E + lane] = hist[lane];
}

// One group of G lanes per token (G = min(64, next pow2 >= E)); each lane owns
// up to 4 experts (e = lane + i*G).  K rounds of a group-wide max over the
// keys pick the experts in descending order.  Block = 256 threads = 4 waves,
// each wave one group of 64 / G tokens, so a block takes 4 * 64 / G tokens:
// the per-token rounds are short dependent shuffle chains, and many small
// blocks keep enough of them in flight to hide their latency.
//
// E <= G (at most 64 experts: one expert per lane): the group maximum is
// taken on the 32-bit order-preserving logit alone, and among the lanes that
// hold it the lowest lane -- the lowest expert id -- wins (one ballot).  Same
// selection, order and weights as the 64-bit keys, with half the shuffles.
template <int G>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int K, int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  constexpr int TPW = kWave / G;  // tokens per wave
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int gl = lane & (G - 1), grp = lane / G;
  const int t = (blockIdx.x * 4 + wave) * TPW + grp;
  const bool valid = t < T;
  if (E <= G) {
    uint32_t v = (valid && gl < E) ? route_ord(logits[(int64_t)t * E + gl]) : 0u;   // 0: none
    const uint64_t gmask = G == kWave ? ~0ull : (((1ull << (G % kWave)) - 1ull) << (grp * G));
    float l0 = 0.f, zsum = 0.f, my_l = 0.f;
    int my_e = 0;
    for (int k = 0; k < K; ++k) {
      uint32_t best = v;
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) best = max(best, (uint32_t)__shfl_xor((int)best, o, kWave));
      const uint64_t cand = __ballot(v != 0u && v == best) & gmask;
      const int e = __ffsll((unsigned long long)cand) - 1 - grp * G;   // lowest id among the ties
      const float l = route_ord_logit(best);
      if (gl == e) v = 0u;  // an expert is picked once
      if (k == 0) l0 = l;
      zsum += expf(l - l0);
      if (gl == k) {
        my_l = l;
        my_e = e;
      }
    }
    if (valid && gl < K) {
      topk_idx[(int64_t)t * K + gl] = my_e;
      topk_w[(int64_t)t * K + gl] = expf(my_l - l0) / zsum;
    }
    return;
  }
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = gl + i * G;
    key[i] = (valid && e < E) ? route_key(logits[(int64_t)t * E + e], e) : 0ull;
  }
  // pick k is kept by lane k % 64 in slot k / 64 (K <= 256)
  float l0 = 0.f, zsum = 0.f, my_l[4] = {0.f, 0.f, 0.f, 0.f};
  int my_e[4] = {0, 0, 0, 0};
  for (int k = 0; k < K; ++k) {
    uint64_t best = umax64(umax64(key[0], key[1]), umax64(key[2], key[3]));
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) {
      const uint64_t other = __shfl_xor(best, o, kWave);
      best = umax64(best, other);
    }
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float l = route_key_logit(best);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e == gl + i * G) key[i] = 0ull;  // an expert is picked once
    if (k == 0) l0 = l;
    zsum += expf(l - l0);
    if (gl == (k & (G - 1))) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((k / G) == c) {
          my_l[c] = l;
          my_e[c] = e;
        }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int k = gl + c * G;
    if (valid && k < K) {
      topk_idx[(int64_t)t * K + k] = my_e[c];
      topk_w[(int64_t)t * K + k] = expf(my_l[c] - l0) / zsum;
    }
  }
}

// One block per expert: exclusive scan of the expert's column of chunk counts
// (chunk_base[c][e] = pairs of lower chunks routed to e) and its total.  Each
// thread sums a contiguous run of chunks, one block scan places the runs.
__global__ __launch_bounds__(256) void route_chunk_scan_kernel(const int32_t* __restrict__ chunk_counts,
                                                               int nchunk, int E,
                                                               int32_t* __restrict__ chunk_base,
                                                               int32_t* __restrict__ counts) {
  __shared__ int buf[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int per = (nchunk + 255) / 256;
  const int c0 = min(nchunk, tid * per), c1 = min(nchunk, c0 + per);
  int mine = 0;
  for (int c = c0; c < c1; ++c) mine += chunk_counts[(int64_t)c * E + e];
  buf[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  int run = buf[tid] - mine;
  for (int c = c0; c < c1; ++c) {
    const int v = chunk_counts[(int64_t)c * E + e];
    chunk_base[(int64_t)c * E + e] = run;
    run += v;
  }
  if (tid == 255) counts[e] = buf[255];
}

// One wave per chunk.  Expert start offsets = exclusive scan of counts (every
// wave recomputes it; chunk 0 publishes offsets).  Then the chunk's pairs are
// taken 64 at a time in (token, k) order: the lanes holding the same expert
// are found with one ballot per bit of the expert id, a lane's rank among
// them is the popcount of lower peers, and the highest peer advances the
// expert's running cursor.  slot = offsets[e] + chunk_base[c][e] + rank.
// chunk_t0 (may be null): chunk c holds tokens [chunk_t0[c], chunk_t0[c+1])
// instead of the uniform chunks of kChunkTokens.
__global__ __launch_bounds__(64) void route_slot_kernel(const int32_t* __restrict__ topk_idx,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ chunk_base,
                                                        const int32_t* __restrict__ chunk_t0,
                                                        int T, int E, int K,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ slot,
                                                        int32_t* __restrict__ slot_src) {
  __shared__ int cur[256];
  const int lane = threadIdx.x, c = blockIdx.x;
  int v[4], lane_total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane * 4 + i;
    v[i] = e < E ? counts[e] : 0;
    lane_total += v[i];
  }
  int incl = lane_total;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  int run = incl - lane_total;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane * 4 + i;
    if (e < E) {
      cur[e] = run + chunk_base[(int64_t)c * E + e];
      if (c == 0) offsets[e] = run;
    }
    run += v[i];
  }
  if (c == 0 && lane == kWave - 1) offsets[E] = incl;
  __syncthreads();

  const int t0 = chunk_t0 ? chunk_t0[c] : c * kChunkTokens;
  const int t1 = chunk_t0 ? chunk_t0[c + 1] : min(T, t0 + kChunkTokens);
  const int n = (t1 - t0) * K;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lower = (1ull << lane) - 1ull;
  const uint64_t higher = ~((2ull << lane) - 1ull);
  int e_next = lane < n ? topk_idx[(int64_t)t0 * K + lane] : 0;   // one group of 64 pairs ahead
  for (int q0 = 0; q0 < n; q0 += kWave) {
    const int q = q0 + lane;
    const int e_in = e_next;
    if (q + kWave < n) e_next = topk_idx[(int64_t)t0 * K + q + kWave];
    const bool act = q < n && (unsigned)e_in < (unsigned)E;   // ids outside [0, E) are skipped
    const int e = act ? e_in : 0;
    uint64_t peers = __ballot(act);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int base = cur[e];
    __syncthreads();
    if (act) {
      const int s = base + __popcll(peers & lower);
      slot[(int64_t)t0 * K + q] = s;
      slot_src[s] = t0 + q / K;
      if ((peers & higher) == 0ull) cur[e] = base + __popcll(peers);
    }
    __syncthreads();
  }
}

hipError_t launch_route(const float* logits, int T, int E, int K, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* slot_src,
                        int32_t* chunk_counts, int32_t* chunk_base, hipStream_t st) {
  const int nchunk = route_nchunk(T);
  int g = 1;
  while (g < E && g < 64) g <<= 1;
  const int per_block = 4 * (kWave / g);
  const dim3 grid((T + per_block - 1) / per_block), block(256);
  const int lane_grid = (T + kWave - 1) / kWave;
  if (E <= 32 && K <= kLaneMaxK) g = E <= 8 ? -8 : E <= 16 ? -16 : -32;   // the lane kernel
  switch (g) {
    case -8:
      route_topk_lane_kernel<8><<<lane_grid, kWave, 0, st>>>(logits, T, E, K, topk_idx, topk_w,
                                                               chunk_counts);
      break;
    case -16:
      route_topk_lane_kernel<16><<<lane_grid, kWave, 0, st>>>(logits, T, E, K, topk_idx, topk_w,
                                                               chunk_counts);
      break;
    case -32:
      route_topk_lane_kernel<32><<<lane_grid, kWave, 0, st>>>(logits, T, E, K, topk_idx, topk_w,
                                                               chunk_counts);
      break;
#define MOE_ROUTE_CASE(G)                                                                      \
  case G:                                                                                      \
    route_topk_kernel<G><<<grid, block, 0, st>>>(logits, T, E, K, topk_idx, topk_w);           \
    break;
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(16)
    MOE_ROUTE_CASE(32)
    MOE_ROUTE_CASE(64)
#undef MOE_ROUTE_CASE
    default:
      return hipErrorInvalidValue;
  }
  if (g > 0) chunk_hist_kernel<<<nchunk, 64, 0, st>>>(topk_idx, nullptr, T, E, K, chunk_counts);
  route_chunk_scan_kernel<<<E, 256, 0, st>>>(chunk_counts, nchunk, E, chunk_base, counts);
  route_slot_kernel<<<nchunk, 64, 0, st>>>(topk_idx, counts, chunk_base, nullptr, T, E, K, offsets,
                                           slot, slot_src);
  return hipGetLastError();
}

// ------------------------------------------------- static scratch variant --
//
// The routing scratch of moe_route_noalloc: a file-scope device array, one per
// device, so that the call allocates nothing.  In host code `scratch` names a
// host-side stand-in, not the device array: the kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and cached.  Every call on a device shares its array; nothing in it
// needs to start at zero (each word the kernels read was written earlier in
// the same call), and calls that overlap in time on one device race.
static __device__ __align__(256) int32_t scratch[kRouteScratchInts];

namespace {
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[64] = {};

hipError_t lookup_scratch_locked(int device) {
  if (g_scratch_ptr[device]) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[device] = static_cast<int32_t*>(p);
  return hipSuccess;
}
}  // namespace

hipError_t route_scratch_prepare(int device) {
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  int prev = 0;
  hipError_t e = hipGetDevice(&prev);
  if (e != hipSuccess) return e;
  if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
  e = lookup_scratch_locked(device);
  const hipError_t r = prev != device ? hipSetDevice(prev) : hipSuccess;
  return e != hipSuccess ? e : r;
}

hipError_t route_scratch_current(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  e = lookup_scratch_locked(dev);   // the current device is the one looked up
  *out = g_scratch_ptr[dev];
  return e;
}

// ---------------------------------------------------------------- G ranks --
//
// Algorithm 1 of the UniEP article (section 2.2) with G explicit ranks, each
// holding the contiguous token block [floor(T r / G), floor(T (r+1) / G)):
// every rank counts its own (token, k) pairs per expert, the counts form a
// [G, E] table (what an all-gather would give each rank), the base offset of
// rank r in expert e is the expert's start plus the counts of lower ranks,
// and a pair's slot is its rank's base plus its stable position among the
// rank's pairs of that expert.  On one GPU each rank is cut into chunks of at
// most kChunkTokens tokens and the chunk kernels above run over the chunks in
// rank-major order, so the slots equal the one-rank map by construction.

// Chunk table: chunk_t0[j] = first token of chunk j (chunk_t0[j] = T for the
// unused chunks up to the bound nmax, and for j = nmax), rank_chunk[r] = first
// chunk of rank r, rank_chunk[G] = number of chunks.  One block; each thread
// owns a run of ranks and a block scan places its chunks.
__global__ __launch_bounds__(256) void rank_chunks_kernel(int T, int G, int nmax,
                                                          int32_t* __restrict__ chunk_t0,
                                                          int32_t* __restrict__ rank_chunk) {
  __shared__ int scan[256];
  const int tid = threadIdx.x;
  const int per = (G + 255) / 256;
  const int r_begin = min(G, tid * per), r_end = min(G, r_begin + per);
  auto bound = [&](int r) { return (int)(((int64_t)T * r) / G); };
  int mine = 0;
  for (int r = r_begin; r < r_end; ++r) mine += (bound(r + 1) - bound(r) + kChunkTokens - 1) / kChunkTokens;
  scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  int j = scan[tid] - mine;
  for (int r = r_begin; r < r_end; ++r) {
    rank_chunk[r] = j;
    for (int t = bound(r); t < bound(r + 1); t += kChunkTokens) chunk_t0[j++] = t;
  }
  const int total = scan[255];
  if (tid == 0) rank_chunk[G] = total;
  for (int i = total + tid; i <= nmax; i += 256) chunk_t0[i] = T;
}

// One wave per chunk: the chunk's per-expert pair counts (zero for unused
// chunks).  chunk_t0 null: uniform chunks of kChunkTokens tokens.
__global__ __launch_bounds__(64) void chunk_hist_kernel(const int32_t* __restrict__ topk_idx,
                                                        const int32_t* __restrict__ chunk_t0, int T,
                                                        int E, int K, int32_t* __restrict__ chunk_counts) {
  __shared__ int hist[256];
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += kWave) hist[e] = 0;
  __syncthreads();
  const int t0 = chunk_t0 ? chunk_t0[c] : c * kChunkTokens;
  const int t1 = chunk_t0 ? chunk_t0[c + 1] : min(T, t0 + kChunkTokens);
  for (int q = lane; q < (t1 - t0) * K; q += kWave) {
    const int e = topk_idx[(int64_t)t0 * K + q];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);   // ids outside [0, E) are skipped
  }
  __syncthreads();
  for (int e = lane; e < E; e += kWave) chunk_counts[(int64_t)c * E + e] = hist[e];
}

// Rank tables from the chunk prefix sums: rank_base[r][e] = expert start +
// pairs of lower ranks routed to e, rank_counts[r][e] = pairs of rank r routed
// to e.  Each block scans the expert totals for the starts, then fills its
// ranks.
__global__ __launch_bounds__(256) void rank_tables_kernel(const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ chunk_base,
                                                          const int32_t* __restrict__ rank_chunk,
                                                          int G, int E, int nmax, int ranks_per_block,
                                                          int32_t* __restrict__ rank_counts,
                                                          int32_t* __restrict__ rank_base) {
  __shared__ int start[256];
  const int tid = threadIdx.x;
  start[tid] = tid < E ? counts[tid] : 0;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? start[tid - off] : 0;
    __syncthreads();
    start[tid] += add;
    __syncthreads();
  }
  const int incl = start[tid];
  __syncthreads();
  start[tid] = incl - (tid < E ? counts[tid] : 0);   // exclusive
  __syncthreads();
  auto cb = [&](int j, int e) { return j < nmax ? chunk_base[(int64_t)j * E + e] : counts[e]; };
  const int r0 = blockIdx.x * ranks_per_block, r1 = min(G, r0 + ranks_per_block);
  for (int i = tid; i < (r1 - r0) * E; i += 256) {
    const int r = r0 + i / E, e = i % E;
    const int lo = cb(rank_chunk[r], e), hi = cb(rank_chunk[r + 1], e);
    rank_base[(int64_t)r * E + e] = start[e] + lo;
    rank_counts[(int64_t)r * E + e] = hi - lo;
  }
}

int route_ranks_nchunk(int T, int G) { return (T + kChunkTokens - 1) / kChunkTokens + G; }

hipError_t launch_route_ranks(const int32_t* topk_idx, int T, int E, int K, int G,
                              int32_t* rank_counts, int32_t* rank_base, int32_t* counts,
                              int32_t* offsets, int32_t* slot, int32_t* slot_src, int32_t* chunk_counts,
                              int32_t* chunk_base, int32_t* chunk_t0, int32_t* rank_chunk,
                              hipStream_t st) {
  const int nmax = route_ranks_nchunk(T, G);
  rank_chunks_kernel<<<1, 256, 0, st>>>(T, G, nmax, chunk_t0, rank_chunk);
  chunk_hist_kernel<<<nmax, 64, 0, st>>>(topk_idx, chunk_t0, T, E, K, chunk_counts);
  route_chunk_scan_kernel<<<E, 256, 0, st>>>(chunk_counts, nmax, E, chunk_base, counts);
  const int rpb = 64;
  rank_tables_kernel<<<(G + rpb - 1) / rpb, 256, 0, st>>>(counts, chunk_base, rank_chunk, G, E, nmax,
                                                          rpb, rank_counts, rank_base);
  route_slot_kernel<<<nmax, 64, 0, st>>>(topk_idx, counts, chunk_base, chunk_t0, T, E, K, offsets,
                                         slot, slot_src);
  return hipGetLastError();
}

}  // namespace moe
