// GPU-built longest-first work lists of the packed call.
//
// The pages build the schedule once per microbatch on the GPU with a
// fixed-pass sort and hand items, costliest first, to the grid
// ([Summary, §3.6.2 Load-Balanced Scheduling]; [Reading, 4.4] last bullet).
// Here each (document, tile) gets a unique 64-bit key
//   (COST_MAX - c) << 44 | doc << 20 | tile
// where c is the tile's cost; sorting the keys gives the pages' order: cost
// descending, then document, then tile.  Three lists are built:
//   0  forward query tiles, that order;
//   1  backward key tiles, that order (the published schedule);
//   2  the backward's dispatch order, a permutation of list 1: c is the cost
//      of the document's costliest (first) key tile, so a document's key
//      tiles stay together (longest document first, tiles in order, so still
//      costliest first inside it) and its query rows are reused from L2 while
//      its tiles run.
// Every key is unique, so exactly one order is correct.
//   * Lists of at most PLAN_MAX_TILES tiles: one workgroup per list
//     enumerates the keys and bitonic-sorts them in LDS (within one wave for
//     at most 64 tiles).
//   * Longer lists: the keys are enumerated into a padded array (tile t of
//     document d at slot floor(cu[d] / 128) + d + t, which never reaches the
//     next document's first slot; empty slots hold the largest key), runs of
//     PLAN_RUN keys are bitonic-sorted in LDS, and merge passes double the run
//     length (each output element finds its source by a co-rank binary search
//     over the two runs).
// A tile later expands to num_heads consecutive grid items (head ascending).
// The forward reads item blockIdx.x / H of list 0, the backward of list 2;
// the hardware dispatcher hands workgroups out in index order, which plays
// the role of the pages' dynamic fetch.
//
// Costs (number of tile pairs the causal tile touches):
//   forward  query tile t of a document of length L: floor((min((t+1)Bq, L)-1)/Bk) + 1
//   backward key tile u:                             ceil(L/Bq) - floor(u Bk / Bq)
// Without the mask every tile of a document touches all ceil(L/Bk) key tiles
// (forward) or all ceil(L/Bq) query tiles (backward).
#include <utility>

#include "flamia_device.hpp"
#include "flamia_internal.hpp"

namespace flamia {

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_WAVES = PLAN_THREADS / 64;

// Inclusive scan of one int per thread over the workgroup: a scan inside each
// wave, then one over the wave totals.  `wsum` holds PLAN_WAVES ints.
__device__ static int block_inclusive_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(v, off, 64);
    if (lane >= off) v += up;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int before = 0;
  total = 0;
  for (int w = 0; w < PLAN_WAVES; ++w) {
    const int t = wsum[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  return v + before;
}

// Inclusive scan of one 64-bit value per thread over the workgroup (same
// scheme; `wsum` holds PLAN_WAVES values).
__device__ static long long block_inclusive_scan64(long long v, long long* wsum, long long& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned lo = __shfl_up((unsigned)v, off, 64), hi = __shfl_up((unsigned)((unsigned long long)v >> 32), off, 64);
    if (lane >= off) v += (long long)(((unsigned long long)hi << 32) | lo);
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  long long before = 0;
  total = 0;
  for (int w = 0; w < PLAN_WAVES; ++w) {
    const long long t = wsum[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  return v + before;
}

// One 64-bit key per lane of wave 0, sorted ascending across the wave with
// the same bitonic network (for lists of at most 64 tiles).
__device__ static unsigned long long wave_bitonic(unsigned long long key) {
  const int lane = threadIdx.x & 63;
  for (int k = 2; k <= 64; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      const unsigned lo = __shfl_xor((unsigned)key, j, 64), hi = __shfl_xor((unsigned)(key >> 32), j, 64);
      const unsigned long long other = ((unsigned long long)hi << 32) | lo;
      const bool up = (lane & k) == 0, first = (lane & j) == 0;
      // the lower lane of the pair keeps the smaller key when sorting up
      const bool keep_min = (first == up);
      key = keep_min ? (other < key ? other : key) : (other > key ? other : key);
    }
  return key;
}

static_assert(FWD_BQ == BWD_BK, "both lists count 128-token tiles");
constexpr int PLAN_TILE = FWD_BQ;

constexpr int PLAN_LISTS = 3;          // forward, backward, backward dispatch

// Plan word holding the tile count of list `lst` (word 2 is the
// deterministic-mode error word).
__device__ __forceinline__ int count_slot(int lst) { return lst == 2 ? 3 : lst; }

// Sort key of tile t of document d (L tokens) in list `lst`.
__device__ __forceinline__ unsigned long long tile_key(int lst, bool causal, int d, int t, int L, int bq, int bk) {
  int cost;
  if (!causal) {
    cost = lst == 0 ? (L + bk - 1) / bk : (L + bq - 1) / bq;
  } else if (lst == 0) {
    const int e = min((t + 1) * bq, L);
    cost = (e - 1) / bk + 1;
  } else if (lst == 1) {
    cost = (L + bq - 1) / bq - (t * bk) / bq;
  } else {
    // dispatch order: every tile of a document carries the cost of its
    // costliest (first) key tile
    cost = (L + bq - 1) / bq;
  }
  return ((unsigned long long)(COST_MAX - cost) << 44) | ((unsigned long long)d << 20) | (unsigned long long)t;
}

__device__ __forceinline__ int2 key_item(unsigned long long key) {
  return make_int2((int)((key >> 20) & 0xffffffull), (int)(key & 0xfffffull));
}

// Ascending bitonic sort of n2 (a power of two) keys in LDS by the whole
// workgroup.
__device__ static void lds_bitonic(unsigned long long* keys, int n2) {
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += PLAN_THREADS) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long a = keys[i], b = keys[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) { keys[i] = b; keys[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
}

__device__ static void build_sorted(const int* __restrict__ cu, int ndocs, int lst, bool causal, int bq, int bk,
                                    unsigned long long* keys, int* wsum, int* count_out,
                                    int2* __restrict__ out) {
  const bool fwd = lst == 0;
  const int tid = threadIdx.x;
  int n_tiles = 0;
  // enumerate tiles, chunk of PLAN_THREADS documents at a time
  for (int base = 0; base < ndocs; base += PLAN_THREADS) {
    const int d = base + tid;
    int L = 0, n = 0;
    if (d < ndocs) {
      L = cu[d + 1] - cu[d];
      n = fwd ? (L + bq - 1) / bq : (L + bk - 1) / bk;
    }
    int total;
    const int first = n_tiles + block_inclusive_scan(n, wsum, total) - n;
    for (int t = 0; t < n; ++t) keys[first + t] = tile_key(lst, causal, d, t, L, bq, bk);
    n_tiles += total;
  }
  __syncthreads();
  if (n_tiles <= 64) {
    // small list: one wave, no workgroup barriers
    if (tid < 64) {
      const unsigned long long key = wave_bitonic(tid < n_tiles ? keys[tid] : ~0ull);
      if (tid < n_tiles) out[tid] = key_item(key);
    }
  } else {
    int n2 = 1;
    while (n2 < n_tiles) n2 <<= 1;
    for (int i = n_tiles + tid; i < n2; i += PLAN_THREADS) keys[i] = ~0ull;
    __syncthreads();
    lds_bitonic(keys, n2);
    for (int i = tid; i < n_tiles; i += PLAN_THREADS) out[i] = key_item(keys[i]);
  }
  if (tid == 0) *count_out = n_tiles;
}

// Workgroup 0 builds the forward list, workgroup 1 the backward list and the
// deterministic-mode step prefix, workgroup 2 the backward dispatch order: document d's dQ partial steps (per head)
// start at det_base[d]; a document of L tokens has n = ceil(L / BWD_BK) key
// tiles and Q = ceil(L / BWD_BQ) query tiles, and key tile u visits query
// tiles 2u .. Q-1, so n Q - n (n - 1) steps (n Q without the mask).  Word 2
// of the plan flags a total beyond det_cap.
// With `large` set the lists are left to the multi-workgroup kernels below
// and this kernel only clears the tile counts.  The step prefix is built only in
// deterministic mode (det_cap > 0).
__global__ void __launch_bounds__(PLAN_THREADS) plan_kernel(const int* __restrict__ cu, int ndocs, int causal,
                                                            int large, int* counts, int2* fwd_items,
                                                            int2* bwd_items, int2* disp_items, float* qk_scale,
                                                            int* det_base, int det_cap) {
  __shared__ unsigned long long keys[PLAN_MAX_TILES];
  __shared__ int wsum[PLAN_WAVES];
  __shared__ long long wsum64[PLAN_WAVES];
  const int lst = blockIdx.x;
  const bool fwd = lst == 0;
  if (large) {                    // the fill kernel adds the counts
    if (threadIdx.x == 0) counts[count_slot(lst)] = 0;
  } else {
    build_sorted(cu, ndocs, lst, causal != 0, fwd ? FWD_BQ : BWD_BQ, fwd ? FWD_BK : BWD_BK, keys, wsum,
                 counts + count_slot(lst), lst == 0 ? fwd_items : lst == 1 ? bwd_items : disp_items);
  }
  if (lst != 1) return;
  if (det_cap == 0 && threadIdx.x == 0) counts[2] = 0;
  if (det_cap > 0) {
    long long done = 0;
    for (int base = 0; base < ndocs; base += PLAN_THREADS) {
      const int d = base + threadIdx.x;
      long long st = 0;
      if (d < ndocs) {
        const long long L = cu[d + 1] - cu[d];
        const long long n = (L + BWD_BK - 1) / BWD_BK, q = (L + BWD_BQ - 1) / BWD_BQ;
        st = causal ? n * q - n * (n - 1) : n * q;
      }
      long long chunk;
      const long long incl = block_inclusive_scan64(st, wsum64, chunk);
      if (d < ndocs) det_base[d] = (int)min(done + incl - st, (long long)INT_MAX);
      done += chunk;
    }
    if (threadIdx.x == 0) {
      det_base[ndocs] = (int)min(done, (long long)INT_MAX);
      counts[2] = done > det_cap ? 1 : 0;
    }
  }
  // mixed path: clear the tensor-amax slots before the amax pass runs
  if (qk_scale != nullptr && threadIdx.x < 2) qk_scale[threadIdx.x] = 0.f;
}

// ---- multi-workgroup path (lists of more than PLAN_MAX_TILES tiles)

// First padded slot of document d: floor(cu[d] / 128) + d.  Strictly
// increasing in d, and slot(d + 1) - slot(d) >= ceil(L_d / 128).
__device__ __forceinline__ int doc_slot(const int* __restrict__ cu, int d) { return cu[d] / PLAN_TILE + d; }

// Keys of the three lists into padded arrays of cap_r slots (blockIdx.y =
// list); each workgroup adds its number of real tiles to the list's count.
__global__ void __launch_bounds__(256) plan_fill_kernel(const int* __restrict__ cu, int ndocs, int causal,
                                                        unsigned long long* __restrict__ keys, int cap_r,
                                                        int* counts) {
  __shared__ int wcount[4];
  const int lst = blockIdx.y;
  const bool fwd = lst == 0;
  const int s = blockIdx.x * 256 + threadIdx.x;
  unsigned long long key = ~0ull;
  if (s < cap_r && s < doc_slot(cu, ndocs - 1) + (cu[ndocs] - cu[ndocs - 1] + PLAN_TILE - 1) / PLAN_TILE) {
    // largest d with doc_slot(d) <= s
    int lo = 0, hi = ndocs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (doc_slot(cu, mid) <= s) lo = mid; else hi = mid - 1;
    }
    const int L = cu[lo + 1] - cu[lo], t = s - doc_slot(cu, lo);
    if (t < (L + PLAN_TILE - 1) / PLAN_TILE)
      key = tile_key(lst, causal != 0, lo, t, L, fwd ? FWD_BQ : BWD_BQ, fwd ? FWD_BK : BWD_BK);
  }
  if (s < cap_r) keys[(size_t)blockIdx.y * cap_r + s] = key;
  const int n = __popcll(__ballot(key != ~0ull));
  if ((threadIdx.x & 63) == 0) wcount[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int tot = wcount[0] + wcount[1] + wcount[2] + wcount[3];
    if (tot) atomicAdd(counts + count_slot(lst), tot);
  }
}

// Each workgroup sorts one run of PLAN_RUN keys in LDS, in place.
__global__ void __launch_bounds__(PLAN_THREADS) plan_sort_runs_kernel(unsigned long long* keys, int cap_r) {
  __shared__ unsigned long long sk[PLAN_RUN];
  unsigned long long* run = keys + (size_t)blockIdx.y * cap_r + (size_t)blockIdx.x * PLAN_RUN;
  for (int i = threadIdx.x; i < PLAN_RUN; i += PLAN_THREADS) sk[i] = run[i];
  __syncthreads();
  lds_bitonic(sk, PLAN_RUN);
  for (int i = threadIdx.x; i < PLAN_RUN; i += PLAN_THREADS) run[i] = sk[i];
}

// One merge pass: sorted runs of `width` keys are merged pairwise from src
// into dst.  Output element k of a pair takes i elements from run A and k - i
// from run B, with i the smallest index where B[k - i - 1] < A[i] (equal keys
// -- only the padding -- come from A first).
__global__ void __launch_bounds__(256) plan_merge_kernel(const unsigned long long* __restrict__ src,
                                                         unsigned long long* __restrict__ dst, int cap_r,
                                                         int width) {
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= cap_r) return;
  const size_t lb0 = (size_t)blockIdx.y * cap_r;
  const int base = g / (2 * width) * (2 * width);
  const int la = min(width, cap_r - base), lb = max(0, min(width, cap_r - base - width));
  const unsigned long long* A = src + lb0 + base;
  const unsigned long long* B = A + la;
  const int k = g - base;
  int lo = max(0, k - lb), hi = min(k, la);
  while (lo < hi) {
    const int i = (lo + hi) >> 1;          // i < la, k - i - 1 >= 0
    if (B[k - i - 1] < A[i]) hi = i; else lo = i + 1;
  }
  const int i = lo, j = k - lo;
  const bool take_a = i < la && (j >= lb || A[i] <= B[j]);
  dst[lb0 + g] = take_a ? A[i] : B[j];
}

// Sorted keys -> (doc, tile) items of the three lists.
__global__ void __launch_bounds__(256) plan_extract_kernel(const unsigned long long* __restrict__ keys, int cap_r,
                                                           int cap, int2* fwd_items, int2* bwd_items,
                                                           int2* disp_items) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= cap) return;
  (blockIdx.y == 0 ? fwd_items : blockIdx.y == 1 ? bwd_items : disp_items)[i] =
      key_item(keys[(size_t)blockIdx.y * cap_r + i]);
}

hipError_t launch_plan(const int* cu, int ndocs, int causal, void* plan, const PlanLayout& pl, float* qk_scale,
                       hipStream_t stream) {
  char* base = static_cast<char*>(plan);
  int* counts = reinterpret_cast<int*>(base);
  int2* fwd_items = reinterpret_cast<int2*>(base + pl.fwd_offset);
  int2* bwd_items = reinterpret_cast<int2*>(base + pl.bwd_offset);
  int2* disp_items = reinterpret_cast<int2*>(base + pl.disp_offset);
  hipLaunchKernelGGL(plan_kernel, dim3(PLAN_LISTS), dim3(PLAN_THREADS), 0, stream, cu, ndocs, causal,
                     pl.cap_r > 0 ? 1 : 0, counts, fwd_items, bwd_items, disp_items, qk_scale,
                     reinterpret_cast<int*>(base + pl.det_offset), pl.det_cap);
  if (pl.cap_r == 0) return hipGetLastError();
  // cap_r: a multiple of PLAN_RUN holding cap_fwd = cap_bwd slots
  unsigned long long* k0 = reinterpret_cast<unsigned long long*>(base + pl.keys_offset);
  unsigned long long* k1 = k0 + PLAN_LISTS * (size_t)pl.cap_r;
  const dim3 g256((unsigned)((pl.cap_r + 255) / 256), PLAN_LISTS);
  hipLaunchKernelGGL(plan_fill_kernel, g256, dim3(256), 0, stream, cu, ndocs, causal, k0, pl.cap_r, counts);
  hipLaunchKernelGGL(plan_sort_runs_kernel, dim3((unsigned)(pl.cap_r / PLAN_RUN), PLAN_LISTS), dim3(PLAN_THREADS), 0,
                     stream, k0, pl.cap_r);
  for (int w = PLAN_RUN; w < pl.cap_r; w *= 2) {
    hipLaunchKernelGGL(plan_merge_kernel, g256, dim3(256), 0, stream, k0, k1, pl.cap_r, w);
    std::swap(k0, k1);
  }
  hipLaunchKernelGGL(plan_extract_kernel, dim3((unsigned)((pl.cap_fwd + 255) / 256), PLAN_LISTS), dim3(256), 0,
                     stream, k0, pl.cap_r, pl.cap_fwd, fwd_items, bwd_items, disp_items);
  return hipGetLastError();
}

}  // namespace flamia
