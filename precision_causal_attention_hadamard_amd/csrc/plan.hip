// GPU-built longest-first work lists of the packed call.
//
// The pages build the schedule once per microbatch on the GPU with a
// fixed-pass sort and hand items, costliest first, to the grid
// ([Summary, §3.6.2 Load-Balanced Scheduling]; [Reading, 4.4] last bullet).
// Here one workgroup enumerates every (document, tile), forms a 64-bit key
//   (COST_MAX - cost) << 44 | doc << 20 | tile
// and bitonic-sorts the keys in LDS.  The key is unique, so the order is the
// single correct one: cost descending, then document, then tile.  A tile
// later expands to num_heads consecutive grid items (head ascending).  The
// attention kernels read item blockIdx.x / H of the sorted list; the
// hardware dispatcher hands workgroups out in index order, which plays the
// role of the pages' dynamic fetch.
//
// Costs (number of tile pairs the causal tile touches):
//   forward  query tile t of a document of length L: floor((min((t+1)Bq, L)-1)/Bk) + 1
//   backward key tile u:                             ceil(L/Bq) - floor(u Bk / Bq)
#include "flamia_device.hpp"
#include "flamia_internal.hpp"

namespace flamia {

constexpr int PLAN_THREADS = 1024;

__device__ static void block_inclusive_scan(int* buf, int tid, int& total) {
  // Hillis-Steele inclusive scan on PLAN_THREADS ints, then shift.
  for (int off = 1; off < PLAN_THREADS; off <<= 1) {
    int v = buf[tid];
    int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] = v + add;
    __syncthreads();
  }
  total = buf[PLAN_THREADS - 1];
  __syncthreads();
}

__device__ static void build_sorted(const int* __restrict__ cu, int ndocs, bool fwd, int bq, int bk,
                                    unsigned long long* keys, int* scan, int* count_out,
                                    int2* __restrict__ out) {
  const int tid = threadIdx.x;
  int n_tiles = 0;
  // enumerate tiles, chunk of PLAN_THREADS documents at a time
  for (int base = 0; base < ndocs; base += PLAN_THREADS) {
    int d = base + tid;
    int L = 0, n = 0;
    if (d < ndocs) {
      L = cu[d + 1] - cu[d];
      n = fwd ? (L + bq - 1) / bq : (L + bk - 1) / bk;
    }
    scan[tid] = n;
    __syncthreads();
    int total;
    block_inclusive_scan(scan, tid, total);
    int first = n_tiles + scan[tid] - n;
    for (int t = 0; t < n; ++t) {
      int cost;
      if (fwd) {
        int e = min((t + 1) * bq, L);
        cost = (e - 1) / bk + 1;
      } else {
        cost = (L + bq - 1) / bq - (t * bk) / bq;
      }
      unsigned long long key = ((unsigned long long)(COST_MAX - cost) << 44) |
                               ((unsigned long long)d << 20) | (unsigned long long)t;
      keys[first + t] = key;
    }
    n_tiles += total;
    __syncthreads();
  }
  int n2 = 1;
  while (n2 < n_tiles) n2 <<= 1;
  for (int i = n_tiles + tid; i < n2; i += PLAN_THREADS) keys[i] = ~0ull;
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += PLAN_THREADS) {
        int ixj = i ^ j;
        if (ixj > i) {
          unsigned long long a = keys[i], b = keys[ixj];
          bool up = (i & k) == 0;
          if ((a > b) == up) { keys[i] = b; keys[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < n_tiles; i += PLAN_THREADS) {
    unsigned long long key = keys[i];
    out[i] = make_int2((int)((key >> 20) & 0xffffffull), (int)(key & 0xfffffull));
  }
  if (tid == 0) *count_out = n_tiles;
  __syncthreads();
}

__global__ void __launch_bounds__(PLAN_THREADS) plan_kernel(const int* __restrict__ cu, int ndocs,
                                                            int* counts, int2* fwd_items,
                                                            int2* bwd_items, float* qk_scale) {
  __shared__ unsigned long long keys[PLAN_MAX_TILES];
  __shared__ int scan[PLAN_THREADS];
  build_sorted(cu, ndocs, true, FWD_BQ, FWD_BK, keys, scan, counts + 0, fwd_items);
  build_sorted(cu, ndocs, false, BWD_BQ, BWD_BK, keys, scan, counts + 1, bwd_items);
  if (threadIdx.x == 0) { counts[2] = 0; counts[3] = 0; }
  // mixed path: clear the tensor-amax slots before the amax pass runs
  if (qk_scale != nullptr && threadIdx.x < 2) qk_scale[threadIdx.x] = 0.f;
}

hipError_t launch_plan(const int* cu, int ndocs, void* plan, const PlanLayout& pl, float* qk_scale,
                       hipStream_t stream) {
  char* base = static_cast<char*>(plan);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, cu, ndocs,
                     reinterpret_cast<int*>(base), reinterpret_cast<int2*>(base + pl.fwd_offset),
                     reinterpret_cast<int2*>(base + pl.bwd_offset), qk_scale);
  return hipGetLastError();
}

}  // namespace flamia
