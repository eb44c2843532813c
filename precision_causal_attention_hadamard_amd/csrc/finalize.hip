// Gradient finalisers of the backward pass.
//
// dQ: the fp16 accumulator holds dQ 2^-sigma (sigma per query block, chosen
// so partial sums stay inside fp16); multiply back by 2^sigma and the
// softmax scale.  dK (mixed path only; the MXFP8 backward kernel writes bf16
// dK itself): fp32 staging already carries the softmax scale.  With
// the Hadamard option on, both are rotated back with the same normalised
// Sylvester matrix as the forward rotation (it is symmetric and orthogonal):
// fp32 butterflies h = 1, 2, ..., d/2 then one multiply by fp32(1/sqrt(d)).
// Outputs are bf16 (round to nearest even).  Four lanes per (token, head) row.
#include "flamia_device.hpp"
#include "flamia_internal.hpp"

namespace flamia {

constexpr int FIN_THREADS = 256;
constexpr int FIN_PARTS = 4;     // lanes per row

template <int D>
__global__ void __launch_bounds__(FIN_THREADS)
finalize_kernel(Problem p, const uint16_t* __restrict__ dq_acc, const int* __restrict__ dq_sigma,
                const float* __restrict__ dk_f32, uint16_t* __restrict__ dq, uint16_t* __restrict__ dk,
                bool do_dq, bool with_dk) {
  constexpr int E = D / FIN_PARTS;
  const size_t rows = (size_t)p.T * p.H;
  const size_t row = ((size_t)blockIdx.x * FIN_THREADS + threadIdx.x) / FIN_PARTS;   // = t * H + h
  const int part = threadIdx.x & (FIN_PARTS - 1);
  // whole quads leave together, so the lane moves below see only live lanes
  if (row >= rows) return;
  const int t = (int)(row / p.H), h = (int)(row % p.H);
  const size_t off = row * D + (size_t)part * E;
  if (do_dq) {
    float x[E];
    const int sig = dq_sigma[(size_t)h * p.T + t];
    v4i acc[E / 8];
#pragma unroll
    for (int c = 0; c < E / 8; ++c) acc[c] = ld16(dq_acc + off + 8 * c);
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
      const v4i w = acc[c];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t u = (uint32_t)w[k];
        _Float16 lo, hi;
        uint16_t ul = (uint16_t)(u & 0xffffu), uh = (uint16_t)(u >> 16);
        __builtin_memcpy(&lo, &ul, 2);
        __builtin_memcpy(&hi, &uh, 2);
        x[8 * c + 2 * k] = __builtin_amdgcn_ldexpf((float)lo, sig) * p.softmax_scale;
        x[8 * c + 2 * k + 1] = __builtin_amdgcn_ldexpf((float)hi, sig) * p.softmax_scale;
      }
    }
    if (p.hadamard) fwht_quarter_row<D>(x, part);
    store_bf16<E>(dq + off, x);
  }
  if (with_dk) {
    float x[E];
#pragma unroll
    for (int c = 0; c < E / 4; ++c) {
      const v4f w = *reinterpret_cast<const v4f*>(dk_f32 + off + 4 * c);
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * c + k] = w[k];
    }
    if (p.hadamard) fwht_quarter_row<D>(x, part);
    store_bf16<E>(dk + off, x);
  }
}

// The rotation of fwht_quarter_row with the row dealt out in 16-byte chunks:
// lane `part` of the quad holds chunks part, part + 4, ..., so element
// 32 c + 8 part + k sits in x[8 c + k].  The butterflies run in the same order
// h = 1, 2, ..., d/2 with the same sums and differences as fwht_quarter_row,
// so the results are the same bit for bit; only which of them cross lanes
// (h = 8, 16) differs.
template <int D>
__device__ __forceinline__ void fwht_chunked_row(float (&x)[D / 4], int part) {
  constexpr int E = D / 4, NC = D / 32;
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int a = 0; a < E; ++a)
      if ((a & h) == 0) {
        const float lo = x[a], hi = x[a + h];
        x[a] = lo + hi;
        x[a + h] = lo - hi;
      }
#pragma unroll
  for (int a = 0; a < E; ++a) {      // h = 8: partner lane part ^ 1
    const float other = __int_as_float(dpp_move<0xb1>(__float_as_int(x[a])));
    x[a] = (part & 1) ? other - x[a] : x[a] + other;
  }
#pragma unroll
  for (int a = 0; a < E; ++a) {      // h = 16: partner lane part ^ 2
    const float other = __int_as_float(dpp_move<0x4e>(__float_as_int(x[a])));
    x[a] = (part & 2) ? other - x[a] : x[a] + other;
  }
#pragma unroll
  for (int hc = 1; hc < NC; hc <<= 1)  // h = 32 (and 64 at d = 128): across the lane's chunks
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if ((c & hc) == 0)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float lo = x[8 * c + k], hi = x[8 * (c + hc) + k];
          x[8 * c + k] = lo + hi;
          x[8 * (c + hc) + k] = lo - hi;
        }
  const float inv_sqrt_d = D == 64 ? 0.125f : __uint_as_float(0x3db504f3u);
#pragma unroll
  for (int a = 0; a < E; ++a) x[a] = x[a] * inv_sqrt_d;
}

// Deterministic mode: the fp16 accumulator of a query row is rebuilt from the
// step partials of every key tile that sees the query, added in fp16 in
// ascending key-tile order, then scaled, rotated back and rounded as in
// finalize_kernel.  A block covers 64 consecutive tokens of one head, four
// lanes a row.  Lane `part` holds the 16-byte chunks part, part + 4, ... of the
// row, so the four lanes of a row read 64 contiguous bytes of a partial per
// instruction and a wave's instruction covers 16 consecutive rows of one
// slot.  The loop has no divergent branches, so the partials of DET_RING key
// tiles stay in flight: its trip count is the wave's largest, a row's loads
// past its last key tile re-read that tile and its adds there are masked.  A
// row one of whose partials did not fit the workspace (max_doc_len
// under-promised) is written as NaN; its loads read its own output row.
constexpr int DET_ROWS = FIN_THREADS / FIN_PARTS;   // tokens per block
constexpr int DET_RING = 4;                         // key tiles in flight per row

template <int D>
__global__ void __launch_bounds__(FIN_THREADS)
finalize_dq_det_kernel(Problem p, const uint16_t* __restrict__ dq_part, const int* __restrict__ det_base,
                       int det_cap, const int* __restrict__ dq_sigma, uint16_t* __restrict__ dq) {
  constexpr int NC = D / 32;          // 16-byte chunks per lane
  constexpr int E = D / 4;
  // token blocks from the last to the first, so each document's longest rows
  // (its last queries, which see the most key tiles) start first
  const int h = (int)(blockIdx.x % (unsigned)p.H);
  const int nblk = (p.T + DET_ROWS - 1) / DET_ROWS;
  const int t_row = (nblk - 1 - (int)(blockIdx.x / (unsigned)p.H)) * DET_ROWS + (int)(threadIdx.x / FIN_PARTS);
  const int part = threadIdx.x & (FIN_PARTS - 1);
  // every lane stays to the end (the wave maximum and the row transform read
  // other lanes); a row past the last token works on the last token and
  // stores nothing
  const bool live = t_row < p.T;
  const int t = live ? t_row : p.T - 1;
  const int d = find_doc(p.cu, p.ndocs, t);
  const int s0 = p.cu[d], L = p.cu[d + 1] - s0, lp = t - s0;
  const int qt = lp / BWD_BQ, r = lp % BWD_BQ;
  const int nq = (L + BWD_BQ - 1) / BWD_BQ, nk = (L + BWD_BK - 1) / BWD_BK;
  const int umax = p.causal ? min(qt / 2, nk - 1) : nk - 1;
  const int base = det_base[d];
  const int sig = dq_sigma[(size_t)h * p.T + t];
  uint16_t* const dst = dq + ((size_t)t * p.H + h) * D + 8 * part;
  // a row's step indices grow with the key tile, so the last one decides
  const bool lost = det_step(base, umax, qt, nq, p.causal) >= det_cap;
  const uint16_t* const row0 = dq_part + ((size_t)h * BWD_BQ + r) * D + 8 * part;
  const size_t per_step = (size_t)p.H * BWD_BQ * D;
  auto load = [&](v4i (&c4)[NC], int u) {
    const uint16_t* src = lost ? dst : row0 + (size_t)det_step(base, min(u, umax), qt, nq, p.causal) * per_step;
#pragma unroll
    for (int c = 0; c < NC; ++c) c4[c] = ld16(src + 32 * c);
  };
  v8h acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = v8h{};
  const int uw = wave_max_i(umax);
  v4i ring[DET_RING][NC];
#pragma unroll
  for (int i = 0; i < DET_RING; ++i) load(ring[i], i);
  for (int u = 0; u <= uw; u += DET_RING) {
#pragma unroll
    for (int i = 0; i < DET_RING; ++i) {
      const bool take = u + i <= umax;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v8h s = acc[c] + __builtin_bit_cast(v8h, ring[i][c]);
        acc[c] = take ? s : acc[c];
      }
      load(ring[i], u + i + DET_RING);
    }
  }
  float x[E];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int k = 0; k < 8; ++k)
      x[8 * c + k] = lost ? __builtin_nanf("") : __builtin_amdgcn_ldexpf((float)acc[c][k], sig) * p.softmax_scale;
  if (p.hadamard) fwht_chunked_row<D>(x, part);
  if (!live) return;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    v4i w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (int)((uint32_t)f32_to_bf16_bits(x[8 * c + 2 * k]) | ((uint32_t)f32_to_bf16_bits(x[8 * c + 2 * k + 1]) << 16));
    st16(dst + 32 * c, w);
  }
}

// dQ without the rotation, deterministic slots or dK: the same arithmetic as
// finalize_kernel, with the accumulator read and dq written in whole 1 KB
// pieces per wave instruction (16 bytes a lane, consecutive lanes on
// consecutive bytes); FIN_FLAT pieces a thread, all loads issued first.
constexpr int FIN_FLAT = 4;
template <int D>
__global__ void __launch_bounds__(FIN_THREADS)
finalize_dq_flat_kernel(Problem p, const uint16_t* __restrict__ dq_acc, const int* __restrict__ dq_sigma,
                        uint16_t* __restrict__ dq) {
  const size_t n8 = (size_t)p.T * p.H * (D / 8);       // 16-byte pieces
  const size_t first = (size_t)blockIdx.x * (FIN_THREADS * FIN_FLAT) + threadIdx.x;
  v4i w[FIN_FLAT];
  int sig[FIN_FLAT];
#pragma unroll
  for (int c = 0; c < FIN_FLAT; ++c) {
    const size_t idx = first + (size_t)c * FIN_THREADS;
    if (idx < n8) {
      w[c] = ld16(dq_acc + idx * 8);
      const size_t row = idx / (D / 8);                 // = t * H + h
      const int t = (int)(row / p.H), h = (int)(row % p.H);
      sig[c] = dq_sigma[(size_t)h * p.T + t];
    }
  }
#pragma unroll
  for (int c = 0; c < FIN_FLAT; ++c) {
    const size_t idx = first + (size_t)c * FIN_THREADS;
    if (idx < n8) {
      float x[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t u = (uint32_t)w[c][k];
        _Float16 lo, hi;
        uint16_t ul = (uint16_t)(u & 0xffffu), uh = (uint16_t)(u >> 16);
        __builtin_memcpy(&lo, &ul, 2);
        __builtin_memcpy(&hi, &uh, 2);
        x[2 * k] = __builtin_amdgcn_ldexpf((float)lo, sig[c]) * p.softmax_scale;
        x[2 * k + 1] = __builtin_amdgcn_ldexpf((float)hi, sig[c]) * p.softmax_scale;
      }
      store_bf16<8>(dq + idx * 8, x);
    }
  }
}

// Split groups (grouped query attention with the group spread over several
// backward items): dK and dV of each (token, key/value head) row are the sums
// of the gsplit fp32 partials, added in part order; dK is rotated back with the
// Hadamard option; both are rounded to bf16 once.  Four lanes per row.
template <int D>
__global__ void __launch_bounds__(FIN_THREADS)
group_reduce_kernel(Problem p, int gsplit, const float* __restrict__ dk_f32, const float* __restrict__ dv_f32,
                    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  constexpr int E = D / FIN_PARTS;
  const size_t rows = (size_t)p.T * p.Hk;
  const size_t row = ((size_t)blockIdx.x * FIN_THREADS + threadIdx.x) / FIN_PARTS;
  const int part = threadIdx.x & (FIN_PARTS - 1);
  if (row >= rows) return;      // whole quads leave together
  const size_t off = row * D + (size_t)part * E, plane = rows * D;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const float* src = (which == 0 ? dk_f32 : dv_f32) + off;
    float x[E];
#pragma unroll
    for (int c = 0; c < E / 4; ++c) {
      const v4f w = *reinterpret_cast<const v4f*>(src + 4 * c);
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * c + k] = w[k];
    }
    for (int s = 1; s < gsplit; ++s) {
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        const v4f w = *reinterpret_cast<const v4f*>(src + (size_t)s * plane + 4 * c);
#pragma unroll
        for (int k = 0; k < 4; ++k) x[4 * c + k] = x[4 * c + k] + w[k];
      }
    }
    if (which == 0 && p.hadamard) fwht_quarter_row<D>(x, part);
    store_bf16<E>((which == 0 ? dk : dv) + off, x);
  }
}

hipError_t launch_group_reduce(const Problem& p, int gsplit, const float* dk_f32, const float* dv_f32, void* dk,
                               void* dv, hipStream_t stream) {
  const size_t rows = (size_t)p.T * p.Hk;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows * FIN_PARTS + FIN_THREADS - 1) / FIN_THREADS));
  if (p.D == 64)
    hipLaunchKernelGGL(group_reduce_kernel<64>, grid, dim3(FIN_THREADS), 0, stream, p, gsplit, dk_f32, dv_f32,
                       (uint16_t*)dk, (uint16_t*)dv);
  else
    hipLaunchKernelGGL(group_reduce_kernel<128>, grid, dim3(FIN_THREADS), 0, stream, p, gsplit, dk_f32, dv_f32,
                       (uint16_t*)dk, (uint16_t*)dv);
  return hipGetLastError();
}

hipError_t launch_finalize(const Problem& p, const void* dq_acc, const int* dq_sigma,
                           const float* dk_f32, void* dq, void* dk, bool with_dk, const void* dq_part,
                           const int* det_base, int det_cap, hipStream_t stream) {
  const size_t rows = (size_t)p.T * p.H;
  if (rows == 0) return hipSuccess;
  if (!p.hadamard && !p.deterministic && !with_dk) {
    const size_t n8 = rows * (size_t)(p.D / 8);
    dim3 gf((unsigned)((n8 + FIN_THREADS * FIN_FLAT - 1) / (FIN_THREADS * FIN_FLAT)));
    if (p.D == 64)
      hipLaunchKernelGGL(finalize_dq_flat_kernel<64>, gf, dim3(FIN_THREADS), 0, stream, p, (const uint16_t*)dq_acc,
                         dq_sigma, (uint16_t*)dq);
    else
      hipLaunchKernelGGL(finalize_dq_flat_kernel<128>, gf, dim3(FIN_THREADS), 0, stream, p, (const uint16_t*)dq_acc,
                         dq_sigma, (uint16_t*)dq);
    return hipGetLastError();
  }
  if (p.deterministic) {
    dim3 gd((unsigned)(((size_t)p.T + DET_ROWS - 1) / DET_ROWS * p.H));
    if (p.D == 64)
      hipLaunchKernelGGL(finalize_dq_det_kernel<64>, gd, dim3(FIN_THREADS), 0, stream, p, (const uint16_t*)dq_part,
                         det_base, det_cap, dq_sigma, (uint16_t*)dq);
    else
      hipLaunchKernelGGL(finalize_dq_det_kernel<128>, gd, dim3(FIN_THREADS), 0, stream, p, (const uint16_t*)dq_part,
                         det_base, det_cap, dq_sigma, (uint16_t*)dq);
    if (!with_dk) return hipGetLastError();
  }
  const bool do_dq = !p.deterministic;
  dim3 grid((unsigned)((rows * FIN_PARTS + FIN_THREADS - 1) / FIN_THREADS));
  if (p.D == 64)
    hipLaunchKernelGGL(finalize_kernel<64>, grid, dim3(FIN_THREADS), 0, stream, p,
                       (const uint16_t*)dq_acc, dq_sigma, dk_f32, (uint16_t*)dq, (uint16_t*)dk, do_dq, with_dk);
  else
    hipLaunchKernelGGL(finalize_kernel<128>, grid, dim3(FIN_THREADS), 0, stream, p,
                       (const uint16_t*)dq_acc, dq_sigma, dk_f32, (uint16_t*)dq, (uint16_t*)dk, do_dq, with_dk);
  return hipGetLastError();
}

}  // namespace flamia
