// Device helpers shared by the flamia HIP kernels (gfx950 / CDNA4 only).
//
// Operand layouts of the gfx950 matrix-core instructions used here, as
// measured on the hardware:
//
// * v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulate).  A is
//   32 x 64 (M x K), B is 64 x 32 (K x N).  Lane l = 32*h + m holds, for A,
//   row m and for B, column m: bytes 0..15 are 16 K-values of K-block 0
//   (K 0..31) and bytes 16..31 are 16 K-values of K-block 1 (K 32..63); the
//   two lane halves h = 0, 1 hold complementary halves of each K-block.
//   Lane (m, h) supplies the UE8M0 scale of K-block h of its row (A) or
//   column (B).  Which 16 K-values a lane half holds inside a block is free,
//   provided A and B agree.  C is 32 x 32: lane (n, h) holds column n and,
//   in accumulator register rr = 4q + r, row 8q + 4h + r.
// * v_mfma_f32_32x32x16_bf16: same A/B/C arrangement with 8 bf16 per lane;
//   no scales, so any K assignment shared by A and B is valid.
// * Swapping A and B yields exactly the transposed C (bit for bit), which
//   lets the forward compute S^T and the backward S from the same products.
//
// The index convention used for every 32-token block of tokens is the
// "pi order": token t = 8q + 4h + r of the block (the row held by lane half h
// in register 4q + r of a C tile) is stored at position 16h + 4q + r, so a
// lane half's 16 tokens are contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flamia {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int TOKEN_BLOCK = 32;   // tokens per scale block
constexpr int FWD_BQ = 128;       // queries per forward work item
constexpr int FWD_BK = 64;        // keys per forward inner step
// Largest deferred rescale of the forward, in powers of two: P^'s operand
// scale 2^(fold reference + P_EXP + FWD_LAZY) stays a finite E8M0 value (at
// most 2^127) and the fp32 accumulators lose at most 2^8 of headroom.
constexpr int FWD_LAZY = 8;
constexpr int BWD_BQ = 64;        // queries per backward inner step
constexpr int BWD_BK = 128;       // keys per backward work item
constexpr int E8M0_BIAS = 127;
constexpr int P_EXP = -8;         // fixed exponent of the probability operand
constexpr int M_NONE = -(1 << 20);  // running row max before any visible key

__device__ __forceinline__ int pi_pos(int t) {   // t in [0, 32)
  return ((t >> 2) & 1) * 16 + (t >> 3) * 4 + (t & 3);
}

// ---------------------------------------------------------------- formats

// Smallest integer e with amax <= 448 * 2^e, from the fp32 bits:
// amax = m 2^k with m in [1, 2): e = k - 8 if m <= 1.75, else k - 7.
// amax == 0 (or an fp32 subnormal) gives -127; clamped to [-127, 127].
__device__ __forceinline__ int roundup_exp(float amax) {
  uint32_t b = __float_as_uint(amax) & 0x7fffffffu;
  int be = (int)(b >> 23);
  if (be == 0) return -127;
  int k = be - 127;
  int e = (b & 0x7fffffu) <= 0x600000u ? k - 8 : k - 7;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Two fp32 values -> two E4M3 codes (round to nearest even; inputs must be
// within +-464 in magnitude, which every caller guarantees).
__device__ __forceinline__ int cvt_fp8x2(float a, float b) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffff;
}
__device__ __forceinline__ int cvt_fp8x4(float a, float b, float c, float d) {
  // the first convert's upper half is overwritten by the second
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
__device__ __forceinline__ float fp8_value(int packed, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(packed, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(packed, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(packed, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(packed, 3);
  }
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}
// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ __bf16 f32_to_bf16(float f) {
  uint16_t b = f32_to_bf16_bits(f);
  return *reinterpret_cast<__bf16*>(&b);
}

// ---------------------------------------------------------------- matrix cores

__device__ __forceinline__ v16f mfma_f8(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave reductions

// Whole-wave maxima with DPP lane moves (no LDS round trips): pairs and quads,
// then halves and whole rows of 16 by mirroring, then rows 0-1 and 0-3 by the
// row broadcasts of lanes 15 and 31; lane 63 ends with the maximum, which is
// returned to every lane.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ float wave_max(float v) {
  auto mx = [](float a, int b) { return fmaxf(a, __int_as_float(b)); };
  v = mx(v, dpp_move<0xb1>(__float_as_int(v)));          // quad_perm [1,0,3,2]
  v = mx(v, dpp_move<0x4e>(__float_as_int(v)));          // quad_perm [2,3,0,1]
  v = mx(v, dpp_move<0x141>(__float_as_int(v)));         // row_half_mirror
  v = mx(v, dpp_move<0x140>(__float_as_int(v)));         // row_mirror
  v = mx(v, dpp_move<0x142, 0xa>(__float_as_int(v)));    // row_bcast:15 -> rows 1, 3
  v = mx(v, dpp_move<0x143, 0xc>(__float_as_int(v)));    // row_bcast:31 -> rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_move<0xb1>(v));
  v = max(v, dpp_move<0x4e>(v));
  v = max(v, dpp_move<0x141>(v));
  v = max(v, dpp_move<0x140>(v));
  v = max(v, dpp_move<0x142, 0xa>(v));
  v = max(v, dpp_move<0x143, 0xc>(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Index of the document containing packed token t (cu[d] <= t < cu[d+1]).
__device__ __forceinline__ int find_doc(const int* __restrict__ cu, int ndocs, int t) {
  int lo = 0, hi = ndocs - 1;   // largest d with cu[d] <= t
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- small loads

__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }
__device__ __forceinline__ void st16(void* p, v4i v) { *reinterpret_cast<v4i*>(p) = v; }

__device__ __forceinline__ v8i cat8(v4i lo, v4i hi) {
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Transpose a 4 x 4 byte block held as four dwords (row i = dword i, byte j
// = column j) into four dwords (dword j = column j, byte i = row i).
__device__ __forceinline__ void transpose4x4_b8(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                                uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3) {
  // interleave bytes of (r0, r1) and (r2, r3), then 16-bit halves
  uint32_t a0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
  uint32_t a1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
  uint32_t b0 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
  uint32_t b1 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
  c0 = __builtin_amdgcn_perm(b0, a0, 0x05040100u);           // a0.lo16 b0.lo16
  c1 = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
  c2 = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
  c3 = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
}

// ---------------------------------------------------------------- NVFP4 expansion
//
// bf16 bits of (E2M1 code) x (E4M3 group scale value s).  The product has at
// most 6 significant bits and lies in [2^-10, 2688], so it is exact in fp32
// and its top 16 bits are the exact bf16 value.
__device__ __forceinline__ uint32_t e2m1_times_bf16(uint32_t nib, float s) {
  const uint32_t e = (nib >> 1) & 3u, m = nib & 1u;
  const uint32_t mag = e == 0 ? (m ? 0x3f000000u : 0u) : (((126u + e) << 23) | (m << 22));
  const uint32_t v = __float_as_uint(__uint_as_float(mag) * s) | ((nib & 8u) << 28);
  return v >> 16;
}

// Eight E2M1 codes (one dword, element 0 in the low nibble) times s, as 8 bf16.
__device__ __forceinline__ v4i e2m1x8_times_bf16(uint32_t codes, float s) {
  v4i r;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = (int)(e2m1_times_bf16((codes >> (8 * k)) & 15u, s) | (e2m1_times_bf16((codes >> (8 * k + 4)) & 15u, s) << 16));
  return r;
}

// ---------------------------------------------------------------- LDS transpose reads
//
// gfx950 ds_read_b64_tr_b8 / _tr_b16, as measured on the hardware: within each
// 16-lane group, lane p receives, for b8, byte (p % 8) of the 8-byte rows
// addressed by lanes 2b + p / 8 (b = 0..7); for b16, element (p % 4) of the
// 8-byte rows addressed by lanes 4e + p / 4 (e = 0..3).  Letting the lanes of
// a group address 8 (or 4) token rows of a token-major tile turns a
// token-major tile into the MN-major operand of a matrix-core product.

__device__ __forceinline__ v2i lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p));
}
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4s lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
}

// 16 one-byte codes of one 32-token block for one column, in accumulator
// order (token 8(rr/4) + 4hh + rr%4 at byte rr), from a token-major byte tile
// (row = token, `stride` bytes).  `col0` is the first column of the lane's
// 16-lane group; the lane receives column col0 + (lane & 15).
__device__ __forceinline__ v4i tr_block16(const uint8_t* tile, int stride, int tok0, int col0, int lane) {
  const int p = lane & 15, hh = lane >> 5;
  const int b = p >> 1;
  const int t = tok0 + 8 * (b >> 2) + 4 * hh + (b & 3);
  const uint8_t* a0 = tile + t * stride + col0 + 8 * (p & 1);
  const v2i lo = lds_tr8(a0);
  const v2i hi = lds_tr8(a0 + 16 * stride);
  return v4i{lo[0], lo[1], hi[0], hi[1]};
}

// 8 bf16 of one column for the 16-token K-step `ks` of a 32-token block
// (tokens 8(2ks + e/4) + 4hh + e%4 at element e), from a token-major bf16
// tile (row = token, `stride` bytes); `col0` as above (in elements).
__device__ __forceinline__ v8bf tr_bf16x8(const uint8_t* tile, int stride, int tok0, int ks, int col0, int lane) {
  const int p = lane & 15, hh = lane >> 5;
  const int e = p >> 2, s = p & 3;
  const int t = tok0 + 16 * ks + 4 * hh + e;
  const uint8_t* a0 = tile + t * stride + 2 * (col0 + 4 * s);
  const v4s lo = lds_tr16(a0);
  const v4s hi = lds_tr16(a0 + 8 * stride);
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(v8bf, both);
}

// ---------------------------------------------------------------- swizzled LDS tiles
//
// Tiles staged by direct global->LDS loads are stored without padding; the
// 16-byte chunk c of row r sits at chunk c ^ key(r) of that row.  The keys
// spread the rows touched by one read instruction over all 64 banks:
// * code tiles (one byte per element, d-byte rows; read by 16-byte operand
//   loads of 32 rows and by 8-bit transpose reads of 16 rows);
// * wide tiles (bf16, 2d-byte rows; read by 16-bit transpose reads of 8 rows);
// * the mixed path's bf16 score operand (2d-byte rows; 16-byte operand loads
//   of 32 rows).
// Every key has period 16 in r or less, so row r + 16 shares the key of row r.

// d = 128: with m = (r >> 1) & 7 = (m2 m1 m0), key = (m0 m2 m1).  Rows of one
// parity get 8 distinct keys (16-byte reads of 16 rows), and the rows
// {0-3, 8-11} (+4) that one half-wave's 8-bit transpose read touches get
// disjoint chunk pairs.
template <int D> __device__ __forceinline__ int code_key(int r) {
  if constexpr (D == 128) {
    const int m = (r >> 1) & 7;
    return ((m & 1) << 2) | (((m >> 2) & 1) << 1) | ((m >> 1) & 1);
  } else {
    return (r >> 2) & 3;
  }
}
template <int D> __device__ __forceinline__ int wide_key(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 1));
}
template <int D> __device__ __forceinline__ int xq_key(int r) {
  return D == 128 ? wide_key<128>(r) : (r >> 1) & 7;
}
template <int D> __device__ __forceinline__ int code_off(int r, int byte) {
  return r * D + ((((byte >> 4) ^ code_key<D>(r))) << 4) + (byte & 15);
}
template <int D> __device__ __forceinline__ int wide_off(int r, int byte) {
  return r * 2 * D + ((((byte >> 4) ^ wide_key<D>(r))) << 4) + (byte & 15);
}
template <int D> __device__ __forceinline__ int xq_off(int r, int byte) {
  return r * 2 * D + ((((byte >> 4) ^ xq_key<D>(r))) << 4) + (byte & 15);
}

// Direct global -> LDS loads: every lane fetches 16 (or 4) bytes from its own
// global address; the wave's 64 results land contiguously at the
// wave-uniform LDS address `lds` (lane l at lds + 16 l, or + 4 l).
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}

// Workgroup barrier for LDS traffic only: outstanding global loads, LDS DMA
// and atomics stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0), vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Workgroup barrier after every outstanding memory operation of the wave
// (global loads, LDS DMA, atomics, LDS) has completed.
__device__ __forceinline__ void full_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// floor(x) as an integer in one instruction (finite x in int range).
__device__ __forceinline__ int cvt_floor_i32(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// ---------------------------------------------------------------- the probability evaluation
// Both passes evaluate P 2^8 = 2^(S' - m~ + 8) for a score S' and integer row
// maximum m~ the same way, so the backward's P^ codes replay the forward's:
// exp2 of S' whole (one transcendental), then the power of two 2^(8 - m~)
// applied exactly, for S' <= P_X_HI (exp2 finite) when either S' >= P_X_LO
// (exp2 a normal fp32 value) or m~ >= P_M_LO (then S' < -126 gives
// P 2^8 < 2^-18, E4M3 code 0, whatever exp2 returns there); otherwise
// 2^floor(S') exp2(fract(S')).  `kofs` = 8 - m~.
constexpr float P_X_LO = -126.f, P_X_HI = 120.f;
constexpr int P_M_LO = -100, P_M_HI = 120;

// exp2 on the FMA pipe (the optional polynomial evaluation of the pages'
// softmax scheduling, [Reading, 4.4] second bullet): 2^f for f in [0, 1) as
// q(f) = 1 + f (c1 + f (c2 + f (c3 + f (c4 + f c5)))), five FMAs in this
// order.  The coefficients minimise the largest relative error of q against
// 2^f on [0, 1] (8.3e-8; 2.4 ulp after fp32 rounding of the Horner steps), and
// q(0) = 1 exactly, so integer arguments give exact powers of two.
__device__ __forceinline__ float exp2_fma_frac(float f) {
  float q = 0.001867053215391934f;
  q = __builtin_fmaf(q, f, 0.00901719182729721f);
  q = __builtin_fmaf(q, f, 0.05579979717731476f);
  q = __builtin_fmaf(q, f, 0.24016447365283966f);
  q = __builtin_fmaf(q, f, 0.6931512951850891f);
  return __builtin_fmaf(q, f, 1.0f);
}
// 2^x = 2^floor(x) q(fract(x)) (rounded once where the result is subnormal)
__device__ __forceinline__ float exp2_fma(float x) {
  return __builtin_amdgcn_ldexpf(exp2_fma_frac(__builtin_amdgcn_fractf(x)), cvt_floor_i32(x));
}
// exp2 of the probability evaluation: the transcendental unit, or (POLY) the
// FMA-pipe polynomial.  Which blocks take the polynomial is fixed per 32 x 32
// (query block, key block) pair, so both passes make the same choice.
template <bool POLY>
__device__ __forceinline__ float exp2_p(float x) {
  if constexpr (POLY) return exp2_fma(x);
  else return __builtin_amdgcn_exp2f(x);
}
template <bool POLY = false>
__device__ __forceinline__ float p_scaled(float x, int kofs) {
  const float frac2 = POLY ? exp2_fma_frac(__builtin_amdgcn_fractf(x)) : __builtin_amdgcn_exp2f(__builtin_amdgcn_fractf(x));
  const float whole = __builtin_amdgcn_ldexpf(exp2_p<POLY>(x), kofs);
  const float split = __builtin_amdgcn_ldexpf(frac2, cvt_floor_i32(x) + kofs);
  return (x <= P_X_HI && (x >= P_X_LO || kofs <= 8 - P_M_LO)) ? whole : split;
}
// The polynomial takes the 32 x 32 blocks whose document-local query-block and
// key-block indices have an odd sum (half of the blocks; none on the diagonal).
__device__ __forceinline__ bool poly_block(int qb, int kb) { return ((qb + kb) & 1) != 0; }
// Rows whose m~ lies in [P_M_LO, P_M_HI] take the fast form, p_scaled's whole
// branch for every visible score (S' <= m~ <= 120), with 2^(8 - m~) applied
// inside the E4M3 convert (same codes as ldexp, then convert) and once to a
// block's sum (sums of 64 such values stay finite).
// ---------------------------------------------------------------- 4-bit probability operand
// The lane's 16 nonnegative values of one 32-key block (register rr = 4g + r
// holds key 8g + 4hh + r) in 4-bit form: groups of 16 consecutive keys are
// registers 0-7 and 8-15 of the two lane halves.  Per group, e = the smallest
// integer with max <= 6 2^e (the group maximum = M 2^k: e = k - 2 for M <= 1.5,
// else k - 1), the E2M1 codes of v / 2^e by the hardware convert (round to
// nearest even, dividing by its scale), and the values code x 2^e back as E4M3
// codes of value / sc (the convert's scale again; exact but below E4M3's
// range).  A group whose maximum is zero, subnormal or needs a scale below
// 2^-126 becomes zero (its values are then far below E4M3's range at any
// scale the callers pass).
__device__ __forceinline__ void p4_block(const float (&v)[16], float sc, int (&pc)[4]) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    float gm = fmaxf(fmaxf(fmaxf(v[8 * h2], v[8 * h2 + 1]), fmaxf(v[8 * h2 + 2], v[8 * h2 + 3])),
                     fmaxf(fmaxf(v[8 * h2 + 4], v[8 * h2 + 5]), fmaxf(v[8 * h2 + 6], v[8 * h2 + 7])));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(gm), __float_as_uint(gm), false, false);
    gm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const uint32_t b = __float_as_uint(gm);
    const int be = (int)(b >> 23);
    const int e = be - 127 - ((b & 0x7fffffu) <= 0x400000u ? 2 : 1);
    if (be == 0 || e < -126) {
      pc[2 * h2] = 0;
      pc[2 * h2 + 1] = 0;
      continue;
    }
    const float s2 = __builtin_amdgcn_ldexpf(1.0f, e);
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      const int g = 2 * h2 + g2;
      uint32_t c4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[4 * g], v[4 * g + 1], s2, 0);
      c4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c4, v[4 * g + 2], v[4 * g + 3], s2, 1);
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c4, s2, 0);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c4, s2, 1);
      v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, lo[0], lo[1], sc, false);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, hi[0], hi[1], sc, true);
      pc[g] = __builtin_bit_cast(int, w);
    }
  }
}

// E4M3 codes of a / sc .. d / sc for a power of two sc: the convert's scale
// divides exactly before its single rounding (the same codes as ldexp, then
// convert).
__device__ __forceinline__ int cvt_fp8x4_scaled(float a, float b, float c, float d, float sc) {
  // (the first convert's upper half is overwritten by the second)
  v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, a), a, b, sc, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, sc, true);
  return __builtin_bit_cast(int, w);
}

// Transpose reads of swizzled tiles: same results as tr_block16 / tr_bf16x8
// on the unswizzled tile.
template <int D>
__device__ __forceinline__ v4i tr_code16(const uint8_t* tile, int tok0, int col0, int lane) {
  const int p = lane & 15, hh = lane >> 5;
  const int b = p >> 1;
  const int t = tok0 + 8 * (b >> 2) + 4 * hh + (b & 3);
  const uint8_t* a0 = tile + code_off<D>(t, col0 + 8 * (p & 1));
  const v2i lo = lds_tr8(a0);
  const v2i hi = lds_tr8(a0 + 16 * D);
  return v4i{lo[0], lo[1], hi[0], hi[1]};
}
template <int D>
__device__ __forceinline__ v8bf tr_wide_bf16x8(const uint8_t* tile, int tok0, int ks, int col0, int lane) {
  const int p = lane & 15, hh = lane >> 5;
  const int e = p >> 2, s = p & 3;
  const int t = tok0 + 16 * ks + 4 * hh + e;
  const int byte = 2 * (col0 + 4 * s);
  const v4s lo = lds_tr16(tile + wide_off<D>(t, byte));
  const v4s hi = lds_tr16(tile + wide_off<D>(t + 8, byte));
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(v8bf, both);
}

// ---------------------------------------------------------------- bf16 rows, Hadamard back-rotation
//
// A (token, head) row of d fp32 values split over the four lanes of a quad,
// lane part k holding elements [k d/4, (k+1) d/4).
// In-place normalised Hadamard transform of a row split over the four lanes
// of a quad: butterflies h = 1 .. d/8 inside the lane, h = d/4 and d/2
// between lanes of the quad (lane part bit 0, then bit 1), then one multiply
// by fp32(1/sqrt(d)); the same butterflies in the same order as a whole-row
// transform, so the same fp32 results.
template <int D>
__device__ __forceinline__ void fwht_quarter_row(float (&x)[D / 4], int part) {
  constexpr int E = D / 4;
#pragma unroll
  for (int h = 1; h < E; h <<= 1)
#pragma unroll
    for (int a = 0; a < E; ++a)
      if ((a & h) == 0) {
        const float lo = x[a], hi = x[a + h];
        x[a] = lo + hi;
        x[a + h] = lo - hi;
      }
#pragma unroll
  for (int a = 0; a < E; ++a) {      // h = d/4: partner lane part ^ 1
    const float other = __int_as_float(dpp_move<0xb1>(__float_as_int(x[a])));   // quad_perm [1,0,3,2]
    x[a] = (part & 1) ? other - x[a] : x[a] + other;
  }
#pragma unroll
  for (int a = 0; a < E; ++a) {      // h = d/2: partner lane part ^ 2
    const float other = __int_as_float(dpp_move<0x4e>(__float_as_int(x[a])));   // quad_perm [2,3,0,1]
    x[a] = (part & 2) ? other - x[a] : x[a] + other;
  }
  const float inv_sqrt_d = D == 64 ? 0.125f : __uint_as_float(0x3db504f3u);
#pragma unroll
  for (int a = 0; a < E; ++a) x[a] = x[a] * inv_sqrt_d;
}

template <int N>
__device__ __forceinline__ void store_bf16(uint16_t* __restrict__ dst, const float (&x)[N]) {
#pragma unroll
  for (int c = 0; c < N / 8; ++c) {
    v4i w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (int)((uint32_t)f32_to_bf16_bits(x[8 * c + 2 * k]) | ((uint32_t)f32_to_bf16_bits(x[8 * c + 2 * k + 1]) << 16));
    st16(dst + 8 * c, w);
  }
}


}  // namespace flamia
