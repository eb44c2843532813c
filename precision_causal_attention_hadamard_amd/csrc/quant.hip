// Fused quantizers of the training call (HBM-bound).
//
// quant_qkv_kernel: one workgroup per (32-token chunk of the packed array,
// tensor in {Q, K, V}); it quantizes every document-local 32-token block
// that STARTS in its chunk, for all heads of the tensor (wave w takes heads
// w, w+4, ...; K and V have the key/value heads).
// A block never crosses a document, so a document boundary may fall
// anywhere inside a chunk and a block may run past the chunk's end.
// Per (block, head): load 32 rows x d bf16 (lane = (row, half-row)),
// optional fp32 Hadamard butterflies on Q and K, amax over the block, the
// round-up exponent, E4M3 codes; for V also the per-key exponents, per-key
// codes and the per-query fold reference (prefix max of the per-key
// exponents inside the block; the block exponent when the call is not
// causal).  [Summary, §3.1 Token-Block Scaling; §3.2 Causally Safe Scales;
// §4.3 Ablation Study]; [Reading, 4.4] first bullet.  Code rows leave as
// whole rows per store instruction through a wave-private LDS tile.
// Exact option: one exponent per token instead of per block (V's block and
// per-key codes then coincide), and K's in-block prefix maximum of the
// per-token exponents for the causal dQ prescale.
//
// quant_do_kernel: the backward's preparation, per block and head: token-block
// codes of dO, D_i = sum_d dO~_id O_id from the same codes ([Summary, §3.3]:
// D uses the quantized dO that dP uses), G_i = dO~_i 2^-8 / l_i in bf16 (the
// right operand of dV = P^T G), the dQ accumulator prescale exponent of the
// block, and zeroes the block's rows of the fp16 dQ accumulator.  G and the
// zeros leave as whole rows per store instruction (G through a wave-private
// LDS tile): half-row stores from each lane left partial lines that doubled
// the write traffic.
#include "flamia_device.hpp"
#include "flamia_internal.hpp"

namespace flamia {

constexpr int QUANT_THREADS = 256;

// Calls f(block_start, block_end, doc_start, doc) for every document-local
// 32-token block that starts inside chunk [c0, c0 + 32).  Uniform across the
// workgroup.
template <typename F>
__device__ __forceinline__ void for_blocks_in_chunk(const int* __restrict__ cu, int ndocs, int T, int c0, F f) {
  const int cend = min(c0 + TOKEN_BLOCK, T);
  int d = find_doc(cu, ndocs, c0);
  int s = cu[d], e = cu[d + 1];
  int p = s + ((c0 - s + TOKEN_BLOCK - 1) / TOKEN_BLOCK) * TOKEN_BLOCK;
  while (true) {
    if (p >= e) {               // document exhausted (or empty): next document
      if (d + 1 >= ndocs) break;
      ++d;
      s = cu[d];
      e = cu[d + 1];
      p = s;
      continue;
    }
    if (p >= cend) break;       // next block of this document starts past the chunk
    f(p, min(p + TOKEN_BLOCK, e), s, d);
    p += TOKEN_BLOCK;
  }
}

template <int D>
__device__ __forceinline__ void load_half_row(const uint16_t* __restrict__ src, bool valid, float (&x)[D / 2]) {
  if (valid) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      v4i w = ld16(src + 8 * c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t u = (uint32_t)w[j];
        x[8 * c + 2 * j] = __uint_as_float(u << 16);
        x[8 * c + 2 * j + 1] = __uint_as_float(u & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < D / 2; ++i) x[i] = 0.f;
  }
}

// In-place normalised Hadamard transform of a d-row split over two lanes
// (lane half `hf` holds channels [hf d/2, (hf+1) d/2)).  For h = 1, 2, ...,
// d/2 every pair (a, a+h) of each aligned 2h-group becomes
// (x_a + x_{a+h}, x_a - x_{a+h}) in fp32 (round to nearest even), then every
// element is multiplied once by fp32(1/sqrt(d)).  The last stage pairs the
// two lanes of a row.
template <int D>
__device__ __forceinline__ void fwht_half_row(float (&x)[D / 2], int hf) {
#pragma unroll
  for (int h = 1; h < D / 2; h <<= 1) {
#pragma unroll
    for (int a = 0; a < D / 2; ++a) {
      if ((a & h) == 0) {
        float lo = x[a], hi = x[a + h];
        x[a] = lo + hi;
        x[a + h] = lo - hi;
      }
    }
  }
#pragma unroll
  for (int a = 0; a < D / 2; ++a) {
    float other = __shfl_xor(x[a], 1, 64);
    x[a] = hf == 0 ? x[a] + other : other - x[a];
  }
  const float inv_sqrt_d = D == 64 ? 0.125f : __uint_as_float(0x3db504f3u);  // fp32(2^-3.5)
#pragma unroll
  for (int a = 0; a < D / 2; ++a) x[a] = x[a] * inv_sqrt_d;
}

// LDS slot (16-byte unit within a d-byte code row) of chunk c of half hf of
// row r of a wave's code tile: XOR-swizzled within the half by the row and the
// half, so the half-row writes (8 lanes per pass) spread over the banks.
template <int D>
__device__ __forceinline__ int code_slot(int r, int hf, int c) {
  constexpr int HC = D / 32;                       // chunks per half-row
  return hf * HC + (c ^ (r & (HC - 1)) ^ (hf * (HC / 2)));
}

// Codes of the half-rows of one 32-token block (lane = (row, half)), scaled
// by 2^-e (exact), to memory as whole rows per store instruction: the
// half-rows go through the wave's LDS tile `stage` (32 x d bytes), then 2d/32
// lanes per row store 16 bytes each.  Rows at or past nrows are not stored.
template <int D>
__device__ __forceinline__ void store_codes(uint8_t* __restrict__ dst_row0, size_t row_stride, int nrows,
                                            uint8_t* stage, const float (&x)[D / 2], int e) {
  constexpr int HC = D / 32, CPR = 2 * HC, RPI = 64 / CPR;
  const int lane = threadIdx.x & 63, row = lane >> 1, hf = lane & 1;
#pragma unroll
  for (int c = 0; c < HC; ++c) {
    v4i w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 16 * c + 4 * j;
      w[j] = cvt_fp8x4(__builtin_amdgcn_ldexpf(x[b], -e), __builtin_amdgcn_ldexpf(x[b + 1], -e),
                       __builtin_amdgcn_ldexpf(x[b + 2], -e), __builtin_amdgcn_ldexpf(x[b + 3], -e));
    }
    st16(stage + row * D + 16 * code_slot<D>(row, hf, c), w);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / CPR, lc = lane % CPR;
    if (r < nrows) st16(dst_row0 + (size_t)r * row_stride + 16 * lc, ld16(stage + r * D + 16 * code_slot<D>(r, lc / HC, lc % HC)));
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int D>
__device__ __forceinline__ float half_row_amax(const float (&x)[D / 2]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < D / 2; ++i) m = fmaxf(m, fabsf(x[i]));
  return m;
}

// ---------------------------------------------------------------- NVFP4 (mixed path)
//
// Score operands of the mixed path: E2M1 elements, one E4M3 scale per 16
// head-dimension elements of a token, one fp32 tensor scale t = amax / 2688
// per tensor ([Summary] opening paragraphs; [Reading, part 一] NVFP4 format).
// The group scale is the smallest E4M3 value >= amax_group / fp32(6 t)
// (the round-up rule for a non-power-of-two scale), capped at 448; element
// codes are E2M1(x / fp32(s t)) rounded to nearest even, saturating at 6.

// E2M1 code (bit 3 = sign) of v, round to nearest even, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t idx = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return ((__float_as_uint(v) >> 28) & 8u) | idx;
}

// Smallest E4M3 code whose value is >= q (q >= 0); 448 when q >= 448.
__device__ __forceinline__ int e4m3_round_up_code(float q) {
  if (q >= 448.f) return 0x7e;
  int code = cvt_fp8x2(q, 0.f) & 0xff;
  if (fp8_value(code, 0) < q) ++code;
  return code;
}

template <int D>
__global__ void __launch_bounds__(QUANT_THREADS)
amax_qk_kernel(Problem p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               float* __restrict__ qk_scale) {
  const int tensor = blockIdx.y;
  const uint16_t* src = tensor == 0 ? q : k;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = lane >> 1, hf = lane & 1;
  const int c0 = blockIdx.x * TOKEN_BLOCK;
  const int H = tensor == 0 ? p.H : p.Hk, T = p.T;
  float m = 0.f;
  for_blocks_in_chunk(p.cu, p.ndocs, T, c0, [&](int bs, int be, int, int) {
    const int tok = bs + row;
    const bool valid = tok < be;
    for (int h = wave; h < H; h += QUANT_THREADS / 64) {
      const size_t off = ((size_t)tok * H + h) * D + hf * (D / 2);
      float x[D / 2];
      load_half_row<D>(src + off, valid, x);
      if (p.hadamard) fwht_half_row<D>(x, hf);
      m = fmaxf(m, half_row_amax<D>(x));
    }
  });
  m = wave_max(m);
  if (lane == 0 && m > 0.f)
    atomicMax(reinterpret_cast<unsigned int*>(qk_scale) + tensor, __float_as_uint(m));
}

// NVFP4 codes and group scales of one half-row (lane half hf of a token row),
// and each element's code x group scale as bf16 (exact).
template <int D>
__device__ __forceinline__ void store_nvfp4(uint8_t* __restrict__ fp4, uint8_t* __restrict__ sf,
                                            uint16_t* __restrict__ xb, const float (&x)[D / 2], float t) {
  const float six_t = 6.0f * t;
  uint32_t packed[D / 16];     // the half-row's D/2 codes, 8 per dword
  uint32_t sfw = 0;
#pragma unroll
  for (int gi = 0; gi < D / 32; ++gi) {
    float gmax = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) gmax = fmaxf(gmax, fabsf(x[16 * gi + e]));
    const int code = e4m3_round_up_code(gmax / six_t);
    sfw |= (uint32_t)code << (8 * gi);
    const float sv = fp8_value(code, 0);
    const float st = sv * t;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = st > 0.f ? x[16 * gi + 8 * w + e] / st : 0.f;
        word |= e2m1_code(v) << (4 * e);
      }
      packed[2 * gi + w] = word;
      st16(xb + 16 * gi + 8 * w, e2m1x8_times_bf16(word, sv));
    }
  }
#pragma unroll
  for (int c = 0; c < D / 64; ++c)
    st16(fp4 + 16 * c, v4i{(int)packed[4 * c], (int)packed[4 * c + 1], (int)packed[4 * c + 2], (int)packed[4 * c + 3]});
  if (D / 32 == 4) *reinterpret_cast<uint32_t*>(sf) = sfw;
  else *reinterpret_cast<uint16_t*>(sf) = (uint16_t)sfw;
}

template <int D>
__global__ void __launch_bounds__(QUANT_THREADS)
quant_qkv_kernel(Problem p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, uint8_t* __restrict__ q_codes,
                 uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes,
                 uint8_t* __restrict__ v_key_codes, uint8_t* __restrict__ q_exp,
                 uint8_t* __restrict__ k_exp, uint8_t* __restrict__ v_exp,
                 uint8_t* __restrict__ v_key_exp, uint8_t* __restrict__ v_ref_exp,
                 uint8_t* __restrict__ k_ref_exp, Fp4Operands f4) {
  __shared__ __attribute__((aligned(16))) uint8_t cstage[QUANT_THREADS / 64][32 * D];   // code rows of a block
  const int tensor = blockIdx.y;
  const bool nvfp4 = p.path == 1 && tensor < 2;
  float t = 1.f;
  if (nvfp4) {
    const float amax = f4.qk_scale[tensor];
    t = amax > 0.f ? amax / 2688.0f : 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) f4.qk_scale[2 + tensor] = t;
  }
  const uint16_t* src = tensor == 0 ? q : (tensor == 1 ? k : v);
  uint8_t* codes = tensor == 0 ? q_codes : (tensor == 1 ? k_codes : v_codes);
  uint8_t* exps = tensor == 0 ? q_exp : (tensor == 1 ? k_exp : v_exp);
  const bool rotate = p.hadamard && tensor < 2;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = lane >> 1, hf = lane & 1;
  const int c0 = blockIdx.x * TOKEN_BLOCK;
  const int H = tensor == 0 ? p.H : p.Hk, T = p.T;      // K and V carry the key/value heads

  for_blocks_in_chunk(p.cu, p.ndocs, T, c0, [&](int bs, int be, int, int) {
    const int tok = bs + row;
    const bool valid = tok < be;
    for (int h = wave; h < H; h += QUANT_THREADS / 64) {
      const size_t off = ((size_t)tok * H + h) * D + hf * (D / 2);
      float x[D / 2];
      load_half_row<D>(src + off, valid, x);
      if (rotate) fwht_half_row<D>(x, hf);
      const float lane_amax = half_row_amax<D>(x);
      // exact option: one exponent per token (the row's two lane halves)
      const int e = roundup_exp(p.exact ? fmaxf(lane_amax, __shfl_xor(lane_amax, 1, 64)) : wave_max(lane_amax));
      store_codes<D>(codes + ((size_t)bs * H + h) * D, (size_t)H * D, be - bs, cstage[wave], x, e);
      if (valid) {
        if (hf == 0) exps[(size_t)h * T + tok] = (uint8_t)(e + E8M0_BIAS);
        if (nvfp4)
          store_nvfp4<D>((tensor == 0 ? f4.q_fp4 : f4.k_fp4) + off / 2,
                         (tensor == 0 ? f4.q_sf : f4.k_sf) + off / 16, (tensor == 0 ? f4.q_x : f4.k_x) + off, x, t);
      }
      if (tensor == 1 && p.exact) {
        // prefix max of the per-token K exponents over rows 0..row of the block
        int ref = valid ? e : -127;
#pragma unroll
        for (int o = 2; o < 64; o <<= 1) {
          int up = __shfl_up(ref, o, 64);
          if (lane >= o) ref = max(ref, up);
        }
        if (valid && hf == 0) k_ref_exp[(size_t)h * T + tok] = (uint8_t)(ref + E8M0_BIAS);
      }
      if (tensor == 2) {
        const float row_amax = fmaxf(lane_amax, __shfl_xor(lane_amax, 1, 64));
        const int ek = roundup_exp(row_amax);
        // prefix max of per-key exponents over rows 0..row of the block
        int ref = valid ? ek : -127;
#pragma unroll
        for (int o = 2; o < 64; o <<= 1) {
          int up = __shfl_up(ref, o, 64);
          if (lane >= o) ref = max(ref, up);
        }
        store_codes<D>(v_key_codes + ((size_t)bs * H + h) * D, (size_t)H * D, be - bs, cstage[wave], x, ek);
        if (valid) {
          if (hf == 0) {
            v_key_exp[(size_t)h * T + tok] = (uint8_t)(ek + E8M0_BIAS);
            // without the mask every key of the block is visible: the
            // reference is the block's largest per-key exponent, i.e. e
            v_ref_exp[(size_t)h * T + tok] = (uint8_t)((p.causal ? ref : e) + E8M0_BIAS);
          }
        }
      }
    }
  });
}

// LDS slot (16-byte unit within a 2d-byte row) of chunk c of half hf of row r
// of a wave's G tile: chunks are XOR-swizzled within their half by the row and
// the half, so that both the half-row writes (8 lanes per pass) and the
// whole-row reads (16 lanes per pass) hit distinct banks.
template <int D>
__device__ __forceinline__ int g_slot(int r, int hf, int c) {
  constexpr int HC = D / 16;                       // chunks per half-row
  return hf * HC + (c ^ (r & (HC - 1)) ^ (hf * (HC / 2)));
}

template <int D>
__global__ void __launch_bounds__(QUANT_THREADS)
quant_do_kernel(Problem p, const uint16_t* __restrict__ dout, const uint16_t* __restrict__ o,
                const int* __restrict__ row_max, const float* __restrict__ row_sum,
                const uint8_t* __restrict__ q_exp,
                const uint8_t* __restrict__ k_exp, const uint8_t* __restrict__ v_exp,
                const uint8_t* __restrict__ v_ref_exp, const uint8_t* __restrict__ k_ref_exp,
                uint8_t* __restrict__ do_codes,
                uint8_t* __restrict__ do_exp, int* __restrict__ kofs, float* __restrict__ delta,
                float* __restrict__ il8,
                int* __restrict__ qexps, uint16_t* __restrict__ g, int* __restrict__ dq_sigma,
                uint16_t* __restrict__ dq_acc) {
  __shared__ __attribute__((aligned(16))) uint8_t cstage[QUANT_THREADS / 64][32 * D];       // dO~ code rows of a block
  __shared__ __attribute__((aligned(16))) uint8_t gstage[QUANT_THREADS / 64][32 * D * 2];   // G rows of a block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = lane >> 1, hf = lane & 1;
  const int c0 = blockIdx.x * TOKEN_BLOCK;
  const int H = p.H, T = p.T;
  constexpr int LOG2D = D == 64 ? 6 : 7;

  for_blocks_in_chunk(p.cu, p.ndocs, T, c0, [&](int bs, int be, int ds, int doc) {
    const int tok = bs + row;
    const bool valid = tok < be;
    const int blk = (bs - ds) / TOKEN_BLOCK;
    const int de = p.cu[doc + 1];
    const int nblk_doc = (de - ds + TOKEN_BLOCK - 1) / TOKEN_BLOCK;
    const int nvis = p.causal_dq_scale ? blk + 1 : nblk_doc;
    for (int h = wave; h < H; h += QUANT_THREADS / 64) {
      const size_t off = ((size_t)tok * H + h) * D + hf * (D / 2);
      float x[D / 2];
      load_half_row<D>(dout + off, valid, x);
      const float lane_amax = half_row_amax<D>(x);
      const int e = roundup_exp(p.exact ? fmaxf(lane_amax, __shfl_xor(lane_amax, 1, 64)) : wave_max(lane_amax));
      // largest K and V block exponents over the visible key blocks (of the
      // key/value head this query head reads)
      const size_t hkT = (size_t)(h / (H / p.Hk)) * T;
      int emax_kv = -254;
      if (p.exact) {
        // per token: the largest K and V exponents over positions j <= tok of the
        // document -- earlier blocks through their last token's in-block prefix
        // maximum, this block through the prefix at tok itself
        int ek = -127, ev = -127;
        for (int J = lane; J < blk; J += 64) {
          const size_t t1 = hkT + ds + J * TOKEN_BLOCK + TOKEN_BLOCK - 1;
          ek = max(ek, (int)k_ref_exp[t1] - E8M0_BIAS);
          ev = max(ev, (int)v_ref_exp[t1] - E8M0_BIAS);
        }
        ek = wave_max_i(ek);
        ev = wave_max_i(ev);
        const size_t tt = hkT + min(tok, be - 1);
        emax_kv = max(ek, (int)k_ref_exp[tt] - E8M0_BIAS) + max(ev, (int)v_ref_exp[tt] - E8M0_BIAS);
      } else {
        int ek = -127, ev = -127;
        for (int J = lane; J < nvis; J += 64) {
          const size_t t0 = hkT + ds + J * TOKEN_BLOCK;
          ek = max(ek, (int)k_exp[t0] - E8M0_BIAS);
          ev = max(ev, (int)v_exp[t0] - E8M0_BIAS);
        }
        emax_kv = wave_max_i(ek) + wave_max_i(ev);
      }
      if (!p.deterministic) {
        // zero the block's rows of the fp16 dQ accumulator (unused in
        // deterministic mode): whole rows per store instruction, 16 lanes
        // per 2d-byte row (d = 128), so every instruction writes full lines
        constexpr int CPR = D / 8, RPI = 64 / CPR;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int r = RPI * i + lane / CPR;
          if (bs + r < be) st16(dq_acc + ((size_t)(bs + r) * H + h) * D + 8 * (lane % CPR), v4i{0, 0, 0, 0});
        }
      }
      // every row of the block has its integer row maximum where the
      // backward may take the fast probability form (p_scaled); one bit,
      // bit 24 of each row's qexps word
      const int mrow = valid ? row_max[(size_t)h * T + tok] : 0;
      const int pfast = __all(mrow >= P_M_LO && mrow <= P_M_HI) ? 1 << 24 : 0;
      if (valid) {
        // codes, dequantized values, D and G
        float oo[D / 2];
        load_half_row<D>(o + off, true, oo);
        float dsum = 0.f;
        const float l = row_sum[(size_t)h * T + tok];
        const float ginv = __builtin_amdgcn_ldexpf(1.0f / l, P_EXP);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          v4i w;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int b = 16 * c + 4 * j;
            w[j] = cvt_fp8x4(__builtin_amdgcn_ldexpf(x[b], -e), __builtin_amdgcn_ldexpf(x[b + 1], -e),
                             __builtin_amdgcn_ldexpf(x[b + 2], -e), __builtin_amdgcn_ldexpf(x[b + 3], -e));
#pragma unroll
            for (int t = 0; t < 4; ++t) x[b + t] = __builtin_amdgcn_ldexpf(fp8_value(w[j], t), e);
          }
          st16(cstage[wave] + row * D + 16 * code_slot<D>(row, hf, c), w);   // rows leave below
        }
#pragma unroll
        for (int i = 0; i < D / 2; ++i) dsum = __builtin_fmaf(x[i], oo[i], dsum);
        dsum += __shfl_xor(dsum, 1, 64);
        // G half-row into the wave's LDS tile (16-byte chunks swizzled so the
        // writes and the row reads below are free of bank conflicts)
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          v4i w;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int b = 8 * c + 2 * j;
            uint32_t lo = f32_to_bf16_bits(x[b] * ginv), hi = f32_to_bf16_bits(x[b + 1] * ginv);
            w[j] = (int)(lo | (hi << 16));
          }
          st16(gstage[wave] + row * (2 * D) + 16 * g_slot<D>(row, hf, c), w);
        }
        if (hf == 0) {
          const size_t mi = (size_t)h * T + tok;
          do_exp[mi] = (uint8_t)(e + E8M0_BIAS);
          delta[mi] = -dsum;           // the backward adds -D
          il8[mi] = ginv;
          kofs[mi] = 8 - mrow;           // -P_EXP - m~: P 2^8 = 2^(S' + kofs)
          qexps[mi] = (int)q_exp[mi] | ((e + E8M0_BIAS) << 8) | ((int)v_ref_exp[hkT + tok] << 16) | pfast;
          // |dQ partial sum| <= 2.2 d 448^3 2^(e_dO + e_V + e_K) < 2^(27.6 + log2 d + ...);
          // the prescale keeps it below 2^15 in fp16
          dq_sigma[mi] = e + emax_kv + LOG2D + 13;
        }
      }
      // dO~ code rows and G rows to memory: whole rows per store instruction
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      {
        constexpr int HC = D / 32, CPR = 2 * HC, RPI = 64 / CPR;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int r = RPI * i + lane / CPR, lc = lane % CPR;
          if (bs + r < be)
            st16(do_codes + ((size_t)(bs + r) * H + h) * D + 16 * lc,
                 ld16(cstage[wave] + r * D + 16 * code_slot<D>(r, lc / HC, lc % HC)));
        }
      }
      {
        constexpr int CPR = D / 8, HC = CPR / 2, RPI = 64 / CPR;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int r = RPI * i + lane / CPR, lc = lane % CPR;
          if (bs + r < be)
            st16(g + ((size_t)(bs + r) * H + h) * D + 8 * lc,
                 ld16(gstage[wave] + r * (2 * D) + 16 * g_slot<D>(r, lc / HC, lc % HC)));
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  });
}

hipError_t launch_quant_qkv(const Problem& p, const void* q, const void* k, const void* v,
                            uint8_t* q_codes, uint8_t* k_codes, uint8_t* v_codes, uint8_t* v_key_codes,
                            uint8_t* q_exp, uint8_t* k_exp, uint8_t* v_exp, uint8_t* v_key_exp,
                            uint8_t* v_ref_exp, uint8_t* k_ref_exp, const Fp4Operands& f4, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  dim3 grid((p.T + TOKEN_BLOCK - 1) / TOKEN_BLOCK, 3);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(QUANT_THREADS), 0, stream, p, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, q_codes, k_codes, v_codes, v_key_codes,
                       q_exp, k_exp, v_exp, v_key_exp, v_ref_exp, k_ref_exp, f4);
  };
  if (p.D == 64) args(quant_qkv_kernel<64>); else args(quant_qkv_kernel<128>);
  return hipGetLastError();
}

hipError_t launch_amax_qk(const Problem& p, const void* q, const void* k, float* qk_scale, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  dim3 grid((p.T + TOKEN_BLOCK - 1) / TOKEN_BLOCK, 2);
  if (p.D == 64)
    hipLaunchKernelGGL(amax_qk_kernel<64>, grid, dim3(QUANT_THREADS), 0, stream, p, (const uint16_t*)q,
                       (const uint16_t*)k, qk_scale);
  else
    hipLaunchKernelGGL(amax_qk_kernel<128>, grid, dim3(QUANT_THREADS), 0, stream, p, (const uint16_t*)q,
                       (const uint16_t*)k, qk_scale);
  return hipGetLastError();
}

hipError_t launch_quant_do(const Problem& p, const void* dout, const void* o, const int* row_max,
                           const float* row_sum, const uint8_t* q_exp, const uint8_t* k_exp,
                           const uint8_t* v_exp, const uint8_t* v_ref_exp, const uint8_t* k_ref_exp,
                           uint8_t* do_codes,
                           uint8_t* do_exp, int* kofs, float* delta,
                           float* il8, int* qexps, void* g, int* dq_sigma, void* dq_acc, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  dim3 grid((p.T + TOKEN_BLOCK - 1) / TOKEN_BLOCK);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(QUANT_THREADS), 0, stream, p, (const uint16_t*)dout,
                       (const uint16_t*)o, row_max, row_sum, q_exp, k_exp, v_exp, v_ref_exp, k_ref_exp, do_codes,
                       do_exp, kofs, delta, il8, qexps, (uint16_t*)g, dq_sigma, (uint16_t*)dq_acc);
  };
  if (p.D == 64) args(quant_do_kernel<64>); else args(quant_do_kernel<128>);
  return hipGetLastError();
}

}  // namespace flamia
