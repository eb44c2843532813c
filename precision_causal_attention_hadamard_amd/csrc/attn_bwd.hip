// Backward kernel of the causal block-scaled MXFP8 attention call.
//
// One workgroup (4 waves) per work item (document, 128-key tile, head), items
// longest first.  Wave w owns the 32 keys of document-local block 4u + w and
// keeps their K~, V~ (block and per-key codes) in registers as the B
// operands of S = Q~ K~^T and dP = dO~ V~^T, and accumulates dK and dV for
// them.  The kernel walks the 64-query tiles from the diagonal to the end of
// the document ([Summary, §3.3 Forward-Backward Numerical Consistency];
// [Reading, 4.3]; [Reading, 4.4] third bullet).
//
// Staging.  Query tiles (Q~ and dO~ codes, G = dO~ 2^-8 / l in bf16, and five
// per-row planes: integer row maximum, 2^-8 / l, D, the dQ prescale exponent,
// the Q / dO / fold-reference exponent bytes) go global -> LDS directly, with
// no register staging, into two named buffers; the loop is unrolled by two so
// each step reads one buffer while the next tile streams into the other.
// Tiles are unpadded and XOR-swizzled per 16-byte chunk.  The fp16 dQ partial
// of a step is added to memory at the start of the next step, so the one
// full wait per step (at its end) finds both the atomics and the next tile's
// loads long finished.
//
// Per query tile:
//   * S is recomputed from the same Q~/K~ codes with the same 32x32x64
//     scaled FP8 products as the forward (the forward computes S^T with the
//     operands swapped, which yields the same bits), then the same
//     P 2^8 = exp2(fract S') 2^(floor S' + 8 - m~) with the stored integer
//     row maximum, the same causal mask, the same diagonal decision (query
//     and key in one document-local 32-token block) and the same per-key
//     fold, so the probability codes are the forward's;
//   * dV += P^_eff^T G on bf16 matrix cores (P^ is exact in bf16; the
//     per-query 1/l cannot be a per-32-block operand scale);
//   * dP = dO~ V~^T on scaled FP8 matrix cores, with the V representation the
//     forward used for the pair (per-key codes on the diagonal block);
//   * dS = (P / l)(dP - D) in fp32; one round-up exponent per 32 x 32 block
//     of dS from the block max-abs (a whole-wave reduction: one C tile is one
//     such block); dS^ in E4M3 ([Summary, §3.3] second bullet);
//   * dK += dS^^T Q~ (scaled FP8; dS^ straight from the accumulator layout,
//     Q~ d-major through the 8-bit LDS transpose read of the same payload);
//   * dS^ goes to LDS key-major; each wave then forms dQ^T for one slice of d
//     over all 128 keys (scaled FP8, dS^ read back transposed), multiplies by
//     2^-sigma (the data-dependent power-of-two prescale of the fp16
//     accumulator, [Reading, 4.4] third bullet) and stages the fp16 tile in
//     LDS; the next step adds it with row-contiguous packed fp16 atomics.
// Blocks strictly below the diagonal and inside the document take a path
// with no mask and no fold.
// Item end: dK (times the softmax scale) goes to an fp32 staging buffer (the
// finaliser rotates it back when the Hadamard option is on); dV to bf16.
#include <type_traits>

#include "flamia_device.hpp"
#include "flamia_internal.hpp"

namespace flamia {

constexpr int BWD_THREADS = 256;
constexpr int NPLANES = 5;          // per-row planes staged with each query tile

struct BwdArgs {
  Problem p;
  const int* counts;
  const int2* items;
  const uint8_t *q_codes, *k_codes, *v_codes, *v_key_codes;
  const uint8_t *k_exp, *v_exp, *v_key_exp;
  const int* row_max;     // [H, T] integer row maxima of the forward
  const float* il8;       // [H, T] 2^-8 / l
  const float* delta;     // [H, T] D
  const int* dq_sigma;    // [H, T] dQ prescale exponent
  const int* qexps;       // [H, T] q_exp | do_exp << 8 | v_ref_exp << 16 (biased bytes)
  const uint8_t* do_codes;
  const uint16_t* g;
  uint16_t* dq_acc;
  float* dk_f32;
  uint16_t* dv;
  const uint16_t *q_x, *k_x;   // mixed path: NVFP4 Q and K expanded to bf16
  const float* qk_scale;       // mixed path: [2], [3] tensor scales
};

// PATH 0: MXFP8 scores.  PATH 1 (mixed): the recomputed scores come from the
// NVFP4 Q and K (expanded exactly to bf16) on bf16 matrix cores with the same
// operand split and order as the forward, then scaled by t_Q t_K; dK and dQ
// still use the E4M3 token-block Q~ and K~.
template <int D, int PATH>
__global__ void __launch_bounds__(BWD_THREADS) attn_bwd_kernel(BwdArgs a) {
  constexpr int DSK = BWD_BQ + 16;           // key-major dS^ row stride (bytes)
  constexpr int NS = D / 64;
  constexpr int ND = D / 32;
  constexpr int CT = BWD_BQ * D;             // bytes of a query code tile
  constexpr int WT = BWD_BQ * 2 * D;         // bytes of a query bf16 tile
  constexpr int RT = NPLANES * BWD_BQ * 4;   // bytes of the per-row planes
  constexpr int DQS = D + 4;                 // fp16 dQ staging row stride (elements): 8 bytes of
                                             // padding put the 32 rows of one store on distinct banks
  constexpr int KQ = BWD_BK * D > BWD_BQ * DQS * 2 ? BWD_BK * D : BWD_BQ * DQS * 2;

  // K~ tile at item start, then the fp16 dQ partial of the current step
  __shared__ __attribute__((aligned(1024))) uint8_t sKQ[KQ];
  __shared__ __attribute__((aligned(1024))) uint8_t sQ0[CT];
  __shared__ __attribute__((aligned(1024))) uint8_t sQ1[CT];
  __shared__ __attribute__((aligned(1024))) uint8_t sO0[CT];
  __shared__ __attribute__((aligned(1024))) uint8_t sO1[CT];
  __shared__ __attribute__((aligned(1024))) uint8_t sG0[WT];
  __shared__ __attribute__((aligned(1024))) uint8_t sG1[WT];
  __shared__ __attribute__((aligned(1024))) uint8_t sX0[PATH ? WT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sX1[PATH ? WT : 16];
  __shared__ __attribute__((aligned(256))) uint8_t sR0[RT];
  __shared__ __attribute__((aligned(256))) uint8_t sR1[RT];
  __shared__ __attribute__((aligned(16))) uint8_t sdSK[BWD_BK * DSK];
  __shared__ int sEds[2][4];
  __shared__ int sKeB[4];

  const Problem& p = a.p;
  const int H = p.H, T = p.T;
  const int tile_idx = blockIdx.x / H, head = blockIdx.x % H;
  if (tile_idx >= a.counts[1]) return;
  const int2 it = a.items[tile_idx];
  const int doc = it.x, u = it.y;
  const int s_d = p.cu[doc];
  const int L = p.cu[doc + 1] - s_d;
  const int k0 = u * BWD_BK;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int colg = 16 * ((lane >> 4) & 1);      // first column of this lane's 16-lane group
  const int j = k0 + 32 * wave + n;             // this lane's key (document-local)
  const bool kv = j < L;
  const bool wave_active = k0 + 32 * wave < L;
  const int KB = 4 * u + wave;
  const size_t rs = (size_t)H * D;
  const size_t hT = (size_t)head * T + s_d;
  const size_t doc0 = (size_t)s_d * rs + (size_t)head * D;   // row 0 of this doc/head
  const uint32_t rs32 = (uint32_t)rs;
  const float c = p.c_log2;
  // per-document bases (uniform); per-lane offsets fit 32 bits (checked on the host)
  const uint8_t* q_doc = a.q_codes + doc0;
  const uint8_t* do_doc = a.do_codes + doc0;
  const uint8_t* k_doc = a.k_codes + doc0;
  const uint8_t* g_doc = reinterpret_cast<const uint8_t*>(a.g + doc0);
  const uint8_t* x_doc = PATH ? reinterpret_cast<const uint8_t*>(a.q_x + doc0) : nullptr;
  uint8_t* dq_doc = reinterpret_cast<uint8_t*>(a.dq_acc + doc0);

  // ---- staging of 64-row tiles: rows row0 + r, clamped to the document's last row
  auto dma_codes = [&](uint8_t* tile, const uint8_t* src, int row0, int nrows) {
    const int ninst = nrows * D / 1024;
    for (int i = wave; i < ninst; i += 4) {
      const int o = i * 1024 + 16 * lane;
      const int r = o / D, slot = (o % D) >> 4;
      const uint32_t gr = (uint32_t)min(row0 + r, L - 1);
      dma16(src + (gr * rs32 + 16u * (uint32_t)(slot ^ code_key<D>(r))), tile + i * 1024);
    }
  };
  auto dma_wide = [&](uint8_t* tile, const uint8_t* src, int row0, bool xq) {
    constexpr int NI = WT / 1024;
#pragma unroll
    for (int i = wave; i < NI; i += 4) {
      const int o = i * 1024 + 16 * lane;
      const int r = o / (2 * D), slot = (o % (2 * D)) >> 4;
      const uint32_t gr = (uint32_t)min(row0 + r, L - 1);
      const int key = xq ? xq_key<D>(r) : wide_key<D>(r);
      dma16(src + (2u * gr * rs32 + 16u * (uint32_t)(slot ^ key)), tile + i * 1024);
    }
  };
  auto dma_planes = [&](uint8_t* tile, int row0) {
    const size_t mi = hT + min(row0 + lane, L - 1);
    for (int pl = wave; pl < NPLANES; pl += 4) {
      const void* src = pl == 0 ? (const void*)(a.row_max + mi)
                      : pl == 1 ? (const void*)(a.il8 + mi)
                      : pl == 2 ? (const void*)(a.delta + mi)
                      : pl == 3 ? (const void*)(a.dq_sigma + mi) : (const void*)(a.qexps + mi);
      dma4(src, tile + pl * BWD_BQ * 4);
    }
  };
  auto issue_tile = [&](auto Bc, int qt) {
    constexpr int B = decltype(Bc)::value;
    const int q0 = qt * BWD_BQ;
    dma_codes(B ? sQ1 : sQ0, q_doc, q0, BWD_BQ);
    dma_codes(B ? sO1 : sO0, do_doc, q0, BWD_BQ);
    dma_wide(B ? sG1 : sG0, g_doc, q0, false);
    if constexpr (PATH == 1) dma_wide(B ? sX1 : sX0, x_doc, q0, true);
    dma_planes(B ? sR1 : sR0, q0);
  };

  // ---- per item: the key tile (for K~^T of dQ) and the first query tile
  const int qt_first = k0 / BWD_BQ;
  const int qt_end = (L + BWD_BQ - 1) / BWD_BQ;
  dma_codes(sKQ, k_doc, k0, BWD_BK);
  issue_tile(std::integral_constant<int, 0>{}, qt_first);
  if (tid < 4) sKeB[tid] = k0 + 32 * tid < L ? (int)a.k_exp[hT + k0 + 32 * tid] : E8M0_BIAS;

  // ---- per wave: K~ (or the mixed path's bf16 K), V~ (block and per-key) as
  // B operands (lane = key)
  v8i kreg[PATH ? 1 : NS], vreg[NS], vkreg[NS];
  v8bf kb16[PATH ? D / 16 : 1];
  int ke = E8M0_BIAS, ve = E8M0_BIAS, vke = E8M0_BIAS;
  float tqk = 1.f;
  if constexpr (PATH == 1) tqk = a.qk_scale[2] * a.qk_scale[3];
  {
    const size_t ro = doc0 + (size_t)min(j, L - 1) * rs;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (PATH == 0)
        kreg[s] = cat8(ld16(a.k_codes + ro + 64 * s + 16 * hh), ld16(a.k_codes + ro + 64 * s + 32 + 16 * hh));
      vreg[s] = cat8(ld16(a.v_codes + ro + 64 * s + 16 * hh), ld16(a.v_codes + ro + 64 * s + 32 + 16 * hh));
      vkreg[s] = cat8(ld16(a.v_key_codes + ro + 64 * s + 16 * hh), ld16(a.v_key_codes + ro + 64 * s + 32 + 16 * hh));
    }
    if constexpr (PATH == 1) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) kb16[s] = __builtin_bit_cast(v8bf, ld16(a.k_x + ro + 16 * s + 8 * hh));
    }
    const size_t mi = hT + min(j, L - 1);
    ke = a.k_exp[mi];
    ve = a.v_exp[mi];
    vke = a.v_key_exp[mi];
    if (!kv) {    // keys past the document: zero operands
#pragma unroll
      for (int s = 0; s < NS; ++s) vreg[s] = vkreg[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (PATH == 0) {
#pragma unroll
        for (int s = 0; s < NS; ++s) kreg[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      } else {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) kb16[s] = __builtin_bit_cast(v8bf, v4i{0, 0, 0, 0});
      }
    }
  }
  const int e_key = vke - E8M0_BIAS;
  full_barrier();

  // K~^T slice for dQ^T: wave -> d-slice ds; lane (d row, half hh), K = keys
  const int ds = wave % ND;
  v8i ktreg[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    ktreg[ks] = cat8(tr_code16<D>(sKQ, 64 * ks, 32 * ds + colg, lane),
                     tr_code16<D>(sKQ, 64 * ks + 32, 32 * ds + colg, lane));

  v16f dk[ND], dv[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) { dk[db] = v16f{}; dv[db] = v16f{}; }

  // fp16 dQ partial of query tile qtp (staged in sKQ) -> memory-side atomics,
  // one wave instruction per row pair run
  auto flush_dq = [&](int qtp) {
    constexpr int PAIRS = D / 2;
    const int q0p = qtp * BWD_BQ;
    const int nqp = min(BWD_BQ, L - q0p);
    const uint16_t* sdQ = reinterpret_cast<const uint16_t*>(sKQ);
    for (int idx = tid; idx < BWD_BQ * PAIRS; idx += BWD_THREADS) {
      const int row = idx / PAIRS, pr = idx % PAIRS;
      if (row < nqp) {
        const v2h hv = *reinterpret_cast<const v2h*>(sdQ + row * DQS + 2 * pr);
        __builtin_amdgcn_global_atomic_fadd_v2f16(
            reinterpret_cast<v2h*>(dq_doc + (2u * ((uint32_t)(q0p + row) * rs32) + 4u * (uint32_t)pr)), hv);
      }
    }
  };

  auto step = [&](auto Bc, int qt) {
    constexpr int B = decltype(Bc)::value;
    const uint8_t* tQ = B ? sQ1 : sQ0;
    const uint8_t* tdO = B ? sO1 : sO0;
    const uint8_t* tG = B ? sG1 : sG0;
    const uint8_t* tX = B ? sX1 : sX0;
    const uint8_t* tR = B ? sR1 : sR0;
    const int* pm = reinterpret_cast<const int*>(tR);
    const float* pil = reinterpret_cast<const float*>(tR + BWD_BQ * 4);
    const float* pdl = reinterpret_cast<const float*>(tR + 2 * BWD_BQ * 4);
    const int* psig = reinterpret_cast<const int*>(tR + 3 * BWD_BQ * 4);
    const int* pqx = reinterpret_cast<const int*>(tR + 4 * BWD_BQ * 4);
    const int q0 = qt * BWD_BQ;
    const int nq = min(BWD_BQ, L - q0);

    // the next tile streams in while this one is computed; last step's dQ goes out
    if (qt + 1 < qt_end) issue_tile(std::integral_constant<int, 1 - B>{}, qt + 1);
    if (qt > qt_first) flush_dq(qt - 1);

    int dsc[2][4];
    int eds[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int QB = 2 * qt + qb;
      const bool act = wave_active && QB >= KB && 32 * qb < nq;
      eds[qb] = -127;
#pragma unroll
      for (int g = 0; g < 4; ++g) dsc[qb][g] = 0;
      if (act) {
        const bool dia = QB == KB;
        const bool fast = !dia && 32 * qb + 32 <= nq;   // no mask, no fold
        const int qx = pqx[32 * qb];
        const int sqe = qx & 255, sdoe = (qx >> 8) & 255;
        v16f sacc = v16f{}, pacc = v16f{};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int row = 32 * qb + n;
          if constexpr (PATH == 0)
            sacc = mfma_f8(cat8(ld16(tQ + code_off<D>(row, 64 * s + 16 * hh)),
                                ld16(tQ + code_off<D>(row, 64 * s + 32 + 16 * hh))),
                           kreg[s], sacc, sqe, ke);
          pacc = mfma_f8(cat8(ld16(tdO + code_off<D>(row, 64 * s + 16 * hh)),
                              ld16(tdO + code_off<D>(row, 64 * s + 32 + 16 * hh))),
                         dia ? vkreg[s] : vreg[s], pacc, sdoe, dia ? vke : ve);
        }
        if constexpr (PATH == 1) {
          const int row = 32 * qb + n;
#pragma unroll
          for (int s = 0; s < D / 16; ++s)
            sacc = mfma_bf16(__builtin_bit_cast(v8bf, ld16(tX + xq_off<D>(row, 32 * s + 16 * hh))), kb16[s], sacc);
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) sacc[rr] = sacc[rr] * tqk;
        }
        float dsv[16];
        uint32_t pe[8];    // bf16 pairs of P^_eff * 2^8, accumulator register order
        float amax = 0.f;
        if (fast) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int r0 = 32 * qb + 8 * g + 4 * hh;      // first of 4 consecutive query rows
            const v4i mv = *reinterpret_cast<const v4i*>(pm + r0);
            const v4f ilv = *reinterpret_cast<const v4f*>(pil + r0);
            const v4f dlv = *reinterpret_cast<const v4f*>(pdl + r0);
            float pf[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int rr = 4 * g + r;
              const float x = sacc[rr] * c;
              const float e2 = __builtin_amdgcn_exp2f(__builtin_amdgcn_fractf(x));
              pf[r] = __builtin_amdgcn_ldexpf(e2, cvt_floor_i32(x) + (8 - mv[r]));   // P 2^8
              dsv[rr] = (pf[r] * ilv[r]) * (pacc[rr] - dlv[r]);
              amax = fmaxf(amax, fabsf(dsv[rr]));
            }
            const int code = cvt_fp8x4(pf[0], pf[1], pf[2], pf[3]);
            pe[2 * g] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, false));
            pe[2 * g + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, true));
          }
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int r0 = 32 * qb + 8 * g + 4 * hh;
            const v4i mv = *reinterpret_cast<const v4i*>(pm + r0);
            const v4f ilv = *reinterpret_cast<const v4f*>(pil + r0);
            const v4f dlv = *reinterpret_cast<const v4f*>(pdl + r0);
            float pf[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int rr = 4 * g + r;
              const int i = q0 + r0 + r;
              float dsr = 0.f, pev = 0.f;
              if (kv && j <= i && i < L) {
                const float x = sacc[rr] * c;
                const float e2 = __builtin_amdgcn_exp2f(__builtin_amdgcn_fractf(x));
                const float p8 = __builtin_amdgcn_ldexpf(e2, cvt_floor_i32(x) + (8 - mv[r]));
                dsr = (p8 * ilv[r]) * (pacc[rr] - dlv[r]);
                if (dia) {
                  const int vref = ((pqx[r0 + r] >> 16) & 255) - E8M0_BIAS;
                  const int code = cvt_fp8x2(__builtin_amdgcn_ldexpf(p8, e_key - vref), 0.f);
                  pev = __builtin_amdgcn_ldexpf(fp8_value(code, 0), vref - e_key);
                } else {
                  pev = fp8_value(cvt_fp8x2(p8, 0.f), 0);
                }
              }
              dsv[rr] = dsr;
              amax = fmaxf(amax, fabsf(dsr));
              pf[r] = pev;
            }
            pe[2 * g] = (uint32_t)f32_to_bf16_bits(pf[0]) | ((uint32_t)f32_to_bf16_bits(pf[1]) << 16);
            pe[2 * g + 1] = (uint32_t)f32_to_bf16_bits(pf[2]) | ((uint32_t)f32_to_bf16_bits(pf[3]) << 16);
          }
        }
        const int e = roundup_exp(wave_max(amax));
        eds[qb] = e;
        if (e >= -126) {
          const float sc2 = __builtin_amdgcn_ldexpf(1.0f, e);    // the convert divides by it
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, dsv[4 * g], dsv[4 * g + 1], sc2, false);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, dsv[4 * g + 2], dsv[4 * g + 3], sc2, true);
            dsc[qb][g] = __builtin_bit_cast(int, w);
          }
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            dsc[qb][g] = cvt_fp8x4(__builtin_amdgcn_ldexpf(dsv[4 * g], -e), __builtin_amdgcn_ldexpf(dsv[4 * g + 1], -e),
                                   __builtin_amdgcn_ldexpf(dsv[4 * g + 2], -e), __builtin_amdgcn_ldexpf(dsv[4 * g + 3], -e));
        }
        // dV += P^_eff^T G  (two K-steps of 16 queries)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const v8bf av = __builtin_bit_cast(
              v8bf, v4i{(int)pe[4 * ks], (int)pe[4 * ks + 1], (int)pe[4 * ks + 2], (int)pe[4 * ks + 3]});
#pragma unroll
          for (int db = 0; db < ND; ++db)
            dv[db] = mfma_bf16(av, tr_wide_bf16x8<D>(tG, 32 * qb, ks, 32 * db + colg, lane), dv[db]);
        }
      }
    }
    // dK += dS^^T Q~ : K = the 64 queries; lane half hh carries query block hh
    if (wave_active) {
      const v8i adk = v8i{dsc[0][0], dsc[0][1], dsc[0][2], dsc[0][3], dsc[1][0], dsc[1][1], dsc[1][2], dsc[1][3]};
      const int sa = (hh == 0 ? eds[0] : eds[1]) + E8M0_BIAS;
      const int sb = pqx[32 * hh] & 255;
#pragma unroll
      for (int db = 0; db < ND; ++db)
        dk[db] = mfma_f8(adk, cat8(tr_code16<D>(tQ, 0, 32 * db + colg, lane), tr_code16<D>(tQ, 32, 32 * db + colg, lane)),
                         dk[db], sa, sb);
    }
    // dS^ to LDS key-major: row = key of the tile, 4 consecutive queries per dword
    {
      uint8_t* row = sdSK + (32 * wave + n) * DSK + 4 * hh;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) *reinterpret_cast<int*>(row + 32 * qb + 8 * g) = dsc[qb][g];
      if (lane == 0) { sEds[0][wave] = eds[0]; sEds[1][wave] = eds[1]; }
    }
    lds_barrier();
    // dQ^T slice: rows d in [32 ds, 32 ds + 32), columns = queries, K = 128 keys
    uint16_t* sdQ = reinterpret_cast<uint16_t*>(sKQ);
    for (int qb = (ND == 4 ? 0 : wave / ND); qb < 2; qb += (ND == 4 ? 1 : 2)) {
      if (32 * qb >= nq) continue;
      v16f acc = v16f{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const v8i bq = cat8(tr_block16(sdSK, DSK, 64 * ks, 32 * qb + colg, lane),
                            tr_block16(sdSK, DSK, 64 * ks + 32, 32 * qb + colg, lane));
        acc = mfma_f8(ktreg[ks], bq, acc, sKeB[2 * ks + hh], sEds[qb][2 * ks + hh] + E8M0_BIAS);
      }
      // prescaled fp16 partial of this query row into LDS (4 consecutive d per store)
      const int iq = 32 * qb + n;
      const int sig = psig[iq];
      uint16_t* dst = sdQ + iq * DQS + 32 * ds + 4 * hh;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v2h h0, h1;
        h0[0] = (_Float16)__builtin_amdgcn_ldexpf(acc[4 * g], -sig);
        h0[1] = (_Float16)__builtin_amdgcn_ldexpf(acc[4 * g + 1], -sig);
        h1[0] = (_Float16)__builtin_amdgcn_ldexpf(acc[4 * g + 2], -sig);
        h1[1] = (_Float16)__builtin_amdgcn_ldexpf(acc[4 * g + 3], -sig);
        *reinterpret_cast<v2i*>(dst + 8 * g) = v2i{__builtin_bit_cast(int, h0), __builtin_bit_cast(int, h1)};
      }
    }
    // the next tile has landed, this step's dQ partial is staged, the
    // previous step's atomics are done
    full_barrier();
  };

  for (int qt = qt_first;;) {
    step(std::integral_constant<int, 0>{}, qt);
    if (++qt >= qt_end) break;
    step(std::integral_constant<int, 1>{}, qt);
    if (++qt >= qt_end) break;
  }
  flush_dq(qt_end - 1);

  // ---- item end: dK (scaled, fp32 staging) and dV (bf16)
  if (wave_active) {
    const float sc = p.softmax_scale;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int jk = k0 + 32 * wave + 8 * (rr >> 2) + 4 * hh + (rr & 3);
        if (jk < L) {
          const size_t o = doc0 + (size_t)jk * rs + 32 * db + n;
          a.dk_f32[o] = dk[db][rr] * sc;
          a.dv[o] = f32_to_bf16_bits(dv[db][rr]);
        }
      }
  }
}

hipError_t launch_attn_bwd(const Problem& p, const void* plan, const PlanLayout& pl, const BwdInputs& in,
                           hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const char* base = static_cast<const char*>(plan);
  BwdArgs a{p, reinterpret_cast<const int*>(base), reinterpret_cast<const int2*>(base + pl.bwd_offset),
            in.q_codes, in.k_codes, in.v_codes, in.v_key_codes, in.k_exp, in.v_exp, in.v_key_exp,
            in.row_max, in.il8, in.delta, in.dq_sigma, in.qexps, in.do_codes,
            static_cast<const uint16_t*>(in.g), static_cast<uint16_t*>(in.dq_acc), in.dk_f32,
            static_cast<uint16_t*>(in.dv), static_cast<const uint16_t*>(in.q_x),
            static_cast<const uint16_t*>(in.k_x), in.qk_scale};
  dim3 grid((unsigned)pl.cap_bwd * (unsigned)p.H);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(BWD_THREADS), 0, stream, a); };
  if (p.path == 1) {
    if (p.D == 64) go(attn_bwd_kernel<64, 1>); else go(attn_bwd_kernel<128, 1>);
  } else {
    if (p.D == 64) go(attn_bwd_kernel<64, 0>); else go(attn_bwd_kernel<128, 0>);
  }
  return hipGetLastError();
}

}  // namespace flamia
