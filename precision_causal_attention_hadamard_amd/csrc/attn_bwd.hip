// Backward kernel of the causal block-scaled MXFP8 attention call.
//
// One workgroup (4 waves) per work item (document, 128-key tile, head), items
// longest first.  Wave w owns the 32 keys of document-local block 4u + w and
// keeps their K~, V~ (block and per-key codes) in registers as the B
// operands of S = Q~ K~^T and dP = dO~ V~^T, and accumulates dK and dV for
// them.  The kernel walks the 64-query tiles from the diagonal to the end of
// the document ([Summary, §3.3 Forward-Backward Numerical Consistency];
// [Reading, 4.3]; [Reading, 4.4] third bullet).  Query tiles (Q~ and dO~
// codes, G = dO~ 2^-8 / l in bf16, per-row statistics) are staged token-major
// and double-buffered; the next tile's global loads are in flight while the
// current one is computed.  Per query tile:
//   * S is recomputed from the same Q~/K~ codes with the same 32x32x64
//     scaled FP8 products as the forward (the forward computes S^T with the
//     operands swapped, which yields the same bits), then the same
//     P = 2^(n - m~) exp2(r) with the stored integer row maximum, the same
//     causal mask, the same diagonal decision (query and key in one
//     document-local 32-token block) and the same per-key fold, so the
//     probability codes are the forward's;
//   * dV += P^_eff^T G on bf16 matrix cores (P^ is exact in bf16; the
//     per-query 1/l cannot be a per-32-block operand scale); G is read
//     d-major from its token-major tile with the 16-bit LDS transpose read;
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
//     accumulator, [Reading, 4.4] third bullet), stages the fp16 tile in LDS
//     and adds it with row-contiguous packed fp16 atomics.
// Item end: dK (times the softmax scale) goes to an fp32 staging buffer (the
// finaliser rotates it back when the Hadamard option is on); dV to bf16.
#include "flamia_device.hpp"
#include "flamia_internal.hpp"

namespace flamia {

constexpr int BWD_THREADS = 256;

struct BwdArgs {
  Problem p;
  const int* counts;
  const int2* items;
  const uint8_t *q_codes, *k_codes, *v_codes, *v_key_codes;
  const uint8_t *q_exp, *k_exp, *v_exp, *v_key_exp, *v_ref_exp;
  const int* row_max;
  const float* row_sum;
  const uint8_t* do_codes;
  const uint8_t* do_exp;
  const float* delta;
  const uint16_t* g;
  const int* dq_sigma;
  uint16_t* dq_acc;
  float* dk_f32;
  uint16_t* dv;
  Fp4Operands f4;
};

// PATH 0: MXFP8 scores.  PATH 1 (mixed): the recomputed scores come from the
// NVFP4 Q and K, expanded exactly to bf16 and multiplied on bf16 matrix cores
// with the same operand split and order as the forward, then scaled by
// t_Q t_K; dK and dQ still use the E4M3 token-block Q~ and K~.
template <int D, int PATH>
__global__ void __launch_bounds__(BWD_THREADS) attn_bwd_kernel(BwdArgs a) {
  constexpr int KS = D + 16;                 // token-major code row stride (bytes)
  constexpr int QSB = 2 * D + 16;            // token-major bf16 row stride of the mixed-path Q tile
  constexpr int GS = 2 * D + 64;             // token-major bf16 row stride (bytes); = 64 mod 256 so the
                                             // four rows of a 16-bit transpose read hit distinct banks
  constexpr int DSK = BWD_BQ + 16;           // key-major dS^ row stride (bytes)
  constexpr int NS = D / 64;
  constexpr int ND = D / 32;
  constexpr int NCQ = BWD_BQ * D / 16 / BWD_THREADS;       // 16-byte code chunks per thread
  constexpr int NCG = BWD_BQ * 2 * D / 16 / BWD_THREADS;   // 16-byte G chunks per thread
  constexpr int NCK = BWD_BK * D / 16 / BWD_THREADS;       // K tile chunks per thread
  __shared__ __attribute__((aligned(16))) uint8_t sK[BWD_BK * KS];
  __shared__ __attribute__((aligned(16))) uint8_t sQ[2][BWD_BQ * KS];
  __shared__ __attribute__((aligned(16))) uint8_t sdO[2][BWD_BQ * KS];
  __shared__ __attribute__((aligned(16))) uint8_t sQb[2][PATH ? BWD_BQ * QSB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sG[2][BWD_BQ * GS];
  __shared__ __attribute__((aligned(16))) uint8_t sdSK[BWD_BK * DSK];
  __shared__ __attribute__((aligned(16))) uint16_t sdQ[BWD_BQ * D];
  __shared__ __attribute__((aligned(16))) int sM[2][BWD_BQ];
  __shared__ __attribute__((aligned(16))) float sIL[2][BWD_BQ];
  __shared__ __attribute__((aligned(16))) float sDl[2][BWD_BQ];
  __shared__ int sSig[2][BWD_BQ];
  __shared__ int sVref[2][BWD_BQ];
  __shared__ int sQeB[2][2], sDOeB[2][2], sKeB[4];
  __shared__ int sEds[2][4];

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
  const float c = p.c_log2;

  // ---- per item: the key tile, token-major, for K~^T of dQ
  {
    const int nk = L - k0;
#pragma unroll
    for (int c2 = 0; c2 < NCK; ++c2) {
      const int ch = tid + BWD_THREADS * c2;
      const int r = ch / (D / 16), c16 = ch % (D / 16);
      st16(sK + r * KS + 16 * c16, r < nk ? ld16(a.k_codes + doc0 + (size_t)(k0 + r) * rs + 16 * c16) : v4i{0, 0, 0, 0});
    }
    if (tid < 4) sKeB[tid] = k0 + 32 * tid < L ? (int)a.k_exp[hT + k0 + 32 * tid] : E8M0_BIAS;
  }

  // ---- per wave: K~ (or the mixed path's bf16 K), V~ (block and per-key) as
  // B operands (lane = key)
  v8i kreg[PATH ? 1 : NS], vreg[NS], vkreg[NS];
  v8bf kb16[PATH ? D / 16 : 1];
  int ke = E8M0_BIAS, ve = E8M0_BIAS, vke = E8M0_BIAS;
  float tqk = 1.f;
  if constexpr (PATH == 1) tqk = a.f4.qk_scale[2] * a.f4.qk_scale[3];
  if (kv) {
    const size_t ro = doc0 + (size_t)j * rs;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (PATH == 0)
        kreg[s] = cat8(ld16(a.k_codes + ro + 64 * s + 16 * hh), ld16(a.k_codes + ro + 64 * s + 32 + 16 * hh));
      vreg[s] = cat8(ld16(a.v_codes + ro + 64 * s + 16 * hh), ld16(a.v_codes + ro + 64 * s + 32 + 16 * hh));
      vkreg[s] = cat8(ld16(a.v_key_codes + ro + 64 * s + 16 * hh), ld16(a.v_key_codes + ro + 64 * s + 32 + 16 * hh));
    }
    if constexpr (PATH == 1) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const uint32_t codes = *reinterpret_cast<const uint32_t*>(a.f4.k_fp4 + ro / 2 + 8 * s + 4 * hh);
        kb16[s] = __builtin_bit_cast(v8bf, e2m1x8_times_bf16(codes, fp8_value(a.f4.k_sf[ro / 16 + s], 0)));
      }
    }
    ke = a.k_exp[hT + j];
    ve = a.v_exp[hT + j];
    vke = a.v_key_exp[hT + j];
  } else {
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
  const int e_key = vke - E8M0_BIAS;

  // ---- register prefetch of one query tile
  v4i pq[NCQ], pdo[NCQ], pg[NCG], pq4;
  uint32_t psf = 0;           // mixed path: NVFP4 Q chunk and its two group scales
  // per-row statistics for threads < BWD_BQ; threads BWD_BQ and BWD_BQ + 1
  // carry the two query blocks' Q and dO exponents in pm / psig
  int pm = 0, psig = 0, pvref = 0;
  float pil = 0.f, pdl = 0.f;
  auto prefetch = [&](int qt) {
    const int q0 = qt * BWD_BQ;
    const int nq = min(BWD_BQ, L - q0);
    const size_t to = doc0 + (size_t)q0 * rs;
#pragma unroll
    for (int c2 = 0; c2 < NCQ; ++c2) {
      const int ch = tid + BWD_THREADS * c2;
      const int r = ch / (D / 16), c16 = ch % (D / 16);
      const bool ok = r < nq;
      pq[c2] = ok ? ld16(a.q_codes + to + r * rs + 16 * c16) : v4i{0, 0, 0, 0};
      pdo[c2] = ok ? ld16(a.do_codes + to + r * rs + 16 * c16) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int c2 = 0; c2 < NCG; ++c2) {
      const int ch = tid + BWD_THREADS * c2;
      const int r = ch / (D / 8), c8 = ch % (D / 8);
      pg[c2] = r < nq ? ld16(a.g + to + r * rs + 8 * c8) : v4i{0, 0, 0, 0};
    }
    if constexpr (PATH == 1) {
      constexpr int CPR = D / 32;       // 16-byte NVFP4 chunks (32 codes) per query row
      if (tid < BWD_BQ * CPR) {
        const int r = tid / CPR, c4 = tid % CPR;
        const bool ok = r < nq;
        pq4 = ok ? ld16(a.f4.q_fp4 + (to + (size_t)r * rs) / 2 + 16 * c4) : v4i{0, 0, 0, 0};
        psf = ok ? *reinterpret_cast<const uint16_t*>(a.f4.q_sf + (to + (size_t)r * rs) / 16 + 2 * c4) : 0u;
      }
    }
    if (tid < BWD_BQ) {
      const bool ok = tid < nq;
      const size_t mi = hT + q0 + tid;
      pm = ok ? a.row_max[mi] : 0;
      pil = ok ? 1.0f / a.row_sum[mi] : 0.f;
      pdl = ok ? a.delta[mi] : 0.f;
      psig = ok ? a.dq_sigma[mi] : 0;
      pvref = ok ? (int)a.v_ref_exp[mi] - E8M0_BIAS : 0;
    } else if (tid < BWD_BQ + 2) {
      const int b = tid - BWD_BQ;
      const bool ok = 32 * b < nq;
      pm = ok ? (int)a.q_exp[hT + q0 + 32 * b] : E8M0_BIAS;
      psig = ok ? (int)a.do_exp[hT + q0 + 32 * b] : E8M0_BIAS;
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int c2 = 0; c2 < NCQ; ++c2) {
      const int ch = tid + BWD_THREADS * c2;
      const int r = ch / (D / 16), c16 = ch % (D / 16);
      st16(&sQ[buf][r * KS + 16 * c16], pq[c2]);
      st16(&sdO[buf][r * KS + 16 * c16], pdo[c2]);
    }
#pragma unroll
    for (int c2 = 0; c2 < NCG; ++c2) {
      const int ch = tid + BWD_THREADS * c2;
      const int r = ch / (D / 8), c8 = ch % (D / 8);
      st16(&sG[buf][r * GS + 16 * c8], pg[c2]);
    }
    if constexpr (PATH == 1) {
      constexpr int CPR = D / 32;
      if (tid < BWD_BQ * CPR) {
        const int r = tid / CPR, c4 = tid % CPR;
        uint8_t* dst = &sQb[buf][r * QSB + 64 * c4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
          st16(dst + 16 * w, e2m1x8_times_bf16((uint32_t)pq4[w], fp8_value((int)psf, w >> 1)));
      }
    }
    if (tid < BWD_BQ) {
      sM[buf][tid] = pm;
      sIL[buf][tid] = pil;
      sDl[buf][tid] = pdl;
      sSig[buf][tid] = psig;
      sVref[buf][tid] = pvref;
    } else if (tid < BWD_BQ + 2) {
      sQeB[buf][tid - BWD_BQ] = pm;
      sDOeB[buf][tid - BWD_BQ] = psig;
    }
  };

  const int qt_first = k0 / BWD_BQ;
  const int qt_end = (L + BWD_BQ - 1) / BWD_BQ;
  prefetch(qt_first);
  commit(0);
  __syncthreads();

  // K~^T slice for dQ^T: wave -> d-slice ds; lane (d row, half hh), K = keys
  const int ds = wave % ND;
  v8i ktreg[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    ktreg[ks] = cat8(tr_block16(sK, KS, 64 * ks, 32 * ds + colg, lane),
                     tr_block16(sK, KS, 64 * ks + 32, 32 * ds + colg, lane));

  v16f dk[ND], dv[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) { dk[db] = v16f{}; dv[db] = v16f{}; }

  for (int qt = qt_first; qt < qt_end; ++qt) {
    const int buf = (qt - qt_first) & 1;
    const int q0 = qt * BWD_BQ;
    const int nq = min(BWD_BQ, L - q0);
    const bool has_next = qt + 1 < qt_end;
    if (has_next) prefetch(qt + 1);
    const uint8_t* tQ = sQ[buf];
    const uint8_t* tdO = sdO[buf];
    const uint8_t* tG = sG[buf];

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
        v16f sacc = v16f{}, pacc = v16f{};
        const int sqe = sQeB[buf][qb], sdoe = sDOeB[buf][qb];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint8_t* dr = tdO + (32 * qb + n) * KS + 64 * s;
          if constexpr (PATH == 0) {
            const uint8_t* qr = tQ + (32 * qb + n) * KS + 64 * s;
            sacc = mfma_f8(cat8(ld16(qr + 16 * hh), ld16(qr + 32 + 16 * hh)), kreg[s], sacc, sqe, ke);
          }
          pacc = mfma_f8(cat8(ld16(dr + 16 * hh), ld16(dr + 32 + 16 * hh)), dia ? vkreg[s] : vreg[s], pacc,
                         sdoe, dia ? vke : ve);
        }
        if constexpr (PATH == 1) {
          const uint8_t* qr = sQb[buf] + (32 * qb + n) * QSB;
#pragma unroll
          for (int s = 0; s < D / 16; ++s)
            sacc = mfma_bf16(__builtin_bit_cast(v8bf, ld16(qr + 2 * (16 * s + 8 * hh))), kb16[s], sacc);
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) sacc[rr] = sacc[rr] * tqk;
        }
        float dsv[16];
        uint32_t pe[8];    // bf16 pairs of P^_eff * 2^8, accumulator register order
        float amax = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = 32 * qb + 8 * g + 4 * hh;      // first of 4 consecutive query rows
          const v4i mv = *reinterpret_cast<const v4i*>(&sM[buf][r0]);
          const v4f ilv = *reinterpret_cast<const v4f*>(&sIL[buf][r0]);
          const v4f dlv = *reinterpret_cast<const v4f*>(&sDl[buf][r0]);
          float pf[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rr = 4 * g + r;
            const int i = q0 + r0 + r;
            float dsr = 0.f, pev = 0.f;
            if (kv && j <= i && i < L) {
              const float x = sacc[rr] * c;
              const float e2 = __builtin_amdgcn_exp2f(__builtin_amdgcn_fractf(x));
              const float pr = __builtin_amdgcn_ldexpf(e2, (int)floorf(x) - mv[r]);
              dsr = (pr * ilv[r]) * (pacc[rr] - dlv[r]);
              if (dia) {
                const int vref = sVref[buf][r0 + r];
                const int code = cvt_fp8x2(__builtin_amdgcn_ldexpf(pr, 8 + e_key - vref), 0.f);
                pev = __builtin_amdgcn_ldexpf(fp8_value(code, 0), vref - e_key);
              } else {
                const int code = cvt_fp8x2(__builtin_amdgcn_ldexpf(pr, 8), 0.f);
                pev = fp8_value(code, 0);
              }
            }
            dsv[rr] = dsr;
            amax = fmaxf(amax, fabsf(dsr));
            pf[r] = pev;
          }
          pe[2 * g] = (uint32_t)f32_to_bf16_bits(pf[0]) | ((uint32_t)f32_to_bf16_bits(pf[1]) << 16);
          pe[2 * g + 1] = (uint32_t)f32_to_bf16_bits(pf[2]) | ((uint32_t)f32_to_bf16_bits(pf[3]) << 16);
        }
        const int e = roundup_exp(wave_max(amax));
        eds[qb] = e;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          dsc[qb][g] = cvt_fp8x4(__builtin_amdgcn_ldexpf(dsv[4 * g], -e), __builtin_amdgcn_ldexpf(dsv[4 * g + 1], -e),
                                 __builtin_amdgcn_ldexpf(dsv[4 * g + 2], -e), __builtin_amdgcn_ldexpf(dsv[4 * g + 3], -e));
        // dV += P^_eff^T G  (two K-steps of 16 queries)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const v8bf av = __builtin_bit_cast(
              v8bf, v4i{(int)pe[4 * ks], (int)pe[4 * ks + 1], (int)pe[4 * ks + 2], (int)pe[4 * ks + 3]});
#pragma unroll
          for (int db = 0; db < ND; ++db)
            dv[db] = mfma_bf16(av, tr_bf16x8(tG, GS, 32 * qb, ks, 32 * db + colg, lane), dv[db]);
        }
      }
    }
    // dK += dS^^T Q~ : K = the 64 queries; lane half hh carries query block hh
    if (wave_active) {
      const v8i adk = v8i{dsc[0][0], dsc[0][1], dsc[0][2], dsc[0][3], dsc[1][0], dsc[1][1], dsc[1][2], dsc[1][3]};
      const int sa = (hh == 0 ? eds[0] : eds[1]) + E8M0_BIAS;
      const int sb = sQeB[buf][hh];
#pragma unroll
      for (int db = 0; db < ND; ++db)
        dk[db] = mfma_f8(adk, cat8(tr_block16(tQ, KS, 0, 32 * db + colg, lane), tr_block16(tQ, KS, 32, 32 * db + colg, lane)),
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
    __syncthreads();
    // dQ^T slice: rows d in [32 ds, 32 ds + 32), columns = queries, K = 128 keys
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
      const int sig = sSig[buf][iq];
      uint16_t* dst = sdQ + iq * D + 32 * ds + 4 * hh;
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
    __syncthreads();
    // row-contiguous packed fp16 atomics: one wave instruction covers whole rows
    {
      constexpr int PAIRS = D / 2;
      for (int idx = tid; idx < BWD_BQ * PAIRS; idx += BWD_THREADS) {
        const int row = idx / PAIRS, pr = idx % PAIRS;
        if (row < nq) {
          const v2h hv = *reinterpret_cast<const v2h*>(sdQ + row * D + 2 * pr);
          __builtin_amdgcn_global_atomic_fadd_v2f16(
              reinterpret_cast<v2h*>(a.dq_acc + doc0 + (size_t)(q0 + row) * rs + 2 * pr), hv);
        }
      }
    }
    if (has_next) commit(buf ^ 1);
    __syncthreads();
  }

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

hipError_t launch_attn_bwd(const Problem& p, const void* plan, const PlanLayout& pl,
                           const uint8_t* q_codes, const uint8_t* k_codes, const uint8_t* v_codes,
                           const uint8_t* v_key_codes, const uint8_t* q_exp, const uint8_t* k_exp,
                           const uint8_t* v_exp, const uint8_t* v_key_exp, const uint8_t* v_ref_exp,
                           const int* row_max, const float* row_sum, const uint8_t* do_codes,
                           const uint8_t* do_exp, const float* delta, const void* g,
                           const int* dq_sigma, void* dq_acc, float* dk_f32, void* dv,
                           const Fp4Operands& f4, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const char* base = static_cast<const char*>(plan);
  BwdArgs a{p, reinterpret_cast<const int*>(base), reinterpret_cast<const int2*>(base + pl.bwd_offset),
            q_codes, k_codes, v_codes, v_key_codes, q_exp, k_exp, v_exp, v_key_exp, v_ref_exp,
            row_max, row_sum, do_codes, do_exp, delta, static_cast<const uint16_t*>(g), dq_sigma,
            static_cast<uint16_t*>(dq_acc), dk_f32, static_cast<uint16_t*>(dv), f4};
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
