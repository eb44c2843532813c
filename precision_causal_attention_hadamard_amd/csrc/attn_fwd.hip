// Forward kernel of the causal block-scaled MXFP8 attention call.
//
// One workgroup (4 waves) per work item (document, 128-query tile, head),
// items taken longest first from the GPU-built list.  With grouped query
// attention the K-side operands are those of key/value head h / (H / Hk).  Wave w owns the 32
// queries of document-local block 4t + w.  The kernel steps over 64-key tiles
// from the document start to the diagonal (to the document end when the call
// is not causal).  Per step:
//   * K~ and V~ codes (and, on the two diagonal key tiles, the per-key V
//     codes) are staged token-major in LDS.  The next tile's global loads are
//     issued into registers before the current tile is computed, and the LDS
//     is double-buffered, so memory latency hides behind the matrix work;
//   * S^T = K~ Q~^T on the scaled FP8 matrix cores (all K operand reads of
//     the tile first, then the products): the token-block exponents
//     are the operand scales, which realises the pages' factorisation
//     S_ij = 2^(eQ(i) + eK(j)) x code dot product ([Reading, 4.1]);
//   * each lane owns one query, so the row maximum is a lane-local max plus
//     one cross-half exchange; it is rounded up to an integer m~ in the
//     log2 domain and every rescale of the running output is a power of two;
//   * P 2^8 = 2^(S' + 8 - m~), S' = S c, evaluated as the backward does
//     (p_scaled): exp2(S') once per score, then the power of two 2^(8 - m~),
//     which rows with m~ in [-100, 120] apply inside the E4M3 convert and once
//     to the tile's sum.  P relative to the final m~ is then exactly P
//     relative to the running m~ times a power of two (the backward's replay
//     relies on it);
//   * P^ = E4M3(P 2^8) enters the P^V product with the constant scale 2^-8;
//     on a query's own 32-token block V uses per-key codes and each key's
//     exponent is folded into P relative to the largest visible per-key
//     exponent of the block, which becomes that query's operand scale
//     ([Summary], opening paragraphs: per-key V scales folded on diagonal
//     tiles; [News, "Key design choices"]);
//   * O^T += V~^T P^^T on the scaled FP8 matrix cores.  P^^T is consumed
//     straight from the S^T accumulator layout; V~^T (d-major) is read from
//     the token-major tile with the LDS transpose read, so the one E4M3
//     payload serves both orientations ([Summary, §3.1 Token-Block Scaling]).
// Epilogue: O = O_acc / l to bf16, integer row max and fp32 l stored.
// Exact option (EXACT): V's codes are per token, and every key block folds
// its keys' exponents into P against a reference -- the query's v_ref_exp on
// its own block, the block's largest exponent on earlier blocks -- which is
// the P operand's scale of that block.
#include "flamia_device.hpp"
#include "flamia_internal.hpp"

namespace flamia {

constexpr int FWD_THREADS = 256;

struct FwdArgs {
  Problem p;
  const int* counts;
  const int2* items;
  const uint8_t *q_codes, *k_codes, *v_codes, *v_key_codes;
  const uint8_t *q_exp, *k_exp, *v_exp, *v_key_exp, *v_ref_exp;
  Fp4Operands f4;
  uint16_t* o;
  int* row_max;
  float* row_sum;
  // diagnostic instantiation only: the P^ codes of every visible (query, key)
  // pair, [H, T, dump_len] by document-local key, and the running integer
  // row maximum each 64-key step used, [H, T, ceil(dump_len / 64)]
  uint8_t* dump;
  int* dump_max;
  int dump_len;
};

// PATH 0: MXFP8 scores.  PATH 1 (mixed): scores from NVFP4 Q and K, expanded
// exactly to bf16 (code x group scale) and multiplied on bf16 matrix cores,
// then scaled by t_Q t_K; the rest of the kernel is shared.
// CAUSAL false: every key of the document is visible (no j <= i mask); the
// diagonal per-key V fold is unchanged, its reference then being the block
// exponent (written so by the quantizer).
// DIAG: also writes each P^ code and the running row maximum it was taken
// against, for the check that the backward replays the forward's codes
// ([Summary, §3.3 Forward-Backward Numerical Consistency]).
// P4: the 4-bit probability operand (log-domain NVFP4, p4_block) in place of
// E4M3 P^ (MXFP8 path, without the exact option).
// POLY: exp2 of the blocks poly_block selects on the FMA-pipe polynomial
// (MXFP8 path, without the exact option or the 4-bit operand).
template <int D, int PATH, bool EXACT, bool CAUSAL, bool DIAG = false, bool P4 = false, bool POLY = false>
__global__ void __launch_bounds__(FWD_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(FwdArgs a) {
  static_assert(!P4 || (PATH == 0 && !EXACT && !DIAG), "4-bit probability operand: MXFP8 path only");
  static_assert(!POLY || (PATH == 0 && !EXACT && !P4), "FMA-pipe exp2: MXFP8 path only");
  constexpr int KS = D + 16;          // token-major row stride (bytes)
  constexpr int KSB = 2 * D + 16;     // token-major bf16 row stride (bytes), mixed path K
  constexpr int NS = D / 64;          // K-steps of the FP8 S product
  constexpr int ND = D / 32;          // d-blocks of the output
  constexpr int NCH = FWD_BK * D / 16 / FWD_THREADS;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][FWD_BK * (PATH ? KSB : KS)];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][FWD_BK * KS];
  __shared__ __attribute__((aligned(16))) uint8_t sVk[2][FWD_BK * KS];
  __shared__ __attribute__((aligned(16))) uint8_t sKe[2][FWD_BK];
  __shared__ __attribute__((aligned(16))) uint8_t sVe[2][FWD_BK];    // read four bytes at a time (exact option)
  __shared__ __attribute__((aligned(16))) uint8_t sVke[2][FWD_BK];
  __shared__ uint8_t sVr[2][2];      // exact option: fold reference (block max) of each key block

  const Problem& p = a.p;
  const int H = p.H, T = p.T;
  const int tile_idx = blockIdx.x / H, head = blockIdx.x % H;
  if (tile_idx >= a.counts[0]) return;
  const int2 it = a.items[tile_idx];
  const int doc = it.x, qt = it.y;
  const int s_d = p.cu[doc];
  const int L = p.cu[doc + 1] - s_d;
  const int q0 = qt * FWD_BQ;

  // the wave index is read into a scalar register, so every per-wave
  // condition below (active key blocks, interior tiles) is a scalar branch
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int qw0 = q0 + 32 * wave;            // this wave's first query
  const int i = qw0 + n;                     // this lane's query (document-local)
  const bool iv = i < L;
  const bool wave_active = qw0 < L;
  const int QB = 4 * qt + wave;              // this wave's query block
  const size_t rs = (size_t)H * D;           // token stride of [T,H,d] codes
  const size_t hT = (size_t)head * T + s_d;  // base of [H,T] metadata of this doc/head
  // K side: the key/value head of this query head ([T,Hk,d] codes, [Hk,T] metadata)
  const int hk = head / (H / p.Hk);
  const size_t rsk = (size_t)p.Hk * D;
  const size_t hTk = (size_t)hk * T + s_d;
  const uint8_t* kdoc = a.k_codes + (size_t)s_d * rsk + (size_t)hk * D;
  const uint8_t* vdoc = a.v_codes + (size_t)s_d * rsk + (size_t)hk * D;
  const uint8_t* vkdoc = a.v_key_codes + (size_t)s_d * rsk + (size_t)hk * D;

  // Q~ as the B operand of S^T = K~ Q~^T (lane = query column)
  v8i qa[PATH ? 1 : NS];
  v8bf qb[PATH ? D / 16 : 1];   // mixed path: NVFP4 Q expanded to bf16, K-step s = d in [16s, 16s + 16)
  int qe = E8M0_BIAS, vref = 0;
  float tqk = 1.f;
  if constexpr (PATH == 1) tqk = a.f4.qk_scale[2] * a.f4.qk_scale[3];
  if (iv) {
    if constexpr (PATH == 0) {
      const uint8_t* qrow = a.q_codes + (size_t)(s_d + i) * rs + (size_t)head * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) qa[s] = cat8(ld16(qrow + 64 * s + 16 * hh), ld16(qrow + 64 * s + 32 + 16 * hh));
      qe = a.q_exp[hT + i];
    } else {
      const size_t qi = (size_t)(s_d + i) * rs + (size_t)head * D;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const uint32_t codes = *reinterpret_cast<const uint32_t*>(a.f4.q_fp4 + qi / 2 + 8 * s + 4 * hh);
        const float sc = fp8_value(a.f4.q_sf[qi / 16 + s], 0);
        qb[s] = __builtin_bit_cast(v8bf, e2m1x8_times_bf16(codes, sc));
      }
    }
    vref = (int)a.v_ref_exp[hTk + i] - E8M0_BIAS;
  } else {
    if constexpr (PATH == 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) qa[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    } else {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qb[s] = __builtin_bit_cast(v8bf, v4i{0, 0, 0, 0});
    }
  }

  v16f oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = v16f{};
  float l_run = 0.f;          // sum of P * 2^8, taken against m_acc
  int m_run = M_NONE;         // running integer row maximum
  int m_acc = M_NONE;         // the maximum oacc and l_run are taken against (<= m_run)
  const float c = p.c_log2;

  const int kt_last = ((CAUSAL ? min(q0 + FWD_BQ, L) : L) - 1) / FWD_BK;

  // ---- register prefetch of one key tile (K side and V side)
  v4i pk[NCH], pv[NCH], pvk[NCH];
  uint32_t psf = 0;           // mixed path: group scales of the prefetched NVFP4 chunk
  uint8_t pke = 0, pve = 0, pvke = 0, pvr = 0;
  const uint8_t* k4doc = PATH ? a.f4.k_fp4 + ((size_t)s_d * rsk + (size_t)hk * D) / 2 : nullptr;
  const uint8_t* ksfdoc = PATH ? a.f4.k_sf + ((size_t)s_d * rsk + (size_t)hk * D) / 16 : nullptr;
  // this thread's 16-byte chunks of a key tile: row, byte offset in the
  // [T, Hk, d] codes from the tile's first key, LDS offset (loop-invariant;
  // a step adds a uniform base)
  int crow[NCH];
  uint32_t cgl[NCH], clds[NCH];
#pragma unroll
  for (int c2 = 0; c2 < NCH; ++c2) {
    const int ch = tid + FWD_THREADS * c2;
    crow[c2] = ch / (D / 16);
    cgl[c2] = (uint32_t)crow[c2] * (uint32_t)rsk + 16u * (uint32_t)(ch % (D / 16));
    clds[c2] = (uint32_t)(crow[c2] * KS + 16 * (ch % (D / 16)));
  }
  auto prefetch_k = [&](int kt) {
    const int j0 = kt * FWD_BK;
    const int nvalid = min(FWD_BK, L - j0);
    if constexpr (PATH == 0) {
      const uint8_t* kt0 = kdoc + (size_t)j0 * rsk;
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2)
        pk[c2] = (nvalid == FWD_BK || crow[c2] < nvalid) ? ld16(kt0 + cgl[c2]) : v4i{0, 0, 0, 0};
    } else {
      // NVFP4 K: 16-byte chunk = 32 codes (d in [32 c, 32 c + 32)) of one key, 2 group scales
      constexpr int CPR = D / 32;       // 16-byte chunks (32 codes) per key row
      if (tid < FWD_BK * CPR) {
        const int r = tid / CPR, c4 = tid % CPR;
        const bool ok = r < nvalid;
        pk[0] = ok ? ld16(k4doc + (size_t)(j0 + r) * rsk / 2 + 16 * c4) : v4i{0, 0, 0, 0};
        psf = ok ? *reinterpret_cast<const uint16_t*>(ksfdoc + (size_t)(j0 + r) * rsk / 16 + 2 * c4) : 0u;
      }
    }
    if (tid < FWD_BK) pke = tid < nvalid ? a.k_exp[hTk + j0 + tid] : (uint8_t)E8M0_BIAS;
  };
  auto prefetch_v = [&](int kt) {
    const int j0 = kt * FWD_BK;
    const int nvalid = min(FWD_BK, L - j0);
    const bool diag_tile = (kt >> 1) == qt;   // holds the query tile's diagonal blocks
    const uint8_t* vt0 = vdoc + (size_t)j0 * rsk;
    const uint8_t* vkt0 = vkdoc + (size_t)j0 * rsk;
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) {
      const bool ok = nvalid == FWD_BK || crow[c2] < nvalid;
      pv[c2] = ok ? ld16(vt0 + cgl[c2]) : v4i{0, 0, 0, 0};
      pvk[c2] = (ok && diag_tile) ? ld16(vkt0 + cgl[c2]) : v4i{0, 0, 0, 0};
    }
    // exact option: the largest per-key exponent of each key block is the
    // in-block prefix maximum at its last token (only read for blocks that
    // lie wholly before the query's own block)
    if (EXACT && tid < 2) pvr = a.v_ref_exp[hTk + min(j0 + 32 * tid + 31, L - 1)];
    if (tid < FWD_BK) {
      const bool kv = tid < nvalid;
      pve = kv ? a.v_exp[hTk + j0 + tid] : (uint8_t)E8M0_BIAS;
      pvke = (kv && diag_tile) ? a.v_key_exp[hTk + j0 + tid] : (uint8_t)E8M0_BIAS;
    }
  };
  auto commit_k = [&](int slot) {
    if constexpr (PATH == 0) {
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) st16(&sK[slot][clds[c2]], pk[c2]);
    } else {
      constexpr int CPR = D / 32;
      if (tid < FWD_BK * CPR) {
        const int r = tid / CPR, c4 = tid % CPR;
        uint8_t* dst = &sK[slot][r * KSB + 64 * c4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
          st16(dst + 16 * w, e2m1x8_times_bf16((uint32_t)pk[0][w], fp8_value((int)psf, w >> 1)));
      }
    }
    if (tid < FWD_BK) sKe[slot][tid] = pke;
  };
  auto commit_v = [&](int buf, bool diag_tile) {
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) {
      st16(&sV[buf][clds[c2]], pv[c2]);
      if (diag_tile) st16(&sVk[buf][clds[c2]], pvk[c2]);   // read on diagonal blocks only
    }
    if (EXACT && tid < 2) sVr[buf][tid] = pvr;
    if (tid < FWD_BK) {
      sVe[buf][tid] = pve;
      sVke[buf][tid] = pvke;
    }
  };

  // ---- S^T of key tile kt for this wave's 32 queries (lane = query column)
  auto scores = [&](int kt, v16f (&st)[2]) {
    const int j0 = kt * FWD_BK;
    const uint8_t* tK = sK[kt & 1];
    const uint8_t* tKe = sKe[kt & 1];
    if constexpr (PATH == 0) {
      // all K operand reads first (one LDS round trip), then the products;
      // a block the wave does not see is computed too (the tile holds its
      // rows, zero past the document end) and ignored by the softmax
      v8i ka[2][NS];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint8_t* krow = tK + (32 * kb + n) * KS;
          ka[kb][s] = cat8(ld16(krow + 64 * s + 16 * hh), ld16(krow + 64 * s + 32 + 16 * hh));
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int ske = tKe[32 * kb + n];
        st[kb] = mfma_f8(ka[kb][0], qa[0], v16f{}, ske, qe);
#pragma unroll
        for (int s = 1; s < NS; ++s) st[kb] = mfma_f8(ka[kb][s], qa[s], st[kb], ske, qe);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = v16f{};
        if ((!CAUSAL || 2 * kt + kb <= QB) && j0 + 32 * kb < L) {
          const uint8_t* krow = tK + (32 * kb + n) * KSB;
#pragma unroll
          for (int s = 0; s < D / 16; ++s)
            st[kb] = mfma_bf16(__builtin_bit_cast(v8bf, ld16(krow + 2 * (16 * s + 8 * hh))), qb[s], st[kb]);
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) st[kb][rr] = st[kb][rr] * tqk;
        }
      }
    }
  };

  // ---- online softmax of key tile kt (scores st) and O^T += V~^T P^^T
  auto softmax_pv = [&](int kt, v16f (&st)[2]) {
    const int buf = kt & 1;
    const int j0 = kt * FWD_BK;
    bool act[2], dia[2], pol[2];
    // interior tile: every key precedes every query of the wave (or, not
    // causal, any key) and lies in the document; both blocks are then active
    // (and, causal, neither is diagonal)
    const bool interior = (!CAUSAL || j0 + FWD_BK <= qw0) && j0 + FWD_BK <= L;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int KB = 2 * kt + kb;
      act[kb] = (!CAUSAL || KB <= QB) && j0 + 32 * kb < L;
      dia[kb] = KB == QB;
      pol[kb] = POLY && poly_block(QB, KB);
    }
    if (!(act[0] || act[1])) return;
    // the tile's maximum over the visible scores (all 64 on an interior tile)
    float tmax = -INFINITY;
    if (interior) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) tmax = fmaxf(tmax, st[kb][rr]);
    } else {
      // key j0 + 32 kb + 8 g + 4 hh + r is visible when its offset 32 kb + 8 g + r
      // (a constant per register) is at most lim
      const int lim = (CAUSAL ? min(i, L - 1) : L - 1) - (j0 + 4 * hh);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (act[kb]) {
#pragma unroll
          for (int rr = 0; rr < 16; rr += 2) {
            const int o0 = 32 * kb + 8 * (rr >> 2) + (rr & 3);
            const float s0 = o0 <= lim ? st[kb][rr] : -INFINITY;
            const float s1 = o0 + 1 <= lim ? st[kb][rr + 1] : -INFINITY;
            tmax = fmaxf(tmax, fmaxf(s0, s1));
          }
        }
    }
    {   // the other lane half holds the query's other 16 keys of each block
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const int m_tile = tmax == -INFINITY ? M_NONE : (int)ceilf(tmax * c);
    m_run = max(m_run, m_tile);
    // The online rescale is deferred: oacc and l_run stay taken against m_acc
    // while m_run - m_acc <= FWD_LAZY, the P^V product carrying the factor
    // 2^(m_run - m_acc) in P^'s operand scale and the sums in their power of
    // two.  Every factor is a power of two, so O is the same bit for bit as
    // with a rescale at every change of m~; when any lane of the wave runs
    // further ahead, all rebase.
    int dl = m_run - m_acc;
    if (__any(dl > FWD_LAZY)) {
      const int sh = m_acc - m_run;   // <= 0
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) oacc[db][rr] = __builtin_amdgcn_ldexpf(oacc[db][rr], sh);
      l_run = __builtin_amdgcn_ldexpf(l_run, sh);
      m_acc = m_run;
      dl = 0;
    }
    const int kofs = 8 - m_run;       // P 2^8 = 2^(S' + 8 - m~)
    // fast form (p_scaled's codes, see there): exp2(S') per score, the row's
    // 2^(8 - m~) applied inside the E4M3 convert and once to the tile's sum
    const bool fast = __all(m_run >= P_M_LO && m_run <= P_M_HI);
    const float psc = __builtin_amdgcn_ldexpf(1.0f, fast ? m_run - 8 : 0);

    // l gains one partial sum per 32-key block, summed in the same order on
    // every path (the fast form sums exp2(S') and scales the sum by 2^(8 - m~),
    // which gives the bits of the sum of the scaled terms)
    int pc[2][4];
    if (fast && interior && !dia[0] && !dia[1]) {
      // the common step, straight-line over both blocks (without the causal
      // mask an interior tile may still hold the query's diagonal block)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float ls = 0.f;
        if constexpr (P4) {
          float e[16];
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            e[rr] = __builtin_amdgcn_exp2f(st[kb][rr] * c);
            ls += e[rr];
          }
          p4_block(e, psc, pc[kb]);
        } else {
          auto block = [&](auto PB) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              float e[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                e[r] = exp2_p<decltype(PB)::value>(st[kb][4 * g + r] * c);
                ls = (g == 0 && r == 0) ? e[r] : ls + e[r];    // exp2 >= +0: the same sum as from 0
              }
              if constexpr (EXACT) {
                // the key's fold against its block's reference, exact before
                // the scaled convert (a product that leaves fp32's normal range
                // here is below 2^-18 after the row's scale: code 0 either way)
                const int fold4 = *reinterpret_cast<const int*>(&sVe[buf][32 * kb + 8 * g + 4 * hh]);
                const int fref = (int)sVr[buf][kb];
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_ldexpf(e[r], ((fold4 >> (8 * r)) & 255) - fref);
              }
              pc[kb][g] = cvt_fp8x4_scaled(e[0], e[1], e[2], e[3], psc);
            }
          };
          if (POLY && pol[kb]) block(std::true_type{}); else block(std::false_type{});
        }
        l_run += __builtin_amdgcn_ldexpf(ls, kofs + dl);
      }
    } else if (PATH == 0 && !EXACT && !P4 && fast) {
      // a step with a diagonal or boundary block, rows in the fast range.  Per
      // 32-key block: one the wave sees none of gives codes 0 and adds 0 to l;
      // one wholly before the wave's queries and inside the document takes
      // the common form; the rest the fast form with the mask (0 for a key the
      // query does not see) and, on the diagonal, the fold as an exact ldexp
      // before the scaled convert -- every fold is <= 0, and a product that
      // leaves fp32's normal range here is below 2^-18 after the row's scale,
      // so the codes are those of the forms below
      const int lim = (CAUSAL ? min(i, L - 1) : L - 1) - (j0 + 4 * hh);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!act[kb]) {
#pragma unroll
          for (int g = 0; g < 4; ++g) pc[kb][g] = 0;
          continue;
        }
        const bool whole = !dia[kb] && j0 + 32 * kb + 32 <= L && (!CAUSAL || 2 * kt + kb < QB);
        float ls = 0.f;
        auto block = [&](auto PB, auto WB) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            // four per-key exponents of the diagonal block's V fold at once
            const int f4 = (!decltype(WB)::value && dia[kb])
                               ? *reinterpret_cast<const int*>(&sVke[buf][32 * kb + 8 * g + 4 * hh]) : 0;
            float e4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              // key j0 + 32 kb + 8 g + 4 hh + r is visible when 32 kb + 8 g + r <= lim
              const bool vis = decltype(WB)::value || 32 * kb + 8 * g + r <= lim;
              const float ev = vis ? exp2_p<decltype(PB)::value>(st[kb][4 * g + r] * c) : 0.f;
              ls = (g == 0 && r == 0) ? ev : ls + ev;     // exp2 >= +0: the same sum as from 0
              e4[r] = (!decltype(WB)::value && dia[kb])
                          ? __builtin_amdgcn_ldexpf(ev, ((f4 >> (8 * r)) & 255) - E8M0_BIAS - vref) : ev;
            }
            pc[kb][g] = cvt_fp8x4_scaled(e4[0], e4[1], e4[2], e4[3], psc);
          }
        };
        if (whole) {
          if (POLY && pol[kb]) block(std::true_type{}, std::true_type{}); else block(std::false_type{}, std::true_type{});
        } else {
          if (POLY && pol[kb]) block(std::true_type{}, std::false_type{}); else block(std::false_type{}, std::false_type{});
        }
        l_run += __builtin_amdgcn_ldexpf(ls, kofs + dl);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float ls = 0.f;
        float pv16[16];          // 4-bit operand: the block's values before its group quantization
        if (interior && !dia[kb]) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            // exact option: the fold of keys 8g + 4hh + r against the block's
            // reference joins the power of two of P (four exponent bytes at once)
            int fold4 = 0;
            if constexpr (EXACT) fold4 = *reinterpret_cast<const int*>(&sVe[buf][32 * kb + 8 * g + 4 * hh]);
            const int fref = EXACT ? (int)sVr[buf][kb] : 0;
            float pv4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float x = st[kb][4 * g + r] * c;
              const float pr = (POLY && pol[kb]) ? p_scaled<POLY>(x, kofs) : p_scaled(x, kofs);
              ls += pr;
              pv4[r] = EXACT ? __builtin_amdgcn_ldexpf(pr, ((fold4 >> (8 * r)) & 255) - fref) : pr;
              pv16[4 * g + r] = pv4[r];
            }
            if constexpr (!P4) pc[kb][g] = cvt_fp8x4(pv4[0], pv4[1], pv4[2], pv4[3]);
          }
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float pv4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int jj = 8 * g + 4 * hh + r;           // key within the 32-block
              const int j = j0 + 32 * kb + jj;
              float pr = 0.f;
              if (act[kb] && (!CAUSAL || j <= i) && j < L) {
                const float x = st[kb][4 * g + r] * c;
                pr = (POLY && pol[kb]) ? p_scaled<POLY>(x, kofs) : p_scaled(x, kofs);
              }
              ls += pr;
              if constexpr (EXACT)   // every block folds V's per-token exponent into P
                pv4[r] = __builtin_amdgcn_ldexpf(pr, ((int)sVe[buf][32 * kb + jj] - E8M0_BIAS) -
                                                         (dia[kb] ? vref : (int)sVr[buf][kb] - E8M0_BIAS));
              else
                pv4[r] = dia[kb] ? __builtin_amdgcn_ldexpf(pr, ((int)sVke[buf][32 * kb + jj] - E8M0_BIAS) - vref) : pr;
              pv16[4 * g + r] = pv4[r];
            }
            if constexpr (!P4) pc[kb][g] = cvt_fp8x4(pv4[0], pv4[1], pv4[2], pv4[3]);
          }
        }
        if constexpr (P4) p4_block(pv16, 1.0f, pc[kb]);
        l_run += __builtin_amdgcn_ldexpf(ls, dl);
      }
    }
    const v8i pb = v8i{pc[0][0], pc[0][1], pc[0][2], pc[0][3], pc[1][0], pc[1][1], pc[1][2], pc[1][3]};
    if constexpr (DIAG) {
      if (a.dump != nullptr && iv) {
        const size_t row = (size_t)head * T + s_d + i;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = j0 + 32 * kb + 8 * g + 4 * hh + r;
              if (act[kb] && j < L && j < a.dump_len && (!CAUSAL || j <= i))
                a.dump[row * a.dump_len + j] = (uint8_t)((pc[kb][g] >> (8 * r)) & 255);
            }
        const int nkt = (a.dump_len + FWD_BK - 1) / FWD_BK;
        if (hh == 0 && kt < nkt) a.dump_max[row * nkt + kt] = m_run;
      }
    }
    // lane half hh supplies the scales of key block hh (with the deferred
    // rescale's 2^(m_run - m_acc) of the lane's query)
    const int sb = dl + (EXACT ? (dia[hh] ? E8M0_BIAS + vref + P_EXP : (int)sVr[buf][hh] + P_EXP)
                               : (dia[hh] ? E8M0_BIAS + vref + P_EXP : E8M0_BIAS + P_EXP));
    const int sa = (EXACT || dia[hh]) ? E8M0_BIAS : (int)sVe[buf][32 * hh];
    // exact option: V's codes are per token everywhere
    const uint8_t* v0 = (!EXACT && dia[0]) ? sVk[buf] : sV[buf];
    const uint8_t* v1 = (!EXACT && dia[1]) ? sVk[buf] : sV[buf];
    const int colg = 16 * ((lane >> 4) & 1);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const v4i va0 = tr_block16(v0, KS, 0, 32 * db + colg, lane);
      const v4i va1 = tr_block16(v1, KS, 32, 32 * db + colg, lane);
      oacc[db] = mfma_f8(cat8(va0, va1), pb, oacc[db], sa, sb);
    }
  };

  // ---- one key step: the next tile's loads go out first, the LDS tiles are
  // double-buffered, one barrier per step
  prefetch_k(0);
  prefetch_v(0);
  commit_k(0);
  commit_v(0, qt == 0);
  __syncthreads();

  for (int kt = 0; kt <= kt_last; ++kt) {
    if (kt < kt_last) {
      prefetch_k(kt + 1);
      prefetch_v(kt + 1);
    }
    if (wave_active) {
      v16f st[2];
      scores(kt, st);
      softmax_pv(kt, st);
    }
    if (kt < kt_last) {
      commit_k((kt + 1) & 1);
      commit_v((kt + 1) & 1, ((kt + 1) >> 1) == qt);
    }
    __syncthreads();
  }

  if (wave_active) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    const float l = __builtin_amdgcn_ldexpf(l_run + (hh ? __uint_as_float(sw[0]) : __uint_as_float(sw[1])), P_EXP);
    // O's 32 rows of the wave go through a free V buffer (the loop's last
    // barrier is behind every wave): row n at 2d bytes, its 16-byte chunks
    // XOR-swizzled by row, then whole rows out with 16-byte stores
    constexpr int CPR = 2 * D / 16;                  // 16-byte chunks per row
    uint8_t* const ot = (wave & 2) ? sVk[wave & 1] : sV[wave & 1];
    static_assert(32 * 2 * D <= FWD_BK * KS, "a wave's O rows fit one V buffer");
    {
      const float inv = 1.0f / l;                    // rows past the document are not stored
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t b0 = f32_to_bf16_bits(oacc[db][4 * g] * inv);
          const uint32_t b1 = f32_to_bf16_bits(oacc[db][4 * g + 1] * inv);
          const uint32_t b2 = f32_to_bf16_bits(oacc[db][4 * g + 2] * inv);
          const uint32_t b3 = f32_to_bf16_bits(oacc[db][4 * g + 3] * inv);
          const int c = 4 * db + g;                  // d = 8c + 4hh .. 8c + 4hh + 3
          *reinterpret_cast<v2i*>(ot + n * (2 * D) + ((c ^ (n & (CPR - 1))) << 4) + 8 * hh) =
              v2i{(int)(b0 | (b1 << 16)), (int)(b2 | (b3 << 16))};
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    {
      constexpr int RPI = 64 / CPR;                  // rows per store instruction
#pragma unroll
      for (int k = 0; k < 32 / RPI; ++k) {
        const int r = RPI * k + lane / CPR, c = lane % CPR;
        const v4i v = *reinterpret_cast<const v4i*>(ot + r * (2 * D) + ((c ^ (r & (CPR - 1))) << 4));
        if (qw0 + r < L) st16(a.o + (size_t)(s_d + qw0 + r) * rs + (size_t)head * D + 8 * c, v);
      }
    }
    if (iv) {
      if (hh == 0) {
        a.row_max[hT + i] = m_run;
        a.row_sum[hT + i] = __builtin_amdgcn_ldexpf(l, m_acc - m_run);   // l is taken against m_acc
      }
    }
  }
}

hipError_t launch_attn_fwd(const Problem& p, const void* plan, const PlanLayout& pl,
                           const uint8_t* q_codes, const uint8_t* k_codes, const uint8_t* v_codes,
                           const uint8_t* v_key_codes, const uint8_t* q_exp, const uint8_t* k_exp,
                           const uint8_t* v_exp, const uint8_t* v_key_exp, const uint8_t* v_ref_exp,
                           const Fp4Operands& f4, void* o, int* row_max, float* row_sum, hipStream_t stream,
                           uint8_t* dump, int* dump_max, int dump_len, bool p4) {
  if (p.T == 0) return hipSuccess;
  const char* base = static_cast<const char*>(plan);
  FwdArgs a{p, reinterpret_cast<const int*>(base), reinterpret_cast<const int2*>(base + pl.fwd_offset),
            q_codes, k_codes, v_codes, v_key_codes, q_exp, k_exp, v_exp, v_key_exp, v_ref_exp, f4,
            static_cast<uint16_t*>(o), row_max, row_sum, dump, dump_max, dump_len};
  dim3 grid((unsigned)pl.cap_fwd * (unsigned)p.H);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(FWD_THREADS), 0, stream, a); };
  if (p.exp2_fma) {        // FMA-pipe exp2 on half of the blocks: MXFP8 path, causal, no exact option
    if (dump_len > 0) {
      if (p.D == 64) go(attn_fwd_kernel<64, 0, false, true, true, false, true>);
      else go(attn_fwd_kernel<128, 0, false, true, true, false, true>);
    } else {
      if (p.D == 64) go(attn_fwd_kernel<64, 0, false, true, false, false, true>);
      else go(attn_fwd_kernel<128, 0, false, true, false, false, true>);
    }
  } else if (p4) {         // 4-bit probability operand: MXFP8 path, no exact option
    if (p.causal) {
      if (p.D == 64) go(attn_fwd_kernel<64, 0, false, true, false, true>);
      else go(attn_fwd_kernel<128, 0, false, true, false, true>);
    } else {
      if (p.D == 64) go(attn_fwd_kernel<64, 0, false, false, false, true>);
      else go(attn_fwd_kernel<128, 0, false, false, false, true>);
    }
  } else if (dump_len > 0) {      // diagnostic instantiation: MXFP8 path, causal, no exact option
    if (p.D == 64) go(attn_fwd_kernel<64, 0, false, true, true>); else go(attn_fwd_kernel<128, 0, false, true, true>);
  } else if (p.path == 1 && p.causal) {
    if (p.D == 64) go(attn_fwd_kernel<64, 1, false, true>); else go(attn_fwd_kernel<128, 1, false, true>);
  } else if (p.path == 1) {
    if (p.D == 64) go(attn_fwd_kernel<64, 1, false, false>); else go(attn_fwd_kernel<128, 1, false, false>);
  } else if (p.exact) {
    if (p.D == 64) go(attn_fwd_kernel<64, 0, true, true>); else go(attn_fwd_kernel<128, 0, true, true>);
  } else if (!p.causal) {
    if (p.D == 64) go(attn_fwd_kernel<64, 0, false, false>); else go(attn_fwd_kernel<128, 0, false, false>);
  } else {
    if (p.D == 64) go(attn_fwd_kernel<64, 0, false, true>); else go(attn_fwd_kernel<128, 0, false, true>);
  }
  return hipGetLastError();
}

}  // namespace flamia
