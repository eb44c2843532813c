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
// per-row planes: 8 - integer row maximum, 2^-8 / l, D, the dQ prescale
// exponent, the Q / dO / fold-reference exponent bytes) go global -> LDS directly, with
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
//     evaluation of P 2^8 = 2^(S' + 8 - m~) (p_scaled; its fast form where
//     the query block's flag allows) with the stored integer
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
  const int* kofs;        // [H, T] 8 - integer row maximum of the forward
  const float* il8;       // [H, T] 2^-8 / l
  const float* delta;     // [H, T] -D
  const int* dq_sigma;    // [H, T] dQ prescale exponent
  const int* qexps;       // [H, T] q_exp | do_exp << 8 | v_ref_exp << 16 (biased bytes) | fast-form flag << 24
  const uint8_t* do_codes;
  const uint16_t* g;
  uint16_t* dq_acc;
  float* dk_f32;          // mixed path: fp32 dK staging; split groups: fp32 dK partials
  uint16_t* dk;           // MXFP8 path: bf16 dK
  uint16_t* dv;
  float* dv_f32;          // split groups: fp32 dV partials [gsplit, T, Hk, d]
  int gsplit;             // items per key/value head group
  uint16_t* dq_part;      // deterministic mode: fp16 dQ partial slots
  const int* det_base;    // deterministic mode: first step of each document
  int det_cap;            // deterministic mode: steps per head in dq_part
  const uint8_t* v_ref_exp;    // exact option: V's in-block prefix maximum (block maxima at block ends)
  const uint16_t *q_x, *k_x;   // mixed path: NVFP4 Q and K expanded to bf16
  const float* qk_scale;       // mixed path: [2], [3] tensor scales
  uint8_t* dump;               // diagnostic instantiation: P^ codes [H, T, dump_len] (or null)
  int dump_len;
  unsigned long long* ds_counts;   // diagnostic instantiation: [0] nonzero dS, [1] those coded 0
};

// PATH 0: MXFP8 scores.  PATH 1 (mixed): the recomputed scores come from the
// NVFP4 Q and K (expanded exactly to bf16) on bf16 matrix cores with the same
// operand split and order as the forward, then scaled by t_Q t_K; dK and dQ
// still use the E4M3 token-block Q~ and K~.
// CAUSAL false: every query tile of the document visits the key tile (no
// j <= i mask), as in attn_bwd8_kernel.
template <int D, int PATH, bool CAUSAL>
__global__ void __launch_bounds__(BWD_THREADS) attn_bwd_kernel(BwdArgs a) {
  constexpr int DSK = BWD_BQ + 16;           // key-major dS^ row stride (bytes)
  constexpr int NS = D / 64;
  constexpr int ND = D / 32;
  constexpr int CT = BWD_BQ * D;             // bytes of a query code tile
  constexpr int WT = BWD_BQ * 2 * D;         // bytes of a query bf16 tile
  constexpr int RT = NPLANES * BWD_BQ * 4;   // bytes of the per-row planes
  constexpr int DQS = D + 4;                 // fp16 dQ staging row stride (elements): 8 bytes of
                                             // padding put the 32 rows of one store on distinct banks

  __shared__ __attribute__((aligned(1024))) uint8_t sK[BWD_BK * D];         // K~ tile of the item
  __shared__ __attribute__((aligned(1024))) uint8_t sKQ[BWD_BQ * DQS * 2];  // fp16 dQ partial of a step
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

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
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
  // K side: the key/value head of this query head ([T,Hk,d] codes, [Hk,T] metadata);
  // with grouped heads (gsplit = H / Hk) dK and dV leave as fp32 partials, one
  // per query head of the group, which the group reduction adds and rounds once
  const int hk = head / (H / p.Hk);
  const size_t rsk = (size_t)p.Hk * D;
  const size_t hTk = (size_t)hk * T + s_d;
  const size_t doc0k = (size_t)s_d * rsk + (size_t)hk * D;
  const uint32_t rsk32 = (uint32_t)rsk;
  const float c = p.c_log2;
  // per-document bases (uniform); per-lane offsets fit 32 bits (checked on the host)
  const uint8_t* q_doc = a.q_codes + doc0;
  const uint8_t* do_doc = a.do_codes + doc0;
  const uint8_t* k_doc = a.k_codes + doc0k;
  const uint8_t* g_doc = reinterpret_cast<const uint8_t*>(a.g + doc0);
  const uint8_t* x_doc = PATH ? reinterpret_cast<const uint8_t*>(a.q_x + doc0) : nullptr;
  uint8_t* dq_doc = reinterpret_cast<uint8_t*>(a.dq_acc + doc0);

  // ---- staging of row tiles: rows row0 + r, clamped to the document's last row.
  // Instruction i of a tile fills tile bytes [1024 i, 1024 i + 1024); lane l
  // brings the 16-byte chunk that the swizzle puts at byte 1024 i + 16 l.
  auto dma_codes = [&](uint8_t* tile, const uint8_t* src, uint32_t stride, int row0, int nrows) {
    const int ninst = nrows * D / 1024;
    for (int i = wave; i < ninst; i += 4) {
      const int o = i * 1024 + 16 * lane;
      const int r = o / D, slot = (o % D) >> 4;
      const uint32_t gr = (uint32_t)min(row0 + r, L - 1);
      dma16(src + (gr * stride + 16u * (uint32_t)(slot ^ code_key<D>(r))), tile + i * 1024);
    }
  };
  // the query tiles: instruction k of this wave is tile instruction wave + 4k;
  // its row and swizzled column are the same for every tile (loop-invariant)
  constexpr int NIC = CT / 1024 / 4;     // code-tile instructions per wave
  constexpr int NIW = WT / 1024 / 4;     // bf16-tile instructions per wave
  // byte offsets: row r of a code tile is r * rs bytes from row 0 (bf16 tiles 2 r rs)
  uint32_t crow[NIC], wrow[NIW], ccol[NIC], wcol[NIW], xcol[NIW];
#pragma unroll
  for (int k = 0; k < NIC; ++k) {
    const int o = (wave + 4 * k) * 1024 + 16 * lane;
    crow[k] = (uint32_t)(o / D) * rs32;
    ccol[k] = 16u * (uint32_t)(((o % D) >> 4) ^ code_key<D>(o / D));
  }
#pragma unroll
  for (int k = 0; k < NIW; ++k) {
    const int o = (wave + 4 * k) * 1024 + 16 * lane;
    const int r = o / (2 * D), slot = (o % (2 * D)) >> 4;
    wrow[k] = 2u * (uint32_t)r * rs32;
    wcol[k] = 16u * (uint32_t)(slot ^ wide_key<D>(r));
    xcol[k] = 16u * (uint32_t)(slot ^ xq_key<D>(r));
  }
  const uint32_t last_c = (uint32_t)(L - 1) * rs32;       // the document's last row
  const uint32_t last_w = 2u * last_c;
  const int* const planes[NPLANES] = {a.kofs + hT, reinterpret_cast<const int*>(a.il8) + hT,
                                      reinterpret_cast<const int*>(a.delta) + hT, a.dq_sigma + hT, a.qexps + hT};
  auto issue_tile = [&](auto Bc, int qt) {
    constexpr int B = decltype(Bc)::value;
    const int q0 = qt * BWD_BQ;
    const uint32_t q0c = (uint32_t)q0 * rs32, q0w = 2u * q0c;   // uniform
#pragma unroll
    for (int k = 0; k < NIC; ++k) {
      const uint32_t off = min(q0c + crow[k], last_c) + ccol[k];
      dma16(q_doc + off, (B ? sQ1 : sQ0) + (wave + 4 * k) * 1024);
      dma16(do_doc + off, (B ? sO1 : sO0) + (wave + 4 * k) * 1024);
    }
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
      const uint32_t rowb = min(q0w + wrow[k], last_w);
      dma16(g_doc + (rowb + wcol[k]), (B ? sG1 : sG0) + (wave + 4 * k) * 1024);
      if constexpr (PATH == 1) dma16(x_doc + (rowb + xcol[k]), (B ? sX1 : sX0) + (wave + 4 * k) * 1024);
    }
    const int mrow = min(q0 + lane, L - 1);
    for (int pl = wave; pl < NPLANES; pl += 4) dma4(planes[pl] + mrow, (B ? sR1 : sR0) + pl * BWD_BQ * 4);
  };

  // ---- per item: the key tile (for K~^T of dQ) and the first query tile
  const int qt_first = CAUSAL ? k0 / BWD_BQ : 0;
  const int qt_end = (L + BWD_BQ - 1) / BWD_BQ;
  dma_codes(sK, k_doc, rsk32, k0, BWD_BK);
  issue_tile(std::integral_constant<int, 0>{}, qt_first);
  if (tid < 4) sKeB[tid] = k0 + 32 * tid < L ? (int)a.k_exp[hTk + k0 + 32 * tid] : E8M0_BIAS;

  // ---- per wave: K~ (or the mixed path's bf16 K) and V~ block codes as B
  // operands (lane = key); the per-key V~ codes are loaded on the diagonal
  // block only
  v8i kreg[PATH ? 1 : NS], vreg[NS];
  v8bf kb16[PATH ? D / 16 : 1];
  int ke = E8M0_BIAS, ve = E8M0_BIAS, vke = E8M0_BIAS;
  float tqk = 1.f;
  if constexpr (PATH == 1) tqk = a.qk_scale[2] * a.qk_scale[3];
  {
    const size_t ro = doc0k + (size_t)min(j, L - 1) * rsk;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (PATH == 0)
        kreg[s] = cat8(ld16(a.k_codes + ro + 64 * s + 16 * hh), ld16(a.k_codes + ro + 64 * s + 32 + 16 * hh));
      vreg[s] = cat8(ld16(a.v_codes + ro + 64 * s + 16 * hh), ld16(a.v_codes + ro + 64 * s + 32 + 16 * hh));
    }
    if constexpr (PATH == 1) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) kb16[s] = __builtin_bit_cast(v8bf, ld16(a.k_x + ro + 16 * s + 8 * hh));
    }
    const size_t mi = hTk + min(j, L - 1);
    ke = a.k_exp[mi];
    ve = a.v_exp[mi];
    vke = a.v_key_exp[mi];
    if (!kv) {    // keys past the document: zero operands
#pragma unroll
      for (int s = 0; s < NS; ++s) vreg[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
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
  // per-key V~ codes of this lane's key (B operand of dP on the diagonal block)
  auto vkey = [&](int s2) {
    const uint8_t* vr = a.v_key_codes + doc0k + (size_t)min(j, L - 1) * rsk + 64 * s2 + 16 * hh;
    return kv ? cat8(ld16(vr), ld16(vr + 32)) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
  };
  full_barrier();

  // dQ^T: wave -> d-slice ds; K~^T of that slice is read from sK each step
  const int ds = wave % ND;

  v16f dk[ND], dv[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) { dk[db] = v16f{}; dv[db] = v16f{}; }

  // fp16 dQ partial of query tile qtp (staged in sKQ) -> memory-side atomics.
  // One wave instruction covers whole rows (one row for d = 128, two for 64),
  // rows wave, wave + 4, ...; the per-lane parts of both addresses are fixed.
  constexpr int RPI = 128 / D;                       // rows per wave instruction
  const int frow = RPI == 1 ? 0 : lane >> 5;
  const int fpair = RPI == 1 ? lane : lane & 31;
  const uint16_t* const fsrc = reinterpret_cast<const uint16_t*>(sKQ) + frow * DQS + 2 * fpair;
  const uint32_t fdst = 2u * (uint32_t)frow * rs32 + 4u * (uint32_t)fpair;
  // (in two halves, so the atomics are spread over the step)
  // deterministic mode: plain stores into the step's own partial slot instead
  const int nq_doc = (L + BWD_BQ - 1) / BWD_BQ;
  auto flush_dq = [&](int qtp, int half) {
    constexpr int NIT = BWD_BQ / (8 * RPI);
    const int q0p = qtp * BWD_BQ;
    const int nqp = min(BWD_BQ, L - q0p);
    v2h hv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      hv[it] = *reinterpret_cast<const v2h*>(fsrc + RPI * (wave + 4 * (it + NIT * half)) * DQS);
    if (p.deterministic) {
      const long long step = det_step(a.det_base[doc], u, qtp, nq_doc, CAUSAL);
      if (step >= a.det_cap) return;      // the plan flags the overflow
      uint8_t* const slot = reinterpret_cast<uint8_t*>(a.dq_part) + ((size_t)step * H + head) * (BWD_BQ * D * 2);
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int row0 = RPI * (wave + 4 * (it + NIT * half));
        *reinterpret_cast<v2h*>(slot + (row0 + frow) * (D * 2) + 4 * fpair) = hv[it];
      }
      return;
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int row0 = RPI * (wave + 4 * (it + NIT * half));    // uniform
      if (row0 + frow < nqp)
        __builtin_amdgcn_global_atomic_fadd_v2f16(
            reinterpret_cast<v2h*>(dq_doc + (2u * (uint32_t)(q0p + row0) * rs32 + fdst)), hv[it]);
    }
  };

  // per-lane LDS offsets of the operand reads (loop-invariant; every swizzle
  // key has period 16 or less in the row, and the reads start at rows that
  // are multiples of 16)
  const int ck = code_key<D>(n);
  int offA[NS][2];                 // row n, 16-byte chunks 4s + hh and 4s + 2 + hh
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
    for (int e = 0; e < 2; ++e) offA[s2][e] = n * D + (((4 * s2 + 2 * e + hh) ^ ck) << 4);
  int offK[ND];                    // 8-bit transpose reads of the Q~ tile (dK operand)
  {
    const int pp = lane & 15, b = pp >> 1;
    const int t = 8 * (b >> 2) + 4 * hh + (b & 3);
#pragma unroll
    for (int db = 0; db < ND; ++db) offK[db] = code_off<D>(t, 32 * db + colg + 8 * (pp & 1));
  }
  int offG[ND][2];                 // 16-bit transpose reads of the G tile (dV operand)
  {
    const int pp = lane & 15, e = pp >> 2, s4 = pp & 3;
    const int t = 4 * hh + e;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      offG[db][0] = wide_off<D>(t, 2 * (32 * db + colg + 4 * s4));
      offG[db][1] = wide_off<D>(t + 8, 2 * (32 * db + colg + 4 * s4));
    }
  }

  auto step = [&](auto Bc, int qt) {
    constexpr int B = decltype(Bc)::value;
    const uint8_t* tQ = B ? sQ1 : sQ0;
    const uint8_t* tdO = B ? sO1 : sO0;
    const uint8_t* tG = B ? sG1 : sG0;
    const uint8_t* tX = B ? sX1 : sX0;
    const uint8_t* tR = B ? sR1 : sR0;
    const int* pko = reinterpret_cast<const int*>(tR);
    const float* pil = reinterpret_cast<const float*>(tR + BWD_BQ * 4);
    const float* pdl = reinterpret_cast<const float*>(tR + 2 * BWD_BQ * 4);
    const int* psig = reinterpret_cast<const int*>(tR + 3 * BWD_BQ * 4);
    const int* pqx = reinterpret_cast<const int*>(tR + 4 * BWD_BQ * 4);
    const int q0 = qt * BWD_BQ;
    const int nq = min(BWD_BQ, L - q0);

    // the next tile streams in while this one is computed (issued once the
    // first block's products are under way); last step's dQ goes out in two
    // halves between the blocks

    int dsc[2][4];
    int eds[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int QB = 2 * qt + qb;
      const bool act = wave_active && (!CAUSAL || QB >= KB) && 32 * qb < nq;
      eds[qb] = -127;
#pragma unroll
      for (int g = 0; g < 4; ++g) dsc[qb][g] = 0;
      const bool dia = QB == KB;
      // no mask, no fold; without the causal mask a key block may also run past the document end
      const bool fast = !dia && 32 * qb + 32 <= nq && (CAUSAL || k0 + 32 * wave + 32 <= L);
      v16f sacc = v16f{}, pacc = v16f{};
      if (act) {
        const int qx = pqx[32 * qb];
        const int sqe = qx & 255, sdoe = (qx >> 8) & 255;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if constexpr (PATH == 0)
            sacc = mfma_f8(cat8(ld16(tQ + 32 * qb * D + offA[s][0]), ld16(tQ + 32 * qb * D + offA[s][1])),
                           kreg[s], sacc, sqe, ke);
          pacc = mfma_f8(cat8(ld16(tdO + 32 * qb * D + offA[s][0]), ld16(tdO + 32 * qb * D + offA[s][1])),
                         dia ? vkey(s) : vreg[s], pacc, sdoe, dia ? vke : ve);
        }
        if constexpr (PATH == 1) {
          const int row = 32 * qb + n;
#pragma unroll
          for (int s = 0; s < D / 16; ++s)
            sacc = mfma_bf16(__builtin_bit_cast(v8bf, ld16(tX + xq_off<D>(row, 32 * s + 16 * hh))), kb16[s], sacc);
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) sacc[rr] = sacc[rr] * tqk;
        }
      }
      if (qb == 0 && qt + 1 < qt_end) issue_tile(std::integral_constant<int, 1 - B>{}, qt + 1);
      float dsv[16];
      uint32_t pe[8];      // bf16 pairs of P^_eff * 2^8, accumulator register order
      if (act) {
        float amax = 0.f;
        if (fast) {
          // one straight-line body per probability form (fast where every
          // row of the query block allows it)
          auto rows = [&](auto PW) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int r0 = 32 * qb + 8 * g + 4 * hh;      // first of 4 consecutive query rows
            const v4i kov = *reinterpret_cast<const v4i*>(pko + r0);
            const v4f ilv = *reinterpret_cast<const v4f*>(pil + r0);
            const v4f dlv = *reinterpret_cast<const v4f*>(pdl + r0);
            float pf[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)      // P 2^8
              pf[r] = decltype(PW)::value
                          ? __builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f(sacc[4 * g + r] * c), kov[r])
                          : p_scaled(sacc[4 * g + r] * c, kov[r]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int rr = 4 * g + r;
              dsv[rr] = (pf[r] * ilv[r]) * (pacc[rr] + dlv[r]);
              amax = fmaxf(amax, fabsf(dsv[rr]));
            }
            const int code = cvt_fp8x4(pf[0], pf[1], pf[2], pf[3]);
            pe[2 * g] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, false));
            pe[2 * g + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, true));
          }
          };
          if ((__builtin_amdgcn_readfirstlane(pqx[32 * qb]) >> 24) & 1)
            rows(std::true_type{});
          else
            rows(std::false_type{});
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int r0 = 32 * qb + 8 * g + 4 * hh;
            const v4i kov = *reinterpret_cast<const v4i*>(pko + r0);
            const v4f ilv = *reinterpret_cast<const v4f*>(pil + r0);
            const v4f dlv = *reinterpret_cast<const v4f*>(pdl + r0);
            float pf[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int rr = 4 * g + r;
              const int i = q0 + r0 + r;
              float dsr = 0.f, pev = 0.f;
              if (kv && (!CAUSAL || j <= i) && i < L) {
                const float p8 = p_scaled(sacc[rr] * c, kov[r]);
                dsr = (p8 * ilv[r]) * (pacc[rr] + dlv[r]);
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
        // amax >= 0, so its bits order like the values
        const int e = roundup_exp(__int_as_float(wave_max_i(__float_as_int(amax))));
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
      }
      if (qt > qt_first) flush_dq(qt - 1, qb);
      if (act) {
        // dV += P^_eff^T G  (two K-steps of 16 queries)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const v8bf av = __builtin_bit_cast(
              v8bf, v4i{(int)pe[4 * ks], (int)pe[4 * ks + 1], (int)pe[4 * ks + 2], (int)pe[4 * ks + 3]});
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            const uint8_t* g0 = tG + (32 * qb + 16 * ks) * 2 * D;
            const v4s lo = lds_tr16(g0 + offG[db][0]);
            const v4s hi = lds_tr16(g0 + offG[db][1]);
            dv[db] = mfma_bf16(av, __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)),
                               dv[db]);
          }
        }
      }
    }
    // dK += dS^^T Q~ : K = the 64 queries; lane half hh carries query block hh
    if (wave_active) {
      const v8i adk = v8i{dsc[0][0], dsc[0][1], dsc[0][2], dsc[0][3], dsc[1][0], dsc[1][1], dsc[1][2], dsc[1][3]};
      const int sa = (hh == 0 ? eds[0] : eds[1]) + E8M0_BIAS;
      const int sb = pqx[32 * hh] & 255;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const uint8_t* q0p = tQ + offK[db];
        const v2i a0 = lds_tr8(q0p), a1 = lds_tr8(q0p + 16 * D), a2 = lds_tr8(q0p + 32 * D), a3 = lds_tr8(q0p + 48 * D);
        dk[db] = mfma_f8(adk, v8i{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]}, dk[db], sa, sb);
      }
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
        const v8i kt = cat8(tr_code16<D>(sK, 64 * ks, 32 * ds + colg, lane),
                            tr_code16<D>(sK, 64 * ks + 32, 32 * ds + colg, lane));
        acc = mfma_f8(kt, bq, acc, sKeB[2 * ks + hh], sEds[qb][2 * ks + hh] + E8M0_BIAS);
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
  flush_dq(qt_end - 1, 0);
  flush_dq(qt_end - 1, 1);

  // ---- item end: dK (scaled, fp32 staging) and dV (bf16)
  if (wave_active) {
    const float sc = p.softmax_scale;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int jk = k0 + 32 * wave + 8 * (rr >> 2) + 4 * hh + (rr & 3);
        if (jk < L && a.gsplit > 1) {
          const size_t o = (size_t)(head % a.gsplit) * T * rsk + doc0k + (size_t)jk * rsk + 32 * db + n;
          a.dk_f32[o] = dk[db][rr] * sc;
          a.dv_f32[o] = dv[db][rr];
        } else if (jk < L) {
          const size_t o = doc0 + (size_t)jk * rs + 32 * db + n;
          a.dk_f32[o] = dk[db][rr] * sc;
          a.dv[o] = f32_to_bf16_bits(dv[db][rr]);
        }
      }
  }
}

// Key-major dS^ tile of the eight-wave kernel: row = key (128 rows of 64 B),
// 16-byte chunk c = 2 hh + qh holds the four dwords one lane of the wave of
// query half qh wrote (queries 32 qh + 8 g + 4 hh + r, g = dword, r = byte).
// Chunks are XOR-swizzled by a key of row bits 1-3 so that the 16-byte writes
// (8-lane passes over 128 B), the 16-byte dK operand reads (16-lane passes
// over 256 B) and the 8-bit transpose reads of the dQ operand (32-lane passes
// over 256 B) all reach every bank once per pass.
// Row of the fp16 dQ staging tile that holds query row q: rows with bit 4 set
// trade places with their neighbour four rows away, so the 16 query rows one
// 16-lane store pass writes (q = 8 a + b + const, a, b < 4, lanes split by
// bit 4 of q) fall on 16 distinct 8-byte bank groups of the 264-byte rows.
__device__ __forceinline__ int stage_row(int q) { return q ^ (((q >> 4) & 1) << 2); }

__device__ __forceinline__ int dsk_off(int r, int chunk) {
  const int key = (((r >> 2) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1);
  return r * 64 + ((chunk ^ key) << 4);
}

// Largest value over the 32 lanes of the calling lane's wave half: four DPP
// rotations inside each 16-lane row, then one swizzle that pairs lane l with
// lane l ^ 16.
// Reduce-scatter of 16 registers over the 32 lanes of a wave half: lane n of
// the half returns the largest value of register (n >> 1) over the half.
// Each level pairs two registers, keeps one in the lanes whose bit is clear
// and the other where it is set, and takes the maximum with the partner lane
// across that bit (bits 4, 3, 2, 1 by swizzle or DPP), then bit 0 finishes.
template <int PAT>
__device__ __forceinline__ float swizzle_f(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), PAT));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float rows_max16(const float (&v)[16], int n) {
  const bool b4 = n & 16, b3 = n & 8, b2 = n & 4, b1 = n & 2;
  float w[8], x[4], y[2];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    w[k] = fmaxf(b4 ? v[k + 8] : v[k], swizzle_f<0x401f>(b4 ? v[k] : v[k + 8]));    // xor 16
#pragma unroll
  for (int k = 0; k < 4; ++k)
    x[k] = fmaxf(b3 ? w[k + 4] : w[k], dpp_f<0x128>(b3 ? w[k] : w[k + 4]));         // xor 8 (row_ror:8)
#pragma unroll
  for (int k = 0; k < 2; ++k)
    y[k] = fmaxf(b2 ? x[k + 2] : x[k], swizzle_f<0x101f>(b2 ? x[k] : x[k + 2]));    // xor 4
  const float z = fmaxf(b1 ? y[1] : y[0], dpp_f<0x4e>(b1 ? y[0] : y[1]));            // xor 2 (quad_perm)
  return fmaxf(z, dpp_f<0xb1>(z));                                                  // xor 1 (quad_perm)
}

__device__ __forceinline__ float half_max32(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x128, 0xf, 0xf, false)));  // row_ror:8
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x124, 0xf, 0xf, false)));  // row_ror:4
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x122, 0xf, 0xf, false)));  // row_ror:2
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x121, 0xf, 0xf, false)));  // row_ror:1
  return fmaxf(m, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x401f)));               // xor 16
}

// ---------------------------------------------------------------------------
// Eight-wave backward (MXFP8 path): two waves per SIMD on the same item.
// Wave w owns key block kb = w & 3 and, of each 64-query tile, query block
// qh = w >> 2.  It forms S, dP, P, dS and the dS^ codes of its 32 x 32 block
// (the block exponent is a whole-wave reduction, as above), and adds
// P^_eff^T G over its 32 queries to a dV accumulator for all of d; the two
// waves of a key block sum their dV at the end of the item.  dK needs both
// query blocks: after the barrier that publishes the dS^ codes key-major, each
// wave of the pair forms dK for half of d over all 64 queries.  dQ^T is one
// (d slice, query block) pair per wave.  K~ and V~ of the item stay in LDS and
// are read as operands each step.
// Grouped query attention: the item is (document, key tile, key/value head,
// part) and the query-tile loop runs over the part's query heads in turn, so
// dK and dV sum them in fp32 registers.  With one part per group (the usual
// case) they are rounded once here; when the grid would be too small the
// group is split over gsplit items, which store fp32 partials that a reduce
// kernel adds in order and rounds once.  GRP = false is the one-head-per-item
// instantiation (H = Hk): the loop runs the query tiles of one head only.
// EXACT (exact option): Q, K, V, dO scales are per token --
// the recomputed S and dP take each row's exponent as its operand scale; every
// key block folds V's exponents into P for dV; dS is quantized twice, with
// K's exponent folded in and one exponent per (query, 32 keys) for dQ, and
// with Q's exponent folded in and one exponent per (key, 32 queries) for dK.
// CAUSAL false: every query tile of the document visits the key tile (no
// j <= i mask); the diagonal per-key V codes and fold stay, against the block
// exponent as the quantizer then writes it.
// DIAG: also writes each recomputed P^ code (the forward's, relative to the
// final row maximum, when the replay is exact: [Summary, §3.3
// Forward-Backward Numerical Consistency]) and counts the nonzero dS and
// those whose E4M3 code is zero ([Summary, §3.3] second bullet).
template <int D, bool DET, bool GRP, bool EXACT, bool CAUSAL, bool DIAG = false, bool POLY = false>
__global__ void __launch_bounds__(2 * BWD_THREADS) attn_bwd8_kernel(BwdArgs a) {
  static_assert(!POLY || (!DET && !GRP && !EXACT && CAUSAL), "FMA-pipe exp2: the default call only");
  constexpr int NS = D / 64;
  constexpr int ND = D / 32;
  constexpr int NDK = ND / 2;                // dK d-blocks per wave
  constexpr int CT = BWD_BQ * D;             // bytes of a query code tile
  constexpr int WT = BWD_BQ * 2 * D;         // bytes of a query bf16 tile
  constexpr int RT = NPLANES * BWD_BQ * 4;   // bytes of the per-row planes
  constexpr int DQS = D + 4;                 // fp16 dQ staging row stride (elements)
  static_assert(WT >= 64 * ND * 16 * 4, "a key block's dV partial sums fit one bf16 tile buffer");

  __shared__ __attribute__((aligned(1024))) uint8_t sK[BWD_BK * D];         // K~ tile of the item
  __shared__ __attribute__((aligned(1024))) uint8_t sV[BWD_BK * D];         // V~ block codes of the item
  // per-key V~ codes of the item (the diagonal blocks' dP operand), same layout
  __shared__ __attribute__((aligned(1024))) uint8_t sVk[EXACT ? 16 : BWD_BK * D];
  // query-tile double buffers (distinct arrays, so reads of one buffer never
  // wait for the loads into the other); after the last step the bf16 pair
  // holds the dV partial sums
  __shared__ __attribute__((aligned(1024))) uint8_t sQ0[CT];
  __shared__ __attribute__((aligned(1024))) uint8_t sQ1[CT];
  __shared__ __attribute__((aligned(1024))) uint8_t sO0[CT];
  __shared__ __attribute__((aligned(1024))) uint8_t sO1[CT];
  __shared__ __attribute__((aligned(1024))) uint8_t sG0[WT];
  __shared__ __attribute__((aligned(1024))) uint8_t sG1[WT];
  __shared__ __attribute__((aligned(256))) uint8_t sR0[RT];
  __shared__ __attribute__((aligned(256))) uint8_t sR1[RT];
  __shared__ __attribute__((aligned(1024))) uint8_t sdSK[BWD_BK * BWD_BQ];
  __shared__ __attribute__((aligned(1024))) uint8_t sKQ[BWD_BQ * DQS * 2];  // fp16 dQ partial of a step
  __shared__ int sEds[2][4];
  __shared__ int sKeB[4];
  // exact option: the dQ payload (same layout as sdSK), its exponents per (key
  // block, query), the dK payload's exponents per (query half, key), and each
  // key block's largest V exponent
  __shared__ __attribute__((aligned(1024))) uint8_t sdSQ[EXACT ? BWD_BK * BWD_BQ : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sRowE[EXACT ? 4 : 1][BWD_BQ];
  __shared__ uint8_t sColE[EXACT ? 2 : 1][BWD_BK];
  __shared__ int sVrB[4];

  const Problem& p = a.p;
  const int H = p.H, T = p.T, Hk = p.Hk;
  const int tile_idx = GRP ? (int)(blockIdx.x / (Hk * a.gsplit)) : (int)(blockIdx.x / H);
  const int hk = GRP ? (int)((blockIdx.x / a.gsplit) % Hk) : (int)(blockIdx.x % H);
  if (tile_idx >= a.counts[1]) return;
  const int2 it = a.items[tile_idx];
  const int doc = it.x, u = it.y;
  const int s_d = p.cu[doc];
  const int L = p.cu[doc + 1] - s_d;
  const int k0 = u * BWD_BK;
  const int hpp = GRP ? H / Hk / a.gsplit : 1;                        // query heads per part
  const int h_first = GRP ? hk * (H / Hk) + (int)(blockIdx.x % a.gsplit) * hpp : hk, h_end = h_first + hpp;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
  const int kb = wave & 3, qh = wave >> 2;
  const int n = lane & 31, hh = lane >> 5;
  const int colg = 16 * ((lane >> 4) & 1);
  const int j = k0 + 32 * kb + n;             // this lane's key (document-local)
  const bool kv = j < L;
  const bool kb_active = k0 + 32 * kb < L;
  const int KB = 4 * u + kb;
  const size_t rs = (size_t)H * D;            // query side: [T,H,d], [H,T]
  const size_t rsk = (size_t)Hk * D;          // key side: [T,Hk,d], [Hk,T]
  const size_t hTk = (size_t)hk * T + s_d;
  const size_t doc0k = (size_t)s_d * rsk + (size_t)hk * D;
  const uint32_t rs32 = (uint32_t)rs, rsk32 = (uint32_t)rsk;
  const float c = p.c_log2;
  // query-side document bases of head 0; a head adds head * d elements
  const size_t docq = (size_t)s_d * rs;
  const uint8_t* q_doc = a.q_codes + docq;
  const uint8_t* do_doc = a.do_codes + docq;
  const uint8_t* g_doc = reinterpret_cast<const uint8_t*>(a.g + docq);
  uint8_t* dq_doc = reinterpret_cast<uint8_t*>(a.dq_acc + docq);

  // ---- item start: K~ and V~ tiles (128 rows), swizzled code layout; the
  // per-key V~ codes too (rows past the document end repeat its last row, as
  // in the other tiles: their P and dS are masked to zero)
  {
    constexpr int NI = BWD_BK * D / 1024;
    constexpr int NTILE = EXACT ? 2 : 3;
    for (int i = wave; i < NTILE * NI; i += 8) {
      const int ti = i / NI, ii = i % NI;
      const int o = ii * 1024 + 16 * lane;
      const int r = o / D, slot = (o % D) >> 4;
      const uint32_t off = (uint32_t)min(k0 + r, L - 1) * rsk32 + 16u * (uint32_t)(slot ^ code_key<D>(r));
      dma16((ti == 0 ? a.k_codes : ti == 1 ? a.v_codes : a.v_key_codes) + doc0k + off,
            (ti == 0 ? sK : ti == 1 ? sV : sVk) + ii * 1024);
    }
  }
  // ---- query tiles: code instruction `wave` (if any), bf16 instructions wave + 8 k, plane `wave`
  constexpr int NIC = CT / 1024;              // code-tile instructions (8 or 4)
  constexpr int NIW = WT / 1024 / 8;          // bf16-tile instructions per wave (2 or 1)
  const bool has_c = wave < NIC;
  uint32_t crow = 0, ccol = 0, wrow[NIW], wcol[NIW];
  {
    const int o = wave * 1024 + 16 * lane;
    crow = (uint32_t)(o / D) * rs32;
    ccol = 16u * (uint32_t)(((o % D) >> 4) ^ code_key<D>(o / D));
  }
#pragma unroll
  for (int k = 0; k < NIW; ++k) {
    const int o = (wave + 8 * k) * 1024 + 16 * lane;
    const int r = o / (2 * D), slot = (o % (2 * D)) >> 4;
    wrow[k] = 2u * (uint32_t)r * rs32;
    wcol[k] = 16u * (uint32_t)(slot ^ wide_key<D>(r));
  }
  const uint32_t last_c = (uint32_t)(L - 1) * rs32, last_w = 2u * last_c;
  const int* const plane = (wave == 0 ? a.kofs
                          : wave == 1 ? reinterpret_cast<const int*>(a.il8)
                          : wave == 2 ? reinterpret_cast<const int*>(a.delta)
                          : wave == 3 ? a.dq_sigma : a.qexps) + s_d;
  // query tile qt of query head h
  auto issue_tile = [&](auto Bc, int qt, int h) {
    constexpr int B = decltype(Bc)::value;
    const int q0 = qt * BWD_BQ;
    const uint32_t q0c = (uint32_t)q0 * rs32, q0w = 2u * q0c;
    const uint32_t hd = (uint32_t)h * D;
    if (has_c) {
      const uint32_t off = min(q0c + crow, last_c) + ccol + hd;
      dma16(q_doc + off, (B ? sQ1 : sQ0) + wave * 1024);
      dma16(do_doc + off, (B ? sO1 : sO0) + wave * 1024);
    }
#pragma unroll
    for (int k = 0; k < NIW; ++k)
      dma16(g_doc + (min(q0w + wrow[k], last_w) + wcol[k] + 2u * hd), (B ? sG1 : sG0) + (wave + 8 * k) * 1024);
    if (wave < NPLANES) dma4(plane + (size_t)h * T + min(q0 + lane, L - 1), (B ? sR1 : sR0) + wave * BWD_BQ * 4);
  };

  const int qt_first = CAUSAL ? k0 / BWD_BQ : 0;
  const int qt_end = (L + BWD_BQ - 1) / BWD_BQ;
  issue_tile(std::integral_constant<int, 0>{}, qt_first, h_first);
  if (tid < 4) sKeB[tid] = k0 + 32 * tid < L ? (int)a.k_exp[hTk + k0 + 32 * tid] : E8M0_BIAS;
  if (EXACT && tid >= 4 && tid < 8) sVrB[tid - 4] = a.v_ref_exp[hTk + min(k0 + 32 * (tid - 4) + 31, L - 1)];
  int ke, ve, vke;
  {
    const size_t mi = hTk + min(j, L - 1);
    ke = a.k_exp[mi];
    ve = a.v_exp[mi];
    vke = a.v_key_exp[mi];
  }
  const int e_key = vke - E8M0_BIAS;
  full_barrier();

  // per-lane LDS offsets (loop-invariant)
  const int ck = code_key<D>(n);
  // row n of the wave's query block (Q~, dO~) and key block (K~, V~), chunks 4s + hh and
  // 4s + 2 + hh, as byte offsets from the tile's start (the tile is then the read's
  // constant offset).  The FMA-pipe exp2 and exact instantiations have no registers to
  // spare for the second array: there the block bases are added at each read
  constexpr bool FOLD = !POLY && !EXACT;
  const int qb0 = FOLD ? 0 : 32 * qh * D, kb0 = FOLD ? 0 : 32 * kb * D;
  int offQ2[NS][2], offK2[NS][2];
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int o = n * D + (((4 * s2 + 2 * e + hh) ^ ck) << 4);
      offQ2[s2][e] = (FOLD ? 32 * qh * D : 0) + o;
      offK2[s2][e] = (FOLD ? 32 * kb * D : 0) + o;
    }
  int offK[NDK];                   // 8-bit transpose reads of the Q~ tile (dK operand), this wave's half of d
  {
    const int pp = lane & 15, b = pp >> 1;
    const int t = 8 * (b >> 2) + 4 * hh + (b & 3);
#pragma unroll
    for (int e = 0; e < NDK; ++e) offK[e] = code_off<D>(t, 32 * (NDK * qh + e) + colg + 8 * (pp & 1));
  }
  int offG[ND][2];                 // 16-bit transpose reads of the G tile (dV operand)
  {
    const int pp = lane & 15, e = pp >> 2, s4 = pp & 3;
    const int t = 4 * hh + e;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      offG[db][0] = wide_off<D>(t, 2 * (32 * db + colg + 4 * s4));
      offG[db][1] = wide_off<D>(t + 8, 2 * (32 * db + colg + 4 * s4));
    }
  }

  // dQ^T: wave -> (d slice, query block); d = 64 uses waves 0-3 only
  const bool dq_wave = D == 128 || wave < 4;
  const int dq_ds = D == 128 ? wave & 3 : wave & 1;
  const int dq_qb = D == 128 ? wave >> 2 : (wave >> 1) & 1;
  // dS^ operand of dQ^T: the lane's 16-lane group reads chunk dq_qb + 2 grp
  // (query half dq_qb, writer lane half grp); column n is query iq
  int offQ;
  {
    const int pp = lane & 15, b = pp >> 1;
    offQ = dsk_off(8 * (b >> 2) + 4 * hh + (b & 3), dq_qb + 2 * ((lane >> 4) & 1)) + 8 * (pp & 1);
  }

  v16f dk[NDK], dv[ND];
  uint32_t ds_nz = 0, ds_zero = 0;       // diagnostic counts of this lane
#pragma unroll
  for (int e = 0; e < NDK; ++e) dk[e] = v16f{};
#pragma unroll
  for (int db = 0; db < ND; ++db) dv[db] = v16f{};

  // fp16 dQ partial of query tile qtp -> memory-side atomics; rows wave, wave + 8, ...
  constexpr int RPI = 128 / D;                       // rows per wave instruction
  const int frow = RPI == 1 ? 0 : lane >> 5;
  const int fpair = RPI == 1 ? lane : lane & 31;
  const uint16_t* const fsrc = reinterpret_cast<const uint16_t*>(sKQ) + frow * DQS + 2 * fpair;
  const uint32_t fdst = 2u * (uint32_t)frow * rs32 + 4u * (uint32_t)fpair;
  // deterministic mode: plain stores into the step's own partial slot instead
  const int nq_doc = (L + BWD_BQ - 1) / BWD_BQ;
  auto flush_dq = [&](int qtp, int h) {
    constexpr int NIT = BWD_BQ / (8 * RPI);
    const int q0p = qtp * BWD_BQ;
    const int nqp = min(BWD_BQ, L - q0p);
    v2h hv[NIT];
#pragma unroll
    for (int t2 = 0; t2 < NIT; ++t2) {
      const int row0 = RPI * (wave + 8 * t2);        // rows row0 + frow share bit 4
      hv[t2] = *reinterpret_cast<const v2h*>(fsrc + stage_row(row0) * DQS);
    }
    if constexpr (DET) {
      const long long step = det_step(a.det_base[doc], u, qtp, nq_doc, CAUSAL);
      if (step >= a.det_cap) return;      // the plan flags the overflow
      uint8_t* const slot = reinterpret_cast<uint8_t*>(a.dq_part) + ((size_t)step * H + h) * (BWD_BQ * D * 2);
#pragma unroll
      for (int t2 = 0; t2 < NIT; ++t2) {
        const int row0 = RPI * (wave + 8 * t2);
        // non-temporal: the partials are read back only by the finaliser, so
        // they must not evict the query tiles later items re-read from L2
        __builtin_nontemporal_store(__builtin_bit_cast(uint32_t, hv[t2]),
                                    reinterpret_cast<uint32_t*>(slot + (row0 + frow) * (D * 2) + 4 * fpair));
      }
      return;
    }
#pragma unroll
    for (int t2 = 0; t2 < NIT; ++t2) {
      const int row0 = RPI * (wave + 8 * t2);        // uniform
      if (row0 + frow < nqp)
        __builtin_amdgcn_global_atomic_fadd_v2f16(
            reinterpret_cast<v2h*>(dq_doc + (2u * (uint32_t)(q0p + row0) * rs32 + fdst + 2u * (uint32_t)h * D)), hv[t2]);
    }
  };

  auto step = [&](auto Bc, int qt, int h) {
    constexpr int B = decltype(Bc)::value;
    const uint8_t* tQ = B ? sQ1 : sQ0;
    const uint8_t* tdO = B ? sO1 : sO0;
    const uint8_t* tG = B ? sG1 : sG0;
    const uint8_t* tR = B ? sR1 : sR0;
    const int* pko = reinterpret_cast<const int*>(tR);
    const float* pil = reinterpret_cast<const float*>(tR + BWD_BQ * 4);
    const float* pdl = reinterpret_cast<const float*>(tR + 2 * BWD_BQ * 4);
    const int* psig = reinterpret_cast<const int*>(tR + 3 * BWD_BQ * 4);
    const int* pqx = reinterpret_cast<const int*>(tR + 4 * BWD_BQ * 4);
    const int q0 = qt * BWD_BQ;
    const int nq = min(BWD_BQ, L - q0);
    const int QB = 2 * qt + qh;
    const bool act = kb_active && (!CAUSAL || QB >= KB) && 32 * qh < nq;
    const bool dia = QB == KB;
    const bool pol = POLY && poly_block(QB, KB);   // the forward's choice for this block
    // no mask (and, but for the exact option, no fold); without the causal
    // mask a block may also hold keys past the document end
    const bool fast = !dia && 32 * qh + 32 <= nq && (CAUSAL || k0 + 32 * kb + 32 <= L);
    int dsc[4] = {0, 0, 0, 0};
    int eds = -127;
    v16f sacc, pacc;     // set (and read) only when act
    if (act) {
      // dP accumulates onto -D (the plane holds -D), so the product yields dP - D directly
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4f dlv = *reinterpret_cast<const v4f*>(pdl + 32 * qh + 8 * g + 4 * hh);
#pragma unroll
        for (int r = 0; r < 4; ++r) pacc[4 * g + r] = dlv[r];
      }
      // exact option: each row's own exponent (lane n supplies row n's scale)
      const int qx = pqx[32 * qh + (EXACT ? n : 0)];
      const int sqe = qx & 255, sdoe = (qx >> 8) & 255;
      auto s_step = [&](int s) {
        const v8i qa = cat8(ld16(tQ + qb0 + offQ2[s][0]), ld16(tQ + qb0 + offQ2[s][1]));
        const v8i kb8 = cat8(ld16(sK + kb0 + offK2[s][0]), ld16(sK + kb0 + offK2[s][1]));
        sacc = s == 0 ? mfma_f8(qa, kb8, v16f{}, sqe, ke) : mfma_f8(qa, kb8, sacc, sqe, ke);
      };
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        s_step(s);
        // diagonal block: per-key V~ codes
        pacc = mfma_f8(cat8(ld16(tdO + qb0 + offQ2[s][0]), ld16(tdO + qb0 + offQ2[s][1])),
                       (!EXACT && dia) ? cat8(ld16(sVk + kb0 + offK2[s][0]), ld16(sVk + kb0 + offK2[s][1]))
                                       : cat8(ld16(sV + kb0 + offK2[s][0]), ld16(sV + kb0 + offK2[s][1])), pacc,
                       sdoe, (!EXACT && dia) ? vke : ve);
      }
    }
    // the next tile streams in while this one is computed; last step's dQ
    // goes out (steps run over the query tiles of one head, then the next head)
    if constexpr (GRP) {
      const bool wrap = qt + 1 >= qt_end;
      const int nh = wrap ? h + 1 : h;
      if (nh < h_end) issue_tile(std::integral_constant<int, 1 - B>{}, wrap ? qt_first : qt + 1, nh);
      const bool first = qt == qt_first;
      const int ph = first ? h - 1 : h;
      if (ph >= h_first) flush_dq(first ? qt_end - 1 : qt - 1, ph);
    } else {
      if (qt + 1 < qt_end) issue_tile(std::integral_constant<int, 1 - B>{}, qt + 1, h);
      if (qt > qt_first) flush_dq(qt - 1, h);
    }
    if (act) {
      float dsv[16];
      uint32_t pe[8];      // bf16 pairs of P^_eff * 2^8, accumulator register order
      float amax = 0.f;
      if (fast) {
        // exact option: the lane's key folds against its block's largest V
        // exponent; the fold is a constant per lane here
        const int fd = EXACT ? e_key - (sVrB[kb] - E8M0_BIAS) : 0;
        const float ufd = __builtin_amdgcn_ldexpf(1.0f, -fd);
        // the block's rows as one straight-line body per probability form
        // (fast where every row of the query block allows it)
        auto rows = [&](auto PW, auto PL) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = 32 * qh + 8 * g + 4 * hh;
          const v4i kov = *reinterpret_cast<const v4i*>(pko + r0);
          const v4f ilv = *reinterpret_cast<const v4f*>(pil + r0);
          float pf[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)        // P 2^8
            pf[r] = decltype(PW)::value
                        ? __builtin_amdgcn_ldexpf(exp2_p<decltype(PL)::value>(sacc[4 * g + r] * c), kov[r])
                        : p_scaled<decltype(PL)::value>(sacc[4 * g + r] * c, kov[r]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rr = 4 * g + r;
            dsv[rr] = (pf[r] * ilv[r]) * pacc[rr];
            amax = fmaxf(amax, fabsf(dsv[rr]));
          }
          const int code = EXACT ? cvt_fp8x4(__builtin_amdgcn_ldexpf(pf[0], fd), __builtin_amdgcn_ldexpf(pf[1], fd),
                                             __builtin_amdgcn_ldexpf(pf[2], fd), __builtin_amdgcn_ldexpf(pf[3], fd))
                                 : cvt_fp8x4(pf[0], pf[1], pf[2], pf[3]);
          if constexpr (DIAG) {
            if (a.dump != nullptr && j < a.dump_len) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                a.dump[((size_t)h * T + s_d + q0 + r0 + r) * a.dump_len + j] = (uint8_t)((code >> (8 * r)) & 255);
            }
          }
          pe[2 * g] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, EXACT ? ufd : 1.0f, false));
          pe[2 * g + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, EXACT ? ufd : 1.0f, true));
        }
        };
        auto rows_pw = [&](auto PW) {
          if (POLY && pol) rows(PW, std::integral_constant<bool, POLY>{});
          else rows(PW, std::false_type{});
        };
        if ((__builtin_amdgcn_readfirstlane(pqx[32 * qh]) >> 24) & 1)
          rows_pw(std::true_type{});
        else
          rows_pw(std::false_type{});
      } else if (!EXACT && ((__builtin_amdgcn_readfirstlane(pqx[32 * qh]) >> 24) & 1)) {
        // a diagonal or ragged block whose rows all take the fast form: the
        // mask as a select (0 for what the query does not see) and, on the
        // diagonal, each row's V fold as exact ldexps around the convert --
        // the values and codes of the per-score form below.  Row 8 g + r of
        // the lane (query q0 + 32 qh + 8 g + 4 hh + r) sees the lane's key
        // when lo <= 8 g + r < hi
        const int qrow0 = q0 + 32 * qh + 4 * hh;
        const int lo = CAUSAL ? j - qrow0 : 0;
        const int hi = kv ? L - qrow0 : 0;
        auto rows_m = [&](auto PL) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int r0 = 32 * qh + 8 * g + 4 * hh;
            const v4i kov = *reinterpret_cast<const v4i*>(pko + r0);
            const v4f ilv = *reinterpret_cast<const v4f*>(pil + r0);
            const v4i qxv = *reinterpret_cast<const v4i*>(pqx + r0);
            float xf[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int rr = 4 * g + r;
              const bool vis = 8 * g + r >= lo && 8 * g + r < hi;
              const float p8 = __builtin_amdgcn_ldexpf(exp2_p<decltype(PL)::value>(sacc[rr] * c), kov[r]);
              const float dsr = vis ? (p8 * ilv[r]) * pacc[rr] : 0.f;
              dsv[rr] = dsr;
              amax = fmaxf(amax, fabsf(dsr));
              const float pv = vis ? p8 : 0.f;
              xf[r] = dia ? __builtin_amdgcn_ldexpf(pv, e_key - (((qxv[r] >> 16) & 255) - E8M0_BIAS)) : pv;
            }
            const int code = cvt_fp8x4(xf[0], xf[1], xf[2], xf[3]);
            if constexpr (DIAG) {
              if (a.dump != nullptr && j < a.dump_len) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (8 * g + r >= lo && 8 * g + r < hi)
                    a.dump[((size_t)h * T + s_d + q0 + r0 + r) * a.dump_len + j] = (uint8_t)((code >> (8 * r)) & 255);
              }
            }
            if (dia) {
              float pf[4];
#pragma unroll
              for (int r = 0; r < 4; ++r)
                pf[r] = __builtin_amdgcn_ldexpf(fp8_value(code, r), (((qxv[r] >> 16) & 255) - E8M0_BIAS) - e_key);
              pe[2 * g] = (uint32_t)f32_to_bf16_bits(pf[0]) | ((uint32_t)f32_to_bf16_bits(pf[1]) << 16);
              pe[2 * g + 1] = (uint32_t)f32_to_bf16_bits(pf[2]) | ((uint32_t)f32_to_bf16_bits(pf[3]) << 16);
            } else {
              pe[2 * g] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, false));
              pe[2 * g + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, true));
            }
          }
        };
        if (POLY && pol) rows_m(std::integral_constant<bool, POLY>{});
        else rows_m(std::false_type{});
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = 32 * qh + 8 * g + 4 * hh;
          const v4i kov = *reinterpret_cast<const v4i*>(pko + r0);
          const v4f ilv = *reinterpret_cast<const v4f*>(pil + r0);
          float pf[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rr = 4 * g + r;
            const int i = q0 + r0 + r;
            float dsr = 0.f, pev = 0.f;
            if (kv && (!CAUSAL || j <= i) && i < L) {
              const float x = sacc[rr] * c;
              const float p8 = (POLY && pol) ? p_scaled<POLY>(x, kov[r]) : p_scaled(x, kov[r]);
              dsr = (p8 * ilv[r]) * pacc[rr];
              int code;
              if (EXACT || dia) {
                const int vref = (EXACT && !dia) ? sVrB[kb] - E8M0_BIAS : ((pqx[r0 + r] >> 16) & 255) - E8M0_BIAS;
                code = cvt_fp8x2(__builtin_amdgcn_ldexpf(p8, e_key - vref), 0.f);
                pev = __builtin_amdgcn_ldexpf(fp8_value(code, 0), vref - e_key);
              } else {
                code = cvt_fp8x2(p8, 0.f);
                pev = fp8_value(code, 0);
              }
              if constexpr (DIAG) {
                if (a.dump != nullptr && j < a.dump_len)
                  a.dump[((size_t)h * T + s_d + i) * a.dump_len + j] = (uint8_t)(code & 255);
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
      if constexpr (EXACT) {
        // dQ payload: K's per-token exponent of the lane's key folded in, one
        // exponent per query row over this block's 32 keys (the lanes of a half)
        const int ekf = ke - E8M0_BIAS;
        int dqc[4];
        {
          float av[16];
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) av[rr] = fabsf(__builtin_amdgcn_ldexpf(dsv[rr], ekf));
          // each row's maximum lands in lanes 2 r, 2 r + 1 of the half; its
          // exponent goes to the table the dQ product reads, and every lane
          // reads back the exponents of its 16 rows (four bytes per dword)
          const int rw = n >> 1;
          const int er = roundup_exp(rows_max16(av, n));
          if (!(n & 1)) sRowE[kb][32 * qh + 8 * (rw >> 2) + 4 * hh + (rw & 3)] = (uint8_t)(er + E8M0_BIAS);
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int e4 = *reinterpret_cast<const int*>(&sRowE[kb][32 * qh + 8 * g + 4 * hh]);
            float xq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              xq[r] = __builtin_amdgcn_ldexpf(dsv[4 * g + r], ekf - (((e4 >> (8 * r)) & 255) - E8M0_BIAS));
            dqc[g] = cvt_fp8x4(xq[0], xq[1], xq[2], xq[3]);
          }
        }
        st16(sdSQ + dsk_off(32 * kb + n, 2 * hh + qh), v4i{dqc[0], dqc[1], dqc[2], dqc[3]});
        // dK payload: Q's per-token exponent of each row folded in, one exponent
        // per key (lane) over the wave's 32 queries (both halves)
        auto eq = [&](int rr) { return (pqx[32 * qh + 8 * (rr >> 2) + 4 * hh + (rr & 3)] & 255) - E8M0_BIAS; };
        float mk = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mk = fmaxf(mk, fabsf(__builtin_amdgcn_ldexpf(dsv[rr], eq(rr))));
        mk = fmaxf(mk, __shfl_xor(mk, 32, 64));
        const int ec = roundup_exp(mk);
        if (hh == 0) sColE[qh][32 * kb + n] = (uint8_t)(ec + E8M0_BIAS);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          dsc[g] = cvt_fp8x4(__builtin_amdgcn_ldexpf(dsv[4 * g], eq(4 * g) - ec),
                             __builtin_amdgcn_ldexpf(dsv[4 * g + 1], eq(4 * g + 1) - ec),
                             __builtin_amdgcn_ldexpf(dsv[4 * g + 2], eq(4 * g + 2) - ec),
                             __builtin_amdgcn_ldexpf(dsv[4 * g + 3], eq(4 * g + 3) - ec));
      } else {
      // amax >= 0, so its bits order like the values; the exponent is the
      // same in every lane, so the rare branch below is a scalar branch
      const int e = __builtin_amdgcn_readfirstlane(roundup_exp(__int_as_float(wave_max_i(__float_as_int(amax)))));
      eds = e;
      if (e >= -126) {
        const float sc2 = __builtin_amdgcn_ldexpf(1.0f, e);    // the convert divides by it
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // (the first convert's other half is overwritten by the second)
          v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, dsv[4 * g]), dsv[4 * g],
                                                          dsv[4 * g + 1], sc2, false);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, dsv[4 * g + 2], dsv[4 * g + 3], sc2, true);
          dsc[g] = __builtin_bit_cast(int, w);
        }
      } else {
        // e = -127 (2^e is no normal fp32 scale): kept out of line -- the
        // empty volatile statement stops the compiler from evaluating this
        // branch on every step
        asm volatile("");
#pragma unroll
        for (int g = 0; g < 4; ++g)
          dsc[g] = cvt_fp8x4(__builtin_amdgcn_ldexpf(dsv[4 * g], -e), __builtin_amdgcn_ldexpf(dsv[4 * g + 1], -e),
                             __builtin_amdgcn_ldexpf(dsv[4 * g + 2], -e), __builtin_amdgcn_ldexpf(dsv[4 * g + 3], -e));
      }
      }
      if constexpr (DIAG) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const bool nz = dsv[rr] != 0.f;      // masked and out-of-range entries are exactly 0
          ds_nz += nz;
          ds_zero += nz && ((dsc[rr >> 2] >> (8 * (rr & 3))) & 0x7f) == 0;
        }
      }
      // dV += P^_eff^T G over this wave's 32 queries (two K-steps of 16)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const v8bf av = __builtin_bit_cast(
            v8bf, v4i{(int)pe[4 * ks], (int)pe[4 * ks + 1], (int)pe[4 * ks + 2], (int)pe[4 * ks + 3]});
        const uint8_t* g0 = tG + (32 * qh + 16 * ks) * 2 * D;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const v4s lo = lds_tr16(g0 + offG[db][0]);
          const v4s hi = lds_tr16(g0 + offG[db][1]);
          dv[db] = mfma_bf16(av, __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)),
                             dv[db]);
        }
      }
    }
    if (EXACT && !act) {     // zero codes; any finite scale
      st16(sdSQ + dsk_off(32 * kb + n, 2 * hh + qh), v4i{0, 0, 0, 0});
      if (n < 16) sRowE[kb][32 * qh + 8 * (n >> 2) + 4 * hh + (n & 3)] = (uint8_t)E8M0_BIAS;
      if (hh == 0) sColE[qh][32 * kb + n] = (uint8_t)E8M0_BIAS;
    }
    // dS^ to LDS key-major: row = key, one 16-byte chunk per lane
    st16(sdSK + dsk_off(32 * kb + n, 2 * hh + qh), v4i{dsc[0], dsc[1], dsc[2], dsc[3]});
    if (lane == 0) sEds[qh][kb] = eds;
    lds_barrier();
    // dK += dS^^T Q~ over the 64 queries, this wave's half of d; lane half hh
    // carries query block hh
    if (kb_active) {
      // K-block 0 = query half 0 (chunk 2 hh), K-block 1 = query half 1 (chunk 2 hh + 1)
      const v8i adk = cat8(ld16(sdSK + dsk_off(32 * kb + n, 2 * hh)), ld16(sdSK + dsk_off(32 * kb + n, 2 * hh + 1)));
      const int sa = EXACT ? (int)sColE[hh][32 * kb + n] : sEds[hh][kb] + E8M0_BIAS;
      const int sb = EXACT ? E8M0_BIAS : pqx[32 * hh] & 255;
#pragma unroll
      for (int e = 0; e < NDK; ++e) {
        const uint8_t* qp = tQ + offK[e];
        const v2i a0 = lds_tr8(qp), a1 = lds_tr8(qp + 16 * D), a2 = lds_tr8(qp + 32 * D), a3 = lds_tr8(qp + 48 * D);
        dk[e] = mfma_f8(adk, v8i{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]}, dk[e], sa, sb);
      }
    }
    // dQ^T slice: rows d in [32 ds, 32 ds + 32), columns = queries of block dq_qb, K = 128 keys
    if (dq_wave && 32 * dq_qb < nq) {
      v16f acc = v16f{};
      const int iq = 32 * dq_qb + 8 * ((n & 15) >> 2) + 4 * ((lane >> 4) & 1) + (n & 3);
      // the dQ prescale of this query block (one value per block but for the
      // exact option, whose prescale is per token)
      const int dq_sig = EXACT ? 0 : __builtin_amdgcn_readfirstlane(psig[32 * dq_qb]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint8_t* b0 = (EXACT ? sdSQ : sdSK) + 64 * 64 * ks + offQ;
        const v2i l0 = lds_tr8(b0), h0 = lds_tr8(b0 + 16 * 64), l1 = lds_tr8(b0 + 32 * 64), h1 = lds_tr8(b0 + 48 * 64);
        const v8i bq = v8i{l0[0], l0[1], h0[0], h0[1], l1[0], l1[1], h1[0], h1[1]};
        const v8i kt = cat8(tr_code16<D>(sK, 64 * ks, 32 * dq_ds + colg, lane),
                            tr_code16<D>(sK, 64 * ks + 32, 32 * dq_ds + colg, lane));
        if constexpr (EXACT) {
          acc = mfma_f8(kt, bq, acc, E8M0_BIAS, sRowE[2 * ks + hh][iq]);
        } else {
          // the prescale 2^-sigma rides in the operands' scales: sigma is one
          // value per 32-query block here.  Only the sum of the two E8M0 bytes
          // matters, so what would leave the dS byte's finite range [0, 254]
          // moves to the K byte; a sum still below 0 scales the product (at
          // most 2^24 in magnitude) below 2^-230, zero in fp16 either way
          int kb = sKeB[2 * ks + hh], sb = sEds[dq_qb][2 * ks + hh] + E8M0_BIAS - dq_sig;
          if (sb < 0) {
            kb += sb;
            sb = 0;
          } else if (sb > 254) {
            kb += sb - 254;
            sb = 254;
          }
          acc = mfma_f8(kt, bq, acc, min(max(kb, 0), 254), sb);
        }
      }
      const int sig = EXACT ? psig[iq] : 0;
      uint16_t* dst = reinterpret_cast<uint16_t*>(sKQ) + stage_row(iq) * DQS + 32 * dq_ds + 4 * hh;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v2h h0, h1;
        if constexpr (EXACT) {
          h0[0] = (_Float16)__builtin_amdgcn_ldexpf(acc[4 * g], -sig);
          h0[1] = (_Float16)__builtin_amdgcn_ldexpf(acc[4 * g + 1], -sig);
          h1[0] = (_Float16)__builtin_amdgcn_ldexpf(acc[4 * g + 2], -sig);
          h1[1] = (_Float16)__builtin_amdgcn_ldexpf(acc[4 * g + 3], -sig);
        } else {
          h0[0] = (_Float16)acc[4 * g];
          h0[1] = (_Float16)acc[4 * g + 1];
          h1[0] = (_Float16)acc[4 * g + 2];
          h1[1] = (_Float16)acc[4 * g + 3];
        }
        *reinterpret_cast<v2i*>(dst + 8 * g) = v2i{__builtin_bit_cast(int, h0), __builtin_bit_cast(int, h1)};
      }
    }
    // the next tile has landed, this step's dQ partial is staged, the
    // previous step's atomics are done
    full_barrier();
  };

  if constexpr (GRP) {
    for (int qt = qt_first, h = h_first;;) {
      step(std::integral_constant<int, 0>{}, qt, h);
      if (++qt >= qt_end) { qt = qt_first; if (++h >= h_end) break; }
      step(std::integral_constant<int, 1>{}, qt, h);
      if (++qt >= qt_end) { qt = qt_first; if (++h >= h_end) break; }
    }
  } else {
    for (int qt = qt_first;;) {
      step(std::integral_constant<int, 0>{}, qt, h_first);
      if (++qt >= qt_end) break;
      step(std::integral_constant<int, 1>{}, qt, h_first);
      if (++qt >= qt_end) break;
    }
  }
  flush_dq(qt_end - 1, h_end - 1);
  if constexpr (DIAG) {
    if (a.ds_counts != nullptr) {
      unsigned long long nz = ds_nz, zr = ds_zero;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        nz += __shfl_xor(nz, off, 64);
        zr += __shfl_xor(zr, off, 64);
      }
      if (lane == 0) {
        atomicAdd(a.ds_counts, nz);
        atomicAdd(a.ds_counts + 1, zr);
      }
    }
  }

  // split groups: this item's part (recomputed here rather than kept live)
  const int GS = GRP ? a.gsplit : 1, part = GRP ? (int)(blockIdx.x % GS) : 0;
  // ---- item end: the two query-half dV partials of each key block meet in
  // the (now free) bf16 tile buffers, key blocks 0-1 first, then 2-3, the
  // sums staying in the registers of the query-half-0 waves; then dK
  for (int round = 0; round < 2; ++round) {
    const bool mine = (kb >> 1) == round;
    // chunk-major: chunk 4 db + q4 of every lane side by side (each
    // instruction moves 1 KB without bank conflicts)
    float* red = reinterpret_cast<float*>((kb & 1) ? sG1 : sG0) + 4 * lane;
    if (mine && qh == 1) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<v4f*>(red + 256 * (4 * db + q4)) =
              v4f{dv[db][4 * q4], dv[db][4 * q4 + 1], dv[db][4 * q4 + 2], dv[db][4 * q4 + 3]};
    }
    __syncthreads();
    if (mine && qh == 0 && kb_active) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const v4f o = *reinterpret_cast<const v4f*>(red + 256 * (4 * db + q4));
#pragma unroll
          for (int r = 0; r < 4; ++r) dv[db][4 * q4 + r] = dv[db][4 * q4 + r] + o[r];
          if (GS != 1) {     // split groups: fp32 partials of this part
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int jk = k0 + 32 * kb + 8 * q4 + 4 * hh + r;
              if (jk < L)
                a.dv_f32[(size_t)part * T * rsk + doc0k + (size_t)jk * rsk + 32 * db + n] = dv[db][4 * q4 + r];
            }
          }
        }
    }
    __syncthreads();
  }
  // dV as bf16 into a key-major tile per key block (the free query code
  // buffers, 2d bytes a row), its 16-byte chunks XOR-swizzled by row so that
  // the column writes here and the row-quarter reads below are free of bank
  // conflicts
  auto dvt = [&](int b) { return b == 0 ? sQ0 : b == 1 ? sQ1 : b == 2 ? sO0 : sO1; };
  static_assert(32 * 2 * D <= CT, "a key block of bf16 dV fits one query code buffer");
  auto dv_off = [](int row, int dcol) {        // byte offset of (row, d) in a key block's tile
    const int sw = D == 128 ? (row & 7) : (((row >> 1) & 1) | (((row >> 2) & 1) << 2));
    return row * (2 * D) + (((dcol >> 3) ^ sw) << 4) + 2 * (dcol & 7);
  };
  if (GS == 1 && qh == 0 && kb_active) {
    uint8_t* const t = dvt(kb);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        *reinterpret_cast<uint16_t*>(t + dv_off(8 * (rr >> 2) + 4 * hh + (rr & 3), 32 * db + n)) =
            f32_to_bf16_bits(dv[db][rr]);
  }
  // fp32 dK tile index of (row, d): 16-byte chunks XOR-swizzled by row (and,
  // d = 128, by the chunk's upper half) so that both the column writes below
  // and the row-quarter reads are free of bank conflicts
  auto dk_idx = [](int row, int col) {
    const int ch = col >> 2;
    const int sw = (row & 3) | (((row >> 2) & 1) << 3) | (D == 128 ? ((ch >> 4) & 1) << 2 : 0);
    return row * D + ((ch ^ sw) << 2) + (col & 3);
  };
  // dK times the softmax scale into a key-major fp32 tile (key block kb in
  // one free buffer, 32 rows of d), then four lanes per key row rotate it
  // back (Hadamard option) with the same butterflies as the dQ finaliser and
  // store bf16 rows
  {
    float* const tile = reinterpret_cast<float*>(kb == 0 ? sK : kb == 1 ? sV : kb == 2 ? sG0 : sG1);
    static_assert(BWD_BK / 4 * D * 4 <= BWD_BK * D && BWD_BK / 4 * D * 4 <= WT, "a key block of fp32 dK fits one buffer");
    const float sc = p.softmax_scale;
#pragma unroll
    for (int e = 0; e < NDK; ++e)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        tile[dk_idx(8 * (rr >> 2) + 4 * hh + (rr & 3), 32 * (NDK * qh + e) + n)] = dk[e][rr] * sc;
  }
  __syncthreads();
  {
    constexpr int E = D / 4;
    const int row = tid >> 2, q4p = tid & 3;          // 128 key rows, four lanes each
    const int jk = k0 + row;
    if (jk < L) {                                     // whole quads leave together
      const int rb = row >> 5;
      const float* const src = reinterpret_cast<const float*>(rb == 0 ? sK : rb == 1 ? sV : rb == 2 ? sG0 : sG1);
      if (GS == 1) {
        float x[E];
#pragma unroll
        for (int c = 0; c < E / 4; ++c) {
          const v4f w = *reinterpret_cast<const v4f*>(src + dk_idx(row & 31, q4p * E + 4 * c));
#pragma unroll
          for (int k = 0; k < 4; ++k) x[4 * c + k] = w[k];
        }
        if (p.hadamard) fwht_quarter_row<D>(x, q4p);
        store_bf16<E>(a.dk + doc0k + (size_t)jk * rsk + q4p * E, x);
        // this row quarter of dV: E bf16 = E / 8 chunks
        const uint8_t* const vt = dvt(rb);
#pragma unroll
        for (int c = 0; c < E / 8; ++c)
          st16(a.dv + doc0k + (size_t)jk * rsk + q4p * E + 8 * c,
               *reinterpret_cast<const v4i*>(vt + dv_off(row & 31, q4p * E + 8 * c)));
      } else {
        float* dst = a.dk_f32 + (size_t)part * T * rsk + doc0k + (size_t)jk * rsk + q4p * E;
#pragma unroll
        for (int c = 0; c < E / 4; ++c)
          *reinterpret_cast<v4f*>(dst + 4 * c) = *reinterpret_cast<const v4f*>(src + dk_idx(row & 31, q4p * E + 4 * c));
      }
    }
  }
}

// Clears n 64-bit counters (a kernel rather than a memset, so a captured
// graph replays it correctly).
__global__ void zero_u64_kernel(unsigned long long* x, int n) {
  if ((int)threadIdx.x < n) x[threadIdx.x] = 0ull;
}

hipError_t launch_attn_bwd(const Problem& p, const void* plan, const PlanLayout& pl, const BwdInputs& in,
                           hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const char* base = static_cast<const char*>(plan);
  // items in the dispatch order (the backward list grouped by document)
  BwdArgs a{p, reinterpret_cast<const int*>(base), reinterpret_cast<const int2*>(base + pl.disp_offset),
            in.q_codes, in.k_codes, in.v_codes, in.v_key_codes, in.k_exp, in.v_exp, in.v_key_exp,
            in.kofs, in.il8, in.delta, in.dq_sigma, in.qexps, in.do_codes,
            static_cast<const uint16_t*>(in.g), static_cast<uint16_t*>(in.dq_acc), in.dk_f32,
            static_cast<uint16_t*>(in.dk), static_cast<uint16_t*>(in.dv), in.dv_f32, in.gsplit,
            static_cast<uint16_t*>(in.dq_part), in.det_base, in.det_cap, in.v_ref_exp, static_cast<const uint16_t*>(in.q_x),
            static_cast<const uint16_t*>(in.k_x), in.qk_scale, in.dump, in.dump_len, in.ds_counts};
  dim3 grid((unsigned)pl.cap_bwd * (unsigned)p.Hk * (unsigned)in.gsplit);   // the mixed path has Hk = H, gsplit = 1
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(BWD_THREADS), 0, stream, a); };
  if (p.path == 1) {
    if (p.causal) {
      if (p.D == 64) go(attn_bwd_kernel<64, 1, true>); else go(attn_bwd_kernel<128, 1, true>);
    } else {
      if (p.D == 64) go(attn_bwd_kernel<64, 1, false>); else go(attn_bwd_kernel<128, 1, false>);
    }
  } else if (in.diag) {
    // diagnostic instantiation: MXFP8, one head per item, causal, atomic dQ
    if (in.ds_counts != nullptr)
      hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(64), 0, stream, in.ds_counts, 2);
    auto go8 = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(2 * BWD_THREADS), 0, stream, a); };
    if (p.exp2_fma) {
      if (p.D == 64) go8(attn_bwd8_kernel<64, false, false, false, true, true, true>);
      else go8(attn_bwd8_kernel<128, false, false, false, true, true, true>);
    } else {
      if (p.D == 64) go8(attn_bwd8_kernel<64, false, false, false, true, true>);
      else go8(attn_bwd8_kernel<128, false, false, false, true, true>);
    }
  } else if (p.exp2_fma) {
    // exp2 of half of the blocks on the FMA pipe: MXFP8, one head per item,
    // causal, atomic dQ
    auto go8 = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(2 * BWD_THREADS), 0, stream, a); };
    if (p.D == 64) go8(attn_bwd8_kernel<64, false, false, false, true, false, true>);
    else go8(attn_bwd8_kernel<128, false, false, false, true, false, true>);
  } else {
    auto go8 = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(2 * BWD_THREADS), 0, stream, a); };
    // one instantiation per (determinism, grouped heads, exact option, causal);
    // the exact option is causal only
    auto pick = [&](auto det, auto grp, auto exact, auto causal) {
      constexpr bool DT = decltype(det)::value, GR = decltype(grp)::value;
      constexpr bool EX = decltype(exact)::value, CA = decltype(causal)::value;
      if (p.D == 64) go8(attn_bwd8_kernel<64, DT, GR, EX, CA>); else go8(attn_bwd8_kernel<128, DT, GR, EX, CA>);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    auto by_causal = [&](auto det, auto grp) {
      if (p.exact) pick(det, grp, T_{}, T_{});
      else if (p.causal) pick(det, grp, F_{}, T_{});
      else pick(det, grp, F_{}, F_{});
    };
    auto by_group = [&](auto det) {
      if (p.Hk != p.H) by_causal(det, T_{}); else by_causal(det, F_{});
    };
    if (p.deterministic) by_group(T_{}); else by_group(F_{});
  }
  return hipGetLastError();
}

}  // namespace flamia
