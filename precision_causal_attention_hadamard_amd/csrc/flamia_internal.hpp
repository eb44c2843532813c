// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace flamia {

constexpr int PLAN_MAX_TILES = 8192;      // LDS capacity of the one-workgroup work-list sort
constexpr int PLAN_RUN = 2048;            // run length of the multi-workgroup sort (sorted in LDS)
constexpr int COST_MAX = (1 << 20) - 1;   // costs must stay below this

// Plan words: [0] forward items, [1] backward items, [2] deterministic-mode
// error word (1: the documents need more dQ partial slots than the
// workspace holds), [3] backward dispatch items (= [1]).
struct PlanLayout {
  size_t fwd_offset;   // bytes from the plan base to the forward (doc, tile) list
  size_t bwd_offset;   // the backward list in the pages' order (cost descending)
  size_t disp_offset;  // the backward's dispatch order: the same items, grouped by document
  size_t det_offset;   // int [num_docs + 1]: first dQ partial step of each document (per head)
  int cap_fwd;         // ceil(T / FWD_BQ) + num_docs
  int cap_bwd;         // ceil(T / BWD_BK) + num_docs
  int det_cap;         // deterministic mode: dQ partial steps per head the workspace holds
  int cap_r;           // lists beyond PLAN_MAX_TILES: padded key slots per list (a multiple of
                       // PLAN_RUN), else 0
  size_t keys_offset;  // with cap_r: two key buffers of 3 x cap_r uint64 (the three lists)
  size_t bytes;
};

// Byte offsets of the backward workspace.
struct BwdLayout {
  size_t do_codes, do_exp, kofs, delta, il8, qexps, g, dq_sigma, dq_acc, dk_f32, dv_f32, dq_part, bytes;
};

struct Problem {
  const int* cu;
  int T, ndocs, H, D;
  int Hk;                  // key/value heads (= H, or a divisor of H: grouped query attention)
  int hadamard, causal_dq_scale, path;
  int deterministic;       // dQ from per-step partials added in a fixed order
  int exact;               // the exact option: per-token scales, all-tile V fold, two dS payloads
  int causal;              // 1: key j visible to query i for j <= i; 0: every key of the document
  int exp2_fma;            // 1: exp2 of the blocks poly_block selects on the FMA-pipe polynomial
  float softmax_scale;     // fp32 softmax scale
  float c_log2;            // fp32(softmax_scale * log2(e))
};

hipError_t launch_plan(const int* cu, int ndocs, int causal, void* plan, const PlanLayout& pl, float* qk_scale,
                       hipStream_t stream);

// Deterministic-mode dQ partials: one fp16 [BWD_BQ, d] slot per (step, head),
// step = first step of the document + u Q - u (u - 1) + (qt - 2 u) for key tile
// u and query tile qt of a document with Q query tiles (causal: key tile u
// visits query tiles 2u .. Q-1), or + u Q + qt without the mask (every key
// tile visits every query tile).
__host__ __device__ inline long long det_step(int base, int u, int qt, int nq_tiles, bool causal) {
  if (!causal) return (long long)base + (long long)u * nq_tiles + qt;
  return (long long)base + (long long)u * nq_tiles - (long long)u * (u - 1) + (qt - 2 * u);
}

// NVFP4 score operands of the mixed path (null when path = 0).
struct Fp4Operands {
  uint8_t *q_fp4, *k_fp4, *q_sf, *k_sf;
  float* qk_scale;     // [0],[1] amax bits of Q and K; [2],[3] tensor scales
  uint16_t *q_x, *k_x; // code x group scale, exactly, as bf16 [T, H, d]
};

hipError_t launch_amax_qk(const Problem& p, const void* q, const void* k, float* qk_scale, hipStream_t stream);

hipError_t launch_quant_qkv(const Problem& p, const void* q, const void* k, const void* v,
                            uint8_t* q_codes, uint8_t* k_codes, uint8_t* v_codes, uint8_t* v_key_codes,
                            uint8_t* q_exp, uint8_t* k_exp, uint8_t* v_exp, uint8_t* v_key_exp,
                            uint8_t* v_ref_exp, uint8_t* k_ref_exp, const Fp4Operands& f4, hipStream_t stream);

hipError_t launch_quant_do(const Problem& p, const void* dout, const void* o, const int* row_max,
                           const float* row_sum, const uint8_t* q_exp, const uint8_t* k_exp,
                           const uint8_t* v_exp, const uint8_t* v_ref_exp, const uint8_t* k_ref_exp,
                           uint8_t* do_codes,
                           uint8_t* do_exp, int* kofs, float* delta,
                           float* il8, int* qexps, void* g, int* dq_sigma, void* dq_acc, hipStream_t stream);

hipError_t launch_attn_fwd(const Problem& p, const void* plan, const PlanLayout& pl,
                           const uint8_t* q_codes, const uint8_t* k_codes, const uint8_t* v_codes,
                           const uint8_t* v_key_codes, const uint8_t* q_exp, const uint8_t* k_exp,
                           const uint8_t* v_exp, const uint8_t* v_key_exp, const uint8_t* v_ref_exp,
                           const Fp4Operands& f4, void* o, int* row_max, float* row_sum, hipStream_t stream,
                           uint8_t* dump = nullptr, int* dump_max = nullptr, int dump_len = 0,
                           bool p4 = false);

// Everything the backward kernel reads and writes.
struct BwdInputs {
  const uint8_t *q_codes, *k_codes, *v_codes, *v_key_codes;
  const uint8_t *k_exp, *v_exp, *v_key_exp;   // [Hk, T]
  const int* kofs;         // [H, T] 8 - integer row maximum
  const float* il8;        // [H, T] 2^-8 / l
  const float* delta;      // [H, T] -D
  const int* dq_sigma;     // [H, T]
  const int* qexps;        // [H, T] q_exp | do_exp << 8 | v_ref_exp << 16 | fast-form flag << 24
  const uint8_t* do_codes;
  const void* g;
  void* dq_acc;
  float* dk_f32;           // mixed path: fp32 dK staging (the finaliser rotates and rounds it);
                           // split groups: fp32 dK partials [gsplit, T, Hk, d]
  float* dv_f32;           // split groups: fp32 dV partials [gsplit, T, Hk, d]
  int gsplit;              // items per key/value head group (1: one item runs the whole group)
  void* dk;                // MXFP8 path: bf16 dK, written by the backward kernel
  void* dv;
  void* dq_part;           // deterministic mode: fp16 dQ partial slots
  const int* det_base;     // deterministic mode: first step of each document (plan)
  int det_cap;             // deterministic mode: steps per head in dq_part
  const uint8_t* v_ref_exp;   // exact option: V's in-block prefix maximum
  const void *q_x, *k_x;   // mixed path only
  const float* qk_scale;   // mixed path only
  // diagnostic instantiation (MXFP8, one head per item, causal, atomic dQ):
  // P^ codes [H, T, dump_len] (may be null) and counts of nonzero dS and of
  // those whose E4M3 code is zero (zeroed here before the launch)
  uint8_t* dump = nullptr;
  int dump_len = 0;
  unsigned long long* ds_counts = nullptr;
  bool diag = false;
};

hipError_t launch_attn_bwd(const Problem& p, const void* plan, const PlanLayout& pl, const BwdInputs& in,
                           hipStream_t stream);

// Split groups: dK, dV of each key/value head = the sum of the gsplit fp32
// partials in order, dK rotated back (Hadamard option), both rounded to bf16.
hipError_t launch_group_reduce(const Problem& p, int gsplit, const float* dk_f32, const float* dv_f32, void* dk,
                               void* dv, hipStream_t stream);

hipError_t launch_finalize(const Problem& p, const void* dq_acc, const int* dq_sigma,
                           const float* dk_f32, void* dq, void* dk, bool with_dk, const void* dq_part,
                           const int* det_base, int det_cap, hipStream_t stream);

}  // namespace flamia
