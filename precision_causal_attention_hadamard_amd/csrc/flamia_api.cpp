// Host side of the flamia C ABI: argument validation, buffer layouts and
// kernel launches.  Nothing here allocates, frees or synchronises.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "../../include/flamia.h"
#include "flamia_internal.hpp"

namespace {

using namespace flamia;

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Tile sizes of the kernels (kept in step with flamia_device.hpp).
constexpr int K_FWD_BQ = 128, K_FWD_BK = 64, K_BWD_BQ = 64, K_BWD_BK = 128;

// Deterministic mode: an upper bound of the dQ partial steps per head.  A
// document of L tokens has n Q - n (n - 1) <= n^2 + n steps (n = ceil(L/128)
// key tiles, Q = ceil(L/64) <= 2n query tiles), and n^2 + n <= L^2/16384 +
// 3L/128 + 2; summed over documents of at most M tokens that is at most
// T M / 16384 + 3 T / 128 + 2 num_docs.  Without the mask a document has
// n Q <= (L/128 + 1)(L/64 + 1) = L^2/8192 + 3L/128 + 1 steps, so at most
// T M / 8192 + 3 T / 128 + num_docs in all.
int64_t det_step_cap(const flamia_attn_desc* d) {
  const int64_t T = d->total_tokens, M = d->max_doc_len > 0 ? d->max_doc_len : d->total_tokens;
  const int64_t div = d->causal ? 16384 : 8192;
  return (T * M + div - 1) / div + (3 * T + 127) / 128 + 2 * (int64_t)d->num_docs;
}

flamia_status validate(const flamia_attn_desc* d) {
  if (!d || !d->cu_seqlens) return FLAMIA_ERR_INVALID_ARG;
  if (d->total_tokens < 0 || d->num_docs < 1 || d->num_heads < 1) return FLAMIA_ERR_INVALID_ARG;
  if (d->max_doc_len < 0 || d->max_doc_len > d->total_tokens) return FLAMIA_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return FLAMIA_ERR_INVALID_ARG;
  if ((d->hadamard | d->causal_dq_scale | d->deterministic | d->causal | d->exact) & ~1) return FLAMIA_ERR_INVALID_ARG;
  if (d->path != 0 && d->path != 1) return FLAMIA_ERR_INVALID_ARG;
  if (!std::isfinite(d->softmax_scale)) return FLAMIA_ERR_INVALID_ARG;
  if (d->num_kv_heads < 0 || d->num_kv_heads > d->num_heads ||
      (d->num_kv_heads > 0 && d->num_heads % d->num_kv_heads != 0))
    return FLAMIA_ERR_INVALID_ARG;
  // without the mask: the causal dQ prescale and the exact option (both
  // defined by which keys a query may see) do not apply
  if (!d->causal && (d->causal_dq_scale || d->exact)) return FLAMIA_ERR_INVALID_ARG;
  // the exact option is built for the MXFP8 path
  if (d->exact && d->path != 0) return FLAMIA_ERR_UNSUPPORTED;
  // the FMA-pipe exp2: 0 or 1; built for the default MXFP8 call (causal, one
  // key/value head per query head, atomic dQ, no exact option)
  if (d->exp2_fma & ~1) return FLAMIA_ERR_INVALID_ARG;
  if (d->exp2_fma && (d->path != 0 || d->exact || !d->causal || d->deterministic ||
                      (d->num_kv_heads > 0 && d->num_kv_heads != d->num_heads)))
    return FLAMIA_ERR_UNSUPPORTED;
  // index limits: documents and tiles are packed into 24 and 20 bits of the
  // sort key, costs into 20 bits; a launch's work-items (up to 512 per
  // workgroup, one workgroup per tile and head) must fit 32 bits
  if (d->num_docs >= (1 << 24) || d->total_tokens >= (1 << 24)) return FLAMIA_ERR_WORKSPACE;
  const int64_t cap = cdiv(d->total_tokens, K_FWD_BQ) + (int64_t)d->num_docs;
  if (cap * d->num_heads * 512 >= (int64_t)1 << 32) return FLAMIA_ERR_WORKSPACE;
  // the backward addresses a document's rows with 32-bit byte offsets of 2-byte elements
  if ((int64_t)d->total_tokens * d->num_heads * d->head_dim >= (int64_t)1 << 30) return FLAMIA_ERR_WORKSPACE;
  // deterministic mode: steps are 32-bit in the plan
  if (d->deterministic && det_step_cap(d) >= ((int64_t)1 << 31)) return FLAMIA_ERR_WORKSPACE;
  return FLAMIA_OK;
}

inline int kv_heads(const flamia_attn_desc* d) { return d->num_kv_heads > 0 ? d->num_kv_heads : d->num_heads; }

// Grouped query attention: the MXFP8 backward item is (document, key tile,
// key/value head) and runs the group's query heads itself.  When that gives
// fewer than K_BWD_MIN_ITEMS items (two per CU of an MI355X), each group is
// split over the smallest divisor s of H/Hk that reaches it, and the s fp32
// partials of dK and dV are reduced afterwards.  The mixed path's item is one
// query head, so its s is H/Hk.
constexpr int64_t K_BWD_MIN_ITEMS = 512;
int bwd_group_split(const flamia_attn_desc* d) {
  const int g = d->num_heads / kv_heads(d);
  if (g == 1) return 1;
  if (d->path == 1) return g;     // the mixed path's backward item is one query head
  const int64_t items = (int64_t)(cdiv(d->total_tokens, K_BWD_BK) + d->num_docs) * kv_heads(d);
  for (int s = 1; s < g; ++s)
    if (g % s == 0 && items * s >= K_BWD_MIN_ITEMS) return s;
  return g;
}

PlanLayout plan_layout(const flamia_attn_desc* d) {
  PlanLayout pl{};
  pl.cap_fwd = cdiv(d->total_tokens, K_FWD_BQ) + d->num_docs;
  pl.cap_bwd = cdiv(d->total_tokens, K_BWD_BK) + d->num_docs;
  pl.fwd_offset = ALIGN;
  pl.bwd_offset = align_up(pl.fwd_offset + sizeof(int) * 2 * (size_t)pl.cap_fwd);
  pl.disp_offset = align_up(pl.bwd_offset + sizeof(int) * 2 * (size_t)pl.cap_bwd);
  pl.det_offset = align_up(pl.disp_offset + sizeof(int) * 2 * (size_t)pl.cap_bwd);
  pl.det_cap = d->deterministic ? (int)det_step_cap(d) : 0;
  pl.bytes = align_up(pl.det_offset + sizeof(int) * ((size_t)d->num_docs + 1));
  // lists beyond one workgroup's LDS: padded keys of the three lists, two buffers
  pl.cap_r = 0;
  pl.keys_offset = 0;
  if (pl.cap_fwd > PLAN_MAX_TILES) {
    pl.cap_r = cdiv(pl.cap_fwd, PLAN_RUN) * PLAN_RUN;
    pl.keys_offset = pl.bytes;
    pl.bytes = align_up(pl.keys_offset + 6 * sizeof(uint64_t) * (size_t)pl.cap_r);
  }
  return pl;
}

struct QLayout {
  size_t codes[4], exps[5], plan, fp4[2], sf[2], qk_scale, fx[2], k_ref, bytes;
};

QLayout q_layout(const flamia_attn_desc* d) {
  QLayout q{};
  const size_t E = (size_t)d->total_tokens * d->num_heads * d->head_dim;
  const size_t M = (size_t)d->total_tokens * d->num_heads;
  const size_t Ek = (size_t)d->total_tokens * kv_heads(d) * d->head_dim;   // K, V: [T, Hk, d]
  const size_t Mk = (size_t)d->total_tokens * kv_heads(d);
  size_t off = 0;
  for (int i = 0; i < 4; ++i) { q.codes[i] = off; off = align_up(off + (i == 0 ? E : Ek)); }
  for (int i = 0; i < 5; ++i) { q.exps[i] = off; off = align_up(off + (i == 0 ? M : Mk)); }
  q.plan = off;
  off = align_up(off + plan_layout(d).bytes);
  q.k_ref = 0;
  if (d->exact) { q.k_ref = off; off = align_up(off + Mk); }
  q.fp4[0] = q.fp4[1] = q.sf[0] = q.sf[1] = q.qk_scale = q.fx[0] = q.fx[1] = 0;
  if (d->path == 1) {
    for (int i = 0; i < 2; ++i) { q.fp4[i] = off; off = align_up(off + E / 2); }
    for (int i = 0; i < 2; ++i) { q.sf[i] = off; off = align_up(off + E / 16); }
    q.qk_scale = off; off = align_up(off + 4 * sizeof(float));
    for (int i = 0; i < 2; ++i) { q.fx[i] = off; off = align_up(off + 2 * E); }
  }
  q.bytes = off;
  return q;
}

BwdLayout bwd_layout(const flamia_attn_desc* d) {
  BwdLayout b{};
  const size_t E = (size_t)d->total_tokens * d->num_heads * d->head_dim;
  const size_t M = (size_t)d->total_tokens * d->num_heads;
  size_t off = 0;
  b.do_codes = off; off = align_up(off + E);
  b.do_exp = off;   off = align_up(off + M);
  b.kofs = off;     off = align_up(off + 4 * M);
  b.delta = off;    off = align_up(off + 4 * M);
  b.il8 = off;      off = align_up(off + 4 * M);
  b.qexps = off;    off = align_up(off + 4 * M);
  b.g = off;        off = align_up(off + 2 * E);
  b.dq_sigma = off; off = align_up(off + 4 * M);
  b.dq_acc = off;   off = align_up(off + 2 * E);
  // fp32 dK staging: the mixed path's dK, or the split-group dK partials
  // (s Hk <= H, so E holds them); the MXFP8 path otherwise writes bf16 dK
  // from the backward kernel and needs none
  const int gs = bwd_group_split(d);
  b.dk_f32 = off;
  if (d->path == 1 || gs > 1) off = align_up(off + 4 * E);
  b.dv_f32 = off;
  if (gs > 1) off = align_up(off + 4 * (size_t)gs * d->total_tokens * kv_heads(d) * d->head_dim);
  b.dq_part = off;
  if (d->deterministic)
    off = align_up(off + (size_t)det_step_cap(d) * d->num_heads * K_BWD_BQ * d->head_dim * 2);
  b.bytes = off;
  return b;
}

Problem problem(const flamia_attn_desc* d) {
  Problem p{};
  p.cu = d->cu_seqlens;
  p.T = d->total_tokens;
  p.ndocs = d->num_docs;
  p.H = d->num_heads;
  p.Hk = kv_heads(d);
  p.D = d->head_dim;
  p.hadamard = d->hadamard;
  p.causal_dq_scale = d->causal_dq_scale;
  p.path = d->path;
  p.deterministic = d->deterministic;
  p.exact = d->exact;
  p.causal = d->causal;
  p.exp2_fma = d->exp2_fma;
  // the exact option carries its own (per-token) causal dQ prescale
  if (p.exact) p.causal_dq_scale = 1;
  p.softmax_scale = d->softmax_scale > 0.f ? d->softmax_scale : (float)(1.0 / std::sqrt((double)d->head_dim));
  p.c_log2 = (float)((double)p.softmax_scale * 1.4426950408889634);
  return p;
}

bool qt_complete(const flamia_attn_desc* d, const flamia_qtensors* q) {
  if (!(q && q->q_codes && q->k_codes && q->v_codes && q->v_key_codes && q->q_exp && q->k_exp &&
        q->v_exp && q->v_key_exp && q->v_ref_exp && q->plan && (!d->exact || q->k_ref_exp)))
    return false;
  return d->path != 1 ||
         (q->q_fp4 && q->k_fp4 && q->q_sf && q->k_sf && q->qk_tensor_scale && q->q_fp4_bf16 && q->k_fp4_bf16);
}

Fp4Operands fp4_operands(const flamia_qtensors* q) {
  return Fp4Operands{q->q_fp4, q->k_fp4, q->q_sf, q->k_sf, q->qk_tensor_scale,
                     static_cast<uint16_t*>(q->q_fp4_bf16), static_cast<uint16_t*>(q->k_fp4_bf16)};
}

flamia_status hip_status(hipError_t e) { return e == hipSuccess ? FLAMIA_OK : FLAMIA_ERR_HIP; }

flamia_status bwd_main(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* dk, void* dv, void* ws,
                       hipStream_t stream, uint8_t* dump, int dump_len, unsigned long long* ds_counts, bool diag);

// The diagnostic instantiations cover the MXFP8 causal call with one
// key/value head per query head, atomic dQ and block scales.
flamia_status diag_supported(const flamia_attn_desc* d, const void* dump, int32_t dump_len) {
  if (d->path != 0 || kv_heads(d) != d->num_heads || d->exact || d->deterministic || !d->causal)
    return FLAMIA_ERR_UNSUPPORTED;
  const int32_t mdl = d->max_doc_len > 0 ? d->max_doc_len : d->total_tokens;
  if (dump != nullptr && dump_len < std::max(mdl, 1)) return FLAMIA_ERR_INVALID_ARG;
  return FLAMIA_OK;
}


// Tensor and workspace pointers may be null only for an empty call (T = 0),
// which launches nothing but the work-list build.
bool tensors_ok(const flamia_attn_desc* d, std::initializer_list<const void*> ps) {
  if (d->total_tokens == 0) return true;
  for (const void* p : ps)
    if (!p) return false;
  return true;
}

}  // namespace

extern "C" {

flamia_status flamia_buffer_sizes(const flamia_attn_desc* desc, size_t* qtensor_bytes,
                                  size_t* fwd_ws_bytes, size_t* bwd_ws_bytes) {
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (qtensor_bytes) *qtensor_bytes = q_layout(desc).bytes;
  if (fwd_ws_bytes) *fwd_ws_bytes = 0;
  if (bwd_ws_bytes) *bwd_ws_bytes = bwd_layout(desc).bytes;
  return FLAMIA_OK;
}

flamia_status flamia_qtensors_layout(const flamia_attn_desc* desc, void* base, flamia_qtensors* out) {
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (!base || !out || (reinterpret_cast<uintptr_t>(base) % ALIGN) != 0) return FLAMIA_ERR_INVALID_ARG;
  const QLayout q = q_layout(desc);
  uint8_t* b = static_cast<uint8_t*>(base);
  out->q_codes = b + q.codes[0];
  out->k_codes = b + q.codes[1];
  out->v_codes = b + q.codes[2];
  out->v_key_codes = b + q.codes[3];
  out->q_exp = b + q.exps[0];
  out->k_exp = b + q.exps[1];
  out->v_exp = b + q.exps[2];
  out->v_key_exp = b + q.exps[3];
  out->v_ref_exp = b + q.exps[4];
  out->plan = b + q.plan;
  const bool mixed = desc->path == 1;
  out->q_fp4 = mixed ? b + q.fp4[0] : nullptr;
  out->k_fp4 = mixed ? b + q.fp4[1] : nullptr;
  out->q_sf = mixed ? b + q.sf[0] : nullptr;
  out->k_sf = mixed ? b + q.sf[1] : nullptr;
  out->qk_tensor_scale = mixed ? reinterpret_cast<float*>(b + q.qk_scale) : nullptr;
  out->q_fp4_bf16 = mixed ? b + q.fx[0] : nullptr;
  out->k_fp4_bf16 = mixed ? b + q.fx[1] : nullptr;
  out->k_ref_exp = desc->exact ? b + q.k_ref : nullptr;
  return FLAMIA_OK;
}

flamia_status flamia_plan_build(const flamia_attn_desc* desc, const flamia_qtensors* out, hipStream_t stream) {
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (!qt_complete(desc, out)) return FLAMIA_ERR_INVALID_ARG;
  const Problem p = problem(desc);
  return hip_status(launch_plan(p.cu, p.ndocs, p.causal, out->plan, plan_layout(desc),
                                p.path == 1 ? out->qk_tensor_scale : nullptr, stream));
}

flamia_status flamia_quantize(const flamia_attn_desc* desc, const void* q, const void* k, const void* v,
                              const flamia_qtensors* out, hipStream_t stream) {
  flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (!tensors_ok(desc, {q, k, v}) || !qt_complete(desc, out)) return FLAMIA_ERR_INVALID_ARG;
  const Problem p = problem(desc);
  s = flamia_plan_build(desc, out, stream);
  if (s != FLAMIA_OK) return s;
  if (p.path == 1) {
    s = hip_status(launch_amax_qk(p, q, k, out->qk_tensor_scale, stream));
    if (s != FLAMIA_OK) return s;
  }
  return hip_status(launch_quant_qkv(p, q, k, v, out->q_codes, out->k_codes, out->v_codes, out->v_key_codes,
                                     out->q_exp, out->k_exp, out->v_exp, out->v_key_exp, out->v_ref_exp,
                                     out->k_ref_exp, fp4_operands(out), stream));
}

flamia_status flamia_attn_fwd(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* o,
                              int32_t* row_max, float* row_sum, void* ws, hipStream_t stream) {
  (void)ws;
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (!qt_complete(desc, qt) || !tensors_ok(desc, {o, row_max, row_sum})) return FLAMIA_ERR_INVALID_ARG;
  const Problem p = problem(desc);
  return hip_status(launch_attn_fwd(p, qt->plan, plan_layout(desc), qt->q_codes, qt->k_codes, qt->v_codes,
                                    qt->v_key_codes, qt->q_exp, qt->k_exp, qt->v_exp, qt->v_key_exp,
                                    qt->v_ref_exp, fp4_operands(qt), o, row_max, row_sum, stream));
}

flamia_status flamia_attn_fwd_p4(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* o,
                                 int32_t* row_max, float* row_sum, void* ws, hipStream_t stream) {
  (void)ws;
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (desc->path != 0 || desc->exact || desc->exp2_fma) return FLAMIA_ERR_UNSUPPORTED;
  if (!qt_complete(desc, qt) || !tensors_ok(desc, {o, row_max, row_sum})) return FLAMIA_ERR_INVALID_ARG;
  const Problem p = problem(desc);
  return hip_status(launch_attn_fwd(p, qt->plan, plan_layout(desc), qt->q_codes, qt->k_codes, qt->v_codes,
                                    qt->v_key_codes, qt->q_exp, qt->k_exp, qt->v_exp, qt->v_key_exp,
                                    qt->v_ref_exp, fp4_operands(qt), o, row_max, row_sum, stream, nullptr, nullptr,
                                    0, true));
}

flamia_status flamia_attn_bwd_prep(const flamia_attn_desc* desc, const flamia_qtensors* qt, const void* o,
                                   const int32_t* row_max, const float* row_sum, const void* dout, void* ws,
                                   hipStream_t stream) {
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (!qt_complete(desc, qt) || !tensors_ok(desc, {o, row_max, row_sum, dout, ws})) return FLAMIA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) % ALIGN) != 0) return FLAMIA_ERR_INVALID_ARG;
  const Problem p = problem(desc);
  const BwdLayout b = bwd_layout(desc);
  uint8_t* w = static_cast<uint8_t*>(ws);
  return hip_status(launch_quant_do(p, dout, o, row_max, row_sum, qt->q_exp, qt->k_exp, qt->v_exp,
                                    qt->v_ref_exp, qt->k_ref_exp, w + b.do_codes, w + b.do_exp, reinterpret_cast<int*>(w + b.kofs),
                                    reinterpret_cast<float*>(w + b.delta),
                                    reinterpret_cast<float*>(w + b.il8), reinterpret_cast<int*>(w + b.qexps),
                                    w + b.g, reinterpret_cast<int*>(w + b.dq_sigma), w + b.dq_acc, stream));
}

flamia_status flamia_attn_bwd_main(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* dk, void* dv,
                                   void* ws, hipStream_t stream) {
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (!qt_complete(desc, qt) || !tensors_ok(desc, {dk, dv, ws})) return FLAMIA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) % ALIGN) != 0) return FLAMIA_ERR_INVALID_ARG;
  return bwd_main(desc, qt, dk, dv, ws, stream, nullptr, 0, nullptr, false);
}

}  // extern "C"

namespace {

flamia_status bwd_main(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* dk, void* dv, void* ws,
                       hipStream_t stream, uint8_t* dump, int dump_len, unsigned long long* ds_counts,
                       bool diag) {
  const Problem p = problem(desc);
  const BwdLayout b = bwd_layout(desc);
  uint8_t* w = static_cast<uint8_t*>(ws);
  BwdInputs in{};
  in.q_codes = qt->q_codes;
  in.k_codes = qt->k_codes;
  in.v_codes = qt->v_codes;
  in.v_key_codes = qt->v_key_codes;
  in.k_exp = qt->k_exp;
  in.v_exp = qt->v_exp;
  in.v_key_exp = qt->v_key_exp;
  in.kofs = reinterpret_cast<const int*>(w + b.kofs);
  in.il8 = reinterpret_cast<const float*>(w + b.il8);
  in.delta = reinterpret_cast<const float*>(w + b.delta);
  in.dq_sigma = reinterpret_cast<const int*>(w + b.dq_sigma);
  in.qexps = reinterpret_cast<const int*>(w + b.qexps);
  in.do_codes = w + b.do_codes;
  in.g = w + b.g;
  in.dq_acc = w + b.dq_acc;
  in.dk_f32 = reinterpret_cast<float*>(w + b.dk_f32);
  in.dk = dk;
  in.dv = dv;
  in.dv_f32 = reinterpret_cast<float*>(w + b.dv_f32);
  in.gsplit = bwd_group_split(desc);
  const PlanLayout pl = plan_layout(desc);
  in.dq_part = w + b.dq_part;
  in.det_base = reinterpret_cast<const int*>(static_cast<const uint8_t*>(qt->plan) + pl.det_offset);
  in.det_cap = pl.det_cap;
  in.v_ref_exp = qt->v_ref_exp;
  in.q_x = qt->q_fp4_bf16;
  in.k_x = qt->k_fp4_bf16;
  in.qk_scale = qt->qk_tensor_scale;
  in.dump = dump;
  in.dump_len = dump_len;
  in.ds_counts = ds_counts;
  in.diag = diag;
  const flamia_status st = hip_status(launch_attn_bwd(p, qt->plan, pl, in, stream));
  if (st != FLAMIA_OK || in.gsplit == 1) return st;
  return hip_status(launch_group_reduce(p, in.gsplit, in.dk_f32, in.dv_f32, dk, dv, stream));
}

}  // namespace

extern "C" {

flamia_status flamia_attn_bwd_finish(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* dq,
                                     void* dk, void* ws, hipStream_t stream) {
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (!qt_complete(desc, qt) || !tensors_ok(desc, {dq, dk, ws})) return FLAMIA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) % ALIGN) != 0) return FLAMIA_ERR_INVALID_ARG;
  const Problem p = problem(desc);
  const BwdLayout b = bwd_layout(desc);
  uint8_t* w = static_cast<uint8_t*>(ws);
  const PlanLayout pl = plan_layout(desc);
  return hip_status(launch_finalize(p, w + b.dq_acc, reinterpret_cast<const int*>(w + b.dq_sigma),
                                    reinterpret_cast<const float*>(w + b.dk_f32), dq, dk,
                                    p.path == 1 && bwd_group_split(desc) == 1,   // else dK came from the group reduction
                                    w + b.dq_part,
                                    reinterpret_cast<const int*>(static_cast<const uint8_t*>(qt->plan) + pl.det_offset),
                                    pl.det_cap, stream));
}

flamia_status flamia_attn_fwd_diag(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* o,
                                   int32_t* row_max, float* row_sum, void* ws, uint8_t* phat, int32_t* phat_max,
                                   int32_t row_len, hipStream_t stream) {
  (void)ws;
  flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if ((s = diag_supported(desc, phat, row_len)) != FLAMIA_OK) return s;
  if (!qt_complete(desc, qt) || !tensors_ok(desc, {o, row_max, row_sum, phat, phat_max}))
    return FLAMIA_ERR_INVALID_ARG;
  const Problem p = problem(desc);
  return hip_status(launch_attn_fwd(p, qt->plan, plan_layout(desc), qt->q_codes, qt->k_codes, qt->v_codes,
                                    qt->v_key_codes, qt->q_exp, qt->k_exp, qt->v_exp, qt->v_key_exp,
                                    qt->v_ref_exp, fp4_operands(qt), o, row_max, row_sum, stream, phat,
                                    phat_max, std::max(row_len, 1)));
}

flamia_status flamia_attn_bwd_main_diag(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* dk,
                                        void* dv, void* ws, uint8_t* phat, int32_t row_len,
                                        uint64_t* ds_counts, hipStream_t stream) {
  flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if ((s = diag_supported(desc, phat, row_len)) != FLAMIA_OK) return s;
  if (!qt_complete(desc, qt) || !tensors_ok(desc, {dk, dv, ws})) return FLAMIA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) % ALIGN) != 0) return FLAMIA_ERR_INVALID_ARG;
  return bwd_main(desc, qt, dk, dv, ws, stream, phat, row_len, reinterpret_cast<unsigned long long*>(ds_counts),
                  true);
}

flamia_status flamia_attn_bwd(const flamia_attn_desc* desc, const flamia_qtensors* qt, const void* o,
                              const int32_t* row_max, const float* row_sum, const void* dout, void* dq,
                              void* dk, void* dv, void* ws, hipStream_t stream) {
  flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (!qt_complete(desc, qt) || !tensors_ok(desc, {o, row_max, row_sum, dout, dq, dk, dv, ws}))
    return FLAMIA_ERR_INVALID_ARG;
  s = flamia_attn_bwd_prep(desc, qt, o, row_max, row_sum, dout, ws, stream);
  if (s != FLAMIA_OK) return s;
  s = flamia_attn_bwd_main(desc, qt, dk, dv, ws, stream);
  if (s != FLAMIA_OK) return s;
  return flamia_attn_bwd_finish(desc, qt, dq, dk, ws, stream);
}

flamia_status flamia_bwd_ws_layout(const flamia_attn_desc* desc, flamia_bwd_ws_offsets* out) {
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  if (!out) return FLAMIA_ERR_INVALID_ARG;
  const BwdLayout b = bwd_layout(desc);
  out->do_codes = b.do_codes;
  out->do_exp = b.do_exp;
  out->neg_delta = b.delta;
  out->inv_l = b.il8;
  out->g = b.g;
  out->dq_sigma = b.dq_sigma;
  out->dq_acc = b.dq_acc;
  return FLAMIA_OK;
}

flamia_status flamia_tile_config(int32_t head_dim, int32_t* fwd_bq, int32_t* fwd_bk, int32_t* bwd_bq,
                                 int32_t* bwd_bk) {
  if (head_dim != 64 && head_dim != 128) return FLAMIA_ERR_INVALID_ARG;
  if (fwd_bq) *fwd_bq = K_FWD_BQ;
  if (fwd_bk) *fwd_bk = K_FWD_BK;
  if (bwd_bq) *bwd_bq = K_BWD_BQ;
  if (bwd_bk) *bwd_bk = K_BWD_BK;
  return FLAMIA_OK;
}

flamia_status flamia_plan_view(const flamia_attn_desc* desc, size_t* fwd_offset, int32_t* cap_fwd,
                               size_t* bwd_offset, int32_t* cap_bwd, size_t* bwd_dispatch_offset) {
  const flamia_status s = validate(desc);
  if (s != FLAMIA_OK) return s;
  const PlanLayout pl = plan_layout(desc);
  if (fwd_offset) *fwd_offset = pl.fwd_offset;
  if (cap_fwd) *cap_fwd = pl.cap_fwd;
  if (bwd_offset) *bwd_offset = pl.bwd_offset;
  if (cap_bwd) *cap_bwd = pl.cap_bwd;
  if (bwd_dispatch_offset) *bwd_dispatch_offset = pl.disp_offset;
  return FLAMIA_OK;
}

const char* flamia_status_string(flamia_status status) {
  switch (status) {
    case FLAMIA_OK: return "ok";
    case FLAMIA_ERR_INVALID_ARG: return "invalid argument";
    case FLAMIA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FLAMIA_ERR_WORKSPACE: return "size exceeds the library's index limits";
    case FLAMIA_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"
