/*
 * flamia.h -- C ABI of the causal block-scaled low-precision attention
 * training call for AMD MI355X (gfx950).
 *
 * The call is three steps over packed variable-length documents:
 *   flamia_quantize   fused quantization of Q, K, V (+ the work list),
 *   flamia_attn_fwd   S = Q K^T, causal (or, with causal = 0, unmasked)
 *                     online softmax, O = P^ V,
 *   flamia_attn_bwd   dO quantization + D, then dV, dP, dS, dQ, dK.
 *
 * Method (from the pages describing FLAMIA; page titles are cited in full
 * once here and shortened after):
 *   [Summary] "FLAMIA: FLAsh MIcroscaling Attention for Fast and Causally
 *             Safe Training on Blackwell" (summary page; its bullets carry
 *             the paper's section numbers, e.g. §3.1 Token-Block Scaling).
 *   [Reading] "因果安全的低精度注意力——FLAMIA Blackwell 训练内核精读",
 *             sections 4.1-4.4.
 *   [News]    "FLAMIA Brings Causally Safe Low-Precision Attention to
 *             Blackwell", "Key design choices".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts.  Per-token tensors are [T, H, d] row-major ("THD": packed tokens,
 *   then heads, then the head dimension), no padding between documents;
 *   k, v, dk, dv and the K-side quantized tensors have Hk = num_kv_heads heads.
 *   Per-token metadata (exponent bytes, row statistics, D) is [H, T].
 *   Documents are given by cu_seqlens (device int32[num_docs + 1],
 *   0 = cu[0] <= cu[1] <= ... <= cu[num_docs] = T).
 * Numbers.  q, k, v, dout, o, dq, dk, dv are bf16.  Codes are E4M3 (OCP FN:
 *   bias 7, largest finite 448).  Exponent bytes are UE8M0 (value e + 127).
 * Ownership.  Every pointer is caller-owned device memory; the library
 *   never allocates, frees or keeps device memory, holds no state between
 *   calls and never synchronises the host.  Each call only enqueues kernels
 *   on `stream`, so a whole training call can be captured in a HIP graph.
 * Errors.  Every function returns a flamia_status and never throws.  Only
 *   host scalars and pointer non-nullness are validated (before anything is
 *   launched); a malformed device-side cu_seqlens is undefined behaviour.
 *   An empty call (total_tokens = 0, cu_seqlens all zero) is valid: tensor
 *   and workspace pointers may then be NULL, and only the work-list build
 *   is launched.
 *   FLAMIA_ERR_HIP reports a failed kernel launch (hipGetLastError).
 * Descriptor.  The same flamia_attn_desc (all fields equal) must be passed
 *   to flamia_quantize, flamia_attn_fwd and flamia_attn_bwd of one call.
 */
#ifndef FLAMIA_H
#define FLAMIA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLAMIA_OK = 0,
  FLAMIA_ERR_INVALID_ARG = 1,   /* bad host scalar or NULL pointer */
  FLAMIA_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement */
  FLAMIA_ERR_WORKSPACE = 3,     /* a size exceeds what the library can index */
  FLAMIA_ERR_HIP = 4            /* a kernel launch failed */
} flamia_status;

typedef struct flamia_attn_desc {
  int32_t total_tokens;         /* T >= 0 */
  int32_t num_docs;             /* >= 1 */
  int32_t max_doc_len;          /* caller's upper bound of any document length, 1..T (0: T);
                                   sizes the deterministic-mode dQ partial buffer */
  const int32_t* cu_seqlens;    /* device int32[num_docs + 1] */
  int32_t num_heads;            /* H >= 1 */
  int32_t head_dim;             /* d: 64 or 128 */
  int32_t causal;               /* 1: query i sees keys j <= i of its document (the call the pages
                                   define); 0: every key of its document, same quantization rules
                                   without the mask -- the diagonal per-key V fold then takes the
                                   whole 32-token block as visible, so its reference is the block
                                   exponent.  Both paths.  0 with causal_dq_scale or exact:
                                   FLAMIA_ERR_INVALID_ARG */
  int32_t path;                 /* 0 = MXFP8; 1 = mixed: QK^T (and its recompute) from NVFP4 Q/K */
  int32_t hadamard;             /* 1: rotate Q and K rows by the normalised Sylvester Hadamard matrix */
  int32_t causal_dq_scale;      /* 1: dQ accumulator prescale from causally visible blocks only */
  int32_t deterministic;        /* 0: dQ reduced with fp16 atomics (order not fixed);
                                   1: each (key tile, query tile) dQ partial is stored in its own
                                   fp16 slot and the finaliser adds the slots of a query in fp16 in
                                   ascending key-tile order -- bitwise reproducible
                                   ([Reading, 6.3]: atomic dQ reduction by default, a slower
                                   deterministic mode beside it) */
  float softmax_scale;          /* <= 0 selects 1/sqrt(head_dim) */
  int32_t num_kv_heads;         /* Hk: heads of k and v; 0 (or H) = one per query head.  A proper
                                   divisor of H gives grouped query attention: query head h reads
                                   key/value head h / (H / Hk), and dk, dv of a key/value head are
                                   the sums over its H / Hk query heads, accumulated in fp32 and
                                   rounded once ([Reading, 5.2] measures GQA workloads).  Both
                                   paths */
  int32_t exact;                /* 1: the exact option ([Summary] bullets on causally safe scales;
                                   [Reading, 4.2]): one exponent per token (and head) for Q, K, V
                                   and dO; V's per-token exponents folded into P on every tile
                                   against the largest exponent of the key block the query may see;
                                   dS quantized twice -- for dQ with the key's K exponent folded in,
                                   one exponent per (query, 32 keys), for dK with the query's Q
                                   exponent folded in, one exponent per (key, 32 queries) -- and a
                                   per-token causal dQ prescale.  No output depends on a later
                                   position's inputs.  MXFP8 path only (path = 1:
                                   FLAMIA_ERR_UNSUPPORTED) */
  int32_t exp2_fma;             /* 1: the exponentials of half of the 32 x 32 (query block, key
                                   block) pairs -- those whose document-local block indices have
                                   an odd sum -- on a degree-5 polynomial on the FMA pipe instead of
                                   the transcendental unit ([Reading, 4.4] second bullet: part of
                                   the exp work emulated on the FMA pipe).  Forward and backward
                                   choose alike, so the backward still replays the forward's P^.
                                   0 or 1; 1 needs path 0, causal, no exact option, one key/value
                                   head per query head and atomic dQ (else
                                   FLAMIA_ERR_UNSUPPORTED) */
} flamia_attn_desc;

/*
 * Quantized operands and the GPU-built schedule: the forward-to-backward
 * saved set together with o, row_max and row_sum.  All pointers point into
 * one caller buffer of `qtensor_bytes` (flamia_buffer_sizes); fill them with
 * flamia_qtensors_layout.
 *
 * K-side tensors (k_codes, v_codes, v_key_codes: [T,Hk,d]; k_exp, v_exp,
 * v_key_exp, v_ref_exp: [Hk,T]) carry the num_kv_heads heads; [T,H,d] and
 * [H,T] below read [T,Hk,d] and [Hk,T] for them.
 *
 *  q_codes, k_codes   [T,H,d] E4M3 token-block codes of Q and K (after the
 *                     optional Hadamard rotation) -- [Summary, §3.1 Token-Block
 *                     Scaling]: one power-of-two exponent per 32 consecutive
 *                     tokens of one document x the full head dimension.
 *  v_codes            [T,H,d] token-block codes of V.
 *  v_key_codes        [T,H,d] per-key codes of V, used on diagonal blocks.
 *  q_exp, k_exp, v_exp  [H,T] UE8M0 block exponent, repeated for every token
 *                     of the block (per-token scale metadata, [Summary, §3.6.2]).
 *  v_key_exp          [H,T] per-key exponent of V.
 *  v_ref_exp          [H,T] per query: largest v_key_exp among the keys of
 *                     its own block it may see (the fold reference of the
 *                     diagonal P^V product).
 *  k_ref_exp          [H,T] exact option only (else NULL): per token, the
 *                     largest k_exp among the tokens of its own block up to
 *                     it (with v_ref_exp, the causal dQ prescale's inputs).
 *  plan               opaque GPU-built longest-first work lists.
 *  Mixed path only (NULL when path = 0), [Summary] opening paragraphs and
 *  [Reading, 4.1]: NVFP4 score operands of Q and K (after the rotation):
 *  q_fp4, k_fp4       [T,H,d/2] E2M1 codes, two per byte (even element in
 *                     the low nibble, bit 3 of a nibble = sign).
 *  q_sf, k_sf         [T,H,d/16] E4M3 scale per 16 head-dim elements of a
 *                     token: the smallest E4M3 value >= amax_group / fp32(6 t).
 *  qk_tensor_scale    float[4]: [0], [1] = bits of the Q and K tensor amax
 *                     (working space), [2], [3] = t_Q, t_K = amax / 2688.
 *  q_fp4_bf16, k_fp4_bf16  [T,H,d] bf16: E2M1 value x E4M3 group scale of
 *                     each element, exact in bf16 (at most 5 significant
 *                     bits), the operands of the score products.
 */
typedef struct flamia_qtensors {
  uint8_t* q_codes;
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint8_t* v_key_codes;
  uint8_t* q_exp;
  uint8_t* k_exp;
  uint8_t* v_exp;
  uint8_t* v_key_exp;
  uint8_t* v_ref_exp;
  void* plan;
  uint8_t* q_fp4;
  uint8_t* k_fp4;
  uint8_t* q_sf;
  uint8_t* k_sf;
  float* qk_tensor_scale;
  void* q_fp4_bf16;
  void* k_fp4_bf16;
  uint8_t* k_ref_exp;
} flamia_qtensors;

/*
 * flamia_buffer_sizes -- bytes the caller must provide.
 *   qtensor_bytes : one buffer for flamia_qtensors (codes, exponents, plan).
 *   fwd_ws_bytes  : workspace of flamia_attn_fwd (may be 0; pass NULL then).
 *   bwd_ws_bytes  : workspace of flamia_attn_bwd (quantized dO, D, dO/l,
 *                   fp16 dQ accumulator, prescale exponents; on the mixed
 *                   path fp32 dK staging;
 *                   with grouped query attention on a grid too small to fill
 *                   the GPU, also fp32 dK and dV partials of the split groups;
 *                   in deterministic mode also the dQ partial slots: 64 x d
 *                   fp16 per head for at most ceil(T M / 16384) + ceil(3T / 128)
 *                   + 2 num_docs steps, M = max_doc_len, a bound of the causal
 *                   (key tile, query tile) steps of documents of at most M tokens;
 *                   ceil(T M / 8192) in the first term when causal = 0).
 * If the documents need more steps than max_doc_len promised, the
 * deterministic backward drops the partials beyond the workspace, writes NaN
 * to every dq row that lost one, and sets word 2 of the plan (int32 at byte 8
 * of qtensors.plan) to 1; the library never reads it back itself.  Any
 * output pointer may be NULL.  Host only; launches nothing.
 */
flamia_status flamia_buffer_sizes(const flamia_attn_desc* desc, size_t* qtensor_bytes,
                                  size_t* fwd_ws_bytes, size_t* bwd_ws_bytes);

/*
 * flamia_qtensors_layout -- carve a qtensor buffer (device address `base`,
 * at least qtensor_bytes long, 256-byte aligned) into the fields of `out`.
 * Host only; writes no device memory.
 */
flamia_status flamia_qtensors_layout(const flamia_attn_desc* desc, void* base,
                                     flamia_qtensors* out);

/*
 * flamia_plan_build -- the GPU-built longest-first work lists alone
 * ([Summary, §3.6.2 Load-Balanced Scheduling]; [Reading, 4.4] last bullet:
 * the schedule is built on the GPU once per microbatch with a fixed-pass
 * sort).  flamia_quantize runs it first; it is exported so the schedule can
 * be rebuilt or timed on its own.  Reads cu_seqlens, writes out->plan (and,
 * on the mixed path, clears the two amax slots of out->qk_tensor_scale).
 * Lists of at most 8192 tiles are sorted by one workgroup in LDS; longer
 * lists by runs of 2048 keys sorted in LDS and merge passes over a key area
 * inside the plan (sized by flamia_buffer_sizes).  No limit on the number
 * of documents beyond the descriptor's.  Enqueues only; errors as for
 * flamia_quantize.
 */
flamia_status flamia_plan_build(const flamia_attn_desc* desc, const flamia_qtensors* out, hipStream_t stream);

/*
 * flamia_quantize -- fused forward-side quantization, [Reading, 4.4] first
 * bullet (rotation, block statistics, codes and scales generated together)
 * and [Summary, §4.3 Ablation Study]; plus the GPU-built work lists of
 * [Summary, §3.6.2 Load-Balanced Scheduling] and [Reading, 4.4] last bullet.
 *   q, k, v : bf16 inputs (device): q [T,H,d]; k, v [T,Hk,d].
 *   out     : filled qtensors (device buffers, caller-owned).
 * Per (document, 32-token block, head): optional fp32 Hadamard rotation of
 * Q and K rows; amax over the 32 x d block; exponent e = the smallest
 * integer with amax <= 448 * 2^e (rounded up so nothing clamps,
 * [Summary, §3.2 Causally Safe Scales]); codes = RNE_E4M3(x * 2^-e).
 * V also gets per-key exponents/codes and the per-query fold reference.
 * Mixed path: Q and K also get NVFP4 codes and scales (see flamia_qtensors);
 * the tensor scale needs the tensor-wide amax, so one more launch computes it
 * first.  Launches: the work-list builder (flamia_plan_build), (mixed path)
 * the amax pass, the quantizer.
 */
flamia_status flamia_quantize(const flamia_attn_desc* desc, const void* q, const void* k,
                              const void* v, const flamia_qtensors* out, hipStream_t stream);

/*
 * flamia_attn_fwd -- forward pass, [Summary] opening paragraphs and
 * [Reading, 4.1]/[Reading, 4.3]: S = Q~ K~^T on scaled FP8 matrix cores with
 * the token-block exponents as operand scales (the factorisation
 * S_ij = 2^(eQ(i)+eK(j)) x code dot product), causal mask within each
 * document, online softmax with an integer (rounded-up, log2-domain) row
 * maximum, P^ = E4M3(P * 2^8), per-key V scales folded into P on diagonal
 * 32-token blocks, O = sum P^ V / l.
 *   qt       : quantized operands from flamia_quantize.
 *   o        : bf16 [T,H,d] output (device).
 *   row_max  : int32 [H,T] integer row maximum m~ of S * softmax_scale * log2(e).
 *   row_sum  : fp32 [H,T] softmax denominator l = sum_j exp2(S'_ij - m~_i).
 *   ws       : fwd workspace (may be NULL when fwd_ws_bytes is 0).
 */
flamia_status flamia_attn_fwd(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* o,
                              int32_t* row_max, float* row_sum, void* ws, hipStream_t stream);

/*
 * flamia_attn_fwd_p4 -- the forward with the 4-bit probability operand,
 * [Summary, §3.5.2 Softmax Throughput and MMA Scheduling] and [Reading, 4.4]
 * second bullet: the probabilities of the NVFP4 path are quantized in the
 * log domain.  Everything is flamia_attn_fwd's but for the operand of the
 * P^V product: per query row and group of 16 consecutive keys (document-
 * aligned), a power-of-two scale 2^e with e the smallest integer such that
 * the group's largest P * 2^8 (times the diagonal fold) is at most 6 * 2^e,
 * E2M1 codes of the values over 2^e (round to nearest even), and the products
 * code x 2^e carried into the FP8 product as E4M3 values.  row_max and
 * row_sum are flamia_attn_fwd's (l sums the unquantized P).  Arguments as for
 * flamia_attn_fwd.  The backward is not defined for this forward's output
 * (its dV would need the same 4-bit operand).
 * Errors: FLAMIA_ERR_UNSUPPORTED on the mixed path, with the exact option or
 * with exp2_fma = 1; otherwise as flamia_attn_fwd.
 */
flamia_status flamia_attn_fwd_p4(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* o,
                                 int32_t* row_max, float* row_sum, void* ws, hipStream_t stream);

/*
 * flamia_attn_bwd -- backward pass, [Summary, §3.3 Forward-Backward Numerical
 * Consistency] and [Reading, 4.3]/[Reading, 4.4] third bullet: dO is
 * token-block quantized and D = rowsum(dO~ * O) is built from that same
 * payload; scores are recomputed from the same Q~/K~ codes with the same
 * matrix-core sequence, mask, exponential evaluation, stored integer row
 * maximum and diagonal fold as the forward, so the probability codes are
 * the forward's; dV = P^T (dO~/l); dP = dO~ V~^T; dS = P/l (dP - D) gets one
 * round-up exponent per 32x32 block; dK = dS^T Q~ and dQ = dS K~ (fp16
 * partials with a data-dependent power-of-two prescale, reduced with
 * atomics); with the rotation on, dQ and dK are rotated back.
 *   o, row_max, row_sum : forward outputs.
 *   dout                : bf16 [T,H,d] upstream gradient.
 *   dq, dk, dv          : bf16 gradients w.r.t. the unrotated q, k, v (dq [T,H,d];
 *                         dk, dv [T,Hk,d]).
 *   ws                  : bwd workspace of bwd_ws_bytes (device).
 * Four kernel launches: dO quantizer, backward, two finalisers.
 */
flamia_status flamia_attn_bwd(const flamia_attn_desc* desc, const flamia_qtensors* qt,
                              const void* o, const int32_t* row_max, const float* row_sum,
                              const void* dout, void* dq, void* dk, void* dv, void* ws,
                              hipStream_t stream);

/*
 * flamia_attn_bwd_noalloc -- flamia_attn_bwd without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a device array inside the library, 32 MiB on each GPU the
 * library runs on, held until the process ends; its address is looked up on
 * the first call on each device.  Same arguments, kernels and results as
 * flamia_attn_bwd otherwise.  Nothing is allocated or freed.
 * Errors: FLAMIA_ERR_WORKSPACE when the call's bwd_ws_bytes
 * (flamia_buffer_sizes) exceed 32 MiB; FLAMIA_ERR_INVALID_ARG when `stream`
 * does not belong to the current device; FLAMIA_ERR_HIP when the array's
 * address cannot be obtained; else as flamia_attn_bwd.
 * Every call on one GPU shares the array: calls that overlap on one GPU race.
 */
flamia_status flamia_attn_bwd_noalloc(const flamia_attn_desc* desc, const flamia_qtensors* qt,
                                      const void* o, const int32_t* row_max, const float* row_sum,
                                      const void* dout, void* dq, void* dk, void* dv, hipStream_t stream);

/*
 * The three stages of flamia_attn_bwd, for callers that schedule them
 * separately (e.g. to overlap the dO preparation with other work).  Calling
 * them in this order on one stream is exactly flamia_attn_bwd.
 *
 * flamia_attn_bwd_prep -- token-block E4M3 codes of dout, D = rowsum(dO~ O)
 *   from those codes ([Summary, §3.3]), G = dO~ 2^-8 / l in bf16, the dQ
 *   accumulator prescale exponent per query block, a zeroed fp16 dQ
 *   accumulator, and the per-query values the backward kernel reads with
 *   each query tile (8 - row_max, 2^-8 / row_sum, D, the prescale exponent,
 *   the Q / dO / fold-reference exponent bytes); all inside ws.  One launch.
 * flamia_attn_bwd_main -- the backward kernel: recompute, dV (bf16, written
 *   to dv), dK and dQ (fp16 accumulator in ws).  On the MXFP8 path dK is
 *   written to dk as bf16, rotated back when the Hadamard option is on; on
 *   the mixed path it goes to fp32 staging in ws and dk is not written here.
 *   Everything else it reads is in qt and ws.  One launch; two when grouped
 *   query attention splits each key/value head's group over several items
 *   (fewer than 512 (document, key tile, key/value head) items): the kernel
 *   then leaves fp32 dK/dV partials in ws and a second launch adds them in a
 *   fixed order and writes dk, dv (still rounded once, still deterministic).
 * flamia_attn_bwd_finish -- dQ to bf16 (rotated back when the Hadamard
 *   option is on; in deterministic mode first summed from the partial slots);
 *   on the mixed path also dK from its staging.  Reads the plan in qt.  One
 *   launch.
 */
flamia_status flamia_attn_bwd_prep(const flamia_attn_desc* desc, const flamia_qtensors* qt,
                                   const void* o, const int32_t* row_max, const float* row_sum,
                                   const void* dout, void* ws, hipStream_t stream);
flamia_status flamia_attn_bwd_main(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* dk,
                                   void* dv, void* ws, hipStream_t stream);
flamia_status flamia_attn_bwd_finish(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* dq,
                                     void* dk, void* ws, hipStream_t stream);

/*
 * Diagnostic entry points: flamia_attn_fwd and flamia_attn_bwd_main run as a
 * second instantiation of the same kernels that also reports what the pages
 * make checkable ([Summary, §3.3 Forward-Backward Numerical Consistency]):
 * the probability codes each pass computes, and the share of nonzero dS that
 * its 32x32 block scale rounds to zero ([Summary, §3.3] second bullet).
 * Same results as the plain calls.  Supported for the MXFP8 causal call
 * with num_kv_heads = num_heads, block scales and atomic dQ (exact = 0,
 * deterministic = 0); anything else returns FLAMIA_ERR_UNSUPPORTED.
 *
 * flamia_attn_fwd_diag -- flamia_attn_fwd, plus (when phat is not NULL):
 *   phat      uint8 [H, T, row_len]: E4M3 code of P^ (with the diagonal
 *             fold) of query token t and document-local key j, for every
 *             key the query sees, taken against the running integer row
 *             maximum of the 64-key step that holds the key; other bytes are
 *             left as they are.
 *   phat_max  int32 [H, T, ceil(row_len / 64)]: that running maximum per step.
 *   row_len   >= max_doc_len (else FLAMIA_ERR_INVALID_ARG).
 * flamia_attn_bwd_main_diag -- flamia_attn_bwd_main, plus:
 *   phat       (may be NULL) as above, the backward's recomputed codes,
 *              taken against the stored final row maximum.  Where P 2^8
 *              (times the fold) is at least 2^-6 (E4M3's normal range) the
 *              forward's code times 2^(run max - final max) equals it.
 *   ds_counts  (may be NULL) uint64[2]: nonzero dS entries, and those whose
 *              E4M3 code is zero; zeroed by the call before it counts.
 */
flamia_status flamia_attn_fwd_diag(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* o,
                                   int32_t* row_max, float* row_sum, void* ws, uint8_t* phat, int32_t* phat_max,
                                   int32_t row_len, hipStream_t stream);
flamia_status flamia_attn_bwd_main_diag(const flamia_attn_desc* desc, const flamia_qtensors* qt, void* dk,
                                        void* dv, void* ws, uint8_t* phat, int32_t row_len,
                                        uint64_t* ds_counts, hipStream_t stream);

/*
 * flamia_bwd_ws_layout -- where flamia_attn_bwd_prep leaves its payload
 * inside the backward workspace: byte offsets from ws, so a caller (or a
 * test) can read it back after the prep stage.  Host only.
 *   do_codes   [T,H,d] E4M3 token-block codes of dO (32 tokens of one
 *              document x d per exponent, no rotation) -- the one payload
 *              that dP and D are formed from ([Summary, §3.3])
 *   do_exp     [H,T] UE8M0 exponent of each token's dO block
 *   neg_delta  [H,T] fp32 -D_i, D_i = sum_d dO~_id O_id summed in fp32 over
 *              the stored bf16 O
 *   inv_l      [H,T] fp32 2^-8 / l_i (row_sum l_i)
 *   g          [T,H,d] bf16 G_i = dO~_i 2^-8 / l_i, the right operand of dV
 *   dq_sigma   [H,T] int32 exponent sigma_i of the fp16 dQ accumulator's
 *              power-of-two prescale ([Reading, 4.4] third bullet):
 *              e_dO(i) + E_V + E_K + log2 d + 13, E_V and E_K the largest V
 *              and K exponents of the document (of its blocks up to i's with
 *              causal_dq_scale; of its tokens up to i with the exact option)
 *   dq_acc     [T,H,d] fp16 dQ 2^-sigma_i, zeroed by the prep stage and summed
 *              by the main stage (atomic mode); flamia_attn_bwd_finish writes
 *              dq from it
 */
typedef struct flamia_bwd_ws_offsets {
  size_t do_codes, do_exp, neg_delta, inv_l, g, dq_sigma, dq_acc;
} flamia_bwd_ws_offsets;
flamia_status flamia_bwd_ws_layout(const flamia_attn_desc* desc, flamia_bwd_ws_offsets* out);

/*
 * flamia_tile_config -- tile sizes the kernels use for a head dim, i.e. the
 * Bq/Bk of the work-list cost model.  Host only.
 */
flamia_status flamia_tile_config(int32_t head_dim, int32_t* fwd_bq, int32_t* fwd_bk,
                                 int32_t* bwd_bq, int32_t* bwd_bk);

/*
 * flamia_plan_view -- where the work lists live inside qt->plan, so a caller
 * (or a test) can copy them back.  Host only.  Layout of the plan:
 *   int32 counts[4]   at byte 0: n_fwd_tiles, n_bwd_tiles, deterministic-mode
 *                     error word (see flamia_buffer_sizes), n_bwd_tiles again
 *                     (the dispatch list's count)
 *   int32 fwd[cap_fwd][2] at fwd_offset: (doc, q tile), longest first
 *   int32 bwd[cap_bwd][2] at bwd_offset: (doc, k tile), longest first
 *   int32 dispatch[cap_bwd][2] at bwd_dispatch_offset: the backward kernel's
 *                     launch order, a permutation of bwd that keeps each
 *                     document's key tiles together: documents by the cost of
 *                     their costliest (first) key tile, descending, then
 *                     document, then tile (so its query rows stay in L2
 *                     while its tiles run)
 * Sort key of fwd and bwd ([Summary, §3.6.2 Load-Balanced Scheduling];
 * [Reading, 4.4] last bullet): cost descending, then doc, then tile; each
 * tile expands to num_heads consecutive items, head ascending.  Any output
 * pointer may be NULL.
 */
flamia_status flamia_plan_view(const flamia_attn_desc* desc, size_t* fwd_offset, int32_t* cap_fwd,
                               size_t* bwd_offset, int32_t* cap_bwd, size_t* bwd_dispatch_offset);

/* Static description of a status code; never NULL. */
const char* flamia_status_string(flamia_status status);

#ifdef __cplusplus
}
#endif

#endif /* FLAMIA_H */
