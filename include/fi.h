/*
 * fi.h -- C ABI of a gfx950 (MI355X) library for batched attention over a
 * paged KV cache, decode and causal prefill, with fp16/bf16 queries and
 * outputs and K/V stored as OCP fp8 (e4m3 or e5m2) with per-tensor scales,
 * widened to the query's 2-byte type as they are loaded.  Beside these: fp8
 * queries with a per-tensor q_scale (the *_fp8q calls), fnuz fp8 caches
 * (decode, and prefill with a 2-byte query), and prefill over ragged
 * (non-paged) K/V or a single request.
 *
 * The problem statement these calls follow comes from three pages:
 *   [A] "Enable Hopper FA3 FP8 attention in decode.py" (flashinfer PR #2148):
 *       the plan()/run() arguments (paged_kv_indptr / indices /
 *       last_page_len, head counts, head_dim, page_size, q/kv/o dtypes,
 *       k_scale / v_scale), the output dtype that defaults to the query's and
 *       is never fp8 (Walkthrough; review comments), the output shape of q
 *       with V's head_dim (Nitpick comments), the split-KV plan knobs
 *       fixed_split_size / disable_split_kv (review comments).
 *   [B] "fallback to fa2 (instead of fa3) for unsupported configuration (bf16
 *       Q, Fp8 KV)" (flashinfer PR #2536): a 2-byte query against an fp8
 *       cache is a configuration a library must serve or refuse explicitly.
 *   [C] "fp8 KV cache in the in-tree prefill kernel" (AMD-Ecosystem/flashinfer
 *       PR #368): the refusal rules and their sentences (Refusals; Test plan),
 *       the k_scale / v_scale folds (Test plan), mixed 2-byte decode
 *       (Architecture / design notes), the OCP exponent biases (Architecture /
 *       design notes), the paged decode and causal prefill workloads
 *       (Benchmark results).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers marked [dev] are device (HBM) pointers on the current HIP
 *    device; [host] pointers are read by the host during the call only.
 *  - q and o are row-major [tokens, num_qo_heads, head_dim], contiguous.
 *    Decode has tokens = batch (one query per request); prefill is ragged by
 *    qo_indptr.  lse is [tokens, num_qo_heads] float32, natural log of the
 *    sum of exp(scaled logits); it may be NULL.
 *  - K and V page pools have element strides (stride_page, stride_token,
 *    stride_head); head_dim is contiguous.  The default layout is
 *    [num_pages, page_size, num_kv_heads, head_dim] ("NHD").
 *  - GQA: num_qo_heads % num_kv_heads == 0 and q head h reads kv head
 *    h / (num_qo_heads / num_kv_heads).
 *  - Token t of request i lives on page indices[indptr[i] + t / page_size],
 *    slot t % page_size; the request holds
 *    (indptr[i+1] - indptr[i] - 1) * page_size + last_page_len[i] tokens,
 *    or none when it has no pages (then o = 0 and lse = -inf).
 *  - Real K = stored K * k_scale, real V = stored V * v_scale ([A] review
 *    comments; [C] Test plan).  The stored fp8 code is widened exactly into
 *    q's 2-byte type; k_scale is folded into the logit scale and v_scale into
 *    the output before its single rounding -- the same arithmetic as scaling
 *    every element, with one rounding fewer.
 *  - sm_scale <= 0 selects 1/sqrt(head_dim).
 *  - Causal prefill: query row r of a request with qo_len queries and kv_len
 *    keys sees key t iff t <= r + kv_len - qo_len (aligned to the end of the
 *    KV sequence).
 *  - head_dim is 64 or 128; page_size is a power of two, 1..128; base
 *    pointers and strides give 16-byte aligned rows.
 *  - Calls are asynchronous on `stream` (a hipStream_t, NULL = the null
 *    stream).  The caller owns every buffer and keeps it alive until the
 *    stream has run the call.  The library allocates no memory and keeps no
 *    state between calls.  Host arrays must hold the same values as their
 *    device twins.
 *  - A call issues kernel launches only (no memory set or copy): the plan it
 *    derives from the host arrays travels in the kernel arguments, so a call
 *    made while `stream` is being captured into a HIP graph records its
 *    kernels, and each replay repeats the same plan on whatever the buffers
 *    then hold.  The host arrays are not read again at replay; a changed
 *    page table or batch needs a new capture.
 *
 * Errors
 * ------
 * Every call returns an fi_status.  On any status other than FI_OK no kernel
 * has been launched and o / lse are untouched (except FI_E_HIP, reported after
 * a launch failed).  fi_last_error() then returns a sentence naming the call,
 * the argument(s) and the dtype(s), e.g.
 *   "fi_batch_decode_paged: k has dtype float16 but v has dtype bfloat16".
 * Checks run in a fixed order: query dtype, output dtype, k/v dtype match,
 * KV dtype, (prefill) 2-byte KV equal to q, then shapes, pointers, alignment,
 * page table and scales, then workspace.  The fp8-query calls check in the
 * same order with their own rules: q in {E4M3, E5M2}, o_dtype given
 * explicitly as F16 or BF16, k == v, an fp8 cache (fnuz in decode only: the
 * fp8-query prefill feeds the raw codes to the OCP fp8 matrix cores),
 * then q_scale with the other scales.
 */
#ifndef FI_H_
#define FI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fi_dtype {
  FI_DTYPE_DEFAULT = 0, /* output only: the query's dtype ([A] Walkthrough) */
  FI_F16 = 1,
  FI_BF16 = 2,
  FI_F8_E4M3 = 3,      /* OCP e4m3 ("e4m3fn"), bias 7 ([C] design notes) */
  FI_F8_E5M2 = 4,      /* OCP e5m2, bias 15 */
  FI_F32 = 5,          /* refused everywhere */
  FI_I8 = 6,           /* refused: no float interpretation ([C] design notes) */
  FI_U8 = 7,           /* refused, as int8 */
  FI_F8_E4M3_FNUZ = 8, /* the gfx942 variant, bias 8 ([C] design notes); not with an fp8-query prefill */
  FI_F8_E5M2_FNUZ = 9  /* the gfx942 variant, bias 16; not with an fp8-query prefill */
} fi_dtype;

typedef enum fi_status {
  FI_OK = 0,
  FI_E_DTYPE = 1,     /* a dtype or dtype combination is refused */
  FI_E_SHAPE = 2,     /* a size, head count, head_dim or page_size is invalid */
  FI_E_ARG = 3,       /* a pointer, alignment, scale or page-table value is invalid */
  FI_E_WORKSPACE = 4, /* workspace present but smaller than fi_decode_workspace_bytes() */
  FI_E_HIP = 5        /* the HIP runtime reported an error (message included) */
} fi_status;

/* The paged K/V cache of one call ([A] plan() arguments). */
typedef struct fi_paged_kv {
  const void* k;                /* [dev] K page pool */
  const void* v;                /* [dev] V page pool (same strides as k) */
  fi_dtype k_dtype, v_dtype;    /* must be equal */
  int64_t stride_page;          /* elements between consecutive pages */
  int64_t stride_token;         /* elements between consecutive slots of a page */
  int64_t stride_head;          /* elements between consecutive kv heads */
  int32_t num_pages;            /* pages in each pool */
  int32_t page_size;            /* power of two, 1..128 */
  int32_t num_kv_heads;
  int32_t head_dim;             /* 64 or 128 */
  const int32_t* indptr;        /* [dev] [batch+1] page ranges per request */
  const int32_t* indices;       /* [dev] [indptr[batch]] page ids, each < num_pages */
  const int32_t* last_page_len; /* [dev] [batch] valid slots of the last page, 1..page_size */
  const int32_t* indptr_h;      /* [host] copy of indptr (planning and checks) */
  const int32_t* last_page_len_h; /* [host] copy of last_page_len */
  float k_scale, v_scale;       /* per-tensor, finite and > 0; 1.0 = none */
} fi_paged_kv;

/* The sentence describing the last non-FI_OK status returned on this thread
 * ("" if none).  The pointer stays valid until the next call on this thread. */
const char* fi_last_error(void);

/* Bytes of device workspace that fi_batch_decode_paged and fi_single_decode
 * may use for split-KV partial states, for any call whose longest request has
 * at most max_kv_len tokens.  Split-KV divides a long request into chunks
 * processed in parallel and merges their (output, log-sum-exp) states
 * ([A] review comments: fixed_split_size / disable_split_kv). */
size_t fi_decode_workspace_bytes(int32_t batch, int32_t num_qo_heads, int32_t head_dim, int32_t max_kv_len);

/* Batched decode: one query token per request against its paged K/V.
 *   q        [dev] [batch, num_qo_heads, head_dim], q_dtype in {FI_F16, FI_BF16}
 *   kv       the paged cache; KV dtype in {F16, BF16, E4M3, E5M2, E4M3_FNUZ,
 *            E5M2_FNUZ} (fnuz: widened exactly, as in prefill).  A 2-byte KV
 *            dtype may differ from q's ([C] design notes: mixed 2-byte decode
 *            is correct); the products then run in bf16 with every fp16
 *            value split exactly into two bf16 parts, so nothing is rounded
 *            and nothing can overflow.
 *   o        [dev] [batch, num_qo_heads, head_dim] of o_dtype
 *            (FI_DTYPE_DEFAULT = q_dtype; fp8 refused)
 *   lse      [dev] [batch, num_qo_heads] float32, or NULL
 *   workspace [dev] split-KV scratch, or NULL to process each request in one
 *            piece (disable_split_kv).  If non-NULL, workspace_bytes must be at
 *            least fi_decode_workspace_bytes(batch, num_qo_heads, head_dim,
 *            longest kv_len).
 * Environment: FI_SPLIT_KV = "off" disables splitting, a positive integer
 * forces that many tokens per chunk (rounded up to a multiple of 64), unset
 * or "auto" lets the planner choose (fixed_split_size).  FI_DECODE_WAVES = 4
 * or 8 forces the decode workgroup size (8: for a 2-byte query over an OCP
 * fp8 cache or one of its own type, under the planner's balanced split);
 * unset, 8 is used where a workgroup's slice holds at least 1 MB of K/V. */
fi_status fi_batch_decode_paged(const void* q, fi_dtype q_dtype, int32_t batch, int32_t num_qo_heads,
                                const fi_paged_kv* kv, void* o, fi_dtype o_dtype, float* lse, float sm_scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Batched decode that allocates nothing and takes no workspace: for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Arguments, dtype rules,
 * results and the split-KV plan are those of fi_batch_decode_paged with a
 * workspace, and the output is bit-identical to it; the split-KV partial
 * states go to a scratch array the library holds in device memory, one copy
 * per GPU, FI_DECODE_SCRATCH_BYTES long, kept until the process ends.
 * A batch whose split needs more scratch than that is refused with
 * FI_E_WORKSPACE (no kernel launched; fi_batch_decode_paged with a workspace
 * of fi_decode_workspace_bytes() has no such limit).  No memory is allocated,
 * set or copied.  Every call on a GPU shares that GPU's scratch, so two calls
 * that overlap in time on one GPU (different streams, or host threads) race:
 * the caller serialises them, e.g. on one stream. */
#define FI_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
fi_status fi_batch_decode_paged_noalloc(const void* q, fi_dtype q_dtype, int32_t batch, int32_t num_qo_heads,
                                        const fi_paged_kv* kv, void* o, fi_dtype o_dtype, float* lse, float sm_scale,
                                        void* stream);

/* Batched decode with an fp8 query ([A]: fp8 attention in decode.py; review
 * comments: q_scale folded into sm_scale for the first product).
 *   q        [dev] [batch, num_qo_heads, head_dim] fp8 codes, q_dtype in
 *            {FI_F8_E4M3, FI_F8_E5M2}; real q = code * q_scale
 *   q_scale  per-tensor, finite and > 0
 *   kv       an fp8 cache: E4M3, E5M2, E4M3_FNUZ or E5M2_FNUZ
 *   o_dtype  FI_F16 or FI_BF16, given explicitly
 * Other arguments, the split-KV workspace and results as
 * fi_batch_decode_paged.  The codes are widened exactly to fp16 as they are
 * loaded and the products run as with an fp16 query, so the result matches
 * fi_batch_decode_paged on the widened values (with sm_scale * q_scale). */
fi_status fi_batch_decode_paged_fp8q(const void* q, fi_dtype q_dtype, float q_scale, int32_t batch,
                                     int32_t num_qo_heads, const fi_paged_kv* kv, void* o, fi_dtype o_dtype,
                                     float* lse, float sm_scale, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Batched prefill over the paged cache ([C] Summary and Refusals).
 *   q          [dev] [qo_indptr[batch], num_qo_heads, head_dim]
 *   qo_indptr  [dev] [batch+1] query ranges; qo_indptr_h its [host] copy.
 *   causal     nonzero: mask aligned to the end of the KV sequence.
 *   A 2-byte KV dtype must equal q_dtype ([C] Refusals: prefill reads KV
 *   fragments as the query type); fp8 KV -- OCP, or the gfx942 fnuz layouts
 *   ([C] Architecture / design notes), widened exactly from their bits -- is
 *   widened on load.
 *   workspace / workspace_bytes are unused (prefill does not split) and may be
 *   NULL / 0. */
fi_status fi_batch_prefill_paged(const void* q, fi_dtype q_dtype, const int32_t* qo_indptr,
                                 const int32_t* qo_indptr_h, int32_t batch, int32_t num_qo_heads,
                                 const fi_paged_kv* kv, int32_t causal, void* o, fi_dtype o_dtype, float* lse,
                                 float sm_scale, void* workspace, size_t workspace_bytes, void* stream);

/* A prefill batch and a decode batch in one launch ("POD"; [C] Refusals and
 * Architecture / design notes: the POD and batch-POD run entry points beside
 * prefill and decode, with the prefill dtype rules and the k/v check).
 *   prefill phase: q_p, qo_indptr / qo_indptr_h, batch_p, kv_p, causal, o_p,
 *     lse_p -- as fi_batch_prefill_paged;
 *   decode phase: q_d, batch_d, kv_d, o_d, lse_d -- as fi_batch_decode_paged,
 *     one query per request;
 *   q_dtype, o_dtype (FI_DTYPE_DEFAULT = q_dtype), num_qo_heads and sm_scale
 *     are shared, as is one KV dtype: kv_p and kv_d must have the same dtype,
 *     num_kv_heads and head_dim (one kernel runs both phases; a mismatch
 *     between the phases is refused, never reinterpreted), and a 2-byte KV
 *     must equal q in both phases ([C]: "on prefill and POD").  fp8 KV (OCP
 *     or fnuz) is widened on load as in the other calls.  kv_p and kv_d may
 *     describe the same pools with different page tables, or different pools;
 *     each phase has its own k_scale / v_scale.
 *   workspace / workspace_bytes: the decode phase's split-KV scratch, as for
 *     fi_batch_decode_paged (NULL: no split).
 * Results are those of the two separate calls (the prefill phase bit for bit;
 * the decode phase within tolerance: it is cut into slices for 8-wave
 * workgroups instead of the decode kernel's 4).  The prefill phase may hold at
 * most 384 (request, block of 256 / heads_per_group query rows) pairs, which
 * the launch's arguments carry; more is refused with FI_E_SHAPE.  Checks run
 * in the order of fi_batch_prefill_paged for the prefill phase, then the same
 * for the decode phase (its sentences name "(decode phase)"), then the
 * cross-phase dtype and head checks, shapes and pointers, then workspace.
 * The launch puts the decode slices first, on a share of the compute units
 * sized so that the decode phase takes about half of the launch's estimated
 * time (a decode stream needs bandwidth more than CUs), and the prefill items
 * on the rest and on the units the decode slices leave.
 * Environment: FI_POD_DECODE_WG = a positive count of decode workgroups to
 * cut the decode phase into (default: that share; two per compute unit when
 * the prefill phase is empty); FI_POD_ORDER = "prefill_first" dispatches the
 * prefill items first. */
fi_status fi_batch_pod_paged(const void* q_p, const int32_t* qo_indptr, const int32_t* qo_indptr_h, int32_t batch_p,
                             const fi_paged_kv* kv_p, int32_t causal, void* o_p, float* lse_p, const void* q_d,
                             int32_t batch_d, const fi_paged_kv* kv_d, void* o_d, float* lse_d, fi_dtype q_dtype,
                             fi_dtype o_dtype, int32_t num_qo_heads, float sm_scale, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Batched prefill over the paged cache with an fp8 query ([A] review
 * comments: q_scale folded into sm_scale for the first product; [A]
 * Walkthrough and review comments: an fp8 input gives a float16 or bfloat16
 * output, never fp8).
 *   q        [dev] [qo_indptr[batch], num_qo_heads, head_dim] fp8 codes,
 *            q_dtype in {FI_F8_E4M3, FI_F8_E5M2}; real q = code * q_scale
 *   q_scale  per-tensor, finite and > 0
 *   kv       the paged cache; KV dtype in {E4M3, E5M2} (either, with either
 *            query format)
 *   o_dtype  FI_F16 or FI_BF16, given explicitly (FI_DTYPE_DEFAULT, the
 *            query's own dtype, is refused)
 *   pv_fp8   0: P V in float16 (P rounded to float16, V widened exactly);
 *            nonzero: P rounded to e4m3 (round to nearest even) and P V on
 *            the fp8 matrix cores with V staying fp8 ([A] and [B]: the FA3
 *            fp8 path quantises the probabilities for the second product)
 * Other arguments, layouts, the causal mask and results as
 * fi_batch_prefill_paged.  S = Q K^T runs on the fp8 matrix cores with K
 * staying fp8 from HBM to the MFMA; the products are exact and summed in
 * fp32 as in the 2-byte path.  With pv_fp8 = 0 the result matches the 2-byte
 * path to the same tolerance.  With pv_fp8 set, each probability carries a
 * relative rounding error of at most 2^-4 (absolute 2^-10 of the row's
 * reference maximum below 2^-6 of it); the output is normalised by the fp32
 * sum of the unrounded probabilities, which also gives lse. */
fi_status fi_batch_prefill_paged_fp8q(const void* q, fi_dtype q_dtype, float q_scale, const int32_t* qo_indptr,
                                      const int32_t* qo_indptr_h, int32_t batch, int32_t num_qo_heads,
                                      const fi_paged_kv* kv, int32_t causal, int32_t pv_fp8, void* o,
                                      fi_dtype o_dtype, float* lse, float sm_scale, void* stream);

/* K/V held contiguously per request ("ragged"): request i owns rows
 * indptr[i] .. indptr[i+1]-1 of each pool, row r of kv head g at element
 * r * stride_token + g * stride_head.  The default layout is
 * [num_tokens, num_kv_heads, head_dim].  Same dtype and scale rules as
 * fi_paged_kv. */
typedef struct fi_ragged_kv {
  const void* k;                /* [dev] K rows */
  const void* v;                /* [dev] V rows (same strides as k) */
  fi_dtype k_dtype, v_dtype;    /* must be equal */
  int64_t stride_token;         /* elements between consecutive rows */
  int64_t stride_head;          /* elements between consecutive kv heads */
  int32_t num_tokens;           /* rows in each pool; indptr[batch] <= num_tokens */
  int32_t num_kv_heads;
  int32_t head_dim;             /* 64 or 128 */
  const int32_t* indptr;        /* [dev] [batch+1] row ranges per request */
  const int32_t* indptr_h;      /* [host] copy of indptr */
  float k_scale, v_scale;       /* per-tensor, finite and > 0; 1.0 = none */
} fi_ragged_kv;

/* Batched prefill over a ragged (non-paged) K/V: the batch-prefill run entry
 * point without a page table ([C] Architecture / design notes: the ragged
 * wrapper and the run entry points that share the k/v dtype check; Test plan:
 * the fp8 equivalence across single, paged and ragged).  Arguments, layouts,
 * refusals and results as fi_batch_prefill_paged, with request i's kv_len =
 * indptr[i+1] - indptr[i] (0: o = 0 and lse = -inf).  The same kernel runs,
 * addressing rows instead of pages, so a ragged call and a paged call over the
 * same K/V values give identical bits. */
fi_status fi_batch_prefill_ragged(const void* q, fi_dtype q_dtype, const int32_t* qo_indptr,
                                  const int32_t* qo_indptr_h, int32_t batch, int32_t num_qo_heads,
                                  const fi_ragged_kv* kv, int32_t causal, void* o, fi_dtype o_dtype, float* lse,
                                  float sm_scale, void* stream);

/* Prefill of one request against a contiguous K/V ([C] Architecture / design
 * notes: the single-prefill run entry point).  q and o are [dev]
 * [qo_len, num_qo_heads, head_dim]; k and v are [dev] [kv_len, num_kv_heads,
 * head_dim]; lse is [qo_len, num_qo_heads] float32 or NULL.  Dtype rules,
 * causal mask and results as fi_batch_prefill_paged with one request; no
 * device index array is needed (the lengths travel in the kernel arguments). */
fi_status fi_single_prefill(const void* q, fi_dtype q_dtype, int32_t qo_len, const void* k, const void* v,
                            fi_dtype k_dtype, fi_dtype v_dtype, int32_t kv_len, int32_t num_qo_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t causal, float k_scale, float v_scale,
                            void* o, fi_dtype o_dtype, float* lse, float sm_scale, void* stream);

/* The ragged and single prefill calls with an fp8 query: q holds e4m3 / e5m2
 * codes with a per-tensor q_scale (real q = code * q_scale), o_dtype is given
 * explicitly as F16 or BF16, and the cache is OCP fp8 -- the dtype rules,
 * q_scale fold and pv_fp8 mode of fi_batch_prefill_paged_fp8q, with the K/V
 * addressing of fi_batch_prefill_ragged / fi_single_prefill.  Over the same
 * values a ragged, single and paged fp8-query call give identical bits. */
fi_status fi_batch_prefill_ragged_fp8q(const void* q, fi_dtype q_dtype, float q_scale, const int32_t* qo_indptr,
                                       const int32_t* qo_indptr_h, int32_t batch, int32_t num_qo_heads,
                                       const fi_ragged_kv* kv, int32_t causal, int32_t pv_fp8, void* o,
                                       fi_dtype o_dtype, float* lse, float sm_scale, void* stream);
fi_status fi_single_prefill_fp8q(const void* q, fi_dtype q_dtype, float q_scale, int32_t qo_len, const void* k,
                                 const void* v, fi_dtype k_dtype, fi_dtype v_dtype, int32_t kv_len,
                                 int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t causal,
                                 int32_t pv_fp8, float k_scale, float v_scale, void* o, fi_dtype o_dtype, float* lse,
                                 float sm_scale, void* stream);

/* Decode of one query against a contiguous K/V ([C] Summary: the single-decode
 * entry point).  k and v are [dev] [kv_len, num_kv_heads, head_dim] with the
 * same dtype rules as fi_batch_decode_paged; q and o are
 * [num_qo_heads, head_dim]; lse is [num_qo_heads] or NULL. */
fi_status fi_single_decode(const void* q, fi_dtype q_dtype, const void* k, const void* v, fi_dtype k_dtype,
                           fi_dtype v_dtype, int32_t kv_len, int32_t num_qo_heads, int32_t num_kv_heads,
                           int32_t head_dim, float k_scale, float v_scale, void* o, fi_dtype o_dtype, float* lse,
                           float sm_scale, void* workspace, size_t workspace_bytes, void* stream);

/* Widen n fp8 codes into a 2-byte type with the same device conversion the
 * attention kernels use (no scaling; the e4m3fnuz values, which the kernels
 * hold as value * 2^-7 with 2^7 folded into their scales, are returned as the
 * values themselves).  src in {E4M3, E5M2, E4M3_FNUZ, E5M2_FNUZ}, dst in
 * {F16, BF16}; the fnuz NaN code 0x80 reads as a quiet NaN;
 * codes [dev] [n] bytes, out [dev] [n] 2-byte values.  This makes the
 * conversion testable code by code ([C] design notes: the vec_cast paragraph
 * records a decoder with the wrong bias and broken denormals that no test
 * could reach). */
fi_status fi_fp8_widen(const uint8_t* codes, int64_t n, fi_dtype src, fi_dtype dst, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FI_H_ */
