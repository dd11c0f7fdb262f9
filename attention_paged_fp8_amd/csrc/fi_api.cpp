// Host front end of the C ABI declared in include/fi.h: argument checks in a
// fixed order (no HIP call before they pass), the split-KV plan, and the
// kernel launches.
//
// The refusal rules and their wording follow "fp8 KV cache in the in-tree
// prefill kernel" (AMD-Ecosystem/flashinfer PR #368), sections Refusals and
// Architecture / design notes: q and o are 2-byte floats; the output is never
// fp8 ("Enable Hopper FA3 FP8 attention in decode.py", flashinfer PR #2148,
// Walkthrough); k and v must share a dtype; int8/uint8 KV has no float
// interpretation; a 2-byte KV must equal q for prefill while decode converts
// it; nothing is ever cast silently.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "fi.h"
#include "fi_internal.h"

namespace {

thread_local std::string g_err;

fi_status fail(fi_status st, const char* fn, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = std::string(fn) + ": " + buf;
  return st;
}

const char* dtype_name(fi_dtype d) {
  switch (d) {
    case FI_DTYPE_DEFAULT: return "default";
    case FI_F16: return "float16";
    case FI_BF16: return "bfloat16";
    case FI_F8_E4M3: return "float8_e4m3fn";
    case FI_F8_E5M2: return "float8_e5m2";
    case FI_F32: return "float32";
    case FI_I8: return "int8";
    case FI_U8: return "uint8";
    case FI_F8_E4M3_FNUZ: return "float8_e4m3fnuz";
    case FI_F8_E5M2_FNUZ: return "float8_e5m2fnuz";
  }
  return "unknown";
}

bool is_2byte(fi_dtype d) { return d == FI_F16 || d == FI_BF16; }
bool is_ocp_fp8(fi_dtype d) { return d == FI_F8_E4M3 || d == FI_F8_E5M2; }
bool is_any_fp8(fi_dtype d) {
  return is_ocp_fp8(d) || d == FI_F8_E4M3_FNUZ || d == FI_F8_E5M2_FNUZ;
}
int elem_bytes(fi_dtype d) { return is_2byte(d) ? 2 : 1; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks 1-5 of the documented order.  `prefill` enables the 2-byte rule.
fi_status check_dtypes(const char* fn, fi_dtype q, fi_dtype* o, fi_dtype k, fi_dtype v, bool prefill) {
  if (!is_2byte(q)) {
    if (is_any_fp8(q))
      return fail(FI_E_DTYPE, fn, "q has dtype %s; an fp8 query is not supported (q must be float16 or bfloat16, "
                  "and it is never cast silently; fi_batch_prefill_paged_fp8q takes an fp8 query with its scale)",
                  dtype_name(q));
    return fail(FI_E_DTYPE, fn, "q has dtype %s; q must be float16 or bfloat16", dtype_name(q));
  }
  if (*o == FI_DTYPE_DEFAULT) *o = q;
  if (is_any_fp8(*o))
    return fail(FI_E_DTYPE, fn, "o has dtype %s; an fp8 output is not supported (o must be float16 or bfloat16)",
                dtype_name(*o));
  if (!is_2byte(*o)) return fail(FI_E_DTYPE, fn, "o has dtype %s; o must be float16 or bfloat16", dtype_name(*o));
  if (k != v) return fail(FI_E_DTYPE, fn, "k has dtype %s but v has dtype %s", dtype_name(k), dtype_name(v));
  if (k == FI_I8 || k == FI_U8)
    return fail(FI_E_DTYPE, fn, "KV cache has dtype %s, which has no float interpretation; KV must be float16, "
                "bfloat16, float8_e4m3fn or float8_e5m2", dtype_name(k));
  if (!is_2byte(k) && !is_any_fp8(k))
    return fail(FI_E_DTYPE, fn, "KV cache has dtype %s; KV must be float16, bfloat16, float8_e4m3fn, float8_e5m2, "
                "float8_e4m3fnuz or float8_e5m2fnuz", dtype_name(k));
  if (prefill && is_2byte(k) && k != q)
    return fail(FI_E_DTYPE, fn, "q has dtype %s but the KV cache has dtype %s; prefill needs a 2-byte KV cache of the "
                "query's dtype (fp8 KV is widened on load)", dtype_name(q), dtype_name(k));
  return FI_OK;
}

// Checks 1-5 for a call that takes an fp8 query: q in {e4m3, e5m2}; o given
// explicitly as a 2-byte type (the default, q's dtype, would be fp8); k == v;
// an fp8 KV cache (fnuz too where `fnuz` is set: decode).
fi_status check_dtypes_fp8q(const char* fn, fi_dtype q, fi_dtype o, fi_dtype k, fi_dtype v, bool fnuz = false) {
  if (!is_ocp_fp8(q))
    return fail(FI_E_DTYPE, fn, "q has dtype %s; this call takes an fp8 query (float8_e4m3fn or float8_e5m2)",
                dtype_name(q));
  if (o == FI_DTYPE_DEFAULT)
    return fail(FI_E_DTYPE, fn, "o_dtype must be given for an fp8 query (float16 or bfloat16; the query's own dtype "
                "is fp8, and an fp8 output is not supported)");
  if (is_any_fp8(o))
    return fail(FI_E_DTYPE, fn, "o has dtype %s; an fp8 output is not supported (o must be float16 or bfloat16)",
                dtype_name(o));
  if (!is_2byte(o)) return fail(FI_E_DTYPE, fn, "o has dtype %s; o must be float16 or bfloat16", dtype_name(o));
  if (k != v) return fail(FI_E_DTYPE, fn, "k has dtype %s but v has dtype %s", dtype_name(k), dtype_name(v));
  if (k == FI_I8 || k == FI_U8)
    return fail(FI_E_DTYPE, fn, "KV cache has dtype %s, which has no float interpretation; KV must be "
                "float8_e4m3fn or float8_e5m2", dtype_name(k));
  if (!fnuz && (k == FI_F8_E4M3_FNUZ || k == FI_F8_E5M2_FNUZ))
    return fail(FI_E_DTYPE, fn, "KV cache has dtype %s, the gfx942 fnuz variant; an fp8-query prefill runs the "
                "OCP fp8 matrix cores on the raw codes (fnuz caches are read with a float16 or bfloat16 query, "
                "or by fi_batch_decode_paged_fp8q)", dtype_name(k));
  if (!is_any_fp8(k))
    return fail(FI_E_DTYPE, fn, "q has dtype %s but the KV cache has dtype %s; an fp8 query needs an fp8 KV cache "
                "(float8_e4m3fn or float8_e5m2)", dtype_name(q), dtype_name(k));
  return FI_OK;
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

fi_status check_heads(const char* fn, int32_t hqo, int32_t hkv, int32_t d) {
  if (hqo <= 0 || hkv <= 0) return fail(FI_E_SHAPE, fn, "head counts must be positive (num_qo_heads=%d, num_kv_heads=%d)", hqo, hkv);
  if (hqo % hkv != 0)
    return fail(FI_E_SHAPE, fn, "num_qo_heads=%d is not a multiple of num_kv_heads=%d", hqo, hkv);
  if (d != 64 && d != 128) return fail(FI_E_SHAPE, fn, "head_dim=%d; supported head_dim values are 64 and 128", d);
  return FI_OK;
}

fi_status check_scales(const char* fn, float k_scale, float v_scale, float sm_scale) {
  if (!std::isfinite(k_scale) || !(k_scale > 0.f)) return fail(FI_E_ARG, fn, "k_scale=%g must be finite and > 0", k_scale);
  if (!std::isfinite(v_scale) || !(v_scale > 0.f)) return fail(FI_E_ARG, fn, "v_scale=%g must be finite and > 0", v_scale);
  if (!std::isfinite(sm_scale)) return fail(FI_E_ARG, fn, "sm_scale=%g must be finite (<= 0 selects 1/sqrt(head_dim))", sm_scale);
  return FI_OK;
}

// Checks on the paged cache: shape, pointers, alignment and the host page table.
// On success *max_kv and *total_kv hold the longest and the summed kv_len.
fi_status check_paged(const char* fn, int32_t batch, const fi_paged_kv* kv, int64_t* max_kv, int64_t* total_kv) {
  const int eb = elem_bytes(kv->k_dtype);
  if (!pow2(kv->page_size) || kv->page_size > 128)
    return fail(FI_E_SHAPE, fn, "page_size=%d; page_size must be a power of two from 1 to 128", kv->page_size);
  if (kv->num_pages < 0) return fail(FI_E_SHAPE, fn, "num_pages=%d is negative", kv->num_pages);
  if (kv->stride_page <= 0 || kv->stride_token <= 0 || kv->stride_head <= 0)
    return fail(FI_E_SHAPE, fn, "strides must be positive (page %lld, token %lld, head %lld)",
                (long long)kv->stride_page, (long long)kv->stride_token, (long long)kv->stride_head);
  if (kv->stride_page * eb >= (1ll << 32) || kv->stride_token * eb >= (1ll << 32) || kv->stride_head * eb >= (1ll << 32))
    return fail(FI_E_SHAPE, fn, "K/V strides must be below 4 GiB");
  if ((kv->stride_page * eb) % 16 || (kv->stride_token * eb) % 16 || (kv->stride_head * eb) % 16)
    return fail(FI_E_ARG, fn, "K/V strides must give 16-byte aligned rows (page %lld, token %lld, head %lld elements "
                "of %d bytes)", (long long)kv->stride_page, (long long)kv->stride_token, (long long)kv->stride_head, eb);
  if (batch > 0) {
    if (!kv->k || !kv->v) return fail(FI_E_ARG, fn, "k and v page pools must not be NULL");
    if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(FI_E_ARG, fn, "k and v page pools must be 16-byte aligned");
    if (!kv->indptr || !kv->indices || !kv->last_page_len)
      return fail(FI_E_ARG, fn, "indptr, indices and last_page_len (device) must not be NULL");
    if (!kv->indptr_h || !kv->last_page_len_h)
      return fail(FI_E_ARG, fn, "indptr_h and last_page_len_h (host copies) must not be NULL");
  }
  int64_t mx = 0, tot = 0;
  if (batch > 0 && kv->indptr_h[0] < 0) return fail(FI_E_ARG, fn, "indptr[0]=%d is negative", kv->indptr_h[0]);
  for (int32_t i = 0; i < batch; ++i) {
    const int32_t a = kv->indptr_h[i], e = kv->indptr_h[i + 1];
    if (e < a) return fail(FI_E_ARG, fn, "indptr is decreasing at request %d (%d > %d)", i, a, e);
    const int32_t np = e - a;
    int64_t len = 0;
    if (np > 0) {
      const int32_t lp = kv->last_page_len_h[i];
      if (lp < 1 || lp > kv->page_size)
        return fail(FI_E_ARG, fn, "last_page_len[%d]=%d is outside [1, page_size=%d]", i, lp, kv->page_size);
      len = (int64_t)(np - 1) * kv->page_size + lp;
    }
    if (len >= (1ll << 30)) return fail(FI_E_SHAPE, fn, "request %d has %lld tokens; at most 2^30 - 1 are supported", i, (long long)len);
    mx = len > mx ? len : mx;
    tot += len;
  }
  *max_kv = mx;
  *total_kv = tot;
  return FI_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

#ifndef FI_DECODE_MIN_CHUNK
#define FI_DECODE_MIN_CHUNK 256
#endif
#ifndef FI_DECODE_TARGET_WG
#define FI_DECODE_TARGET_WG 2048
#endif
constexpr int kMinAutoChunk = FI_DECODE_MIN_CHUNK;  // smallest chunk the planner picks by itself
#ifndef FI_DECODE_INTERLEAVE
#define FI_DECODE_INTERLEAVE 1
#endif
constexpr int kTargetWorkgroups = FI_DECODE_TARGET_WG;  // workgroups the planner aims for

// Split-KV plan: tokens per chunk (a multiple of kChunkQuantum); a chunk that
// covers the longest request means no split.  `groups` workgroups share each
// token (kv head groups x row-slice groups).
int64_t plan_chunk(int64_t max_kv, int64_t total_kv, int64_t groups, bool have_ws) {
  const int64_t q = fi::kChunkQuantum;
  const int64_t whole = std::max<int64_t>(q, round_up(std::max<int64_t>(max_kv, 1), q));
  if (!have_ws) return whole;
  const char* env = std::getenv("FI_SPLIT_KV");
  if (env && *env && std::strcmp(env, "auto") != 0) {
    if (std::strcmp(env, "off") == 0) return whole;
    const long n = std::strtol(env, nullptr, 10);
    if (n > 0) return std::min(whole, std::max<int64_t>(q, round_up(n, q)));
  }
  const int64_t work = total_kv * groups;
  int64_t c = round_up(std::max<int64_t>(1, ceil_div(work, kTargetWorkgroups)), q);
  c = std::max<int64_t>(c, kMinAutoChunk);
  return std::min(c, whole);
}

size_t partial_bytes(int64_t batch, int64_t max_chunks, int64_t hqo, int64_t d) {
  if (max_chunks <= 1) return 0;
  return (size_t)(batch * max_chunks * hqo * (d + 1) * 4);
}

// The split-KV plan of a decode batch, for NW-wave workgroups: workgroup
// shape (kv heads and GQA row slices per workgroup), then either the balanced
// split (equal slices of the (group, request, token) space, one per
// workgroup slot; needs a workspace) or fixed chunks.  `slots` > 0 gives the
// number of balanced slices to aim for; 0 takes the device's resident
// capacity for the 4-wave decode kernel with the rule below.  On return
// *merge says whether some segment was split (or a request is empty) and
// *need is the workspace the partial states take.
template <class DP>
fi_status plan_decode(const char* fn, DP& p, int nw, int slots, fi_dtype q_dtype, fi_dtype kv_dtype,
                      fi_dtype o_dtype, int32_t batch, int32_t head_dim, const int32_t* indptr_h,
                      const int32_t* last_page_len_h, int32_t page_size, int64_t max_kv, int64_t total_kv,
                      bool have_ws, bool* merge_out, size_t* need_out) {
  // Workgroup shape: up to nw waves, one per (kv head, 16-row slice of its GQA
  // group); the heads of a workgroup are adjacent, so each token's rows of
  // those heads are read as one contiguous run.
  const int nsub = (p.group + fi::kDecodeRows - 1) / fi::kDecodeRows;
  p.nsub = nsub;
  p.spw = nsub <= nw ? nsub : nw;
  const int max_hpw = nw / p.spw;
  const int max_shift = ilog2(nw);
  int hpw_shift = 0;
  while (hpw_shift < max_shift && (2 << hpw_shift) <= max_hpw && p.num_kv_heads % (2 << hpw_shift) == 0) ++hpw_shift;
  p.hpw_shift = hpw_shift;
  p.n_hgroups = p.num_kv_heads >> hpw_shift;
  p.n_sgroups = (nsub + p.spw - 1) / p.spw;
  const int64_t groups = (int64_t)p.n_hgroups * p.n_sgroups;
  p.batch = batch;

  // kv length of request i from the host copy of the page table
  auto kv_of = [&](int i) -> int64_t {
    if (!indptr_h) return total_kv;
    const int32_t np = indptr_h[i + 1] - indptr_h[i];
    return np > 0 ? (int64_t)(np - 1) * page_size + last_page_len_h[i] : 0;
  };
  const char* env = std::getenv("FI_SPLIT_KV");
  const bool forced = env && *env && std::strcmp(env, "auto") != 0;
  bool merge = false;
  bool empty_any = false;
  for (int32_t i = 0; i < batch; ++i) empty_any |= (kv_of(i) == 0);

  // Balanced split: equal slices of the (group, request, token) space, one per
  // workgroup slot of the device (the default whenever a workspace is given).
  p.balanced = 0;
  if (have_ws && !forced && batch <= fi::kBalancedMaxBatch && total_kv > 0) {
    if (slots <= 0) {
      // Workgroups: the device's resident capacity (CUs x occupancy), except
      // that short streams run better at 2 per CU -- fewer, longer slices split
      // fewer requests and spread start-up over more bytes (measured: a slice
      // under ~640 KB of K/V loses at 3 per CU, one over ~850 KB gains).
      slots = fi::decode_slots(q_dtype, kv_dtype, o_dtype, head_dim, nw);
      const int cus = fi::device_cus();
      if (slots > 0 && cus > 0 && slots / cus > 2) {
        const int64_t row_bytes = (int64_t)(1 << hpw_shift) * head_dim * elem_bytes(kv_dtype) * 2;  // K + V per item
        if (ceil_div(total_kv * groups, slots) * row_bytes < (640 << 10)) slots = 2 * cus;
      }
    }
    if (slots > 0) {
      const int64_t W = total_kv * groups;
      int64_t slice = round_up(ceil_div(W, slots), fi::kDecodeStep);
      slice = std::max<int64_t>(slice, fi::kChunkQuantum);
      p.balanced = 1;
      p.slice = slice;
      p.pre_n = 0;
      if (batch <= DP::kPrefixMax && total_kv < 0x7fffffff) {
        int64_t run = 0;
        for (int32_t i = 0; i < batch; ++i) {
          p.pre[i] = (int32_t)run;
          run += kv_of(i);
        }
        p.pre[batch] = (int32_t)run;
        p.pre_n = batch + 1;
      }
      p.spg = 0;
      if (FI_DECODE_INTERLEAVE && groups > 1) {
        // every group cut into the same token slices (a few more workgroups than
        // the group-major cut at most: widen the slice until they fit the slots)
        while (groups * ceil_div(total_kv, slice) > slots && slice < total_kv) slice += fi::kDecodeStep;
        p.slice = slice;
        p.spg = (int32_t)ceil_div(total_kv, slice);
        p.n_wg = (int32_t)(groups * p.spg);
      } else {
        p.n_wg = (int32_t)ceil_div(W, slice);
      }
      p.max_chunks = (int32_t)(ceil_div(std::max<int64_t>(max_kv, 1), slice) + 1);
      p.chunk = 0;
      // a merge is needed if some (request, group) segment spans several slices
      int64_t pre = 0;
      for (int32_t i = 0; i < batch && !merge; ++i) {
        const int64_t len = kv_of(i);
        for (int64_t gi = 0; gi < groups && len > 0; ++gi) {
          const int64_t s0 = (p.spg ? 0 : gi * total_kv) + pre, s1 = s0 + len;
          if (s0 / slice != (s1 - 1) / slice) {
            merge = true;
            break;
          }
        }
        pre += len;
      }
      merge |= empty_any;  // the merge kernel also writes requests without keys
    }
  }
  if (!p.balanced) {
    const int64_t chunk = plan_chunk(max_kv, total_kv, groups, have_ws);
    const int64_t max_chunks = std::max<int64_t>(1, ceil_div(max_kv, chunk));
    if (max_chunks * groups * (int64_t)batch > 0x7fffffff)
      return fail(FI_E_SHAPE, fn, "the split needs more than 2^31 workgroups");
    p.chunk = (int32_t)chunk;
    p.max_chunks = (int32_t)max_chunks;
    merge = max_chunks > 1;
  }
  *merge_out = merge;
  *need_out = merge ? partial_bytes(batch, p.max_chunks, p.num_qo_heads, head_dim) + (size_t)batch * groups * 4 : 0;
  return FI_OK;
}

// Decode workgroups of a plan (the grid of the decode kernel or the decode
// part of a fused launch).
template <class DP>
int64_t decode_workgroups(const DP& p, int32_t batch) {
  return p.balanced ? (int64_t)p.n_wg : (int64_t)p.max_chunks * p.n_hgroups * p.n_sgroups * batch;
}

// Scales and the partial-state pointers of a planned decode.
template <class DP>
void finish_decode(DP& p, fi_dtype kv_dtype, int32_t batch, int32_t head_dim, float sm_scale, float k_scale,
                   float v_scale, void* workspace, size_t need) {
  const float scale = (sm_scale > 0.f) ? sm_scale : 1.0f / std::sqrt((float)head_dim);
  // e4m3fnuz codes are widened to value * 2^-7 (exactly); the 2^7 joins the scales
  if (kv_dtype == FI_F8_E4M3_FNUZ) {
    k_scale *= 128.f;
    v_scale *= 128.f;
  }
  p.scale_log2 = scale * k_scale * fi::kLog2eHost;
  p.v_scale = v_scale;
  float* ws = reinterpret_cast<float*>(workspace);
  const size_t npart = (size_t)batch * p.num_qo_heads * p.max_chunks;
  p.part_o = need ? ws : nullptr;
  p.part_lse = need ? ws + npart * head_dim : nullptr;
  p.nch = need ? reinterpret_cast<int32_t*>(ws + npart * (head_dim + 1)) : nullptr;
}

// The split-KV merge of a planned decode (after its decode workgroups ran).
template <class DP>
hipError_t launch_decode_merge(const DP& p, fi_dtype o_dtype, int32_t batch, int32_t head_dim, hipStream_t stream) {
  fi::MergeParams mp{};
  mp.o = p.o;
  mp.lse = p.lse;
  mp.part_o = p.part_o;
  mp.part_lse = p.part_lse;
  mp.nch = p.nch;
  mp.batch = batch;
  mp.num_qo_heads = p.num_qo_heads;
  mp.group = p.group;
  mp.hpw_shift = p.hpw_shift;
  mp.spw = p.spw;
  mp.n_hgroups = p.n_hgroups;
  mp.n_sgroups = p.n_sgroups;
  mp.max_chunks = p.max_chunks;
  mp.v_scale = p.v_scale;
  return fi::launch_merge(mp, o_dtype, head_dim, batch, stream);
}

// Workspace checks of a planned decode; for the allocation-free call
// (use_scratch) the scratch array's address is looked up here, after every
// check has passed.
fi_status decode_workspace(const char* fn, size_t need, void** workspace, size_t workspace_bytes, bool use_scratch,
                           int32_t batch) {
  if (need > 0 && use_scratch && need > workspace_bytes)
    return fail(FI_E_WORKSPACE, fn, "this batch's split-KV state needs %zu bytes; the allocation-free call holds at "
                "most %zu bytes of scratch (FI_DECODE_SCRATCH_BYTES): call fi_batch_decode_paged with a workspace "
                "of fi_decode_workspace_bytes() instead", need, workspace_bytes);
  if (need > 0 && workspace_bytes < need)
    return fail(FI_E_WORKSPACE, fn, "workspace_bytes=%zu is smaller than the %zu bytes this split needs "
                "(fi_decode_workspace_bytes gives the bound)", workspace_bytes, need);
  if (need > 0 && !use_scratch && !aligned16(*workspace))
    return fail(FI_E_ARG, fn, "workspace must be 16-byte aligned");
  if (need > 0 && use_scratch && batch > 0) {
    hipError_t e = fi::decode_scratch(workspace);
    if (e != hipSuccess) return fail(FI_E_HIP, fn, "scratch address lookup failed: %s", hipGetErrorString(e));
  }
  return FI_OK;
}

// use_scratch: the allocation-free call -- the split-KV state goes to the
// library's own per-device scratch array (at most fi::kDecodeScratchBytes)
// instead of a caller's workspace; `workspace` is then NULL and its address
// is looked up only once every check has passed.
fi_status run_decode(const char* fn, fi::DecodeParams& p, fi_dtype q_dtype, fi_dtype kv_dtype, fi_dtype o_dtype,
                     int32_t batch, int32_t head_dim, const int32_t* indptr_h, const int32_t* last_page_len_h,
                     int32_t page_size, int64_t max_kv, int64_t total_kv, void* workspace, size_t workspace_bytes,
                     float sm_scale, float k_scale, float v_scale, hipStream_t stream, bool use_scratch = false) {
  const bool have_ws = workspace != nullptr || use_scratch;
  if (use_scratch) workspace_bytes = fi::kDecodeScratchBytes;
  bool merge = false;
  size_t need = 0;
  int nw = fi::kDecodeWaves;
  fi_status st = plan_decode(fn, p, nw, 0, q_dtype, kv_dtype, o_dtype, batch, head_dim, indptr_h, last_page_len_h,
                             page_size, max_kv, total_kv, have_ws, &merge, &need);
  if (st != FI_OK) return st;
  // Long per-workgroup streams (a balanced slice of at least 1 MB of K/V) run
  // on 8-wave workgroups that read whole rows of 8 heads: the long-context
  // workload streams 4% faster that way, while short slices (the
  // batch-decode workload's ~600 KB) gain nothing.
  // FI_DECODE_WAVES = 4 or 8 forces the workgroup size (8 only where it exists).
  const char* wv = std::getenv("FI_DECODE_WAVES");
  const int force_nw = wv ? std::atoi(wv) : 0;
  if (p.balanced && fi::decode_long_supported(q_dtype, kv_dtype) && force_nw != fi::kDecodeWaves) {
    const int64_t row_bytes = (int64_t)(1 << p.hpw_shift) * head_dim * elem_bytes(kv_dtype) * 2;
    if (force_nw == fi::kDecodeWavesLong || p.slice * row_bytes >= (1 << 20)) {
      fi::DecodeParams p8 = p;
      bool merge8 = false;
      size_t need8 = 0;
      if (plan_decode(fn, p8, fi::kDecodeWavesLong, 0, q_dtype, kv_dtype, o_dtype, batch, head_dim, indptr_h,
                      last_page_len_h, page_size, max_kv, total_kv, have_ws, &merge8, &need8) == FI_OK &&
          p8.balanced) {
        p = p8;
        merge = merge8;
        need = need8;
        nw = fi::kDecodeWavesLong;
      }
    }
  }
  if ((st = decode_workspace(fn, need, &workspace, workspace_bytes, use_scratch, batch)) != FI_OK) return st;
  finish_decode(p, kv_dtype, batch, head_dim, sm_scale, k_scale, v_scale, workspace, need);
  if (batch == 0) return FI_OK;
  hipError_t err = fi::launch_decode(p, q_dtype, kv_dtype, o_dtype, head_dim, batch, nw, stream);
  if (err != hipSuccess) return fail(FI_E_HIP, fn, "decode kernel launch failed: %s", hipGetErrorString(err));
  if (merge) {
    err = launch_decode_merge(p, o_dtype, batch, head_dim, stream);
    if (err != hipSuccess) return fail(FI_E_HIP, fn, "merge kernel launch failed: %s", hipGetErrorString(err));
  }
  return FI_OK;
}

// Dispatch order of causal / full prefill: the (request, query block) pairs
// sorted by the number of K/V tiles they walk, heaviest first, so that the
// hardware's in-order dispatch approximates longest-processing-time
// scheduling and no workgroup is launched for an empty query block.  Left
// empty (grid order) when the pairs do not fit in the kernel arguments.
template <class PP>
void plan_prefill_order(PP& p, int32_t batch, const int32_t* qo_indptr_h, const std::vector<int64_t>& kv_len) {
  p.n_items = 0;
  if (batch >= 65536) return;
  int64_t pairs = 0;
  for (int32_t i = 0; i < batch; ++i) pairs += ceil_div(qo_indptr_h[i + 1] - qo_indptr_h[i], p.q_per_wg);
  if (pairs > PP::kOrderMax) return;
  std::vector<std::pair<int64_t, uint32_t>> items;  // (tiles, request << 16 | block)
  items.reserve((size_t)pairs);
  for (int32_t i = 0; i < batch; ++i) {
    const int64_t qo = qo_indptr_h[i + 1] - qo_indptr_h[i];
    const int64_t kvl = kv_len[i];
    for (int64_t qb = ceil_div(qo, p.q_per_wg) - 1; qb >= 0; --qb) {
      const int64_t q_last = std::min<int64_t>((qb + 1) * p.q_per_wg, qo) - 1;
      const int64_t key_end = p.causal ? std::min<int64_t>(kvl, q_last + (kvl - qo) + 1) : kvl;
      items.emplace_back(key_end > 0 ? ceil_div(key_end, 64) : 0, (uint32_t)i << 16 | (uint32_t)qb);
    }
  }
  std::stable_sort(items.begin(), items.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
  for (size_t k = 0; k < items.size(); ++k) p.order[k] = items[k].second;
  p.n_items = (int32_t)items.size();
}

// Query-side checks shared by the prefill calls (after the dtype and head
// checks): the host query ranges, then q / o pointers.  *max_qo receives the
// longest request's query count.
fi_status check_queries(const char* fn, const void* q, void* o, int32_t batch, const int32_t* qo_indptr,
                               const int32_t* qo_indptr_h, int64_t* max_qo) {
  if (batch > 0 && (!qo_indptr || !qo_indptr_h)) return fail(FI_E_ARG, fn, "qo_indptr and qo_indptr_h must not be NULL");
  int64_t mx = 0, total = 0;
  if (batch > 0 && qo_indptr_h[0] < 0) return fail(FI_E_ARG, fn, "qo_indptr[0]=%d is negative", qo_indptr_h[0]);
  for (int32_t i = 0; i < batch; ++i) {
    const int64_t n = (int64_t)qo_indptr_h[i + 1] - qo_indptr_h[i];
    if (n < 0) return fail(FI_E_ARG, fn, "qo_indptr is decreasing at request %d", i);
    mx = n > mx ? n : mx;
    total += n;
  }
  if (total > 0) {
    if (!q || !o) return fail(FI_E_ARG, fn, "q and o must not be NULL");
    if (!aligned16(q) || !aligned16(o)) return fail(FI_E_ARG, fn, "q and o must be 16-byte aligned");
  }
  *max_qo = mx;
  return FI_OK;
}

// Work-group shape, scales and dispatch order of a prefill batch; p already
// holds the tensors and the K/V addressing.
// kv_base_h: the host copy of the cache's indptr (a request's first page, or
// first row of a ragged cache), or NULL for a single request (row 0).
template <class PP>
fi_status plan_prefill(const char* fn, PP& p, fi_dtype kv_dtype, int32_t batch, int32_t num_qo_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t causal, int64_t max_qo,
                       const int32_t* qo_indptr_h, const std::vector<int64_t>& kv_len, float sm_scale, float k_scale,
                       float v_scale, const int32_t* kv_base_h) {
  p.num_qo_heads = num_qo_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_qo_heads / num_kv_heads;
  p.heads_per_wg = (p.group % 4 == 0) ? 4 : (p.group % 2 == 0) ? 2 : 1;
  p.q_per_wg = 32 * fi::kPrefillWaves / p.heads_per_wg;
  p.n_qblocks = (int32_t)ceil_div(max_qo, p.q_per_wg);
  p.causal = causal ? 1 : 0;
  const float scale = (sm_scale > 0.f) ? sm_scale : 1.0f / std::sqrt((float)head_dim);
  // e4m3fnuz codes are widened to value * 2^-7 (exactly); the 2^7 joins the scales
  if (kv_dtype == FI_F8_E4M3_FNUZ) {
    k_scale *= 128.f;
    v_scale *= 128.f;
  }
  p.scale_log2 = scale * k_scale * fi::kLog2eHost;
  p.v_scale = v_scale;
  if (p.n_qblocks > 65535) return fail(FI_E_SHAPE, fn, "longest request has %lld queries; at most %d are supported",
                                       (long long)max_qo, 65535 * p.q_per_wg);
  plan_prefill_order(p, batch, qo_indptr_h, kv_len);
  p.n_geo = 0;
  if (batch <= PP::kGeoMax) {
    for (int32_t i = 0; i < batch; ++i) {
      p.geo[i][0] = qo_indptr_h[i];
      p.geo[i][1] = qo_indptr_h[i + 1] - qo_indptr_h[i];
      p.geo[i][2] = kv_base_h ? kv_base_h[i] : 0;
      p.geo[i][3] = (int32_t)kv_len[i];
    }
    p.n_geo = batch;
  }
  return FI_OK;
}

// Common tail of the prefill calls: the plan, then the launch.
fi_status run_prefill(const char* fn, fi::PrefillParams& p, fi_dtype q_dtype, fi_dtype kv_dtype,
                             fi_dtype o_dtype, int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t causal, int64_t max_qo, const int32_t* qo_indptr_h,
                             const std::vector<int64_t>& kv_len, float sm_scale, float k_scale, float v_scale,
                             bool ragged, hipStream_t stream, const int32_t* kv_base_h) {
  fi_status st = plan_prefill(fn, p, kv_dtype, batch, num_qo_heads, num_kv_heads, head_dim, causal, max_qo,
                              qo_indptr_h, kv_len, sm_scale, k_scale, v_scale, kv_base_h);
  if (st != FI_OK) return st;
  hipError_t err = fi::launch_prefill(p, q_dtype, kv_dtype, o_dtype, head_dim, batch, ragged, stream);
  if (err != hipSuccess) return fail(FI_E_HIP, fn, "prefill kernel launch failed: %s", hipGetErrorString(err));
  return FI_OK;
}

// Checks on contiguous K/V rows (ragged or single): strides, pointers and
// alignment of two pools of `rows` rows.
fi_status check_rows(const char* fn, const void* k, const void* v, fi_dtype kv_dtype, int64_t stride_token,
                            int64_t stride_head, int64_t rows) {
  const int eb = elem_bytes(kv_dtype);
  if (stride_token <= 0 || stride_head <= 0)
    return fail(FI_E_SHAPE, fn, "strides must be positive (token %lld, head %lld)", (long long)stride_token,
                (long long)stride_head);
  if (stride_token * eb >= (1ll << 32) || stride_head * eb >= (1ll << 32))
    return fail(FI_E_SHAPE, fn, "K/V strides must be below 4 GiB");
  if ((stride_token * eb) % 16 || (stride_head * eb) % 16)
    return fail(FI_E_ARG, fn, "K/V strides must give 16-byte aligned rows (token %lld, head %lld elements of %d bytes)",
                (long long)stride_token, (long long)stride_head, eb);
  if (rows > 0) {
    if (!k || !v) return fail(FI_E_ARG, fn, "k and v must not be NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(FI_E_ARG, fn, "k and v must be 16-byte aligned");
  }
  return FI_OK;
}

}  // namespace

extern "C" {

const char* fi_last_error(void) { return g_err.c_str(); }

size_t fi_decode_workspace_bytes(int32_t batch, int32_t num_qo_heads, int32_t head_dim, int32_t max_kv_len) {
  if (batch <= 0 || num_qo_heads <= 0 || head_dim <= 0 || max_kv_len <= 0) return 0;
  // every plan uses pieces of at least kChunkQuantum tokens; a balanced slice
  // boundary can add one more piece to a request
  const int64_t max_chunks = ceil_div(max_kv_len, fi::kChunkQuantum) + 1;
  return partial_bytes(batch, max_chunks, num_qo_heads, head_dim) + (size_t)batch * num_qo_heads * 4;
}

// Batched paged decode after the dtype checks (q_scale: 1 for a 2-byte query).
static fi_status decode_paged(const char* fn, const void* q, fi_dtype q_dtype, float q_scale, int32_t batch,
                              int32_t num_qo_heads, const fi_paged_kv* kv, void* o, fi_dtype o_dtype, float* lse,
                              float sm_scale, void* workspace, size_t workspace_bytes, void* stream,
                              bool use_scratch = false) {
  fi_status st;
  if (batch < 0) return fail(FI_E_SHAPE, fn, "batch=%d is outside [0, 2^31)", batch);
  if ((st = check_heads(fn, num_qo_heads, kv->num_kv_heads, kv->head_dim)) != FI_OK) return st;
  if (batch > 0) {
    if (!q || !o) return fail(FI_E_ARG, fn, "q and o must not be NULL");
    if (!aligned16(q) || !aligned16(o)) return fail(FI_E_ARG, fn, "q and o must be 16-byte aligned");
  }
  if ((st = check_scales(fn, kv->k_scale, kv->v_scale, sm_scale)) != FI_OK) return st;
  int64_t max_kv = 0, total_kv = 0;
  if ((st = check_paged(fn, batch, kv, &max_kv, &total_kv)) != FI_OK) return st;
  const int eb = elem_bytes(kv->k_dtype);
  fi::DecodeParams p{};
  p.q = q;
  p.o = o;
  p.lse = lse;
  p.k = reinterpret_cast<const uint8_t*>(kv->k);
  p.v = reinterpret_cast<const uint8_t*>(kv->v);
  p.sp = kv->stride_page * eb;
  p.st = kv->stride_token * eb;
  p.sh = kv->stride_head * eb;
  p.indptr = kv->indptr;
  p.indices = kv->indices;
  p.last_page_len = kv->last_page_len;
  p.page_shift = ilog2(kv->page_size);
  p.page_size = kv->page_size;
  p.single_kv_len = 0;
  p.num_qo_heads = num_qo_heads;
  p.num_kv_heads = kv->num_kv_heads;
  p.group = num_qo_heads / kv->num_kv_heads;
  // q_scale joins k_scale in the logit scale (both multiply the fp32 products)
  return run_decode(fn, p, q_dtype, kv->k_dtype, o_dtype, batch, kv->head_dim, kv->indptr_h, kv->last_page_len_h,
                    kv->page_size, max_kv, total_kv, workspace, workspace_bytes, sm_scale, kv->k_scale * q_scale,
                    kv->v_scale, reinterpret_cast<hipStream_t>(stream), use_scratch);
}

fi_status fi_batch_decode_paged(const void* q, fi_dtype q_dtype, int32_t batch, int32_t num_qo_heads,
                                const fi_paged_kv* kv, void* o, fi_dtype o_dtype, float* lse, float sm_scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "fi_batch_decode_paged";
  if (!kv) return fail(FI_E_ARG, fn, "kv must not be NULL");
  fi_status st = check_dtypes(fn, q_dtype, &o_dtype, kv->k_dtype, kv->v_dtype, false);
  if (st != FI_OK) return st;
  return decode_paged(fn, q, q_dtype, 1.0f, batch, num_qo_heads, kv, o, o_dtype, lse, sm_scale, workspace,
                      workspace_bytes, stream);
}

fi_status fi_batch_decode_paged_noalloc(const void* q, fi_dtype q_dtype, int32_t batch, int32_t num_qo_heads,
                                        const fi_paged_kv* kv, void* o, fi_dtype o_dtype, float* lse, float sm_scale,
                                        void* stream) {
  static const char* fn = "fi_batch_decode_paged_noalloc";
  if (!kv) return fail(FI_E_ARG, fn, "kv must not be NULL");
  fi_status st = check_dtypes(fn, q_dtype, &o_dtype, kv->k_dtype, kv->v_dtype, false);
  if (st != FI_OK) return st;
  return decode_paged(fn, q, q_dtype, 1.0f, batch, num_qo_heads, kv, o, o_dtype, lse, sm_scale, nullptr, 0, stream,
                      true);
}

fi_status fi_batch_decode_paged_fp8q(const void* q, fi_dtype q_dtype, float q_scale, int32_t batch,
                                     int32_t num_qo_heads, const fi_paged_kv* kv, void* o, fi_dtype o_dtype,
                                     float* lse, float sm_scale, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  static const char* fn = "fi_batch_decode_paged_fp8q";
  if (!kv) return fail(FI_E_ARG, fn, "kv must not be NULL");
  fi_status st = check_dtypes_fp8q(fn, q_dtype, o_dtype, kv->k_dtype, kv->v_dtype, true);
  if (st != FI_OK) return st;
  if (!std::isfinite(q_scale) || !(q_scale > 0.f)) return fail(FI_E_ARG, fn, "q_scale=%g must be finite and > 0", q_scale);
  return decode_paged(fn, q, q_dtype, q_scale, batch, num_qo_heads, kv, o, o_dtype, lse, sm_scale, workspace,
                      workspace_bytes, stream);
}

fi_status fi_single_decode(const void* q, fi_dtype q_dtype, const void* k, const void* v, fi_dtype k_dtype,
                           fi_dtype v_dtype, int32_t kv_len, int32_t num_qo_heads, int32_t num_kv_heads,
                           int32_t head_dim, float k_scale, float v_scale, void* o, fi_dtype o_dtype, float* lse,
                           float sm_scale, void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "fi_single_decode";
  fi_status st = check_dtypes(fn, q_dtype, &o_dtype, k_dtype, v_dtype, false);
  if (st != FI_OK) return st;
  if ((st = check_heads(fn, num_qo_heads, num_kv_heads, head_dim)) != FI_OK) return st;
  if (kv_len < 0 || kv_len >= (1 << 30)) return fail(FI_E_SHAPE, fn, "kv_len=%d is outside [0, 2^30)", kv_len);
  if (!q || !o) return fail(FI_E_ARG, fn, "q and o must not be NULL");
  if (!aligned16(q) || !aligned16(o)) return fail(FI_E_ARG, fn, "q and o must be 16-byte aligned");
  if (kv_len > 0 && (!k || !v)) return fail(FI_E_ARG, fn, "k and v must not be NULL");
  if (kv_len > 0 && (!aligned16(k) || !aligned16(v))) return fail(FI_E_ARG, fn, "k and v must be 16-byte aligned");
  if ((st = check_scales(fn, k_scale, v_scale, sm_scale)) != FI_OK) return st;
  const int eb = elem_bytes(k_dtype);
  fi::DecodeParams p{};
  p.q = q;
  p.o = o;
  p.lse = lse;
  p.k = reinterpret_cast<const uint8_t*>(k);
  p.v = reinterpret_cast<const uint8_t*>(v);
  p.sp = 0;
  p.st = (int64_t)num_kv_heads * head_dim * eb;
  p.sh = (int64_t)head_dim * eb;
  p.indptr = nullptr;
  p.indices = nullptr;
  p.last_page_len = nullptr;
  p.page_shift = 30;
  p.page_size = 1 << 30;
  p.single_kv_len = kv_len;
  p.num_qo_heads = num_qo_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_qo_heads / num_kv_heads;
  return run_decode(fn, p, q_dtype, k_dtype, o_dtype, 1, head_dim, nullptr, nullptr, 1 << 30, kv_len, kv_len,
                    workspace, workspace_bytes, sm_scale, k_scale, v_scale, reinterpret_cast<hipStream_t>(stream));
}

fi_status fi_batch_prefill_paged(const void* q, fi_dtype q_dtype, const int32_t* qo_indptr,
                                 const int32_t* qo_indptr_h, int32_t batch, int32_t num_qo_heads,
                                 const fi_paged_kv* kv, int32_t causal, void* o, fi_dtype o_dtype, float* lse,
                                 float sm_scale, void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "fi_batch_prefill_paged";
  (void)workspace;
  (void)workspace_bytes;
  if (!kv) return fail(FI_E_ARG, fn, "kv must not be NULL");
  fi_status st = check_dtypes(fn, q_dtype, &o_dtype, kv->k_dtype, kv->v_dtype, true);
  if (st != FI_OK) return st;
  if (batch < 0) return fail(FI_E_SHAPE, fn, "batch=%d is negative", batch);
  if ((st = check_heads(fn, num_qo_heads, kv->num_kv_heads, kv->head_dim)) != FI_OK) return st;
  if (batch > 0 && (!qo_indptr || !qo_indptr_h)) return fail(FI_E_ARG, fn, "qo_indptr and qo_indptr_h must not be NULL");
  if ((st = check_scales(fn, kv->k_scale, kv->v_scale, sm_scale)) != FI_OK) return st;
  int64_t max_kv = 0, total_kv = 0;
  if ((st = check_paged(fn, batch, kv, &max_kv, &total_kv)) != FI_OK) return st;
  int64_t max_qo = 0;
  if ((st = check_queries(fn, q, o, batch, qo_indptr, qo_indptr_h, &max_qo)) != FI_OK) return st;
  if (batch == 0 || max_qo == 0) return FI_OK;
  std::vector<int64_t> kv_len((size_t)batch);
  for (int32_t i = 0; i < batch; ++i) {
    const int64_t np = kv->indptr_h[i + 1] - kv->indptr_h[i];
    kv_len[i] = np > 0 ? (np - 1) * kv->page_size + kv->last_page_len_h[i] : 0;
  }
  const int eb = elem_bytes(kv->k_dtype);
  fi::PrefillParams p{};
  p.q = q;
  p.o = o;
  p.lse = lse;
  p.k = reinterpret_cast<const uint8_t*>(kv->k);
  p.v = reinterpret_cast<const uint8_t*>(kv->v);
  p.sp = kv->stride_page * eb;
  p.st = kv->stride_token * eb;
  p.sh = kv->stride_head * eb;
  p.qo_indptr = qo_indptr;
  p.indptr = kv->indptr;
  p.indices = kv->indices;
  p.last_page_len = kv->last_page_len;
  p.page_shift = ilog2(kv->page_size);
  p.page_size = kv->page_size;
  return run_prefill(fn, p, q_dtype, kv->k_dtype, o_dtype, batch, num_qo_heads, kv->num_kv_heads, kv->head_dim,
                     causal, max_qo, qo_indptr_h, kv_len, sm_scale, kv->k_scale, kv->v_scale, false,
                     reinterpret_cast<hipStream_t>(stream), kv->indptr_h);
}

fi_status fi_batch_prefill_paged_fp8q(const void* q, fi_dtype q_dtype, float q_scale, const int32_t* qo_indptr,
                                      const int32_t* qo_indptr_h, int32_t batch, int32_t num_qo_heads,
                                      const fi_paged_kv* kv, int32_t causal, int32_t pv_fp8, void* o,
                                      fi_dtype o_dtype, float* lse, float sm_scale, void* stream) {
  static const char* fn = "fi_batch_prefill_paged_fp8q";
  if (!kv) return fail(FI_E_ARG, fn, "kv must not be NULL");
  fi_status st = check_dtypes_fp8q(fn, q_dtype, o_dtype, kv->k_dtype, kv->v_dtype);
  if (st != FI_OK) return st;
  if (batch < 0) return fail(FI_E_SHAPE, fn, "batch=%d is negative", batch);
  if ((st = check_heads(fn, num_qo_heads, kv->num_kv_heads, kv->head_dim)) != FI_OK) return st;
  if (batch > 0 && (!qo_indptr || !qo_indptr_h)) return fail(FI_E_ARG, fn, "qo_indptr and qo_indptr_h must not be NULL");
  if (!std::isfinite(q_scale) || !(q_scale > 0.f)) return fail(FI_E_ARG, fn, "q_scale=%g must be finite and > 0", q_scale);
  if ((st = check_scales(fn, kv->k_scale, kv->v_scale, sm_scale)) != FI_OK) return st;
  int64_t max_kv = 0, total_kv = 0;
  if ((st = check_paged(fn, batch, kv, &max_kv, &total_kv)) != FI_OK) return st;
  int64_t max_qo = 0;
  if ((st = check_queries(fn, q, o, batch, qo_indptr, qo_indptr_h, &max_qo)) != FI_OK) return st;
  if (batch == 0 || max_qo == 0) return FI_OK;
  std::vector<int64_t> kv_len((size_t)batch);
  for (int32_t i = 0; i < batch; ++i) {
    const int64_t np = kv->indptr_h[i + 1] - kv->indptr_h[i];
    kv_len[i] = np > 0 ? (np - 1) * kv->page_size + kv->last_page_len_h[i] : 0;
  }
  fi::PrefillParams p{};
  p.q = q;
  p.o = o;
  p.lse = lse;
  p.k = reinterpret_cast<const uint8_t*>(kv->k);
  p.v = reinterpret_cast<const uint8_t*>(kv->v);
  p.sp = kv->stride_page;  // fp8: one byte per element
  p.st = kv->stride_token;
  p.sh = kv->stride_head;
  p.qo_indptr = qo_indptr;
  p.indptr = kv->indptr;
  p.indices = kv->indices;
  p.last_page_len = kv->last_page_len;
  p.page_shift = ilog2(kv->page_size);
  p.page_size = kv->page_size;
  p.pv_fp8 = pv_fp8 ? 1 : 0;
  // q_scale joins k_scale in the logit scale (both multiply the fp32 products)
  return run_prefill(fn, p, q_dtype, kv->k_dtype, o_dtype, batch, num_qo_heads, kv->num_kv_heads, kv->head_dim,
                     causal, max_qo, qo_indptr_h, kv_len, sm_scale, kv->k_scale * q_scale, kv->v_scale, false,
                     reinterpret_cast<hipStream_t>(stream), kv->indptr_h);
}

// Prefill and decode batches in one launch.  Both phases must agree on the
// query, output and KV dtypes and on the head layout (they run one kernel);
// each has its own page table and scales.  The prefill phase takes the
// prefill rules (a 2-byte KV equal to q), and so does the decode phase, as the
// pages' POD entry points do.
fi_status fi_batch_pod_paged(const void* q_p, const int32_t* qo_indptr, const int32_t* qo_indptr_h, int32_t batch_p,
                             const fi_paged_kv* kv_p, int32_t causal, void* o_p, float* lse_p, const void* q_d,
                             int32_t batch_d, const fi_paged_kv* kv_d, void* o_d, float* lse_d, fi_dtype q_dtype,
                             fi_dtype o_dtype, int32_t num_qo_heads, float sm_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  static const char* fn = "fi_batch_pod_paged";
  static const char* fn_d = "fi_batch_pod_paged (decode phase)";
  if (!kv_p || !kv_d) return fail(FI_E_ARG, fn, "kv_p and kv_d must not be NULL");
  fi_status st = check_dtypes(fn, q_dtype, &o_dtype, kv_p->k_dtype, kv_p->v_dtype, true);
  if (st != FI_OK) return st;
  fi_dtype o_d_dtype = o_dtype;
  if ((st = check_dtypes(fn_d, q_dtype, &o_d_dtype, kv_d->k_dtype, kv_d->v_dtype, true)) != FI_OK) return st;
  if (kv_d->k_dtype != kv_p->k_dtype)
    return fail(FI_E_DTYPE, fn, "the prefill phase's KV cache has dtype %s but the decode phase's has dtype %s; both "
                "phases of one call run one kernel over one KV dtype", dtype_name(kv_p->k_dtype),
                dtype_name(kv_d->k_dtype));
  if (batch_p < 0 || batch_d < 0)
    return fail(FI_E_SHAPE, fn, "batch sizes must not be negative (prefill %d, decode %d)", batch_p, batch_d);
  if ((st = check_heads(fn, num_qo_heads, kv_p->num_kv_heads, kv_p->head_dim)) != FI_OK) return st;
  if (kv_d->num_kv_heads != kv_p->num_kv_heads || kv_d->head_dim != kv_p->head_dim)
    return fail(FI_E_SHAPE, fn, "the decode phase's cache has %d kv heads of head_dim %d but the prefill phase's has "
                "%d of head_dim %d; both phases share the head layout", kv_d->num_kv_heads, kv_d->head_dim,
                kv_p->num_kv_heads, kv_p->head_dim);
  if (batch_p > 0 && (!qo_indptr || !qo_indptr_h)) return fail(FI_E_ARG, fn, "qo_indptr and qo_indptr_h must not be NULL");
  if ((st = check_scales(fn, kv_p->k_scale, kv_p->v_scale, sm_scale)) != FI_OK) return st;
  if ((st = check_scales(fn_d, kv_d->k_scale, kv_d->v_scale, sm_scale)) != FI_OK) return st;
  int64_t max_kv_p = 0, total_kv_p = 0, max_kv_d = 0, total_kv_d = 0;
  if ((st = check_paged(fn, batch_p, kv_p, &max_kv_p, &total_kv_p)) != FI_OK) return st;
  if ((st = check_paged(fn_d, batch_d, kv_d, &max_kv_d, &total_kv_d)) != FI_OK) return st;
  int64_t max_qo = 0;
  if ((st = check_queries(fn, q_p, o_p, batch_p, qo_indptr, qo_indptr_h, &max_qo)) != FI_OK) return st;
  if (batch_d > 0) {
    if (!q_d || !o_d) return fail(FI_E_ARG, fn_d, "q and o must not be NULL");
    if (!aligned16(q_d) || !aligned16(o_d)) return fail(FI_E_ARG, fn_d, "q and o must be 16-byte aligned");
  }
  const int eb = elem_bytes(kv_p->k_dtype);
  const int32_t hd = kv_p->head_dim;
  fi::PodParams pp{};
  // prefill phase: every (request, query block) pair in the dispatch order
  if (batch_p > 0 && max_qo > 0) {
    auto& f = pp.pf;
    f.q = q_p;
    f.o = o_p;
    f.lse = lse_p;
    f.k = reinterpret_cast<const uint8_t*>(kv_p->k);
    f.v = reinterpret_cast<const uint8_t*>(kv_p->v);
    f.sp = kv_p->stride_page * eb;
    f.st = kv_p->stride_token * eb;
    f.sh = kv_p->stride_head * eb;
    f.qo_indptr = qo_indptr;
    f.indptr = kv_p->indptr;
    f.indices = kv_p->indices;
    f.last_page_len = kv_p->last_page_len;
    f.page_shift = ilog2(kv_p->page_size);
    f.page_size = kv_p->page_size;
    std::vector<int64_t> kv_len((size_t)batch_p);
    for (int32_t i = 0; i < batch_p; ++i) {
      const int64_t np = kv_p->indptr_h[i + 1] - kv_p->indptr_h[i];
      kv_len[i] = np > 0 ? (np - 1) * kv_p->page_size + kv_p->last_page_len_h[i] : 0;
    }
    if ((st = plan_prefill(fn, f, kv_p->k_dtype, batch_p, num_qo_heads, kv_p->num_kv_heads, hd, causal, max_qo,
                           qo_indptr_h, kv_len, sm_scale, kv_p->k_scale, kv_p->v_scale, kv_p->indptr_h)) != FI_OK)
      return st;
    if (f.n_items == 0)
      return fail(FI_E_SHAPE, fn, "the prefill phase has more than %d (request, query block) pairs of %d queries, the "
                  "most one launch's arguments carry; fi_batch_prefill_paged has no such limit", fi::kPodOrderMax,
                  f.q_per_wg);
    pp.n_prefill_wg = f.n_items * kv_p->num_kv_heads * (f.group / f.heads_per_wg);
  }
  // decode phase: balanced slices over 8-wave workgroups, two per CU unless
  // FI_POD_DECODE_WG names a count
  bool merge = false;
  if (batch_d > 0) {
    fi::DecodeParamsT<fi::kPodPrefixMax>& d = pp.dc;
    d.q = q_d;
    d.o = o_d;
    d.lse = lse_d;
    d.k = reinterpret_cast<const uint8_t*>(kv_d->k);
    d.v = reinterpret_cast<const uint8_t*>(kv_d->v);
    d.sp = kv_d->stride_page * eb;
    d.st = kv_d->stride_token * eb;
    d.sh = kv_d->stride_head * eb;
    d.indptr = kv_d->indptr;
    d.indices = kv_d->indices;
    d.last_page_len = kv_d->last_page_len;
    d.page_shift = ilog2(kv_d->page_size);
    d.page_size = kv_d->page_size;
    d.num_qo_heads = num_qo_heads;
    d.num_kv_heads = kv_d->num_kv_heads;
    d.group = num_qo_heads / kv_d->num_kv_heads;
    // Decode slices first, on a share of the CUs: the decode stream needs HBM
    // bandwidth rather than CUs, so a fraction of the CUs streams it while the
    // rest start the prefill items, which then fill the CUs the decode
    // workgroups leave.  The decode phase costs about the same CU time however
    // many workgroups share it (each streams at its own rate), so the launch
    // takes about (decode + prefill CU time) / CUs as long as the decode
    // workgroups finish within it; they are sized to take half that estimate,
    // which keeps them off the critical path (measured on the mixed batch:
    // fewer workgroups, sized to end with the prefill, made the decode phase
    // the longer one on some runs).  Decode bytes at kPodDecodeWgRate per 8-wave
    // workgroup, prefill flops at kPodPrefillCuRate per CU (both measured on
    // MI355X under sustained load: the causal-prefill workload at ~890 TFLOP/s
    // over 256 CUs; a lone decode workgroup streams ~20 GB/s).  A decode-only
    // call takes two workgroups per CU.  FI_POD_DECODE_WG overrides the count.
    constexpr double kPodPrefillCuRate = 3.5e12, kPodDecodeWgRate = 20e9;
    const int cus = std::max(1, fi::device_cus());
    int slots = 2 * cus;
    if (pp.n_prefill_wg > 0) {
      double flops = 0;
      for (int32_t i = 0; i < batch_p; ++i) {
        const int64_t qo = qo_indptr_h[i + 1] - qo_indptr_h[i];
        const int64_t np = kv_p->indptr_h[i + 1] - kv_p->indptr_h[i];
        const int64_t kvl = np > 0 ? (np - 1) * kv_p->page_size + kv_p->last_page_len_h[i] : 0;
        for (int64_t r = 0; r < qo; ++r)  // keys row r sees
          flops += (double)(causal ? std::max<int64_t>(0, std::min<int64_t>(kvl, r + 1 + kvl - qo)) : kvl);
      }
      flops *= 4.0 * hd * num_qo_heads;
      const double bytes = (double)total_kv_d * kv_d->num_kv_heads * hd * eb * 2;
      const double dec_cu = bytes / kPodDecodeWgRate, pf_cu = flops / kPodPrefillCuRate;  // CU-seconds
      const double nd = 2.0 * cus * dec_cu / (dec_cu + pf_cu);
      slots = (int)std::lround(std::min<double>(2.0 * cus, std::max<double>(std::max(8, cus / 16), nd)));
    }
    if (const char* env = std::getenv("FI_POD_DECODE_WG")) {
      const long n = std::strtol(env, nullptr, 10);
      if (n > 0 && n < (1 << 20)) slots = (int)n;
    }
    size_t need = 0;
    if ((st = plan_decode(fn_d, d, fi::kPodDecodeWaves, std::max(slots, 1), q_dtype, kv_d->k_dtype, o_dtype, batch_d,
                          hd, kv_d->indptr_h, kv_d->last_page_len_h, kv_d->page_size, max_kv_d, total_kv_d,
                          workspace != nullptr, &merge, &need)) != FI_OK)
      return st;
    if ((st = decode_workspace(fn_d, need, &workspace, workspace_bytes, false, batch_d)) != FI_OK) return st;
    finish_decode(d, kv_d->k_dtype, batch_d, hd, sm_scale, kv_d->k_scale, kv_d->v_scale, workspace, need);
    const int64_t nwg = decode_workgroups(d, batch_d);
    if (nwg + pp.n_prefill_wg > 0x7fffffff) return fail(FI_E_SHAPE, fn, "the launch needs more than 2^31 workgroups");
    pp.n_decode_wg = (int32_t)nwg;
  }
  if (pp.n_prefill_wg + (int64_t)pp.n_decode_wg == 0) return FI_OK;
  {
    const char* env = std::getenv("FI_POD_ORDER");
    pp.decode_first = (env && std::strcmp(env, "prefill_first") == 0) ? 0 : 1;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t err = fi::launch_pod(pp, q_dtype, kv_p->k_dtype, o_dtype, hd, s);
  if (err != hipSuccess) return fail(FI_E_HIP, fn, "prefill + decode kernel launch failed: %s", hipGetErrorString(err));
  if (merge) {
    err = launch_decode_merge(pp.dc, o_dtype, batch_d, hd, s);
    if (err != hipSuccess) return fail(FI_E_HIP, fn, "merge kernel launch failed: %s", hipGetErrorString(err));
  }
  return FI_OK;
}

}  // extern "C"

// Ragged and single prefill, with a 2-byte query or (q8) an fp8 query with
// its q_scale, which joins k_scale in the logit scale as in the paged call.
static fi_status ragged_prefill(const char* fn, bool q8, const void* q, fi_dtype q_dtype, float q_scale,
                                const int32_t* qo_indptr, const int32_t* qo_indptr_h, int32_t batch,
                                int32_t num_qo_heads, const fi_ragged_kv* kv, int32_t causal, int32_t pv_fp8, void* o,
                                fi_dtype o_dtype, float* lse, float sm_scale, void* stream) {
  if (!kv) return fail(FI_E_ARG, fn, "kv must not be NULL");
  fi_status st = q8 ? check_dtypes_fp8q(fn, q_dtype, o_dtype, kv->k_dtype, kv->v_dtype)
                    : check_dtypes(fn, q_dtype, &o_dtype, kv->k_dtype, kv->v_dtype, true);
  if (st != FI_OK) return st;
  if (batch < 0) return fail(FI_E_SHAPE, fn, "batch=%d is negative", batch);
  if ((st = check_heads(fn, num_qo_heads, kv->num_kv_heads, kv->head_dim)) != FI_OK) return st;
  if (batch > 0 && (!qo_indptr || !qo_indptr_h)) return fail(FI_E_ARG, fn, "qo_indptr and qo_indptr_h must not be NULL");
  if (q8 && (!std::isfinite(q_scale) || !(q_scale > 0.f)))
    return fail(FI_E_ARG, fn, "q_scale=%g must be finite and > 0", q_scale);
  if ((st = check_scales(fn, kv->k_scale, kv->v_scale, sm_scale)) != FI_OK) return st;
  if (kv->num_tokens < 0) return fail(FI_E_SHAPE, fn, "num_tokens=%d is negative", kv->num_tokens);
  if ((st = check_rows(fn, kv->k, kv->v, kv->k_dtype, kv->stride_token, kv->stride_head,
                       batch > 0 ? kv->num_tokens : 0)) != FI_OK)
    return st;
  if (batch > 0 && (!kv->indptr || !kv->indptr_h))
    return fail(FI_E_ARG, fn, "indptr (device) and indptr_h (host copy) must not be NULL");
  std::vector<int64_t> kv_len((size_t)batch);
  if (batch > 0 && kv->indptr_h[0] < 0) return fail(FI_E_ARG, fn, "indptr[0]=%d is negative", kv->indptr_h[0]);
  for (int32_t i = 0; i < batch; ++i) {
    const int32_t a = kv->indptr_h[i], e = kv->indptr_h[i + 1];
    if (e < a) return fail(FI_E_ARG, fn, "indptr is decreasing at request %d (%d > %d)", i, a, e);
    if (e - a >= (1 << 30))
      return fail(FI_E_SHAPE, fn, "request %d has %d tokens; at most 2^30 - 1 are supported", i, e - a);
    kv_len[i] = e - a;
  }
  if (batch > 0 && kv->indptr_h[batch] > kv->num_tokens)
    return fail(FI_E_ARG, fn, "indptr[%d]=%d exceeds num_tokens=%d", batch, kv->indptr_h[batch], kv->num_tokens);
  int64_t max_qo = 0;
  if ((st = check_queries(fn, q, o, batch, qo_indptr, qo_indptr_h, &max_qo)) != FI_OK) return st;
  if (batch == 0 || max_qo == 0) return FI_OK;
  const int eb = elem_bytes(kv->k_dtype);
  fi::PrefillParams p{};
  p.q = q;
  p.o = o;
  p.lse = lse;
  p.k = reinterpret_cast<const uint8_t*>(kv->k);
  p.v = reinterpret_cast<const uint8_t*>(kv->v);
  p.st = kv->stride_token * eb;
  p.sh = kv->stride_head * eb;
  p.qo_indptr = qo_indptr;
  p.indptr = kv->indptr;
  p.pv_fp8 = (q8 && pv_fp8) ? 1 : 0;
  return run_prefill(fn, p, q_dtype, kv->k_dtype, o_dtype, batch, num_qo_heads, kv->num_kv_heads, kv->head_dim,
                     causal, max_qo, qo_indptr_h, kv_len, sm_scale, kv->k_scale * (q8 ? q_scale : 1.0f), kv->v_scale,
                     true, reinterpret_cast<hipStream_t>(stream), kv->indptr_h);
}

static fi_status single_prefill(const char* fn, bool q8, const void* q, fi_dtype q_dtype, float q_scale,
                                int32_t qo_len, const void* k, const void* v, fi_dtype k_dtype, fi_dtype v_dtype,
                                int32_t kv_len, int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t causal, int32_t pv_fp8, float k_scale, float v_scale, void* o,
                                fi_dtype o_dtype, float* lse, float sm_scale, void* stream) {
  fi_status st = q8 ? check_dtypes_fp8q(fn, q_dtype, o_dtype, k_dtype, v_dtype)
                    : check_dtypes(fn, q_dtype, &o_dtype, k_dtype, v_dtype, true);
  if (st != FI_OK) return st;
  if ((st = check_heads(fn, num_qo_heads, num_kv_heads, head_dim)) != FI_OK) return st;
  if (qo_len < 0) return fail(FI_E_SHAPE, fn, "qo_len=%d is negative", qo_len);
  if (kv_len < 0 || kv_len >= (1 << 30)) return fail(FI_E_SHAPE, fn, "kv_len=%d is outside [0, 2^30)", kv_len);
  if (q8 && (!std::isfinite(q_scale) || !(q_scale > 0.f)))
    return fail(FI_E_ARG, fn, "q_scale=%g must be finite and > 0", q_scale);
  if ((st = check_scales(fn, k_scale, v_scale, sm_scale)) != FI_OK) return st;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if ((st = check_rows(fn, k, v, k_dtype, row, head_dim, kv_len)) != FI_OK) return st;
  if (qo_len > 0) {
    if (!q || !o) return fail(FI_E_ARG, fn, "q and o must not be NULL");
    if (!aligned16(q) || !aligned16(o)) return fail(FI_E_ARG, fn, "q and o must be 16-byte aligned");
  }
  if (qo_len == 0) return FI_OK;
  const int eb = elem_bytes(k_dtype);
  fi::PrefillParams p{};
  p.q = q;
  p.o = o;
  p.lse = lse;
  p.k = reinterpret_cast<const uint8_t*>(k);
  p.v = reinterpret_cast<const uint8_t*>(v);
  p.st = row * eb;
  p.sh = (int64_t)head_dim * eb;
  p.single_qo_len = qo_len;
  p.single_kv_len = kv_len;
  p.pv_fp8 = (q8 && pv_fp8) ? 1 : 0;
  const int32_t qo_indptr_h[2] = {0, qo_len};
  const std::vector<int64_t> lens(1, kv_len);
  return run_prefill(fn, p, q_dtype, k_dtype, o_dtype, 1, num_qo_heads, num_kv_heads, head_dim, causal, qo_len,
                     qo_indptr_h, lens, sm_scale, k_scale * (q8 ? q_scale : 1.0f), v_scale, true,
                     reinterpret_cast<hipStream_t>(stream), nullptr);
}

extern "C" {

fi_status fi_batch_prefill_ragged(const void* q, fi_dtype q_dtype, const int32_t* qo_indptr,
                                  const int32_t* qo_indptr_h, int32_t batch, int32_t num_qo_heads,
                                  const fi_ragged_kv* kv, int32_t causal, void* o, fi_dtype o_dtype, float* lse,
                                  float sm_scale, void* stream) {
  return ragged_prefill("fi_batch_prefill_ragged", false, q, q_dtype, 1.0f, qo_indptr, qo_indptr_h, batch,
                        num_qo_heads, kv, causal, 0, o, o_dtype, lse, sm_scale, stream);
}

fi_status fi_batch_prefill_ragged_fp8q(const void* q, fi_dtype q_dtype, float q_scale, const int32_t* qo_indptr,
                                       const int32_t* qo_indptr_h, int32_t batch, int32_t num_qo_heads,
                                       const fi_ragged_kv* kv, int32_t causal, int32_t pv_fp8, void* o,
                                       fi_dtype o_dtype, float* lse, float sm_scale, void* stream) {
  return ragged_prefill("fi_batch_prefill_ragged_fp8q", true, q, q_dtype, q_scale, qo_indptr, qo_indptr_h, batch,
                        num_qo_heads, kv, causal, pv_fp8, o, o_dtype, lse, sm_scale, stream);
}

fi_status fi_single_prefill(const void* q, fi_dtype q_dtype, int32_t qo_len, const void* k, const void* v,
                            fi_dtype k_dtype, fi_dtype v_dtype, int32_t kv_len, int32_t num_qo_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t causal, float k_scale, float v_scale,
                            void* o, fi_dtype o_dtype, float* lse, float sm_scale, void* stream) {
  return single_prefill("fi_single_prefill", false, q, q_dtype, 1.0f, qo_len, k, v, k_dtype, v_dtype, kv_len,
                        num_qo_heads, num_kv_heads, head_dim, causal, 0, k_scale, v_scale, o, o_dtype, lse, sm_scale,
                        stream);
}

fi_status fi_single_prefill_fp8q(const void* q, fi_dtype q_dtype, float q_scale, int32_t qo_len, const void* k,
                                 const void* v, fi_dtype k_dtype, fi_dtype v_dtype, int32_t kv_len,
                                 int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t causal,
                                 int32_t pv_fp8, float k_scale, float v_scale, void* o, fi_dtype o_dtype, float* lse,
                                 float sm_scale, void* stream) {
  return single_prefill("fi_single_prefill_fp8q", true, q, q_dtype, q_scale, qo_len, k, v, k_dtype, v_dtype, kv_len,
                        num_qo_heads, num_kv_heads, head_dim, causal, pv_fp8, k_scale, v_scale, o, o_dtype, lse,
                        sm_scale, stream);
}

fi_status fi_fp8_widen(const uint8_t* codes, int64_t n, fi_dtype src, fi_dtype dst, void* out, void* stream) {
  static const char* fn = "fi_fp8_widen";
  if (!is_any_fp8(src))
    return fail(FI_E_DTYPE, fn, "src has dtype %s; src must be float8_e4m3fn, float8_e5m2, float8_e4m3fnuz or "
                "float8_e5m2fnuz", dtype_name(src));
  if (!is_2byte(dst)) return fail(FI_E_DTYPE, fn, "dst has dtype %s; dst must be float16 or bfloat16", dtype_name(dst));
  if (n < 0) return fail(FI_E_SHAPE, fn, "n=%lld is negative", (long long)n);
  if (n == 0) return FI_OK;
  if (!codes || !out) return fail(FI_E_ARG, fn, "codes and out must not be NULL");
  if (reinterpret_cast<uintptr_t>(out) & 1u) return fail(FI_E_ARG, fn, "out must be 2-byte aligned");
  hipError_t err = fi::launch_fp8_widen(codes, n, src, dst, out, reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(FI_E_HIP, fn, "widen kernel launch failed: %s", hipGetErrorString(err));
  return FI_OK;
}

}  // extern "C"
