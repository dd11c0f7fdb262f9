// Internal interface between the host front end (fi_api.cpp) and the kernel
// translation units.  Plain structs passed to kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fi {

// Stored element formats; the values match fi_dtype.
enum Fmt : int { FMT_F16 = 1, FMT_BF16 = 2, FMT_E4M3 = 3, FMT_E5M2 = 4, FMT_E4M3_FNUZ = 8, FMT_E5M2_FNUZ = 9 };

constexpr int kDecodeWaves = 4;         // waves per decode workgroup, one (kv head, row slice) each
constexpr int kDecodeWavesLong = 8;     // the same for long per-workgroup streams (whole 1 KB rows of 8 heads)
constexpr int kDecodeStep = 16;         // tokens staged per step
constexpr int kChunkQuantum = 64;       // split-KV chunk granularity (tokens)
constexpr int kDecodeRows = 16;         // q rows per decode MFMA tile (one GQA slice)
constexpr float kLog2eHost = 1.4426950408889634f;
constexpr int kBalancedMaxBatch = 1024; // largest batch the balanced decode split handles
constexpr int kDecodePrefixMax = 768;   // largest batch whose token prefix sums travel in the kernel arguments

// NPRE: capacity of the token prefix sums carried in the arguments
template <int NPRE>
struct DecodeParamsT {
  static constexpr int kPrefixMax = NPRE;
  const void* q;          // [tokens, Hqo, D]
  void* o;                // [tokens, Hqo, D]
  float* lse;             // [tokens, Hqo] or null
  const uint8_t* k;       // pool base (bytes)
  const uint8_t* v;
  int64_t sp, st, sh;     // strides in bytes: page, token, head
  const int32_t* indptr;  // null: single contiguous sequence of single_kv_len tokens
  const int32_t* indices;
  const int32_t* last_page_len;
  int32_t page_shift;     // log2(page_size)
  int32_t page_size;
  int32_t single_kv_len;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group;          // Hqo / Hkv
  int32_t nsub;           // 16-row slices of a GQA group: ceil(group / 16)
  int32_t hpw_shift;      // log2(kv heads per workgroup): 0, 1 or 2
  int32_t spw;            // slices per workgroup (waves = heads x slices <= 4)
  int32_t n_hgroups;      // kv head groups: num_kv_heads >> hpw_shift
  int32_t n_sgroups;      // slice groups: ceil(nsub / spw)
  int32_t chunk;          // fixed chunks: tokens per workgroup (multiple of kChunkQuantum)
  int32_t max_chunks;     // pieces a (request, group) segment can have: partial buffer stride
  int32_t batch;
  int32_t balanced;       // 1: equal slices of the (group, request, token) space
  int32_t n_wg;           // balanced: workgroups launched
  int64_t slice;          // balanced: (group x token) items per workgroup
  int32_t spg;            // balanced, interleaved: token slices per group (workgroup w: group w % groups,
                          // slice w / groups); 0: slices of the group-major item space
  int32_t* nch;           // [batch, groups] pieces per segment, written for the merge (or null)
  float scale_log2;       // sm_scale * k_scale * log2(e)
  float v_scale;
  float* part_o;          // [batch, Hqo, max_chunks, D] fp32, normalised, unscaled by v_scale
  float* part_lse;        // [batch, Hqo, max_chunks] base-2 log-sum-exp
  // balanced: token prefix sums of the requests, from the host's page table
  // (pre[i] = tokens of requests < i, i <= batch) when they fit; else
  // pre_n = 0 and every workgroup scans the device page table itself
  int32_t pre_n;
  int32_t pre[NPRE + 1];
};
using DecodeParams = DecodeParamsT<kDecodePrefixMax>;

struct MergeParams {
  void* o;
  float* lse;
  const float* part_o;
  const float* part_lse;
  const int32_t* nch;     // [batch, groups] pieces per segment (0: a request without keys)
  int32_t batch;
  int32_t num_qo_heads;
  int32_t group;          // q heads per kv head
  int32_t hpw_shift, spw, n_hgroups, n_sgroups;
  int32_t max_chunks;
  float v_scale;
};

// Prefill workgroups: waves of 32 query rows sharing each K/V tile.
constexpr int kPrefillWaves = 8;
// Largest number of (request, query block) pairs whose dispatch order travels
// in the kernel arguments (4 bytes each), and of requests whose geometry does
// (16 bytes each).
constexpr int kPrefillOrderMax = 512;
constexpr int kPrefillGeoMax = 96;

// NORD: capacity of the dispatch order carried in the arguments; NGEO: of
// the request geometry
template <int NORD, int NGEO>
struct PrefillParamsT {
  static constexpr int kOrderMax = NORD;
  static constexpr int kGeoMax = NGEO;
  const void* q;          // [total_q, Hqo, D]
  void* o;
  float* lse;
  const uint8_t* k;
  const uint8_t* v;
  int64_t sp, st, sh;     // bytes
  const int32_t* qo_indptr;
  const int32_t* indptr;  // pages per request; token rows per request when ragged
  const int32_t* indices;
  const int32_t* last_page_len;
  int32_t page_shift;
  int32_t page_size;
  int32_t single_qo_len;  // when qo_indptr (and indptr) are NULL: the one request's
  int32_t single_kv_len;  // queries and keys (ragged K/V from row 0)
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t heads_per_wg;   // 1, 2 or 4
  int32_t q_per_wg;       // 32 * kPrefillWaves / heads_per_wg query tokens per workgroup
  int32_t n_qblocks;      // grid.y when n_items == 0
  int32_t causal;
  int32_t pv_fp8;         // fp8 queries: P rounded to e4m3 and P V on the fp8 MFMA
  float scale_log2;
  float v_scale;
  // Dispatch order: when n_items > 0, workgroup x serves pair order[x / (kv
  // heads * head groups)] = request << 16 | query block, listed heaviest
  // first; otherwise x = (request, kv head, head group) and y = query block.
  int32_t n_items;
  uint32_t order[NORD];
  // Request geometry from the host's copies of the index arrays, so that a
  // workgroup's first page-id loads need no device load before them: per
  // request, its first query row, queries, first page (ragged: first K/V row)
  // and keys.  n_geo = batch when it fits, else 0 (read from the device).
  int32_t n_geo;
  int32_t geo[NGEO][4];
};
using PrefillParams = PrefillParamsT<kPrefillOrderMax, kPrefillGeoMax>;

// One launch over a prefill batch and a decode batch ("POD"): n_prefill_wg
// workgroups run prefill work items in the heaviest-first order and
// n_decode_wg run decode slices with kPodDecodeWaves waves each, the prefill
// items first unless decode_first.  The
// two plans share the kernel-argument budget of one launch, so their lists
// are shorter than the separate calls'.
constexpr int kPodDecodeWaves = 8;
constexpr int kPodOrderMax = 384;
constexpr int kPodGeoMax = 48;
constexpr int kPodPrefixMax = 256;
struct PodParams {
  PrefillParamsT<kPodOrderMax, kPodGeoMax> pf;
  DecodeParamsT<kPodPrefixMax> dc;
  int32_t n_prefill_wg;
  int32_t n_decode_wg;
  int32_t decode_first;  // 1: the decode slices take the first workgroup indices
};
static_assert(sizeof(PodParams) <= 4096, "POD kernel arguments exceed 4 KB");
static_assert(sizeof(PrefillParams) <= 4096, "prefill kernel arguments exceed 4 KB");
static_assert(sizeof(DecodeParams) <= 4096, "decode kernel arguments exceed 4 KB");

// Kernel launchers (defined in the .hip translation units).  They return the
// hipError_t of the launch.
// nw: kDecodeWaves, or kDecodeWavesLong where decode_long_supported().
hipError_t launch_decode(const DecodeParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, int batch, int nw,
                         hipStream_t s);
// The 8-wave decode kernel exists for a 2-byte query over an OCP fp8 cache or
// a cache of the query's own type.
inline bool decode_long_supported(int q_fmt, int kv_fmt) {
  return (q_fmt == FMT_F16 || q_fmt == FMT_BF16) && (kv_fmt == FMT_E4M3 || kv_fmt == FMT_E5M2 || kv_fmt == q_fmt);
}
hipError_t launch_merge(const MergeParams& p, int o_fmt, int head_dim, int batch, hipStream_t s);
// Workgroups of the decode kernel for these types that fit on the current device at once.
int decode_slots(int q_fmt, int kv_fmt, int o_fmt, int head_dim, int nw = kDecodeWaves);
int device_cus();  // compute units of the current device (0 on error), cached
// ragged: K/V rows addressed as indptr[b] + t (stride st) instead of a page table
hipError_t launch_prefill(const PrefillParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, int batch,
                          bool ragged, hipStream_t s);
hipError_t launch_fp8_widen(const uint8_t* codes, int64_t n, int src_fmt, int dst_fmt, void* out, hipStream_t s);
// POD: q in {f16, bf16}, KV q's 2-byte type or any fp8, paged prefill with a 2-byte query
hipError_t launch_pod(const PodParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, hipStream_t s);

// Split-KV scratch of the allocation-free decode call: a file-scope device
// array of kDecodeScratchBytes in the decode translation unit, one copy per
// GPU.  decode_scratch() returns the current device's address of it (looked
// up once per device with hipGetSymbolAddress and cached).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace fi
