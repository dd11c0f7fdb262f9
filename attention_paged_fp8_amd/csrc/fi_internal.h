// Internal interface between the host front end (fi_api.cpp) and the kernel
// translation units.  Plain structs passed to kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fi {

// Stored element formats; the values match fi_dtype.
enum Fmt : int { FMT_F16 = 1, FMT_BF16 = 2, FMT_E4M3 = 3, FMT_E5M2 = 4 };

constexpr int kDecodeWaves = 4;         // waves per decode workgroup
constexpr int kDecodeBlock = 32;        // tokens per wave step
constexpr int kChunkQuantum = kDecodeWaves * kDecodeBlock;  // split-KV chunk granularity
constexpr int kDecodeRows = 16;         // q rows per decode MFMA tile (one GQA subgroup)
constexpr float kLog2eHost = 1.4426950408889634f;

struct DecodeParams {
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
  int32_t nsub;           // ceil(group / 16)
  int32_t chunk;          // tokens per workgroup (multiple of kChunkQuantum)
  int32_t max_chunks;     // chunks of the longest request
  int32_t batch;
  float scale_log2;       // sm_scale * k_scale * log2(e)
  float v_scale;
  float* part_o;          // [batch, max_chunks, Hqo, D] fp32, normalised, unscaled by v_scale
  float* part_lse;        // [batch, max_chunks, Hqo] base-2 log-sum-exp
};

struct MergeParams {
  void* o;
  float* lse;
  const float* part_o;
  const float* part_lse;
  const int32_t* indptr;
  const int32_t* last_page_len;
  int32_t page_size;
  int32_t single_kv_len;
  int32_t num_qo_heads;
  int32_t chunk;
  int32_t max_chunks;
  float v_scale;
};

struct PrefillParams {
  const void* q;          // [total_q, Hqo, D]
  void* o;
  float* lse;
  const uint8_t* k;
  const uint8_t* v;
  int64_t sp, st, sh;     // bytes
  const int32_t* qo_indptr;
  const int32_t* indptr;
  const int32_t* indices;
  const int32_t* last_page_len;
  int32_t page_shift;
  int32_t page_size;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t heads_per_wg;   // 1, 2 or 4
  int32_t q_per_wg;       // 128 / heads_per_wg query tokens per workgroup
  int32_t n_qblocks;      // grid.y
  int32_t causal;
  float scale_log2;
  float v_scale;
};

// Kernel launchers (defined in the .hip translation units).  They return the
// hipError_t of the launch.
hipError_t launch_decode(const DecodeParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, int batch,
                         hipStream_t s);
hipError_t launch_merge(const MergeParams& p, int o_fmt, int head_dim, int batch, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, int batch,
                          hipStream_t s);
hipError_t launch_fp8_widen(const uint8_t* codes, int64_t n, int src_fmt, int dst_fmt, void* out, hipStream_t s);

}  // namespace fi
