// Batched (causal) prefill over a paged KV cache for gfx950.
//
// What is computed: for every query token of every request and every q head,
// softmax(q K^T * sm_scale) V over the keys the (optional) causal mask leaves
// visible, with K and V stored as OCP fp8, as the gfx942 fnuz fp8 layouts
// (widened exactly from their bits) or as q's 2-byte type ("fp8 KV cache in
// the in-tree prefill kernel", AMD-Ecosystem/flashinfer PR #368: Summary,
// Kernel, Architecture / design notes, Benchmark results).  The causal mask is aligned to
// the end of the KV sequence: row r sees key t iff t <= r + kv_len - qo_len.
//
// Mapping.  A workgroup of 8 waves owns one (request, kv head, group of heads,
// block of query tokens); every wave holds 32 query rows of one q head, so the
// 8 waves (256 rows, up to 4 q heads of a GQA group) share each K/V tile and
// its gather, widening and LDS stores.
// Per 64-token K/V tile:
//   * the workgroup gathers the tile's rows from their pages with coalesced
//     16-byte loads (8 lanes per 128-byte fp8 row), four tiles ahead, widens
//     fp8 to q's type in registers and stores 2-byte K and V tiles in LDS --
//     the dequantize-on-load design the PR describes (Kernel; Architecture /
//     design notes), with the wide loads its Known limitations ask for.
//     The LDS traffic is laid out to be free of bank conflicts (measured with
//     the SQ_LDS_BANK_CONFLICT counter on gfx950): each row's stores are two
//     contiguous 128-byte runs (the fp8 head dimensions are permuted to make
//     them so; Q is loaded in the same order and the output undoes it), the K
//     pitch is 16 mod 256 bytes for the 16-byte reads of 32 rows, and the V
//     pitch 64 mod 256 bytes for the transposed reads of 4 rows x 32 bytes,
//     which then take 2 cycles each; every read address is a per-lane base
//     plus a compile-time offset;
//   * each wave computes S^T = K Q^T on MFMA 32x32x16 (tokens x rows), runs
//     the online softmax in base 2 and accumulates O^T += V^T P^T, the
//     probabilities feeding the MFMA straight from the S^T registers and V
//     gathered column-wise by ds_read_b64_tr_b16;
//   * the softmax is kept lean: the mask is applied only on tiles that cross
//     the causal diagonal or the end of the sequence; the logit scale and the
//     running max enter exp2 through one FMA; the output accumulator is
//     rescaled only when a row max grows by more than 2^8 (the exponents stay
//     below 2^8, so nothing overflows, and the final division by the same sum
//     makes the result independent of when the max was taken).
// The row sums of the probabilities as rounded for the PV MFMA are taken
// with v_dot2 against (1, 1), two values per instruction, exact products and
// an fp32 sum; they normalise the output and, for fp16 (rounding 2^-11), give
// the log-sum-exp.  With a bf16 query (rounding 2^-9) the log-sum-exp uses a
// separate sum of the fp32 values.
// Each wave also overlaps its two phases: the QK MFMAs of the next tile are
// issued between the exponentials of the current one.
//
// Variants (template flags):
//   * RAGGED: K/V rows contiguous per request (row indptr[b] + t), the page
//     walk reduced to an addition; with NULL index arrays a single request
//     takes its lengths from the kernel arguments.
//   * Q8 (an fp8 query, q_scale folded into the logit scale -- "Enable Hopper
//     FA3 FP8 attention in decode.py", flashinfer PR #2148, review comments):
//     K stays fp8 from HBM to the matrix cores (raw LDS tile) and S^T = K Q^T
//     runs on v_mfma_f32_32x32x64_f8f6f4, twice the 16-bit rate; P V stays fp16.
//   * P8 (with Q8): V stays fp8 too, the probabilities are rounded to e4m3
//     in registers and P V runs on the same fp8 MFMA; the output is
//     normalised by the fp32 sum of the unrounded probabilities.
#include <type_traits>

#include "fi_prefill_body.hpp"

namespace fi {

template <int QF, int KVF, bool OBF16, int D, bool RAGGED, bool P8>
__global__ __launch_bounds__(64 * kPrefillWaves, 1) void prefill_kernel(const PrefillParams p) {
  constexpr bool Q8 = QF == FMT_E4M3 || QF == FMT_E5M2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[PrefillCfg<QF == FMT_BF16, KVF, OBF16, D, Q8, P8>::LDS];
  prefill_body<QF, KVF, OBF16, D, RAGGED, P8>(p, blockIdx.x, blockIdx.y, smem);
}

template <int QF, int KVF, bool OBF16, int D>
static hipError_t launch_prefill_t(const PrefillParams& p, int batch, bool ragged, hipStream_t s) {
  const int nsg = p.group / p.heads_per_wg;
  const dim3 grid = (p.n_items > 0) ? dim3(p.n_items * p.num_kv_heads * nsg, 1)
                                    : dim3(batch * p.num_kv_heads * nsg, p.n_qblocks);
  if constexpr (QF == FMT_E4M3 || QF == FMT_E5M2) {
    if (p.pv_fp8) {
      if (ragged)
        hipLaunchKernelGGL((prefill_kernel<QF, KVF, OBF16, D, true, true>), grid, dim3(64 * kPrefillWaves), 0, s, p);
      else
        hipLaunchKernelGGL((prefill_kernel<QF, KVF, OBF16, D, false, true>), grid, dim3(64 * kPrefillWaves), 0, s, p);
    } else {
      if (ragged)
        hipLaunchKernelGGL((prefill_kernel<QF, KVF, OBF16, D, true, false>), grid, dim3(64 * kPrefillWaves), 0, s, p);
      else
        hipLaunchKernelGGL((prefill_kernel<QF, KVF, OBF16, D, false, false>), grid, dim3(64 * kPrefillWaves), 0, s, p);
    }
  } else {
    if (p.pv_fp8) return hipErrorInvalidValue;
    if (ragged)
      hipLaunchKernelGGL((prefill_kernel<QF, KVF, OBF16, D, true, false>), grid, dim3(64 * kPrefillWaves), 0, s, p);
    else
      hipLaunchKernelGGL((prefill_kernel<QF, KVF, OBF16, D, false, false>), grid, dim3(64 * kPrefillWaves), 0, s, p);
  }
  return hipGetLastError();
}

template <int QF, int KVF, bool OBF16>
static hipError_t launch_prefill_d(const PrefillParams& p, int head_dim, int batch, bool ragged, hipStream_t s) {
  if (head_dim == 128) return launch_prefill_t<QF, KVF, OBF16, 128>(p, batch, ragged, s);
  return launch_prefill_t<QF, KVF, OBF16, 64>(p, batch, ragged, s);
}

template <int QF, int KVF>
static hipError_t launch_prefill_o(const PrefillParams& p, int o_fmt, int head_dim, int batch, bool ragged,
                                   hipStream_t s) {
  if (o_fmt == FMT_BF16) return launch_prefill_d<QF, KVF, true>(p, head_dim, batch, ragged, s);
  return launch_prefill_d<QF, KVF, false>(p, head_dim, batch, ragged, s);
}

hipError_t launch_prefill(const PrefillParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, int batch,
                          bool ragged, hipStream_t s) {
  // Prefill admits a 2-byte KV only when it equals q's type, and an fp8
  // query only with an fp8 KV.
  if (q_fmt == FMT_E4M3 || q_fmt == FMT_E5M2) {
    if (kv_fmt != FMT_E4M3 && kv_fmt != FMT_E5M2) return hipErrorInvalidValue;
    if (q_fmt == FMT_E4M3) {
      if (kv_fmt == FMT_E4M3) return launch_prefill_o<FMT_E4M3, FMT_E4M3>(p, o_fmt, head_dim, batch, ragged, s);
      return launch_prefill_o<FMT_E4M3, FMT_E5M2>(p, o_fmt, head_dim, batch, ragged, s);
    }
    if (kv_fmt == FMT_E4M3) return launch_prefill_o<FMT_E5M2, FMT_E4M3>(p, o_fmt, head_dim, batch, ragged, s);
    return launch_prefill_o<FMT_E5M2, FMT_E5M2>(p, o_fmt, head_dim, batch, ragged, s);
  }
  if (q_fmt == FMT_BF16) {
    switch (kv_fmt) {
      case FMT_BF16: return launch_prefill_o<FMT_BF16, FMT_BF16>(p, o_fmt, head_dim, batch, ragged, s);
      case FMT_E4M3: return launch_prefill_o<FMT_BF16, FMT_E4M3>(p, o_fmt, head_dim, batch, ragged, s);
      case FMT_E4M3_FNUZ: return launch_prefill_o<FMT_BF16, FMT_E4M3_FNUZ>(p, o_fmt, head_dim, batch, ragged, s);
      case FMT_E5M2_FNUZ: return launch_prefill_o<FMT_BF16, FMT_E5M2_FNUZ>(p, o_fmt, head_dim, batch, ragged, s);
      default: return launch_prefill_o<FMT_BF16, FMT_E5M2>(p, o_fmt, head_dim, batch, ragged, s);
    }
  }
  switch (kv_fmt) {
    case FMT_F16: return launch_prefill_o<FMT_F16, FMT_F16>(p, o_fmt, head_dim, batch, ragged, s);
    case FMT_E4M3: return launch_prefill_o<FMT_F16, FMT_E4M3>(p, o_fmt, head_dim, batch, ragged, s);
    case FMT_E4M3_FNUZ: return launch_prefill_o<FMT_F16, FMT_E4M3_FNUZ>(p, o_fmt, head_dim, batch, ragged, s);
    case FMT_E5M2_FNUZ: return launch_prefill_o<FMT_F16, FMT_E5M2_FNUZ>(p, o_fmt, head_dim, batch, ragged, s);
    default: return launch_prefill_o<FMT_F16, FMT_E5M2>(p, o_fmt, head_dim, batch, ragged, s);
  }
}

}  // namespace fi
