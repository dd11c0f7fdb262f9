// One launch over a prefill batch and a decode batch ("POD": prefill and
// decode attention in one kernel).  "fp8 KV cache in the in-tree prefill
// kernel" (AMD-Ecosystem/flashinfer PR #368) lists the POD and batch-POD run
// entry points beside prefill and decode (Refusals; Architecture / design
// notes): one call whose two phases share the query and KV dtypes, a 2-byte
// KV equal to the query as in prefill, and the k/v dtype check; that fork
// refuses fp8 KV there because its POD kernels instantiate the prefill
// kernel's fragment traits, a limitation of that code and not of the method.
//
// Mapping onto gfx950.  A prefill workgroup (8 waves, up to 256 VGPRs each)
// fills a CU's register file, so a decode workgroup cannot share a CU with
// one; the two phases share the GPU by CUs instead.  The decode stream is
// bound by HBM, not by CUs: a few CUs stream it (each decode workgroup
// reaching ~20 GB/s while the memory system is far from saturated) while the
// other CUs compute prefill items, which then also take the CUs the decode
// workgroups leave.  The hardware dispatches workgroups in index order, so
// by default the decode slices come first, cut for a decode share of CUs that
// balances the two phases' estimated durations, then the prefill items
// (heaviest first); the prefill-first order remains selectable.  The kernel
// runs 512 threads per workgroup: the decode workgroups run the decode body
// with 8 waves, each wave one (kv head, 16-row slice) as in the decode
// kernel, the workgroup reading up to 8 heads' rows of each token; the others
// run the prefill body's items.  Split decode rows are combined by the decode
// merge kernel afterwards, as for fi_batch_decode_paged.
#include <type_traits>

#include "fi_decode_body.hpp"
#include "fi_prefill_body.hpp"

namespace fi {

static_assert(kPodDecodeWaves == kPrefillWaves, "the fused launch has one workgroup size");

template <int QF, int KVF, bool OBF16, int D>
__global__ __launch_bounds__(64 * kPrefillWaves, 1) void pod_kernel(const PodParams p) {
  constexpr bool QBF16 = QF == FMT_BF16;
  using PC = PrefillCfg<QBF16, KVF, OBF16, D, false, false>;
  using DC = DecodeCfg<QBF16, KVF, OBF16, D, kPodDecodeWaves>;
  constexpr int kLds = PC::LDS > DC::LDS ? PC::LDS : DC::LDS;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  const int x = blockIdx.x;
  const int xp = p.decode_first ? x - p.n_decode_wg : x;  // prefill item, if >= 0
  if (xp >= 0 && xp < p.n_prefill_wg)
    prefill_body<QF, KVF, OBF16, D, false, false>(p.pf, xp, 0, smem);
  else
    decode_body<QBF16, KVF, OBF16, D, 0, kPodDecodeWaves>(p.dc, p.decode_first ? x : x - p.n_prefill_wg,
                                                          p.n_decode_wg, smem);
}

template <int QF, int KVF, bool OBF16, int D>
static hipError_t launch_pod_t(const PodParams& p, hipStream_t s) {
  const unsigned n = (unsigned)p.n_prefill_wg + (unsigned)p.n_decode_wg;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((pod_kernel<QF, KVF, OBF16, D>), dim3(n), dim3(64 * kPrefillWaves), 0, s, p);
  return hipGetLastError();
}

template <int QF, int KVF>
static hipError_t launch_pod_o(const PodParams& p, int o_fmt, int head_dim, hipStream_t s) {
  if (o_fmt == FMT_BF16)
    return head_dim == 128 ? launch_pod_t<QF, KVF, true, 128>(p, s) : launch_pod_t<QF, KVF, true, 64>(p, s);
  return head_dim == 128 ? launch_pod_t<QF, KVF, false, 128>(p, s) : launch_pod_t<QF, KVF, false, 64>(p, s);
}

template <int QF>
static hipError_t launch_pod_kv(const PodParams& p, int kv_fmt, int o_fmt, int head_dim, hipStream_t s) {
  switch (kv_fmt) {
    case FMT_E4M3: return launch_pod_o<QF, FMT_E4M3>(p, o_fmt, head_dim, s);
    case FMT_E5M2: return launch_pod_o<QF, FMT_E5M2>(p, o_fmt, head_dim, s);
    case FMT_E4M3_FNUZ: return launch_pod_o<QF, FMT_E4M3_FNUZ>(p, o_fmt, head_dim, s);
    case FMT_E5M2_FNUZ: return launch_pod_o<QF, FMT_E5M2_FNUZ>(p, o_fmt, head_dim, s);
  }
  if (kv_fmt != QF) return hipErrorInvalidValue;  // a 2-byte KV must be q's type
  return launch_pod_o<QF, QF>(p, o_fmt, head_dim, s);
}

hipError_t launch_pod(const PodParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, hipStream_t s) {
  if (q_fmt == FMT_BF16) return launch_pod_kv<FMT_BF16>(p, kv_fmt, o_fmt, head_dim, s);
  if (q_fmt == FMT_F16) return launch_pod_kv<FMT_F16>(p, kv_fmt, o_fmt, head_dim, s);
  return hipErrorInvalidValue;
}

}  // namespace fi
