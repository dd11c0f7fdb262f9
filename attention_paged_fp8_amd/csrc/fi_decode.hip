// Batched paged decode for gfx950, the split-KV state merge, and the fp8 widen
// kernel used to test the conversion code by code.
//
// What is computed: for each request and q head, softmax(q K^T * sm_scale) V
// over the request's paged K/V, with K and V stored as OCP fp8 (or a 2-byte
// type) and per-tensor k_scale / v_scale ("fp8 KV cache in the in-tree
// prefill kernel", AMD-Ecosystem/flashinfer PR #368: Summary, Test plan;
// "Enable Hopper FA3 FP8 attention in decode.py", flashinfer PR #2148:
// plan()/run() arguments and split-KV knobs).
//
// Mapping onto the hardware.  A workgroup of 4 waves owns one (request, chunk
// of C tokens, group of adjacent kv heads); each wave owns one (kv head,
// 16-row slice of its GQA group).  The chunk is walked in 16-token steps:
//   * the whole workgroup loads the step's rows of its heads -- for fp8 K/V
//     and head_dim 128, 4 heads x 128 B = 512 contiguous bytes per token and
//     pool, the access pattern that measured closest to whole-page streaming
//     on MI355X -- with 16-byte loads, two steps ahead, and stores them into an
//     LDS stage whose 16-byte chunks are XOR-swizzled by row;
//   * each wave reads its head's K rows from LDS (conflict-free 16-byte reads),
//     widens fp8 in registers and multiplies on MFMA 16x16x32 as
//     S^T = K * Q^T: the group's q rows (padded to 16) are the N dimension,
//     the step's tokens the M dimension, and Q^T and K use the same
//     permutation of head_dim;
//   * the probabilities of the S^T accumulators are exactly the P^T operand of
//     MFMA 16x16x16, so O^T += V^T * P^T needs V column-wise: one transposed
//     LDS read (ds_read_b64_tr_b8) yields a lane's 4-token column of two
//     16-wide head_dim blocks at once (tr_b16 for 2-byte V);
//   * the MFMA type is bf16 when q or a 2-byte cache is bf16, else fp16; an
//     fp16 operand meeting a bf16 one (mixed 2-byte decode) is split exactly
//     into two bf16 MFMA operands, so no value is rounded;
//   * the online softmax keeps a running max per row in base 2 (the logit
//     scale sm_scale * k_scale * log2(e) folded into one multiply) and two
//     sums: of the fp32 probabilities, for the log-sum-exp, and of the
//     probabilities after rounding to the MFMA type, which are the weights the
//     PV MFMA applies, to normalise the output (so a constant V comes out
//     unchanged).
// Each wave writes either its rows' final output (v_scale applied before the
// single rounding) or, when the request is split into several chunks, an fp32
// partial (output, log-sum-exp) that merge_kernel combines.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "fi_decode_body.hpp"

namespace fi {

// Workgroups per CU the register allocation is sized for (4 waves each).
#ifndef FI_DECODE_MIN_WG_PER_CU
#define FI_DECODE_MIN_WG_PER_CU 3
#endif

// Q8: an fp8 query (see decode_body).  NW: waves per workgroup -- 4, or 8
// for long per-workgroup streams, where a workgroup reading whole 1 KB rows
// of 8 heads streams faster (long-context workload 287 -> 275 us).
// The second launch bound is waves per SIMD: a 4-wave workgroup puts one wave
// on each SIMD, an 8-wave one two.  The fnuz forms hold a step's codes in
// registers before widening them, and get the registers of two workgroups per
// CU; an 8-wave workgroup runs one per CU (its stage is twice as wide).
template <bool QBF16, int KVF, bool OBF16, int D, int Q8 = 0, int NW = kDecodeWaves>
__global__ __launch_bounds__(64 * NW, (KVF == FMT_E4M3_FNUZ || KVF == FMT_E5M2_FNUZ) || NW == 8
                                          ? 2
                                          : FI_DECODE_MIN_WG_PER_CU) void
decode_kernel(
    const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DecodeCfg<QBF16, KVF, OBF16, D, NW>::LDS];
  decode_body<QBF16, KVF, OBF16, D, Q8, NW>(p, blockIdx.x, gridDim.x, smem);
}

// ---------------------------------------------------------------------------
// Split-KV merge: L = log2 sum_c 2^lse_c, o = v_scale * sum_c 2^(lse_c - L) o_c
// (the natural-log form of the same identity is the oracle's merge_states).
// One wave per (request, q head), kMergeWaves per workgroup.  The segment's
// piece count says what to do: 0 = a request without keys (o = 0, lse =
// -inf), 1 = the decode kernel already wrote the result, n > 1 = merge n
// partials.  Lane c holds chunk c's log-sum-exp (64 chunks per pass), the
// lanes split head_dim, and the weights reach every lane through shuffles:
// two dependent memory round trips (the count, then the partials), no LDS.
// ---------------------------------------------------------------------------
constexpr int kMergeWaves = 4;

template <bool OBF16, int D>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(const MergeParams p) {
  constexpr int PL = D / 64;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (pair >= p.batch * p.num_qo_heads) return;
  const int hq = pair % p.num_qo_heads;
  const int b = pair / p.num_qo_heads;
  // the (head group, slice group) this q head belongs to, as the decode kernel numbers them
  const int gkv = hq / p.group;
  const int sub = (hq - gkv * p.group) / kDecodeRows;
  const int grp = (sub / p.spw) * p.n_hgroups + (gkv >> p.hpw_shift);
  const int n = min(p.max_chunks, p.nch[(int64_t)b * p.n_hgroups * p.n_sgroups + grp]);
  uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)b * p.num_qo_heads + hq) * D + PL * lane;
  float* lsep = p.lse ? p.lse + (int64_t)b * p.num_qo_heads + hq : nullptr;
  if (n == 1) return;
  if (n <= 0) {
    if constexpr (PL == 2) *reinterpret_cast<uint32_t*>(op) = 0u;
    else *op = 0;
    if (lsep && lane == 0) *lsep = kNegInf;
    return;
  }
  const int64_t base = ((int64_t)b * p.num_qo_heads + hq) * p.max_chunks;
  const float* lse = p.part_lse + base;
  const float* po = p.part_o + base * D + PL * lane;
  float M = kNegInf;
  for (int c0 = 0; c0 < n; c0 += 64)
    if (c0 + lane < n) M = fmaxf(M, lse[c0 + lane]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float L = 0.f;
  float acc[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const float lc = (c0 + lane < n) ? lse[c0 + lane] : kNegInf;
    const float wl = (lc == kNegInf) ? 0.f : fast_exp2(lc - M);
    L += wl;
    const int cn = min(64, n - c0);
    // blocks of 8 partials: all 8 loads in flight before the first is used
    for (int k0 = 0; k0 < cn; k0 += 8) {
      float v[8][PL];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int i = 0; i < PL; ++i) v[k][i] = (k0 + k < cn) ? po[(int64_t)(c0 + k0 + k) * D + i] : 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float wk = __shfl(wl, k0 + k);
#pragma unroll
        for (int i = 0; i < PL; ++i) acc[i] += wk * v[k][i];
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  // L is 0 only when every piece is empty; a NaN partial makes it NaN
  const float f = (L != 0.f) ? p.v_scale / L : 0.f;
  if constexpr (PL == 2) *reinterpret_cast<uint32_t*>(op) = pack2<OBF16>(acc[0] * f, acc[1] * f);
  else *op = to_bits<OBF16>(acc[0] * f);
  if (lsep && lane == 0) *lsep = (L != 0.f) ? (M + fast_log2(L)) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------------------
// fp8 -> 2-byte widening of a code buffer (conformance of widen4).
// ---------------------------------------------------------------------------
template <bool BF16, int KVF>
__global__ __launch_bounds__(256) void widen_kernel(const uint8_t* codes, int64_t n, uint16_t* out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (i + j < n) w |= (uint32_t)codes[i + j] << (8 * j);
  uint2 r = widen4<BF16, KVF>(w);
  if constexpr (KVF == FMT_E4M3_FNUZ) {  // the attention kernels fold this 2^7 into their scales
    r.x = pack2<BF16>(unpack2<BF16>(r.x).x * 128.f, unpack2<BF16>(r.x).y * 128.f);
    r.y = pack2<BF16>(unpack2<BF16>(r.y).x * 128.f, unpack2<BF16>(r.y).y * 128.f);
  }
  const uint16_t v[4] = {(uint16_t)(r.x & 0xffff), (uint16_t)(r.x >> 16), (uint16_t)(r.y & 0xffff),
                         (uint16_t)(r.y >> 16)};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (i + j < n) out[i + j] = v[j];
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode call (fi_batch_decode_paged_noalloc):
// the split-KV partial states and piece counts live in this array instead of
// a caller's workspace.  Every GPU holds its own copy until the process ends.
// Host code never names the array itself (on the host the name is only a
// stand-in, not a device address): it asks the runtime for the current
// device's address once per device and passes that pointer to the kernels as
// the workspace.  Nothing in it needs to start at zero: a call writes every
// piece count and every partial state it later reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <bool QBF16, int KVF, bool OBF16, int D, int Q8, int NW>
static hipError_t launch_decode_t(const DecodeParams& p, int batch, hipStream_t s) {
  dim3 grid(p.balanced ? (unsigned)p.n_wg : (unsigned)p.max_chunks * p.n_hgroups * p.n_sgroups * batch);
  if (grid.x == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<QBF16, KVF, OBF16, D, Q8, NW>), grid, dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

// the 8-wave kernel where it exists (decode_long_supported), else the 4-wave one
template <bool QBF16, int KVF, int Q8>
constexpr bool kHasLong = Q8 == 0 && (KVF == FMT_E4M3 || KVF == FMT_E5M2 || KVF == (QBF16 ? FMT_BF16 : FMT_F16));

template <bool QBF16, int KVF, bool OBF16, int Q8>
static hipError_t launch_decode_d(const DecodeParams& p, int head_dim, int batch, int nw, hipStream_t s) {
  if constexpr (kHasLong<QBF16, KVF, Q8>) {
    if (nw == kDecodeWavesLong) {
      if (head_dim == 128) return launch_decode_t<QBF16, KVF, OBF16, 128, Q8, kDecodeWavesLong>(p, batch, s);
      return launch_decode_t<QBF16, KVF, OBF16, 64, Q8, kDecodeWavesLong>(p, batch, s);
    }
  }
  if (nw != kDecodeWaves) return hipErrorInvalidValue;
  if (head_dim == 128) return launch_decode_t<QBF16, KVF, OBF16, 128, Q8, kDecodeWaves>(p, batch, s);
  return launch_decode_t<QBF16, KVF, OBF16, 64, Q8, kDecodeWaves>(p, batch, s);
}

template <bool QBF16, int KVF, int Q8>
static hipError_t launch_decode_o(const DecodeParams& p, int o_fmt, int head_dim, int batch, int nw, hipStream_t s) {
  if (o_fmt == FMT_BF16) return launch_decode_d<QBF16, KVF, true, Q8>(p, head_dim, batch, nw, s);
  return launch_decode_d<QBF16, KVF, false, Q8>(p, head_dim, batch, nw, s);
}

template <bool QBF16, int Q8>
static hipError_t launch_decode_kv(const DecodeParams& p, int kv_fmt, int o_fmt, int head_dim, int batch, int nw,
                                   hipStream_t s) {
  switch (kv_fmt) {
    case FMT_E4M3: return launch_decode_o<QBF16, FMT_E4M3, Q8>(p, o_fmt, head_dim, batch, nw, s);
    case FMT_E5M2: return launch_decode_o<QBF16, FMT_E5M2, Q8>(p, o_fmt, head_dim, batch, nw, s);
    case FMT_E4M3_FNUZ: return launch_decode_o<QBF16, FMT_E4M3_FNUZ, Q8>(p, o_fmt, head_dim, batch, nw, s);
    case FMT_E5M2_FNUZ: return launch_decode_o<QBF16, FMT_E5M2_FNUZ, Q8>(p, o_fmt, head_dim, batch, nw, s);
  }
  if constexpr (Q8 != 0) {
    return hipErrorInvalidValue;  // an fp8 query needs an fp8 cache
  } else {
    if (kv_fmt == FMT_F16) return launch_decode_o<QBF16, FMT_F16, 0>(p, o_fmt, head_dim, batch, nw, s);
    return launch_decode_o<QBF16, FMT_BF16, 0>(p, o_fmt, head_dim, batch, nw, s);
  }
}

template <bool QBF16, int KVF, bool OBF16, int D, int Q8, int NW>
static int occupancy_t() {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ,
                                                   reinterpret_cast<const void*>(&decode_kernel<QBF16, KVF, OBF16, D, Q8, NW>),
                                                   64 * NW, 0) != hipSuccess)
    return 0;
  return occ;
}

template <bool QBF16, int KVF, bool OBF16, int Q8>
static int occupancy_d(int d, int nw) {
  if constexpr (kHasLong<QBF16, KVF, Q8>) {
    if (nw == kDecodeWavesLong)
      return d == 128 ? occupancy_t<QBF16, KVF, OBF16, 128, Q8, kDecodeWavesLong>()
                      : occupancy_t<QBF16, KVF, OBF16, 64, Q8, kDecodeWavesLong>();
  }
  if (nw != kDecodeWaves) return 0;
  return d == 128 ? occupancy_t<QBF16, KVF, OBF16, 128, Q8, kDecodeWaves>()
                  : occupancy_t<QBF16, KVF, OBF16, 64, Q8, kDecodeWaves>();
}

template <bool QBF16, int KVF, int Q8>
static int occupancy_o(int o, int d, int nw) {
  return o == FMT_BF16 ? occupancy_d<QBF16, KVF, true, Q8>(d, nw) : occupancy_d<QBF16, KVF, false, Q8>(d, nw);
}

template <bool QBF16, int Q8>
static int occupancy_kv(int kv, int o, int d, int nw) {
  switch (kv) {
    case FMT_E4M3: return occupancy_o<QBF16, FMT_E4M3, Q8>(o, d, nw);
    case FMT_E5M2: return occupancy_o<QBF16, FMT_E5M2, Q8>(o, d, nw);
    case FMT_E4M3_FNUZ: return occupancy_o<QBF16, FMT_E4M3_FNUZ, Q8>(o, d, nw);
    case FMT_E5M2_FNUZ: return occupancy_o<QBF16, FMT_E5M2_FNUZ, Q8>(o, d, nw);
  }
  if constexpr (Q8 != 0) {
    return 0;
  } else {
    return kv == FMT_F16 ? occupancy_o<QBF16, FMT_F16, 0>(o, d, nw) : occupancy_o<QBF16, FMT_BF16, 0>(o, d, nw);
  }
}

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

int decode_slots(int q_fmt, int kv_fmt, int o_fmt, int head_dim, int nw) {
  // cached per (device, instantiation): the values cannot change while the process runs
  static std::atomic<int> cache[64][4][10][2][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || kv_fmt < 0 || kv_fmt >= 10) return 0;
  const int qi = q_fmt == FMT_BF16 ? 1 : q_fmt == FMT_E4M3 ? 2 : q_fmt == FMT_E5M2 ? 3 : 0;
  std::atomic<int>& slot = cache[dev][qi][kv_fmt][o_fmt == FMT_BF16][head_dim == 128][nw == kDecodeWavesLong];
  int v = slot.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int occ = qi == 1   ? occupancy_kv<true, 0>(kv_fmt, o_fmt, head_dim, nw)
                  : qi == 2 ? occupancy_kv<false, FMT_E4M3>(kv_fmt, o_fmt, head_dim, nw)
                  : qi == 3 ? occupancy_kv<false, FMT_E5M2>(kv_fmt, o_fmt, head_dim, nw)
                            : occupancy_kv<false, 0>(kv_fmt, o_fmt, head_dim, nw);
  v = cus * occ;
  slot.store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_decode(const DecodeParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, int batch, int nw,
                         hipStream_t s) {
  if (q_fmt == FMT_BF16) return launch_decode_kv<true, 0>(p, kv_fmt, o_fmt, head_dim, batch, nw, s);
  if (q_fmt == FMT_E4M3) return launch_decode_kv<false, FMT_E4M3>(p, kv_fmt, o_fmt, head_dim, batch, nw, s);
  if (q_fmt == FMT_E5M2) return launch_decode_kv<false, FMT_E5M2>(p, kv_fmt, o_fmt, head_dim, batch, nw, s);
  return launch_decode_kv<false, 0>(p, kv_fmt, o_fmt, head_dim, batch, nw, s);
}

hipError_t launch_merge(const MergeParams& p, int o_fmt, int head_dim, int batch, hipStream_t s) {
  dim3 grid((unsigned)(((int64_t)p.num_qo_heads * batch + kMergeWaves - 1) / kMergeWaves));
  dim3 block(64 * kMergeWaves);
  if (o_fmt == FMT_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((merge_kernel<true, 128>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((merge_kernel<true, 64>), grid, block, 0, s, p);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((merge_kernel<false, 128>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((merge_kernel<false, 64>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_widen(const uint8_t* codes, int64_t n, int src_fmt, int dst_fmt, void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  dim3 grid((unsigned)((threads + 255) / 256));
  uint16_t* o = reinterpret_cast<uint16_t*>(out);
  auto go = [&](auto fmt) {
    constexpr int KVF = decltype(fmt)::value;
    if (dst_fmt == FMT_BF16)
      hipLaunchKernelGGL((widen_kernel<true, KVF>), grid, dim3(256), 0, s, codes, n, o);
    else
      hipLaunchKernelGGL((widen_kernel<false, KVF>), grid, dim3(256), 0, s, codes, n, o);
  };
  switch (src_fmt) {
    case FMT_E4M3: go(std::integral_constant<int, FMT_E4M3>{}); break;
    case FMT_E5M2: go(std::integral_constant<int, FMT_E5M2>{}); break;
    case FMT_E4M3_FNUZ: go(std::integral_constant<int, FMT_E4M3_FNUZ>{}); break;
    default: go(std::integral_constant<int, FMT_E5M2_FNUZ>{}); break;
  }
  return hipGetLastError();
}

}  // namespace fi
