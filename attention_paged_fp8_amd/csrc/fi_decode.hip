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
// Mapping onto the hardware.  A workgroup of 4 waves owns one (request, kv
// head, 16-row slice of the GQA group, chunk of C tokens).  Each wave walks
// 32-token blocks of the chunk (blocks w, w+4, ...):
//   * each lane fetches, for two tokens of the block, a DL = head_dim/4
//     element slice of the K and V rows (16-byte loads), straight from the
//     page the token lives on;
//   * K is widened in registers and multiplied on MFMA 16x16x32 as
//     S^T = K * Q^T: the group's q rows (padded to 16) are the N dimension, the
//     block's tokens the M dimension; both operands see the same permutation of
//     head_dim, so no data movement is needed for QK;
//   * V goes through a small per-wave LDS tile in its stored format; one
//     transposed LDS read (ds_read_b64_tr_b8 for fp8, two tr_b16 for 2-byte)
//     gives each lane one column over the eight tokens its P^T operand holds,
//     so that O^T += V^T * P^T runs on the same MFMA shape with the
//     probabilities taken directly from the S^T accumulator registers;
//   * the MFMA type is bf16 when q or a 2-byte cache is bf16, else fp16; an
//     fp16 operand meeting a bf16 one (mixed 2-byte decode) is split exactly
//     into two bf16 MFMA operands, so no value is rounded;
//   * the online softmax keeps a running max per row in base 2 (the logit
//     scale sm_scale * k_scale * log2(e) folded into one multiply) and two
//     sums: of the fp32 probabilities, for the log-sum-exp, and of the
//     probabilities after rounding to q's type, which are the weights the PV
//     MFMA applies, to normalise the output (so a constant V comes out
//     unchanged).
// The four waves' states are merged through LDS; the result is either the
// final output (v_scale applied before the single rounding) or, when the
// request is split into several chunks, an fp32 partial (output, log-sum-exp)
// merged by merge_kernel.
#include "fi_device.hpp"

namespace fi {

// Page ids staged in LDS per window; a window spans kPidWindow pages.
constexpr int kPidWindow = 1024;

template <bool QBF16, int KVF, bool OBF16, int D>
struct DecodeCfg {
  static constexpr bool kFp8 = (KVF == FMT_E4M3 || KVF == FMT_E5M2);
  // MFMA operand type: bf16 whenever q or a 2-byte cache is bf16.  An fp16
  // operand meeting a bf16 one is split exactly into bf16 hi + lo.
  static constexpr bool MBF16 = QBF16 || KVF == FMT_BF16;
  static constexpr bool kSplitQ = !QBF16 && MBF16;            // fp16 q, bf16 cache
  static constexpr bool kSplitKV = (KVF == FMT_F16) && MBF16;  // fp16 cache, bf16 q
  static constexpr int KVB = kFp8 ? 1 : 2;  // bytes per stored element
  static constexpr int DL = D / 4;          // elements of a row per lane
  static constexpr int ROWB = DL * KVB;     // bytes of a row per lane
  static constexpr int U = ROWB / 16;       // 16-byte loads per row per lane
  static constexpr int NS = D / 32;         // MFMA k-steps for QK
  static constexpr int NDB = D / 16;        // 16-wide head_dim blocks for PV
  static constexpr int VROW = D * KVB + 16; // LDS row pitch of the V tile (bytes)
  static constexpr int VTILE = 32 * VROW;   // LDS bytes per wave
  static constexpr int MERGE = kDecodeWaves * kDecodeRows * (D + 3) * 4;
  static constexpr int PIDS = kDecodeWaves * VTILE;            // byte offset of the page-id window
  static constexpr int LOOP = PIDS + (kPidWindow + 2) * 4;      // LDS used by the main loop
  static constexpr int LDS = (LOOP > MERGE) ? LOOP : MERGE;
};

template <bool QBF16, int KVF, int D>
struct KvRegs {
  using Cfg = DecodeCfg<QBF16, KVF, false, D>;
  uint4 k[2][Cfg::U];
  uint4 v[2][Cfg::U];
};

// Issue the K and V loads of block `blk` for this lane's two tokens
// (16*h + c, h = 0, 1).  Page ids come from the LDS window `pids` whose first
// entry is page `pg_lo` of the request; past the chunk end the token index is
// clamped, and compute() zeroes those rows.
template <bool QBF16, int KVF, int D>
__device__ __forceinline__ void issue_kv(const DecodeParams& p, const uint8_t* kb, const uint8_t* vb, int t_begin,
                                         int t_end, int blk, int c, const int* pids, int pg_lo,
                                         KvRegs<QBF16, KVF, D>& r) {
  using Cfg = DecodeCfg<QBF16, KVF, false, D>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = min(t_begin + 32 * blk + 16 * h + c, t_end - 1);
    const int pid = pids[(t >> p.page_shift) - pg_lo];
    const int64_t off = (int64_t)pid * p.sp + (int64_t)(t & (p.page_size - 1)) * p.st;
    const uint4* kp = reinterpret_cast<const uint4*>(kb + off);
    const uint4* vp = reinterpret_cast<const uint4*>(vb + off);
#pragma unroll
    for (int u = 0; u < Cfg::U; ++u) r.k[h][u] = load16_stream(kp + u);
#pragma unroll
    for (int u = 0; u < Cfg::U; ++u) r.v[h][u] = load16_stream(vp + u);
  }
}

// K operand of k-step s for token half h (fp8 widened to the MFMA type; a
// 2-byte cache as stored).
template <bool QBF16, int KVF, int D>
__device__ __forceinline__ uint4 k_operand(const KvRegs<QBF16, KVF, D>& r, int h, int s) {
  using Cfg = DecodeCfg<QBF16, KVF, false, D>;
  if constexpr (Cfg::kFp8) {
    const uint4& x = r.k[h][s >> 1];
    return (s & 1) ? widen8<Cfg::MBF16, KVF>(x.z, x.w) : widen8<Cfg::MBF16, KVF>(x.x, x.y);
  } else {
    return r.k[h][s];
  }
}

// Workgroups per CU the register allocation is sized for (4 waves each).
#ifndef FI_DECODE_MIN_WG_PER_CU
#define FI_DECODE_MIN_WG_PER_CU 2
#endif
// Order of the 1-D grid: chunk index slowest (1) or fastest (0).
#ifndef FI_DECODE_CHUNK_SLOWEST
#define FI_DECODE_CHUNK_SLOWEST 0
#endif

template <bool QBF16, int KVF, bool OBF16, int D>
__global__ __launch_bounds__(256, FI_DECODE_MIN_WG_PER_CU) void decode_kernel(const DecodeParams p) {
  using Cfg = DecodeCfg<QBF16, KVF, OBF16, D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::LDS];

  // 1-D grid, chunk index slowest: consecutive workgroups (which the hardware
  // deals round-robin to the 8 XCDs) walk (kv head slice, request) first, so
  // the chunk-0 workgroups every request has are spread over all XCDs whatever
  // the number of chunks.
  const int units = p.num_kv_heads * p.nsub;
#if FI_DECODE_CHUNK_SLOWEST
  const int per_chunk = units * p.batch;
  const int chunk_id = blockIdx.x / per_chunk;
  const int rem = blockIdx.x - chunk_id * per_chunk;
  const int b = rem / units;
  const int gy = rem - b * units;
#else
  const int chunk_id = blockIdx.x % p.max_chunks;
  const int rem = blockIdx.x / p.max_chunks;
  const int gy = rem % units;
  const int b = rem / units;
#endif
  const int g = gy / p.nsub;
  const int sub = gy - g * p.nsub;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int qg = lane >> 4;

  int kv_len, pg_base;
  if (p.indptr) {
    const int a = p.indptr[b], e = p.indptr[b + 1];
    pg_base = a;
    kv_len = (e > a) ? (e - a - 1) * p.page_size + p.last_page_len[b] : 0;
  } else {
    pg_base = 0;
    kv_len = p.single_kv_len;
  }
  // the host plan sizes the grid from its copy of the page table; clamping keeps
  // a workgroup inside the partial buffers even if the two copies disagree
  const int nchunks = min(p.max_chunks, max(1, (kv_len + p.chunk - 1) / p.chunk));
  if (chunk_id >= nchunks) return;
  const int t_begin = chunk_id * p.chunk;
  const int t_end = min(kv_len, t_begin + p.chunk);
  const int nblk = (t_end > t_begin) ? (t_end - t_begin + 31) / 32 : 0;

  const int rig = sub * kDecodeRows + c;  // row within the GQA group
  const bool row_ok = rig < p.group;
  const int h = g * p.group + (row_ok ? rig : 0);

  // Q^T operand: lane (qg, c) holds q[row c][DL*qg + 8s + j], j = 0..7.
  uint4 qop[Cfg::NS];
  uint4 qlo[Cfg::kSplitQ ? Cfg::NS : 1];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.q) +
                                                     ((int64_t)b * p.num_qo_heads + h) * D + Cfg::DL * qg);
#pragma unroll
    for (int s = 0; s < Cfg::NS; ++s) {
      const uint4 raw = row_ok ? qp[s] : make_uint4(0, 0, 0, 0);
      if constexpr (Cfg::kSplitQ) {
        split_f16x8(raw, qop[s], qlo[s]);
      } else {
        qop[s] = raw;
      }
    }
  }

  const uint8_t* kb = p.k + (int64_t)g * p.sh + qg * Cfg::ROWB;
  const uint8_t* vb = p.v + (int64_t)g * p.sh + qg * Cfg::ROWB;
  uint8_t* vt = smem + w * Cfg::VTILE;
  // transposed-read addresses: fp8 tiles give 8 rows per read (lanes 2r, 2r+1
  // name row r), 2-byte tiles 4 rows per read (lanes 4r..4r+3 name row r)
  const uint8_t* v_tr;
  const uint8_t* v_tr2;
  if constexpr (Cfg::kFp8) {
    const int rr = c >> 1;
    const int tok = (rr < 4) ? 4 * qg + rr : 16 + 4 * qg + (rr - 4);
    v_tr = vt + tok * Cfg::VROW + 8 * (c & 1);
    v_tr2 = v_tr;
  } else {
    v_tr = vt + (4 * qg + (c >> 2)) * Cfg::VROW + 8 * (c & 3);
    v_tr2 = vt + (16 + 4 * qg + (c >> 2)) * Cfg::VROW + 8 * (c & 3);
  }

  float m_run = kNegInf;
  float l_run = 0.f;   // sum of fp32 probabilities (log-sum-exp)
  float lr_run = 0.f;  // sum of the rounded probabilities (output normalisation)
  f32x4_t acc[Cfg::NDB];
#pragma unroll
  for (int i = 0; i < Cfg::NDB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One 32-token block: QK on MFMA, online softmax, V through LDS, PV on MFMA.
  auto compute = [&](int blk, KvRegs<QBF16, KVF, D>& r) {
    const int tb = t_begin + 32 * blk;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bool ok = tb + 16 * hh + c < t_end;
#pragma unroll
      for (int u = 0; u < Cfg::U; ++u) {
        if (!ok) {
          r.k[hh][u] = make_uint4(0, 0, 0, 0);
          r.v[hh][u] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    // V rows -> LDS (row 16*hh + c, bytes [qg*ROWB, +ROWB)).
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint4* dst = reinterpret_cast<uint4*>(vt + (16 * hh + c) * Cfg::VROW + qg * Cfg::ROWB);
#pragma unroll
      for (int u = 0; u < Cfg::U; ++u) dst[u] = r.v[hh][u];
    }
    // S^T = K Q^T
    f32x4_t s[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      s[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < Cfg::NS; ++st) {
        if constexpr (Cfg::kSplitKV) {
          uint4 khi, klo;
          split_f16x8(r.k[hh][st], khi, klo);
          s[hh] = mfma16x16x32<true>(khi, qop[st], s[hh]);
          s[hh] = mfma16x16x32<true>(klo, qop[st], s[hh]);
        } else {
          const uint4 kop = k_operand(r, hh, st);
          s[hh] = mfma16x16x32<Cfg::MBF16>(kop, qop[st], s[hh]);
          if constexpr (Cfg::kSplitQ) s[hh] = mfma16x16x32<true>(kop, qlo[st], s[hh]);
        }
      }
    }
    // online softmax over the block's 32 tokens (row c; 8 values per lane)
    float x[2][4];
    float bm = kNegInf;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = tb + 16 * hh + 4 * qg + i < t_end;
        x[hh][i] = ok ? s[hh][i] * p.scale_log2 : kNegInf;
        bm = fmaxf(bm, x[hh][i]);
      }
    bm = xor_max(bm, 16);
    bm = xor_max(bm, 32);
    const float m_new = fmaxf(m_run, bm);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float pe[2][4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) pe[hh][i] = fast_exp2(x[hh][i] - m_use);
    uint4 pop;
    pop.x = pack2<Cfg::MBF16>(pe[0][0], pe[0][1]);
    pop.y = pack2<Cfg::MBF16>(pe[0][2], pe[0][3]);
    pop.z = pack2<Cfg::MBF16>(pe[1][0], pe[1][1]);
    pop.w = pack2<Cfg::MBF16>(pe[1][2], pe[1][3]);
    float2 f0 = unpack2<Cfg::MBF16>(pop.x), f1 = unpack2<Cfg::MBF16>(pop.y), f2 = unpack2<Cfg::MBF16>(pop.z),
           f3 = unpack2<Cfg::MBF16>(pop.w);
    lr_run = lr_run * alpha + ((f0.x + f0.y) + (f1.x + f1.y)) + ((f2.x + f2.y) + (f3.x + f3.y));
    l_run = l_run * alpha + ((pe[0][0] + pe[0][1]) + (pe[0][2] + pe[0][3])) +
            ((pe[1][0] + pe[1][1]) + (pe[1][2] + pe[1][3]));
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < Cfg::NDB; ++i) acc[i] *= alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P^T: lane (qg, c) needs column 16*db + c of the tile over
    // tokens 4qg..4qg+3 and 16+4qg..16+4qg+3 (the order its P^T slots hold).
    // One transposed LDS read per 16-column block gathers exactly that.
#pragma unroll
    for (int db = 0; db < Cfg::NDB; ++db) {
      if constexpr (Cfg::kFp8) {
        const uint2 x = lds_tr8(v_tr + 16 * db);
        acc[db] = mfma16x16x32<Cfg::MBF16>(widen8<Cfg::MBF16, KVF>(x.x, x.y), pop, acc[db]);
      } else {
        const uint2 x1 = lds_tr16(v_tr + 32 * db);
        const uint2 x2 = lds_tr16(v_tr2 + 32 * db);
        const uint4 vraw = make_uint4(x1.x, x1.y, x2.x, x2.y);
        if constexpr (Cfg::kSplitKV) {
          uint4 vhi, vlo;
          split_f16x8(vraw, vhi, vlo);
          acc[db] = mfma16x16x32<true>(vhi, pop, acc[db]);
          acc[db] = mfma16x16x32<true>(vlo, pop, acc[db]);
        } else {
          acc[db] = mfma16x16x32<Cfg::MBF16>(vraw, pop, acc[db]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // The chunk's page ids are staged in LDS, a window of kPidWindow pages at a
  // time, so that no K/V load waits on a page-id load.  Each wave then runs a
  // two-deep software pipeline over its blocks (w, w+4, ...): the loads of the
  // next block are in flight while a block is computed, and the wait before a
  // block covers only that block's loads.  Past the wave's last block the
  // index is clamped to it, so the extra loads re-read cached lines.
  int* pids_s = reinterpret_cast<int*>(smem + Cfg::PIDS);
  const int shift = p.page_shift;
  const int win_blocks =
      (int)min((int64_t)max(nblk, 1), max((int64_t)kDecodeWaves, ((int64_t)kPidWindow << shift) / 32));
  for (int wb0 = 0; wb0 < nblk; wb0 += win_blocks) {
    const int wb1 = min(nblk, wb0 + win_blocks);
    const int pg_lo = (t_begin + 32 * wb0) >> shift;
    const int pg_hi = ((min(t_begin + 32 * wb1, t_end) - 1) >> shift) + 1;
    const int cnt = min(pg_hi - pg_lo, kPidWindow + 2);
    __syncthreads();  // the previous window's page ids are no longer read
    for (int i = threadIdx.x; i < cnt; i += 256) pids_s[i] = p.indices ? p.indices[pg_base + pg_lo + i] : 0;
    __syncthreads();
    const int my_n = (wb1 - wb0 > w) ? (wb1 - wb0 - w + kDecodeWaves - 1) / kDecodeWaves : 0;
    if (my_n > 0) {
      auto blk_of = [&](int k) { return wb0 + w + kDecodeWaves * min(k, my_n - 1); };
      KvRegs<QBF16, KVF, D> ra, rb;
      issue_kv(p, kb, vb, t_begin, t_end, blk_of(0), c, pids_s, pg_lo, ra);
      for (int k = 0; k < my_n; k += 2) {
        issue_kv(p, kb, vb, t_begin, t_end, blk_of(k + 1), c, pids_s, pg_lo, rb);
        compute(blk_of(k), ra);
        if (k + 1 >= my_n) break;
        issue_kv(p, kb, vb, t_begin, t_end, blk_of(k + 2), c, pids_s, pg_lo, ra);
        compute(blk_of(k + 1), rb);
      }
    }
  }

  // Per-wave state -> LDS, then merge the four waves.
  l_run = xor_sum(l_run, 16);
  l_run = xor_sum(l_run, 32);
  lr_run = xor_sum(lr_run, 16);
  lr_run = xor_sum(lr_run, 32);
  __syncthreads();
  float* ms = reinterpret_cast<float*>(smem);                 // [4][16]
  float* ls = ms + kDecodeWaves * kDecodeRows;                 // [4][16]
  float* lrs = ls + kDecodeWaves * kDecodeRows;                // [4][16]
  float* accs = lrs + kDecodeWaves * kDecodeRows;              // [4][16][D]
  if (qg == 0) {
    ms[w * kDecodeRows + c] = m_run;
    ls[w * kDecodeRows + c] = l_run;
    lrs[w * kDecodeRows + c] = lr_run;
  }
#pragma unroll
  for (int db = 0; db < Cfg::NDB; ++db) {
    *reinterpret_cast<f32x4_t*>(accs + (w * kDecodeRows + c) * D + 16 * db + 4 * qg) = acc[db];
  }
  __syncthreads();

  constexpr int EPT = D * kDecodeRows / 256;  // outputs per thread (8 or 4)
  const int row = threadIdx.x / 16;
  const int d0 = (threadIdx.x % 16) * EPT;
  const int rrow = sub * kDecodeRows + row;
  if (rrow >= p.group) return;
  const int hq = g * p.group + rrow;
  float M = kNegInf;
#pragma unroll
  for (int ww = 0; ww < kDecodeWaves; ++ww) M = fmaxf(M, ms[ww * kDecodeRows + row]);
  float wt[kDecodeWaves];
  float L = 0.f, Lr = 0.f;
#pragma unroll
  for (int ww = 0; ww < kDecodeWaves; ++ww) {
    const float mw = ms[ww * kDecodeRows + row];
    wt[ww] = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
    L += wt[ww] * ls[ww * kDecodeRows + row];
    Lr += wt[ww] * lrs[ww * kDecodeRows + row];
  }
  float out[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    float a = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecodeWaves; ++ww) a += wt[ww] * accs[(ww * kDecodeRows + row) * D + d0 + e];
    out[e] = a;
  }
  const float inv = (Lr > 0.f) ? 1.f / Lr : 0.f;
  const float lse2 = (L > 0.f) ? M + fast_log2(L) : kNegInf;
  if (nchunks == 1) {
    const float f = inv * p.v_scale;
    uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)b * p.num_qo_heads + hq) * D + d0;
    uint32_t packed[EPT / 2];
#pragma unroll
    for (int e = 0; e < EPT / 2; ++e) packed[e] = pack2<OBF16>(out[2 * e] * f, out[2 * e + 1] * f);
    if constexpr (EPT == 8) {
      *reinterpret_cast<uint4*>(op) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    } else {
      *reinterpret_cast<uint2*>(op) = make_uint2(packed[0], packed[1]);
    }
    if (p.lse && (threadIdx.x % 16) == 0) p.lse[(int64_t)b * p.num_qo_heads + hq] = lse2 * kLn2;
  } else {
    const int64_t pidx = ((int64_t)b * p.max_chunks + chunk_id) * p.num_qo_heads + hq;
    float* po = p.part_o + pidx * D + d0;
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
      *reinterpret_cast<f32x4_t*>(po + e) = f32x4_t{out[e] * inv, out[e + 1] * inv, out[e + 2] * inv, out[e + 3] * inv};
    if ((threadIdx.x % 16) == 0) p.part_lse[pidx] = lse2;
  }
}

// ---------------------------------------------------------------------------
// Split-KV merge: L = log2 sum_c 2^lse_c, o = v_scale * sum_c 2^(lse_c - L) o_c
// (the natural-log form of the same identity is the oracle's merge_states).
// One wave per (request, q head); lanes cover head_dim.
// ---------------------------------------------------------------------------
template <bool OBF16, int D>
__global__ __launch_bounds__(64) void merge_kernel(const MergeParams p) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  int kv_len;
  if (p.indptr) {
    const int a = p.indptr[b], e = p.indptr[b + 1];
    kv_len = (e > a) ? (e - a - 1) * p.page_size + p.last_page_len[b] : 0;
  } else {
    kv_len = p.single_kv_len;
  }
  const int nchunks = min(p.max_chunks, max(1, (kv_len + p.chunk - 1) / p.chunk));
  if (nchunks <= 1) return;
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x;
  const int64_t base = (int64_t)b * p.max_chunks * p.num_qo_heads + hq;
  float M = kNegInf;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, p.part_lse[base + (int64_t)c * p.num_qo_heads]);
  float L = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int c = 0; c < nchunks; ++c) {
    const int64_t idx = base + (int64_t)c * p.num_qo_heads;
    const float lc = p.part_lse[idx];
    const float wgt = (lc == kNegInf) ? 0.f : fast_exp2(lc - M);
    L += wgt;
    const float* po = p.part_o + idx * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += wgt * po[e];
  }
  const float f = (L > 0.f) ? p.v_scale / L : 0.f;
  uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)b * p.num_qo_heads + hq) * D + lane * EPL;
  if constexpr (EPL == 2) {
    *reinterpret_cast<uint32_t*>(op) = pack2<OBF16>(acc[0] * f, acc[1] * f);
  } else {
    op[0] = to_bits<OBF16>(acc[0] * f);
  }
  if (p.lse && lane == 0) p.lse[(int64_t)b * p.num_qo_heads + hq] = (L > 0.f) ? (M + fast_log2(L)) * kLn2 : kNegInf;
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
  const uint16_t v[4] = {(uint16_t)(r.x & 0xffff), (uint16_t)(r.x >> 16), (uint16_t)(r.y & 0xffff),
                         (uint16_t)(r.y >> 16)};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (i + j < n) out[i + j] = v[j];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <bool QBF16, int KVF, bool OBF16, int D>
static hipError_t launch_decode_t(const DecodeParams& p, int batch, hipStream_t s) {
  dim3 grid((unsigned)p.max_chunks * p.num_kv_heads * p.nsub * batch);
  hipLaunchKernelGGL((decode_kernel<QBF16, KVF, OBF16, D>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool QBF16, int KVF, bool OBF16>
static hipError_t launch_decode_d(const DecodeParams& p, int head_dim, int batch, hipStream_t s) {
  if (head_dim == 128) return launch_decode_t<QBF16, KVF, OBF16, 128>(p, batch, s);
  return launch_decode_t<QBF16, KVF, OBF16, 64>(p, batch, s);
}

template <bool QBF16, int KVF>
static hipError_t launch_decode_o(const DecodeParams& p, int o_fmt, int head_dim, int batch, hipStream_t s) {
  if (o_fmt == FMT_BF16) return launch_decode_d<QBF16, KVF, true>(p, head_dim, batch, s);
  return launch_decode_d<QBF16, KVF, false>(p, head_dim, batch, s);
}

template <bool QBF16>
static hipError_t launch_decode_kv(const DecodeParams& p, int kv_fmt, int o_fmt, int head_dim, int batch,
                                   hipStream_t s) {
  switch (kv_fmt) {
    case FMT_F16: return launch_decode_o<QBF16, FMT_F16>(p, o_fmt, head_dim, batch, s);
    case FMT_BF16: return launch_decode_o<QBF16, FMT_BF16>(p, o_fmt, head_dim, batch, s);
    case FMT_E4M3: return launch_decode_o<QBF16, FMT_E4M3>(p, o_fmt, head_dim, batch, s);
    default: return launch_decode_o<QBF16, FMT_E5M2>(p, o_fmt, head_dim, batch, s);
  }
}

hipError_t launch_decode(const DecodeParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, int batch,
                         hipStream_t s) {
  if (q_fmt == FMT_BF16) return launch_decode_kv<true>(p, kv_fmt, o_fmt, head_dim, batch, s);
  return launch_decode_kv<false>(p, kv_fmt, o_fmt, head_dim, batch, s);
}

hipError_t launch_merge(const MergeParams& p, int o_fmt, int head_dim, int batch, hipStream_t s) {
  dim3 grid(p.num_qo_heads, batch);
  if (o_fmt == FMT_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((merge_kernel<true, 128>), grid, dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL((merge_kernel<true, 64>), grid, dim3(64), 0, s, p);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((merge_kernel<false, 128>), grid, dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL((merge_kernel<false, 64>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_widen(const uint8_t* codes, int64_t n, int src_fmt, int dst_fmt, void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  dim3 grid((unsigned)((threads + 255) / 256));
  uint16_t* o = reinterpret_cast<uint16_t*>(out);
  if (dst_fmt == FMT_BF16) {
    if (src_fmt == FMT_E4M3)
      hipLaunchKernelGGL((widen_kernel<true, FMT_E4M3>), grid, dim3(256), 0, s, codes, n, o);
    else
      hipLaunchKernelGGL((widen_kernel<true, FMT_E5M2>), grid, dim3(256), 0, s, codes, n, o);
  } else {
    if (src_fmt == FMT_E4M3)
      hipLaunchKernelGGL((widen_kernel<false, FMT_E4M3>), grid, dim3(256), 0, s, codes, n, o);
    else
      hipLaunchKernelGGL((widen_kernel<false, FMT_E5M2>), grid, dim3(256), 0, s, codes, n, o);
  }
  return hipGetLastError();
}

}  // namespace fi
