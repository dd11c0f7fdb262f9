// Batched (causal) prefill over a paged KV cache for gfx950.
//
// What is computed: for every query token of every request and every q head,
// softmax(q K^T * sm_scale) V over the keys the (optional) causal mask leaves
// visible, with K and V stored as OCP fp8 or as q's 2-byte type
// ("fp8 KV cache in the in-tree prefill kernel", AMD-Ecosystem/flashinfer
// PR #368: Summary, Kernel, Benchmark results).  The causal mask is aligned to
// the end of the KV sequence: row r sees key t iff t <= r + kv_len - qo_len.
//
// Mapping.  A workgroup of 4 waves owns one (request, kv head, group of heads,
// block of query tokens); every wave holds 32 query rows of one q head, so the
// 4 waves share each K/V tile (GQA packing: one tile serves up to 4 q heads).
// Per 64-token K/V tile:
//   * the workgroup gathers the tile's rows from their pages, widens fp8 to
//     q's type in registers and stores a 2-byte tile in LDS -- the
//     dequantize-on-load design the PR describes (Kernel; Architecture /
//     design notes), here with 16-byte loads per lane, which the PR's Known
//     limitations name as what its 4-byte loads lacked;
//   * each wave computes S^T = K Q^T on MFMA 32x32x16 (tokens x rows), masks,
//     runs the online softmax in base 2 and accumulates O^T += V^T P^T, the
//     probabilities feeding the MFMA straight from the S^T registers; the
//     log-sum-exp comes from the sum of the fp32 probabilities, the output is
//     normalised by the sum of the rounded ones the MFMA applied.
#include "fi_device.hpp"

namespace fi {

template <bool QBF16, int KVF, bool OBF16, int D>
struct PrefillCfg {
  static constexpr bool kFp8 = (KVF == FMT_E4M3 || KVF == FMT_E5M2);
  static constexpr int KVB = kFp8 ? 1 : 2;
  static constexpr int TK = 64;              // keys per tile
  static constexpr int KP = D * 2 + 16;      // LDS row pitch (bytes) of the 2-byte tiles
  static constexpr int FILL_E = D / 4;       // elements each thread moves per tile row
  static constexpr int FILL_U = FILL_E * KVB / 16;  // 16-byte loads per thread per tensor
  static constexpr int NS = D / 16;          // QK k-steps (MFMA k = 16)
  static constexpr int NDB = D / 32;         // PV head_dim blocks of 32
  static constexpr int LDS = 2 * TK * KP;
};

template <bool QBF16, int KVF, int D>
struct TileRegs {
  using Cfg = PrefillCfg<QBF16, KVF, false, D>;
  uint4 k[Cfg::FILL_U];
  uint4 v[Cfg::FILL_U];
};

template <bool QBF16, int KVF, bool OBF16, int D>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillParams p) {
  using Cfg = PrefillCfg<QBF16, KVF, OBF16, D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::LDS];
  uint8_t* ks = smem;
  uint8_t* vs = smem + Cfg::TK * Cfg::KP;

  const int nsg = p.group / p.heads_per_wg;
  const int x = blockIdx.x;
  const int sg = x % nsg;
  const int g = (x / nsg) % p.num_kv_heads;
  const int b = x / (nsg * p.num_kv_heads);
  const int qb = p.n_qblocks - 1 - blockIdx.y;  // heaviest (latest) query blocks first

  const int q_begin = p.qo_indptr[b];
  const int qo_len = p.qo_indptr[b + 1] - q_begin;
  const int q0 = qb * p.q_per_wg;
  if (q0 >= qo_len) return;
  const int a = p.indptr[b], e = p.indptr[b + 1];
  const int kv_len = (e > a) ? (e - a - 1) * p.page_size + p.last_page_len[b] : 0;
  const int prefix = kv_len - qo_len;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int rho = lane & 31;
  const int hh = lane >> 5;
  const int head_local = w % p.heads_per_wg;
  const int tsub = w / p.heads_per_wg;
  const int hq = g * p.group + sg * p.heads_per_wg + head_local;
  const int qpos = q0 + 32 * tsub + rho;  // this lane's query row
  const bool row_ok = qpos < qo_len;

  // last key any row of the workgroup can see
  const int q_last = min(q0 + p.q_per_wg, qo_len) - 1;
  const int key_end = p.causal ? min(kv_len, q_last + prefix + 1) : kv_len;
  const int ntiles = (key_end > 0) ? (key_end + Cfg::TK - 1) / Cfg::TK : 0;
  // last key this lane's row can see (exclusive bound)
  const int row_key_end = p.causal ? min(kv_len, qpos + prefix + 1) : kv_len;

  // Q^T operand: lane (hh, rho) holds q[row rho][(D/2)*hh + 8s + j].
  uint4 qop[Cfg::NS];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.q) +
                                                     ((int64_t)(q_begin + (row_ok ? qpos : 0)) * p.num_qo_heads + hq) * D +
                                                     (D / 2) * hh);
#pragma unroll
    for (int s = 0; s < Cfg::NS; ++s) qop[s] = row_ok ? qp[s] : make_uint4(0, 0, 0, 0);
  }

  // transposed-read address of this lane for the V^T operand: within each
  // 16-lane group, lanes 4r..4r+3 name the four 8-byte pieces of row r
  const uint8_t* v_tr = vs + (4 * hh + ((rho & 15) >> 2)) * Cfg::KP + (16 * (rho >> 4) + 4 * (rho & 3)) * 2;

  // tile fill: thread -> (token row = tid / 4, element range part * D/4)
  const int f_tok = tid >> 2;
  const int f_part = tid & 3;
  const uint8_t* kb = p.k + (int64_t)g * p.sh + f_part * Cfg::FILL_E * Cfg::KVB;
  const uint8_t* vb = p.v + (int64_t)g * p.sh + f_part * Cfg::FILL_E * Cfg::KVB;

  auto load_pid = [&](int tile) -> int {
    const int t = min(tile * Cfg::TK + f_tok, max(kv_len - 1, 0));
    return p.indices[a + (t >> p.page_shift)];
  };
  auto issue = [&](int tile, int pid, TileRegs<QBF16, KVF, D>& r) {
    const int t = min(tile * Cfg::TK + f_tok, max(kv_len - 1, 0));
    const int64_t off = (int64_t)pid * p.sp + (int64_t)(t & (p.page_size - 1)) * p.st;
    const uint4* kp = reinterpret_cast<const uint4*>(kb + off);
    const uint4* vp = reinterpret_cast<const uint4*>(vb + off);
#pragma unroll
    for (int u = 0; u < Cfg::FILL_U; ++u) r.k[u] = kp[u];
#pragma unroll
    for (int u = 0; u < Cfg::FILL_U; ++u) r.v[u] = vp[u];
  };
  // widen into q's type and store the row slice into the LDS tiles
  auto store = [&](int tile, TileRegs<QBF16, KVF, D>& r) {
    const bool ok = tile * Cfg::TK + f_tok < kv_len;
    uint4* kd = reinterpret_cast<uint4*>(ks + f_tok * Cfg::KP + f_part * Cfg::FILL_E * 2);
    uint4* vd = reinterpret_cast<uint4*>(vs + f_tok * Cfg::KP + f_part * Cfg::FILL_E * 2);
    const uint4 z = make_uint4(0, 0, 0, 0);
    if constexpr (Cfg::kFp8) {
#pragma unroll
      for (int u = 0; u < Cfg::FILL_U; ++u) {
        kd[2 * u] = ok ? widen8<QBF16, KVF>(r.k[u].x, r.k[u].y) : z;
        kd[2 * u + 1] = ok ? widen8<QBF16, KVF>(r.k[u].z, r.k[u].w) : z;
        vd[2 * u] = ok ? widen8<QBF16, KVF>(r.v[u].x, r.v[u].y) : z;
        vd[2 * u + 1] = ok ? widen8<QBF16, KVF>(r.v[u].z, r.v[u].w) : z;
      }
    } else {
#pragma unroll
      for (int u = 0; u < Cfg::FILL_U; ++u) {
        kd[u] = ok ? r.k[u] : z;
        vd[u] = ok ? r.v[u] : z;
      }
    }
  };

  float m_run = kNegInf;
  float l_run = 0.f;   // sum of fp32 probabilities (log-sum-exp)
  float lr_run = 0.f;  // sum of the probabilities rounded to q's type (output normalisation)
  f32x16_t acc[Cfg::NDB];
#pragma unroll
  for (int i = 0; i < Cfg::NDB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;

  auto compute = [&](int tile) {
    const int kbase = tile * Cfg::TK;
    // S^T = K Q^T, two 32-token halves
    f32x16_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[sub][j] = 0.f;
      const uint8_t* krow = ks + (32 * sub + rho) * Cfg::KP + D * hh;
#pragma unroll
      for (int st = 0; st < Cfg::NS; ++st) {
        const uint4 kop = *reinterpret_cast<const uint4*>(krow + 16 * st);
        s[sub] = mfma32x32x16<QBF16>(kop, qop[st], s[sub]);
      }
    }
    // mask + online softmax; lane holds keys 32*sub + 8*(i/4) + 4*hh + i%4
    float bm = kNegInf;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = kbase + 32 * sub + 8 * (i >> 2) + 4 * hh + (i & 3);
        const float v = (t < row_key_end) ? s[sub][i] * p.scale_log2 : kNegInf;
        s[sub][i] = v;
        bm = fmaxf(bm, v);
      }
    bm = xor_max(bm, 32);
    const float m_new = fmaxf(m_run, bm);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    uint4 pop[4];
    float psum = 0.f, prsum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t wds[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i0 = 8 * (u & 1) + 2 * jj;
        const float e0 = fast_exp2(s[u >> 1][i0] - m_use), e1 = fast_exp2(s[u >> 1][i0 + 1] - m_use);
        wds[jj] = pack2<QBF16>(e0, e1);
        const float2 f = unpack2<QBF16>(wds[jj]);
        prsum += f.x + f.y;
        psum += e0 + e1;
      }
      pop[u] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    }
    l_run = l_run * alpha + psum;
    lr_run = lr_run * alpha + prsum;
#pragma unroll
    for (int i = 0; i < Cfg::NDB; ++i) acc[i] *= alpha;
    // O^T += V^T P^T.  Lane (hh, rho) needs column 32*db + rho of the V tile
    // over tokens r0..r0+3 and r0+8..r0+11 (r0 = 32*(u/2) + 16*(u%2) + 4*hh),
    // the order its P^T slots hold: two transposed LDS reads of 4 rows each.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r0 = 32 * (u >> 1) + 16 * (u & 1);
      const uint8_t* a1 = v_tr + r0 * Cfg::KP;
      const uint8_t* a2 = a1 + 8 * Cfg::KP;
#pragma unroll
      for (int db = 0; db < Cfg::NDB; ++db) {
        const uint2 x1 = lds_tr16(a1 + 64 * db);
        const uint2 x2 = lds_tr16(a2 + 64 * db);
        acc[db] = mfma32x32x16<QBF16>(make_uint4(x1.x, x1.y, x2.x, x2.y), pop[u], acc[db]);
      }
    }
  };

  if (ntiles > 0) {
    TileRegs<QBF16, KVF, D> ra;
    int pid = load_pid(0);
    issue(0, pid, ra);
    int pid_next = load_pid(min(1, ntiles - 1));
    for (int tile = 0; tile < ntiles; ++tile) {
      store(tile, ra);
      __syncthreads();
      if (tile + 1 < ntiles) {
        issue(tile + 1, pid_next, ra);
        pid_next = load_pid(min(tile + 2, ntiles - 1));
      }
      compute(tile);
      __syncthreads();
    }
  }

  // epilogue
  l_run = xor_sum(l_run, 32);
  lr_run = xor_sum(lr_run, 32);
  if (!row_ok) return;
  const float inv = (lr_run > 0.f) ? p.v_scale / lr_run : 0.f;
  uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)(q_begin + qpos) * p.num_qo_heads + hq) * D;
#pragma unroll
  for (int db = 0; db < Cfg::NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * db + 8 * i4 + 4 * hh;
      *reinterpret_cast<uint2*>(op + d) = make_uint2(pack2<OBF16>(acc[db][4 * i4] * inv, acc[db][4 * i4 + 1] * inv),
                                                     pack2<OBF16>(acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv));
    }
  if (p.lse && hh == 0)
    p.lse[(int64_t)(q_begin + qpos) * p.num_qo_heads + hq] =
        (l_run > 0.f) ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
}

template <bool QBF16, int KVF, bool OBF16, int D>
static hipError_t launch_prefill_t(const PrefillParams& p, int batch, hipStream_t s) {
  const int nsg = p.group / p.heads_per_wg;
  dim3 grid(batch * p.num_kv_heads * nsg, p.n_qblocks);
  hipLaunchKernelGGL((prefill_kernel<QBF16, KVF, OBF16, D>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool QBF16, int KVF, bool OBF16>
static hipError_t launch_prefill_d(const PrefillParams& p, int head_dim, int batch, hipStream_t s) {
  if (head_dim == 128) return launch_prefill_t<QBF16, KVF, OBF16, 128>(p, batch, s);
  return launch_prefill_t<QBF16, KVF, OBF16, 64>(p, batch, s);
}

template <bool QBF16, int KVF>
static hipError_t launch_prefill_o(const PrefillParams& p, int o_fmt, int head_dim, int batch, hipStream_t s) {
  if (o_fmt == FMT_BF16) return launch_prefill_d<QBF16, KVF, true>(p, head_dim, batch, s);
  return launch_prefill_d<QBF16, KVF, false>(p, head_dim, batch, s);
}

hipError_t launch_prefill(const PrefillParams& p, int q_fmt, int kv_fmt, int o_fmt, int head_dim, int batch,
                          hipStream_t s) {
  // Prefill admits a 2-byte KV only when it equals q's type.
  if (q_fmt == FMT_BF16) {
    switch (kv_fmt) {
      case FMT_BF16: return launch_prefill_o<true, FMT_BF16>(p, o_fmt, head_dim, batch, s);
      case FMT_E4M3: return launch_prefill_o<true, FMT_E4M3>(p, o_fmt, head_dim, batch, s);
      default: return launch_prefill_o<true, FMT_E5M2>(p, o_fmt, head_dim, batch, s);
    }
  }
  switch (kv_fmt) {
    case FMT_F16: return launch_prefill_o<false, FMT_F16>(p, o_fmt, head_dim, batch, s);
    case FMT_E4M3: return launch_prefill_o<false, FMT_E4M3>(p, o_fmt, head_dim, batch, s);
    default: return launch_prefill_o<false, FMT_E5M2>(p, o_fmt, head_dim, batch, s);
  }
}

}  // namespace fi
