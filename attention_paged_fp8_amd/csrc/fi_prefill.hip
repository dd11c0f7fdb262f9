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
//   * the workgroup gathers the tile's rows from their pages with coalesced
//     16-byte loads (8 lanes per 128-byte fp8 row), two tiles ahead, widens
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
// The row sums of the probabilities as rounded for the PV MFMA come from the
// MFMA itself (an all-ones operand against P^T), exact in fp32; they normalise
// the output and, for fp16 (rounding 2^-11), give the log-sum-exp.  With a
// bf16 query (rounding 2^-9) the log-sum-exp uses a separate fp32 sum.
#include "fi_device.hpp"

namespace fi {

template <bool QBF16, int KVF, bool OBF16, int D>
struct PrefillCfg {
  static constexpr bool kFp8 = (KVF == FMT_E4M3 || KVF == FMT_E5M2);
  static constexpr bool kF32Sum = QBF16;        // bf16 probabilities round at 2^-9: LSE from an fp32 sum
  static constexpr int KVB = kFp8 ? 1 : 2;
  static constexpr int TK = 64;                 // keys per tile
  static constexpr int DB = D * KVB;            // stored bytes of a row
  static constexpr int ROW = D * 2;             // bytes of a 2-byte row
  static constexpr int KP = ROW + 16;           // K tile pitch, 16 mod 256 bytes
  static constexpr int VP = (ROW + 191) / 256 * 256 + 64;  // V tile pitch, 64 mod 256 bytes
  static constexpr int KTILE = TK * KP;
  static constexpr int STAGE = KTILE + TK * VP; // K then V
  static constexpr int PER = TK * DB / (16 * 256);  // 16-byte global loads per thread per tensor
  static constexpr int NS = D / 16;             // QK k-steps (MFMA k = 16)
  static constexpr int NDB = D / 32;            // PV head_dim blocks of 32
  static constexpr int LDS = 2 * STAGE;
  // Head-dimension order of the LDS tiles.  An fp8 lane holds 16 consecutive
  // dimensions (16c .. 16c+15) and stores their widened halves 128 bytes
  // apart, so the 8 lanes of a row write two contiguous 128-byte runs: tile
  // position p holds dimension dim_of(p).  2-byte tiles keep the natural order.
  __host__ __device__ static constexpr int dim_of(int p) {
    if (!kFp8) return p;
    return p < D / 2 ? 16 * (p / 8) + p % 8 : 16 * ((p - D / 2) / 8) + 8 + (p - D / 2) % 8;
  }
};

template <bool QBF16, int KVF, bool OBF16, int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillParams p) {
  using Cfg = PrefillCfg<QBF16, KVF, OBF16, D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::LDS];

  const int nsg = p.group / p.heads_per_wg;
  const int x = blockIdx.x;
  const int sg = x % nsg;
  const int g = (x / nsg) % p.num_kv_heads;
  const int b = x / (nsg * p.num_kv_heads);
  const int qb = p.n_qblocks - 1 - blockIdx.y;  // heaviest (latest) query blocks first

  // request geometry: uniform over the workgroup, kept in scalar registers so
  // that the tile loop and its branches stay scalar
  const int q_begin = uniform(p.qo_indptr[b]);
  const int qo_len = uniform(p.qo_indptr[b + 1]) - q_begin;
  const int q0 = qb * p.q_per_wg;
  if (q0 >= qo_len) return;
  const int a = uniform(p.indptr[b]), e = uniform(p.indptr[b + 1]);
  const int kv_len = (e > a) ? (e - a - 1) * p.page_size + uniform(p.last_page_len[b]) : 0;
  const int prefix = kv_len - qo_len;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int lane = tid & 63;
  const int rho = lane & 31;
  const int hh = lane >> 5;
  const int head_local = w % p.heads_per_wg;
  const int tsub = w / p.heads_per_wg;
  const int hq = g * p.group + sg * p.heads_per_wg + head_local;
  const int qw0 = q0 + 32 * tsub;         // this wave's first query row
  const int qpos = qw0 + rho;             // this lane's query row
  const bool row_ok = qpos < qo_len;

  // keys the workgroup needs, and the keys every / some row of this wave sees
  const int q_last = min(q0 + p.q_per_wg, qo_len) - 1;
  const int key_end = p.causal ? min(kv_len, q_last + prefix + 1) : kv_len;
  const int ntiles = uniform((key_end > 0) ? (key_end + Cfg::TK - 1) / Cfg::TK : 0);
  const int row_key_end = p.causal ? min(kv_len, qpos + prefix + 1) : kv_len;
  const int wave_full_end = uniform(p.causal ? min(kv_len, qw0 + prefix + 1) : kv_len);  // all rows see keys below
  const int wave_any_end =
      uniform(p.causal ? min(kv_len, min(qw0 + 31, qo_len - 1) + prefix + 1) : kv_len);  // no row sees keys at or above
  const bool wave_ok = qw0 < qo_len;

  // Q^T operand: lane (hh, rho) holds q[row rho] at the dimensions of K tile
  // positions (D/2)*hh + 8s + j, j = 0..7 (8 consecutive dimensions).
  uint4 qop[Cfg::NS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) +
                         ((int64_t)(q_begin + (row_ok ? qpos : 0)) * p.num_qo_heads + hq) * D;
#pragma unroll
    for (int s = 0; s < Cfg::NS; ++s)
      qop[s] = row_ok ? *reinterpret_cast<const uint4*>(qp + Cfg::dim_of((D / 2) * hh + 8 * s)) : make_uint4(0, 0, 0, 0);
  }

  // tile loads: chunk ci = j*256 + tid of a tensor's tile is row ci / (DB/16),
  // 16-byte column ci % (DB/16); 8 lanes read one 128-byte fp8 row
  constexpr int SC = Cfg::DB / 16;  // stored 16-byte chunks per row
  int ld_row[Cfg::PER], ld_col[Cfg::PER];
#pragma unroll
  for (int j = 0; j < Cfg::PER; ++j) {
    const int ci = j * 256 + tid;
    ld_row[j] = ci / SC;
    ld_col[j] = ci % SC;
  }
  const uint8_t* kb = p.k + (int64_t)g * p.sh;
  const uint8_t* vb = p.v + (int64_t)g * p.sh;
  // One register set per LDS stage: the tile's data and the page ids of the
  // tile two loads later.  Page ids are fetched a whole tile ahead of the data
  // they address, so waiting for them never waits for the data loads issued
  // after them (vector memory counters retire in order).
  struct Regs {
    uint4 k[Cfg::PER];
    uint4 v[Cfg::PER];
    uint32_t pid[Cfg::PER];
  };
  auto row_token = [&](int tile, int j) { return min(tile * Cfg::TK + ld_row[j], max(kv_len - 1, 0)); };
  auto load_pids = [&](int tile, Regs& r) {
#pragma unroll
    for (int j = 0; j < Cfg::PER; ++j) r.pid[j] = (uint32_t)p.indices[a + (row_token(tile, j) >> p.page_shift)];
  };
  auto load_tile = [&](int tile, Regs& r) {
#pragma unroll
    for (int j = 0; j < Cfg::PER; ++j) {
      const int t = row_token(tile, j);
      const uint64_t off = (uint64_t)r.pid[j] * (uint32_t)p.sp +
                           (uint32_t)((t & (p.page_size - 1)) * (uint32_t)p.st) + (uint32_t)(ld_col[j] * 16);
      r.k[j] = load16(kb + off);
      r.v[j] = load16(vb + off);
    }
  };
  // widen into q's type and store into an LDS stage.  Rows past kv_len hold
  // the last valid token again (row_token clamps): finite values whose keys
  // the mask sets to -inf, so their probabilities are exactly 0.
  auto store_tile = [&](Regs& r, uint8_t* stage) {
#pragma unroll
    for (int j = 0; j < Cfg::PER; ++j) {
      const int row = ld_row[j];
      const uint4 kx = r.k[j], vx = r.v[j];
      uint8_t* kd = stage + row * Cfg::KP;
      uint8_t* vd = stage + Cfg::KTILE + row * Cfg::VP;
      if constexpr (Cfg::kFp8) {  // dimensions 16c..16c+7 to position 8c, 16c+8.. to D/2 + 8c
        const int c0 = 16 * ld_col[j];
        *reinterpret_cast<uint4*>(kd + c0) = widen8<QBF16, KVF>(kx.x, kx.y);
        *reinterpret_cast<uint4*>(kd + D + c0) = widen8<QBF16, KVF>(kx.z, kx.w);
        *reinterpret_cast<uint4*>(vd + c0) = widen8<QBF16, KVF>(vx.x, vx.y);
        *reinterpret_cast<uint4*>(vd + D + c0) = widen8<QBF16, KVF>(vx.z, vx.w);
      } else {
        *reinterpret_cast<uint4*>(kd + 16 * ld_col[j]) = kx;
        *reinterpret_cast<uint4*>(vd + 16 * ld_col[j]) = vx;
      }
    }
  };

  float m_run = kNegInf;  // running max (base-2 scaled logits), updated lazily
  float l_run = 0.f;      // sum of fp32 probabilities (bf16 only)
  f32x16_t acc[Cfg::NDB];
  f32x16_t accs;          // row sums of the rounded probabilities (every element of a lane alike)
#pragma unroll
  for (int i = 0; i < Cfg::NDB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) accs[j] = 0.f;
  const uint32_t one2 = QBF16 ? 0x3f803f80u : 0x3c003c00u;  // two 1.0 in the MFMA type
  const uint4 ones = make_uint4(one2, one2, one2, one2);

  // per-lane LDS read bases (stage 0); everything else is a constant offset.
  // K: lane (hh, rho) reads row 32*sub + rho, bytes [D*hh + 16*st, +16).
  // V^T transposed reads: within each 16-lane group (same hh, same rho / 16),
  // lanes 4r..4r+3 name the four 8-byte pieces of row r of a 16-column block.
  const int k_base = rho * Cfg::KP + D * hh;
  const int v_base = Cfg::KTILE + (4 * hh + ((rho & 15) >> 2)) * Cfg::VP + 32 * (rho >> 4) + 8 * (rho & 3);

  auto compute = [&](int tile, const uint8_t* stage) {
    const int kbase = tile * Cfg::TK;
    if (kbase >= wave_any_end) return;  // no row of this wave sees this tile
    const uint8_t* kl = stage + k_base;
    const uint8_t* vl = stage + v_base;
    // S^T = K Q^T, two 32-token halves
    f32x16_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[sub][j] = 0.f;
#pragma unroll
      for (int st = 0; st < Cfg::NS; ++st) {
        const uint4 kop = *reinterpret_cast<const uint4*>(kl + 32 * sub * Cfg::KP + 16 * st);
        s[sub] = mfma32x32x16<QBF16>(kop, qop[st], s[sub]);
      }
    }
    // lane (hh, rho) holds keys kbase + 32*sub + 8*(i/4) + 4*hh + i%4 of row rho
    if (kbase + Cfg::TK > wave_full_end) {  // the tile crosses the diagonal or the end
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = kbase + 32 * sub + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (t >= row_key_end) s[sub][i] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[sub][i], s[sub][i + 1]));
    mx = xor_max(mx, 32) * p.scale_log2;  // base-2 logits (scale > 0 keeps the order)
    // lazy rescale: move the reference max only when some row's max grows by
    // more than 8 (log2) -- then exp2 stays below 2^8
    const bool grow = mx > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      if constexpr (Cfg::kF32Sum) l_run *= alpha;
      accs *= alpha;
#pragma unroll
      for (int i = 0; i < Cfg::NDB; ++i) acc[i] *= alpha;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    uint4 pop[4];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t wds[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i0 = 8 * (u & 1) + 2 * jj;
        const float e0 = fast_exp2(__builtin_fmaf(s[u >> 1][i0], p.scale_log2, -m_use));
        const float e1 = fast_exp2(__builtin_fmaf(s[u >> 1][i0 + 1], p.scale_log2, -m_use));
        wds[jj] = pack2<QBF16>(e0, e1);
        if constexpr (Cfg::kF32Sum) psum += e0 + e1;
      }
      pop[u] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
      accs = mfma32x32x16<QBF16>(ones, pop[u], accs);
    }
    if constexpr (Cfg::kF32Sum) l_run += psum;
    // O^T += V^T P^T.  Lane (hh, rho) needs column 32*db + rho of the V tile
    // over tokens r0..r0+3 and r0+8..r0+11 (r0 = 32*(u/2) + 16*(u%2) + 4*hh),
    // the order its P^T slots hold: two transposed LDS reads of 4 rows each.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint8_t* a1 = vl + (32 * (u >> 1) + 16 * (u & 1)) * Cfg::VP;
#pragma unroll
      for (int db = 0; db < Cfg::NDB; ++db) {
        const uint2 x1 = lds_tr16(a1 + 64 * db);
        const uint2 x2 = lds_tr16(a1 + 8 * Cfg::VP + 64 * db);
        acc[db] = mfma32x32x16<QBF16>(make_uint4(x1.x, x1.y, x2.x, x2.y), pop[u], acc[db]);
      }
    }
  };

  // two LDS stages, tile loads two tiles ahead (page ids four), one barrier per tile (it
  // publishes the stage just written and tells the writer of the other stage
  // that its previous readers are done); past the last tile the index is
  // clamped, so the extra loads re-read cached lines
  if (ntiles > 0) {
    auto tile_of = [&](int k) { return min(k, ntiles - 1); };
    Regs ra, rb;
    load_pids(0, ra);
    load_pids(tile_of(1), rb);
    load_tile(0, ra);
    load_pids(tile_of(2), ra);
    load_tile(tile_of(1), rb);
    load_pids(tile_of(3), rb);
    // Tiles go in pairs and both halves always load (an odd count re-reads
    // the last tile once), so every path round the loop issues the same
    // loads and the memory waits stay one tile deep.
    for (int k = 0; k < ntiles; k += 2) {
      store_tile(ra, smem);
      load_tile(tile_of(k + 2), ra);
      load_pids(tile_of(k + 4), ra);
      __syncthreads();
      if (wave_ok) compute(k, smem);
      store_tile(rb, smem + Cfg::STAGE);
      load_tile(tile_of(k + 3), rb);
      load_pids(tile_of(k + 5), rb);
      __syncthreads();
      if (wave_ok && k + 1 < ntiles) compute(k + 1, smem + Cfg::STAGE);
    }
  }

  // epilogue
  const float lr_run = accs[0];
  if constexpr (Cfg::kF32Sum) l_run = xor_sum(l_run, 32);
  else l_run = lr_run;
  if (!row_ok) return;
  const float inv = (lr_run > 0.f) ? p.v_scale / lr_run : 0.f;
  uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)(q_begin + qpos) * p.num_qo_heads + hq) * D;
#pragma unroll
  for (int db = 0; db < Cfg::NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = Cfg::dim_of(32 * db + 8 * i4 + 4 * hh);  // 4 positions, 4 consecutive dimensions
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
