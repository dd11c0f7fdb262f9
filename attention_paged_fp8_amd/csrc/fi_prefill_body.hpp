// The batched (causal) prefill over a paged or ragged KV cache as a device
// function: the work of one prefill workgroup (kPrefillWaves waves), shared
// by the prefill kernel and the fused prefill + decode kernel.  What it
// computes and how it maps onto gfx950 is described at the top of
// fi_prefill.hip.
#pragma once

#include <type_traits>

#include "fi_device.hpp"

namespace fi {

// Q8: an fp8 query; K stays fp8 in LDS and S = K Q^T runs on the fp8 MFMA,
// while P V runs in fp16 (QBF16 is then false).  P8 (with Q8): V stays fp8
// in LDS too, the probabilities are rounded to e4m3 and P V also runs on the
// fp8 MFMA; the output is then normalised by the fp32 sum.
template <bool QBF16, int KVF, bool OBF16, int D, bool Q8, bool P8 = false>
struct PrefillCfg {
  static constexpr bool kFp8 = (KVF == FMT_E4M3 || KVF == FMT_E5M2 || KVF == FMT_E4M3_FNUZ || KVF == FMT_E5M2_FNUZ);
  static_assert(!Q8 || KVF == FMT_E4M3 || KVF == FMT_E5M2, "an fp8 query needs an OCP fp8 KV cache");
  static_assert(!P8 || Q8, "fp8 P V needs the fp8 query path");
  static constexpr bool kP8 = P8;
  // The output is normalised by the sum of the probabilities as rounded for
  // the PV MFMA.  fp16 rounds at 2^-11 and that sum also gives the
  // log-sum-exp; bf16 rounds at 2^-9, so its log-sum-exp uses a separate sum
  // of the fp32 values.
  static constexpr bool kF32Lse = QBF16 || P8;
  static constexpr int KVB = kFp8 ? 1 : 2;
  static constexpr int TK = 64;                 // keys per tile
  static constexpr int DB = D * KVB;            // stored bytes of a row
  static constexpr int ROW = D * 2;             // bytes of a 2-byte row
  // K tile pitch: 16 mod 256 bytes for 2-byte rows; raw fp8 rows (Q8) take
  // D + 16, an odd multiple of 16 bytes, so the 16-byte reads of 16
  // consecutive rows fall in distinct bank groups
  static constexpr int KP = Q8 ? D + 16 : ROW + 16;
  // V tile pitch: 64 mod 256 bytes for 2-byte rows; raw fp8 rows (P8) take
  // D + 32, an odd multiple of 32 bytes, so 8 consecutive rows fall in distinct
  // 32-byte bank groups for the transposed byte reads
  static constexpr int VP = P8 ? D + 32 : (ROW + 191) / 256 * 256 + 64;
  static constexpr int KTILE = TK * KP;
  static constexpr int VTILE = TK * VP;
  // two K slots, then two V slots
  static constexpr int K0 = 0, K1 = KTILE, V0 = 2 * KTILE, V1 = 2 * KTILE + VTILE;
  // The epilogue stages the normalised output in the same memory: the
  // workgroup's 256 rows as its query tokens, each token's heads_per_wg rows
  // contiguous (as in o) and the token pitch padded by 16 bytes (16-byte
  // aligned pieces; the 32 tokens of a wave's rows spread over 16 bank
  // groups).  Largest with one head per workgroup (256 tokens).
  static constexpr int OSTAGE = 256 * (ROW + 16);
  // The prologue brings the query block in the same way, into its own area
  // after the slots: each token's heads_per_wg query rows contiguous, token
  // pitch padded by 16 bytes.
  static constexpr int QROW = Q8 ? D : 2 * D;       // bytes of a query row
  static constexpr int QS = 2 * KTILE + 2 * VTILE;  // offset of the query area
  static constexpr int QSTAGE = 256 * (QROW + 16);
  static constexpr int QPER = 256 * QROW / 16 / (64 * kPrefillWaves);  // 16-byte query pieces per thread
  static constexpr int LDS = (QS + QSTAGE > OSTAGE) ? QS + QSTAGE : OSTAGE;
  static constexpr int NT = 64 * kPrefillWaves;     // threads per workgroup
  static constexpr int CHUNKS = TK * DB / 16;       // 16-byte pieces of a tile of one tensor
  static constexpr int PER = (CHUNKS + NT - 1) / NT;  // per thread (the last round may be partial)
  static constexpr int NS = D / 16;             // QK k-steps (MFMA k = 16)
  static constexpr int NS8 = D / 64;            // QK k-steps of the fp8 MFMA (k = 64)
  static constexpr int NDB = D / 32;            // PV head_dim blocks of 32
  // Head-dimension order of the LDS tiles: position p holds dimension
  // dim_of(p), each run of 16 dimensions split into halves D/2 positions
  // apart.  An fp8 lane holds 16 consecutive dimensions and stores their
  // widened halves 128 bytes apart; a 2-byte lane holds 8 and stores them in
  // one of the halves -- either way the lanes of a row write two contiguous
  // runs, and both cache types produce the same tile for the same values.
  __host__ __device__ static constexpr int dim_of(int p) {
    return p < D / 2 ? 16 * (p / 8) + p % 8 : 16 * ((p - D / 2) / 8) + 8 + (p - D / 2) % 8;
  }
};

// Instruction order of the two blocks of a step (sched_group_barrier masks:
// 0x008 MFMA, 0x002 VALU, 0x400 transcendental, 0x100 LDS read, 0x200 LDS
// write).  Block 1 computes S(j+1) = K Q^T while the probabilities of S(j)
// are formed: a few K reads ahead, then each QK MFMA followed by a share of
// the exponential work and one more LDS read.  Block 2 accumulates P V while
// the row max of S(j+1) is taken and the next K tile is widened into LDS:
// each PV MFMA with its two transposed reads and a share of that VALU work.
template <int NQK>
__device__ __forceinline__ void schedule_qk_exp() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}
// Block 1 with the fp8 QK MFMA (k = 64, twice the work of a 16-bit one):
// each MFMA with its two 16-byte K reads and a larger share of the
// exponential work.
template <int NQK>
__device__ __forceinline__ void schedule_qk8_exp() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, 20, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}
// Block 2 with the fp8 PV MFMA: each MFMA with its four transposed byte
// reads and a share of the row max work, then the K stores.
template <int NPV>
__device__ __forceinline__ void schedule_pv8_max() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);
}
template <int NPV>
__device__ __forceinline__ void schedule_pv_max() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);
}

// RAGGED: K/V rows are contiguous per request -- token t of request b is row
// indptr[b] + t of the pools (or row t when indptr is NULL) -- so the page
// walk reduces to an addition and no index is loaded.
// Workgroup (bx, by) of the prefill grid: bx = dispatch-order item x (kv head,
// head group) when the host passed an order, else (request, kv head, head
// group) with by the query block; LDS at smem (PrefillCfg::LDS bytes).
template <int QF, int KVF, bool OBF16, int D, bool RAGGED, bool P8, class P>
__device__ __forceinline__ void prefill_body(const P& p, const int bx, const int by, uint8_t* smem) {
  constexpr bool QBF16 = QF == FMT_BF16;
  constexpr bool Q8 = QF == FMT_E4M3 || QF == FMT_E5M2;
  using Cfg = PrefillCfg<QBF16, KVF, OBF16, D, Q8, P8>;

  const int nsg = p.group / p.heads_per_wg;
  const int x = bx;
  const int sg = x % nsg;
  const int g = (x / nsg) % p.num_kv_heads;
  int b, qb;
  if (p.n_items > 0) {  // (request, query block) pairs in the host's heaviest-first order
    const uint32_t item = p.order[x / (nsg * p.num_kv_heads)];
    b = (int)(item >> 16);
    qb = (int)(item & 0xffffu);
  } else {
    b = x / (nsg * p.num_kv_heads);
    qb = p.n_qblocks - 1 - by;  // latest query blocks first
  }

  // request geometry: uniform over the workgroup, kept in scalar registers so
  // that the tile loop and its branches stay scalar
  // (a single request passes its lengths in the arguments instead of indptrs)
  // (from the kernel arguments when the host passed them: the first page-id
  // loads then wait for no device load)
  int q_begin, qo_len, a, kv_len;
  if (b < p.n_geo) {
    q_begin = p.geo[b][0];
    qo_len = p.geo[b][1];
    a = p.geo[b][2];
    kv_len = p.geo[b][3];
  } else {
    q_begin = p.qo_indptr ? uniform(p.qo_indptr[b]) : 0;
    qo_len = p.qo_indptr ? uniform(p.qo_indptr[b + 1]) - q_begin : p.single_qo_len;
    a = p.indptr ? uniform(p.indptr[b]) : 0;
    if (RAGGED) {
      kv_len = p.indptr ? uniform(p.indptr[b + 1]) - a : p.single_kv_len;
    } else {
      const int e = uniform(p.indptr[b + 1]);
      kv_len = (e > a) ? (e - a - 1) * p.page_size + uniform(p.last_page_len[b]) : 0;
    }
  }
  const int q0 = qb * p.q_per_wg;
  if (q0 >= qo_len) return;
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
  // tiles this wave computes (a prefix of the workgroup's tiles)
  const int ntw = uniform((qw0 < qo_len && wave_any_end > 0) ? (wave_any_end + Cfg::TK - 1) / Cfg::TK : 0);

  // Q^T operand: lane (hh, rho) holds q[row rho] at the dimensions of K tile
  // positions (D/2)*hh + 8s + j, j = 0..7 (8 consecutive dimensions).
  // fp8 query (Q8): for k-step c, lane (hh, rho) holds the 32 bytes of
  // dimensions 64c + 32hh .. +31, in memory order (K rows are read the same way).
  // Filled in the prologue from the query area of LDS (rows past the block's
  // queries are zero there).
  uint4 qop[Cfg::NS];
  const int qtokp = p.heads_per_wg * Cfg::QROW + 16;  // query area pitch of a token

  // ---- tile gather ---------------------------------------------------------
  // Chunk ci = j*NT + tid of a tensor's tile is row ci / (DB/16), 16-byte
  // column ci % (DB/16): 8 lanes read one 128-byte fp8 row (whole waves sit
  // out a partial last round).  Rows past kv_len re-read the last valid token
  // (finite values whose keys the mask sets to -inf, so their probabilities
  // are exactly 0).
  constexpr int SC = Cfg::DB / 16;
  int ld_row[Cfg::PER], ld_col[Cfg::PER];
#pragma unroll
  for (int j = 0; j < Cfg::PER; ++j) {
    const int ci = j * Cfg::NT + tid;
    ld_row[j] = ci / SC;
    ld_col[j] = ci % SC;
  }
  // does round j of this thread hold a chunk? (uniform per wave)
  auto ld_on = [&](int j) { return Cfg::CHUNKS % Cfg::NT == 0 || j * Cfg::NT + w * 64 < Cfg::CHUNKS; };
  const uint8_t* kb = p.k + (int64_t)g * p.sh;
  const uint8_t* vb = p.v + (int64_t)g * p.sh;
  // a tile's K and V on their way from memory to LDS
  struct Fetch {
    uint4 k[Cfg::PER], v[Cfg::PER];
  };
  uint64_t goff[Cfg::PER];  // byte offsets of this thread's rows of the tile being fetched
  auto tile_of = [&](int t) { return min(t, ntiles - 1); };
  auto row_token = [&](int tile, int j) { return min(tile * Cfg::TK + ld_row[j], max(kv_len - 1, 0)); };
  auto load_pids = [&](int tile, uint32_t(&pid)[Cfg::PER]) {
#pragma unroll
    for (int j = 0; j < Cfg::PER; ++j)
      if (ld_on(j)) {
        if (RAGGED)
          pid[j] = (uint32_t)(a + row_token(tile, j));  // the row itself
        else
          pid[j] = (uint32_t)p.indices[a + (row_token(tile, j) >> p.page_shift)];
      }
  };
  auto offset = [&](int tile, int j, uint32_t pid) -> uint64_t {
    if (RAGGED) return (uint64_t)pid * (uint32_t)p.st + (uint32_t)(ld_col[j] * 16);
    // byte strides are below 4 GiB, page ids and slots non-negative: each term
    // is a 32 x 32 -> 64-bit product (a slot times the token stride can pass
    // 4 GiB, e.g. 127 slots of a token-major pool)
    const int t = row_token(tile, j);
    return (uint64_t)pid * (uint32_t)p.sp + (uint64_t)(uint32_t)(t & (p.page_size - 1)) * (uint32_t)p.st +
           (uint32_t)(ld_col[j] * 16);
  };
  auto locate = [&](int tile, const uint32_t(&pid)[Cfg::PER]) {
#pragma unroll
    for (int j = 0; j < Cfg::PER; ++j)
      if (ld_on(j)) goff[j] = offset(tile, j, pid[j]);
  };
  auto load_k = [&](Fetch& f) {
#pragma unroll
    for (int j = 0; j < Cfg::PER; ++j)
      if (ld_on(j)) f.k[j] = load16(kb + goff[j]);
  };
  auto load_v = [&](Fetch& f) {
#pragma unroll
    for (int j = 0; j < Cfg::PER; ++j)
      if (ld_on(j)) f.v[j] = load16(vb + goff[j]);
  };
  // store rows into an LDS slot in the dim_of order, fp8 widened to q's type
  // (raw: fp8 rows for the fp8 MFMA, as loaded; fp8 V rows (P8) go to row
  // v8_row(t), which lists each 16-token block as tokens 0-3, 8-11, 4-7,
  // 12-15, so that every transposed read of P V takes 8 consecutive rows)
  auto v8_row = [](int t) { return (t & ~15) | (t & 3) | (((t >> 3) & 1) << 2) | (((t >> 2) & 1) << 3); };
  auto store_rows_with = [&](const uint4(&r)[Cfg::PER], uint8_t* slot, int pitch, auto raw, auto vperm, auto w4) {
    auto w8 = [&](uint32_t lo, uint32_t hi) {
      const uint2 a = w4(lo), b = w4(hi);
      return make_uint4(a.x, a.y, b.x, b.y);
    };
#pragma unroll
    for (int j = 0; j < Cfg::PER; ++j) {
      if (!ld_on(j)) continue;
      uint8_t* d = slot + (decltype(vperm)::value ? v8_row(ld_row[j]) : ld_row[j]) * pitch;
      if constexpr (decltype(raw)::value) {
        *reinterpret_cast<uint4*>(d + 16 * ld_col[j]) = r[j];
      } else if constexpr (Cfg::kFp8) {  // dimensions 16c..16c+7 to position 8c, 16c+8.. to D/2 + 8c
        *reinterpret_cast<uint4*>(d + 16 * ld_col[j]) = w8(r[j].x, r[j].y);
        *reinterpret_cast<uint4*>(d + D + 16 * ld_col[j]) = w8(r[j].z, r[j].w);
      } else {  // dimensions 8c..8c+7 to position 8(c/2) (c even) or D/2 + 8(c/2) (c odd)
        *reinterpret_cast<uint4*>(d + 16 * (ld_col[j] >> 1) + D * (ld_col[j] & 1)) = r[j];
      }
    }
  };
  // fnuz caches widen through the OCP converter (fast form) unless a code of
  // the wave's chunks lies outside the OCP reading; the two forms give
  // identical values
  auto store_rows = [&](const uint4(&r)[Cfg::PER], uint8_t* slot, int pitch, auto raw, auto vperm) {
    auto exact = [](uint32_t w) { return widen4<QBF16, KVF>(w); };
    if constexpr ((KVF == FMT_E4M3_FNUZ || KVF == FMT_E5M2_FNUZ) && !decltype(raw)::value) {
      uint32_t out = 0;
#pragma unroll
      for (int j = 0; j < Cfg::PER; ++j)
        if (ld_on(j))
          out |= fnuz_outside_ocp<KVF>(r[j].x) | fnuz_outside_ocp<KVF>(r[j].y) | fnuz_outside_ocp<KVF>(r[j].z) |
                 fnuz_outside_ocp<KVF>(r[j].w);
      if (__builtin_amdgcn_ballot_w64(out != 0) == 0)
        store_rows_with(r, slot, pitch, raw, vperm, [](uint32_t w) { return widen4_fnuz_ocp<QBF16, KVF>(w); });
      else
        store_rows_with(r, slot, pitch, raw, vperm, exact);
    } else {
      store_rows_with(r, slot, pitch, raw, vperm, exact);
    }
  };
  auto store_k = [&](const Fetch& f, uint8_t* slot) {
    store_rows(f.k, slot, Cfg::KP, std::integral_constant<bool, Q8>{}, std::false_type{});
  };
  auto store_v = [&](const Fetch& f, uint8_t* slot) {
    store_rows(f.v, slot, Cfg::VP, std::integral_constant<bool, P8>{}, std::integral_constant<bool, P8>{});
  };

  // ---- per-wave attention state --------------------------------------------
  float m_run = kNegInf;  // running max (base-2 scaled logits), updated lazily
  float lr_run = 0.f;     // this lane's share of the sum of rounded probabilities
  float l_run = 0.f;      // bf16: this lane's share of the fp32 probability sum
  f32x16_t acc[Cfg::NDB];
#pragma unroll
  for (int i = 0; i < Cfg::NDB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;

  // per-lane LDS read bases within a slot; everything else is a constant offset.
  // K: lane (hh, rho) reads row 32*sub + rho, bytes [D*hh + 16*st, +16).
  // V^T transposed reads: within each 16-lane group (same hh, same rho / 16),
  // lanes 4r..4r+3 name the four 8-byte pieces of row r of a 16-column block.
  const int k_base = rho * Cfg::KP + (Q8 ? 32 : D) * hh;
  const int v_base = (4 * hh + ((rho & 15) >> 2)) * Cfg::VP + 32 * (rho >> 4) + 8 * (rho & 3);
  // fp8 V^T (P8) transposed byte reads: in 16-lane group G = lane / 16 (hh =
  // G / 2), lanes 2r and 2r+1 name the two 8-byte halves of row 8hh + r of a
  // 16-row block at dimensions 16(G % 2) .. +15 of a 32-dimension block
  const int v8_base = (8 * hh + ((rho & 15) >> 1)) * Cfg::VP + 16 * (rho >> 4) + 8 * (rho & 1);

  // S^T = K Q^T for one tile, two 32-token halves; lane (hh, rho) then holds
  // keys 32*sub + 8*(i/4) + 4*hh + i%4 of row rho
  auto qk = [&](const uint8_t* kslot, f32x16_t(&s)[2]) {
    const uint8_t* kl = kslot + k_base;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[sub][j] = 0.f;
      if constexpr (Q8) {
#pragma unroll
        for (int c = 0; c < Cfg::NS8; ++c) {
          const uint8_t* a = kl + 32 * sub * Cfg::KP + 64 * c;
          s[sub] = mfma32x32x64_f8<KVF, QF>(*reinterpret_cast<const uint4*>(a), *reinterpret_cast<const uint4*>(a + 16),
                                            qop[2 * c], qop[2 * c + 1], s[sub]);
        }
      } else {
#pragma unroll
        for (int st = 0; st < Cfg::NS; ++st) {
          const uint4 kop = *reinterpret_cast<const uint4*>(kl + 32 * sub * Cfg::KP + 16 * st);
          s[sub] = mfma32x32x16<QBF16>(kop, qop[st], s[sub]);
        }
      }
    }
  };
  // mask of the keys a row does not see (only tiles that cross the diagonal
  // or the end of the sequence)
  auto mask = [&](int tile, f32x16_t(&s)[2]) {
    const int kbase = tile * Cfg::TK;
    if (kbase + Cfg::TK > wave_full_end) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = kbase + 32 * sub + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (t >= row_key_end) s[sub][i] = kNegInf;
        }
    }
  };
  // row max in base-2 logit units (scale > 0 keeps the order)
  auto row_max = [&](const f32x16_t(&s)[2]) -> float {
    float mx = fmaxf(s[0][0], s[0][1]);  // then three-operand maxima over pairs
#pragma unroll
    for (int i = 2; i < 32; i += 2) mx = fmaxf(mx, fmaxf(s[i >> 4][i & 15], s[i >> 4][(i & 15) + 1]));
    return max_half_swap(mx) * p.scale_log2;
  };
  // lazy rescale: the reference max moves only when some row's max grows by
  // more than 8 (log2), so exp2 stays below 2^8; returns the max the
  // exponents subtract
  auto rebase = [&](float mx) -> float {
    const bool grow = mx > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      lr_run *= alpha;
      if constexpr (Cfg::kF32Lse) l_run *= alpha;
#pragma unroll
      for (int i = 0; i < Cfg::NDB; ++i) acc[i] *= alpha;
    }
    return (m_run == kNegInf) ? 0.f : m_run;
  };
  // probabilities, rounded to the MFMA type and packed as the P^T operand
  // (slot u = tokens 16u .. 16u+15), and their row sums
  auto exp_pack = [&](const f32x16_t(&s)[2], float m_use, uint4(&pop)[4]) {
    float rsum = 0.f, psum = 0.f;
    if constexpr (P8) {
      // e4m3 probabilities, byte 16*sub + i of the P^T operand holding S(j)
      // register s[sub][i] (keys 32sub + 8(i/4) + 4hh + i%4)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        uint32_t wds[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int i0 = 4 * d;
          const float e0 = fast_exp2(__builtin_fmaf(s[sub][i0], p.scale_log2, -m_use));
          const float e1 = fast_exp2(__builtin_fmaf(s[sub][i0 + 1], p.scale_log2, -m_use));
          const float e2 = fast_exp2(__builtin_fmaf(s[sub][i0 + 2], p.scale_log2, -m_use));
          const float e3 = fast_exp2(__builtin_fmaf(s[sub][i0 + 3], p.scale_log2, -m_use));
          int wd = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
          wd = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, wd, true);
          wds[d] = (uint32_t)wd;
          psum += (e0 + e1) + (e2 + e3);
        }
        pop[sub] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
      }
      l_run += psum;
      return;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t wds[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i0 = 8 * (u & 1) + 2 * jj;
        const float e0 = fast_exp2(__builtin_fmaf(s[u >> 1][i0], p.scale_log2, -m_use));
        const float e1 = fast_exp2(__builtin_fmaf(s[u >> 1][i0 + 1], p.scale_log2, -m_use));
        wds[jj] = pack2<QBF16>(e0, e1);
        rsum = sum2<QBF16>(wds[jj], rsum);
        if constexpr (Cfg::kF32Lse) psum += e0 + e1;
      }
      pop[u] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    }
    lr_run += rsum;
    if constexpr (Cfg::kF32Lse) l_run += psum;
  };
  // O^T += V^T P^T.  Lane (hh, rho) needs column 32*db + rho of the V tile
  // over tokens r0..r0+3 and r0+8..r0+11 (r0 = 32*(u/2) + 16*(u%2) + 4*hh),
  // the order its P^T slots hold: two transposed LDS reads of 4 rows each.
  auto pv = [&](const uint8_t* vslot, const uint4(&pop)[4]) {
    if constexpr (P8) {
      // O^T += V^T P^T on the fp8 MFMA, one per 32 dimensions: A byte 8r + b
      // is dimension 32db + lane%32 of token 32(r/2) + 16(r%2) + 8(b/4) + 4hh
      // + b%4, the key order of the P^T bytes
      const uint8_t* vl = vslot + v8_base;
#pragma unroll
      for (int db = 0; db < Cfg::NDB; ++db) {
        uint2 x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = lds_tr8(vl + (32 * (r >> 1) + 16 * (r & 1)) * Cfg::VP + 32 * db);
        acc[db] = mfma32x32x64_f8<KVF, FMT_E4M3>(make_uint4(x[0].x, x[0].y, x[1].x, x[1].y),
                                                  make_uint4(x[2].x, x[2].y, x[3].x, x[3].y), pop[0], pop[1], acc[db]);
      }
      return;
    }
    const uint8_t* vl = vslot + v_base;
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

  // ---- the tile pipeline ---------------------------------------------------
  // Step j: issue S(j+1) = K(j+1) Q^T on the matrix cores while the same wave
  // turns S(j) into probabilities; accumulate P(j) V(j) while it masks S(j+1),
  // takes its row max and stores K(j+2) into the slot K(j) used; move the
  // reference max for S(j+1) (after P(j) V(j), which a rescale applies to);
  // fetch K(j+4); one barrier; store V(j+2) into the slot V(j) used and fetch
  // V(j+4).
  // K and V each have two LDS slots; the barrier orders every slot's readers
  // before its next writer and every writer before its readers.  Two register
  // sets keep tiles in flight two steps ahead; page ids are fetched one step
  // before the data they address.
  auto step = [&](int j, f32x16_t(&sc)[2], f32x16_t(&sn)[2], Fetch& f, const uint32_t(&pcur)[Cfg::PER],
                  uint32_t(&pnext)[Cfg::PER], uint8_t* k_this, const uint8_t* k_next, uint8_t* v_this,
                  float& m_use) {
    locate(tile_of(j + 4), pcur);
    if (j < ntw) {
      uint4 pop[4];
      // S(j+1) even past this wave's last tile (the slot then holds a
      // clamped copy and the result goes unused): no branch splits the
      // matrix-core work from the VALU work it overlaps
      qk(k_next, sn);
      exp_pack(sc, m_use, pop);
      // the probabilities are materialised here, beside the QK products,
      // rather than sunk past the mask branch into the PV block (emits nothing)
#pragma unroll
      for (int u = 0; u < (P8 ? 2 : 4); ++u) asm volatile("" ::"v"(pop[u].x), "v"(pop[u].y), "v"(pop[u].z), "v"(pop[u].w));
      if constexpr (Q8)
        schedule_qk8_exp<2 * Cfg::NS8>();
      else
        schedule_qk_exp<2 * Cfg::NS>();
      mask(j + 1, sn);
      pv(v_this, pop);
      const float mx = row_max(sn);
      store_k(f, k_this);
      if constexpr (P8)
        schedule_pv8_max<Cfg::NDB>();
      else
        schedule_pv_max<4 * Cfg::NDB>();
      m_use = rebase(mx);  // after P(j) V(j): a rescale applies to it
    } else {
      store_k(f, k_this);
    }
    load_k(f);
    load_pids(tile_of(j + 5), pnext);
    __syncthreads();
    store_v(f, v_this);
    load_v(f);
  };

  if (ntiles > 0) {
    uint8_t* const K0 = smem + Cfg::K0;
    uint8_t* const K1 = smem + Cfg::K1;
    uint8_t* const V0 = smem + Cfg::V0;
    uint8_t* const V1 = smem + Cfg::V1;
    uint32_t pa[Cfg::PER], pb[Cfg::PER];
    f32x16_t s0[2], s1[2];
    Fetch fa, fb;
    {
      // tiles 0..3 go out together; 0 and 1 land in LDS, 2 and 3 stay in
      // the register sets of steps 0 and 1
      uint32_t i0[Cfg::PER], i1[Cfg::PER], i2[Cfg::PER], i3[Cfg::PER];
      load_pids(0, i0);
      load_pids(tile_of(1), i1);
      load_pids(tile_of(2), i2);
      load_pids(tile_of(3), i3);
      load_pids(tile_of(4), pb);
      // the query block, after the page ids (which the K/V addresses wait
      // for): whole 16-byte pieces of each token's contiguous head rows
      const int qshift = __builtin_ctz(p.heads_per_wg * Cfg::QROW / 16);  // pieces per token
      const int ntok = min(p.q_per_wg, qo_len - q0);
      const uint8_t* qsrc =
          reinterpret_cast<const uint8_t*>(p.q) + ((int64_t)(q_begin + q0) * p.num_qo_heads + hq - head_local) * Cfg::QROW;
      const int64_t qtok_stride = (int64_t)p.num_qo_heads * Cfg::QROW;
      uint4 qst[Cfg::QPER];
#pragma unroll
      for (int k = 0; k < Cfg::QPER; ++k) {
        const int pc = k * Cfg::NT + tid;
        const int t = pc >> qshift;
        qst[k] = t < ntok ? load16(qsrc + t * qtok_stride + 16 * (pc - (t << qshift))) : make_uint4(0, 0, 0, 0);
      }
      Fetch f0, f1;
      locate(0, i0);
      load_k(f0);
      load_v(f0);
      locate(tile_of(1), i1);
      load_k(f1);
      load_v(f1);
      locate(tile_of(2), i2);
      load_k(fa);
      load_v(fa);
      locate(tile_of(3), i3);
      load_k(fb);
      load_v(fb);
#pragma unroll
      for (int k = 0; k < Cfg::QPER; ++k) {
        const int pc = k * Cfg::NT + tid;
        const int t = pc >> qshift;
        *reinterpret_cast<uint4*>(smem + Cfg::QS + t * qtokp + 16 * (pc - (t << qshift))) = qst[k];
      }
      store_k(f0, K0);
      store_v(f0, V0);
      store_k(f1, K1);
      store_v(f1, V1);
    }
    __syncthreads();
    {
      const uint8_t* qrow = smem + Cfg::QS + (qpos - q0) * qtokp + head_local * Cfg::QROW;
      if constexpr (Q8) {
#pragma unroll
        for (int s = 0; s < 2 * Cfg::NS8; ++s)
          qop[s] = *reinterpret_cast<const uint4*>(qrow + 32 * hh + 64 * (s >> 1) + 16 * (s & 1));
      } else {
#pragma unroll
        for (int s = 0; s < Cfg::NS; ++s)
          qop[s] = *reinterpret_cast<const uint4*>(qrow + 2 * Cfg::dim_of((D / 2) * hh + 8 * s));
      }
    }
    float m_use = 0.f;
    if (ntw > 0) {
      qk(K0, s0);
      mask(0, s0);
      m_use = rebase(row_max(s0));
    }
    __syncthreads();  // every wave has read K(0) before step 0 overwrites its slot
    // Steps go in pairs (the register roles swap) and every step stores,
    // loads and waits whether or not this wave computes, so every path
    // round the loop issues the same memory operations.
    for (int j = 0; j < ntiles; j += 2) {
      step(j, s0, s1, fa, pb, pa, K0, K1, V0, m_use);
      step(j + 1, s1, s0, fb, pa, pb, K1, K0, V1, m_use);
    }
  }

  // ---- epilogue ------------------------------------------------------------
  lr_run = sum_half_swap(lr_run);
  l_run = Cfg::kF32Lse ? sum_half_swap(l_run) : lr_run;
  const float lnorm = P8 ? l_run : lr_run;  // fp8 probabilities: the fp32 sum
  // a row without visible keys has sums of exactly +0; a NaN read from the
  // cache makes them NaN, which then carries into o and lse
  const float inv = has_weight(lnorm) ? p.v_scale / lnorm : 0.f;
  // The output goes out through LDS: a lane's own values are 4 dimensions of
  // one row, and storing them directly scatters each wave store over 32 rows
  // 32 * num_qo_heads * D bytes apart; staged, a token's heads_per_wg rows
  // (contiguous in o) leave as whole 16-byte pieces of one run.
  const int tokp = p.heads_per_wg * Cfg::ROW + 16;  // staging pitch of a token
  __syncthreads();  // every wave is done with the K/V slots
  {
    uint8_t* orow = smem + (qpos - q0) * tokp + head_local * Cfg::ROW;
#pragma unroll
    for (int db = 0; db < Cfg::NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        // 4 positions, 4 consecutive dimensions (fp8 V^T rows are dimensions)
        const int d = P8 ? 32 * db + 8 * i4 + 4 * hh : Cfg::dim_of(32 * db + 8 * i4 + 4 * hh);
        *reinterpret_cast<uint2*>(orow + 2 * d) =
            make_uint2(pack2<OBF16>(acc[db][4 * i4] * inv, acc[db][4 * i4 + 1] * inv),
                       pack2<OBF16>(acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv));
      }
  }
  __syncthreads();
  {
    const int pieces_shift = __builtin_ctz(p.heads_per_wg * Cfg::ROW / 16);  // 16-byte pieces per token
    const int ntok = min(p.q_per_wg, qo_len - q0);
    const int64_t tok_stride = (int64_t)p.num_qo_heads * Cfg::ROW;
    uint8_t* ob = reinterpret_cast<uint8_t*>(p.o) + ((int64_t)(q_begin + q0) * p.num_qo_heads + hq - head_local) * Cfg::ROW;
    for (int k = tid; k < (ntok << pieces_shift); k += Cfg::NT) {
      const int t = k >> pieces_shift;
      const int c = k - (t << pieces_shift);
      *reinterpret_cast<uint4*>(ob + t * tok_stride + 16 * c) = *reinterpret_cast<const uint4*>(smem + t * tokp + 16 * c);
    }
  }
  if (p.lse && hh == 0 && row_ok)
    p.lse[(int64_t)(q_begin + qpos) * p.num_qo_heads + hq] =
        has_weight(l_run) ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
  // ---- end of item
}

}  // namespace fi
