// The batched paged decode as a device function: the work of one decode
// workgroup of NW waves, shared by the decode kernel (4 waves) and the fused
// prefill + decode kernel (8 waves).  What it computes and how it maps onto
// gfx950 is described at the top of fi_decode.hip.
#pragma once

#include "fi_device.hpp"

namespace fi {

// Page ids staged in LDS per window; a window spans kPidWindow pages.
constexpr int kPidWindow = 1024;

template <bool QBF16, int KVF, bool OBF16, int D, int NW = kDecodeWaves>
struct DecodeCfg {
  static constexpr int NT = 64 * NW;          // threads per workgroup
  static constexpr bool kFp8 = (KVF == FMT_E4M3 || KVF == FMT_E5M2 || KVF == FMT_E4M3_FNUZ || KVF == FMT_E5M2_FNUZ);
  // MFMA operand type: bf16 whenever q or a 2-byte cache is bf16.  An fp16
  // operand meeting a bf16 one is split exactly into bf16 hi + lo.
  static constexpr bool MBF16 = QBF16 || KVF == FMT_BF16;
  static constexpr bool kSplitQ = !QBF16 && MBF16;            // fp16 q, bf16 cache
  static constexpr bool kSplitKV = (KVF == FMT_F16) && MBF16;  // fp16 cache, bf16 q
  static constexpr int KVB = kFp8 ? 1 : 2;    // bytes per stored element
  static constexpr int DB = D * KVB;          // bytes of one head's row
  static constexpr int DB16 = DB / 16;        // 16-byte chunks of one head's row
  static constexpr int DL = D / 4;            // elements of a row a lane multiplies
  static constexpr int NS = D / 32;           // QK k-steps (MFMA 16x16x32)
  static constexpr int NDB = D / 16;          // PV head_dim blocks (MFMA 16x16x16)
  static constexpr int PITCH = NW * DB;             // LDS row pitch: up to NW heads
  static constexpr int TILE = kDecodeStep * PITCH;  // one pool, one step
  static constexpr int STAGE = 2 * TILE;            // K then V
  static constexpr int PER = kDecodeStep * PITCH / (16 * NT);  // 16-byte loads per thread per pool per step
  static constexpr int PIDS = 2 * STAGE;            // byte offset of the page-id window
  static constexpr int PREFIX = PIDS + (kPidWindow + 2) * 4;  // request prefix sums (balanced mode)
  static constexpr int WSUM = PREFIX + (kBalancedMaxBatch + 1) * 8;  // per-wave sums of the prefix scan
  static constexpr int LDS = WSUM + NW * 8;
};

// Tokens of request b (0 when it has no pages).
template <class P>
__device__ __forceinline__ int request_kv_len(const P& p, int b) {
  if (!p.indptr) return p.single_kv_len;
  const int a = p.indptr[b], e = p.indptr[b + 1];
  return (e > a) ? (e - a - 1) * p.page_size + p.last_page_len[b] : 0;
}

// Q8: an fp8 query (FMT_E4M3 / FMT_E5M2 codes, q_scale folded into the logit
// scale by the host), widened exactly to fp16 as it is loaded; QBF16 is then
// false and the kernel runs its fp16 path.  NW waves per workgroup (NT = 64 *
// NW threads): workgroup `bid` of `nblocks` decode workgroups, LDS at smem
// (DecodeCfg::LDS bytes).
template <bool QBF16, int KVF, bool OBF16, int D, int Q8, int NW, class P>
__device__ __forceinline__ void decode_body(const P& p, const int bid, const int nblocks, uint8_t* smem) {
  using Cfg = DecodeCfg<QBF16, KVF, OBF16, D, NW>;
  constexpr bool MB = Cfg::MBF16;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 15;
  const int qg = lane >> 4;
  const int groups = p.n_hgroups * p.n_sgroups;
  int* pids_s = reinterpret_cast<int*>(smem + Cfg::PIDS);
  const int shift = p.page_shift;
  const int hpw = 1 << p.hpw_shift;
  const int cpr_shift = __builtin_ctz(Cfg::DB16) + p.hpw_shift;
  const int cpr = 1 << cpr_shift;    // 16-byte chunks per token row of the workgroup's heads
  const int swz = min(cpr - 1, 7);   // XOR swizzle of a row's 16-byte chunks

  // Work on one piece: tokens [t_begin, t_end) of request b, head/slice group
  // grp, which is chunk `chunk_id` of the `nchunks` pieces of its segment.
  auto process = [&](int b, int grp, int t_begin, int t_end, int chunk_id, int nchunks) {
    const int hgrp = grp % p.n_hgroups;
    const int sgrp = grp / p.n_hgroups;
    const int pg_base = p.indptr ? p.indptr[b] : 0;
    const int nsteps = uniform((t_end > t_begin) ? (t_end - t_begin + kDecodeStep - 1) / kDecodeStep : 0);

    // this wave's (kv head, slice) and the workgroup's heads
    const int g0 = hgrp << p.hpw_shift;
    const int hl = w / p.spw;                         // head within the workgroup
    const int sub = sgrp * p.spw + (w - hl * p.spw);  // 16-row slice of the GQA group
    const bool wave_ok = hl < hpw && sub < p.nsub;
    const int g = g0 + (wave_ok ? hl : 0);
    const int rig = sub * kDecodeRows + c;            // row within the GQA group
    const bool row_ok = wave_ok && rig < p.group;
    const int h = g * p.group + (row_ok ? rig : 0);

    // Q^T operand: lane (qg, c) holds q[row c][DL*qg + 8s + j], j = 0..7.
    uint4 qop[Cfg::NS];
    uint4 qlo[Cfg::kSplitQ ? Cfg::NS : 1];
    if constexpr (Q8 != 0) {
      const uint2* qp = reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(p.q) +
                                                       ((int64_t)b * p.num_qo_heads + h) * D + Cfg::DL * qg);
#pragma unroll
      for (int s = 0; s < Cfg::NS; ++s) {
        const uint2 raw = row_ok ? qp[s] : make_uint2(0, 0);
        qop[s] = widen8<false, Q8>(raw.x, raw.y);
      }
    } else {
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

    // Cooperative loads: thread tid moves 16-byte chunks ci = j*NT + tid
    // (j < PER) of each pool; chunk ci is row ci / cpr, 16-byte column
    // ci % cpr of the workgroup's contiguous heads.  With fewer than NW heads
    // the surplus threads repeat a chunk another thread moves (same address,
    // same value).
    int ld_row[Cfg::PER], ld_col[Cfg::PER];
    int64_t ld_off[Cfg::PER];
#pragma unroll
    for (int j = 0; j < Cfg::PER; ++j) {
      const int ci = (j * Cfg::NT + tid) & (kDecodeStep * cpr - 1);
      ld_row[j] = ci >> cpr_shift;
      ld_col[j] = ci & (cpr - 1);
      const int hh = ld_col[j] / Cfg::DB16;
      ld_off[j] = (int64_t)(g0 + hh) * p.sh + (ld_col[j] - hh * Cfg::DB16) * 16;
    }
    int pg_lo = 0;
    struct Regs {
      uint4 k[Cfg::PER];
      uint4 v[Cfg::PER];
    };
    auto load_step = [&](int st, Regs& r) {
#pragma unroll
      for (int j = 0; j < Cfg::PER; ++j) {
        const int t = min(t_begin + st * kDecodeStep + ld_row[j], t_end - 1);
        const int pid = pids_s[(t >> shift) - pg_lo];
        // byte strides are below 4 GiB and page ids and slots are non-negative:
        // two 32 x 32 -> 64-bit multiply-adds instead of full 64-bit products
        const uint64_t off = (uint64_t)(uint32_t)pid * (uint32_t)p.sp +
                             ((uint64_t)(uint32_t)(t & (p.page_size - 1)) * (uint32_t)p.st + (uint64_t)ld_off[j]);
        r.k[j] = load16_stream(p.k + off);
        r.v[j] = load16_stream(p.v + off);
      }
    };
    auto store_step = [&](int st, Regs& r, uint8_t* stage) {
#pragma unroll
      for (int j = 0; j < Cfg::PER; ++j) {
        const bool ok = t_begin + st * kDecodeStep + ld_row[j] < t_end;
        const int o = ld_row[j] * Cfg::PITCH + 16 * (ld_col[j] ^ (ld_row[j] & swz));
        *reinterpret_cast<uint4*>(stage + o) = ok ? r.k[j] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(stage + Cfg::TILE + o) = ok ? r.v[j] : make_uint4(0, 0, 0, 0);
      }
    };

    float m_run = kNegInf;
    float l_run = 0.f;   // sum of fp32 probabilities (log-sum-exp)
    float lr_run = 0.f;  // sum of the rounded probabilities (output normalisation)
    f32x4_t acc[Cfg::NDB];
#pragma unroll
    for (int i = 0; i < Cfg::NDB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // K: lane (qg, c) reads token c, bytes [hl*DB + qg*DL*KVB, +DL*KVB) of its head
    const int kcol0 = hl * Cfg::DB16 + qg * (Cfg::DL * Cfg::KVB / 16);
    const int k_off = c * Cfg::PITCH;
    // V: transposed reads, see the PV step
    int v_off[Cfg::kFp8 ? Cfg::NDB / 2 : Cfg::NDB];
    if constexpr (Cfg::kFp8) {
      // lanes 2r, 2r+1 name row r: token 4qg + (r & 3), head_dim block 2i + (r >> 2)
      const int r = c >> 1;
      const int tok = 4 * qg + (r & 3);
#pragma unroll
      for (int i = 0; i < Cfg::NDB / 2; ++i) {
        const int col = hl * Cfg::DB16 + 2 * i + (r >> 2);
        v_off[i] = Cfg::TILE + tok * Cfg::PITCH + 16 * (col ^ (tok & swz)) + 8 * (c & 1);
      }
    } else {
      // lanes 4r..4r+3 name row r: token 4qg + r, the four 8-byte pieces of a
      // 16-wide head_dim block (32 bytes)
      const int r = c >> 2, q4 = c & 3;
      const int tok = 4 * qg + r;
#pragma unroll
      for (int i = 0; i < Cfg::NDB; ++i) {
        const int col = hl * Cfg::DB16 + 2 * i + (q4 >> 1);
        v_off[i] = Cfg::TILE + tok * Cfg::PITCH + 16 * (col ^ (tok & swz)) + 8 * (q4 & 1);
      }
    }

    // One step: kget(u) gives the u-th 16 bytes of this lane's K row, vget(i)
    // the i-th transposed V read, w4 widens 4 fp8 codes.
    auto compute_with = [&](int st, const uint8_t* stage, auto kget, auto vget, auto w4) {
      auto w8 = [&](uint32_t lo, uint32_t hi) {
        const uint2 a = w4(lo), b = w4(hi);
        return make_uint4(a.x, a.y, b.x, b.y);
      };
      const int tb = t_begin + st * kDecodeStep;
      // S^T = K Q^T over the step's 16 tokens
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < Cfg::DL * Cfg::KVB / 16; ++u) {
        const uint4 x = kget(u);
        if constexpr (Cfg::kFp8) {
          s = mfma16x16x32<MB>(w8(x.x, x.y), qop[2 * u], s);
          if constexpr (Cfg::kSplitQ) s = mfma16x16x32<true>(w8(x.x, x.y), qlo[2 * u], s);
          s = mfma16x16x32<MB>(w8(x.z, x.w), qop[2 * u + 1], s);
          if constexpr (Cfg::kSplitQ) s = mfma16x16x32<true>(w8(x.z, x.w), qlo[2 * u + 1], s);
        } else if constexpr (Cfg::kSplitKV) {
          uint4 khi, klo;
          split_f16x8(x, khi, klo);
          s = mfma16x16x32<true>(khi, qop[u], s);
          s = mfma16x16x32<true>(klo, qop[u], s);
        } else {
          s = mfma16x16x32<MB>(x, qop[u], s);
          if constexpr (Cfg::kSplitQ) s = mfma16x16x32<true>(x, qlo[u], s);
        }
      }
      // online softmax: lane (qg, c) holds tokens tb + 4qg + i of row c
      float x[4];
      float bm = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (tb + 4 * qg + i < t_end) ? s[i] * p.scale_log2 : kNegInf;
        bm = fmaxf(bm, x[i]);
      }
      bm = xor_max(bm, 16);
      bm = xor_max(bm, 32);
      const float m_new = fmaxf(m_run, bm);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float pe[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pe[i] = fast_exp2(x[i] - m_use);
      const uint2 pop = make_uint2(pack2<MB>(pe[0], pe[1]), pack2<MB>(pe[2], pe[3]));
      const float2 f0 = unpack2<MB>(pop.x), f1 = unpack2<MB>(pop.y);
      lr_run = lr_run * alpha + ((f0.x + f0.y) + (f1.x + f1.y));
      l_run = l_run * alpha + ((pe[0] + pe[1]) + (pe[2] + pe[3]));
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < Cfg::NDB; ++i) acc[i] *= alpha;
      // O^T += V^T P^T (MFMA 16x16x16): lane (qg, c) needs column 16*db + c of
      // tokens 4qg..4qg+3, the order its P^T slots hold.
      if constexpr (Cfg::kFp8) {
#pragma unroll
        for (int i = 0; i < Cfg::NDB / 2; ++i) {
          const uint2 v = vget(i);
          acc[2 * i] = mfma16x16x16<MB>(w4(v.x), pop, acc[2 * i]);
          acc[2 * i + 1] = mfma16x16x16<MB>(w4(v.y), pop, acc[2 * i + 1]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < Cfg::NDB; ++i) {
          const uint2 v = lds_tr16(stage + v_off[i]);
          if constexpr (Cfg::kSplitKV) {
            uint2 vhi, vlo;
            split_f16x2(v.x, vhi.x, vlo.x);
            split_f16x2(v.y, vhi.y, vlo.y);
            acc[i] = mfma16x16x16<true>(vhi, pop, acc[i]);
            acc[i] = mfma16x16x16<true>(vlo, pop, acc[i]);
          } else {
            acc[i] = mfma16x16x16<MB>(v, pop, acc[i]);
          }
        }
      }
    };

    auto k_lds = [&](const uint8_t* stage) {
      return [=](int u) { return *reinterpret_cast<const uint4*>(stage + k_off + 16 * ((kcol0 + u) ^ (c & swz))); };
    };
    auto compute = [&](int st, const uint8_t* stage) {
      if constexpr (KVF == FMT_E4M3_FNUZ || KVF == FMT_E5M2_FNUZ) {
        // The step's codes are read first; unless one of them lies outside
        // the OCP reading (e4m3fnuz: +-240, the extremes of the tensor;
        // e5m2fnuz: exponent 0 or 1, values below 2^-14 -- both rare), the
        // OCP converter widens them, else the exact bit form does -- the two
        // give identical values.
        constexpr int KU = Cfg::DL * Cfg::KVB / 16;
        uint4 kx[KU];
        uint2 vx[Cfg::NDB / 2];
        auto outside = [](uint32_t w) { return fnuz_outside_ocp<KVF>(w); };
        uint32_t hit = 0;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          kx[u] = k_lds(stage)(u);
          hit |= outside(kx[u].x) | outside(kx[u].y) | outside(kx[u].z) | outside(kx[u].w);
        }
#pragma unroll
        for (int i = 0; i < Cfg::NDB / 2; ++i) {
          vx[i] = lds_tr8(stage + v_off[i]);
          hit |= outside(vx[i].x) | outside(vx[i].y);
        }
        auto kreg = [&](int u) { return kx[u]; };
        auto vreg = [&](int i) { return vx[i]; };
        if (__builtin_amdgcn_ballot_w64(hit != 0) == 0)
          compute_with(st, stage, kreg, vreg, [](uint32_t w) { return widen4_fnuz_ocp<MB, KVF>(w); });
        else
          compute_with(st, stage, kreg, vreg, [](uint32_t w) { return widen4<MB, KVF>(w); });
      } else {
        compute_with(st, stage, k_lds(stage), [&](int i) { return lds_tr8(stage + v_off[i]); },
                     [](uint32_t w) { return widen4<MB, KVF>(w); });
      }
    };

    // Page ids are staged in LDS a window of kPidWindow pages at a time, so
    // that no K/V load waits on a page-id load.  Within a window the loads of
    // the next two steps are in flight while a step is computed; every step
    // costs one barrier (it publishes the stage just written, and tells the
    // writer of the other stage that its previous readers are done).  Past
    // the last step the step index is clamped, so the extra loads re-read
    // cached lines.
    const int win_steps =
        (int)min((int64_t)max(nsteps, 1), max((int64_t)1, ((int64_t)kPidWindow << shift) / kDecodeStep));
    for (int ws0 = 0; ws0 < nsteps; ws0 += win_steps) {
      const int ws1 = min(nsteps, ws0 + win_steps);
      pg_lo = (t_begin + ws0 * kDecodeStep) >> shift;
      const int pg_hi = ((min(t_begin + ws1 * kDecodeStep, t_end) - 1) >> shift) + 1;
      const int cnt = min(pg_hi - pg_lo, kPidWindow + 2);
      __syncthreads();  // the previous stages and page ids are no longer read
      for (int i = tid; i < cnt; i += Cfg::NT) pids_s[i] = p.indices ? p.indices[pg_base + pg_lo + i] : 0;
      __syncthreads();
      const int n = uniform(ws1 - ws0);
      auto step_of = [&](int k) { return ws0 + min(k, n - 1); };
      Regs ra, rb;
      load_step(step_of(0), ra);
      __builtin_amdgcn_sched_barrier(0);  // step 0's loads go out first, so waiting for them leaves step 1's in flight
      load_step(step_of(1), rb);
      // Steps go in pairs and both halves always store and load (an odd
      // count repeats the last step's data into an unread stage), so every
      // path round the loop issues the same memory operations and the waits
      // for a step's data stay two steps behind its loads.  The last pair is
      // peeled off the loop, which leaves the loop body without the test for
      // an odd count (measured: batch decode 63.9 -> 63.1 us).
      int k = 0;
      for (; k + 2 < n; k += 2) {
        store_step(step_of(k), ra, smem);
        load_step(step_of(k + 2), ra);
        __syncthreads();
        if (wave_ok) compute(step_of(k), smem);
        store_step(step_of(k + 1), rb, smem + Cfg::STAGE);
        load_step(step_of(k + 3), rb);
        __syncthreads();
        if (wave_ok) compute(step_of(k + 1), smem + Cfg::STAGE);
      }
      store_step(step_of(k), ra, smem);
      load_step(step_of(k + 2), ra);
      __syncthreads();
      if (wave_ok) compute(step_of(k), smem);
      store_step(step_of(k + 1), rb, smem + Cfg::STAGE);
      load_step(step_of(k + 3), rb);
      __syncthreads();
      if (wave_ok && k + 1 < n) compute(step_of(k + 1), smem + Cfg::STAGE);
    }

    // every wave writes its own rows
    if (chunk_id == 0 && tid == 0 && p.nch) p.nch[(int64_t)b * groups + grp] = nchunks;
    l_run = xor_sum(l_run, 16);
    l_run = xor_sum(l_run, 32);
    lr_run = xor_sum(lr_run, 16);
    lr_run = xor_sum(lr_run, 32);
    if (!row_ok) return;
    // a row without keys has sums of exactly 0; a NaN read from the cache
    // makes them NaN, which then carries into o and lse
    const float inv = has_weight(lr_run) ? 1.f / lr_run : 0.f;
    const float lse2 = has_weight(l_run) ? m_run + fast_log2(l_run) : kNegInf;
    if (nchunks == 1) {
      const float f = inv * p.v_scale;
      uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)b * p.num_qo_heads + h) * D + 4 * qg;
#pragma unroll
      for (int i = 0; i < Cfg::NDB; ++i)
        *reinterpret_cast<uint2*>(op + 16 * i) =
            make_uint2(pack2<OBF16>(acc[i][0] * f, acc[i][1] * f), pack2<OBF16>(acc[i][2] * f, acc[i][3] * f));
      if (p.lse && qg == 0) p.lse[(int64_t)b * p.num_qo_heads + h] = lse2 * kLn2;
    } else if (p.part_o && chunk_id < p.max_chunks) {
      const int64_t pidx = ((int64_t)b * p.num_qo_heads + h) * p.max_chunks + chunk_id;
      float* po = p.part_o + pidx * D + 4 * qg;
#pragma unroll
      for (int i = 0; i < Cfg::NDB; ++i) *reinterpret_cast<f32x4_t*>(po + 16 * i) = acc[i] * inv;
      if (qg == 0) p.part_lse[pidx] = lse2;
    }
  };

  if (!p.balanced) {
    // Fixed chunks: 1-D grid, chunk index fastest, then group, then request.
    const int chunk_id = bid % p.max_chunks;
    const int rem = bid / p.max_chunks;
    const int grp = rem % groups;
    const int b = rem / groups;
    const int kv_len = request_kv_len(p, b);
    // the host sizes the grid from its copy of the page table; clamping keeps a
    // workgroup inside the partial buffers even if the two copies disagree
    const int nchunks = min(p.max_chunks, max(1, (kv_len + p.chunk - 1) / p.chunk));
    if (chunk_id >= nchunks) return;
    const int t_begin = chunk_id * p.chunk;
    process(b, grp, t_begin, min(kv_len, t_begin + p.chunk), chunk_id, nchunks);
    return;
  }

  // Balanced slices: the (group, request, token) space of groups x T items
  // (T = total tokens) is cut into equal slices of p.slice items, one per
  // workgroup, so every workgroup streams the same number of bytes.  A slice
  // may cover the end of one request and the start of the next; each such
  // piece is a chunk of its (request, group) segment.
  int64_t* pre_lds = reinterpret_cast<int64_t*>(smem + Cfg::PREFIX);  // [batch + 1] token prefix sums
  if (p.pre_n == 0) {
    const int B = p.batch;
    const int per = (B + Cfg::NT - 1) / Cfg::NT;
    int64_t local = 0;
    for (int k = 0; k < per; ++k) {
      const int i = tid * per + k;
      if (i < B) local += request_kv_len(p, i);
    }
    int64_t v = local;  // inclusive scan over the workgroup
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t n = __shfl_up(v, o);
      if (lane >= o) v += n;
    }
    int64_t* wsum = reinterpret_cast<int64_t*>(smem + Cfg::WSUM);  // [NW]
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    for (int ww = 0; ww < w; ++ww) v += wsum[ww];
    int64_t run = v - local;  // exclusive prefix of this thread's first element
    for (int k = 0; k < per; ++k) {
      const int i = tid * per + k;
      if (i < B) {
        pre_lds[i] = run;
        run += request_kv_len(p, i);
      }
    }
    if (tid == 0) {
      int64_t tot = 0;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) tot += wsum[ww];
      pre_lds[B] = tot;
    }
    __syncthreads();
  }
  // every index below is uniform: with host prefix sums these are scalar
  // loads from the kernel arguments
  auto pre = [&](int i) -> int64_t { return p.pre_n ? (int64_t)p.pre[i] : pre_lds[i]; };
  const int64_t T = pre(p.batch);
  const int64_t W = T * groups;
  // requests without keys own no slice; their piece count 0 tells the merge
  // kernel to write o = 0 and lse = -inf
  if (p.nch)
    for (int i = bid; i < p.batch; i += nblocks)
      if (pre(i + 1) == pre(i))
        for (int k = tid; k < groups; k += Cfg::NT) p.nch[(int64_t)i * groups + k] = 0;
  if (p.spg > 0) {
    // Interleaved: each group's T tokens are cut into spg slices of its own and
    // workgroup w takes group w % groups, slice w / groups, so the workgroups
    // that read one token's kv head groups (its row's parts) run side by side.
    const int g = (int)(bid % groups);
    const int sl = (int)(bid / groups);
    int64_t t0 = (int64_t)sl * p.slice;
    const int64_t t1 = min(T, t0 + p.slice);
    while (t0 < t1) {
      int lo = 0, hi = p.batch;  // largest b with pre[b] <= t0
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre(mid) <= t0) lo = mid; else hi = mid;
      }
      const int b = lo;
      const int64_t seg0 = pre(b), seg1 = pre(b + 1);
      const int64_t end = min(seg1, t1);
      const int64_t s_first = seg0 / p.slice;
      const int nchunks = (int)((seg1 - 1) / p.slice - s_first + 1);
      process(b, g, (int)(t0 - seg0), (int)(end - seg0), (int)(sl - s_first), nchunks);
      t0 = end;
    }
    return;
  }
  int64_t x0 = (int64_t)bid * p.slice;
  const int64_t x1 = min(W, x0 + p.slice);
  while (x0 < x1) {
    const int grp = (int)(x0 / T);
    const int64_t pos = x0 - grp * T;
    int lo = 0, hi = p.batch;  // largest b with pre[b] <= pos (then pos < pre[b + 1])
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre(mid) <= pos) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int64_t seg0 = grp * T + pre(b);
    const int64_t seg1 = grp * T + pre(b + 1);
    const int64_t end = min(seg1, x1);
    const int64_t w_first = seg0 / p.slice;
    const int nchunks = (int)((seg1 - 1) / p.slice - w_first + 1);
    process(b, grp, (int)(pos - pre(b)), (int)(end - seg0), (int)(bid - w_first), nchunks);
    x0 = end;
  }
}

}  // namespace fi
