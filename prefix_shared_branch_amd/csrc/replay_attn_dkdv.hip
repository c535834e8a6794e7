// Replay attention backward, dK/dV part, on gfx950. The prompt-side gradient is the d l / d z_P
// term of the gradient decomposition in the LongStraw study notes (§2-2); serial replay adds it
// into resident accumulators response after response (§2-1 step 4, §3-2 (4)), and each
// accumulator element is owned by the prompt page it belongs to (§4-3 (2), page-owner dK/dV).
//
// With P = exp(S scale - LSE), dP = dO V^T, Delta = rowsum(dO * O), dS = P (dP - Delta):
//   dV_j += sum_rows P_rj dO_r,   dK_j += scale sum_rows dS_rj Q_r.
//
// replay_bwd_dkdv: key-tile owner. One workgroup = 4 waves x 32 keys of one kv head, one wave per
// SIMD; each wave keeps its keys' K and V fragments and its dK^T, dV^T accumulators in registers for
// the whole sweep over every query row that sees those keys, 32 GQA-packed rows per step. It serves
// the response keys and head dim 64; the prompt keys at head dim 128 (the long sweeps) run the
// 64-keys-per-wave form in replay_attn_dkdv64.hip, on the same packed rows. The rows were repacked per
// kv head before the launch (pack.hip): row-major Q and dO (A operands of S = Q K^T and
// dP = dO V^T) and dimension-major, slot-permuted Q^T and dO^T (A operands of dV^T += dO^T P and
// dK^T += Q^T dS, whose B operands come straight from the S / dP accumulators), plus each row's LSE
// and Delta as bf16 row terms (pack_rowext) that one 32x32x8 MFMA each turns into the starting
// values of the S and dP accumulators. Per step all of them stream global -> LDS by direct loads
// into a three-stage ring of XOR-swizzled tiles shared by the eight waves, so every MFMA operand is
// one 16-byte LDS read.
// The dV / dK products run in fp16 (11 significant bits; bf16's 8 would cost ~1.7e-3 relative error
// in the fp32 sums over 10^6-10^7 terms, fp16 ~2e-4) with exact power-of-two scaling so every
// operand sits in fp16's normal range: 2^15 P (folded into the exponent; dS is formed from the same
// fp16 2^15 P), dO s_dO and Q s_Q
// (s from max |dO|, max |Q|), and 2^15 P (dP - Delta) s_dS with s_dS from the bound
// |dP - Delta| <= 2 max_r |dO_r| max_j |V_j| (pack.hip computes the scales per call). Prompt keys:
// the sums are added to dKp / dVp in place (each element is read and written by exactly one
// workgroup per call). Response keys: causal, bf16 dKs / dVs stores.
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

template <int D, int DV, int NW_>
struct DkvCfg {
  static constexpr int NW = NW_;              // waves per workgroup (4: one per SIMD)
  static constexpr int BN = NW * 32;          // keys per workgroup (32 per wave)
  static constexpr int BR = 32;               // packed query rows per step
  static constexpr int QCH = D / 8;           // 16-byte chunks per Q row
  static constexpr int OCH = DV / 8;
  static constexpr int QROW = D * 2;
  static constexpr int OROW = DV * 2;
  static constexpr int TROW = BR * 2;         // bytes per packed Q^T / dO^T row of a step (32 slots)
  static constexpr int QBYTES = BR * QROW;
  static constexpr int OBYTES = BR * OROW;
  static constexpr int QTBYTES = D * TROW;
  static constexpr int OTBYTES = DV * TROW;
  static constexpr int LDBYTES = BR * 32;     // bf16 row terms of S and dP, 32 bytes per row
  static constexpr int OFF_O = QBYTES;
  static constexpr int OFF_QT = OFF_O + OBYTES;
  static constexpr int OFF_OT = OFF_QT + QTBYTES;
  static constexpr int OFF_LD = OFF_OT + OTBYTES;
  static constexpr int STAGE = OFF_LD + LDBYTES;
  static constexpr int NSTAGE = 4;
  // 1 KB direct loads of a step's Q, dO, Q^T and dO^T tiles, in that order, spread evenly over the
  // waves; each wave also loads a 256-byte quarter of the row terms
  static constexpr int QJ = QBYTES / 1024, OJ = OBYTES / 1024, QTJ = QTBYTES / 1024, OTJ = OTBYTES / 1024;
  static constexpr int NJOB = QJ + OJ + QTJ + OTJ;
  static constexpr int JPW = NJOB / NW;
  static_assert(NJOB % NW == 0 && LDBYTES == 4 * 256, "loads per wave");
  static constexpr int LPS = JPW + 1;         // direct loads per wave and step
  static constexpr int KS = D / 16;
  static constexpr int VS = DV / 16;
  static constexpr int DB = D / 32;
  static constexpr int VB = DV / 32;
};

// 4 waves, 128 keys per workgroup; the plan's key tiles match (attn_plan.cpp).
constexpr int kDkvWaves = 4;

template <int D, int DV, bool PROMPT>
__global__ __launch_bounds__(64 * kDkvWaves, 1) void replay_bwd_dkdv(BwdArgs a) {
  using C = DkvCfg<D, DV, kDkvWaves>;
  __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * C::STAGE];

  const AttnGeom& G = a.geo;
  const int nk = PROMPT ? a.ktiles_prompt : a.ktile0[G.n_resp];
  const int W = nk * G.Hkv;
  const int per_xcd = (W + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= W) return;
  const int kvh = w / nk;
  const int kt = w - kvh * nk;
  const int g = G.g;

  int key0, nkeys, tokb = 0, R = 0, ktokb = 0, qo = 0, row_begin, row_end;
  if (PROMPT) {
    key0 = kt * C::BN;
    nkeys = min(C::BN, G.P - key0);
    row_begin = 0;
    row_end = G.T * g;
  } else {
    int ri = 0;
    while (kt >= a.ktile0[ri + 1]) ++ri;
    tokb = G.tok0[ri];
    R = G.tok0[ri + 1] - tokb;
    ktokb = G.ktok0[ri];
    const int Rk = G.ktok0[ri + 1] - ktokb;  // response keys; query row t sits at key position t + qo
    qo = Rk - R;
    key0 = (kt - a.ktile0[ri]) * C::BN;  // within the response's keys
    nkeys = min(C::BN, Rk - key0);
    // the first row that sees key key0 sits at key position key0; steps start on 32-row
    // boundaries of the packed rows (the slot permutation of the packed Q^T / dO^T repeats every
    // 16 rows); rows of other responses are masked below
    row_begin = ((tokb + max(0, key0 - qo)) * g) & ~(C::BR - 1);
    row_end = (tokb + R) * g;
  }

  const int lane = threadIdx.x & 63;
  // wave index as a scalar: the load assignment below branches on it
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int mykey = wv * 32 + l32;  // within the tile
  const bool kvalid = mykey < nkeys;

  // K, V fragments of this wave's 32 keys (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[C::KS], vf[C::VS];
  {
    const uint16_t* kr = PROMPT ? G.Kp + (int64_t)(key0 + mykey) * G.ldk + kvh * D
                                : G.Ks + (int64_t)(ktokb + key0 + mykey) * G.ldk + kvh * D;
    const uint16_t* vr = PROMPT ? G.Vp + (int64_t)(key0 + mykey) * G.ldv + kvh * DV
                                : G.Vs + (int64_t)(ktokb + key0 + mykey) * G.ldv + kvh * DV;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kf[ks] = kvalid ? ld_bf16x8(kr + ks * 16 + hl * 8) : zero_bf16x8();
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) vf[ks] = kvalid ? ld_bf16x8(vr + ks * 16 + hl * 8) : zero_bf16x8();
  }

  f32x16 dk[C::DB], dv[C::VB];
#pragma unroll
  for (int b = 0; b < C::DB; ++b) dk[b] = f32x16{};
#pragma unroll
  for (int b = 0; b < C::VB; ++b) dv[b] = f32x16{};

  // Direct loads of a step go through buffer resources over this kv head's packed slabs (one base
  // per slab; the step moves the scalar offset, which stays inside the slab: the last step's rows
  // end at or before the slab's padded row count).
  const int64_t mpad = a.mpad;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(a.Qr + (int64_t)kvh * mpad * D, mpad * C::QROW);
  const __amdgpu_buffer_rsrc_t ro = buf_rsrc(a.dOr + (int64_t)kvh * mpad * DV, mpad * C::OROW);
  const __amdgpu_buffer_rsrc_t rqt = buf_rsrc(a.QT + (int64_t)kvh * D * mpad, (int64_t)D * mpad * 2);
  const __amdgpu_buffer_rsrc_t rot = buf_rsrc(a.dOT + (int64_t)kvh * DV * mpad, (int64_t)DV * mpad * 2);
  const __amdgpu_buffer_rsrc_t rld = buf_rsrc(a.rowstat + (int64_t)kvh * mpad * 8, mpad * 32);
  // load u of this wave's JPW 1 KB loads of the step at packed row m0 into stage buffer buf: job
  // j = u * NW + wv of the step's Q, dO, Q^T, dO^T tiles (row-major rows with XOR-swizzled chunks,
  // transposed rows of 32 slots). Each tile is a whole number of loads per wave, so the tile of load
  // u is known at compile time and the loop body has no branches (a branch there splits the loop into
  // blocks at whose joins the compiler copies the accumulators).
  static_assert(C::QJ % C::NW == 0 && C::OJ % C::NW == 0 && C::QTJ % C::NW == 0 && C::OTJ % C::NW == 0,
                "whole tiles per wave");
  auto issue_load = [&](int u, int m0, char* buf) {
    const int j0 = u * C::NW;  // compile-time: the tile of this load
    if (j0 < C::QJ) {
      const int jj = j0 + wv;
      const int row = jj * (64 / C::QCH) + lane / C::QCH;
      const uint32_t off = (uint32_t)(row * C::QROW + (((lane % C::QCH) ^ swz<C::QCH>(row)) << 4));
      lds_dma16_buf(rq, off, buf + jj * 1024, m0 * C::QROW);
    } else if (j0 < C::QJ + C::OJ) {
      const int jj = j0 - C::QJ + wv;
      const int row = jj * (64 / C::OCH) + lane / C::OCH;
      const uint32_t off = (uint32_t)(row * C::OROW + (((lane % C::OCH) ^ swz<C::OCH>(row)) << 4));
      lds_dma16_buf(ro, off, buf + C::OFF_O + jj * 1024, m0 * C::OROW);
    } else if (j0 < C::QJ + C::OJ + C::QTJ) {
      const int jj = j0 - C::QJ - C::OJ + wv;
      const int row = jj * 16 + (lane >> 2);
      const uint32_t off = (uint32_t)(row * mpad * 2 + (((lane & 3) ^ swz<4>(row)) << 4));
      lds_dma16_buf(rqt, off, buf + C::OFF_QT + jj * 1024, m0 * 2);
    } else {
      const int jj = j0 - C::QJ - C::OJ - C::QTJ + wv;
      const int row = jj * 16 + (lane >> 2);
      const uint32_t off = (uint32_t)(row * mpad * 2 + (((lane & 3) ^ swz<4>(row)) << 4));
      lds_dma16_buf(rot, off, buf + C::OFF_OT + jj * 1024, m0 * 2);
    }
  };
  auto issue_step = [&](int m0, char* buf) {
#pragma unroll
    for (int u = 0; u < C::JPW; ++u) issue_load(u, m0, buf);
    // row terms in dwords: wave wv loads the 256-byte quarter wv
    static_assert(C::NW == 4, "one row-term quarter per wave");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rld, (LSR_LDS void*)(buf + C::OFF_LD + wv * 256), 4, wv * 256 + lane * 4,
                                             m0 * 32, 0, 0);
  };

  const float c2 = G.scale_log2;
  const int nsteps = row_end > row_begin ? (row_end - row_begin + C::BR - 1) / C::BR : 0;
  const float s_ds = a.scales[2];  // fp16 scale of dS

  // Response keys: packed row m (token t = m / g - tokb, at key position t + qo) sees this lane's key
  // (position kp) iff 0 <= t < R and kp <= t + qo, i.e. iff m_lo <= m < m_hi with the bounds below;
  // rows of other responses see none of these keys.
  const int kp = key0 + mykey;
  const int m_lo = (tokb + max(0, kp - qo)) * g, m_hi = (tokb + R) * g;
  auto p_elem = [&](const f32x16& s, int r, int m0) {
    float pv = fast_exp2(s[r] * c2);
    if (!PROMPT) {
      const int m = m0 + 8 * (r >> 2) + 4 * hl + (r & 3);  // the packed row of register r
      pv = (m >= m_lo && m < m_hi) ? pv : 0.0f;
    }
    return pv;
  };
  // B operand of the row-term products: [1, 1, 1, 0] over k = 0..3 for every key, zero for k = 4..7
  const s16x4 ones = hl ? s16x4{0, 0, 0, 0} : s16x4{0x3F80, 0x3F80, 0x3F80, 0};
  // LDS byte offsets of a lane's fragments within a stage. Row-major tiles store logical 16-byte
  // chunk c of row r at chunk c ^ swz(r); the lane's fragment k (chunks 2k + hl of row l32) sits at
  // xb ^ (k << 5) with xb = row offset | ((hl ^ swz(l32)) << 4): the XOR touches bits 5..7 only, so
  // it commutes with adding the stage offset and the tile offsets (multiples of 1 KB). The packed
  // Q^T / dO^T tiles (64-byte rows of 32 slots) work the same way with k = the row half h.
  static_assert(C::STAGE % 1024 == 0 && C::OFF_O % 1024 == 0 && C::OFF_QT % 1024 == 0 && C::OFF_OT % 1024 == 0,
                "stage and tile offsets must not touch bits 5..7");
  const int qx0 = (l32 * C::QROW) | ((hl ^ swz<C::QCH>(l32)) << 4);
  const int ox0 = C::OFF_O + ((l32 * C::OROW) | ((hl ^ swz<C::OCH>(l32)) << 4));
  const int tx0 = (l32 * C::TROW) | ((hl ^ swz<4>(l32)) << 4);

  // One step: 32 packed rows against this wave's 32 keys, in two phases
  //   X:  S = row term + Q K^T;  2^15 P = exp2(c S)      (the row term holds -(LSE log2 e - 15) / c)
  //       dP - Delta = row term + dO V^T;  dS' = 2^15 P (dP - Delta) s_dS
  //   Y:  dV^T += dO^T (2^15 P),  dK^T += Q^T dS'         (fp16 operands)
  // X holds all of the step's VALU work, Y only MFMAs. Every MFMA takes one 16-byte LDS fragment,
  // read PD slots ahead (LDS latency under this load is several MFMAs long); a slot is one MFMA with
  // its read, fenced so the compiler keeps the reads (and their registers) where they are written.
  // Y reads the same stage as X, so its first fragments are read during X's last slots, across the
  // barrier between the phases.
  constexpr int NQ = C::KS, NO = C::VS, NOT = 2 * C::VB, NQT = 2 * C::DB;
  constexpr int NX = NQ + NO, NF = NX + NOT + NQT;
  constexpr int PD = 2;

  // Four-stage ring; every phase starts at a workgroup barrier:
  //  * each wave waits for its own loads of step j + 1 at the end of its X(j) (loads of steps j + 1
  //    and j + 2 in flight), so step j + 1's tiles are complete at the barrier before X(j + 1);
  //  * a wave issues its loads of step j + 3 at the barrier before Y(j), into the stage of step
  //    j - 1, which every wave has finished reading by then (each wave's reads of a stage have
  //    returned before the barrier that precedes its next X).
  // Past the last step the last step's rows are loaded again, so every step issues the same number
  // of loads and the wait count is fixed.
  auto stage = [&](int j) { return smem + (j & 3) * C::STAGE; };
  auto mrow = [&](int t) { return row_begin + min(t, nsteps - 1) * C::BR; };

  auto step = [&](int j) {
    const char* buf = stage(j);
    const int m0 = row_begin + j * C::BR;
    // per-step fragment bases (the opaque copy keeps them from being hoisted out of the loop as one
    // live register per fragment)
    int qx = qx0, ox = ox0, tx = tx0;
    asm volatile("" : "+v"(qx), "+v"(ox), "+v"(tx));
    const int stg = (int)(buf - smem);
    qx += stg;
    ox += stg;
    tx += stg;
    const int tx1 = tx ^ 32;
    auto rd = [&](int i) {
      int off;
      if (i < NQ) off = qx ^ (i << 5);
      else if (i < NX) off = ox ^ ((i - NQ) << 5);
      else if (i < NX + NOT) {
        const int k = i - NX, h = k / C::VB, b = k % C::VB;
        off = (h ? tx1 : tx) + C::OFF_OT + b * 32 * C::TROW;
      } else {
        const int k = i - NX - NOT, h = k / C::DB, b = k % C::DB;
        off = (h ? tx1 : tx) + C::OFF_QT + b * 32 * C::TROW;
      }
      return __builtin_bit_cast(u32x4, lds_b128_at(smem, off));
    };
    u32x4 fr[NF];
    const s16x4 xq = lds_s16x4_at(buf, C::OFF_LD + hl * 256 + l32 * 8);
#pragma unroll
    for (int i = 0; i < PD; ++i) fr[i] = rd(i);
    f32x16 s = mfma32x8(xq, ones, f32x16{}), dp;
    f16x8 h0, h1, d0, d1;  // fp16 2^15 P and dS'
    s16x4 xo;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      if (i == NX) {
        // between the phases: own loads of step j + 1 complete, then the barrier before Y(j), then
        // this wave's loads of step j + 3 into the stage of step j - 1
        wait_vmem_le<C::LPS>();
        bare_barrier();
        issue_step(mrow(j + 3), stage(j + 3));
      }
      if (i + PD < NF) fr[i + PD] = rd(i + PD);
      if (i == NQ - 1) xo = lds_s16x4_at(buf, C::OFF_LD + 512 + hl * 256 + l32 * 8);
      if (i < NQ) {
        s = mfma32(__builtin_bit_cast(bf16x8, fr[i]), kf[i], s);
        if (i == NQ - 1) {
          // 2^15 P, kept in fp16 only (the B operand of the dV products; dS' below is formed from it)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = p_elem(s, r, m0);
          h0 = c_regs_to_f16x8(s, 0);
          h1 = c_regs_to_f16x8(s, 8);
        }
      } else if (i < NX) {
        if (i == NQ) dp = mfma32x8(xo, ones, f32x16{});
        dp = mfma32(__builtin_bit_cast(bf16x8, fr[i]), vf[i - NQ], dp);
        if (i == NX - 1) {
          // dS' = 2^15 P (dP - Delta) s_dS in place of dP, from the fp16 2^15 P: its halves are
          // unpacked here from the packed operand (the opaque copy keeps the compiler from holding a
          // second, unpacked copy of P since the exponentials)
          u32x4 hu0 = __builtin_bit_cast(u32x4, h0), hu1 = __builtin_bit_cast(u32x4, h1);
          asm volatile("" : "+v"(hu0), "+v"(hu1));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t u = r < 8 ? hu0[(r & 7) >> 1] : hu1[(r & 7) >> 1];
            const float pv = (float)__builtin_bit_cast(_Float16, (uint16_t)((r & 1) ? (u >> 16) : (u & 0xffffu)));
            dp[r] = pv * (dp[r] * s_ds);
          }
          h0 = __builtin_bit_cast(f16x8, hu0);
          h1 = __builtin_bit_cast(f16x8, hu1);
          d0 = c_regs_to_f16x8(dp, 0);
          d1 = c_regs_to_f16x8(dp, 8);
        }
      } else if (i < NX + NOT) {
        const int k = i - NX, h = k / C::VB, b = k % C::VB;
        dv[b] = mfma32h(__builtin_bit_cast(f16x8, fr[i]), h ? h1 : h0, dv[b]);
      } else {
        const int k = i - NX - NOT, h = k / C::DB, b = k % C::DB;
        dk[b] = mfma32h(__builtin_bit_cast(f16x8, fr[i]), h ? d1 : d0, dk[b]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nsteps > 0) {
    issue_step(mrow(0), stage(0));
    issue_step(mrow(1), stage(1));
    issue_step(mrow(2), stage(2));
    wait_vmem_le<2 * C::LPS>();  // own loads of step 0
  }
  for (int j = 0; j < nsteps; ++j) {
    wait_lds();      // this wave's reads of the previous stage have returned
    bare_barrier();  // before X(j); no fence: it would wait for every direct load in flight
    step(j);
  }
  // no direct load may still be writing into LDS when the waves end
  wait_vmem();

  if (!kvalid) return;
  // C layout of dV^T / dK^T: lane holds key (lane & 31), dims 32b + 8(r/4) + 4hl + r%4.
  // Undo the operand scales: dV = sum / (2^15 s_dO), dK = scale * sum / (2^15 s_dS s_Q).
  const float fv = 0x1p-15f / a.scales[0];
  const float sc = G.scale * 0x1p-15f / (s_ds * a.scales[1]);
  if (PROMPT) {
    float* dvr = a.dVp + ((int64_t)(key0 + mykey) * G.Hkv + kvh) * DV + 4 * hl;
    float* dkr = a.dKp + ((int64_t)(key0 + mykey) * G.Hkv + kvh) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::VB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4* ptr = reinterpret_cast<f32x4*>(dvr + b * 32 + 8 * q);
        const f32x4 add = {dv[b][4 * q] * fv, dv[b][4 * q + 1] * fv, dv[b][4 * q + 2] * fv, dv[b][4 * q + 3] * fv};
        *ptr = *ptr + add;
      }
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4* ptr = reinterpret_cast<f32x4*>(dkr + b * 32 + 8 * q);
        const f32x4 add = {dk[b][4 * q] * sc, dk[b][4 * q + 1] * sc, dk[b][4 * q + 2] * sc, dk[b][4 * q + 3] * sc};
        *ptr = *ptr + add;
      }
  } else if (a.dKs_acc) {
    // blocks of one response: fp32 sums added into the response-key accumulators
    const int64_t tok = ktokb + key0 + mykey;
    float* dvr = a.dVs_acc + (tok * G.Hkv + kvh) * DV + 4 * hl;
    float* dkr = a.dKs_acc + (tok * G.Hkv + kvh) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::VB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4* ptr = reinterpret_cast<f32x4*>(dvr + b * 32 + 8 * q);
        const f32x4 add = {dv[b][4 * q] * fv, dv[b][4 * q + 1] * fv, dv[b][4 * q + 2] * fv, dv[b][4 * q + 3] * fv};
        *ptr = *ptr + add;
      }
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4* ptr = reinterpret_cast<f32x4*>(dkr + b * 32 + 8 * q);
        const f32x4 add = {dk[b][4 * q] * sc, dk[b][4 * q + 1] * sc, dk[b][4 * q + 2] * sc, dk[b][4 * q + 3] * sc};
        *ptr = *ptr + add;
      }
  } else {
    const int64_t tok = ktokb + key0 + mykey;
    uint16_t* dvr = a.dVs + (tok * G.Hkv + kvh) * DV + 4 * hl;
    uint16_t* dkr = a.dKs + (tok * G.Hkv + kvh) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::VB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v = {pack_bf16x2(dv[b][4 * q] * fv, dv[b][4 * q + 1] * fv),
                         pack_bf16x2(dv[b][4 * q + 2] * fv, dv[b][4 * q + 3] * fv)};
        *reinterpret_cast<u32x2*>(dvr + b * 32 + 8 * q) = v;
      }
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v = {pack_bf16x2(dk[b][4 * q] * sc, dk[b][4 * q + 1] * sc),
                         pack_bf16x2(dk[b][4 * q + 2] * sc, dk[b][4 * q + 3] * sc)};
        *reinterpret_cast<u32x2*>(dkr + b * 32 + 8 * q) = v;
      }
  }
}

template <int D, int DV>
hipError_t dkdv_go(BwdArgs& a, hipStream_t st) {
  const AttnGeom& G = a.geo;
  hipError_t e;
  // fp16 operand scales of this call
  ScaleArgs sa;
  sa.dO = a.dO;
  sa.Q = G.Q;
  sa.Vp = G.Vp;
  sa.Vs = G.Vs;
  sa.ldv = G.ldv;
  sa.T = G.T;
  sa.Tk = G.Tk;
  sa.P = G.P;
  sa.Hq = G.Hq;
  sa.Hkv = G.Hkv;
  sa.Dqk = D;
  sa.Dv = DV;
  sa.partial = a.scale_part;
  sa.scales = a.scales;
  if ((e = launch_bwd_scales(sa, st)) != hipSuccess) return e;
  // packed query rows of every kv head: row-major Q / dO (bf16), dimension-major Q^T / dO^T (fp16,
  // scaled), statistics
  const int64_t M = (int64_t)G.T * G.g;
  PackArgs p;
  p.f16_scale = nullptr;
  p.ld = (int64_t)G.Hq * D;
  p.grp = G.g;
  p.gstride = D;
  p.hstride = (int64_t)G.g * D;
  p.dim = D;
  p.heads = G.Hkv;
  p.nseg = 1;
  p.row0[0] = 0;
  p.n[0] = (int32_t)M;
  p.col0[0] = 0;
  p.out_ld = a.mpad;
  p.cols = a.mpad;
  p.src = G.Q;
  p.out = a.Qr;
  if ((e = launch_pack_rows(p, st)) != hipSuccess) return e;
  p.out = a.QT;
  p.f16_scale = a.scales + 1;
  if ((e = launch_pack_keys_t(p, st)) != hipSuccess) return e;
  p.f16_scale = nullptr;
  p.ld = (int64_t)G.Hq * DV;
  p.gstride = DV;
  p.hstride = (int64_t)G.g * DV;
  p.dim = DV;
  p.src = a.dO;
  p.out = a.dOr;
  if ((e = launch_pack_rows(p, st)) != hipSuccess) return e;
  p.out = a.dOT;
  p.f16_scale = a.scales + 0;
  if ((e = launch_pack_keys_t(p, st)) != hipSuccess) return e;
  RowStatArgs r;
  r.c2 = G.scale_log2;
  r.lse = a.lse;
  r.delta = a.delta;
  r.scales = a.scales;
  r.out = a.rowstat;
  r.T = G.T;
  r.Hq = G.Hq;
  r.g = G.g;
  r.Hkv = G.Hkv;
  r.M = M;
  r.mpad = a.mpad;
  if ((e = launch_pack_rowext(r, st)) != hipSuccess) return e;

  if (a.ktiles_prompt > 0) {
    const long long W = (long long)a.ktiles_prompt * G.Hkv;
    timer_mark(LS_KERNEL_DKDV_PROMPT, st, false);
    if constexpr (D == 128) {
      e = launch_dkdv_prompt_w64(a, st);
    } else {
      hipLaunchKernelGGL((replay_bwd_dkdv<D, DV, true>), dim3((unsigned)(((W + 7) / 8) * 8)), dim3(64 * kDkvWaves),
                         0, st, a);
      e = hipGetLastError();
    }
    timer_mark(LS_KERNEL_DKDV_PROMPT, st, true);
    if (e != hipSuccess) return e;
  }
  const long long W = (long long)a.ktile0[G.n_resp] * G.Hkv;
  if (W > 0) {
    hipLaunchKernelGGL((replay_bwd_dkdv<D, DV, false>), dim3((unsigned)(((W + 7) / 8) * 8)), dim3(64 * kDkvWaves), 0,
                       st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_dkdv(BwdArgs& a, int Dqk, int Dv, hipStream_t st) {
  if (Dqk == kWideDqk && Dv == kWideDv) return launch_bwd_dkdv_wide(a, st);
  if (Dqk == 64 && Dv == 64) return dkdv_go<64, 64>(a, st);
  if (Dqk == 128 && Dv == 128) return dkdv_go<128, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lsr
