// Replay attention backward, dK/dV of the prompt keys at head dim 128, 64 keys per wave (gfx950).
// The prompt-side gradient is the d l / d z_P term of the gradient decomposition in the LongStraw
// study notes (§2-2), added into resident accumulators response after response (§2-1 step 4,
// §3-2 (4)) by the owner of each prompt page (§4-3 (2)).
//
// With P = exp(S scale - LSE), dP = dO V^T, Delta = rowsum(dO * O), dS = P (dP - Delta):
//   dV_j += sum_rows P_rj dO_r,   dK_j += scale sum_rows dS_rj Q_r.
//
// replay_bwd_dkdv_w64: one workgroup = 4 waves x 64 keys = 256 keys of one kv head, one wave per
// SIMD. A wave's keys are two 32-key blocks, and every 16-byte LDS fragment of the streamed rows
// (row-major Q and dO, packed Q^T and dO^T, the same tiles and ring as the 32-key kernel in
// replay_attn_dkdv.hip) feeds one MFMA per block: half the LDS bytes per MFMA of the 32-key form.
// The price is the register file: the K and V fragments of 64 keys take 128 registers and the
// dK^T, dV^T accumulators 256 of the 512 (VGPRs and AGPRs) a lane has, so a SIMD holds one wave, and
// its VALU work (P, dS) is interleaved with its own MFMAs rather than with another wave's. Per
// 32-row step and wave:
//   S = row term + Q K^T (two 32x32 tiles), 2^15 P = exp2(c S) as fp16 B operands;
//   (dP - Delta) s_dS = row term + dO (s_dS V)^T, dS' = 2^15 P (dP - Delta) s_dS from the fp16 P;
//   dV^T += dO^T (2^15 P), dK^T += Q^T dS' (fp16, exact power-of-two operand scales).
// Operand layouts, scales, row terms and accumulator updates are those of the 32-key kernel, whose
// results this kernel reproduces bit for bit (s_dS is a power of two, so folding it into V and the
// row term's operand changes no rounding).
#include <utility>

#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{}): a loop whose index
// is a constant expression in the body
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// first element of half-slot hs in a window of 32 elements spread evenly over hn half-slots from h0
constexpr int win_lo(int hs, int h0, int hn) {
  return hs < h0 ? 0 : (hs >= h0 + hn ? 32 : ((hs - h0) * 32 + hn - 1) / hn);
}

struct W64Cfg {
  static constexpr int D = 128, DV = 128;
  static constexpr int NW = 4;                // waves per workgroup, one per SIMD
  static constexpr int KPW = 64;              // keys per wave: two 32-key blocks
  static constexpr int BN = NW * KPW;         // keys per workgroup
  static constexpr int BR = 32;               // packed query rows per step
  static constexpr int QCH = D / 8, OCH = DV / 8;
  static constexpr int QROW = D * 2, OROW = DV * 2;
  static constexpr int TROW = BR * 2;         // bytes per packed Q^T / dO^T row of a step
  static constexpr int QBYTES = BR * QROW, OBYTES = BR * OROW;
  static constexpr int QTBYTES = D * TROW, OTBYTES = DV * TROW;
  static constexpr int LDBYTES = BR * 32;     // bf16 row terms of S and dP
  static constexpr int OFF_O = QBYTES;
  static constexpr int OFF_QT = OFF_O + OBYTES;
  static constexpr int OFF_OT = OFF_QT + QTBYTES;
  static constexpr int OFF_LD = OFF_OT + OTBYTES;
  static constexpr int STAGE = OFF_LD + LDBYTES;
  static constexpr int NSTAGE = 4;
  static constexpr int QJ = QBYTES / 1024, OJ = OBYTES / 1024, QTJ = QTBYTES / 1024, OTJ = OTBYTES / 1024;
  static constexpr int NJOB = QJ + OJ + QTJ + OTJ;
  static constexpr int JPW = NJOB / NW;
  static_assert(NJOB % NW == 0 && LDBYTES == 4 * 256, "loads per wave");
  static constexpr int LPS = JPW + 1;         // direct loads per wave and step (tiles, row-term quarter)
  static constexpr int KS = D / 16, VS = DV / 16;
  static constexpr int DB = D / 32, VB = DV / 32;
};

__global__ __launch_bounds__(64 * W64Cfg::NW, 1) void replay_bwd_dkdv_w64(BwdArgs a) {
  using C = W64Cfg;
  constexpr int D = C::D, DV = C::DV;
  __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * C::STAGE];

  const AttnGeom& G = a.geo;
  const int nk = a.ktiles_prompt;
  const int W = nk * G.Hkv;
  const int per_xcd = (W + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= W) return;
  const int kvh = w / nk;
  const int kt = w - kvh * nk;
  const int g = G.g;
  const int key0 = kt * C::BN;
  const int nkeys = min(C::BN, G.P - key0);
  const int row_begin = 0, row_end = G.T * g;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  // this lane's key in block kb: wv * 64 + 32 kb + l32 (within the tile)
  auto mykey = [&](int kb) { return wv * C::KPW + 32 * kb + l32; };

  // K, V fragments of the wave's 64 keys (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[2][C::KS], vf[2][C::VS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const bool ok = mykey(kb) < nkeys;
    const uint16_t* kr = G.Kp + (int64_t)(key0 + mykey(kb)) * G.ldk + kvh * D;
    const uint16_t* vr = G.Vp + (int64_t)(key0 + mykey(kb)) * G.ldv + kvh * DV;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kf[kb][ks] = ok ? ld_bf16x8(kr + ks * 16 + hl * 8) : zero_bf16x8();
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) vf[kb][ks] = ok ? ld_bf16x8(vr + ks * 16 + hl * 8) : zero_bf16x8();
  }

  f32x16 dk[2][C::DB], dv[2][C::VB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int b = 0; b < C::DB; ++b) dk[kb][b] = f32x16{};
#pragma unroll
    for (int b = 0; b < C::VB; ++b) dv[kb][b] = f32x16{};
  }

  // Direct loads of a step through buffer resources over this kv head's packed slabs (the scalar
  // offset moves per step and stays inside the slab)
  const int64_t mpad = a.mpad;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(a.Qr + (int64_t)kvh * mpad * D, mpad * C::QROW);
  const __amdgpu_buffer_rsrc_t ro = buf_rsrc(a.dOr + (int64_t)kvh * mpad * DV, mpad * C::OROW);
  const __amdgpu_buffer_rsrc_t rqt = buf_rsrc(a.QT + (int64_t)kvh * D * mpad, (int64_t)D * mpad * 2);
  const __amdgpu_buffer_rsrc_t rot = buf_rsrc(a.dOT + (int64_t)kvh * DV * mpad, (int64_t)DV * mpad * 2);
  const __amdgpu_buffer_rsrc_t rld = buf_rsrc(a.rowstat + (int64_t)kvh * mpad * 8, mpad * 32);
  // load u of this wave's JPW 1 KB loads of the step at packed row m0: job jj = u * NW + wv of the
  // Q, dO, Q^T, dO^T tiles in that order (two loads per tile and wave; the tile of load u is a
  // compile-time constant). The lane part of the offset is the same for both loads of a tile and for
  // Q and dO (rows of 16 chunks, jj % 4 = wv fixes the swizzle) and for Q^T and dO^T (rows of four
  // chunks, swizzled by lane / 16 alone); the load's own part goes to the scalar offset.
  static_assert(C::QJ == 2 * C::NW && C::OJ == 2 * C::NW && C::QTJ == 2 * C::NW && C::OTJ == 2 * C::NW &&
                C::QCH == 16 && C::OCH == 16, "two loads per tile and wave");
  const uint32_t voff_rm = (uint32_t)((wv * 4 + (lane >> 4)) * C::QROW +
                                      (((lane & 15) ^ swz<16>(wv * 4 + (lane >> 4))) << 4));
  const uint32_t voff_tr = (uint32_t)((lane >> 2) * mpad * 2 + (((lane & 3) ^ swz<4>(lane >> 2)) << 4));
  auto issue_load = [&](int u, int m0, char* buf) {
    const int t = u >> 1, half = u & 1;  // tile, which of its two loads
    const int jj = half * C::NW + wv;
    if (t == 0) lds_dma16_buf(rq, voff_rm, buf + jj * 1024, m0 * C::QROW + half * 16 * C::QROW);
    else if (t == 1) lds_dma16_buf(ro, voff_rm, buf + C::OFF_O + jj * 1024, m0 * C::OROW + half * 16 * C::OROW);
    else if (t == 2)
      lds_dma16_buf(rqt, voff_tr, buf + C::OFF_QT + jj * 1024, m0 * 2 + (half * C::NW + wv) * 16 * (int)mpad * 2);
    else
      lds_dma16_buf(rot, voff_tr, buf + C::OFF_OT + jj * 1024, m0 * 2 + (half * C::NW + wv) * 16 * (int)mpad * 2);
  };
  auto issue_step = [&](int m0, char* buf) {
#pragma unroll
    for (int u = 0; u < C::JPW; ++u) issue_load(u, m0, buf);
    // row terms in dwords: wave wv loads the 256-byte quarter wv
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rld, (LSR_LDS void*)(buf + C::OFF_LD + wv * 256), 4, wv * 256 + lane * 4,
                                             m0 * 32, 0, 0);
  };

  const float c2 = G.scale_log2;
  const int nsteps = row_end > row_begin ? (row_end - row_begin + C::BR - 1) / C::BR : 0;
  const float s_ds = a.scales[2];  // fp16 scale of dS: a power of two
  // B operands of the row-term products: [1, 1, 1, 0] over k = 0..3 for every key, zero for k = 4..7;
  // for dP the same with s_dS in place of 1 (exact), so that the dP tile comes out as
  // (dP - Delta) s_dS
  const s16x4 ones = hl ? s16x4{0, 0, 0, 0} : s16x4{0x3F80, 0x3F80, 0x3F80, 0};
  const short sd16 = (short)(__float_as_uint(s_ds) >> 16);
  const s16x4 ones_ds = hl ? s16x4{0, 0, 0, 0} : s16x4{sd16, sd16, sd16, 0};
  // V fragments times s_dS (a power of two: exact in bf16 within its exponent range)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) {
      u32x4 u = __builtin_bit_cast(u32x4, vf[kb][ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        u[e] = (__float_as_uint(bf16_lo(u[e]) * s_ds) >> 16) | (__float_as_uint(bf16_hi(u[e]) * s_ds) & 0xffff0000u);
      vf[kb][ks] = __builtin_bit_cast(bf16x8, u);
    }
  // V fragments are MFMA operands only: start them in AGPRs (an empty asm with an AGPR constraint). With
  // 512 registers per lane split between the accumulators, the K and V fragments and the step's S /
  // dP tiles and VALU work, this hint is what lets the register allocator keep the loop free of
  // copies between the two register files and of spills (checked in the generated code)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) asm volatile("" : "+a"(vf[kb][ks]));
  // lane fragment offsets within a stage: fragment k of a row-major tile at xb ^ (k << 5) (the
  // swizzle touches bits 5..7 only, which commute with the stage and tile offsets)
  static_assert(C::STAGE % 1024 == 0 && C::OFF_O % 1024 == 0 && C::OFF_QT % 1024 == 0 && C::OFF_OT % 1024 == 0,
                "stage and tile offsets must not touch bits 5..7");
  const int qx0 = (l32 * C::QROW) | ((hl ^ swz<C::QCH>(l32)) << 4);
  const int ox0 = C::OFF_O + ((l32 * C::OROW) | ((hl ^ swz<C::OCH>(l32)) << 4));
  const int tx0 = (l32 * C::TROW) | ((hl ^ swz<4>(l32)) << 4);

  // Slots of a step: one 16-byte fragment each, feeding one MFMA per key block:
  //   S:  Q fragments        s[kb]  += Q K^T        (started from the S row term)
  //   dP: dO fragments       dp[kb] += dO (s_dS V)^T (started from the scaled Delta row term)
  //   dV: dO^T fragments     dv[kb] += dO^T (2^15 P)
  //   dK: Q^T fragments      dk[kb] += Q^T dS'
  // A slot runs as MFMA (block 0), VALU half, MFMA (block 1), VALU half: with one wave per SIMD the
  // VALU work of the step (2^15 P = exp2(c S) to fp16, dS' = 2^15 P (dP - Delta) s_dS to fp16) is
  // issued while the matrix unit works on the slot's MFMAs. P elements are spread over the dP slots
  // and the first half of the dV slots (register halves h = 0 first: the first dV slots read them),
  // dS' elements over the second half of the dV slots and the first half of the dK slots. Fragments
  // are read PD slots ahead; the last PD slots of step j read the first fragments of step j + 1, after
  // the barrier that publishes them, and the last slot starts step j + 1's S tile from its row term.
  constexpr int NQ = C::KS, NO = C::VS, NOT = 2 * C::VB, NQT = 2 * C::DB;
  constexpr int NX = NQ + NO, NF = NX + NOT + NQT;
  constexpr int PD = 2;
  static_assert(NQ >= PD && NOT == 8 && NQT == 8, "slot plan for head dim 128");
  // half-slot windows (half-slot 2 i + half of slot i) of the VALU work; element e of a window is
  // register half h = e / 16, block kb = (e / 8) % 2, register 8 h + e % 8 of that block's tile
  constexpr int P_H0 = 2 * NQ, P_HN = 2 * (NOT / 2 + NO);       // dP slots + first half of dV
  constexpr int D_H0 = 2 * (NX + NOT / 2), D_HN = 2 * (NOT / 2 + NQT / 2);
  auto stage = [&](int j) { return smem + (j & 3) * C::STAGE; };
  auto mrow = [&](int t) { return row_begin + min(t, nsteps - 1) * C::BR; };

  // Four-stage ring: steps 0-2 are loaded up front; at slot NF - PD of step j each wave waits for its
  // own loads of step j + 1 (those of step j + 2 may still be in flight), passes a workgroup barrier
  // (every wave has finished its reads of step j - 1 and published step j + 1) and issues its loads
  // of step j + 3 into the stage of step j - 1. Past the last step the last step's rows are loaded
  // again, so every step issues the same number of loads and the waits are fixed.
  u32x4 fr[NF];
  f32x16 s_init;
  if (nsteps > 0) {
    issue_step(mrow(0), stage(0));
    issue_step(mrow(1), stage(1));
    issue_step(mrow(2), stage(2));
    wait_vmem_le<2 * C::LPS>();  // own loads of step 0
    bare_barrier();
    int qx = qx0;
    asm volatile("" : "+v"(qx));
#pragma unroll
    for (int i = 0; i < PD; ++i) fr[i] = __builtin_bit_cast(u32x4, lds_b128_at(smem, qx ^ (i << 5)));
    s_init = mfma32x8(lds_s16x4_at(smem, C::OFF_LD + hl * 256 + l32 * 8), ones, f32x16{});
  }
  for (int j = 0; j < nsteps; ++j) {
    const int stg = (int)(stage(j) - smem);
    const int dn = (int)(stage(j + 1) - smem) - stg;  // to the next step's stage
    // per-step fragment bases (an opaque copy keeps them from being hoisted as one register per
    // fragment)
    int qx = qx0, ox = ox0, tx = tx0;
    asm volatile("" : "+v"(qx), "+v"(ox), "+v"(tx));
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
    f32x16 s[2], dp[2], dp_init;
    uint32_t hw[2][2][4], dw[2][2][4];  // fp16 pairs of 2^15 P and dS': [block][register half][word]
    float pend[2], dend[2];               // the even element of a pair, until its odd partner is formed
    s16x4 xo, xq;
    // VALU work of half-slot hs: P elements [win_lo(hs), win_lo(hs + 1)) of the P window, then dS'
    // elements of the dS' window
    auto valu = [&](auto hsc) {
      constexpr int hs = decltype(hsc)::value;
      static_for<32>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        constexpr int h = e >> 4, kb = (e >> 3) & 1, r = 8 * h + (e & 7);
        if constexpr (e >= win_lo(hs, P_H0, P_HN) && e < win_lo(hs + 1, P_H0, P_HN)) {
          const float pv = fast_exp2(s[kb][r] * c2);
          if constexpr (r & 1) {
            f16x2 x;
            x[0] = (_Float16)pend[kb];
            x[1] = (_Float16)pv;
            hw[kb][h][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, x);
          } else {
            pend[kb] = pv;
          }
        }
        if constexpr (e >= win_lo(hs, D_H0, D_HN) && e < win_lo(hs + 1, D_H0, D_HN)) {
          const uint32_t u = hw[kb][h][(r & 7) >> 1];
          const float pv = (float)__builtin_bit_cast(_Float16, (uint16_t)((r & 1) ? (u >> 16) : (u & 0xffffu)));
          const float dv_ = pv * dp[kb][r];
          if constexpr (r & 1) {
            f16x2 x;
            x[0] = (_Float16)dend[kb];
            x[1] = (_Float16)dv_;
            dw[kb][h][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, x);
          } else {
            dend[kb] = dv_;
          }
        }
      });
    };
    auto h16 = [](const uint32_t* w) { return __builtin_bit_cast(f16x8, u32x4{w[0], w[1], w[2], w[3]}); };
    static_for<NF>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (i == NF - PD) {
        wait_vmem_le<C::LPS>();
        bare_barrier();
        issue_step(mrow(j + 3), stage(j + 3));
      }
      if constexpr (i == D_H0 / 2) {
        // dS' is formed from the packed fp16 2^15 P: the opaque in-place redefinition keeps the compiler
        // from holding an unpacked fp16 copy of every P element since the exponentials
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            asm volatile("" : "+v"(hw[kb][h][0]), "+v"(hw[kb][h][1]), "+v"(hw[kb][h][2]), "+v"(hw[kb][h][3]));
      }
      if (i == 0) xo = lds_s16x4_at(smem, stg + C::OFF_LD + 512 + hl * 256 + l32 * 8);
      if (i == NF - PD) xq = lds_s16x4_at(smem, stg + dn + C::OFF_LD + hl * 256 + l32 * 8);
      // MFMA of block 0
      if (i < NQ) s[0] = mfma32(__builtin_bit_cast(bf16x8, fr[i]), kf[0][i], i == 0 ? s_init : s[0]);
      else if (i < NX) dp[0] = mfma32(__builtin_bit_cast(bf16x8, fr[i]), vf[0][i - NQ], i == NQ ? dp_init : dp[0]);
      else if (i < NX + NOT) {
        const int k = i - NX, h = k / C::VB, b = k % C::VB;
        dv[0][b] = mfma32h(__builtin_bit_cast(f16x8, fr[i]), h16(hw[0][h]), dv[0][b]);
      } else {
        const int k = i - NX - NOT, h = k / C::DB, b = k % C::DB;
        dk[0][b] = mfma32h(__builtin_bit_cast(f16x8, fr[i]), h16(dw[0][h]), dk[0][b]);
      }
      __builtin_amdgcn_sched_barrier(0);
      valu(std::integral_constant<int, 2 * i>{});
      __builtin_amdgcn_sched_barrier(0);
      // MFMA of block 1
      if (i < NQ) s[1] = mfma32(__builtin_bit_cast(bf16x8, fr[i]), kf[1][i], i == 0 ? s_init : s[1]);
      else if (i < NX) dp[1] = mfma32(__builtin_bit_cast(bf16x8, fr[i]), vf[1][i - NQ], i == NQ ? dp_init : dp[1]);
      else if (i < NX + NOT) {
        const int k = i - NX, h = k / C::VB, b = k % C::VB;
        dv[1][b] = mfma32h(__builtin_bit_cast(f16x8, fr[i]), h16(hw[1][h]), dv[1][b]);
      } else {
        const int k = i - NX - NOT, h = k / C::DB, b = k % C::DB;
        dk[1][b] = mfma32h(__builtin_bit_cast(f16x8, fr[i]), h16(dw[1][h]), dk[1][b]);
      }
      // row terms: the dP tile's start for this step, the S tile's start for the next step
      if (i == 2) dp_init = mfma32x8(xo, ones_ds, f32x16{});
      if (i == NF - 1) s_init = mfma32x8(xq, ones, f32x16{});
      // the slot's fragment register is free once its second MFMA has issued: read the fragment of
      // slot i + PD into it (the next step's first fragments at the step's end)
      __builtin_amdgcn_sched_barrier(0);
      if (i + PD < NF) fr[i + PD] = rd(i + PD);
      else fr[i + PD - NF] = __builtin_bit_cast(u32x4, lds_b128_at(smem, (qx + dn) ^ ((i + PD - NF) << 5)));
      __builtin_amdgcn_sched_barrier(0);
      valu(std::integral_constant<int, 2 * i + 1>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  // no direct load may still be writing into LDS when the waves end
  wait_vmem();

  // C layout of dV^T / dK^T: lane holds key (lane & 31) of block kb, dims 32b + 8(r/4) + 4hl + r%4.
  // Undo the operand scales: dV = sum / (2^15 s_dO), dK = scale * sum / (2^15 s_dS s_Q).
  const float fv = 0x1p-15f / a.scales[0];
  const float sc = G.scale * 0x1p-15f / (s_ds * a.scales[1]);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (mykey(kb) >= nkeys) continue;
    float* dvr = a.dVp + ((int64_t)(key0 + mykey(kb)) * G.Hkv + kvh) * DV + 4 * hl;
    float* dkr = a.dKp + ((int64_t)(key0 + mykey(kb)) * G.Hkv + kvh) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::VB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4* ptr = reinterpret_cast<f32x4*>(dvr + b * 32 + 8 * q);
        const f32x4 add = {dv[kb][b][4 * q] * fv, dv[kb][b][4 * q + 1] * fv, dv[kb][b][4 * q + 2] * fv,
                           dv[kb][b][4 * q + 3] * fv};
        *ptr = *ptr + add;
      }
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4* ptr = reinterpret_cast<f32x4*>(dkr + b * 32 + 8 * q);
        const f32x4 add = {dk[kb][b][4 * q] * sc, dk[kb][b][4 * q + 1] * sc, dk[kb][b][4 * q + 2] * sc,
                           dk[kb][b][4 * q + 3] * sc};
        *ptr = *ptr + add;
      }
  }
}

}  // namespace

hipError_t launch_dkdv_prompt_w64(BwdArgs& a, hipStream_t st) {
  const long long W = (long long)a.ktiles_prompt * a.geo.Hkv;
  if (W == 0) return hipSuccess;
  hipLaunchKernelGGL(replay_bwd_dkdv_w64, dim3((unsigned)(((W + 7) / 8) * 8)), dim3(64 * W64Cfg::NW), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsr
