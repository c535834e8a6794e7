// Replay attention backward, dK/dV part, on gfx950. The prompt-side gradient is the d l / d z_P
// term of the gradient decomposition in the LongStraw study notes (§2-2); serial replay adds it
// into resident accumulators response after response (§2-1 step 4, §3-2 (4)), and each
// accumulator element is owned by the prompt page it belongs to (§4-3 (2), page-owner dK/dV).
//
// With P = exp(S scale - LSE), dP = dO V^T, Delta = rowsum(dO * O), dS = P (dP - Delta):
//   dV_j += sum_rows P_rj dO_r,   dK_j += scale sum_rows dS_rj Q_r.
//
// replay_bwd_dkdv: key-tile owner. One workgroup = 4 waves x 32 keys of one kv head (one wave per
// SIMD); the wave keeps its keys' K and V fragments (AGPRs) and dK^T, dV^T accumulators for the
// whole sweep over every query row that sees those keys, 32 GQA-packed rows per step, software
// pipelined so that step j's dV / dK products overlap step j + 1's S / dP and softmax. The rows
// were repacked per kv head before the launch (pack.hip): row-major Q and dO (A operands of
// S = Q K^T and dP = dO V^T) and dimension-major, slot-permuted Q^T and dO^T (A operands of
// dV^T += dO^T P and dK^T += Q^T dS, whose B operands come straight from the S / dP accumulators),
// plus each row's LSE and Delta as bf16 row terms (pack_rowext) that one 32x32x8 MFMA each turns
// into the starting values of the S and dP accumulators. Per step all of them stream global -> LDS
// by direct DMA into
// a three-stage ring of XOR-swizzled tiles, so every MFMA operand is one 16-byte LDS read.
// The dV / dK products run in fp16 (11 significant bits; bf16's 8 would cost ~1.7e-3 relative error
// in the fp32 sums over 10^6-10^7 terms, fp16 ~2e-4) with exact power-of-two scaling so every
// operand sits in fp16's normal range: 2^15 P (folded into the exponent), dO s_dO and Q s_Q
// (s from max |dO|, max |Q|), and 2^15 P (dP - Delta) s_dS with s_dS from the bound
// |dP - Delta| <= 2 max_r |dO_r| max_j |V_j| (pack.hip computes the scales per call). Prompt keys:
// the sums are added to dKp / dVp in place (each element is read and written by exactly one
// workgroup per call). Response keys: causal, bf16 dKs / dVs stores.
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

template <int D, int DV>
struct DkvCfg {
  static constexpr int BN = 128;              // keys per workgroup (32 per wave)
  static constexpr int BR = 32;               // query rows per step
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
  static constexpr int NSTAGE = 3;
  static constexpr int QINS = QBYTES / 4096;  // 1 KB direct loads per wave per step
  static constexpr int OINS = OBYTES / 4096;
  static constexpr int QTINS = QTBYTES / 4096;
  static constexpr int OTINS = OTBYTES / 4096;
  static constexpr int KS = D / 16;
  static constexpr int VS = DV / 16;
  static constexpr int DB = D / 32;
  static constexpr int VB = DV / 32;
};

template <int D, int DV, bool PROMPT>
__global__ __launch_bounds__(256, 1) void replay_bwd_dkdv(BwdArgs a) {
  using C = DkvCfg<D, DV>;
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
  const int wv = threadIdx.x >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int mykey = wv * 32 + l32;  // within the tile
  const bool kvalid = mykey < nkeys;

  // K, V fragments of this wave's 32 keys (B operands of S = Q K^T and dP = dO V^T), in AGPRs
  bf16x8 kf[C::KS], vf[C::VS];
  {
    const uint16_t* kr = PROMPT ? G.Kp + (int64_t)(key0 + mykey) * G.ldk + kvh * D
                                : G.Ks + (int64_t)(ktokb + key0 + mykey) * G.ldk + kvh * D;
    const uint16_t* vr = PROMPT ? G.Vp + (int64_t)(key0 + mykey) * G.ldv + kvh * DV
                                : G.Vs + (int64_t)(ktokb + key0 + mykey) * G.ldv + kvh * DV;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      kf[ks] = kvalid ? ld_bf16x8(kr + ks * 16 + hl * 8) : zero_bf16x8();
      asm volatile("" : "+a"(kf[ks]));
    }
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) {
      vf[ks] = kvalid ? ld_bf16x8(vr + ks * 16 + hl * 8) : zero_bf16x8();
      asm volatile("" : "+a"(vf[ks]));
    }
  }

  f32x16 dk[C::DB], dv[C::VB];
#pragma unroll
  for (int b = 0; b < C::DB; ++b) dk[b] = f32x16{};
#pragma unroll
  for (int b = 0; b < C::VB; ++b) dv[b] = f32x16{};

  // lane-constant LDS byte offsets within a stage
  int qoff[C::KS], ooff[C::VS], toff[2];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) qoff[ks] = l32 * C::QROW + (((2 * ks + hl) ^ swz<C::QCH>(l32)) << 4);
#pragma unroll
  for (int ks = 0; ks < C::VS; ++ks) ooff[ks] = C::OFF_O + l32 * C::OROW + (((2 * ks + hl) ^ swz<C::OCH>(l32)) << 4);
#pragma unroll
  for (int h = 0; h < 2; ++h) toff[h] = l32 * C::TROW + (((2 * h + hl) ^ swz<4>(l32)) << 4);

  // Direct loads of a step go through buffer resources over this kv head's packed slabs (one base
  // per slab; the step moves the scalar offset; loads past a slab's end read as zeros).
  const int64_t mpad = a.mpad;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(a.Qr + (int64_t)kvh * mpad * D, mpad * C::QROW);
  const __amdgpu_buffer_rsrc_t ro = buf_rsrc(a.dOr + (int64_t)kvh * mpad * DV, mpad * C::OROW);
  const __amdgpu_buffer_rsrc_t rqt = buf_rsrc(a.QT + (int64_t)kvh * D * mpad, (int64_t)D * mpad * 2);
  const __amdgpu_buffer_rsrc_t rot = buf_rsrc(a.dOT + (int64_t)kvh * DV * mpad, (int64_t)DV * mpad * 2);
  const __amdgpu_buffer_rsrc_t rld = buf_rsrc(a.rowstat + (int64_t)kvh * mpad * 8, mpad * 32);
  // lane-constant byte offsets of the direct loads within one step's slabs: Q / dO rows row-major
  // with XOR-swizzled chunks, Q^T / dO^T rows of 32 slots, 4 bytes of row terms per lane
  uint32_t qdo[C::QINS], odo[C::OINS], qtdo[C::QTINS], otdo[C::OTINS];
#pragma unroll
  for (int u = 0; u < C::QINS; ++u) {
    const int row = (wv * C::QINS + u) * (64 / C::QCH) + lane / C::QCH;
    qdo[u] = (uint32_t)(row * C::QROW + (((lane % C::QCH) ^ swz<C::QCH>(row)) << 4));
  }
#pragma unroll
  for (int u = 0; u < C::OINS; ++u) {
    const int row = (wv * C::OINS + u) * (64 / C::OCH) + lane / C::OCH;
    odo[u] = (uint32_t)(row * C::OROW + (((lane % C::OCH) ^ swz<C::OCH>(row)) << 4));
  }
#pragma unroll
  for (int u = 0; u < C::QTINS; ++u) {
    const int row = (wv * C::QTINS + u) * 16 + (lane >> 2);
    qtdo[u] = (uint32_t)(row * mpad * 2 + (((lane & 3) ^ swz<4>(row)) << 4));
  }
#pragma unroll
  for (int u = 0; u < C::OTINS; ++u) {
    const int row = (wv * C::OTINS + u) * 16 + (lane >> 2);
    otdo[u] = (uint32_t)(row * mpad * 2 + (((lane & 3) ^ swz<4>(row)) << 4));
  }
  const uint32_t ldo = (uint32_t)(wv * 256 + lane * 4);
  // load i of this wave's kPerStep loads of the step at packed row m0 into stage buffer buf; the
  // last one is this wave's quarter of the step's 1 KB of row terms.
  constexpr int kPerStep = C::QINS + C::OINS + C::QTINS + C::OTINS + 1;
  auto issue_load = [&](int i, int m0, char* buf) {
    if (i < C::QINS) {
      lds_dma16_buf(rq, qdo[i], buf + (wv * C::QINS + i) * 1024, m0 * C::QROW);
    } else if (i < C::QINS + C::OINS) {
      const int u = i - C::QINS;
      lds_dma16_buf(ro, odo[u], buf + C::OFF_O + (wv * C::OINS + u) * 1024, m0 * C::OROW);
    } else if (i < C::QINS + C::OINS + C::QTINS) {
      const int u = i - C::QINS - C::OINS;
      lds_dma16_buf(rqt, qtdo[u], buf + C::OFF_QT + (wv * C::QTINS + u) * 1024, m0 * 2);
    } else if (i < kPerStep - 1) {
      const int u = i - C::QINS - C::OINS - C::QTINS;
      lds_dma16_buf(rot, otdo[u], buf + C::OFF_OT + (wv * C::OTINS + u) * 1024, m0 * 2);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rld, (LSR_LDS void*)(buf + C::OFF_LD + wv * 256), 4, (int)ldo, m0 * 32, 0, 0);
    }
  };
  auto issue_step = [&](int m0, char* buf) {
#pragma unroll
    for (int i = 0; i < kPerStep; ++i) issue_load(i, m0, buf);
  };

  const float c2 = G.scale_log2;
  const int nsteps = row_end > row_begin ? (row_end - row_begin + C::BR - 1) / C::BR : 0;

  // fp16 operand scales of this call
  const float s_ds = a.scales[2];

  // Software-pipelined steps. Step j's dV and dK products run while step j + 1's S and dP are
  // formed, so every phase pairs one run of MFMAs with VALU work that does not depend on it and
  // with the LDS reads of a later phase:
  //   A  dV(j) MFMAs         | scaled dS(j), first half      | Q rows of step j + 1
  //   B  S(j + 1) MFMAs      | scaled dS(j), second half     | dO rows of step j + 1, tile loads
  //   C  dK(j) MFMAs         | 2^15 P(j + 1), first half     | row statistics, dO^T of step j + 1
  //   D  dP(j + 1) MFMAs     | 2^15 P(j + 1), second half    | Q^T of step j + 1
  // Within one wave only about a dozen cycles of VALU hide under each MFMA, so the VALU work is
  // spread over all four runs instead of following the MFMAs it depends on.
  // an empty asm use keeps a value's computation in the MFMA run it is written in (instruction
  // selection would otherwise sink it to its first real use)
  auto pin = [](float v) {
    asm volatile("" : "+v"(v));
    return v;
  };
  auto p_elem = [&](const f32x16& s, int r, int m0) {
    const int q = r >> 2, e = r & 3;
    float pv = fast_exp2(s[r] * c2);
    if (!PROMPT) {
      // causal within the response (row t at key position t + qo); rows of other responses see
      // none of these keys
      const int t = (m0 + 8 * q + 4 * hl + e) / g - tokb;
      pv = (t >= 0 && t < R && key0 + mykey <= t + qo) ? pv : 0.0f;
    }
    return pv;
  };
  auto ds_elem = [&](const f32x16& p, const f32x16& dpv, int r) { return p[r] * (dpv[r] * s_ds); };
  // row terms of the step's 32 rows, as the A operands of the 32x32x8 products that start the S and
  // dP accumulators (lanes 32..63 read the zero quarters; each half-wave reads 256 contiguous bytes)
  auto read_terms = [&](const char* buf, s16x4& xq, s16x4& xo) {
    xq = lds_s16x4_at(buf, C::OFF_LD + hl * 256 + l32 * 8);
    xo = lds_s16x4_at(buf, C::OFF_LD + 512 + hl * 256 + l32 * 8);
  };
  // B operand of those products: [1, 1, 1, 0] over k = 0..3 for every key, zero for k = 4..7
  const s16x4 ones = hl ? s16x4{0, 0, 0, 0} : s16x4{0x3F80, 0x3F80, 0x3F80, 0};

  // State carried from one step to the next: 2^15 P (fp32 and fp16), dP - Delta, and the dO^T and
  // Q^T fragments of the step whose dV / dK products are still to run.
  f32x16 p, dp;
  f16x8 pf[2];
  f16x8 ot[2][C::VB], qt[2][C::DB];

  // Three-stage ring. The barrier of step j + 1 (top of pipelined step j) publishes step j + 1's
  // tiles (each wave first waits for its own loads of it) and frees step j's stage: every read
  // of that stage was issued during pipelined step j - 1 and has returned (lgkmcnt(0) before the
  // barrier). That stage then receives step j + 3, issued under the S(j + 1) MFMAs, two steps
  // before it is read. Past the last step the last step's rows are loaded again, so every step
  // issues the same number of loads and the wait count is fixed.
  char* const st0 = smem;
  char* const st1 = smem + C::STAGE;
  char* const st2 = smem + 2 * C::STAGE;
  auto mrow = [&](int t) { return row_begin + min(t, nsteps - 1) * C::BR; };

  // the reads and products of one step's S and dP, 2^15 P and its fp16 copy, with the fragments
  // of the step's dV / dK products; used once, for step 0
  auto first_step = [&](const char* buf) {
    bf16x8 af[C::KS], bfr[C::VS];
    s16x4 xq, xo;
    read_terms(buf, xq, xo);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) af[ks] = lds_b128_at(buf, qoff[ks]);
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) bfr[ks] = lds_b128_at(buf, ooff[ks]);
    f32x16 s = mfma32x8(xq, ones, f32x16{});
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s = mfma32(af[ks], kf[ks], s);
    dp = mfma32x8(xo, ones, f32x16{});
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) dp = mfma32(bfr[ks], vf[ks], dp);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < C::VB; ++b) ot[h][b] = lds_h128_at(buf, C::OFF_OT + b * 32 * C::TROW + toff[h]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < C::DB; ++b) qt[h][b] = lds_h128_at(buf, C::OFF_QT + b * 32 * C::TROW + toff[h]);
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = p_elem(s, r, row_begin);
    pf[0] = c_regs_to_f16x8(p, 0);
    pf[1] = c_regs_to_f16x8(p, 8);
  };

  // pipelined step j: finishes step j (buf of step j + 1 = nb, free stage fb receives step j + 3)
  auto step = [&](int j, const char* nb, char* fb) {
    const int mn = row_begin + (j + 1) * C::BR;  // first packed row of step j + 1
    const int ml = mrow(j + 3);
    constexpr int NA = 2 * C::VB, NB = C::KS, NC = 2 * C::DB, ND = C::VS;
    // A: dV(j) += dO^T P; scaled dS(j) rows 0..7; row terms and Q rows of step j + 1
    bf16x8 af[C::KS];
    s16x4 xq, xo;
    read_terms(nb, xq, xo);
    f32x16 ds = dp;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      dv[i % C::VB] = mfma32h(ot[i / C::VB][i % C::VB], pf[i / C::VB], dv[i % C::VB]);
#pragma unroll
      for (int k = 0; k < C::KS; ++k)
        if (k * NA / C::KS == i) af[k] = lds_b128_at(nb, qoff[k]);
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r * NA / 8 == i) ds[r] = pin(ds_elem(p, dp, r));
      __builtin_amdgcn_sched_barrier(0);
    }
    // B: S(j + 1) = Q K^T; scaled dS(j) rows 8..15; dO rows of step j + 1; step j + 3's tiles
    const f16x8 d0 = c_regs_to_f16x8(ds, 0);
    bf16x8 bfr[C::VS];
    f32x16 sn = mfma32x8(xq, ones, f32x16{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      sn = mfma32(af[i], kf[i], sn);
#pragma unroll
      for (int k = 0; k < C::VS; ++k)
        if (k * NB / C::VS == i) bfr[k] = lds_b128_at(nb, ooff[k]);
#pragma unroll
      for (int r = 8; r < 16; ++r)
        if ((r - 8) * NB / 8 == i) ds[r] = pin(ds_elem(p, dp, r));
#pragma unroll
      for (int l = 0; l < kPerStep; ++l)
        if (l * NB / kPerStep == i) issue_load(l, ml, fb);
      __builtin_amdgcn_sched_barrier(0);
    }
    const f16x8 d1 = c_regs_to_f16x8(ds, 8);
    // C: dK(j) += Q^T dS; dO^T of step j + 1; 2^15 P(j + 1) rows 0..7
    f16x8 otn[2][C::VB];
    f32x16 pn;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      dk[i % C::DB] = mfma32h(qt[i / C::DB][i % C::DB], i / C::DB ? d1 : d0, dk[i % C::DB]);
#pragma unroll
      for (int k = 0; k < 2 * C::VB; ++k)
        if (k * NC / (2 * C::VB) == i) otn[k / C::VB][k % C::VB] = lds_h128_at(nb, C::OFF_OT + (k % C::VB) * 32 * C::TROW + toff[k / C::VB]);
      // P needs the S MFMAs' results: start it half-way through the run
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (NC / 2 + r * (NC - NC / 2) / 8 == i) pn[r] = pin(p_elem(sn, r, mn));
      __builtin_amdgcn_sched_barrier(0);
    }
    pf[0] = c_regs_to_f16x8(pn, 0);
    // D: dP(j + 1) = dO V^T; Q^T of step j + 1; 2^15 P(j + 1) rows 8..15
    f16x8 qtn[2][C::DB];
    f32x16 dpn = mfma32x8(xo, ones, f32x16{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      dpn = mfma32(bfr[i], vf[i], dpn);
#pragma unroll
      for (int k = 0; k < 2 * C::DB; ++k)
        if (k * ND / (2 * C::DB) == i) qtn[k / C::DB][k % C::DB] = lds_h128_at(nb, C::OFF_QT + (k % C::DB) * 32 * C::TROW + toff[k / C::DB]);
#pragma unroll
      for (int r = 8; r < 16; ++r)
        if ((r - 8) * ND / 8 == i) pn[r] = pin(p_elem(sn, r, mn));
      __builtin_amdgcn_sched_barrier(0);
    }
    pf[1] = c_regs_to_f16x8(pn, 8);
    p = pn;
    dp = dpn;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int b = 0; b < C::VB; ++b) ot[h][b] = otn[h][b];
#pragma unroll
      for (int b = 0; b < C::DB; ++b) qt[h][b] = qtn[h][b];
    }
  };

  if (nsteps > 0) {
    issue_step(mrow(0), st0);
    issue_step(mrow(1), st1);
    issue_step(mrow(2), st2);
    wait_vmem_le<2 * kPerStep>();
    bare_barrier();
    first_step(st0);
  }
  // Pipelined step j runs whether or not step j + 1 exists: past the last step it forms S and dP
  // of a repeated tile (rows clamped, results unused), so every wave passes the same barriers.
  for (int it = 0; it < nsteps; it += 3) {
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      const int j = it + jj;
      if (j >= nsteps) break;
      char* nb = jj == 0 ? st1 : (jj == 1 ? st2 : st0);  // stage of step j + 1
      char* fb = jj == 0 ? st0 : (jj == 1 ? st1 : st2);  // stage of step j, free after the barrier
      wait_vmem_le<kPerStep>();
      wait_lds();      // this wave's reads of step j's stage have returned
      bare_barrier();  // no fence: it would wait for every direct load in flight
      step(j, nb, fb);
    }
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
    hipLaunchKernelGGL((replay_bwd_dkdv<D, DV, true>), dim3((unsigned)(((W + 7) / 8) * 8)), dim3(256), 0, st, a);
    timer_mark(LS_KERNEL_DKDV_PROMPT, st, true);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const long long W = (long long)a.ktile0[G.n_resp] * G.Hkv;
  if (W > 0) {
    hipLaunchKernelGGL((replay_bwd_dkdv<D, DV, false>), dim3((unsigned)(((W + 7) / 8) * 8)), dim3(256), 0, st, a);
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
