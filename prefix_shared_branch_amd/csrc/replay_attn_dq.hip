// Replay attention backward, dQ part, on gfx950 (LongStraw study notes, §2-1 step 4 and §2-2):
// with P = exp(S scale - LSE), dP = dO V^T, Delta = rowsum(dO * O) and dS = P (dP - Delta),
//   dQ_r = scale sum_j dS_rj K_j
// over the prompt keys and the response's own (causal) keys. Query-tile owner with split-K over
// the prompt, like the forward; split partials are summed in a fixed order by
// replay_bwd_dq_reduce (deterministic), which also applies the scale and rounds to bf16.
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

// ------------------------------------------------------------------ dQ (query owner, split-K)
template <int D, int DV>
struct DqCfg {
  static constexpr int RB = 2;                // 32-row blocks per wave
  static constexpr int BM = 4 * 32 * RB;      // packed query rows per workgroup
  static_assert(BM == kQTileDq, "dQ tile must match the plan");
  static constexpr int BN = 64;               // keys per tile
  static constexpr int KCH = D / 8;           // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;
  static constexpr int KROW = D * 2;
  static constexpr int VROW = DV * 2;
  static constexpr int TROW = BN * 2;         // bytes per packed K^T row (one dim, 64 keys)
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = BN * VROW;
  static constexpr int TBYTES = D * TROW;
  static constexpr int STAGE = KBYTES + VBYTES + TBYTES;
  static constexpr int NSTAGE = 3;
  static constexpr int KINS = KBYTES / 4096;  // 1 KB direct loads per wave per tile
  static constexpr int VINS = VBYTES / 4096;
  static constexpr int TINS = TBYTES / 4096;
  static constexpr int KS = D / 16;
  static constexpr int VS = DV / 16;
  static constexpr int DB = D / 32;
};

// One workgroup = 4 waves x 64 GQA-packed query rows (one wave per SIMD) over the key tiles of one
// split. Per 64-key tile, K and V (key-major) and the packed K^T (dimension-major, pack.hip layout)
// stream global -> LDS by direct DMA into a three-stage ring of XOR-swizzled tiles. Per 32-key
// block each wave recomputes S^T = K Q^T and dP^T = V dO^T for its two row blocks (Q and dO
// fragments stay in AGPRs; every K or V fragment feeds two MFMAs), forms dS = P (dP - Delta) with
// P = exp(S scale - LSE), and accumulates dQ^T += K^T dS^T with every K^T fragment a single
// 16-byte LDS read feeding two MFMAs.
template <int D, int DV>
__global__ __launch_bounds__(256, 1) void replay_bwd_dq(BwdArgs a) {
  using C = DqCfg<D, DV>;
  __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * C::STAGE];

  const AttnGeom& G = a.geo;
  const int W = a.qtiles * G.Hkv * a.splits;
  const int per_xcd = (W + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= W) return;
  const int strm = w / a.qtiles;
  const int qt = w - strm * a.qtiles;
  const int kvh = strm / a.splits;
  const int sp = strm - kvh * a.splits;
  int ri = 0;
  while (qt >= a.tile0[ri + 1]) ++ri;
  const int tokb = G.tok0[ri];
  const int R = G.tok0[ri + 1] - tokb;
  const int g = G.g;
  const int M = R * g;
  const int m0 = (qt - a.tile0[ri]) * C::BM;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  bool rvalid[C::RB];
  int trow[C::RB], hq[C::RB];
  float lrow[C::RB], drow[C::RB];
  bf16x8 qf[C::RB][C::KS], of[C::RB][C::VS];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    const int mrow = m0 + wv * 32 * C::RB + rb * 32 + l32;
    rvalid[rb] = mrow < M;
    trow[rb] = rvalid[rb] ? mrow / g : 0;
    hq[rb] = kvh * g + (rvalid[rb] ? mrow - trow[rb] * g : 0);
    const int64_t tok = tokb + trow[rb];
    const uint16_t* qrow = G.Q + (tok * G.Hq + hq[rb]) * D + hl * 8;
    const uint16_t* orow = a.dO + (tok * G.Hq + hq[rb]) * DV + hl * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[rb][ks] = rvalid[rb] ? ld_bf16x8(qrow + ks * 16) : zero_bf16x8();
      asm volatile("" : "+a"(qf[rb][ks]));  // MFMA operands only: AGPRs
    }
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) {
      of[rb][ks] = rvalid[rb] ? ld_bf16x8(orow + ks * 16) : zero_bf16x8();
      asm volatile("" : "+a"(of[rb][ks]));
    }
    // padding rows: LSE = +inf makes P = 0
    lrow[rb] = rvalid[rb] ? a.lse[(int64_t)hq[rb] * G.T + tok] * kLog2e : INFINITY;
    drow[rb] = rvalid[rb] ? a.delta[(int64_t)hq[rb] * G.T + tok] : 0.0f;
  }

  // lane-constant LDS byte offsets within a stage (block offsets are immediates)
  int koff[C::KS], voff[C::VS], toff[2][2];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) koff[ks] = l32 * C::KROW + (((2 * ks + hl) ^ swz<C::KCH>(l32)) << 4);
#pragma unroll
  for (int ks = 0; ks < C::VS; ++ks) voff[ks] = C::KBYTES + l32 * C::VROW + (((2 * ks + hl) ^ swz<C::VCH>(l32)) << 4);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      toff[kb][h] = C::KBYTES + C::VBYTES + l32 * C::TROW + (((4 * kb + 2 * h + hl) ^ swz<8>(l32)) << 4);

  const int pt0 = sp * a.ptiles_per_split;
  const int np = max(0, min(a.ptiles, pt0 + a.ptiles_per_split) - pt0);
  const int t_lo = m0 / g;
  const int t_hi = (min(M, m0 + C::BM) - 1) / g;
  const int ns = (sp == a.splits - 1) ? (t_hi / C::BN + 1) : 0;
  const int nit = np + ns;

  // Direct loads go through buffer resources that end with the key arrays: K / V rows past the last
  // key read as zeros (masked out: P = 0 there); packed K^T slots past the keys hold zeros.
  // Lane-constant byte offsets within a tile: K and V rows key-major with XOR-swizzled chunks,
  // packed K^T rows dimension-major (prompt and response pitches).
  uint32_t kdo[C::KINS], vdo[C::VINS], tdo[C::TINS], tdr[C::TINS];
#pragma unroll
  for (int u = 0; u < C::KINS; ++u) {
    const int row = (wv * C::KINS + u) * (64 / C::KCH) + lane / C::KCH;
    kdo[u] = (uint32_t)(row * G.ldk * 2 + (((lane % C::KCH) ^ swz<C::KCH>(row)) << 4));
  }
#pragma unroll
  for (int u = 0; u < C::VINS; ++u) {
    const int row = (wv * C::VINS + u) * (64 / C::VCH) + lane / C::VCH;
    vdo[u] = (uint32_t)(row * G.ldv * 2 + (((lane % C::VCH) ^ swz<C::VCH>(row)) << 4));
  }
#pragma unroll
  for (int u = 0; u < C::TINS; ++u) {
    const int row = (wv * C::TINS + u) * 8 + (lane >> 3);
    tdo[u] = (uint32_t)(row * a.ppad * 2 + (((lane & 7) ^ swz<8>(row)) << 4));
    tdr[u] = (uint32_t)(row * a.tpad * 2 + (((lane & 7) ^ swz<8>(row)) << 4));
  }
  const char* const kp0 = reinterpret_cast<const char*>(G.Kp + kvh * D);
  const char* const ks0 = reinterpret_cast<const char*>(G.Ks + (int64_t)tokb * G.ldk + kvh * D);
  const char* const vp0 = reinterpret_cast<const char*>(G.Vp + kvh * DV);
  const char* const vs0 = reinterpret_cast<const char*>(G.Vs + (int64_t)tokb * G.ldv + kvh * DV);
  const char* const tp0 = reinterpret_cast<const char*>(a.KTp + (int64_t)kvh * D * a.ppad);
  const char* const ts0 = reinterpret_cast<const char*>(a.KTs + (int64_t)kvh * D * a.tpad + a.spos[ri]);
  const int64_t kp_end = ((int64_t)(G.P - 1) * G.ldk + (int64_t)(G.Hkv - kvh) * D) * 2;
  const int64_t ks_end = ((int64_t)(G.T - 1 - tokb) * G.ldk + (int64_t)(G.Hkv - kvh) * D) * 2;
  const int64_t vp_end = ((int64_t)(G.P - 1) * G.ldv + (int64_t)(G.Hkv - kvh) * DV) * 2;
  const int64_t vs_end = ((int64_t)(G.T - 1 - tokb) * G.ldv + (int64_t)(G.Hkv - kvh) * DV) * 2;
  const int64_t tp_end = (int64_t)(G.Hkv - kvh) * D * a.ppad * 2;
  const int64_t ts_end = ((int64_t)(G.Hkv - kvh) * D * a.tpad - a.spos[ri]) * 2;
  struct TileSrc {
    __amdgpu_buffer_rsrc_t k, v, t;
    uint32_t mask;  // all ones for a prompt tile (prompt pitch of the packed K^T), else zero
  };
  auto tile_src = [&](int it) {
    TileSrc ts;
    const bool pr = it < np;
    ts.mask = pr ? 0xFFFFFFFFu : 0u;
    const int key0 = pr ? (pt0 + it) * C::BN : (it - np) * C::BN;
    const int64_t ko = key0 * G.ldk * 2, vo = key0 * G.ldv * 2, to = (int64_t)key0 * 2;
    ts.k = buf_rsrc((pr ? kp0 : ks0) + ko, (pr ? kp_end : ks_end) - ko);
    ts.v = buf_rsrc((pr ? vp0 : vs0) + vo, (pr ? vp_end : vs_end) - vo);
    ts.t = buf_rsrc((pr ? tp0 : ts0) + to, (pr ? tp_end : ts_end) - to);
    return ts;
  };
  // load i of this wave's kPerTile loads of a tile into stage buffer buf (branch-free: loads are
  // issued between MFMAs)
  constexpr int kPerTile = C::KINS + C::VINS + C::TINS;
  auto issue_load = [&](int i, const TileSrc& ts, char* buf) {
    if (i < C::KINS) {
      lds_dma16_buf(ts.k, kdo[i], buf + (wv * C::KINS + i) * 1024);
    } else if (i < C::KINS + C::VINS) {
      const int u = i - C::KINS;
      lds_dma16_buf(ts.v, vdo[u], buf + C::KBYTES + (wv * C::VINS + u) * 1024);
    } else {
      const int u = i - C::KINS - C::VINS;
      lds_dma16_buf(ts.t, (tdo[u] & ts.mask) | (tdr[u] & ~ts.mask), buf + C::KBYTES + C::VBYTES + (wv * C::TINS + u) * 1024);
    }
  };

  f32x16 dq[C::RB][C::DB];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
    for (int b = 0; b < C::DB; ++b) dq[rb][b] = f32x16{};
  const float c2 = G.scale_log2;

  // Per 32-key block: S MFMAs; dP MFMAs with P formed under them; then per row block dS and its dQ
  // MFMAs, row block 1's dS formed under row block 0's MFMAs.
  // The loads of the tile two ahead (source nts, stage nbuf) are issued between the score MFMAs of
  // the first 32-key block, one at a time.
  auto compute = [&](const char* buf, bool masked, int key0, int nvalid, bool causal, const TileSrc& nts,
                     char* nbuf) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T = K Q^T for both row blocks (each K fragment feeds two MFMAs)
      f32x16 st[C::RB], dp[C::RB];
      {
        bf16x8 kf[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) kf[ks] = lds_b128_at(buf, kb * 32 * C::KROW + koff[ks]);
        __builtin_amdgcn_sched_barrier(0);
        if (kb == 0) {
#pragma unroll
          for (int i = 0; i < kPerTile; ++i) issue_load(i, nts, nbuf);
        }
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          st[rb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) st[rb] = mfma32(kf[ks], qf[rb][ks], st[rb]);
        }
        if (kb == 0) {
          static_assert(kPerTile <= C::RB * C::KS, "one load after each MFMA at most");
#pragma unroll
          for (int i = 0; i < C::RB * C::KS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < kPerTile) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        }
      }
      // dP^T = V dO^T
      {
        bf16x8 vf[C::VS];
#pragma unroll
        for (int ks = 0; ks < C::VS; ++ks) vf[ks] = lds_b128_at(buf, kb * 32 * C::VROW + voff[ks]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          dp[rb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < C::VS; ++ks) dp[rb] = mfma32(vf[ks], of[rb][ks], dp[rb]);
        }
      }
      if (__builtin_expect(masked, 0)) {
        asm volatile("");  // a real (wave-uniform) branch, not per-element selects
        // register r holds tile key kb*32 + 8(r/4) + 4hl + r%4: visible iff below nvalid and
        // (causal tiles) key0 + key <= the row's token. Hidden keys get S = -inf, so P = 0.
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          const int lim = min(nvalid, causal ? trow[rb] - key0 + 1 : nvalid) - kb * 32 - 4 * hl;
#pragma unroll
          for (int r = 0; r < 16; ++r) st[rb][r] = (8 * (r >> 2) + (r & 3)) < lim ? st[rb][r] : -INFINITY;
        }
      }
      // P = exp(S scale - LSE), under the dP MFMAs
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[rb][r] = fast_exp2(__builtin_fmaf(st[rb][r], c2, -lrow[rb]));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        // dS = P (dP - Delta) as the bf16 B operands of dQ^T += K^T dS^T
#pragma unroll
        for (int r = 0; r < 16; ++r) st[rb][r] = st[rb][r] * (dp[rb][r] - drow[rb]);
        const bf16x8 d0 = c_regs_to_bf16x8(st[rb], 0), d1 = c_regs_to_bf16x8(st[rb], 8);
        // K^T fragments: one 16-byte read of packed slots each
        bf16x8 tf[2][C::DB];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int b = 0; b < C::DB; ++b) tf[h][b] = lds_b128_at(buf, b * 32 * C::TROW + toff[kb][h]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) dq[rb][b] = mfma32(tf[0][b], d0, dq[rb][b]);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) dq[rb][b] = mfma32(tf[1][b], d1, dq[rb][b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Three-stage ring: before tile t each wave waits for its own loads of tile t (tile t + 1's may
  // be in flight) and the barrier publishes the tile; every wave is then past tile t - 1, whose
  // stage receives tile t + 2 (issued inside the tile's first MFMAs). Past the last tile the last
  // tile is loaded again into that free stage, so the wait count is fixed.
  char* const st0 = smem;
  char* const st1 = smem + C::STAGE;
  char* const st2 = smem + 2 * C::STAGE;
  if (nit > 0) {
    const TileSrc t0 = tile_src(0), t1 = tile_src(min(1, nit - 1));
#pragma unroll
    for (int i = 0; i < kPerTile; ++i) issue_load(i, t0, st0);
#pragma unroll
    for (int i = 0; i < kPerTile; ++i) issue_load(i, t1, st1);
  }
  for (int it = 0; it < nit; it += 3) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int t = it + j;
      if (t >= nit) break;
      char* cur = j == 0 ? st0 : (j == 1 ? st1 : st2);
      char* nxt = j == 0 ? st2 : (j == 1 ? st0 : st1);
      const TileSrc nts = tile_src(min(t + 2, nit - 1));
      wait_vmem_le<kPerTile>();
      wait_lds();      // this wave's reads of the stage refilled next have returned
      bare_barrier();  // no fence: it would wait for every direct load in flight
      const bool sfx = t >= np;
      const int key0 = sfx ? (t - np) * C::BN : (pt0 + t) * C::BN;
      const int nvalid = min(C::BN, (sfx ? R : G.P) - key0);
      const bool causal = sfx && (key0 + C::BN - 1 > t_lo);
      compute(cur, causal || nvalid < C::BN, key0, nvalid, causal, nts, nxt);
    }
  }

  // C layout of dQ^T: lane holds row (lane & 31), dims 32b + 8(r/4) + 4hl + r%4
  const float sc = G.scale;
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    if (!rvalid[rb]) continue;
    const int64_t tok = tokb + trow[rb];
    if (a.splits == 1) {
      uint16_t* dst = a.dQ + (tok * G.Hq + hq[rb]) * D + 4 * hl;
#pragma unroll
      for (int b = 0; b < C::DB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 v = {pack_bf16x2(dq[rb][b][4 * q] * sc, dq[rb][b][4 * q + 1] * sc),
                           pack_bf16x2(dq[rb][b][4 * q + 2] * sc, dq[rb][b][4 * q + 3] * sc)};
          *reinterpret_cast<u32x2*>(dst + b * 32 + 8 * q) = v;
        }
    } else {
      float* dst = a.dq_part + (((int64_t)sp * G.T + tok) * G.Hq + hq[rb]) * D + 4 * hl;
#pragma unroll
      for (int b = 0; b < C::DB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {dq[rb][b][4 * q], dq[rb][b][4 * q + 1], dq[rb][b][4 * q + 2], dq[rb][b][4 * q + 3]};
          *reinterpret_cast<f32x4*>(dst + b * 32 + 8 * q) = v;
        }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void replay_bwd_dq_reduce(BwdArgs a) {
  const AttnGeom& G = a.geo;
  const int64_t n4 = (int64_t)G.T * G.Hq * D / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n4) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.splits; ++s) acc += reinterpret_cast<const f32x4*>(a.dq_part)[(int64_t)s * n4 + idx];
  acc *= G.scale;
  const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  reinterpret_cast<u32x2*>(a.dQ)[idx] = v;
}

template <int D, int DV>
hipError_t dq_go(BwdArgs& a, hipStream_t st) {
  const AttnGeom& G = a.geo;
  const long long W = (long long)a.qtiles * G.Hkv * a.splits;
  if (W == 0) return hipSuccess;
  hipError_t e;
  // dimension-major packed K of the prompt and of every response (dQ^T = K^T dS^T operand)
  PackArgs p;
  p.f16_scale = nullptr;
  p.src = G.Kp;
  p.ld = G.ldk;
  p.dim = D;
  p.heads = G.Hkv;
  p.grp = 1;
  p.gstride = 0;
  p.hstride = D;
  p.out_ld = a.ppad;
  p.cols = a.ppad;
  p.out = const_cast<uint16_t*>(a.KTp);
  p.nseg = 1;
  p.row0[0] = 0;
  p.n[0] = G.P;
  p.col0[0] = 0;
  if (G.P > 0 && (e = launch_pack_keys_t(p, st)) != hipSuccess) return e;
  p.src = G.Ks;
  p.out_ld = a.tpad;
  p.cols = a.tpad;
  p.out = const_cast<uint16_t*>(a.KTs);
  p.nseg = G.n_resp;
  for (int i = 0; i < G.n_resp; ++i) {
    p.row0[i] = G.tok0[i];
    p.n[i] = G.tok0[i + 1] - G.tok0[i];
    p.col0[i] = a.spos[i];
  }
  if ((e = launch_pack_keys_t(p, st)) != hipSuccess) return e;
  timer_mark(LS_KERNEL_DQ, st, false);
  hipLaunchKernelGGL((replay_bwd_dq<D, DV>), dim3((unsigned)(((W + 7) / 8) * 8)), dim3(256), 0, st, a);
  timer_mark(LS_KERNEL_DQ, st, true);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.splits > 1) {
    const long long n4 = (long long)G.T * G.Hq * D / 4;
    hipLaunchKernelGGL((replay_bwd_dq_reduce<D>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_dq(BwdArgs& a, int Dqk, int Dv, hipStream_t st) {
  if (Dqk == 64 && Dv == 64) return dq_go<64, 64>(a, st);
  if (Dqk == 128 && Dv == 128) return dq_go<128, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lsr
