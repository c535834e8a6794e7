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
  static constexpr int NW = 8;                // waves per workgroup, two per SIMD
  static constexpr int BM = NW * 32;          // packed query rows per workgroup (32 per wave)
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
  static constexpr int KP = KBYTES / 1024;    // 1 KB direct-load pieces: K, then V, then K^T
  static constexpr int VP = VBYTES / 1024;
  static constexpr int NP = STAGE / 1024;
  static constexpr int PPW = NP / NW;         // pieces per wave per tile
  static_assert(KP % NW == 0 && VP % NW == 0 && NP % NW == 0, "pieces split evenly over the waves");
  static_assert(STAGE % (16 * 64 * NW) == 0, "a stage is zero-filled in whole 16-byte stores");
  static constexpr int KS = D / 16;
  static constexpr int VS = DV / 16;
  static constexpr int DB = D / 32;
};

// compile-time half (32-key block) of a tile
template <int H>
using Half = std::integral_constant<int, H>;

// One workgroup = 8 waves x 32 GQA-packed query rows over the key tiles of one split. Per 64-key
// tile, K and V (key-major) and the packed K^T (dimension-major, pack.hip layout) stream
// global -> LDS by direct buffer loads into a three-stage ring of XOR-swizzled tiles. Per 32-key
// block each wave recomputes S^T = K Q^T and dP^T = V dO^T for its rows (Q and dO fragments stay in
// registers), forms dS = P (dP - Delta) with P = exp(S scale - LSE), and accumulates
// dQ^T += K^T dS^T with every K^T fragment a single 16-byte LDS read. The two waves on a SIMD run
// half a step apart (workgroup barriers between phases): one wave's MFMAs overlap the other's
// exp / dS VALU work.
template <int D, int DV>
__global__ __launch_bounds__(64 * 8, 1) void replay_bwd_dq(BwdArgs a) {
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
  const int ktokb = G.ktok0[ri];
  const int Rk = G.ktok0[ri + 1] - ktokb;  // response keys; query row t sits at key position t + qo
  const int qo = Rk - R;
  const int g = G.g;
  const int M = R * g;
  const int m0 = (qt - a.tile0[ri]) * C::BM;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const bool lead = wv < 4;  // waves 0-3 run half a step ahead of waves 4-7

  // query row of this lane: packed row m0 + 32 wv + (lane % 32); Q and dO stay in registers
  const int mrow = m0 + wv * 32 + l32;
  const bool rvalid = mrow < M;
  const int trow = rvalid ? mrow / g : 0;
  const int hq = kvh * g + (rvalid ? mrow - trow * g : 0);
  const int64_t tok = tokb + trow;
  bf16x8 qf[C::KS], of[C::VS];
  {
    const uint16_t* qrow = G.Q + (tok * G.Hq + hq) * D + hl * 8;
    const uint16_t* orow = a.dO + (tok * G.Hq + hq) * DV + hl * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = rvalid ? ld_bf16x8(qrow + ks * 16) : zero_bf16x8();
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) of[ks] = rvalid ? ld_bf16x8(orow + ks * 16) : zero_bf16x8();
  }
  // padding rows: LSE = +inf makes P = 0
  const float lrow = rvalid ? a.lse[(int64_t)hq * G.T + tok] * kLog2e : INFINITY;
  const float drow = rvalid ? a.delta[(int64_t)hq * G.T + tok] : 0.0f;

  // lane-constant LDS byte offsets within a stage. A K (V) fragment ks of a lane sits at chunk
  // (2 ks + hl) ^ swz(l32) of row l32 of its 32-key half; 2 ks and hl occupy different bits, so its
  // offset is base ^ (ks << 5).
  const int kbase = l32 * C::KROW + ((hl ^ swz<C::KCH>(l32)) << 4);
  const int vbase = C::KBYTES + l32 * C::VROW + ((hl ^ swz<C::VCH>(l32)) << 4);
  int toff[2][2];  // [32-key half][16-key part]: packed slots 32 kb + 16 h + 8 hl .. +7 of dim row l32
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      toff[kb][h] = C::KBYTES + C::VBYTES + l32 * C::TROW + (((4 * kb + 2 * h + hl) ^ swz<8>(l32)) << 4);

  const int pt0 = sp * a.ptiles_per_split;
  const int np = max(0, min(a.ptiles, pt0 + a.ptiles_per_split) - pt0);
  const int t_lo = m0 / g + qo;                         // key positions of the tile's first and
  const int t_hi = (min(M, m0 + C::BM) - 1) / g + qo;   // last query rows
  const int ns = (sp == a.splits - 1) ? (t_hi / C::BN + 1) : 0;
  const int nit = np + ns;

  // Direct loads: a tile is NP pieces of 1 KB, wave wv moving pieces wv, wv + NW, ... (piece k of
  // the wave). They go through buffer resources that end with the key arrays: K / V rows past the
  // last key read as zeros (masked out: P = 0 there); packed K^T slots past the keys hold zeros.
  // Lane byte offsets within a tile are fixed per piece (prompt and response pitches of K^T).
  uint32_t pdo[C::PPW], rdo[C::PPW];
#pragma unroll
  for (int k = 0; k < C::PPW; ++k) {
    const int pc = k * C::NW + wv;
    if (pc < C::KP) {
      const int row = pc * (64 / C::KCH) + lane / C::KCH;
      pdo[k] = rdo[k] = (uint32_t)(row * G.ldk * 2 + (((lane % C::KCH) ^ swz<C::KCH>(row)) << 4));
    } else if (pc < C::KP + C::VP) {
      const int row = (pc - C::KP) * (64 / C::VCH) + lane / C::VCH;
      pdo[k] = rdo[k] = (uint32_t)(row * G.ldv * 2 + (((lane % C::VCH) ^ swz<C::VCH>(row)) << 4));
    } else {
      const int row = (pc - C::KP - C::VP) * 8 + (lane >> 3);
      pdo[k] = (uint32_t)(row * a.ppad * 2 + (((lane & 7) ^ swz<8>(row)) << 4));
      rdo[k] = (uint32_t)(row * a.tpad * 2 + (((lane & 7) ^ swz<8>(row)) << 4));
    }
  }
  const char* const kp0 = reinterpret_cast<const char*>(G.Kp + kvh * D);
  const char* const ks0 = reinterpret_cast<const char*>(G.Ks + (int64_t)ktokb * G.ldk + kvh * D);
  const char* const vp0 = reinterpret_cast<const char*>(G.Vp + kvh * DV);
  const char* const vs0 = reinterpret_cast<const char*>(G.Vs + (int64_t)ktokb * G.ldv + kvh * DV);
  const char* const tp0 = reinterpret_cast<const char*>(a.KTp + (int64_t)kvh * D * a.ppad);
  const char* const ts0 = reinterpret_cast<const char*>(a.KTs + (int64_t)kvh * D * a.tpad + a.spos[ri]);
  const int64_t kp_end = ((int64_t)(G.P - 1) * G.ldk + (int64_t)(G.Hkv - kvh) * D) * 2;
  const int64_t ks_end = ((int64_t)(G.Tk - 1 - ktokb) * G.ldk + (int64_t)(G.Hkv - kvh) * D) * 2;
  const int64_t vp_end = ((int64_t)(G.P - 1) * G.ldv + (int64_t)(G.Hkv - kvh) * DV) * 2;
  const int64_t vs_end = ((int64_t)(G.Tk - 1 - ktokb) * G.ldv + (int64_t)(G.Hkv - kvh) * DV) * 2;
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
  // piece k of this wave for tile `it` (branch-free: pieces are issued between MFMAs)
  auto issue_piece = [&](int it, const TileSrc& ts, int k) {
    char* dst = smem + (it % C::NSTAGE) * C::STAGE + (k * C::NW + wv) * 1024;
    if (k * C::NW < C::KP) lds_dma16_buf(ts.k, pdo[k], dst);
    else if (k * C::NW < C::KP + C::VP) lds_dma16_buf(ts.v, pdo[k], dst);
    else lds_dma16_buf(ts.t, (pdo[k] & ts.mask) | (rdo[k] & ~ts.mask), dst);
  };

  f32x16 dq[C::DB];
#pragma unroll
  for (int b = 0; b < C::DB; ++b) dq[b] = f32x16{};
  f32x16 st, dp;   // S^T then P; dP^T then dS (block of the next softmax phase)
  bf16x8 d0, d1;   // dS^T of the block whose dQ MFMAs come next (two 16-key B operands)
  const float c2 = G.scale_log2;

  // MFMA phase of 32-key block j = 2t + hs: S^T and dP^T of block j, dQ^T += K^T dS^T of block j - 1
  // (block -1 has dS = 0 and reads a zero-filled stage; the scores of block 2 nit, past the last
  // tile, come from stale LDS data and are never used). With LOADS, the phase also issues this
  // wave's pieces of tile pt, one after every few MFMAs.
  auto mma = [&](int t, auto half, auto loads, int pt, const TileSrc& nts) {
    constexpr int hs = decltype(half)::value, hp = 1 - hs;
    constexpr bool LOADS = decltype(loads)::value;
    const char* bs = smem + (t % C::NSTAGE) * C::STAGE + hs * 32 * C::KROW;
    const char* bv = smem + (t % C::NSTAGE) * C::STAGE + hs * 32 * C::VROW;
    const char* bp = smem + ((hs == 0 ? t + C::NSTAGE - 1 : t) % C::NSTAGE) * C::STAGE;
    // Three MFMA runs, each following the reads of its fragments; the next run's fragment reads
    // are interleaved with the current run's MFMAs (a read lands in the registers an MFMA has just
    // consumed), so few fragments are live at once and LDS latency hides under the MFMAs.
    bf16x8 kf[C::KS], vf[C::VS], tf[2][C::DB];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kf[ks] = lds_b128_at(bs, kbase ^ (ks << 5));
    __builtin_amdgcn_sched_barrier(0);
    st = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) st = mfma32(kf[ks], qf[ks], st);
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) vf[ks] = lds_b128_at(bv, vbase ^ (ks << 5));
    static_assert(C::KS == C::VS && C::VS == 2 * C::DB, "one fragment read per MFMA of the previous run");
#pragma unroll
    for (int i = 0; i < C::KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) dp = mfma32(vf[ks], of[ks], dp);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < C::DB; ++b) tf[h][b] = lds_b128_at(bp, b * 32 * C::TROW + toff[hp][h]);
#pragma unroll
    for (int i = 0; i < C::VS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < C::DB; ++b) dq[b] = mfma32(tf[0][b], d0, dq[b]);
#pragma unroll
    for (int b = 0; b < C::DB; ++b) dq[b] = mfma32(tf[1][b], d1, dq[b]);
    if constexpr (LOADS) {
#pragma unroll
      for (int k = 0; k < C::PPW; ++k) issue_piece(pt, nts, k);
#pragma unroll
      for (int i = 0; i < 2 * C::DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < C::PPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the waits that follow stay after the MFMAs
  };

  // softmax phase of block (t, kb): mask, P = exp(S scale - LSE), dS = P (dP - Delta) as bf16
  auto softmax = [&](int t, int kb) {
    const bool sfx = t >= np;
    const int key0 = sfx ? (t - np) * C::BN : (pt0 + t) * C::BN;
    const int nvalid = min(C::BN, (sfx ? Rk : G.P) - key0);
    const bool causal = sfx && (key0 + C::BN - 1 > t_lo);
    if (__builtin_expect(causal || nvalid < C::BN, 0)) {
      asm volatile("");  // a real (wave-uniform) branch, not per-element selects
      // register r holds tile key 32 kb + 8(r/4) + 4hl + r%4: visible iff below nvalid and
      // (causal tiles) key0 + key <= the row's key position. Hidden keys get S = -inf, so P = 0.
      const int lim = min(nvalid, causal ? trow + qo - key0 + 1 : nvalid) - kb * 32 - 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = (8 * (r >> 2) + (r & 3)) < lim ? st[r] : -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = fast_exp2(__builtin_fmaf(st[r], c2, -lrow)) * (dp[r] - drow);
    d0 = c_regs_to_bf16x8(dp, 0);
    d1 = c_regs_to_bf16x8(dp, 8);
  };

  // Both groups run the same program: per 32-key block j, an MFMA phase then a softmax phase, each
  // opened by a workgroup barrier; the trailing group passes one extra barrier first, so at every
  // barrier the groups swap roles. Barrier n opens block n / 2 for the leading group.
  // Ring of three stages: tiles 0 and 1 are loaded up front; in loop step t (four barriers, the two
  // blocks of tile t) every wave issues its pieces of tile t + 2 inside its MFMA phase after the
  // first barrier of the step, into the stage of tile t - 1, which no wave reads after barrier
  // 4t + 2. Past the last tile the last tile is loaded again into that free stage, so the waits are
  // fixed. Tile t + 1 is first read after barrier 4t + 4; before the second barrier of step t each
  // wave waits until its pieces of tile t + 1 have landed (only tile t + 2's may be in flight), so
  // that barrier publishes the whole tile for both groups. Every MFMA phase ends with its LDS reads
  // retired.
  using Off = std::integral_constant<bool, false>;
  using On = std::integral_constant<bool, true>;
  if (nit > 0) {
    const TileSrc t0 = tile_src(0), t1 = tile_src(min(1, nit - 1));
#pragma unroll
    for (int k = 0; k < C::PPW; ++k) issue_piece(0, t0, k);
#pragma unroll
    for (int k = 0; k < C::PPW; ++k) issue_piece(1, t1, k);
  }
  {  // the stage read as "tile -1" holds zeros
    char* z = smem + (C::NSTAGE - 1) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::STAGE / (16 * 64 * C::NW); ++i)
      *reinterpret_cast<LSR_LDS u32x4*>(reinterpret_cast<uintptr_t>(z + (i * 64 * C::NW + threadIdx.x) * 16)) =
          u32x4{0u, 0u, 0u, 0u};
  }
  d0 = zero_bf16x8();
  d1 = d0;
  wait_lds();
  wait_vmem_le<C::PPW>();  // tile 0 before barrier 0: tile 1 may be in flight
  if (!lead) bare_barrier();
  const TileSrc tsz = tile_src(0);
  bare_barrier();
  mma(0, Half<0>{}, Off{}, 0, tsz);
  wait_lds();
  bare_barrier();
  for (int t = 0; t < nit; ++t) {
    const TileSrc nts = tile_src(min(t + 2, nit - 1));
    softmax(t, 0);
    bare_barrier();
    mma(t, Half<1>{}, On{}, t + 2, nts);
    wait_lds();
    wait_vmem_le<C::PPW>();  // tile t + 1 landed; tile t + 2's pieces may be in flight
    bare_barrier();
    softmax(t, 1);
    bare_barrier();
    mma(t + 1, Half<0>{}, Off{}, 0, nts);
    wait_lds();
    bare_barrier();
  }
  if (lead) bare_barrier();

  // C layout of dQ^T: lane holds row (lane & 31), dims 32b + 8(r/4) + 4hl + r%4
  if (!rvalid) return;
  const float sc = G.scale;
  if (a.splits == 1) {
    uint16_t* dst = a.dQ + (tok * G.Hq + hq) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v = {pack_bf16x2(dq[b][4 * q] * sc, dq[b][4 * q + 1] * sc),
                         pack_bf16x2(dq[b][4 * q + 2] * sc, dq[b][4 * q + 3] * sc)};
        *reinterpret_cast<u32x2*>(dst + b * 32 + 8 * q) = v;
      }
  } else {
    float* dst = a.dq_part + (((int64_t)sp * G.T + tok) * G.Hq + hq) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {dq[b][4 * q], dq[b][4 * q + 1], dq[b][4 * q + 2], dq[b][4 * q + 3]};
        *reinterpret_cast<f32x4*>(dst + b * 32 + 8 * q) = v;
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
    p.row0[i] = G.ktok0[i];
    p.n[i] = G.ktok0[i + 1] - G.ktok0[i];
    p.col0[i] = a.spos[i];
  }
  if ((e = launch_pack_keys_t(p, st)) != hipSuccess) return e;
  timer_mark(LS_KERNEL_DQ, st, false);
  hipLaunchKernelGGL((replay_bwd_dq<D, DV>), dim3((unsigned)(((W + 7) / 8) * 8)), dim3(64 * DqCfg<D, DV>::NW), 0, st, a);
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
  if (Dqk == kWideDqk && Dv == kWideDv) {
    hipError_t e = launch_bwd_dq_wide(a, st);
    if (e != hipSuccess || a.splits == 1 || a.qtiles == 0) return e;
    const long long n4 = (long long)a.geo.T * a.geo.Hq * kWideDqk / 4;
    hipLaunchKernelGGL((replay_bwd_dq_reduce<kWideDqk>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (Dqk == 64 && Dv == 64) return dq_go<64, 64>(a, st);
  if (Dqk == 128 && Dv == 128) return dq_go<128, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lsr
