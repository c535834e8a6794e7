// Replay attention forward on gfx950 (LongStraw study notes, §2-1 step 4 and §3-2 (2)/(4)):
// the queries of one response attend to all prompt keys and, causally, to the response's
// own keys.
//
// replay_fwd: one workgroup = 8 waves x 32 = 256 GQA-packed query rows of one kv head, over the
// prompt key tiles of one split (plus, in the last split, the response's causal key tiles). Per
// 64-key tile, K (key-major) and V (dimension-major, packed by pack.hip) stream global -> LDS by
// direct buffer loads into a four-stage ring of XOR-swizzled tiles. Per 32-key block each wave
// computes S^T = K Q^T for its 32 rows (MFMA 32x32x16 bf16; Q fragments stay in registers), an
// online softmax whose row statistics are lane-local (one query row per lane), and O^T += V^T P^T
// where P^T comes straight from the score accumulators and every V^T fragment is one 16-byte LDS
// read. Two waves share each SIMD and run half a step apart, so one wave's softmax (VALU) overlaps
// the other's MFMAs.
// The PV product runs in fp16 (MFMA 32x32x16 f16, the same rate as bf16): the packed V^T holds
// fp16 of V s_V, s_V a power of two with max |V| s_V <= 2^15 (fwd_vscale in pack.hip), so the
// conversion is exact wherever the exponent fits, and P keeps 11 significant bits instead of 8.
// The backward's row term Delta = rowsum(dO O) is formed from this output, and a single heavy
// prompt key (very short prompts) passes the weight rounding straight into the prompt gradient.
// The softmax stabiliser is only moved when a row maximum exceeds it by more than 2^8 (in exp2
// units), so the O rescale is rare; probabilities stay <= 256, far inside fp32/bf16 range.
// Workgroup ids are mapped so that each XCD owns a contiguous run of (kv head, split) streams:
// concurrently resident query tiles sweep the same prompt K/V tiles, which are then fetched from
// HBM once per XCD and served to its CUs from L2.
//
// replay_fwd_merge: log-sum-exp merge of the split partials,
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s.
#include <cstring>

#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

// Eight waves per workgroup, two per SIMD (waves w and w + 4 share a SIMD), 32 query rows each.
// The waves form two groups, 0-3 and 4-7, that run half a step apart: while one group's wave on a
// SIMD issues MFMAs, the other group's wave on the same SIMD runs its softmax on the VALU (on gfx950
// a wave's MFMAs keep their full rate while the SIMD's other wave executes VALU work; within one
// wave the two serialise). Workgroup barriers separate the phases and keep the groups in step.
constexpr int kFwdWaves = 8;

template <int D, int DV>
struct FwdCfg {
  static constexpr int NW = kFwdWaves;
  static constexpr int BM = NW * 32;          // packed query rows per workgroup
  static_assert(BM == kQTileFwd, "forward tile must match the plan");
  static constexpr int BN = 64;               // keys per tile
  static constexpr int KCH = D / 8;           // 16-byte chunks per K row
  static constexpr int KROW = D * 2;          // bytes per K row in LDS
  static constexpr int VTROW = BN * 2;        // bytes per packed V^T row (one dim, 64 keys)
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = DV * VTROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NSTAGE = 4;
  static constexpr int KP = KBYTES / 1024;     // 1 KB direct-load pieces of a tile: K pieces first,
  static constexpr int NP = STAGE / 1024;      // then V^T pieces
  static constexpr int PPW = NP / NW;          // pieces per wave per tile (one after each of PPW barriers)
  static_assert(NP % NW == 0 && KP % NW == 0 && PPW <= 4, "pieces split evenly over the waves");
  static_assert(STAGE % (16 * 64 * NW) == 0, "a stage is zero-filled in whole 16-byte stores");
  static constexpr int KS = D / 16;           // MFMA k-steps over the head dim
  static constexpr int NB = DV / 32;          // 32-wide blocks of the value dim
  static constexpr float kStale = 8.0f;       // stabiliser slack (exp2 units)
};

// max / sum of a value over lanes l and l ^ 32. The swap of two copies of v leaves, in each lane,
// the lane's own value in one result and its partner's in the other; combining the two results
// with a commutative operation gives both lanes the same bits.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// compile-time selector of one part of an MFMA phase: present or not, and which 32-key half of a tile
template <bool ON, int HALF>
struct Part {
  static constexpr bool on = ON;
  static constexpr int half = HALF;
};

template <int D, int DV>
__global__ __launch_bounds__(64 * kFwdWaves, 1) void replay_fwd(FwdArgs a) {
  using C = FwdCfg<D, DV>;
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
  const bool lead = wv < 4;  // group 0 (waves 0-3) runs half a step ahead of group 1

  // query row of this lane: packed row m0 + 32 wv + (lane % 32); Q stays in registers
  const int mrow = m0 + wv * 32 + l32;
  const bool rvalid = mrow < M;
  const int trow = rvalid ? mrow / g : 0;
  const int hq = kvh * g + (rvalid ? mrow - trow * g : 0);
  bf16x8 qf[C::KS];
  {
    const uint16_t* qrow = G.Q + ((int64_t)(tokb + trow) * G.Hq + hq) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qf[ks] = rvalid ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + ks * 16))
                      : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  // lane-constant LDS byte offsets within a stage (block and tile offsets are immediates)
  // K fragment ks of a lane sits at chunk (2 ks + hl) ^ swz(l32) of row l32; since 2 ks and hl
  // occupy different bits, its offset is kbase ^ (ks << 5) (only chunk bits change)
  const int kbase = l32 * C::KROW + ((hl ^ swz<C::KCH>(l32)) << 4);
  int voff[2][2];  // [32-key block][16-key half]: packed slots 32 kb + 16 h + 8 hl .. +7 of dim row l32
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h) voff[kb][h] = C::KBYTES + l32 * C::VTROW + (((4 * kb + 2 * h + hl) ^ swz<8>(l32)) << 4);

  // key range: prompt tiles of this split, then (last split) the response's causal tiles
  const int pt0 = sp * a.ptiles_per_split;
  const int np = max(0, min(a.ptiles, pt0 + a.ptiles_per_split) - pt0);
  const int t_lo = m0 / g + qo;                         // key positions of the tile's first and
  const int t_hi = (min(M, m0 + C::BM) - 1) / g + qo;   // last query rows
  const int ns = (sp == a.splits - 1) ? (t_hi / C::BN + 1) : 0;
  const int nit = np + ns;

  // Direct loads: a tile is NP pieces of 1 KB (one 16-byte load per lane), K pieces first, then
  // packed V^T pieces. Wave wv moves pieces wv, wv + NW, wv + 2 NW, ... (piece k of the wave). K rows
  // are key-major (1024 / KROW rows per piece), packed V^T rows dimension-major (8 rows of 128 bytes
  // per piece); lane byte offsets within the tile are 32-bit and fixed per piece (prompt pitch).
  uint32_t pdo[C::PPW], rdo[C::PPW];  // prompt pitch; V^T pieces of response tiles: response pitch
#pragma unroll
  for (int k = 0; k < C::PPW; ++k) {
    const int pc = k * C::NW + wv;
    if (pc < C::KP) {
      const int row = pc * (64 / C::KCH) + lane / C::KCH;
      pdo[k] = rdo[k] = (uint32_t)(row * G.ldk * 2 + (((lane % C::KCH) ^ swz<C::KCH>(row)) << 4));
    } else {
      const int row = (pc - C::KP) * 8 + (lane >> 3);
      pdo[k] = (uint32_t)(row * a.ppad * 2 + (((lane & 7) ^ swz<8>(row)) << 4));
      rdo[k] = (uint32_t)(row * a.tpad * 2 + (((lane & 7) ^ swz<8>(row)) << 4));
    }
  }

  // global -> LDS sources of a tile: buffer resources that end with the key arrays, so K rows past
  // the last key read as zeros (those keys are masked out of the softmax); packed V^T slots past the
  // keys hold zeros. Bases and extents are formed once; per tile only the start moves.
  const char* const kp0 = reinterpret_cast<const char*>(G.Kp + kvh * D);
  const char* const ks0 = reinterpret_cast<const char*>(G.Ks + (int64_t)ktokb * G.ldk + kvh * D);
  const char* const vp0 = reinterpret_cast<const char*>(a.VTp + (int64_t)kvh * DV * a.ppad);
  const char* const vs0 = reinterpret_cast<const char*>(a.VTs + (int64_t)kvh * DV * a.tpad + a.spos[ri]);
  const int64_t kp_end = ((int64_t)(G.P - 1) * G.ldk + (int64_t)(G.Hkv - kvh) * D) * 2;
  const int64_t ks_end = ((int64_t)(G.Tk - 1 - ktokb) * G.ldk + (int64_t)(G.Hkv - kvh) * D) * 2;
  const int64_t vp_end = (int64_t)(G.Hkv - kvh) * DV * a.ppad * 2;
  const int64_t vs_end = ((int64_t)(G.Hkv - kvh) * DV * a.tpad - a.spos[ri]) * 2;
  const int64_t ldk2 = G.ldk * 2;
  struct TileSrc {
    __amdgpu_buffer_rsrc_t k, v;
    bool prompt;
  };
  auto tile_src = [&](int it) {
    TileSrc ts;
    ts.prompt = it < np;
    const int key0 = ts.prompt ? (pt0 + it) * C::BN : (it - np) * C::BN;
    const int64_t ko = key0 * ldk2, vo = (int64_t)key0 * 2;
    ts.k = buf_rsrc((ts.prompt ? kp0 : ks0) + ko, (ts.prompt ? kp_end : ks_end) - ko);
    ts.v = buf_rsrc((ts.prompt ? vp0 : vs0) + vo, (ts.prompt ? vp_end : vs_end) - vo);
    return ts;
  };
  // piece k of this wave for tile `it` (branch-free: it is issued between MFMAs)
  auto issue_piece = [&](int it, const TileSrc& ts, auto kc) {
    constexpr int k = decltype(kc)::value;
    char* dst = smem + (it % C::NSTAGE) * C::STAGE + (k * C::NW + wv) * 1024;
    if constexpr (k * C::NW < C::KP) lds_dma16_buf(ts.k, pdo[k], dst);
    else {
      // a bit blend rather than a select, which the compiler would turn into a select of array
      // addresses (and move both arrays to scratch memory)
      const uint32_t m = ts.prompt ? 0xFFFFFFFFu : 0u;
      lds_dma16_buf(ts.v, (pdo[k] & m) | (rdo[k] & ~m), dst);
    }
  };

  f32x16 o[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) o[nb] = f32x16{};
  float mu = -INFINITY;  // stabiliser (score * scale * log2 e)
  float l_run = 0.0f;    // row sum of this lane's keys
  f32x16 st;             // S^T of the 32-key block whose softmax comes next
  f16x8 p0, p1;          // P^T of the block whose PV product comes next (two 16-key B operands)
  const float c2 = G.scale_log2;

  // MFMA phase of 32-key block j = 2t + h: S^T = K Q^T for block j (tile t, half h) and
  // O^T += V^T P^T for block j - 1 (its probabilities from the previous softmax phase). Block -1 has
  // zero probabilities and reads a zero-filled stage; the scores of block 2 nit (past the last tile)
  // are formed from stale LDS data and never used.
  // The phase also issues this wave's direct-load pieces K0 .. K0 + NK - 1 of tile `pt` (source ts),
  // spread between its MFMAs so that the loads enter the memory pipeline one at a time.
  auto mma = [&](int t, auto half, int pt, const TileSrc& ts, auto k0c, auto nkc) {
    constexpr int hs = decltype(half)::value, hp = 1 - hs;
    constexpr int K0 = decltype(k0c)::value, NK = decltype(nkc)::value;
    const int bs = (int)((t % C::NSTAGE) * C::STAGE + hs * 32 * C::KROW) + kbase;  // no chunk bits
    const char* bp = smem + ((hs == 0 ? t + C::NSTAGE - 1 : t) % C::NSTAGE) * C::STAGE;
    bf16x8 kf[C::KS], vf[2][C::NB];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kf[ks] = lds_b128_at(smem, bs ^ (ks << 5));
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) vf[h][nb] = lds_b128_at(bp, nb * 32 * C::VTROW + voff[hp][h]);
    if constexpr (NK > 0) issue_piece(pt, ts, std::integral_constant<int, K0>{});
    if constexpr (NK > 1) issue_piece(pt, ts, std::integral_constant<int, K0 + 1>{});
    st = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) st = mfma32(kf[ks], qf[ks], st);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) o[nb] = mfma32h(__builtin_bit_cast(f16x8, vf[0][nb]), p0, o[nb]);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) o[nb] = mfma32h(__builtin_bit_cast(f16x8, vf[1][nb]), p1, o[nb]);
    // Issue order: the K fragment reads, then the score MFMAs each followed by V^T fragment reads
    // (a direct load after the second and the sixth), then the PV MFMAs; LDS latency hides under
    // the MFMA chain.
    static_assert(NK <= 2, "at most two direct loads per MFMA phase");
    __builtin_amdgcn_sched_group_barrier(0x100, C::KS, 0);
#pragma unroll
    for (int i = 0; i < C::KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, (2 * C::NB) / C::KS, 0);
      if ((NK > 0 && i == 1) || (NK > 1 && i == C::KS - 3)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::NB, 0);
    __builtin_amdgcn_sched_barrier(0);  // the waits that follow stay after the MFMAs
  };

  // softmax phase of 32-key block j (tile t = j / 2, half kb = j % 2): mask, online softmax of the
  // lane's row (the other half-wave holds the row's other keys), P^T as bf16 B operands
  auto softmax = [&](int t, int kb) {
    const bool sfx = t >= np;
    const int key0 = sfx ? (t - np) * C::BN : (pt0 + t) * C::BN;
    const int nvalid = min(C::BN, (sfx ? Rk : G.P) - key0);
    const bool causal = sfx && (key0 + C::BN - 1 > t_lo);
    if (__builtin_expect(causal || nvalid < C::BN, 0)) {
      asm volatile("");  // keeps this a real (wave-uniform) branch instead of per-element selects
      // register r holds tile key 32 kb + 8(r/4) + 4hl + r%4; it is visible iff that key is below
      // nvalid and (causal tiles) key0 + key <= the row's key position
      const int lim = min(nvalid, causal ? trow + qo - key0 + 1 : nvalid) - kb * 32 - 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = (8 * (r >> 2) + (r & 3)) < lim ? st[r] : -INFINITY;
    }
    float mx = __builtin_elementwise_maximum(st[0], st[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, st[r]);
    mx = pair_max(mx) * c2;
    const bool move = mx > mu + C::kStale;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(move) != 0, 0)) {
      asm volatile("");  // rare: a real branch, never speculated into unconditional multiplies
      const float mnew = move ? mx : mu;
      const float alpha = move ? fast_exp2(mu - mnew) : 1.0f;   // 0 on a row's first visible keys
      mu = mnew;
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[nb] *= alpha;
    }
    const float msub = mu == -INFINITY ? 0.0f : mu;
    // the row sum is taken in fp32 (the LSE must hold to ~1e-6 even over a few keys)
    float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      st[r] = fast_exp2(__builtin_fmaf(st[r], c2, -msub));
      st[r + 1] = fast_exp2(__builtin_fmaf(st[r + 1], c2, -msub));
      ls0 += st[r];
      ls1 += st[r + 1];
    }
    l_run += ls0 + ls1;
    p0 = c_regs_to_f16x8(st, 0);
    p1 = c_regs_to_f16x8(st, 8);
  };

  // Both groups run the same program: per 32-key block j, an MFMA phase then a softmax phase, each
  // opened by a workgroup barrier. The trailing group passes one extra barrier first, so at every
  // barrier the groups swap roles: while the leading group forms the scores of block j, the
  // trailing group runs the softmax of block j - 1, and so on. Barrier n (counted over the
  // workgroup) opens block n / 2 for the leading group.
  // Ring of four stages: tiles 0-2 are loaded up front; in loop step t (four barriers, two blocks of
  // tile t) every wave issues its pieces of tile t + 3 into the stage of tile t - 1, which no wave
  // reads after barrier 4t + 2: half of them inside its MFMA phase after the first barrier of the
  // step, the rest inside its MFMA phase after the third. Past the last tile the same pieces of
  // the last tile are loaded again into the unused stage, so every step issues the same number of
  // loads and the waits below are fixed. Tile t + 1 is first read after barrier 4t + 4; before the
  // second barrier of step t each wave waits until its pieces of tile t + 1 have landed (only
  // later tiles' pieces may still be in flight), so that barrier publishes the whole tile for both
  // groups. Every MFMA phase ends with its LDS reads retired.
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  using N0 = std::integral_constant<int, 0>;
  constexpr int PA = (C::PPW + 1) / 2, PB = C::PPW - PA;  // pieces in the first / second MFMA phase
  using KA = std::integral_constant<int, 0>;
  using NA = std::integral_constant<int, PA>;
  using KB = std::integral_constant<int, PA>;
  using NB2 = std::integral_constant<int, PB>;
  auto issue_tile = [&](int t) {
    const int tt = min(t, nit - 1);
    const TileSrc ts = tile_src(tt);
    issue_piece(t, ts, std::integral_constant<int, 0>{});
    if constexpr (C::PPW > 1) issue_piece(t, ts, std::integral_constant<int, 1>{});
    if constexpr (C::PPW > 2) issue_piece(t, ts, std::integral_constant<int, 2>{});
    if constexpr (C::PPW > 3) issue_piece(t, ts, std::integral_constant<int, 3>{});
  };
  if (nit > 0) {
    issue_tile(0);
    issue_tile(1);
    issue_tile(2);
  }
  {  // the stage read as "tile -1" holds zeros
    char* z = smem + (C::NSTAGE - 1) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::STAGE / (16 * 64 * C::NW); ++i)
      *reinterpret_cast<LSR_LDS u32x4*>(reinterpret_cast<uintptr_t>(z + (i * 64 * C::NW + threadIdx.x) * 16)) =
          u32x4{0u, 0u, 0u, 0u};
  }
  p0 = __builtin_bit_cast(f16x8, u32x4{0u, 0u, 0u, 0u});
  p1 = p0;
  wait_lds();
  wait_vmem_le<2 * C::PPW>();  // tile 0 before barrier 0: tiles 1 and 2 may be in flight
  if (!lead) bare_barrier();
  bare_barrier();
  const TileSrc ts0 = tile_src(0);
  mma(0, H0{}, 0, ts0, N0{}, N0{});
  wait_lds();
  bare_barrier();
  for (int t = 0; t < nit; ++t) {
    const TileSrc ts = tile_src(min(t + 3, nit - 1));
    softmax(t, 0);
    bare_barrier();
    mma(t, H1{}, t + 3, ts, KA{}, NA{});
    wait_lds();
    wait_vmem_le<C::PPW + PA>();  // tile t + 1: tile t + 2's pieces and PA of tile t + 3 may be in flight
    bare_barrier();
    softmax(t, 1);
    bare_barrier();
    mma(t + 1, H0{}, t + 3, ts, KB{}, NB2{});
    wait_lds();
    bare_barrier();
  }
  if (lead) bare_barrier();

  const float l = pair_sum(l_run);
  if (!rvalid) return;
  const int64_t tok = tokb + trow;
  const float inv = l > 0.0f ? a.vscale[1] / l : 0.0f;   // O = (V s_V)^T P^T / (l s_V)
  const float lse = l > 0.0f ? (mu + fast_log2(l)) * kLn2 : -INFINITY;
  if (a.splits == 1) {
    const int64_t off = (tok * G.Hq + hq) * DV + 4 * hl;
    uint16_t* orow = a.O + off;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = o[nb][4 * q] * inv, x1 = o[nb][4 * q + 1] * inv;
        const float x2 = o[nb][4 * q + 2] * inv, x3 = o[nb][4 * q + 3] * inv;
        const u32x2 v = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        *reinterpret_cast<u32x2*>(orow + nb * 32 + 8 * q) = v;
        if (a.O_lo) {
          const u32x2 r = {pack_bf16x2_residual(x0, x1, v[0]), pack_bf16x2_residual(x2, x3, v[1])};
          *reinterpret_cast<u32x2*>(a.O_lo + off + nb * 32 + 8 * q) = r;
        }
      }
    if (hl == 0) a.lse[(int64_t)hq * G.T + tok] = lse;
  } else {
    float* orow = a.o_part + (((int64_t)sp * G.T + tok) * G.Hq + hq) * DV + 4 * hl;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {o[nb][4 * q] * inv, o[nb][4 * q + 1] * inv, o[nb][4 * q + 2] * inv,
                         o[nb][4 * q + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + nb * 32 + 8 * q) = v;
      }
    if (hl == 0) a.lse_part[((int64_t)sp * G.Hq + hq) * G.T + tok] = lse;
  }
}

template <int DV>
__global__ __launch_bounds__(256) void replay_fwd_merge(FwdArgs a) {
  const AttnGeom& G = a.geo;
  constexpr int CH = DV / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)G.T * G.Hq * CH;
  if (idx >= total) return;
  const int c = (int)(idx % CH);
  const int64_t th = idx / CH;
  const int h = (int)(th % G.Hq);
  const int64_t t = th / G.Hq;
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.lse_part[((int64_t)s * G.Hq + h) * G.T + t]);
  float den = 0.0f;
  for (int s = 0; s < a.splits; ++s) den += expf(a.lse_part[((int64_t)s * G.Hq + h) * G.T + t] - mx);
  const float lse = mx + logf(den);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.splits; ++s) {
    const float wgt = expf(a.lse_part[((int64_t)s * G.Hq + h) * G.T + t] - lse);
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.o_part + (((int64_t)s * G.T + t) * G.Hq + h) * DV + 4 * c);
    acc += wgt * v;
  }
  const u32x2 ov = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  *reinterpret_cast<u32x2*>(a.O + (t * G.Hq + h) * DV + 4 * c) = ov;
  if (a.O_lo) {
    const u32x2 r = {pack_bf16x2_residual(acc[0], acc[1], ov[0]), pack_bf16x2_residual(acc[2], acc[3], ov[1])};
    *reinterpret_cast<u32x2*>(a.O_lo + (t * G.Hq + h) * DV + 4 * c) = r;
  }
  if (c == 0) a.lse[(int64_t)h * G.T + t] = lse;
}

template <int D, int DV>
hipError_t fwd_go(FwdArgs& a, hipStream_t st) {
  const long long W = (long long)a.qtiles * a.geo.Hkv * a.splits;
  if (W == 0) return hipSuccess;
  // V scale, then dimension-major packed fp16 V s_V of the prompt and of every response
  const AttnGeom& G = a.geo;
  {
    ScaleArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.Vp = G.Vp;
    sa.Vs = G.Vs;
    sa.ldv = G.ldv;
    sa.P = G.P;
    sa.Tk = G.Tk;
    sa.Hkv = G.Hkv;
    sa.Dqk = D;
    sa.Dv = DV;
    sa.partial = a.vscale_part;
    sa.scales = a.vscale;
    hipError_t e = launch_fwd_vscale(sa, st);
    if (e != hipSuccess) return e;
  }
  if (G.P > 0) {
    PackArgs p;
    p.f16_scale = a.vscale;
    p.src = G.Vp;
    p.ld = G.ldv;
    p.dim = DV;
    p.heads = G.Hkv;
    p.grp = 1;
    p.gstride = 0;
    p.hstride = DV;
    p.nseg = 1;
    p.row0[0] = 0;
    p.n[0] = G.P;
    p.col0[0] = 0;
    p.out = const_cast<uint16_t*>(a.VTp);
    p.out_ld = a.ppad;
    p.cols = a.ppad;
    hipError_t e = launch_pack_keys_t(p, st);
    if (e != hipSuccess) return e;
  }
  {
    PackArgs p;
    p.f16_scale = a.vscale;
    p.src = G.Vs;
    p.ld = G.ldv;
    p.dim = DV;
    p.heads = G.Hkv;
    p.grp = 1;
    p.gstride = 0;
    p.hstride = DV;
    p.nseg = G.n_resp;
    for (int i = 0; i < G.n_resp; ++i) {
      p.row0[i] = G.ktok0[i];
      p.n[i] = G.ktok0[i + 1] - G.ktok0[i];
      p.col0[i] = a.spos[i];
    }
    p.out = const_cast<uint16_t*>(a.VTs);
    p.out_ld = a.tpad;
    p.cols = a.tpad;
    hipError_t e = launch_pack_keys_t(p, st);
    if (e != hipSuccess) return e;
  }
  const long long per_xcd = (W + 7) / 8;
  timer_mark(LS_KERNEL_ATTN_FWD, st, false);
  hipLaunchKernelGGL((replay_fwd<D, DV>), dim3((unsigned)(per_xcd * 8)), dim3(64 * kFwdWaves), 0, st, a);
  timer_mark(LS_KERNEL_ATTN_FWD, st, true);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const long long total = (long long)a.geo.T * a.geo.Hq * (DV / 4);
  hipLaunchKernelGGL((replay_fwd_merge<DV>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(FwdArgs& a, int Dqk, int Dv, hipStream_t st) {
  if (Dqk == kWideDqk && Dv == kWideDv) {
    // latent KV: V^T fragments come from the K tiles themselves (no packing pass)
    const hipError_t e = launch_attn_fwd_wide(a, st);
    if (e != hipSuccess || a.splits == 1 || a.qtiles == 0) return e;
    const long long total = (long long)a.geo.T * a.geo.Hq * (kWideDv / 4);
    hipLaunchKernelGGL((replay_fwd_merge<kWideDv>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (Dqk == 64 && Dv == 64) return fwd_go<64, 64>(a, st);
  if (Dqk == 128 && Dv == 128) return fwd_go<128, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lsr
