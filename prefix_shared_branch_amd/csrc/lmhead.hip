// LM head fused with the clipped-GRPO token objective (LongStraw study notes, §1-1, L_policy
// equation). The objective reads each token's logits row over the whole vocabulary; the rows are
// the products logits = H W^T of the last hidden states H [T, d] and the vocabulary projection
// W [V, d]. One call handles a response's tokens in chunks of up to kLmChunk:
//
//   1. logits GEMM (this file): C = W H_c^T on MFMA, 256 x 256 tiles. The epilogue rounds each logit
//      to bf16 and reduces it in registers: per token and 128-word vocabulary slab the max and the
//      sum of exp(x - max), and the target's logit. In the gradient pass it also stores
//      e = exp(x - slab max) (bf16) into the chunk's dlogits buffer. The logits themselves are never
//      written to memory.
//   2. row kernel (grpo_loss.hip): merges a row's slab partials into its log-sum-exp, forms the
//      row's loss term, log-prob, clip flag and dlogits coefficient c, and turns the stored e into
//      dlogits = c (e exp(slab max - lse) - onehot(y)) in place (bf16).
//   3. dH_c = dlogits W and dW += dlogits^T H_c, the same GEMM core with the other operand layouts
//      (split over the vocabulary for dH, summed in a fixed order; dW added in place in fp32).
//
// All three products run in the GEMM core below: 4 waves per workgroup, each wave a 128 x 128 block
// of C as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane), operand tiles of
// 256 rows x 32 k streamed by direct global -> LDS loads through a ring of LDS stages, one workgroup
// barrier per k tile. An operand whose rows run along k is read into MFMA fragments with 16-byte
// LDS reads; one whose rows run along m (or n) with ds_read_b64_tr_b16.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <climits>
#include <cstdint>
#include <type_traits>

#include "../../include/ls_replay.h"
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

constexpr int kBM = 256, kBN = 256, kBK = 32;
#ifndef LM_STAGES
#define LM_STAGES 5
#endif
constexpr int kNst = LM_STAGES;              // LDS ring stages (all 160 KB of a CU's LDS at 5)
constexpr int kOpBytes = 256 * kBK * 2;      // one operand's tile: 16 KB
constexpr int kStage = 2 * kOpBytes;         // A tile, then B tile
constexpr int kLpw = 8;                      // direct loads per wave per stage (32 KB / 1 KB / 4 waves)
constexpr uint32_t kOob = 0xFFFFFFF0u;       // buffer offset past every operand: the load returns zeros
constexpr int kSlabWords = 128;              // vocabulary words per softmax partial (one wave's rows)
constexpr int kGroupM = 8;                   // m tiles per group of the tile order

enum { kKMajor = 0, kMNMajor = 1 };
enum { kEpiSoftmax = 0, kEpiStore = 1, kEpiAccum = 2 };

struct LmGemm {
  // A: kKMajor [M][lda] (k contiguous) or kMNMajor [K][lda] (m contiguous); B likewise with N.
  const uint16_t* a;
  const uint16_t* b;
  uint32_t a_bytes, b_bytes;  // extents: loads past them return zeros
  int32_t lda, ldb;
  int32_t M, N, K;
  int32_t mt, nt, splits, kts;  // tiles along M and N, K splits, k tiles per split (a multiple of kNst)
  // C is stored transposed, out[n][m]. kEpiStore: splits == 1 -> out16 [N][ldo] bf16; else
  // out + split * split_stride, [N][ldo] fp32. kEpiAccum: out [N][ldo] fp32 += C^T.
  float* out;
  uint16_t* out16;
  int64_t ldo, split_stride;
  // kEpiSoftmax (A = W, B = H_c, C = logits^T [V][T_c])
  float2* part;            // [T_c][nslab]: (max, sum exp(x - max)) of each 128-word slab
  int32_t nslab;
  float* xtgt;             // [T_c] the target's logit (bf16 value)
  const int32_t* targets;  // [T_c]
  uint16_t* ebuf;          // [T_c][M] bf16 exp(x - slab max), or null (scoring)
};

// Workgroup -> (m tile, n tile, split). Workgroups are dealt to the 8 XCDs in turn; each XCD gets a
// contiguous range of tile ids. Within a split, ids run over groups of 8 m tiles: down the group's m
// tiles, then to the next n tile. The 32 workgroups an XCD runs at once then cover about 8 m tiles x
// 4 n tiles, whose 12 operand stripes (instead of 32 or more) its L2 serves to all of them.
struct TileId {
  int m, n, s;
};
__device__ __forceinline__ TileId tile_of(const LmGemm& g) {
  const int total = g.mt * g.nt * g.splits;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  const int L = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + loc;
  const int mn = g.mt * g.nt;
  TileId t;
  t.s = L / mn;
  const int r = L - t.s * mn;
  const int gm = r / (kGroupM * g.nt);
  const int i = r - gm * kGroupM * g.nt;
  const int gsz = min(kGroupM, g.mt - gm * kGroupM);
  t.n = i / gsz;
  t.m = gm * kGroupM + (i - t.n * gsz);
  return t;
}

struct Frag {
  bf16x8 a[4], b[4];
};

// Fragment reads. K-major tile: row r (of 256) holds 32 k values as 4 chunks of 16 B, logical chunk
// c at physical chunk c ^ ((r >> 2) & 3), so 16 consecutive rows reading one logical chunk hit 16
// distinct bank groups. MN-major tile: k row r (of 32) holds 256 values as 32 chunks, logical chunk
// c at c ^ (4 (r & 3)), so the 4 rows x 64 B of one ds_read_b64_tr_b16 phase hit all 64 banks.
struct LaneOffsets {
  int k0, k1;   // K-major: step 0 / step 1 lane offset (block and wave offsets are immediates)
  int tr[4];    // MN-major: lane offset of block bi (the row swizzle permutes blocks per lane)
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
  LaneOffsets o;
  const int sw = (lane >> 2) & 3, h = lane >> 5;
  o.k0 = (lane & 31) * 64 + ((h ^ sw) << 4);
  o.k1 = (lane & 31) * 64 + (((2 + h) ^ sw) << 4);
  const int j = lane & 15, kq = j >> 2, g2 = (lane >> 4) & 1;
  const int lb = (8 * h + kq) * 512 + (2 * g2 + ((j & 3) >> 1)) * 16 + (j & 1) * 8;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) o.tr[bi] = lb + 64 * (bi ^ kq);
  return o;
}

// fragment of 32 rows (block bi of wave slot w) for k16 step s from an operand tile at `t`
template <int LAYOUT>
__device__ __forceinline__ bf16x8 read_frag(const char* t, const LaneOffsets& o, int w, int bi, int s) {
  if constexpr (LAYOUT == kKMajor) {
    return lds_b128_as(t, (s ? o.k1 : o.k0) + w * 8192 + bi * 2048);
  } else {
    const int base = o.tr[bi] + 256 * w + 16 * s * 512;
    return join_tr(lds_tr_as(t, base), lds_tr_as(t, base + 4 * 512));
  }
}

// Direct loads of one operand's k tiles, 4 of the 16 1-KB pieces per wave. K-major: piece p holds
// rows 16p .. 16p+15; MN-major: k rows 2p, 2p+1. Per lane and piece, `base` is the byte offset at
// k = 0 and `klim` the first k at which the piece's chunk leaves the operand (INT_MIN for a row or
// column outside it); a tile at k0 loads base + k0 * kstride bytes where k0 < klim, else zeros.
template <int LAYOUT>
struct OperandLoads {
  uint32_t base[4];
  int klim[4];
  uint32_t kstride;  // bytes per unit of k

  __device__ __forceinline__ void init(int wv, int lane, int x0, int xvalid, int ld, int K) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = wv * 4 + q;
      if constexpr (LAYOUT == kKMajor) {
        const int row = x0 + 16 * p + (lane >> 2);
        const int c = (lane & 3) ^ ((lane >> 4) & 3);
        base[q] = (uint32_t)row * (uint32_t)ld * 2u + (uint32_t)c * 16u;
        klim[q] = row < xvalid ? K - 8 * c : INT_MIN;
      } else {
        const int kr = 2 * p + (lane >> 5);
        const int c = (lane & 31) ^ (4 * (kr & 3));
        const int col = x0 + 8 * c;
        base[q] = (uint32_t)kr * (uint32_t)ld * 2u + (uint32_t)col * 2u;
        klim[q] = col < xvalid ? K - kr : INT_MIN;
      }
    }
    kstride = LAYOUT == kKMajor ? 2u : (uint32_t)ld * 2u;
  }
  // piece q of the tile at k0 (k0 = INT_MAX loads nothing: zeros)
  __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t rs, char* dst, int wv, int k0, int q) const {
    const uint32_t off = k0 < klim[q] ? base[q] + (uint32_t)k0 * kstride : kOob;
    lds_dma16_buf(rs, off, dst + (wv * 4 + q) * 1024);
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* dst, int wv, int k0) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_one(rs, dst, wv, k0, q);
  }
};

template <int LA, int LB, int EPI>
__global__ __launch_bounds__(256) void lm_gemm(LmGemm g) {
  // one array per ring stage: an LDS read of one stage does not wait for direct loads into another
  __shared__ __attribute__((aligned(1024))) char st0[kStage];
  __shared__ __attribute__((aligned(1024))) char st1[kStage];
  __shared__ __attribute__((aligned(1024))) char st2[kStage];
  __shared__ __attribute__((aligned(1024))) char st3[kStage];
  __shared__ __attribute__((aligned(1024))) char st4[kNst > 4 ? kStage : 16];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const TileId tid = tile_of(g);
  const int mi = tid.m, ni = tid.n, si = tid.s;
  const int m0 = mi * kBM, n0 = ni * kBN;
  const int kt0 = si * g.kts;
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(g.a, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = buf_rsrc(g.b, g.b_bytes);
  const LaneOffsets lo = lane_offsets(lane);
  OperandLoads<LA> la;
  OperandLoads<LB> lb;
  la.init(wv, lane, m0, g.M, g.lda, g.K);
  lb.init(wv, lane, n0, g.N, g.ldb, g.K);
  const int kts = g.kts;

  auto issue = [&](int kt, char* s) {
    // prefetches past this split's range load nothing
    const int k0 = kt < kts ? (kt0 + kt) * kBK : INT_MAX;
    la.issue(ra, s, wv, k0);
    lb.issue(rb, s + kOpBytes, wv, k0);
  };
  auto frags = [&](Frag& f, const char* s, int step) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) f.a[bi] = read_frag<LA>(s, lo, wm, bi, step);
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) f.b[bi] = read_frag<LB>(s + kOpBytes, lo, wn, bi, step);
  };
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto mfmas = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
  };

  issue(0, st0);
  issue(1, st1);
  issue(2, st2);
  issue(3, st3);
  if constexpr (kNst > 4) issue(4, st4);
  wait_vmem_le<(kNst - 1) * kLpw>();
  bare_barrier();
  Frag f0, f1;
  frags(f0, st0, 0);
  wait_lds();
  // One k tile in two steps of 16 MFMAs. Step 0 runs on f0 while f1 is read (step 1 of this tile);
  // then, once every wave has read this tile's stage and the next tile has landed, step 1 runs on f1
  // while the stage is refilled (tile kt + kNst) and f0 is read (step 0 of the next tile). Each
  // LDS read and direct load is issued between two MFMAs, so the wave issues them while the matrix
  // core is busy instead of in a burst at the barrier. (Scheduling barriers hold this order.)
  auto read_one = [&](Frag& f, const char* s, int step, int p) {
    if (p < 4) f.a[p] = read_frag<LA>(s, lo, wm, p, step);
    else f.b[p - 4] = read_frag<LB>(s + kOpBytes, lo, wn, p - 4, step);
  };
  auto mfma_pair = [&](const Frag& f, int p) {
#pragma unroll
    for (int q = 2 * p; q < 2 * p + 2; ++q) acc[q >> 2][q & 3] = mfma32(f.a[q >> 2], f.b[q & 3], acc[q >> 2][q & 3]);
  };
  auto tile = [&](int kt, char* cur, char* nxt) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      read_one(f1, cur, 1, p);
      __builtin_amdgcn_sched_barrier(0);
      mfma_pair(f0, p);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lds();
    wait_vmem_le<(kNst - 2) * kLpw>();
    bare_barrier();
    const int k0 = kt + kNst < kts ? (kt0 + kt + kNst) * kBK : INT_MAX;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (p < 4) la.issue_one(ra, cur, wv, k0, p);
      else lb.issue_one(rb, cur + kOpBytes, wv, k0, p - 4);
      read_one(f0, nxt, 0, p);
      __builtin_amdgcn_sched_barrier(0);
      mfma_pair(f1, p);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lds();
  };
  for (int kt = 0; kt < kts; kt += kNst) {
    tile(kt, st0, st1);
    tile(kt + 1, st1, st2);
    tile(kt + 2, st2, st3);
    if constexpr (kNst > 4) {
      tile(kt + 3, st3, st4);
      tile(kt + 4, st4, st0);
    } else {
      tile(kt + 3, st3, st0);
    }
  }
  wait_vmem();

  const int h = lane >> 5, c = lane & 31;
  if constexpr (EPI == kEpiSoftmax) {
    // every wave is past its last LDS reads and direct loads: the ring is free for the epilogue
    __syncthreads();
    float* xs = reinterpret_cast<float*>((wv < 2 ? st0 : st1) + (wv & 1) * 16384);
    const int slab = 2 * mi + wm;
    const int v0 = m0 + wm * 128;
    const int vlim = g.M - v0;  // rows of this wave's slab inside the vocabulary
    const __amdgpu_buffer_rsrc_t re = buf_rsrc(g.ebuf, g.ebuf ? (int64_t)g.N * g.M * 2 : 0);
    auto epi = [&](auto masked_c) {
      constexpr bool kMasked = decltype(masked_c)::value;
      (void)vlim;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int t = n0 + wn * 128 + nb * 32 + c;
        const bool t_ok = t < g.N;
        // logits rounded to bf16 (the precision the objective reads); rows past V are -inf
        float x[4][16];
        float mx = -INFINITY;
        // rows of the slab left for this lane half: value (mb, r) is valid iff its offset
        // mb*32 + 8(r/4) + r%4 < lim. Each use takes its own opaque copy of lim, so the compares
        // are formed at their use rather than kept as 64 live lane masks.
        int lim = vlim - 4 * h;
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const uint32_t u = pack_bf16x2(acc[mb][nb][r], acc[mb][nb][r + 1]);
            x[mb][r] = bf16_lo(u);
            x[mb][r + 1] = bf16_hi(u);
            if constexpr (kMasked) {
              const int rel = mb * 32 + 8 * (r >> 2) + (r & 3);
              x[mb][r] = rel < lim ? x[mb][r] : -INFINITY;
              x[mb][r + 1] = rel + 1 < lim ? x[mb][r + 1] : -INFINITY;
            }
            mx = fmaxf(mx, fmaxf(x[mb][r], x[mb][r + 1]));
          }
        __builtin_amdgcn_sched_barrier(0);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mb2 = mx * kLog2e;
        float s = 0.0f;
        // e stores through a resource over the chunk's buffer (empty when scoring); a token past
        // the chunk gets an offset outside it
        const uint32_t eo = t_ok ? ((uint32_t)t * (uint32_t)g.M + (uint32_t)v0) * 2u : kOob;
        int lim2 = vlim - 4 * h;
        asm volatile("" : "+v"(lim2));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float e[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              e[q] = fast_exp2(__builtin_fmaf(x[mb][4 * i + q], kLog2e, -mb2));
              s += e[q];
            }
            const int rel = mb * 32 + 8 * i;
            const u32x2 w = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
            const uint32_t o =
                (kMasked && rel >= lim2) || eo == kOob ? kOob : eo + (uint32_t)(rel + 4 * h) * 2u;
            __builtin_amdgcn_raw_buffer_store_b64(w, re, (int)o, 0, 0);
          }
        __builtin_amdgcn_sched_barrier(0);
        s += __shfl_xor(s, 32, 64);
        if (h == 0 && t_ok && slab < g.nslab) g.part[(int64_t)t * g.nslab + slab] = make_float2(mx, s);
        // the target's logit: held by one lane of one wave in the whole grid; that wave passes its
        // values through LDS to pick it out
        const int y = t_ok ? g.targets[t] : -1;
        const int ry = y - v0;
        const bool mine = ry >= 0 && ry < 128 && ry < vlim && ((ry >> 2) & 1) == h;
        if (__any(mine)) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) xs[(mb * 16 + r) * 64 + lane] = x[mb][r];
          const int yi = (ry >> 5) * 16 + ((ry >> 3) & 3) * 4 + (ry & 3);
          if (mine) g.xtgt[t] = xs[(yi & 63) * 64 + lane];
        }
      }
    };
    epi(std::true_type{});
  } else {
    // C is stored transposed, out[n][m]: a lane's registers 4j .. 4j+3 are 4 consecutive m of one n,
    // one 16-byte (fp32) or 8-byte (bf16) access. The accesses go through a buffer resource over this
    // wave's 128 rows n of the output: rows past N fall outside it and columns past M get an offset
    // outside it, so no access needs a branch.
    const bool b16 = EPI == kEpiStore && g.splits == 1;
    const int esz = b16 ? 2 : 4;
    const int nbase = n0 + wn * 128;
    const int64_t rows_left = (int64_t)g.N - nbase;
    const int64_t span = rows_left <= 0 ? 0 : rows_left * g.ldo * esz;
    char* obase = b16 ? reinterpret_cast<char*>(g.out16) + (int64_t)nbase * g.ldo * 2
                      : reinterpret_cast<char*>(g.out) +
                            ((EPI == kEpiStore ? si * g.split_stride : 0) + (int64_t)nbase * g.ldo) * 4;
    const __amdgpu_buffer_rsrc_t ro = buf_rsrc(obase, span);
    const uint32_t rowb = (uint32_t)g.ldo * (uint32_t)esz;
    const int mw = m0 + wm * 128 + 4 * h;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint32_t orow = (uint32_t)(nb * 32 + c) * rowb;
      if constexpr (EPI == kEpiAccum) {
        // all 16 loads of the column block first, then the adds and stores
        f32x4 v[4][4];
        uint32_t off[4][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = mw + mb * 32 + 8 * i;
            off[mb][i] = m < g.M ? orow + (uint32_t)m * 4u : kOob;
            v[mb][i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, (int)off[mb][i], 0, 0));
          }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 w = v[mb][i];
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] += acc[mb][nb][4 * i + q];
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), ro, (int)off[mb][i], 0, 0);
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = mw + mb * 32 + 8 * i;
            const uint32_t o = m < g.M ? orow + (uint32_t)m * (uint32_t)esz : kOob;
            const f32x16& a = acc[mb][nb];
            if (b16) {
              const u32x2 w = {pack_bf16x2(a[4 * i], a[4 * i + 1]), pack_bf16x2(a[4 * i + 2], a[4 * i + 3])};
              __builtin_amdgcn_raw_buffer_store_b64(w, ro, (int)o, 0, 0);
            } else {
              const f32x4 w = {a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]};
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), ro, (int)o, 0, 0);
            }
          }
      }
      // one column block at a time: its offsets and loaded values are all that is live
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// dH = bf16(sum over splits of the fp32 partials), in split order; 4 consecutive values per thread
__global__ __launch_bounds__(256) void lm_split_sum(const float* part, int splits, int64_t stride, int64_t n4,
                                                    uint16_t* out) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 s = *reinterpret_cast<const f32x4*>(part + 4 * i);
    for (int k = 1; k < splits; ++k) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + k * stride + 4 * i);
      s[0] += v[0];
      s[1] += v[1];
      s[2] += v[2];
      s[3] += v[3];
    }
    *reinterpret_cast<u32x2*>(out + 4 * i) = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  }
}

template <int LA, int LB, int EPI>
hipError_t go(const LmGemm& g, hipStream_t st) {
  const unsigned grid = (unsigned)(g.mt * g.nt * g.splits);
  hipLaunchKernelGGL((lm_gemm<LA, LB, EPI>), dim3(grid), dim3(256), 0, st, g);
  return hipGetLastError();
}

constexpr int64_t kLmChunk = 4096;             // tokens per chunk
constexpr int32_t kLmMaxVocab = 1 << 24;
constexpr int32_t kLmMaxHidden = 65536;
constexpr int kMaxSplits = 8;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }
int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
int round_up(int a, int b) { return (a + b - 1) / b * b; }

// tokens per chunk: at most kLmChunk, and a chunk's [T_c, V] bf16 buffer stays under 2 GiB (32-bit
// buffer offsets)
int64_t chunk_tokens(int64_t T, int32_t V) {
  int64_t tc = ((int64_t)1 << 30) / V;
  if (tc > kLmChunk) tc = kLmChunk;
  return T < tc ? T : tc;
}

// K splits of the dH product (K = V): enough workgroups for whole rounds over the 256 CUs, each split
// at least 64 k tiles, at most max_splits
void dh_split(int64_t tc, int32_t V, int32_t d, int max_splits, int* splits, int* kts) {
  const int tiles = cdiv(tc, kBM) * cdiv(d, kBN);
  const int ktiles = cdiv(V, kBK);
  int best = 1;
  double best_eff = 0.0;
  for (int s = 1; s <= max_splits; ++s) {
    if (s > 1 && ktiles / s < 64) break;
    const int wgs = tiles * s;
    const double eff = (double)wgs / (double)(cdiv(wgs, 256) * 256);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = s;
    }
  }
  int k = round_up(cdiv(ktiles, best), kNst);
  *splits = cdiv(ktiles, k);
  *kts = k;
}

struct LmLayout {
  int64_t tc;
  int nslab, splits, kts_dh;
  size_t ebuf, part, xtgt, row_loss, dhpart, total;
};

LmLayout lm_layout(int64_t T, int32_t V, int32_t d) {
  LmLayout l;
  l.tc = chunk_tokens(T, V);
  const int64_t tc = l.tc > 0 ? l.tc : 1;
  l.nslab = cdiv(V, kSlabWords);
  dh_split(tc, V, d, kMaxSplits, &l.splits, &l.kts_dh);
  l.ebuf = 0;
  l.part = l.ebuf + align256((size_t)tc * V * 2);
  l.xtgt = l.part + align256((size_t)tc * l.nslab * 8);
  l.row_loss = l.xtgt + align256((size_t)tc * 4);
  l.dhpart = l.row_loss + align256(grpo_workspace_bytes(tc));
  l.total = l.dhpart + (l.splits > 1 ? align256((size_t)l.splits * tc * d * 4) : 0);
  return l;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

}  // namespace lsr

using namespace lsr;

extern "C" {

int ls_grpo_lmhead_workspace_bytes(int64_t T, int32_t V, int32_t d, size_t* bytes) {
  if (!bytes || T < 0 || V < 1 || d < 1) return LS_ERR_INVALID_ARG;
  *bytes = lm_layout(T, V, d).total;
  return LS_OK;
}

int ls_grpo_lmhead_loss(void* stream, int32_t V, int32_t d, int32_t G, const int32_t* R, const float* rewards,
                        float eps, int32_t first, int32_t count, const void* H, const void* W,
                        const int32_t* targets, const float* old_logp, float* loss_accum, void* dH,
                        float* dW_accum, float* logp_out, uint8_t* clipped_out, void* workspace,
                        size_t workspace_bytes) {
  if (V < 1 || d < 1 || G < 1 || !R || !rewards) return LS_ERR_INVALID_ARG;
  if (V > kLmMaxVocab || d > kLmMaxHidden) return LS_ERR_UNSUPPORTED;
  if ((V % 8) != 0 || (d % 8) != 0) return LS_ERR_UNSUPPORTED;   // 16-byte operand chunks
  if (!std::isfinite(eps) || !(eps > 0.0f) || !(eps < 1.0f)) return LS_ERR_INVALID_ARG;
  if (first < 0 || count < 1 || (int64_t)first + count > G) return LS_ERR_INVALID_ARG;
  for (int i = 0; i < G; ++i)
    if (R[i] < 1 || !std::isfinite(rewards[i])) return LS_ERR_INVALID_ARG;
  if ((dH == nullptr) != (dW_accum == nullptr)) return LS_ERR_INVALID_ARG;
  int64_t T = 0;
  for (int i = first; i < first + count; ++i) T += R[i];
  if (T > INT32_MAX || (int64_t)V * d > INT32_MAX) return LS_ERR_UNSUPPORTED;
  if (!H || !W || !targets || !old_logp || !loss_accum) return LS_ERR_INVALID_ARG;
  const void* a16[] = {H, W, dH, dW_accum};
  for (const void* p : a16)
    if (p && !aligned(p, 16)) return LS_ERR_INVALID_ARG;
  if (!aligned(targets, 4) || !aligned(old_logp, 4) || !aligned(loss_accum, 4) || (logp_out && !aligned(logp_out, 4)))
    return LS_ERR_INVALID_ARG;
  const LmLayout lay = lm_layout(T, V, d);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total) return LS_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint16_t* ebuf = reinterpret_cast<uint16_t*>(ws + lay.ebuf);
  float2* part = reinterpret_cast<float2*>(ws + lay.part);
  float* xtgt = reinterpret_cast<float*>(ws + lay.xtgt);
  float* row_loss = reinterpret_cast<float*>(ws + lay.row_loss);
  float* dhpart = reinterpret_cast<float*>(ws + lay.dhpart);
  const uint16_t* Hb = static_cast<const uint16_t*>(H);
  const uint16_t* Wb = static_cast<const uint16_t*>(W);
  uint16_t* dHb = static_cast<uint16_t*>(dH);
  const bool grad = dH != nullptr;
  const uint32_t w_bytes = (uint32_t)((int64_t)V * d * 2);

  for (int64_t c0 = 0; c0 < T; c0 += lay.tc) {
    const int tc = (int)((T - c0) < lay.tc ? (T - c0) : lay.tc);
    const uint16_t* Hc = Hb + c0 * d;
    const uint32_t h_bytes = (uint32_t)((int64_t)tc * d * 2);
    const uint32_t e_bytes = (uint32_t)((int64_t)tc * V * 2);

    // 1. logits^T [V][tc] = W H_c^T with the softmax partials in the epilogue
    LmGemm g = {};
    g.a = Wb;
    g.a_bytes = w_bytes;
    g.lda = d;
    g.b = Hc;
    g.b_bytes = h_bytes;
    g.ldb = d;
    g.M = V;
    g.N = tc;
    g.K = d;
    g.mt = cdiv(V, kBM);
    g.nt = cdiv(tc, kBN);
    g.splits = 1;
    g.kts = round_up(cdiv(d, kBK), kNst);
    g.part = part;
    g.nslab = lay.nslab;
    g.xtgt = xtgt;
    g.targets = targets + c0;
    g.ebuf = grad ? ebuf : nullptr;
    if (go<kKMajor, kKMajor, kEpiSoftmax>(g, st) != hipSuccess) return LS_ERR_HIP;

    // 2. per row: log-sum-exp, loss term, log-prob, clip flag; dlogits in place of e
    const bool ok = grpo_batches(G, R, rewards, eps, first, count, c0, c0 + tc, [&](GrpoArgs& a, int64_t brow0) {
      const int64_t r0 = brow0 - c0;
      LmRowArgs ra;
      a.V = V;
      a.logits = nullptr;
      a.dlogits = grad ? ebuf + r0 * V : nullptr;
      a.targets = targets + brow0;
      a.old_logp = old_logp + brow0;
      a.row_loss = row_loss + r0;
      a.logp_out = logp_out ? logp_out + brow0 : nullptr;
      a.clipped_out = clipped_out ? clipped_out + brow0 : nullptr;
      a.loss_accum = loss_accum;
      ra.g = a;
      ra.part = part + r0 * lay.nslab;
      ra.nslab = lay.nslab;
      ra.xtgt = xtgt + r0;
      return launch_lm_rows(ra, st) == hipSuccess;
    });
    if (!ok) return LS_ERR_HIP;
    if (!grad) continue;

    // 3. dH_c [tc][d] = dlogits [tc][V] W [V][d], formed as C = W^T dlogits^T [d][tc] and stored
    //    transposed; split over V, the partials summed in split order
    LmGemm h = {};
    h.a = Wb;
    h.a_bytes = w_bytes;
    h.lda = d;
    h.b = ebuf;
    h.b_bytes = e_bytes;
    h.ldb = V;
    h.M = d;
    h.N = tc;
    h.K = V;
    h.mt = cdiv(d, kBM);
    h.nt = cdiv(tc, kBN);
    // the partial buffer holds lay.splits x lay.tc rows of d: a shorter last chunk may take more splits
    const int64_t cap = lay.splits > 1 ? (int64_t)lay.splits * lay.tc : 0;
    const int max_splits = (int)std::min<int64_t>(kMaxSplits, std::max<int64_t>(1, cap / tc));
    dh_split(tc, V, d, max_splits, &h.splits, &h.kts);
    h.out = dhpart;
    h.out16 = dHb + c0 * d;
    h.ldo = d;
    h.split_stride = (int64_t)tc * d;
    if (go<kMNMajor, kKMajor, kEpiStore>(h, st) != hipSuccess) return LS_ERR_HIP;
    if (h.splits > 1) {
      const int64_t n4 = (int64_t)tc * d / 4;
      const int64_t grid = std::min<int64_t>((n4 + 255) / 256, 4096);
      hipLaunchKernelGGL(lm_split_sum, dim3((unsigned)grid), dim3(256), 0, st, (const float*)dhpart, h.splits,
                         h.split_stride, n4, dHb + c0 * d);
      if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
    }

    // 4. dW [V][d] += dlogits^T H_c, formed as C = H_c^T dlogits [d][V] and added in transposed;
    //    both operands are read along their rows (k = tokens)
    LmGemm w = {};
    w.a = Hc;
    w.a_bytes = h_bytes;
    w.lda = d;
    w.b = ebuf;
    w.b_bytes = e_bytes;
    w.ldb = V;
    w.M = d;
    w.N = V;
    w.K = tc;
    w.mt = cdiv(d, kBM);
    w.nt = cdiv(V, kBN);
    w.splits = 1;
    w.kts = round_up(cdiv(tc, kBK), kNst);
    w.out = dW_accum;
    w.ldo = d;
    if (go<kMNMajor, kMNMajor, kEpiAccum>(w, st) != hipSuccess) return LS_ERR_HIP;
  }
  return LS_OK;
}

}  // extern "C"
