// Fused clipped-GRPO token objective (LongStraw study notes, §1-1, L_policy equation).
//
// A workgroup handles one token row at a time. The bf16 logits row is read from HBM exactly once into
// VGPRs (16-byte loads, consecutive threads on consecutive 16-byte chunks); the row max
// and the sum of exponentials are wave reductions combined through LDS; the exponentials replace
// the logits in the registers (bf16), and the dlogits row is produced from them with one multiply
// per element and written once. HBM traffic per token is the algorithmic minimum: 2V bytes in, 2V
// bytes out, plus target, old log-prob, log-prob.
//
// Per row t of response i (A = A_i, w = 1/(G R_i)):
//   lse = max + log(sum exp(x - max)),  logp = x_y - lse,  rho = exp(logp - old)
//   term = min(rho A, clip(rho, 1-eps, 1+eps) A);  row_loss = -w term
//   clipped = clip(rho) A < rho A  (then the gradient is zero)
//   dlogits = c (softmax(x) - onehot(y)),  c = clipped ? 0 : w A rho
// The loss is summed by a second single-workgroup kernel in a fixed order (deterministic).
// Without a dlogits buffer (scoring old or reference policies) the row kernels stop after the
// per-row outputs: the logits are read once and nothing of size V is written.
#include "common.h"
#include "grpo_row.h"
#include "kernels.h"

namespace lsr {

namespace {

template <int NT>
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  constexpr int NW = NT / 64;
  v = is_max ? wave_max(v) : wave_sum(v);
  const int wv = threadIdx.x / 64;
  __syncthreads();  // red[] may still be read from a previous reduction
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) r = is_max ? fmaxf(r, red[k]) : r + red[k];
  return r;
}

// Vector path: V % 8 == 0, 16-byte aligned rows; NCH 16-byte chunks per thread in registers.
// Rows are read through a buffer resource over the row (no per-chunk 64-bit addresses stay live);
// chunks past the row end read zeros, are masked to -inf after the load and never stored.
// A row fills most of a CU's registers at the large vocabularies, so one workgroup per CU loops
// over rows (row = blockIdx.x, + gridDim.x, ...). In the gradient pass the registers of chunk j
// are reloaded with chunk j of the next row as soon as chunk j's dlogits are stored: the next
// row streams in while this row's output is formed and written, and the stores drain while the
// next row's max and sum are taken.
template <int NT, int NCH, bool SCORE>
__global__ __launch_bounds__(NT) void grpo_rows_vec(GrpoArgs a) {
  __shared__ float red[NT / 64];
  const int nch = a.V >> 3;
  const int voff = threadIdx.x * 16;
  const int64_t stride = gridDim.x;
  int64_t row = blockIdx.x;
  if (row >= a.T) return;
  auto row_src = [&](int64_t r) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a.logits + r * (int64_t)a.V), 0, a.V * 2, kBufferWord3);
  };

  // 16 bytes of chunk j of a row for this thread. The whole byte offset goes in the VGPR offset,
  // which the buffer range check covers (the SGPR offset is not range-checked), so chunks past the
  // row end read zeros without touching memory. The offset is materialised at the load (opaque z)
  // rather than hoisted out of the row loop as one live register per chunk.
  auto ld_chunk = [&](__amdgpu_buffer_rsrc_t r, int j, int z) {
    int o = voff + j * NT * 16 + z;
    asm volatile("" : "+v"(o));
    return __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, kSlc);
  };
  // Per-row scalars (target, target logit, old log-prob) of this workgroup's first NT rows, one row
  // per thread, preloaded into LDS before the row loop: those rows read them where they are used,
  // so no row waits for the dependent gather of its target logit or for its old_logp, and none of
  // them holds a register across the row's passes. Rows past the first NT (calls of more than
  // NT x grid rows) load them at their use.
  __shared__ int s_y[NT];
  __shared__ float s_xy[NT], s_old[NT];
  {
    const int64_t r = row + (int64_t)threadIdx.x * stride;
    if (r < a.T) {
      const int y = a.targets[r];
      s_y[threadIdx.x] = y;
      s_xy[threadIdx.x] = (y >= 0 && y < a.V) ? bf16_to_f32(a.logits[r * (int64_t)a.V + y]) : 0.0f;
      s_old[threadIdx.x] = a.old_logp[r];
    }
    // published by the barriers of the first row's reductions, before their first read
  }
  u32x4 v[NCH];
  {
    const __amdgpu_buffer_rsrc_t src = row_src(row);
#pragma unroll
    for (int j = 0; j < NCH; ++j) v[j] = ld_chunk(src, j, 0);
  }
  for (int it = 0;; ++it) {
    // chunk offsets and chunk-validity masks are formed from a value the compiler cannot see
    // through, so they are materialised at their use instead of being hoisted out of the row loop
    // (where 19 lane masks and offsets would be live SGPRs across it)
    int zoff = 0;
    asm volatile("" : "+s"(zoff));
    const int64_t next = row + stride;
    const bool more = next < a.T;  // uniform
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      if ((int)threadIdx.x + j * NT + zoff >= nch) v[j] = u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};

    // after the last row the reloads go through an empty resource: no memory access, zeros returned
    const __amdgpu_buffer_rsrc_t nsrc =
        more ? row_src(next) : __builtin_amdgcn_make_buffer_rsrc((void*)a.logits, 0, 0, kBufferWord3);
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      m = fmaxf(m, fmaxf(fmaxf(bf16_lo(v[j].x), bf16_hi(v[j].x)), fmaxf(bf16_lo(v[j].y), bf16_hi(v[j].y))));
      m = fmaxf(m, fmaxf(fmaxf(bf16_lo(v[j].z), bf16_hi(v[j].z)), fmaxf(bf16_lo(v[j].w), bf16_hi(v[j].w))));
    }
    m = block_reduce<NT>(m, red, true);
    // keep only the packed row live across the passes (re-derive floats on use, no spills)
#pragma unroll
    for (int j = 0; j < NCH; ++j) asm volatile("" : "+v"(v[j]));
    const float mb = m * kLog2e;
    // e = exp2((x - max) log2 e), summed; the gradient pass keeps e (bf16) in place of the logits, so
    // each element takes one exponential; the scoring pass needs only the sum, and reloads each
    // chunk's registers with the next row's chunk as soon as its exponentials are summed. Both passes
    // sum in the same order, so scoring gives bit-identical log-probs and loss.
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float e0 = fast_exp2(__builtin_fmaf(bf16_lo(v[j][q]), kLog2e, -mb));
        const float e1 = fast_exp2(__builtin_fmaf(bf16_hi(v[j][q]), kLog2e, -mb));
        s += e0;
        s += e1;
        if (!SCORE) v[j][q] = pack_bf16x2(e0, e1);
      }
      if (SCORE) {
        // the reload of chunk j after its exponentials (not hoisted above them: two copies live)
        __builtin_amdgcn_sched_barrier(0);
        v[j] = ld_chunk(nsrc, j, zoff);
      } else {
        asm volatile("" : "+v"(v[j]));  // the packed exponentials are formed here, not at their use
      }
      // chunk by chunk, so that only one chunk's floats are live beside the packed row
      __builtin_amdgcn_sched_barrier(0);
    }
    s = block_reduce<NT>(s, red, false);
    const float lse = m + fast_log2(s) * kLn2;
    int y;
    float xy, old_lp;
    if (it < NT) {
      y = s_y[it];
      xy = s_xy[it];
      old_lp = s_old[it];
    } else {
      y = a.targets[row];
      xy = (y >= 0 && y < a.V) ? bf16_to_f32(a.logits[row * (int64_t)a.V + y]) : 0.0f;
      old_lp = a.old_logp[row];
    }
    const bool y_ok = (y >= 0) && (y < a.V);
    const float c = row_scalar(a, row, xy, y_ok, lse, old_lp, threadIdx.x == 0);
    if (!SCORE) {
      // dlogits = c softmax(x) = (c / sum) e, with the target's element c (p_y - 1) formed from the
      // logit itself
      const float f = c / s;
      const float lb = lse * kLog2e;
#pragma unroll
      for (int j = 0; j < NCH; ++j) asm volatile("" : "+v"(v[j]));
      const int yc = y_ok ? (y >> 3) : -1;  // the chunk holding the target (one lane of the row)
      // Stores are global (FLAT) stores: the compiler protects their data registers from the
      // next VALU write, which it does not do for buffer stores with an SGPR offset.
      char* dst = reinterpret_cast<char*>(a.dlogits + row * (int64_t)a.V);
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int cj = (int)threadIdx.x + j * NT + zoff;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(f * bf16_lo(v[j][q]), f * bf16_hi(v[j][q]));
        if (cj == yc) {
          // the one-hot term (one lane of the row): the target's element becomes c (p_y - 1)
          const float py = fast_exp2(__builtin_fmaf(xy, kLog2e, -lb)) - 1.0f;
          const uint32_t t = pack_bf16x2(c * py, 0.0f) & 0xffffu;
          const int qy = (y & 7) >> 1;
          const uint32_t keep = (y & 1) ? 0x0000ffffu : 0xffff0000u;
          const uint32_t ins = (y & 1) ? (t << 16) : t;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = (q == qy) ? ((o[q] & keep) | ins) : o[q];
        }
        if (cj < nch) __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst + voff + j * NT * 16));
        v[j] = ld_chunk(nsrc, j, zoff);
        // chunk by chunk: the reload of chunk j is not hoisted above the output of chunks < j,
        // which would keep two rows' chunks live at once
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!more) break;
    row = next;
  }
}

// Rows too long for registers (V > 196608, V % 8 == 0, 16-byte aligned): two passes over the row.
// The first keeps a per-thread running max and sum of exponentials (the sum rescaled whenever the
// max moves) and combines them over the workgroup; the second forms dlogits. The row is read twice
// and written once.
template <int NT>
__global__ __launch_bounds__(NT) void grpo_rows_stream(GrpoArgs a) {
  __shared__ float red[NT / 64];
  const int64_t row = blockIdx.x;
  const int nch = a.V >> 3;
  const u32x4* x = reinterpret_cast<const u32x4*>(a.logits + row * (int64_t)a.V);
  const int y = a.targets[row];
  const bool y_ok = (y >= 0) && (y < a.V);
  float m = -INFINITY, s = 0.0f;
  for (int cj = threadIdx.x; cj < nch; cj += NT) {
    const u32x4 v = x[cj];
    float cm = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) cm = fmaxf(cm, fmaxf(bf16_lo(v[q]), bf16_hi(v[q])));
    if (cm > m) {
      s = (m == -INFINITY) ? 0.0f : s * fast_exp2((m - cm) * kLog2e);
      m = cm;
    }
    if (m != -INFINITY) {  // while every value so far is -inf the sum stays 0
      const float mb = m * kLog2e;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s += fast_exp2(__builtin_fmaf(bf16_lo(v[q]), kLog2e, -mb));
        s += fast_exp2(__builtin_fmaf(bf16_hi(v[q]), kLog2e, -mb));
      }
    }
  }
  const float M = block_reduce<NT>(m, red, true);
  const float sl = (m == -INFINITY) ? 0.0f : s * fast_exp2((m - M) * kLog2e);
  const float S = block_reduce<NT>(sl, red, false);
  const float lse = M + fast_log2(S) * kLn2;
  const float xy = y_ok ? bf16_to_f32(a.logits[row * (int64_t)a.V + y]) : 0.0f;
  const float c = row_scalar(a, row, xy, y_ok, lse, a.old_logp[row], threadIdx.x == 0);
  if (a.dlogits == nullptr) return;  // scoring only: no gradient pass
  const float lb = lse * kLog2e;
  const int yc = y_ok ? (y >> 3) : -1;
  u32x4* d = reinterpret_cast<u32x4*>(a.dlogits + row * (int64_t)a.V);
  for (int cj = threadIdx.x; cj < nch; cj += NT) {
    const u32x4 v = x[cj];
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float p0 = fast_exp2(__builtin_fmaf(bf16_lo(v[q]), kLog2e, -lb));
      const float p1 = fast_exp2(__builtin_fmaf(bf16_hi(v[q]), kLog2e, -lb));
      o[q] = pack_bf16x2(c * p0, c * p1);
    }
    if (cj == yc) {  // the one-hot term, as in grpo_rows_vec
      const float py = fast_exp2(__builtin_fmaf(xy, kLog2e, -lb)) - 1.0f;
      const uint32_t t = pack_bf16x2(c * py, 0.0f) & 0xffffu;
      const int qy = (y & 7) >> 1;
      const uint32_t keep = (y & 1) ? 0x0000ffffu : 0xffff0000u;
      const uint32_t ins = (y & 1) ? (t << 16) : t;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = (q == qy) ? ((o[q] & keep) | ins) : o[q];
    }
    __builtin_nontemporal_store(o, d + cj);
  }
}

// Element-wise path for any V / alignment: three passes over the row (L2-resident).
__global__ __launch_bounds__(256) void grpo_rows_scalar(GrpoArgs a) {
  constexpr int NT = 256;
  __shared__ float red[NT / 64];
  const int64_t row = blockIdx.x;
  const uint16_t* x = a.logits + row * (int64_t)a.V;
  const int y = a.targets[row];
  const bool y_ok = (y >= 0) && (y < a.V);
  float m = -INFINITY;
  for (int e = threadIdx.x; e < a.V; e += NT) m = fmaxf(m, bf16_to_f32(x[e]));
  m = block_reduce<NT>(m, red, true);
  float s = 0.0f;
  for (int e = threadIdx.x; e < a.V; e += NT) s += fast_exp2((bf16_to_f32(x[e]) - m) * kLog2e);
  s = block_reduce<NT>(s, red, false);
  const float lse = m + fast_log2(s) * kLn2;
  const float xy = y_ok ? bf16_to_f32(x[y]) : 0.0f;
  const float c = row_scalar(a, row, xy, y_ok, lse, a.old_logp[row], threadIdx.x == 0);
  if (a.dlogits == nullptr) return;  // scoring only: no gradient pass
  uint16_t* d = a.dlogits + row * (int64_t)a.V;
  for (int e = threadIdx.x; e < a.V; e += NT) {
    float p = fast_exp2((bf16_to_f32(x[e]) - lse) * kLog2e) - ((e == y) ? 1.0f : 0.0f);
    d[e] = (uint16_t)(pack_bf16x2(c * p, 0.0f) & 0xffffu);
  }
}

// Fixed-order sum of the per-row losses, added to *loss_accum.
__global__ __launch_bounds__(256) void grpo_sum(const float* row_loss, int64_t T, float* loss_accum) {
  __shared__ double part[256];
  double acc = 0.0;
  for (int64_t r = threadIdx.x; r < T; r += 256) acc += (double)row_loss[r];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss_accum = (float)((double)*loss_accum + part[0]);
}

// LM-head row pass: one workgroup per row. The row's log-sum-exp merges the slab partials
// (max_k, s_k) of the logits GEMM: lse = M + log sum_k s_k exp(max_k - M), M = max_k max_k. With a
// dlogits buffer, each 16-byte chunk of stored e = exp(x - slab max) becomes
// dlogits = c exp(x - lse) = c exp(slab max - lse) e, the target's element c (p_y - 1).
template <int NT>
__global__ __launch_bounds__(NT) void lm_rows(LmRowArgs la) {
  __shared__ float red[NT / 64];
  const GrpoArgs& a = la.g;
  const int64_t row = blockIdx.x;
  const float2* p = la.part + row * la.nslab;
  float m = -INFINITY;
  for (int i = threadIdx.x; i < la.nslab; i += NT) m = fmaxf(m, p[i].x);
  m = block_reduce<NT>(m, red, true);
  const float mb = m * kLog2e;
  float s = 0.0f;
  for (int i = threadIdx.x; i < la.nslab; i += NT) {
    const float2 q = p[i];
    s += q.y * fast_exp2(__builtin_fmaf(q.x, kLog2e, -mb));
  }
  s = block_reduce<NT>(s, red, false);
  const float lse = m + fast_log2(s) * kLn2;
  const int y = a.targets[row];
  const bool y_ok = (y >= 0) && (y < a.V);
  const float xy = y_ok ? la.xtgt[row] : 0.0f;
  const float c = row_scalar(a, row, xy, y_ok, lse, a.old_logp[row], threadIdx.x == 0);
  if (a.dlogits == nullptr) return;  // scoring only
  const float lb = lse * kLog2e;
  const int nch = a.V >> 3;
  const int yc = y_ok ? (y >> 3) : -1;
  u32x4* d = reinterpret_cast<u32x4*>(a.dlogits + row * (int64_t)a.V);
#pragma unroll 4
  for (int cj = threadIdx.x; cj < nch; cj += NT) {
    const float f = c * fast_exp2(__builtin_fmaf(p[cj >> 4].x, kLog2e, -lb));
    const u32x4 v = d[cj];
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(f * bf16_lo(v[q]), f * bf16_hi(v[q]));
    if (cj == yc) {  // the one-hot term, as in grpo_rows_vec
      const float py = fast_exp2(__builtin_fmaf(xy, kLog2e, -lb)) - 1.0f;
      const uint32_t t = pack_bf16x2(c * py, 0.0f) & 0xffffu;
      const int qy = (y & 7) >> 1;
      const uint32_t keep = (y & 1) ? 0x0000ffffu : 0xffff0000u;
      const uint32_t ins = (y & 1) ? (t << 16) : t;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = (q == qy) ? ((o[q] & keep) | ins) : o[q];
    }
    d[cj] = o;
  }
}

// Workgroups of the row loop: one per CU at 1024 threads (a row fills most of a CU's registers),
// four per CU at 256 threads.
constexpr int64_t kLossCUs = 256;

template <int NT, int NCH>
hipError_t go_vec(const GrpoArgs& a, hipStream_t st) {
  const int64_t wgs = kLossCUs * (NT == 1024 ? 1 : 4);
  const int64_t grid = a.T < wgs ? a.T : wgs;
  if (a.dlogits) hipLaunchKernelGGL((grpo_rows_vec<NT, NCH, false>), dim3((unsigned)grid), dim3(NT), 0, st, a);
  else hipLaunchKernelGGL((grpo_rows_vec<NT, NCH, true>), dim3((unsigned)grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grpo(const GrpoArgs& a, bool vec, hipStream_t st) {
  hipError_t e = hipSuccess;
  timer_mark(LS_KERNEL_GRPO_ROWS, st, false);
  if (vec) {
    const int nch = a.V / 8;
    if (nch <= 256) e = go_vec<256, 1>(a, st);
    else if (nch <= 512) e = go_vec<256, 2>(a, st);
    else if (nch <= 1024) e = go_vec<256, 4>(a, st);
    else if (nch <= 2048) e = go_vec<256, 8>(a, st);
    else if (nch <= 4096) e = go_vec<256, 16>(a, st);
    else if (nch <= 1024 * 8) e = go_vec<1024, 8>(a, st);
    else if (nch <= 1024 * 12) e = go_vec<1024, 12>(a, st);
    else if (nch <= 1024 * 16) e = go_vec<1024, 16>(a, st);
    else if (nch <= 1024 * 19) e = go_vec<1024, 19>(a, st);
    else if (nch <= 1024 * 24) e = go_vec<1024, 24>(a, st);
    else {
      hipLaunchKernelGGL((grpo_rows_stream<1024>), dim3((unsigned)a.T), dim3(1024), 0, st, a);
      e = hipGetLastError();
    }
  } else {
    hipLaunchKernelGGL(grpo_rows_scalar, dim3((unsigned)a.T), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  timer_mark(LS_KERNEL_GRPO_ROWS, st, true);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(grpo_sum, dim3(1), dim3(256), 0, st, (const float*)a.row_loss, a.T, a.loss_accum);
  return hipGetLastError();
}

hipError_t launch_lm_rows(const LmRowArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((lm_rows<256>), dim3((unsigned)a.g.T), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(grpo_sum, dim3(1), dim3(256), 0, st, (const float*)a.g.row_loss, a.g.T, a.g.loss_accum);
  return hipGetLastError();
}

}  // namespace lsr
