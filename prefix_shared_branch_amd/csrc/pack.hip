// Operand packing for the replay kernels. pack_keys_t rewrites a key-major bf16 matrix (logical
// rows addressed as described for PackArgs) dimension-major, one row of keys per (head, dim):
//
//   out[(h * DIM + d) * out_ld + col0_s + p] = row (row0_s + key(p)) of head h, dim d
//
// for every segment s (the prompt, or one response's own keys), with zeros for the slots past the
// segment's n_s keys (each segment occupies a multiple of 64 slots). Within every 16-slot group the
// slots 4..7 and 8..11 are exchanged (key(p) = p with those two quads swapped): an MFMA 32x32x16
// accumulator tile, converted to bf16, enumerates its contraction index in exactly that order
// (register halves h: rows 16h + 4g + 0..3 then 16h + 8 + 4g + 0..3 for lane group g), so the
// matching operand becomes eight consecutive bf16 -- one 16-byte LDS read per fragment.
// pack_rows gathers the same logical rows row-major per head (the GQA-packed query rows of one kv
// head become one contiguous matrix), and pack_rowstats lays out the per-row softmax statistics
// of those rows next to each other.
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

constexpr int kPackKeys = 64;   // slots per block
constexpr int kPackDims = 64;   // dims per block
constexpr int kPackPitch = kPackDims + 8;  // LDS row pitch (elements) of the key-major staging tile

__device__ __forceinline__ int slot_key(int p) {
  const int q = (p >> 2) & 3;
  return q == 1 ? p + 4 : (q == 2 ? p - 4 : p);
}

__device__ __forceinline__ int64_t src_row(const PackArgs& a, int64_t r, int h) {
  const int64_t q = r / a.grp;
  return q * a.ld + (r - q * a.grp) * a.gstride + (int64_t)h * a.hstride;
}

__global__ __launch_bounds__(256) void pack_keys_t(PackArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kPackKeys * kPackPitch];
  const int64_t c0 = (int64_t)blockIdx.x * kPackKeys;   // first slot of this block
  const int d0 = blockIdx.y * kPackDims;
  const int h = blockIdx.z;
  int s = 0;
  while (s + 1 < a.nseg && c0 >= a.col0[s + 1]) ++s;
  const int kk = (int)(c0 - a.col0[s]);                 // first key of the block within the segment
  const int n = a.n[s];
  const int64_t row0 = a.row0[s];

#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = threadIdx.x + u * 256;   // 512 chunks of 8 dims
    const int key = q >> 3, ch = q & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (kk + key < n) v = *reinterpret_cast<const u32x4*>(a.src + src_row(a, row0 + kk + key, h) + d0 + ch * 8);
    *reinterpret_cast<u32x4*>(&tile[key * kPackPitch + ch * 8]) = v;
  }
  __syncthreads();
  const float f16s = a.f16_scale ? *a.f16_scale : 0.0f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = threadIdx.x + u * 256;   // 64 dims x 8 chunks of 8 slots
    const int d = q >> 3, pc = q & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[slot_key(pc * 8 + 2 * e) * kPackPitch + d];
      const uint32_t hi = tile[slot_key(pc * 8 + 2 * e + 1) * kPackPitch + d];
      if (a.f16_scale) {
        // power-of-two scaling is exact; the fp16 rounding is to nearest even
        f16x2 h;
        h[0] = (_Float16)(bf16_to_f32((uint16_t)lo) * f16s);
        h[1] = (_Float16)(bf16_to_f32((uint16_t)hi) * f16s);
        w[e] = __builtin_bit_cast(uint32_t, h);
      } else {
        w[e] = lo | (hi << 16);
      }
    }
    *reinterpret_cast<u32x4*>(a.out + ((int64_t)h * a.dim + d0 + d) * a.out_ld + c0 + pc * 8) =
        u32x4{w[0], w[1], w[2], w[3]};
  }
}

// row-major copy, 16 bytes per thread: out row (h, col0_s + r) <- logical row row0_s + r of head h
// (bf16, or fp16 of value * (*f16_scale))
__global__ __launch_bounds__(256) void pack_rows(PackArgs a) {
  const int cpr = a.dim / 8;                         // 16-byte chunks per row
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y;
  const int64_t slot = idx / cpr;
  const int ch = (int)(idx - slot * cpr);
  if (slot >= a.cols) return;
  int s = 0;
  while (s + 1 < a.nseg && slot >= a.col0[s + 1]) ++s;
  const int64_t r = slot - a.col0[s];
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < a.n[s]) v = *reinterpret_cast<const u32x4*>(a.src + src_row(a, a.row0[s] + r, h) + ch * 8);
  if (a.f16_scale) {
    // fp16 rows of value * scale (power of two: exact up to the fp16 rounding, to nearest even)
    const float f = *a.f16_scale;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f16x2 x;
      x[0] = (_Float16)(bf16_lo(v[q]) * f);
      x[1] = (_Float16)(bf16_hi(v[q]) * f);
      v[q] = __builtin_bit_cast(uint32_t, x);
    }
  }
  *reinterpret_cast<u32x4*>(a.out + ((int64_t)h * a.out_ld + slot) * a.dim + ch * 8) = v;
}

__global__ __launch_bounds__(256) void pack_rowstats(RowStatArgs a) {
  const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int k = blockIdx.y;
  if (m >= a.mpad) return;
  float l = INFINITY, d = 0.0f;   // padding rows: P = exp2(s - inf) = 0
  if (m < a.M) {
    const int64_t t = m / a.g;
    const int h = k * a.g + (int)(m - t * a.g);
    // 2^15 P = exp2(S scale log2 e - (LSE log2 e - 15)); Delta in the units of the scaled dS
    l = a.lse[(int64_t)h * a.T + t] * kLog2e - 15.0f;
    d = a.delta[(int64_t)h * a.T + t] * a.scales[2];
  }
  reinterpret_cast<float2*>(a.out)[(int64_t)k * a.mpad + m] = make_float2(l, d);
}

// bf16 parts hi, mid, lo of v (hi + mid + lo = v to about 24 significant bits), then a zero; a
// non-finite v keeps hi = v and zero parts
__device__ __forceinline__ u32x2 split3_bf16(float v) {
  const float hi = (float)(__bf16)v;
  const float r1 = __builtin_isfinite(v) ? v - hi : 0.0f;
  const float mid = (float)(__bf16)r1;
  const float lo = r1 - mid;
  return u32x2{pack_bf16x2(hi, mid), pack_bf16x2(lo, 0.0f)};
}

__global__ __launch_bounds__(256) void pack_rowext(RowStatArgs a) {
  const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int k = blockIdx.y;
  if (m >= a.mpad) return;
  float x = -INFINITY, d = 0.0f;  // padding rows: S starts at -inf, so P = 0
  if (m < a.M) {
    const int64_t t = m / a.g;
    const int h = k * a.g + (int)(m - t * a.g);
    // 2^15 P = exp2(scale log2 e (S + x)) with x = -(LSE log2 e - 15) / (scale log2 e)
    x = -(a.lse[(int64_t)h * a.T + t] * kLog2e - 15.0f) / a.c2;
    d = -a.delta[(int64_t)h * a.T + t];
  }
  // 32-row blocks of 1 KB, each [x parts of rows 0..31 | zeros | d parts | zeros] at 8 bytes per row,
  // so the 32 lanes that read one quarter read 256 contiguous bytes
  const u32x2 xs = split3_bf16(x), ds = split3_bf16(d);
  u32x2* o = reinterpret_cast<u32x2*>(a.out + ((int64_t)k * a.mpad + (m & ~(int64_t)31)) * 8) + (m & 31);
  o[0] = xs;
  o[32] = u32x2{0u, 0u};
  o[64] = ds;
  o[96] = u32x2{0u, 0u};
}

// Partial maxima for the fp16 operand scales: {max |dO|, max row norm of dO, max |Q|, max row norm
// of V over the prompt and the responses}. Rows are read 16 bytes per thread; a row's squared
// norm is summed over the DIM / 8 consecutive lanes that hold it.
template <int DIM>
__device__ __forceinline__ void rows_max(const uint16_t* base, int64_t nrows, int64_t ld, int heads, int64_t start,
                                         int64_t stride, float& amax, float& nmax) {
  constexpr int TPR = DIM / 8;  // threads per row
  const int64_t nchunks = nrows * heads * TPR;
  for (int64_t c = start; c < nchunks; c += stride) {
    const int64_t rh = c / TPR;
    const int part = (int)(c - rh * TPR);
    const int64_t r = rh / heads;
    const int h = (int)(rh - r * heads);
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + r * ld + (int64_t)h * DIM + part * 8);
    float ss = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x0 = bf16_lo(v[q]), x1 = bf16_hi(v[q]);
      amax = __builtin_elementwise_maximum(amax, __builtin_elementwise_maximum(__builtin_fabsf(x0), __builtin_fabsf(x1)));
      ss = __builtin_fmaf(x0, x0, __builtin_fmaf(x1, x1, ss));
    }
    // the TPR lanes of a row are consecutive (stride and start are multiples of TPR per lane group)
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    nmax = __builtin_elementwise_maximum(nmax, __builtin_sqrtf(ss));
  }
}

template <int D, int DV>
__global__ __launch_bounds__(256) void bwd_scale_partials(ScaleArgs a) {
  const int64_t start = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float dummy = 0.0f;
  rows_max<DV>(a.dO, a.T, (int64_t)a.Hq * DV, a.Hq, start, stride, v[0], v[1]);
  rows_max<D>(a.Q, a.T, (int64_t)a.Hq * D, a.Hq, start, stride, v[2], dummy);
  if (a.P > 0) rows_max<DV>(a.Vp, a.P, a.ldv, a.Hkv, start, stride, dummy, v[3]);
  rows_max<DV>(a.Vs, a.Tk, a.ldv, a.Hkv, start, stride, dummy, v[3]);
  __shared__ float red[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = v[i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = __builtin_elementwise_maximum(x, __shfl_xor(x, o, 64));
    if ((threadIdx.x & 63) == 0) red[i][threadIdx.x >> 6] = x;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    const int i = threadIdx.x;
    a.partial[blockIdx.x * 4 + i] = __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(red[i][0], red[i][1]), __builtin_elementwise_maximum(red[i][2], red[i][3]));
  }
}

// exponent k (as the float 2^k) with x * 2^k <= 2^15, clamped; 1 for x == 0
__device__ __forceinline__ float pow2_fit(float x) {
  if (!(x > 0.0f)) return 1.0f;                       // zero: any scale; NaN: propagates anyway
  int e;
  (void)frexpf(x, &e);                               // x = m 2^e, 0.5 <= m < 1, so x < 2^e
  const int k = min(60, max(-60, 15 - e));
  return ldexpf(1.0f, k);
}

__global__ __launch_bounds__(256) void bwd_scale_final(ScaleArgs a) {
  __shared__ float red[4][4];
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int b = threadIdx.x; b < kScaleBlocks; b += 256)
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_elementwise_maximum(v[i], a.partial[b * 4 + i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = v[i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = __builtin_elementwise_maximum(x, __shfl_xor(x, o, 64));
    if ((threadIdx.x & 63) == 0) red[i][threadIdx.x >> 6] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m[i] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(red[i][0], red[i][1]),
                                           __builtin_elementwise_maximum(red[i][2], red[i][3]));
    a.scales[0] = pow2_fit(m[0]);
    a.scales[1] = pow2_fit(m[2]);
    // |2^15 P (dP - Delta)| <= 2^15 * 2 * max|dO_r| * max|V_j|: scale that bound down to 2^15
    a.scales[2] = pow2_fit(2.0f * m[1] * m[3]) * 0x1p-15f;
    a.scales[3] = 0.0f;
  }
}

// Forward: partial maxima of |V| over the prompt and response V rows (one per block).
template <int DV>
__global__ __launch_bounds__(256) void fwd_vscale_partials(ScaleArgs a) {
  const int64_t start = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  float amax = 0.0f, nmax = 0.0f;
  if (a.P > 0) rows_max<DV>(a.Vp, a.P, a.ldv, a.Hkv, start, stride, amax, nmax);
  rows_max<DV>(a.Vs, a.Tk, a.ldv, a.Hkv, start, stride, amax, nmax);
  __shared__ float red[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = __builtin_elementwise_maximum(amax, __shfl_xor(amax, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0)
    a.partial[blockIdx.x * 8] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(red[0], red[1]),
                                                              __builtin_elementwise_maximum(red[2], red[3]));
}

// s_V = 2^k with max |V| s_V <= 2^15 (fp16 holds V s_V exactly where its exponent fits; products
// with probabilities <= 2^8 accumulate in fp32), and its exact inverse
__global__ __launch_bounds__(256) void fwd_vscale_final(ScaleArgs a) {
  __shared__ float red[4];
  float v = 0.0f;
  for (int b = threadIdx.x; b < kScaleBlocks; b += 256) v = __builtin_elementwise_maximum(v, a.partial[b * 8]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_elementwise_maximum(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(red[0], red[1]),
                                                  __builtin_elementwise_maximum(red[2], red[3]));
    const float s = pow2_fit(m);
    a.scales[0] = s;
    a.scales[1] = 1.0f / s;
  }
}

}  // namespace

hipError_t launch_fwd_vscale(const ScaleArgs& a, hipStream_t st) {
  if (a.Dv == 64) hipLaunchKernelGGL((fwd_vscale_partials<64>), dim3(kScaleBlocks), dim3(256), 0, st, a);
  else if (a.Dv == 128) hipLaunchKernelGGL((fwd_vscale_partials<128>), dim3(kScaleBlocks), dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd_vscale_final, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_scales(const ScaleArgs& a, hipStream_t st) {
  if (a.Dqk == 64 && a.Dv == 64) hipLaunchKernelGGL((bwd_scale_partials<64, 64>), dim3(kScaleBlocks), dim3(256), 0, st, a);
  else if (a.Dqk == 128 && a.Dv == 128) hipLaunchKernelGGL((bwd_scale_partials<128, 128>), dim3(kScaleBlocks), dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scale_final, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pack_rows(const PackArgs& a, hipStream_t st) {
  if (a.cols == 0) return hipSuccess;
  const int64_t n = a.cols * (a.dim / 8);
  hipLaunchKernelGGL(pack_rows, dim3((unsigned)((n + 255) / 256), (unsigned)a.heads), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pack_rowstats(const RowStatArgs& a, hipStream_t st) {
  if (a.mpad == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_rowstats, dim3((unsigned)((a.mpad + 255) / 256), (unsigned)a.Hkv), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pack_rowext(const RowStatArgs& a, hipStream_t st) {
  if (a.mpad == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_rowext, dim3((unsigned)((a.mpad + 255) / 256), (unsigned)a.Hkv), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pack_keys_t(const PackArgs& a, hipStream_t st) {
  if (a.cols == 0) return hipSuccess;
  dim3 grid((unsigned)(a.cols / kPackKeys), (unsigned)(a.dim / kPackDims), (unsigned)a.heads);
  hipLaunchKernelGGL(pack_keys_t, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsr
