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
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = threadIdx.x + u * 256;   // 64 dims x 8 chunks of 8 slots
    const int d = q >> 3, pc = q & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[slot_key(pc * 8 + 2 * e) * kPackPitch + d];
      const uint32_t hi = tile[slot_key(pc * 8 + 2 * e + 1) * kPackPitch + d];
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(a.out + ((int64_t)h * a.dim + d0 + d) * a.out_ld + c0 + pc * 8) =
        u32x4{w[0], w[1], w[2], w[3]};
  }
}

// row-major copy, 16 bytes per thread: out row (h, col0_s + r) <- logical row row0_s + r of head h
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
    l = a.lse[(int64_t)h * a.T + t] * kLog2e;
    d = a.delta[(int64_t)h * a.T + t];
  }
  reinterpret_cast<float2*>(a.out)[(int64_t)k * a.mpad + m] = make_float2(l, d);
}

}  // namespace

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

hipError_t launch_pack_keys_t(const PackArgs& a, hipStream_t st) {
  if (a.cols == 0) return hipSuccess;
  dim3 grid((unsigned)(a.cols / kPackKeys), (unsigned)(a.dim / kPackDims), (unsigned)a.heads);
  hipLaunchKernelGGL(pack_keys_t, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsr
