// Operand packing for the replay kernels: a key-major bf16 matrix (token rows of stride `ld`, H
// heads of DIM values each) is rewritten dimension-major, one row of keys per (head, dim):
//
//   out[(h * DIM + d) * out_ld + col0_s + p] = in[(row0_s + key(p)) * ld + h * DIM + d]
//
// for every segment s (the prompt, or one response's own keys), with zeros for the slots past the
// segment's n_s keys (each segment occupies a multiple of 64 slots). Within every 16-slot group the
// slots 4..7 and 8..11 are exchanged (key(p) = p with those two quads swapped): an MFMA 32x32x16
// accumulator tile, converted to bf16, enumerates its contraction index in exactly that order
// (register halves h: rows 16h + 4g + 0..3 then 16h + 8 + 4g + 0..3 for lane group g), so the
// matching operand becomes eight consecutive bf16 -- one 16-byte LDS read per fragment.
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
    if (kk + key < n) v = *reinterpret_cast<const u32x4*>(a.src + (row0 + kk + key) * a.ld + (int64_t)h * a.dim + d0 + ch * 8);
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

}  // namespace

hipError_t launch_pack_keys_t(const PackArgs& a, hipStream_t st) {
  if (a.cols == 0) return hipSuccess;
  dim3 grid((unsigned)(a.cols / kPackKeys), (unsigned)(a.dim / kPackDims), (unsigned)a.heads);
  hipLaunchKernelGGL(pack_keys_t, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsr
