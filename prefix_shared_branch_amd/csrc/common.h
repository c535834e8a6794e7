// Device helpers shared by the gfx950 kernels of liblsreplay.
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A[m][k] (32x16): lane l holds A[l%32][8*(l/32) + 0..7]   (8 bf16, one 16-byte LDS read
//                    when a row's k values are contiguous)
//   B[k][n] (16x32): lane l holds B[8*(l/32) + 0..7][l%32]
//   C[m][n] (32x32): lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l%32]
// So a C tile keeps one n index per lane. The kernels put the softmax row (query) on n
// whenever per-row statistics are needed, so row max/sum/rescale stay lane-local.
//
// A C tile's 16 registers, converted to bf16 in order, form the B operand of the next
// MFMA whose k index runs over C's m index permuted as
//   k position (g = l/32, j) <-> m = 16*h + 4*g + j        (j = 0..3)
//                                 m = 16*h + 8 + 4*g + j-4  (j = 4..7)
// for register half h (registers 8h..8h+7). The matching A operand is fetched with the
// same permutation via ds_read_b64_tr_b16 (two 4-element transposed reads).
//
// ds_read_b64_tr_b16 (gfx950): within each 16-lane group, lane j passes the address of
// element (k0 + j/4, n0 + 4*(j%4)) of a row-major [k][n] LDS tile and receives the four
// values (k0 + e, n0 + j), e = 0..3 -- a transposed 4x16 block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsr {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LSR_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
// Buffer resource word 3 for the gfx9 family (raw buffer, 32-bit data format) and the
// cache-policy bit that marks streaming (non-temporal) accesses.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kSlc = 2;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x8(const s16x4& a, const s16x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32h(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// Round-to-nearest-even pack (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// bf16 of the rounding residuals x0 - bf16(x0), x1 - bf16(x1), given rounded = pack_bf16x2(x0, x1):
// the pair (rounded, residual) carries x to about 16 significant bits.
__device__ __forceinline__ uint32_t pack_bf16x2_residual(float x0, float x1, uint32_t rounded) {
  return pack_bf16x2(x0 - bf16_lo(rounded), x1 - bf16_hi(rounded));
}

// 8 consecutive registers of a C tile (r0..r0+7) -> bf16 B/A operand.
__device__ __forceinline__ bf16x8 c_regs_to_bf16x8(const f32x16& c, int r0) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (__bf16)c[r0 + j];
  return v;
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t* lds_elem_ptr) {
  return *reinterpret_cast<const LSR_LDS bf16x8*>(reinterpret_cast<uintptr_t>(lds_elem_ptr));
}

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* lds_elem_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<LSR_LDS s16x4*>(reinterpret_cast<uintptr_t>(lds_elem_ptr)));
}

__device__ __forceinline__ bf16x8 join_tr(const s16x4& a, const s16x4& b) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ---- LDS tiles without padding: logical 16-byte chunk c of row r is stored at chunk c ^ swz<CH>(r),
// CH = chunks per row. ds_read_b128 serves 16 lanes (256 bytes, all 64 banks) per phase; for 16
// consecutive rows reading the same logical chunk the swizzle puts the 16 reads in 16 distinct
// 16-byte bank groups, for rows of 16 chunks (256 B), 8 chunks (128 B) and 4 chunks (64 B).
// (The 16-chunk form is also conflict-free for ds_read_b64_tr_b16, 4 rows x 64 contiguous bytes.)
template <int CH>
__device__ __forceinline__ int swz(int r) {
  static_assert(CH == 4 || CH == 8 || CH == 16, "row length");
  if constexpr (CH == 16) return (((r & 3) << 2) ^ ((r >> 2) & 3) ^ (r & 2)) & 15;
  else if constexpr (CH == 8) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// ---- Padded LDS tiles of 64 rows: row r starts at byte 16 * PCH * r (PCH >= CH chunks of 16 B).
// PCH = CH + 1 makes 16-byte row-wise reads conflict-free (8 lanes on 8 rows hit 8 distinct
// 16-byte bank groups); PCH = CH + 4 makes ds_read_b64_tr_b16 conflict-free (4 rows x 64 B).
// Every fragment offset is then a per-lane base plus a compile-time immediate.
// A 64-row tile is exactly PCH 1 KB direct-load instructions; lanes that fall on a pad chunk
// reload the row's last real chunk (never read). Rows past nvalid reload row nvalid - 1.
template <int CH, int PCH>
__device__ __forceinline__ void dma_tile64(const uint16_t* base, int64_t ld, int nvalid, char* lds, int wv, int lane);

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i's bytes land at
// lds_wave_base + 16 i. lds_wave_base must be wave-uniform.
// Raw buffer resource over the `bytes` bytes from `base` (clamped to 2^32 - 1): loads at offsets past
// the end return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)(uint32_t)n, kBufferWord3);
}
// 16 bytes per lane from buffer offset voff + soff into LDS at lds_wave_base + 16 * lane (direct load)
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_wave_base,
                                              int soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LSR_LDS void*)lds_wave_base, 16, (int)voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <int CH, int PCH>
__device__ __forceinline__ void dma_tile64(const uint16_t* base, int64_t ld, int nvalid, char* lds, int wv, int lane) {
  static_assert(PCH >= CH, "pitch");
  // opaque lane id: the per-lane row/chunk arithmetic is recomputed for every tile (a few ALU ops)
  // instead of being hoisted out of the tile loop, where it would pin registers for the whole kernel
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int k = 0; k < (PCH + 3) / 4; ++k) {
    const int ins = wv + 4 * k;  // wave-uniform
    if (ins < PCH) {
      const int q = ins * 64 + ln;
      int row = q / PCH;
      int c = q - row * PCH;
      c = c < CH ? c : CH - 1;
      row = row < nvalid ? row : nvalid - 1;
      lds_dma16(base + (int64_t)row * ld + c * 8, lds + ins * 1024);
    }
  }
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maxima): this wave's LDS reads have returned
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// workgroup barrier that orders this wave's memory operations in program order around it but
// waits for nothing (no s_waitcnt); callers wait for the counters they need first
__device__ __forceinline__ void bare_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave still outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// 8 consecutive registers of a C tile (r0..r0+7) -> fp16 B/A operand (round to nearest even).
__device__ __forceinline__ f16x8 c_regs_to_f16x8(const f32x16& c, int r0) {
  f16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (_Float16)c[r0 + j];
  return v;
}

__device__ __forceinline__ f16x8 lds_h128_at(const char* base, int byte_off) {
  return *reinterpret_cast<const LSR_LDS f16x8*>(reinterpret_cast<uintptr_t>(base + byte_off));
}

__device__ __forceinline__ bf16x8 lds_b128_at(const char* base, int byte_off) {
  return *reinterpret_cast<const LSR_LDS bf16x8*>(reinterpret_cast<uintptr_t>(base + byte_off));
}

__device__ __forceinline__ s16x4 lds_s16x4_at(const char* base, int byte_off) {
  return *reinterpret_cast<const LSR_LDS s16x4*>(reinterpret_cast<uintptr_t>(base + byte_off));
}

__device__ __forceinline__ s16x4 lds_tr_at(const char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<LSR_LDS s16x4*>(reinterpret_cast<uintptr_t>(base + byte_off)));
}

// LDS reads through LDS-typed pointers derived from a __shared__ array (rather than from an integer
// address): the compiler keeps the array's identity, so a kernel whose ring stages are separate
// arrays does not wait, before reading one stage, for direct loads in flight into another.
__device__ __forceinline__ bf16x8 lds_b128_as(const char* base, int off) {
  return *(const LSR_LDS bf16x8*)((const LSR_LDS char*)base + off);
}
__device__ __forceinline__ f16x8 lds_h128_as(const char* base, int off) {
  return *(const LSR_LDS f16x8*)((const LSR_LDS char*)base + off);
}
__device__ __forceinline__ f32x4 lds_f32x4_as(const char* base, int off) {
  return *(const LSR_LDS f32x4*)((const LSR_LDS char*)base + off);
}
__device__ __forceinline__ s16x4 lds_tr_as(const char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LSR_LDS s16x4*)((LSR_LDS char*)base + off));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace lsr
