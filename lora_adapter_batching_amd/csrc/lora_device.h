// lora_device.h -- gfx950 device helpers: 16-byte global accesses, bf16
// conversions and the bf16 MFMA wrappers used by the LoRA kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------------------
// Buffer-resource access. A raw buffer resource covers [base, base + bytes);
// an access whose byte offset is at or beyond `bytes` reads zeros and a store
// there is dropped, without a branch. Lanes with nothing to load or store use
// kOff (outside every resource: spans stay below 2 GiB).
// ---------------------------------------------------------------------------
constexpr uint32_t kOff = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer, 32-bit data format

// Both arguments must be wave-uniform (they are moved to scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mk_rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7ffffff0;
  const int n = __builtin_amdgcn_readfirstlane((int)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)));
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, kRsrcWord3);
}
// The same descriptor as four scalar words, for the LDS-destination load
// below (issued as inline assembly so that the compiler neither reorders it
// nor inserts its own conservative waits for it: callers wait explicitly).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 mk_rsrc_words(const void* base, int64_t bytes) {
  const int64_t cap = 0x7ffffff0;
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)));
  r[3] = kRsrcWord3;
  return r;
}
// Loads 16 bytes per lane from byte offset voff of the buffer straight into
// LDS: lane l's bytes land at LDS byte address lds_addr + 16 l (lds_addr
// wave-uniform). Lanes whose offset is outside the buffer write zeros. The
// load counts in vmcnt like any vector load.
// M0 (which holds the LDS address) is declared as an output of the
// statement, so the compiler keeps no value of its own in it across the load.
// The descriptor words pass through readfirstlane so that they are SGPR
// values even where the compiler has kept a copy of them in VGPRs.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  int m0_out;
  i32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = __builtin_amdgcn_readfirstlane(rsrc[q]);
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds"
               : "={m0}"(m0_out)
               : "s"(lds_addr), "v"(voff), "s"(r)
               : "memory");
  (void)m0_out;
}
// The same with the non-temporal bit, for data that the launch reads once.
__device__ __forceinline__ void load_lds16_stream(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  int m0_out;
  i32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = __builtin_amdgcn_readfirstlane(rsrc[q]);
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen nt lds"
               : "={m0}"(m0_out)
               : "s"(lds_addr), "v"(voff), "s"(r)
               : "memory");
  (void)m0_out;
}

// Buffer loads and stores of 16 bytes. The _stream forms set the
// non-temporal bit: the output rows y, which every launch reads and writes
// exactly once, go through the caches as streamed data, so they neither
// displace the adapter weights and the hand-off parts that are reused nor
// linger as dirty lines. Measured on the decode MLP-up launch (2560 -> 19456,
// 8 adapters, cold inputs) 13.9 -> 12.0 us, on the MLP-up batch of 32 mixed
// ranks 85 -> 75 us, on the 8192-token prefill 52 -> 46 us.
constexpr int kNT = 2;
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4 bld16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNT);
}
__device__ __forceinline__ void bst16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kNT);
}
__device__ __forceinline__ uint32_t bld2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf2f(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}
// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f2bf(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

// Unpack 8 bf16 (one 16-byte chunk) to floats.
__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __builtin_bit_cast(float, v[q] << 16);
    f[2 * q + 1] = __builtin_bit_cast(float, v[q] & 0xffff0000u);
  }
}
// Pack 8 floats to 8 bf16 (round to nearest even), two per conversion.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    v[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{f[2 * q], f[2 * q + 1]}, bf16x2_t));
  return v;
}

// Split 8 fp32 values into bf16 hi + lo parts (hi = rne(f), lo = rne(f - hi)),
// so an MFMA pair on (hi, lo) carries ~16 mantissa bits of the fp32 operand.
__device__ __forceinline__ void split8(const float (&f)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h = static_cast<__bf16>(f[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(f[e] - static_cast<float>(h));
  }
}

// D = A(32x16) * B(16x32) + C. Lane l supplies A[l%32][8(l/32)+e] and
// B[8(l/32)+e][l%32] (e = 0..7) and holds D[8(i/4)+4(l/32)+(i%4)][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D = A(16x32) * B(32x16) + C. Lane l supplies A[l%16][8(l/16)+e] and
// B[8(l/16)+e][l%16] and holds D[4(l/16)+i][l%16] (i = 0..3).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero_acc16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Expand-output permutation. Row m of a 32x32 MFMA output block is written
// to column colmap(m) of the block, so that lane l's 16 results (rows
// 8(i/4)+4h+(i%4), h = l/32) land on columns 16(i/8) + 8h + (i%8): two runs
// of 8 contiguous bf16, i.e. two 16-byte accesses per lane.
__device__ __forceinline__ int colmap(int m) {
  return (m & 16) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

}  // namespace lora
