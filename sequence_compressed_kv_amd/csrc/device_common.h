// Device helpers shared by the gfx950 kernels: storage codecs, MFMA wrappers,
// wavefront reductions and block scans.  Wavefronts are 64 lanes wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sckv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int32_t i32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs; inf/nan keep their class).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ------------------------------------------------------------------ OCP e4m3 ("fn")
// Saturating round-to-nearest-even fp32 -> e4m3 code.  Built from the format
// definition: 3 mantissa bits, bias 7, subnormal step 2^-9, largest finite 448.
// Normal range (|x| >= 2^-6): the fp32 bits rounded to nearest even at bit 20
// (a carry moves into the exponent), exponent rebased from bias 127 to 7; below
// 2^-6 the code is the count of 2^-9 steps.  Branch-free.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  const uint32_t u = __float_as_uint(a);
  const uint32_t normal = ((u + 0x7ffffu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  return sign | (a < 0.015625f ? sub : normal);
}

__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 v) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v[1], 1.0f, true));
  return r;
}

// ------------------------------------------------------------------ order-preserving score keys
// Monotone map fp32 -> uint32 (larger float -> larger key); -0 is ranked as +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------------ MFMA (gfx950)
// 16x16x32: A lane l holds row l%16, B lane l holds column l%16, each with 8 K
// elements of K-group l/16; D lane l holds column l%16, rows 4*(l/16) + i.
__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 16x16x4 fp32: A lane l holds row l%16, B lane l column l%16, each the K element
// l/16; D as for 16x16x32.
__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// 32x32x16: A lane l holds row l%32, B column l%32, 8 K elements of K-group l/32;
// D lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4 for register i.
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <typename T, typename S>
__device__ __forceinline__ T bitcast(const S& s) {
  static_assert(sizeof(T) == sizeof(S), "size");
  return __builtin_bit_cast(T, s);
}

// Global-memory byte pointer whose origin the compiler cannot see.  Loads through
// it are not known to read memory that stays unchanged during the kernel, so the
// compiler cannot re-issue them next to their use (rematerialisation): a
// prefetched value stays in the registers it was loaded into and its load stays
// where it was issued.  The address space stays global (not flat), so these
// loads never hold up LDS waits.
typedef __attribute__((address_space(1))) const uint8_t* gbytes;

__device__ __forceinline__ gbytes opaque_global(const void* p) {
  asm volatile("" : "+s"(p));
  return (gbytes)p;
}

template <typename V>
__device__ __forceinline__ V gload(gbytes base, int64_t byte_off) {
  return *reinterpret_cast<__attribute__((address_space(1))) const V*>(base + byte_off);
}

// Redefines a register value through an empty asm statement (the value must be
// ready: this waits for its load).  Later uses then carry no dependency on the
// original load.
template <typename T>
__device__ __forceinline__ void pin(T& v) {
  static_assert(sizeof(T) == 16, "128-bit values");
  u32x4 x = __builtin_bit_cast(u32x4, v);
  asm volatile("" : "+v"(x));
  v = __builtin_bit_cast(T, x);
}

// ------------------------------------------------------------------ asynchronous global -> LDS copies
// One instruction copies 16 bytes per lane (1 KB per wavefront) from global memory
// straight into LDS at lds_row + 16 * lane (lds_row must be wave-uniform).  The
// copy is tracked by the vector-memory counter only: consumers wait with
// wait_vm_lgkm() and publish with block_barrier().
typedef __attribute__((address_space(3))) void* lds_ptr;

//
// The copy is written as inline assembly on purpose: the compiler then does not
// see an asynchronous LDS writer, so it does not make every later LDS read wait
// for all copies in flight (which would leave nothing in flight during the
// math).  The caller owns the waits.  lds_row must be wave-uniform: it is
// handed to the instruction in M0, which the compiler loads itself (the {m0}
// operand), so it never holds a value of its own there across the copy.
__device__ __forceinline__ void copy_to_lds16(gbytes src, void* lds_row) {
  const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>((lds_ptr)lds_row);
  const uint64_t addr = reinterpret_cast<uint64_t>(src);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(addr), "{m0}"(dst) : "memory");
}

// gfx950 transposing LDS read of four 16-bit values per lane (see the P.V
// operand in the attention kernel for the lane mapping); byte_off is a
// compile-time offset added to every lane's address.
__device__ __forceinline__ u32x2 lds_read_tr16(lds_ptr base, int byte_off) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4)((__attribute__((address_space(3))) uint8_t*)base + byte_off));
  return __builtin_bit_cast(u32x2, v);
}

// s_waitcnt: at most VM vector-memory operations and LGKM LDS/scalar operations
// still outstanding (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int VM, int LGKM>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (LGKM << 8) | ((VM >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (which would wait
// for every copy still in flight).  The empty asm statements keep the compiler
// from moving memory operations across it; the hardware ordering comes from an
// explicit wait_vm_lgkm() before it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ wave / block helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

// maximum over the four 16-lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float group_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// max(x, 0) in one instruction: on the bit pattern, a signed integer max with 0
// keeps non-negative floats and maps every negative one (sign bit set) to +0
// (fmaxf costs a NaN-quieting step besides the max)
__device__ __forceinline__ float relu(float x) {
  const int b = __float_as_int(x);
  return __int_as_float(b > 0 ? b : 0);
}

// v[l] + v[l ^ 32] on every lane, through the gfx950 half-wave swap (no LDS)
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave.
// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round trips):
// shifts by 1, 2, 4 and 8 lanes within each row of 16, then the row totals are
// carried by row_bcast:15 (lane 15 of a row into the next row, rows 1 and 3)
// and row_bcast:31 (lane 31 into rows 2 and 3).  Out-of-row sources read 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Value of lane 63 (a wave-uniform result in a scalar register).
__device__ __forceinline__ uint32_t last_lane(uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, 63); }

// Exclusive prefix sum across the block (blockDim.x = NT threads, NT/64 <= 64 waves).
// `sh` needs NT/64 + 1 words of LDS.  Returns the thread's exclusive prefix and
// writes the block total to *total.  Contains barriers: call from every thread.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  constexpr int NW = NT / kWave;
  const uint32_t inc = wave_incl_scan(v);
  const int w = wave_id(), l = lane_id();
  if (l == kWave - 1) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    uint32_t x = (l < NW) ? sh[l] : 0u;
    uint32_t xi = wave_incl_scan(x);
    if (l < NW) sh[l] = xi - x;
    if (l == NW - 1) sh[NW] = xi;
  }
  __syncthreads();
  const uint32_t r = sh[w] + inc - v;
  *total = sh[NW];
  __syncthreads();
  return r;
}

}  // namespace sckv
