// Device-side building blocks shared by the gfx950 attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __fp16 f16x4_lds __attribute__((__vector_size__(4 * sizeof(__fp16))));

#define MIATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// v_exp_f32 / v_log_f32: base-2 transcendental unit.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Two floats -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16lo_to_f32(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
__device__ __forceinline__ float f16hi_to_f32(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }
// Eight bf16 -> eight fp16 (exact for magnitudes in fp16's normal range).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_f16x2(bf16lo_to_f32(v[i]), bf16hi_to_f32(v[i]));
  return r;
}
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x2 a, u32x2 b) {
  u32x4 v = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(f16x8, v);
}

// Value held by lane (lane ^ 32): v_permlane32_swap exchanges the upper half
// wave's first operand with the lower half's second; passing x twice gives
// each lane its partner's copy in the element it did not keep.
__device__ __forceinline__ float xor32(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __builtin_bit_cast(float, lane < 32 ? (int)r[1] : (int)r[0]);
}

// Value held by lane (lane ^ 16): ds_swizzle in bit-mask mode with xor mask 16.
__device__ __forceinline__ float xor16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// 16-byte global load / store through plain vector types.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Non-temporal 16-byte store for output no kernel of the call reads back
// (keeps it from displacing K/V tiles in L2).
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
// Non-temporal 16-byte load for data that is read exactly once.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// Direct HBM -> LDS copy of 16 bytes per lane through a buffer resource
// (MUBUF "lds" form): lane i's 16 bytes from base + voff land at
// lds + 16 i. The buffer form, unlike the global one, is tracked by the
// compiler as a plain vector-memory load, so LDS reads issued while it is in
// flight keep their own fine-grained lgkmcnt waits. base must be uniform.
__device__ __forceinline__ void dma16_to_lds(const void* base, uint32_t voff, MIATTN_LDS void* lds) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 0, 0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Direct HBM -> LDS copy of 16 bytes per lane (buffer load, LDS form) issued
// from inline asm: lane i's 16 bytes from base + voff land at LDS byte
// address lds + 16 i. The compiler does not track these writes, so a loop
// that reads one LDS buffer while a copy fills the other needs no waits from
// it; the caller waits (s_waitcnt vmcnt) before reading what was copied.
// base and lds must be uniform.
__device__ __forceinline__ void dma16_to_lds_asm(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t addr = (uint64_t)base;
  const i32x4 rs = {(int)(uint32_t)addr, (int)((addr >> 32) & 0xffff), 0x7fffffff, 0x00020000};
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}

__device__ __forceinline__ u32x4 lds_ld16(const MIATTN_LDS void* p) {
  return *reinterpret_cast<const MIATTN_LDS u32x4*>(p);
}
__device__ __forceinline__ void lds_st16(MIATTN_LDS void* p, u32x4 v) {
  *reinterpret_cast<MIATTN_LDS u32x4*>(p) = v;
}

// ds_read_b64_tr_b16. Within each block of 16 lanes, lane k names 4 consecutive
// 16-bit elements (row k/4, columns 4(k%4)..4(k%4)+3 of a 4 x 16 tile when the
// addresses are laid out that way); lane j receives column j of the 4 rows.
__device__ __forceinline__ u32x2 lds_ld_tr16(const MIATTN_LDS void* p) {
  f16x4_lds v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((MIATTN_LDS f16x4_lds*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x2 a, u32x2 b) {
  u32x4 v = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x4 as_bf16x4(u32x2 v) { return __builtin_bit_cast(bf16x4, v); }

// Probabilities for the P.V product: two floats -> a packed pair of fp16
// (F16) or bf16, round to nearest even.
template <bool F16>
__device__ __forceinline__ uint32_t pack_p(float lo, float hi) {
  if constexpr (F16) return pack_f16x2(lo, hi);
  else return pack_bf16x2(lo, hi);
}
// O^T += V^T P^T on 32x32x16 MFMAs: V^T operand halves lo/hi and P operand p
// in fp16 (F16) or bf16.
template <bool F16>
__device__ __forceinline__ f32x16 mfma_pv(u32x2 lo, u32x2 hi, u32x4 p, f32x16 acc) {
  if constexpr (F16) return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(lo, hi), as_f16x8(p), acc, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lo, hi), as_bf16x8(p), acc, 0, 0, 0);
}

// bf16 -> fp16 copy of n8 groups of eight elements (16 bytes each), one
// group per thread and grid stride: exact for magnitudes in [2^-14, 65504];
// smaller ones become fp16 subnormals (absolute error at most 2^-25), larger
// ones overflow to inf.
// Words of a work queue: per-XCD counters and an exit count.
constexpr int kWorkQueueWords = 9;

// Sets n words to zero (the work queues' first initialisation).
__global__ __launch_bounds__(64) void miattn_zero_u32_kernel(unsigned* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}

__global__ __launch_bounds__(256) void miattn_bf16_to_f16_kernel(const uint16_t* __restrict__ src,
                                                                 uint16_t* __restrict__ dst, long n8) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256)
    st16(dst + 8 * i, bf16x8_to_f16x8(ld16_stream(src + 8 * i)));
}

}  // namespace miattn
