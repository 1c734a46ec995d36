// Device-side building blocks shared by the MLA kernels (gfx950 / CDNA4).
//
// Register layouts of the matrix instructions used here (wave of 64 lanes,
// lane l, half = l / 32):
//   v_mfma_f32_32x32x16_bf16  A[32 x 16]: lane l holds row l%32, k = 8*half + s (s = 0..7)
//                             B[16 x 32]: lane l holds col l%32, k = 8*half + s
//                             C[32 x 32]: lane l, reg r holds row 8*(r/4) + 4*half + r%4,
//                                         col l%32
//   ds_read_b64_tr_b16        in each group of 16 lanes, lane q supplies the address of
//                             4 consecutive bf16 (row q/4 of a 4 x 16 block, columns
//                             4*(q%4) .. +3) and receives column q of the block:
//                             [row0[q], row1[q], row2[q], row3[q]].
// These are what makes the key tile serve both as the A operand of the score
// product (rows = tokens, 8 consecutive latent values per lane: one 16-byte
// LDS read) and, read transposed, as the A operand of the value product
// (rows = latent columns, 4 consecutive tokens per lane per transposed read).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned char __attribute__((address_space(3))) lds_u8;

// Generic pointer to a __shared__ object -> LDS address-space pointer.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
__device__ __forceinline__ lds_u8* to_lds(const void* p) { return (lds_u8*)(p); }
#pragma clang diagnostic pop

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value-product MFMAs accumulating into AGPRs, written as inline asm by the
// decode kernel, where every AGPR holds an output accumulator and the
// compiler's own MFMAs are kept in VGPR form (-mllvm -amdgpu-mfma-vgpr-form
// for that translation unit).  The compiler does not see them as MFMAs, so
// the kernel keeps these rules:
//  * the B operand written by VALU is passed through valu_to_mfma_settle()
//    first (VALU write -> MFMA operand read needs wait states);
//  * every accumulator goes through agpr_settle16() before anything other
//    than another of these MFMAs reads it, and after a VALU/accvgpr write of
//    it before the next MFMA reads it (MFMA write -> read: 32 wait states).
__device__ __forceinline__ void valu_to_mfma_settle(bf16x8& b0, bf16x8& b1) {
  asm volatile("s_nop 4" : "+v"(b0), "+v"(b1));
}
__device__ __forceinline__ void agpr_settle16(f32x16 (&a)[16]) {
  asm volatile("s_nop 15\n\ts_nop 15"
               : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(a[4]), "+a"(a[5]),
                 "+a"(a[6]), "+a"(a[7]), "+a"(a[8]), "+a"(a[9]), "+a"(a[10]), "+a"(a[11]),
                 "+a"(a[12]), "+a"(a[13]), "+a"(a[14]), "+a"(a[15]));
}

// In-place scaling of one accumulator element held in an AGPR (VALU cannot
// read AGPRs directly); a run of these is bracketed by agpr_settle16().
#define MLA_AGPR_SCALE(elem, factor)                                         \
  do {                                                                       \
    float mla_tmp_;                                                          \
    asm volatile(                                                            \
        "v_accvgpr_read_b32 %1, %0\n\t"                                       \
        "v_mul_f32 %1, %1, %2\n\t"                                            \
        "v_accvgpr_write_b32 %0, %1"                                         \
        : "+a"(elem), "=&v"(mla_tmp_)                                        \
        : "v"(factor));                                                      \
  } while (0)

// 16-byte global load reinterpreted as 8 bf16.
__device__ __forceinline__ bf16x8 ld_global_bf16x8(const uint16_t* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 ld_lds_bf16x8(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

__device__ __forceinline__ void st_lds16(lds_u8* p, uint4 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p) = u32x4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ void st_lds_zero16(lds_u8* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p) = u32x4{0u, 0u, 0u, 0u};
}

// Transposed LDS read (see the layout note above).
__device__ __forceinline__ bf16x4 ld_lds_tr(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(const_cast<lds_u8*>(p)));
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Direct global -> LDS copy of 16 bytes per lane.  `lds` must be the same for
// every lane of the wave; lane j's bytes land at lds + 16 * j.
__device__ __forceinline__ void g2lds16(const void* g, lds_u8* lds) {
  __builtin_amdgcn_global_load_lds(g, reinterpret_cast<__attribute__((address_space(3))) void*>(lds),
                                   16, 0, 0);
}

// The same load written as an instruction the compiler does not see.  The
// builtin is a FLAT-class instruction that may write LDS, so after it the
// compiler's wait-count model turns every later LDS wait into lgkmcnt(0),
// which serialises operand reads issued ahead.  The hardware counts this load
// in vmcnt only; callers wait for it with wait_vmcnt.  It writes no register.
// M0 is a reserved register the compiler does not track through inline asm:
// a kernel that uses this form must not also use the builtin (whose M0 set-up
// the asm could land between).  `lds` must be wave-uniform.
__device__ __forceinline__ void g2lds16_opaque(const void* g, lds_u8* lds) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(m0)
               : "m0");
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in [3:0] and
// [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Work-group barrier for LDS hand-over: this wave's LDS reads are complete,
// then all waves meet.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum / sum of v over lanes l and l ^ 32 (the two halves of a row of an
// MFMA 32x32 result), in every lane, with v_permlane32_swap (a VALU exchange,
// no LDS round trip): the swap exchanges the upper half of its first register
// with the lower half of its second, so with both holding v the two hold
// [v_lo, v_lo] and [v_hi, v_hi], and one max / add gives the pair's result in
// every lane.  Written as inline asm: through the compiler builtin, the
// optimiser folds the builtin's second result into its first (a max of the two
// then returns the lower half's value), a miscompilation seen with this
// toolchain.  The s_nop's give the wait states between a VALU write and the
// swap's read, and between the swap and the VALU read of its results.
__device__ __forceinline__ float pair32_max(float v) {
  unsigned a = __builtin_bit_cast(unsigned, v), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a);
}
__device__ __forceinline__ float pair32_sum(float v) {
  unsigned a = __builtin_bit_cast(unsigned, v), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_add_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a);
}

}  // namespace mla
