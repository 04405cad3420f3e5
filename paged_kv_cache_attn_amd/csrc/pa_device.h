// pa_device.h -- device helpers shared by the gfx950 kernels of libpagedattn.
//
// Wave64 conventions used throughout: lane = threadIdx.x & 63, and the 64
// lanes are viewed as 4 rows of 16 (r = lane >> 4, c = lane & 15), which is
// how the 16x16 MFMA instructions distribute their operands:
//   v_mfma_f32_16x16x32_bf16  A: lane holds A[m = c][k = 8r .. 8r+7]
//                             B: lane holds B[k = 8r .. 8r+7][n = c]
//   v_mfma_f32_16x16x16_bf16  A: lane holds A[m = c][k = 4r .. 4r+3]
//                             B: lane holds B[k = 4r .. 4r+3][n = c]
//   both                      C: lane holds C[m = 4r + i][n = c], i = 0..3
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 of two values, packed lo | hi << 16
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Round-to-nearest-even fp32 -> fp16 of two values, packed lo | hi << 16
// (v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 p = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Two packed bf16 to two packed fp16.  Exact for magnitudes in fp16's normal
// range [2^-14, 65504] (8 significant bits fit in 11); smaller magnitudes
// land on fp16's subnormal grid (an absolute error below 2^-25), larger ones
// overflow to infinity.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// -- Debug build ---------------------------------------------------------------
// Built with PAGED_ATTN_DEBUG=1, the kernels also report what their bounds
// checks mask (they never dereference it, in either build): each bit below is
// set in a flag word when the condition is met at least once.  Every
// translation unit has its own word (a file-scope device variable); the host
// reads them all through pa_debug_flags.  In the release build the reports
// compile to nothing.
#ifndef PAGED_ATTN_DEBUG
#define PAGED_ATTN_DEBUG 0
#endif
enum : unsigned {
  kDbgSlotRange = 1u << 0,     // a slot at or past num_blocks * block_size (skipped)
  kDbgSlotDup = 1u << 1,       // two tokens of one kv_cache_write with the same slot
  kDbgBlockRange = 1u << 2,    // a block-table entry outside [0, num_blocks) (masked)
  kDbgPairRange = 1u << 3,     // a block_copy id outside [0, num_blocks) (skipped)
  kDbgPairConflict = 1u << 4,  // a dst used twice, or a dst that is another pair's src
  kDbgLenClamped = 1u << 5,    // a sequence length < 0 or past the call's bound (clamped)
  kDbgQueryLoc = 1u << 6,      // query_start_loc not a valid partition of the query rows
  kDbgSwapRange = 1u << 7,     // a swap id outside [0, num_blocks)
  kDbgPlan = 1u << 8,          // a plan record outside the call's cache or rows (masked)
};
#if PAGED_ATTN_DEBUG
static __device__ unsigned pa_debug_word;
// Device address of this translation unit's flag word (host).
#define PA_DEBUG_WORD_ACCESSOR(name) \
  hipError_t name(void **p) { return hipGetSymbolAddress(p, HIP_SYMBOL(pa_debug_word)); }
#endif
__device__ __forceinline__ void debug_report(bool cond, unsigned bit) {
#if PAGED_ATTN_DEBUG
  // a wave-uniform branch (so values the caller keeps in scalar registers
  // stay uniform), then one lane's vector atomic in global memory
  if (__builtin_amdgcn_ballot_w64(cond) != 0) {
    if (cond && __builtin_amdgcn_readfirstlane(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u))) ==
                    __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)))
      atomicOr(&pa_debug_word, bit);
  }
#else
  (void)cond;
  (void)bit;
#endif
}

// A sequence length clamped to [0, cap] (cap: the tokens the table and the
// host bound admit).
__device__ __forceinline__ int clamp_len(int L, int cap) {
  debug_report(L < 0 || L > cap, kDbgLenClamped);
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// One 16-byte load per lane from global memory straight into LDS: lane i's
// bytes land at lds_base + 16 i (lds_base is the same for the whole wave).
// Written as inline assembly so that the compiler does not track it: its
// wait-count pass cannot tell loads into one LDS stage from reads of another
// across a loop header and would wait there for every load in flight.  The
// caller therefore owns the waits: vm_wait for this wave's loads (they count
// in vmcnt like any vector load), then a workgroup barrier before any wave
// reads the stage.  M0 holds the LDS base; the compiler sets it afresh before
// each of its own uses.
__device__ __forceinline__ void load_lds16(const void *src, void *lds_base) {
  const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds_base;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m), "v"(src) : "memory", "m0");
#pragma clang diagnostic pop
}

// The same load with the address split into a wave-uniform base (scalar
// registers) and a 32-bit per-lane byte offset.
__device__ __forceinline__ void load_lds16_sv(const void *sbase, uint32_t voff, void *lds_base) {
  const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds_base;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m), "v"(voff), "s"(sbase) : "memory", "m0");
#pragma clang diagnostic pop
}

// Waits until at most N of this wave's vector-memory operations are still in
// flight (they complete in issue order).  Loads straight into LDS count here.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// vm_wait<N> that also waits for every LDS (and scalar-memory) operation of
// this wave, so LDS stores issued before it are done when a barrier follows.
template <int N>
__device__ __forceinline__ void vm_lgkm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0x0 << 8) | ((N >> 4) << 14));
}

// All waves of the workgroup meet; the compiler moves no memory access across
// it.  Unlike __syncthreads it waits for none of this wave's loads, so loads
// into LDS stages that are not read yet stay in flight.
__device__ __forceinline__ void workgroup_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ floatx4 mfma_16x16x32_bf16(const bf16x8 &a, const bf16x8 &b,
                                                      const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_16x16x32_f16(const f16x8 &a, const f16x8 &b,
                                                     const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_16x16x16_bf16(const u32x2 &a, const u32x2 &b,
                                                      const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// The four lanes of a column (c, c+16, c+32, c+48) combine through the
// gfx950 row swaps: v_permlane16_swap exchanges rows 1 and 3 of its first
// operand with rows 0 and 2 of its second, v_permlane32_swap the upper half
// of the first with the lower half of the second.  Fed v twice, the returned
// pair is, in every lane, {v[l & ~16], v[l | 16]} (resp. bit 32), so both
// lanes of a partner pair combine the same two values in the same order and
// agree bit for bit.  (The pair's elements are copied out as integers before
// the bit cast: a bit cast applied directly to an element of the returned
// vector reads element 0 whatever the index.)
__device__ __forceinline__ float xor16_first(float v, float &second) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t s0 = s[0], s1 = s[1];
  second = __builtin_bit_cast(float, s1);
  return __builtin_bit_cast(float, s0);
}
__device__ __forceinline__ float xor32_first(float v, float &second) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t s0 = s[0], s1 = s[1];
  second = __builtin_bit_cast(float, s1);
  return __builtin_bit_cast(float, s0);
}

__device__ __forceinline__ float row_max4(float v) {
  // max over the four rows (lanes c, c+16, c+32, c+48)
  float b;
  const float a = xor16_first(v, b);
  v = fmaxf(a, b);
  float d;
  const float c = xor32_first(v, d);
  return fmaxf(c, d);
}

__device__ __forceinline__ float row_sum4(float v) {
  float b;
  const float a = xor16_first(v, b);
  v = a + b;
  float d;
  const float c = xor32_first(v, d);
  return c + d;
}

// Work items in a 1-D grid: consecutive workgroup ids are dealt round-robin
// to the eight XCDs, each with its own L2.  Item L is renumbered so that every
// XCD receives one contiguous run of the work list; neighbouring items, which
// tend to read the same K/V blocks (the query tiles of one head, sequences
// forked from one prompt), then share an L2 and run close together in time.
__device__ __forceinline__ unsigned xcd_contiguous(unsigned L, unsigned N) {
  constexpr unsigned kXcds = 8;
  const unsigned q = N / kXcds, rem = N % kXcds, xcd = L % kXcds, pos = L / kXcds;
  return xcd < rem ? xcd * (q + 1) + pos : rem * (q + 1) + (xcd - rem) * q + pos;
}

// 16-byte global load/store through a plain vector type (global_load_dwordx4).
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x2 ld8(const void *p) { return *reinterpret_cast<const u32x2 *>(p); }
// The same loads with the non-temporal hint, for data read once per call (the
// K/V stream): they leave the L2 to what is reused across calls and kernels
// (plans, partial results, queries).
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x2 ld8_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}

// -- FP8 E4M3 (OCP: bias 7, no infinities, S.1111.111 = NaN, max 448) ------
// Two codes (bytes 0-1 of w, or bytes 2-3 with kHigh) to two bf16, exactly:
// every E4M3 value is a bf16 value (v_cvt_scalef32_pk_bf16_fp8, scale 1).
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}
// Eight codes (two dwords) to eight bf16 (four dwords), in order.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t a, uint32_t b) {
  return u32x4{fp8x2_to_bf16x2<false>(a), fp8x2_to_bf16x2<true>(a), fp8x2_to_bf16x2<false>(b),
               fp8x2_to_bf16x2<true>(b)};
}
// The same eight codes to eight fp16, exactly: every E4M3 value (at most 448
// in magnitude, at least 2^-9 apart from zero) is an fp16 value.
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHigh));
}
__device__ __forceinline__ u32x4 fp8x8_to_f16x8(uint32_t a, uint32_t b) {
  return u32x4{fp8x2_to_f16x2<false>(a), fp8x2_to_f16x2<true>(a), fp8x2_to_f16x2<false>(b),
               fp8x2_to_f16x2<true>(b)};
}
// fp32 -> code, nearest with ties to even and saturation at +-448: the clamp
// supplies the saturation (v_cvt_pk_fp8_f32 rounds to nearest-even and turns
// magnitudes of 464 and up into NaN).  NaN inputs give an unspecified code.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  auto sat = [](float x) { return fminf(fmaxf(x, -448.f), 448.f); };
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
}
__device__ __forceinline__ void st16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Select halves of two packed-bf16 dwords: lo16(a) | lo16(b) << 16 and
// hi16(a) | hi16(b) << 16 (v_perm_b32).
__device__ __forceinline__ uint32_t pack_lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

}  // namespace pa
