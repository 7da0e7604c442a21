// Device helpers shared by the attention kernels (gfx950): element types,
// MFMA wrappers, direct global-to-LDS loads, waits, lane swaps.
// Included by the HIP sources only.
#ifndef KVC_DEVICE_H
#define KVC_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_kernels.h"
#include "kvc_plan_layout.h"

namespace kvc {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = KVC_KV_TILE;

// Element type of the pools, k, v, q, o and the split partials: E = 0
// bfloat16, E = 1 float16.  Operands travel as raw 16-bit pairs (bf16x8
// registers) and take their type only in the MFMA, the probability packing,
// the row-sum dot product and the conversions to and from float32.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int E>
struct El;

template <>
struct El<0> {
  static constexpr uint32_t ONE2 = 0x3f803f80u;   // two bf16 ones
  static __device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // bf16 pair of p (lo, hi): the upper halves of the float32 values (rounded
  // toward zero), one byte permute per pair
  static __device__ __forceinline__ uint32_t pack_p(float lo, float hi) {
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
  }
  static __device__ __forceinline__ float dot_ones(uint32_t w, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
  }
  // round to nearest even
  static __device__ __forceinline__ u32x2 cvt4(const f32x4& v) {
    const bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    return __builtin_bit_cast(u32x2, b);
  }
  static __device__ __forceinline__ f32x4 widen4(const u32x2& x) {
    const bf16x4 b = __builtin_bit_cast(bf16x4, x);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
  }
};

template <>
struct El<1> {
  static constexpr uint32_t ONE2 = 0x3c003c00u;   // two f16 ones
  static __device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  }
  // f16 pair of p (lo, hi), rounded toward zero in one packing conversion;
  // p <= 2^8 here, inside the f16 range
  static __device__ __forceinline__ uint32_t pack_p(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  static __device__ __forceinline__ float dot_ones(uint32_t w, float acc) {
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), ones, acc, false);
  }
  static __device__ __forceinline__ u32x2 cvt4(const f32x4& v) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const f16x4 b = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    return __builtin_bit_cast(u32x2, b);
  }
  static __device__ __forceinline__ f32x4 widen4(const u32x2& x) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const f16x4 b = __builtin_bit_cast(f16x4, x);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
  }
};

// The ring of stages is filled by direct global->LDS loads that the kernel
// issues, waits for and publishes itself: the compiler would otherwise treat
// every LDS read as depending on every load in flight and drain the ring at
// each barrier.  Completion is tracked with vmcnt (vector memory operations
// retire in issue order), then a barrier makes a stage visible to all waves.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One work-unit entry of the plan (16 bytes at a wave-uniform address) read
// into scalar registers.  The load completes asynchronously: unit_wait must
// run before the value is used (it names the registers, so every use follows
// it).  Scalar loads share the lgkm counter with LDS reads; an extra scalar
// load in flight only makes the compiler's own LDS waits stricter.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 unit_load(const int32_t* entry) {
  const uint64_t b = (uint64_t)entry;
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  i32x4 e;
  asm volatile("s_load_dwordx4 %0, %1, 0x0" : "=s"(e) : "s"((const int32_t*)sb) : "memory");
  return e;
}
__device__ __forceinline__ void unit_wait(i32x4& e) { asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(e)::"memory"); }

// 16 bytes from base + offset (per lane) to LDS byte address
// lds_base + 16 * lane.  base and lds_base are wave-uniform; they are read
// from the first lane so that they always sit in scalar registers.
__device__ __forceinline__ void load_lds16(const void* base, uint32_t offset, uint32_t lds_base) {
  const uint64_t b = (uint64_t)base;
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t sl = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(offset), "s"((const void*)sb),
               "s"(sl)
               : "memory", "m0");
}

// Maximum of scores (never NaN: masked slots are -inf).  Written with the
// compiler's own max so that its hazard tracking sees the MFMA results these
// read (an opaque instruction reading an MFMA accumulator too early would see
// a partially written register).
__device__ __forceinline__ float max2(float a, float b) { return __builtin_fmaxf(a, b); }

__device__ __forceinline__ uint32_t lds_addr(const void* generic) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)generic;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ i16x4 ds_read_tr16(const uint8_t* lds_generic) {
  const lds_i16x4* p = (const lds_i16x4*)(__attribute__((address_space(3))) const uint8_t*)lds_generic;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

// Exchange with the lane 32 (or 16) apart: after the swap, each lane holds
// its own value and its partner's in (a, b).  Issued directly because the
// compiler builtin's second result is not usable.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// max / sum over lanes l, l^16, l^32, l^48: the four lane groups that hold
// one query column of an MFMA accumulator
__device__ __forceinline__ float lane_swap_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  x = max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  swap16(a, b);
  return max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

__device__ __forceinline__ float lane_swap_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  x = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  swap16(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// The stream record of an attention work item: the stream is the last one
// whose first item is at most `item` (item0 ascends over the streams).  Taken
// from the launch arguments when the plan has at most KVC_ARG_STREAMS
// streams, so that the work-group's first memory round trip is the one for
// its unit entries; else read from the plan.
__device__ __forceinline__ kvc_dev_stream stream_of_item(const AttnParams& p, int item) {
  const int nstreams = p.num_streams;
  kvc_dev_stream st;
  if (nstreams <= KVC_ARG_STREAMS) {
    st = p.recs[0];
#pragma unroll
    for (int i = 1; i < KVC_ARG_STREAMS; ++i)
      if (i < nstreams && item >= p.recs[i].item0) st = p.recs[i];
  } else {
    const kvc_dev_stream* recs = reinterpret_cast<const kvc_dev_stream*>(p.plan + KVC_PLAN_HEADER_INTS);
    int si = 0;
    while (si + 1 < nstreams && item >= recs[si + 1].item0) ++si;
    st = recs[si];
  }
  return st;
}

// Lazy renormalisation.  Each query tile keeps a reference value ref in log2
// units (the running maximum as last renormalised); a stage's probabilities
// are p = 2^(s * scale - ref), with scale = log2(e)/sqrt(D) applied in fp32 to
// the exact MFMA scores.  The stage is first exponentiated against the
// current ref; only when a lane's sum of those probabilities exceeds 2^8 (a
// score more than a few units above ref, or an overflow to infinity) is it
// redone against the exact column maximum.  A tile's first stage with a valid
// slot always takes the exact path.  The own tiles test the whole column's
// sum over the stage (the four lane groups' 64 slots), against four times the
// lane limit.
constexpr float LAZY_SUM_LIMIT = 256.0f;
constexpr float LAZY_COL_LIMIT = 4.0f * LAZY_SUM_LIMIT;

// The lazy checks compare a sum's bit pattern with the limit's: a sum of
// non-negative terms orders like its bits, and so an infinite sum and a NaN
// one (an overflowed probability times a 0 entry of a mask operand) exceed
// the limit too, which a float compare in a build that assumes no NaN can
// miss.
__device__ __forceinline__ bool sum_exceeds(float x, float limit) {
  return __builtin_bit_cast(uint32_t, x) > __builtin_bit_cast(uint32_t, limit);
}

}  // namespace dev
}  // namespace kvc

#endif
