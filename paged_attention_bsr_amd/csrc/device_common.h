// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bsa {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// int32 in the constant address space (read-only for the kernel's lifetime)
typedef __attribute__((address_space(4))) int32_t cint32_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Per-storage-type vector types and the 32x32x16 MFMA (fp32 accumulate).
template <typename T>
struct MfmaType;

template <>
struct MfmaType<_Float16> {
  using v8 = f16x8;
  using v4 = f16x4;
  static __device__ __forceinline__ f32x16 mfma32(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct MfmaType<__bf16> {
  using v8 = bf16x8;
  using v4 = bf16x4;
  static __device__ __forceinline__ f32x16 mfma32(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& x) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, x);
}

// Two OCP e4m3 bytes (the low or high 16-bit half of `w`) -> two values of T
// packed in one dword (gfx950's scaled conversion at scale 1: exact, every
// e4m3 value is an fp16 and a bf16 value).
template <typename T, bool HI>
__device__ __forceinline__ uint32_t fp8x2_widen(uint32_t w) {
  if constexpr (sizeof(T) == 2 && static_cast<T>(1.0009765625f) != static_cast<T>(1.f))
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Eight e4m3 bytes -> eight values of T (16 bytes).
template <typename T>
__device__ __forceinline__ u32x4 fp8x8_widen(u32x2 w) {
  return u32x4{fp8x2_widen<T, false>(w[0]), fp8x2_widen<T, true>(w[0]), fp8x2_widen<T, false>(w[1]),
               fp8x2_widen<T, true>(w[1])};
}

// Trace build (BSA_TRACE, a separate library that only tests load): each
// kernel records per planner tile what its loops did, 16 int32 per tile,
// {times processed, first column entry loaded, last entry loaded + 1, valid
// keys loaded, partial offset written (-1: o/lse), kv head, first row, rows,
// key tokens outside [0, N) met, unused...}; the host fills every record with
// {0, INT_MAX, 0, 0, ..., 0 at 8} before the launch.  The build also checks
// every key token a kernel derives from the tables against [0, N): one
// outside is counted and replaced by a masked key (the zero row), so a
// corrupted table never makes a load leave the cache.  In the product build
// every trace statement is dead code.
#ifdef BSA_TRACE
constexpr bool kTrace = true;
#else
constexpr bool kTrace = false;
#endif
struct TraceAcc {
  int lo = 0x7fffffff, end = 0, n = 0, bad = 0;
  // a key token (-1 = masked) checked against [0, num_keys): outside -> masked,
  // and counted when `count` (one of the lanes that derive the same token)
  __device__ __forceinline__ int check(int tok, int64_t num_keys, bool count) {
    if (!kTrace) return tok;
    if (tok < -1 || static_cast<int64_t>(tok) >= num_keys) {
      if (count) ++bad;
      return -1;
    }
    return tok;
  }
  __device__ __forceinline__ void keys(int entry, int count) {
    if (kTrace && count > 0) {
      lo = entry < lo ? entry : lo;
      end = entry + 1 > end ? entry + 1 : end;
      n += count;
    }
  }
};
__device__ __forceinline__ void trace_flush(int32_t* trace, int tile, const TraceAcc& acc, bool owner, int part,
                                            int kvh, int row0, int nrows) {
  if (!kTrace) return;
  int32_t* r = trace + static_cast<int64_t>(tile) * 16;
  if (acc.n > 0) {
    atomicMin(r + 1, acc.lo);
    atomicMax(r + 2, acc.end);
    atomicAdd(r + 3, acc.n);
  }
  if (acc.bad > 0) atomicAdd(r + 8, acc.bad);
  if (owner) {
    atomicAdd(r + 0, 1);
    r[4] = part;
    r[5] = kvh;
    r[6] = row0;
    r[7] = nrows;
  }
}

// v_exp_f32: 2^x, with 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane reductions on the VALU (gfx950's lane swaps) instead of LDS
// permutes: v_permlane32_swap a, b exchanges the upper 32 lanes of a with the
// lower 32 of b, v_permlane16_swap a, b the odd 16-lane rows of a with the
// even rows of b.  With b a copy of a, the two registers then hold, per lane,
// its own value and its partner's (lane ^ 32, resp. ^ 16); max / sum are
// commutative, so the results equal x op (x of the partner) bit for bit.
// The swaps are written as inline asm with both registers tied in and out
// (through the compiler builtins, this toolchain combined the two results as
// if they were one value, x op x, in some kernels).  The hazard checks do not
// look inside inline asm, so each swap is preceded by the two wait states the
// compiler itself puts between a VALU write and a swap reading that register
// (without them the swap read stale values).
template <typename Op>
__device__ __forceinline__ float reduce_xor32(float x, Op op) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return op(a, b);
}
template <typename Op>
__device__ __forceinline__ float reduce_xor16(float x, Op op) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return op(a, b);
}
struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};
// x combined with the lane l ^ 32
__device__ __forceinline__ float max_xor32(float x) { return reduce_xor32(x, MaxOp{}); }
__device__ __forceinline__ float sum_xor32(float x) { return reduce_xor32(x, AddOp{}); }
// x combined over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48):
// (x op x^16) op (that)^32
__device__ __forceinline__ float max_rows4(float x) { return max_xor32(reduce_xor16(x, MaxOp{})); }
__device__ __forceinline__ float sum_rows4(float x) { return sum_xor32(reduce_xor16(x, AddOp{})); }

}  // namespace bsa
