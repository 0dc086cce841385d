// hr_internal.h -- helpers shared by libhr's translation units (not exported).
//
// Binary16 arithmetic here is the hardware's: a packed pair of _Float16
// lowers to one v_pk_add_f16, which adds two lanes with IEEE
// round-to-nearest-even and keeps subnormals (the default f16 denormal mode
// is left untouched; the library is built without fast-math).
//
// bfloat16 has no packed add on gfx950: a pair of __bf16 is widened to two
// binary32 values (exact), added with v_add_f32 and narrowed by one
// v_cvt_pk_bf16_f32 (round to nearest even).  Rounding to binary32 and then
// to bfloat16 equals one correct rounding of the exact sum because
// 24 >= 2 * 8 + 2; binary32 denormals are kept (default mode), so bfloat16
// subnormals are exact.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#define HR_BUILDING_LIBRARY 1
#include "hr.h"

namespace hr {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Bytes per vector unit: one 16-byte global_load/store_dwordx4 = 8 binary16.
constexpr int kVecElems = 8;

// fl16(a + b) on two packed binary16 lanes.
__device__ __forceinline__ uint32_t add_pk(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) + __builtin_bit_cast(f16x2, b));
}

// fl16(a + b) on eight binary16 lanes, lane by lane, `a` first.
__device__ __forceinline__ u32x4 add_f16x8(u32x4 a, u32x4 b) {
    u32x4 r;
    r.x = add_pk(a.x, b.x);
    r.y = add_pk(a.y, b.y);
    r.z = add_pk(a.z, b.z);
    r.w = add_pk(a.w, b.w);
    return r;
}

// fl16(a + b) on one binary16 value.
__device__ __forceinline__ uint16_t add_f16x1(uint16_t a, uint16_t b) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(__builtin_bit_cast(_Float16, a) +
                                                              __builtin_bit_cast(_Float16, b)));
}

// bfloat16 counterparts of the three adds above.
__device__ __forceinline__ uint32_t add_pk_bf16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(bf16x2, a) + __builtin_bit_cast(bf16x2, b));
}

__device__ __forceinline__ u32x4 add_bf16x8(u32x4 a, u32x4 b) {
    u32x4 r;
    r.x = add_pk_bf16(a.x, b.x);
    r.y = add_pk_bf16(a.y, b.y);
    r.z = add_pk_bf16(a.z, b.z);
    r.w = add_pk_bf16(a.w, b.w);
    return r;
}

__device__ __forceinline__ uint16_t add_bf16x1(uint16_t a, uint16_t b) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(static_cast<float>(__builtin_bit_cast(__bf16, a)) +
                                                            static_cast<float>(__builtin_bit_cast(__bf16, b))));
}

// The element type of a combine: its 8-wide and 1-wide adds, `a` first.
struct F16 {
    static __device__ __forceinline__ u32x4 add8(u32x4 a, u32x4 b) { return add_f16x8(a, b); }
    static __device__ __forceinline__ uint16_t add1(uint16_t a, uint16_t b) { return add_f16x1(a, b); }
};

struct BF16 {
    static __device__ __forceinline__ u32x4 add8(u32x4 a, u32x4 b) { return add_bf16x8(a, b); }
    static __device__ __forceinline__ uint16_t add1(uint16_t a, uint16_t b) { return add_bf16x1(a, b); }
};

// Compute units of a device, cached after the first query.
hipError_t device_cu_count(int device, int *cus);

// Device that work enqueued on `stream` runs on.
hipError_t stream_device(hr_stream_t stream, int *device);

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// True when [a, a+bytes) and [b, b+bytes) share a byte but a != b.
inline bool partial_overlap(const void *a, const void *b, size_t bytes) {
    uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    if (x == y) return false;
    return x < y + bytes && y < x + bytes;
}

}  // namespace hr
