// Internal helpers shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "sag.h"

namespace sag {

// ---- error reporting ---------------------------------------------------------

void set_error(const std::string& msg);
sag_status fail(sag_status s, const std::string& msg);

#define SAG_CHECK_HIP(expr)                                                        \
    do {                                                                           \
        hipError_t e_ = (expr);                                                    \
        if (e_ != hipSuccess)                                                      \
            return ::sag::fail(SAG_E_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
    } while (0)

#define SAG_LAUNCH_CHECK()                                                         \
    do {                                                                           \
        hipError_t e_ = hipGetLastError();                                         \
        if (e_ != hipSuccess)                                                      \
            return ::sag::fail(SAG_E_HIP, std::string("launch: ") + hipGetErrorString(e_)); \
    } while (0)

#define SAG_TRY(expr)                                                              \
    do {                                                                           \
        sag_status s_ = (expr);                                                    \
        if (s_ != SAG_OK) return s_;                                               \
    } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t elt_size(sag_dtype t) { return t == SAG_BF16 ? 2 : 4; }
inline int64_t vec_elems(sag_dtype t) { return t == SAG_BF16 ? 8 : 4; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }
inline int bits_for(uint64_t max_value) {   // bits needed to hold values 0..max_value
    int b = 0;
    while (b < 64 && (max_value >> b) != 0) ++b;
    return b;
}

// Checks a dense operand: non-null (unless empty), ld >= d, 16-B aligned
// pointer and row pitch.
sag_status check_dense(const char* name, const void* p, int64_t rows, int64_t d, int64_t ld,
                       sag_dtype t);

// Workspace carving: 256-B aligned sub-buffers from one caller buffer.  With a
// null base it only measures.
struct Carver {
    char* base;
    size_t size;
    size_t off = 0;
    Carver(void* b, size_t s) : base(static_cast<char*>(b)), size(s) {}
    template <class T>
    T* take(size_t count) {
        off = (off + 255) & ~size_t(255);
        T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
        off += count * sizeof(T);
        return p;
    }
    size_t used() const { return (off + 255) & ~size_t(255); }
    bool fits() const { return off <= size; }
};

// ---- bf16 <-> fp32 (device) ----------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even, NaN to a quiet NaN, in one hardware conversion
// (on every fp32 bit pattern the same bits as the rounding written out:
// add 0x7fff plus the kept low bit, keep the high half, set the quiet bit
// of a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }

// Elements of type T in one 16-byte vector.
template <class T> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; };
template <> struct Vec<uint16_t> { static constexpr int N = 8; };

// Unpacks a 16-B vector into fp32 values.
__device__ __forceinline__ void unpack16(const uint4& v, float* f, float*) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(const uint4& v, float* f, uint16_t*) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}
template <class T>
__device__ __forceinline__ void unpack(const uint4& v, float* f) {
    unpack16(v, f, static_cast<T*>(nullptr));
}

// Stores n (<= Vec<T>::N) fp32 values as type T at p (16-B aligned when n
// is a full vector).
template <class T>
__device__ __forceinline__ void store_vals(T* p, const float* f, int n) {
    constexpr int V = Vec<T>::N;
    if (n == V) {
        if constexpr (V == 4) {
            *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
        } else {
            uint4 o;
            o.x = uint32_t(f32_to_bf16(f[0])) | (uint32_t(f32_to_bf16(f[1])) << 16);
            o.y = uint32_t(f32_to_bf16(f[2])) | (uint32_t(f32_to_bf16(f[3])) << 16);
            o.z = uint32_t(f32_to_bf16(f[4])) | (uint32_t(f32_to_bf16(f[5])) << 16);
            o.w = uint32_t(f32_to_bf16(f[6])) | (uint32_t(f32_to_bf16(f[7])) << 16);
            *reinterpret_cast<uint4*>(p) = o;
        }
    } else {
        for (int e = 0; e < n; ++e) p[e] = from_f32<T>(f[e]);
    }
}

// Exclusive scan of int32 counts into int64 offsets (out[n] = total).
// tmp: scan_workspace_bytes(n) bytes.
size_t scan_workspace_bytes(int64_t n);
sag_status exclusive_scan(const int32_t* in, int64_t* out, int64_t n, void* tmp, hipStream_t s);

// Stable LSD radix sort of n uint64 keys on their low `bits` bits.  Sorts
// between `keys` and `alt`; *result points at whichever holds the output.
size_t radix_sort_workspace_bytes(int64_t n);
sag_status radix_sort_u64(uint64_t* keys, uint64_t* alt, int64_t n, int bits, void* tmp,
                          size_t tmp_bytes, hipStream_t s, uint64_t** result);

// Row pointers of a sorted key list: row of entry i is keys[i] / divisor;
// writes indptr[0..n_rows] (n_rows + 1 entries).
sag_status rows_from_sorted_keys(const uint64_t* keys, int64_t n, uint64_t divisor,
                                 int64_t n_rows, int64_t* indptr, hipStream_t s);

}  // namespace sag
