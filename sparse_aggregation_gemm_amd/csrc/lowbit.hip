// Low-bit halo messages: Sylvie's Quantizer and Dequantizer (Sylvie, system
// overview, "Quantizer", "Communicator" and "Dequantizer" paragraphs).  Each
// node feature vector h that leaves its partition becomes b-bit integers
// (B = 2^b - 1 bins) by stochastic rounding, with a per-row scale
// (max(h) - min(h)) / B and zero-point min(h); the receiver recovers
// zero + code * scale.  The page's equations are missing from the text; the
// plain reading is taken: t = (h - zero) / scale, the position in bins (the
// inverse of the recovery), code = floor(t) + 1 with probability
// t - floor(t) (at most B), every step an fp32 operation rounded to nearest
// even in that order, so that the integer decisions are reproducible.  The
// uniform draws come from the Philox4x32-10 counter-based generator (Salmon,
// Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC'11): element j of node `node` in call `epoch` uses the top 24 bits of
// word j % 4 of the block at counter (j / 4, node, epoch, 0) under key
// (seed low, seed high), times 2^-24 -- the fp32 uniform on [0, 1), whose
// values all lie on the grid of every fp32 fraction of a position >= 1/2, so
// the rounding is exactly unbiased there (the page's unbiased Low-bit
// Module).  Two blocks per eight elements.
//
// A group of G lanes handles a row, each lane eight consecutive elements at
// a time (one 16-byte bf16 vector or two fp32 vectors), so that a lane's
// codes are b whole bytes: element j of the row occupies bits
// [b j, b j + b) of the row's codes, little-endian.
#include "common.h"
#include "trace.h"

// Every fp32 step below is rounded on its own: no multiply-add contraction
// (the recovered value is zero + code * scale with two roundings).  The
// operations are written out here rather than through library helpers so
// that this setting governs them.
#pragma clang fp contract(off)

namespace sag {
namespace {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

// Philox4x32 with 10 rounds: c is the counter in and the block out.  Each
// round's two 32 x 32 -> 64-bit products are taken whole, so one
// instruction gives both halves of each.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * c[0];
        const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * c[2];
        const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = static_cast<uint32_t>(p1);
        c[2] = n2;
        c[3] = static_cast<uint32_t>(p0);
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
    }
}

// The eight elements [8g, 8g + 8) of a row as fp32 (elements past d read
// as 0).  Loads are whole 16-byte vectors: the vector that holds the row's
// last element lies inside the row's pitch (a multiple of 16 bytes), so only
// an fp32 vector that starts at or past d is skipped.
template <class T>
__device__ __forceinline__ void load8(const T* row, int64_t g, int64_t d, float (&f)[8]) {
    const int64_t j0 = 8 * g;
    unpack<T>(*reinterpret_cast<const uint4*>(row + j0), f);
    if constexpr (sizeof(T) == 4) {
        if (j0 + 4 < d) {
            unpack<T>(*reinterpret_cast<const uint4*>(row + j0 + 4), f + 4);
        } else {
#pragma unroll
            for (int e = 4; e < 8; ++e) f[e] = 0.f;
        }
    }
    if (j0 + 8 > d) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = j0 + e < d ? f[e] : 0.f;
    }
}

// Writes the BITS bytes that hold eight BITS-bit codes.
template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* p, uint64_t packed) {
    if constexpr (BITS == 1) *p = static_cast<uint8_t>(packed);
    else if constexpr (BITS == 2) *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(packed);
    else if constexpr (BITS == 4) *reinterpret_cast<uint32_t*>(p) = static_cast<uint32_t>(packed);
    else *reinterpret_cast<uint64_t*>(p) = packed;
}

// The codes of eight elements f (the first `live` of them real; the others
// get code 0) with the uniform draws of element e in the top 24 bits of w[e],
// packed BITS bits each.  The division by the scale is the correctly rounded
// fp32 quotient (the compiler's default for '/' on this target; no fast-math
// flags).
template <int BITS, bool FULL>
__device__ __forceinline__ uint64_t code_group(const float (&f)[8], int live, float z, float s, float B,
                                               const uint32_t (&w)[8]) {
    uint32_t part[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float t = (f[e] - z) / s;
        const float fl = floorf(t);
        const float fr = t - fl;
        const float u = static_cast<float>(w[e] >> 8) * 5.9604644775390625e-8f;   // 2^-24
        float q = u < fr ? fl + 1.f : fl;
        q = q < B ? q : B;
        uint32_t c = static_cast<uint32_t>(q);
        if constexpr (!FULL) c = e < live ? c : 0u;
        part[(BITS * e) / 32] |= c << ((BITS * e) % 32);
    }
    return static_cast<uint64_t>(part[0]) | (static_cast<uint64_t>(part[1]) << 32);
}

__device__ __forceinline__ uint64_t load_codes(const uint8_t* p, int bits) {
    switch (bits) {
        case 1: return *p;
        case 2: return *reinterpret_cast<const uint16_t*>(p);
        case 4: return *reinterpret_cast<const uint32_t*>(p);
        default: return *reinterpret_cast<const uint64_t*>(p);
    }
}

struct QArgs {
    const char* src;
    int64_t ld_src;          // elements
    const int32_t* rows;     // nullable: row k
    int64_t n_src;
    const int32_t* nodes;    // nullable: stream id k
    int64_t n, d;
    int bits;
    uint32_t key0, key1, epoch;
    uint8_t* codes;
    int64_t ld_codes;        // bytes
    float* scale;
    float* zero;
};

// x from another lane through a DPP lane permutation (one VALU operand
// modifier, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Min and max over the G lanes (aligned) of a row: swaps within quads, then
// mirrors within 8 and 16 lanes (after each step all lanes of the block hold
// its value, so a mirror brings in the other half's), then lane shuffles.
template <int G>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
    if constexpr (G >= 2) { mn = fminf(mn, dpp<0xb1>(mn)); mx = fmaxf(mx, dpp<0xb1>(mx)); }     // quad_perm [1,0,3,2]
    if constexpr (G >= 4) { mn = fminf(mn, dpp<0x4e>(mn)); mx = fmaxf(mx, dpp<0x4e>(mx)); }     // quad_perm [2,3,0,1]
    if constexpr (G >= 8) { mn = fminf(mn, dpp<0x141>(mn)); mx = fmaxf(mx, dpp<0x141>(mx)); }   // row_half_mirror
    if constexpr (G >= 16) { mn = fminf(mn, dpp<0x140>(mn)); mx = fmaxf(mx, dpp<0x140>(mx)); }  // row_mirror
    if constexpr (G >= 32) {
        mn = fminf(mn, __shfl_xor(mn, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    }
    if constexpr (G >= 64) {
        mn = fminf(mn, __shfl_xor(mn, 32, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    }
}

template <class T, int G, int BITS>
__global__ __launch_bounds__(256) void quantize_rows(QArgs a) {
    constexpr int kRowsPerBlock = 256 / G;
    const int gl = threadIdx.x % G;
    const int64_t k = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / G;
    const bool valid = k < a.n;
    const int64_t r = valid ? (a.rows ? static_cast<int64_t>(a.rows[k]) : k) : 0;
    const bool ok = valid && r >= 0 && r < a.n_src;
    const T* row = reinterpret_cast<const T*>(a.src) + (ok ? r : 0) * a.ld_src;
    const int64_t groups = (a.d + 7) / 8;
    // a lane's first group stays in registers for the coding pass (the only
    // one when d <= 8 G); later groups are loaded again
    float f0[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
    if (ok) {
        for (int64_t g = gl; g < groups; g += G) {
            float f[8];
            load8<T>(row, g, a.d, f);
            if (g == gl) {
#pragma unroll
                for (int e = 0; e < 8; ++e) f0[e] = f[e];
            }
            const int live = static_cast<int>(a.d - 8 * g < 8 ? a.d - 8 * g : 8);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (live == 8 || e < live) {
                    mn = fminf(mn, f[e]);
                    mx = fmaxf(mx, f[e]);
                }
        }
    }
    group_minmax<G>(mn, mx);
    const float B = static_cast<float>((1 << BITS) - 1);
    const float z = ok && a.d > 0 ? mn : 0.f;
    const float R = ok && a.d > 0 ? mx - mn : 0.f;
    const float s = R / B;
    if (!valid) return;
    const uint32_t node = static_cast<uint32_t>(a.nodes ? a.nodes[k] : k);
    uint8_t* out = a.codes + k * a.ld_codes;
    for (int64_t g = gl; g < groups; g += G) {
        uint64_t packed = 0;
        if (R > 0.f) {
            float f[8];
            if (g == gl) {
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = f0[e];
            } else {
                load8<T>(row, g, a.d, f);
            }
            // elements 8g .. 8g + 7 draw from blocks 2g and 2g + 1
            uint32_t b0[4] = {static_cast<uint32_t>(2 * g), node, a.epoch, 0u};
            uint32_t b1[4] = {static_cast<uint32_t>(2 * g + 1), node, a.epoch, 0u};
            philox4x32_10(b0, a.key0, a.key1);
            const int live = static_cast<int>(a.d - 8 * g < 8 ? a.d - 8 * g : 8);
            if (live > 4) philox4x32_10(b1, a.key0, a.key1);
            const uint32_t w[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            packed = live == 8 ? code_group<BITS, true>(f, 8, z, s, B, w)
                               : code_group<BITS, false>(f, live, z, s, B, w);
        }
        store_codes<BITS>(out + g * BITS, packed);
    }
    if (gl == 0) {
        a.scale[k] = s;
        a.zero[k] = z;
    }
}

struct DArgs {
    const uint8_t* codes;
    int64_t ld_codes;
    const float* scale;
    const float* zero;
    int64_t n, d;
    int bits;
    const int32_t* ids;      // nullable: target row k
    int64_t row_base, n_dst;
    char* dst;
    int64_t ld_dst;          // elements
};

template <class T, int G, bool ACC>
__global__ __launch_bounds__(256) void dequantize_rows(DArgs a) {
    constexpr int kRowsPerBlock = 256 / G;
    const int gl = threadIdx.x % G;
    const int64_t k = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / G;
    if (k >= a.n) return;
    const int64_t t = a.ids ? static_cast<int64_t>(a.ids[k]) - a.row_base : k;
    if (t < 0 || t >= a.n_dst) return;
    const float s = a.scale[k], z = a.zero[k];
    const uint8_t* in = a.codes + k * a.ld_codes;
    T* row = reinterpret_cast<T*>(a.dst) + t * a.ld_dst;
    const int64_t groups = (a.d + 7) / 8;
    const uint64_t mask = (1ull << a.bits) - 1;
    for (int64_t g = gl; g < groups; g += G) {
        const uint64_t packed = load_codes(in + g * a.bits, a.bits);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float q = static_cast<float>(static_cast<uint32_t>((packed >> (a.bits * e)) & mask));
            const float prod = q * s;
            v[e] = prod + z;
        }
        const int64_t j0 = 8 * g;
        if constexpr (ACC) {
            float old[8];
            load8<T>(row, g, a.d, old);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = old[e] + v[e];
        }
        if (j0 + 8 <= a.d) {
            if constexpr (sizeof(T) == 2) {
                store_vals<T>(row + j0, v, 8);
            } else {
                store_vals<T>(row + j0, v, 4);
                store_vals<T>(row + j0 + 4, v + 4, 4);
            }
        } else {
            for (int e = 0; j0 + e < a.d; ++e) row[j0 + e] = from_f32<T>(v[e]);
        }
    }
}

template <class T, int BITS>
sag_status launch_q(const QArgs& a, hipStream_t s) {
    const int64_t groups = (a.d + 7) / 8;
    auto go = [&](auto gc) {
        constexpr int G = decltype(gc)::value;
        quantize_rows<T, G, BITS><<<dim3(static_cast<unsigned>(cdiv(a.n, 256 / G))), dim3(256), 0, s>>>(a);
    };
    if (groups <= 4) go(std::integral_constant<int, 4>{});
    else if (groups <= 8) go(std::integral_constant<int, 8>{});
    else if (groups <= 16) go(std::integral_constant<int, 16>{});
    else if (groups <= 32) go(std::integral_constant<int, 32>{});
    else go(std::integral_constant<int, 64>{});
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

template <class T, bool ACC>
sag_status launch_dq(const DArgs& a, hipStream_t s) {
    const int64_t groups = (a.d + 7) / 8;
    auto go = [&](auto gc) {
        constexpr int G = decltype(gc)::value;
        dequantize_rows<T, G, ACC><<<dim3(static_cast<unsigned>(cdiv(a.n, 256 / G))), dim3(256), 0, s>>>(a);
    };
    if (groups <= 4) go(std::integral_constant<int, 4>{});
    else if (groups <= 8) go(std::integral_constant<int, 8>{});
    else if (groups <= 16) go(std::integral_constant<int, 16>{});
    else if (groups <= 32) go(std::integral_constant<int, 32>{});
    else go(std::integral_constant<int, 64>{});
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

bool bits_ok(int bits) { return bits == 1 || bits == 2 || bits == 4 || bits == 8; }

int64_t code_row_bytes(int64_t d, int bits) { return round_up(((d + 7) / 8) * bits, 16); }

}  // namespace
}  // namespace sag

extern "C" size_t sag_code_row_bytes(int64_t d, int bits) {
    using namespace sag;
    if (d < 0 || !bits_ok(bits)) return 0;
    return static_cast<size_t>(code_row_bytes(d, bits));
}

extern "C" sag_status sag_quantize_rows(const void* src, int64_t ld_src, sag_dtype dt, const int32_t* rows,
                                        int64_t n_src, const int32_t* nodes, int64_t n, int64_t d, int bits,
                                        uint64_t seed, uint32_t epoch, uint8_t* codes, int64_t ld_codes,
                                        float* scale, float* zero, void* stream) {
    using namespace sag;
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "quantize_rows: bad dtype");
    if (!bits_ok(bits)) return fail(SAG_E_INVALID, "quantize_rows: bits must be 1, 2, 4 or 8");
    if (n < 0 || d < 0 || n_src < 0) return fail(SAG_E_INVALID, "quantize_rows: negative size");
    if (n == 0) return SAG_OK;
    if (!codes || !scale || !zero) return fail(SAG_E_INVALID, "quantize_rows: null output");
    if (!aligned16(codes) || ld_codes % 16 != 0 || ld_codes < code_row_bytes(d, bits))
        return fail(SAG_E_ALIGN, "quantize_rows: codes must be 16-byte aligned with ld_codes >= sag_code_row_bytes");
    if (n_src > 0) SAG_TRY(check_dense("quantize_rows src", src, n_src, d > 0 ? d : 1, ld_src, dt));
    QArgs a{static_cast<const char*>(src), ld_src, rows, n_src, nodes, n, d, bits,
            static_cast<uint32_t>(seed & 0xffffffffu), static_cast<uint32_t>(seed >> 32), epoch,
            codes, ld_codes, scale, zero};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t e = elt_size(dt);
    TraceScope trace(trace_enabled() ? shape_name("quantize", dt == SAG_BF16 ? "bf16" : "f32", n, d, bits)
                                     : std::string(),
                     s, n * (d * e + (d * bits + 7) / 8 + 8 + (rows ? 4 : 0) + (nodes ? 4 : 0)), 0);
    auto go = [&](auto bc) {
        constexpr int BITS = decltype(bc)::value;
        return dt == SAG_BF16 ? launch_q<uint16_t, BITS>(a, s) : launch_q<float, BITS>(a, s);
    };
    switch (bits) {
        case 1: return go(std::integral_constant<int, 1>{});
        case 2: return go(std::integral_constant<int, 2>{});
        case 4: return go(std::integral_constant<int, 4>{});
        default: return go(std::integral_constant<int, 8>{});
    }
}

extern "C" sag_status sag_dequantize_rows(const uint8_t* codes, int64_t ld_codes, const float* scale,
                                          const float* zero, int64_t n, int64_t d, int bits, const int32_t* ids,
                                          int64_t row_base, int accumulate, sag_dtype dt, void* dst,
                                          int64_t ld_dst, int64_t n_dst, void* stream) {
    using namespace sag;
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "dequantize_rows: bad dtype");
    if (!bits_ok(bits)) return fail(SAG_E_INVALID, "dequantize_rows: bits must be 1, 2, 4 or 8");
    if (n < 0 || d < 0 || n_dst < 0) return fail(SAG_E_INVALID, "dequantize_rows: negative size");
    if (n == 0 || d == 0 || n_dst == 0) return SAG_OK;
    if (!codes || !scale || !zero) return fail(SAG_E_INVALID, "dequantize_rows: null input");
    if (!aligned16(codes) || ld_codes % 16 != 0 || ld_codes < code_row_bytes(d, bits))
        return fail(SAG_E_ALIGN, "dequantize_rows: codes must be 16-byte aligned with ld_codes >= sag_code_row_bytes");
    SAG_TRY(check_dense("dequantize_rows dst", dst, n_dst, d, ld_dst, dt));
    DArgs a{codes, ld_codes, scale, zero, n, d, bits, ids, row_base, n_dst, static_cast<char*>(dst), ld_dst};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t e = elt_size(dt);
    TraceScope trace(trace_enabled() ? shape_name("dequantize", dt == SAG_BF16 ? "bf16" : "f32", n, d, bits)
                                     : std::string(),
                     s, n * (d * e * (accumulate ? 2 : 1) + (d * bits + 7) / 8 + 8 + (ids ? 4 : 0)), 0);
    if (dt == SAG_BF16)
        return accumulate ? launch_dq<uint16_t, true>(a, s) : launch_dq<uint16_t, false>(a, s);
    return accumulate ? launch_dq<float, true>(a, s) : launch_dq<float, false>(a, s);
}
