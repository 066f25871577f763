// common.h -- device helpers shared by the gfx950 kernels of libmssm.
//
// Storage types: float (MSSM_F32) and bfloat16 carried as uint16_t
// (MSSM_BF16).  All arithmetic is float32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));

// --- scalar conversions ----------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint16_t to_bf16(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// 2^x with the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait for every outstanding LDS / scalar-memory operation (s_waitcnt
// lgkmcnt(0): vmcnt and expcnt fields at their maximum, gfx9 encoding), and
// keep the scheduler from moving instructions across this point.
__device__ __forceinline__ void lgkm_wait_all() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
}

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(w), w = e^-|v| in (0, 1].
// With u = 1 + w rounded to float and c = w - (u - 1) its rounding error
// (|c| <= 2^-24), log1p(w) = log(u) + log(1 + c / u).  The last term is c / u
// to first order; c (1 - w) stands in for it with an error below 2^-24 w^2,
// so no division is needed (when u rounds to 1 the result is w - w^2).
__device__ __forceinline__ float softplus_f(float v) {
    const float w = fast_exp2(-fabsf(v) * kLog2e);
    const float u = 1.0f + w;
    const float c = w - (u - 1.0f);
    return fmaxf(v, 0.0f) + fmaf(__builtin_amdgcn_logf(u), kLn2, fmaf(-c, w, c));
}

// silu(g) = g * sigmoid(g) = g / (1 + e^-g).
__device__ __forceinline__ float silu(float g) {
    const float e = fast_exp2(-g * kLog2e);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// --- range-checked buffer access ----------------------------------------------
// A raw buffer resource (stride 0) covering `bytes` bytes from `base`.  Loads
// at offsets >= bytes return zero and stores there are dropped by the
// hardware, so tails and idle lanes need no branches (which also keeps the
// compiler's wait counting exact).  Offsets are 32-bit byte offsets.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;   // any offset >= every buffer size used
constexpr int kRsrcWord3 = 0x00020000;          // raw 32-bit data format

// `off` if `ok`, else kOutOfRange.  The value goes through an empty asm, so
// the compiler must keep the choice a select: left visible, it may rewrite
// the select as a branch around the load and then, at the join, wait for
// every load in flight -- prefetched ones included.
__device__ __forceinline__ uint32_t off_if(bool ok, uint32_t off) {
    uint32_t v = ok ? off : kOutOfRange;
    asm("" : "+v"(v));
    return v;
}

// Makes `v` opaque to the optimiser, so a later `cond ? v : 0` stays a
// select instead of a branch around the code that computes v.
__device__ __forceinline__ void keep_select(float& v) { asm("" : "+v"(v)); }

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

typedef unsigned int u32x2_t __attribute__((__vector_size__(2 * sizeof(unsigned int))));
typedef unsigned int u32x4_t __attribute__((__vector_size__(4 * sizeof(unsigned int))));

// Cache-policy bits of a buffer access: kStream marks data touched once
// (non-temporal), so streamed outputs do not displace reused lines in L2.
constexpr int kCached = 0;
constexpr int kStream = 2;

// Load / store KW 32-bit words (KW = 2, 4 or 8) at byte offset `off`.
template <int KW, int AUX = kCached>
__device__ __forceinline__ void buf_load(rsrc_t r, uint32_t off, uint32_t* w) {
    static_assert(KW == 2 || KW == 4 || KW == 8, "2, 4 or 8 words");
    if constexpr (KW == 2) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
        w[0] = v[0]; w[1] = v[1];
    } else {
#pragma unroll
        for (int i = 0; i < KW / 4; ++i) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, AUX);
            w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
        }
    }
}
template <int KW, int AUX = kCached>
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t off, const uint32_t* w) {
    static_assert(KW == 2 || KW == 4 || KW == 8, "2, 4 or 8 words");
    if constexpr (KW == 2) {
        const u32x2_t v = {w[0], w[1]};
        __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, AUX);
    } else {
#pragma unroll
        for (int i = 0; i < KW / 4; ++i) {
            const u32x4_t v = {w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(v, r, off + 16 * i, 0, AUX);
        }
    }
}
__device__ __forceinline__ uint32_t buf_load1(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Pack CNT floats into storage words of type T (bf16 pairs or fp32 bits).
template <typename T, int CNT>
__device__ __forceinline__ void pack_words(const float (&v)[CNT], uint32_t (&w)[CNT * sizeof(T) / 4]) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < CNT; ++i) w[i] = __float_as_uint(v[i]);
    } else {
#pragma unroll
        for (int i = 0; i < CNT / 2; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    }
}

// --- per-dtype element access over packed 32-bit words ----------------------
// A run of CNT elements of type T held as CNT*sizeof(T)/4 words.
template <typename T> struct Elem;

template <> struct Elem<float> {
    static constexpr int kPerWord = 1;
    __device__ __forceinline__ static float get(const uint32_t* w, int j) { return __uint_as_float(w[j]); }
    __device__ __forceinline__ static float load1(const float* p) { return *p; }
    __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

template <> struct Elem<uint16_t> {
    static constexpr int kPerWord = 2;
    __device__ __forceinline__ static float get(const uint32_t* w, int j) {
        const uint32_t x = w[j >> 1];
        return (j & 1) ? bf16_hi(x) : bf16_lo(x);
    }
    __device__ __forceinline__ static float load1(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }
    __device__ __forceinline__ static void store1(uint16_t* p, float v) { *p = to_bf16(v); }
};

// Load CNT consecutive elements starting at src into words w (CNT*sizeof(T)
// must be a multiple of 8).  `valid` elements are in range; the rest read
// as zero.  `vec` says src is aligned to the vector width used (16 bytes
// when CNT*sizeof(T) is a multiple of 16, else 8).
template <typename T, int CNT>
__device__ __forceinline__ void load_run(const T* __restrict__ src, int valid, bool vec,
                                         uint32_t (&w)[CNT * sizeof(T) / 4]) {
    constexpr int kWords = CNT * sizeof(T) / 4;
    static_assert(kWords % 2 == 0, "runs are whole 8-byte vectors");
    if (vec && valid >= CNT) {
        if constexpr (kWords % 4 == 0) {
            const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
            for (int i = 0; i < kWords / 4; ++i) {
                const uint4 v = s4[i];
                w[4 * i + 0] = v.x;
                w[4 * i + 1] = v.y;
                w[4 * i + 2] = v.z;
                w[4 * i + 3] = v.w;
            }
        } else {
            const uint2* s2 = reinterpret_cast<const uint2*>(src);
#pragma unroll
            for (int i = 0; i < kWords / 2; ++i) {
                const uint2 v = s2[i];
                w[2 * i + 0] = v.x;
                w[2 * i + 1] = v.y;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kWords; ++i) w[i] = 0u;
#pragma unroll
        for (int j = 0; j < CNT; ++j) {
            if (j < valid) {
                if constexpr (sizeof(T) == 4) {
                    w[j] = __float_as_uint(reinterpret_cast<const float*>(src)[j]);
                } else {
                    const uint32_t bits = reinterpret_cast<const uint16_t*>(src)[j];
                    w[j >> 1] |= (j & 1) ? (bits << 16) : bits;
                }
            }
        }
    }
}

// Store CNT floats as T (only the first `valid`), vectorised when aligned.
template <typename T, int CNT>
__device__ __forceinline__ void store_run(T* __restrict__ dst, int valid, bool vec, const float (&v)[CNT]) {
    if (vec && valid >= CNT) {
        if constexpr (sizeof(T) == 2 && CNT == 4) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else if constexpr (sizeof(T) == 4) {
            float4* d4 = reinterpret_cast<float4*>(dst);
#pragma unroll
            for (int i = 0; i < CNT / 4; ++i)
                d4[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        } else {
            uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
            for (int i = 0; i < CNT / 8; ++i)
                d4[i] = make_uint4(pack_bf16x2(v[8 * i + 0], v[8 * i + 1]), pack_bf16x2(v[8 * i + 2], v[8 * i + 3]),
                                   pack_bf16x2(v[8 * i + 4], v[8 * i + 5]), pack_bf16x2(v[8 * i + 6], v[8 * i + 7]));
        }
    } else {
#pragma unroll
        for (int j = 0; j < CNT; ++j)
            if (j < valid) Elem<T>::store1(dst + j, v[j]);
    }
}

}  // namespace mssm
