// Device-side helpers for the KDA kernels (gfx950 / CDNA4 only).
//
// Matrix cores: every dense contraction in the library goes through one of
// two MFMA shapes, both producing a 16x16 fp32 tile per wavefront of 64:
//   bf16: v_mfma_f32_16x16x32_bf16  (contraction 32, 8 values per lane)
//   fp32: v_mfma_f32_16x16x4_f32    (contraction 4,  1 value  per lane)
// Operand layout used throughout (lane = 0..63, grp = lane / 16):
//   A fragment: row  = lane % 16, k = kbase + grp * KPL + j   (j < KPL)
//   B fragment: col  = lane % 16, k = kbase + grp * KPL + j
//   D tile:     row  = 4 * grp + r (r < 4), col = lane % 16
// A and B always use the same k mapping, so the contraction is correct for
// any assignment of k to (grp, j); only the D layout is relied upon.
// Both operands are therefore stored "k-contiguous": A as [rows][k] and B as
// [cols][k], so one fragment is one contiguous 16-byte (bf16) read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kTile = 16;  // MFMA tile edge, and the 16-token decay tile

// Lanes of one wave that exchange values through LDS with no workgroup
// barrier: a wave's LDS accesses execute in program order, and this point
// (wavefront-scope release and acquire around a wave barrier) keeps the
// compiler from moving any of the wave's memory accesses across it.  It
// emits no instruction that waits.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

template <class T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int K = 32;   // contraction per instruction
    static constexpr int KPL = 8;  // operand values per lane
    typedef bf16x8 Frag;
    static __device__ __forceinline__ floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ void set(Frag &f, int j, float x) { f[j] = static_cast<bf16>(x); }
    static __device__ __forceinline__ Frag load(const bf16 *p) {
        return *reinterpret_cast<const bf16x8 *>(p);
    }
    // 8 consecutive fp32 values rounded to an operand fragment
    static __device__ __forceinline__ Frag load_f32(const float *p) {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        Frag f;
        f[0] = static_cast<bf16>(a.x); f[1] = static_cast<bf16>(a.y);
        f[2] = static_cast<bf16>(a.z); f[3] = static_cast<bf16>(a.w);
        f[4] = static_cast<bf16>(b.x); f[5] = static_cast<bf16>(b.y);
        f[6] = static_cast<bf16>(b.z); f[7] = static_cast<bf16>(b.w);
        return f;
    }
};

template <> struct Mma<float> {
    static constexpr int K = 4;
    static constexpr int KPL = 1;
    typedef float Frag;
    static __device__ __forceinline__ floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ void set(Frag &f, int, float x) { f = x; }
    static __device__ __forceinline__ Frag load(const float *p) { return *p; }
    static __device__ __forceinline__ Frag load_f32(const float *p) { return *p; }
};

// fp32 16x16x4 MFMA, used for the fp32 triangular-inverse block products on
// both paths.
__device__ __forceinline__ floatx4 mma_f32(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// Natural exponential through the hardware base-2 exponential.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float exp_e(float x) { return exp2_hw(x * kLog2e); }

// Store four consecutive values of type T (8 bytes for bf16, 16 for fp32).
__device__ __forceinline__ void store4(bf16 *p, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = static_cast<bf16>(a); v[1] = static_cast<bf16>(b);
    v[2] = static_cast<bf16>(c); v[3] = static_cast<bf16>(d);
    *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

// Four consecutive values of one column (four tokens of a channel), rounded
// to T as they are produced, so that fewer registers hold them until the
// column is stored at once.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <class T> struct Col4 {
    float v[4];
    __device__ __forceinline__ void set(int r, float x) { v[r] = x; }
    __device__ __forceinline__ void store(T *p) const { store4(p, v[0], v[1], v[2], v[3]); }
};
template <> struct Col4<bf16> {
    bf16x2 h[2];
    float lo;
    __device__ __forceinline__ void set(int r, float x) {
        if (r & 1) h[r >> 1] = bf16x2{static_cast<bf16>(lo), static_cast<bf16>(x)};
        else lo = x;
    }
    __device__ __forceinline__ void store(bf16 *p) const {
        *reinterpret_cast<bf16x4 *>(p) = bf16x4{h[0][0], h[0][1], h[1][0], h[1][1]};
    }
};

// 16-byte vector of T (8 bf16 or 4 fp32) for coalesced global <-> LDS copies.
template <class T> struct Vec16 {
    static constexpr int N = 16 / sizeof(T);
    uint4 raw;
    __device__ __forceinline__ float get(int i) const {
        const T *p = reinterpret_cast<const T *>(&raw);
        return to_f32(p[i]);
    }
};

}  // namespace kda
