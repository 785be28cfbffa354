// Device helpers shared by the gfx950 kernels of this library.
//
// Cross-workgroup communication (the decoupled look-back) follows the gfx942 /
// gfx950 memory model: the L2 is per XCD and an agent-scope fence writes back
// and invalidates it, which is slow.  Status words and payloads are
// therefore written and read with relaxed agent-scope atomics of at most 64
// bits (sc1, device coherent: single-copy atomic, and seen by every XCD
// without a fence).  A status word of more than 64 bits is made of halves
// that each carry its tag, and a reader accepts it only when the tags agree.
// Larger payloads are written with such stores, completed with a vmcnt wait
// and a workgroup barrier, and only then announced by a flag store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cls {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Payloads larger than a status word are written and read with compiler-
// generated relaxed agent-scope 64-bit atomics (sc1, device coherent).  They
// must not be written with inline-asm stores that leave the store in flight:
// the compiler cannot see that such an instruction still reads its data
// registers and may overwrite them before the hardware has read the last
// dwords.  Publish with wait_vmem() + a barrier before the flag store.
__device__ __forceinline__ void store_payload(float* p, f32x4 v) {
    const uint64_t lo = uint64_t(__builtin_bit_cast(uint32_t, float(v.x))) |
                        (uint64_t(__builtin_bit_cast(uint32_t, float(v.y))) << 32);
    const uint64_t hi = uint64_t(__builtin_bit_cast(uint32_t, float(v.z))) |
                        (uint64_t(__builtin_bit_cast(uint32_t, float(v.w))) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p) + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 load_payload(const float* p) {
    const uint64_t lo = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p) + 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    f32x4 v;
    v.x = __builtin_bit_cast(float, uint32_t(lo));
    v.y = __builtin_bit_cast(float, uint32_t(lo >> 32));
    v.z = __builtin_bit_cast(float, uint32_t(hi));
    v.w = __builtin_bit_cast(float, uint32_t(hi >> 32));
    return v;
}

// Wait for every outstanding vector memory operation of this wave, and keep
// the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
}

__device__ __forceinline__ uint32_t load_coherent_u32(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent_u32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t atomic_add_u32(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reinterpret 32-bit words.  Always pass by value: __builtin_bit_cast applied
// directly to an ext_vector_type element (v[k]) reads element 0 in this
// compiler, so vector elements must be copied out first.
__device__ __forceinline__ float as_float(uint32_t w) { return __builtin_bit_cast(float, w); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---------------------------------------------------------------------------
// Wave helpers (64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float shfl_up(float v, int d) { return __shfl_up(v, d, 64); }
__device__ __forceinline__ float shfl_down(float v, int d) { return __shfl_down(v, d, 64); }
__device__ __forceinline__ int shfl_up_i(int v, int d) { return __shfl_up(v, d, 64); }

__device__ __forceinline__ float bcast_lane0(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// ---------------------------------------------------------------------------
// bf16 packing (round to nearest even, as the MFMA operands expect).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ldg_b128(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Inclusive sum over the first 256 threads of a 256-thread block (one value
// per thread).  `scratch` holds 4 floats of LDS.  Ends with a barrier.
__device__ __forceinline__ float block_inclusive_sum_256(float v, float* scratch) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    if (lane == 63) scratch[wave] = v;
    __syncthreads();
    float add = 0.0f;
#pragma unroll
    for (int q = 0; q < 3; ++q)
        if (q < wave) add += scratch[q];
    __syncthreads();
    return v + add;
}

// Transpose an 8x8 block of 16-bit values held as 8 rows of 16 bytes: on
// return out[c] holds column c (8 values, row 0 in the low half-word).
__device__ __forceinline__ void transpose8x8_b16(const u32x4 (&r)[8], u32x4 (&out)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = r[2 * m][k];
            const uint32_t hi = r[2 * m + 1][k];
            out[2 * k][m] = (lo & 0xffffu) | (hi << 16);
            out[2 * k + 1][m] = (lo >> 16) | (hi & 0xffff0000u);
        }
    }
}

}  // namespace cls
