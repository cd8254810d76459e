// Device-side helpers shared by the gfx950 kernels of liblcsi.
// Wave64 only: every helper assumes 64 lanes per wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcsi {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Number of set bits of `mask` strictly below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (lo in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 (the same rounding as f32_to_bf16_bits for finite
// inputs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Two fp32 -> two IEEE fp16 (lo in the low half), round to nearest even,
// and back (exact).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
__device__ __forceinline__ float f16_lo(uint32_t v) { return (float)__builtin_bit_cast(f16x2, v)[0]; }
__device__ __forceinline__ float f16_hi(uint32_t v) { return (float)__builtin_bit_cast(f16x2, v)[1]; }

// Four OCP E4M3 bytes (one dword) -> four bf16 values packed in two dwords
// (byte i -> half i), with the hardware conversion at scale 1.  Every finite
// E4M3 value (3 mantissa bits, exponents 2^-9 .. 2^8) is exactly a bf16
// value, so the conversion is exact.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w)
{
    u32x2 r{0, 0};
#if defined(__HIP_DEVICE_COMPILE__)
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
#else
    (void)w;
#endif
    return r;
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 is
// mapped like +0 so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float x)
{
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// x[lane] + x[lane ^ 32], formed as (lower half + upper half) in every lane,
// with v_permlane32_swap (a VALU op: no LDS traffic, no lgkmcnt wait).  With
// old = src = x the swap returns, in every lane, the lower-half value in
// element 0 and the upper-half value in element 1.
__device__ __forceinline__ float sum_lane_halves(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 32-bit store through a buffer resource over [base, base + bytes): a lane
// whose byte offset is not below `bytes` has its store dropped by the
// hardware's range check, so per-lane masking needs no branch (and the
// compiler can count outstanding memory operations exactly).  base and
// bytes must be wave-uniform; bytes < 2^31.
__device__ __forceinline__ void store_b32_ranged(float *base, uint32_t bytes, uint32_t off, float v)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000),
                                          (int)off, 0, 0);
#else
    (void)base;
    (void)bytes;
    (void)off;
    (void)v;
#endif
}

// 64-bit store through a buffer resource, with the same range rule as above.
__device__ __forceinline__ void store_b64_ranged(void *base, uint32_t bytes, uint32_t off, u32x2 v)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_buffer_store_b64(v, __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000), (int)off,
                                          0, 0);
#else
    (void)base;
    (void)bytes;
    (void)off;
    (void)v;
#endif
}

// Direct global->LDS load (global_load_lds_dwordx4): every lane loads 16
// bytes from its own address; lane l's bytes land at lds + 16*l (lds is
// wave-uniform).  The builtin is only spelled out for the device pass: in
// the host pass of the same source an LDS builtin on a computed pointer
// suppresses the host-side launch stub of the kernel that calls it, and a
// __device__ function never runs on the host.
__device__ __forceinline__ void load_to_lds16(const void *src, uint8_t *lds)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#else
    (void)src;
    (void)lds;
#endif
}

// Direct buffer->LDS load (buffer_load_dwordx4 ... lds) of 16 bytes per lane
// from base + off, through a buffer resource of `bytes` bytes: a lane whose
// 16 bytes lie past the end gets zeros.  Lane l's bytes land at lds + 16*l
// (base, bytes and lds wave-uniform; bytes < 2^31).  Device pass only, as
// above.
__device__ __forceinline__ void buffer_load_to_lds16(const void *base, uint32_t bytes, uint32_t off, uint8_t *lds)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000),
        (__attribute__((address_space(3))) void *)lds, 16, (int)off, 0, 0, 0);
#else
    (void)base;
    (void)bytes;
    (void)off;
    (void)lds;
#endif
}

// 16-byte load through a buffer resource over [base, base + bytes): bytes
// past the end read as zero, so a guarded load needs no branch (and the
// compiler can count outstanding loads exactly).  base and bytes
// wave-uniform; bytes < 2^31.
__device__ __forceinline__ u32x4 ld16_ranged(const void *base, uint32_t bytes, uint32_t off)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000),
                                         (int)off, 0, 0));
#else
    (void)base;
    (void)bytes;
    (void)off;
    return u32x4{0, 0, 0, 0};
#endif
}

// ld16_ranged with the non-temporal hint: for data read once, in whole cache
// lines per load instruction.
__device__ __forceinline__ u32x4 ld16_ranged_nt(const void *base, uint32_t bytes, uint32_t off)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000),
                                         (int)off, 0, 2));
#else
    (void)base;
    (void)bytes;
    (void)off;
    return u32x4{0, 0, 0, 0};
#endif
}

__device__ __forceinline__ float ld4_ranged(const void *base, uint32_t bytes, uint32_t off)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000),
                                         (int)off, 0, 0));
#else
    (void)base;
    (void)bytes;
    (void)off;
    return 0.f;
#endif
}

// Workgroup barrier for LDS hand-offs only: no memory-model fence, so the
// compiler does not wait for this wave's outstanding global stores or
// direct-to-LDS loads (the caller waits for what it needs first); the empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt on the LDS/scalar-memory counter only: this wave's LDS writes
// have completed (vector-memory loads still in flight are not waited on).
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

// s_waitcnt on the vector-memory counter only: wait until at most N vector
// memory operations of this wave are outstanding (N < 64); LDS and export
// counters are not waited on.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int wave_sum_int(int v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace lcsi
