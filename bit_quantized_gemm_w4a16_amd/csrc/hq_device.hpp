// Device-side helpers for the gfx950 kernels: vector types, MFMA wrappers,
// 4-bit decode, stores.  Header-only, included by the *.hip files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace hq {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v6u __attribute__((ext_vector_type(6)));
typedef unsigned v16u __attribute__((ext_vector_type(16)));

union Frag8 {  // eight 16-bit values = one MFMA A/B operand of 16x16x32 f16/bf16
    v4u u;
    v8h h;
    v8bf b;
};

// One 16x16x32 MFMA step with fp32 accumulation.  Lane l supplies row/column
// (l & 15) and eight K values; A and B use the same K labelling, so any
// consistent assignment of K values to (lane >> 4, element) is a valid GEMM.
template <bool BF16>
__device__ __forceinline__ v4f mfma16(const Frag8& a, const Frag8& b, v4f c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.b, b.b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.h, b.h, c, 0, 0, 0);
}

// fp32 -> bf16 / fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}
template <bool BF16>
__device__ __forceinline__ uint16_t f32_to_16(float f) {
    if constexpr (BF16) return f32_to_bf16_bits(f);
    else return f32_to_f16_bits(f);
}
template <bool BF16>
__device__ __forceinline__ float bits16_to_f32(uint16_t v) {
    if constexpr (BF16) return __uint_as_float((uint32_t)v << 16);
    else return (float)__builtin_bit_cast(_Float16, v);
}

// Buffer-resource loads: base and size live in scalar registers, each lane
// supplies a 32-bit offset and a wave-uniform offset goes in an SGPR, so a
// staged load costs one VGPR of address instead of two.  A lane offset at or
// beyond `bytes` reads zeros instead of touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // word 3 = 0x00020000: raw (untyped) 32-bit data format, as the gfx9 ISA requires for range checks
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef __attribute__((address_space(3))) void* lds_ptr;  // LDS destination of a direct global->LDS load
typedef __attribute__((address_space(3))) char lds_char;

// Direct HBM -> LDS loads (buffer_load ... lds) of 16 or 4 bytes per lane:
// lane l of the wave writes lds + l * size; `lds` must be the same for the
// whole wave, and is an LDS-space pointer taken straight from the __shared__
// array (through a generic pointer the compiler loses which array a load
// writes, and then makes every later LDS read wait for it).  The _nt form
// marks the data non-temporal.  The builtin exists
// only in the device pass (the host pass rejects its operands, and inside a
// kernel template that rejection silently drops the kernel's launch stub),
// and its size operand must be a literal, hence one helper per size.
__device__ __forceinline__ void dma16(rsrc_t r, lds_ptr lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
#endif
}
__device__ __forceinline__ void dma16_nt(rsrc_t r, lds_ptr lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 2);
#endif
}
__device__ __forceinline__ void dma4(rsrc_t r, lds_ptr lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, soff, 0, 0);
#endif
}
template <bool NT = false>
__device__ __forceinline__ v4u buf16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? 2 : 0));
}
__device__ __forceinline__ uint64_t buf8(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf4(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf2(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf1(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// Direct global -> LDS loads through a flat pointer (16 or 4 bytes per lane):
// lane l writes lds_wave_base + l * size; the base must be wave-uniform.
__device__ __forceinline__ void lds_dma16(const void* g, char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* g, char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 4, 0, 0);
}

// 16-byte global loads: a non-temporal hint for data read exactly once.
__device__ __forceinline__ v4u ld_nt(const v4u* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ v4u ld16(const void* p) { return *(const v4u*)p; }

}  // namespace hq
