// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace nf4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two float32 -> one dword of two bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l holds A row (l % 32), B column (l % 32), both at k = 8*(l/32) .. +7;
// accumulator element e of lane l is D[8*(e/4) + 4*(l/32) + e%4][l % 32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l holds A row (l % 16), B column (l % 16), both at k = 8*(l/16) .. +7;
// accumulator element e of lane l is D[4*(l/16) + e][l % 16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Split an fp32 value v into bf16 hi + lo with hi = RNbf(v), lo = RNbf(v - hi);
// hi + lo equals v to about 2^-17 relative, so an MFMA fed with both keeps fp32-like
// accuracy for the small LoRA operands (u, g).
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
    hi = (__bf16)v;
    lo = (__bf16)(v - (float)hi);
}

// The dispatcher hands workgroups to the 8 XCDs (each with its own L2) round-robin
// in linear-id order. xcd_tile_order maps linear id L of a grid of `total`
// workgroups to a tile index such that each XCD runs one contiguous range of tile
// indices, in order: tiles that share operands and sit next to each other in the
// tile order then meet in the same L2 at about the same time. A bijection on
// [0, total) for any total.
constexpr uint32_t kXcds = 8;

__host__ __device__ __forceinline__ uint32_t xcd_tile_order(uint32_t L, uint32_t total) {
    const uint32_t q = total / kXcds, rem = total % kXcds;
    const uint32_t xcd = L % kXcds, local = L / kXcds;
    return xcd < rem ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
}

// Balanced two-round split (pick_balanced on the host): workgroups [0, 2 x round) of
// the split tiles, round = the CU count; linear ids L and L + round run on one CU.
// Round 0 (L < round) holds the
// a * pa pieces of tiles [0, a) (pa pieces each) and then pieces of the other tiles
// (pa + 1 each), round 1 only the latter; within a round the logical order is
// XCD-aware (xcd_tile_order), so neighbouring tiles - the token tiles of one weight
// slice - meet in one L2. Piece z of P covers steps [z S / P, (z + 1) S / P): all
// pieces of a tile are non-empty and differ by at most one step.
__host__ __device__ __forceinline__ void balanced_piece(uint32_t L, uint32_t round, int tail, int a, int pa, int steps,
                                                        int& q, int& z, int& s0, int& s1) {
    const int l = int(xcd_tile_order(L % round, round));
    const int na = a * pa, b = tail - a;
    int P;
    if (L < round && l < na) {
        q = l % a;
        z = l / a;
        P = pa;
    } else {
        const int v = L < round ? l - na : int(round) - na + l;
        q = a + v % b;
        z = v / b;
        P = pa + 1;
    }
    s0 = int(int64_t(z) * steps / P);
    s1 = int(int64_t(z + 1) * steps / P);
}

// Raw buffer resource over [base, base + bytes): loads at or beyond `bytes` return 0
// in hardware, which replaces per-load bounds branches. Third-dword flags for the
// gfx9 family (gfx950 included).
// The base and size must be wave-uniform; they are passed through readfirstlane so
// the descriptor lives in SGPRs (no per-load waterfall loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    void* p = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, int(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000);
}

// A byte offset past every buffer the entry points accept (they cap each operand a
// kernel wraps in one descriptor at 2^30 bytes): loads from it return zero.
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
}

__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, 0));
}

// Non-temporal variants (the load's nt cache-policy bit): for data each kernel reads once
// while streaming, such as a weight matrix read by a few-token kernel.
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 2));
}

__device__ __forceinline__ u32x2 buf_load8_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, 2));
}

__device__ __forceinline__ uint32_t buf_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0));
}

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0));
}

// Direct global -> LDS copy of 16 bytes per lane (gfx950 buffer_load_dwordx4 ... lds):
// lane i of the wave writes lds_wave_base + 16 * i; out-of-range reads write zeros.
// lds_wave_base must be wave-uniform. Completion is tracked by vmcnt of the issuing wave.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, int(off), 0, 0,
                                             0);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained); N is a compile-time constant.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace nf4
