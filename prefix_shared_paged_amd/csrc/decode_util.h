// decode_util.h -- device helpers shared by the split-K decode kernels
// (kernels_decode.hip: one KV head per workgroup; kernels_decode_rows.hip:
// all KV heads of a slot row per workgroup).
#pragma once

#include "common.h"

namespace sgl_decode {

// Position of 16-byte chunk c of K/V row r (within a tile) is c ^ swz<D>(r).
// A K operand read touches one chunk of all 16 rows; a V^T read touches two
// adjacent chunks of 8 rows per half wave.  For 16 chunks per row the swizzle
// puts the row's low three bits on chunk bits 1..3 and bit 3 on chunk bit 0.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
    return (r & 7) ^ ((r >> 3) & 1);                                // 8 chunks per row
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 ld_q(const __bf16 *p) {
    return __builtin_bit_cast(bf16x8, *(const u32x4 *)p);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));

// LDS reads of the tiles written by direct loads, as inline asm: the kernel
// itself waits for those loads (vmcnt) and, with several waves, meets at a
// barrier before reading, so the compiler must not add a wait for every
// direct load still in flight into the other buffer (its alias tracking of
// direct-to-LDS loads cannot tell the two buffers apart).  Each group of
// reads ends with lgkmcnt(0) tied to its results.
template <int N>
__device__ __forceinline__ void lds_read_b128(bf16x8 (&out)[N], const uint32_t (&addr)[N]) {
    u32x4 r[N];
#pragma unroll
    for (int i = 0; i < N; i++) asm volatile("ds_read_b128 %0, %1" : "=v"(r[i]) : "v"(addr[i]));
    if constexpr (N == 4)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]));
#pragma unroll
    for (int i = 0; i < N; i++) out[i] = __builtin_bit_cast(bf16x8, r[i]);
}
template <int N>
__device__ __forceinline__ void lds_read_tr16(i16x4 (&out)[N], const uint32_t (&addr)[N]) {
    i32x2 r[N];
#pragma unroll
    for (int i = 0; i < N; i++) asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r[i]) : "v"(addr[i]));
    if constexpr (N == 8)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
#pragma unroll
    for (int i = 0; i < N; i++) out[i] = __builtin_bit_cast(i16x4, r[i]);
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const SGL_LDS void *)p;
}

// s_waitcnt vmcnt(N), other counters untouched
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void lgkm_wait0() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
}

// Position of 16-byte chunk c of fp8 row r (within a tile) is c ^ swz8<D>(r):
// the 16 rows of a K operand read and the 8 rows of each V^T read fall on
// distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int swz8(int r) {
    if (D == 128) return ((r >> 1) ^ (r >> 3)) & 7;
    return ((r >> 2) ^ (r >> 3)) & 3;                                // 4 chunks per row
}

// 8 e4m3fn codes (little-endian in two words) -> 8 exact bf16 values
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// LDS reads as inline asm (see lds_read_b128), results tied to one wait
template <class T, int N>
__device__ __forceinline__ void lgkm_wait_tied(T (&r)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; i++) asm volatile("" : "+v"(r[i]));
}
template <int N>
__device__ __forceinline__ void lds_read_raw128(u32x4 (&r)[N], const uint32_t (&addr)[N]) {
#pragma unroll
    for (int i = 0; i < N; i++) asm volatile("ds_read_b128 %0, %1" : "=v"(r[i]) : "v"(addr[i]));
    lgkm_wait_tied(r);
}
template <int N>
__device__ __forceinline__ void lds_read_tr8(i32x2 (&r)[N], const uint32_t (&addr)[N]) {
#pragma unroll
    for (int i = 0; i < N; i++) asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(r[i]) : "v"(addr[i]));
    lgkm_wait_tied(r);
}

}  // namespace sgl_decode
