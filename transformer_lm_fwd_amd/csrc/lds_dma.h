// gfx950 helpers shared by the LDS-staged kernels: buffer loads straight into LDS
// and the transposed LDS read.
#pragma once

#include "common.h"

namespace gpt2 {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4_t;

// Buffer resource over [base, base + bytes): loads at or past the end return zero.
typedef uint32_t dsc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ dsc_t make_dsc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    dsc_t d;
    d[0] = (uint32_t)b;
    d[1] = (uint32_t)(b >> 32) & 0xffffu;  // stride 0
    d[2] = bytes;
    d[3] = 0x00020000u;
    return d;
}

// One wave load of 64 x 16 bytes from d + voff + soff (per lane) into LDS at the
// wave-uniform byte address `lds_addr` (lane i writes lds_addr + 16 i).  Written as
// inline assembly on purpose: the compiler, seeing an LDS write it cannot place,
// would otherwise wait for every load in flight before each ds_read_b64_tr_b16 and
// serialise the pipeline.  Callers order these loads themselves: wait_loads + a
// barrier before a stage is read, lgkmcnt(0) + a barrier before it is overwritten.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const dsc_t& d, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(d), "s"(soff)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a pointer into shared memory, made wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)p);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): all but this wave's N most recent loads into LDS
// have landed, and its own LDS reads are done.
template <int N> __device__ __forceinline__ void wait_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// ds_read_b64_tr_b16 at byte offset o of an LDS array: within each 16-lane group,
// lane j receives element j % 4 of the 8-byte words addressed by lanes j/4, 4 + j/4,
// 8 + j/4, 12 + j/4 of the group.  With lane i addressing (row k0 + i/4, columns
// n0 + 4 (i%4) .. +3) of a row-major bf16 tile, lane j gets rows k0..k0+3 of column
// n0 + j.
__device__ __forceinline__ v4i16 read_tr(const void* base, int o) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_t)((const char*)base + o));
}
// Two transposed reads joined into one 8 x bf16 MFMA operand.
__device__ __forceinline__ u32x4 read_tr2(const void* base, int o0, int o1) {
    const v4i16 lo = read_tr(base, o0), hi = read_tr(base, o1);
    u32x4 r;
    r[0] = (uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    r[1] = (uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    r[2] = (uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    r[3] = (uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return r;
}

}  // namespace gpt2
