// common.hpp -- device-side vocabulary shared by the gfx950 kernels of the
// Maglev attention path: vector types, bf16 conversion, MFMA wrappers, the
// LDS transpose read, and small helpers.
//
// MFMA lane layouts (checked on gfx950 by an in-bounds probe):
//   v_mfma_f32_32x32x16_bf16: operand lane l holds row/column (l % 32) and the
//     8 consecutive K entries 8*(l/32) .. +7; result lane l holds column l % 32,
//     rows 8*(e/4) + 4*(l/32) + (e % 4) for e = 0..15.
//   ds_read_tr16_b64: inside each group of 16 lanes, lane i receives element
//     (i % 4) of the 4-element rows addressed by lanes i/4 + 4k, k = 0..3. With
//     lane j addressing row k0 + j/4 at column n0 + 4*(j%4), lane i receives the
//     4 consecutive rows k0..k0+3 of column n0 + i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace maglev {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define MAGLEV_DEV __device__ __forceinline__

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// float -> bf16, round to nearest even (the gfx950 conversion instruction).
MAGLEV_DEV bf16 f2bf(float x) { return (bf16)x; }
MAGLEV_DEV float bf2f(bf16 x) { return (float)x; }

// Storage-type agnostic load/store of one element.
template <typename T> MAGLEV_DEV float to_f(T x);
template <> MAGLEV_DEV float to_f<float>(float x) { return x; }
template <> MAGLEV_DEV float to_f<bf16>(bf16 x) { return (float)x; }
template <typename T> MAGLEV_DEV T from_f(float x);
template <> MAGLEV_DEV float from_f<float>(float x) { return x; }
template <> MAGLEV_DEV bf16 from_f<bf16>(float x) { return (bf16)x; }

// 8 consecutive elements of type T as floats (16-byte or 32-byte loads).
MAGLEV_DEV void load8(const bf16 *p, float *out)
{
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
}
MAGLEV_DEV void load8(const float *p, float *out)
{
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
}
MAGLEV_DEV void store8(bf16 *p, const float *in)
{
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)in[i];
    *reinterpret_cast<bf16x8 *>(p) = v;
}
MAGLEV_DEV void store8(float *p, const float *in)
{
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = in[i]; b[i] = in[4 + i]; }
    *reinterpret_cast<f32x4 *>(p) = a;
    *reinterpret_cast<f32x4 *>(p + 4) = b;
}

MAGLEV_DEV bf16x8 pack8(const float *in)
{
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)in[i];
    return v;
}

MAGLEV_DEV f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

MAGLEV_DEV f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read of four 16-bit values (see the layout note above).
MAGLEV_DEV i16x4 lds_read_tr16(const bf16 *p)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// Two transpose reads joined into one 8-entry MFMA operand.
MAGLEV_DEV bf16x8 join_tr(i16x4 lo, i16x4 hi)
{
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    return __builtin_bit_cast(bf16x8, v);
}

MAGLEV_DEV float gate_sigmoid(float g) { return 1.0f / (1.0f + __expf(-g)); }

// Wave-wide exchange with the lane 32 positions away.
MAGLEV_DEV float xor32(float x) { return __shfl_xor(x, 32, 64); }

MAGLEV_DEV float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

typedef __attribute__((address_space(3))) bf16 lds_bf16;

// 16 bytes from global memory straight into LDS: lane L's bytes land at
// lds_wave_base + 16 L (global_load_lds_dwordx4, LDS base in M0; counted by
// vmcnt). Written as inline assembly so that the compiler does not track it
// as an LDS store: it would otherwise wait for every load in flight before
// the next LDS read, which defeats multi-stage pipelining. The callers wait
// explicitly (wait_vmcnt) before a barrier that publishes the stage. The
// instruction has no register results.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; it is clobbered on purpose
MAGLEV_DEV void dma16(const bf16 *src, bf16 *lds_wave_base)
{
    const unsigned m = (unsigned)(uintptr_t)(lds_bf16 *)lds_wave_base;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m)
                 : "memory", "m0");
}
// As dma16, from a raw buffer: lane L's 16 bytes at byte offset voff of the
// buffer described by rs (buffer_load_dwordx4 ... lds). The callers keep
// every offset inside the buffer.
MAGLEV_DEV void dma16_buf(__amdgpu_buffer_rsrc_t rs, unsigned voff, bf16 *lds_wave_base)
{
    const unsigned m = (unsigned)(uintptr_t)(lds_bf16 *)lds_wave_base;
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
                 "s"(m)
                 : "memory", "m0");
}
// As dma16_buf for data read once (nontemporal: not kept in the caches that
// hold re-read tiles).
MAGLEV_DEV void dma16_buf_once(__amdgpu_buffer_rsrc_t rs, unsigned voff, bf16 *lds_wave_base)
{
    const unsigned m = (unsigned)(uintptr_t)(lds_bf16 *)lds_wave_base;
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff),
                 "s"(rs), "s"(m)
                 : "memory", "m0");
}
// 4 bytes a lane from global memory straight into LDS: lane L's word lands at
// lds_wave_base + 4 L (global_load_lds_dword); otherwise as dma16.
MAGLEV_DEV void dma4(const float *src, void *lds_wave_base)
{
    const unsigned m = (unsigned)(uintptr_t)(lds_bf16 *)static_cast<bf16 *>(lds_wave_base);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
MAGLEV_DEV void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Map a linear workgroup id so that consecutive logical tiles share an XCD
// (workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2): XCD x receives the nwg/8 (+1 for x < nwg mod 8) consecutive items from
// x * (nwg/8) + min(x, nwg mod 8), in dispatch order.
MAGLEV_DEV int xcd_remap(int wg, int nwg)
{
    const int q = nwg >> 3, r = nwg & 7, x = wg & 7;
    return x * q + (x < r ? x : r) + (wg >> 3);
}

}  // namespace maglev
