// gdn_device.h - device helpers shared by the libgdn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------------------------
// bf16 <-> f32.  bf16 is the top half of an f32; f32 -> bf16 rounds to nearest, ties to even.
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_act(const void *p, size_t i)
{
    if constexpr (BF16)
        return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
    else
        return static_cast<const float *>(p)[i];
}

// ---------------------------------------------------------------------------------------------
// Cross-lane sums inside a row of 16 lanes with DPP (no LDS traffic):
//   quad_perm [1,0,3,2] and [2,3,0,1] give every lane its quad's sum, row_ror 4 and row_ror 8
//   then fold the four quads of the row.  All 16 lanes end with the row total.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x124>(x);  // row_ror:4
    x += dpp_mov<0x128>(x);  // row_ror:8
    return x;
}

// Sum over the whole 64-lane wave (prologue use only).
__device__ __forceinline__ float wave_sum(float x)
{
    x = row16_sum(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// A 16-byte store for write-once streams that no later kernel re-reads soon: global_store_dwordx4
// with the nontemporal and system-scope (sc1) cache-policy bits.  Measured on MI355X, plain stores
// of the 2 GiB verify capture, or of the state a rollback copies, leave dirty lines in L2 and the
// Infinity Cache that the next kernel pays to write back; nt alone keeps that cost off the next
// kernel, and sc1 with it streams faster still.  The compiler does not see this store in its
// memory-counter bookkeeping, so use it only where no later wait in the kernel depends on it.
// Nor does it see the ISA's wait-state rule for stores of more than 64 bits of data: a VALU
// instruction may not write the store's data registers in the cycle after it issues.  The compiler
// does reuse those registers at once when they die with the store (seen on a final-state store
// whose data came back corrupted), so the s_nop that it would insert for a store it knows about
// is part of the asm.
__device__ __forceinline__ void store_stream(void *p, f4 v)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
#else
    (void)p;
    (void)v;
#endif
}

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4).  The LDS address must be
// the same for the whole wave up to lane * 16: lane i lands at lds + 16 i of the first active lane.
// Tracked by the vector-memory counter like any load.  The builtin exists only for the device
// compilation pass; the host pass just needs the declaration to emit launch stubs.
__device__ __forceinline__ void lds_dma16(const void *g, void *lds)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
#else
    (void)g;
    (void)lds;
#endif
}

// Workgroup barrier for data exchanged through LDS by ds_read / ds_write: waits for this wave's
// own LDS operations, then meets the other waves.  No wait on the vector-memory counter, so
// outstanding global stores and global_load_lds prefetches stay in flight across it; LDS filled
// by global_load_lds must be waited for explicitly (s_waitcnt vmcnt) before the barrier that
// publishes it.  The memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
}

// Same, 4 bytes per lane: lane i lands at lds + 4 i of the first active lane.  The global address
// must be 4-byte aligned.
__device__ __forceinline__ void lds_dma4(const void *g, void *lds)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
#else
    (void)g;
    (void)lds;
#endif
}

// Depthwise causal conv tap sum, oldest input first; tap 3 multiplies the current token.  One
// fixed rounding order so every kernel produces identical bits for identical windows.
__device__ __forceinline__ float conv4(f4 w, float x0, float x1, float x2, float x3)
{
    return __builtin_fmaf(w[3], x3, __builtin_fmaf(w[2], x2, __builtin_fmaf(w[1], x1, w[0] * x0)));
}

__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }
// The logistic function on the vector ALU's exp2 and reciprocal: two transcendental instructions
// against ~25 for a correctly rounded expf and division.  Rounding the product -x log2(e) costs a
// relative error of about |x| 2^-24 in exp(-x), and the reciprocal about an ulp, so the result is
// within ~1e-6 relative for |x| < 16; where exp2 overflows the result is 0, as the limit is.
__device__ __forceinline__ float sigmoid_f(float x)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.44269504088896341f));
}
// 1 / sqrt(x) on the vector ALU's reciprocal square root (about an ulp).
__device__ __forceinline__ float rsqrt_f(float x) { return __builtin_amdgcn_rsqf(x); }

}  // namespace gdn
