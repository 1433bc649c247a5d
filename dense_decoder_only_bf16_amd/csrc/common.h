// Shared device-side definitions for the gfx950 kernels: vector types, MFMA wrappers,
// wave reductions, conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// A "chunk" is 8 consecutive elements along the contraction axis held by one lane as an
// MFMA operand: 16 bytes for bf16, 32 bytes for fp32.
template <typename T> struct Chunk;
template <> struct Chunk<bf16> { typedef bf16x8 type; typedef bf16x4 half; };
template <> struct Chunk<float> { typedef f32x8 type; typedef f32x4 half; };

// 32x32 output tile, 16-deep contraction.  Operand layout (both element types): lane l
// holds row/column (l % 32) and contraction indices 8*(l/32) .. 8*(l/32)+7.
// Output layout: lane l, register j holds row 8*(j/4) + 4*(l/32) + (j%4), column l % 32.
// For fp32 the 16-deep step is eight 2-deep MFMAs; MFMA i contracts element i of every
// lane, so both element types sum over the same 16 indices.
__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(f32x8 a, f32x8 b, f32x16 c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
    return c;
}

// 32x32 output tile, 64-deep contraction of e4m3 operands (gfx950's scaled f8f6f4 MFMA):
// c + 2^(sa - 127) 2^(sb - 127) sum_k a_k b_k.  Each lane holds 32 bytes of its row (A) or
// column (B); the instruction pairs byte p of lane l in A with byte p of lane l' = column +
// 32 (l / 32) in B, so any assignment of k to (l / 32, p) that both operands share gives the
// same product.  Measured on gfx950: subnormal inputs are kept, and the accumulator is added
// at fp32 precision (within 2 ulp).
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mma32_e4m3(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
// Four fp32 values -> four e4m3 bytes of x 2^shift (round to nearest even), clamped to the
// largest finite e4m3 value (448): the conversion itself gives NaN beyond it.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float scale) {
    auto cl = [&](float x) { return fminf(fmaxf(x * scale, -448.f), 448.f); };
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), v, true);
    return (uint32_t)v;
}
// Eight bf16 values -> eight e4m3 bytes (two dwords) of w / inv_scale (round to nearest
// even); |w / inv_scale| must stay within 448 (larger values give NaN).  The values go
// through fp32 (a shift or a mask per value): the conversion builtin that takes bf16 pairs
// directly was compiled here as if every pair were the first one.
__device__ __forceinline__ void e4m3x8_bf16(bf16x8 w, float inv_scale, int& d0, int& d1) {
    typedef short s2 __attribute__((ext_vector_type(2)));
    const u32x4 u = __builtin_bit_cast(u32x4, w);  // bf16 pairs, element 2i in the low half
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __builtin_bit_cast(float, u[i] << 16);
        f[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xffff0000u);
    }
    s2 o = {0, 0};
    o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, f[0], f[1], inv_scale, false);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, f[2], f[3], inv_scale, true);
    d0 = __builtin_bit_cast(int, o);
    s2 o2 = {0, 0};
    o2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o2, f[4], f[5], inv_scale, false);
    o2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o2, f[6], f[7], inv_scale, true);
    d1 = __builtin_bit_cast(int, o2);
}

// 16x16 output tile, 32-deep contraction.  Operand layout: lane l holds row/column (l % 16)
// and contraction indices 8*(l/16) .. 8*(l/16)+7.  Output: lane l, register j holds row
// 4*(l/16) + j, column l % 16.
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
    return c;
}

// Same-size unsigned vector of a chunk, for branch-free masking of loaded values.
template <typename T> struct ChunkBits;
template <> struct ChunkBits<bf16> { typedef uint32_t type __attribute__((ext_vector_type(4))); };
template <> struct ChunkBits<float> { typedef uint32_t type __attribute__((ext_vector_type(8))); };

// Load a chunk and zero it where `keep` is false, without a branch around the load (the
// address must be valid either way).
template <typename T>
__device__ __forceinline__ typename Chunk<T>::type load_masked(const T* p, bool keep) {
    typedef typename ChunkBits<T>::type U;
    U v = *(const U*)p;
    v &= (U)(keep ? 0xffffffffu : 0u);
    return __builtin_bit_cast(typename Chunk<T>::type, v);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename V> __device__ __forceinline__ V zero_vec() {
    V v;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(V) / sizeof(v[0])); ++i) v[i] = 0;
    return v;
}

// Sum / max over the 64 lanes of a wave, the same value in every lane (call with the whole
// wave active).  Inside each 16-lane row, four DPP lane exchanges (quad xor 1, quad xor 2,
// half-row mirror, row mirror) leave the row's result in all its lanes; these are VALU
// operand modifiers, with none of the LDS round trips of a shuffle.  The four row results
// are then read as scalars.
template <int CTRL> __device__ __forceinline__ float dpp_lane(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float read_lane(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
constexpr int DPP_QUAD_XOR1 = 0xB1, DPP_QUAD_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
constexpr int DPP_ROW_BCAST15 = 0x142;
// sum over the 16 lanes of each row, in every lane of the row
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_lane<DPP_QUAD_XOR1>(v);
    v += dpp_lane<DPP_QUAD_XOR2>(v);
    v += dpp_lane<DPP_HALF_MIRROR>(v);
    return v + dpp_lane<DPP_MIRROR>(v);
}
// sum over each 32-lane half, valid in lanes 16..31 (first half) and 48..63 (second half):
// the row sums of rows 0 and 2 are broadcast from their lane 15 into rows 1 and 3
__device__ __forceinline__ float half_sum_hi_rows(float v) {
    v = row_sum(v);
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), DPP_ROW_BCAST15,
                                                                     0xA, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum(v);
    return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_lane<DPP_QUAD_XOR1>(v));
    v = fmaxf(v, dpp_lane<DPP_QUAD_XOR2>(v));
    v = fmaxf(v, dpp_lane<DPP_HALF_MIRROR>(v));
    v = fmaxf(v, dpp_lane<DPP_MIRROR>(v));
    return fmaxf(fmaxf(read_lane(v, 0), read_lane(v, 16)), fmaxf(read_lane(v, 32), read_lane(v, 48)));
}

// Wait for every outstanding vector-memory load of this wave (including direct-to-LDS
// loads, which the compiler does not track).
#define NC_WAIT_VM_ALL() __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8))
// Wait until at most n (a constant, <= 63) vector-memory loads of this wave are outstanding
// (expcnt and lgkmcnt left at their maxima), in the gfx9 s_waitcnt encoding.
#define NC_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// Device-scope plain accesses (relaxed atomics at agent scope): the store is written
// through to the level where the dies' L2 caches are coherent and the load reads from it,
// so data passed between workgroups on different dies needs no cache-wide fence.
__device__ __forceinline__ void store_device(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_device(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory access this wave has issued is complete (device-scope stores
// have reached the coherent level); the compiler may move no memory access across it.
__device__ __forceinline__ void wait_stores_complete() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    NC_WAIT_VM_ALL();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup barrier for LDS data: this wave's LDS accesses complete, then s_barrier.  Unlike
// __syncthreads() it leaves the wave's outstanding global loads alone, so the direct-to-LDS
// loads of later pipeline stages stay in flight across it (their own waits are explicit).
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maximum
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Cache-policy operand of a direct-to-LDS load that reads at device scope (sc1: the bits the
// compiler gives a relaxed agent-scope atomic load), for data another workgroup stored with
// store_device.
#define NC_CPOL_DEVICE 16

// 16-byte device-scope accesses (sc1) through a buffer resource: base must be the same in
// every lane (it goes to scalar registers), the byte offset may differ per lane.  Word 3 of
// the resource selects the 32-bit data format for raw (untyped) access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void store_device4(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, NC_CPOL_DEVICE);
}
__device__ __forceinline__ f32x4 load_device4(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, NC_CPOL_DEVICE));
}

typedef __attribute__((address_space(1))) void gvoid;  // global memory, for direct-to-LDS loads
typedef __attribute__((address_space(3))) void lvoid;  // LDS

// Row scale of the parameter-free RMSNorm, r = 1/sqrt(sum_p ss[p * stride + m] / dim + eps),
// from `parts` partial sums of squares.  Wave-cooperative: lane q loads parts q, q+64, ...
// (all loads independent), then a butterfly sum; every lane returns r.  Must be called by
// all 64 lanes of the wave.
__device__ __forceinline__ float row_scale_wave(const float* ss, int parts, int stride, int m,
                                                int dim, float eps) {
    const int lane = threadIdx.x & 63;
    float s = 0.f;
    for (int q = lane; q < parts; q += 64) s += ss[(long long)q * stride + m];
    return 1.0f / sqrtf(wave_sum(s) / (float)dim + eps);
}

// Gate of a value embedding for value head j of a row (every lane of the wave calls it):
// 3 sigmoid(r xin[:ch] . gate[j]).
template <typename T>
__device__ __forceinline__ float value_embed_gate(const T* __restrict__ gate, int j, int ch,
                                                  const float* __restrict__ xin, float r, int lane) {
    float dot = lane < ch ? to_f32(gate[(long long)j * ch + lane]) * xin[lane] : 0.f;
    dot = wave_sum(dot) * r;
    return 3.0f / (1.0f + expf(-dot));
}

// 2^x on the hardware exponential unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh from the identity tanh(y) = sign(y) (1 - e^(-2|y|)) / (1 + e^(-2|y|)), with the
// exponential taken as 2^(-2|y| log2 e) and the quotient through the hardware reciprocal
// (1 ulp).  Relative error a few ulp away from 0; for |y| < 2^-4 the odd Taylor series
// y - y^3/3 + 2y^5/15 is taken instead (a select, no branch), which avoids the
// cancellation in 1 - e^(-2|y|).
__device__ __forceinline__ float tanh_f32(float y) {
    const float a = fabsf(y);
    const float y2 = y * y;
    const float series = y * (1.0f + y2 * (-1.0f / 3.0f + y2 * (2.0f / 15.0f)));
    const float e = fast_exp2(-2.8853900817779268f * a);  // e^(-2a)
    const float q = copysignf((1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e), y);
    return a < 0.0625f ? series : q;
}
// The logit softcap cap tanh(x / cap), with inv_cap = 1 / cap computed once by the caller.
__device__ __forceinline__ float softcap_f32(float x, float cap, float inv_cap) {
    return cap * tanh_f32(x * inv_cap);
}
