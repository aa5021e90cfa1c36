// bqd_kernels.hip -- gfx950 kernels and C ABI of libbqd.so (see include/bqd.h).
//
// Pages cited by title and section:
//   [Orin]   "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s"
//   [Ascend] "在香橙派上跑 Gemma4：vLLM 适配昇腾 310B 的内核开发实录"
//
// Design (CDNA4, wave64):
//   * Weights stream once from HBM as 16-byte chunks (32 INT4 codes).  A row
//     is split over L lanes (16/32/64); a "lane group" of L lanes owns r rows
//     and keeps r int32 accumulators per lane, so every activation chunk read
//     from LDS feeds r rows ([Orin] "o2-all 和 o4-all 为什么能加速").
//   * The INT8 activation is staged once per workgroup in LDS in a permuted
//     order: for each group of 8 codes, word A = codes {0,2,4,6}, word B =
//     codes {1,3,5,7}.  A packed weight word w then meets the activation
//     through two v_dot4_i32_i8:  (w << 4) & 0xF0F0F0F0 holds 16*q{0,2,4,6}
//     as signed bytes and w & 0xF0F0F0F0 holds 16*q{1,3,5,7}, so
//       sdot4(lo16(w), A) + sdot4(hi16(w), B) = 16 * sum_k q_k x_k
//     exactly, with three bit operations per word and no sign-extension
//     ([Orin] "DP4A 做了什么" splits the word into two int8x4 for two DP4A).
//     Each lane divides its partial by 16 (exact) before the cross-lane sum.
//   * Cross-lane sums use DPP row rotations inside each 16-lane row, then
//     lane shuffles across rows; the fp32 epilogue is fused.
//   * Activation quantisation ([Orin] derivation section) is either its own
//     kernel or folded into the GEMV prologue (each workgroup recomputes
//     max|x|, the fp32 scale and the RNE codes; correctly rounded fp32
//     division, so every workgroup's codes are identical).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "bqd.h"

namespace {

constexpr int kThreads = 256;          // 4 waves per workgroup
constexpr int kWave = 64;
constexpr int kLdsBytes = 65536;       // activation staging limit per workgroup
constexpr int kLdsMaxBytes = 160 * 1024;  // LDS of one CU (gfx950)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

// fp16 pair from a 32-bit word.  The word goes in by value: __builtin_bit_cast
// of an ext-vector element (v.y) was compiled as a read of element 0.
__device__ __forceinline__ h16x2 as_h16x2(uint32_t v)
{
    return __builtin_bit_cast(h16x2, v);
}

// Global address space.  Pointers read from memory (the pass descriptors) are
// generic; casting them keeps loads on the global path (global_load_*, which
// count only in vmcnt) instead of flat loads, which also count in lgkmcnt and
// so would be drained by every LDS wait.
#define BQD_GLOBAL __attribute__((address_space(1)))
#define BQD_LDS __attribute__((address_space(3)))
template <typename T>
__device__ __forceinline__ const BQD_GLOBAL T* gptr(const T* p)
{
    return (const BQD_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ BQD_GLOBAL T* gptr_mut(T* p)
{
    return (BQD_GLOBAL T*)p;
}

// Raw buffer resources.  A buffer load at an offset past the resource's
// size returns zeros and makes no memory access: loads that must not read
// can still be issued unconditionally, so the compiler counts them exactly.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kDeviceScope = 16;          // buffer-load cache-policy bit sc1
constexpr int kBufferPast = 0x7FFFFFF0;   // an offset past every resource this file makes
constexpr int kNonTemporal = 2;           // buffer-load cache-policy bit nt: streamed once, not kept in L2

__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes)
{
    // the address is wave-uniform: keep the resource in scalar registers
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0, bytes, kBufferWord3);
}

// ------------------------------------------------------------------------
// Bit helpers
// ------------------------------------------------------------------------

// Signed INT4 codes {0,2,4,6} of w, each times 16, as four signed bytes.
__device__ __forceinline__ int lo16(uint32_t w) { return (int)((w << 4) & 0xF0F0F0F0u); }
// Signed INT4 codes {1,3,5,7} of w, each times 16, as four signed bytes.
__device__ __forceinline__ int hi16(uint32_t w) { return (int)(w & 0xF0F0F0F0u); }

// Activation bytes b0..b7 (lo = b0..b3, hi = b4..b7) -> A = [b0 b2 b4 b6].
__device__ __forceinline__ uint32_t perm_even(uint32_t lo, uint32_t hi)
{
    return (lo & 0xFFu) | ((lo >> 8) & 0xFF00u) | ((hi & 0xFFu) << 16) | ((hi << 8) & 0xFF000000u);
}
// -> B = [b1 b3 b5 b7].
__device__ __forceinline__ uint32_t perm_odd(uint32_t lo, uint32_t hi)
{
    return ((lo >> 8) & 0xFFu) | ((lo >> 16) & 0xFF00u) | ((hi << 8) & 0xFF0000u) | (hi & 0xFF000000u);
}

// 16 x (sum over the 32 codes of one chunk of w times the staged activation).
// xa = [A0 B0 A1 B1], xb = [A2 B2 A3 B3] of the chunk's four 8-code groups.
__device__ __forceinline__ int dot_chunk16(u32x4 w, u32x4 xa, u32x4 xb, int acc)
{
    acc = __builtin_amdgcn_sdot4(lo16(w.x), (int)xa.x, acc, false);
    acc = __builtin_amdgcn_sdot4(hi16(w.x), (int)xa.y, acc, false);
    acc = __builtin_amdgcn_sdot4(lo16(w.y), (int)xa.z, acc, false);
    acc = __builtin_amdgcn_sdot4(hi16(w.y), (int)xa.w, acc, false);
    acc = __builtin_amdgcn_sdot4(lo16(w.z), (int)xb.x, acc, false);
    acc = __builtin_amdgcn_sdot4(hi16(w.z), (int)xb.y, acc, false);
    acc = __builtin_amdgcn_sdot4(lo16(w.w), (int)xb.z, acc, false);
    acc = __builtin_amdgcn_sdot4(hi16(w.w), (int)xb.w, acc, false);
    return acc;
}

// ------------------------------------------------------------------------
// Cross-lane reductions
// ------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over L consecutive lanes (L = 16, 32, 64); every lane gets the sum.
// Inside a 16-lane DPP row: rotations by 8, 4, 2, 1 (row_ror); across rows:
// lane shuffles.  Integer sums are exact, so the order is immaterial.
template <int L>
__device__ __forceinline__ int sum_lanes(int v)
{
    v += dpp_i<0x128>(v);
    v += dpp_i<0x124>(v);
    v += dpp_i<0x122>(v);
    v += dpp_i<0x121>(v);
    if (L >= 32) v += __shfl_xor(v, 16);
    if (L >= 64) v += __shfl_xor(v, 32);
    return v;
}
template <int L>
__device__ __forceinline__ float sum_lanes_f(float v)
{
    v += dpp_f<0x128>(v);
    v += dpp_f<0x124>(v);
    v += dpp_f<0x122>(v);
    v += dpp_f<0x121>(v);
    if (L >= 32) v += __shfl_xor(v, 16);
    if (L >= 64) v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1)
        v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

// The same maximum without LDS traffic (lane shuffles are LDS permutes):
// DPP row rotations 8, 4, 2, 1 inside each row of 16 lanes, then the four
// row maxima read as scalars.  Needs every lane of the wave active.
__device__ __forceinline__ float wave_max_dpp(float v)
{
    v = fmaxf(v, dpp_f<0x128>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x122>(v));
    v = fmaxf(v, dpp_f<0x121>(v));
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Max over the workgroup (every thread gets it).  red: 4 floats of LDS.
__device__ __forceinline__ float block_max(float v, float* red)
{
    v = wave_max(v);
    if ((threadIdx.x & (kWave - 1)) == 0)
        red[threadIdx.x / kWave] = v;
    __syncthreads();
    float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return m;
}

// ------------------------------------------------------------------------
// Activation input: 8 consecutive values of x as fp32 (fp16 widens exactly)
// ------------------------------------------------------------------------
enum XIn { X_Q8 = 0, X_F32 = 1, X_F16 = 2, X_RMS = 3 };

// Operands of the RMSNorm activation (X_RMS): x = RMSNorm(h + delta) * gamma.
struct RmsIn {
    const float* h;      // residual stream [K]
    const float* delta;  // added to h first, or NULL
    const float* gamma;  // [K]
    float* h_out;        // h + delta, written by workgroup 0, or NULL
    float eps;
};

template <int XIN>
__device__ __forceinline__ void load8(const void* x, int g, float v[8])
{
    if constexpr (XIN == X_F32) {
        const BQD_GLOBAL f32x4* p = gptr(reinterpret_cast<const f32x4*>(x)) + 2 * g;
        f32x4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        u32x4 h = gptr(reinterpret_cast<const u32x4*>(x))[g];
        uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hw[k] & 0xFFFFu));
            v[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hw[k] >> 16));
        }
    }
}

// Activation scale s = max|x| / 127 (correctly rounded fp32 division) with
// what the code computation needs.  [Orin] derivation section.
struct ActScale {
    float s;    // s^x
    float inv;  // fl(1 / s), valid when fast
    bool fast;  // s is a normal number: the reciprocal route below applies
};

__device__ __forceinline__ ActScale act_scale(float amax)
{
    ActScale a;
    a.s = amax / 127.0f;
    a.fast = a.s >= 0x1p-126f;
    a.inv = a.fast ? 1.0f / a.s : 0.0f;
    return a;
}

// clip(round_half_even(fl(v / s)), -127, 127), bit-identical to the correctly
// rounded fp32 division followed by RNE; 0 when s == 0.
// Route: r = v * fl(1/s) is within 2^-16 of v/s (|v/s| <= 127 * (1 + 2^-23),
// two roundings of relative size 2^-24 each), and fl(v/s) within 2^-17 of
// v/s, so whenever r is more than 2^-15 away from a half-integer, rint(r)
// and rint(fl(v/s)) agree.  Only closer to a tie is the exact quotient taken.
// r - rint(r) is exact (Sterbenz), so the test itself does not round.
__device__ __forceinline__ uint32_t act_code(float v, const ActScale& a)
{
    float m;
    if (a.fast) {
        const float r = v * a.inv;
        m = rintf(r);
        if (fabsf(r - m) > 0.5f - 0x1p-15f)
            m = rintf(v / a.s);
    } else {
        if (a.s == 0.0f)
            return 0u;
        m = rintf(v / a.s);
    }
    m = fminf(fmaxf(m, -127.0f), 127.0f);
    return (uint32_t)((int)m) & 0xFFu;
}

// Quantise 8 values into bytes lo = codes 0..3, hi = codes 4..7.
__device__ __forceinline__ void quant8(const float v[8], const ActScale& a, uint32_t& lo, uint32_t& hi)
{
    lo = act_code(v[0], a) | (act_code(v[1], a) << 8) | (act_code(v[2], a) << 16) | (act_code(v[3], a) << 24);
    hi = act_code(v[4], a) | (act_code(v[5], a) << 8) | (act_code(v[6], a) << 16) | (act_code(v[7], a) << 24);
}

// Codes of 8 values, bytes lo = codes 0..3, hi = codes 4..7, bit-identical to
// act_code: the reciprocal route for all 8, then one (rare) branch to the
// exact quotient if any of them lies within 2^-15 of a rounding tie.
__device__ __forceinline__ void quant8_fast(const float v[8], const ActScale& a, uint32_t& lo, uint32_t& hi)
{
    float m[8];
    bool near = !a.fast;
    if (a.fast) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float r = v[e] * a.inv;
            m[e] = rintf(r);
            near |= fabsf(r - m[e]) > 0.5f - 0x1p-15f;
        }
    }
    if (near) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            m[e] = a.s == 0.0f ? 0.0f : rintf(v[e] / a.s);
    }
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        b[e] = (uint32_t)((int)__builtin_amdgcn_fmed3f(m[e], -127.0f, 127.0f)) & 0xFFu;
    lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
}


// Four values, the same rule: the exact quotient for all four whenever one
// of them lies near a rounding tie.
__device__ __forceinline__ uint32_t quant4_fast(f32x4 v, const ActScale& a)
{
    const float x[4] = {v.x, v.y, v.z, v.w};
    float m[4];
    bool near = !a.fast;
    if (a.fast) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float r = x[e] * a.inv;
            m[e] = rintf(r);
            near |= fabsf(r - m[e]) > 0.5f - 0x1p-15f;
        }
    }
    if (near) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            m[e] = a.s == 0.0f ? 0.0f : rintf(x[e] / a.s);
    }
    uint32_t q = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        q |= ((uint32_t)((int)__builtin_amdgcn_fmed3f(m[e], -127.0f, 127.0f)) & 0xFFu) << (8 * e);
    return q;
}

// Stage G8 = K/8 groups of INT8 codes into LDS (permuted), from int8 memory.
__device__ __forceinline__ void stage_q8(u32x2* xs, const int8_t* qx, int G8)
{
    const u32x2* q = reinterpret_cast<const u32x2*>(qx);
    for (int g = threadIdx.x; g < G8; g += kThreads) {
        u32x2 v = q[g];
        xs[g] = u32x2{perm_even(v.x, v.y), perm_odd(v.x, v.y)};
    }
}

// Codes a producer already wrote, for K <= 16 * kThreads * kQ8Pre: every
// 16-byte load (two 8-value groups) issued at once, before the kernel's
// first weight step, and waited for once.  A CU serves its loads in order,
// so codes loaded after that step (stage_q8's loop, one round trip per
// iteration) wait for its weights first.
constexpr int kQ8Pre = 5;
__device__ __forceinline__ void preload_q8(const void* qx, int G16, u32x4 (&v)[kQ8Pre])
{
    const __amdgpu_buffer_rsrc_t r = uniform_rsrc(qx, 16 * G16);
#pragma unroll
    for (int k = 0; k < kQ8Pre; ++k) {
        const int g = (int)threadIdx.x + k * kThreads;
        v[k] = u32x4{0u, 0u, 0u, 0u};
        if (k * kThreads < G16)  // uniform: only the rounds the activation needs
            v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, g < G16 ? 16 * g : kBufferPast,
                                                                                   0, 0));
    }
}

__device__ __forceinline__ void write_q8(u32x2* xs, const u32x4 (&v)[kQ8Pre], int G16)
{
#pragma unroll
    for (int k = 0; k < kQ8Pre; ++k) {
        const int g = (int)threadIdx.x + k * kThreads;
        if (g < G16) {
            xs[2 * g] = u32x2{perm_even(v[k].x, v[k].y), perm_odd(v[k].x, v[k].y)};
            xs[2 * g + 1] = u32x2{perm_even(v[k].z, v[k].w), perm_odd(v[k].z, v[k].w)};
        }
    }
}

// Quantise x (fp32/fp16, [K]) in the workgroup and stage the codes into LDS.
// Returns s^x.  Workgroup 0 optionally writes the codes and scale out.
// Up to K = 8192 each thread keeps its (at most 4) 8-value groups in
// registers: every load is issued before the first use (one memory round
// trip), and the codes come from the registers.  Longer activations take
// two passes over x (the second from cache), 4 groups per thread at a time.
// A short activation (G8 <= 4 * kThreads groups of 8) in registers: the
// loads alone, so that a kernel can issue them ahead of its weight loads
// (a CU serves its loads in order, and the activation is on the critical
// path: its maximum and codes come before the first dot product).
template <int XIN>
__device__ __forceinline__ void preload_x(const void* x, int G8, float (&v)[4][8])
{
#pragma unroll
    for (int k = 0; k < 4; ++k)
        load8<XIN>(x, min((int)threadIdx.x + k * kThreads, G8 - 1), v[k]);
}

// Codes and scale of a short activation already in registers (preload_x).
__device__ float quant_from_regs(u32x2* xs, const float (&v)[4][8], int G8, float* red, int8_t* qx_out,
                                 float* sx_out)
{
    const bool out = (qx_out != nullptr) && blockIdx.x == 0;
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            m = fmaxf(m, fabsf(v[k][e]));  // clamped groups repeat a real one
    const ActScale a = act_scale(block_max(m, red));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int g = threadIdx.x + k * kThreads;
        if (g < G8) {
            uint32_t lo, hi;
            quant8_fast(v[k], a, lo, hi);
            xs[g] = u32x2{perm_even(lo, hi), perm_odd(lo, hi)};
            if (out)
                reinterpret_cast<u32x2*>(qx_out)[g] = u32x2{lo, hi};
        }
    }
    if (sx_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *sx_out = a.s;
    return a.s;
}

template <int XIN>
__device__ float stage_quant(u32x2* xs, const void* x, int G8, float* red, int8_t* qx_out,
                             float* sx_out)
{
    if (G8 <= 4 * kThreads) {
        float v[4][8];
        preload_x<XIN>(x, G8, v);
        return quant_from_regs(xs, v, G8, red, qx_out, sx_out);
    }
    const bool out = (qx_out != nullptr) && blockIdx.x == 0;
    // batches of 4 groups per thread, the batch's loads issued together
    float amax = 0.0f;
    for (int g0 = threadIdx.x; g0 < G8; g0 += 4 * kThreads) {
        float v[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            load8<XIN>(x, min(g0 + k * kThreads, G8 - 1), v[k]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                amax = fmaxf(amax, fabsf(v[k][e]));  // clamped groups repeat a real one
    }
    amax = block_max(amax, red);
    const ActScale a = act_scale(amax);
    const float s = a.s;
    for (int g0 = threadIdx.x; g0 < G8; g0 += 4 * kThreads) {
        float v[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            load8<XIN>(x, min(g0 + k * kThreads, G8 - 1), v[k]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int g = g0 + k * kThreads;
            if (g < G8) {
                uint32_t lo, hi;
                quant8_fast(v[k], a, lo, hi);
                xs[g] = u32x2{perm_even(lo, hi), perm_odd(lo, hi)};
                if (out)
                    reinterpret_cast<u32x2*>(qx_out)[g] = u32x2{lo, hi};
            }
        }
    }
    if (sx_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *sx_out = s;
    return s;
}

// ------------------------------------------------------------------------
// Load-time weight quantisation
// ------------------------------------------------------------------------

// One wave per row: s = max|W_row| / 7, codes clip(rne(W/s), -8, 7), packed.
__global__ __launch_bounds__(kThreads) void k_quantize_weights_int4_rowwise(
    const float* __restrict__ W, int N, int K, uint32_t* __restrict__ wq, float* __restrict__ sw)
{
    const int row = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    if (row >= N)
        return;  // whole wave exits together: no cross-wave sync below
    const float* w = W + (size_t)row * K;
    const int G8 = K / 8;
    float amax = 0.0f;
    for (int g = lane; g < G8; g += kWave) {
        float v[8];
        load8<X_F32>(w, g, v);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            amax = fmaxf(amax, fabsf(v[k]));
    }
    amax = wave_max(amax);
    const float s = amax / 7.0f;
    if (lane == 0)
        sw[row] = s;
    uint32_t* out = wq + (size_t)row * G8;
    for (int g = lane; g < G8; g += kWave) {
        float v[8];
        load8<X_F32>(w, g, v);
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            int q = 0;
            if (s != 0.0f)
                q = (int)fminf(fmaxf(rintf(v[k] / s), -8.0f), 7.0f);
            word |= ((uint32_t)q & 0xFu) << (4 * k);
        }
        out[g] = word;
    }
}

// One thread per block of 32 weights: fp16 scale fp16(max|W_block| / D),
// codes against the stored fp16 value.  INT4 (packed) or INT8 output.
template <bool INT8>
__global__ __launch_bounds__(kThreads) void k_quantize_weights_group32(
    const float* __restrict__ W, int N, int K, void* __restrict__ out, uint16_t* __restrict__ s16)
{
    const int G = K / 32;
    const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= (long long)N * G)
        return;
    const int row = (int)(idx / G), g = (int)(idx % G);
    const float* w = W + (size_t)row * K + (size_t)g * 32;
    float v[32];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        load8<X_F32>(w, t, v + 8 * t);
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k)
        amax = fmaxf(amax, fabsf(v[k]));
    const float D = INT8 ? 31.0f : 7.0f;
    const float lo = INT8 ? -32.0f : -8.0f, hi = INT8 ? 31.0f : 7.0f;
    const _Float16 h = (_Float16)(amax / D);
    s16[(size_t)row * G + g] = __builtin_bit_cast(uint16_t, h);
    const float s = (float)h;
    int q[32];
#pragma unroll
    for (int k = 0; k < 32; ++k)
        q[k] = (s != 0.0f) ? (int)fminf(fmaxf(rintf(v[k] / s), lo), hi) : 0;
    if constexpr (INT8) {
        u32x4* o = reinterpret_cast<u32x4*>(reinterpret_cast<int8_t*>(out) + (size_t)row * K + (size_t)g * 32);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            uint32_t wv[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int b = 16 * t + 4 * d;
                wv[d] = ((uint32_t)q[b] & 0xFFu) | (((uint32_t)q[b + 1] & 0xFFu) << 8) |
                        (((uint32_t)q[b + 2] & 0xFFu) << 16) | (((uint32_t)q[b + 3] & 0xFFu) << 24);
            }
            o[t] = u32x4{wv[0], wv[1], wv[2], wv[3]};
        }
    } else {
        uint32_t wv[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t word = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                word |= ((uint32_t)q[8 * d + k] & 0xFu) << (4 * k);
            wv[d] = word;
        }
        reinterpret_cast<u32x4*>(reinterpret_cast<uint32_t*>(out) + (size_t)row * (K / 8))[g] =
            u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
}

// ------------------------------------------------------------------------
// Activation quantisation: one workgroup per token row.
// ------------------------------------------------------------------------
template <int XIN>
__global__ __launch_bounds__(kThreads) void k_quantize_act(const void* __restrict__ x, int K,
                                                           int8_t* __restrict__ qx, float* __restrict__ sx)
{
    __shared__ float red[4];
    const int m = blockIdx.x;
    const int G8 = K / 8;
    const size_t esz = XIN == X_F32 ? 4 : 2;
    const void* xr = reinterpret_cast<const char*>(x) + (size_t)m * K * esz;
    float amax = 0.0f;
    for (int g = threadIdx.x; g < G8; g += kThreads) {
        float v[8];
        load8<XIN>(xr, g, v);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            amax = fmaxf(amax, fabsf(v[k]));
    }
    amax = block_max(amax, red);
    const ActScale a = act_scale(amax);
    u32x2* q = reinterpret_cast<u32x2*>(qx + (size_t)m * K);
    for (int g = threadIdx.x; g < G8; g += kThreads) {
        float v[8];
        load8<XIN>(xr, g, v);
        uint32_t lo, hi;
        quant8(v, a, lo, hi);
        q[g] = u32x2{lo, hi};
    }
    if (threadIdx.x == 0)
        sx[m] = a.s;
}

// ------------------------------------------------------------------------
// Producers of a linear's activation fused with its quantisation ([Orin]
// "后续还能继续优化什么", items 1 and 2: the residual add, RMSNorm and SwiGLU
// still end in their own kernels, and the quantisation could be folded into
// the operator before it).  Textbook forms: RMSNorm y = h / sqrt(mean h^2 +
// eps) * gamma, SwiGLU h = silu(g) * u.  Every value that decides a code is
// an fp32 result of a fixed sequence of IEEE operations (the sum of squares
// aside, which is accumulated in fp64, where each square is exact), so the
// codes do not depend on the order of the reductions.
//   RMSNorm: one workgroup of 1024 threads per token holds the token in
//   registers (ITEMS 16-byte items per thread, every load issued before the
//   first use): one memory round trip, a sum and a max over the workgroup,
//   then the codes.
//   SwiGLU: the elementwise part is spread over many workgroups (it costs
//   ~30 VALU operations per value); a second kernel then takes the row's max
//   in each of a few workgroups and quantises one slice per workgroup.
// ------------------------------------------------------------------------
constexpr int kProdThreads = 1024;
constexpr int kProdWaves = kProdThreads / kWave;
constexpr int kProdMaxK = BQD_MAX_PROD_K;
static_assert(kProdMaxK <= 8 * 4 * kProdThreads, "at most 8 items of 4 values per thread");

__device__ __forceinline__ float prod_block_max(float v, float* red)
{
    v = wave_max(v);
    if ((threadIdx.x & (kWave - 1)) == 0)
        red[threadIdx.x / kWave] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kProdWaves; ++w)
        m = fmaxf(m, red[w]);
    __syncthreads();
    return m;
}

// fp64 sum over the workgroup, the same value in every thread.
__device__ __forceinline__ double prod_block_sum(double v, double* red)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1)
        v += __shfl_xor(v, m);
    if ((threadIdx.x & (kWave - 1)) == 0)
        red[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kProdWaves; ++w)
        t += red[w];
    __syncthreads();
    return t;
}

// e^x in fp32 (W. J. Cody and W. Waite, "Software Manual for the Elementary
// Functions", 1980: x = n ln2 + r, n = round(x / ln2), ln2 split into a
// 9-significant-bit head, exact against any |n| < 2^15, and a tail), then
// e^r by its degree-7 Taylor polynomial in Horner form (|r| <= ln2 / 2:
// truncation below 6e-9 relative) and a final scaling by 2^n.  Each step is
// one IEEE operation (fmaf rounds once), so the result is reproducible bit
// for bit; the argument is clamped to [-104, 89], beyond which the result is
// already 0 or +Inf.
__device__ __forceinline__ float exp_cw(float x)
{
    x = fminf(fmaxf(x, -104.0f), 89.0f);
    const float n = rintf(x * 1.44269504088896341f);
    float r = __builtin_fmaf(-n, 0.693359375f, x);
    r = __builtin_fmaf(-n, -2.12194440054690583e-4f, r);
    float p = (float)(1.0 / 5040.0);
    p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return (g / (1.0f + exp_cw(-g))) * u;  // correctly rounded division
}

__device__ __forceinline__ float max_abs4(f32x4 v)
{
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// h1 = h + delta; r = fp32(1 / sqrt(sum h1^2 / K + eps)) (fp64 sum, root
// and division); y = (h1 * r) * gamma; then the codes.  Token blockIdx.x;
// thread t holds items t, t + 1024, ... (ITEMS of them, K/4 <= 1024 ITEMS);
// items past the row are loaded clamped and never used.  Outputs optional.
template <int ITEMS>
__global__ __launch_bounds__(kProdThreads) void k_add_rmsnorm_quant(
    const float* __restrict__ h, const float* __restrict__ delta, const float* __restrict__ gamma,
    float eps, int K, float* h_out, float* y_out, int8_t* __restrict__ qx, float* __restrict__ sx)
{
    __shared__ double dred[kProdWaves];
    __shared__ float fred[kProdWaves];
    const int K4 = K / 4;
    const size_t base = (size_t)blockIdx.x * K4;
    const f32x4* hp = reinterpret_cast<const f32x4*>(h) + base;
    const f32x4* gp = reinterpret_cast<const f32x4*>(gamma);
    f32x4 a[ITEMS], g[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const int i = min((int)threadIdx.x + k * kProdThreads, K4 - 1);
        a[k] = hp[i];
        g[k] = gp[i];
    }
    if (delta) {
        const f32x4* dp = reinterpret_cast<const f32x4*>(delta) + base;
        f32x4 d[ITEMS];
#pragma unroll
        for (int k = 0; k < ITEMS; ++k)
            d[k] = dp[min((int)threadIdx.x + k * kProdThreads, K4 - 1)];
#pragma unroll
        for (int k = 0; k < ITEMS; ++k)
            a[k] = f32x4{a[k].x + d[k].x, a[k].y + d[k].y, a[k].z + d[k].z, a[k].w + d[k].w};
    }
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const int i = threadIdx.x + k * kProdThreads;
        if (i < K4) {
            if (h_out)
                reinterpret_cast<f32x4*>(h_out)[base + i] = a[k];
            ss += (double)a[k].x * (double)a[k].x;
            ss += (double)a[k].y * (double)a[k].y;
            ss += (double)a[k].z * (double)a[k].z;
            ss += (double)a[k].w * (double)a[k].w;
        }
    }
    ss = prod_block_sum(ss, dred);
    const double v = ss / (double)K + (double)eps;
    const float r = v > 0.0 ? (float)(1.0 / sqrt(v)) : 0.0f;
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        a[k] = f32x4{(a[k].x * r) * g[k].x, (a[k].y * r) * g[k].y, (a[k].z * r) * g[k].z, (a[k].w * r) * g[k].w};
        amax = fmaxf(amax, max_abs4(a[k]));  // clamped items repeat a real one
    }
    amax = prod_block_max(amax, fred);
    const ActScale as = act_scale(amax);
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const int i = threadIdx.x + k * kProdThreads;
        if (i < K4) {
            if (y_out)
                reinterpret_cast<f32x4*>(y_out)[base + i] = a[k];
            if (qx)
                reinterpret_cast<uint32_t*>(qx)[base + i] = quant4_fast(a[k], as);
        }
    }
    if (sx && threadIdx.x == 0)
        sx[blockIdx.x] = as.s;
}

// h = silu(g) * u over a token's fused gate/up output [g | u] (2I fp32):
// thread (blockIdx.x, threadIdx.x) of token blockIdx.y computes one 16-byte
// item (4 values) into h.
__global__ __launch_bounds__(kThreads) void k_swiglu(const float* __restrict__ gu, int I,
                                                     float* __restrict__ h)
{
    const int I4 = I / 4;
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= I4)
        return;
    const f32x4* gp = reinterpret_cast<const f32x4*>(gu) + (size_t)blockIdx.y * 2 * I4;
    const f32x4 g = gp[i], u = gp[I4 + i];
    reinterpret_cast<f32x4*>(h)[(size_t)blockIdx.y * I4 + i] =
        f32x4{silu_mul(g.x, u.x), silu_mul(g.y, u.y), silu_mul(g.z, u.z), silu_mul(g.w, u.w)};
}

// Per-token quantisation of fp32 rows [M, K], the row spread over
// gridDim.x workgroups: each takes the max over the whole row (thread t holds
// items t, t + 1024, ..., ITEMS of them, loads issued before the first use)
// and writes the codes of its own slice of 1024 items; workgroup 0 writes s^x.
template <int ITEMS>
__global__ __launch_bounds__(kProdThreads) void k_quantize_rows(const float* __restrict__ x, int K,
                                                                int8_t* __restrict__ qx, float* __restrict__ sx)
{
    __shared__ float fred[kProdWaves];
    const int K4 = K / 4;
    const f32x4* xr = reinterpret_cast<const f32x4*>(x) + (size_t)blockIdx.y * K4;
    f32x4 v[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k)
        v[k] = xr[min((int)threadIdx.x + k * kProdThreads, K4 - 1)];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k)
        amax = fmaxf(amax, max_abs4(v[k]));  // clamped items repeat a real one
    amax = prod_block_max(amax, fred);
    const ActScale as = act_scale(amax);
    const int i = blockIdx.x * kProdThreads + threadIdx.x;
    if (i < K4) {
        f32x4 t = v[0];
#pragma unroll
        for (int k = 1; k < ITEMS; ++k)
            if (k == (int)blockIdx.x)
                t = v[k];
        reinterpret_cast<uint32_t*>(qx)[(size_t)blockIdx.y * K4 + i] = quant4_fast(t, as);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0)
        sx[blockIdx.y] = as.s;
}

// ------------------------------------------------------------------------
// W4A8 GEMV, per-row scales.
//   R: rows per lane group; L: lanes per row; U: chunk iterations per
//   pipeline step; XIN: activation input form.
//   Workgroup tile = (256/L) lane groups x R rows; workgroups walk tiles in a
//   grid-stride loop.  Each lane streams its rows in steps of U chunks
//   (R*U 16-byte loads); step s+1 (possibly of the next tile) is loaded while
//   step s is computed, and the first step is issued before the activation
//   prologue so that its latency overlaps the staging.  Rows past N read
//   row N-1 (in bounds) and are never written.  Weights are read once, with
//   non-temporal loads (the single [3584, 3584] GEMV 4.41 -> 4.09 us, the
//   per-linear 28-layer stream 1.222 -> 1.177 ms).
// ------------------------------------------------------------------------
template <int R, int L, int U>
__device__ __forceinline__ void load_step(u32x4 (&buf)[U][R], const u32x4* __restrict__ wq, int N,
                                          int C, int row0, int step, int lane)
{
    const u32x4* wrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        wrow[r] = wq + (size_t)min(row0 + r, N - 1) * C;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (step * U + u) * L + lane;
        const bool ok = c < C;
#pragma unroll
        for (int r = 0; r < R; ++r)
            buf[u][r] = ok ? __builtin_nontemporal_load(wrow[r] + c) : u32x4{0u, 0u, 0u, 0u};
    }
}

template <int R, int L, int U>
__device__ __forceinline__ void load_scales(uint16_t (&buf)[U][R], const uint16_t* __restrict__ s16,
                                            int N, int C, int row0, int step, int lane)
{
    const uint16_t* srow[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        srow[r] = s16 + (size_t)min(row0 + r, N - 1) * C;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (step * U + u) * L + lane;
        const bool ok = c < C;
#pragma unroll
        for (int r = 0; r < R; ++r)
            buf[u][r] = ok ? srow[r][c] : (uint16_t)0;
    }
}

// Residual add + RMSNorm + quantisation in the GEMV prologue (K <= 8192):
// each thread holds its (at most 4) groups of h + delta and of gamma in
// registers, all loaded before the first use; the binary64 sum of squares
// over the workgroup gives r = fp32(1 / sqrt(ss / K + eps)), then y =
// (a * r) * gamma and the codes -- the same fp32 operations as
// add_rmsnorm_quant, so the same codes.  Workgroup 0 writes h + delta (and
// optionally the codes and scale).
__device__ float stage_rms_quant(u32x2* xs, const RmsIn& p, int G8, float* red, int8_t* qx_out, float* sx_out)
{
    __shared__ double dred[kThreads / kWave];
    float a[4][8], gm[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int g = min((int)threadIdx.x + k * kThreads, G8 - 1);
        load8<X_F32>(p.h, g, a[k]);
        load8<X_F32>(p.gamma, g, gm[k]);
    }
    if (p.delta) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float d[8];
            load8<X_F32>(p.delta, min((int)threadIdx.x + k * kThreads, G8 - 1), d);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a[k][e] = a[k][e] + d[e];
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if ((int)threadIdx.x + k * kThreads < G8)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ss += (double)a[k][e] * (double)a[k][e];
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1)
        ss += __shfl_xor(ss, m);
    if ((threadIdx.x & (kWave - 1)) == 0)
        dred[threadIdx.x / kWave] = ss;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w)
        t += dred[w];
    const double v = t / (double)(8 * G8) + (double)p.eps;
    const float r = v > 0.0 ? (float)(1.0 / sqrt(v)) : 0.0f;
    const bool w0 = blockIdx.x == 0;
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int g = threadIdx.x + k * kThreads;
        if (w0 && p.h_out && g < G8) {
            f32x4* o = reinterpret_cast<f32x4*>(p.h_out) + 2 * g;
            o[0] = f32x4{a[k][0], a[k][1], a[k][2], a[k][3]};
            o[1] = f32x4{a[k][4], a[k][5], a[k][6], a[k][7]};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[k][e] = (a[k][e] * r) * gm[k][e];
            m = fmaxf(m, fabsf(a[k][e]));  // clamped groups repeat a real one
        }
    }
    const ActScale as = act_scale(block_max(m, red));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int g = threadIdx.x + k * kThreads;
        if (g < G8) {
            uint32_t lo, hi;
            quant8_fast(a[k], as, lo, hi);
            xs[g] = u32x2{perm_even(lo, hi), perm_odd(lo, hi)};
            if (w0 && qx_out)
                reinterpret_cast<u32x2*>(qx_out)[g] = u32x2{lo, hi};
        }
    }
    if (w0 && sx_out && threadIdx.x == 0)
        *sx_out = as.s;
    return as.s;
}

template <int XIN>
__device__ __forceinline__ float stage_activation(u32x4* xs, const void* xin, const float* sx_in, int C,
                                                  float* red, int8_t* qx_out, float* sx_out,
                                                  const RmsIn& rms = RmsIn{})
{
    if constexpr (XIN == X_Q8) {
        stage_q8(reinterpret_cast<u32x2*>(xs), reinterpret_cast<const int8_t*>(xin), 4 * C);
        return *sx_in;
    } else if constexpr (XIN == X_RMS) {
        return stage_rms_quant(reinterpret_cast<u32x2*>(xs), rms, 4 * C, red, qx_out, sx_out);
    } else {
        return stage_quant<XIN>(reinterpret_cast<u32x2*>(xs), xin, 4 * C, red, qx_out, sx_out);
    }
}

template <int R, int L, int U, int XIN>
__global__ __launch_bounds__(kThreads) void k_gemv_w4a8(
    const u32x4* __restrict__ wq, const float* __restrict__ sw, const float* __restrict__ bias,
    const void* __restrict__ xin, const float* __restrict__ sx_in, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int8_t* __restrict__ qx_out, float* __restrict__ sx_out, int N,
    int C, RmsIn rms)
{
    extern __shared__ u32x4 xs[];  // 2*C chunks' activation = K bytes
    __shared__ float red[4];
    constexpr int GROUPS = kThreads / L;
    constexpr int ROWS = GROUPS * R;
    const int lane = threadIdx.x % L;
    const int grp = threadIdx.x / L;
    const int tiles = (N + ROWS - 1) / ROWS;
    const int iters = (C + L - 1) / L;
    const int steps = (iters + U - 1) / U;

    int tile = blockIdx.x;
    u32x4 cur[U][R];
    float sx;
    bool staged = false;
    if constexpr (XIN == X_F32 || XIN == X_F16) {
        if (C <= kThreads) {
            // the activation's loads first, then the first weight step's
            float v[4][8];
            preload_x<XIN>(xin, 4 * C, v);
            load_step<R, L, U>(cur, wq, N, C, tile * ROWS + grp * R, 0, lane);
            sx = quant_from_regs(reinterpret_cast<u32x2*>(xs), v, 4 * C, red, qx_out, sx_out);
            staged = true;
        }
    } else if constexpr (XIN == X_Q8) {
        if (2 * C <= kQ8Pre * kThreads) {
            u32x4 v[kQ8Pre];
            preload_q8(xin, 2 * C, v);
            load_step<R, L, U>(cur, wq, N, C, tile * ROWS + grp * R, 0, lane);
            write_q8(reinterpret_cast<u32x2*>(xs), v, 2 * C);
            sx = *sx_in;
            staged = true;
        }
    }
    if (!staged) {
        load_step<R, L, U>(cur, wq, N, C, tile * ROWS + grp * R, 0, lane);
        sx = stage_activation<XIN>(xs, xin, sx_in, C, red, qx_out, sx_out, rms);
    }
    __syncthreads();

    for (; tile < tiles; tile += gridDim.x) {
        const int row0 = tile * ROWS + grp * R;
        int acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = 0;
        for (int st = 0; st < steps; ++st) {
            u32x4 nxt[U][R];
            int ntile = tile, nst = st + 1;
            if (nst == steps) {
                ntile += gridDim.x;
                nst = 0;
            }
            const bool more = ntile < tiles;
            if (more)
                load_step<R, L, U>(nxt, wq, N, C, ntile * ROWS + grp * R, nst, lane);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (st * U + u < iters) {  // uniform across the wave
                    const int c = min((st * U + u) * L + lane, C - 1);
                    const u32x4 xa = xs[2 * c], xb = xs[2 * c + 1];
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r] = dot_chunk16(cur[u][r], xa, xb, acc[r]);
                }
            }
            if (more) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        cur[u][r] = nxt[u][r];
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = sum_lanes<L>(acc[r] >> 4);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r;
            if (lane == r && row < N) {
                if (acc_out)
                    acc_out[row] = acc[r];
                const float t = sw[row] * sx;
                y[row] = fmaf(t, (float)acc[r], bias ? bias[row] : 0.0f);
            }
        }
    }
}

// ------------------------------------------------------------------------
// One fused linear in wide workgroups: TH threads, one wave per output
// row (TH / 64 rows per workgroup), U 16-byte chunks per lane (K <= 64 * 32
// * U, at most 24576).  Every thread first loads its 8-value groups of x
// (fp32 / fp16; NG of them) or its 16-byte pieces of codes (NQ), then its
// wave's row chunks, so the activation's loads go out ahead of the weights
// in the CU's in-order queue; the whole workgroup finds max|x| and writes
// the codes in one round, and every weight of the workgroup is in flight
// while it does.  Same codes and, the accumulator being exact, the same y
// bits as k_gemv_w4a8.
// ------------------------------------------------------------------------
constexpr int kWideThreads = 1024;  // on a producer's codes
constexpr int kWideThreadsX = 512;  // quantising x in the prologue (single [3584, 3584]: 4.10 -> 3.96 us; on
                                    // codes 512 threads were slower, 3.38 -> 3.45 us)
constexpr int kWideMaxN = 8192;   // linear_w4a8 / gemv_w4a8 take the wide kernel up to this many rows
constexpr int kWideMaxK = 24576;  // and this K (U <= 12 chunks per lane: 16 spilled)
// On a producer's codes only up to this K: at K = 18944 the 256-thread
// kernel, which preloads the codes too, was faster ([3584, 18944] 9.0
// against 9.6 us), while for the fused linear the wide one was ([3584, 18944]
// in the per-linear 28-layer stream 1.18 -> 1.10 ms per token).
constexpr int kWideMaxKQ8 = 8192;

// One wave's row of the wide kernels: U chunks per lane against the staged
// codes, the lanes' exact sum, the fp32 epilogue.
template <int U>
__device__ __forceinline__ void wide_dot(const u32x4 (&w)[U], const u32x2* xs, int C, int lane, int r, int N,
                                         const float* sw, const float* bias, float sx, float* y, int32_t* acc_out)
{
    int acc = 0;
    const u32x4* xq = reinterpret_cast<const u32x4*>(xs);
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int c = lane + kWave * j;
        if (c < C)
            acc = dot_chunk16(w[j], xq[2 * c], xq[2 * c + 1], acc);
    }
    acc = sum_lanes<kWave>(acc >> 4);
    if (lane == 0 && r < N) {
        if (acc_out)
            acc_out[r] = acc;
        y[r] = fmaf(sw[r] * sx, (float)acc, bias ? bias[r] : 0.0f);
    }
}

template <int U, int XIN, int TH>
__global__ __launch_bounds__(TH) void k_linear_wide(
    const u32x4* __restrict__ wq, const float* __restrict__ sw, const float* __restrict__ bias,
    const void* __restrict__ x, const float* __restrict__ sx_in, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int8_t* __restrict__ qx_out, float* __restrict__ sx_out, int N, int C)
{
    constexpr int ROWS = TH / kWave;                     // one wave per row
    constexpr int NG = (4 * kWave * U + TH - 1) / TH;  // 8-value groups of x per thread: 4C <= TH NG
    constexpr int NQ = (2 * kWave * U + TH - 1) / TH;  // 16-byte pieces of codes per thread: 2C <= TH NQ
    extern __shared__ u32x4 xsd[];   // codes of 8 values per group, permuted (K bytes)
    u32x2* xs = reinterpret_cast<u32x2*>(xsd);
    __shared__ float red[ROWS];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int G8 = 4 * C;
    const int row = min(blockIdx.x * ROWS + wave, N - 1);
    float sxv;
    if constexpr (XIN == X_Q8) {
        // codes already made (a producer's)
        const int G16 = 2 * C;
        const __amdgpu_buffer_rsrc_t r = uniform_rsrc(x, 16 * G16);
        u32x4 q[NQ];
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int g = tid + k * TH;
            q[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, g < G16 ? 16 * g : kBufferPast,
                                                                                   0, 0));
        }
        u32x4 w[U];
#pragma unroll
        for (int j = 0; j < U; ++j)
            w[j] = __builtin_nontemporal_load(wq + (size_t)row * C + min(lane + kWave * j, C - 1));
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int g = tid + k * TH;
            if (g < G16) {
                xs[2 * g] = u32x2{perm_even(q[k].x, q[k].y), perm_odd(q[k].x, q[k].y)};
                xs[2 * g + 1] = u32x2{perm_even(q[k].z, q[k].w), perm_odd(q[k].z, q[k].w)};
            }
        }
        sxv = *sx_in;
        __syncthreads();
        wide_dot<U>(w, xs, C, lane, blockIdx.x * ROWS + wave, N, sw, bias, sxv, y, acc_out);
        return;
    } else {
        float v[NG][8];
#pragma unroll
        for (int k = 0; k < NG; ++k)
            load8<XIN>(x, min(tid + k * TH, G8 - 1), v[k]);  // a clamped group repeats a real one
        u32x4 w[U];
#pragma unroll
        for (int j = 0; j < U; ++j)
            w[j] = __builtin_nontemporal_load(wq + (size_t)row * C + min(lane + kWave * j, C - 1));
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < NG; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                m = fmaxf(m, fabsf(v[k][e]));
        m = wave_max_dpp(m);
        if (lane == 0)
            red[wave] = m;
        __syncthreads();
        float amax = red[0];
#pragma unroll
        for (int i = 1; i < ROWS; ++i)
            amax = fmaxf(amax, red[i]);
        const ActScale a = act_scale(amax);
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const int g = tid + k * TH;
            if (g < G8) {
                uint32_t lo, hi;
                quant8_fast(v[k], a, lo, hi);
                xs[g] = u32x2{perm_even(lo, hi), perm_odd(lo, hi)};
                if (qx_out && blockIdx.x == 0)
                    reinterpret_cast<u32x2*>(qx_out)[g] = u32x2{lo, hi};
            }
        }
        if (sx_out && blockIdx.x == 0 && tid == 0)
            *sx_out = a.s;
        __syncthreads();
        wide_dot<U>(w, xs, C, lane, blockIdx.x * ROWS + wave, N, sw, bias, a.s, y, acc_out);
    }
}

// ------------------------------------------------------------------------
// W4A8 GEMV for any K % 8 == 0 up to the int32 bound of the page "Jetson
// Orin AGX INT4 ..." (section "INT32 accumulator 是否安全"), the shapes the
// kernels above refuse (K % 32 != 0, or more codes than LDS holds): one wave
// per row, four rows per workgroup, the row read as 4-byte words (a row
// needs only 4-byte alignment) and the activation from memory, one 8-value
// group per word.  For an fp32 / fp16 x each workgroup first finds max|x|
// over the whole activation, then codes every group it meets with
// quantize_act's arithmetic (the same codes).  A correctness path: it keeps
// no activation on chip and streams no wider than 4 bytes per lane.
// ------------------------------------------------------------------------
constexpr int kAnyRows = kThreads / kWave;

template <int XIN>
__global__ __launch_bounds__(kThreads) void k_gemv_w4a8_any(
    const uint32_t* __restrict__ wq, const float* __restrict__ sw, const float* __restrict__ bias,
    const void* __restrict__ x, const float* __restrict__ sx_in, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int8_t* __restrict__ qx_out, float* __restrict__ sx_out, int N, int K)
{
    __shared__ float red[4];
    const int G8 = K / 8;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    ActScale a{0.0f, 0.0f, false};
    float s;
    if constexpr (XIN == X_Q8) {
        s = *sx_in;
    } else {
        float amax = 0.0f;
        for (int g = threadIdx.x; g < G8; g += kThreads) {
            float v[8];
            load8<XIN>(x, g, v);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                amax = fmaxf(amax, fabsf(v[e]));
        }
        a = act_scale(block_max(amax, red));
        s = a.s;
        if (blockIdx.x == 0) {
            if (qx_out) {
                for (int g = threadIdx.x; g < G8; g += kThreads) {
                    float v[8];
                    load8<XIN>(x, g, v);
                    uint32_t lo, hi;
                    quant8_fast(v, a, lo, hi);
                    reinterpret_cast<u32x2*>(qx_out)[g] = u32x2{lo, hi};
                }
            }
            if (sx_out && threadIdx.x == 0)
                *sx_out = a.s;
        }
    }
    for (int row = blockIdx.x * kAnyRows + wave; row < N; row += gridDim.x * kAnyRows) {  // wave-uniform
        const uint32_t* wr = wq + (size_t)row * G8;
        int acc = 0;
        for (int g = lane; g < G8; g += kWave) {
            const uint32_t wv = __builtin_nontemporal_load(wr + g);
            uint32_t lo, hi;
            if constexpr (XIN == X_Q8) {
                const u32x2 q = reinterpret_cast<const u32x2*>(x)[g];
                lo = q.x;
                hi = q.y;
            } else {
                float v[8];
                load8<XIN>(x, g, v);
                quant8_fast(v, a, lo, hi);
            }
            acc = __builtin_amdgcn_sdot4(lo16(wv), (int)perm_even(lo, hi), acc, false);
            acc = __builtin_amdgcn_sdot4(hi16(wv), (int)perm_odd(lo, hi), acc, false);
        }
        acc = sum_lanes<kWave>(acc >> 4);
        if (lane == 0) {
            if (acc_out)
                acc_out[row] = acc;
            y[row] = fmaf(sw[row] * s, (float)acc, bias ? bias[row] : 0.0f);
        }
    }
}

// ------------------------------------------------------------------------
// W4A8 GEMV, one fp16 scale per 32 codes (= per 16-byte chunk).
//   y = sx * sum_g s_g * acc_g + b; acc_g exact int32, the scaled sum fp32.
//   Same pipeline as k_gemv_w4a8, with each chunk's scale loaded beside it.
// ------------------------------------------------------------------------
template <int R, int L, int U, int XIN>
__global__ __launch_bounds__(kThreads) void k_gemv_w4a8_g32(
    const u32x4* __restrict__ wq, const uint16_t* __restrict__ s16, const float* __restrict__ bias,
    const void* __restrict__ xin, const float* __restrict__ sx_in, float* __restrict__ y,
    int32_t* __restrict__ accg_out, int8_t* __restrict__ qx_out, float* __restrict__ sx_out, int N,
    int C)
{
    extern __shared__ u32x4 xs[];
    __shared__ float red[4];
    constexpr int GROUPS = kThreads / L;
    constexpr int ROWS = GROUPS * R;
    const int lane = threadIdx.x % L;
    const int grp = threadIdx.x / L;
    const int tiles = (N + ROWS - 1) / ROWS;
    const int iters = (C + L - 1) / L;
    const int steps = (iters + U - 1) / U;

    int tile = blockIdx.x;
    u32x4 cur[U][R];
    uint16_t scur[U][R];
    float sx;
    bool staged = false;
    if constexpr (XIN == X_F32 || XIN == X_F16) {
        if (C <= kThreads) {
            // the activation's loads first, then the first weight step's
            float v[4][8];
            preload_x<XIN>(xin, 4 * C, v);
            load_step<R, L, U>(cur, wq, N, C, tile * ROWS + grp * R, 0, lane);
            load_scales<R, L, U>(scur, s16, N, C, tile * ROWS + grp * R, 0, lane);
            sx = quant_from_regs(reinterpret_cast<u32x2*>(xs), v, 4 * C, red, qx_out, sx_out);
            staged = true;
        }
    } else if constexpr (XIN == X_Q8) {
        if (2 * C <= kQ8Pre * kThreads) {
            u32x4 v[kQ8Pre];
            preload_q8(xin, 2 * C, v);
            load_step<R, L, U>(cur, wq, N, C, tile * ROWS + grp * R, 0, lane);
            load_scales<R, L, U>(scur, s16, N, C, tile * ROWS + grp * R, 0, lane);
            write_q8(reinterpret_cast<u32x2*>(xs), v, 2 * C);
            sx = *sx_in;
            staged = true;
        }
    }
    if (!staged) {
        load_step<R, L, U>(cur, wq, N, C, tile * ROWS + grp * R, 0, lane);
        load_scales<R, L, U>(scur, s16, N, C, tile * ROWS + grp * R, 0, lane);
        sx = stage_activation<XIN>(xs, xin, sx_in, C, red, qx_out, sx_out);
    }
    __syncthreads();

    for (; tile < tiles; tile += gridDim.x) {
        const int row0 = tile * ROWS + grp * R;
        float facc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            facc[r] = 0.0f;
        for (int st = 0; st < steps; ++st) {
            u32x4 nxt[U][R];
            uint16_t snxt[U][R];
            int ntile = tile, nst = st + 1;
            if (nst == steps) {
                ntile += gridDim.x;
                nst = 0;
            }
            const bool more = ntile < tiles;
            if (more) {
                load_step<R, L, U>(nxt, wq, N, C, ntile * ROWS + grp * R, nst, lane);
                load_scales<R, L, U>(snxt, s16, N, C, ntile * ROWS + grp * R, nst, lane);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (st * U + u < iters) {
                    const int c = (st * U + u) * L + lane;
                    const int cc = min(c, C - 1);
                    const u32x4 xa = xs[2 * cc], xb = xs[2 * cc + 1];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const int ag = dot_chunk16(cur[u][r], xa, xb, 0) >> 4;
                        const float sg = (float)__builtin_bit_cast(_Float16, scur[u][r]);
                        facc[r] = fmaf((float)ag, sg, facc[r]);
                        if (accg_out != nullptr && c < C && row0 + r < N)
                            accg_out[(size_t)(row0 + r) * C + c] = ag;
                    }
                }
            }
            if (more) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        cur[u][r] = nxt[u][r];
                        scur[u][r] = snxt[u][r];
                    }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            facc[r] = sum_lanes_f<L>(facc[r]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r;
            if (lane == r && row < N)
                y[row] = fmaf(sx, facc[r], bias ? bias[row] : 0.0f);
        }
    }
}

// ------------------------------------------------------------------------
// W8A16 GEMV (int8 codes, fp16 group-32 scales, fp16 activation).
//   A lane handles whole 32-code groups (two 16-byte chunks).  Each byte
//   code q becomes an exact fp16 by the magic-number route: u = q ^ 0x80 =
//   q + 128 in [0, 255], fp16 bits 0x6400 | u = 1024 + u (spacing 1 there),
//   minus 1152.  One v_perm_b32 against the constant 0x64 bytes builds the
//   fp16 pair of two codes; pairs then go through v_dot2_f32_f16 against the
//   staged fp16 x.  (Masking the 6-bit code and assembling the pairs with
//   shifts took 3.65 VALU instructions per code; this takes 1.75.)
// ------------------------------------------------------------------------
__device__ __forceinline__ float dot4_w8_f16(uint32_t w, uint32_t x01, uint32_t x23, float acc)
{
    const uint32_t u = w ^ 0x80808080u;
    // selector bytes 0-3 take u's bytes, 4 a byte of 0x64646464
    const uint32_t h01 = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // [u0, 64, u1, 64]
    const uint32_t h23 = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // [u2, 64, u3, 64]
    const h16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    const h16x2 q01 = __builtin_bit_cast(h16x2, h01) - bias;
    const h16x2 q23 = __builtin_bit_cast(h16x2, h23) - bias;
    acc = __builtin_amdgcn_fdot2(q01, __builtin_bit_cast(h16x2, x01), acc, false);
    acc = __builtin_amdgcn_fdot2(q23, __builtin_bit_cast(h16x2, x23), acc, false);
    return acc;
}

template <int R, int L>
__global__ __launch_bounds__(kThreads) void k_gemv_w8a16_g32(
    const u32x4* __restrict__ w8, const uint16_t* __restrict__ s16, const u32x4* __restrict__ x16,
    float* __restrict__ y, int N, int G)
{
    extern __shared__ u32x4 xs[];  // 4 chunks (32 fp16) per group
    for (int i = threadIdx.x; i < 4 * G; i += kThreads)
        xs[i] = x16[i];
    __syncthreads();

    constexpr int GROUPS = kThreads / L;
    constexpr int ROWS = GROUPS * R;
    constexpr int U = 2;
    const int lane = threadIdx.x % L;
    const int grp = threadIdx.x / L;
    const int tiles = (N + ROWS - 1) / ROWS;
    const int iters = (G + L - 1) / L;

    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int row0 = tile * ROWS + grp * R;
        const u32x4* wrow[R];
        const uint16_t* srow[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const size_t rr = (size_t)min(row0 + r, N - 1);
            wrow[r] = w8 + rr * (2 * (size_t)G);
            srow[r] = s16 + rr * G;
        }
        float facc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            facc[r] = 0.0f;
        for (int it = 0; it < iters; it += U) {
            u32x4 w[U][R][2];
            uint16_t sc[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = (it + u) * L + lane;
                const bool ok = (it + u < iters) && (g < G);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    w[u][r][0] = ok ? wrow[r][2 * g] : u32x4{0u, 0u, 0u, 0u};
                    w[u][r][1] = ok ? wrow[r][2 * g + 1] : u32x4{0u, 0u, 0u, 0u};
                    sc[u][r] = ok ? srow[r][g] : (uint16_t)0;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = min((it + u) * L + lane, G - 1);
                const u32x4 x0 = xs[4 * g], x1 = xs[4 * g + 1], x2 = xs[4 * g + 2], x3 = xs[4 * g + 3];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const u32x4 a = w[u][r][0], b = w[u][r][1];
                    float p = 0.0f;
                    p = dot4_w8_f16(a.x, x0.x, x0.y, p);
                    p = dot4_w8_f16(a.y, x0.z, x0.w, p);
                    p = dot4_w8_f16(a.z, x1.x, x1.y, p);
                    p = dot4_w8_f16(a.w, x1.z, x1.w, p);
                    p = dot4_w8_f16(b.x, x2.x, x2.y, p);
                    p = dot4_w8_f16(b.y, x2.z, x2.w, p);
                    p = dot4_w8_f16(b.z, x3.x, x3.y, p);
                    p = dot4_w8_f16(b.w, x3.z, x3.w, p);
                    facc[r] = fmaf((float)__builtin_bit_cast(_Float16, sc[u][r]), p, facc[r]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            facc[r] = sum_lanes_f<L>(facc[r]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r;
            if (lane == r && row < N)
                y[row] = facc[r];
        }
    }
}

// ------------------------------------------------------------------------
// Packed 6-bit lm_head ("在香橙派上跑 Gemma4 ..." section 3.2 sizes a Q6_K
// weight at 210 bytes per 256: 4-bit low and 2-bit high fields of each code,
// an int8 scale per 16 weights, an fp16 scale per 256; the page expands it to
// int8 because decoding the fields was vector-instruction bound there).  This
// library's layout: separate aligned arrays per row,
//   ql [K/2]: low nibble of u = q + 32 in byte i/2 (bits 0-3 even i, 4-7 odd)
//   qh [K/4]: per 16 weights a uint32; weight 8k + e (k in {0,1}) puts bits
//             4-5 of u at bit 2(e mod 4) + 8k + 16[e >= 4]
//   sc [K/16] int8, d [K/256] fp16;  value = d * sc * q.
// The high-bit placement makes one shift and one mask bring the high bits of
// the code pair (e, e + 4) of a low-nibble word to bits 4-5 of both 16-bit
// halves, so a pair costs: shift + and-or (low nibbles, fp16 exponent 0x64),
// shift + and-or (high bits), a packed fp16 subtract of 1056 (fp16 bits
// 0x6400 | u = 1024 + u) and one v_dot2_f32_f16.
// ------------------------------------------------------------------------

// Load-time quantisation, one thread per 16-weight sub-block, 16 lanes per
// 256-weight super-block (K % 256 == 0 keeps super-blocks on 16-lane
// boundaries):  t = max|w| / 31;  d = fp16(max t / 127);  sc = clip(round(t /
// d), 0, 127);  q = clip(round(w / (d * sc)), -32, 31) (fp32 divisions, RNE;
// a zero scale gives zero codes).
__global__ __launch_bounds__(kThreads) void k_quantize_weights_q6k(const float* __restrict__ W, int K,
                                                                   long long subblocks, u32x2* __restrict__ ql,
                                                                   uint32_t* __restrict__ qh,
                                                                   int8_t* __restrict__ sc,
                                                                   uint16_t* __restrict__ d)
{
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= subblocks)  // whole 16-lane super-blocks leave together
        return;
    const f32x4* wp = reinterpret_cast<const f32x4*>(W) + 4 * gid;
    float v[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x4 t = wp[k];
        v[4 * k] = t.x;
        v[4 * k + 1] = t.y;
        v[4 * k + 2] = t.z;
        v[4 * k + 3] = t.w;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        m = fmaxf(m, fabsf(v[i]));
    const float t = m / 31.0f;
    float tmax = t;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
        tmax = fmaxf(tmax, __shfl_xor(tmax, o));
    const _Float16 dh = (_Float16)(tmax / 127.0f);
    const float df = (float)dh;
    const float scf = df == 0.0f ? 0.0f : fminf(fmaxf(rintf(t / df), 0.0f), 127.0f);
    const float e = df * scf;  // exact: 11 x 7 significant bits
    uint32_t lo = 0, hi = 0, hw = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float qf = e == 0.0f ? 0.0f : fminf(fmaxf(rintf(v[i] / e), -32.0f), 31.0f);
        const uint32_t u = (uint32_t)((int)qf + 32);
        if (i < 8)
            lo |= (u & 15u) << (4 * i);
        else
            hi |= (u & 15u) << (4 * (i - 8));
        const int k = i / 8, ee = i % 8;
        hw |= (u >> 4) << (2 * (ee % 4) + 8 * k + 16 * (ee >= 4));
    }
    ql[gid] = u32x2{lo, hi};
    qh[gid] = hw;
    sc[gid] = (int8_t)(int)scf;
    if ((gid & 15) == 0)
        d[gid / 16] = __builtin_bit_cast(uint16_t, dh);
}

// Eight codes of one low-nibble word w (weights 8k..8k+7) with their high
// bits hq (already shifted so that pair e sits at bits 2e and 16 + 2e),
// against the staged activation pairs (x_e, x_{e+4}), e = 0..3.
// (a & m) | (b & ~m) in one instruction (the compiler splits it into and/or3
// when b is a constant).
__device__ __forceinline__ uint32_t bfi32(uint32_t m, uint32_t a, uint32_t b)
{
    uint32_t d;
    __asm__("v_bfi_b32 %0, %1, %2, %3" : "=v"(d) : "s"(m), "v"(a), "v"(b));
    return d;
}

__device__ __forceinline__ float dot8_q6(uint32_t w, uint32_t hq, uint32_t x04, uint32_t x15, uint32_t x26,
                                         uint32_t x37, float acc)
{
    const h16x2 bias = {(_Float16)1056.0f, (_Float16)1056.0f};
    const uint32_t xp[4] = {x04, x15, x26, x37};
    const uint32_t expo = 0x64006400u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // low nibbles into the fp16 exponent word, then the high bits over them
        const uint32_t hs = 2 * e <= 4 ? hq << (4 - 2 * e) : hq >> (2 * e - 4);
        const uint32_t u2 = bfi32(0x00300030u, hs, bfi32(0x000F000Fu, w >> (4 * e), expo));
        acc = __builtin_amdgcn_fdot2(as_h16x2(u2) - bias, as_h16x2(xp[e]), acc, false);
    }
    return acc;
}

// Lane reduction for 8 lanes per row (the wave64 DPP row reduction of
// sum_lanes_f covers 16).
template <int L>
__device__ __forceinline__ float sum_lanes_q6(float v)
{
    if constexpr (L == 8) {
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        return v;
    } else {
        return sum_lanes_f<L>(v);
    }
}

// A lane takes units of 64 weights (two 32-weight chunks): low fields 2 x 16
// bytes, high fields 16 bytes, the four sub-block scales as one 4-byte word
// and the fp16 super-block scale -- five loads per 64 weights; U units per
// step, R rows per lane group, L lanes per row.
template <int R, int U>
struct Q6Step {
    u32x4 la[U][R], lb[U][R], hw[U][R];
    uint32_t s4[U][R], dd[U][R];
};

// The loads of step `it` of the rows rr (clamped rows; a unit past the row
// loads at a clamped unit with its scales zeroed, so it adds nothing).
template <int R, int L, int U>
__device__ __forceinline__ void q6k_load(Q6Step<R, U>& s, const u32x4* __restrict__ ql, const u32x4* __restrict__ qh,
                                         const uint32_t* __restrict__ sc4, const uint16_t* __restrict__ d16,
                                         const size_t (&rr)[R], int it, int iters, int C, int lane)
{
    const int C2 = C / 2, D = C / 8;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c2 = (it + u) * L + lane;
        const bool ok = (it + u < iters) && (c2 < C2);
        const int cc = min(c2, C2 - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            s.la[u][r] = ql[rr[r] * C + 2 * cc];
            s.lb[u][r] = ql[rr[r] * C + 2 * cc + 1];
            s.hw[u][r] = qh[rr[r] * C2 + cc];
            const uint32_t sv = sc4[rr[r] * C2 + cc];
            s.s4[u][r] = ok ? sv : 0u;
            s.dd[u][r] = d16[rr[r] * D + cc / 4];
        }
    }
}

template <int R, int L, int U>
__device__ __forceinline__ void q6k_dot(const Q6Step<R, U>& s, const u32x4* xs, int it, int C, int lane,
                                        float (&facc)[R])
{
    const int C2 = C / 2;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = 2 * min((it + u) * L + lane, C2 - 1);
        const u32x4 g0 = xs[4 * c], g1 = xs[4 * c + 1], g2 = xs[4 * c + 2], g3 = xs[4 * c + 3];
        const u32x4 g4 = xs[4 * c + 4], g5 = xs[4 * c + 5], g6 = xs[4 * c + 6], g7 = xs[4 * c + 7];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4 wa = s.la[u][r], wb = s.lb[u][r], h = s.hw[u][r];
            float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f, p3 = 0.0f;
            p0 = dot8_q6(wa.x, h.x, g0.x, g0.y, g0.z, g0.w, p0);
            p0 = dot8_q6(wa.y, h.x >> 8, g1.x, g1.y, g1.z, g1.w, p0);
            p1 = dot8_q6(wa.z, h.y, g2.x, g2.y, g2.z, g2.w, p1);
            p1 = dot8_q6(wa.w, h.y >> 8, g3.x, g3.y, g3.z, g3.w, p1);
            p2 = dot8_q6(wb.x, h.z, g4.x, g4.y, g4.z, g4.w, p2);
            p2 = dot8_q6(wb.y, h.z >> 8, g5.x, g5.y, g5.z, g5.w, p2);
            p3 = dot8_q6(wb.z, h.w, g6.x, g6.y, g6.z, g6.w, p3);
            p3 = dot8_q6(wb.w, h.w >> 8, g7.x, g7.y, g7.z, g7.w, p3);
            const float df = (float)__builtin_bit_cast(_Float16, (uint16_t)s.dd[u][r]);
            const uint32_t sv = s.s4[u][r];
            float a = facc[r];
            a = fmaf(df * (float)(int8_t)(sv & 0xFFu), p0, a);
            a = fmaf(df * (float)(int8_t)((sv >> 8) & 0xFFu), p1, a);
            a = fmaf(df * (float)(int8_t)((sv >> 16) & 0xFFu), p2, a);
            a = fmaf(df * (float)(int8_t)(sv >> 24), p3, a);
            facc[r] = a;
        }
    }
}

// Up to 2 rows per lane group the next step's loads are issued before the
// current step's decode (two register sets; with more rows one set, as the
// registers run out).
template <int R, int L>
__global__ __launch_bounds__(kThreads) void k_gemv_q6k(const u32x4* __restrict__ ql, const u32x4* __restrict__ qh,
                                                       const uint32_t* __restrict__ sc4,
                                                       const uint16_t* __restrict__ d16,
                                                       const u32x4* __restrict__ x16, float* __restrict__ y, int N,
                                                       int C)
{
    extern __shared__ u32x4 xs[];  // per 8 weights: (x0,x4) (x1,x5) (x2,x6) (x3,x7)
    constexpr int GROUPS = kThreads / L;
    constexpr int ROWS = GROUPS * R;
    constexpr bool kPipe = R <= 2;
    constexpr int U = kPipe ? 1 : 2;
    const int lane = threadIdx.x % L;
    const int grp = threadIdx.x / L;
    const int tiles = (N + ROWS - 1) / ROWS;
    const int C2 = C / 2;  // 64-weight units per row
    const int iters = (C2 + L - 1) / L;
    const int steps = (iters + U - 1) / U;
    auto rows_of = [&](int tile, size_t (&rr)[R]) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            rr[r] = (size_t)min(tile * ROWS + grp * R + r, N - 1);
    };

    int tile = blockIdx.x;
    size_t rr[R];
    rows_of(tile, rr);
    Q6Step<R, U> cur;
    if (kPipe && tile < tiles)
        q6k_load<R, L, U>(cur, ql, qh, sc4, d16, rr, 0, iters, C, lane);  // ahead of the staging
    for (int g = threadIdx.x; g < 4 * C; g += kThreads) {
        const u32x4 v = x16[g];
        xs[g] = u32x4{(v.x & 0xFFFFu) | (v.z << 16), (v.x >> 16) | (v.z & 0xFFFF0000u),
                      (v.y & 0xFFFFu) | (v.w << 16), (v.y >> 16) | (v.w & 0xFFFF0000u)};
    }
    __syncthreads();

    for (; tile < tiles; tile += gridDim.x) {
        rows_of(tile, rr);
        float facc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            facc[r] = 0.0f;
        for (int st = 0; st < steps; ++st) {
            if constexpr (kPipe) {
                int ntile = tile, nst = st + 1;
                if (nst == steps) {
                    ntile += gridDim.x;
                    nst = 0;
                }
                Q6Step<R, U> nxt;
                const bool more = ntile < tiles;  // uniform across the workgroup
                if (more) {
                    size_t nr[R];
                    rows_of(ntile, nr);
                    q6k_load<R, L, U>(nxt, ql, qh, sc4, d16, nr, nst * U, iters, C, lane);
                }
                q6k_dot<R, L, U>(cur, xs, st * U, C, lane, facc);
                if (more)
                    cur = nxt;
            } else {
                q6k_load<R, L, U>(cur, ql, qh, sc4, d16, rr, st * U, iters, C, lane);
                q6k_dot<R, L, U>(cur, xs, st * U, C, lane, facc);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            facc[r] = sum_lanes_q6<L>(facc[r]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = tile * ROWS + grp * R + r;
            if (lane == r && row < N)
                y[row] = facc[r];
        }
    }
}

// ------------------------------------------------------------------------
// INT8-X (3,5,8) lossless INT8 weights ("定長無損 INT8 壓縮與 Triton 融合解碼",
// sections 2.1-2.5), decoded inside a W8A8 GEMV.  Over the row-major
// flattened tensor: B1 (a bit per weight, 1 = not level 1), B2 (a bit per
// non-level-1 weight, 1 = level 3), L1 (3-bit two's complement codes of
// |v| <= 3), L2 (5-bit codes of |v| <= 15), L3 (raw bytes), all bit streams
// LSB-first; per block of BQD_INT8X_BLOCK weights the set bits of B1 and B2
// before it.  A wave decodes one block, 8 weights per lane: the lane's B1
// byte gives its non-level-1 count, a wave prefix scan its place among the
// block's, its B2 bits (a 64-bit window) its level-3 count and a second
// scan; the block sums then locate its runs in L1, L2 and L3, read through
// 64/96-bit windows; the 8 codes are selected branch-free, dotted with the
// int8 activation (two v_dot4_i32_i8) and summed exactly per row in LDS.
// Every stream index is clamped to its stream, so a malformed encoding
// cannot read out of bounds.
// ------------------------------------------------------------------------
constexpr int kInt8xBlock = BQD_INT8X_BLOCK;
static_assert(kInt8xBlock == 8 * kWave, "one wave decodes one block, 8 weights per lane");

__device__ __forceinline__ int wave_excl_scan(int v)
{
    const int lane = threadIdx.x & (kWave - 1);
    int inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(inc, o);
        inc += lane >= o ? t : 0;
    }
    return inc - v;
}

struct Int8xStreams {
    const uint32_t* b1;
    const uint32_t* b2;
    const uint32_t* l1;
    const uint32_t* l2;
    const uint32_t* l3;  // bytes, read as words
    const int32_t* b1_blk;
    const int32_t* b2_blk;
    int nb2, nl1, nl2, nl3;  // words in b2, l1, l2, l3 (>= 3: padding included)
};

// 64 bits of a word stream from bit pos, as (hi, lo); the first word index
// is clamped to [0, n - 3] so the three reads stay inside the stream.
__device__ __forceinline__ void window(const uint32_t* s, int pos, int n, uint32_t& lo, uint32_t& hi)
{
    const int w = min(max(pos >> 5, 0), n - 3);
    const uint32_t a = s[w], b = s[w + 1], c = s[w + 2];
    const uint32_t off = (uint32_t)pos & 31u;
    lo = __builtin_amdgcn_alignbit(b, a, off);
    hi = __builtin_amdgcn_alignbit(c, b, off);
}

template <int R>
__global__ __launch_bounds__(kThreads) void k_gemv_int8x(Int8xStreams st, const int8_t* __restrict__ qx,
                                                         const float* __restrict__ sx, float sw,
                                                         float* __restrict__ y, int32_t* __restrict__ acc_out,
                                                         int N, int K)
{
    __shared__ int racc[R];
    if (threadIdx.x < R)
        racc[threadIdx.x] = 0;
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int bpr = K / kInt8xBlock;  // blocks per row
    const int row0 = blockIdx.x * R;
    const int items = min(R, N - row0) * bpr;
    for (int item = wave; item < items; item += kThreads / kWave) {
        const int rr = item / bpr, bi = item % bpr;
        const long long g = (long long)(row0 + rr) * bpr + bi;  // global block
        const long long t0 = g * kInt8xBlock;
        const uint32_t b1w = st.b1[(t0 >> 5) + (lane >> 2)];
        const uint32_t bits8 = (b1w >> (8 * (lane & 3))) & 0xFFu;
        const int nn = __builtin_popcount(bits8);
        const int pre_nn = wave_excl_scan(nn);
        const int blk1 = st.b1_blk[g], blk2 = st.b2_blk[g];
        uint32_t b2lo, b2hi;
        window(st.b2, blk1 + pre_nn, st.nb2, b2lo, b2hi);
        const uint32_t b2bits = b2lo & ((1u << nn) - 1u);
        const int n3 = __builtin_popcount(b2bits);
        const int pre3 = wave_excl_scan(n3);
        // first stream index of the lane's weights of each level
        const int i1 = (int)(t0 - blk1) + (8 * lane - pre_nn);
        const int i2 = (blk1 - blk2) + (pre_nn - pre3);
        const int i3 = blk2 + pre3;
        uint32_t w1, w1h, lo2, hi2, lo3, hi3;
        window(st.l1, 3 * i1, st.nl1, w1, w1h);
        window(st.l2, 5 * i2, st.nl2, lo2, hi2);
        window(st.l3, 8 * i3, st.nl3, lo3, hi3);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // rank of weight e among the lane's non-level-1 weights, and
            // among its level-3 ones, from the bitmap bits below it
            const int rn = __builtin_popcount(bits8 & ((1u << e) - 1u));
            const int r3 = __builtin_popcount(b2bits & ((1u << rn) - 1u));
            const bool n1 = (bits8 >> e) & 1u;
            const bool l3 = (b2bits >> rn) & 1u;
            const int r1 = e - rn, r2 = rn - r3;
            const int c1 = __builtin_amdgcn_sbfe((int)w1, 3 * r1, 3);
            const int o2 = 5 * r2;  // <= 30 unless e == 7
            const uint32_t f2 = (e == 7 && o2 >= 32) ? hi2 >> (o2 - 32) : __builtin_amdgcn_alignbit(hi2, lo2, o2);
            const int c2 = __builtin_amdgcn_sbfe((int)f2, 0, 5);
            const int c3 = __builtin_amdgcn_sbfe((int)__builtin_amdgcn_perm(hi3, lo3, 0x0C0C0C00u | (uint32_t)r3), 0, 8);
            const int v = n1 ? (l3 ? c3 : c2) : c1;
            if (e < 4)
                lo |= ((uint32_t)v & 0xFFu) << (8 * e);
            else
                hi |= ((uint32_t)v & 0xFFu) << (8 * (e - 4));
        }
        const u32x2 xv = *reinterpret_cast<const u32x2*>(qx + (size_t)bi * kInt8xBlock + 8 * lane);
        int a = __builtin_amdgcn_sdot4((int)lo, (int)xv.x, 0, false);
        a = __builtin_amdgcn_sdot4((int)hi, (int)xv.y, a, false);
        a = sum_lanes<64>(a);
        if (lane == 0)
            atomicAdd(&racc[rr], a);
    }
    __syncthreads();
    if (threadIdx.x < R && row0 + (int)threadIdx.x < N) {
        const int row = row0 + threadIdx.x;
        const int a = racc[threadIdx.x];
        if (acc_out)
            acc_out[row] = a;
        y[row] = (sw * sx[0]) * (float)a;
    }
}

// ------------------------------------------------------------------------
// W4A16 comparison GEMV: the same packed per-row INT4 weights against an
// fp16 activation, unpacked to fp16 and multiplied in floating point
// ("Jetson Orin AGX INT4 ..." section "为什么 INT4 float 解包不快" weighs this
// route against the integer dot; "在香橙派上跑 Gemma4 ..." section 3.1
// dequantises to fp16 and uses fp16 MACs).
//   Per word: u = w ^ 0x88888888 turns each signed nibble q into q + 8;
//   bytes (u & 0x0F0F0F0F) hold codes {0,2,4,6}, ((u >> 4) & 0x0F0F0F0F)
//   codes {1,3,5,7}; one v_perm_b32 spreads a byte pair into fp16 bits
//   0x6400 | (q+8) = 1024 + q + 8, and a packed subtract of 1032 gives q
//   exactly; then v_dot2_f32_f16 against x staged per 8-group as [x0 x2 |
//   x4 x6 | x1 x3 | x5 x7].  The compiled loop issues about 2.0 VALU
//   instructions per code (3.4 when the pairs were assembled with shifts
//   and masks), against about 1.1 for the integer dot.  y = fmaf(sw, acc, b)
//   with acc the fp32 sum.
// ------------------------------------------------------------------------
__device__ __forceinline__ float dot8_w4_f16(uint32_t w, u32x4 xg, float acc)
{
    const uint32_t u = w ^ 0x88888888u;
    const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
    // fp16 pairs [1024 + c_a, 1024 + c_b] from bytes a, b of a code word:
    // one v_perm_b32 each against the constant 0x64 bytes.
    const h16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h16x2 q02 = __builtin_bit_cast(h16x2, __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u)) - bias;
    const h16x2 q46 = __builtin_bit_cast(h16x2, __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u)) - bias;
    const h16x2 q13 = __builtin_bit_cast(h16x2, __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u)) - bias;
    const h16x2 q57 = __builtin_bit_cast(h16x2, __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)) - bias;
    acc = __builtin_amdgcn_fdot2(q02, as_h16x2(xg.x), acc, false);
    acc = __builtin_amdgcn_fdot2(q46, as_h16x2(xg.y), acc, false);
    acc = __builtin_amdgcn_fdot2(q13, as_h16x2(xg.z), acc, false);
    acc = __builtin_amdgcn_fdot2(q57, as_h16x2(xg.w), acc, false);
    return acc;
}

template <int R, int L>
__global__ __launch_bounds__(kThreads) void k_gemv_w4a16(const u32x4* __restrict__ wq, const float* __restrict__ sw,
                                                         const float* __restrict__ bias,
                                                         const u32x4* __restrict__ x16, float* __restrict__ y,
                                                         int N, int C)
{
    extern __shared__ u32x4 xs[];  // one 16-byte group of 8 fp16 per 8 codes, permuted
    for (int g = threadIdx.x; g < 4 * C; g += kThreads) {
        const u32x4 v = x16[g];  // x0..x7 as fp16 pairs (x0,x1) (x2,x3) (x4,x5) (x6,x7)
        xs[g] = u32x4{(v.x & 0xFFFFu) | (v.y << 16), (v.z & 0xFFFFu) | (v.w << 16),
                      (v.x >> 16) | (v.y & 0xFFFF0000u), (v.z >> 16) | (v.w & 0xFFFF0000u)};
    }
    __syncthreads();

    constexpr int GROUPS = kThreads / L;
    constexpr int ROWS = GROUPS * R;
    constexpr int U = 2;
    const int lane = threadIdx.x % L;
    const int grp = threadIdx.x / L;
    const int tiles = (N + ROWS - 1) / ROWS;
    const int iters = (C + L - 1) / L;

    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int row0 = tile * ROWS + grp * R;
        const u32x4* wrow[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            wrow[r] = wq + (size_t)min(row0 + r, N - 1) * C;
        float facc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            facc[r] = 0.0f;
        for (int it = 0; it < iters; it += U) {
            u32x4 w[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = (it + u) * L + lane;
                const bool ok = (it + u < iters) && (c < C);
#pragma unroll
                for (int r = 0; r < R; ++r)
                    w[u][r] = ok ? wrow[r][c] : u32x4{0u, 0u, 0u, 0u};  // codes 0
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = min((it + u) * L + lane, C - 1);
                const u32x4 g0 = xs[4 * c], g1 = xs[4 * c + 1], g2 = xs[4 * c + 2], g3 = xs[4 * c + 3];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float p = facc[r];
                    p = dot8_w4_f16(w[u][r].x, g0, p);
                    p = dot8_w4_f16(w[u][r].y, g1, p);
                    p = dot8_w4_f16(w[u][r].z, g2, p);
                    p = dot8_w4_f16(w[u][r].w, g3, p);
                    facc[r] = p;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            facc[r] = sum_lanes_f<L>(facc[r]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r;
            if (lane == r && row < N)
                y[row] = fmaf(sw[row], facc[r], bias ? bias[row] : 0.0f);
        }
    }
}

// ------------------------------------------------------------------------
// M-token verify GEMM, integer dot products.  MT >= M tokens are staged in
// LDS per K-segment (padding tokens are zero); each weight chunk is loaded
// and split once and meets all MT tokens.
// ------------------------------------------------------------------------
template <int MT, int R, int L>
__global__ __launch_bounds__(kThreads) void k_verify_w4a8(
    const u32x4* __restrict__ wq, const float* __restrict__ sw, const float* __restrict__ bias,
    const int8_t* __restrict__ qx, const float* __restrict__ sx, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int M, int N, int C, int SEGC)
{
    extern __shared__ u32x4 xs[];  // [MT][SEGC][2] chunks
    constexpr int GROUPS = kThreads / L;
    constexpr int ROWS = GROUPS * R;
    const int lane = threadIdx.x % L;
    const int grp = threadIdx.x / L;
    const int tiles = (N + ROWS - 1) / ROWS;
    const int K = 32 * C;
    const bool single = SEGC >= C;

    // Stage tokens' codes of chunks [c0, c0 + nc) into LDS (zeros for m >= M).
    auto stage = [&](int c0, int nc) {
        const int groups = 4 * nc;
        u32x2* xs2 = reinterpret_cast<u32x2*>(xs);
        for (int i = threadIdx.x; i < MT * groups; i += kThreads) {
            const int m = i / groups, g = i % groups;
            u32x2 v = {0u, 0u};
            if (m < M)
                v = reinterpret_cast<const u32x2*>(qx + (size_t)m * K)[4 * c0 + g];
            xs2[(size_t)m * 4 * SEGC + g] = u32x2{perm_even(v.x, v.y), perm_odd(v.x, v.y)};
        }
    };
    if (single) {
        stage(0, C);
        __syncthreads();
    }

    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int row0 = tile * ROWS + grp * R;
        const u32x4* wrow[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            wrow[r] = wq + (size_t)min(row0 + r, N - 1) * C;
        int acc[MT][R];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[m][r] = 0;

        for (int c0 = 0; c0 < C; c0 += SEGC) {
            const int nc = min(SEGC, C - c0);
            if (!single) {
                __syncthreads();
                stage(c0, nc);
                __syncthreads();
            }
            for (int cl = lane; cl < nc; cl += L) {
                u32x4 w[R];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    w[r] = wrow[r][c0 + cl];
                int lo[R][4], hi[R][4];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    lo[r][0] = lo16(w[r].x); hi[r][0] = hi16(w[r].x);
                    lo[r][1] = lo16(w[r].y); hi[r][1] = hi16(w[r].y);
                    lo[r][2] = lo16(w[r].z); hi[r][2] = hi16(w[r].z);
                    lo[r][3] = lo16(w[r].w); hi[r][3] = hi16(w[r].w);
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const u32x4 xa = xs[((size_t)m * SEGC + cl) * 2];
                    const u32x4 xb = xs[((size_t)m * SEGC + cl) * 2 + 1];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        int a = acc[m][r];
                        a = __builtin_amdgcn_sdot4(lo[r][0], (int)xa.x, a, false);
                        a = __builtin_amdgcn_sdot4(hi[r][0], (int)xa.y, a, false);
                        a = __builtin_amdgcn_sdot4(lo[r][1], (int)xa.z, a, false);
                        a = __builtin_amdgcn_sdot4(hi[r][1], (int)xa.w, a, false);
                        a = __builtin_amdgcn_sdot4(lo[r][2], (int)xb.x, a, false);
                        a = __builtin_amdgcn_sdot4(hi[r][2], (int)xb.y, a, false);
                        a = __builtin_amdgcn_sdot4(lo[r][3], (int)xb.z, a, false);
                        a = __builtin_amdgcn_sdot4(hi[r][3], (int)xb.w, a, false);
                        acc[m][r] = a;
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[m][r] = sum_lanes<L>(acc[m][r] >> 4);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r;
            if (lane == r && row < N) {
                const float swr = sw[row];
                const float b = bias ? bias[row] : 0.0f;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < M) {
                        if (acc_out)
                            acc_out[(size_t)m * N + row] = acc[m][r];
                        y[(size_t)m * N + row] = fmaf(swr * sx[m], (float)acc[m][r], b);
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------------
// M-token verify GEMM on the matrix cores.
//   v_mfma_i32_16x16x64_i8 computes D[i][j] += sum over 4 lane groups g and
//   16 bytes t of A_lane(i + 16g)[t] * B_lane(j + 16g)[t]; lane l receives
//   D[4*(l/16) + e][l % 16], e = 0..3.  A is a 16-row weight tile (lane l:
//   row l % 16), B the 16 token columns (lane l: token l % 16, zeros past
//   M); both take, per lane, the same 16 code positions.  A lane loads one
//   16-byte chunk (32 codes) of its row and feeds two MFMAs: words x, y as
//   [lo16(x) hi16(x) lo16(y) hi16(y)] against the staged activation chunk
//   half [A0 B0 A1 B1], then words z, w against [A2 B2 A3 B3] -- the pairing
//   of dot_chunk16, so the int32 result is 16 * acc exactly.
//   The 4 lane groups of a wave take 4 consecutive chunks of each of 16 rows
//   (64 contiguous bytes per row per load).  SPLIT consecutive waves share
//   a 16-row tile's K range and add their exact partials through LDS
//   (SPLIT = 1: each wave owns a tile).  The M tokens'
//   codes are staged per K segment in LDS; weight loads run U chunks ahead
//   of the MFMAs.
// ------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 mfma_chunk(u32x4 w, u32x4 xa, u32x4 xb, i32x4 acc)
{
    const i32x4 a0 = {lo16(w.x), hi16(w.x), lo16(w.y), hi16(w.y)};
    const i32x4 a1 = {lo16(w.z), hi16(w.z), lo16(w.w), hi16(w.w)};
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, __builtin_bit_cast(i32x4, xa), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, __builtin_bit_cast(i32x4, xb), acc, 0, 0, 0);
    return acc;
}

template <int U>
__device__ __forceinline__ void load_quads(u32x4 (&buf)[U], const u32x4* __restrict__ wrow, int c0,
                                           int nc, int q, int q1, int g)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = 4 * (q + u) + g;
        buf[u] = (q + u < q1 && c < nc) ? wrow[c0 + c] : u32x4{0u, 0u, 0u, 0u};
    }
}

template <int SPLIT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_verify_mfma(
    const u32x4* __restrict__ wq, const float* __restrict__ sw, const float* __restrict__ bias,
    const int8_t* __restrict__ qx, const float* __restrict__ sx, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int M, int N, int C, int SEGC)
{
    // Staged codes of the M tokens: token m's chunk c at xs[m * TS + 2c] and
    // [.. + 1]; the 16-byte pad per token row spreads the 16 token columns of
    // one read over the LDS banks.
    extern __shared__ u32x4 xs[];
    __shared__ i32x4 part[WAVES][kWave];
    constexpr int U = 8;
    constexpr int NT = WAVES * kWave;
    // Staging loads in flight per thread.  With up to 8 waves, 16 per thread
    // take the M = 16 activation in one round trip ([18944, 3584]: 17.3 ->
    // 16.1 us); 16-wave workgroups have 128 registers per lane, and more than
    // 4 spill (the [3584, 18944] verify then runs 2-3x slower).
    constexpr int kStageBatch = WAVES > 8 ? 4 : 16;
    constexpr int TPW = WAVES / SPLIT;  // row tiles per workgroup
    const int TS = 2 * SEGC + 1;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int g = lane >> 4, col = lane & 15;
    const bool tok = col < M;           // lanes past M feed zero columns
    const int xrow = (tok ? col : 0) * TS;
    const int tiles = (N + 15) >> 4;
    const int groups = (tiles + TPW - 1) / TPW;
    const int K = 32 * C;

    for (int grp = blockIdx.x; grp < groups; grp += gridDim.x) {
        const int tile = grp * TPW + wave / SPLIT;
        const int sub = wave % SPLIT;
        const u32x4* wrow = wq + (size_t)min(tile * 16 + col, N - 1) * C;
        i32x4 acc = {0, 0, 0, 0};
        for (int c0 = 0; c0 < C; c0 += SEGC) {
            const int nc = min(SEGC, C - c0);
            const int nq = (nc + 3) >> 2;
            const int q0 = sub * nq / SPLIT, q1 = (sub + 1) * nq / SPLIT;
            u32x4 cur[U];
            load_quads<U>(cur, wrow, c0, nc, q0, q1, g);  // overlaps the staging
            __syncthreads();                              // readers of the last segment are done
            const int nh = 2 * nc;                        // 16-code halves per token
            for (int i0 = threadIdx.x; i0 < M * nh; i0 += kStageBatch * NT) {
                u32x4 v[kStageBatch];                     // all loads in flight, then the stores
#pragma unroll
                for (int j = 0; j < kStageBatch; ++j) {
                    const int i = i0 + j * NT;
                    v[j] = u32x4{0u, 0u, 0u, 0u};
                    if (i < M * nh)
                        v[j] = reinterpret_cast<const u32x4*>(qx + (size_t)(i / nh) * K)[2 * c0 + i % nh];
                }
#pragma unroll
                for (int j = 0; j < kStageBatch; ++j) {
                    const int i = i0 + j * NT;
                    if (i < M * nh)
                        xs[(i / nh) * TS + i % nh] = u32x4{perm_even(v[j].x, v[j].y), perm_odd(v[j].x, v[j].y),
                                                           perm_even(v[j].z, v[j].w), perm_odd(v[j].z, v[j].w)};
                }
            }
            __syncthreads();
            for (int q = q0; q < q1; q += U) {
                u32x4 nxt[U];
                const bool more = q + U < q1;  // uniform across the wave
                if (more)
                    load_quads<U>(nxt, wrow, c0, nc, q + U, q1, g);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (q + u < q1) {
                        const int c = min(4 * (q + u) + g, nc - 1);
                        u32x4 xa = xs[xrow + 2 * c], xb = xs[xrow + 2 * c + 1];
                        if (!tok)
                            xa = xb = u32x4{0u, 0u, 0u, 0u};
                        acc = mfma_chunk(cur[u], xa, xb, acc);
                    }
                }
                if (more) {
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        cur[u] = nxt[u];
                }
            }
        }
        if (SPLIT > 1) {  // waves wave - sub .. wave - sub + SPLIT - 1 share a tile
            part[wave][lane] = acc;
            __syncthreads();
            if (sub == 0) {
#pragma unroll
                for (int s2 = 1; s2 < SPLIT; ++s2)
                    acc += part[wave + s2][lane];
            }
            __syncthreads();
        }
        if (sub == 0 && tok) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = tile * 16 + 4 * g + e;
                if (row < N) {
                    const int a = acc[e] >> 4;
                    if (acc_out)
                        acc_out[(size_t)col * N + row] = a;
                    y[(size_t)col * N + row] = fmaf(sw[row] * sx[col], (float)a, bias ? bias[row] : 0.0f);
                }
            }
        }
    }
}

// ------------------------------------------------------------------------
// Verify on the matrix cores in balanced blocks.  The tiles x K work (16-row
// tiles; a "quad" is 4 chunks = 128 codes of a tile, one pair of MFMAs) is
// cut into one block per workgroup: a range of tiles times a K slice, all
// blocks holding about the same number of quads.  A workgroup stages only
// its slice's codes of the M tokens (issued before its weight loads, so they
// do not queue behind them), its 16 waves split the block's 4-quad groups
// into contiguous runs, one group's weight loads in flight per wave, and
// each wave adds its exact int32 partials into per-tile LDS accumulators.
// With one K slice the workgroup owns its tiles and writes y directly.
// With several, each block counts in on its tiles as it starts (the count's
// round trip overlaps its staging and MFMAs); the block that counted in
// last on a tile gathers it: it loads the other slices' partials, adds its
// own (integers: the order does not matter), writes y and clears the
// tile's count and the partials, so the whole workspace is zero again for
// the next call, of any shape.  The others store their partials and leave.
// A gatherer only waits for blocks that have already counted in, hence
// started; the blocks of a tile group walk the tiles' words in the same
// order, and at each word one block waits for what the others store at that
// same word, so every wait ends without any assumption about which blocks
// are resident together.
// ------------------------------------------------------------------------
constexpr int kVbWaves = 16;
constexpr int kVbThreads = kVbWaves * kWave;
constexpr int kVbMaxTiles = 16;             // tiles per block (LDS accumulators)
constexpr int kVbGroups = 1;                // 4-quad groups a wave has in flight: with more, the later waves'
                                            // staging loads queue behind them (16 tokens, [3584, 18944] /
                                            // [18944, 3584]: 3 groups 15.3 / 14.1 us, 2 15.0 / 13.9, 1 13.9 / 12.9)
constexpr int kVbQ = 4 * kVbGroups;         // their registers (one quad each)
constexpr int kVbStage = 8;                 // staging loads per thread per batch
constexpr int kVbXsBytes = 112 * 1024;      // LDS for the staged codes
constexpr int kVbCountWords = 64;           // tile counts are padded to 256 bytes
constexpr int kVbSpinLimit = 1 << 20;       // polls of one partial word (its store is already issued)
constexpr int kVbSplitCost = 600;           // fixed charge of a K split in vb_plan, sixths of a quad
static_assert(kVbStage * kVbThreads * 16 >= kVbXsBytes, "one staging batch holds a whole slice");

// Weights stream in groups: a group is one tile's 16 rows times 16 chunks
// (256 bytes of each row, 4 quads), read by 4 loads of 4 rows x 256
// contiguous bytes each (load p, lane l: row 4p + l / 16, chunk l % 16):
// a 16-lane quarter of a load covers two whole 128-byte lines, where the
// matrix cores' own operand order (16 rows x 64 bytes per load) touches 16
// half lines.  Measured at [3584, 18944], 16 tokens, 3 groups in flight:
// 16.2 us in operand order, 15.3 us in row order with the transpose below.
// Slots past ue, rows past the matrix and chunks past the slice load at an
// offset past the resource: zeros, no memory access.  The loads are
// non-temporal (read once; 16 tokens: 14.0 / 12.8 -> 13.5 / 12.2 us at
// [3584, 18944] / [18944, 3584]).  wr covers this block's tiles' rows
// (16-byte chunks, row pitch C).
__device__ __forceinline__ void vb_load(u32x4 (&buf)[kVbQ], __amdgpu_buffer_rsrc_t wr, int u0, int ue, int qg,
                                        int nrows, int C, int c0, int nc, int lane)
{
#pragma unroll
    for (int h = 0; h < kVbGroups; ++h) {
        const int u = u0 + h;
        const int lt = u / qg, c = 16 * (u - lt * qg) + (lane & 15);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = lt * 16 + 4 * p + (lane >> 4);
            const int off = u < ue && row < nrows && c < nc ? 16 * (row * C + c0 + c) : kBufferPast;
            buf[4 * h + p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, kNonTemporal));
        }
    }
}

// Exchange between registers a and b across lane distance D (4 or 8, inside
// a 16-lane row): lanes with bit D set take b from D lanes below into a,
// lanes with it clear take a from D lanes above into b.
template <int D>
__device__ __forceinline__ void vb_xchg(uint32_t& a, uint32_t& b, bool hi)
{
    constexpr int kHi = D == 4 ? 0xA : 0xC, kLo = D == 4 ? 0x5 : 0x3;  // banks with / without lane bit D
    const uint32_t na = (uint32_t)__builtin_amdgcn_update_dpp((int)a, (int)b, 0x110 | D, 0xF, kHi, false);
    const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp((int)b, (int)a, 0x100 | D, 0xF, kLo, false);
    a = na;
    b = nb;
}

// A group from its load order (register p, lane l: row 4p + l / 16, chunk
// l % 16) into the matrix cores' (register t, lane 16g + i: row i, chunk
// 4t + g).  With the index bits written out, a load's element sits at
// register (r2 r3), lane (c0 c1 c2 c3 r0 r1) and must go to register
// (c2 c3), lane (r0 r1 r2 r3 c0 c1): a lane permutation swapping lane bits
// 0,1 with 4,5, then register bit 0 exchanged with lane bit 2 and register
// bit 1 with lane bit 3.  The lane permutation goes through the wave's own
// LDS scratch (each register written in lane order and read back permuted:
// two 16-byte LDS accesses per lane, where ds_bpermute takes four 4-byte
// ones and measured slower); the exchanges are DPP row shifts whose bank
// masks pick the lanes (lane bits 2 and 3 select 4-lane banks).
constexpr int kVbScratch = 68;  // 16-byte slots per wave: 4 rows of 16 lanes, each + 1 against bank conflicts
static_assert(kVbXsBytes + kVbMaxTiles * 256 * 4 + kVbWaves * kVbScratch * 16 + kVbMaxTiles * 4 <= kLdsMaxBytes,
              "verify LDS: staged codes, tile sums, transpose scratch");

__device__ __forceinline__ int vb_slot(int l)
{
    return 17 * (l >> 4) + (l & 15);
}

__device__ __forceinline__ void vb_transpose(u32x4& w0, u32x4& w1, u32x4& w2, u32x4& w3, u32x4* sc, int rd, int lane)
{
    // sc: this wave's scratch; rd: this lane's read slot (its source lane's write slot)
    const int wr = vb_slot(lane);
    sc[wr] = w0;
    w0 = sc[rd];
    sc[wr] = w1;
    w1 = sc[rd];
    sc[wr] = w2;
    w2 = sc[rd];
    sc[wr] = w3;
    w3 = sc[rd];
    uint32_t v[4][4] = {{w0.x, w0.y, w0.z, w0.w}, {w1.x, w1.y, w1.z, w1.w},
                        {w2.x, w2.y, w2.z, w2.w}, {w3.x, w3.y, w3.z, w3.w}};
    const bool b2 = (lane >> 2) & 1, b3 = (lane >> 3) & 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        vb_xchg<4>(v[0][e], v[1][e], b2);
        vb_xchg<4>(v[2][e], v[3][e], b2);
        vb_xchg<8>(v[0][e], v[2][e], b3);
        vb_xchg<8>(v[1][e], v[3][e], b3);
    }
    w0 = u32x4{v[0][0], v[0][1], v[0][2], v[0][3]};
    w1 = u32x4{v[1][0], v[1][1], v[1][2], v[1][3]};
    w2 = u32x4{v[2][0], v[2][1], v[2][2], v[2][3]};
    w3 = u32x4{v[3][0], v[3][1], v[3][2], v[3][3]};
}

__global__ __launch_bounds__(kVbThreads) void k_verify_blocks(
    const u32x4* __restrict__ wq, const float* __restrict__ sw, const float* __restrict__ bias,
    const int8_t* __restrict__ qx, const float* __restrict__ sx, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int M, int N, int C, int ksplit, int kslice, int ntg,
    uint32_t* __restrict__ ws)
{
    extern __shared__ u32x4 xs[];  // token m's slice chunk c: xs[m * TS + 2c], [.. + 1]
    __shared__ int32_t tacc[kVbMaxTiles * 256];  // [tile][row 16][token 16]
    __shared__ uint32_t s_last[kVbMaxTiles];
    __shared__ u32x4 vbt[kVbWaves * kVbScratch];  // the waves' transpose scratch
    const int T = (N + 15) >> 4;
    const int ks = blockIdx.x % ksplit, tg = blockIdx.x / ksplit;
    const int t0 = (int)((long long)tg * T / ntg), nt = (int)((long long)(tg + 1) * T / ntg) - t0;
    const int c0 = ks * kslice, nc = min(kslice, C - c0);
    if (nt <= 0 || nc <= 0)
        return;  // uniform: a block with no tiles contributes to none
    const int qg = (nc + 15) >> 4;  // 4-quad groups per tile in this slice
    const int total = nt * qg;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int g = lane >> 4, col = lane & 15;
    const bool tok = col < M;
    const int TS = 2 * kslice + 1;
    const int nh = 2 * nc, items = M * nh;
    const u32x4* qv = reinterpret_cast<const u32x4*>(qx);
    const int K2 = 2 * C;  // 16-byte halves per token row
    // 0. with a split, count in on this block's tiles; the old count is
    //    first used after the MFMAs, when wave 0's loads have all landed
    uint32_t* cnt = ws;
    uint32_t cnt_old = 0;
    if (ksplit > 1 && wave == 0 && lane < nt)
        cnt_old = __hip_atomic_fetch_add(&cnt[t0 + lane], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // 1. the staging loads (one batch holds the whole slice), ahead of the weights
    u32x4 sv[kVbStage];
#pragma unroll
    for (int j = 0; j < kVbStage; ++j) {
        const int i = min(tid + j * kVbThreads, items - 1);
        sv[j] = qv[(size_t)(i / nh) * K2 + 2 * c0 + i % nh];
    }
    for (int i = tid; i < nt * 256; i += kVbThreads)
        tacc[i] = 0;
    // 2. this wave's run of groups [ga, gb): the first kVbGroups of them in flight
    const int ga = (int)((long long)wave * total / kVbWaves), gb = (int)((long long)(wave + 1) * total / kVbWaves);
    const int nrows = min(nt * 16, N - t0 * 16);
    const __amdgpu_buffer_rsrc_t wr = uniform_rsrc(wq + (size_t)t0 * 16 * C, nrows * C * 16);
    u32x4 wb[kVbQ];
    vb_load(wb, wr, ga, min(gb, ga + kVbGroups), qg, nrows, C, c0, nc, lane);
    // 3. staged codes into LDS, permuted for the unpacked weight halves
#pragma unroll
    for (int j = 0; j < kVbStage; ++j) {
        const int i = tid + j * kVbThreads;
        if (i < items)
            xs[(i / nh) * TS + i % nh] = u32x4{perm_even(sv[j].x, sv[j].y), perm_odd(sv[j].x, sv[j].y),
                                               perm_even(sv[j].z, sv[j].w), perm_odd(sv[j].z, sv[j].w)};
    }
    __syncthreads();
    // 4. the MFMAs; a change of tile flushes the wave's partial into LDS
    i32x4 acc = {0, 0, 0, 0};
    int cur = -1;
    const int xrow = col * TS;
    u32x4* const sc = vbt + kVbScratch * wave;
    const int rd = vb_slot(((lane & 3) << 4) | ((lane >> 4) & 3) | (lane & 12));  // lane bits 0,1 <-> 4,5
    for (int u0 = ga; u0 < gb; u0 += kVbGroups) {
#pragma unroll
        for (int h = 0; h < kVbGroups; ++h) {
            const int u = u0 + h;
            if (u < gb) {  // uniform across the wave
                vb_transpose(wb[4 * h], wb[4 * h + 1], wb[4 * h + 2], wb[4 * h + 3], sc, rd, lane);
                const int lt = u / qg, cg = 16 * (u - lt * qg);
                if (lt != cur) {
                    if (cur >= 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            __hip_atomic_fetch_add(&tacc[cur * 256 + (4 * g + e) * 16 + col], acc[e],
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    }
                    acc = i32x4{0, 0, 0, 0};
                    cur = lt;
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int c = cg + 4 * t + g;
                    u32x4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
                    if (tok && c < nc) {
                        xa = xs[xrow + 2 * c];
                        xb = xs[xrow + 2 * c + 1];
                    }
                    acc = mfma_chunk(wb[4 * h + t], xa, xb, acc);
                }
            }
        }
        if (u0 + kVbGroups < gb)  // the run's next groups
            vb_load(wb, wr, u0 + kVbGroups, min(gb, u0 + 2 * kVbGroups), qg, nrows, C, c0, nc, lane);
    }
    if (cur >= 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            __hip_atomic_fetch_add(&tacc[cur * 256 + (4 * g + e) * 16 + col], acc[e], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (ksplit > 1 && wave == 0 && lane < nt) {
        const bool last = cnt_old == (uint32_t)(ksplit - 1);
        if (last)  // every slice of the tile has counted in: ready for the next call
            __hip_atomic_store(&cnt[t0 + lane], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last[lane] = last;
    }
    __syncthreads();
    // 5. outputs
    if (ksplit == 1) {
        for (int i = tid; i < nt * 256; i += kVbThreads) {
            const int row = (t0 + (i >> 8)) * 16 + ((i >> 4) & 15), m = i & 15;
            if (row < N && m < M) {
                const int a = tacc[i] >> 4;
                if (acc_out)
                    acc_out[(size_t)m * N + row] = a;
                y[(size_t)m * N + row] = fmaf(sw[row] * sx[m], (float)a, bias ? bias[row] : 0.0f);
            }
        }
        return;
    }
    // Each partial word goes out as one 64-bit atomic store {1, value}: its
    // high half says it is there, so no store needs to be ordered before
    // another and no fence is needed.  The gatherer loads each other slice's
    // word until its high half is set, then clears it.  (Loading all slices'
    // words at once, and those not there yet again together, was measured
    // slower: the gatherer mostly waits for the slowest other slice, and
    // one word at a time finds the later slices' words already there.)
    uint64_t* part = reinterpret_cast<uint64_t*>(ws + (((size_t)T + kVbCountWords - 1) / kVbCountWords) * kVbCountWords);
    for (int i = tid; i < nt * 256; i += kVbThreads) {
        const int lt = i >> 8;  // uniform across the wave
        if (!s_last[lt]) {
            __hip_atomic_store(&part[((size_t)ks * T + t0 + lt) * 256 + (i & 255)], (1ull << 32) | (uint32_t)tacc[i],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        int s = tacc[i];
        for (int k = 0; k < ksplit; ++k) {
            if (k == ks)
                continue;
            uint64_t* pp = &part[((size_t)k * T + t0 + lt) * 256 + (i & 255)];
            uint64_t v = __hip_atomic_load(pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int spin = 0; (v >> 32) == 0 && spin < kVbSpinLimit; ++spin) {
                __builtin_amdgcn_s_sleep(1);
                v = __hip_atomic_load(pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            s += (int32_t)(uint32_t)v;
            __hip_atomic_store(pp, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const int row = (t0 + lt) * 16 + ((i >> 4) & 15), m = i & 15;
        if (row < N && m < M) {
            const int a = s >> 4;
            if (acc_out)
                acc_out[(size_t)m * N + row] = a;
            y[(size_t)m * N + row] = fmaf(sw[row] * sx[m], (float)a, bias ? bias[row] : 0.0f);
        }
    }
}

// ------------------------------------------------------------------------
// Persistent token pass: every linear of a decode step in one launch, one
// 1024-thread workgroup per CU, all resident at once.
//
// Dependencies travel with the data.  When linear t reads an output of an
// earlier linear k of the same pass (a decoder's chain: each GEMV's input is
// derived from the previous GEMV's output), it does not read k's output
// buffer: every row k's workgroups compute is also stored into an exchange
// array in the synchronisation workspace, as the bitwise NOT of its fp32
// bits, with a relaxed device-scope atomic store, and an exchange word holds
// 0 until its row has been written in this pass.  Linear t's workgroups load
// the words of their activation with device-scope loads and load again the
// ones still 0.  Each word is an atomic object that carries its own value,
// so nothing relies on the order in which stores to different locations
// become visible: no fences, no store-completion waits, no counters.  The
// chain from a writer's store to a reader's use is one store and one load.
// Two exchange sets alternate between passes (epoch parity): the writer of a
// row also stores 0 to that row in the other set, which the previous pass
// used and this pass never reads, so a set is all zero when its pass starts
// (consecutive passes are ordered by the kernel boundary).  An activation
// written before the launch is read through the caches, with no wait.
//
// The weights depend on nothing, so when a workgroup finishes its share of
// a linear its worker waves issue the loads of the first step of their
// share of the next one; they stream from HBM while the activation is
// awaited and quantised.
//   Work split: workgroup w owns a contiguous, balanced range of rows of
//   every linear; its lane groups (2^lshift lanes per row, r rows per group)
//   take the range in batches; a lane streams its rows in steps of 8
//   16-byte chunks, double-buffered in registers.  Shapes are chosen and
//   encoded on the host for the grid the launch uses (checked in the kernel).
//   Workspace (32-bit words): err at 0; epoch[w] at 64 + 16 w (w < 1024,
//   one 64-byte line each); exchange set s at kXchBase + s * xch_words.
//   Each workgroup writes its epoch word once per pass, so all of them hold
//   the same value e between passes; a pass runs as epoch e + 1 and uses
//   exchange set (e + 1) & 1.  A wait that exceeds its spin limit sets err
//   bit 0 and proceeds, so every wave always reaches the end of the kernel;
//   descriptors for another grid or another n set bit 1 and the kernel
//   returns at once, as do descriptors whose exchange does not fit the
//   workspace the launch was given.
// ------------------------------------------------------------------------
struct PassHeader {
    int32_t n, grid, max_k, xch_words;  // xch_words: 32-bit words per exchange set
    int32_t slots;                      // chunks per lane per step: the kernel instance (k_decode_pass<slots>)
    int32_t pad[3];
};
static_assert(sizeof(PassHeader) == 32, "descriptor header layout");

struct PassTask {
    const u32x4* wq;
    const void* scales;             // float s^W [N] (kind 0) or fp16 group scales [N, C] (kind 1)
    const float* bias;
    const void* x;                  // activation written before the launch (xin < 0)
    float* y;
    int32_t N, C;                   // rows; 16-byte chunks per row (K / 32)
    int32_t rows_base, rows_extra;  // workgroup w owns rows_base + (w < rows_extra) rows
    int32_t lshift, r;              // 2^lshift lanes per row; r rows per lane group
    int32_t iters, batches;         // chunk iterations per row per lane; row batches
    int32_t steps;                  // pipeline steps per batch
    int32_t xin;                    // exchange word of x[0] (x is an output of the pass), or -1
    int32_t xout;                   // exchange word of y[0] (a later linear reads y), or -1
    int32_t x_dtype;                // X_F32 or X_F16 (xin < 0)
    int32_t kind;                   // 0: per-row fp32 scales; 1: one fp16 scale per 32 weights
    int32_t reserved;
};
static_assert(sizeof(PassTask) == 96, "descriptor layout");

constexpr int kPassThreads = 1024;    // 16 waves: one workgroup per CU
// Waves 0..11 stream weights; waves 12..15 stage the activation.  The
// staging waves never hold weight loads: vmcnt completes in order, so an
// activation load issued behind a wave's own prefetch could not be used
// until that prefetch had landed.
constexpr int kPassWorkers = 768;
constexpr int kPassControl = kPassThreads - kPassWorkers;
constexpr int kPassSlots = 8;         // 16-byte chunks per lane per pipeline step
// Passes whose linears are all group-32 (small per-CU shares: 6-37 KB in the
// Gemma-shaped stream) run an instance with 4: a step's fixed work (the
// predicated loads, the register copy) sits on every small linear's
// critical path (Gemma-shaped pass 0.65 against 0.71 ms); per-row passes
// keep 8 (4 there: 1.06 against 1.00 ms, the large linears stream slower).
constexpr int kPassSlotsSmall = 4;
constexpr int kPassMaxGrid = 1024;
constexpr int kPassSpinLimit = 1 << 21;
constexpr int kPassWgPerCu = 1;
constexpr int kPassMaxK = BQD_MAX_PASS_K;  // LDS: codes (K bytes) + fp32 activation (4K bytes)
static_assert(5 * kPassMaxK <= 160 * 1024, "pass activation must fit LDS");
// Workspace layout (32-bit words).
constexpr int kEpochBase = 64;        // after err's 256-byte line
constexpr int kSyncStride = 16;       // one 64-byte line per epoch word
constexpr int kXchBase = kEpochBase + kPassMaxGrid * kSyncStride;  // 16448 words = 65792 bytes
// 8-value groups a staging thread loads at once (all issued before the first
// use): 3 covers K = 3584 on the 4 staging waves and K = 18944 on all 16 in
// one round and holds fewer registers than 4 (Gemma-shaped pass 0.733 ->
// 0.725 ms, Qwen2-7B-shaped unchanged; 2 needs a second round at K = 18944).
constexpr int kStageGroups = 3;

inline size_t pass_lds_bytes(int max_k) { return (size_t)((max_k + 15) & ~15) + 4 * (size_t)max_k; }

// Descriptors are read from a ring in LDS, not with scalar loads: a scalar
// load misses the scalar cache once per linear and per CU in every pass,
// and LDS waits (lgkmcnt) also wait for scalar loads, so its latency would
// land on each linear's staging.  The ring holds kDescRing descriptors;
// the staging waves refill half of it every kDescRing / 2 linears.
constexpr int kDescRing = 64;
// A group-32 linear's scales for this workgroup's rows, staged in LDS.
constexpr int kPassScaleLds = 16384;
static_assert(kPassScaleLds % (16 * 256) == 0, "scale block: whole registers per staging thread");
constexpr int kDescWords = (int)(sizeof(PassTask) / 4);
static_assert(sizeof(PassTask) % 4 == 0, "descriptor words");
static_assert(5 * kPassMaxK + kDescRing * (int)sizeof(PassTask) + kPassScaleLds + 1024 <= 160 * 1024, "pass LDS");

// Copies descriptors [lo, hi) into their ring slots, threads t, t + nt, ...
__device__ __forceinline__ void ring_fill(uint32_t* dring, const PassTask* tasks, int lo, int hi, int t, int nt)
{
    const BQD_GLOBAL uint32_t* src = gptr(reinterpret_cast<const uint32_t*>(tasks));
    for (int i = t; i < (hi - lo) * kDescWords; i += nt) {
        const int d = lo + i / kDescWords, k = i % kDescWords;
        dring[(d % kDescRing) * kDescWords + k] = src[(size_t)d * kDescWords + k];
    }
}

// Descriptor i from the ring, every field wave-uniform (scalar registers).
__device__ __forceinline__ PassTask ring_get(const uint32_t* dring, int i)
{
    uint32_t w[kDescWords];
    const uint32_t* d = dring + (i % kDescRing) * kDescWords;
#pragma unroll
    for (int k = 0; k < kDescWords; ++k)
        w[k] = __builtin_amdgcn_readfirstlane(d[k]);
    PassTask t;
    __builtin_memcpy(&t, w, sizeof t);
    return t;
}

__device__ __forceinline__ void pass_range(const PassTask& t, int w, int& row_start, int& rows)
{
    rows = t.rows_base + (w < t.rows_extra ? 1 : 0);
    row_start = w * t.rows_base + (w < t.rows_extra ? w : t.rows_extra);
}

// Streamed once: non-temporal, so weights do not push the activation out of L2.
__device__ __forceinline__ u32x4 ld_stream(const BQD_GLOBAL u32x4* p)
{
    return __builtin_nontemporal_load(p);
}

// Loads step j of row batch b into buf; with the first step of a batch, lane
// rr of each lane group also loads the scale and bias of the group's row rr
// (the epilogue's operands arrive with the weights, not after them).
template <int R, int S>
__device__ __forceinline__ void pass_load(u32x4 (&buf)[S], float& esw, float& eb, const PassTask& t,
                                          int row_start, int rows, int b, int j)
{
    constexpr int U = S / R;
    const int L = 1 << t.lshift;
    const int lane = threadIdx.x & (L - 1);
    const int groups = kPassWorkers >> t.lshift;
    const int grp = threadIdx.x >> t.lshift;
    const BQD_GLOBAL u32x4* wrow[R];
    bool vr[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int rl = (b * groups + grp) * R + rr;
        vr[rr] = rl < rows;
        wrow[rr] = gptr(t.wq) + (size_t)(row_start + (vr[rr] ? rl : 0)) * t.C;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (j * U + u) * L + lane;
        const bool ok = c < t.C;
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
            buf[u * R + rr] = (ok && vr[rr]) ? ld_stream(wrow[rr] + c) : u32x4{0u, 0u, 0u, 0u};
    }
    if (j == 0) {
        const int rl = (b * groups + grp) * R + lane;
        const bool own = lane < R && rl < rows;
        esw = (own && t.kind == 0) ? gptr(reinterpret_cast<const float*>(t.scales))[row_start + rl] : 0.0f;
        eb = (own && t.bias) ? gptr(t.bias)[row_start + rl] : 0.0f;
    }
}

// One linear's share of this workgroup: batches of rows, each streamed in
// steps with the next step's loads in flight during the current step.  Each
// row's y goes to the output buffer and, when a later linear of the pass
// reads it, to the exchange (xcur) as ~bits, with the same row of the other
// set (xold) cleared for the next pass.
template <int R, int S>
__device__ __forceinline__ void pass_run(u32x4 (&cur)[S], float& esw, float& eb, bool have_cur,
                                         const PassTask& t, int row_start, int rows, const u32x4* xs, float sx,
                                         uint32_t* xcur, uint32_t* xold)
{
    constexpr int U = S / R;
    const int L = 1 << t.lshift;
    const int lane = threadIdx.x & (L - 1);
    const int groups = kPassWorkers >> t.lshift;
    const int grp = threadIdx.x >> t.lshift;
    if (!have_cur)
        pass_load<R, S>(cur, esw, eb, t, row_start, rows, 0, 0);
    float nsw = 0.0f, nbv = 0.0f;  // next batch's epilogue operands
    for (int b = 0; b < t.batches; ++b) {
        int acc[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
            acc[rr] = 0;
        for (int j = 0; j < t.steps; ++j) {
            u32x4 nxt[S];
            int nb = b, nj = j + 1;
            if (nj == t.steps) {
                nb = b + 1;
                nj = 0;
            }
            const bool more = nb < t.batches;
            if (more)
                pass_load<R, S>(nxt, nsw, nbv, t, row_start, rows, nb, nj);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = j * U + u;
                if (i < t.iters) {  // uniform across the wave
                    const int c = min(i * L + lane, t.C - 1);
                    const u32x4 xa = xs[2 * c], xb = xs[2 * c + 1];
#pragma unroll
                    for (int rr = 0; rr < R; ++rr)
                        acc[rr] = dot_chunk16(cur[u * R + rr], xa, xb, acc[rr]);
                }
            }
            if (more) {
#pragma unroll
                for (int k = 0; k < S; ++k)
                    cur[k] = nxt[k];
            }
        }
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            int v = acc[rr] >> 4;
            v += dpp_i<0x128>(v);
            v += dpp_i<0x124>(v);
            v += dpp_i<0x122>(v);
            v += dpp_i<0x121>(v);
            if (L >= 32)
                v += __shfl_xor(v, 16);
            if (L >= 64)
                v += __shfl_xor(v, 32);
            const int rl = (b * groups + grp) * R + rr;
            if (lane == rr && rl < rows) {
                const float yv = fmaf(esw * sx, (float)v, eb);
                const int row = row_start + rl;
                gptr_mut(t.y)[row] = yv;
                if (t.xout >= 0) {
                    __hip_atomic_store(gptr_mut(xcur) + t.xout + row, ~__builtin_bit_cast(uint32_t, yv),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(gptr_mut(xold) + t.xout + row, 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        esw = nsw;
        eb = nbv;
    }
}

// A group-32 linear ("在香橙派上跑 Gemma4 ..." section 3.1: INT4 with one fp16
// scale per 32 weights): per 16-byte chunk the exact int32 partial acc_g
// times its scale s_g, accumulated in fp32 in the lane's chunk order, the
// lanes' sums added by the same DPP and shuffle tree, and y = s^x sum + b:
// the arithmetic and order, hence the bits, of k_gemv_w4a8_g32 at 32
// lanes per row (the encoder fixes 32 lanes and one row per lane group).
// sl holds the workgroup's rows' scales, staged in LDS.
template <int S>
__device__ __forceinline__ void pass_run_g32(u32x4 (&cur)[S], float& esw, float& eb, bool have_cur,
                                             const PassTask& t, int row_start, int rows, const u32x4* xs, float sx,
                                             const uint16_t* sl, uint32_t* xcur, uint32_t* xold)
{
    constexpr int L = 32;
    const int lane = threadIdx.x & (L - 1);
    const int groups = kPassWorkers / L;
    const int grp = threadIdx.x / L;
    if (!have_cur)
        pass_load<1, S>(cur, esw, eb, t, row_start, rows, 0, 0);
    float nsw = 0.0f, nbv = 0.0f;
    for (int b = 0; b < t.batches; ++b) {
        const int rl = b * groups + grp;
        const uint16_t* srow = sl + (size_t)min(rl, rows - 1) * t.C;
        float facc = 0.0f;
        for (int j = 0; j < t.steps; ++j) {
            u32x4 nxt[S];
            int nb = b, nj = j + 1;
            if (nj == t.steps) {
                nb = b + 1;
                nj = 0;
            }
            const bool more = nb < t.batches;
            if (more)
                pass_load<1, S>(nxt, nsw, nbv, t, row_start, rows, nb, nj);
#pragma unroll
            for (int u = 0; u < S; ++u) {
                const int i = j * S + u;
                if (i < t.iters) {  // uniform across the wave
                    const int c = min(i * L + lane, t.C - 1);
                    const int ag = dot_chunk16(cur[u], xs[2 * c], xs[2 * c + 1], 0) >> 4;
                    const float sg = (float)__builtin_bit_cast(_Float16, srow[c]);
                    facc = fmaf((float)ag, sg, facc);
                }
            }
            if (more) {
#pragma unroll
                for (int k = 0; k < S; ++k)
                    cur[k] = nxt[k];
            }
        }
        facc = sum_lanes_f<L>(facc);
        if (lane == 0 && rl < rows) {
            const float yv = fmaf(sx, facc, eb);
            const int row = row_start + rl;
            gptr_mut(t.y)[row] = yv;
            if (t.xout >= 0) {
                __hip_atomic_store(gptr_mut(xcur) + t.xout + row, ~__builtin_bit_cast(uint32_t, yv),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(gptr_mut(xold) + t.xout + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        esw = nsw;
        eb = nbv;
    }
}

// Activation staging, phase 1, by `nst` threads (index st): x is read once
// from memory into LDS as fp32 (xf; fp16 widens exactly) and max |x| is
// reduced per thread.  Each thread loads up to kStageGroups of its 8-value
// groups at once.
//
// From the exchange (XCH): words of rows not yet written in this pass are 0;
// they are loaded again (device scope, sc1: coherent with the writers'
// device-scope stores on every XCD, where a plain load could be served a
// stale line by this CU's L1 or this XCD's L2) until none is left.  A word
// is a relaxed atomic load: every 32-bit word of an aligned 16-byte load is
// read single-copy atomically.  After spin_limit rounds the wait gives up,
// sets err bit 0 and takes the words as they are; so does every wait of a
// workgroup that finds bit 0 already set.
__device__ __forceinline__ bool written8(u32x4 a, u32x4 b)
{
    return a.x && a.y && a.z && a.w && b.x && b.y && b.z && b.w;
}

template <int XIN, bool XCH>
__device__ __forceinline__ float stage_load(const void* x, f32x4* xf, int G8, int st, int nst, uint32_t* err,
                                            int spin_limit)
{
    constexpr int kGroupBytes = XIN == X_F16 ? 16 : 32;
    const __amdgpu_buffer_rsrc_t r = uniform_rsrc(x, G8 * kGroupBytes);
    float amax = 0.0f;
    for (int g0 = st; g0 < G8; g0 += kStageGroups * nst) {
        u32x4 v[kStageGroups][2];
        uint32_t todo = 0;
#pragma unroll
        for (int k = 0; k < kStageGroups; ++k) {
            const int g = g0 + k * nst;
            v[k][0] = v[k][1] = u32x4{0u, 0u, 0u, 0u};
            if (g < G8) {
                todo |= 1u << k;
                if constexpr (XCH) {
                    v[k][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 32 * g, 0, kDeviceScope));
                    v[k][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 32 * g + 16, 0, kDeviceScope));
                } else if constexpr (XIN == X_F32) {
                    v[k][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 32 * g, 0, 0));
                    v[k][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 32 * g + 16, 0, 0));
                } else {
                    v[k][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * g, 0, 0));
                }
            }
        }
        if constexpr (XCH) {
            int spins = 0;
            while (true) {
                uint32_t left = 0;
#pragma unroll
                for (int k = 0; k < kStageGroups; ++k)
                    if (((todo >> k) & 1u) && !written8(v[k][0], v[k][1]))
                        left |= 1u << k;
                if (!left)
                    break;
                ++spins;
                if (spins >= spin_limit ||
                    ((spins & 255) == 0 && (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1u))) {
                    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
#pragma unroll
                for (int k = 0; k < kStageGroups; ++k) {
                    if ((left >> k) & 1u) {
                        const int g = g0 + k * nst;
                        v[k][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 32 * g, 0, kDeviceScope));
                        v[k][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 32 * g + 16, 0, kDeviceScope));
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kStageGroups; ++k) {
            if ((todo >> k) & 1u) {
                const int g = g0 + k * nst;
                float u[8];
                if constexpr (XIN == X_F32) {
                    // whole-vector casts: a bit cast of one ext-vector
                    // element (a.y) was compiled as a read of element 0
                    const f32x4 a = __builtin_bit_cast(f32x4, XCH ? ~v[k][0] : v[k][0]);
                    const f32x4 b = __builtin_bit_cast(f32x4, XCH ? ~v[k][1] : v[k][1]);
                    u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w;
                    u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
                } else {
                    const uint32_t hw[4] = {v[k][0].x, v[k][0].y, v[k][0].z, v[k][0].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        u[2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hw[e] & 0xFFFFu));
                        u[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hw[e] >> 16));
                    }
                }
                xf[2 * g] = f32x4{u[0], u[1], u[2], u[3]};
                xf[2 * g + 1] = f32x4{u[4], u[5], u[6], u[7]};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    amax = fmaxf(amax, fabsf(u[e]));
            }
        }
    }
    return amax;
}

// Phase 2: the permuted codes from the fp32 values in LDS.
__device__ __forceinline__ void stage_codes(u32x2* xs, const f32x4* xf, int G8, int st, int nst,
                                            const ActScale& a)
{
    for (int g = st; g < G8; g += nst) {
        const f32x4 p = xf[2 * g], q = xf[2 * g + 1];
        const float u[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
        uint32_t lo, hi;
        quant8_fast(u, a, lo, hi);
        xs[g] = u32x2{perm_even(lo, hi), perm_odd(lo, hi)};
    }
}

// Above this many 8-value groups (K > 4096) every wave stages; below, only
// the staging waves, which hold no weight loads.  (From K > 8192 before:
// the Gemma-shaped pass, whose down projection has K = 6144, 0.747 -> 0.731
// ms per token; the Qwen2-7B-shaped one, K = 3584 or 18944, unchanged.)
constexpr int kPassStageAllAbove = 512;

template <int R, int S>
__device__ __forceinline__ void pass_prefetch(u32x4 (&cur)[S], float& esw, float& eb, const PassTask& t,
                                              int w)
{
    int row_start, rows;
    pass_range(t, w, row_start, rows);
    if (rows > 0)
        pass_load<R, S>(cur, esw, eb, t, row_start, rows, 0, 0);
}

template <int S>
__global__ __launch_bounds__(kPassThreads) void k_decode_pass(const PassHeader* __restrict__ hdr,
                                                              const PassTask* __restrict__ tasks, int n_launch,
                                                              int max_k_launch, uint32_t* __restrict__ sync,
                                                              size_t sync_words, int spin_limit)
{
    extern __shared__ u32x4 xs[];  // codes: max_k bytes, then fp32 x at xf_offset
    const int xf_offset = (hdr->max_k + 15) & ~15;
    __shared__ float red[2][kPassThreads / kWave];
    __shared__ uint32_t s_epoch;
    __shared__ uint32_t dring[kDescRing * kDescWords];
    __shared__ u32x4 sl16[kPassScaleLds / 16];  // group-32 scales of this workgroup's rows
    const int n = hdr->n;
    const int G = gridDim.x;
    const int w = blockIdx.x;
    const int tid = threadIdx.x;
    const bool worker = tid < kPassWorkers;  // uniform per wave
    const int ct = tid - kPassWorkers;       // staging-thread index (>= 0 on the staging waves)
    uint32_t* err = sync;
    uint32_t* epochs = sync + kEpochBase;    // epochs[w * kSyncStride]
    if (hdr->grid != G || n != n_launch || hdr->max_k != max_k_launch || hdr->slots != S || G > kPassMaxGrid ||
        (size_t)kXchBase + 2 * (size_t)(uint32_t)hdr->xch_words > sync_words) {
        // uniform: every workgroup leaves
        if (tid == 0 && w == 0)
            __hip_atomic_fetch_or(err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    // Every workgroup writes its epoch word once per pass, so all of them
    // hold the same value between passes: this pass writes that value + 1.
    if (tid == 0)
        s_epoch = __hip_atomic_load(&epochs[(size_t)w * kSyncStride], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    ring_fill(dring, tasks, 0, n < kDescRing ? n : kDescRing, tid, kPassThreads);
    __syncthreads();
    const uint32_t epoch = s_epoch;
    const size_t xw = (size_t)(uint32_t)hdr->xch_words;
    uint32_t* xcur = sync + kXchBase + (epoch & 1u) * xw;
    uint32_t* xold = sync + kXchBase + ((epoch & 1u) ^ 1u) * xw;

    u32x4 cur[S];
    float esw = 0.0f, eb = 0.0f;  // first batch's epilogue operands, loaded with cur
    PassTask t = ring_get(dring, 0);
    bool have_cur = false;
    if (worker) {
        int rs, rw;
        pass_range(t, w, rs, rw);
        if (rw > 0) {
            if (t.r == 2)
                pass_prefetch<2, S>(cur, esw, eb, t, w);
            else
                pass_prefetch<1, S>(cur, esw, eb, t, w);
            have_cur = true;
        }
    }
    f32x4* xf = reinterpret_cast<f32x4*>(reinterpret_cast<char*>(xs) + xf_offset);
    for (int ti = 0; ti < n; ++ti) {
        if (ti > 0 && ti % (kDescRing / 2) == 0 && ct >= 0)
            ring_fill(dring, tasks, ti + kDescRing / 2, min(n, ti + kDescRing), ct, kPassControl);
        const PassTask tn = ring_get(dring, ti + 1 < n ? ti + 1 : ti);
        int row_start, rows;
        pass_range(t, w, row_start, rows);
        const int G8 = 4 * t.C;
        float* rd = red[ti & 1];
        // 1. the activation into LDS (fp32) and max |x|: staging waves, or
        //    every wave for long activations
        const bool all_stage = G8 > kPassStageAllAbove;
        const int st = all_stage ? tid : ct;
        const int nst = all_stage ? kPassThreads : kPassControl;
        // this workgroup's rows' group scales: rows * C fp16 values,
        // contiguous and 16-byte aligned (C % 8 == 0, checked on the host),
        // copied straight into LDS (no registers) ahead of the activation's
        // loads, so the two overlap; the staging waves wait for every load
        // before the barrier that hands the scales to the workers
        if (t.kind == 1 && rows > 0 && ct >= 0) {
            const int nsc = rows * t.C / 8;
            const BQD_GLOBAL u32x4* src =
                gptr(reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(t.scales) + (size_t)row_start * t.C));
            // The lane number is made inside the loop (v_mbcnt, nothing
            // loaded): hoisted out of it, the per-lane values were among the
            // kernel's spills, and their scratch reloads joined the CU's
            // memory queue behind the weight prefetch at the start of every
            // group-32 linear (Gemma-shaped pass 0.723 -> 0.707 ms; the
            // kernel now keeps no value in scratch).
            for (int base = __builtin_amdgcn_readfirstlane(ct) & ~(kWave - 1); base < nsc; base += kPassControl) {
                int ln;
                asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
                if (base + ln < nsc)
                    __builtin_amdgcn_global_load_lds(const_cast<BQD_GLOBAL u32x4*>(src + base + ln),
                                                     (BQD_LDS void*)(sl16 + base), 16, 0, 0);
            }
        }
        if (rows > 0 && st >= 0) {
            float m;
            if (t.xin >= 0)
                m = stage_load<X_F32, true>(xcur + t.xin, xf, G8, st, nst, err, spin_limit);
            else if (t.x_dtype == X_F16)
                m = stage_load<X_F16, false>(t.x, xf, G8, st, nst, err, spin_limit);
            else
                m = stage_load<X_F32, false>(t.x, xf, G8, st, nst, err, spin_limit);
            m = wave_max_dpp(m);
            if ((st & (kWave - 1)) == 0)
                rd[st / kWave] = m;
        }
        if (t.kind == 1 && rows > 0 && ct >= 0)
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the scale copies are in LDS
        __syncthreads();
        float amax = rd[0];
        const int nw = all_stage ? kPassThreads / kWave : kPassControl / kWave;
        for (int i = 1; i < nw; ++i)
            amax = fmaxf(amax, rd[i]);
        const ActScale a = act_scale(amax);
        // 2. codes into LDS
        if (rows > 0)
            stage_codes(reinterpret_cast<u32x2*>(xs), xf, G8, tid, kPassThreads, a);
        __syncthreads();
        // 3. workers: stream the weights, write the rows
        if (rows > 0 && worker) {
            if (t.kind == 1)
                pass_run_g32<S>(cur, esw, eb, have_cur, t, row_start, rows, xs, a.s,
                             reinterpret_cast<const uint16_t*>(sl16), xcur, xold);
            else if (t.r == 2)
                pass_run<2, S>(cur, esw, eb, have_cur, t, row_start, rows, xs, a.s, xcur, xold);
            else
                pass_run<1, S>(cur, esw, eb, have_cur, t, row_start, rows, xs, a.s, xcur, xold);
        }
        // 4. workers prefetch ti+1
        have_cur = false;
        if (worker && ti + 1 < n) {
            int rs, rw;
            pass_range(tn, w, rs, rw);
            if (rw > 0) {
                if (tn.r == 2)
                    pass_prefetch<2, S>(cur, esw, eb, tn, w);
                else
                    pass_prefetch<1, S>(cur, esw, eb, tn, w);
                have_cur = true;
            }
        }
        // The next activation is staged after this workgroup's share of ti:
        // its LDS is free, and the staging waves poll only once the
        // workgroup has nothing else to do.
        __syncthreads();
        t = tn;
    }
    if (tid == 0)
        __hip_atomic_store(&epochs[(size_t)w * kSyncStride], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------
// Streaming-read reference: the measured read ceiling the GEMV rooflines are
// set against.  Each thread reads 16-byte words in a grid-stride loop, U in
// flight, and folds them with XOR; one word per workgroup is written so no
// load is dead.
// ------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(kThreads) void k_read_probe(const u32x4* __restrict__ p, long long n, uint32_t* out)
{
    uint32_t a = 0;
    const long long stride = (long long)gridDim.x * kThreads;
    long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u)
            a ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const u32x4 v = p[i];
        a ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    a ^= __shfl_xor(a, 1);
    if (threadIdx.x == 0)
        out[blockIdx.x] = a;
}

// ------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 rejected
int g_dev_cus[kMaxDevices];
std::mutex g_dev_mutex;

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline int current_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 256;
    return g_dev_cus[dev] > 0 ? g_dev_cus[dev] : 256;
}

inline int launched()
{
    return hipGetLastError() == hipSuccess ? BQD_OK : BQD_ERR_LAUNCH;
}

inline int check_k(int K, int mult = 32)
{
    if (K <= 0 || K % mult)
        return BQD_ERR_SHAPE;
    if (K > BQD_MAX_K)
        return BQD_ERR_BOUND;
    return BQD_OK;
}

// The entry points with a general path (gemv_w4a8, linear_w4a8,
// quantize_act, gemm_w4a8_verify) take any K % 8 == 0 up to the int32 bound;
// the fast kernels take K % 32 == 0 up to BQD_MAX_K.
inline int check_k_any(int K)
{
    if (K <= 0 || K % 8)
        return BQD_ERR_SHAPE;
    if (K > BQD_MAX_K_ANY)
        return BQD_ERR_BOUND;
    return BQD_OK;
}
inline bool fast_k(int K) { return K % 32 == 0 && K <= BQD_MAX_K; }

// Launch of the general-K GEMV (rows in a grid-stride loop).
template <int XIN>
int launch_gemv_any(const uint32_t* wq, const float* sw, const float* bias, const void* x, const float* sx,
                    float* y, int32_t* acc, int8_t* qx_out, float* sx_out, int N, int K, hipStream_t st)
{
    const long long tiles = ((long long)N + kAnyRows - 1) / kAnyRows;
    const long long cap = (long long)current_cus() * 8;
    hipLaunchKernelGGL(k_gemv_w4a8_any<XIN>, dim3((unsigned)(tiles < cap ? tiles : cap)), dim3(kThreads), 0, st, wq,
                       sw, bias, x, sx, y, acc, qx_out, sx_out, N, K);
    return launched();
}

// Launch shape of a GEMV: r rows per lane group, L lanes per row, U chunk
// iterations per pipeline step, and the number of workgroups.
struct GemvCfg {
    int r, L, U, grid;
};

constexpr int kWgPerCu = 8;  // grid cap: workgroups per CU in the grid-stride loop

inline int pow2ceil(int v)
{
    int p = 1;
    while (p < v)
        p <<= 1;
    return p;
}

// Largest U for r rows: R*U 16-byte loads are double-buffered in VGPRs.
inline int max_unroll(int r) { return r >= 8 ? 2 : (r >= 4 ? 4 : 8); }

inline bool valid_config(int r, int L)
{
    return (r == 0 || r == 1 || r == 2 || r == 4 || r == 8) && (L == 0 || L == 16 || L == 32 || L == 64);
}

// Automatic choice where the caller passes 0 (measured on MI355X in the
// decode streams, one graph-replayed launch per linear): 32 lanes per row;
// one row per lane group, except r_large rows from 8192 rows on (per-row
// INT4: 1 -- the Qwen-shaped stream takes 1.42 ms per token with 1 and
// 1.51 ms with 2; group-32: 2, which the Gemma-shaped stream prefers).  U
// covers a lane's whole row when it fits the register budget.
// Chunks per lane of the wide kernel's instances (the smallest that covers C / 64 is launched).
#define BQD_WIDE_CASES(X) X(1) X(2) X(3) X(4) X(6) X(8) X(10) X(12)

inline GemvCfg make_cfg(int N, int C, int r, int L, int r_large)
{
    GemvCfg c;
    c.L = L ? L : 32;
    c.r = r ? r : (N >= 8192 ? r_large : 1);
    const int iters = (C + c.L - 1) / c.L;
    c.U = pow2ceil(iters) < max_unroll(c.r) ? pow2ceil(iters) : max_unroll(c.r);
    const long long rows = (long long)(kThreads / c.L) * c.r;
    const long long tiles = (N + rows - 1) / rows;
    const long long cap = (long long)current_cus() * kWgPerCu;
    c.grid = (int)(tiles < cap ? tiles : cap);
    return c;
}

inline unsigned grid_for(long long tiles)
{
    const long long cap = 1LL << 30;
    return (unsigned)(tiles < cap ? tiles : cap);
}

// Every (R, L, U) instance: R*U <= 16 loads per step.
#define BQD_FOR_CFGS_L(X, LL)                                                                     \
    X(1, LL, 1) X(1, LL, 2) X(1, LL, 4) X(1, LL, 8) X(2, LL, 1) X(2, LL, 2) X(2, LL, 4) X(2, LL, 8) \
    X(4, LL, 1) X(4, LL, 2) X(4, LL, 4) X(8, LL, 1) X(8, LL, 2)
#define BQD_FOR_CFGS(X) BQD_FOR_CFGS_L(X, 16) BQD_FOR_CFGS_L(X, 32) BQD_FOR_CFGS_L(X, 64)

template <int XIN>
int launch_gemv_rowwise(const uint32_t* wq, const float* sw, const float* bias, const void* xin,
                        const float* sx, float* y, int32_t* acc, int8_t* qx_out, float* sx_out,
                        int N, int K, const GemvCfg& c, hipStream_t st, const RmsIn& rms = RmsIn{})
{
    const int C = K / 32;
    const dim3 grid(c.grid), block(kThreads);
    const size_t lds = (size_t)K;
    const u32x4* w = reinterpret_cast<const u32x4*>(wq);
#define BQD_GEMV_CASE(RR, LL, UU)                                                                \
    if (c.r == RR && c.L == LL && c.U == UU) {                                                   \
        hipLaunchKernelGGL((k_gemv_w4a8<RR, LL, UU, XIN>), grid, block, lds, st, w, sw, bias, xin, \
                           sx, y, acc, qx_out, sx_out, N, C, rms);                               \
        return launched();                                                                       \
    }
    BQD_FOR_CFGS(BQD_GEMV_CASE)
#undef BQD_GEMV_CASE
    return BQD_ERR_CONFIG;
}

template <int XIN>
int launch_gemv_group32(const uint32_t* wq, const uint16_t* s16, const float* bias, const void* xin,
                        const float* sx, float* y, int32_t* accg, int8_t* qx_out, float* sx_out,
                        int N, int K, const GemvCfg& c, hipStream_t st)
{
    const int C = K / 32;
    const dim3 grid(c.grid), block(kThreads);
    const size_t lds = (size_t)K;
    const u32x4* w = reinterpret_cast<const u32x4*>(wq);
#define BQD_G32_CASE(RR, LL, UU)                                                                    \
    if (c.r == RR && c.L == LL && c.U == UU) {                                                      \
        hipLaunchKernelGGL((k_gemv_w4a8_g32<RR, LL, UU, XIN>), grid, block, lds, st, w, s16, bias,    \
                           xin, sx, y, accg, qx_out, sx_out, N, C);                                 \
        return launched();                                                                          \
    }
    BQD_FOR_CFGS(BQD_G32_CASE)
#undef BQD_G32_CASE
    return BQD_ERR_CONFIG;
}

int check_x_dtype(int d) { return (d == BQD_F32 || d == BQD_F16) ? BQD_OK : BQD_ERR_DTYPE; }

}  // namespace

// Workspace of decode_pass_w4a8_static, for callers that cannot allocate
// device memory: one copy per GPU, held until the process ends.  Host code
// never uses this name as an address (on the host it is a stand-in); it
// uses the device address bqd_init looked up for the current GPU.
static __device__ __align__(256) uint32_t scratch[BQD_STATIC_PASS_BYTES / 4];

namespace {

uint32_t* g_scratch[kMaxDevices];  // device address of `scratch` on each GPU, or NULL

// Zero-fills n 16-byte words (graph-capture safe, unlike hipMemsetAsync).
__global__ __launch_bounds__(kThreads) void k_zero16(u32x4* p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

// The pass's error word, copied out to the caller's buffer.
__global__ void k_copy_word(const uint32_t* src, uint32_t* dst)
{
    if (threadIdx.x == 0)
        *dst = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// ==========================================================================
// C ABI
// ==========================================================================
extern "C" {

int bqd_abi_version(void) { return BQD_ABI_VERSION; }

const char* bqd_status_string(int status)
{
    switch (status) {
    case BQD_OK: return "ok";
    case BQD_ERR_NULL: return "a required pointer is NULL";
    case BQD_ERR_SHAPE: return "bad shape: N/M < 0, K <= 0 or K not a multiple of 32, or bad count";
    case BQD_ERR_ALIGN: return "a pointer is not aligned as required";
    case BQD_ERR_BOUND: return "K above BQD_MAX_K or token count above BQD_MAX_TOKENS";
    case BQD_ERR_DTYPE: return "unknown dtype or scale kind";
    case BQD_ERR_CONFIG: return "unsupported r / lanes_per_row";
    case BQD_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case BQD_ERR_DEVICE: return "no HIP device, or the current device is not a gfx950";
    default: return "unknown status";
    }
}

int bqd_init(void)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return BQD_ERR_DEVICE;
    int s = g_dev_state[dev].load(std::memory_order_acquire);
    if (s == 1)
        return BQD_OK;
    if (s == -1)
        return BQD_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    s = g_dev_state[dev].load(std::memory_order_relaxed);
    if (s == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
            s = -1;
        } else {
            s = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
            g_dev_cus[dev] = p.multiProcessorCount;
            // This device's copy of the static workspace (its address
            // differs per GPU); NULL if the lookup fails, which only
            // decode_pass_w4a8_static reports.
            void* ptr = nullptr;
            if (s == 1 && hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess)
                g_scratch[dev] = static_cast<uint32_t*>(ptr);
            else
                (void)hipGetLastError();
        }
        g_dev_state[dev].store(s, std::memory_order_release);
    }
    return s == 1 ? BQD_OK : BQD_ERR_DEVICE;
}

int quantize_weights_int4_rowwise(const float* W, int32_t N, int32_t K, uint32_t* wq, float* sw,
                                  void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K);
    if (rc)
        return rc;
    if (N == 0)
        return BQD_OK;
    if (!W || !wq || !sw)
        return BQD_ERR_NULL;
    if (!aligned(W, 16) || !aligned(wq, 16) || !aligned(sw, 4))
        return BQD_ERR_ALIGN;
    if ((rc = bqd_init()))
        return rc;
    const int rows_per_block = kThreads / kWave;
    hipLaunchKernelGGL(k_quantize_weights_int4_rowwise, dim3((N + rows_per_block - 1) / rows_per_block),
                       dim3(kThreads), 0, (hipStream_t)stream, W, N, K, wq, sw);
    return launched();
}

static int quantize_group32_common(bool int8, const float* W, int32_t N, int32_t K, void* out,
                                   uint16_t* s16, void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K);
    if (rc)
        return rc;
    if (N == 0)
        return BQD_OK;
    if (!W || !out || !s16)
        return BQD_ERR_NULL;
    if (!aligned(W, 16) || !aligned(out, 16) || !aligned(s16, 2))
        return BQD_ERR_ALIGN;
    if ((rc = bqd_init()))
        return rc;
    const long long n = (long long)N * (K / 32);
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    if (int8)
        hipLaunchKernelGGL(k_quantize_weights_group32<true>, grid, dim3(kThreads), 0, (hipStream_t)stream,
                           W, N, K, out, s16);
    else
        hipLaunchKernelGGL(k_quantize_weights_group32<false>, grid, dim3(kThreads), 0, (hipStream_t)stream,
                           W, N, K, out, s16);
    return launched();
}

int quantize_weights_int4_group32(const float* W, int32_t N, int32_t K, uint32_t* wq, uint16_t* s16,
                                  void* stream)
{
    return quantize_group32_common(false, W, N, K, wq, s16, stream);
}

int quantize_weights_int8_group32(const float* W, int32_t N, int32_t K, int8_t* w8, uint16_t* s16,
                                  void* stream)
{
    return quantize_group32_common(true, W, N, K, w8, s16, stream);
}

int int8x_counts_host(const int8_t* q, int64_t n, int64_t* counts)
{
    if (!q || !counts)
        return BQD_ERR_NULL;
    if (n <= 0)
        return BQD_ERR_SHAPE;
    int64_t c[3] = {0, 0, 0};
    for (int64_t t = 0; t < n; ++t) {
        const int a = q[t] < 0 ? -(int)q[t] : (int)q[t];
        c[(a > 3) + (a > 15)]++;
    }
    counts[0] = c[0];
    counts[1] = c[1];
    counts[2] = c[2];
    return BQD_OK;
}

int int8x_stream_bytes_host(int64_t n, const int64_t* counts, int64_t* bytes)
{
    if (!counts || !bytes)
        return BQD_ERR_NULL;
    if (n <= 0 || counts[0] < 0 || counts[1] < 0 || counts[2] < 0 || counts[0] + counts[1] + counts[2] != n)
        return BQD_ERR_SHAPE;
    auto words = [](int64_t bits) { return (bits + 31) / 32 + 3; };  // + padding for the read windows
    const int64_t blocks = (n + kInt8xBlock - 1) / kInt8xBlock;
    bytes[0] = 4 * words(n);                            // b1
    bytes[1] = 4 * words(counts[1] + counts[2]);        // b2
    bytes[2] = 4 * words(3 * counts[0]);                // l1
    bytes[3] = 4 * words(5 * counts[1]);                // l2
    bytes[4] = 4 * words(8 * counts[2]);                // l3
    bytes[5] = 4 * (blocks + 1);                        // b1_blk
    bytes[6] = 4 * (blocks + 1);                        // b2_blk
    return BQD_OK;
}

// Bit writer over a zeroed word stream, LSB-first.
struct BitSink {
    uint32_t* w;
    int64_t pos = 0;
    void put(uint32_t v, int width)
    {
        v &= (1u << width) - 1u;
        const int64_t i = pos >> 5;
        const int off = (int)(pos & 31);
        w[i] |= v << off;
        if (off + width > 32)
            w[i + 1] |= v >> (32 - off);
        pos += width;
    }
};

int int8x_encode_host(const int8_t* q, int64_t n, uint32_t* b1, uint32_t* b2, uint32_t* l1, uint32_t* l2,
                      uint8_t* l3, int32_t* b1_blk, int32_t* b2_blk)
{
    if (!q || !b1 || !b2 || !l1 || !l2 || !l3 || !b1_blk || !b2_blk)
        return BQD_ERR_NULL;
    int64_t counts[3], bytes[7];
    int rc = int8x_counts_host(q, n, counts);
    if (rc || (rc = int8x_stream_bytes_host(n, counts, bytes)))
        return rc;
    if (counts[1] + counts[2] > INT32_MAX)
        return BQD_ERR_BOUND;
    std::memset(b1, 0, bytes[0]);
    std::memset(b2, 0, bytes[1]);
    std::memset(l1, 0, bytes[2]);
    std::memset(l2, 0, bytes[3]);
    std::memset(l3, 0, bytes[4]);
    BitSink s1{l1}, s2{l2}, sb2{b2};
    int64_t n3 = 0;
    for (int64_t t = 0; t < n; ++t) {
        if (t % kInt8xBlock == 0) {
            b1_blk[t / kInt8xBlock] = (int32_t)sb2.pos;  // non-level-1 weights so far
            b2_blk[t / kInt8xBlock] = (int32_t)n3;
        }
        const int v = q[t];
        const int a = v < 0 ? -v : v;
        if (a <= 3) {
            s1.put((uint32_t)v, 3);
            continue;
        }
        b1[t >> 5] |= 1u << (t & 31);
        if (a <= 15) {
            sb2.put(0u, 1);
            s2.put((uint32_t)v, 5);
        } else {
            sb2.put(1u, 1);
            l3[n3++] = (uint8_t)v;
        }
    }
    const int64_t blocks = (n + kInt8xBlock - 1) / kInt8xBlock;
    b1_blk[blocks] = (int32_t)sb2.pos;
    b2_blk[blocks] = (int32_t)n3;
    return BQD_OK;
}

int gemv_int8x(const uint32_t* b1, const uint32_t* b2, const uint32_t* l1, const uint32_t* l2, const uint8_t* l3,
               const int32_t* b1_blk, const int32_t* b2_blk, const int64_t* stream_bytes, const int8_t* qx,
               const float* sx, float sw, float* y, int32_t* acc, int32_t N, int32_t K, int32_t rows,
               void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K, kInt8xBlock);
    if (rc)
        return rc;
    if (K > BQD_MAX_K)
        return BQD_ERR_BOUND;
    if (N == 0)
        return BQD_OK;
    if (!b1 || !b2 || !l1 || !l2 || !l3 || !b1_blk || !b2_blk || !stream_bytes || !qx || !sx || !y)
        return BQD_ERR_NULL;
    if (!aligned(b1, 4) || !aligned(b2, 4) || !aligned(l1, 4) || !aligned(l2, 4) || !aligned(l3, 4) ||
        !aligned(qx, 8) || !aligned(y, 4) || !aligned(acc, 4))
        return BQD_ERR_ALIGN;
    for (int i = 1; i < 5; ++i)  // three words at least (the encoder's padding)
        if (stream_bytes[i] < 12 || stream_bytes[i] % 4)
            return BQD_ERR_SHAPE;
    // bit positions are int32 in the kernel: every stream below 2^26 words
    if ((int64_t)N * K >= ((int64_t)1 << 31))
        return BQD_ERR_BOUND;
    for (int i = 1; i < 5; ++i)
        if (stream_bytes[i] / 4 > ((int64_t)1 << 26))
            return BQD_ERR_BOUND;
    if (stream_bytes[0] < 4 * (((int64_t)N * K + 31) / 32) ||
        stream_bytes[5] < 4 * ((int64_t)N * K / kInt8xBlock + 1) ||
        stream_bytes[6] < 4 * ((int64_t)N * K / kInt8xBlock + 1))
        return BQD_ERR_SHAPE;
    if (rows != 0 && rows != 1 && rows != 2 && rows != 4 && rows != 8)
        return BQD_ERR_CONFIG;
    // automatic: one row per workgroup keeps enough waves in flight for short
    // matrices (measured: [3584, 18944] 69 us with 1, 103 with 4); 4 from 8192 rows
    const int R = rows ? rows : (N >= 8192 ? 4 : 1);
    if ((rc = bqd_init()))
        return rc;
    Int8xStreams st{b1, b2, l1, l2, reinterpret_cast<const uint32_t*>(l3), b1_blk, b2_blk,
                    (int)(stream_bytes[1] / 4), (int)(stream_bytes[2] / 4), (int)(stream_bytes[3] / 4),
                    (int)(stream_bytes[4] / 4)};
    const dim3 grid((N + R - 1) / R), block(kThreads);
    hipStream_t sm = (hipStream_t)stream;
#define BQD_I8X_CASE(RR)                                                                              \
    if (R == RR) {                                                                                    \
        hipLaunchKernelGGL(k_gemv_int8x<RR>, grid, block, 0, sm, st, qx, sx, sw, y, acc, N, K);       \
        return launched();                                                                            \
    }
    BQD_I8X_CASE(1) BQD_I8X_CASE(2) BQD_I8X_CASE(4) BQD_I8X_CASE(8)
#undef BQD_I8X_CASE
    return BQD_ERR_CONFIG;
}

int pack_int4_rows_host(const int8_t* q, int32_t N, int32_t K, uint32_t* out)
{
    if (!q || !out)
        return BQD_ERR_NULL;
    if (N < 0 || K <= 0 || K % 8)
        return BQD_ERR_SHAPE;
    const size_t n = (size_t)N * (size_t)K;
    for (size_t i = 0; i < n; ++i)
        if (q[i] < -8 || q[i] > 7)
            return BQD_ERR_SHAPE;
    for (size_t t = 0; t < n / 8; ++t) {
        uint32_t w = 0;
        for (int k = 0; k < 8; ++k)
            w |= ((uint32_t)(uint8_t)q[8 * t + k] & 0xFu) << (4 * k);
        out[t] = w;
    }
    return BQD_OK;
}

int unpack_int4_rows_host(const uint32_t* w, int32_t N, int32_t K, int8_t* out)
{
    if (!w || !out)
        return BQD_ERR_NULL;
    if (N < 0 || K <= 0 || K % 8)
        return BQD_ERR_SHAPE;
    const size_t words = (size_t)N * (size_t)K / 8;
    for (size_t t = 0; t < words; ++t)
        for (int k = 0; k < 8; ++k) {
            // sign-extend the nibble: shift it to the top of a 32-bit int, then back
            const int32_t v = (int32_t)(w[t] << (28 - 4 * k)) >> 28;
            out[8 * t + k] = (int8_t)v;
        }
    return BQD_OK;
}

inline int prod_items(int K);

static bool bytes_overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

// One buffer of a launch: address and bytes (NULL or empty: absent).
struct Span {
    const void* p;
    size_t n;
};

// True when an output overlaps anything the launch reads or another output.
// Every workgroup of these kernels reads the activation (and its own rows'
// weights) while other workgroups already write outputs, so an overlap
// would make the results depend on timing.
static bool io_overlap(std::initializer_list<Span> ins, std::initializer_list<Span> outs)
{
    for (const Span* o = outs.begin(); o != outs.end(); ++o) {
        if (!o->p || !o->n)
            continue;
        for (const Span& i : ins)
            if (i.p && i.n && bytes_overlap(o->p, o->n, i.p, i.n))
                return true;
        for (const Span* o2 = o + 1; o2 != outs.end(); ++o2)
            if (o2->p && o2->n && bytes_overlap(o->p, o->n, o2->p, o2->n))
                return true;
    }
    return false;
}

int quantize_act(const void* x, int32_t x_dtype, int32_t M, int32_t K, int8_t* qx, float* sx,
                 void* stream)
{
    int rc = check_x_dtype(x_dtype);
    if (rc)
        return rc;
    if (M < 0)
        return BQD_ERR_SHAPE;
    if ((rc = check_k_any(K)))
        return rc;
    if (M == 0)
        return BQD_OK;
    if (!x || !qx || !sx)
        return BQD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(qx, 16) || !aligned(sx, 4))
        return BQD_ERR_ALIGN;
    if (io_overlap({{x, (size_t)M * K * (x_dtype == BQD_F32 ? 4 : 2)}}, {{qx, (size_t)M * K}, {sx, 4 * (size_t)M}}))
        return BQD_ERR_SHAPE;
    if ((rc = bqd_init()))
        return rc;
    if (x_dtype == BQD_F32 && K % 32 == 0 && K <= BQD_MAX_PROD_K && M <= 65535) {
        // fp32 tokens up to 32768 values: the producers' quantiser, ceil(K/4096)
        // workgroups of 1024 threads per token, each holding the whole token in
        // registers (one memory round trip; K = 18944: 8.7 -> ~3 us), the
        // same codes and scale.
        const dim3 grid((K / 4 + kProdThreads - 1) / kProdThreads, M);
        const float* xf = static_cast<const float*>(x);
#define BQD_QACT_CASE(IT)                                                                                        \
        if (prod_items(K) == IT) {                                                                               \
            hipLaunchKernelGGL(k_quantize_rows<IT>, grid, dim3(kProdThreads), 0, (hipStream_t)stream, xf, K, qx, sx); \
            return launched();                                                                                   \
        }
        BQD_QACT_CASE(1) BQD_QACT_CASE(2) BQD_QACT_CASE(4) BQD_QACT_CASE(8)
#undef BQD_QACT_CASE
    }
    if (x_dtype == BQD_F32)
        hipLaunchKernelGGL(k_quantize_act<X_F32>, dim3(M), dim3(kThreads), 0, (hipStream_t)stream, x, K, qx, sx);
    else
        hipLaunchKernelGGL(k_quantize_act<X_F16>, dim3(M), dim3(kThreads), 0, (hipStream_t)stream, x, K, qx, sx);
    return launched();
}

// Items of 4 values per thread of a 1024-thread workgroup covering K values.
inline int prod_items(int K)
{
    const int per = (K / 4 + kProdThreads - 1) / kProdThreads;
    return per <= 1 ? 1 : (per <= 2 ? 2 : (per <= 4 ? 4 : 8));
}

int add_rmsnorm_quant(const float* h, const float* delta, const float* gamma, float eps, float* h_out,
                      float* y_out, int8_t* qx, float* sx, int32_t M, int32_t K, void* stream)
{
    if (M < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K);
    if (rc)
        return rc;
    if (K > kProdMaxK)
        return BQD_ERR_BOUND;
    if (!(eps >= 0.0f) || !(eps <= FLT_MAX))
        return BQD_ERR_SHAPE;
    if (M == 0)
        return BQD_OK;
    if (!h || !gamma || (qx && !sx))
        return BQD_ERR_NULL;
    if (!aligned(h, 16) || !aligned(delta, 16) || !aligned(gamma, 16) || !aligned(h_out, 16) ||
        !aligned(y_out, 16) || !aligned(qx, 16) || !aligned(sx, 4))
        return BQD_ERR_ALIGN;
    {
        // h_out and y_out may each be h or delta itself (every element is read
        // by the thread that later writes it), never a shifted view of them.
        const size_t tb = 4 * (size_t)M * K;
        const auto same_or_apart = [tb](const void* o, const void* i) {
            return !o || !i || o == i || !bytes_overlap(o, tb, i, tb);
        };
        if (!same_or_apart(h_out, h) || !same_or_apart(h_out, delta) || !same_or_apart(y_out, h) ||
            !same_or_apart(y_out, delta))
            return BQD_ERR_SHAPE;
        if (io_overlap({{gamma, 4 * (size_t)K}}, {{h_out, tb}, {y_out, tb}}) ||
            io_overlap({{h, tb}, {delta, tb}, {gamma, 4 * (size_t)K}, {h_out, tb}, {y_out, tb}},
                       {{qx, (size_t)M * K}, {sx, 4 * (size_t)M}}))
            return BQD_ERR_SHAPE;
    }
    if ((rc = bqd_init()))
        return rc;
    hipStream_t st = (hipStream_t)stream;
#define BQD_RMS_CASE(IT)                                                                                  \
    if (prod_items(K) == IT) {                                                                            \
        hipLaunchKernelGGL(k_add_rmsnorm_quant<IT>, dim3(M), dim3(kProdThreads), 0, st, h, delta, gamma, eps, \
                           K, h_out, y_out, qx, sx);                                                     \
        return launched();                                                                                \
    }
    BQD_RMS_CASE(1) BQD_RMS_CASE(2) BQD_RMS_CASE(4) BQD_RMS_CASE(8)
#undef BQD_RMS_CASE
    return BQD_ERR_CONFIG;
}

int swiglu_quant(const float* gu, float* h_out, int8_t* qx, float* sx, int32_t M, int32_t I, void* stream)
{
    if (M < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(I);
    if (rc)
        return rc;
    if (I > kProdMaxK)
        return BQD_ERR_BOUND;
    if (M == 0)
        return BQD_OK;
    if (!gu || !h_out || (qx && !sx))
        return BQD_ERR_NULL;
    if (!aligned(gu, 16) || !aligned(h_out, 16) || !aligned(qx, 16) || !aligned(sx, 4))
        return BQD_ERR_ALIGN;
    if (io_overlap({{gu, 8 * (size_t)M * I}}, {{h_out, 4 * (size_t)M * I}, {qx, (size_t)M * I}, {sx, 4 * (size_t)M}}))
        return BQD_ERR_SHAPE;
    if ((rc = bqd_init()))
        return rc;
    hipStream_t st = (hipStream_t)stream;
    const int I4 = I / 4;
    hipLaunchKernelGGL(k_swiglu, dim3((I4 + kThreads - 1) / kThreads, M), dim3(kThreads), 0, st, gu, I, h_out);
    if ((rc = launched()) || !qx)
        return rc;
    const dim3 grid((I4 + kProdThreads - 1) / kProdThreads, M);
#define BQD_QROWS_CASE(IT)                                                                              \
    if (prod_items(I) == IT) {                                                                          \
        hipLaunchKernelGGL(k_quantize_rows<IT>, grid, dim3(kProdThreads), 0, st, h_out, I, qx, sx);     \
        return launched();                                                                              \
    }
    BQD_QROWS_CASE(1) BQD_QROWS_CASE(2) BQD_QROWS_CASE(4) BQD_QROWS_CASE(8)
#undef BQD_QROWS_CASE
    return BQD_ERR_CONFIG;
}

int gemv_w4a8(const uint32_t* wq, const float* sw, const float* bias, const int8_t* qx,
              const float* sx, float* y, int32_t* acc, int32_t N, int32_t K, int32_t r,
              int32_t lanes_per_row, void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k_any(K);
    if (rc)
        return rc;
    if (!valid_config(r, lanes_per_row))
        return BQD_ERR_CONFIG;
    if (N == 0)
        return BQD_OK;
    if (!wq || !sw || !qx || !sx || !y)
        return BQD_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(qx, 16) || !aligned(sw, 4) || !aligned(sx, 4) ||
        !aligned(y, 4) || !aligned(bias, 4) || !aligned(acc, 4))
        return BQD_ERR_ALIGN;
    if (io_overlap({{wq, (size_t)N * K / 2}, {sw, 4 * (size_t)N}, {bias, 4 * (size_t)N}, {qx, (size_t)K}, {sx, 4}},
                   {{y, 4 * (size_t)N}, {acc, 4 * (size_t)N}}))
        return BQD_ERR_SHAPE;
    if ((rc = bqd_init()))
        return rc;
    if (!fast_k(K))
        return launch_gemv_any<X_Q8>(wq, sw, bias, qx, sx, y, acc, nullptr, nullptr, N, K, (hipStream_t)stream);
    if (r == 0 && lanes_per_row == 0 && N <= kWideMaxN && K <= kWideMaxKQ8) {
        // wide workgroups, as for linear_w4a8
        const int C = K / 32, U = (C + kWave - 1) / kWave;
        constexpr int rows = kWideThreads / kWave;
        const dim3 grid((N + rows - 1) / rows), block(kWideThreads);
        const u32x4* w = reinterpret_cast<const u32x4*>(wq);
#define BQD_WIDE_Q8_CASE(UU)                                                                               \
        if (U <= UU) {                                                                                     \
            hipLaunchKernelGGL((k_linear_wide<UU, X_Q8, kWideThreads>), grid, block, (size_t)K, (hipStream_t)stream, w, sw, \
                               bias, qx, sx, y, acc, nullptr, nullptr, N, C);                              \
            return launched();                                                                             \
        }
        BQD_WIDE_Q8_CASE(1) BQD_WIDE_Q8_CASE(2) BQD_WIDE_Q8_CASE(3) BQD_WIDE_Q8_CASE(4)
#undef BQD_WIDE_Q8_CASE
    }
    return launch_gemv_rowwise<X_Q8>(wq, sw, bias, qx, sx, y, acc, nullptr, nullptr, N, K,
                                     make_cfg(N, K / 32, r, lanes_per_row, 1), (hipStream_t)stream);
}

int linear_w4a8(const uint32_t* wq, const float* sw, const float* bias, const void* x,
                int32_t x_dtype, float* y, int8_t* qx_out, float* sx_out, int32_t* acc, int32_t N,
                int32_t K, int32_t r, int32_t lanes_per_row, void* stream)
{
    int rc = check_x_dtype(x_dtype);
    if (rc)
        return rc;
    if (N < 0)
        return BQD_ERR_SHAPE;
    if ((rc = check_k_any(K)))
        return rc;
    if (N == 0)
        return BQD_OK;
    if (!wq || !sw || !x || !y)
        return BQD_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(x, 16) || !aligned(qx_out, 16) || !aligned(sw, 4) ||
        !aligned(sx_out, 4) || !aligned(y, 4) || !aligned(bias, 4) || !aligned(acc, 4))
        return BQD_ERR_ALIGN;
    if (!valid_config(r, lanes_per_row))
        return BQD_ERR_CONFIG;
    if (io_overlap({{wq, (size_t)N * K / 2}, {sw, 4 * (size_t)N}, {bias, 4 * (size_t)N},
                    {x, (size_t)K * (x_dtype == BQD_F32 ? 4 : 2)}},
                   {{y, 4 * (size_t)N}, {qx_out, (size_t)K}, {sx_out, 4}, {acc, 4 * (size_t)N}}))
        return BQD_ERR_SHAPE;
    if ((rc = bqd_init()))
        return rc;
    if (!fast_k(K)) {
        if (x_dtype == BQD_F32)
            return launch_gemv_any<X_F32>(wq, sw, bias, x, nullptr, y, acc, qx_out, sx_out, N, K, (hipStream_t)stream);
        return launch_gemv_any<X_F16>(wq, sw, bias, x, nullptr, y, acc, qx_out, sx_out, N, K, (hipStream_t)stream);
    }
    if (r == 0 && lanes_per_row == 0 && N <= kWideMaxN && K <= kWideMaxK) {
        // wide workgroups for few rows (measured, the single Q projection
        // [3584, 3584] graph-replayed: 5.54 -> 4.38 us, cold 8.6 -> 7.6 us;
        // the per-linear 28-layer stream 1.266 -> 1.215 ms; with gate/up and
        // the lm_head also wide the stream is slower, 1.279 ms)
        const int C = K / 32, U = (C + kWave - 1) / kWave;
        constexpr int rows = kWideThreadsX / kWave;
        const dim3 grid((N + rows - 1) / rows), block(kWideThreadsX);
        hipStream_t st = (hipStream_t)stream;
        const u32x4* w = reinterpret_cast<const u32x4*>(wq);
#define BQD_WIDE_CASE(UU)                                                                                 \
        if (U <= UU) {                                                                                    \
            if (x_dtype == BQD_F32)                                                                       \
                hipLaunchKernelGGL((k_linear_wide<UU, X_F32, kWideThreadsX>), grid, block, (size_t)K, st, w, sw, \
                                   bias, x, nullptr, y, acc, qx_out, sx_out, N, C);                       \
            else                                                                                          \
                hipLaunchKernelGGL((k_linear_wide<UU, X_F16, kWideThreadsX>), grid, block, (size_t)K, st, w, sw, \
                                   bias, x, nullptr, y, acc, qx_out, sx_out, N, C);                       \
            return launched();                                                                            \
        }
        BQD_WIDE_CASES(BQD_WIDE_CASE)
#undef BQD_WIDE_CASE
    }
    const GemvCfg c = make_cfg(N, K / 32, r, lanes_per_row, 1);
    if (x_dtype == BQD_F32)
        return launch_gemv_rowwise<X_F32>(wq, sw, bias, x, nullptr, y, acc, qx_out, sx_out, N, K, c,
                                          (hipStream_t)stream);
    return launch_gemv_rowwise<X_F16>(wq, sw, bias, x, nullptr, y, acc, qx_out, sx_out, N, K, c,
                                      (hipStream_t)stream);
}


int linear_rmsnorm_w4a8(const uint32_t* wq, const float* sw, const float* bias, const float* h,
                        const float* delta, const float* gamma, float eps, float* h_out, float* y,
                        int8_t* qx_out, float* sx_out, int32_t* acc, int32_t N, int32_t K, int32_t r,
                        int32_t lanes_per_row, void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K);
    if (rc)
        return rc;
    if (K > 4 * 8 * kThreads)
        return BQD_ERR_BOUND;
    if (!(eps >= 0.0f) || !(eps <= FLT_MAX))
        return BQD_ERR_SHAPE;
    if (N == 0)
        return BQD_OK;
    if (!wq || !sw || !h || !gamma || !y)
        return BQD_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(h, 16) || !aligned(delta, 16) || !aligned(gamma, 16) ||
        !aligned(h_out, 16) || !aligned(qx_out, 16) || !aligned(sw, 4) || !aligned(sx_out, 4) ||
        !aligned(y, 4) || !aligned(bias, 4) || !aligned(acc, 4))
        return BQD_ERR_ALIGN;
    if (!valid_config(r, lanes_per_row))
        return BQD_ERR_CONFIG;
    if (io_overlap({{wq, (size_t)N * K / 2}, {sw, 4 * (size_t)N}, {bias, 4 * (size_t)N}, {h, 4 * (size_t)K},
                    {delta, 4 * (size_t)K}, {gamma, 4 * (size_t)K}},
                   {{y, 4 * (size_t)N}, {h_out, 4 * (size_t)K}, {qx_out, (size_t)K}, {sx_out, 4},
                    {acc, 4 * (size_t)N}}))
        return BQD_ERR_SHAPE;
    if ((rc = bqd_init()))
        return rc;
    const GemvCfg c = make_cfg(N, K / 32, r, lanes_per_row, 1);
    const RmsIn rms{h, delta, gamma, h_out, eps};
    return launch_gemv_rowwise<X_RMS>(wq, sw, bias, nullptr, nullptr, y, acc, qx_out, sx_out, N, K, c,
                                      (hipStream_t)stream, rms);
}

int gemv_w4a8_group32(const uint32_t* wq, const uint16_t* s16, const float* bias, const int8_t* qx,
                      const float* sx, float* y, int32_t* acc_g, int32_t N, int32_t K, int32_t r,
                      int32_t lanes_per_row, void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K);
    if (rc)
        return rc;
    if (N == 0)
        return BQD_OK;
    if (!wq || !s16 || !qx || !sx || !y)
        return BQD_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(qx, 16) || !aligned(s16, 2) || !aligned(sx, 4) ||
        !aligned(y, 4) || !aligned(bias, 4) || !aligned(acc_g, 4))
        return BQD_ERR_ALIGN;
    if (!valid_config(r, lanes_per_row))
        return BQD_ERR_CONFIG;
    if (io_overlap({{wq, (size_t)N * K / 2}, {s16, (size_t)N * (K / 32) * 2}, {bias, 4 * (size_t)N},
                    {qx, (size_t)K}, {sx, 4}},
                   {{y, 4 * (size_t)N}, {acc_g, (size_t)N * (K / 32) * 4}}))
        return BQD_ERR_SHAPE;
    if ((rc = bqd_init()))
        return rc;
    return launch_gemv_group32<X_Q8>(wq, s16, bias, qx, sx, y, acc_g, nullptr, nullptr, N, K,
                                     make_cfg(N, K / 32, r, lanes_per_row, 2), (hipStream_t)stream);
}

int linear_w4a8_group32(const uint32_t* wq, const uint16_t* s16, const float* bias, const void* x,
                        int32_t x_dtype, float* y, int8_t* qx_out, float* sx_out, int32_t* acc_g,
                        int32_t N, int32_t K, int32_t r, int32_t lanes_per_row, void* stream)
{
    int rc = check_x_dtype(x_dtype);
    if (rc)
        return rc;
    if (N < 0)
        return BQD_ERR_SHAPE;
    if ((rc = check_k(K)))
        return rc;
    if (N == 0)
        return BQD_OK;
    if (!wq || !s16 || !x || !y)
        return BQD_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(x, 16) || !aligned(qx_out, 16) || !aligned(s16, 2) ||
        !aligned(sx_out, 4) || !aligned(y, 4) || !aligned(bias, 4) || !aligned(acc_g, 4))
        return BQD_ERR_ALIGN;
    if (!valid_config(r, lanes_per_row))
        return BQD_ERR_CONFIG;
    if (io_overlap({{wq, (size_t)N * K / 2}, {s16, (size_t)N * (K / 32) * 2}, {bias, 4 * (size_t)N},
                    {x, (size_t)K * (x_dtype == BQD_F32 ? 4 : 2)}},
                   {{y, 4 * (size_t)N}, {qx_out, (size_t)K}, {sx_out, 4}, {acc_g, (size_t)N * (K / 32) * 4}}))
        return BQD_ERR_SHAPE;
    if ((rc = bqd_init()))
        return rc;
    const GemvCfg c = make_cfg(N, K / 32, r, lanes_per_row, 2);
    if (x_dtype == BQD_F32)
        return launch_gemv_group32<X_F32>(wq, s16, bias, x, nullptr, y, acc_g, qx_out, sx_out, N, K,
                                          c, (hipStream_t)stream);
    return launch_gemv_group32<X_F16>(wq, s16, bias, x, nullptr, y, acc_g, qx_out, sx_out, N, K, c,
                                      (hipStream_t)stream);
}

int gemv_w8a16_group32(const int8_t* w8, const uint16_t* s16, const uint16_t* x16, float* y,
                       int32_t N, int32_t K, int32_t r, int32_t lanes_per_row, void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K);
    if (rc)
        return rc;
    if (2 * (size_t)K > (size_t)kLdsBytes)
        return BQD_ERR_BOUND;
    if (N == 0)
        return BQD_OK;
    if (!w8 || !s16 || !x16 || !y)
        return BQD_ERR_NULL;
    if (!aligned(w8, 16) || !aligned(x16, 16) || !aligned(s16, 2) || !aligned(y, 4))
        return BQD_ERR_ALIGN;
    if (io_overlap({{w8, (size_t)N * K}, {s16, (size_t)N * (K / 32) * 2}, {x16, 2 * (size_t)K}}, {{y, 4 * (size_t)N}}))
        return BQD_ERR_SHAPE;
    if (!valid_config(r, lanes_per_row))
        return BQD_ERR_CONFIG;
    const int L = lanes_per_row ? lanes_per_row : 16;
    if (r == 0)
        r = 1;  // [262144, 1536], 16 lanes per row: 70.4 / 73.7 / 77.5 us for r = 1 / 2 / 4
    if ((rc = bqd_init()))
        return rc;
    const int G = K / 32;
    const int rows = (kThreads / L) * r;
    const dim3 grid(grid_for((N + rows - 1) / rows)), block(kThreads);
    const size_t lds = 2 * (size_t)K;
    const u32x4* w = reinterpret_cast<const u32x4*>(w8);
    const u32x4* xv = reinterpret_cast<const u32x4*>(x16);
    hipStream_t st = (hipStream_t)stream;
#define BQD_W8_CASE(RR, LL)                                                                     \
    if (r == RR && L == LL) {                                                                   \
        hipLaunchKernelGGL((k_gemv_w8a16_g32<RR, LL>), grid, block, lds, st, w, s16, xv, y, N, G); \
        return launched();                                                                      \
    }
    BQD_W8_CASE(1, 16) BQD_W8_CASE(2, 16) BQD_W8_CASE(4, 16) BQD_W8_CASE(8, 16)
    BQD_W8_CASE(1, 32) BQD_W8_CASE(2, 32) BQD_W8_CASE(4, 32) BQD_W8_CASE(8, 32)
    BQD_W8_CASE(1, 64) BQD_W8_CASE(2, 64) BQD_W8_CASE(4, 64) BQD_W8_CASE(8, 64)
#undef BQD_W8_CASE
    return BQD_ERR_CONFIG;
}

int quantize_weights_q6k(const float* W, int32_t N, int32_t K, uint8_t* ql, uint8_t* qh, int8_t* sc,
                         uint16_t* d, void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K, 256);
    if (rc)
        return rc;
    if (K > BQD_MAX_K)
        return BQD_ERR_BOUND;
    if (N == 0)
        return BQD_OK;
    if (!W || !ql || !qh || !sc || !d)
        return BQD_ERR_NULL;
    if (!aligned(W, 16) || !aligned(ql, 8) || !aligned(qh, 4) || !aligned(d, 2))
        return BQD_ERR_ALIGN;
    if ((rc = bqd_init()))
        return rc;
    const long long subblocks = (long long)N * (K / 16);
    hipLaunchKernelGGL(k_quantize_weights_q6k, dim3((unsigned)((subblocks + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, (hipStream_t)stream, W, K, subblocks, reinterpret_cast<u32x2*>(ql),
                       reinterpret_cast<uint32_t*>(qh), sc, d);
    return launched();
}

int gemv_q6k_f16(const uint8_t* ql, const uint8_t* qh, const int8_t* sc, const uint16_t* d, const uint16_t* x16,
                 float* y, int32_t N, int32_t K, int32_t r, int32_t lanes_per_row, void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K, 256);
    if (rc)
        return rc;
    if (2 * (size_t)K > (size_t)kLdsBytes)
        return BQD_ERR_BOUND;
    if (N == 0)
        return BQD_OK;
    if (!ql || !qh || !sc || !d || !x16 || !y)
        return BQD_ERR_NULL;
    if (!aligned(ql, 16) || !aligned(qh, 16) || !aligned(sc, 4) || !aligned(d, 2) || !aligned(x16, 16) ||
        !aligned(y, 4))
        return BQD_ERR_ALIGN;
    if (!valid_config(r, lanes_per_row == 8 ? 16 : lanes_per_row))
        return BQD_ERR_CONFIG;
    // automatic: 2 rows per lane group, 8 lanes per row (the [262144, 1536]
    // head, us: 63.3 against 70.1 at 16 lanes and 77.6 at 1 row x 16 lanes)
    const int L = lanes_per_row ? lanes_per_row : 8;
    if (r == 0)
        r = 2;
    if ((rc = bqd_init()))
        return rc;
    const int C = K / 32;
    const int rows = (kThreads / L) * r;
    const dim3 grid(grid_for((N + rows - 1) / rows)), block(kThreads);
    const size_t lds = 2 * (size_t)K;
    const u32x4* qlv = reinterpret_cast<const u32x4*>(ql);
    const u32x4* qhv = reinterpret_cast<const u32x4*>(qh);
    const uint32_t* scv = reinterpret_cast<const uint32_t*>(sc);
    const u32x4* xv = reinterpret_cast<const u32x4*>(x16);
    hipStream_t st = (hipStream_t)stream;
#define BQD_Q6K_CASE(RR, LL)                                                                                    \
    if (r == RR && L == LL) {                                                                                   \
        hipLaunchKernelGGL((k_gemv_q6k<RR, LL>), grid, block, lds, st, qlv, qhv, scv, d, xv, y, N, C);           \
        return launched();                                                                                      \
    }
    BQD_Q6K_CASE(1, 8) BQD_Q6K_CASE(2, 8) BQD_Q6K_CASE(4, 8) BQD_Q6K_CASE(8, 8)
    BQD_Q6K_CASE(1, 16) BQD_Q6K_CASE(2, 16) BQD_Q6K_CASE(4, 16) BQD_Q6K_CASE(8, 16)
    BQD_Q6K_CASE(1, 32) BQD_Q6K_CASE(2, 32) BQD_Q6K_CASE(4, 32) BQD_Q6K_CASE(8, 32)
    BQD_Q6K_CASE(1, 64) BQD_Q6K_CASE(2, 64) BQD_Q6K_CASE(4, 64) BQD_Q6K_CASE(8, 64)
#undef BQD_Q6K_CASE
    return BQD_ERR_CONFIG;
}

int gemv_w4a16(const uint32_t* wq, const float* sw, const float* bias, const uint16_t* x16, float* y,
               int32_t N, int32_t K, int32_t r, int32_t lanes_per_row, void* stream)
{
    if (N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k(K);
    if (rc)
        return rc;
    if (2 * (size_t)K > (size_t)kLdsBytes)
        return BQD_ERR_BOUND;
    if (N == 0)
        return BQD_OK;
    if (!wq || !sw || !x16 || !y)
        return BQD_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(x16, 16) || !aligned(sw, 4) || !aligned(bias, 4) || !aligned(y, 4))
        return BQD_ERR_ALIGN;
    if (!valid_config(r, lanes_per_row))
        return BQD_ERR_CONFIG;
    // Automatic shape, from a sweep over the Qwen2-7B layer shapes: full
    // waves per row; two rows per wave once N alone fills the chip.
    const int L = lanes_per_row ? lanes_per_row : 64;
    if (r == 0)
        r = N >= 16384 ? 2 : 1;
    if ((rc = bqd_init()))
        return rc;
    const int C = K / 32;
    const int rows = (kThreads / L) * r;
    const dim3 grid(grid_for((N + rows - 1) / rows)), block(kThreads);
    const size_t lds = 2 * (size_t)K;
    const u32x4* w = reinterpret_cast<const u32x4*>(wq);
    const u32x4* xv = reinterpret_cast<const u32x4*>(x16);
    hipStream_t st = (hipStream_t)stream;
#define BQD_W4A16_CASE(RR, LL)                                                                        \
    if (r == RR && L == LL) {                                                                         \
        hipLaunchKernelGGL((k_gemv_w4a16<RR, LL>), grid, block, lds, st, w, sw, bias, xv, y, N, C);  \
        return launched();                                                                            \
    }
    BQD_W4A16_CASE(1, 16) BQD_W4A16_CASE(2, 16) BQD_W4A16_CASE(4, 16) BQD_W4A16_CASE(8, 16)
    BQD_W4A16_CASE(1, 32) BQD_W4A16_CASE(2, 32) BQD_W4A16_CASE(4, 32) BQD_W4A16_CASE(8, 32)
    BQD_W4A16_CASE(1, 64) BQD_W4A16_CASE(2, 64) BQD_W4A16_CASE(4, 64) BQD_W4A16_CASE(8, 64)
#undef BQD_W4A16_CASE
    return BQD_ERR_CONFIG;
}

// Blocks of k_verify_blocks for M tokens over N x C chunks: the K split,
// the slice length (a multiple of 4 chunks) and the number of tile groups
// with the least work on the busiest CU, counted in sixths of a quad (1 KB
// of weights from HBM): the block's quads, its staged codes (from L2, about
// a sixth of the cost per byte) and, with a split, its partials plus a
// fixed charge for the count and the gathering (measured: [3584, 18944]
// with two tokens, 224 blocks of whole tiles 13.4 us, 256 half-K blocks
// 16.1 us).  Tile groups are at
// least ceil(T / kVbMaxTiles) and, when there are more than one round of
// them, fill whole rounds.  Splits are tried while the tiles alone do not
// fill the CUs, or until one lets the codes fit.  False when no slice's
// codes fit the LDS.
struct VbPlan {
    int ksplit, kslice, ntg;
};
static bool vb_plan(int M, int N, int C, VbPlan& p)
{
    const long long T = (N + 15) / 16, G = current_cus();
    const int maxc = (kVbXsBytes / (16 * M) - 1) / 2;
    const long long need = (T + kVbMaxTiles - 1) / kVbMaxTiles;
    long long best = -1;
    for (int s = 1; s <= 64 && s <= C; ++s) {
        const int ksl = (((C + s - 1) / s) + 15) & ~15;  // whole 4-quad groups
        if (ksl > maxc || (C + ksl - 1) / ksl != s)
            continue;
        if (s > 1 && T * s > 2 * G && best >= 0)
            break;  // enough tiles: no further split unless the codes need one
        const long long per_round = G / s > 0 ? G / s : 1;
        long long ng = need > per_round ? (need + per_round - 1) / per_round * per_round : per_round;
        ng = ng > T ? T : ng;
        const long long rounds = (ng * s + G - 1) / G;
        const long long tmax = (T + ng - 1) / ng;
        const long long cost = rounds * (6 * tmax * ((ksl + 3) / 4) + (long long)ksl * M / 32 +
                                         (s > 1 ? kVbSplitCost + tmax * (6 + 3 * s / 2) : 0));
        if (best < 0 || cost < best) {
            best = cost;
            p = VbPlan{s, ksl, (int)ng};
        }
    }
    return best >= 0;
}

static size_t vb_workspace_bytes(int N, const VbPlan& p)
{
    if (p.ksplit <= 1)
        return 0;
    const size_t T = (size_t)(N + 15) / 16;
    return 4 * (((T + kVbCountWords - 1) / kVbCountWords) * kVbCountWords) + 8 * (size_t)p.ksplit * T * 256;
}

size_t gemm_w4a8_verify_workspace_bytes(int32_t M, int32_t N, int32_t K)
{
    if (M < 1 || M > BQD_MAX_TOKENS || N < 1 || check_k_any(K) || !fast_k(K) || bqd_init())
        return 0;
    VbPlan p;
    return vb_plan(M, N, K / 32, p) ? vb_workspace_bytes(N, p) : 0;
}

int gemm_w4a8_verify(const uint32_t* wq, const float* sw, const float* bias, const int8_t* qx,
                     const float* sx, float* y, int32_t* acc, int32_t M, int32_t N, int32_t K,
                     int32_t impl, void* workspace, size_t workspace_bytes, void* stream)
{
    if (M < 0 || N < 0)
        return BQD_ERR_SHAPE;
    int rc = check_k_any(K);
    if (rc)
        return rc;
    if (M > BQD_MAX_TOKENS)
        return BQD_ERR_BOUND;
    if (impl < 0 || impl > 3)
        return BQD_ERR_CONFIG;
    if (M == 0 || N == 0)
        return BQD_OK;
    if (!wq || !sw || !qx || !sx || !y)
        return BQD_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(qx, 16) || !aligned(sw, 4) || !aligned(sx, 4) ||
        !aligned(y, 4) || !aligned(bias, 4) || !aligned(acc, 4) || !aligned(workspace, 256))
        return BQD_ERR_ALIGN;
    if (io_overlap({{wq, (size_t)N * K / 2}, {sw, 4 * (size_t)N}, {bias, 4 * (size_t)N}, {qx, (size_t)M * K},
                    {sx, 4 * (size_t)M}},
                   {{y, 4 * (size_t)M * N}, {acc, 4 * (size_t)M * N}, {workspace, workspace_bytes}}))
        return BQD_ERR_SHAPE;
    if (!fast_k(K) && impl != 0)
        return BQD_ERR_CONFIG;
    if ((rc = bqd_init()))
        return rc;
    hipStream_t st = (hipStream_t)stream;
    if (!fast_k(K)) {
        // the general-K GEMV once per token
        for (int m = 0; m < M && rc == BQD_OK; ++m)
            rc = launch_gemv_any<X_Q8>(wq, sw, bias, qx + (size_t)m * K, sx + m, y + (size_t)m * N,
                                       acc ? acc + (size_t)m * N : nullptr, nullptr, nullptr, N, K, st);
        return rc;
    }
    const int C = K / 32;
    const u32x4* w = reinterpret_cast<const u32x4*>(wq);
    VbPlan vp{1, C, 1};
    const bool vb_ok = vb_plan(M, N, C, vp);
    const bool vb_fits = vb_ok && (vb_workspace_bytes(N, vp) == 0 ||
                                   (workspace && workspace_bytes >= vb_workspace_bytes(N, vp)));
    if (impl == 0) {
        // One token is the decode GEMV; from two tokens on the matrix cores
        // beat the dot-product kernel on both verify shapes (measured), and
        // the balanced blocks beat the per-tile kernel at every token count
        // (us, impl 2 / 3: [18944, 3584] M = 2 12.2 / 11.9, M = 4 12.8 /
        // 11.9, M = 16 16.1 / 12.9; [3584, 18944] M = 2 13.5 / 11.6, M = 16
        // 21.7 / 13.9).  The per-tile kernel remains for a split plan whose
        // workspace the caller did not give.
        if (M == 1)
            return gemv_w4a8(wq, sw, bias, qx, sx, y, acc, N, K, 0, 0, stream);
        impl = vb_fits ? 3 : 2;
    }
    if (impl == 3) {
        if (!vb_ok)
            return BQD_ERR_CONFIG;
        if (!vb_fits)
            return workspace ? BQD_ERR_BOUND : BQD_ERR_NULL;
        const size_t lds = (size_t)M * (2 * vp.kslice + 1) * 16;
        hipLaunchKernelGGL(k_verify_blocks, dim3(vp.ntg * vp.ksplit), dim3(kVbThreads), lds, st, w, sw, bias, qx,
                           sx, y, acc, M, N, C, vp.ksplit, vp.kslice, vp.ntg, static_cast<uint32_t*>(workspace));
        return launched();
    }
    if (impl == 2) {
        // Matrix cores, 16-row tiles x 16 token columns.  The smallest K split
        // over waves that still gives about 8 waves per CU (each wave's chain
        // of dependent weight steps shortens as the split grows); with more
        // than 8 tokens and at least 4 tiles per CU, 4 waves per CU (every
        // workgroup stages all tokens' codes: fewer, larger workgroups).  A
        // workgroup holds max(4, split) waves.
        const long long tiles = (N + 15) / 16;
        const long long cus = current_cus();
        const long long want = (M > 8 && tiles >= 4 * cus ? 4 : 8) * cus;
        int split = 16;
        for (int sp = 1; sp < 16; sp *= 2)
            if (tiles * sp >= want) {
                split = sp;
                break;
            }
        // From 4 to 8 tokens, 8-wave workgroups stage 16 loads per thread
        // where 16-wave ones stage 4 (three staging round trips per K instead
        // of nine at K = 18944): [3584, 18944] M = 4 / 8 14.6 / 17.5 ->
        // 13.9 / 16.4 us.  At 16 tokens the longer chains per wave cost more
        // (22.0 -> 23.3 us).
        if (M >= 4 && M <= 8 && split > 8)
            split = 8;
        const int waves = split < 4 ? 4 : split;
        const long long groups = (tiles + waves / split - 1) / (waves / split);
        // One workgroup per CU at most: stage longer segments (fewer barriers).
        const int budget = groups <= current_cus() ? kLdsMaxBytes - (waves + 2) * 1024 : kLdsBytes;
        int segc = (budget / M - 16) / 32;  // chunks per staged segment
        if (segc > C)
            segc = C;
        const size_t lds = (size_t)M * (32 * segc + 16);
        const dim3 grid(grid_for(groups)), block(waves * kWave);
#define BQD_MFMA_CASE(SP, WV)                                                                      \
    if (split == SP) {                                                                             \
        hipLaunchKernelGGL((k_verify_mfma<SP, WV>), grid, block, lds, st, w, sw, bias, qx, sx, y, acc, \
                           M, N, C, segc);                                                         \
        return launched();                                                                         \
    }
        BQD_MFMA_CASE(1, 4) BQD_MFMA_CASE(2, 4) BQD_MFMA_CASE(4, 4) BQD_MFMA_CASE(8, 8)
        BQD_MFMA_CASE(16, 16)
#undef BQD_MFMA_CASE
        return BQD_ERR_CONFIG;
    }
    const int MT = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    constexpr int L = 16, R = 2;
    // LDS holds MT tokens x SEGC chunks x 32 bytes; SEGC a multiple of L.
    int segc = kLdsBytes / (MT * 32);
    segc -= segc % L;
    if (segc >= C)
        segc = C;
    const size_t lds = (size_t)MT * segc * 32;
    const int rows = (kThreads / L) * R;
    const dim3 grid(grid_for((N + rows - 1) / rows)), block(kThreads);
#define BQD_VER_CASE(MM)                                                                          \
    if (MT == MM) {                                                                               \
        hipLaunchKernelGGL((k_verify_w4a8<MM, R, L>), grid, block, lds, st, w, sw, bias, qx, sx, y, \
                           acc, M, N, C, segc);                                                   \
        return launched();                                                                        \
    }
    BQD_VER_CASE(1) BQD_VER_CASE(2) BQD_VER_CASE(4) BQD_VER_CASE(8) BQD_VER_CASE(16)
#undef BQD_VER_CASE
    return BQD_ERR_CONFIG;
}

int layer_w4a8_forward(const bqd_linear_w4a8* lin, int32_t n, const void* const* x,
                       int32_t x_dtype, float* const* y, void* stream)
{
    if (n < 0 || n > 64)
        return BQD_ERR_SHAPE;
    if (n == 0)
        return BQD_OK;
    if (!lin || !x || !y)
        return BQD_ERR_NULL;
    int rc = check_x_dtype(x_dtype);
    if (rc)
        return rc;
    // Validate every linear before launching any of them.
    for (int i = 0; i < n; ++i) {
        const bqd_linear_w4a8& l = lin[i];
        if (!l.wq || !l.scales || !x[i] || !y[i])
            return BQD_ERR_NULL;
        if (l.scale_kind != BQD_SCALE_ROW_F32 && l.scale_kind != BQD_SCALE_GROUP32_F16)
            return BQD_ERR_DTYPE;
        if (l.N < 0)
            return BQD_ERR_SHAPE;
        if ((rc = check_k(l.K)))
            return rc;
        if (!aligned(l.wq, 16) || !aligned(x[i], 16) || !aligned(l.scales, 2) ||
            !aligned(l.bias, 4) || !aligned(y[i], 4))
            return BQD_ERR_ALIGN;
        if (!valid_config(l.r, l.lanes_per_row))
            return BQD_ERR_CONFIG;
        // each linear is its own launch, so only a linear's own output may
        // not overlap what that launch reads
        const size_t sb = l.scale_kind == BQD_SCALE_ROW_F32 ? 4 * (size_t)l.N : (size_t)l.N * (l.K / 32) * 2;
        if (io_overlap({{l.wq, (size_t)l.N * l.K / 2}, {l.scales, sb}, {l.bias, 4 * (size_t)l.N},
                        {x[i], (size_t)l.K * (x_dtype == BQD_F32 ? 4 : 2)}},
                       {{y[i], 4 * (size_t)l.N}}))
            return BQD_ERR_SHAPE;
    }
    for (int i = 0; i < n; ++i) {
        const bqd_linear_w4a8& l = lin[i];
        if (l.scale_kind == BQD_SCALE_ROW_F32)
            rc = linear_w4a8(l.wq, (const float*)l.scales, l.bias, x[i], x_dtype, y[i], nullptr,
                             nullptr, nullptr, l.N, l.K, l.r, l.lanes_per_row, stream);
        else
            rc = linear_w4a8_group32(l.wq, (const uint16_t*)l.scales, l.bias, x[i], x_dtype, y[i],
                                     nullptr, nullptr, nullptr, l.N, l.K, l.r, l.lanes_per_row,
                                     stream);
        if (rc)
            return rc;
    }
    return BQD_OK;
}

size_t decode_pass_desc_bytes(int32_t n)
{
    return n > 0 ? sizeof(PassHeader) + (size_t)n * sizeof(PassTask) : 0;
}

// Grid of the pass on the current device: co-resident workgroups, at most
// kPassWgPerCu per CU, for a given activation staging size.
static int pass_grid(int max_k, int* grid)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_pass<kPassSlots>, kPassThreads, pass_lds_bytes(max_k)) !=
            hipSuccess ||
        per_cu < 1)
        return BQD_ERR_LAUNCH;
    *grid = current_cus() * (per_cu < kPassWgPerCu ? per_cu : kPassWgPerCu);
    return BQD_OK;
}

// Lanes per row and rows per lane group for one linear on a grid of G
// workgroups: fewest loads per lane, plus a charge per pipeline step (small
// linears then take one step, whose loads are all issued before the wait).
static void pass_shape_host(int N, int C, int G, int slots, PassTask& t)
{
    const int rows_max = (N + G - 1) / G;
    long best = -1;
    for (int ls = 4; ls <= 6; ++ls) {
        for (int r = 2; r >= 1; --r) {
            const int L = 1 << ls, groups = kPassWorkers >> ls;
            const int iters = (C + L - 1) / L;
            const int batches = (rows_max + groups * r - 1) / (groups * r);
            const int steps = (iters * r + slots - 1) / slots;
            const long cost = (long)batches * r * iters + 4L * batches * steps;
            if (best < 0 || cost < best) {
                best = cost;
                t.lshift = ls;
                t.r = r;
                t.iters = iters;
                t.batches = batches;
                t.steps = steps;
            }
        }
    }
    t.rows_base = N / G;
    t.rows_extra = N % G;
}

static bool contains(const void* outer, size_t no, const void* inner, size_t ni)
{
    const uintptr_t a = (uintptr_t)outer, b = (uintptr_t)inner;
    return b >= a && b + ni <= a + no;
}

int decode_pass_encode(const bqd_linear_w4a8* lin, int32_t n, const void* const* x, int32_t x_dtype,
                       float* const* y, void* desc_host, size_t desc_bytes, int32_t* max_k, size_t* sync_bytes,
                       int32_t* slots_out)
{
    if (n <= 0 || n > BQD_MAX_PASS_LINEARS)
        return BQD_ERR_SHAPE;
    if (!lin || !x || !y || !desc_host || !max_k || !sync_bytes || !slots_out)
        return BQD_ERR_NULL;
    int rc = check_x_dtype(x_dtype);
    if (rc)
        return rc;
    if (desc_bytes < decode_pass_desc_bytes(n))
        return BQD_ERR_SHAPE;
    const size_t xe = x_dtype == BQD_F32 ? 4 : 2;
    int kmax = 0;
    for (int i = 0; i < n; ++i) {
        const bqd_linear_w4a8& l = lin[i];
        if (l.scale_kind != BQD_SCALE_ROW_F32 && l.scale_kind != BQD_SCALE_GROUP32_F16)
            return BQD_ERR_DTYPE;
        const bool g32 = l.scale_kind == BQD_SCALE_GROUP32_F16;
        if (l.N <= 0)
            return BQD_ERR_SHAPE;
        if ((rc = check_k(l.K)))
            return rc;
        if (g32 && l.K % 256)
            return BQD_ERR_SHAPE;  // a row's group scales fill whole 16-byte words
        if (!l.wq || !l.scales || !x[i] || !y[i])
            return BQD_ERR_NULL;
        if (!aligned(l.wq, 16) || !aligned(x[i], 16) || !aligned(l.scales, g32 ? 16 : 4) || !aligned(l.bias, 4) ||
            !aligned(y[i], 4))
            return BQD_ERR_ALIGN;
        if (l.r != 0 || l.lanes_per_row != 0)
            return BQD_ERR_CONFIG;  // the pass chooses its own work split
        if (l.K > kPassMaxK)
            return BQD_ERR_BOUND;
        kmax = l.K > kmax ? l.K : kmax;
    }
    // Outputs are disjoint, and none overlaps weights, scales or biases
    // (read, and prefetched before the activation is ready, through the
    // caches): each output is written once per pass.
    for (int i = 0; i < n; ++i) {
        const size_t ny = (size_t)lin[i].N * 4;
        for (int j = 0; j < n; ++j) {
            const bqd_linear_w4a8& l = lin[j];
            const size_t scale_bytes =
                l.scale_kind == BQD_SCALE_GROUP32_F16 ? (size_t)l.N * (l.K / 32) * 2 : (size_t)l.N * 4;
            if ((j > i && bytes_overlap(y[i], ny, y[j], (size_t)l.N * 4)) ||
                bytes_overlap(y[i], ny, l.wq, (size_t)l.N * l.K / 2) ||
                bytes_overlap(y[i], ny, l.scales, scale_bytes) ||
                (l.bias && bytes_overlap(y[i], ny, l.bias, (size_t)l.N * 4)))
                return BQD_ERR_SHAPE;
        }
    }
    // Where each activation comes from: written before the launch (it
    // overlaps no output), or a contiguous part of one earlier linear's
    // output (read from the exchange; fp32 only).  Overlapping its own or a
    // later output, or more than one output, is refused: workgroups run
    // ahead of each other between dependent linears, so a later output may
    // be written while the activation is still being read.
    std::vector<int> src(n, -1);
    std::vector<int64_t> off(n, 0);
    for (int i = 0; i < n; ++i) {
        const size_t nx = (size_t)lin[i].K * xe;
        for (int k = 0; k < n; ++k) {
            const size_t ny = (size_t)lin[k].N * 4;
            if (!bytes_overlap(x[i], nx, y[k], ny))
                continue;
            if (k >= i || src[i] >= 0 || !contains(y[k], ny, x[i], nx))
                return BQD_ERR_SHAPE;
            if (x_dtype != BQD_F32)
                return BQD_ERR_DTYPE;
            const uintptr_t d = (uintptr_t)x[i] - (uintptr_t)y[k];
            if (d % 4)
                return BQD_ERR_ALIGN;
            src[i] = k;
            off[i] = (int64_t)(d / 4);
        }
    }
    // Exchange offsets: each output a later linear reads gets N words, placed
    // so that an exchange word and its output element share their position
    // modulo 16 bytes (a 16-byte-aligned activation is a 16-byte-aligned run
    // of exchange words); every output starts a 256-byte line.
    std::vector<int64_t> xout(n, -1);
    int64_t words = 0;
    for (int i = 0; i < n; ++i)
        if (src[i] >= 0 && xout[src[i]] < 0) {
            const int k = src[i];
            xout[k] = words + (int64_t)(((uintptr_t)y[k] >> 2) & 3);
            words += ((int64_t)lin[k].N + 3 + 63) / 64 * 64;
        }
    for (int k = 0; k < n; ++k)
        if (src[k] >= 0 && xout[src[k]] < 0)
            return BQD_ERR_SHAPE;  // unreachable: every source has an offset
    if (words > (int64_t)(INT32_MAX / 2) - kXchBase)
        return BQD_ERR_BOUND;
    if ((rc = bqd_init()))
        return rc;
    // the kernel instance: 4 chunks per step when every linear is group-32
    bool all_g32 = true;
    for (int i = 0; i < n; ++i)
        all_g32 = all_g32 && lin[i].scale_kind == BQD_SCALE_GROUP32_F16;
    const int slots = all_g32 ? kPassSlotsSmall : kPassSlots;
    int G = 0;
    if ((rc = pass_grid(kmax, &G)))
        return rc;
    if (G > kPassMaxGrid)
        return BQD_ERR_LAUNCH;
    PassHeader h{n, G, kmax, (int32_t)words, slots, {0, 0, 0}};
    std::memcpy(desc_host, &h, sizeof h);
    PassTask* d = reinterpret_cast<PassTask*>(reinterpret_cast<char*>(desc_host) + sizeof(PassHeader));
    for (int i = 0; i < n; ++i) {
        const bqd_linear_w4a8& l = lin[i];
        PassTask t;
        std::memset(&t, 0, sizeof t);
        t.wq = reinterpret_cast<const u32x4*>(l.wq);
        t.scales = l.scales;
        t.kind = l.scale_kind == BQD_SCALE_GROUP32_F16 ? 1 : 0;
        t.bias = l.bias;
        t.x = x[i];
        t.y = y[i];
        t.N = l.N;
        t.C = l.K / 32;
        t.x_dtype = x_dtype == BQD_F16 ? X_F16 : X_F32;
        t.xin = src[i] >= 0 ? (int32_t)(xout[src[i]] + off[i]) : -1;
        t.xout = (int32_t)xout[i];
        pass_shape_host(t.N, t.C, G, slots, t);
        if (t.kind == 1) {
            // the per-linear group-32 kernel's lanes per row (its sums run
            // in that order), one row per lane group
            const int rows_max = (t.N + G - 1) / G;
            if ((size_t)rows_max * t.C * 2 > (size_t)kPassScaleLds)
                return BQD_ERR_BOUND;
            t.lshift = 5;
            t.r = 1;
            t.iters = (t.C + 31) / 32;
            t.batches = (rows_max + (kPassWorkers >> 5) - 1) / (kPassWorkers >> 5);
            t.steps = (t.iters + slots - 1) / slots;
        }
        std::memcpy(d + i, &t, sizeof t);
    }
    *max_k = kmax;
    *sync_bytes = ((size_t)kXchBase + 2 * (size_t)words) * sizeof(uint32_t);
    *slots_out = slots;
    return BQD_OK;
}

static int pass_check_launch(const void* desc_dev, int32_t n, int32_t max_k, int32_t slots, size_t sync_bytes,
                             int32_t spin_limit)
{
    if (n <= 0 || n > BQD_MAX_PASS_LINEARS)
        return BQD_ERR_SHAPE;
    if (slots != kPassSlots && slots != kPassSlotsSmall)
        return BQD_ERR_CONFIG;
    if (!desc_dev)
        return BQD_ERR_NULL;
    int rc = check_k(max_k);
    if (rc)
        return rc;
    if (max_k > kPassMaxK)
        return BQD_ERR_BOUND;
    if (sync_bytes < (size_t)kXchBase * 4 || sync_bytes % 256)
        return BQD_ERR_SHAPE;
    if (spin_limit < 0)
        return BQD_ERR_CONFIG;
    if (!aligned(desc_dev, 16))
        return BQD_ERR_ALIGN;
    return BQD_OK;
}

static int pass_launch(const void* desc_dev, int32_t n, int32_t max_k, int32_t slots, uint32_t* sync,
                       size_t sync_bytes, int32_t spin_limit, hipStream_t stream)
{
    int G = 0;
    int rc = pass_grid(max_k, &G);
    if (rc)
        return rc;
    const PassHeader* hdr = reinterpret_cast<const PassHeader*>(desc_dev);
    const PassTask* tasks =
        reinterpret_cast<const PassTask*>(reinterpret_cast<const char*>(desc_dev) + sizeof(PassHeader));
    int spin = spin_limit ? spin_limit : kPassSpinLimit;
    int nn = n, mk = max_k;
    size_t words = sync_bytes / 4;
    void* args[] = {(void*)&hdr, (void*)&tasks, (void*)&nn, (void*)&mk, (void*)&sync, (void*)&words, (void*)&spin};
    // An ordinary launch: the grid is what the occupancy query says fits at
    // once (one workgroup per CU), so on a device with no other work every
    // workgroup is resident from the start; were some held back by other
    // work, the bounded waits end them with bit 0 of the error word instead
    // of a hang.  (A cooperative launch gives the same residency, costs
    // about 1.5 % per pass and has made the profiler's exit handlers crash.)
    const void* fn = slots == kPassSlotsSmall ? (const void*)k_decode_pass<kPassSlotsSmall>
                                              : (const void*)k_decode_pass<kPassSlots>;
    if (hipLaunchKernel(fn, dim3(G), dim3(kPassThreads), args,
                        (size_t)pass_lds_bytes(max_k), stream) != hipSuccess)
        return BQD_ERR_LAUNCH;
    return launched();
}

int decode_pass_w4a8(const void* desc_dev, int32_t n, int32_t max_k, int32_t slots, uint32_t* sync_dev,
                     size_t sync_bytes, int32_t spin_limit, void* stream)
{
    int rc = pass_check_launch(desc_dev, n, max_k, slots, sync_bytes, spin_limit);
    if (rc)
        return rc;
    if (!sync_dev)
        return BQD_ERR_NULL;
    if (!aligned(sync_dev, 256))
        return BQD_ERR_ALIGN;
    if ((rc = bqd_init()))
        return rc;
    return pass_launch(desc_dev, n, max_k, slots, sync_dev, sync_bytes, spin_limit, (hipStream_t)stream);
}

int decode_pass_w4a8_static(const void* desc_dev, int32_t n, int32_t max_k, int32_t slots, size_t sync_bytes,
                            int32_t spin_limit, uint32_t* err_dev, void* stream)
{
    int rc = pass_check_launch(desc_dev, n, max_k, slots, sync_bytes, spin_limit);
    if (rc)
        return rc;
    if (sync_bytes > (size_t)BQD_STATIC_PASS_BYTES)
        return BQD_ERR_BOUND;
    if (!err_dev)
        return BQD_ERR_NULL;
    if (!aligned(err_dev, 4))
        return BQD_ERR_ALIGN;
    if ((rc = bqd_init()))
        return rc;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return BQD_ERR_DEVICE;
    uint32_t* ws = g_scratch[dev];
    if (!ws)
        return BQD_ERR_LAUNCH;
    hipStream_t st = (hipStream_t)stream;
    // The array keeps the previous call's contents (any descriptors):
    // every call starts from a zeroed workspace of its own size.
    const size_t n16 = sync_bytes / 16;
    const long long want = (long long)((n16 + kThreads - 1) / kThreads);
    const unsigned grid = (unsigned)(want < 1024 ? want : 1024);
    hipLaunchKernelGGL(k_zero16, dim3(grid), dim3(kThreads), 0, st, reinterpret_cast<u32x4*>(ws), n16);
    if ((rc = launched()))
        return rc;
    if ((rc = pass_launch(desc_dev, n, max_k, slots, ws, sync_bytes, spin_limit, st)))
        return rc;
    hipLaunchKernelGGL(k_copy_word, dim3(1), dim3(kWave), 0, st, ws, err_dev);
    return launched();
}

int read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t grid, int32_t unroll, void* stream)
{
    if (grid < 1 || grid > (1 << 20) || bytes % 16 != 0)
        return BQD_ERR_SHAPE;
    if (unroll != 1 && unroll != 4 && unroll != 8)
        return BQD_ERR_CONFIG;
    if (bytes == 0)
        return BQD_OK;
    if (!buf || !sink)
        return BQD_ERR_NULL;
    if (!aligned(buf, 16) || !aligned(sink, 4))
        return BQD_ERR_ALIGN;
    int rc = bqd_init();
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    const u32x4* p = reinterpret_cast<const u32x4*>(buf);
    const long long n = (long long)(bytes / 16);
    if (unroll == 1)
        hipLaunchKernelGGL(k_read_probe<1>, dim3(grid), dim3(kThreads), 0, st, p, n, sink);
    else if (unroll == 4)
        hipLaunchKernelGGL(k_read_probe<4>, dim3(grid), dim3(kThreads), 0, st, p, n, sink);
    else
        hipLaunchKernelGGL(k_read_probe<8>, dim3(grid), dim3(kThreads), 0, st, p, n, sink);
    return launched();
}

}  // extern "C"
