// Device-side building blocks shared by the sparse MLA kernels (gfx950).
//
// Operand layouts of the bf16 MFMA used throughout, v_mfma_f32_16x16x32_bf16
// (checked on the hardware): with lane l, g = l / 16 and n = l % 16,
//   A (16 x 32): lane holds A[n][8g .. 8g+7]
//   B (32 x 16): lane holds B[8g .. 8g+7][n]
//   C (16 x 16): lane holds C[4g .. 4g+3][n]
// The contraction index is always the in-lane one.  ds_read_b64_tr_b16 reads
// a 4 x 16 block of 16-bit values spread over a 16-lane group (lanes 4e..4e+3
// name row e, four columns each) and returns to lane i of the group the column
// i of that block (rows 0..3), i.e. a transposed operand straight from LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) __bf16 lds_bf16;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BLK = 64;           // top-k slots per block
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 zero8() {
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Streaming (non-temporal) loads, for the Delta pass, which reads O and dO
// once and nothing else: -11 % at the headline.  Measured elsewhere they cost
// time or only moved it: the gather kernels' q, dO and dS loads (+1 to +28 %),
// the reduce's partial rows (+11 %: some are still cached from the dKV
// kernel), the dKV kernel's staging of q, dO, P and dS (-3 % there, +7 % in
// the reduce after it); streaming stores of 8-byte pieces were up to 2.6x
// slower (not combined into whole lines).
__device__ __forceinline__ bf16x8 ld8_nt(const __bf16* p) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ bf16x8 lds8(const __bf16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Transposed 4-element read from LDS (see the file comment).
__device__ __forceinline__ bf16x4 lds_tr4(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)((lds_bf16*)p));
}

__device__ __forceinline__ bf16x8 cat44(bf16x4 lo, bf16x4 hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ bf16x4 cvt4(float a, float b, float c, float d) {
    return bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}

__device__ __forceinline__ bf16x8 cvt8(f32x4 lo, f32x4 hi) {
    return bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                  (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
}

__device__ __forceinline__ void st4(__bf16* p, bf16x4 v) {
    *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v);
}


__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Wait until every vector-memory operation of this wave has completed
// (including direct global->LDS loads).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70 & ~0xC000); }

__device__ __forceinline__ float xor_max(float v, int m) {
    return fmaxf(v, __shfl_xor(v, m, 64));
}

// Number of valid-candidate slots of token t: the compact length clamped to
// [0, W], or W for the non-compact layout.
__device__ __forceinline__ int row_length(const int32_t* len, int t, int W) {
    if (len == nullptr) return W;
    int L = len[t];
    return L < 0 ? 0 : (L > W ? W : L);
}

// KV row of slot j, or -1 when the slot is not valid.
__device__ __forceinline__ int slot_row(const int32_t* idx, int t, int W, int L, int S_kv, int j) {
    if (j >= L) return -1;
    int v = idx[(size_t)t * W + j];
    return (v >= 0 && v < S_kv) ? v : -1;
}

// Stage the raw top-k indices of slots 64 b .. 64 b + 63 of token t into dst
// (LDS) with one buffer load that writes LDS directly (a whole wave calls it;
// slots past the end of the row read 0).  It completes with the caller's
// vector-memory count.  A slot's validity is decided where it is used.
__device__ __forceinline__ void stage_slot_idx(int* dst, const int32_t* idx, int t, int W, int b,
                                               int lane) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(idx + (size_t)t * W), (short)0, W * 4, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 4, (b * 64 + lane) * 4, 0, 0, 0);
}

// Store the KV rows of one block's 64 slots (a whole wave: lane = slot; -1
// for a slot that is not valid) and whether any of them is valid.  A block
// with no valid slot adds exact zeros to every sum, so its math is skipped.
__device__ __forceinline__ void put_rows(int* rows, int* live, int r, int lane) {
    rows[lane] = r;
    const bool any = __builtin_amdgcn_ballot_w64(r >= 0) != 0;
    if (lane == 0) *live = any;
}

// Block storage of fp32 values in 16 bits each (the dKV partials): a group of
// four values keeps E = max(13, the largest fp32 exponent field among them)
// (8 bits) and each value as a 14-bit signed multiple of 2^(E - 139), i.e. of
// 2^-12 times the group's leading power of two.  A value's error is at most
// 2^-13 of the group's largest magnitude (2^-12 where rounding reaches the
// end of the range); groups below 2^-114 are kept to 2^-127 absolute.  A group
// holding a non-finite value has E = 255 and decodes as NaN.  Layout:
// w0 = E | q0 << 8 | (q1 & 0x3FF) << 22, w1 = q1 >> 10 | q2 << 4 | q3 << 18
// (q in 14-bit two's complement).
__device__ __forceinline__ u32x2 pack_blk4(f32x4 v) {
    // E from the exponent fields (through scalars: a bit cast of a vector
    // element can read the wrong element with this compiler)
    float x[4];
    uint32_t e4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = v[i];
        e4[i] = __builtin_amdgcn_ubfe(__builtin_bit_cast(uint32_t, x[i]), 23, 8);
    }
    const uint32_t e01 = e4[0] > e4[1] ? e4[0] : e4[1];
    const uint32_t e23 = e4[2] > e4[3] ? e4[2] : e4[3];
    uint32_t e = e01 > e23 ? e01 : e23;
    e = e > 13u ? e : 13u;
    const float sc = __builtin_bit_cast(float, (266u - e) << 23);   // 2^(139 - E), a normal number
    // |x sc| < 2^13: adding 1.5 * 2^23 in one rounding leaves round-to-
    // nearest-even(x sc) in the low bits, as rint(x sc) would; the result,
    // clamped to +-8191 (a float median: r is an integer plus 1.5 * 2^23),
    // holds q in two's complement in its low 14 bits
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float r = __builtin_fmaf(x[i], sc, 12582912.0f);
        u[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(r, 12582912.0f - 8191.0f, 12582912.0f + 8191.0f));
    }
    const uint32_t w0 = e | ((u[0] << 8) & 0x3FFF00u) | (u[1] << 22);
    const uint32_t w1 = ((u[1] >> 10) & 0xFu) | ((u[2] << 4) & 0x3FFF0u) | (u[3] << 18);
    return u32x2{w0, w1};
}

__device__ __forceinline__ f32x4 unpack_blk4(u32x2 w) {
    const uint32_t e = w[0] & 0xFFu;
    float sc = e > 12u ? __builtin_bit_cast(float, (e - 12u) << 23) : 0.f;       // 2^(E - 139)
    sc = e == 255u ? __builtin_nanf("") : sc;
    const int q0 = __builtin_amdgcn_sbfe((int)w[0], 8, 14);
    const int q1 = __builtin_amdgcn_sbfe((int)((w[0] >> 22) | (w[1] << 10)), 0, 14);
    const int q2 = __builtin_amdgcn_sbfe((int)w[1], 4, 14);
    const int q3 = __builtin_amdgcn_sbfe((int)w[1], 18, 14);
    return f32x4{(float)q0 * sc, (float)q1 * sc, (float)q2 * sc, (float)q3 * sc};
}

// Finite-max-guarded logaddexp: ln(e^a + e^b); an infinite maximum is returned
// as is, so no inf - inf is formed.
__device__ __forceinline__ float glae(float a, float b) {
    float m = fmaxf(a, b);
    if (m == INFINITY || m == -INFINITY) return m;
    return m + logf(expf(a - m) + expf(b - m));
}

// sigma(x) = 1 / (1 + e^-x), saturating cleanly at both ends.
__device__ __forceinline__ float sigmoid(float x) {
    return 1.0f / (1.0f + expf(-x));
}

}  // namespace smla
