// q4moe_dev.h -- device helpers shared by the gfx950 kernels of the routed
// MoE Q4 layer: bf16 conversions, the on-chip group-64 affine 4-bit
// dequantisation, MFMA operand types and wave reductions.
//
// Source for the weight format: [Lily-M5] = "Perplexity's Lily beats MLX-LM
// on MacBook M5 because it only runs one model", section "Prefill: keep
// routing on the GPU, dequantize in flight" -- every group of 64 weights
// shares a bf16 scale and a bf16 bias, w = q * scale + bias, and the tensor
// ops take the weights as bf16 operands.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 64;
constexpr int kWave = 64;
constexpr int kMaxExperts = 256;  // MOE_MAX_EXPERTS
constexpr int kMaxTopK = 8;       // MOE_MAX_TOPK
constexpr int kBlockRows = 32;    // MOE_BLOCK_ROWS
constexpr int kTileRows = 128;    // MOE_TILE_ROWS

struct Q4 {  // device view of one stack of Q4 matrices (see moe_q4mat)
    const uint32_t* q;
    const uint16_t* scale;
    const uint16_t* bias;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
    return __uint_as_float(bits << 16);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32), two at a time.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// Two floats as two round-to-nearest-even fp16 values in one word (low half =
// lo): one v_cvt_pk_f16_f32 on gfx950, the same bits as two scalar casts.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const float __attribute__((ext_vector_type(2))) v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// A group's scale as dequant8 takes it: scale * 2^9 (exact for |scale| < 2^119).
__device__ __forceinline__ float dq_scale(uint32_t bf16_bits) {
    return bf16_to_f32(bf16_bits) * 512.0f;
}

// Dequantise one 32-bit word of eight 4-bit codes (lowest nibble = lowest k)
// with the group's scale and bias into eight bf16 weights in k order:
// w = bf16(q * scale + bias).  s9 is scale * 2^9 (dq_scale).
//
// A byte holding a code q in 0..15, read as an fp8 e4m3 value (the OCP
// format gfx950 converts: 3 mantissa bits, exponent bias 7), is exactly
// q * 2^-9: codes 0..7 are the subnormals m * 2^-9 and codes 8..15 the first
// normal binade (1 + m/8) * 2^-6 = (8 + m) * 2^-9.  So v_cvt_pk_f32_fp8 turns
// two codes into two exact floats in one instruction, and
// fma(q * 2^-9, scale * 2^9, bias) = fma(q, scale, bias): q * scale is exact in
// fp32 (at most 12 significant bits) and so is the sum whenever the exponents
// of scale and bias lie within 12 of each other; the single rounding of the
// fma followed by the round-to-nearest-even conversion gives the nearest bf16
// to the exact affine value.
//
// 19 VALU instructions per word: 3 to split the even and odd codes into the
// four bytes of two words, 4 v_cvt_pk_f32_fp8, 8 v_fma_f32 and 4
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s9, float b) {
    const uint32_t ev = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6 in bytes 0..3
    const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
    const f32x2 e01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)ev, false);  // q0, q2 (* 2^-9)
    const f32x2 e23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)ev, true);   // q4, q6
    const f32x2 o01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)od, false);  // q1, q3
    const f32x2 o23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)od, true);   // q5, q7
    u32x4 r;
    r[0] = pack_bf16x2(__builtin_fmaf(e01[0], s9, b), __builtin_fmaf(o01[0], s9, b));
    r[1] = pack_bf16x2(__builtin_fmaf(e01[1], s9, b), __builtin_fmaf(o01[1], s9, b));
    r[2] = pack_bf16x2(__builtin_fmaf(e23[0], s9, b), __builtin_fmaf(o23[0], s9, b));
    r[3] = pack_bf16x2(__builtin_fmaf(e23[1], s9, b), __builtin_fmaf(o23[1], s9, b));
    return __builtin_bit_cast(bf16x8, r);
}

// acc + sum over the eight weights of one code word of bf16(q*s + b) * v (s9 =
// dq_scale of s), with
// v the matching eight bf16 activations as four packed pairs in k order
// (v_dot2_f32_bf16: both products and the sum in fp32).
// (The activations are reinterpreted as one bf16x8 and split with shuffles:
// a bit cast of each 32-bit element separately was compiled into four uses of
// element 0.)
__device__ __forceinline__ float dot8_bf16(uint32_t w, float s9, float b, u32x4 v, float acc) {
    const bf16x8 wv = dequant8(w, s9, b);
    const bf16x8 xv = __builtin_bit_cast(bf16x8, v);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 0, 1),
                                          __builtin_shufflevector(xv, xv, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 2, 3),
                                          __builtin_shufflevector(xv, xv, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 4, 5),
                                          __builtin_shufflevector(xv, xv, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 6, 7),
                                          __builtin_shufflevector(xv, xv, 6, 7), acc, false);
    return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Sum of v over the wave, returned to every lane, in a fixed order: four DPP
// steps leave every lane with the sum of its row of 16 lanes (add the
// neighbour, the other pair, the mirrored quad, the mirrored half row), then
// the four row sums are added through scalar registers.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm 1,0,3,2
    v += dpp_f32<0x4E>(v);   // quad_perm 2,3,0,1
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float silu(float g) {
    return __fdividef(g, 1.0f + __expf(-g));
}

// Order-preserving 32-bit key of an fp32 logit: a larger logit has a larger
// key.  -0.0 is folded onto +0.0 so that the two tie; key 0 belongs to no
// finite logit.
__device__ __forceinline__ uint32_t logit_key(float v) {
    if (v == 0.0f) v = 0.0f;
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Maximum of v over the wave, returned to every lane: four DPP steps give
// every lane the maximum of its row of 16 lanes (swap neighbours, swap
// pairs, mirror within 8, mirror within 16), then the four row maxima meet in
// scalar registers.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false)); // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false)); // row_mirror
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// ---------------------------------------------------------------------------
// Wave-wide reductions on the vector ALUs only: DPP within rows of 16 lanes,
// then gfx950's row swaps (v_permlane16_swap: rows 0<->1, 2<->3;
// v_permlane32_swap: lanes 0-31 <-> 32-63).  Every lane gets the result; no
// scalar round trip.
// ---------------------------------------------------------------------------
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(r16[0], r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return op(r32[0], r32[1]);
}

// ---------------------------------------------------------------------------
// Top-k of one token's logits by one wave (E <= 256: lane l holds experts
// 4l .. 4l + 3, so lane order is expert order).  Selection compares fp32
// logits: larger first, equal logits -> lower expert index.  Each of the k
// rounds takes every lane's largest remaining key, the wave maximum of those
// (one reduction on the vector ALUs), and the lowest lane holding it (a
// ballot): that lane's lowest expert with the maximum key is the round's
// pick, and the lane retires it.
// Scores: softmax over the experts renormalised over the k selected ones,
// computed as exp(l_s - l_max) / sum_s' exp(l_s' - l_max) with the sum taken
// in slot order (the full-softmax normaliser cancels).  Lane s < k returns
// slot s.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_topk(const float* __restrict__ lrow, int E, int k, int lane,
                                          int* out_e, float* out_w) {
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * lane + i;
        key[i] = e < E ? logit_key(lrow[e]) : 0u;  // key 0: no finite logit, never chosen
    }
    auto umax = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
    float sel_l[kMaxTopK];
    int my_e = 0;
    float my_l = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        sel_l[s] = 0.0f;
        if (s < k) {
            const uint32_t h = umax(umax(key[0], key[1]), umax(key[2], key[3]));
            const uint32_t m = wave_reduce_u32(h, umax);
            // the lowest lane whose largest key is m holds the lowest expert with key m
            const int win = (int)__builtin_ctzll(__ballot(h == m));
            const int i_lo = key[0] == m ? 0 : key[1] == m ? 1 : key[2] == m ? 2 : 3;
            const int e = 4 * win + __builtin_amdgcn_readlane(i_lo, win);
            if (lane == win) {
#pragma unroll
                for (int i = 0; i < 4; ++i) key[i] = i == i_lo ? 0u : key[i];
            }
            sel_l[s] = key_logit(m);
            if (s == lane) {
                my_e = e;
                my_l = sel_l[s];
            }
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) sum += s < k ? expf(sel_l[s] - sel_l[0]) : 0.0f;
    *out_e = lane < k ? my_e : 0;
    *out_w = lane < k ? expf(my_l - sel_l[0]) / sum : 0.0f;
}

}  // namespace q4moe
