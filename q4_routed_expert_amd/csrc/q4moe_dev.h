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

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Dequantise one 32-bit word of eight 4-bit codes (lowest nibble = lowest k)
// with the group's scale s and bias b into eight bf16 weights in k order:
// w = bf16(q * s + b).  q*s is exact in fp32 (at most 12 significant bits) and
// so is the sum whenever the exponents of s and b lie within 12 of each other,
// so the single fp32 fma followed by the round-to-nearest-even conversion
// gives the nearest bf16 to the exact affine value.
//
// 23 VALU instructions per word: 3 to split the even and odd codes into the
// four bytes of two words, 8 v_cvt_f32_ubyte{0..3} (each converts one byte in
// place), 8 v_fma_f32 and 4 v_cvt_pk_bf16_f32.  The empty asm statements hide
// the masks from known-bits analysis, which would otherwise turn each byte
// read into a 4-bit extract plus a separate convert.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s, float b) {
    uint32_t ev = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6 in bytes 0..3
    uint32_t od = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
    asm("" : "+v"(ev));
    asm("" : "+v"(od));
    u32x4 r;
    r[0] = pack_bf16x2(__builtin_fmaf((float)(ev & 0xFFu), s, b),
                       __builtin_fmaf((float)(od & 0xFFu), s, b));
    r[1] = pack_bf16x2(__builtin_fmaf((float)((ev >> 8) & 0xFFu), s, b),
                       __builtin_fmaf((float)((od >> 8) & 0xFFu), s, b));
    r[2] = pack_bf16x2(__builtin_fmaf((float)((ev >> 16) & 0xFFu), s, b),
                       __builtin_fmaf((float)((od >> 16) & 0xFFu), s, b));
    r[3] = pack_bf16x2(__builtin_fmaf((float)(ev >> 24), s, b),
                       __builtin_fmaf((float)(od >> 24), s, b));
    return __builtin_bit_cast(bf16x8, r);
}

// acc + sum over the eight weights of one code word of bf16(q*s + b) * v, with
// v the matching eight bf16 activations as four packed pairs in k order
// (v_dot2_f32_bf16: both products and the sum in fp32).
// (The activations are reinterpreted as one bf16x8 and split with shuffles:
// a bit cast of each 32-bit element separately was compiled into four uses of
// element 0.)
__device__ __forceinline__ float dot8_bf16(uint32_t w, float s, float b, u32x4 v, float acc) {
    const bf16x8 wv = dequant8(w, s, b);
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

// Ordering key for "larger logit first, equal logits -> lower expert index":
// a larger key wins.  -0.0 is folded onto +0.0 so that the two tie.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
    if (v == 0.0f) v = 0.0f;
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0xFFFFu - (uint32_t)e);
}

__device__ __forceinline__ int topk_key_expert(uint64_t key) {
    return (int)(0xFFFFu - (uint32_t)(key & 0xFFFFu));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
        uint64_t w = ((uint64_t)hi << 32) | lo;
        v = w > v ? w : v;
    }
    return v;
}

// ---------------------------------------------------------------------------
// Top-k of one token's logits by one wave (E <= 256: four logits per lane).
// Selection compares fp32 logits: larger first, equal -> lower expert index.
// Scores: softmax over the experts renormalised over the k selected ones,
// computed as exp(l_s - l_max) / sum_s' exp(l_s' - l_max) (the full-softmax
// normaliser cancels).  Lane s < k returns slot s.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_topk(const float* __restrict__ lrow, int E, int k, int lane,
                                          int* out_e, float* out_w) {
    uint64_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? topk_key(lrow[e], e) : 0ull;
    }
    float sel_l[kMaxTopK];
    int sel_e[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        sel_l[s] = 0.0f;
        sel_e[s] = 0;
        if (s < k) {
            uint64_t b = key[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) b = key[i] > b ? key[i] : b;
            b = wave_max_u64(b);
            const int e = topk_key_expert(b);
            if ((e & 63) == lane) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (i == (e >> 6)) key[i] = 0ull;
            }
            sel_e[s] = e;
            sel_l[s] = lrow[e];
        }
    }
    float ex[kMaxTopK], sum = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        ex[s] = s < k ? expf(sel_l[s] - sel_l[0]) : 0.0f;
        sum += ex[s];
    }
    *out_e = 0;
    *out_w = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
        if (s == lane) {
            *out_e = sel_e[s];
            *out_w = ex[s] / sum;
        }
}

}  // namespace q4moe
