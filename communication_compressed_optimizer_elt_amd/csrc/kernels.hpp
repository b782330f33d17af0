// kernels.hpp -- kernel arguments and the streaming helpers shared by the
// encode kernels (encode.hpp: DeToNATION notes, Algorithm 1 steps 3-5) and the
// decode kernels (decode.hpp: steps 6-7) of the DeMo / FlexDeMo optimizer step.
//
// One wavefront owns one group of 64 chunks and a block of 4 waves takes 4
// consecutive groups; the grid covers the shard once.  Every array is read and
// written once, in coalesced float4 order; the per-chunk work (transform,
// selection, packing) runs one chunk per lane on an LDS-transposed copy.
#pragma once

#include <hip/hip_fp16.h>

#include "device_common.hpp"

namespace demo {

enum { VF_TERNARY = 0, VF_F16 = 1, VF_F32 = 2 };

struct EncArgs {
    const float* g;
    float* m;
    uint8_t* pay;
    float* q_out;
    uint64_t n, C, G;
    uint64_t idx_off, nz_off, neg_off, val_off;
    uint64_t chunk_offset, seed;
    uint32_t step_lo;
    uint32_t mask;  // shared positions of STRIDE / DILOCO
    float beta;
    float gamma;    // u = beta*m + gamma*g: 1, or 1 - beta1 for AdamW's first moment
    float* v;       // AdamW second moment (nullptr: plain momentum)
    float beta2;
    int k;
    int random;     // 1: positions from random_mask per chunk
    int sign;       // 1: slots carry sign(value); 0: the value itself
};

struct DecArgs {
    float* theta;
    const uint8_t* pay;
    uint64_t stride;
    uint64_t n, C, G;
    uint64_t idx_off, nz_off, neg_off, val_off;
    uint64_t chunk_offset, seed;
    uint32_t step_lo;
    uint32_t mask;
    float lr, invR;
    int k, R;
    int random;
    const float* v;         // AdamW second moment (nullptr: theta -= lr*Q)
    float c1, c2, eps, wd;  // AdamW bias corrections 1/(1-beta^t), eps, weight decay
};

// ---------------------------------------------------------------- streaming --

typedef float f32x4 __attribute__((ext_vector_type(4)));

// read-once stream (gradients): non-temporal load
__device__ __forceinline__ float4 load_stream(const float4* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// write-once stream: non-temporal store (the line is not read again in the
// launch, and the next step reaches it only after gigabytes of other traffic).
// Measured on the OLMo2-1B half shard, one box, interleaved minima: the
// momentum read and rewritten by non-temporal loads and stores, DeMo k = 1
// encode 1.248 -> 1.160 ms, Random n = 8 encode 1.269 -> 1.168 ms, DiLoCo
// momentum pass 1.315 -> 1.241 ms (non-temporal loads alone 1.228 -> 1.278
// ms, stores alone 1.269 -> 1.323 ms on the Random encode: only the pair
// pays); theta stored so in the decodes, DeMo k = 1 0.847 -> 0.803 ms, R = 64
// 1.207 -> 1.139 ms, Random n = 8 0.858 -> 0.822 ms.  Decoupled AdamW, fp32
// values: the second moment read and rewritten so, DCT encode 2.198 -> 2.055
// ms, Random n = 8 encode 2.352 -> 2.295 ms; its momentum too in the Random
// encode (-> 2.189 ms) but not in the DCT encode (2.300 ms with it); its
// decodes read theta after Q and rewrite it the same way (DCT 1.329 -> 1.206
// ms, Random n = 8 1.507 -> 1.433 ms).
__device__ __forceinline__ void store_stream(float4* p, float4 v) {
    __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}

// AdamW second moment: beta2*v + (1 - beta2)*g^2
__device__ __forceinline__ float second_moment(const EncArgs& a, float v, float g) {
    return fmaf(a.beta2, v, (1.f - a.beta2) * (g * g));
}

// u = beta*m + gamma*g for the wave's group, coalesced order; zero beyond n
// (with AdamW the second moment is updated in the same pass, read and
// written by non-temporal loads and stores).  NTM: m is read by non-temporal
// loads (its lines are rewritten by the same wave; pays only together with
// non-temporal stores of m).
template <bool AD, bool NTM>
__device__ __forceinline__ void load_u(const EncArgs& a, uint64_t base, bool full, int lane, float4 (&uc)[8]) {
    if (full) {
        const float4* g4 = reinterpret_cast<const float4*>(a.g + base);
        const float4* m4 = reinterpret_cast<const float4*>(a.m + base);
        float4 gv[8], mv[8];
#pragma unroll
        for (int r = 0; r < 8; r++) {
            gv[r] = load_stream(g4 + r * kWave + lane);
            mv[r] = NTM ? load_stream(m4 + r * kWave + lane) : m4[r * kWave + lane];
        }
        if constexpr (AD) {
            float4* v4 = reinterpret_cast<float4*>(a.v + base);
#pragma unroll
            for (int r = 0; r < 8; r++) {
                float4 vv = load_stream(v4 + r * kWave + lane);
                vv.x = second_moment(a, vv.x, gv[r].x);
                vv.y = second_moment(a, vv.y, gv[r].y);
                vv.z = second_moment(a, vv.z, gv[r].z);
                vv.w = second_moment(a, vv.w, gv[r].w);
                store_stream(v4 + r * kWave + lane, vv);
            }
        }
#pragma unroll
        for (int r = 0; r < 8; r++) {
            uc[r].x = fmaf(a.beta, mv[r].x, AD ? a.gamma * gv[r].x : gv[r].x);
            uc[r].y = fmaf(a.beta, mv[r].y, AD ? a.gamma * gv[r].y : gv[r].y);
            uc[r].z = fmaf(a.beta, mv[r].z, AD ? a.gamma * gv[r].z : gv[r].z);
            uc[r].w = fmaf(a.beta, mv[r].w, AD ? a.gamma * gv[r].w : gv[r].w);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 8; r++) {
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint64_t e = base + r * 256 + lane * 4 + t;
                v[t] = 0.f;
                if (e < a.n) {
                    if constexpr (AD) a.v[e] = second_moment(a, a.v[e], a.g[e]);
                    v[t] = fmaf(a.beta, a.m[e], AD ? a.gamma * a.g[e] : a.g[e]);
                }
            }
            uc[r] = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

// coalesced tile -> LDS (chunk-swizzled)
__device__ __forceinline__ void put_coalesced(float* st, int lane, const float4 (&v)[8]) {
#pragma unroll
    for (int r = 0; r < 8; r++)
        *reinterpret_cast<float4*>(st + swz(8 * r + (lane >> 3), 4 * (lane & 7))) = v[r];
}

__device__ __forceinline__ void get_coalesced(const float* st, int lane, float4 (&v)[8]) {
#pragma unroll
    for (int r = 0; r < 8; r++)
        v[r] = *reinterpret_cast<const float4*>(st + swz(8 * r + (lane >> 3), 4 * (lane & 7)));
}

__device__ __forceinline__ void put_chunk(float* st, int lane, const float (&x)[32]) {
#pragma unroll
    for (int q = 0; q < 8; q++)
        *reinterpret_cast<float4*>(st + swz(lane, 4 * q)) =
            make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
}

__device__ __forceinline__ void get_chunk(const float* st, int lane, float (&x)[32]) {
#pragma unroll
    for (int q = 0; q < 8; q++) {
        const float4 v = *reinterpret_cast<const float4*>(st + swz(lane, 4 * q));
        x[4 * q] = v.x;
        x[4 * q + 1] = v.y;
        x[4 * q + 2] = v.z;
        x[4 * q + 3] = v.w;
    }
}

// store a coalesced tile to dst[base ...], guarded beyond n (NT: whole tiles
// by non-temporal stores)
template <bool NT = false>
__device__ __forceinline__ void store_tile(float* dst, uint64_t base, uint64_t n, bool full, int lane,
                                           const float4 (&v)[8]) {
    if (full) {
        float4* d4 = reinterpret_cast<float4*>(dst + base);
#pragma unroll
        for (int r = 0; r < 8; r++) {
            if constexpr (NT)
                store_stream(d4 + r * kWave + lane, v[r]);
            else
                d4[r * kWave + lane] = v[r];
        }
    } else {
#pragma unroll
        for (int r = 0; r < 8; r++) {
            const float t[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const uint64_t e = base + r * 256 + lane * 4 + s;
                if (e < n) dst[e] = t[s];
            }
        }
    }
}

__device__ __forceinline__ void fill_basis_table(float* tab) {
    for (int t = threadIdx.x; t < kChunk * kChunk; t += blockDim.x)
        tab[(t >> 5) * kTabStride + (t & 31)] = kBasisT[t >> 5][t & 31];
    __syncthreads();
}

__device__ __forceinline__ uint16_t f16_of_sign(float v) {
    return v > 0.f ? (uint16_t)0x3C00u : (v < 0.f ? (uint16_t)0xBC00u : (uint16_t)0u);
}

// binary16 bits of v, rounded to nearest even (subnormals kept)
__device__ __forceinline__ uint16_t f16_bits(float v) {
    return __half_as_ushort(__float2half_rn(v));
}

// what a value-format slot carries: sign(v) or v itself
__device__ __forceinline__ float wire_f32(float v, int sign) {
    return sign ? sgnf(v) : v;
}
__device__ __forceinline__ uint16_t wire_f16(float v, int sign) {
    return sign ? f16_of_sign(v) : f16_bits(v);
}

}  // namespace demo
