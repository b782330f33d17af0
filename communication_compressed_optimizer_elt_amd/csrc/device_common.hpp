// device_common.hpp -- device helpers of libdemo (gfx950, wave64).
//
// Work unit: one wavefront owns a "group" of 64 consecutive chunks (2048
// elements, 8 KB per fp32 array).  Global memory is streamed in the coalesced
// order (lane l, register r holds elements 256r + 4l .. +3 of the group) and
// turned into one-chunk-per-lane order through a per-wave LDS tile in which
// chunk c's float4 number q sits at slot q ^ (c & 7).  With that XOR swizzle
// both the coalesced float4 accesses (8 lanes cover one chunk) and the
// per-lane accesses (8 lanes cover 8 chunks) hit all 32 banks once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace demo {

constexpr int kChunk = 32;
constexpr int kWave = 64;
constexpr int kGroupElems = kWave * kChunk;  // 2048
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kTabStride = 33;  // LDS basis table row stride (floats)

#include "dct32_consts.inc"

// float index inside a wave's 2048-float LDS tile of chunk c, position i
__device__ __forceinline__ int swz(int c, int i) {
    return c * kChunk + ((((i >> 2) ^ (c & 7))) << 2) + (i & 3);
}

// Order LDS traffic of one wavefront: wait for its LDS operations and keep
// the compiler from moving memory accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Workgroups are handed to the chip's 8 XCDs round-robin by id.  Renumber
// them so that each XCD takes runs of S consecutive ids: block b, the
// (b / 8)-th block XCD b % 8 receives, goes to run (b / 8) / S of that XCD,
// and the runs of the 8 XCDs interleave, so the whole chip sweeps the shard
// front to back while each XCD works on S blocks in a row.  Payload words
// that neighbouring groups share in one 128-byte line (the 8-byte plane words
// of 16 groups = 4 blocks at k = 1) are then written, or fetched, through one
// L2.  Ids past the last whole set of 8*S runs keep their number.
//
// The run length is the kernel's: on the OLMo2-1B half shard (639,697,920
// parameters) the encodes measured fastest with S = 4 (DeMo k = 1: 1.244 ms
// against 1.302 ms with one contiguous range per XCD; Random n = 8: 1.273
// against 1.308 ms; with non-temporal momentum streams 1.160 against 1.184 ms
// at S = 8 and 1.203 ms at S = 2).  The decodes, whose theta is stored by
// non-temporal stores, run fastest with S = 8 (DeMo k = 1: 0.786 against
// 0.804 ms at S = 16 and 0.838 ms at S = 4; Random n = 8: 0.790 against 0.815
// ms; R = 64 equal or faster), except the Decoupled AdamW few-entry DCT decode
// (plain theta stores), which keeps S = 16 (1.317 against 1.376 ms at S = 8).
// Run lengths that are not powers of two (2, 3, 6, 12, 24) measured slower.
constexpr uint32_t kXcds = 8;
constexpr uint32_t kEncodeRun = 4;
constexpr uint32_t kDecodeRun = 8;
constexpr uint32_t kDecodeRunAdamwDct = 16;
// The DiLoCo momentum pass (m <- beta*m + g, one group per wave, one block
// per CU): S = 16, 1.135 ms against 1.161 ms at S = 4, 1.153 at 32 and 1.183
// at 64 (the earlier one-float4-per-work-item grid: 1.190 ms).
constexpr uint32_t kMomentumRun = 16;

template <uint32_t S>
__device__ __forceinline__ uint32_t xcd_block(uint32_t b, uint32_t nb) {
    const uint32_t whole = nb - nb % (kXcds * S);
    if (b >= whole) return b;
    const uint32_t x = b % kXcds, pos = b / kXcds;
    return ((pos / S) * kXcds + x) * S + pos % S;
}

__device__ __forceinline__ float sgnf(float x) {
    return x > 0.f ? 1.f : (x < 0.f ? -1.f : 0.f);
}

// ------------------------------------------------------------------------
// 32-point orthonormal DCT-II and its inverse by even/odd splitting.
// ------------------------------------------------------------------------

template <int H>
__device__ __forceinline__ float odd_row(const float (&M)[H][H], int p, const float* b) {
    float acc = M[p][0] * b[0];
#pragma unroll
    for (int i = 1; i < H; i++) acc = fmaf(M[p][i], b[i], acc);
    return acc;
}

template <int H>
__device__ __forceinline__ float odd_col(const float (&M)[H][H], int i, const float* y) {
    float acc = M[0][i] * y[0];
#pragma unroll
    for (int p = 1; p < H; p++) acc = fmaf(M[p][i], y[p], acc);
    return acc;
}

__device__ __forceinline__ void dct32(const float (&u)[32], float (&X)[32]) {
    float a[16], b[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        a[i] = u[i] + u[31 - i];
        b[i] = u[i] - u[31 - i];
    }
#pragma unroll
    for (int p = 0; p < 16; p++) X[2 * p + 1] = odd_row<16>(kOdd32, p, b);
    float a2[8], b2[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        a2[i] = a[i] + a[15 - i];
        b2[i] = a[i] - a[15 - i];
    }
#pragma unroll
    for (int p = 0; p < 8; p++) X[4 * p + 2] = odd_row<8>(kOdd16, p, b2);
    float a3[4], b3[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        a3[i] = a2[i] + a2[7 - i];
        b3[i] = a2[i] - a2[7 - i];
    }
#pragma unroll
    for (int p = 0; p < 4; p++) X[8 * p + 4] = odd_row<4>(kOdd8, p, b3);
    float a4[2], b4[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        a4[i] = a3[i] + a3[3 - i];
        b4[i] = a3[i] - a3[3 - i];
    }
#pragma unroll
    for (int p = 0; p < 2; p++) X[16 * p + 8] = odd_row<2>(kOdd4, p, b4);
    X[0] = kDC * (a4[0] + a4[1]);
    X[16] = kOdd2 * (a4[0] - a4[1]);
}

__device__ __forceinline__ void idct32(const float (&X)[32], float (&u)[32]) {
    float e2[2];
    {
        float E = kDC * X[0], O = kOdd2 * X[16];
        e2[0] = E + O;
        e2[1] = E - O;
    }
    float e4[4];
    {
        float y[2] = {X[8], X[24]};
#pragma unroll
        for (int i = 0; i < 2; i++) {
            float O = odd_col<2>(kOdd4, i, y);
            e4[i] = e2[i] + O;
            e4[3 - i] = e2[i] - O;
        }
    }
    float e8[8];
    {
        float y[4] = {X[4], X[12], X[20], X[28]};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float O = odd_col<4>(kOdd8, i, y);
            e8[i] = e4[i] + O;
            e8[7 - i] = e4[i] - O;
        }
    }
    float e16[16];
    {
        float y[8];
#pragma unroll
        for (int p = 0; p < 8; p++) y[p] = X[4 * p + 2];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float O = odd_col<8>(kOdd16, i, y);
            e16[i] = e8[i] + O;
            e16[15 - i] = e8[i] - O;
        }
    }
    {
        float y[16];
#pragma unroll
        for (int p = 0; p < 16; p++) y[p] = X[2 * p + 1];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            float O = odd_col<16>(kOdd32, i, y);
            u[i] = e16[i] + O;
            u[31 - i] = e16[i] - O;
        }
    }
}

// ------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 products with the
// Weyl key schedule.
// ------------------------------------------------------------------------

__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1, uint32_t (&w)[4]) {
#pragma unroll
    for (int r = 0; r < 10; r++) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    w[0] = c0;
    w[1] = c1;
    w[2] = c2;
    w[3] = c3;
}

// Position of the r-th (from 0) clear bit of mask, r < number of clear bits:
// a binary search on population counts of the complement.
__device__ __forceinline__ uint32_t nth_clear_bit(uint32_t mask, uint32_t r) {
    uint32_t z = ~mask, pos = 0, c;
    c = __popc(z & 0xFFFFu);
    if (r >= c) { r -= c; z >>= 16; pos += 16; }
    c = __popc(z & 0xFFu);
    if (r >= c) { r -= c; z >>= 8; pos += 8; }
    c = __popc(z & 0xFu);
    if (r >= c) { r -= c; z >>= 4; pos += 4; }
    c = __popc(z & 0x3u);
    if (r >= c) { r -= c; z >>= 2; pos += 2; }
    c = z & 1u;
    if (r >= c) { pos += 1; }
    return pos;
}

constexpr uint32_t kTagSelect = 1u;

// n shared-seed positions of chunk `chunk` at step `step_lo` (Random scheme):
// draw i takes word i%4 of block i/4, scales it to the 32-i free positions
// by a 32x32 high product and marks that free position.
__device__ __forceinline__ uint32_t random_mask(uint64_t seed, uint32_t step_lo, uint64_t chunk, int n) {
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const uint32_t c0 = (uint32_t)chunk, c1 = (uint32_t)(chunk >> 32);
    uint32_t mask = 0;
    for (int blk = 0; blk * 4 < n; blk++) {
        uint32_t w[4];
        philox4x32_10(c0, c1, step_lo, (kTagSelect << 24) | (uint32_t)blk, k0, k1, w);
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int i = blk * 4 + t;
            if (i < n) {
                const uint32_t r = __umulhi(w[t], (uint32_t)(kChunk - i));
                mask |= 1u << nth_clear_bit(mask, r);
            }
        }
    }
    return mask;
}

}  // namespace demo
