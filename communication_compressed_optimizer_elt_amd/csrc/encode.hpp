// encode.hpp -- encode kernels of libdemo for gfx950: momentum (or AdamW's
// moments), chunk transform, slot selection, payload packing and error
// feedback (DeToNATION notes, Algorithm 1 steps 3-5).
#pragma once

#include "kernels.hpp"

namespace demo {

// ------------------------------------------------------------ encode (DCT) --
//
// KS > 0: k <= KS, selection by k argmax passes, q by sparse inverse
//         transform from the LDS basis table.
// KS = 0: any k, selection mask, q by the full inverse transform.

template <int KS, int VF, bool WQ, bool AD>
__global__ __launch_bounds__(kBlock) void encode_dct_kernel(EncArgs a) {
    __shared__ float tab[kChunk * kTabStride];
    __shared__ __attribute__((aligned(16))) float stage_all[kWavesPerBlock * kGroupElems];
    if (KS > 0) fill_basis_table(tab);

    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float* st = stage_all + wv * kGroupElems;
    const int k = a.k;

    {
        const uint64_t grp = (uint64_t)xcd_block<kEncodeRun>(blockIdx.x, gridDim.x) * kWavesPerBlock + wv;
        if (grp >= a.G) return;
        const uint64_t base = grp * kGroupElems;
        const bool full = base + kGroupElems <= a.n;
        const uint64_t c = grp * kWave + lane;
        const bool valid = c < a.C;

        float4 uc[8];
        load_u<AD, !AD>(a, base, full, lane, uc);
        wave_lds_sync();
        put_coalesced(st, lane, uc);
        wave_lds_sync();
        float u[32];
        get_chunk(st, lane, u);

        float X[32];
        dct32(u, X);

        float q[32], mo[32];  // extracted component and feedback m' = u - q
#pragma unroll
        for (int i = 0; i < 32; i++) q[i] = 0.f;
        bool mo_done = false;  // the generic-k form may produce m' directly

        uint64_t mynz = 0, myneg = 0;

        if constexpr (KS > 0) {
            int selj[KS];
            float selv[KS];
            float ax[32];
#pragma unroll
            for (int j = 0; j < 32; j++) ax[j] = fabsf(X[j]);
#pragma unroll
            for (int p = 0; p < KS; p++) {
                if (p < k) {
                    float best = -1.f, bx = 0.f;
                    int bj = 0;
#pragma unroll
                    for (int j = 0; j < 32; j++) {
                        const bool gt = ax[j] > best;
                        best = gt ? ax[j] : best;
                        bx = gt ? X[j] : bx;
                        bj = gt ? j : bj;
                    }
                    selj[p] = bj;
                    selv[p] = bx;
                    if (p + 1 < k) {
#pragma unroll
                        for (int j = 0; j < 32; j++) ax[j] = (j == bj) ? -1.f : ax[j];
                    }
                } else {
                    selj[p] = kChunk + p;
                    selv[p] = 0.f;
                }
            }
            // ascending position order
#pragma unroll
            for (int pass = 0; pass < KS; pass++) {
#pragma unroll
                for (int i = pass & 1; i + 1 < KS; i += 2) {
                    const bool sw = selj[i] > selj[i + 1];
                    const int j0 = sw ? selj[i + 1] : selj[i];
                    const int j1 = sw ? selj[i] : selj[i + 1];
                    const float v0 = sw ? selv[i + 1] : selv[i];
                    const float v1 = sw ? selv[i] : selv[i + 1];
                    selj[i] = j0;
                    selj[i + 1] = j1;
                    selv[i] = v0;
                    selv[i + 1] = v1;
                }
            }
            // q = sum_s X_js * B[js][:]
#pragma unroll
            for (int p = 0; p < KS; p++) {
                if (p < k) {
                    const float x = selv[p];
                    const float* t = tab + selj[p];
#pragma unroll
                    for (int i = 0; i < 32; i++) q[i] = fmaf(x, t[i * kTabStride], q[i]);
                }
            }
            // payload
            if (valid) {
                uint8_t* idx = a.pay + a.idx_off + c * (uint64_t)k;
                if constexpr (KS == 1) {
                    idx[0] = (uint8_t)selj[0];
                } else if constexpr (KS == 2) {
                    *reinterpret_cast<uint16_t*>(idx) = (uint16_t)(selj[0] | (selj[1] << 8));
                } else {
                    if (KS == 4 && k == 4) {
                        *reinterpret_cast<uint32_t*>(idx) = (uint32_t)selj[0] | ((uint32_t)selj[1] << 8) |
                                                            ((uint32_t)selj[2] << 16) | ((uint32_t)selj[KS - 1] << 24);
                    } else {
#pragma unroll
                        for (int p = 0; p < KS; p++)
                            if (p < k) idx[p] = (uint8_t)selj[p];
                    }
                }
                if (VF == VF_F32) {
                    float* val = reinterpret_cast<float*>(a.pay + a.val_off) + c * (uint64_t)k;
#pragma unroll
                    for (int p = 0; p < KS; p++)
                        if (p < k) val[p] = wire_f32(selv[p], a.sign);
                } else if (VF == VF_F16) {
                    uint16_t* val = reinterpret_cast<uint16_t*>(a.pay + a.val_off) + c * (uint64_t)k;
#pragma unroll
                    for (int p = 0; p < KS; p++)
                        if (p < k) val[p] = wire_f16(selv[p], a.sign);
                }
            }
            if (VF == VF_TERNARY) {
#pragma unroll
                for (int p = 0; p < KS; p++) {
                    if (p < k) {
                        const uint64_t nzb = __ballot(valid && selv[p] != 0.f);
                        const uint64_t negb = __ballot(valid && selv[p] < 0.f);
                        if (lane == p) {
                            mynz = nzb;
                            myneg = negb;
                        }
                    }
                }
            }
        } else {
            // generic k: k argmax passes build the selection mask
            float ax[32];
#pragma unroll
            for (int j = 0; j < 32; j++) ax[j] = fabsf(X[j]);
            uint32_t S = 0;
            for (int p = 0; p < k; p++) {
                float best = -1.f;
                int bj = 0;
#pragma unroll
                for (int j = 0; j < 32; j++) {
                    const bool gt = ax[j] > best;
                    best = gt ? ax[j] : best;
                    bj = gt ? j : bj;
                }
                S |= 1u << bj;
#pragma unroll
                for (int j = 0; j < 32; j++) ax[j] = (j == bj) ? -1.f : ax[j];
            }
            // With more than half the coefficients kept, m' is taken as the
            // inverse transform of the ones left behind and q = u - m' (the same
            // values: its rounding then scales with the smaller, unselected
            // coefficients, and k = 32 gives m' = 0 and q = u exactly).
            const bool rest = 2 * k > kChunk;
            float Xs[32];
#pragma unroll
            for (int j = 0; j < 32; j++) Xs[j] = (((S >> j) & 1u) != 0u) != rest ? X[j] : 0.f;
            if (rest) {
                idct32(Xs, mo);
#pragma unroll
                for (int i = 0; i < 32; i++) q[i] = u[i] - mo[i];
                mo_done = true;
            } else {
                idct32(Xs, q);
            }
            // slots in ascending position order
            uint32_t nzv = 0, negv = 0;
            int s = 0;
            uint8_t* idx = a.pay + a.idx_off + c * (uint64_t)k;
#pragma unroll
            for (int j = 0; j < 32; j++) {
                if ((S >> j) & 1u) {
                    nzv |= (X[j] != 0.f ? 1u : 0u) << s;
                    negv |= (X[j] < 0.f ? 1u : 0u) << s;
                    if (valid) {
                        idx[s] = (uint8_t)j;
                        if (VF == VF_F32)
                            (reinterpret_cast<float*>(a.pay + a.val_off) + c * (uint64_t)k)[s] = wire_f32(X[j], a.sign);
                        else if (VF == VF_F16)
                            (reinterpret_cast<uint16_t*>(a.pay + a.val_off) + c * (uint64_t)k)[s] = wire_f16(X[j], a.sign);
                    }
                    s++;
                }
            }
            if (VF == VF_TERNARY) {
                for (int p = 0; p < k; p++) {
                    const uint64_t nzb = __ballot(valid && ((nzv >> p) & 1u));
                    const uint64_t negb = __ballot(valid && ((negv >> p) & 1u));
                    if (lane == p) {
                        mynz = nzb;
                        myneg = negb;
                    }
                }
            }
        }

        if (VF == VF_TERNARY && lane < k) {
            reinterpret_cast<uint64_t*>(a.pay + a.nz_off)[grp * (uint64_t)k + lane] = mynz;
            reinterpret_cast<uint64_t*>(a.pay + a.neg_off)[grp * (uint64_t)k + lane] = myneg;
        }

        // m <- u - q, back through LDS to coalesced order
        if (!mo_done) {
#pragma unroll
            for (int i = 0; i < 32; i++) mo[i] = u[i] - q[i];
        }
        put_chunk(st, lane, mo);
        wave_lds_sync();
        float4 outc[8];
        get_coalesced(st, lane, outc);
        store_tile<!AD>(a.m, base, a.n, full, lane, outc);
        if constexpr (WQ) {
            wave_lds_sync();
            put_chunk(st, lane, q);
            wave_lds_sync();
            get_coalesced(st, lane, outc);
            store_tile(a.q_out, base, a.n, full, lane, outc);
        }
    }
}

// Ternary slot values (bit s of nzv / negv) of chunk c as fp32 or fp16
// numbers, 16-byte stores where k allows.
template <int VF>
__device__ __forceinline__ void store_slot_values(uint8_t* val, uint64_t c, int k, uint32_t nzv, uint32_t negv) {
    auto value = [&](int s) { return ((nzv >> s) & 1u) ? (((negv >> s) & 1u) ? -1.f : 1.f) : 0.f; };
    if (VF == VF_F32) {
        float* v = reinterpret_cast<float*>(val) + c * (uint64_t)k;
        if ((k & 3) == 0) {
#pragma unroll
            for (int s = 0; s < 32; s += 4)
                if (s < k) *reinterpret_cast<float4*>(v + s) = make_float4(value(s), value(s + 1), value(s + 2), value(s + 3));
        } else {
            for (int s = 0; s < k; s++) v[s] = value(s);
        }
    } else {
        uint16_t* v = reinterpret_cast<uint16_t*>(val) + c * (uint64_t)k;
        if ((k & 7) == 0) {
#pragma unroll
            for (int s = 0; s < 32; s += 8)
                if (s < k) {
                    uint32_t w[4];
#pragma unroll
                    for (int t = 0; t < 4; t++)
                        w[t] = (uint32_t)f16_of_sign(value(s + 2 * t)) | ((uint32_t)f16_of_sign(value(s + 2 * t + 1)) << 16);
                    *reinterpret_cast<uint4*>(v + s) = make_uint4(w[0], w[1], w[2], w[3]);
                }
        } else {
            for (int s = 0; s < k; s++) v[s] = f16_of_sign(value(s));
        }
    }
}

// Slot values of chunk c taken as they are (sign off): slot s is the s-th
// set position of mask, read from the lane's row of the LDS tile holding u.
template <int VF>
__device__ __forceinline__ void store_slot_raw(uint8_t* val, uint64_t c, int k, const float* st, int lane,
                                               uint32_t mask) {
    uint32_t mm = mask;
    for (int s = 0; s < k; s++) {
        const uint32_t j = __builtin_ctz(mm) & 31u;  // mm keeps k set bits for k draws
        mm &= mm - 1u;
        const float x = st[swz(lane, (int)j)];
        if (VF == VF_F32)
            reinterpret_cast<float*>(val)[c * (uint64_t)k + s] = x;
        else
            reinterpret_cast<uint16_t*>(val)[c * (uint64_t)k + s] = f16_bits(x);
    }
}

// ---------------------------------------- encode (Random / Striding / DiLoCo) --

template <int VF, bool WQ, bool AD>
__global__ __launch_bounds__(kBlock) void encode_sel_kernel(EncArgs a) {
    __shared__ __attribute__((aligned(16))) float stage_all[kWavesPerBlock * kGroupElems];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float* st = stage_all + wv * kGroupElems;
    const int k = a.k;

    {
        const uint64_t grp = (uint64_t)xcd_block<kEncodeRun>(blockIdx.x, gridDim.x) * kWavesPerBlock + wv;
        if (grp >= a.G) return;
        const uint64_t base = grp * kGroupElems;
        const bool full = base + kGroupElems <= a.n;
        const uint64_t c = grp * kWave + lane;
        const bool valid = c < a.C;

        float4 uc[8];
        load_u<AD, true>(a, base, full, lane, uc);
        wave_lds_sync();
        put_coalesced(st, lane, uc);
        wave_lds_sync();
        float u[32];
        get_chunk(st, lane, u);

        const uint32_t mask = a.random ? random_mask(a.seed, a.step_lo, a.chunk_offset + c, k) : a.mask;

        uint32_t nzpos = 0, negpos = 0;
        float mo[32];
#pragma unroll
        for (int j = 0; j < 32; j++) {
            const bool sel = (mask >> j) & 1u;
            nzpos |= ((sel && u[j] != 0.f) ? 1u : 0u) << j;
            negpos |= ((sel && u[j] < 0.f) ? 1u : 0u) << j;
            mo[j] = sel ? 0.f : u[j];
        }
        // slot s = s-th selected position in ascending order
        uint32_t nzv = 0, negv = 0, mm = mask;
        for (int s = 0; s < k; s++) {
            const uint32_t j = __builtin_ctz(mm) & 31u;  // mm keeps k set bits for k draws
            mm &= mm - 1u;
            nzv |= ((nzpos >> j) & 1u) << s;
            negv |= ((negpos >> j) & 1u) << s;
        }

        if (VF == VF_TERNARY) {
            uint64_t mynz = 0, myneg = 0;
            for (int s = 0; s < k; s++) {
                const uint64_t nzb = __ballot(valid && ((nzv >> s) & 1u));
                const uint64_t negb = __ballot(valid && ((negv >> s) & 1u));
                if (lane == s) {
                    mynz = nzb;
                    myneg = negb;
                }
            }
            if (lane < k) {
                reinterpret_cast<uint64_t*>(a.pay + a.nz_off)[grp * (uint64_t)k + lane] = mynz;
                reinterpret_cast<uint64_t*>(a.pay + a.neg_off)[grp * (uint64_t)k + lane] = myneg;
            }
        } else if (valid) {
            if (a.sign)
                store_slot_values<VF>(a.pay + a.val_off, c, k, nzv, negv);
            else
                store_slot_raw<VF>(a.pay + a.val_off, c, k, st, lane, mask);
        }

        put_chunk(st, lane, mo);
        wave_lds_sync();
        float4 outc[8];
        get_coalesced(st, lane, outc);
        store_tile<true>(a.m, base, a.n, full, lane, outc);
        if constexpr (WQ) {
            float q[32];
#pragma unroll
            for (int j = 0; j < 32; j++) q[j] = ((mask >> j) & 1u) ? u[j] : 0.f;
            wave_lds_sync();
            put_chunk(st, lane, q);
            wave_lds_sync();
            get_coalesced(st, lane, outc);
            store_tile(a.q_out, base, a.n, full, lane, outc);
        }
    }
}

// DiLoCo between synchronisations: m <- beta*m + g (with AdamW also v),
// nothing extracted.  One wave per 2048-element group, through the encodes'
// load and store paths.
template <bool WQ, bool AD>
__global__ __launch_bounds__(kBlock) void momentum_kernel(EncArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint64_t grp = (uint64_t)xcd_block<kMomentumRun>(blockIdx.x, gridDim.x) * kWavesPerBlock + wv;
    if (grp >= a.G) return;
    const uint64_t base = grp * kGroupElems;
    const bool full = base + kGroupElems <= a.n;
    float4 uc[8];
    load_u<AD, !AD>(a, base, full, lane, uc);
    store_tile<!AD>(a.m, base, a.n, full, lane, uc);
    if constexpr (WQ) {
        const float4 z[8] = {};
        store_tile(a.q_out, base, a.n, full, lane, z);
    }
}

}  // namespace demo
