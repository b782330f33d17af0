// decode.hpp -- decode kernels of libdemo for gfx950: the R replicas'
// payloads summed per chunk, inverse transform and parameter update
// (DeToNATION notes, Algorithm 1 steps 6-7), and the shared-seed position
// kernel behind demo_random_select.
#pragma once

#include "kernels.hpp"

namespace demo {

// ------------------------------------------------------------------ decode --

// Words of a payload, which no kernel of the launch writes, read through the
// constant address space: wave-uniform addresses become scalar loads.
__device__ __forceinline__ uint64_t load_const_u64(const uint8_t* base, uint64_t word) {
    typedef const __attribute__((address_space(4))) uint64_t* const_u64_ptr;
    return ((const_u64_ptr)base)[word];
}

// k slot values of one chunk in a value-format payload (fp32 / fp16), added to
// A; val points at the group's first entry, loff is the lane's entry offset
template <int VF>
__device__ __forceinline__ void add_slot_values(const uint8_t* val, uint32_t loff, int k, float (&A)[32]) {
    if (VF == VF_F32) {
        const float* v = reinterpret_cast<const float*>(val) + loff;
        if ((k & 3) == 0) {
#pragma unroll
            for (int s = 0; s < 32; s += 4)
                if (s < k) {
                    const float4 x = *reinterpret_cast<const float4*>(v + s);
                    A[s] += x.x;
                    A[s + 1] += x.y;
                    A[s + 2] += x.z;
                    A[s + 3] += x.w;
                }
        } else {
#pragma unroll
            for (int s = 0; s < 32; s++)
                if (s < k) A[s] += v[s];
        }
    } else {
        const uint16_t* v = reinterpret_cast<const uint16_t*>(val) + loff;
        if ((k & 7) == 0) {
#pragma unroll
            for (int s = 0; s < 32; s += 8)
                if (s < k) {
                    const uint4 x = *reinterpret_cast<const uint4*>(v + s);
                    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        A[s + 2 * t] += __half2float(__ushort_as_half((uint16_t)(w[t] & 0xFFFFu)));
                        A[s + 2 * t + 1] += __half2float(__ushort_as_half((uint16_t)(w[t] >> 16)));
                    }
                }
        } else {
#pragma unroll
            for (int s = 0; s < 32; s++)
                if (s < k) A[s] += __half2float(__ushort_as_half(v[s]));
        }
    }
}

// this lane's slot value from a plane word pair: NZ ? (NEG ? -1 : +1) : 0
__device__ __forceinline__ float ternary_of(uint64_t nzw, uint64_t negw, int lane) {
    const bool nz = (nzw >> lane) & 1ull;
    const bool ng = (negw >> lane) & 1ull;
    return nz ? (ng ? -1.f : 1.f) : 0.f;
}

// Per-chunk entries (IDX bytes, VAL values) of slot s in replica payload pr:
// a wave-uniform base (replica, group, slot) plus the lane's own offset
// loff = lane*k (0 for lanes past the last chunk), so the loads take a scalar
// base and a 32-bit lane offset.
__device__ __forceinline__ uint64_t group_entry(const DecArgs& a, uint64_t grp, int s) {
    return grp * (uint64_t)(kWave * a.k) + (uint64_t)s;
}

__device__ __forceinline__ int slot_index(const DecArgs& a, const uint8_t* pr, uint64_t grp, int s, uint32_t loff) {
    return (pr + a.idx_off + group_entry(a, grp, s))[loff] & 31;
}

template <int VF>
__device__ __forceinline__ float slot_value(const DecArgs& a, const uint8_t* pr, uint64_t grp, int s, uint32_t loff,
                                            int lane) {
    if (VF == VF_TERNARY) {
        // plain (vector) loads of the wave-uniform words: measured faster here
        // than scalar loads, whose waits also cover the LDS table reads
        const uint64_t w = grp * (uint64_t)a.k + s;
        return ternary_of(reinterpret_cast<const uint64_t*>(pr + a.nz_off)[w],
                          reinterpret_cast<const uint64_t*>(pr + a.neg_off)[w], lane);
    } else if (VF == VF_F32) {
        return (reinterpret_cast<const float*>(pr + a.val_off) + group_entry(a, grp, s))[loff];
    } else {
        return __half2float(
            __ushort_as_half((reinterpret_cast<const uint16_t*>(pr + a.val_off) + group_entry(a, grp, s))[loff]));
    }
}

// One parameter's update: theta - lr*Q, or with AdamW
// theta - lr*(c1*Q/(sqrt(c2*v) + eps) + wd*theta).
template <bool AD>
__device__ __forceinline__ float param_step(const DecArgs& a, float th, float q, float v) {
    if constexpr (AD) return th - a.lr * (a.c1 * q / (sqrtf(a.c2 * v) + a.eps) + a.wd * th);
    return fmaf(-a.lr, q, th);
}

__device__ __forceinline__ float4 adamw_step4(const DecArgs& a, float4 th, float4 q, float4 v) {
    return make_float4(param_step<true>(a, th.x, q.x, v.x), param_step<true>(a, th.y, q.y, v.y),
                       param_step<true>(a, th.z, q.z, v.z), param_step<true>(a, th.w, q.w, v.w));
}

// theta <- theta - lr * Q (param_step) with Q in coalesced order from the LDS tile
template <bool AD>
__device__ __forceinline__ void apply_update(const DecArgs& a, const float* st, uint64_t base, bool full, int lane) {
    float4 qc[8];
    get_coalesced(st, lane, qc);
    if (full) {
        float4* t4 = reinterpret_cast<float4*>(a.theta + base);
        float4 tv[8], vv[8];
#pragma unroll
        for (int r = 0; r < 8; r++) tv[r] = t4[r * kWave + lane];
        if constexpr (AD) {
            const float4* v4 = reinterpret_cast<const float4*>(a.v + base);
#pragma unroll
            for (int r = 0; r < 8; r++) vv[r] = v4[r * kWave + lane];
        }
#pragma unroll
        for (int r = 0; r < 8; r++) {
            if constexpr (AD)
                tv[r] = adamw_step4(a, tv[r], qc[r], vv[r]);
            else {
                tv[r].x = fmaf(-a.lr, qc[r].x, tv[r].x);
                tv[r].y = fmaf(-a.lr, qc[r].y, tv[r].y);
                tv[r].z = fmaf(-a.lr, qc[r].z, tv[r].z);
                tv[r].w = fmaf(-a.lr, qc[r].w, tv[r].w);
            }
            t4[r * kWave + lane] = tv[r];
        }
    } else {
#pragma unroll
        for (int r = 0; r < 8; r++) {
            const float qq[4] = {qc[r].x, qc[r].y, qc[r].z, qc[r].w};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint64_t e = base + r * 256 + lane * 4 + t;
                if (e < a.n) a.theta[e] = param_step<AD>(a, a.theta[e], qq[t], AD ? a.v[e] : 0.f);
            }
        }
    }
}

// The same update with the theta tile loaded up front (prefetch_theta at the
// start of every decode kernel, so its latency overlaps the payload work), by
// non-temporal loads: each theta line is read once and then rewritten by the
// same wave.  On the OLMo2-1B half shard the non-temporal prefetch measured
// 4-8% faster than plain loads for the R = 2 decodes (DeMo k = 1 0.902 ->
// 0.850 ms, Random n = 8 0.921 -> 0.863 ms, fp32 values 1.124 -> 1.040 ms)
// and the R = 64 Random decode (1.436 -> 1.373 ms); a plain-load prefetch was
// no faster than loading theta after Q in the few-entry DCT decode, and
// non-temporal loads there after Q were 5% slower.
struct ThetaTile {
    float4 v[8];
};

__device__ __forceinline__ void prefetch_theta(const DecArgs& a, uint64_t base, bool full, int lane, ThetaTile& t) {
    if (full) {
        const float4* t4 = reinterpret_cast<const float4*>(a.theta + base);
#pragma unroll
        for (int r = 0; r < 8; r++) t.v[r] = load_stream(t4 + r * kWave + lane);
    }
}

// Decoupled AdamW decodes: the read-only second moment v is the tile loaded up
// front (non-temporal, like theta elsewhere) and theta is read after Q, by
// non-temporal loads, and stored the same way.  Measured on the OLMo2-1B half
// shard, few-entry DCT decode: 1.265 ms against 1.336 ms with both loaded
// after Q and 1.506 ms with theta prefetched (plain theta accesses); with the
// non-temporal theta load and store 1.329 -> 1.206 ms (the load alone: 1.440
// ms).  Selection decode (Random n = 8): 1.507 ms with theta prefetched too
// and stored plainly, 1.433 ms this way.
__device__ __forceinline__ void prefetch_moment2(const DecArgs& a, uint64_t base, bool full, int lane, ThetaTile& t) {
    if (full) {
        const float4* v4 = reinterpret_cast<const float4*>(a.v + base);
#pragma unroll
        for (int r = 0; r < 8; r++) t.v[r] = load_stream(v4 + r * kWave + lane);
    }
}

__device__ __forceinline__ void apply_adamw_moment2_prefetched(const DecArgs& a, const float* st, uint64_t base,
                                                               bool full, int lane, const ThetaTile& v) {
    if (!full) {
        apply_update<true>(a, st, base, full, lane);
        return;
    }
    float4 qc[8], tv[8];
    get_coalesced(st, lane, qc);
    float4* t4 = reinterpret_cast<float4*>(a.theta + base);
#pragma unroll
    for (int r = 0; r < 8; r++) tv[r] = load_stream(t4 + r * kWave + lane);
#pragma unroll
    for (int r = 0; r < 8; r++) store_stream(t4 + r * kWave + lane, adamw_step4(a, tv[r], qc[r], v.v[r]));
}

template <bool AD>
__device__ __forceinline__ void apply_update_prefetched(const DecArgs& a, const float* st, uint64_t base, bool full,
                                                        int lane, ThetaTile& t) {
    if (!full) {
        apply_update<AD>(a, st, base, full, lane);
        return;
    }
    float4 qc[8];
    get_coalesced(st, lane, qc);
    float4* t4 = reinterpret_cast<float4*>(a.theta + base);
    if constexpr (AD) {
        const float4* v4 = reinterpret_cast<const float4*>(a.v + base);
#pragma unroll
        for (int r = 0; r < 8; r++) t4[r * kWave + lane] = adamw_step4(a, t.v[r], qc[r], v4[r * kWave + lane]);
        return;
    }
#pragma unroll
    for (int r = 0; r < 8; r++) {
        float4 tv = t.v[r];
        tv.x = fmaf(-a.lr, qc[r].x, tv.x);
        tv.y = fmaf(-a.lr, qc[r].y, tv.y);
        tv.z = fmaf(-a.lr, qc[r].z, tv.z);
        tv.w = fmaf(-a.lr, qc[r].w, tv.w);
        store_stream(t4 + r * kWave + lane, tv);
    }
}

// Ternary words of many payload entries (entry e = r*k + s: replica r, slot
// s of the wave's group) staged through LDS: each lane fetches whole words
// with coalesced vector loads that all go out together, and stores them as
// {nz.lo, neg.lo, nz.hi, neg.hi}, so that every lane then reads the halves
// holding its own chunk's bits with one LDS read (two addresses per wave).
struct WordStage {
    int lr, ls, rpr;  // this lane's replica and slot within a round; replicas per round
};

__device__ __forceinline__ WordStage word_stage(int k, int lane) {
    WordStage w;
    w.rpr = kWave / k;
    w.lr = lane / k;
    w.ls = lane - w.lr * k;
    return w;
}

// stage replicas [r0, r0 + nrep) of group grp, nrep <= ROUNDS * rpr
template <int ROUNDS>
__device__ __forceinline__ void stage_words(const DecArgs& a, uint64_t grp, uint4* ws, const WordStage& w, int r0,
                                            int nrep) {
    uint64_t nzv[ROUNDS], ngv[ROUNDS];
#pragma unroll
    for (int i = 0; i < ROUNDS; i++) {
        const int r = r0 + i * w.rpr + w.lr;
        const int rc = r < a.R ? r : a.R - 1;  // clamped: every address stays inside the payloads
        const uint8_t* pr = a.pay + (uint64_t)rc * a.stride;
        const uint64_t word = grp * (uint64_t)a.k + w.ls;
        nzv[i] = reinterpret_cast<const uint64_t*>(pr + a.nz_off)[word];
        ngv[i] = reinterpret_cast<const uint64_t*>(pr + a.neg_off)[word] & nzv[i];  // NZ decides
    }
#pragma unroll
    for (int i = 0; i < ROUNDS; i++) {
        const int rl = i * w.rpr + w.lr;
        if (w.lr < w.rpr && rl < nrep)
            ws[rl * a.k + w.ls] = make_uint4((uint32_t)nzv[i], (uint32_t)ngv[i], (uint32_t)(nzv[i] >> 32),
                                             (uint32_t)(ngv[i] >> 32));
    }
}

// ternary value {-1, 0, 1} of bit sh of the halves h = {nz, neg}: NZ - 2 NEG
// (the staged NEG halves are masked with NZ)
__device__ __forceinline__ int lane_ternary(uint2 h, uint32_t sh) {
    const int nz = (int)__builtin_amdgcn_ubfe(h.x, sh, 1u);
    const int ng = (int)__builtin_amdgcn_ubfe(h.y, sh, 1u);
    return nz - 2 * ng;
}

// this lane's ternary value of staged entry e
__device__ __forceinline__ int staged_ternary(const uint4* ws, int e, int lane) {
    const uint2 h = reinterpret_cast<const uint2*>(ws)[2 * e + (lane >> 5)];
    return lane_ternary(h, (uint32_t)lane & 31u);
}

// DCT scheme, few entries per chunk (R*k <= kSparseEntries): Q accumulated
// directly from basis rows of an LDS table.  Measured on the OLMo2-1B half
// shard (DeMo, ternary) against the many-entry decode, both with non-temporal
// theta stores: 4 entries 0.793 against 0.834 ms (R = 4, k = 1) and 0.794
// against 0.835 ms (R = 2, k = 2); 6 entries 0.840 against 0.835 ms; 8
// entries 0.911 against 0.839 ms (R = 8, k = 1) and 0.893 against 0.838 ms
// (R = 4, k = 2).
constexpr int kSparseEntries = 4;

template <int VF, bool AD>
__global__ __launch_bounds__(kBlock) void decode_dct_kernel(DecArgs a) {
    __shared__ float tab[kChunk * kTabStride];
    __shared__ __attribute__((aligned(16))) float stage_all[kWavesPerBlock * kGroupElems];
    fill_basis_table(tab);
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float* st = stage_all + wv * kGroupElems;
    const int k = a.k, R = a.R;

    constexpr uint32_t run = AD ? kDecodeRunAdamwDct : kDecodeRun;
    const uint64_t grp = (uint64_t)xcd_block<run>(blockIdx.x, gridDim.x) * kWavesPerBlock + wv;
    if (grp >= a.G) return;
    const uint64_t base = grp * kGroupElems;
    const bool full = base + kGroupElems <= a.n;
    const uint64_t c = grp * kWave + lane;
    const bool valid = c < a.C;
    const uint32_t loff = valid ? (uint32_t)(lane * k) : 0u;

    // theta loads go out first; the Decoupled AdamW instances (3 blocks per
    // CU, v read beside theta) load v first and theta after Q instead: with
    // plain theta accesses a theta prefetch measured 13% slower there (1.506
    // against 1.329 ms on the OLMo2-1B half shard)
    ThetaTile th;
    if constexpr (AD)
        prefetch_moment2(a, base, full, lane, th);
    else
        prefetch_theta(a, base, full, lane, th);
    float Q[32];
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 32; i++) Q[i] = 0.f;
    for (int r = 0; r < R; r++) {
        const uint8_t* pr = a.pay + (uint64_t)r * a.stride;
        for (int s = 0; s < k; s++) {
            const int j = slot_index(a, pr, grp, s, loff);
            const float v = valid ? slot_value<VF>(a, pr, grp, s, loff, lane) : 0.f;
            const float* t = tab + j;
#pragma unroll
            for (int i = 0; i < 32; i++) Q[i] = fmaf(v, t[i * kTabStride], Q[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 32; i++) Q[i] *= a.invR;
    put_chunk(st, lane, Q);
    wave_lds_sync();
    if constexpr (AD)
        apply_adamw_moment2_prefetched(a, st, base, full, lane, th);
    else
        apply_update_prefetched<AD>(a, st, base, full, lane, th);
}

// DCT scheme, many entries per chunk: the entries are summed per frequency in
// the lane's own counters in the LDS tile, Q is one full inverse transform of
// them.  The counters belong to one lane, so the sums are plain LDS
// read-add-writes (LDS float atomics measured 4x slower here).
//
// Ternary payloads: passes of up to 64 entries stage both the plane words and
// the index bytes of the pass through LDS with coalesced vector loads; each
// lane then reads its index byte and its two plane bits per entry from LDS and
// adds NZ - 2 NEG to its counter of that frequency.  The tile's 8 KB hold the
// counters (4 KB) and the staged index bytes (4 KB).
//  - R < 128 (count_entries8): two banks of int8 counters, entries alternating
//    between them; counter j of a lane sits in a dword of its own column
//    ((j & 7) * 64 + lane), so a wave's accesses hit 64 distinct banks for any
//    positions; four entries share one LDS round trip (two per bank, a repeated
//    position folded into the later write).  The wave runs at raised priority
//    while its theta and payload loads go out.  Measured on the OLMo2-1B half
//    shard at R = 64 against int16 rows with one round trip per entry: 1.198
//    against 1.248 ms, bit-identical (1.211 ms with the priority alone; the
//    conflict-free layout alone 1.236 ms; more waves per CU without the theta
//    prefetch, or block-wide staging of the payload, were slower).
//  - larger R (< 2^15): int16 rows, one read-add-write per entry.
// Value payloads (and ternary with more replicas): fp32 rows, entries in
// batches of 16 whose index and value loads go out before the batch's adds.
constexpr int kDenseBatch = 16;
constexpr int kRowBytes = kWave * kChunk * 2;  // int16 rows of one wave
constexpr int kCount8MaxR = 127;               // |counter| <= R fits int8

// index bytes of replicas [r0, r0 + nrep) of group grp (nrep*k <= 64) into
// is[rl*64k + c*k + s], by 16-byte units; units past the region's entries
// (the last group) are skipped.  From 16 entries per chunk (R*k) on, the
// loads are non-temporal.  Measured on the OLMo2-1B half shard, DeMo decode,
// one box: k = 1, R = 16 879 -> 866 us, R = 48 1030 -> 1010 us; k = 2, R = 8
// 885 -> 868 us, R = 32 1110 -> 1059 us, R = 64 1917 -> 1558 us; with fewer
// entries they were 2-3% slower (k = 1, R = 8 815 -> 841 us).
constexpr int kStreamIndexEntries = 16;

__device__ __forceinline__ void stage_index(const DecArgs& a, uint64_t grp, uint8_t* is, int r0, int nrep,
                                            int lane) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const int k = a.k;
    const int upr = 4 * k;  // 16-byte units per replica row of 64k bytes
    const uint64_t g0 = grp * (uint64_t)(kWave * k);
    const uint64_t lim = a.C * (uint64_t)k;
    const int units = nrep * upr;  // <= 256
    const bool stream = a.R * k >= kStreamIndexEntries;
    uint4 v[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int u = lane + i * kWave;
        const int rl = u / upr, off = (u - rl * upr) * 16;
        ok[i] = u < units && g0 + off < lim;
        const int rc = ok[i] ? r0 + rl : r0;
        const uint64_t oc = ok[i] ? (uint64_t)off : 0;
        const u32x4* p = reinterpret_cast<const u32x4*>(a.pay + (uint64_t)rc * a.stride + a.idx_off + g0 + oc);
        const u32x4 t = stream ? __builtin_nontemporal_load(p) : *p;
        v[i] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
        if (ok[i]) *reinterpret_cast<uint4*>(is + (lane + i * kWave) * 16) = v[i];
}

// Ternary entries of all R replicas into two banks of int8 counters (bank A
// at the tile's bytes [0, 2 KB), bank B at [2 KB, 4 KB); counter j of this
// lane at byte 4 * ((j & 7) * 64 + lane) + (j >> 3) of its bank), staged index
// bytes at [4 KB, 8 KB).  Entries 4i, 4i+2 go to bank A, 4i+1, 4i+3 to bank
// B; the four reads are issued together and, where a bank's two positions
// coincide, the later write carries both values.  A_j = bank A + bank B.
// Drops the wave's priority once a pass's loads have landed.
__device__ __forceinline__ void count_entries8(const DecArgs& a, uint64_t grp, float* st, uint4* ws, int lane,
                                               float (&A)[32]) {
    const int k = a.k, R = a.R;
    uint32_t* cw = reinterpret_cast<uint32_t*>(st);
    int8_t* cA = reinterpret_cast<int8_t*>(st) + 4 * lane;
    int8_t* cB = cA + 2048;
    uint8_t* is = reinterpret_cast<uint8_t*>(st) + kRowBytes;
#pragma unroll
    for (int q = 0; q < 16; q++) cw[q * kWave + lane] = 0u;
    const WordStage w = word_stage(k, lane);
    const int pass = w.rpr;  // replicas per pass: rpr*k <= 64 entries
    const uint2* ws2 = reinterpret_cast<const uint2*>(ws) + (lane >> 5);
    const uint32_t sh = (uint32_t)lane & 31u;
    const int rowstep = kWave * k - k;  // index-byte offset step when the slot wraps
    auto at = [](int8_t* bank, int j) { return bank + (j & 7) * (4 * kWave) + (j >> 3); };
    for (int r0 = 0; r0 < R; r0 += pass) {
        const int nrep = R - r0 < pass ? R - r0 : pass;
        const int ne = nrep * k;
        wave_lds_sync();
        stage_words<1>(a, grp, ws, w, r0, nrep);
        stage_index(a, grp, is, r0, nrep, lane);
        __builtin_amdgcn_s_setprio(0);
        wave_lds_sync();
        const uint8_t* il = is + lane * k;  // entry (rl, s) at il[rl*64k + s]
        int off = 0, s = 0;
        const int nfull = ne - ne % kDenseBatch;
        for (int e0 = 0; e0 < nfull; e0 += kDenseBatch) {
            int jj[kDenseBatch], vi[kDenseBatch];
#pragma unroll
            for (int t = 0; t < kDenseBatch; t++) {
                jj[t] = il[off] & 31;
                const uint2 h = ws2[2 * (e0 + t)];
                vi[t] = (int)__builtin_amdgcn_ubfe(h.x, sh, 1u) - 2 * (int)__builtin_amdgcn_ubfe(h.y, sh, 1u);
                off++;
                if (++s == k) {
                    s = 0;
                    off += rowstep;
                }
            }
#pragma unroll
            for (int t = 0; t < kDenseBatch; t += 4) {
                int8_t* pa0 = at(cA, jj[t]);
                int8_t* pb0 = at(cB, jj[t + 1]);
                int8_t* pa1 = at(cA, jj[t + 2]);
                int8_t* pb1 = at(cB, jj[t + 3]);
                const int8_t xa0 = *pa0, xb0 = *pb0, xa1 = *pa1, xb1 = *pb1;
                const int ya1 = vi[t + 2] + (jj[t] == jj[t + 2] ? vi[t] : 0);
                const int yb1 = vi[t + 3] + (jj[t + 1] == jj[t + 3] ? vi[t + 1] : 0);
                *pa0 = (int8_t)(xa0 + vi[t]);
                *pb0 = (int8_t)(xb0 + vi[t + 1]);
                *pa1 = (int8_t)(xa1 + ya1);
                *pb1 = (int8_t)(xb1 + yb1);
            }
        }
        for (int e = nfull; e < ne; e++) {
            int8_t* p = at(cA, il[off] & 31);
            *p = (int8_t)(*p + lane_ternary(ws2[2 * e], sh));
            off++;
            if (++s == k) {
                s = 0;
                off += rowstep;
            }
        }
    }
    wave_lds_sync();
#pragma unroll
    for (int q = 0; q < 8; q++) {
        const uint32_t va = cw[q * kWave + lane], vb = cw[512 + q * kWave + lane];
#pragma unroll
        for (int b = 0; b < 4; b++)
            A[q + 8 * b] = (float)((int)(int8_t)((va >> (8 * b)) & 0xFFu) + (int)(int8_t)((vb >> (8 * b)) & 0xFFu));
    }
}

template <int VF, bool AD>
__global__ __launch_bounds__(kBlock) void decode_dct_dense_kernel(DecArgs a) {
    __shared__ __attribute__((aligned(16))) float stage_all[kWavesPerBlock * kGroupElems];
    __shared__ uint4 words_all[VF == VF_TERNARY ? kWavesPerBlock * kWave : 1];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float* st = stage_all + wv * kGroupElems;
    uint4* ws = words_all + (VF == VF_TERNARY ? wv * kWave : 0);
    const int k = a.k, R = a.R;

    const uint64_t grp = (uint64_t)xcd_block<kDecodeRun>(blockIdx.x, gridDim.x) * kWavesPerBlock + wv;
    if (grp >= a.G) return;
    const bool counts8 = VF == VF_TERNARY && R <= kCount8MaxR;
    if (counts8) __builtin_amdgcn_s_setprio(3);  // while the loads go out
    const uint64_t base = grp * kGroupElems;
    const bool full = base + kGroupElems <= a.n;
    ThetaTile th;  // theta loads go out first
    prefetch_theta(a, base, full, lane, th);
    const uint64_t c = grp * kWave + lane;
    const bool valid = c < a.C;
    const uint32_t loff = valid ? (uint32_t)(lane * k) : 0u;
    const int rowx = (lane & 7) << 2;  // swz(lane, j) = 32 lane + (j ^ rowx)

    float A[32], Q[32];
    wave_lds_sync();
    if (counts8) {
        count_entries8(a, grp, st, ws, lane, A);
    } else if (VF == VF_TERNARY && R < (1 << 15)) {
        int16_t* row = reinterpret_cast<int16_t*>(st) + lane * kChunk;
        uint8_t* is = reinterpret_cast<uint8_t*>(st) + kRowBytes;
#pragma unroll
        for (int q = 0; q < 4; q++) reinterpret_cast<uint4*>(row)[q] = make_uint4(0u, 0u, 0u, 0u);
        const WordStage w = word_stage(k, lane);
        const int pass = w.rpr;  // replicas per pass: rpr*k <= 64 entries
        const uint2* ws2 = reinterpret_cast<const uint2*>(ws) + (lane >> 5);
        const uint32_t sh = (uint32_t)lane & 31u;
        const int rowstep = kWave * k - k;  // index-byte offset step when the slot wraps
        for (int r0 = 0; r0 < R; r0 += pass) {
            const int nrep = R - r0 < pass ? R - r0 : pass;
            const int ne = nrep * k;
            wave_lds_sync();
            stage_words<1>(a, grp, ws, w, r0, nrep);
            stage_index(a, grp, is, r0, nrep, lane);
            wave_lds_sync();
            const uint8_t* il = is + lane * k;  // entry (rl, s) at il[rl*64k + s]
            int off = 0, s = 0;
            const int nfull = ne - ne % kDenseBatch;
            for (int e0 = 0; e0 < nfull; e0 += kDenseBatch) {
                int jj[kDenseBatch], vi[kDenseBatch];
#pragma unroll
                for (int t = 0; t < kDenseBatch; t++) {
                    jj[t] = il[off] & 31;
                    vi[t] = lane_ternary(ws2[2 * (e0 + t)], sh);
                    off++;
                    if (++s == k) {
                        s = 0;
                        off += rowstep;
                    }
                }
#pragma unroll
                for (int t = 0; t < kDenseBatch; t++) row[jj[t] ^ rowx] += (int16_t)vi[t];
            }
            for (int e = nfull; e < ne; e++) {
                row[(il[off] & 31) ^ rowx] += (int16_t)lane_ternary(ws2[2 * e], sh);
                off++;
                if (++s == k) {
                    s = 0;
                    off += rowstep;
                }
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 32; i++) A[i] = (float)row[i ^ rowx];
    } else {
#pragma unroll
        for (int q = 0; q < 8; q++)
            *reinterpret_cast<float4*>(st + swz(lane, 4 * q)) = make_float4(0.f, 0.f, 0.f, 0.f);
        int r = 0, s = 0;  // replica and slot of the next entry (wave-uniform)
        const int ne = R * k;
        for (int e0 = 0; e0 < ne; e0 += kDenseBatch) {
            int jj[kDenseBatch];
            float vv[kDenseBatch];
#pragma unroll
            for (int t = 0; t < kDenseBatch; t++) {
                const bool live = e0 + t < ne;
                // past the last entry r reaches R with s = 0: clamp the replica
                const int rc = __builtin_amdgcn_readfirstlane(live ? r : R - 1);
                const int sc = __builtin_amdgcn_readfirstlane(s);
                const uint8_t* pr = a.pay + (uint64_t)rc * a.stride;
                jj[t] = slot_index(a, pr, grp, sc, loff);
                const float v = slot_value<VF>(a, pr, grp, sc, loff, lane);
                vv[t] = (live && valid) ? v : 0.f;
                if (++s == k) {
                    s = 0;
                    r++;
                }
            }
#pragma unroll
            for (int t = 0; t < kDenseBatch; t++)
                if (e0 + t < ne) st[lane * kChunk + (jj[t] ^ rowx)] += vv[t];  // the row is this lane's alone
        }
        wave_lds_sync();
        get_chunk(st, lane, A);
    }
    idct32(A, Q);
#pragma unroll
    for (int i = 0; i < 32; i++) Q[i] *= a.invR;
    wave_lds_sync();
    put_chunk(st, lane, Q);
    wave_lds_sync();
    apply_update_prefetched<AD>(a, st, base, full, lane, th);
}

// ---- bit-sliced counting of ternary planes over many replicas -------------
//
// For the position-aligned schemes every replica's slot s covers the same
// chunk positions, so the decode needs, per chunk and slot, the number of set
// NZ bits and set NEG bits over the R replicas (value = #NZ - 2 #NEG).  Lanes
// count whole 32-bit plane halves (32 chunks per operation) into vertical
// bit-plane counters: unit u = 2s + h (slot s, chunk half h) is shared by lpu
// lanes, each adding every lpu-th replica with carry-save adders; a butterfly
// over the unit's lanes adds their counters; the chunk lanes then read their
// bit of each counter plane back from LDS.
constexpr int kSelRounds = 8;  // the 8 KB tile holds the words of 8*64 entries
constexpr int kCountPlanes = 8;  // counters up to 255 replicas
constexpr int kMaxCountLanes = 8;
constexpr int kCountMinR = 8;    // below it per-entry sums are cheaper (measured at R = 2)

// (h, l) = a + b + c as a two-bit column sum, bitwise (carry-save adder)
__device__ __forceinline__ void csa(uint32_t& h, uint32_t& l, uint32_t a, uint32_t b, uint32_t c) {
    const uint32_t u = a ^ b;
    h = (u & c) | (~u & a);
    l = u ^ c;
}

// c += w[0] + ... + w[7], per bit position
__device__ __forceinline__ void count8(uint32_t (&c)[kCountPlanes], const uint32_t (&w)[8]) {
    uint32_t twosA, twosB, foursA, foursB, eights;
    csa(twosA, c[0], c[0], w[0], w[1]);
    csa(twosB, c[0], c[0], w[2], w[3]);
    csa(foursA, c[1], c[1], twosA, twosB);
    csa(twosA, c[0], c[0], w[4], w[5]);
    csa(twosB, c[0], c[0], w[6], w[7]);
    csa(foursB, c[1], c[1], twosA, twosB);
    csa(eights, c[2], c[2], foursA, foursB);
#pragma unroll
    for (int b = 3; b < kCountPlanes; b++) {
        const uint32_t t = c[b] & eights;
        c[b] ^= eights;
        eights = t;
    }
}

// c += (counter of lane ^ d), per bit position
__device__ __forceinline__ void add_partner(uint32_t (&c)[kCountPlanes], int d) {
    uint32_t cy = 0;
#pragma unroll
    for (int b = 0; b < kCountPlanes; b++) {
        const uint32_t o = (uint32_t)__shfl_xor((int)c[b], d);
        const uint32_t t = c[b] ^ o;
        const uint32_t sum = t ^ cy;
        cy = (t & cy) | (~t & c[b]);
        c[b] = sum;
    }
}

// this lane's count (bit sh of every plane) from 8 planes in LDS
__device__ __forceinline__ int read_count(const uint4* planes, uint32_t sh) {
    const uint4 p0 = planes[0], p1 = planes[1];
    const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < kCountPlanes; b++) v |= ((w[b] >> sh) & 1u) << b;
    return (int)v;
}

// T[s] = sum over the R replicas of slot s's ternary value for this lane's
// chunk, R <= 255; st is the wave's 8 KB tile (staging, then counters)
__device__ __forceinline__ void count_ternary(const DecArgs& a, uint64_t grp, float* st, int lane, int (&T)[32]) {
    const int k = a.k, R = a.R;
    uint4* ws = reinterpret_cast<uint4*>(st);
    const WordStage w = word_stage(k, lane);
    const int pass = kSelRounds * w.rpr;
    const int units = 2 * k;
    int lpu = 1;
    while (lpu * 2 * units <= kWave && lpu * 2 <= kMaxCountLanes) lpu *= 2;
    const int u = lane / lpu, j = lane - u * lpu;
    const bool active = u < units;
    const int us = active ? u >> 1 : 0, uh = active ? u & 1 : 0;

    uint32_t cz[kCountPlanes], cn[kCountPlanes];
#pragma unroll
    for (int b = 0; b < kCountPlanes; b++) cz[b] = cn[b] = 0;
    for (int r0 = 0; r0 < R; r0 += pass) {
        const int nrep = R - r0 < pass ? R - r0 : pass;
        wave_lds_sync();
        stage_words<kSelRounds>(a, grp, ws, w, r0, nrep);
        wave_lds_sync();
        const uint2* ws2 = reinterpret_cast<const uint2*>(ws);
        for (int i0 = 0; i0 * lpu < nrep; i0 += 8) {
            uint32_t wz[8], wn[8];
#pragma unroll
            for (int t = 0; t < 8; t++) {
                const int rl = j + (i0 + t) * lpu;
                const bool live = active && rl < nrep;
                const uint2 h = ws2[2 * ((live ? rl : 0) * k + us) + uh];
                wz[t] = live ? h.x : 0u;
                wn[t] = live ? h.y : 0u;
            }
            count8(cz, wz);
            count8(cn, wn);
        }
    }
    for (int d = 1; d < lpu; d *= 2) {
        add_partner(cz, d);
        add_partner(cn, d);
    }
    // counters to LDS: unit u's NZ planes at [4u, 4u+2), NEG planes at [4u+2, 4u+4)
    wave_lds_sync();
    if (active && j == 0) {
        ws[4 * u + 0] = make_uint4(cz[0], cz[1], cz[2], cz[3]);
        ws[4 * u + 1] = make_uint4(cz[4], cz[5], cz[6], cz[7]);
        ws[4 * u + 2] = make_uint4(cn[0], cn[1], cn[2], cn[3]);
        ws[4 * u + 3] = make_uint4(cn[4], cn[5], cn[6], cn[7]);
    }
    wave_lds_sync();
    const uint32_t sh = (uint32_t)lane & 31u;
    const int half = lane >> 5;
#pragma unroll
    for (int s = 0; s < 32; s++)
        if (s < k) {
            const uint4* pl = ws + 4 * (2 * s + half);
            T[s] = read_count(pl, sh) - 2 * read_count(pl + 2, sh);
        }
}

// Random / Striding / DiLoCo: every replica's slot s sits at the s-th selected
// position, so the replicas are summed per slot in registers first (value
// formats: the lane's own k values; ternary planes: few entries as
// wave-uniform scalar word loads; many entries (STAGED) through the word
// stage, by bit-sliced counting from 8 replicas on), then each slot sum is
// written once to its position in the lane's LDS tile and the tile updates
// theta in coalesced order.

template <int VF, bool STAGED, bool AD>
__global__ __launch_bounds__(kBlock) void decode_sel_kernel(DecArgs a) {
    __shared__ __attribute__((aligned(16))) float stage_all[kWavesPerBlock * kGroupElems];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float* st = stage_all + wv * kGroupElems;
    const int k = a.k, R = a.R;

    const uint64_t grp = (uint64_t)xcd_block<kDecodeRun>(blockIdx.x, gridDim.x) * kWavesPerBlock + wv;
    if (grp >= a.G) return;
    const uint64_t base = grp * kGroupElems;
    const bool full = base + kGroupElems <= a.n;
    ThetaTile th;  // theta (AdamW: the read-only v) loads go out first
    if constexpr (AD)
        prefetch_moment2(a, base, full, lane, th);
    else
        prefetch_theta(a, base, full, lane, th);
    const uint64_t c = grp * kWave + lane;
    const bool valid = c < a.C;
    const uint64_t cv = valid ? c : 0;
    const uint32_t loff = valid ? (uint32_t)(lane * k) : 0u;
    const uint32_t mask = a.random ? random_mask(a.seed, a.step_lo, a.chunk_offset + cv, k) : a.mask;

    float A[32];
#pragma unroll
    for (int s = 0; s < 32; s++) A[s] = 0.f;
    if (VF == VF_TERNARY && STAGED && R >= kCountMinR && R < (1 << kCountPlanes)) {
        int T[32];
        count_ternary(a, grp, st, lane, T);
#pragma unroll
        for (int s = 0; s < 32; s++) A[s] = (float)T[s];
    } else if (VF == VF_TERNARY && STAGED) {
        uint4* ws = reinterpret_cast<uint4*>(st);
        const WordStage w = word_stage(k, lane);
        const int pass = kSelRounds * w.rpr;
        int T[32];
#pragma unroll
        for (int s = 0; s < 32; s++) T[s] = 0;
        for (int r0 = 0; r0 < R; r0 += pass) {
            const int nrep = R - r0 < pass ? R - r0 : pass;
            wave_lds_sync();
            stage_words<kSelRounds>(a, grp, ws, w, r0, nrep);
            wave_lds_sync();
            for (int rl = 0; rl < nrep; rl++) {
#pragma unroll
                for (int s = 0; s < 32; s++)
                    if (s < k) T[s] += staged_ternary(ws, rl * k + s, lane);
            }
        }
#pragma unroll
        for (int s = 0; s < 32; s++) A[s] = (float)T[s];
    } else if (VF != VF_TERNARY) {
        // value formats: two replicas' values loaded before either is added
        // (measured 3-6% faster than one replica at a time)
        const uint64_t voff = a.val_off + group_entry(a, grp, 0) * (VF == VF_F32 ? 4 : 2);
        int r = 0;
        for (; r + 1 < R; r += 2) {
            float V0[32], V1[32];
#pragma unroll
            for (int s = 0; s < 32; s++) V0[s] = V1[s] = 0.f;
            add_slot_values<VF>(a.pay + (uint64_t)r * a.stride + voff, loff, k, V0);
            add_slot_values<VF>(a.pay + (uint64_t)(r + 1) * a.stride + voff, loff, k, V1);
#pragma unroll
            for (int s = 0; s < 32; s++) A[s] += V0[s] + V1[s];
        }
        if (r < R) add_slot_values<VF>(a.pay + (uint64_t)r * a.stride + voff, loff, k, A);
    } else {  // ternary, few entries: wave-uniform plane words as scalar loads
        for (int r = 0; r < R; r++) {
            const uint8_t* pr = a.pay + (uint64_t)r * a.stride;
#pragma unroll
            for (int s = 0; s < 32; s++)
                if (s < k) {
                    const uint64_t wd = grp * (uint64_t)k + s;
                    A[s] += ternary_of(load_const_u64(pr + a.nz_off, wd), load_const_u64(pr + a.neg_off, wd), lane);
                }
        }
    }

    wave_lds_sync();
#pragma unroll
    for (int q = 0; q < 8; q++)
        *reinterpret_cast<float4*>(st + swz(lane, 4 * q)) = make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t mm = mask;
#pragma unroll
    for (int s = 0; s < 32; s++)
        if (s < k) {
            const uint32_t j = __builtin_ctz(mm) & 31u;  // mm keeps k set bits for k draws
            mm &= mm - 1u;
            st[swz(lane, (int)j)] = valid ? A[s] * a.invR : 0.f;
        }
    wave_lds_sync();
    if constexpr (AD)
        apply_adamw_moment2_prefetched(a, st, base, full, lane, th);
    else
        apply_update_prefetched<AD>(a, st, base, full, lane, th);
}

// ------------------------------------------------------------------ select --

// ------------------------------------------------------------- validation --

// Payload check for a receiver (demo_payload_validate): one wave per group of
// 64 chunks, lane = chunk; every violation of the format counts once:
// a NEG bit without its NZ bit (chunks < C), any NZ / NEG bit of a chunk >= C,
// an IDX byte above 31 or not above the previous slot's, a sign-on value other
// than -1 / 0 / +1, a sign-off value that is not finite.  The wave's total is
// added to *out (cleared beforehand by zero_u64_kernel).
struct CheckArgs {
    const uint8_t* pay;
    unsigned long long* out;
    uint64_t C, G;
    uint64_t idx_off, nz_off, neg_off, val_off;
    int k;
    int dct;
    int sign;
};

template <int VF>
__global__ __launch_bounds__(kBlock) void validate_kernel(CheckArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t grp = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (grp >= a.G) return;
    const uint64_t c = grp * kWave + lane;
    const bool valid = c < a.C;
    uint32_t bad = 0;
    int prev = -1;
    for (int s = 0; s < a.k; s++) {
        const uint64_t e = c * (uint64_t)a.k + (uint64_t)s;
        if (VF == VF_TERNARY) {
            const uint64_t w = grp * (uint64_t)a.k + (uint64_t)s;
            const bool nz = (reinterpret_cast<const uint64_t*>(a.pay + a.nz_off)[w] >> lane) & 1ull;
            const bool ng = (reinterpret_cast<const uint64_t*>(a.pay + a.neg_off)[w] >> lane) & 1ull;
            bad += valid ? (uint32_t)(ng && !nz) : (uint32_t)nz + (uint32_t)ng;
        } else if (valid) {
            const float v = VF == VF_F32 ? reinterpret_cast<const float*>(a.pay + a.val_off)[e]
                                         : __half2float(__ushort_as_half(
                                               reinterpret_cast<const uint16_t*>(a.pay + a.val_off)[e]));
            bad += a.sign ? (uint32_t)!(v == 0.f || v == 1.f || v == -1.f) : (uint32_t)!isfinite(v);
        }
        if (a.dct && valid) {
            const int b = a.pay[a.idx_off + e];
            bad += (uint32_t)(b > 31) + (uint32_t)(b <= prev);
            prev = b;
        }
    }
    unsigned long long total = bad;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) total += __shfl_xor(total, d);
    if (lane == 0 && total) atomicAdd(a.out, total);
}

__global__ void zero_u64_kernel(unsigned long long* p) { *p = 0ull; }

__global__ __launch_bounds__(256) void select_kernel(uint32_t* out, uint64_t n_chunks, uint64_t chunk_offset,
                                                     uint64_t seed, uint32_t step_lo, int k, int random,
                                                     uint32_t mask) {
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n_chunks;
         c += (uint64_t)gridDim.x * blockDim.x)
        out[c] = random ? random_mask(seed, step_lo, chunk_offset + c, k) : mask;
}

}  // namespace demo
