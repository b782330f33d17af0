// demo.hip -- host side of libdemo: argument validation, payload layout,
// launch configuration and the extern "C" entry points declared in
// include/demo.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "demo.h"
#include "kernels.hpp"

namespace {

using demo::DecArgs;
using demo::EncArgs;

constexpr uint64_t kMaxElems = (uint64_t)1 << 40;  // 4 TB of fp32 per array

uint64_t up256(uint64_t x) { return (x + 255u) & ~(uint64_t)255u; }

bool is_sync_step(const demo_cfg* cfg) { return cfg->step % cfg->period == (uint64_t)(cfg->period - 1); }

int slots_per_chunk(const demo_cfg* cfg) { return cfg->scheme == DEMO_SCHEME_DILOCO ? 32 : (int)cfg->k; }

int check_cfg(const demo_cfg* cfg) {
    if (!cfg) return DEMO_EINVAL;
    if (cfg->abi_version != DEMO_ABI_VERSION) return DEMO_EABI;
    if (cfg->chunk != DEMO_CHUNK) return DEMO_EUNSUPPORTED;
    if (cfg->reserved != 0) return DEMO_EINVAL;
    switch (cfg->scheme) {
    case DEMO_SCHEME_DCT:
    case DEMO_SCHEME_RANDOM:
        if (cfg->k < 1 || cfg->k > 32) return DEMO_EINVAL;
        break;
    case DEMO_SCHEME_STRIDE:
        if (cfg->k < 1 || cfg->k > 32 || 32 % cfg->k != 0) return DEMO_EINVAL;
        break;
    case DEMO_SCHEME_DILOCO:
        if (cfg->period < 1) return DEMO_EINVAL;
        break;
    default:
        return DEMO_EINVAL;
    }
    if (cfg->value_fmt > DEMO_VAL_F32) return DEMO_EINVAL;
    if (cfg->sign > 1) return DEMO_EINVAL;
    if (cfg->sign == 0 && cfg->value_fmt == DEMO_VAL_TERNARY) return DEMO_EINVAL;
    if (!std::isfinite(cfg->beta) || !std::isfinite(cfg->lr)) return DEMO_EINVAL;
    return DEMO_OK;
}

int check_size(const demo_cfg* cfg, uint64_t n) {
    if (n == 0 || n > kMaxElems) return DEMO_EINVAL;
    const uint64_t C = (n + 31) / 32;
    if (cfg->chunk_offset > UINT64_MAX - C) return DEMO_EINVAL;
    return DEMO_OK;
}

void layout_of(const demo_cfg* cfg, uint64_t n, demo_layout* L) {
    const uint64_t C = (n + 31) / 32;
    const uint64_t G = (C + 63) / 64;
    const uint64_t k = (uint64_t)slots_per_chunk(cfg);
    *L = demo_layout{};
    uint64_t off = 0;
    if (cfg->scheme == DEMO_SCHEME_DCT) {
        L->idx_off = off;
        L->idx_bytes = C * k;
        off = up256(off + L->idx_bytes);
    }
    if (cfg->value_fmt == DEMO_VAL_TERNARY) {
        L->plane_bytes = G * k * 8;
        L->nz_off = off;
        off = up256(off + L->plane_bytes);
        L->neg_off = off;
        off = up256(off + L->plane_bytes);
    } else {
        L->val_bytes = C * k * (cfg->value_fmt == DEMO_VAL_F16 ? 2 : 4);
        L->val_off = off;
        off = up256(off + L->val_bytes);
    }
    L->total_bytes = off;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// One block of 4 waves per 4 consecutive groups; the grid covers the shard
// once (a one-pass grid streams markedly faster than persistent blocks on
// MI355X).
unsigned grid_for_groups(uint64_t G) {
    return (unsigned)((G + demo::kWavesPerBlock - 1) / demo::kWavesPerBlock);
}

// The encode kernels stream 16 KB of loads per wave (g and m); measured on
// MI355X they run fastest with 2 blocks (8 waves) per CU, while the decode
// kernels (8 KB per wave) run fastest at the 4 blocks per CU their own LDS
// allows.  Reserving this much extra LDS per encode block holds the encode at
// 2 blocks per CU (160 KB of LDS per CU).
constexpr size_t kEncodeLdsReserve = 24 * 1024;

uint32_t stride_mask(uint64_t step, uint32_t n) {
    const uint32_t s = 32 / n;
    const uint32_t off = (uint32_t)(step % s);
    uint32_t m = 0;
    for (uint32_t j = off; j < 32; j += s) m |= 1u << j;
    return m;
}

// shared (chunk-independent) positions of STRIDE / DILOCO for this step
uint32_t shared_mask(const demo_cfg* cfg) {
    if (cfg->scheme == DEMO_SCHEME_STRIDE) return stride_mask(cfg->step, cfg->k);
    if (cfg->scheme == DEMO_SCHEME_DILOCO) return 0xFFFFFFFFu;
    return 0;
}

int launch_status() { return hipGetLastError() == hipSuccess ? DEMO_OK : DEMO_EHIP; }

template <int KS, int VF>
void launch_encode_dct_q(const EncArgs& a, bool wq, unsigned grid, hipStream_t s) {
    if (wq)
        hipLaunchKernelGGL((demo::encode_dct_kernel<KS, VF, true>), dim3(grid), dim3(demo::kBlock), kEncodeLdsReserve,
                           s, a);
    else
        hipLaunchKernelGGL((demo::encode_dct_kernel<KS, VF, false>), dim3(grid), dim3(demo::kBlock), kEncodeLdsReserve,
                           s, a);
}

template <int VF>
void launch_encode_dct(const EncArgs& a, bool wq, unsigned grid, hipStream_t s) {
    switch (a.k) {
    case 1: launch_encode_dct_q<1, VF>(a, wq, grid, s); break;
    case 2: launch_encode_dct_q<2, VF>(a, wq, grid, s); break;
    case 3:
    case 4: launch_encode_dct_q<4, VF>(a, wq, grid, s); break;
    default:
        if (a.k <= 8) launch_encode_dct_q<8, VF>(a, wq, grid, s);
        else launch_encode_dct_q<0, VF>(a, wq, grid, s);
    }
}

template <int VF>
void launch_encode_sel(const EncArgs& a, bool wq, unsigned grid, hipStream_t s) {
    if (wq)
        hipLaunchKernelGGL((demo::encode_sel_kernel<VF, true>), dim3(grid), dim3(demo::kBlock), kEncodeLdsReserve, s,
                           a);
    else
        hipLaunchKernelGGL((demo::encode_sel_kernel<VF, false>), dim3(grid), dim3(demo::kBlock), kEncodeLdsReserve, s,
                           a);
}

// Selection-scheme decode with ternary planes: up to this many payload entries
// per chunk (R*k) the plane words are read as wave-uniform scalar loads; beyond
// it they are staged through LDS with coalesced vector loads.
constexpr uint64_t kSelScalarEntries = 8;

}  // namespace

extern "C" {

int demo_abi_version(void) { return DEMO_ABI_VERSION; }

const char* demo_strerror(int code) {
    switch (code) {
    case DEMO_OK: return "ok";
    case DEMO_EINVAL: return "invalid argument or configuration";
    case DEMO_EALIGN: return "pointer or stride misaligned";
    case DEMO_EUNSUPPORTED: return "configuration not supported by this build";
    case DEMO_EHIP: return "HIP runtime or launch error";
    case DEMO_EABI: return "demo_cfg.abi_version does not match the library";
    default: return "unknown error code";
    }
}

int demo_payload_layout(const demo_cfg* cfg, uint64_t n_elems, demo_layout* out) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    if ((rc = check_size(cfg, n_elems))) return rc;
    if (!out) return DEMO_EINVAL;
    layout_of(cfg, n_elems, out);
    return DEMO_OK;
}

int demo_encode(const demo_cfg* cfg, uint64_t n_elems, const float* grad, float* momentum, void* payload_out,
                float* q_out, void* hip_stream) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    if ((rc = check_size(cfg, n_elems))) return rc;
    const bool sends = cfg->scheme != DEMO_SCHEME_DILOCO || is_sync_step(cfg);
    if (!grad || !momentum || (sends && !payload_out)) return DEMO_EINVAL;
    if (!aligned16(grad) || !aligned16(momentum) || (q_out && !aligned16(q_out)) ||
        (sends && !aligned16(payload_out)))
        return DEMO_EALIGN;
    demo_layout L;
    layout_of(cfg, n_elems, &L);
    const uint64_t nb = n_elems * 4;
    const uint64_t pb = sends ? L.total_bytes : 0;
    if (overlap(grad, nb, momentum, nb) || overlap(grad, nb, q_out, nb) || overlap(momentum, nb, q_out, nb) ||
        overlap(payload_out, pb, grad, nb) || overlap(payload_out, pb, momentum, nb) ||
        overlap(payload_out, pb, q_out, nb))
        return DEMO_EINVAL;

    const uint64_t C = (n_elems + 31) / 32;
    EncArgs a{};
    a.g = grad;
    a.m = momentum;
    a.pay = static_cast<uint8_t*>(payload_out);
    a.q_out = q_out;
    a.n = n_elems;
    a.C = C;
    a.G = (C + 63) / 64;
    a.idx_off = L.idx_off;
    a.nz_off = L.nz_off;
    a.neg_off = L.neg_off;
    a.val_off = L.val_off;
    a.chunk_offset = cfg->chunk_offset;
    a.seed = cfg->seed;
    a.step_lo = (uint32_t)cfg->step;
    a.mask = shared_mask(cfg);
    a.beta = cfg->beta;
    a.k = slots_per_chunk(cfg);
    a.random = cfg->scheme == DEMO_SCHEME_RANDOM;
    a.sign = (int)cfg->sign;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const unsigned grid = grid_for_groups(a.G);
    const bool wq = q_out != nullptr;

    if (!sends) {
        const uint64_t blocks = (n_elems / 4 + 3 + 255) / 256;
        if (wq)
            hipLaunchKernelGGL((demo::momentum_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((demo::momentum_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, s, a);
        return launch_status();
    }
    if (cfg->scheme == DEMO_SCHEME_DCT) {
        switch (cfg->value_fmt) {
        case DEMO_VAL_TERNARY: launch_encode_dct<demo::VF_TERNARY>(a, wq, grid, s); break;
        case DEMO_VAL_F16: launch_encode_dct<demo::VF_F16>(a, wq, grid, s); break;
        default: launch_encode_dct<demo::VF_F32>(a, wq, grid, s); break;
        }
    } else {
        switch (cfg->value_fmt) {
        case DEMO_VAL_TERNARY: launch_encode_sel<demo::VF_TERNARY>(a, wq, grid, s); break;
        case DEMO_VAL_F16: launch_encode_sel<demo::VF_F16>(a, wq, grid, s); break;
        default: launch_encode_sel<demo::VF_F32>(a, wq, grid, s); break;
        }
    }
    return launch_status();
}

int demo_decode_apply(const demo_cfg* cfg, uint64_t n_elems, float* params, const void* payloads, uint64_t stride,
                      uint32_t R, void* hip_stream) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    if ((rc = check_size(cfg, n_elems))) return rc;
    if (R < 1 || R > (1u << 20)) return DEMO_EINVAL;
    const bool sends = cfg->scheme != DEMO_SCHEME_DILOCO || is_sync_step(cfg);
    if (!params || (sends && !payloads)) return DEMO_EINVAL;
    if (!aligned16(params) || (sends && (!aligned16(payloads) || (stride & 15u) != 0))) return DEMO_EALIGN;
    demo_layout L;
    layout_of(cfg, n_elems, &L);
    if (!sends) return DEMO_OK;
    if (stride < L.total_bytes) return DEMO_EINVAL;
    if ((uint64_t)(R - 1) > (UINT64_MAX - L.total_bytes) / (stride ? stride : 1)) return DEMO_EINVAL;
    if (overlap(params, n_elems * 4, payloads, (uint64_t)(R - 1) * stride + L.total_bytes)) return DEMO_EINVAL;

    const uint64_t C = (n_elems + 31) / 32;
    DecArgs a{};
    a.theta = params;
    a.pay = static_cast<const uint8_t*>(payloads);
    a.stride = stride;
    a.n = n_elems;
    a.C = C;
    a.G = (C + 63) / 64;
    a.idx_off = L.idx_off;
    a.nz_off = L.nz_off;
    a.neg_off = L.neg_off;
    a.val_off = L.val_off;
    a.chunk_offset = cfg->chunk_offset;
    a.seed = cfg->seed;
    a.step_lo = (uint32_t)cfg->step;
    a.mask = shared_mask(cfg);
    a.lr = cfg->lr;
    a.invR = 1.0f / (float)R;
    a.k = slots_per_chunk(cfg);
    a.R = (int)R;
    a.random = cfg->scheme == DEMO_SCHEME_RANDOM;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const dim3 grid(grid_for_groups(a.G)), block(demo::kBlock);
    const uint64_t entries = (uint64_t)R * (uint64_t)a.k;  // payload entries per chunk
    if (cfg->scheme == DEMO_SCHEME_DCT && entries <= (uint64_t)demo::kSparseEntries) {
        switch (cfg->value_fmt) {
        case DEMO_VAL_TERNARY: hipLaunchKernelGGL((demo::decode_dct_kernel<demo::VF_TERNARY>), grid, block, 0, s, a); break;
        case DEMO_VAL_F16: hipLaunchKernelGGL((demo::decode_dct_kernel<demo::VF_F16>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((demo::decode_dct_kernel<demo::VF_F32>), grid, block, 0, s, a); break;
        }
    } else if (cfg->scheme == DEMO_SCHEME_DCT) {
        switch (cfg->value_fmt) {
        case DEMO_VAL_TERNARY: hipLaunchKernelGGL((demo::decode_dct_dense_kernel<demo::VF_TERNARY>), grid, block, 0, s, a); break;
        case DEMO_VAL_F16: hipLaunchKernelGGL((demo::decode_dct_dense_kernel<demo::VF_F16>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((demo::decode_dct_dense_kernel<demo::VF_F32>), grid, block, 0, s, a); break;
        }
    } else {
        switch (cfg->value_fmt) {
        case DEMO_VAL_TERNARY:
            if (entries > kSelScalarEntries)
                hipLaunchKernelGGL((demo::decode_sel_kernel<demo::VF_TERNARY, true>), grid, block, 0, s, a);
            else
                hipLaunchKernelGGL((demo::decode_sel_kernel<demo::VF_TERNARY, false>), grid, block, 0, s, a);
            break;
        case DEMO_VAL_F16: hipLaunchKernelGGL((demo::decode_sel_kernel<demo::VF_F16, false>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((demo::decode_sel_kernel<demo::VF_F32, false>), grid, block, 0, s, a); break;
        }
    }
    return launch_status();
}

int demo_random_select(const demo_cfg* cfg, uint64_t seed, uint64_t step, uint64_t n_chunks, uint32_t* masks_out,
                       void* hip_stream) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    if (cfg->scheme != DEMO_SCHEME_RANDOM && cfg->scheme != DEMO_SCHEME_STRIDE) return DEMO_EINVAL;
    if (n_chunks == 0 || n_chunks > kMaxElems / 32 || cfg->chunk_offset > UINT64_MAX - n_chunks) return DEMO_EINVAL;
    if (!masks_out) return DEMO_EINVAL;
    if (((uintptr_t)masks_out & 3u) != 0) return DEMO_EALIGN;
    const int random = cfg->scheme == DEMO_SCHEME_RANDOM;
    const uint32_t mask = random ? 0u : stride_mask(step, cfg->k);
    uint64_t blocks = (n_chunks + 255) / 256;
    if (blocks > (1u << 20)) blocks = 1u << 20;
    hipLaunchKernelGGL(demo::select_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(hip_stream), masks_out, n_chunks, cfg->chunk_offset, seed,
                       (uint32_t)step, (int)cfg->k, random, mask);
    return launch_status();
}

}  // extern "C"
