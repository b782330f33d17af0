// demo.hip -- host side of libdemo: argument validation, payload layout,
// launch configuration and the extern "C" entry points declared in
// include/demo.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "decode.hpp"
#include "demo.h"
#include "encode.hpp"

namespace {

using demo::DecArgs;
using demo::EncArgs;

constexpr uint64_t kMaxElems = DEMO_MAX_ELEMS;
// the one-pass grids of the group kernels (64 work-items per 2048 elements)
// must stay below 2^32 work-items at the largest shard
static_assert((kMaxElems / 2048) * 64 < ((uint64_t)1 << 32), "one-pass grid exceeds 2^32 work-items");

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

// Decoupled AdamW streams one more array (v) through each kernel.  Its DCT
// encode (24 KB of loads per wave: g, m, v) measured fastest at 1 block per CU
// (2.11 ms against 2.20 ms at 2 blocks on a 639,697,920-parameter shard), its
// DCT decode (v beside theta) at 3 blocks (1.336 ms against 1.381 ms at 4);
// its selection decode at the 4 blocks its own LDS allows (1.375 ms against
// 1.534 ms at 3, Random n = 8), so the reserve applies to the DCT decodes only.
constexpr size_t kEncodeAdamwLdsReserve = 48 * 1024;
constexpr size_t kDecodeAdamwLdsReserve = 16 * 1024;

// The DiLoCo momentum pass (two read streams, one write stream, no transform)
// measured fastest at 1 block (4 waves) per CU: 1.161 ms against 1.236 ms at
// 2 blocks and 1.292 ms at 4 (S = 4).  It uses no LDS of its own; this much
// reserved holds it at one block per CU.
constexpr size_t kMomentumLdsReserve = 96 * 1024;

template <bool AD>
constexpr size_t encode_lds_reserve() { return AD ? kEncodeAdamwLdsReserve : kEncodeLdsReserve; }
template <bool AD>
constexpr size_t decode_lds_reserve() { return AD ? kDecodeAdamwLdsReserve : 0; }

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

template <class T>
struct same_type {
    using type = T;
};

// One kernel launch through hipLaunchKernel, whose return code belongs to this
// launch alone (hipGetLastError would also report an error that an earlier,
// unrelated HIP call left pending on the thread).  The parameter types come
// from the kernel; the arguments are converted to them.
template <class... P>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                  typename same_type<P>::type... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, s);
}

int status_of(hipError_t e) { return e == hipSuccess ? DEMO_OK : DEMO_EHIP; }

// AD: Decoupled AdamW (second moment in EncArgs::v / DecArgs::v)
template <int KS, int VF, bool AD>
hipError_t launch_encode_dct_q(const EncArgs& a, bool wq, unsigned grid, hipStream_t s) {
    return launch(wq ? demo::encode_dct_kernel<KS, VF, true, AD> : demo::encode_dct_kernel<KS, VF, false, AD>,
                  dim3(grid), dim3(demo::kBlock), encode_lds_reserve<AD>(), s, a);
}

template <int VF, bool AD>
hipError_t launch_encode_dct(const EncArgs& a, bool wq, unsigned grid, hipStream_t s) {
    switch (a.k) {
    case 1: return launch_encode_dct_q<1, VF, AD>(a, wq, grid, s);
    case 2: return launch_encode_dct_q<2, VF, AD>(a, wq, grid, s);
    case 3:
    case 4: return launch_encode_dct_q<4, VF, AD>(a, wq, grid, s);
    default:
        if (a.k <= 8) return launch_encode_dct_q<8, VF, AD>(a, wq, grid, s);
        return launch_encode_dct_q<0, VF, AD>(a, wq, grid, s);
    }
}

template <int VF, bool AD>
hipError_t launch_encode_sel(const EncArgs& a, bool wq, unsigned grid, hipStream_t s) {
    return launch(wq ? demo::encode_sel_kernel<VF, true, AD> : demo::encode_sel_kernel<VF, false, AD>, dim3(grid),
                  dim3(demo::kBlock), encode_lds_reserve<AD>(), s, a);
}

// the encode launch for one configuration: momentum only (DiLoCo between
// syncs), DCT or position selection, by value format
template <bool AD>
hipError_t launch_encode(const demo_cfg* cfg, const EncArgs& a, bool sends, bool wq, hipStream_t s) {
    if (!sends)
        return launch(wq ? demo::momentum_kernel<true, AD> : demo::momentum_kernel<false, AD>,
                      dim3(grid_for_groups(a.G)), dim3(demo::kBlock), kMomentumLdsReserve, s, a);
    const unsigned grid = grid_for_groups(a.G);
    if (cfg->scheme == DEMO_SCHEME_DCT) {
        switch (cfg->value_fmt) {
        case DEMO_VAL_TERNARY:
            if constexpr (!AD) return launch_encode_dct<demo::VF_TERNARY, false>(a, wq, grid, s);
            return hipErrorInvalidValue;  // AdamW carries values (check_adamw)
        case DEMO_VAL_F16: return launch_encode_dct<demo::VF_F16, AD>(a, wq, grid, s);
        default: return launch_encode_dct<demo::VF_F32, AD>(a, wq, grid, s);
        }
    }
    switch (cfg->value_fmt) {
    case DEMO_VAL_TERNARY:
        if constexpr (!AD) return launch_encode_sel<demo::VF_TERNARY, false>(a, wq, grid, s);
        return hipErrorInvalidValue;
    case DEMO_VAL_F16: return launch_encode_sel<demo::VF_F16, AD>(a, wq, grid, s);
    default: return launch_encode_sel<demo::VF_F32, AD>(a, wq, grid, s);
    }
}

// AdamW's bias correction 1/(1 - beta1^t) needs beta1 = cfg->beta in [0, 1);
// its slots carry values (a ternary Q has no magnitude for sqrt(v) to scale)
int check_adamw(const demo_cfg* cfg, const demo_adamw* w) {
    if (!w) return DEMO_EINVAL;
    if (w->reserved != 0) return DEMO_EINVAL;
    if (cfg->sign != 0) return DEMO_EINVAL;
    if (!(cfg->beta >= 0.f && cfg->beta < 1.f)) return DEMO_EINVAL;
    if (!(w->beta2 >= 0.f && w->beta2 < 1.f)) return DEMO_EINVAL;
    if (!(w->eps >= 0.f) || !std::isfinite(w->eps) || !std::isfinite(w->weight_decay)) return DEMO_EINVAL;
    return DEMO_OK;
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
    case DEMO_EUNSUPPORTED: return "configuration not supported by this library version";
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

}  // extern "C"

namespace {

// demo_encode, and with w (second moment v) demo_encode_adamw
int encode_impl(const demo_cfg* cfg, const demo_adamw* w, uint64_t n_elems, const float* grad, float* momentum,
                float* v, void* payload_out, float* q_out, void* hip_stream) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    if ((rc = check_size(cfg, n_elems))) return rc;
    if (w && (rc = check_adamw(cfg, w))) return rc;
    const bool sends = cfg->scheme != DEMO_SCHEME_DILOCO || is_sync_step(cfg);
    if (!grad || !momentum || (w && !v) || (sends && !payload_out)) return DEMO_EINVAL;
    if (!aligned16(grad) || !aligned16(momentum) || (q_out && !aligned16(q_out)) || (w && !aligned16(v)) ||
        (sends && !aligned16(payload_out)))
        return DEMO_EALIGN;
    demo_layout L;
    layout_of(cfg, n_elems, &L);
    const uint64_t nb = n_elems * 4;
    const uint64_t pb = sends ? L.total_bytes : 0;
    const uint64_t vb = w ? nb : 0;
    if (overlap(grad, nb, momentum, nb) || overlap(grad, nb, q_out, nb) || overlap(momentum, nb, q_out, nb) ||
        overlap(payload_out, pb, grad, nb) || overlap(payload_out, pb, momentum, nb) ||
        overlap(payload_out, pb, q_out, nb) || overlap(v, vb, grad, nb) || overlap(v, vb, momentum, nb) ||
        overlap(v, vb, q_out, nb) || overlap(v, vb, payload_out, pb))
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
    a.gamma = w ? 1.f - cfg->beta : 1.f;  // AdamW's first moment weighs g by 1 - beta1
    a.v = w ? v : nullptr;
    a.beta2 = w ? w->beta2 : 0.f;
    a.k = slots_per_chunk(cfg);
    a.random = cfg->scheme == DEMO_SCHEME_RANDOM;
    a.sign = (int)cfg->sign;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const bool wq = q_out != nullptr;
    return status_of(w ? launch_encode<true>(cfg, a, sends, wq, s) : launch_encode<false>(cfg, a, sends, wq, s));
}

template <bool AD>
hipError_t launch_decode(const demo_cfg* cfg, const DecArgs& a, dim3 grid, dim3 block, hipStream_t s) {
    const uint64_t entries = (uint64_t)a.R * (uint64_t)a.k;  // payload entries per chunk
    const size_t lds = decode_lds_reserve<AD>();  // DCT decodes; the selection decode takes none
    if (cfg->value_fmt == DEMO_VAL_TERNARY) {
        if constexpr (AD) return hipErrorInvalidValue;  // AdamW carries values (check_adamw)
        else {
            if (cfg->scheme == DEMO_SCHEME_DCT && entries <= (uint64_t)demo::kSparseEntries)
                return launch(demo::decode_dct_kernel<demo::VF_TERNARY, false>, grid, block, lds, s, a);
            if (cfg->scheme == DEMO_SCHEME_DCT)
                return launch(demo::decode_dct_dense_kernel<demo::VF_TERNARY, false>, grid, block, lds, s, a);
            if (entries > kSelScalarEntries)
                return launch(demo::decode_sel_kernel<demo::VF_TERNARY, true, false>, grid, block, 0, s, a);
            return launch(demo::decode_sel_kernel<demo::VF_TERNARY, false, false>, grid, block, 0, s, a);
        }
    }
    if (cfg->scheme == DEMO_SCHEME_DCT && entries <= (uint64_t)demo::kSparseEntries) {
        if (cfg->value_fmt == DEMO_VAL_F16)
            return launch(demo::decode_dct_kernel<demo::VF_F16, AD>, grid, block, lds, s, a);
        return launch(demo::decode_dct_kernel<demo::VF_F32, AD>, grid, block, lds, s, a);
    }
    if (cfg->scheme == DEMO_SCHEME_DCT) {
        if (cfg->value_fmt == DEMO_VAL_F16)
            return launch(demo::decode_dct_dense_kernel<demo::VF_F16, AD>, grid, block, lds, s, a);
        return launch(demo::decode_dct_dense_kernel<demo::VF_F32, AD>, grid, block, lds, s, a);
    }
    if (cfg->value_fmt == DEMO_VAL_F16)
        return launch(demo::decode_sel_kernel<demo::VF_F16, false, AD>, grid, block, 0, s, a);
    return launch(demo::decode_sel_kernel<demo::VF_F32, false, AD>, grid, block, 0, s, a);
}

// demo_decode_apply, and with w (second moment v) demo_decode_apply_adamw
int decode_impl(const demo_cfg* cfg, const demo_adamw* w, uint64_t n_elems, float* params, const float* v,
                const void* payloads, uint64_t stride, uint32_t R, void* hip_stream) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    if ((rc = check_size(cfg, n_elems))) return rc;
    if (w && (rc = check_adamw(cfg, w))) return rc;
    if (R < 1 || R > (1u << 20)) return DEMO_EINVAL;
    const bool sends = cfg->scheme != DEMO_SCHEME_DILOCO || is_sync_step(cfg);
    if (!params || (w && !v) || (sends && !payloads)) return DEMO_EINVAL;
    if (!aligned16(params) || (w && !aligned16(v)) ||
        (sends && (!aligned16(payloads) || (stride & 15u) != 0)))
        return DEMO_EALIGN;
    demo_layout L;
    layout_of(cfg, n_elems, &L);
    if (!sends) return DEMO_OK;
    if (stride < L.total_bytes) return DEMO_EINVAL;
    if ((uint64_t)(R - 1) > (UINT64_MAX - L.total_bytes) / (stride ? stride : 1)) return DEMO_EINVAL;
    const uint64_t payb = (uint64_t)(R - 1) * stride + L.total_bytes;
    if (overlap(params, n_elems * 4, payloads, payb) || (w && overlap(params, n_elems * 4, v, n_elems * 4)))
        return DEMO_EINVAL;

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
    if (w) {  // AdamW bias corrections of step t = step + 1, in double, then fp32
        const double t = (double)cfg->step + 1.0;
        a.v = v;
        a.c1 = (float)(1.0 / (1.0 - std::pow((double)cfg->beta, t)));
        a.c2 = (float)(1.0 / (1.0 - std::pow((double)w->beta2, t)));
        a.eps = w->eps;
        a.wd = w->weight_decay;
    }
    a.k = slots_per_chunk(cfg);
    a.R = (int)R;
    a.random = cfg->scheme == DEMO_SCHEME_RANDOM;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const dim3 grid(grid_for_groups(a.G)), block(demo::kBlock);
    return status_of(w ? launch_decode<true>(cfg, a, grid, block, s) : launch_decode<false>(cfg, a, grid, block, s));
}

}  // namespace

extern "C" {

int demo_encode(const demo_cfg* cfg, uint64_t n_elems, const float* grad, float* momentum, void* payload_out,
                float* q_out, void* hip_stream) {
    return encode_impl(cfg, nullptr, n_elems, grad, momentum, nullptr, payload_out, q_out, hip_stream);
}

int demo_encode_adamw(const demo_cfg* cfg, const demo_adamw* adamw, uint64_t n_elems, const float* grad,
                      float* moment1, float* moment2, void* payload_out, float* q_out, void* hip_stream) {
    if (!adamw) return DEMO_EINVAL;
    return encode_impl(cfg, adamw, n_elems, grad, moment1, moment2, payload_out, q_out, hip_stream);
}

int demo_decode_apply(const demo_cfg* cfg, uint64_t n_elems, float* params, const void* payloads, uint64_t stride,
                      uint32_t R, void* hip_stream) {
    return decode_impl(cfg, nullptr, n_elems, params, nullptr, payloads, stride, R, hip_stream);
}

int demo_decode_apply_adamw(const demo_cfg* cfg, const demo_adamw* adamw, uint64_t n_elems, float* params,
                            const float* moment2, const void* payloads, uint64_t stride, uint32_t R,
                            void* hip_stream) {
    if (!adamw) return DEMO_EINVAL;
    return decode_impl(cfg, adamw, n_elems, params, moment2, payloads, stride, R, hip_stream);
}

int demo_payload_validate(const demo_cfg* cfg, uint64_t n_elems, const void* payload, uint64_t* violations_out,
                          void* hip_stream) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    if ((rc = check_size(cfg, n_elems))) return rc;
    const bool sends = cfg->scheme != DEMO_SCHEME_DILOCO || is_sync_step(cfg);
    if (!violations_out || (sends && !payload)) return DEMO_EINVAL;
    if (((uintptr_t)violations_out & 7u) != 0 || (sends && !aligned16(payload))) return DEMO_EALIGN;
    demo_layout L;
    layout_of(cfg, n_elems, &L);
    if (sends && overlap(payload, L.total_bytes, violations_out, 8)) return DEMO_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    unsigned long long* out = reinterpret_cast<unsigned long long*>(violations_out);
    // cleared by a kernel rather than a memset, so the call can be captured in a HIP graph
    hipError_t e = launch(demo::zero_u64_kernel, dim3(1), dim3(1), 0, s, out);
    if (e != hipSuccess || !sends) return status_of(e);
    const uint64_t C = (n_elems + 31) / 32;
    demo::CheckArgs a{};
    a.pay = static_cast<const uint8_t*>(payload);
    a.out = out;
    a.C = C;
    a.G = (C + 63) / 64;
    a.idx_off = L.idx_off;
    a.nz_off = L.nz_off;
    a.neg_off = L.neg_off;
    a.val_off = L.val_off;
    a.k = slots_per_chunk(cfg);
    a.dct = cfg->scheme == DEMO_SCHEME_DCT;
    a.sign = (int)cfg->sign;
    const dim3 grid(grid_for_groups(a.G)), block(demo::kBlock);
    switch (cfg->value_fmt) {
    case DEMO_VAL_TERNARY: return status_of(launch(demo::validate_kernel<demo::VF_TERNARY>, grid, block, 0, s, a));
    case DEMO_VAL_F16: return status_of(launch(demo::validate_kernel<demo::VF_F16>, grid, block, 0, s, a));
    default: return status_of(launch(demo::validate_kernel<demo::VF_F32>, grid, block, 0, s, a));
    }
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
    return status_of(launch(demo::select_kernel, dim3((unsigned)blocks), dim3(256), 0,
                            static_cast<hipStream_t>(hip_stream), masks_out, n_chunks, cfg->chunk_offset, seed,
                            (uint32_t)step, (int)cfg->k, random, mask));
}

}  // extern "C"
