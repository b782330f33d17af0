/*
 * demo.h -- C ABI of libdemo: the DeMo / FlexDeMo optimizer step on one
 * accelerator's parameter shard, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the DeToNATION paper notes (AAAI 2026), section
 * "FlexDeMo optimizer", Algorithm 1, steps 3-7:
 *   3. momentum accumulation      m <- beta*m + g
 *   4. extract fast components    q  (DCT-II + top-k, or another scheme)
 *   5. error feedback             m <- m - q
 *   6. synchronise q over the replication group R (the payload exchange)
 *   7. parameter update           theta <- theta - lr*Q
 * and the same notes' "Replication schemes" table (DeMo, Random, Striding,
 * DiLoCo) and "Sign function" section (sign before sync: ternary values,
 * chunk size 32).  The DeMo abstract ("DeMo: Decoupled Momentum
 * Optimization") fixes the transform as a fast orthonormal DCT with top-k.
 *
 * Conventions shared by every entry point
 *  - All tensors are flat fp32 arrays of n_elems elements in device memory
 *    (hipMalloc / PyTorch allocations), 16-byte aligned, with
 *    1 <= n_elems <= DEMO_MAX_ELEMS (2^36, 256 GB per array; larger shards
 *    are split by the caller, for instance at tensor boundaries, each part
 *    with its own chunk_offset).  The caller owns all memory; the library
 *    never allocates, frees or keeps pointers.
 *  - A chunk is 32 consecutive elements; C = ceil(n_elems/32) chunks; the last
 *    chunk is zero-padded inside the kernels and padded outputs are dropped.
 *  - Calls are asynchronous on the given HIP stream (hipStream_t passed as
 *    void*, NULL = the default stream).  A configuration or argument error is
 *    returned synchronously as a negative code and nothing is launched; a
 *    launch failure returns DEMO_EHIP; device faults surface at the caller's
 *    next synchronisation.  No C++ exception crosses the ABI.
 *  - Buffers passed to one call must not overlap.  Calls on distinct buffers
 *    may be made from several threads.
 *  - Values are not checked: NaN or infinity in an input propagates into that
 *    chunk's outputs (which slots a DCT chunk with a NaN transform selects is
 *    unspecified); every memory access stays inside the buffers described.
 */
#ifndef DEMO_H
#define DEMO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DEMO_ABI_VERSION 1
#define DEMO_CHUNK 32
#define DEMO_MAX_ELEMS ((uint64_t)1 << 36)

/* Replication schemes ("Replication schemes" table of the DeToNATION notes). */
enum {
    DEMO_SCHEME_DCT = 0,    /* DeMo: DCT-II per chunk, top-k, indices sent      */
    DEMO_SCHEME_RANDOM = 1, /* k random positions from a shared seed, no indices */
    DEMO_SCHEME_STRIDE = 2, /* every (32/k)-th position, offset = step mod 32/k  */
    DEMO_SCHEME_DILOCO = 3  /* everything once every `period` steps, else nothing */
};

/* Wire format of the slot values.  Sign before sync makes every value
 * ternary (-1, 0, +1); TERNARY packs it into two bit-planes, F16 / F32 store
 * it as a number (the notes compare fp16 and fp32 communication). */
enum { DEMO_VAL_TERNARY = 0, DEMO_VAL_F16 = 1, DEMO_VAL_F32 = 2 };

enum {
    DEMO_OK = 0,
    DEMO_EINVAL = -1,       /* bad configuration value, size or null pointer */
    DEMO_EALIGN = -2,       /* pointer or stride not aligned as required      */
    DEMO_EUNSUPPORTED = -3, /* valid request this library does not implement  */
    DEMO_EHIP = -4,         /* HIP launch / runtime error                     */
    DEMO_EABI = -5          /* cfg->abi_version != DEMO_ABI_VERSION           */
};

typedef struct demo_cfg {
    uint32_t abi_version;  /* must be DEMO_ABI_VERSION */
    uint32_t scheme;       /* DEMO_SCHEME_* */
    uint32_t chunk;        /* must be 32 ("chunk size = 32", notes' hyper-parameters) */
    uint32_t k;            /* DCT: top-k in [1,32]; RANDOM: n in [1,32];
                              STRIDE: n with 32 % n == 0; DILOCO: ignored (32) */
    uint32_t period;       /* DILOCO: sync when step % period == period-1; >= 1 */
    uint32_t sign;         /* 1 = sign before sync: every slot carries sign(value)
                              in {-1, 0, +1} ("Sign function" section).
                              0 = slots carry the selected values themselves:
                              the DCT coefficient (DCT) or u (others), stored
                              as fp32 or as fp16 rounded to nearest even with
                              subnormals kept; needs value_fmt F16 or F32
                              (TERNARY with sign 0 is DEMO_EINVAL). */
    uint32_t value_fmt;    /* DEMO_VAL_* */
    float beta;            /* momentum decay, finite (offset 28) */
    float lr;              /* learning rate eta, finite (offset 32) */
    uint32_t reserved;     /* must be 0; keeps seed at its natural offset 40 */
    uint64_t seed;         /* shared selection seed (RANDOM) */
    uint64_t step;         /* optimizer step t, from 0 (hashed mod 2^32) */
    uint64_t chunk_offset; /* global chunk index of this shard's element 0 */
} demo_cfg;

/*
 * Payload of one replica for one step: one byte buffer whose regions start at
 * multiples of 256 bytes, in the order IDX, NZ, NEG (TERNARY) or IDX, VAL
 * (F16/F32); its size is rounded up to 256 bytes.  With k slots per chunk
 * (k = 32 for DILOCO) and G = ceil(C/64):
 *   IDX  uint8 [C][k]   DCT scheme only: chunk-local position of slot s of
 *                       chunk c at byte c*k+s; the k positions ascend.
 *   NZ   uint64 [G][k]  TERNARY: bit b of word g*k+s is set iff slot s of chunk
 *   NEG  uint64 [G][k]  64g+b is nonzero / negative.  Value = NZ ? (NEG ? -1 :
 *                       +1) : 0.  NEG without NZ and bits of chunks >= C are 0
 *                       (the encoder never sets them; the decoder reads a NEG
 *                       bit without its NZ bit as 0 and index bytes mod 32).
 *   VAL  fp16|fp32 [C][k] F16/F32: value of slot s of chunk c at entry c*k+s:
 *                       +-1 or 0 with sign 1, the value itself with sign 0.
 * RANDOM, STRIDE and DILOCO carry no IDX: every replica recomputes the slot
 * positions from (seed, step, chunk) and slots follow ascending position.
 */
typedef struct demo_layout {
    uint64_t idx_off, idx_bytes;
    uint64_t nz_off, neg_off, plane_bytes;
    uint64_t val_off, val_bytes;
    uint64_t total_bytes; /* minimum stride between replicas */
} demo_layout;

/*
 * Decoupled AdamW (DeToNATION notes, "Decoupled AdamW": an AdamW variant whose
 * first and second moments are not synchronised).  The notes give no formula;
 * the reading implemented: both moments stay local and are never exchanged;
 * the first moment m = beta1*m + (1-beta1)*g (beta1 = demo_cfg.beta) takes the
 * momentum's place in the extraction, the payload and the error feedback of
 * demo_encode; v = beta2*v + (1-beta2)*g^2; the decode applies the exchanged
 * mean Q as AdamW applies its first moment:
 *   theta -= lr * ((Q / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *                  + weight_decay * theta),   t = demo_cfg.step + 1.
 * The slots carry the selected values (demo_cfg.sign 0, value_fmt F16 or
 * F32): with the sign before sync ("Sign function" section) Q is a mean of
 * ternary values that has lost the first moment's magnitude, and dividing it
 * by sqrt(v) would scale the step by 1/|g|, so demo_cfg.sign 1 is DEMO_EINVAL
 * for both AdamW calls.  beta1 (demo_cfg.beta) and beta2 in [0, 1); eps >= 0
 * and weight_decay finite; reserved must be 0.
 */
typedef struct demo_adamw {
    float beta2;
    float eps;
    float weight_decay;
    uint32_t reserved;
} demo_adamw;

/* Library version; equals DEMO_ABI_VERSION. */
int demo_abi_version(void);

/* Static string for a DEMO_* code (never NULL). */
const char *demo_strerror(int code);

/* Payload layout of one replica for n_elems >= 1 elements under cfg.
 * Host-only (touches no device).  Returns DEMO_OK or a negative code. */
int demo_payload_layout(const demo_cfg *cfg, uint64_t n_elems, demo_layout *out);

/*
 * Encoder side of one optimizer step (Algorithm 1 steps 3-5 and the sender
 * half of step 6):
 *   u = beta*momentum + grad; per chunk select slots (DCT: the k largest |DCT-II
 *   coefficients|, equal magnitudes to the lower index; RANDOM / STRIDE: the
 *   shared positions; DILOCO: all 32 on a sync step, none otherwise);
 *   q = inverse DCT of the selected coefficients (DCT) or u on the selected
 *   positions (others); momentum <- u - q; payload <- the slot values, as
 *   ternary signs or (sign 0) the values themselves, and positions for DCT.
 * grad      [n_elems] read-only.
 * momentum  [n_elems] updated in place.
 * payload_out  >= demo_payload_layout(...).total_bytes bytes, 16-byte aligned.
 *           On a DILOCO non-sync step it is not written.
 * q_out     [n_elems] or NULL: receives q (diagnostics; costs 4 bytes/element).
 */
int demo_encode(const demo_cfg *cfg, uint64_t n_elems, const float *grad, float *momentum,
                void *payload_out, float *q_out, void *hip_stream);

/*
 * Receiver side (Algorithm 1 steps 6-7): payloads holds R >= 1 replicas'
 * payloads for this step, replica r at payloads + r*stride (own payload among
 * them; the layout an all-gather produces).  Per chunk the slot values are
 * summed over replicas into the slot positions, divided by R, taken back
 * through the inverse DCT (DCT scheme) and applied as params -= lr*Q.
 * On a DILOCO non-sync step nothing is read or written.
 * stride >= total_bytes and a multiple of 16.
 */
int demo_decode_apply(const demo_cfg *cfg, uint64_t n_elems, float *params, const void *payloads,
                      uint64_t stride, uint32_t R, void *hip_stream);

/*
 * demo_encode for Decoupled AdamW (see demo_adamw): moment1 [n_elems] is the
 * first moment (extracted from and updated in place like demo_encode's
 * momentum), moment2 [n_elems] the second moment, updated in place (also on
 * DiLoCo steps without a payload).  16-byte aligned; no argument may alias
 * another.  Same payload, codes and asynchrony as demo_encode.
 */
int demo_encode_adamw(const demo_cfg *cfg, const demo_adamw *adamw, uint64_t n_elems, const float *grad,
                      float *moment1, float *moment2, void *payload_out, float *q_out, void *hip_stream);

/*
 * demo_decode_apply for Decoupled AdamW: the same Q, applied with this
 * replica's second moment moment2 [n_elems] (read-only, 16-byte aligned, not
 * aliasing params) and weight decay, as stated at demo_adamw.  On a DILOCO
 * non-sync step nothing is read or written.
 */
int demo_decode_apply_adamw(const demo_cfg *cfg, const demo_adamw *adamw, uint64_t n_elems, float *params,
                            const float *moment2, const void *payloads, uint64_t stride, uint32_t R,
                            void *hip_stream);

/*
 * Receiver-side check of one replica's payload before demo_decode_apply: the
 * payload comes from another replica (the exchange of Algorithm 1 step 6 in
 * the DeToNATION notes), and this call counts, into *violations_out, every
 * violation of the format stated at demo_layout for this cfg and n_elems:
 * a NEG bit without its NZ bit (chunks c < C); each NZ or NEG bit of a chunk
 * c >= C; an IDX byte above 31; an IDX byte not above the previous slot's
 * (positions must ascend strictly); with cfg->sign 1 an F16/F32 value other
 * than -1, 0 or +1 (the ternary values of sign before sync); with cfg->sign 0
 * a value that is not finite.  0 means well formed.  A DILOCO step that sends
 * nothing has no payload: payload may be NULL and the count is 0.
 * payload: device buffer of at least demo_payload_layout's total_bytes,
 * 16-byte aligned, read-only.  violations_out: device uint64, 8-byte aligned,
 * written asynchronously on hip_stream (read it after synchronising); it must
 * not overlap the payload.  The count is cleared by a kernel, not a memset.
 */
int demo_payload_validate(const demo_cfg *cfg, uint64_t n_elems, const void *payload, uint64_t *violations_out,
                          void *hip_stream);

/*
 * Shared-seed slot positions of n_chunks chunks (global ids chunk_offset +
 * c, c < n_chunks): masks_out[c] bit j set iff chunk-local position j is
 * selected.  cfg->scheme RANDOM: k positions drawn without replacement by
 * Philox4x32-10 (Salmon et al., SC'11) keyed by `seed`, counter (chunk_lo,
 * chunk_hi, step_lo, (1 << 24) | i/4), draw i taking word i%4 w and picking
 * free position number floor(w*(32-i)/2^32) counted from bit 0.  STRIDE:
 * positions j % (32/k) == step % (32/k).  `seed` and `step` override
 * cfg->seed and cfg->step.  masks_out: device uint32 [n_chunks], 4-byte aligned;
 * 1 <= n_chunks <= DEMO_MAX_ELEMS / 32.
 */
int demo_random_select(const demo_cfg *cfg, uint64_t seed, uint64_t step, uint64_t n_chunks,
                       uint32_t *masks_out, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* DEMO_H */
