/*
 * oracle.c -- plain, slow, fp64 CPU reference of the DeMo / FlexDeMo optimizer
 * step on one parameter shard.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, link or call
 * this file: only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * GPU library; it is written directly from the method description.
 *
 * Sources (the pages this oracle follows):
 *  - DeToNATION paper notes (Paper-Notes, AAAI 2026), "Method / FlexDeMo
 *    optimizer", Algorithm 1: momentum m <- beta*m + Delta, extract the fast
 *    components q of m by DCT-II (or another scheme), m <- m - q, synchronise q
 *    over the replication group R, theta <- theta - eta*Q.
 *  - same notes, "Replication schemes" table: DeMo (DCT-II, indices sent),
 *    Random (n random indices, shared seed, no indices sent), Striding (equally
 *    spaced), DiLoCo (full synchronisation once every n steps).
 *  - same notes, "Sign function and hyper-parameters": sign before sync
 *    (ternary -1/0/+1), chunk size 32, TopK = 4 on T5.
 *  - "DeMo: Decoupled Momentum Optimization" abstract: fast orthonormal
 *    transform (DCT) + top-k sparsification, momentum subtraction as error
 *    feedback.
 *  - same notes, "Decoupled AdamW": an AdamW variant whose first and second
 *    moments (the EMAs of the gradient and of its square) are not
 *    synchronised.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - Delta is the plain gradient; eta appears only in the parameter update.
 *  - chunks are 32 consecutive elements of the flat shard; the last chunk is
 *    zero-padded, padded outputs are discarded and no state is kept for pads.
 *  - DCT-II is the orthonormal one, B[j][i] = s_j cos(pi (2i+1) j / 64),
 *    s_0 = sqrt(1/32), s_j = sqrt(2/32); its inverse is B transposed.
 *  - top-k keeps the k largest |X_j|; equal magnitudes go to the lower index.
 *    The comparison is taken on |X_j| rounded to fp32, the precision the GPU
 *    decides in (the pages fix none); slots are emitted in ascending index.
 *  - several selections are correct where the k-th and (k+1)-th |X_j| lie
 *    within a rounding of each other, and a sign is open where the selected
 *    value lies within a rounding of 0: the guided encode below takes another
 *    implementation's choice in exactly those cases (and rejects it in every
 *    other), so the two trajectories stay comparable.
 *  - q uses the unsigned coefficients; only the payload carries signs.
 *  - sign(0) = 0; the aggregate is the plain mean over all R payloads
 *    (own included) with no second sign.
 *  - Random: counter-based selection from a shared seed (Philox4x32-10,
 *    Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11);
 *    Striding: every (32/n)-th position, offset = step mod (32/n);
 *    DiLoCo: q = 0 except on steps with step mod period = period-1, where
 *    q = u (all 32 positions).  Random/Striding/DiLoCo work in the parameter
 *    domain (no transform).
 *  - beta and eta are the fp32 configuration values widened to fp64.
 *  - Decoupled AdamW (the notes give no formula): both moments are local and
 *    never exchanged; the first moment m = beta1*m + (1-beta1)*g takes the
 *    momentum's place in extraction and error feedback; v = beta2*v +
 *    (1-beta2)*g^2; the exchanged Q is applied as AdamW applies its first
 *    moment: theta -= eta*((Q/(1-beta1^t)) / (sqrt(v/(1-beta2^t)) + eps)
 *    + wd*theta), t = step + 1.  The slots carry the values themselves (sign
 *    off): a ternary Q has already lost the first moment's magnitude, and
 *    dividing it by sqrt(v) would scale the step by 1/|g| (a sign-on
 *    configuration is rejected).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_CHUNK 32

enum { OR_DCT = 0, OR_RANDOM = 1, OR_STRIDE = 2, OR_DILOCO = 3 };
enum { OR_TERNARY = 0, OR_F16 = 1, OR_F32 = 2 };

/* Configuration as seen by the oracle (its own struct; not the library's). */
typedef struct oracle_params {
    int32_t scheme;
    int32_t k;          /* DCT top-k, or n for Random / Striding */
    int32_t period;     /* DiLoCo period */
    int32_t sign;       /* 1: send sign(value); 0: send the value itself */
    int32_t value_fmt;  /* wire format of values when sign == 0 matters */
    float beta;
    float lr;
    uint64_t seed;
    uint64_t step;
} oracle_params;

/* Decoupled AdamW's extra hyper-parameters (beta1 is oracle_params.beta). */
typedef struct oracle_adamw {
    float beta2;
    float eps;
    float weight_decay;
    int32_t reserved;
} oracle_adamw;

/* threads the OpenMP loops below run on */
int oracle_threads(void) { return omp_get_max_threads(); }

/* run the loops below on n threads (timing the oracle on one core) */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ------------------------------------------------------------------------ */
/* DCT-II basis, straight from its definition.                               */
/* ------------------------------------------------------------------------ */

void oracle_basis(double *B /* [32][32], B[j*32+i] */)
{
    const double pi = 3.14159265358979323846;
    for (int j = 0; j < OR_CHUNK; j++) {
        double s = (j == 0) ? sqrt(1.0 / OR_CHUNK) : sqrt(2.0 / OR_CHUNK);
        for (int i = 0; i < OR_CHUNK; i++)
            B[j * OR_CHUNK + i] = s * cos(pi * (2 * i + 1) * j / (2.0 * OR_CHUNK));
    }
}

/* X_j = sum_i B[j][i] u_i */
static void dct_with(const double *B, const double *u, double *X)
{
    for (int j = 0; j < OR_CHUNK; j++) {
        double acc = 0.0;
        for (int i = 0; i < OR_CHUNK; i++)
            acc += B[j * OR_CHUNK + i] * u[i];
        X[j] = acc;
    }
}

/* u_i = sum_j B[j][i] X_j   (B is orthonormal, so this is the inverse) */
static void idct_with(const double *B, const double *X, double *u)
{
    for (int i = 0; i < OR_CHUNK; i++) {
        double acc = 0.0;
        for (int j = 0; j < OR_CHUNK; j++)
            acc += B[j * OR_CHUNK + i] * X[j];
        u[i] = acc;
    }
}

void oracle_dct(const double *u, double *X)
{
    double B[OR_CHUNK * OR_CHUNK];
    oracle_basis(B);
    dct_with(B, u, X);
}

void oracle_idct(const double *X, double *u)
{
    double B[OR_CHUNK * OR_CHUNK];
    oracle_basis(B);
    idct_with(B, X, u);
}

/* ------------------------------------------------------------------------ */
/* Top-k: order all 32 positions by (|X| rounded to fp32, descending; index  */
/* ascending), keep the first k, and return them in ascending index order.   */
/* ------------------------------------------------------------------------ */

static int ranks_before(const double *X, int a, int b)
{
    /* does position a come before position b in the ranking? */
    float fa = fabsf((float)X[a]);
    float fb = fabsf((float)X[b]);
    if (fa != fb)
        return fa > fb;
    return a < b;
}

int oracle_topk(const double *X, int k, int32_t *out /* [k], ascending */)
{
    if (k < 1 || k > OR_CHUNK)
        return -1;
    int order[OR_CHUNK];
    for (int i = 0; i < OR_CHUNK; i++)
        order[i] = i;
    /* insertion sort by the ranking above */
    for (int i = 1; i < OR_CHUNK; i++) {
        int v = order[i];
        int p = i;
        while (p > 0 && ranks_before(X, v, order[p - 1])) {
            order[p] = order[p - 1];
            p--;
        }
        order[p] = v;
    }
    /* the first k, re-sorted by index */
    int sel[OR_CHUNK];
    for (int s = 0; s < k; s++)
        sel[s] = order[s];
    for (int i = 1; i < k; i++) {
        int v = sel[i];
        int p = i;
        while (p > 0 && sel[p - 1] > v) {
            sel[p] = sel[p - 1];
            p--;
        }
        sel[p] = v;
    }
    for (int s = 0; s < k; s++)
        out[s] = sel[s];
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), from its definition.   */
/* ------------------------------------------------------------------------ */

void oracle_philox4x32(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; round++) {
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)x0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ x1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ x3 ^ k1;
        uint32_t n3 = lo0;
        x0 = n0; x1 = n1; x2 = n2; x3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

#define OR_TAG_SELECT 1u

/* n distinct positions of a chunk, drawn one by one without replacement:
 * draw i picks uniformly (multiply-shift of a 32-bit Philox word) among the
 * 32-i positions not yet taken, counting the free positions from bit 0 up. */
uint32_t oracle_select_mask(uint64_t seed, uint64_t step, uint64_t chunk, int n)
{
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t w[4] = { 0, 0, 0, 0 };
    uint32_t mask = 0;
    for (int i = 0; i < n && i < OR_CHUNK; i++) {
        if (i % 4 == 0) {
            uint32_t ctr[4] = { (uint32_t)chunk, (uint32_t)(chunk >> 32), (uint32_t)step,
                                (OR_TAG_SELECT << 24) | (uint32_t)(i / 4) };
            oracle_philox4x32(ctr, key, w);
        }
        uint32_t r = (uint32_t)(((uint64_t)w[i % 4] * (uint64_t)(OR_CHUNK - i)) >> 32);
        uint32_t seen = 0;
        for (int b = 0; b < OR_CHUNK; b++) {
            if (mask & (1u << b))
                continue;
            if (seen == r) {
                mask |= 1u << b;
                break;
            }
            seen++;
        }
    }
    return mask;
}

/* positions j with j mod (32/n) == step mod (32/n) */
uint32_t oracle_stride_mask(uint64_t step, int n)
{
    if (n < 1 || n > OR_CHUNK || OR_CHUNK % n != 0)
        return 0;
    int stride = OR_CHUNK / n;
    int offset = (int)(step % (uint64_t)stride);
    uint32_t mask = 0;
    for (int j = 0; j < OR_CHUNK; j++)
        if (j % stride == offset)
            mask |= 1u << j;
    return mask;
}

static int is_sync_step(const oracle_params *p)
{
    return p->period >= 1 && (p->step % (uint64_t)p->period) == (uint64_t)(p->period - 1);
}

/* positions selected in the parameter domain for the non-DCT schemes */
static uint32_t param_domain_mask(const oracle_params *p, uint64_t chunk_id)
{
    switch (p->scheme) {
    case OR_RANDOM: return oracle_select_mask(p->seed, p->step, chunk_id, p->k);
    case OR_STRIDE: return oracle_stride_mask(p->step, p->k);
    case OR_DILOCO: return is_sync_step(p) ? 0xFFFFFFFFu : 0u;
    default: return 0u;
    }
}

/* slots per chunk carried by one payload for this step */
int oracle_slots(const oracle_params *p)
{
    if (p->scheme == OR_DILOCO)
        return is_sync_step(p) ? OR_CHUNK : 0;
    return p->k;
}

/* ------------------------------------------------------------------------ */
/* fp16 (IEEE binary16) round-to-nearest-even, written from the format.      */
/* ------------------------------------------------------------------------ */

uint16_t oracle_to_f16_bits(double x)
{
    /* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;
     * subnormal quantum 2^-24, smallest normal 2^-14, largest finite 65504 */
    uint16_t sgn = (uint16_t)(signbit(x) ? 0x8000u : 0u);
    if (isnan(x))
        return 0x7E00u;
    double a = fabs(x);
    if (a == 0.0)
        return sgn;
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    int E = e - 1; /* a in [2^E, 2^(E+1)) */
    if (E < -14)
        E = -14; /* subnormal range shares the quantum of the smallest binade */
    double quantum = ldexp(1.0, E - 10);
    double q = a / quantum; /* exact: division by a power of two */
    double fl = floor(q);
    double rem = q - fl;
    double n = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))
        n = fl + 1.0;
    if (n >= 2048.0) { /* rounded up into the next binade */
        n = 1024.0;
        E += 1;
    }
    if (n < 1024.0) /* subnormal (E == -14): the bits are the count itself */
        return (uint16_t)(sgn | (uint16_t)n);
    if (E > 15)
        return (uint16_t)(sgn | 0x7C00u);
    return (uint16_t)(sgn | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0));
}

double oracle_from_f16_bits(uint16_t h)
{
    int s = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int mant = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)mant, -24);
    else if (ex == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp(1.0 + mant / 1024.0, ex - 15);
    return s ? -v : v;
}

static double sgn_of(double x)
{
    float f = (float)x;
    if (f > 0.0f)
        return 1.0;
    if (f < 0.0f)
        return -1.0;
    return 0.0;
}

/* the value a slot carries on the wire */
double oracle_wire_value(const oracle_params *p, double x)
{
    if (p->sign)
        return sgn_of(x);
    if (p->value_fmt == OR_F16)
        return oracle_from_f16_bits(oracle_to_f16_bits(x));
    return (double)(float)x;
}

/* ------------------------------------------------------------------------ */
/* Guide: where more than one result is correct, take the one another        */
/* implementation chose, and only there.                                     */
/*  - positions (DCT): the guide's k positions must be distinct, ascending   */
/*    and in [0, 32), and every guided |X_j| must be at least every unguided */
/*    |X_j| less near * max_j |X_j| (fp64 coefficients): then they are a     */
/*    valid top-k up to rounding and are adopted (GUIDE_POSITIONS);          */
/*  - signs (sign before sync): a slot whose guided ternary value differs    */
/*    from sign(x) is adopted if |x| <= near * max_j |x_j| (x = X for DCT,   */
/*    u otherwise; GUIDE_SIGNS);                                             */
/*  - anything else that differs is GUIDE_REJECTED and the oracle keeps its  */
/*    own choice.  Values with the sign off are not guided.                  */
/* ------------------------------------------------------------------------ */

enum { OR_GUIDE_POSITIONS = 1, OR_GUIDE_SIGNS = 2, OR_GUIDE_REJECTED = 4 };

static int guide_is_near_topk(const double *X, const int32_t *gidx, int k, double near)
{
    uint32_t in = 0;
    for (int s = 0; s < k; s++) {
        if (gidx[s] < 0 || gidx[s] >= OR_CHUNK)
            return 0;
        if (s > 0 && gidx[s] <= gidx[s - 1])
            return 0;
        in |= 1u << gidx[s];
    }
    double top = 0.0, min_in = INFINITY, max_out = 0.0;
    for (int j = 0; j < OR_CHUNK; j++) {
        double a = fabs(X[j]);
        if (a > top)
            top = a;
        if (in & (1u << j)) {
            if (a < min_in)
                min_in = a;
        } else if (a > max_out) {
            max_out = a;
        }
    }
    return min_in >= max_out - near * top;
}

/* ------------------------------------------------------------------------ */
/* Encode: Algorithm 1 steps 3-5 for a list of chunks.                       */
/*   g      : fp32 gradients, [n][32], padded positions ignored              */
/*   m      : fp64 momentum state, [n][32], updated in place (pads kept 0)   */
/*   nvalid : valid elements of each chunk (1..32)                           */
/*   chunk_id: global chunk index of each chunk (Random hashing)             */
/* Outputs (any may be NULL):                                                */
/*   slot_idx [n][slots] chunk-local position of each slot (ascending)       */
/*   slot_val [n][slots] the value the slot carries on the wire              */
/*   q_out    [n][32]    extracted component q                               */
/*   x_out    [n][32]    DCT coefficients (DCT scheme) or u (others)         */
/* Guide (all NULL for a plain encode): guide_idx / guide_val [n][slots] in   */
/* the layout of slot_idx / slot_val, tolerance near, and guide_status [n]    */
/* receiving the OR_GUIDE_* bits of each chunk (0: nothing differed).         */
/* Returns slots per chunk, or -1 on a bad configuration.                    */
/* ------------------------------------------------------------------------ */

static int encode_impl(const oracle_params *p, double gamma, int64_t n, const uint64_t *chunk_id,
                       const int32_t *nvalid, const float *g, double *m, int32_t *slot_idx, double *slot_val,
                       double *q_out, double *x_out, const int32_t *guide_idx, const double *guide_val,
                       double near, int32_t *guide_status)
{
    if (p->scheme < OR_DCT || p->scheme > OR_DILOCO)
        return -1;
    if (p->scheme != OR_DILOCO && (p->k < 1 || p->k > OR_CHUNK))
        return -1;
    if (p->scheme == OR_STRIDE && OR_CHUNK % p->k != 0)
        return -1;
    if (p->scheme == OR_DILOCO && p->period < 1)
        return -1;
    const int slots = oracle_slots(p);
    const int guided = guide_idx != NULL && guide_val != NULL;
    const double beta = (double)p->beta;
    double B[OR_CHUNK * OR_CHUNK];
    oracle_basis(B);

#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n; c++) {
        const int nv = nvalid[c];
        const float *gc = g + c * OR_CHUNK;
        double *mc = m + c * OR_CHUNK;
        double u[OR_CHUNK], q[OR_CHUNK], X[OR_CHUNK];
        int32_t sel[OR_CHUNK];
        double val[OR_CHUNK];
        double raw[OR_CHUNK]; /* the selected value of each slot, before the wire */
        int status = 0;

        /* step 3: momentum accumulation (pads are zero); gamma = 1, or 1 - beta1
         * for the AdamW first moment */
        for (int i = 0; i < OR_CHUNK; i++)
            u[i] = (i < nv) ? beta * mc[i] + gamma * (double)gc[i] : 0.0;

        /* step 4: extract q */
        for (int i = 0; i < OR_CHUNK; i++)
            q[i] = 0.0;
        if (p->scheme == OR_DCT) {
            double Xs[OR_CHUNK];
            dct_with(B, u, X);
            oracle_topk(X, p->k, sel);
            if (guided) {
                const int32_t *gs = guide_idx + c * slots;
                int differs = 0;
                for (int s = 0; s < slots; s++)
                    differs |= gs[s] != sel[s];
                if (differs) {
                    if (guide_is_near_topk(X, gs, slots, near)) {
                        for (int s = 0; s < slots; s++)
                            sel[s] = gs[s];
                        status |= OR_GUIDE_POSITIONS;
                    } else {
                        status |= OR_GUIDE_REJECTED;
                    }
                }
            }
            for (int j = 0; j < OR_CHUNK; j++)
                Xs[j] = 0.0;
            for (int s = 0; s < slots; s++) {
                Xs[sel[s]] = X[sel[s]];
                raw[s] = X[sel[s]];
            }
            idct_with(B, Xs, q);
        } else {
            uint32_t mask = param_domain_mask(p, chunk_id[c]);
            int s = 0;
            for (int j = 0; j < OR_CHUNK; j++) {
                X[j] = u[j];
                if (mask & (1u << j)) {
                    q[j] = u[j];
                    sel[s] = j;
                    raw[s] = u[j];
                    s++;
                }
            }
        }
        for (int s = 0; s < slots; s++)
            val[s] = oracle_wire_value(p, raw[s]);
        if (guided && p->sign) {
            const double *gv = guide_val + c * slots;
            double top = 0.0;
            for (int j = 0; j < OR_CHUNK; j++)
                if (fabs(X[j]) > top)
                    top = fabs(X[j]);
            for (int s = 0; s < slots; s++) {
                if (gv[s] == val[s])
                    continue;
                int ternary = gv[s] == 1.0 || gv[s] == -1.0 || gv[s] == 0.0;
                if (ternary && fabs(raw[s]) <= near * top) {
                    val[s] = gv[s];
                    status |= OR_GUIDE_SIGNS;
                } else {
                    status |= OR_GUIDE_REJECTED;
                }
            }
        }

        /* step 5: error feedback */
        for (int i = 0; i < OR_CHUNK; i++)
            mc[i] = (i < nv) ? u[i] - q[i] : 0.0;

        for (int s = 0; s < slots; s++) {
            if (slot_idx)
                slot_idx[c * slots + s] = sel[s];
            if (slot_val)
                slot_val[c * slots + s] = val[s];
        }
        if (q_out)
            for (int i = 0; i < OR_CHUNK; i++)
                q_out[c * OR_CHUNK + i] = (i < nv) ? q[i] : 0.0;
        if (x_out)
            for (int i = 0; i < OR_CHUNK; i++)
                x_out[c * OR_CHUNK + i] = X[i];
        if (guide_status)
            guide_status[c] = status;
    }
    return slots;
}

int oracle_encode(const oracle_params *p, int64_t n, const uint64_t *chunk_id, const int32_t *nvalid,
                  const float *g, double *m, int32_t *slot_idx, double *slot_val, double *q_out,
                  double *x_out, const int32_t *guide_idx, const double *guide_val, double near,
                  int32_t *guide_status)
{
    return encode_impl(p, 1.0, n, chunk_id, nvalid, g, m, slot_idx, slot_val, q_out, x_out, guide_idx, guide_val,
                       near, guide_status);
}

/* Decoupled AdamW encode: the second moment v (fp64, [n][32], pads kept 0)
 * takes g^2; the first moment m then goes through the same steps 3-5. */
int oracle_encode_adamw(const oracle_params *p, const oracle_adamw *w, int64_t n, const uint64_t *chunk_id,
                        const int32_t *nvalid, const float *g, double *m, double *v, int32_t *slot_idx,
                        double *slot_val, double *q_out, double *x_out, const int32_t *guide_idx,
                        const double *guide_val, double near, int32_t *guide_status)
{
    if (p->sign)
        return -1;
    const double beta2 = (double)w->beta2;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n; c++)
        for (int i = 0; i < OR_CHUNK; i++) {
            const double gi = (double)g[c * OR_CHUNK + i];
            v[c * OR_CHUNK + i] = (i < nvalid[c]) ? beta2 * v[c * OR_CHUNK + i] + (1.0 - beta2) * gi * gi : 0.0;
        }
    return encode_impl(p, 1.0 - (double)p->beta, n, chunk_id, nvalid, g, m, slot_idx, slot_val, q_out, x_out,
                       guide_idx, guide_val, near, guide_status);
}

/* ------------------------------------------------------------------------ */
/* Decode: Algorithm 1 steps 6-7 for a list of chunks.                       */
/*   R payloads, each given as slot_idx [R][n][slots] (DCT only; the other   */
/*   schemes recompute positions from the shared seed) and slot_val          */
/*   [R][n][slots].  theta is fp64 [n][32], updated in place.                */
/*   Q_out (may be NULL) receives the aggregate Q, [n][32].                  */
/* ------------------------------------------------------------------------ */

static int decode_impl(const oracle_params *p, const oracle_adamw *w, const double *v, int64_t n,
                       const uint64_t *chunk_id, const int32_t *nvalid, int32_t R, const int32_t *slot_idx,
                       const double *slot_val, double *theta, double *Q_out)
{
    if (R < 1)
        return -1;
    /* AdamW: bias corrections of step t = step + 1 */
    const double t = (double)p->step + 1.0;
    const double c1 = w ? 1.0 / (1.0 - pow((double)p->beta, t)) : 1.0;
    const double c2 = w ? 1.0 / (1.0 - pow((double)w->beta2, t)) : 1.0;
    const int slots = oracle_slots(p);
    if (slots == 0) { /* DiLoCo between syncs: no payload, no update */
        if (Q_out)
            memset(Q_out, 0, sizeof(double) * (size_t)n * OR_CHUNK);
        return 0;
    }
    const double lr = (double)p->lr;
    double B[OR_CHUNK * OR_CHUNK];
    oracle_basis(B);

#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n; c++) {
        const int nv = nvalid[c];
        double A[OR_CHUNK], Q[OR_CHUNK];
        for (int j = 0; j < OR_CHUNK; j++)
            A[j] = 0.0;
        if (p->scheme == OR_DCT) {
            for (int r = 0; r < R; r++)
                for (int s = 0; s < slots; s++) {
                    int64_t e = ((int64_t)r * n + c) * slots + s;
                    A[slot_idx[e]] += slot_val[e];
                }
            for (int j = 0; j < OR_CHUNK; j++)
                A[j] = A[j] / (double)R;
            idct_with(B, A, Q);
        } else {
            uint32_t mask = param_domain_mask(p, chunk_id[c]);
            int s = 0;
            for (int j = 0; j < OR_CHUNK; j++) {
                Q[j] = 0.0;
                if (mask & (1u << j)) {
                    double sum = 0.0;
                    for (int r = 0; r < R; r++)
                        sum += slot_val[((int64_t)r * n + c) * slots + s];
                    Q[j] = sum / (double)R;
                    s++;
                }
            }
        }
        for (int i = 0; i < nv; i++) {
            double *th = &theta[c * OR_CHUNK + i];
            if (w)
                *th -= lr * (c1 * Q[i] / (sqrt(c2 * v[c * OR_CHUNK + i]) + (double)w->eps) +
                             (double)w->weight_decay * *th);
            else
                *th -= lr * Q[i];
        }
        if (Q_out)
            for (int i = 0; i < OR_CHUNK; i++)
                Q_out[c * OR_CHUNK + i] = (i < nv) ? Q[i] : 0.0;
    }
    return 0;
}

int oracle_decode(const oracle_params *p, int64_t n, const uint64_t *chunk_id, const int32_t *nvalid,
                  int32_t R, const int32_t *slot_idx, const double *slot_val, double *theta,
                  double *Q_out)
{
    return decode_impl(p, NULL, NULL, n, chunk_id, nvalid, R, slot_idx, slot_val, theta, Q_out);
}

/* Decoupled AdamW decode: Q as above, applied with the own second moment v. */
int oracle_decode_adamw(const oracle_params *p, const oracle_adamw *w, int64_t n, const uint64_t *chunk_id,
                        const int32_t *nvalid, int32_t R, const int32_t *slot_idx, const double *slot_val,
                        const double *v, double *theta, double *Q_out)
{
    if (p->sign)
        return -1;
    return decode_impl(p, w, v, n, chunk_id, nvalid, R, slot_idx, slot_val, theta, Q_out);
}

/* ------------------------------------------------------------------------ */
/* Payload codec (one replica, one step, a whole shard of C chunks).         */
/* Regions, each starting at a multiple of 256 bytes, in this order:         */
/*   IDX (DCT only): uint8 [C][k], the chunk-local position of each slot     */
/*   NZ, NEG (ternary): uint64 [G][k], G = ceil(C/64); word g*k+s, bit b is  */
/*       slot s of chunk 64g+b; value = NZ ? (NEG ? -1 : +1) : 0             */
/*   VAL (fp16 / fp32 formats): [C][k] values                                */
/* The total is rounded up to 256 bytes.                                     */
/* ------------------------------------------------------------------------ */

static uint64_t up256(uint64_t x) { return (x + 255u) & ~(uint64_t)255u; }

/* out[0..7] = idx_off, idx_bytes, nz_off, neg_off, plane_bytes, val_off, val_bytes, total */
int oracle_payload_regions(const oracle_params *p, uint64_t n_elems, uint64_t *out)
{
    uint64_t C = (n_elems + OR_CHUNK - 1) / OR_CHUNK;
    uint64_t G = (C + 63) / 64;
    uint64_t k = (uint64_t)(p->scheme == OR_DILOCO ? OR_CHUNK : p->k);
    uint64_t off = 0;
    uint64_t idx_off = 0, idx_bytes = 0, nz_off = 0, neg_off = 0, plane_bytes = 0, val_off = 0,
             val_bytes = 0;
    if (p->scheme == OR_DCT) {
        idx_off = off;
        idx_bytes = C * k;
        off = up256(off + idx_bytes);
    }
    if (p->value_fmt == OR_TERNARY) {
        plane_bytes = G * k * 8u;
        nz_off = off;
        off = up256(off + plane_bytes);
        neg_off = off;
        off = up256(off + plane_bytes);
    } else {
        val_bytes = C * k * (p->value_fmt == OR_F16 ? 2u : 4u);
        val_off = off;
        off = up256(off + val_bytes);
    }
    out[0] = idx_off; out[1] = idx_bytes; out[2] = nz_off; out[3] = neg_off;
    out[4] = plane_bytes; out[5] = val_off; out[6] = val_bytes; out[7] = off;
    return 0;
}

/* slot_idx / slot_val as produced by oracle_encode for chunks 0..C-1 */
int oracle_pack(const oracle_params *p, uint64_t n_elems, const int32_t *slot_idx,
                const double *slot_val, uint8_t *buf)
{
    uint64_t reg[8];
    oracle_payload_regions(p, n_elems, reg);
    memset(buf, 0, reg[7]);
    uint64_t C = (n_elems + OR_CHUNK - 1) / OR_CHUNK;
    int k = (p->scheme == OR_DILOCO) ? OR_CHUNK : p->k;
    for (uint64_t c = 0; c < C; c++) {
        for (int s = 0; s < k; s++) {
            uint64_t e = c * (uint64_t)k + (uint64_t)s;
            if (p->scheme == OR_DCT)
                buf[reg[0] + e] = (uint8_t)slot_idx[e];
            double v = slot_val[e];
            if (p->value_fmt == OR_TERNARY) {
                if (v != 1.0 && v != -1.0 && v != 0.0)
                    return -1;
                uint64_t word = (c / 64) * (uint64_t)k + (uint64_t)s;
                uint64_t bit = c % 64;
                uint64_t *nz = (uint64_t *)(buf + reg[2]);
                uint64_t *neg = (uint64_t *)(buf + reg[3]);
                if (v != 0.0)
                    nz[word] |= (uint64_t)1 << bit;
                if (v < 0.0)
                    neg[word] |= (uint64_t)1 << bit;
            } else if (p->value_fmt == OR_F16) {
                ((uint16_t *)(buf + reg[5]))[e] = oracle_to_f16_bits(v);
            } else {
                ((float *)(buf + reg[5]))[e] = (float)v;
            }
        }
    }
    return 0;
}

/* Inverse of oracle_pack for the chunks listed in chunks[0..nchunks) (all C
 * chunks in order when chunks is NULL): row i of slot_idx / slot_val receives
 * chunk chunks[i].  Returns -1 if the buffer is malformed anywhere (a NEG bit
 * set without its NZ bit, or a plane bit set for a chunk c >= C), whichever
 * chunks were asked for. */
int oracle_unpack_chunks(const oracle_params *p, uint64_t n_elems, const uint8_t *buf,
                         const uint64_t *chunks, uint64_t nchunks, int32_t *slot_idx, double *slot_val)
{
    uint64_t reg[8];
    oracle_payload_regions(p, n_elems, reg);
    uint64_t C = (n_elems + OR_CHUNK - 1) / OR_CHUNK;
    uint64_t G = (C + 63) / 64;
    int k = (p->scheme == OR_DILOCO) ? OR_CHUNK : p->k;
    const uint64_t *nz = (const uint64_t *)(buf + reg[2]);
    const uint64_t *neg = (const uint64_t *)(buf + reg[3]);
    int bad = 0;
    if (p->value_fmt == OR_TERNARY) {
        /* chunks of the last group at or past C: bits C-64(G-1) .. 63 */
        uint64_t used = C - 64 * (G - 1);
        uint64_t past = used == 64 ? 0 : ~(((uint64_t)1 << used) - 1);
        for (uint64_t w = 0; w < G * (uint64_t)k; w++) {
            if (neg[w] & ~nz[w])
                bad = 1;
            if (w / (uint64_t)k == G - 1 && (nz[w] & past))
                bad = 1;
        }
    }
    uint64_t rows = chunks ? nchunks : C;
    for (uint64_t i = 0; i < rows; i++) {
        uint64_t c = chunks ? chunks[i] : i;
        if (c >= C)
            return -2;
        for (int s = 0; s < k; s++) {
            uint64_t e = c * (uint64_t)k + (uint64_t)s;
            uint64_t o = i * (uint64_t)k + (uint64_t)s;
            if (slot_idx)
                slot_idx[o] = (p->scheme == OR_DCT) ? (int32_t)buf[reg[0] + e] : -1;
            double v;
            if (p->value_fmt == OR_TERNARY) {
                uint64_t word = (c / 64) * (uint64_t)k + (uint64_t)s;
                uint64_t bit = c % 64;
                int isnz = (int)((nz[word] >> bit) & 1u);
                int isneg = (int)((neg[word] >> bit) & 1u);
                v = isnz ? (isneg ? -1.0 : 1.0) : 0.0;
            } else if (p->value_fmt == OR_F16) {
                v = oracle_from_f16_bits(((const uint16_t *)(buf + reg[5]))[e]);
            } else {
                v = (double)((const float *)(buf + reg[5]))[e];
            }
            if (slot_val)
                slot_val[o] = v;
        }
    }
    return bad ? -1 : 0;
}

/* inverse of oracle_pack over the whole shard; -1 for a malformed buffer */
int oracle_unpack(const oracle_params *p, uint64_t n_elems, const uint8_t *buf, int32_t *slot_idx,
                  double *slot_val)
{
    return oracle_unpack_chunks(p, n_elems, buf, NULL, 0, slot_idx, slot_val);
}

/* Violations of the payload format (the statement above and the library
 * header's), counted one by one over the whole buffer:
 *  - TERNARY: a NEG bit without its NZ bit, for a chunk c < C;
 *  - TERNARY: every NZ or NEG bit set for a chunk c >= C (the last group);
 *  - DCT: an IDX byte above 31;
 *  - DCT: slot s >= 1 of a chunk whose IDX byte is not above slot s-1's
 *    (positions must ascend strictly; compared as raw bytes);
 *  - F16 / F32 with the sign on: a value other than -1, 0 or +1;
 *  - F16 / F32 with the sign off: a value that is not finite.
 * A DILOCO step that sends nothing has no payload and no violation. */
uint64_t oracle_payload_violations(const oracle_params *p, uint64_t n_elems, const uint8_t *buf)
{
    if (p->scheme == OR_DILOCO && !is_sync_step(p))
        return 0;
    uint64_t reg[8];
    oracle_payload_regions(p, n_elems, reg);
    uint64_t C = (n_elems + OR_CHUNK - 1) / OR_CHUNK;
    uint64_t G = (C + 63) / 64;
    int k = (p->scheme == OR_DILOCO) ? OR_CHUNK : p->k;
    uint64_t bad = 0;
    for (uint64_t c = 0; c < G * 64; c++) {
        for (int s = 0; s < k; s++) {
            uint64_t e = c * (uint64_t)k + (uint64_t)s;
            if (p->value_fmt == OR_TERNARY) {
                uint64_t word = (c / 64) * (uint64_t)k + (uint64_t)s;
                int nz = (int)((((const uint64_t *)(buf + reg[2]))[word] >> (c % 64)) & 1u);
                int ng = (int)((((const uint64_t *)(buf + reg[3]))[word] >> (c % 64)) & 1u);
                if (c < C)
                    bad += (uint64_t)(ng && !nz);
                else
                    bad += (uint64_t)nz + (uint64_t)ng;
            } else if (c < C) {
                double v = (p->value_fmt == OR_F16) ? oracle_from_f16_bits(((const uint16_t *)(buf + reg[5]))[e])
                                                    : (double)((const float *)(buf + reg[5]))[e];
                if (p->sign)
                    bad += (uint64_t)!(v == 0.0 || v == 1.0 || v == -1.0);
                else
                    bad += (uint64_t)!isfinite(v);
            }
            if (p->scheme == OR_DCT && c < C) {
                uint8_t b = buf[reg[0] + e];
                bad += (uint64_t)(b > 31);
                if (s > 0)
                    bad += (uint64_t)(b <= buf[reg[0] + e - 1]);
            }
        }
    }
    return bad;
}
