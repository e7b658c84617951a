/*
 * hpo_oracle.c -- plain, slow CPU oracle for the mixed-precision AdamW step.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this file's library.  The product library never
 * links, calls or includes anything from here, and this file includes nothing
 * from the product.  It is written straight from the pages below, one step at
 * a time, with no blocking, fusion or reordering.
 *
 * Sources (web pages):
 *   [OPT-INFRA]  "02 · Optimizer：算法与 infra" (llm-infra-atlas, train/02_optimizer)
 *   [HANDBOOK]   "优化器：AdamW、Muon 与分布式优化器" (ai-infra-handbooks, train/algo/optimizer)
 *   [FP32-RFC]   "支持FP32优化器" / "AutoModels Trainer 支持 FP32 main_param 优化器"
 *                (hyper-parallel issue)
 *
 * Two arithmetic variants of the update:
 *   O32 -- every operation the formulas print is one IEEE binary32 operation,
 *          rounded to nearest even, in the printed order, no fused
 *          multiply-add (built with -ffp-contract=off, no fast-math).  The
 *          pages' state (fp32 master, fp32 m and v) is fp32, so this is the
 *          reading used for element-by-element parity.
 *   O64 -- the same formulas evaluated in binary64 with the exact (double)
 *          hyperparameters and no intermediate fp32 rounding; only the state
 *          written back is rounded to fp32.  It is the exact shadow that the
 *          tests use to bound O32's own rounding.
 *
 * Derived scalars (both variants of the hyperparameters' fp32 images) are
 * formed in binary64 and rounded to binary32 once.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_ADAMW 0   /* decoupled weight decay ([OPT-INFRA] §3 AdamW equation) */
#define ORC_ADAM_L2 1 /* L2 term folded into the gradient ([OPT-INFRA] §3, first form) */

int32_t orc_version(void) { return 1; }

/* ------------------------------------------------------------------------ */
/* fp32 -> bf16 write-back.  The pages only say the master is cast to the   */
/* 16-bit model dtype ([OPT-INFRA] §9.2 table, "参数写回"; [FP32-RFC] case  */
/* 1 check "model param equals bf16(main_param)").  Reading: IEEE binary32  */
/* -> bfloat16 round to nearest, ties to even; subnormals kept; overflow to */
/* infinity; NaN mapped to the quiet NaN 0x7FC0 with the input's sign.      */
/* Written from the definition: keep the top 16 bits (truncation toward     */
/* zero in magnitude), then look at the 16 discarded bits: more than half   */
/* an ulp rounds the magnitude up, exactly half rounds to the even result.  */
/* A carry out of the mantissa moves into the exponent, which is what IEEE  */
/* rounding asks for (up to and including infinity).                        */
/* ------------------------------------------------------------------------ */
uint16_t orc_bf16_rne(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, sizeof bits);
    uint32_t sign = bits & 0x80000000u;
    uint32_t mag = bits & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) /* NaN */
        return (uint16_t)((sign >> 16) | 0x7FC0u);
    uint32_t kept = mag >> 16;          /* truncated magnitude, 15 bits */
    uint32_t discarded = mag & 0xFFFFu; /* the 16 bits that are dropped */
    int round_up = 0;
    if (discarded > 0x8000u)
        round_up = 1;
    else if (discarded == 0x8000u && (kept & 1u))
        round_up = 1; /* tie: go to the even neighbour */
    kept += (uint32_t)round_up;
    return (uint16_t)((sign >> 16) | kept);
}

void orc_bf16_rne_array(const float* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_rne(x[i]);
}

/* Same, over the 2^count consecutive fp32 bit patterns starting at first
 * (used by the exhaustive write-back pin; no array of inputs needed). */
void orc_bf16_rne_patterns(uint32_t first, int64_t count, uint16_t* out)
{
    for (int64_t i = 0; i < count; ++i) {
        uint32_t b = first + (uint32_t)i;
        float x;
        memcpy(&x, &b, sizeof x);
        out[i] = orc_bf16_rne(x);
    }
}

/* ------------------------------------------------------------------------ */
/* fp32 -> fp16 write-back for fp16 model params ([OPT-INFRA] §9.2: the     */
/* master is cast to the 16-bit model dtype, fp16 or bf16).  Reading: IEEE  */
/* binary32 -> binary16 round to nearest, ties to even, with binary16       */
/* subnormals, overflow to infinity, NaN -> quiet NaN 0x7E00 with the sign. */
/* Written from the definition: the value is sig * 2^(e - 23) with a 24-bit */
/* significand; the binary16 quantum is 2^(e - 10) for normal results and   */
/* 2^-24 below 2^-14; the significand is divided by the quantum with the    */
/* dropped bits deciding the rounding, and the encoding is built by adding  */
/* the kept significand to the biased exponent field, so a carry moves into */
/* the exponent (up to infinity).                                           */
/* ------------------------------------------------------------------------ */
uint16_t orc_fp16_rne(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, sizeof bits);
    const uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    const uint32_t mag = bits & 0x7FFFFFFFu;
    if (mag > 0x7F800000u)
        return (uint16_t)(sign | 0x7E00u);
    if (mag == 0x7F800000u)
        return (uint16_t)(sign | 0x7C00u);
    const int biased = (int)(mag >> 23);
    if (biased == 0) /* fp32 zero or subnormal: far below 2^-25, rounds to zero */
        return sign;
    const uint32_t sig = (mag & 0x7FFFFFu) | 0x800000u;
    const int e = biased - 127;                /* value = sig * 2^(e - 23) */
    const int q = e >= -14 ? e - 10 : -24;     /* log2 of the binary16 quantum */
    const int shift = q - (e - 23);            /* significand bits dropped, >= 13 */
    if (shift > 24)
        return sign;                           /* below half the smallest subnormal */
    uint32_t kept = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (kept & 1u)))
        kept += 1u;
    uint32_t enc;
    if (q == -24)
        enc = kept;                            /* subnormal; kept == 1024 is the smallest normal */
    else
        enc = ((uint32_t)(e + 15) << 10) + (kept - 1024u);
    if (enc >= 0x7C00u)
        enc = 0x7C00u;                         /* overflow */
    return (uint16_t)(sign | enc);
}

void orc_fp16_rne_array(const float* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_fp16_rne(x[i]);
}

void orc_fp16_rne_patterns(uint32_t first, int64_t count, uint16_t* out)
{
    for (int64_t i = 0; i < count; ++i) {
        uint32_t b = first + (uint32_t)i;
        float x;
        memcpy(&x, &b, sizeof x);
        out[i] = orc_fp16_rne(x);
    }
}

/* bf16 bits -> fp32 value (exact: bf16 is the top half of binary32). */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return x;
}

/* ------------------------------------------------------------------------ */
/* a1: non-finite check over the stored (still scaled) gradients.           */
/* [OPT-INFRA] §9.2 table (unscale row) and §10.2: one pass sets found_inf  */
/* when any main grad is inf or NaN; the values checked are the stored ones.*/
/* ------------------------------------------------------------------------ */
int32_t orc_any_nonfinite(const float* G, int64_t n)
{
    int32_t found = 0;
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(G[i]))
            found = 1;
    return found;
}

/* a1, the pages' in-place form: G <- fp32(G * inv_scale). */
void orc_unscale_inplace(float* G, int64_t n, float inv_scale)
{
    for (int64_t i = 0; i < n; ++i)
        G[i] = G[i] * inv_scale;
}

/* ------------------------------------------------------------------------ */
/* a2: sum of squares of the unscaled gradient, [OPT-INFRA] §11.1 (total    */
/* norm is the square root of the sum of every grad's squared L2 norm).     */
/* The unscaled value g = fp32(G * inv) is squared exactly in binary64 (a   */
/* product of two 24-bit significands fits in 53 bits) and summed in order  */
/* in binary64.  For n terms the relative error of this plain sum is at     */
/* most n * 2^-53, i.e. 1e-6 at n = 8.75e9.                                 */
/* ------------------------------------------------------------------------ */
double orc_sumsq(const float* G, int64_t n, float inv_scale)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        float g = G[i] * inv_scale;
        double gd = (double)g;
        s = s + gd * gd;
    }
    return s;
}

/* ------------------------------------------------------------------------ */
/* Zero count of the step's gradient ([OPT-INFRA] §10.2: an applied step     */
/* returns (success, grad_norm, num_zeros); §17: log_num_zeros_in_grad).     */
/* The pages do not say which gradient is counted.  Reading: the unscaled    */
/* fp32 grad g = fp32(G * inv_scale), the same vector whose norm the step    */
/* returns; +0 and -0 both count (they compare equal), so a subnormal that   */
/* the unscale rounds to zero counts too.  NaN and inf are not zero.         */
/* ------------------------------------------------------------------------ */
int64_t orc_count_zeros(const float* G, int64_t n, float inv_scale)
{
    int64_t zeros = 0;
    for (int64_t i = 0; i < n; ++i) {
        float g = G[i] * inv_scale;
        if (g == 0.0f)
            zeros = zeros + 1;
    }
    return zeros;
}

/* ------------------------------------------------------------------------ */
/* a3: clip coefficient, [OPT-INFRA] §11.1: c = max_norm / (total + 1e-6),  */
/* applied only when c < 1; a non-positive max_norm turns clipping off.     */
/* The fp32 norm handed in is widened to binary64, c is formed in binary64  */
/* and rounded once to binary32.  Returns 1 when clipping applies.          */
/* ------------------------------------------------------------------------ */
int32_t orc_clip_coeff(double max_norm, float norm32, float* C_out, double* c64_out)
{
    *C_out = 1.0f;
    if (c64_out)
        *c64_out = 1.0;
    if (!(max_norm > 0.0))
        return 0;
    double c = max_norm / ((double)norm32 + 1e-6);
    if (c64_out)
        *c64_out = c;
    if (c < 1.0) {
        *C_out = (float)c;
        return 1;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a4 + a5: one Adam/AdamW step over n elements of one parameter group.     */
/*                                                                          */
/*   [OPT-INFRA] §2 equations: m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;*/
/*     m_hat = m / (1 - b1^t);  v_hat = v / (1 - b2^t);                     */
/*     update = m_hat / (sqrt(v_hat) + eps)   (eps outside the root).       */
/*   [OPT-INFRA] §3 AdamW equation with the step size eta = lr and the      */
/*     Adam factor alpha = 1:  theta <- theta - lr (update + wd theta).     */
/*     The decay per step is lr*wd, which the [HANDBOOK] experiment fixes   */
/*     through its (1 - lr*wd)^1000 closed form.                            */
/*   [OPT-INFRA] §3 L2 form: g <- g + wd theta before the moments, then     */
/*     theta <- theta - lr * update.                                        */
/*   Gradient entering the step: g = G * inv_scale, then g * C when the    */
/*     clip applies ([OPT-INFRA] §10.2 and §11.1: unscale, then clip, then  */
/*     the inner optimizer).                                                */
/*   t is the 1-based count of applied steps ([OPT-INFRA] §10.2: a skipped */
/*     step runs no inner step).                                            */
/*   Write-back: p <- bf16(theta) when p is given ([OPT-INFRA] §9.2);       */
/*     fp32 params are their own master and get no write-back ([FP32-RFC]   */
/*     §7.2, native fp32 params).                                           */
/* ------------------------------------------------------------------------ */
typedef struct {
    double lr, wd, beta1, beta2, eps;
    int64_t t;         /* 1-based applied-step count */
    int32_t mode;      /* ORC_ADAMW or ORC_ADAM_L2 */
    int32_t do_clip;   /* 1 when the clip coefficient applies */
    float inv_scale;   /* unscale multiplier (fp32, as the caller holds it) */
    float clip_C;      /* fp32 clip coefficient (O32) */
    double clip_c64;   /* binary64 clip coefficient (O64) */
    int32_t state_bf16;  /* O32 only: exp_avg / exp_avg_sq held as bf16 (uint16 arrays) */
    int32_t param_fp16;  /* the 16-bit model param is fp16 instead of bf16 */
} orc_update_args;

/* m and v point at fp32 arrays, or at bf16 (uint16) arrays when
 * a->state_bf16 is set ([OPT-INFRA] §16: the precision-aware optimizer may
 * keep exp_avg / exp_avg_sq in a lower precision).  Reading for bf16 moments:
 * they are widened exactly to fp32, the update runs in fp32 as above, and the
 * new moments are stored with the bf16 write-back rounding. */
void orc_update_f32(int64_t n, float* theta, void* m_ptr, void* v_ptr, const float* G,
                    uint16_t* p16, const orc_update_args* a)
{
    /* scalars: binary64 once, rounded to binary32 once */
    const float B1 = (float)a->beta1;
    const float B2 = (float)a->beta2;
    const float C1 = (float)(1.0 - a->beta1);
    const float C2 = (float)(1.0 - a->beta2);
    const float BC1 = (float)(1.0 - pow(a->beta1, (double)a->t));
    const float BC2 = (float)(1.0 - pow(a->beta2, (double)a->t));
    const float EPS = (float)a->eps;
    const float LR = (float)a->lr;
    const float WD = (float)a->wd;
    const float INV = a->inv_scale;
    const float C = a->clip_C;
    float* m32 = (float*)m_ptr;
    float* v32 = (float*)v_ptr;
    uint16_t* m16 = (uint16_t*)m_ptr;
    uint16_t* v16 = (uint16_t*)v_ptr;

    for (int64_t i = 0; i < n; ++i) {
        float g = G[i] * INV;
        if (a->do_clip)
            g = g * C;
        float th = theta[i];
        if (a->mode == ORC_ADAM_L2)
            g = g + WD * th;
        const float m_old = a->state_bf16 ? bf16_to_f32(m16[i]) : m32[i];
        const float v_old = a->state_bf16 ? bf16_to_f32(v16[i]) : v32[i];
        float mi = B1 * m_old + C1 * g;
        float vi = B2 * v_old + C2 * (g * g);
        float mh = mi / BC1;
        float vh = vi / BC2;
        float denom = sqrtf(vh) + EPS;
        float u = mh / denom;
        if (a->mode == ORC_ADAMW)
            th = th - LR * (u + WD * th);
        else
            th = th - LR * u;
        if (a->state_bf16) {
            m16[i] = orc_bf16_rne(mi);
            v16[i] = orc_bf16_rne(vi);
        } else {
            m32[i] = mi;
            v32[i] = vi;
        }
        theta[i] = th;
        if (p16)
            p16[i] = a->param_fp16 ? orc_fp16_rne(th) : orc_bf16_rne(th);
    }
}

void orc_update_f64(int64_t n, float* theta, float* m, float* v, const float* G,
                    uint16_t* p_bf16, const orc_update_args* a)
{
    const double b1 = a->beta1, b2 = a->beta2;
    const double bc1 = 1.0 - pow(b1, (double)a->t);
    const double bc2 = 1.0 - pow(b2, (double)a->t);
    for (int64_t i = 0; i < n; ++i) {
        double g = (double)G[i] * (double)a->inv_scale;
        if (a->do_clip)
            g = g * a->clip_c64;
        double th = (double)theta[i];
        if (a->mode == ORC_ADAM_L2)
            g = g + a->wd * th;
        double mi = b1 * (double)m[i] + (1.0 - b1) * g;
        double vi = b2 * (double)v[i] + (1.0 - b2) * (g * g);
        double u = (mi / bc1) / (sqrt(vi / bc2) + a->eps);
        if (a->mode == ORC_ADAMW)
            th = th - a->lr * (u + a->wd * th);
        else
            th = th - a->lr * u;
        m[i] = (float)mi;
        v[i] = (float)vi;
        theta[i] = (float)th;
        if (p_bf16)
            p_bf16[i] = a->param_fp16 ? orc_fp16_rne(theta[i]) : orc_bf16_rne(theta[i]);
    }
}
