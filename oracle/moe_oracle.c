/*
 * moe_oracle.c -- plain, slow, obviously correct CPU oracle for MoE token
 * dispatch layout, dispatch (bf16 and e4m3) and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the
 * HIP library; it is compiled by gcc (not hipcc) with -O2 -ffp-contract=off so
 * that every floating-point operation happens exactly as written below.
 *
 * What it computes, and where the pages define it:
 *
 *  - Combine (the "计算公式" formula and the expert_scales / shared_expert_x
 *    parameter notes of the torch_npu npu_moe_distribute_combine API page):
 *    each output row is the sum over the token's K experts of
 *    expert_scales[t,k] times that expert's output row, plus the shared-expert
 *    row added without a weight.  With one device the page's ReduceScatterV and
 *    AlltoAllv steps are identities, so only the local weighted sum remains.
 *  - Layout (same page, parameters expert_ids, expand_idx, ep_send_counts):
 *    per-expert token counts kept in prefix-sum form and a per-(token, k)
 *    index.  The per-expert segment is rounded up to the 128-row M-tile of the
 *    grouped GEMM that consumes it (TEMPO summary, section 1, "padded
 *    compute"; section 2, tile-aware cost model).
 *  - Dispatch: the mirror of combine ("returns along the path the dispatch op
 *    collected the data on", function description of the same page): token
 *    row t is copied to row slot(t,k) = ep_send_counts[e] + expand_idx[t*K+k]
 *    of the expert-contiguous buffer, for e = expert_ids[t,k].
 *  - FP8 dispatch: the page's comm_quant_mode parameter names a quantised
 *    transfer but its dtype is unreadable; the reading adopted is OCP e4m3fn
 *    with one fp32 scale amax/448 per (token, 128-channel block).
 *  - FP8 combine: the same quantised transfer on the return path; expert
 *    output rows in that e4m3 + scale format are dequantised term by term.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - expand_idx[t*K+k] is the number of earlier pairs (t',k') < (t,k), in
 *    row-major order, routed to the same expert: the stable within-expert rank.
 *  - ep_send_counts has E+1 entries: the exclusive prefix of the padded counts,
 *    the last entry being the padded total.
 *  - Combine accumulates in fp32 with a fused multiply-add chain starting from
 *    +0 in ascending k, then adds the shared row once, then rounds to bf16 with
 *    round-to-nearest-even.
 *  - Padding rows are never written.
 *
 * Every function below is checked by the not-gpu tests against brute force,
 * closed forms, invariants and library conversions (torch's bf16 and
 * float8_e4m3fn casts).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* Status codes and device-flag bits; the numbers are part of the documented
 * C interface (same meaning as the library's), restated here on purpose. */
#define ORC_OK 0
#define ORC_ERR_INVALID_ARG 1
#define ORC_ERR_UNSUPPORTED 3

#define ORC_FLAG_ID_RANGE 1
#define ORC_FLAG_DUP_ID 2
#define ORC_FLAG_GUARD 4

#define ORC_DTYPE_BF16 0
#define ORC_DTYPE_FP8_E4M3 1

/* ------------------------------------------------------------------------ */
/* Number formats, written from their definitions.                          */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* bfloat16 is the upper half of an IEEE binary32: widening appends 16 zero
 * mantissa bits. */
float oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* Narrowing binary32 -> bfloat16, round to nearest, ties to even.  The
 * discarded low 16 bits are compared against one half of the kept unit in the
 * last place; IEEE's sign-magnitude encoding makes "round the magnitude up" an
 * increment of the kept bits (a carry into the exponent, or to infinity, is
 * the correct result).  NaN stays NaN (quiet bit forced). */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u = f32_bits(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits.  Exponent field 0 holds subnormals m/8 * 2^-6; exponent 15 with
 * mantissa 7 is NaN (both signs); there is no infinity; the largest finite
 * magnitude is 1.75 * 2^8 = 448. */
float oracle_e4m3_to_f32(uint8_t c) {
    int sign = (c >> 7) & 1;
    int exp = (c >> 3) & 0xF;
    int man = c & 0x7;
    double mag;
    if (exp == 0xF && man == 0x7) return sign ? -NAN : NAN;
    if (exp == 0)
        mag = ldexp((double)man / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)man / 8.0, exp - 7);
    return (float)(sign ? -mag : mag);
}

/* Round a non-negative double to the nearest integer, ties to even. */
static double round_half_even(double q) {
    double fl = floor(q);
    double frac = q - fl;
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* binary32 -> e4m3fn, round to nearest even, saturating: magnitudes above 448
 * become 448 (the format has no infinity), NaN becomes the NaN code.  A value
 * that rounds to zero keeps its sign. */
uint8_t oracle_f32_to_e4m3(float f) {
    if (isnan(f)) return 0x7F;
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a = fabs((double)f);
    if (a > 448.0) a = 448.0;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: spacing 2^-9, n = 8 is the smallest normal */
        double n = round_half_even(a / ldexp(1.0, -9));
        if (n >= 8.0) return (uint8_t)(sign | 0x08);
        return (uint8_t)(sign | (uint8_t)n);
    }
    int e2;
    (void)frexp(a, &e2);        /* a = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;             /* a in [2^e, 2^(e+1)), e in [-6, 8] */
    double n = round_half_even(a / ldexp(1.0, e - 3)); /* 8 <= n <= 16 */
    if (n >= 16.0) {
        e += 1;
        n = 8.0;
    }
    /* a <= 448 keeps (e, n) at or below (8, 14): never the NaN code. */
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)((int)n - 8));
}

/* ------------------------------------------------------------------------ */
/* Argument rules (the pages' shape and range rules, plus the library's own). */
/* ------------------------------------------------------------------------ */

/* Segment capacity that always holds the padded layout:
 * sum_e ceil(c_e/a)*a <= a*floor((n + (a-1)*min(E, n)) / a) with n = bs*k. */
int64_t oracle_capacity(int32_t bs, int32_t k, int32_t num_experts, int32_t align) {
    int64_t n = (int64_t)bs * (int64_t)k;
    int64_t used = n < num_experts ? n : num_experts;
    return (int64_t)align * ((n + (int64_t)(align - 1) * used) / align);
}

static int is_pow2(int32_t v) { return v > 0 && (v & (v - 1)) == 0; }

/* Layout arguments: 0 <= bs; 1 <= num_experts <= 512 and 0 < k <= num_experts
 * (npu_moe_distribute_combine parameter and constraint notes); the library
 * further caps k at 16 (the widest top-K limit on that page) and requires the
 * alignment to be a power of two in [1, 1024]; bs*k and the padded total must
 * not exceed 2^30. */
int oracle_check_layout_args(int32_t bs, int32_t k, int32_t num_experts, int32_t align) {
    if (bs < 0) return ORC_ERR_INVALID_ARG;
    if (num_experts < 1 || num_experts > 512) return ORC_ERR_INVALID_ARG;
    if (k < 1 || k > 16 || k > num_experts) return ORC_ERR_INVALID_ARG;
    if (!is_pow2(align) || align > 1024) return ORC_ERR_INVALID_ARG;
    if (oracle_capacity(bs, k, num_experts, align) > (1LL << 30)) return ORC_ERR_INVALID_ARG;
    return ORC_OK;
}

/* Row arguments: 0 < hidden, hidden a multiple of 32 (the page's rule for H);
 * e4m3 output additionally needs hidden a multiple of 128 (whole scale
 * blocks).  Row strides are at least hidden. */
int oracle_check_row_args(int32_t hidden, int32_t dtype) {
    if (hidden <= 0 || hidden % 32 != 0 || hidden > 65536) return ORC_ERR_INVALID_ARG;
    if (dtype != ORC_DTYPE_BF16 && dtype != ORC_DTYPE_FP8_E4M3) return ORC_ERR_UNSUPPORTED;
    if (dtype == ORC_DTYPE_FP8_E4M3 && hidden % 128 != 0) return ORC_ERR_INVALID_ARG;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Layout: counts, padded prefix, stable ranks.                              */
/* ------------------------------------------------------------------------ */

/* expert_counts[e]  = number of valid pairs routed to e
 * ep_send_counts[e] = sum over e' < e of ceil(count[e']/align)*align, e in [0, E]
 * expand_idx[t*K+k] = number of earlier valid pairs routed to the same expert,
 *                     or -1 when expert_ids[t,k] lies outside [0, E)
 * flags            |= ORC_FLAG_ID_RANGE for any id outside [0, E),
 *                     ORC_FLAG_DUP_ID when an id repeats within a row. */
int oracle_layout(const int32_t* expert_ids, int32_t bs, int32_t k, int32_t num_experts,
                  int32_t align, int32_t* expert_counts, int32_t* ep_send_counts,
                  int32_t* expand_idx, int32_t* flags) {
    int rc = oracle_check_layout_args(bs, k, num_experts, align);
    if (rc != ORC_OK) return rc;
    int32_t f = 0;

    /* counts */
    for (int32_t e = 0; e < num_experts; ++e) expert_counts[e] = 0;
    for (int32_t t = 0; t < bs; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = expert_ids[(int64_t)t * k + j];
            if (e >= 0 && e < num_experts) expert_counts[e] += 1;
        }

    /* padded exclusive prefix */
    ep_send_counts[0] = 0;
    for (int32_t e = 0; e < num_experts; ++e) {
        int32_t padded = ((expert_counts[e] + align - 1) / align) * align;
        ep_send_counts[e + 1] = ep_send_counts[e] + padded;
    }

    /* stable ranks: visit pairs in row-major (t, k) order */
    int32_t next[512];
    for (int32_t e = 0; e < num_experts; ++e) next[e] = 0;
    for (int32_t t = 0; t < bs; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int64_t i = (int64_t)t * k + j;
            int32_t e = expert_ids[i];
            if (e < 0 || e >= num_experts) {
                expand_idx[i] = -1;
                f |= ORC_FLAG_ID_RANGE;
                continue;
            }
            expand_idx[i] = next[e];
            next[e] += 1;
            for (int32_t j2 = 0; j2 < j; ++j2)
                if (expert_ids[(int64_t)t * k + j2] == e) f |= ORC_FLAG_DUP_ID;
        }

    if (flags) *flags = f;
    return ORC_OK;
}

/* Destination row of pair (t, j), or -1 when the pair is skipped.  A slot
 * outside [0, capacity_rows) is a guard hit: skipped and flagged. */
static int64_t pair_slot(const int32_t* expert_ids, const int32_t* expand_idx,
                         const int32_t* ep_send_counts, int32_t k, int32_t num_experts,
                         int64_t capacity_rows, int32_t t, int32_t j, int32_t* f) {
    int64_t i = (int64_t)t * k + j;
    int32_t e = expert_ids[i];
    int32_t r = expand_idx[i];
    if (e < 0 || e >= num_experts || r < 0) return -1;
    int64_t slot = (int64_t)ep_send_counts[e] + r;
    if (slot < 0 || slot >= capacity_rows) {
        *f |= ORC_FLAG_GUARD;
        return -1;
    }
    return slot;
}

/* ------------------------------------------------------------------------ */
/* Dispatch.                                                                 */
/* ------------------------------------------------------------------------ */

/* bf16: expand_x[slot(t,k), :] = x[t, :], a bit copy.  Padding rows and rows
 * of skipped pairs are left untouched. */
int oracle_dispatch_bf16(const uint16_t* x, int64_t x_stride, int32_t bs, int32_t hidden,
                         const int32_t* expert_ids, const int32_t* expand_idx,
                         const int32_t* ep_send_counts, int32_t k, int32_t num_experts,
                         uint16_t* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                         int32_t* flags) {
    int rc = oracle_check_layout_args(bs, k, num_experts, 1);
    if (rc == ORC_OK) rc = oracle_check_row_args(hidden, ORC_DTYPE_BF16);
    if (rc != ORC_OK) return rc;
    int32_t f = 0;
    for (int32_t t = 0; t < bs; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int64_t slot = pair_slot(expert_ids, expand_idx, ep_send_counts, k, num_experts,
                                     capacity_rows, t, j, &f);
            if (slot < 0) continue;
            for (int32_t h = 0; h < hidden; ++h)
                expand_x[slot * expand_x_stride + h] = x[(int64_t)t * x_stride + h];
        }
    if (flags) *flags |= f;
    return ORC_OK;
}

/* Quantise one token row: for each block of 128 channels,
 *   amax = max |x|,  s = amax / 448 (binary32 division),
 *   q    = e4m3(x / s) (binary32 division, then round-to-nearest-even with
 *          saturation); an all-zero block has s = 0 and every code 0x00.
 * Dequantisation is e4m3_to_f32(q) * s. */
void oracle_quantize_row_e4m3(const uint16_t* x_row, int32_t hidden, uint8_t* q_row,
                              float* scale_row) {
    for (int32_t b = 0; b < hidden / 128; ++b) {
        float amax = 0.0f;
        for (int32_t h = 0; h < 128; ++h) {
            float v = fabsf(oracle_bf16_to_f32(x_row[b * 128 + h]));
            if (v > amax) amax = v;
        }
        float s = amax / 448.0f;
        scale_row[b] = s;
        for (int32_t h = 0; h < 128; ++h) {
            if (amax == 0.0f) {
                q_row[b * 128 + h] = 0x00;
            } else {
                float v = oracle_bf16_to_f32(x_row[b * 128 + h]) / s;
                q_row[b * 128 + h] = oracle_f32_to_e4m3(v);
            }
        }
    }
}

/* e4m3: each of the token's K slots receives the same code row and the same
 * scale row (quant_scales is [capacity_rows, hidden/128] row-major). */
int oracle_dispatch_fp8(const uint16_t* x, int64_t x_stride, int32_t bs, int32_t hidden,
                        const int32_t* expert_ids, const int32_t* expand_idx,
                        const int32_t* ep_send_counts, int32_t k, int32_t num_experts,
                        uint8_t* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                        float* quant_scales, int32_t* flags, uint8_t* q_tmp, float* s_tmp) {
    int rc = oracle_check_layout_args(bs, k, num_experts, 1);
    if (rc == ORC_OK) rc = oracle_check_row_args(hidden, ORC_DTYPE_FP8_E4M3);
    if (rc != ORC_OK) return rc;
    int32_t f = 0;
    int32_t nb = hidden / 128;
    for (int32_t t = 0; t < bs; ++t) {
        oracle_quantize_row_e4m3(x + (int64_t)t * x_stride, hidden, q_tmp, s_tmp);
        for (int32_t j = 0; j < k; ++j) {
            int64_t slot = pair_slot(expert_ids, expand_idx, ep_send_counts, k, num_experts,
                                     capacity_rows, t, j, &f);
            if (slot < 0) continue;
            for (int32_t h = 0; h < hidden; ++h) expand_x[slot * expand_x_stride + h] = q_tmp[h];
            for (int32_t b = 0; b < nb; ++b) quant_scales[slot * nb + b] = s_tmp[b];
        }
    }
    if (flags) *flags |= f;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Combine.                                                                  */
/* ------------------------------------------------------------------------ */

/* x_out[t,h] = bf16( fma-chain over k ascending of expert_scales[t,k] *
 *                    y[slot(t,k), h], started from +0, then + shared[t,h] ).
 * Skipped pairs contribute nothing; shared == NULL means no shared row. */
int oracle_combine(const uint16_t* y, int64_t y_stride, int64_t capacity_rows,
                   const int32_t* expert_ids, const int32_t* expand_idx,
                   const int32_t* ep_send_counts, const float* expert_scales,
                   const uint16_t* shared, int64_t shared_stride, int32_t bs, int32_t hidden,
                   int32_t k, int32_t num_experts, uint16_t* x_out, int32_t* flags) {
    int rc = oracle_check_layout_args(bs, k, num_experts, 1);
    if (rc == ORC_OK) rc = oracle_check_row_args(hidden, ORC_DTYPE_BF16);
    if (rc != ORC_OK) return rc;
    int32_t f = 0;
    int64_t slots[16];
    for (int32_t t = 0; t < bs; ++t) {
        for (int32_t j = 0; j < k; ++j)
            slots[j] = pair_slot(expert_ids, expand_idx, ep_send_counts, k, num_experts,
                                 capacity_rows, t, j, &f);
        for (int32_t h = 0; h < hidden; ++h) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
                if (slots[j] < 0) continue;
                float w = expert_scales[(int64_t)t * k + j];
                float v = oracle_bf16_to_f32(y[slots[j] * y_stride + h]);
                acc = fmaf(w, v, acc);
            }
            if (shared) acc = acc + oracle_bf16_to_f32(shared[(int64_t)t * shared_stride + h]);
            x_out[(int64_t)t * hidden + h] = oracle_f32_to_bf16(acc);
        }
    }
    if (flags) *flags |= f;
    return ORC_OK;
}

/* Quantised-transfer combine (the combine page's comm_quant_mode on the return
 * path; the dtype is unreadable there, read as the same e4m3 + per-128-channel
 * fp32 scale format the dispatch emits): expert output rows arrive as codes
 * y[slot, :] with scales y_scales[slot, h/128] ([capacity_rows, hidden/128]
 * row-major).  Each term is dequantised with one binary32 multiply,
 *   deq = e4m3_to_f32(code) * scale,
 * then summed exactly like the bf16 combine: fma chain over k ascending from
 * +0, + shared, round to nearest even into bf16. */
int oracle_combine_fp8(const uint8_t* y, int64_t y_stride, int64_t capacity_rows,
                       const float* y_scales, const int32_t* expert_ids,
                       const int32_t* expand_idx, const int32_t* ep_send_counts,
                       const float* expert_scales, const uint16_t* shared,
                       int64_t shared_stride, int32_t bs, int32_t hidden, int32_t k,
                       int32_t num_experts, uint16_t* x_out, int32_t* flags) {
    int rc = oracle_check_layout_args(bs, k, num_experts, 1);
    if (rc == ORC_OK) rc = oracle_check_row_args(hidden, ORC_DTYPE_FP8_E4M3);
    if (rc != ORC_OK) return rc;
    int32_t f = 0;
    int32_t nb = hidden / 128;
    int64_t slots[16];
    for (int32_t t = 0; t < bs; ++t) {
        for (int32_t j = 0; j < k; ++j)
            slots[j] = pair_slot(expert_ids, expand_idx, ep_send_counts, k, num_experts,
                                 capacity_rows, t, j, &f);
        for (int32_t h = 0; h < hidden; ++h) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
                if (slots[j] < 0) continue;
                float w = expert_scales[(int64_t)t * k + j];
                float code = oracle_e4m3_to_f32(y[slots[j] * y_stride + h]);
                float deq = code * y_scales[slots[j] * nb + h / 128];
                acc = fmaf(w, deq, acc);
            }
            if (shared) acc = acc + oracle_bf16_to_f32(shared[(int64_t)t * shared_stride + h]);
            x_out[(int64_t)t * hidden + h] = oracle_f32_to_bf16(acc);
        }
    }
    if (flags) *flags |= f;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Rank-partitioned layout (combine page, ep_send_counts for the A3 series:  */
/* ep_world_size * local_expert_num entries; moe_expert_num divisible by the  */
/* number of expert ranks).                                                   */
/* ------------------------------------------------------------------------ */

/* Expert e lives on rank e / L with L = E / ep_world_size experts per rank,
 * so the expert-contiguous layout is already rank-major.  The rows bound for
 * rank r are [rank_offsets[r], rank_offsets[r+1]) with
 * rank_offsets[r] = ep_send_counts[r*L] (and rank_offsets[ws] = the total):
 * the per-destination send offsets of an all-to-all(v).  E must be a
 * multiple of ep_world_size. */
int oracle_layout_ep(const int32_t* expert_ids, int32_t bs, int32_t k, int32_t num_experts,
                     int32_t ep_world_size, int32_t align, int32_t* expert_counts,
                     int32_t* ep_send_counts, int32_t* rank_offsets, int32_t* expand_idx,
                     int32_t* flags) {
    if (ep_world_size < 1 || ep_world_size > num_experts || num_experts % ep_world_size != 0)
        return ORC_ERR_INVALID_ARG;
    int rc = oracle_layout(expert_ids, bs, k, num_experts, align, expert_counts,
                           ep_send_counts, expand_idx, flags);
    if (rc != ORC_OK) return rc;
    int32_t per_rank = num_experts / ep_world_size;
    for (int32_t r = 0; r <= ep_world_size; ++r) rank_offsets[r] = ep_send_counts[r * per_rank];
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Replica-aware dispatch (TEMPO summary, section 2, system integration: one  */
/* in-graph kernel does the probabilistic replica choice and the counting).  */
/* ------------------------------------------------------------------------ */

/* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): the generator's state advances by the golden
 * gamma 0x9E3779B97F4A7C15 per draw and each state is finalised by the
 * variant-13 mixer.  Draw i (0-based) of the stream seeded with `seed` is the
 * finalised state seed + (i+1)*gamma, so any draw can be computed directly
 * from its counter. */
uint64_t oracle_splitmix64(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

#define ORC_FLAG_REPLICA 8

/* Each valid pair (t, j) with logical expert e draws u = the upper 32 bits of
 * draw t*K+j of the SplitMix64 stream, and goes to the first replica r of e
 * (r in [replica_offsets[e], replica_offsets[e+1])) whose cumulative
 * threshold satisfies u <= replica_thresholds[r].  A logical id outside
 * [0, E), or an expert whose thresholds never reach u (an empty or malformed
 * range), gives -1 (the latter also ORC_FLAG_REPLICA).  Then the ordinary
 * layout runs over the num_replicas physical replicas. */
int oracle_layout_replicated(const int32_t* expert_ids, int32_t bs, int32_t k,
                             int32_t num_experts, const int32_t* replica_offsets,
                             const uint32_t* replica_thresholds, int32_t num_replicas,
                             uint64_t seed, int32_t align, int32_t* replica_ids,
                             int32_t* replica_counts, int32_t* ep_send_counts,
                             int32_t* expand_idx, int32_t* flags) {
    int rc = oracle_check_layout_args(bs, k, num_experts, align);
    if (rc == ORC_OK) rc = oracle_check_layout_args(bs, k, num_replicas, align);
    if (rc != ORC_OK) return rc;
    int32_t f = 0;
    for (int32_t t = 0; t < bs; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int64_t i = (int64_t)t * k + j;
            int32_t e = expert_ids[i];
            replica_ids[i] = -1;
            if (e < 0 || e >= num_experts) {
                f |= ORC_FLAG_ID_RANGE;
                continue;
            }
            for (int32_t j2 = 0; j2 < j; ++j2)
                if (expert_ids[(int64_t)t * k + j2] == e) f |= ORC_FLAG_DUP_ID;
            uint32_t u = (uint32_t)(oracle_splitmix64(seed, (uint64_t)i) >> 32);
            int32_t lo = replica_offsets[e], hi = replica_offsets[e + 1];
            int32_t chosen = -1;
            for (int32_t r = lo; r < hi; ++r)
                if (r >= 0 && r < num_replicas && u <= replica_thresholds[r]) {
                    chosen = r;
                    break;
                }
            if (chosen < 0) f |= ORC_FLAG_REPLICA;
            replica_ids[i] = chosen;
        }
    int32_t f2 = 0;
    rc = oracle_layout(replica_ids, bs, k, num_replicas, align, replica_counts, ep_send_counts,
                       expand_idx, &f2);
    if (rc != ORC_OK) return rc;
    /* -1 replica ids were already accounted for above; repeated replicas in a
     * row can only come from repeated logical experts */
    if (flags) *flags = f;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the codecs, so the tests can sweep whole code spaces.      */
/* ------------------------------------------------------------------------ */

void oracle_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]);
}

void oracle_f32_to_e4m3_array(const float* in, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e4m3(in[i]);
}

void oracle_e4m3_to_f32_array(const uint8_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_f32(in[i]);
}
