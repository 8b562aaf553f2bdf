/*
 * oracle.c -- plain, slow CPU definition of one rank's share of a
 * small-message bf16 allreduce with fp32 accumulation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP library; each side implements the definitions below on its own.
 *
 * What is computed, and where it comes from:
 *
 *  - The reduction: every output element is the sum of the P peer inputs at
 *    that index.  For an allreduce every rank is owed the whole buffer and
 *    keeps the whole result (torchcomms PR #3850 "Add HIP-graph capture
 *    coverage for the sharded-relay collectives", commit summary
 *    D117629707: allreduce as the srcStride == 0 case of the one-shot
 *    push-reduce kernel).  Helion PR #245 "One shot all reduce Example"
 *    computes the same one-shot sum.
 *  - Precision and order: each bf16 input is widened exactly to binary32,
 *    the P values are added in rank order 0..P-1 starting from rank 0's value
 *    (IEEE binary32 addition, round to nearest even, subnormals kept, no
 *    contraction), and the binary32 sum is rounded to bf16 with round to
 *    nearest, ties to even.  Every NaN becomes the canonical quiet NaN 0x7FC0.
 *  - Write mode: stage 2 stores the reduced data straight into every peer's
 *    output, whose pointers are handed to the kernel (aiter PR #1910
 *    "optimize allreduce write mode by broadcast output ptr", Motivation and
 *    Technical Details).  Here: P identical output buffers.
 *  - Two-shot share: the slice a rank owns is floored to a multiple of 128
 *    elements and the last slice absorbs the remainder, so every slice
 *    boundary is 128-element aligned (torchcomms PR #3850, commit summary
 *    D117629683: directA aligned down, directB absorbs the remainder).
 *  - LL packets: data and flag travel together, so arrival is read off the
 *    data itself (ARK PR #254 "Add monolithic fused packet allreduce kernel
 *    and Model::all_reduce_packet API", description).  A packet is 16 bytes,
 *    four little-endian u32 words {data0, flag, data1, flag}; data0 holds
 *    elements 4k (low half) and 4k+1 (high half), data1 holds 4k+2 and 4k+3;
 *    elements past n are encoded as 0x0000.
 *  - Fused packet allreduce: scatter, reduce and broadcast in one pass,
 *    synchronised only by the packet flags (ARK PR #254, description).  The
 *    flag of call c is c+1; scratch is zeroed once and never cleared, so a
 *    stale packet reads as not yet arrived (torchcomms PR #3850, commit
 *    summary D117629704: the epoch advances per launch and flags are never
 *    cleared; ARK PR #254, Known limitations: per-call flag rotation).
 *
 * Build: gcc -O1 -std=c11 -ffp-contract=off, never -ffast-math.
 * Each exported function checks that the x86 MXCSR is in its IEEE default
 * state (round to nearest, no flush-to-zero, no denormals-are-zero) and
 * returns ORC_EFPENV otherwise.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_EFLAG (-2)   /* a packet's flag words do not equal the expected flag */
#define ORC_ENOMEM (-3)
#define ORC_EFPENV (-5)  /* host floating-point environment is not IEEE default */

/* ---- floating-point environment guard ---------------------------------- */

static int fp_env_ok(void)
{
    unsigned int csr = _mm_getcsr();
    /* bit 15 FTZ, bit 6 DAZ, bits 13-14 rounding control (00 = nearest). */
    return (csr & 0x8000u) == 0 && (csr & 0x0040u) == 0 && (csr & 0x6000u) == 0;
}

/* ---- scalar definitions ------------------------------------------------- */

/* bf16 bit pattern -> binary32 value: the bf16 bits are the upper half of the
 * binary32 bits, so this is exact for every input, NaN and Inf included. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* binary32 -> bf16, round to nearest, ties to even. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    if ((bits & 0x7F800000u) == 0x7F800000u && (bits & 0x007FFFFFu) != 0)
        return 0x7FC0; /* NaN -> canonical quiet NaN */
    uint32_t kept = bits >> 16;          /* sign, exponent, top 7 mantissa bits */
    uint32_t dropped = bits & 0xFFFFu;   /* the 16 bits rounded away */
    int round_up = dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u));
    /* A carry out of the mantissa bumps the exponent, which is the correct
     * next representable value (up to and including +-Inf). */
    return (uint16_t)(kept + (round_up ? 1u : 0u));
}

/* Sum of element i over the P inputs, binary32, rank order 0..P-1. */
static float sum_in_rank_order(const uint16_t *const *x, int P, int64_t i)
{
    float acc = bf16_to_f32(x[0][i]);
    for (int r = 1; r < P; ++r)
        acc = acc + bf16_to_f32(x[r][i]);
    return acc;
}

/* ---- one-shot, write mode ----------------------------------------------- */

int orc_oneshot_sum(const uint16_t *const *x, int P, int64_t n, uint16_t *y)
{
    if (!fp_env_ok()) return ORC_EFPENV;
    if (P < 1 || n < 0 || !x || (n > 0 && !y)) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        y[i] = f32_to_bf16_rne(sum_in_rank_order(x, P, i));
    return ORC_OK;
}

int orc_write_bcast(const uint16_t *const *x, int P, int64_t n, uint16_t *const *out)
{
    if (!fp_env_ok()) return ORC_EFPENV;
    if (P < 1 || n < 0 || !x || !out) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        uint16_t v = f32_to_bf16_rne(sum_in_rank_order(x, P, i));
        for (int j = 0; j < P; ++j)
            out[j][i] = v;
    }
    return ORC_OK;
}

/* ---- two-shot slice ----------------------------------------------------- */

int orc_slice(int P, int64_t n, int r, int64_t *begin, int64_t *end)
{
    if (P < 1 || n < 0 || r < 0 || r >= P || !begin || !end) return ORC_EINVAL;
    int64_t L = (n / (128 * (int64_t)P)) * 128; /* floored to a 128 multiple */
    *begin = (int64_t)r * L;
    *end = (r == P - 1) ? n : (int64_t)(r + 1) * L;
    return ORC_OK;
}

/* Rank r reduces its slice over the P inputs and writes it into all P
 * outputs; every element outside the slice is left as the caller had it. */
int orc_twoshot_share(const uint16_t *const *x, int P, int64_t n, int r, uint16_t *const *out)
{
    if (!fp_env_ok()) return ORC_EFPENV;
    int64_t b, e;
    if (!x || !out || orc_slice(P, n, r, &b, &e) != ORC_OK) return ORC_EINVAL;
    for (int64_t i = b; i < e; ++i) {
        uint16_t v = f32_to_bf16_rne(sum_in_rank_order(x, P, i));
        for (int j = 0; j < P; ++j)
            out[j][i] = v;
    }
    return ORC_OK;
}

/* ---- one-shot reduce-scatter -------------------------------------------- */

/* Each input holds P blocks of rc elements; rank r keeps the rank-order sum of
 * block r: the reduce-scatter case of the one-shot push-reduce kernel, with a
 * per-peer source stride of rc and an owner offset of r * rc (torchcomms PR
 * #3850, commit summary D117629707). */
int orc_reduce_scatter(const uint16_t *const *x, int P, int64_t rc, int r, uint16_t *y)
{
    if (!fp_env_ok()) return ORC_EFPENV;
    if (P < 1 || rc < 0 || r < 0 || r >= P || !x || (rc > 0 && !y)) return ORC_EINVAL;
    for (int64_t i = 0; i < rc; ++i)
        y[i] = f32_to_bf16_rne(sum_in_rank_order(x, P, (int64_t)r * rc + i));
    return ORC_OK;
}

/* ---- LL packets --------------------------------------------------------- */

int64_t orc_ll_packets(int64_t n)
{
    return n <= 0 ? 0 : (n + 3) / 4;
}

/* Packet k = words 4k..4k+3 of pk (u32, little-endian). */
int orc_ll_encode(const uint16_t *y, int64_t n, uint32_t flag, uint32_t *pk)
{
    if (n < 0 || (n > 0 && (!y || !pk))) return ORC_EINVAL;
    for (int64_t k = 0; k < orc_ll_packets(n); ++k) {
        uint32_t e[4];
        for (int t = 0; t < 4; ++t) {
            int64_t i = 4 * k + t;
            e[t] = i < n ? y[i] : 0u;
        }
        pk[4 * k + 0] = e[0] | (e[1] << 16);
        pk[4 * k + 1] = flag;
        pk[4 * k + 2] = e[2] | (e[3] << 16);
        pk[4 * k + 3] = flag;
    }
    return ORC_OK;
}

/* Inverse of orc_ll_encode.  Every packet must carry `flag` in both flag
 * words; otherwise returns ORC_EFLAG (y is then partially written). */
int orc_ll_decode(const uint32_t *pk, int64_t n, uint32_t flag, uint16_t *y)
{
    if (n < 0 || (n > 0 && (!y || !pk))) return ORC_EINVAL;
    for (int64_t k = 0; k < orc_ll_packets(n); ++k) {
        if (pk[4 * k + 1] != flag || pk[4 * k + 3] != flag) return ORC_EFLAG;
        uint32_t d[2] = {pk[4 * k + 0], pk[4 * k + 2]};
        for (int t = 0; t < 4; ++t) {
            int64_t i = 4 * k + t;
            if (i < n)
                y[i] = (uint16_t)(d[t / 2] >> (16 * (t % 2)));
        }
    }
    return ORC_OK;
}

/* ---- fused packet allreduce --------------------------------------------- */

/* Packets per slot: each slot is sized for the largest slice, the last one. */
int64_t orc_packet_slot_packets(int P, int64_t n)
{
    int64_t b, e;
    if (orc_slice(P, n, P - 1, &b, &e) != ORC_OK) return ORC_EINVAL;
    return orc_ll_packets(e - b);
}

/* Per-rank scratch: [inbox: P slots][resbox: P slots], 16 B per packet. */
int64_t orc_packet_scratch_bytes(int P, int64_t n)
{
    int64_t S = orc_packet_slot_packets(P, n);
    if (S < 0) return S;
    return 2 * (int64_t)P * S * 16;
}

static uint32_t *inbox_slot(uint8_t *scratch_j, int64_t S, int s)
{
    return (uint32_t *)(scratch_j + (int64_t)s * S * 16);
}

static uint32_t *resbox_slot(uint8_t *scratch_j, int P, int64_t S, int s)
{
    return (uint32_t *)(scratch_j + ((int64_t)P + s) * S * 16);
}

/*
 * One fused call for all P ranks, in the order the phases happen:
 *   scatter:   rank r encodes x_r[slice j] into inbox_j[slot r] for every j
 *              (its own inbox included);
 *   reduce:    rank j decodes inbox_j[slot 0..P-1] and sums in rank order;
 *   broadcast: rank j encodes its reduced slice into resbox_k[slot j] for
 *              every k (its own resbox included);
 *   receive:   rank k decodes resbox_k[slot 0..P-1] into out_k.
 * `scratch[j]` is rank j's scratch image (orc_packet_scratch_bytes bytes); it
 * is updated in place, so a sequence of calls threads it from call to call.
 * Packets past a slice's length keep whatever the image held before.
 */
int orc_packet_fused(const uint16_t *const *x, int P, int64_t n, uint32_t flag,
                     uint8_t *const *scratch, uint16_t *const *out)
{
    if (!fp_env_ok()) return ORC_EFPENV;
    if (P < 1 || n < 0 || !x || !scratch || !out || flag == 0) return ORC_EINVAL;
    int64_t S = orc_packet_slot_packets(P, n);
    int64_t b[8 + 1], e[8 + 1];
    if (P > 8) return ORC_EINVAL;
    for (int j = 0; j < P; ++j)
        orc_slice(P, n, j, &b[j], &e[j]);

    /* scatter */
    for (int r = 0; r < P; ++r)
        for (int j = 0; j < P; ++j)
            orc_ll_encode(x[r] + b[j], e[j] - b[j], flag, inbox_slot(scratch[j], S, r));

    /* reduce + broadcast, one owner j at a time */
    for (int j = 0; j < P; ++j) {
        int64_t len = e[j] - b[j];
        if (len == 0) continue;
        uint16_t *staged[8] = {0};
        uint16_t *part = (uint16_t *)malloc((size_t)len * sizeof(uint16_t));
        int rc = part ? ORC_OK : ORC_ENOMEM;
        for (int s = 0; s < P && rc == ORC_OK; ++s) {
            staged[s] = (uint16_t *)malloc((size_t)len * sizeof(uint16_t));
            rc = staged[s] ? orc_ll_decode(inbox_slot(scratch[j], S, s), len, flag, staged[s])
                           : ORC_ENOMEM;
        }
        if (rc == ORC_OK) {
            for (int64_t i = 0; i < len; ++i)
                part[i] = f32_to_bf16_rne(sum_in_rank_order((const uint16_t *const *)staged, P, i));
            for (int k = 0; k < P; ++k)
                orc_ll_encode(part, len, flag, resbox_slot(scratch[k], P, S, j));
        }
        for (int s = 0; s < P; ++s) free(staged[s]);
        free(part);
        if (rc != ORC_OK) return rc;
    }

    /* receive */
    for (int k = 0; k < P; ++k)
        for (int s = 0; s < P; ++s) {
            int rc = orc_ll_decode(resbox_slot(scratch[k], P, S, s), e[s] - b[s], flag,
                                   out[k] + b[s]);
            if (rc != ORC_OK) return rc;
        }
    return ORC_OK;
}
