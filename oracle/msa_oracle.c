/*
 * msa_oracle.c -- plain CPU oracle for the MiniMax Sparse Attention (MSA)
 * forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this file:
 * only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no code, header, table or constant with the
 * HIP library; it decodes its own inputs from raw storage.
 *
 * Every routine is the plain definition written out, slow and in page order:
 *
 *   block scores   "MiniMax Sparse Attention (MSA)", Deep Dive > Index Branch
 *                  Architecture (score = index query . index key / sqrt(d_idx),
 *                  max-pooled over the causally visible tokens of each block);
 *                  "MiniMax Sparse Attention", sec. 2.2 (block partition
 *                  B = ceil(N / B_k)).
 *   selection      same Deep Dive section (TopK over block scores, the local
 *                  block always kept) and Training Stability Mechanisms
 *                  (the forced local block takes one of the k slots);
 *                  "Flash-MSA" blog, Forward > Proxy attention (the local
 *                  block's score is set to +inf inside the top-k).
 *   attention      "MiniMax Sparse Attention", sec. 2.1 (causal softmax
 *                  attention, GQA: G adjacent query heads share KV head r) and
 *                  sec. 2.2 (attention restricted to the causally visible
 *                  tokens of the selected blocks, using the group's KV head).
 *   combine        "MiniMax Sparse Attention (MSA)", Deep Dive > KV-Outer
 *                  Sparse Attention, step 6 (split-K log-sum-exp merge of the
 *                  per-block partial outputs).
 *   inversion      "Flash-MSA" blog, Backward (B[batch, head, query, slot] ->
 *                  block inverted into B*[batch, head, block] -> queries);
 *                  a stable counting sort, entries ascending in query.
 *
 * Precision: block scores are summed in fp32 in index order, the precision in
 * which the block choice is taken on both sides (bf16 x bf16 products are
 * exact in fp32).  Attention and combine run in fp64.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *   - k counts the local block: selection = {L} + the k-1 best other blocks.
 *   - equal scores rank the smaller block id first.
 *   - output rows list the chosen ids ascending, padded with -1.
 *   - fewer than k-1 earlier blocks: all of them are selected.
 *   - the selection ignores the 1/sqrt(d_idx) factor (a positive constant
 *     preserves the order); reported scores include it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- storage decoders (written from the format definitions) ------------ */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
static float dec_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; exponent 0 is subnormal (m/8 * 2^-6). */
static double dec_e4m3(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

enum { ORC_BF16 = 0, ORC_FP8 = 1 };

static double dec_elem(const void *base, int64_t idx, int dtype, double scale)
{
    if (dtype == ORC_BF16)
        return (double)dec_bf16(((const uint16_t *)base)[idx]) * scale;
    return dec_e4m3(((const uint8_t *)base)[idx]) * scale;
}

/* ---- index branch ------------------------------------------------------- */

/*
 * Block scores M[row][r][b], b in [0, B):
 *   b <  L : max over tokens j of block b of sum_t qidx[row][r][t] * kidx[j][t]
 *            (unscaled fp32 sum; every token of an earlier block is visible)
 *   b == L : +inf  (the local block is forced)
 *   b >  L : -inf  (not causal)
 * with L = pos[row] / B_k.  q_idx_rows holds only the rows asked for.
 */
void oracle_block_scores(int64_t N, int H_kv, int d_idx, int B_k, int64_t n_rows,
                         const int64_t *pos, const uint16_t *q_idx_rows,
                         const uint16_t *k_idx, int64_t B, float *M)
{
    int64_t job;
#pragma omp parallel for schedule(dynamic, 1)
    for (job = 0; job < n_rows * H_kv; job++) {
        int64_t row = job / H_kv;
        int r = (int)(job % H_kv);
        int64_t L = pos[row] / B_k;
        const uint16_t *q = q_idx_rows + (row * H_kv + r) * (int64_t)d_idx;
        float *out = M + (row * H_kv + r) * B;
        int64_t b;
        for (b = 0; b < B; b++) {
            if (b > L) {
                out[b] = -INFINITY;
            } else if (b == L) {
                out[b] = INFINITY;
            } else {
                float best = -INFINITY;
                int64_t j;
                for (j = b * B_k; j < (b + 1) * B_k && j < N; j++) {
                    float acc = 0.0f;
                    int t;
                    for (t = 0; t < d_idx; t++)
                        acc += dec_bf16(q[t]) * dec_bf16(k_idx[j * d_idx + t]);
                    if (acc > best)
                        best = acc;
                }
                out[b] = best;
            }
        }
    }
}

/*
 * TopK with the forced local block.  For each (r, row): pick k-1 blocks among
 * 0..L-1 by repeatedly taking the largest remaining score (first, i.e.
 * smallest, id wins a tie), then add L.  Output block_idx[r][row][0..k) is
 * ascending with -1 padding.  rel_margin[r][row] is the relative gap between
 * the (k-1)-th and k-th best non-local scores, +inf when no choice was made.
 */
void oracle_select(int64_t n_rows, int H_kv, int64_t B, int B_k, int k,
                   const int64_t *pos, const float *M, int32_t *block_idx,
                   double *rel_margin)
{
    int64_t job;
#pragma omp parallel for schedule(dynamic, 4)
    for (job = 0; job < n_rows * H_kv; job++) {
        int64_t row = job / H_kv;
        int r = (int)(job % H_kv);
        int64_t L = pos[row] / B_k;
        const float *m = M + (row * H_kv + r) * B;
        int32_t *out = block_idx + ((int64_t)r * n_rows + row) * k;
        unsigned char *taken = calloc((size_t)(L > 0 ? L : 1), 1);
        int32_t *picked = malloc(sizeof(int32_t) * (size_t)k);
        int npicked = 0, s;
        int64_t b, c;
        while (npicked < k - 1 && npicked < L) {
            int64_t best = -1;
            for (b = 0; b < L; b++)
                if (!taken[b] && (best < 0 || m[b] > m[best]))
                    best = b;
            taken[best] = 1;
            picked[npicked++] = (int32_t)best;
        }
        /* margin */
        if (L >= k && k >= 2) {
            double ck1 = m[picked[k - 2]];
            int64_t nb = -1;
            for (b = 0; b < L; b++)
                if (!taken[b] && (nb < 0 || m[b] > m[nb]))
                    nb = b;
            {
                double ck = m[nb];
                double den = fmax(fmax(fabs(ck1), fabs(ck)), 1e-6);
                rel_margin[(int64_t)r * n_rows + row] = (ck1 - ck) / den;
            }
        } else {
            rel_margin[(int64_t)r * n_rows + row] = INFINITY;
        }
        /* ascending ids: walk the taken flags in order, then the local block */
        s = 0;
        for (c = 0; c < L; c++)
            if (taken[c])
                out[s++] = (int32_t)c;
        out[s++] = (int32_t)L;
        while (s < k)
            out[s++] = -1;
        free(taken);
        free(picked);
    }
}

/* ---- main branch -------------------------------------------------------- */

/*
 * Exact softmax attention of every query head over the causally visible
 * tokens of the row's selected blocks.  Head h uses KV head r = h / G and the
 * selection of its index head m = h / (H_q / H_sel): H_sel index (proxy)
 * heads each choose blocks for the adjacent query heads assigned to them
 * ("Flash-MSA", What's next > Note about scheduler requiring proxy heads >=
 * KV heads: an MSA group is the set of query heads of one proxy head); with
 * H_sel = H_kv the groups are the GQA groups.
 * q_rows [n_rows][H_q][d_h]; K, V [N][H_kv][d_h] (bf16 or fp8 codes times the
 * per-tensor scale); block_idx [H_sel][n_rows][k] (-1 = empty slot).
 * Output O [n_rows][H_q][d_h] and natural-log LSE [n_rows][H_q] in fp64.
 */
void oracle_attention(int64_t N, int H_q, int H_kv, int H_sel, int d_h, int B_k, int k,
                      int64_t n_rows, const int64_t *pos, const void *q_rows,
                      const void *K, const void *V, int dtype, double q_scale,
                      double k_scale, double v_scale, const int32_t *block_idx,
                      double softmax_scale, double *O, double *lse)
{
    int G = H_q / H_kv, Gs = H_q / H_sel;
    int64_t job;
#pragma omp parallel for schedule(dynamic, 1)
    for (job = 0; job < n_rows * H_q; job++) {
        int64_t row = job / H_q;
        int h = (int)(job % H_q);
        int r = h / G, m = h / Gs;
        int64_t i = pos[row];
        const int32_t *sel = block_idx + ((int64_t)m * n_rows + row) * k;
        int64_t cap = (int64_t)k * B_k, nt = 0, j, t;
        int64_t *tok = malloc(sizeof(int64_t) * (size_t)cap);
        double *sc = malloc(sizeof(double) * (size_t)cap);
        double *q = malloc(sizeof(double) * (size_t)d_h);
        double mx = -INFINITY, l = 0.0;
        int s, d;
        for (d = 0; d < d_h; d++)
            q[d] = dec_elem(q_rows, (row * H_q + h) * (int64_t)d_h + d, dtype, q_scale);
        /* T = union of selected blocks, intersected with [0, i] */
        for (s = 0; s < k; s++) {
            int64_t b = sel[s];
            if (b < 0)
                continue;
            for (j = b * B_k; j < (b + 1) * B_k && j < N && j <= i; j++)
                tok[nt++] = j;
        }
        for (t = 0; t < nt; t++) {
            double acc = 0.0;
            for (d = 0; d < d_h; d++)
                acc += q[d] * dec_elem(K, (tok[t] * H_kv + r) * (int64_t)d_h + d, dtype, k_scale);
            sc[t] = softmax_scale * acc;
            if (sc[t] > mx)
                mx = sc[t];
        }
        for (t = 0; t < nt; t++) {
            sc[t] = exp(sc[t] - mx);
            l += sc[t];
        }
        for (d = 0; d < d_h; d++) {
            double acc = 0.0;
            for (t = 0; t < nt; t++)
                acc += sc[t] * dec_elem(V, (tok[t] * H_kv + r) * (int64_t)d_h + d, dtype, v_scale);
            O[(row * H_q + h) * (int64_t)d_h + d] = acc / l;
        }
        lse[row * H_q + h] = mx + log(l);
        free(tok);
        free(sc);
        free(q);
    }
}

/*
 * Split-K log-sum-exp merge of per-slot partials.  For each row and head:
 *   LSE = ln sum_{valid s} exp(lse_s),  O = sum_{valid s} exp(lse_s - LSE) * Obar_s
 * o_part [H_kv][n_rows][k][G][d_h] (bf16), lse_part [H_kv][n_rows][k][G]
 * (fp32), a slot is valid when block_idx [H_kv][n_rows][k] >= 0.
 */
void oracle_combine(int H_kv, int G, int d_h, int k, int64_t n_rows,
                    const int32_t *block_idx, const uint16_t *o_part,
                    const float *lse_part, double *O, double *lse)
{
    int H_q = H_kv * G;
    int64_t job;
#pragma omp parallel for schedule(static)
    for (job = 0; job < n_rows * H_q; job++) {
        int64_t row = job / H_q;
        int h = (int)(job % H_q), r = h / G, g = h % G, s, d;
        const int32_t *sel = block_idx + ((int64_t)r * n_rows + row) * k;
        double mx = -INFINITY, sum = 0.0, LSE;
        for (s = 0; s < k; s++) {
            if (sel[s] < 0)
                continue;
            {
                double v = lse_part[(((int64_t)r * n_rows + row) * k + s) * G + g];
                if (v > mx)
                    mx = v;
            }
        }
        for (s = 0; s < k; s++)
            if (sel[s] >= 0)
                sum += exp((double)lse_part[(((int64_t)r * n_rows + row) * k + s) * G + g] - mx);
        LSE = mx + log(sum);
        lse[row * H_q + h] = LSE;
        for (d = 0; d < d_h; d++) {
            double acc = 0.0;
            for (s = 0; s < k; s++) {
                int64_t base;
                if (sel[s] < 0)
                    continue;
                base = ((((int64_t)r * n_rows + row) * k + s) * G + g) * d_h;
                acc += exp((double)lse_part[(((int64_t)r * n_rows + row) * k + s) * G + g] - LSE) *
                       (double)dec_bf16(o_part[base + d]);
            }
            O[(row * H_q + h) * (int64_t)d_h + d] = acc;
        }
    }
}

/*
 * Inverted index.  block_idx [n_seq][n_rows][k] (n_seq = batch * H_kv
 * independent (sequence, group) lists, block ids < B or -1) becomes a CSR
 * over bins (seq, block): offsets [n_seq][B + 1] are absolute positions in
 * entries; entries hold row * k + slot, ascending in row within a bin.
 * A stable counting sort: count, exclusive prefix, then place in row order.
 */
void oracle_invert(int64_t n_seq, int64_t n_rows, int k, int64_t B,
                   const int32_t *block_idx, int32_t *offsets, int32_t *entries)
{
    int64_t *cursor = calloc((size_t)(n_seq * B), sizeof(int64_t));
    int64_t q, i, b, total = 0;
    int s;
    for (q = 0; q < n_seq; q++)
        for (i = 0; i < n_rows; i++)
            for (s = 0; s < k; s++) {
                int32_t v = block_idx[(q * n_rows + i) * k + s];
                if (v >= 0)
                    cursor[q * B + v]++;
            }
    for (q = 0; q < n_seq; q++) {
        for (b = 0; b < B; b++) {
            int64_t c = cursor[q * B + b];
            offsets[q * (B + 1) + b] = (int32_t)total;
            cursor[q * B + b] = total;
            total += c;
        }
        offsets[q * (B + 1) + B] = (int32_t)total;
    }
    for (q = 0; q < n_seq; q++)
        for (i = 0; i < n_rows; i++)
            for (s = 0; s < k; s++) {
                int32_t v = block_idx[(q * n_rows + i) * k + s];
                if (v >= 0)
                    entries[cursor[q * B + v]++] = (int32_t)(i * k + s);
            }
    free(cursor);
}

/* Decoders exposed for their own pins. */
float oracle_decode_bf16(uint16_t h) { return dec_bf16(h); }
double oracle_decode_e4m3(uint8_t c) { return dec_e4m3(c); }

int oracle_num_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
