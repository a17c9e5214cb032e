/*
 * lora_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU statement of the heterogeneous-adapter
 * LoRA delta, used to check the HIP library.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no source
 * with the GPU library and must never be used as a fallback for it.
 *
 * Everything is the plain definition: bf16 inputs are decoded exactly to
 * double, every product of two bf16 values is exact in double, and sums run in
 * ascending index order in double.  No blocking, no fusion, no reordering.
 *
 * Sources (the pages this library's method comes from):
 *  - "m07 -- Multi-Adapter (LoRA) Serving", section "2. Scale Numbers": a
 *    weight W of shape (d_out, d_in) gains B.A with A (r, d_in) and
 *    B (d_out, r).
 *  - same page, "6. Deep Dive A: Batching Heterogeneous Adapters": the forward
 *    is y = Wx + (B.A)x.(alpha/r); the adapter term is per row; the batched
 *    kernel takes the batch, an index vector mapping each sequence to an
 *    adapter slot, and the adapter buffer, and gathers inside the kernel.
 *  - "12. Adapter Serving and Multi-Tenant Customization", section
 *    "Scheduling with adapter awareness": requests are grouped by adapter,
 *    base-only requests form their own group, and the adapter products are a
 *    second, indexed operation after the shared base product.
 *  - "LoRA, quotas and noisy neighbours", section "One weight read, many
 *    adapters": rows are tagged with their adapter and grouped (segmented
 *    gather matrix-vector).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - rows whose id is negative are base-only: no segment, y unchanged;
 *  - ids >= num_slots are errors: the row is skipped and counted;
 *  - segments are in ascending adapter id, rows ascending inside a segment;
 *  - rank 0 means the module is not targeted: zero delta;
 *  - a table rank outside [0, max_rank] is an error: skipped and counted;
 *  - scale (alpha/r) multiplies the delta, 1.0 when unspecified;
 *  - the oracle keeps y in double with no output rounding;
 *  - int8 factors: one fp32 scale per row (see the int8 functions below);
 *  - a 4-bit base weight: signed values in [-8, 7], two per byte (the lower
 *    input index in the low nibble), one fp32 scale per output row and group
 *    of consecutive inputs (see oracle_base_q4 below).
 */
#include <stdint.h>
#include <string.h>

/* bf16 is the upper half of an IEEE-754 binary32; decoding is exact. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Segment build: group rows by adapter.  For each adapter a in ascending
 * order, the rows b with ids[b] == a are appended to perm in ascending b; a
 * segment opens for every adapter with at least one row.
 *   perm[n_valid], seg_offsets[nseg + 1], seg_adapter[nseg], *num_segments.
 * Returns the number of rows whose id is >= num_slots (errors).
 */
int32_t oracle_build_segments(const int32_t *ids, int32_t num_rows,
                              int32_t num_slots, int32_t *perm,
                              int32_t *seg_offsets, int32_t *seg_adapter,
                              int32_t *num_segments)
{
    int32_t bad = 0, pos = 0, nseg = 0;
    for (int32_t b = 0; b < num_rows; ++b)
        if (ids[b] >= num_slots)
            ++bad;
    for (int32_t a = 0; a < num_slots; ++a) {
        int32_t start = pos;
        for (int32_t b = 0; b < num_rows; ++b)
            if (ids[b] == a)
                perm[pos++] = b;
        if (pos > start) {
            seg_offsets[nseg] = start;
            seg_adapter[nseg] = a;
            ++nseg;
        }
    }
    seg_offsets[nseg] = pos;
    *num_segments = nseg;
    return bad;
}

/* v[j] = sum_k A[j][k] * x[k] for j < rank  (A row-major, leading dim d_in). */
void oracle_shrink_row(const uint16_t *x, int32_t d_in, const uint16_t *A,
                       int32_t rank, double *v)
{
    for (int32_t j = 0; j < rank; ++j) {
        double s = 0.0;
        const uint16_t *a = A + (int64_t)j * d_in;
        for (int32_t k = 0; k < d_in; ++k)
            s += bf16_value(a[k]) * bf16_value(x[k]);
        v[j] = s;
    }
}

/* delta[n] = scale * sum_j B[n][j] * v[j]  (B row-major; its rows are
 * stored rank rounded up to a multiple of 8 apart, the columns past the rank
 * being padding that is never read). */
void oracle_expand_row(const double *v, int32_t rank, const uint16_t *B,
                       int32_t d_out, double scale, double *delta)
{
    const int64_t ldb = ((int64_t)rank + 7) / 8 * 8;
    for (int32_t n = 0; n < d_out; ++n) {
        double s = 0.0;
        const uint16_t *b = B + (int64_t)n * ldb;
        for (int32_t j = 0; j < rank; ++j)
            s += bf16_value(b[j]) * v[j];
        delta[n] = scale * s;
    }
}

/*
 * Adapters stored in int8 ("m07 -- Multi-Adapter (LoRA) Serving", "9.
 * Bottlenecks and Evolution", item 3: quantised adapters halve the bytes;
 * the page fixes no scheme).  Reading taken: symmetric int8 with one fp32
 * scale per row, value = scale[row] * q[row][col].  A factor block holds the
 * row scales first (their count rounded up to a multiple of 4, so the int8
 * values start 16-byte aligned), then the int8 rows, each padded to a
 * multiple of 16 bytes:
 *   A block: float sA[round_up(rank, 4)];  int8 A[rank][lda8],
 *            lda8 = round_up(d_in, 16) (columns past d_in never read)
 *   B block: float sB[round_up(d_out, 4)]; int8 B[d_out][ldb8],
 *            ldb8 = round_up(rank, 16) (columns past the rank never read)
 * Each dequantised value scale * q is exact in double, and so is its product
 * with a bf16 value.
 */
enum { ORACLE_FMT_BF16 = 0, ORACLE_FMT_INT8_ROWS = 1 };

static int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

/* v[j] = sum_k (sA[j] * qA[j][k]) * x[k] for j < rank. */
void oracle_shrink_row_q8(const uint16_t *x, int32_t d_in, const void *A_block,
                          int32_t rank, double *v)
{
    const float *sa = (const float *)A_block;
    const int8_t *qa = (const int8_t *)(sa + round_up(rank, 4));
    const int64_t lda8 = round_up(d_in, 16);
    for (int32_t j = 0; j < rank; ++j) {
        double s = 0.0;
        const int8_t *a = qa + (int64_t)j * lda8;
        for (int32_t k = 0; k < d_in; ++k)
            s += ((double)sa[j] * (double)a[k]) * bf16_value(x[k]);
        v[j] = s;
    }
}

/* delta[n] = scale * sum_j (sB[n] * qB[n][j]) * v[j]. */
void oracle_expand_row_q8(const double *v, int32_t rank, const void *B_block,
                          int32_t d_out, double scale, double *delta)
{
    const float *sb = (const float *)B_block;
    const int8_t *qb = (const int8_t *)(sb + round_up(d_out, 4));
    const int64_t ldb8 = round_up(rank, 16);
    for (int32_t n = 0; n < d_out; ++n) {
        double s = 0.0;
        const int8_t *b = qb + (int64_t)n * ldb8;
        for (int32_t j = 0; j < rank; ++j)
            s += ((double)sb[n] * (double)b[j]) * v[j];
        delta[n] = scale * s;
    }
}

/*
 * One projection (module) over a set of rows.
 *
 *   x      bf16 [num_rows][ldx]        input rows
 *   y0     bf16 [num_rows][ldy]        base output W.x
 *   ids    int32 [num_rows]            row -> adapter slot (-1 = base only)
 *   A_ptr, B_ptr, rank, scale  [num_slots]   the adapter table for this module
 *   fmt    int32 [num_slots] or NULL   factor format per slot (NULL: all bf16;
 *                                      an unknown code is an error, skipped)
 *   rows   int32 [n_sel]               which rows to compute (any order)
 * Outputs, one line per selected row (in the order of `rows`):
 *   v      double [n_sel][max_rank]    shrink result, 0 beyond the rank
 *   delta  double [n_sel][d_out]       scale * B.v   (0 for skipped rows)
 *   y      double [n_sel][d_out]       y0 + delta    (y0 for skipped rows)
 * Any of v, delta, y may be NULL.  Returns the number of selected rows
 * skipped because the table rank is outside [0, max_rank] or the format is
 * unknown.
 */
int32_t oracle_lora_module(const uint16_t *x, int64_t ldx, int32_t num_rows,
                           int32_t d_in, const uint16_t *y0, int64_t ldy,
                           int32_t d_out, const int32_t *ids, int32_t num_slots,
                           const uint16_t *const *A_ptr,
                           const uint16_t *const *B_ptr, const int32_t *rank,
                           const float *scale, const int32_t *fmt,
                           int32_t max_rank, const int32_t *rows, int32_t n_sel,
                           double *v, double *delta, double *y, double *scratch)
{
    int32_t bad = 0;
    /* scratch holds max_rank + d_out doubles */
    double *vr = scratch;
    double *dr = scratch + max_rank;
    for (int32_t i = 0; i < n_sel; ++i) {
        int32_t b = rows[i];
        int32_t a = (b >= 0 && b < num_rows) ? ids[b] : -1;
        int32_t r = 0;
        int ok = 0;
        int32_t f = ORACLE_FMT_BF16;
        if (a >= 0 && a < num_slots) {
            r = rank[a];
            f = fmt ? fmt[a] : ORACLE_FMT_BF16;
            if (r < 0 || r > max_rank ||
                (r > 0 && f != ORACLE_FMT_BF16 && f != ORACLE_FMT_INT8_ROWS))
                ++bad;
            else if (r > 0)
                ok = 1;
        }
        for (int32_t j = 0; j < max_rank; ++j)
            vr[j] = 0.0;
        for (int32_t n = 0; n < d_out; ++n)
            dr[n] = 0.0;
        if (ok && f == ORACLE_FMT_BF16) {
            oracle_shrink_row(x + (int64_t)b * ldx, d_in, A_ptr[a], r, vr);
            oracle_expand_row(vr, r, B_ptr[a], d_out, (double)scale[a], dr);
        } else if (ok) {
            oracle_shrink_row_q8(x + (int64_t)b * ldx, d_in, A_ptr[a], r, vr);
            oracle_expand_row_q8(vr, r, B_ptr[a], d_out, (double)scale[a], dr);
        }
        if (v)
            for (int32_t j = 0; j < max_rank; ++j)
                v[(int64_t)i * max_rank + j] = vr[j];
        if (delta)
            for (int32_t n = 0; n < d_out; ++n)
                delta[(int64_t)i * d_out + n] = dr[n];
        if (y)
            for (int32_t n = 0; n < d_out; ++n)
                y[(int64_t)i * d_out + n] =
                    bf16_value(y0[(int64_t)b * ldy + n]) + dr[n];
    }
    return bad;
}

/*
 * Base projection of a linear layer, the shared term of the forward
 * y = Wx + (B.A)x.(alpha/r) ("m07 -- Multi-Adapter (LoRA) Serving", "6. Deep
 * Dive A"): for each selected row b = rows[i] and output n,
 *     out[i][n] = sum over k ascending of W[n][k] * x[b][k]
 * in double.  W is bf16 [d_out][ldw] (row n: the weights of output n).
 */
void oracle_base_bf16(const uint16_t *W, int64_t ldw, int32_t d_out, int32_t d_in,
                      const uint16_t *x, int64_t ldx, const int32_t *rows, int32_t n_sel,
                      double *out)
{
    for (int32_t i = 0; i < n_sel; ++i) {
        const uint16_t *xr = x + (int64_t)rows[i] * ldx;
        for (int32_t n = 0; n < d_out; ++n) {
            const uint16_t *w = W + (int64_t)n * ldw;
            double s = 0.0;
            for (int32_t k = 0; k < d_in; ++k)
                s += bf16_value(w[k]) * bf16_value(xr[k]);
            out[(int64_t)i * d_out + n] = s;
        }
    }
}

/* The signed 4-bit value k of a packed row: byte k/2, low nibble for even k. */
static int32_t q4_value(const uint8_t *row, int32_t k)
{
    uint32_t nib = (k % 2 == 0) ? (row[k / 2] & 0xFu) : (row[k / 2] >> 4);
    return nib >= 8 ? (int32_t)nib - 16 : (int32_t)nib;
}

/*
 * The same with a 4-bit base weight ("12. Adapter Serving and Multi-Tenant
 * Customization", "Interactions with other engine mechanisms", Quantization:
 * the base in INT4, the adapter in BF16, the base dequantised and the sum
 * accumulated wide).  W[n][k] = Ws[n][k / group] * q[n][k], with q the signed
 * 4-bit value k of row n of Wq ([d_out][ldwq] bytes) and Ws fp32
 * [d_out][lds]; the product of an fp32 scale and a 4-bit integer is exact in
 * double.
 */
void oracle_base_q4(const uint8_t *Wq, int64_t ldwq, const float *Ws, int64_t lds,
                    int32_t group, int32_t d_out, int32_t d_in, const uint16_t *x,
                    int64_t ldx, const int32_t *rows, int32_t n_sel, double *out)
{
    for (int32_t i = 0; i < n_sel; ++i) {
        const uint16_t *xr = x + (int64_t)rows[i] * ldx;
        for (int32_t n = 0; n < d_out; ++n) {
            const uint8_t *q = Wq + (int64_t)n * ldwq;
            const float *sc = Ws + (int64_t)n * lds;
            double s = 0.0;
            for (int32_t k = 0; k < d_in; ++k)
                s += ((double)sc[k / group] * (double)q4_value(q, k)) * bf16_value(xr[k]);
            out[(int64_t)i * d_out + n] = s;
        }
    }
}
