// table_checks.cpp - host-side checks of the index tables' values.
//
// The device calls check arguments, never values: page ids, positions,
// lengths and indptr entries are read as given (the launcher note on the
// flashinfer.quantization module page's materializer section says the same
// of FlashInfer's kernels). These functions are the debugging aid for that
// gap: they read host copies of the tables, report the first value a call
// would use out of range, and touch no device memory. Plain host C++ with no
// HIP dependency, so that it also builds with the host sanitizers.
#include <stdint.h>
#include <string.h>

#include "../../include/kvfp4.h"

namespace {

kvfp4_status_t fail(kvfp4_table_report_t *r, int32_t problem, int64_t index, int64_t value)
{
    r->problem = problem;
    r->index = index;
    r->value = value;
    return KVFP4_EVALUE;
}

kvfp4_status_t ok(kvfp4_table_report_t *r)
{
    memset(r, 0, sizeof(*r));
    return KVFP4_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t table_entry(const void *bt, int32_t bt_dtype, int64_t i)
{
    return bt_dtype == KVFP4_I64 ? ((const int64_t *)bt)[i] : (int64_t)((const int32_t *)bt)[i];
}

// indptr[0] == 0 and non-decreasing; problem index = the entry that breaks it
kvfp4_status_t check_indptr(const int32_t *indptr, int32_t batch, kvfp4_table_report_t *r)
{
    if (indptr[0] != 0)
        return fail(r, KVFP4_TABLE_INDPTR_START, 0, indptr[0]);
    for (int32_t b = 0; b < batch; ++b)
        if (indptr[b + 1] < indptr[b])
            return fail(r, KVFP4_TABLE_INDPTR_ORDER, b + 1, indptr[b + 1]);
    return KVFP4_OK;
}

// sort (key) ascending, in place: heapsort, no allocation
void sort_keys(int64_t *a, int64_t n)
{
    auto sift = [a](int64_t i, int64_t end) {
        for (;;) {
            int64_t c = 2 * i + 1;
            if (c >= end)
                return;
            if (c + 1 < end && a[c + 1] > a[c])
                ++c;
            if (a[i] >= a[c])
                return;
            const int64_t t = a[i];
            a[i] = a[c];
            a[c] = t;
            i = c;
        }
    };
    for (int64_t i = n / 2 - 1; i >= 0; --i)
        sift(i, n);
    for (int64_t end = n - 1; end > 0; --end) {
        const int64_t t = a[0];
        a[0] = a[end];
        a[end] = t;
        sift(0, end);
    }
}

}  // namespace

extern "C" {

kvfp4_status_t kvfp4_check_append_tables(const int32_t *batch_indices, const int32_t *positions, int64_t nnz,
                                         const int32_t *kv_indices, const int32_t *kv_indptr,
                                         const int32_t *kv_last_page_len, int32_t batch_size, int32_t page_size,
                                         int32_t num_pages, int64_t *scratch, kvfp4_table_report_t *report)
{
    if (!report)
        return KVFP4_EINVAL;
    if (nnz < 0 || batch_size < 0 || page_size <= 0 || num_pages < 0)
        return KVFP4_EINVAL;
    if (!kv_indptr || (batch_size > 0 && !kv_last_page_len) || (nnz > 0 && (!batch_indices || !positions)))
        return KVFP4_EINVAL;
    kvfp4_status_t s = check_indptr(kv_indptr, batch_size, report);
    if (s != KVFP4_OK)
        return s;
    const int64_t n_entries = kv_indptr[batch_size];
    if (n_entries > 0 && !kv_indices)
        return KVFP4_EINVAL;
    for (int64_t i = 0; i < n_entries; ++i)
        if (kv_indices[i] < 0 || kv_indices[i] >= num_pages)
            return fail(report, KVFP4_TABLE_PAGE_RANGE, i, kv_indices[i]);
    for (int32_t b = 0; b < batch_size; ++b) {
        const int64_t pages = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
        const int32_t last = kv_last_page_len[b];
        if (pages > 0 ? (last < 1 || last > page_size) : last != 0)
            return fail(report, KVFP4_TABLE_LAST_PAGE_LEN, b, last);
    }
    for (int64_t r = 0; r < nnz; ++r) {
        const int32_t b = batch_indices[r];
        if (b < 0 || b >= batch_size)
            return fail(report, KVFP4_TABLE_BATCH_RANGE, r, b);
        const int64_t pages = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
        const int64_t space = pages > 0 ? (pages - 1) * page_size + kv_last_page_len[b] : 0;
        if (positions[r] < 0 || positions[r] >= space)
            return fail(report, KVFP4_TABLE_POSITION_RANGE, r, positions[r]);
    }
    if (scratch && nnz > 1) {
        // rows writing the same (request, position) race: sort the pairs
        for (int64_t r = 0; r < nnz; ++r)
            scratch[r] = ((int64_t)batch_indices[r] << 32) | (uint32_t)positions[r];
        sort_keys(scratch, nnz);
        for (int64_t r = 1; r < nnz; ++r)
            if (scratch[r] == scratch[r - 1]) {
                // report the first row (in row order) holding that pair
                for (int64_t q = 0; q < nnz; ++q)
                    if ((((int64_t)batch_indices[q] << 32) | (uint32_t)positions[q]) == scratch[r])
                        return fail(report, KVFP4_TABLE_DUPLICATE_ROW, q, positions[q]);
            }
    }
    return ok(report);
}

kvfp4_status_t kvfp4_check_step_rows(const int32_t *batch_indices, const int32_t *positions, int64_t nnz,
                                     const int32_t *seq_lens, int32_t batch_size, int64_t *scratch,
                                     kvfp4_table_report_t *report)
{
    if (!report)
        return KVFP4_EINVAL;
    if (nnz != batch_size || batch_size < 0 || (batch_size > 0 && (!batch_indices || !positions || !seq_lens)))
        return KVFP4_EINVAL;
    for (int64_t r = 0; r < nnz; ++r) {
        const int32_t b = batch_indices[r];
        if (b < 0 || b >= batch_size)
            return fail(report, KVFP4_TABLE_BATCH_RANGE, r, b);
        if ((int64_t)positions[r] != (int64_t)seq_lens[b] - 1)
            return fail(report, KVFP4_TABLE_STEP_POSITION, r, positions[r]);
    }
    if (scratch) {
        // one row per request: with nnz == batch_size a request seen twice
        // is the same as a request missing
        for (int32_t b = 0; b < batch_size; ++b)
            scratch[b] = -1;
        for (int64_t r = 0; r < nnz; ++r) {
            const int32_t b = batch_indices[r];
            if (scratch[b] >= 0)
                return fail(report, KVFP4_TABLE_DUPLICATE_ROW, r, b);
            scratch[b] = r;
        }
    }
    return ok(report);
}

kvfp4_status_t kvfp4_check_paged_tables(const void *block_tables, int32_t bt_dtype, int64_t bt_row_stride,
                                        int32_t bt_cols, const int32_t *seq_lens, int32_t batch_size,
                                        int32_t page_size, int32_t num_pages, int32_t max_seq_len,
                                        kvfp4_table_report_t *report)
{
    if (!report)
        return KVFP4_EINVAL;
    if (bt_dtype != KVFP4_I32 && bt_dtype != KVFP4_I64)
        return KVFP4_EINVAL;
    if (batch_size < 0 || page_size <= 0 || num_pages < 0 || bt_cols < 0 || bt_row_stride < bt_cols ||
        max_seq_len < 0)
        return KVFP4_EINVAL;
    if (batch_size > 0 && (!seq_lens || (bt_cols > 0 && !block_tables)))
        return KVFP4_EINVAL;
    for (int32_t b = 0; b < batch_size; ++b) {
        const int32_t len = seq_lens[b];
        const int64_t used = len < max_seq_len ? len : max_seq_len;
        if (len < 0 || ceil_div(used, page_size) > bt_cols)
            return fail(report, KVFP4_TABLE_LENGTH_RANGE, b, len);
        const int64_t need = ceil_div(used, page_size);
        for (int64_t j = 0; j < need; ++j) {
            const int64_t page = table_entry(block_tables, bt_dtype, b * bt_row_stride + j);
            if (page < 0 || page >= num_pages)
                return fail(report, KVFP4_TABLE_PAGE_RANGE, b * bt_row_stride + j, page);
        }
    }
    return ok(report);
}

kvfp4_status_t kvfp4_check_materialize_tables(const int32_t *block_tables, int32_t uses_shared_paged_kv_idx,
                                              int64_t bt_row_stride, int64_t bt_kv_stride, int32_t bt_cols,
                                              const int32_t *seq_lens, const int32_t *kv_page_indptr,
                                              int32_t batch_size, int32_t page_size, int32_t num_pages,
                                              int32_t max_pages_per_seq, int64_t num_out_pages,
                                              kvfp4_table_report_t *report)
{
    if (!report)
        return KVFP4_EINVAL;
    if (batch_size < 0 || page_size <= 0 || num_pages < 0 || max_pages_per_seq < 0 || bt_cols < max_pages_per_seq ||
        num_out_pages < 1)
        return KVFP4_EINVAL;
    if (uses_shared_paged_kv_idx ? bt_row_stride < bt_cols
                                 : (bt_kv_stride < bt_cols || bt_row_stride < bt_kv_stride + bt_cols))
        return KVFP4_EINVAL;
    if (!kv_page_indptr || (batch_size > 0 && (!seq_lens || (bt_cols > 0 && !block_tables))))
        return KVFP4_EINVAL;
    kvfp4_status_t s = check_indptr(kv_page_indptr, batch_size, report);
    if (s != KVFP4_OK)
        return s;
    if ((int64_t)kv_page_indptr[batch_size] + 1 > num_out_pages)
        return fail(report, KVFP4_TABLE_OUT_PAGES, batch_size, kv_page_indptr[batch_size]);
    for (int32_t b = 0; b < batch_size; ++b) {
        const int32_t len = seq_lens[b];
        if (len < 0 || (int64_t)len > (int64_t)max_pages_per_seq * page_size)
            return fail(report, KVFP4_TABLE_LENGTH_RANGE, b, len);
        const int64_t need = ceil_div(len, page_size);
        if ((int64_t)kv_page_indptr[b + 1] - kv_page_indptr[b] < need)
            return fail(report, KVFP4_TABLE_RESERVATION, b, (int64_t)kv_page_indptr[b + 1] - kv_page_indptr[b]);
        for (int kv = 0; kv < (uses_shared_paged_kv_idx ? 1 : 2); ++kv)
            for (int64_t j = 0; j < need; ++j) {
                const int64_t at = b * bt_row_stride + kv * bt_kv_stride + j;
                if (block_tables[at] < 0 || block_tables[at] >= num_pages)
                    return fail(report, KVFP4_TABLE_PAGE_RANGE, at, block_tables[at]);
            }
    }
    return ok(report);
}

const char *kvfp4_table_problem_string(int32_t problem)
{
    switch (problem) {
    case KVFP4_TABLE_OK: return "no problem";
    case KVFP4_TABLE_INDPTR_START: return "the indptr array does not start at 0";
    case KVFP4_TABLE_INDPTR_ORDER: return "the indptr array decreases";
    case KVFP4_TABLE_PAGE_RANGE: return "a page id outside [0, num_pages)";
    case KVFP4_TABLE_BATCH_RANGE: return "a row's request index outside [0, batch_size)";
    case KVFP4_TABLE_POSITION_RANGE: return "a row's position outside its request's reserved space";
    case KVFP4_TABLE_LAST_PAGE_LEN: return "kv_last_page_len outside [1, page_size] (0 for a request without pages)";
    case KVFP4_TABLE_DUPLICATE_ROW: return "two rows write the same (request, position)";
    case KVFP4_TABLE_LENGTH_RANGE: return "a length below 0 or longer than its table row addresses";
    case KVFP4_TABLE_RESERVATION: return "kv_page_indptr reserves fewer pages than the request needs";
    case KVFP4_TABLE_OUT_PAGES: return "out has fewer than kv_page_indptr[batch_size] + 1 pages";
    case KVFP4_TABLE_STEP_POSITION: return "a decode-step row's position is not its request's newest token";
    default: return "unknown problem";
    }
}

}  // extern "C"
