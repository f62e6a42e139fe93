// Page-table format conversions on the device (FlashInfer CSR paging drill,
// sections 2 and 3): a padded block table with per-sequence token counts, as
// vLLM keeps it, to the CSR triple (indptr, indices, last_page_len) the paged
// calls take, and back.  No host synchronization; nothing is allocated.
//
// Sequence b of ctx tokens owns ceil(ctx / page_size) pages; indptr is the
// running sum of those counts (indptr[0] = 0), the indices are the first that
// many entries of every table row, rows in order, and the last page holds
// ctx - (pages - 1) * page_size tokens (1 .. page_size, never 0).  Backwards,
// the page counts are adjacent differences of indptr, a row is its pages
// followed by zeros, and ctx = (pages - 1) * page_size + last_page_len.
//
// Rows the formats cannot describe (ctx < 1, more pages than the table has
// columns, no pages, last_page_len outside 1 .. page_size) become empty rows
// (no pages, ctx or last_page_len 0) and are counted, so that no kernel reads
// outside the arrays it was given.
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kTabThreads = 1024;

// Pages of a sequence of ctx tokens, 0 when the table cannot hold it.
__device__ __forceinline__ int pages_of(int ctx, int ps, int max_blocks) {
  if (ctx < 1) return 0;
  const int n = (int)(((int64_t)ctx + ps - 1) / ps);
  return n <= max_blocks ? n : 0;
}

// One workgroup: page counts -> indptr (scan), last_page_len, bad-row count.
__global__ __launch_bounds__(kTabThreads) void csr_plan_kernel(
    const int32_t* __restrict__ ctx, int B, int ps, int max_blocks, int32_t* __restrict__ indptr,
    int32_t* __restrict__ lpl, int32_t* __restrict__ bad) {
  int carry = 0, nbad = 0;
  if (threadIdx.x == 0) indptr[0] = 0;
  for (int base = 0; base < B; base += kTabThreads) {
    const int b = base + (int)threadIdx.x;
    int n = 0, invalid = 0;
    if (b < B) {
      const int c = ctx[b];
      n = pages_of(c, ps, max_blocks);
      invalid = n == 0;
      lpl[b] = n ? c - (n - 1) * ps : 0;
    }
    int tot, tbad;
    const int ex = block_exclusive_scan(n, &tot);
    block_exclusive_scan(invalid, &tbad);
    if (b < B) indptr[b + 1] = carry + ex + n;
    carry += tot;
    nbad += tbad;
  }
  if (bad && threadIdx.x == 0) *bad = nbad;
}

// One workgroup per row: the row's pages into indices[indptr[b] ..].
__global__ __launch_bounds__(256) void csr_fill_kernel(const int32_t* __restrict__ table,
                                                       int64_t row_stride,
                                                       const int32_t* __restrict__ indptr,
                                                       int32_t* __restrict__ indices) {
  const int b = blockIdx.x;
  const int beg = indptr[b], n = indptr[b + 1] - beg;
  const int32_t* row = table + (int64_t)b * row_stride;
  for (int j = threadIdx.x; j < n; j += blockDim.x) indices[beg + j] = row[j];
}

// One workgroup per row: pages then zero padding, and the context length.
__global__ __launch_bounds__(256) void table_fill_kernel(
    const int32_t* __restrict__ indptr, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ lpl, int ps, int max_blocks, int32_t* __restrict__ table,
    int64_t row_stride, int32_t* __restrict__ ctx) {
  const int b = blockIdx.x;
  const int beg = indptr[b], n = indptr[b + 1] - beg;
  const int last = lpl[b];
  const bool valid = n >= 1 && n <= max_blocks && last >= 1 && last <= ps;
  const int m = valid ? n : 0;
  int32_t* row = table + (int64_t)b * row_stride;
  for (int j = threadIdx.x; j < max_blocks; j += blockDim.x) row[j] = j < m ? indices[beg + j] : 0;
  if (threadIdx.x == 0) ctx[b] = valid ? (n - 1) * ps + last : 0;
}

// One workgroup: rows table_fill_kernel leaves empty.
__global__ __launch_bounds__(kTabThreads) void table_bad_kernel(const int32_t* __restrict__ indptr,
                                                                const int32_t* __restrict__ lpl,
                                                                int B, int ps, int max_blocks,
                                                                int32_t* __restrict__ bad) {
  int nbad = 0;
  for (int base = 0; base < B; base += kTabThreads) {
    const int b = base + (int)threadIdx.x;
    int invalid = 0;
    if (b < B) {
      const int n = indptr[b + 1] - indptr[b], last = lpl[b];
      invalid = !(n >= 1 && n <= max_blocks && last >= 1 && last <= ps);
    }
    int t;
    block_exclusive_scan(invalid, &t);
    nbad += t;
  }
  if (threadIdx.x == 0) *bad = nbad;
}

}  // namespace

hipError_t launch_block_table_to_csr(const int32_t* table, int64_t row_stride, const int32_t* ctx,
                                     int B, int max_blocks, int ps, int32_t* indptr,
                                     int32_t* indices, int32_t* lpl, int32_t* bad,
                                     hipStream_t s) {
  csr_plan_kernel<<<1, kTabThreads, 0, s>>>(ctx, B, ps, max_blocks, indptr, lpl, bad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || B == 0) return e;
  csr_fill_kernel<<<(unsigned)B, 256, 0, s>>>(table, row_stride, indptr, indices);
  return hipGetLastError();
}

hipError_t launch_csr_to_block_table(const int32_t* indptr, const int32_t* indices,
                                     const int32_t* lpl, int B, int ps, int max_blocks,
                                     int32_t* table, int64_t row_stride, int32_t* ctx,
                                     int32_t* bad, hipStream_t s) {
  if (B > 0) {
    table_fill_kernel<<<(unsigned)B, 256, 0, s>>>(indptr, indices, lpl, ps, max_blocks, table,
                                                  row_stride, ctx);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (bad) {
    table_bad_kernel<<<1, kTabThreads, 0, s>>>(indptr, lpl, B, ps, max_blocks, bad);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdn
