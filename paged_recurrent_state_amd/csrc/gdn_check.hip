// Debug validation of a paged batch on the device (flashinfer.gdn_paged,
// "Page table": page tables hold real page ids, never -1 padding; "Slot
// arguments": a row one sequence writes is touched by no other sequence of the
// call; the gaudi-cookbook gdn-prefix-cache note, "The fix": refuse rather
// than guess).  One workgroup writes a bitmask of what it finds; the paged
// calls, when asked to check, run it first and every later kernel of the call
// returns before touching memory if the mask is not zero.
//
// What a sequence b of a paged batch touches, from its n pages and
// last_page_len (it holds (n - 1) page_size + last_page_len tokens):
//   prefill (L new tokens, prefix p):  reads the page holding token p - 1 when
//     p > 0; writes the pages ending after p (entries p / page_size .. n - 1)
//     when L > 0
//   decode:  reads entry n - 2 when last_page_len == 1, else n - 1; writes n - 1
#include "gdn_internal.h"
#include "gdn_paged.h"

namespace gdn {

namespace {

constexpr int kCheckThreads = 1024;
constexpr int kCheckMaxSeqs = 2048;      // sequences the pairwise row check covers
constexpr int kCheckMaxTouched = 4096;   // touched entries the pairwise row check covers

struct CheckSmem {
  int id[kCheckMaxTouched];     // page id of each touched entry
  int owner[kCheckMaxTouched];  // its sequence, with bit 30 set for a write
};

__device__ __forceinline__ int block_or(int x) {
  __shared__ int acc;
  if (threadIdx.x == 0) acc = 0;
  __syncthreads();
  if (x) atomicOr(&acc, x);
  __syncthreads();
  const int r = acc;
  __syncthreads();
  return r;
}

// Touched entries of sequence b (offsets into page_indices): the read entry
// (or -1) and the written range [w0, w1).
struct Touch {
  int rd, w0, w1;
};

__device__ __forceinline__ Touch touched(const int32_t* cu, const int32_t* ptr, const int32_t* lpl,
                                         int b, int ps) {
  const int beg = ptr[b], end = ptr[b + 1], n = end - beg;
  Touch t{-1, 0, 0};
  if (cu) {
    const int L = cu[b + 1] - cu[b];
    const int p = (n - 1) * ps + lpl[b] - L;
    if (p > 0) t.rd = beg + (p - 1) / ps;
    if (L > 0) {
      t.w0 = beg + p / ps;
      t.w1 = end;
    }
  } else {
    t.rd = lpl[b] == 1 ? end - 2 : end - 1;
    t.w0 = end - 1;
    t.w1 = end;
  }
  return t;
}

__global__ __launch_bounds__(kCheckThreads) void check_paged_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ lpl, int B, int ps,
    int num_pages, int32_t* __restrict__ word) {
  __shared__ CheckSmem sm;
  const int tid = threadIdx.x;
  // 1. the CSR structure and the token counts, sequence by sequence
  int f = 0;
  if (tid == 0 && ptr[0] != 0) f |= GDN_CHECK_INDPTR;
  for (int b = tid; b < B; b += kCheckThreads) {
    const int beg = ptr[b], end = ptr[b + 1];
    if (end <= beg) {
      f |= GDN_CHECK_INDPTR;  // decreasing, or a sequence without pages
      continue;
    }
    const int l = lpl[b];
    if (l < 1 || l > ps) f |= GDN_CHECK_LAST_PAGE_LEN;
    const int total = (end - beg - 1) * ps + l;
    if (cu) {
      const int L = cu[b + 1] - cu[b];
      if (L < 0 || L > total) f |= GDN_CHECK_TOKENS;
    } else if (total < 2) {
      f |= GDN_CHECK_TOKENS;  // no token before the decoded one
    }
  }
  if (cu && tid == 0 && cu[0] != 0) f |= GDN_CHECK_TOKENS;
  f = block_or(f);
  if (f & (GDN_CHECK_INDPTR | GDN_CHECK_TOKENS | GDN_CHECK_LAST_PAGE_LEN)) {
    if (tid == 0) *word = f;  // ranges unknown: nothing further is read
    return;
  }
  // 2. every page id of the table is a row of the pool
  const int n_entries = ptr[B];
  for (int e = tid; e < n_entries; e += kCheckThreads) {
    const int x = idx[e];
    if (x < 0 || x >= num_pages) f |= GDN_CHECK_PAGE_ID;
  }
  f = block_or(f);
  if (f) {
    if (tid == 0) *word = f;
    return;
  }
  // 3. rows written by one sequence and read or written by another: list the
  // touched entries in LDS, then compare every written one with all others
  int total = 0;
  if (B <= kCheckMaxSeqs) {
    int carry = 0;
    for (int base = 0; base < B; base += kCheckThreads) {
      const int b = base + tid;
      int cnt = 0;
      Touch t{-1, 0, 0};
      if (b < B) {
        t = touched(cu, ptr, lpl, b, ps);
        cnt = (t.rd >= 0 && (t.rd < t.w0 || t.rd >= t.w1)) + (t.w1 - t.w0);
      }
      int tot;
      const int off = carry + block_exclusive_scan(cnt, &tot);
      if (b < B) {
        int k = off;
        if (off + cnt <= kCheckMaxTouched) {
          if (t.rd >= 0 && (t.rd < t.w0 || t.rd >= t.w1)) {
            sm.id[k] = idx[t.rd];
            sm.owner[k++] = b;
          }
          for (int e = t.w0; e < t.w1; ++e) {
            sm.id[k] = idx[e];
            sm.owner[k++] = b | (1 << 30);
          }
        }
      }
      carry += tot;
    }
    total = carry;
    __syncthreads();
  }
  if (B > kCheckMaxSeqs || total > kCheckMaxTouched) {
    f |= GDN_CHECK_NOT_CHECKED;
  } else {
    for (int i = tid; i < total; i += kCheckThreads) {
      if (!(sm.owner[i] & (1 << 30))) continue;  // compare from the written entries
      const int x = sm.id[i], o = sm.owner[i] & ~(1 << 30);
      for (int j = 0; j < total; ++j)
        if (sm.id[j] == x && (sm.owner[j] & ~(1 << 30)) != o) f |= GDN_CHECK_SHARED_ROW;
    }
  }
  f = block_or(f);
  if (tid == 0) *word = f;
}

}  // namespace

hipError_t launch_check_paged(const int32_t* cu, const int32_t* idx, const int32_t* ptr,
                              const int32_t* lpl, int B, int page_size, int num_pages,
                              int32_t* word, hipStream_t s) {
  check_paged_kernel<<<1, kCheckThreads, 0, s>>>(cu, idx, ptr, lpl, B, page_size, num_pages, word);
  return hipGetLastError();
}

}  // namespace gdn
