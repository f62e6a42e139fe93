// Slot derivation: the pool rows a paged call reads and writes, derived on the
// device in one launch with no host synchronization (flashinfer.gdn_paged,
// gdn_paged_prefill_slots / gdn_paged_decode_slots and "Page table").
//
// Sequence b owns n = indptr[b+1] - indptr[b] pages and holds
// (n - 1) * page_size + last_page_len[b] tokens after the call; its L new
// tokens are the last ones, so its prefix is p = total - L.
//   read   = page holding token p - 1, or -1 when p == 0
//   write  = last page, or -1 when L == 0 (a zero-length sequence writes nothing)
//   ckpt   = indptr[b] + p / page_size  (the pages ending inside the call
//            follow in page_indices; the paged call checkpoints every
//            page_size tokens into page_indices from there)
//   prefix = p
//   chunk  = exclusive scan of ceil(((p mod 64) + L) / 64): chunks sit at
//            absolute multiples of 64, the first one padded on the left.
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kScanThreads = 1024;

__device__ __forceinline__ int chunks_of(int p, int L) {
  return L > 0 ? ((p & (kChunk - 1)) + L + kChunk - 1) / kChunk : 0;
}

__global__ __launch_bounds__(kScanThreads) void prefill_slots_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ lpl, int B, int ps,
    int32_t* __restrict__ read, int32_t* __restrict__ write, int32_t* __restrict__ ckpt,
    int32_t* __restrict__ prefix, int32_t* __restrict__ chunk_start, const int32_t* guard) {
  if (guarded(guard)) return;
  int carry = 0;
  for (int base = 0; base < B; base += kScanThreads) {
    const int b = base + (int)threadIdx.x;
    int nch = 0;
    if (b < B) {
      const int beg = ptr[b], end = ptr[b + 1];
      const int L = cu[b + 1] - cu[b];
      const int total = (end - beg - 1) * ps + lpl[b];
      const int p = total - L;
      read[b] = p > 0 ? idx[beg + (p - 1) / ps] : -1;
      write[b] = L > 0 ? idx[end - 1] : -1;
      ckpt[b] = beg + p / ps;
      prefix[b] = p;
      nch = chunks_of(p, L);
    }
    int tot;
    const int ex = block_exclusive_scan(nch, &tot);
    if (b < B) chunk_start[b] = carry + ex;
    carry += tot;
  }
}

__global__ __launch_bounds__(256) void decode_slots_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ ptr,
    const int32_t* __restrict__ lpl, int B, int32_t* __restrict__ read,
    int32_t* __restrict__ write) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int end = ptr[b + 1];
  const int last = idx[end - 1];
  // A token that opens a new page reads the previous page, else the last one.
  read[b] = lpl[b] == 1 ? idx[end - 2] : last;
  write[b] = last;
}

__device__ __forceinline__ int64_t ld_index(const void* p, int i, int idx64) {
  return idx64 ? ((const int64_t*)p)[i] : (int64_t)((const int32_t*)p)[i];
}

// Rows of the slot-argument prefill, normalised to int32 plus the chunk scan.
__global__ __launch_bounds__(kScanThreads) void general_slots_kernel(
    const int32_t* __restrict__ cu, int B, const void* sidx, const void* oidx,
    const void* cstart, const void* plen, int idx64, int has_init, int write_final,
    int32_t* __restrict__ read, int32_t* __restrict__ write, int32_t* __restrict__ ckpt,
    int32_t* __restrict__ prefix, int32_t* __restrict__ chunk_start) {
  int carry = 0;
  for (int base = 0; base < B; base += kScanThreads) {
    const int b = base + (int)threadIdx.x;
    int nch = 0;
    if (b < B) {
      const int L = cu[b + 1] - cu[b];
      const int rrow = sidx ? (int)ld_index(sidx, b, idx64) : b;
      read[b] = has_init ? rrow : -1;
      int w = -1;
      if (write_final && L > 0) w = oidx ? (int)ld_index(oidx, b, idx64) : rrow;
      write[b] = w;
      ckpt[b] = cstart ? (int)ld_index(cstart, b, idx64) : 0;
      const int p = plen ? (int)ld_index(plen, b, idx64) : 0;
      prefix[b] = p;
      nch = chunks_of(p, L);
    }
    int tot;
    const int ex = block_exclusive_scan(nch, &tot);
    if (b < B) chunk_start[b] = carry + ex;
    carry += tot;
  }
}

}  // namespace

hipError_t launch_prefill_slots(const int32_t* cu, const int32_t* idx, const int32_t* ptr,
                                const int32_t* lpl, int B, int page_size, int32_t* read,
                                int32_t* write, int32_t* ckpt, int32_t* prefix,
                                int32_t* chunk_start, const int32_t* guard, hipStream_t s) {
  if (B == 0) return hipSuccess;
  prefill_slots_kernel<<<1, kScanThreads, 0, s>>>(cu, idx, ptr, lpl, B, page_size, read, write,
                                                  ckpt, prefix, chunk_start, guard);
  return hipGetLastError();
}

hipError_t launch_decode_slots(const int32_t* idx, const int32_t* ptr, const int32_t* lpl,
                               int B, int32_t* read, int32_t* write, hipStream_t s) {
  if (B == 0) return hipSuccess;
  decode_slots_kernel<<<(B + 255) / 256, 256, 0, s>>>(idx, ptr, lpl, B, read, write);
  return hipGetLastError();
}

hipError_t launch_general_slots(const int32_t* cu, int B, const void* sidx, const void* oidx,
                                const void* cstart, const void* plen, int idx64, int has_init,
                                int write_final, int32_t* read, int32_t* write, int32_t* ckpt,
                                int32_t* prefix, int32_t* chunk_start, hipStream_t s) {
  if (B == 0) return hipSuccess;
  general_slots_kernel<<<1, kScanThreads, 0, s>>>(cu, B, sidx, oidx, cstart, plen, idx64,
                                                  has_init, write_final, read, write, ckpt,
                                                  prefix, chunk_start);
  return hipGetLastError();
}

}  // namespace gdn
