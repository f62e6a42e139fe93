// Single-token Gated Delta-Rule decode on a paged pool (flashinfer.gdn_paged,
// gated_delta_rule_decode_paged): a streaming read-update-write of the fp32
// [V, K] state of every (sequence, v-head).
//
// For each state row v (alpha = exp(g), all in fp32):
//   s_k = S[v].k,  s_q = S[v].q
//   delta = beta (v_v - alpha s_k)
//   S'[v] = alpha S[v] + delta k
//   o_v   = scale (alpha s_q + delta (k.q))        (= scale S'[v].q)
// so the state is read once and written once.  Rows: paged mode derives them
// in the kernel (last_page_len == 1 -> read page n-2, write page n-1; else the
// last page in place); explicit mode takes index arrays.  A read row of -1
// starts from literal zeros; a write row of -1 skips the store.
//
// Layout: one 256-thread workgroup per (sequence, head); each half-wave owns a
// 512-byte state row at a time (32 lanes x 16 B, coalesced), 8 rows per
// workgroup per step, all 16 steps' loads issued before any arithmetic.
// Loads and stores bypass the caches' retention (non-temporal): every byte is
// touched once.
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerLane = kDim / 8;  // 16

__device__ __forceinline__ int64_t ld_index(const void* p, int i, int idx64) {
  return idx64 ? ((const int64_t*)p)[i] : (int64_t)((const int32_t*)p)[i];
}

__device__ __forceinline__ float sum32(float x) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ void unpack4(u32x2 w, float (&f)[4]) {
  f[0] = bf2f(u16(w.x & 0xffffu));
  f[1] = bf2f(u16(w.x >> 16));
  f[2] = bf2f(u16(w.y & 0xffffu));
  f[3] = bf2f(u16(w.y >> 16));
}

__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeParams p) {
  const int bid = blockIdx.x;
  const int b = bid / p.H;
  const int h = bid - b * p.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int half = lane >> 5;
  const int kl = lane & 31;

  int64_t rd, wr;
  if (p.mode == 1) {
    const int end = p.page_indptr[b + 1];
    const int last = p.page_indices[end - 1];
    wr = last;
    rd = p.last_page_len[b] == 1 ? p.page_indices[end - 2] : last;
  } else {
    const int64_t r0 = p.rd_idx ? ld_index(p.rd_idx, b, p.idx64) : (int64_t)b;
    rd = p.init ? r0 : -1;
    wr = p.out ? (p.wr_idx ? ld_index(p.wr_idx, b, p.idx64) : r0) : -1;
  }

  const int hq = h / p.group;
  float k4[4], q4[4];
  unpack4(*(const u32x2*)(p.k + ((int64_t)b * p.Hqk + hq) * kDim + 4 * kl), k4);
  unpack4(*(const u32x2*)(p.q + ((int64_t)b * p.Hqk + hq) * kDim + 4 * kl), q4);
  const int64_t bh = (int64_t)b * p.H + h;
  const float alpha = p.g ? expf(p.g[bh]) : 1.f;
  const float bt = p.beta ? p.beta[bh] : 1.f;

  f32x4 s[kRowsPerLane];
  if (rd >= 0) {
    const float* src = p.init + rd * p.init_stride + (int64_t)h * kDim * kDim + 4 * kl;
#pragma unroll
    for (int it = 0; it < kRowsPerLane; ++it) {
      const int row = it * 8 + wid * 2 + half;
      s[it] = __builtin_nontemporal_load((const f32x4*)(src + row * kDim));
    }
  } else {
#pragma unroll
    for (int it = 0; it < kRowsPerLane; ++it) s[it] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float vv[kRowsPerLane];
#pragma unroll
  for (int it = 0; it < kRowsPerLane; ++it) vv[it] = bf2f(p.v[bh * kDim + it * 8 + wid * 2 + half]);

  const float kq = sum32(k4[0] * q4[0] + k4[1] * q4[1] + k4[2] * q4[2] + k4[3] * q4[3]);

  float* dst = wr >= 0 ? p.out + wr * p.out_stride + (int64_t)h * kDim * kDim + 4 * kl : nullptr;
#pragma unroll
  for (int it = 0; it < kRowsPerLane; ++it) {
    const int row = it * 8 + wid * 2 + half;
    const f32x4 x = s[it];
    float sk = x[0] * k4[0] + x[1] * k4[1] + x[2] * k4[2] + x[3] * k4[3];
    float sq = x[0] * q4[0] + x[1] * q4[1] + x[2] * q4[2] + x[3] * q4[3];
    sk = sum32(sk);
    sq = sum32(sq);
    const float delta = bt * (vv[it] - alpha * sk);
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = alpha * x[i] + delta * k4[i];
    if (dst) __builtin_nontemporal_store(y, (f32x4*)(dst + row * kDim));
    if (kl == 0) p.o[bh * kDim + row] = f2bf(p.scale * (alpha * sq + delta * kq));
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.num_seqs * p.H;
  if (blocks <= 0) return hipSuccess;
  decode_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace gdn
