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
// Layout: one 256-thread workgroup per (sequence, head).  Each 16-lane group
// owns one 512-byte state row at a time: lane c holds k = 4c..4c+3 and
// 64+4c..64+4c+3, so one 16-byte load instruction covers 4 whole rows and
// the row's dot products reduce inside the 16-lane group with 4 DPP steps
// (no LDS traffic).  16 rows per workgroup per step, all 8 steps' loads
// issued before any arithmetic.
// Loads and stores bypass the caches' retention (non-temporal): every byte is
// touched once.
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kSteps = kDim / 16;  // 8: 16 rows per workgroup per step

__device__ __forceinline__ int64_t ld_index(const void* p, int i, int idx64) {
  return idx64 ? ((const int64_t*)p)[i] : (int64_t)((const int32_t*)p)[i];
}

// Sum over the 16 lanes of a DPP row, returned to all of them: swap
// neighbours, swap pairs, mirror within 8, mirror within 16.
template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xb1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4e>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
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
  const int g = lane >> 4;  // row within the wave's 4 rows of a step
  const int c = lane & 15;  // k = 4c..4c+3 and 64+4c..64+4c+3

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
  float k8[8], q8[8];
  {
    const u16* kp = p.k + ((int64_t)b * p.Hqk + hq) * kDim + 4 * c;
    const u16* qp = p.q + ((int64_t)b * p.Hqk + hq) * kDim + 4 * c;
    float t[4];
    unpack4(*(const u32x2*)kp, t);
    for (int i = 0; i < 4; ++i) k8[i] = t[i];
    unpack4(*(const u32x2*)(kp + 64), t);
    for (int i = 0; i < 4; ++i) k8[4 + i] = t[i];
    unpack4(*(const u32x2*)qp, t);
    for (int i = 0; i < 4; ++i) q8[i] = t[i];
    unpack4(*(const u32x2*)(qp + 64), t);
    for (int i = 0; i < 4; ++i) q8[4 + i] = t[i];
  }
  const int64_t bh = (int64_t)b * p.H + h;
  const float alpha = p.g ? expf(p.g[bh]) : 1.f;
  const float bt = p.beta ? p.beta[bh] : 1.f;

  // step it covers rows 16*it + 4*wid + g
  f32x4 s[kSteps][2];
  if (rd >= 0) {
    const float* src = p.init + rd * p.init_stride + (int64_t)h * kDim * kDim + 4 * c;
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
      const int row = 16 * it + 4 * wid + g;
      s[it][0] = __builtin_nontemporal_load((const f32x4*)(src + row * kDim));
      s[it][1] = __builtin_nontemporal_load((const f32x4*)(src + row * kDim + 64));
    }
  } else {
#pragma unroll
    for (int it = 0; it < kSteps; ++it) s[it][0] = s[it][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float vv[kSteps];
#pragma unroll
  for (int it = 0; it < kSteps; ++it) vv[it] = bf2f(p.v[bh * kDim + 16 * it + 4 * wid + g]);

  float kq = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) kq += k8[i] * q8[i];
  kq = sum16(kq);

  float* dst = wr >= 0 ? p.out + wr * p.out_stride + (int64_t)h * kDim * kDim + 4 * c : nullptr;
  float o_mine = 0.f;  // o of row 16*c + 4*wid + g (lanes c < 8)
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int row = 16 * it + 4 * wid + g;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sk += s[it][hh][i] * k8[4 * hh + i];
        sq += s[it][hh][i] * q8[4 * hh + i];
      }
    sk = sum16(sk);
    sq = sum16(sq);
    const float delta = bt * (vv[it] - alpha * sk);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = alpha * s[it][hh][i] + delta * k8[4 * hh + i];
      if (dst) __builtin_nontemporal_store(y, (f32x4*)(dst + row * kDim + 64 * hh));
    }
    if (c == it) o_mine = p.scale * (alpha * sq + delta * kq);
  }
  if (c < kSteps) p.o[bh * kDim + 16 * c + 4 * wid + g] = f2bf(o_mine);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.num_seqs * p.H;
  if (blocks <= 0) return hipSuccess;
  decode_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace gdn
