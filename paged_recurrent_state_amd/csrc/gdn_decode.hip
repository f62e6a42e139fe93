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
// Layout: one workgroup of NW waves per (sequence, head).  Each 16-lane group
// owns one state row at a time: for an fp32 state (512-byte rows) lane c
// holds k = 4c..4c+3 and 64+4c..64+4c+3, so one 16-byte load instruction
// covers 4 whole rows; for a bf16 state (256-byte rows) lane c holds
// k = 8c..8c+7, one 16-byte load a row.  The row's dot products reduce inside
// the 16-lane group with 4 DPP steps (no LDS traffic).  4 NW rows per
// workgroup per step, all 128 / (4 NW) steps' loads issued before any
// arithmetic; the update runs in fp32 either way and a bf16 row is stored
// rounded to nearest even.
// Loads and stores bypass the caches' retention (non-temporal): every byte is
// touched once.
#include <algorithm>

#include "gdn_internal.h"

namespace gdn {

namespace {


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
__device__ __forceinline__ void unpack8(u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Rows of sequence b: paged mode derives them from the page table; explicit
// mode takes index arrays (null: row b, and the write row = the read row).
struct DecRows {
  int64_t rd, wr;
};
__device__ __forceinline__ DecRows decode_rows(const DecodeParams& p, int b) {
  if (p.mode == 1) {
    const int end = p.page_indptr[b + 1];
    const int last = p.page_indices[end - 1];
    return DecRows{p.last_page_len[b] == 1 ? p.page_indices[end - 2] : last, last};
  }
  const int64_t r0 = p.rd_idx ? ld_index(p.rd_idx, b, p.idx64) : (int64_t)b;
  return DecRows{p.init ? r0 : -1, p.out ? (p.wr_idx ? ld_index(p.wr_idx, b, p.idx64) : r0) : -1};
}

// What a lane holds of one (sequence, v-head): its state values (step it
// covers rows kRowsPerStep * it + 4 * wid + g), its 8 k and q values, the
// v of its rows, alpha and beta.
template <bool BF16, int NW>
struct DecItem {
  static constexpr int kRowsPerStep = 4 * NW;
  static constexpr int kSteps = kDim / kRowsPerStep;
  f32x4 s[kSteps][2];  // fp32 rows
  u32x4 sb[kSteps];    // bf16 rows
  float k8[8], q8[8], vv[kSteps];
  float alpha, bt;
};

// Issues every load of (b, h) with read row rd (-1: zeros): the state first,
// then the token's inputs.
template <bool BF16, int NW>
__device__ __forceinline__ void decode_load(const DecodeParams& p, int b, int h, int64_t rd,
                                            int wid, int g, int c, DecItem<BF16, NW>& d) {
  using D = DecItem<BF16, NW>;
  if (rd >= 0) {
    if constexpr (BF16) {
      const u16* src = (const u16*)p.init + rd * p.init_stride + (int64_t)h * kDim * kDim + 8 * c;
#pragma unroll
      for (int it = 0; it < D::kSteps; ++it)
        d.sb[it] = __builtin_nontemporal_load((const u32x4*)(src + (D::kRowsPerStep * it + 4 * wid + g) * kDim));
    } else {
      const float* src = (const float*)p.init + rd * p.init_stride + (int64_t)h * kDim * kDim + 4 * c;
#pragma unroll
      for (int it = 0; it < D::kSteps; ++it) {
        const int row = D::kRowsPerStep * it + 4 * wid + g;
        d.s[it][0] = __builtin_nontemporal_load((const f32x4*)(src + row * kDim));
        d.s[it][1] = __builtin_nontemporal_load((const f32x4*)(src + row * kDim + 64));
      }
    }
  } else {
#pragma unroll
    for (int it = 0; it < D::kSteps; ++it) {
      d.s[it][0] = d.s[it][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      d.sb[it] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int hq = h / p.group;
  if constexpr (BF16) {
    const u16* kp = p.k + ((int64_t)b * p.Hqk + hq) * kDim + 8 * c;
    const u16* qp = p.q + ((int64_t)b * p.Hqk + hq) * kDim + 8 * c;
    unpack8(*(const u32x4*)kp, d.k8);
    unpack8(*(const u32x4*)qp, d.q8);
  } else {
    const u16* kp = p.k + ((int64_t)b * p.Hqk + hq) * kDim + 4 * c;
    const u16* qp = p.q + ((int64_t)b * p.Hqk + hq) * kDim + 4 * c;
    float t[4];
    unpack4(*(const u32x2*)kp, t);
    for (int i = 0; i < 4; ++i) d.k8[i] = t[i];
    unpack4(*(const u32x2*)(kp + 64), t);
    for (int i = 0; i < 4; ++i) d.k8[4 + i] = t[i];
    unpack4(*(const u32x2*)qp, t);
    for (int i = 0; i < 4; ++i) d.q8[i] = t[i];
    unpack4(*(const u32x2*)(qp + 64), t);
    for (int i = 0; i < 4; ++i) d.q8[4 + i] = t[i];
  }
  const int64_t bh = (int64_t)b * p.H + h;
  d.alpha = p.g ? expf(p.g[bh]) : 1.f;
  d.bt = p.beta ? p.beta[bh] : 1.f;
#pragma unroll
  for (int it = 0; it < D::kSteps; ++it) d.vv[it] = bf2f(p.v[bh * kDim + D::kRowsPerStep * it + 4 * wid + g]);
}

// The update of (b, h) from its loaded values: the new rows to write row wr
// (-1: no store) and o.  Every product-sum is an explicit fused multiply-add,
// so the result does not depend on how the compiler contracts an instance.
template <bool BF16, int NW>
__device__ __forceinline__ void decode_update(const DecodeParams& p, int b, int h, int64_t wr,
                                              const DecItem<BF16, NW>& d, int wid, int g, int c) {
  using D = DecItem<BF16, NW>;
  float kq = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) kq = __builtin_fmaf(d.k8[i], d.q8[i], kq);
  kq = sum16(kq);
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t doff = wr >= 0 ? wr * p.out_stride + (int64_t)h * kDim * kDim : 0;
  float o_mine = 0.f;  // o of row kRowsPerStep*c + 4*wid + g (lanes c < kSteps)
#pragma unroll
  for (int it = 0; it < D::kSteps; ++it) {
    const int row = D::kRowsPerStep * it + 4 * wid + g;
    float sv[8];  // the lane's 8 state values, in k8's order
    if constexpr (BF16) {
      unpack8(d.sb[it], sv);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = d.s[it][i >> 2][i & 3];
    }
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sk = __builtin_fmaf(sv[i], d.k8[i], sk);
      sq = __builtin_fmaf(sv[i], d.q8[i], sq);
    }
    sk = sum16(sk);
    sq = sum16(sq);
    const float delta = d.bt * __builtin_fmaf(-d.alpha, sk, d.vv[it]);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = __builtin_fmaf(d.alpha, sv[i], delta * d.k8[i]);
    if (wr >= 0) {
      if constexpr (BF16) {
        u16* dst = (u16*)p.out + doff + 8 * c;
        __builtin_nontemporal_store(u32x4{f2bf2(y[0], y[1]), f2bf2(y[2], y[3]), f2bf2(y[4], y[5]), f2bf2(y[6], y[7])},
                                    (u32x4*)(dst + row * kDim));
      } else {
        float* dst = (float*)p.out + doff + 4 * c;
        __builtin_nontemporal_store(f32x4{y[0], y[1], y[2], y[3]}, (f32x4*)(dst + row * kDim));
        __builtin_nontemporal_store(f32x4{y[4], y[5], y[6], y[7]}, (f32x4*)(dst + row * kDim + 64));
      }
    }
    if (c == it) o_mine = p.scale * __builtin_fmaf(d.alpha, sq, delta * kq);
  }
  if (c < D::kSteps) p.o[bh * kDim + D::kRowsPerStep * c + 4 * wid + g] = f2bf(o_mine);
}

// One (sequence, v-head) per workgroup.
template <bool BF16, int NW>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeParams p) {
  if (guarded(p.guard)) return;
  const int b = blockIdx.x / p.H, h = blockIdx.x - b * p.H;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g = lane >> 4;  // row within the wave's 4 rows of a step
  const int c = lane & 15;  // k = 4c..4c+3 and 64+4c..64+4c+3 (fp32), 8c..8c+7 (bf16)
  const DecRows r = decode_rows(p, b);
  DecItem<BF16, NW> d;
  decode_load(p, b, h, r.rd, wid, g, c, d);
  decode_update(p, b, h, r.wr, d, wid, g, c);
}

// A fixed grid walking the (sequence, v-head) pairs blockIdx, blockIdx +
// gridDim, ...: the next pair's loads (and the rows of the one after) are
// issued before the current pair is updated, so each workgroup keeps loads
// in flight instead of waiting on its row indices and state at every start.
template <bool BF16, int NW>
__global__ __launch_bounds__(NW * 64) void decode_stream_kernel(const DecodeParams p) {
  const int items = p.num_seqs * p.H;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  int it = blockIdx.x;
  if (it >= items || guarded(p.guard)) return;
  DecRows r0 = decode_rows(p, it / p.H);
  DecItem<BF16, NW> cur;
  decode_load(p, it / p.H, it % p.H, r0.rd, wid, g, c, cur);
  int nx = it + (int)gridDim.x;
  DecRows r1 = nx < items ? decode_rows(p, nx / p.H) : DecRows{-1, -1};
  for (;;) {
    DecItem<BF16, NW> nxt;
    if (nx < items) decode_load(p, nx / p.H, nx % p.H, r1.rd, wid, g, c, nxt);
    const int nx2 = nx + (int)gridDim.x;
    const DecRows r2 = nx2 < items ? decode_rows(p, nx2 / p.H) : DecRows{-1, -1};
    decode_update(p, it / p.H, it % p.H, r0.wr, cur, wid, g, c);
    if (nx >= items) break;
    it = nx;
    nx = nx2;
    r0 = r1;
    r1 = r2;
    cur = nxt;
  }
}

}  // namespace

template <int NW>
hipError_t launch_decode_nw(const DecodeParams& p, unsigned blocks, hipStream_t s) {
  if (p.state_bf16) decode_kernel<true, NW><<<blocks, NW * 64, 0, s>>>(p);
  else decode_kernel<false, NW><<<blocks, NW * 64, 0, s>>>(p);
  return hipGetLastError();
}

// fp32 pools: the streaming kernel with 6 workgroups of 16 waves per compute
// unit, 6.0 TB/s on the hybrid step's decode batch (the one-pair kernel: 5.6;
// 1-12 per unit: 5.75-6.0); the extra workgroups beyond the resident ones
// even out the walk's tail.  bf16 pools (half the bytes a pair): the
// walking kernel with 4 waves and a grid of one workgroup per pair, 5.6
// TB/s; its compiled form keeps a pair's 8 row loads a lane in flight in 175
// VGPRs, 2 workgroups per compute unit (the one-pair kernel: 5.3 with 16
// waves, 5.1-5.4 with 4 or 8; streaming with fewer workgroups than pairs:
// 4.9-5.3).  The shape arguments pick another (tests, tuning); every choice
// gives bit-identical results.
hipError_t launch_decode(const DecodeParams& p, const DecodeShape& shape, hipStream_t s) {
  const int64_t blocks = (int64_t)p.num_seqs * p.H;
  if (blocks <= 0) return hipSuccess;
  if (p.state_bf16 && shape.waves == 0 && shape.stream_per_cu == 0 && shape.stream_grid == 0) {
    decode_stream_kernel<true, 4><<<(unsigned)blocks, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  // a one-pair width asked for alone selects the one-pair kernel
  int per_cu = p.state_bf16 || shape.waves ? 0 : 6;
  if (shape.stream_per_cu > 0) per_cu = shape.stream_per_cu;
  if (shape.stream_per_cu < 0) per_cu = 0;
  int64_t grid = (int64_t)device_cus() * per_cu;
  if (shape.stream_grid > 0) grid = shape.stream_grid;
  if (grid > 0) {
    const unsigned n = (unsigned)std::min<int64_t>(blocks, grid);
    if (p.state_bf16) decode_stream_kernel<true, 16><<<n, 1024, 0, s>>>(p);
    else decode_stream_kernel<false, 16><<<n, 1024, 0, s>>>(p);
    return hipGetLastError();
  }
  switch (shape.waves) {
    case 2: return launch_decode_nw<2>(p, (unsigned)blocks, s);
    case 4: return launch_decode_nw<4>(p, (unsigned)blocks, s);
    case 8: return launch_decode_nw<8>(p, (unsigned)blocks, s);
    default: return launch_decode_nw<16>(p, (unsigned)blocks, s);
  }
}
}  // namespace gdn
