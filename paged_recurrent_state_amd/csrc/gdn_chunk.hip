// Intra-chunk step of chunked Gated Delta-Rule prefill (one workgroup per
// 64-token chunk and v-head; all chunks of the batch in parallel).
//
// Chunks sit at absolute token positions that are multiples of 64, so that
// every page boundary is a chunk end (flashinfer.gdn_paged, "Page table":
// page_size is a multiple of 64 and the kernels pad the first chunk on the
// left when the prefix is not).  Rows outside the sequence are padding with
// q = k = v = 0, g = 0 and beta = 0: exact identities of the recurrence.
//
// Within a chunk, with G_i the running sum of g over rows 0..i, gamma_i =
// exp(G_i) and D_ij = exp(G_i - G_j) for i >= j, the per-token updates
// S_t = alpha_t S_{t-1} + e_t k_t^T,  e_t = beta_t (v_t - alpha_t S_{t-1} k_t)
// unroll to
//   (I + A) E = diag(beta) (V - diag(gamma) K S0^T),   A_ij = beta_i D_ij k_i.k_j (i > j)
//   O = diag(gamma) Q S0^T + P E,                     P_ij = D_ij q_i.k_j (i >= j)
//   S_end = gamma_last S0 + (diag(exp(G_last - G)) E)^T K
// This kernel produces everything that does not depend on S0: T = (I + A)^-1,
// P, beta, gamma and exp(G_last - G), and a transposed copy of K, laid out as
// ready-to-load MFMA operand fragments for the recurrence kernel.
//
// K K^T and Q K^T are exact bf16 products on MFMA (v_mfma_f32_16x16x32_bf16);
// the triangular inverse runs in fp32 on the vector ALUs (blocked forward
// substitution over 16x16 blocks).  T and P are stored as bf16 hi + lo pairs
// so the recurrence keeps ~fp32 accuracy on MFMA.
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kKPad = kDim + 8;    // bf16 row pitch of the K / Q tiles in LDS
constexpr int kAPad = kChunk + 1;  // fp32 row pitch of the 64x64 matrices

struct ChunkSmem {
  u16 K[kChunk][kKPad];
  union {
    u16 Q[kChunk][kKPad];  // dead after the Gram products
    float T[kChunk][kAPad];
  } u;
  float A[kChunk][kAPad];
  float P[kChunk][kAPad];
  float X[3][16][17];
  float G[kChunk];
  float beta[kChunk];
  int meta[4];
};

// Lower-triangle block pairs (i >= j) of a 4x4 block grid.
__constant__ int kTriI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kTriJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

__global__ __launch_bounds__(kThreads) void chunk_kernel(const ChunkParams p) {
  __shared__ __align__(16) ChunkSmem sm;
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;

  // ---- which sequence owns chunk slot c (one round of parallel loads)
  if (tid == 0) sm.meta[0] = -1;
  __syncthreads();
  for (int b = tid; b < p.num_seqs; b += kThreads) {
    const int cs = p.slots.chunk_start[b];
    if (cs <= c) {
      const int t0 = p.cu_seqlens[b];
      const int L = p.cu_seqlens[b + 1] - t0;
      const int pre = p.slots.prefix[b];
      const int n = L > 0 ? ((pre & (kChunk - 1)) + L + kChunk - 1) / kChunk : 0;
      if (c < cs + n) {
        sm.meta[0] = b;
        sm.meta[1] = (pre & ~(kChunk - 1)) + kChunk * (c - cs) - pre;  // row 0 -> new token idx
        sm.meta[2] = L;
        sm.meta[3] = t0;
      }
    }
  }
  __syncthreads();
  if (sm.meta[0] < 0) return;  // slot beyond this batch's chunks (uniform exit)
  const int n0 = sm.meta[1];
  const int L = sm.meta[2];
  const int tok0 = sm.meta[3];
  const int hq = h / p.group;
  const int64_t ch = (int64_t)c * p.H + h;

  // ---- decay and beta; lane = row of the chunk
  if (wid == 0) {
    const int n = n0 + lane;
    const bool valid = n >= 0 && n < L;
    const int64_t t = (int64_t)tok0 + n;
    float gi = 0.f, bi = 0.f;
    if (valid) {
      gi = p.g ? p.g[t * p.H + h] : 0.f;
      bi = p.beta ? p.beta[t * p.H + h] : 1.f;
    }
    // running sum in log2 units, so every decay factor is one native exp2
    float G = gi * 1.4426950408889634f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(G, off, 64);
      if (lane >= off) G += y;
    }
    const float Glast = __shfl(G, 63, 64);
    sm.G[lane] = G;
    sm.beta[lane] = bi;
    float* sc = p.ws.scal + ch * kScal;
    sc[lane] = bi;
    sc[kChunk + lane] = exp2f(G);
    sc[2 * kChunk + lane] = exp2f(Glast - G);
  }

  // ---- K and Q tiles -> LDS, zero rows outside the sequence
  for (int it = tid; it < kChunk * (kDim / 8); it += kThreads) {
    const int row = it >> 4;
    const int seg = it & 15;
    const int n = n0 + row;
    u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
    if (n >= 0 && n < L) {
      const int64_t off = (((int64_t)tok0 + n) * p.Hqk + hq) * kDim + seg * 8;
      kv = *(const u32x4*)(p.k + off);
      qv = *(const u32x4*)(p.q + off);
    }
    *(u32x4*)&sm.K[row][seg * 8] = kv;
    *(u32x4*)&sm.u.Q[row][seg * 8] = qv;
  }
  __syncthreads();

  // ---- Gram blocks on MFMA: A from K K^T, P from Q K^T (lower blocks only)
  const int n16 = lane & 15;
  const int gq = lane >> 4;
  for (int job = wid; job < 20; job += 4) {
    const int which = job >= 10;
    const int blk = job - 10 * which;
    const int bi = kTriI[blk], bj = kTriJ[blk];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u16* arow = which ? &sm.u.Q[16 * bi + n16][0] : &sm.K[16 * bi + n16][0];
      const bf16x8 a = as_bf16x8(*(const u32x4*)(arow + 32 * ks + 8 * gq));
      const bf16x8 bb = as_bf16x8(*(const u32x4*)(&sm.K[16 * bj + n16][32 * ks + 8 * gq]));
      acc = mfma16x16x32(a, bb, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * bi + 4 * gq + r;
      const int col = 16 * bj + n16;
      const float d = exp2f(sm.G[row] - sm.G[col]);
      if (which)
        sm.P[row][col] = row >= col ? d * acc[r] : 0.f;
      else
        sm.A[row][col] = row > col ? sm.beta[row] * d * acc[r] : 0.f;
    }
  }
  __syncthreads();

  if (wid == 0) {
    // ---- inverses of the four 16x16 diagonal blocks of I + A (one column per lane)
    const int d = lane >> 4, col = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == col) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j) s -= sm.A[16 * d + i][16 * d + j] * x[j];
      x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.u.T[16 * d + i][16 * d + col] = x[i];
  } else {
    // ---- meanwhile: P fragments (hi/lo) and the transposed-K fragments
    const int t2 = tid - 64;
    u16* Pw = p.ws.P + ch * kMatWords;
    for (int it = t2; it < kTFragsPerMat * 64; it += kThreads - 64) {
      const int frag = it >> 6, ln = it & 63;
      const int mt = frag >> 1, ks = frag & 1;
      const int row = 16 * mt + (ln & 15), g4 = ln >> 4;
      float vals[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = perm_row(ks, g4, j);
        vals[j] = s <= row ? sm.P[row][s] : 0.f;
      }
      bf16x8 hi, lo;
      split8(vals, hi, lo);
      *(bf16x8*)(Pw + (frag * 64 + ln) * 8) = hi;
      *(bf16x8*)(Pw + kTFragsPerMat * kFragElems + (frag * 64 + ln) * 8) = lo;
    }
    if (h % p.group == 0) {
      u16* Kw = p.ws.Kt + ((int64_t)c * p.Hqk + hq) * kKtWords;
      for (int it = t2; it < kKtFrags * 64; it += kThreads - 64) {
        const int frag = it >> 6, ln = it & 63;
        const int mk = frag >> 1, ks = frag & 1;
        const int col = 16 * mk + (ln & 15), g4 = ln >> 4;
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = pack2(sm.K[perm_row(ks, g4, 2 * i)][col], sm.K[perm_row(ks, g4, 2 * i + 1)][col]);
        *(u32x4*)(Kw + (frag * 64 + ln) * 8) = w;
      }
    }
  }
  __syncthreads();

  // ---- off-diagonal blocks: T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj
  for (int dist = 1; dist < 4; ++dist) {
    const int nb = 4 - dist;
    for (int it = tid; it < nb * 256; it += kThreads) {
      const int j = it >> 8, e = it & 255, r = e >> 4, cc = e & 15;
      const int i = j + dist;
      float s = 0.f;
      for (int m = j; m < i; ++m) {
#pragma unroll
        for (int q = 0; q < 16; ++q) s += sm.A[16 * i + r][16 * m + q] * sm.u.T[16 * m + q][16 * j + cc];
      }
      sm.X[j][r][cc] = s;
    }
    __syncthreads();
    for (int it = tid; it < nb * 256; it += kThreads) {
      const int j = it >> 8, e = it & 255, r = e >> 4, cc = e & 15;
      const int i = j + dist;
      float s = 0.f;
      for (int q = 0; q <= r; ++q) s += sm.u.T[16 * i + r][16 * i + q] * sm.X[j][q][cc];
      sm.u.T[16 * i + r][16 * j + cc] = -s;
    }
    __syncthreads();
  }

  // ---- T fragments (hi/lo)
  u16* Tw = p.ws.T + ch * kMatWords;
  for (int it = tid; it < kTFragsPerMat * 64; it += kThreads) {
    const int frag = it >> 6, ln = it & 63;
    const int mt = frag >> 1, ks = frag & 1;
    const int row = 16 * mt + (ln & 15), g4 = ln >> 4;
    float vals[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = perm_row(ks, g4, j);
      vals[j] = s <= row ? sm.u.T[row][s] : 0.f;
    }
    bf16x8 hi, lo;
    split8(vals, hi, lo);
    *(bf16x8*)(Tw + (frag * 64 + ln) * 8) = hi;
    *(bf16x8*)(Tw + kTFragsPerMat * kFragElems + (frag * 64 + ln) * 8) = lo;
  }
}

}  // namespace

hipError_t launch_chunk(const ChunkParams& p, int64_t num_chunk_slots, hipStream_t s) {
  if (num_chunk_slots <= 0) return hipSuccess;
  dim3 grid((unsigned)num_chunk_slots, (unsigned)p.H);
  chunk_kernel<<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace gdn
