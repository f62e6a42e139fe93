// Chunked Gated Delta-Rule prefill, fused: one workgroup per (sequence, v-head)
// walks the sequence's 64-token chunks, computing each chunk's intra-chunk
// (WY) quantities in LDS and advancing the fp32 state held in MFMA
// accumulators.  Inputs are read once and outputs written once: nothing
// round-trips through memory between the two steps.
//
// Chunks sit at absolute token positions that are multiples of 64, so every
// page boundary (page_size is a multiple of 64) and every checkpoint position
// (checkpoint_every_n_tokens a multiple of 64) is a chunk end; the first chunk
// is padded on the left when the prefix is not a multiple of 64
// (flashinfer.gdn_paged, "Page table").  Rows outside the sequence are
// padding with q = k = v = 0, g = 0 and beta = 0: exact identities.
//
// Within a chunk, with G_i the running sum of g over rows 0..i, gamma_i =
// exp(G_i) and D_ij = exp(G_i - G_j) (i >= j), the token updates
// S_t = alpha_t S_{t-1} + e_t k_t^T with e_t = beta_t (v_t - alpha_t S_{t-1} k_t)
// unroll to
//   E = T diag(beta) (V - diag(gamma) K S0^T),  T = (I + A)^-1,
//                                              A_ij = beta_i D_ij k_i.k_j (i > j)
//   O = scale (diag(gamma) Q S0^T + P E),       P_ij = D_ij q_i.k_j (i >= j)
//   S_end = gamma_last S0 + (diag(exp(G_last - G)) E)^T K
//
// Work split of the 8 waves, per chunk:
//   WY step   K K^T and Q K^T on bf16 MFMA (exact products of bf16 inputs),
//             decay masks, T by blocked forward substitution in fp32 (16x16
//             diagonal blocks, then the off-diagonal blocks), and the T, P and
//             K^T operand fragments for the recurrence (T and P as bf16 hi + lo).
//   recurrence wave w owns state rows v = 16w..16w+15 (rows of S evolve
//             independently); S^T lives in accumulators (lane: column v,
//             rows k), which is the B-operand layout the next chunk needs.
//             fp32 operands are split into bf16 hi + lo so the MFMA products
//             keep ~fp32 accuracy (3 passes when both sides are fp32, 2 when
//             one side is exact bf16).
//   prefetch  the next chunk's K, Q tiles, g, beta and v are loaded into
//             registers while the recurrence runs, then staged into LDS.
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kTileWords = 4 * 4 * kFragElems;  // 64 x 128 bf16, fragment order
constexpr int kKtWordsL = 8 * 2 * kFragElems;   // K^T fragments
constexpr int kMatFrag = 8 * kFragElems;        // one 64x64 operand (8 fragments)

constexpr int kAP = kChunk + 4;  // fp32 row pitch of the 64x64 matrices (16-byte rows)

struct Smem {
  u16 Kf[kTileWords];   // K tile: [row block][k-step][lane][8]
  u16 Qf[kTileWords];   // Q tile, same order
  u16 Ktf[kKtWordsL];   // K^T fragments: [k block][t-step][lane][8]
  u16 Tf[2 * kMatFrag]; // T fragments, hi then lo
  u16 Pf[2 * kMatFrag]; // P fragments, hi then lo
  u16 Vs[kWaves][64][16]; // v tile: wave w's columns, lane's 16 rows 16*mt + 4*gq + r
  float A[kChunk][kAP];   // strictly lower beta_i D_ij k_i.k_j
  float T[kChunk][kAP];   // (I + A)^-1, lower triangle (upper blocks never read)
  float Xs[4][16][17];    // lower-left 32x32 block of A.T during the inverse
  float scal[3][kChunk];  // beta, gamma, exp(G_last - G)
};

// Fragment-ordered 64x128 tile: element (t, k) sits in fragment (t/16, k/32),
// lane (t%16) + 16*gq, slot j, where k%32 = 16*(j/4) + 4*gq + j%4 (perm_row).
// Offset (in bf16 elements) of the 4-run k..k+3 (k % 4 == 0) of row t.
__device__ __forceinline__ int tile_off(int t, int k) {
  const int ks = k >> 5, w = k & 31;
  const int gq = (w & 15) >> 2, jh = w >> 4;
  return (((t >> 4) * 4 + ks) * 64 + (t & 15) + 16 * gq) * 8 + 4 * jh;
}

__device__ __forceinline__ int64_t ld_index(const void* p, int i, int idx64) {
  return idx64 ? ((const int64_t*)p)[i] : (int64_t)((const int32_t*)p)[i];
}

__device__ __forceinline__ void store_state(float* dst, const f32x4 (&accS)[8]) {
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) *(f32x4*)(dst + 16 * mb) = accS[mb];
}

__device__ __forceinline__ void split_rows(const f32x4 (&x)[4], int ks, bf16x8& hi, bf16x8& lo) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = x[2 * ks + (j >> 2)][j & 3];
  split8(v, hi, lo);
}

// Next chunk's inputs, held in registers while the current chunk computes.
struct Prefetch {
  u32x4 kq[4];  // two 16-byte pieces of the K tile, two of the Q tile
  u32x4 v[2];   // two 16-byte pieces of the v tile
  float g, b;   // row = lane
};

struct Seq {
  int tok0, L, hq, h;
};

// Issue the loads of a chunk whose row 0 is new token n0.  Rows outside the
// sequence read token 0 of the sequence (always in bounds); their values are
// replaced by zeros where they are consumed, so nothing here waits on memory.
__device__ __forceinline__ void load_chunk(Prefetch& pf, const PrefillParams& p, const Seq& s,
                                           int n0, int tid, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int it = tid + kThreads * i;
    const int row = it >> 4, seg = it & 15;
    const int n = n0 + row;
    const bool valid = (unsigned)n < (unsigned)s.L;
    const int64_t tok = (int64_t)s.tok0 + (valid ? n : 0);
    const int64_t off = (tok * p.Hqk + s.hq) * kDim + seg * 8;
    pf.kq[i] = *(const u32x4*)(p.k + off);
    pf.kq[2 + i] = *(const u32x4*)(p.q + off);
    pf.v[i] = *(const u32x4*)(p.v + (tok * p.H + s.h) * kDim + seg * 8);
  }
  const int n = n0 + lane;
  const bool valid = (unsigned)n < (unsigned)s.L;
  const int64_t t = ((int64_t)s.tok0 + (valid ? n : 0)) * p.H + s.h;
  pf.g = p.g ? p.g[t] : 0.f;
  pf.b = p.beta ? p.beta[t] : 1.f;
}

__device__ __forceinline__ void store_tiles(const Prefetch& pf, Smem& sm, const Seq& s, int n0,
                                            int tid) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int it = tid + kThreads * i;
    const int row = it >> 4, seg = it & 15, k0 = seg * 8;
    const bool valid = (unsigned)(n0 + row) < (unsigned)s.L;
    const u32x4 kv = valid ? pf.kq[i] : z;
    const u32x4 qv = valid ? pf.kq[2 + i] : z;
    const u32x4 vv = valid ? pf.v[i] : z;
    *(u32x2*)&sm.Kf[tile_off(row, k0)] = u32x2{kv.x, kv.y};
    *(u32x2*)&sm.Kf[tile_off(row, k0 + 4)] = u32x2{kv.z, kv.w};
    *(u32x2*)&sm.Qf[tile_off(row, k0)] = u32x2{qv.x, qv.y};
    *(u32x2*)&sm.Qf[tile_off(row, k0 + 4)] = u32x2{qv.z, qv.w};
    // v: columns seg*8 .. seg*8+7 of token row `row` go to wave seg/2, lanes
    // 8*(seg&1) + c + 16*gq, slot 4*mt + r (row = 16*mt + 4*gq + r)
    const int w = seg >> 1;
    const int lbase = 8 * (seg & 1) + 16 * ((row & 15) >> 2);
    const int slot = 4 * (row >> 4) + (row & 3);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t word = vv[c >> 1];
      sm.Vs[w][lbase + c][slot] = u16((c & 1) ? (word >> 16) : (word & 0xffffu));
    }
  }
}

// hi/lo 3-pass product of two fp32 operand fragments (~fp32 accuracy)
__device__ __forceinline__ f32x4 mma3(const float (&a)[8], const float (&b)[8], f32x4 c) {
  bf16x8 ah, al, bh, bl;
  split8(a, ah, al);
  split8(b, bh, bl);
  c = mfma16x16x32(ah, bh, c);
  c = mfma16x16x32(ah, bl, c);
  c = mfma16x16x32(al, bh, c);
  return c;
}

__device__ __forceinline__ bf16x8 lds_frag(const u16* base, int frag, int lane) {
  return *(const bf16x8*)(base + (frag * 64 + lane) * 8);
}

// Lower-triangle block pair (i >= j) number blk (0..9) of the 4x4 block grid.
__device__ __forceinline__ int tri_i(int blk) { return blk >= 6 ? 3 : blk >= 3 ? 2 : blk >= 1 ? 1 : 0; }
__device__ __forceinline__ int tri_j(int blk) { const int i = tri_i(blk); return blk - i * (i + 1) / 2; }

__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int n16 = lane & 15, gq = lane >> 4;

  // Longest sequences first: blockIdx walks p.order (sorted by chunk count).
  const int item = blockIdx.x;
  const int b = p.order[item / p.H];
  Seq s;
  s.h = item - (item / p.H) * p.H;
  s.tok0 = p.cu_seqlens[b];
  s.L = p.cu_seqlens[b + 1] - s.tok0;
  if (s.L <= 0) return;  // a zero-length sequence writes nothing
  s.hq = s.h / p.group;
  const int pre = p.slots.prefix[b];
  const int nch = ((pre & (kChunk - 1)) + s.L + kChunk - 1) / kChunk;
  const int rd = p.slots.read[b];
  const int wr = p.slots.write[b];
  const int vrow = 16 * wid + n16;
  const int64_t head_off = ((int64_t)s.h * kDim + vrow) * kDim + 4 * gq;

  f32x4 accS[8];
  if (rd >= 0 && p.init) {
    const float* src = p.init + (int64_t)rd * p.init_stride + head_off;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) accS[mb] = *(const f32x4*)(src + 16 * mb);
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) accS[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  Prefetch pf;
  load_chunk(pf, p, s, (pre & ~(kChunk - 1)) - pre, tid, lane);
  store_tiles(pf, sm, s, (pre & ~(kChunk - 1)) - pre, tid);
  __syncthreads();

  for (int ci = 0; ci < nch; ++ci) {
    const int n0 = (pre & ~(kChunk - 1)) + kChunk * ci - pre;  // new-token index of row 0

    // ================= WY step =================
    // running log2-decay, every wave keeps it in registers (lane = row)
    const bool row_valid = (unsigned)(n0 + lane) < (unsigned)s.L;
    float G = row_valid ? pf.g * kLog2e : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(G, off, 64);
      if (lane >= off) G += y;
    }
    const float bet = row_valid ? pf.b : 0.f;
    if (wid == 0) {
      const float Glast = __shfl(G, 63, 64);
      sm.scal[0][lane] = bet;
      sm.scal[1][lane] = exp2f(G);
      sm.scal[2][lane] = exp2f(Glast - G);
    }

    if (wid < 4) {
      // K K^T lower blocks -> A (fp32), masked, decayed, scaled by beta_row
      for (int blk = wid; blk < 10; blk += 4) {
        const int bi = tri_i(blk), bj = tri_j(blk);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = mfma16x16x32(lds_frag(sm.Kf, bi * 4 + ks, lane), lds_frag(sm.Kf, bj * 4 + ks, lane), acc);
        const int col = 16 * bj + n16;
        const float Gc = __shfl(G, col, 64);
        // shuffles stay outside the masks: a lane-divergent bpermute reads 0
        // from inactive source lanes
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * bi + 4 * gq + r;
          const float Gr = __shfl(G, row, 64);
          const float br = __shfl(bet, row, 64);
          const float val = br * exp2f(Gr - Gc) * acc[r];
          sm.A[row][col] = row > col ? val : 0.f;
        }
      }
    } else {
      // P^T blocks (K rows x Q rows): the accumulator of block (t-block bt,
      // s-block bs) holds, in lane (t, gq), P[16bt + t][16bs + 4gq + r] -- exactly
      // slots 4*(bs&1) + r of P fragment (bt, bs/2).  Written hi/lo, no transpose.
      const int bt = wid - 4;
      const int t = 16 * bt + n16;
      const float Gt = __shfl(G, t, 64);
#pragma unroll
      for (int bs = 0; bs < 4; ++bs) {
        uint32_t hw[2] = {0u, 0u}, lw[2] = {0u, 0u};
        if (bs <= bt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc = mfma16x16x32(lds_frag(sm.Kf, bs * 4 + ks, lane), lds_frag(sm.Qf, bt * 4 + ks, lane), acc);
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int sr = 16 * bs + 4 * gq + r;
            const float Gs = __shfl(G, sr, 64);
            const float val = exp2f(Gt - Gs) * acc[r];
            v[r] = t >= sr ? val : 0.f;
          }
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint32_t w = f2bf2(v[2 * i], v[2 * i + 1]);
            hw[i] = w;
            lw[i] = f2bf2(v[2 * i] - __uint_as_float(w << 16), v[2 * i + 1] - __uint_as_float(w & 0xffff0000u));
          }
        }
        const int f = bt * 2 + (bs >> 1);
        *(u32x2*)&sm.Pf[(f * 64 + lane) * 8 + 4 * (bs & 1)] = u32x2{hw[0], hw[1]};
        *(u32x2*)&sm.Pf[kMatFrag + (f * 64 + lane) * 8 + 4 * (bs & 1)] = u32x2{lw[0], lw[1]};
      }
    }
    // the next chunk's inputs load while this one computes (issued after the
    // Gram products so no register reload there waits behind them)
    if (ci + 1 < nch) load_chunk(pf, p, s, n0 + kChunk, tid, lane);
    // K^T fragments: K[t][k] gathered from the fragment-ordered K tile
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int it = tid + kThreads * i;
      const int frag = it >> 6, ln = it & 63;
      const int mk = frag >> 1, ks = frag & 1;
      const int kcol = 16 * mk + (ln & 15), g4 = ln >> 4;
      const int kin = tile_off(0, kcol & ~3) + (kcol & 3);  // offset of (row 0, kcol)
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t0 = perm_row(ks, g4, 2 * e), t1 = perm_row(ks, g4, 2 * e + 1);
        const u16 a0 = sm.Kf[kin + ((t0 >> 4) * 4 * 64 + (t0 & 15)) * 8];
        const u16 a1 = sm.Kf[kin + ((t1 >> 4) * 4 * 64 + (t1 & 15)) * 8];
        w[e] = pack2(a0, a1);
      }
      *(u32x4*)&sm.Ktf[(frag * 64 + ln) * 8] = w;
    }
    __syncthreads();

    // ---- T = (I + A)^-1.  Diagonal 16x16 blocks by forward substitution
    // (wave 0, lane = (block, column)), short dependency chains.
    if (wid == 0) {
      const int dblk = lane >> 4, col = lane & 15;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < i; ++j) part[j & 3] += sm.A[16 * dblk + i][16 * dblk + j] * x[j];
        x[i] = (i == col ? 1.f : 0.f) - ((part[0] + part[1]) + (part[2] + part[3]));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.T[16 * dblk + i][16 * dblk + col] = x[i];
    }
    __syncthreads();

    // Off-diagonal blocks by doubling, on MFMA with hi/lo splits:
    //   T_10 = -T_11 A_10 T_00,  T_32 = -T_33 A_32 T_22            (waves 0, 1)
    //   X = A[32:64, 0:32] T[0:32, 0:32]                          (waves 0-3)
    //   T[32:64, 0:32] = -T[32:64, 32:64] X                        (waves 0-3)
    // Operand slots follow perm_row; a 16-deep product leaves slots 4..7 zero.
    if (wid < 2) {
      const int I = 1 + 2 * wid, J = I - 1;
      float a[8], bb[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = sm.A[16 * I + n16][16 * J + 4 * gq + j];
        bb[j] = sm.T[16 * J + 4 * gq + j][16 * J + n16];
        a[j + 4] = 0.f;
        bb[j + 4] = 0.f;
      }
      const f32x4 X = mma3(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = sm.T[16 * I + n16][16 * I + 4 * gq + j];
        bb[j] = X[j];
      }
      const f32x4 Y = mma3(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.T[16 * I + 4 * gq + r][16 * J + n16] = -Y[r];
    }
    __syncthreads();
    if (wid < 4) {
      const int I = 2 + (wid >> 1), J = wid & 1;
      float a[8], bb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = perm_row(0, gq, j);  // 0..31 over column blocks 0, 1
        const bool use = J == 0 || kk >= 16;  // T_01 = 0
        a[j] = use ? sm.A[16 * I + n16][kk] : 0.f;
        bb[j] = use ? sm.T[kk][16 * J + n16] : 0.f;
      }
      const f32x4 X = mma3(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.Xs[wid][4 * gq + r][n16] = X[r];
    }
    __syncthreads();
    if (wid < 4) {
      const int I = 2 + (wid >> 1), J = wid & 1;
      float a[8], bb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = perm_row(0, gq, j);  // 0..31 over rows/columns 32..63
        const bool use = I == 3 || kk < 16;  // T_23 = 0
        a[j] = use ? sm.T[16 * I + n16][32 + kk] : 0.f;
        bb[j] = use ? sm.Xs[(kk >> 4) * 2 + J][kk & 15][n16] : 0.f;
      }
      const f32x4 Y = mma3(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.T[16 * I + 4 * gq + r][16 * J + n16] = -Y[r];
    }
    __syncthreads();

    // T fragments (hi/lo), one (fragment, lane) per thread
    {
      const int frag = tid >> 6, ln = tid & 63;
      const int mt = frag >> 1, ks = frag & 1;
      const int row = 16 * mt + (ln & 15), g4 = ln >> 4;
      float vals[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = perm_row(ks, g4, j);
        vals[j] = c <= row ? sm.T[row][c] : 0.f;
      }
      bf16x8 hi, lo;
      split8(vals, hi, lo);
      *(bf16x8*)&sm.Tf[(frag * 64 + ln) * 8] = hi;
      *(bf16x8*)&sm.Tf[kMatFrag + (frag * 64 + ln) * 8] = lo;
    }
    __syncthreads();

    // ================= recurrence =================

    // Y = K S^T, Z = Q S^T
    bf16x8 Shi[4], Slo[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = accS[2 * ks + (j >> 2)][j & 3];
      split8(v, Shi[ks], Slo[ks]);
    }
    // Y = K S^T, then R = beta (V - gamma Y)
    f32x4 R[4];
    {
      const u32x4 va = *(const u32x4*)&sm.Vs[wid][lane][0];
      const u32x4 vb = *(const u32x4*)&sm.Vs[wid][lane][8];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 ak = lds_frag(sm.Kf, mt * 4 + ks, lane);
          y = mfma16x16x32(ak, Shi[ks], y);
          y = mfma16x16x32(ak, Slo[ks], y);
        }
        const f32x4 bt = *(const f32x4*)&sm.scal[0][16 * mt + 4 * gq];
        const f32x4 gm = *(const f32x4*)&sm.scal[1][16 * mt + 4 * gq];
        const uint32_t w0 = mt < 2 ? va[2 * mt] : vb[2 * mt - 4];
        const uint32_t w1 = mt < 2 ? va[2 * mt + 1] : vb[2 * mt - 3];
        const float vx[4] = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xffff0000u),
                             __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xffff0000u)};
#pragma unroll
        for (int r = 0; r < 4; ++r) R[mt][r] = bt[r] * (vx[r] - gm[r] * y[r]);
      }
    }

    // E = T R
    f32x4 E[4];
    {
      bf16x8 Rhi[2], Rlo[2];
      split_rows(R, 0, Rhi[0], Rlo[0]);
      split_rows(R, 1, Rhi[1], Rlo[1]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        E[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int f = mt * 2 + ks;
          const bf16x8 th = lds_frag(sm.Tf, f, lane);
          const bf16x8 tl = lds_frag(sm.Tf + kMatFrag, f, lane);
          E[mt] = mfma16x16x32(th, Rhi[ks], E[mt]);
          E[mt] = mfma16x16x32(th, Rlo[ks], E[mt]);
          E[mt] = mfma16x16x32(tl, Rhi[ks], E[mt]);
        }
      }
    }

    // O = scale (gamma Q S^T + P E), stored row by row block
    {
      bf16x8 Ehi[2], Elo[2];
      split_rows(E, 0, Ehi[0], Elo[0]);
      split_rows(E, 1, Ehi[1], Elo[1]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 aq = lds_frag(sm.Qf, mt * 4 + ks, lane);
          z = mfma16x16x32(aq, Shi[ks], z);
          z = mfma16x16x32(aq, Slo[ks], z);
        }
        const f32x4 gm = *(const f32x4*)&sm.scal[1][16 * mt + 4 * gq];
        f32x4 O;
#pragma unroll
        for (int r = 0; r < 4; ++r) O[r] = gm[r] * z[r];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int f = mt * 2 + ks;
          const bf16x8 ph = lds_frag(sm.Pf, f, lane);
          const bf16x8 pl = lds_frag(sm.Pf + kMatFrag, f, lane);
          O = mfma16x16x32(ph, Ehi[ks], O);
          O = mfma16x16x32(ph, Elo[ks], O);
          O = mfma16x16x32(pl, Ehi[ks], O);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + 16 * mt + 4 * gq + r;
          if ((unsigned)n < (unsigned)s.L)
            p.o[(((int64_t)s.tok0 + n) * p.H + s.h) * kDim + vrow] = f2bf(p.scale * O[r]);
        }
      }
    }

    // S <- gamma_last S + (dec E)^T K
    {
      const float gC = sm.scal[1][kChunk - 1];
      f32x4 Ed[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 dc = *(const f32x4*)&sm.scal[2][16 * mt + 4 * gq];
#pragma unroll
        for (int r = 0; r < 4; ++r) Ed[mt][r] = dc[r] * E[mt][r];
      }
      bf16x8 Dhi[2], Dlo[2];
      split_rows(Ed, 0, Dhi[0], Dlo[0]);
      split_rows(Ed, 1, Dhi[1], Dlo[1]);
#pragma unroll
      for (int mk = 0; mk < 8; ++mk) {
        accS[mk] = accS[mk] * gC;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 kt = lds_frag(sm.Ktf, mk * 2 + ks, lane);
          accS[mk] = mfma16x16x32(kt, Dhi[ks], accS[mk]);
          accS[mk] = mfma16x16x32(kt, Dlo[ks], accS[mk]);
        }
      }
    }

    // checkpoint at this chunk's end?
    if (p.ckpt_idx) {
      const int pos = (pre & ~(kChunk - 1)) + kChunk * (ci + 1);
      if (pos % p.ckpt_every == 0 && pos > pre && pos <= pre + s.L) {
        const int j = pos / p.ckpt_every - pre / p.ckpt_every - 1;
        const int64_t row = ld_index(p.ckpt_idx, p.slots.ckpt_start[b] + j, p.ckpt_idx64);
        if (row >= 0) store_state(p.ckpt + row * p.ckpt_stride + head_off, accS);
      }
    }
    __syncthreads();  // every wave is done with this chunk's LDS operands
    if (ci + 1 < nch) {
      store_tiles(pf, sm, s, n0 + kChunk, tid);
      __syncthreads();
    }
  }
  if (wr >= 0 && p.out) store_state(p.out + (int64_t)wr * p.out_stride + head_off, accS);
}

// Longest-first order of the sequences (by chunk count; ties by index).
__global__ __launch_bounds__(1024) void order_kernel(const int32_t* __restrict__ cu,
                                                     const int32_t* __restrict__ prefix, int B,
                                                     int32_t* __restrict__ order) {
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int L = cu[b + 1] - cu[b];
    const int nb = L > 0 ? ((prefix[b] & (kChunk - 1)) + L + kChunk - 1) / kChunk : 0;
    int rank = 0;
    for (int o = 0; o < B; ++o) {
      const int Lo = cu[o + 1] - cu[o];
      const int no = Lo > 0 ? ((prefix[o] & (kChunk - 1)) + Lo + kChunk - 1) / kChunk : 0;
      rank += (no > nb) || (no == nb && o < b);
    }
    order[rank] = b;
  }
}

}  // namespace

size_t prefill_lds_bytes() { return sizeof(Smem); }

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.num_seqs * p.H;
  if (blocks <= 0) return hipSuccess;
  order_kernel<<<1, 1024, 0, s>>>(p.cu_seqlens, p.slots.prefix, p.num_seqs, (int32_t*)p.order);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static bool attr_set = false;  // raised once per process; idempotent if raced
  if (!attr_set) {
    e = hipFuncSetAttribute((const void*)prefill_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  prefill_kernel<<<(unsigned)blocks, kThreads, sizeof(Smem), s>>>(p);
  return hipGetLastError();
}

}  // namespace gdn
