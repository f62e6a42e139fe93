// Chunked Gated Delta-Rule prefill on gfx950, in two kernels.
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
// plan_kernel: the longest-first sequence order, a table from chunk slot to
//   (sequence, row-0 token) and a zeroed row that padding rows read.
// wy_kernel (all chunks of the batch in parallel, one workgroup per chunk and
//   v-head): K K^T on bf16 MFMA (exact products of bf16 inputs), the decay
//   mask, and T by forward substitution in fp32 on the 16x16 diagonal blocks
//   plus a two-level doubling on MFMA (hi/lo bf16 splits) for the
//   off-diagonal blocks.  T diag(beta) leaves as ready-to-load MFMA fragments
//   (hi and lo bf16 halves; the all-zero ones dropped, the two half-empty
//   ones packed into one), with the per-row scalars beta, G, gamma and
//   exp(G_last - G).
// rec_kernel (one workgroup per (sequence, v-head), longest sequences first):
//   walks the chunks in order.  Per chunk, the P = D * (Q K^T) fragments come
//   straight out of MFMA accumulators (computed as P^T blocks), K^T fragments
//   come from K fragments times a 0/1 selection operand, and eight waves each
//   advance 16 rows of the state, whose fp32 transpose lives in MFMA
//   accumulators (the layout the next chunk's B operand needs).  The
//   products that feed the state keep ~2^-17 relative accuracy by splitting
//   fp32 operands into bf16 hi + lo (3 passes when both sides are fp32, 2
//   when one side is exact bf16): E = T R and the state update.  Y = K S^T
//   and the output-only products (Z = S Q^T, P E) take S and E rounded to
//   bf16 in one pass.
//   The next chunk's tiles load straight from global memory into
//   double-buffered LDS while the current one computes.
#include <atomic>

#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// chunk decay exp(G_last) above which Y = K S^T takes a second (lo) pass
constexpr float kYLoGamma = 0x1p-10f;
// A first-pass transition M whose spectral norm is below 2^-300 leaves no
// trace on a start state: a state's Frobenius norm is below 2^135 in fp32,
// so start * M is below 2^-165, under the smallest fp32 denormal.
constexpr float kSkipLog2 = -300.f;
constexpr int kTileWords = 4 * 4 * kFragElems;  // 64 x 128 bf16, fragment order
constexpr int kKtWordsL = 8 * 2 * kFragElems;   // K^T fragments
constexpr int kMatFrag = 8 * kFragElems;        // one 64x64 operand (8 fragments)

// T is lower triangular: of its 8 operand fragments (row block mt, k-step
// ks) the two with mt < 2, ks = 1 are zero, and two more, (0, 0) and (2, 1),
// are zero in slots 4..7 of every lane (the blocks above the diagonal).  The
// record keeps 5: (0, 0) and (2, 1) share fragment 0 (slots 0..3 of each),
// then (1, 0), (2, 0), (3, 0), (3, 1); hi halves then lo halves.
constexpr int kTFrags = 5;
static_assert(kRecWords == 2 * kTFrags * kFragElems, "T record size");
// operand slot of nonzero fragment (mt, ks) in the unpacked set of 6
__device__ __forceinline__ int t_slot(int mt, int ks) { return mt < 2 ? mt : 2 * mt - 2 + ks; }

// The 6 nonzero operand fragments of T from the record's 5: slots 0 and 3
// take their nonzero halves out of fragment 0.
__device__ __forceinline__ void unpack_t(const bf16x8 (&r)[kTFrags], bf16x8 (&t)[6]) {
  const u32x4 w = __builtin_bit_cast(u32x4, r[0]);
  t[0] = as_bf16x8(u32x4{w[0], w[1], 0u, 0u});
  t[1] = r[1];
  t[2] = r[2];
  t[3] = as_bf16x8(u32x4{w[2], w[3], 0u, 0u});
  t[4] = r[3];
  t[5] = r[4];
}

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

__device__ __forceinline__ void split_rows(const f32x4 (&x)[4], int ks, bf16x8& hi, bf16x8& lo) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = x[2 * ks + (j >> 2)][j & 3];
  split8(v, hi, lo);
}

// the same fragment rounded to bf16 (operand of an output-only product)
__device__ __forceinline__ bf16x8 round_rows(const f32x4 (&x)[4], int ks) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = f2bf2(x[2 * ks + (i >> 1)][2 * (i & 1)], x[2 * ks + (i >> 1)][2 * (i & 1) + 1]);
  return as_bf16x8(w);
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

// v-head of the j-th block of a sequence (or chunk).  Workgroups go to the
// 8 XCDs round-robin by block index, so the g = H / Hqk v-heads that read the
// same q/k head are placed 8 blocks apart: same XCD (and L2), dispatched
// close together, so the second read of q and k hits in L2.  When H is not a
// multiple of 8g the order is the identity.
__device__ __forceinline__ int head_of(int j, int H, int g) {
  if (g == 1 || H % (8 * g) != 0) return j;
  const int qk = 8 * (j / (8 * g)) + (j & 7);
  return qk * g + (j >> 3) % g;
}

__device__ __forceinline__ int chunks_of(int prefix, int L) {
  return L > 0 ? ((prefix & (kChunk - 1)) + L + kChunk - 1) / kChunk : 0;
}

// The 64x128 bf16 token tiles are row-major in 16-byte units (8
// consecutive k), unit k8 of row t at position t*16 + (k8 ^ (t % 16)): four
// whole rows fill the 1 KiB that one global->LDS load writes (lane l to
// position 64j + l), and each 16-lane group of an MFMA operand read (16
// consecutive t, one k8) covers all 16 four-bank groups of the 64 banks.  The state's k index is
// relabelled to match the operand layout: accumulator block mb, lane group
// gq, row r holds k = 32*(mb/2) + 8*gq + 4*(mb%2) + r, so blocks 2ks and
// 2ks+1 of a lane are exactly the 8 consecutive k its B operand needs for
// k-step ks.
__device__ __forceinline__ int tile_pos(int t, int k8) { return t * 16 + (k8 ^ (t & 15)); }

// operand fragment f: lane (tt, gq) gets row 16*(f/4) + tt, k = 32*(f%4) + 8*gq ..
__device__ __forceinline__ bf16x8 tile_frag(const u16* base, int f, int lane) {
  return *(const bf16x8*)(base + tile_pos(16 * (f >> 2) + (lane & 15), 4 * (f & 3) + (lane >> 4)) * 8);
}

struct Seq {
  int tok0, L, hq, h;
};

// One 16-byte global->LDS load a lane: lane l's bytes land at byte 16*l of
// the instruction's 1 KiB destination block (M0 holds its LDS address).
// Issued as inline assembly: these loads retire through the vector-memory
// counter only, and hidden from the compiler they do not make it drain
// every outstanding LDS read at each later wait.  Their completion is
// awaited explicitly (wait_loads, then a barrier) before the data is read.
// NT: the non-temporal policy, for the last read of a tile or record (the
// stores of o, records and states carry it too); the streams then leave the
// caches to what is read again: the g and beta lines, the chunk table, the K
// tiles the intra-chunk step reads before the recurrence does, and the tiles
// a sequence-parallel first pass reads again in its second pass.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ __forceinline__ void lds_load16(u16* dst_block, const void* src) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)dst_block);
  // (one wait state between the M0 write and the load that reads it)
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds), "v"(src)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src)
                 : "memory", "m0");
}
// Same with a wave-uniform 64-bit base and a 32-bit per-lane byte offset.
template <bool NT>
__device__ __forceinline__ void lds_load16_at(uint32_t lds, const void* sbase, uint32_t voff) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds), "v"(voff),
                 "s"(sbase)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a shared-memory pointer, as a wave-uniform value
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

// global-memory pointer (stores through it are global, not flat, stores)
template <typename T>
using gptr = __attribute__((address_space(1))) T*;

// a pointer the whole wave agrees on, held in scalar registers
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Per-lane byte offset, from the first row of block j, of what lane l loads
// in block j: row 4j + l/16, k-group (l%16) ^ (row%16).  Depends on j only
// through j%4.
__device__ __forceinline__ uint32_t tile_lane_off(int q, int lane, int64_t stride) {
  const int r = lane >> 4;
  const int k8 = (lane & 15) ^ ((4 * q + r) & 15);
  return (uint32_t)(r * stride * 2 + k8 * 16);
}


// Rows 4j..4j+3 of a token tile whose row 0 is new token n0 into block j of
// `tile`.  Rows outside the sequence read 256 bytes of zeros (the padding
// rows are exact identities of the recurrence).
template <bool NT>
__device__ __forceinline__ void load_rows(u16* tile, const u16* src, int64_t stride, const u16* zero,
                                          const Seq& s, int n0, int j, int lane) {
  const int row = 4 * j + (lane >> 4);
  const int n = n0 + row;
  const int k8 = (lane & 15) ^ (row & 15);
  const u16* rp = (unsigned)n < (unsigned)s.L ? src + ((int64_t)s.tok0 + n) * stride : zero;
  lds_load16<NT>(tile + j * 512, rp + k8 * 8);
}

// Blocks j0 .. j0 + NB - 1 (j0 a multiple of 4) of a token tile whose row 0
// is new token n0.  Chunks with every row inside the sequence take uniform
// bases and the precomputed lane offsets; the first and last chunk of a
// sequence check rows one by one.
template <int NB, bool NT>
__device__ __forceinline__ void load_tile(u16* tile, const u16* src, int64_t stride,
                                          const uint32_t (&voff)[4], const u16* zero, const Seq& s,
                                          int n0, int j0, int lane) {
  if (n0 >= 0 && n0 + kChunk <= s.L) {
    const char* base = uniform_ptr(src + ((int64_t)s.tok0 + n0 + 4 * j0) * stride);
    const uint32_t lds = lds_addr(tile + j0 * 512);
#pragma unroll
    for (int i = 0; i < NB; ++i) lds_load16_at<NT>(lds + i * 1024, base + (int64_t)i * 8 * stride, voff[i & 3]);
  } else {
#pragma unroll 1
    for (int i = 0; i < NB; ++i) load_rows<NT>(tile, src, stride, zero, s, n0, j0 + i, lane);
  }
}

// The wait goes through the compiler's own builtin (vmcnt 0, the other
// counters untouched), so the compiler knows that nothing is outstanding after
// it: its own waits for stores it issued earlier (whose data registers it must
// not overwrite before they are read) are then not placed later, where they
// would also wait for the loads above that it does not know of.
__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
  asm volatile("" ::: "memory");
}

// Scheduling fence for hand-pipelined products: MFMAs and LDS accesses stay
// on their side (so the next step's operand reads are in flight while this
// step's MFMAs run); plain VALU and SALU work may move across.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0x6); }

// ============================================================== wy_kernel
constexpr int kWyThreads = 256;

// A and T are lower triangular: only their 10 blocks (bi >= bj) of 16x16
// are kept, at a pitch of 20 floats (16-byte rows; the 4 row groups of an
// MFMA result land in different banks).  tri_idx(bi, bj) of an upper block
// still names one of the 10 (its contents are then masked off by the reader).
constexpr int kBP = 20;
__device__ __forceinline__ int tri_idx(int bi, int bj) { return bi * (bi + 1) / 2 + bj; }

// The K tile's LDS is reused: once every wave holds its K K^T blocks in
// registers, A is written over the tile, and each block of T is then formed
// in place of the A block it replaces (every A block is read -- by the same
// wave, or before a barrier -- before its T block is written).
struct WySmem {
  union {
    u16 Kb[kTileWords];      // K tile (row-major, swizzled) ...
    float AT[10][16][kBP];   // ... then A, turning into T block by block
  } u;                       // (X = A[32:64, 0:32] T[0:32, 0:32] goes over the A blocks it consumes)
  float G[kChunk];           // log2-scale running decay sum
  float B[kChunk];           // beta (0 on padding rows)
  float kn[kChunk];          // k.k of each row (the diagonal of K K^T)
};

template <int W>
__device__ __forceinline__ void wy_body(const PrefillParams& p, WySmem& sm) {
  if (guarded(p.guard)) return;
  // Workgroups go to the 8 XCDs round-robin by block index: block b runs on
  // XCD b % 8, and every v-head of chunk slot c runs on XCD c % 8, so the
  // cache lines of g and beta (all heads of a token side by side) and of K
  // (heads of a q/k group) are fetched into one L2 per chunk, not eight.
  const int xcd = blockIdx.x & 7, r = blockIdx.x >> 3;
  const int cg = r / p.H;
  const int c = 8 * cg + xcd;
  if (c >= p.num_chunk_slots) return;  // the grid is rounded up to 8 chunk slots
  const int h = r - cg * p.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = W;
  const int n16 = lane & 15, gq = lane >> 4;

  const int4 e = p.chunk_tab[c];  // the same for every lane
  if (e.x < 0) return;            // slot beyond this batch's chunks
  Seq s;
  s.L = e.z;
  s.tok0 = e.w;
  s.h = h;
  s.hq = h / p.group;
  const int n0 = e.y;
  const int64_t ch = (int64_t)c * p.H + h;

  // K tile straight to LDS (padding rows read zeros); wave 0 loads g and
  // beta alongside and scans the decay
  {
    const int64_t stride = (int64_t)p.Hqk * kDim;
    uint32_t off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) off[q] = tile_lane_off(q, lane, stride);
    load_tile<4, false>(sm.u.Kb, p.k + (int64_t)s.hq * kDim, stride, off, p.zero_row, s, n0, 4 * wid, lane);
  }
  if (wid == 0) {
    const int n = n0 + lane;
    const bool valid = (unsigned)n < (unsigned)s.L;
    const int64_t t = ((int64_t)s.tok0 + (valid ? n : 0)) * p.H + h;
    const float gv = p.g ? p.g[t] : 0.f;
    const float bv = p.beta ? p.beta[t] : 1.f;
    float G = valid ? gv * kLog2e : 0.f;
    const float bet = valid ? bv : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(G, off, 64);
      if (lane >= off) G += y;
    }
    const float Glast = __shfl(G, 63, 64);
    float* sc = p.ws_scal + ch * kRecScal;
    __builtin_nontemporal_store(bet, sc + lane);
    __builtin_nontemporal_store(G, sc + kChunk + lane);
    __builtin_nontemporal_store(exp2f(G), sc + 2 * kChunk + lane);
    __builtin_nontemporal_store(exp2f(Glast - G), sc + 3 * kChunk + lane);
    sm.G[lane] = G;
    sm.B[lane] = bet;
  }
  wait_loads();
  __syncthreads();

  // K K^T lower blocks -> A = beta_row D k.k, strictly lower: the blocks of
  // wave w (w, w + 4, w + 8) stay in registers until every wave is done
  // reading the K tile, then A goes over it.
  f32x4 kk[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int blk = wid + 4 * i;
    kk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (blk < 10) {
      const int bi = tri_i(blk), bj = tri_j(blk);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kk[i] = mfma16x16x32(tile_frag(sm.u.Kb, bi * 4 + ks, lane), tile_frag(sm.u.Kb, bj * 4 + ks, lane), kk[i]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int blk = wid + 4 * i;
    if (blk < 10) {
      const int bi = tri_i(blk), bj = tri_j(blk);
      const int col = 16 * bj + n16;
      const float Gc = sm.G[col];
      const f32x4 Gr = *(const f32x4*)&sm.G[16 * bi + 4 * gq];
      const f32x4 br = *(const f32x4*)&sm.B[16 * bi + 4 * gq];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * bi + 4 * gq + r;
        const float val = br[r] * __builtin_amdgcn_exp2f(Gr[r] - Gc) * kk[i][r];
        sm.u.AT[blk][4 * gq + r][n16] = row > col ? val : 0.f;
        if (bi == bj && row == col) sm.kn[row] = kk[i][r];
      }
    }
  }
  __syncthreads();

  // For the sequence-parallel first pass: a bound on log2 of the spectral
  // norm of the chunk's transition prod_t alpha_t (I - beta_t k_t k_t^T),
  // sum_t (log2 alpha_t + log2 max(1, |1 - beta_t k_t.k_t|)) (the eigenvalues
  // of I - beta k k^T are 1 and 1 - beta k.k).  Wave 1, idle during the
  // substitution below, computes it.
  if (wid == 1 && p.ws_bound) {
    const float x = fabsf(1.f - sm.B[lane] * sm.kn[lane]);
    float f = __builtin_amdgcn_logf(fmaxf(1.f, x)) + (x - x);  // log2; + NaN when x is NaN or inf
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) f += __shfl_xor(f, off, 64);
    if (lane == 0) p.ws_bound[ch] = f + sm.G[kChunk - 1];
  }

  // diagonal 16x16 blocks of (I + A)^-1 by forward substitution, all four in
  // wave 0: lane group d solves block d, one column a lane
  if (wid == 0) {
    const int d = gq;
    const int col = n16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float* Ar = sm.u.AT[tri_idx(d, d)][i];
      const f32x4 r0 = *(const f32x4*)(Ar + 0);
      const f32x4 r1 = *(const f32x4*)(Ar + 4);
      const f32x4 r2 = *(const f32x4*)(Ar + 8);
      const f32x4 r3 = *(const f32x4*)(Ar + 12);
      const float a[16] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3],
                           r2[0], r2[1], r2[2], r2[3], r3[0], r3[1], r3[2], r3[3]};
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < i; ++j) part[j & 3] += a[j] * x[j];
      x[i] = (i == col ? 1.f : 0.f) - ((part[0] + part[1]) + (part[2] + part[3]));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.u.AT[tri_idx(d, d)][i][col] = x[i];
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
      a[j] = sm.u.AT[tri_idx(I, J)][n16][4 * gq + j];
      bb[j] = sm.u.AT[tri_idx(J, J)][4 * gq + j][n16];
      a[j + 4] = 0.f;
      bb[j + 4] = 0.f;
    }
    const f32x4 X = mma3(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = sm.u.AT[tri_idx(I, I)][n16][4 * gq + j];
      bb[j] = X[j];
    }
    const f32x4 Y = mma3(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.u.AT[tri_idx(I, J)][4 * gq + r][n16] = -Y[r];
  }
  __syncthreads();
  {
    const int I = 2 + (wid >> 1), J = wid & 1;
    float a[8], bb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = perm_row(0, gq, j);  // 0..31 over column blocks 0, 1
      const bool use = J == 0 || kk >= 16;  // T_01 = 0
      const float av = sm.u.AT[tri_idx(I, kk >> 4)][n16][kk & 15];
      const float tv = sm.u.AT[tri_idx(kk >> 4, J)][kk & 15][n16];
      a[j] = use ? av : 0.f;
      bb[j] = use ? tv : 0.f;
    }
    const f32x4 X = mma3(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
    __syncthreads();  // every wave has read its A blocks: X goes over block (I, J)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.u.AT[tri_idx(I, J)][4 * gq + r][n16] = X[r];
  }
  __syncthreads();
  {
    const int I = 2 + (wid >> 1), J = wid & 1;
    float a[8], bb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = perm_row(0, gq, j);  // 0..31 over rows/columns 32..63
      const bool use = I == 3 || kk < 16;  // T_23 = 0
      const float tv = sm.u.AT[tri_idx(I, 2 + (kk >> 4))][n16][kk & 15];
      const float xv = sm.u.AT[tri_idx(2 + (kk >> 4), J)][kk & 15][n16];  // X
      a[j] = use ? tv : 0.f;
      bb[j] = use ? xv : 0.f;
    }
    const f32x4 Y = mma3(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
    __syncthreads();  // every wave has read its X blocks: T goes over block (I, J)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.u.AT[tri_idx(I, J)][4 * gq + r][n16] = -Y[r];
  }
  __syncthreads();

  // the record's 5 fragments of T diag(beta) (hi/lo) straight to the
  // workspace: slots 4h..4h+3 of record fragment f hold columns 4g4..4g4+3
  // of block (bi, bj) = (0, 0), (2, 2) for f = 0 and (mt, 2 (f == 4) + h)
  // with mt = 1, 2, 3, 3 for f = 1..4 (lane = row within the block + 16 g4)
  u16* Tw = p.ws_T + ch * kRecWords;
  for (int f = wid; f < kTFrags; f += 4) {
    const int rr = lane & 15, g4 = lane >> 4;
    float vals[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int bi = f == 0 ? 2 * h : (f < 3 ? f : 3);
      const int bj = f == 0 ? 2 * h : (f == 4 ? 2 : 0) + h;
      const f32x4 tv = *(const f32x4*)&sm.u.AT[tri_idx(bi, bj)][rr][4 * g4];
      const f32x4 bv = *(const f32x4*)&sm.B[16 * bj + 4 * g4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vals[4 * h + e] = tv[e] * bv[e];  // T diag(beta)
    }
    bf16x8 hi, lo;
    split8(vals, hi, lo);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, hi), (u32x4*)(Tw + (f * 64 + lane) * 8));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, lo),
                                (u32x4*)(Tw + kTFrags * kFragElems + (f * 64 + lane) * 8));
  }
}

// Each of the four waves runs its own compiled copy of the body (its K K^T
// blocks, substitution and doubling steps then have constant offsets):
// 1.5% less time than one copy with a run-time wave index.
__global__ __launch_bounds__(kWyThreads) void wy_kernel(const PrefillParams p) {
  __shared__ __align__(16) WySmem sm;
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: wy_body<0>(p, sm); break;
    case 1: wy_body<1>(p, sm); break;
    case 2: wy_body<2>(p, sm); break;
    default: wy_body<3>(p, sm); break;
  }
}

// ============================================================== rec_kernel
// A workgroup of NW waves advances NW x 16 state rows (a V-tile) of one
// (sequence, v-head); with NW < 8 the 128 rows split over 8 / NW workgroups,
// for batches too small to fill the chip with whole heads.
constexpr int kOsPitch = kDim + 8;  // bf16 row pitch of the output tile

// k of accumulator row (block mb, lane group gq, r = 0)
__device__ __forceinline__ int state_k(int mb, int gq) { return 32 * (mb >> 1) + 8 * gq + 4 * (mb & 1); }

// dst points at the lane's state row (v), k = 0
// (NT: non-temporal, for rows the caller reads later; the workspace states
// the next kernel of the call reads keep the default policy)
template <bool NT = true>
__device__ __forceinline__ void store_state(float* dst, const f32x4 (&accS)[8], int gq) {
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    if constexpr (NT) __builtin_nontemporal_store(accS[mb], (f32x4*)(dst + state_k(mb, gq)));
    else *(f32x4*)(dst + state_k(mb, gq)) = accS[mb];
  }
}

// The lane's state row in a caller's state buffer (fp32, or bf16 rounded to
// nearest even when bf16), element offset `off` = the row's k = 0
__device__ __forceinline__ void store_state_buf(void* base, int64_t off, const f32x4 (&accS)[8], int gq,
                                                bool bf16) {
  if (bf16) {
    u16* dst = (u16*)base + off;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      *(u32x2*)(dst + state_k(mb, gq)) = u32x2{f2bf2(accS[mb][0], accS[mb][1]), f2bf2(accS[mb][2], accS[mb][3])};
  } else {
    store_state((float*)base + off, accS, gq);
  }
}
__device__ __forceinline__ void load_state_buf(const void* base, int64_t off, f32x4 (&accS)[8], int gq,
                                               bool bf16) {
  if (bf16) {
    const u16* src = (const u16*)base + off;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const u32x2 w = *(const u32x2*)(src + state_k(mb, gq));
      accS[mb] = f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
    }
  } else {
    const float* src = (const float*)base + off;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) accS[mb] = *(const f32x4*)(src + state_k(mb, gq));
  }
}

struct RecSmem {
  u16 Kb[2][kTileWords];               // K tiles, double-buffered by chunk parity
  u16 Qb[2][kTileWords];               // Q tiles
  u16 Tf[2][2 * kTFrags * kFragElems]; // T fragments (wy_kernel's record), hi then lo
  float scal[2][4][kChunk];            // beta, G, gamma, exp(G_last - G)
  u16 Vb[kTileWords];                  // V tile (reloaded after the mid-chunk barrier)
  u16 Ktf[kKtWordsL];                  // K^T fragments: [k block][t-step][lane][8]
  u16 Pf[kMatFrag];                    // P fragments (bf16)
  u16 Os[kChunk][kOsPitch];            // output tile, stored during the next chunk
};

// Half `part` (0 or 1) of the T fragments of chunk slot c (already in LDS
// order), with the per-row scalars in half 0.
template <bool NT>
__device__ __forceinline__ void load_rec(u16* Tdst, float* sdst, const PrefillParams& p, const Seq& s,
                                         int64_t c, int part, int lane) {
  const int64_t ch = c * p.H + s.h;
  const char* Tw = uniform_ptr(p.ws_T + ch * kRecWords + kTFrags * part * 512);
  const uint32_t lds = lds_addr(Tdst + kTFrags * part * 512);
#pragma unroll
  for (int i = 0; i < kTFrags; ++i) lds_load16_at<NT>(lds + i * 1024, Tw + i * 1024, lane * 16);
  if (part == 0) lds_load16_at<NT>(lds_addr(sdst), uniform_ptr(p.ws_scal + ch * kRecScal), lane * 16);
}

// o rows 4j..4j+3 of a finished chunk (row 0 = new token n0), j = j0 ..
// j0 + NJ - 1: 16 bytes a lane, 4 whole rows per store instruction.
// o rows of a finished chunk (row 0 = new token n0) for the workgroup's
// columns v0 .. v0 + 16 NW - 1, all lanes of the workgroup: 16-byte units u =
// tid + 64 NW i, row u / (2 NW), piece u % (2 NW).
template <int NW>
__device__ __forceinline__ void write_o_tile(const PrefillParams& p, const RecSmem& sm, const Seq& s,
                                             int n0, int v0, int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = tid + 64 * NW * i;
    const int row = u / (2 * NW), seg = u % (2 * NW);
    const int nn = n0 + row;
    const u32x4 w = *(const u32x4*)&sm.Os[row][seg * 8];
    if ((unsigned)nn < (unsigned)s.L)
      __builtin_nontemporal_store(w, (u32x4*)(p.o + (((int64_t)s.tok0 + nn) * p.H + s.h) * kDim + v0 + seg * 8));
  }
}

template <int NJ>
__device__ __forceinline__ void write_o(const PrefillParams& p, const RecSmem& sm, const Seq& s,
                                        int n0, int j0, int lane) {
  if (n0 >= 0 && n0 + kChunk <= s.L) {  // every row inside the sequence
    const int64_t rs = (int64_t)p.H * kDim * 2;  // o row stride, bytes
    gptr<char> base = (gptr<char>)uniform_ptr(p.o + (((int64_t)s.tok0 + n0 + 4 * j0) * p.H + s.h) * kDim);
    const uint32_t vo = (uint32_t)((lane >> 4) * rs + (lane & 15) * 16);
    u32x4 w[NJ];
#pragma unroll
    for (int i = 0; i < NJ; ++i) w[i] = *(const u32x4*)&sm.Os[4 * (j0 + i) + (lane >> 4)][(lane & 15) * 8];
#pragma unroll
    for (int i = 0; i < NJ; ++i) __builtin_nontemporal_store(w[i], (gptr<u32x4>)(base + i * 4 * rs + vo));
    return;
  }
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    const int row = 4 * (j0 + i) + (lane >> 4), seg = lane & 15;
    const int nn = n0 + row;
    const u32x4 w = *(const u32x4*)&sm.Os[row][seg * 8];  // pitch keeps 16-byte alignment
    if ((unsigned)nn < (unsigned)s.L)
      __builtin_nontemporal_store(w, (u32x4*)(p.o + (((int64_t)s.tok0 + nn) * p.H + s.h) * kDim + seg * 8));
  }
}


// OUT: the run produces outputs, checkpoints and its final state (whole
// sequences, and the sequence-parallel second pass); without, it is a
// first-pass segment run (offset or transition) that only ends in a state.
// ROLE (8 waves): the wave pair 2 ROLE, 2 ROLE + 1 this copy of the body
// runs for, wsel the wave within the pair; -1 (narrower tiles): wsel is
// the wave index.
template <int NW, bool OUT, int ROLE>
__device__ __forceinline__ void rec_body(const PrefillParams& p, int wsel) {
  constexpr int kThreads = NW * 64;
  constexpr int kTiles = 8 / NW;  // V-tiles per head
  extern __shared__ __align__(16) unsigned char smem_raw[];
  RecSmem& sm = *reinterpret_cast<RecSmem*>(smem_raw);
  if (guarded(p.guard)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = ROLE >= 0 ? 2 * ROLE + wsel : wsel;  // wave index (its pair compile-time)
  const int n16 = lane & 15, gq = lane >> 4;

  // Longest sequences first: blockIdx walks p.order (sorted by chunk count);
  // the V-tiles of a head sit H blocks apart (same XCD when H % 8 == 0).
  // With p.vseq the items are segments of sequences instead (the
  // sequence-parallel passes), each described by its own record.
  const int per_seq = p.H * kTiles;
  const int item = blockIdx.x;
  const int r_in = item - (item / per_seq) * per_seq;
  const int vt = r_in / p.H;
  Seq s;
  s.h = head_of(r_in - vt * p.H, p.H, p.group);
  int pre, cs0, rd, wr, ck_base, mode = kSegNormal;
  if (p.vseq) {
    const int vi = item / per_seq;
    const int ri = p.vhalf > 0 && vi >= p.vhalf ? vi - p.vhalf : vi;  // index within its half
    if (ri >= *p.vcount) return;  // beyond this pass's segments
    const int32_t* d = p.vseq + kSegWords * vi;
    s.tok0 = d[0];
    s.L = d[1];
    pre = d[2];
    cs0 = d[3];
    rd = d[4];
    wr = d[5];
    ck_base = d[6];
    mode = d[7];
  } else {
    const int b = p.order[item / per_seq];
    s.tok0 = p.cu_seqlens[b];
    s.L = p.cu_seqlens[b + 1] - s.tok0;
    pre = p.slots.prefix[b];
    cs0 = p.slots.chunk_start[b];
    rd = p.slots.read[b];
    wr = p.slots.write[b];
    ck_base = p.ckpt_idx ? p.slots.ckpt_start[b] : 0;
  }
  if (s.L <= 0) return;  // a zero-length sequence writes nothing
  // First-pass runs with the chunks' transition bounds at hand (log2 of the
  // norm of prod_t alpha_t (I - beta_t k_t k_t^T), one per chunk and head):
  // a transition run whose whole bound is below kSkipLog2 stores zeros; an
  // offset run starts from zero at the latest chunk from which the rest of
  // the segment's bound is below it (what came before is wiped out at fp32
  // resolution), instead of at the segment's first chunk.  A NaN or infinity
  // in g, beta or k makes the bound of its chunk NaN, so no sum through it
  // counts; v does not enter the bound, so a NaN in v inside chunks an offset
  // run leaves out does not reach the later states (through the full
  // recurrence it would).
  bool map_is_zero = false;
  if constexpr (!OUT) {
    if (p.ws_bound && mode != kSegNormal) {
      const int c_all = chunks_of(pre, s.L);
      const float* bnd = p.ws_bound + (int64_t)cs0 * p.H + s.h;
      if (mode == kSegMap) {
        float t = 0.f;
        for (int base = 0; base < c_all; base += 64) {
          float v = base + lane < c_all ? bnd[(int64_t)(base + lane) * p.H] : 0.f;
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
          t += v;  // the same in every lane and wave
        }
        map_is_zero = __builtin_amdgcn_readfirstlane((int)(t < kSkipLog2)) != 0;
      } else {
        int k = 0;  // trailing chunks to run (0: all of them)
        float carry = 0.f;
        for (int base = 0; base < c_all && k == 0; base += 64) {
          const int c = c_all - 1 - (base + lane);
          float v = c >= 0 ? bnd[(int64_t)c * p.H] : 0.f;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(v, off, 64);
            if (lane >= off) v += y;
          }
          v += carry;  // bound of chunks c .. c_all - 1
          const uint64_t hit = __ballot(c >= 0 && v < kSkipLog2);
          if (hit) k = base + __builtin_ctzll(hit) + 1;
          carry = __shfl(v, 63, 64);
        }
        k = __builtin_amdgcn_readfirstlane(k);
        if (k > 0 && k < c_all) {  // run chunks c_all - k .. c_all - 1 from zero
          const int a = (pre & ~(kChunk - 1)) - pre + kChunk * (c_all - k);
          s.tok0 += a;
          s.L -= a;
          pre += a;
          cs0 += c_all - k;
        }
      }
    }
  }
  s.hq = s.h / p.group;
  const int nch = chunks_of(pre, s.L);
  // a transition-map segment: identity start, v = 0; first-pass runs skip Q
  // and every product that only feeds o
  const bool vzero = !OUT && mode == kSegMap;
  constexpr bool outs = OUT;
  const int vb = vt * NW + wid;  // this wave's 16-row block of the state
  const int vrow = 16 * vb + n16;
  const int64_t head_off = ((int64_t)s.h * kDim + vrow) * kDim;
  if (map_is_zero) {
    const f32x4 zeros[8] = {};
    store_state<false>(p.ws_state + (int64_t)(-2 - wr) * p.ws_state_stride + head_off, zeros, gq);
    return;
  }
  const u16* ksrc = p.k + (int64_t)s.hq * kDim;
  const u16* qsrc = p.q + (int64_t)s.hq * kDim;
  const u16* vsrc = p.v + (int64_t)s.h * kDim;
  const int64_t qk_stride = (int64_t)p.Hqk * kDim, v_stride = (int64_t)p.H * kDim;
  uint32_t off_qk[4], off_v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    off_qk[q] = tile_lane_off(q, lane, qk_stride);
    off_v[q] = tile_lane_off(q, lane, v_stride);
  }

  const int nbase = (pre & ~(kChunk - 1)) - pre;  // new-token index of chunk 0's row 0
  const float log2_scale = __builtin_amdgcn_logf(p.scale);  // log2
  // chunk 0's inputs
#pragma unroll 1
  for (int j = wid; j < 16; j += NW) {
    load_rows<OUT>(sm.Kb[0], ksrc, qk_stride, p.zero_row, s, nbase, j, lane);
    if (outs) load_rows<OUT>(sm.Qb[0], qsrc, qk_stride, p.zero_row, s, nbase, j, lane);
    if (!vzero) load_rows<OUT>(sm.Vb, vsrc, v_stride, p.zero_row, s, nbase, j, lane);
  }
  if (vzero)
    for (int i = tid; i < kTileWords / 8; i += kThreads) *(u32x4*)&sm.Vb[8 * i] = u32x4{0u, 0u, 0u, 0u};
  for (int part = wid; part < 2; part += NW) load_rec<OUT>(sm.Tf[0], &sm.scal[0][0][0], p, s, cs0, part, lane);

  f32x4 accS[8];
  if (vzero) {  // the identity: row vrow has its 1 at k = vrow
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) accS[mb][r] = state_k(mb, gq) + r == vrow ? 1.f : 0.f;
  } else if (rd >= 0 && p.init) {
    load_state_buf(p.init, (int64_t)rd * p.init_stride + head_off, accS, gq, p.state_bf16);
  } else if (rd <= -2) {  // a state of the sequence-parallel workspace
    const float* src = p.ws_state + (int64_t)(-2 - rd) * p.ws_state_stride + head_off;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) accS[mb] = *(const f32x4*)(src + state_k(mb, gq));
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) accS[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // 0/1 operand that picks this wave's 16 v columns out of a V fragment:
  // B[8*gq + j][n] = 1 where 8*gq + j == 16*(vb%2) + n
  bf16x8 vsel;
#pragma unroll
  for (int j = 0; j < 8; ++j) vsel[j] = 8 * gq + j == 16 * (vb & 1) + n16 ? (__bf16)1.0f : (__bf16)0.0f;

  // 0/1 operands that pick, for lane column i, the k of accumulator row
  // state_k(mk, i/4) + i%4 out of a 32-deep K fragment (mk%2 = h):
  // B[8*gq + j][i] = 1 where gq == i/4 and j == 4h + i%4
  bf16x8 ksel[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ksel[h][j] = gq == (n16 >> 2) && j == 4 * h + (n16 & 3) ? (__bf16)1.0f : (__bf16)0.0f;

  // P's blocks above the diagonal are zero for every chunk
  for (int i = tid; i < kMatFrag / 4; i += kThreads) {  // 8-byte units: fragment, lane, half
    const int f = i >> 7, ln = (i >> 1) & 63, half = i & 1;
    const int bt = f >> 1, bs = 2 * (f & 1) + half;
    if (bs > bt) *(u32x2*)&sm.Pf[(f * 64 + ln) * 8 + 4 * half] = u32x2{0u, 0u};
  }
  wait_loads();
  __syncthreads();

  // the next checkpoint position (the first multiple of the interval past the
  // prefix: the state after the token at that many tokens of the sequence)
  // and its index among the call's checkpoints of this sequence
  int ck_next = OUT && p.ckpt_idx ? (pre / p.ckpt_every + 1) * p.ckpt_every : -1;
  int ck_j = 0;
  for (int ci = 0; ci < nch; ++ci) {
    const int X = ci & 1;
    const int n0 = nbase + kChunk * ci;
    const bool more = ci + 1 < nch;
    const u16* Kb = sm.Kb[X];
    const u16* Qb = sm.Qb[X];
    const u16* Tf = sm.Tf[X];
    const float(*sc)[kChunk] = sm.scal[X];
    // position after the chunk's last row; checkpoints strictly inside the
    // chunk (intervals that are not multiples of 64) are taken from the
    // chunk's start state, so its decay then waits until they are done
    const int a_end = (pre & ~(kChunk - 1)) + kChunk * (ci + 1);
    const bool ck_inside = ck_next > 0 && ck_next < a_end && ck_next <= pre + s.L;

    // Memory traffic of the iteration, by wave pairs at different points so
    // that of the two waves sharing a SIMD (w and w + 4) one computes while
    // the other waits to issue: at the top, waves 0-1 load the next K; after
    // Y, waves 2-3 store the previous chunk's o, waves 4-5 load the next Q
    // and waves 6-7 the next T; after the mid-chunk barrier, waves 0-3 load
    // the next V.
    if constexpr (NW == 8) {
      if (wid < 2 && more) load_tile<8, OUT>(sm.Kb[X ^ 1], ksrc, qk_stride, off_qk, p.zero_row, s, n0 + kChunk, 8 * wid, lane);
    } else if (more) {
      // every wave loads 16 / NW consecutive blocks of the next K and Q
      load_tile<16 / NW, OUT>(sm.Kb[X ^ 1], ksrc, qk_stride, off_qk, p.zero_row, s, n0 + kChunk, wid * (16 / NW), lane);
      if (outs) load_tile<16 / NW, OUT>(sm.Qb[X ^ 1], qsrc, qk_stride, off_qk, p.zero_row, s, n0 + kChunk, wid * (16 / NW), lane);
    }

    // ---- recurrence: wave w owns state rows 16w..16w+15
    // Each MFMA run below has vector work beside it that does not depend on
    // it, so the two can overlap: S's decay beside Y, R and its split beside
    // Z = S Q^T, the z scaling beside E, E's splits beside the P and K^T
    // products.  The products keep 4 to 16 independent accumulators in
    // flight (a chain of dependent MFMAs issues at about a third of the
    // rate), and each step's operand fragments are read while the previous
    // step multiplies.
    // S as bf16 operands: Shi (rounded) for Y = K S^T and Z = S Q^T, plus
    // Slo = S - Shi for a second Y pass in chunks with weak decay.  Y enters
    // the state through R = V - gamma Y and E = T R, whose rows reach the
    // chunk's end state scaled by exp(G_last - G_t): every row's Y error
    // arrives there scaled by gamma_last = exp(G_last), the chunk's whole
    // decay.  Below 2^-10 the single pass's 2^-9 error is out of sight
    // (measured against the fp64 oracle: hybrid-step states 4.5e-6 either
    // way); above it -- weak or no decay, short tail chunks -- the second
    // pass keeps states near 1e-5 (one pass: 6.9e-5 with decay / 10, over
    // 1e-3 with none).  A single-pass E or state update would cost 0.7e-3 ..
    // 2.4e-3 at any decay, so those always take hi/lo passes.
    const bool y_lo = __builtin_amdgcn_readfirstlane(
        __builtin_bit_cast(int, sc[2][kChunk - 1]) > __builtin_bit_cast(int, kYLoGamma));
    bf16x8 Shi[4], Slo[4];
    if (y_lo) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = accS[2 * ks + (j >> 2)][j & 3];
        split8(v, Shi[ks], Slo[ks]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = accS[2 * ks + (j >> 2)][j & 3];
        Shi[ks] = round8(v);
        Slo[ks] = Shi[ks];  // not read on this path (keeps it initialised)
      }
    }

    // Y = K S^T (the lo pass only where the decay is weak)
    f32x4 y[4];
    bf16x8 vf[4];
    {
      bf16x8 kf[2][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        y[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        kf[0][mt] = tile_frag(Kb, mt * 4, lane);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // operands of the next step (the V fragments after the last)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (ks < 3) kf[(ks + 1) & 1][mt] = tile_frag(Kb, mt * 4 + ks + 1, lane);
          else vf[mt] = tile_frag(sm.Vb, mt * 4 + (vb >> 1), lane);
        }
        sched_fence();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) y[mt] = mfma16x16x32(kf[ks & 1][mt], Shi[ks], y[mt]);
        if (y_lo) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) y[mt] = mfma16x16x32(kf[ks & 1][mt], Slo[ks], y[mt]);
        }
        sched_fence();
      }
    }
    // S's decay over the chunk (the update adds onto it at the end)
    if (!ck_inside) {
      const float gC = sc[2][kChunk - 1];
#pragma unroll
      for (int mk = 0; mk < 8; ++mk) accS[mk] = accS[mk] * gC;
    }

    if constexpr (NW == 8) {
      if (wid == 2 || wid == 3) {
        if (ci > 0 && OUT) write_o<8>(p, sm, s, n0 - kChunk, 8 * (wid - 2), lane);
      } else if (more && wid >= 4) {
        if (wid < 6) {
          if (outs) load_tile<8, OUT>(sm.Qb[X ^ 1], qsrc, qk_stride, off_qk, p.zero_row, s, n0 + kChunk, 8 * (wid - 4), lane);
        } else {
          load_rec<OUT>(sm.Tf[X ^ 1], &sm.scal[X ^ 1][0][0], p, s, (int64_t)cs0 + ci + 1, wid - 6, lane);
        }
      }
    } else {
      if (ci > 0 && OUT) write_o_tile<NW>(p, sm, s, n0 - kChunk, 16 * NW * vt, tid);
      if (more) {
        for (int part = wid; part < 2; part += NW)
          load_rec<OUT>(sm.Tf[X ^ 1], &sm.scal[X ^ 1][0][0], p, s, (int64_t)cs0 + ci + 1, part, lane);
      }
    }

    // Z = S Q^T with the state's hi part (an output-only product: the bf16
    // output rounding dominates its error); beside it R = V - gamma Y (beta
    // is folded into the T record; V's 16 columns enter through the
    // selection operand, exact) and R's hi/lo split
    f32x4 z[4];
    bf16x8 Rhi[2], Rlo[2];
    {
      bf16x8 qf[2][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        z[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (outs) qf[0][mt] = tile_frag(Qb, mt * 4, lane);
      }
      f32x4 R[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 gm = *(const f32x4*)&sc[2][16 * mt + 4 * gq];
#pragma unroll
        for (int r = 0; r < 4; ++r) R[mt][r] = -gm[r] * y[mt][r];
        R[mt] = mfma16x16x32(vf[mt], vsel, R[mt]);
      }
      if (outs) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if (ks < 3) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) qf[(ks + 1) & 1][mt] = tile_frag(Qb, mt * 4 + ks + 1, lane);
          }
          sched_fence();
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) z[mt] = mfma16x16x32(Shi[ks], qf[ks & 1][mt], z[mt]);
          sched_fence();
        }
      }
      split_rows(R, 0, Rhi[0], Rlo[0]);
      split_rows(R, 1, Rhi[1], Rlo[1]);
    }

    // E = (T diag(beta)) R (row blocks 0 and 1 have no columns in k-step 1);
    // beside it, z *= scale * gamma (the output scale rides on gamma here and
    // on P's exponent)
    f32x4 E[4];
    {
      bf16x8 th[6], tl[6];
      {
        bf16x8 rh[kTFrags], rl[kTFrags];
#pragma unroll
        for (int f = 0; f < kTFrags; ++f) {
          rh[f] = lds_frag(Tf, f, lane);
          rl[f] = lds_frag(Tf + kTFrags * kFragElems, f, lane);
        }
        unpack_t(rh, th);
        unpack_t(rl, tl);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) E[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int mt = ks ? 2 : 0; mt < 4; ++mt) E[mt] = mfma16x16x32(th[t_slot(mt, ks)], Rhi[ks], E[mt]);
#pragma unroll
        for (int mt = ks ? 2 : 0; mt < 4; ++mt) E[mt] = mfma16x16x32(th[t_slot(mt, ks)], Rlo[ks], E[mt]);
#pragma unroll
        for (int mt = ks ? 2 : 0; mt < 4; ++mt) E[mt] = mfma16x16x32(tl[t_slot(mt, ks)], Rhi[ks], E[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float gm = p.scale * sc[2][16 * mt + n16];
#pragma unroll
        for (int r = 0; r < 4; ++r) z[mt][r] *= gm;
      }
    }

    // P^T blocks (K rows x Q rows): the accumulator of block (t-block bt,
    // s-block bs) holds, in lane (t, gq), P[16bt + t][16bs + 4gq + r] --
    // slots 4*(bs&1) + r of P fragment (bt, bs/2).  The ten blocks on and
    // below the diagonal: block w to wave w, and with 8 waves blocks 8 and 9
    // to waves 2 and 3 (which have no loads of the next chunk to issue); the
    // blocks above it stay at the zeros written before the first chunk.  A
    // block's eight operand fragments are read before its four products, so
    // the reads overlap instead of each waiting in turn.
#pragma unroll
    for (int bi = 0; bi < (NW == 8 ? 2 : (10 + NW - 1) / NW); ++bi) {
      const int blk = NW == 8 ? (bi == 0 ? wid : (wid == 2 || wid == 3 ? wid + 6 : 10)) : wid + NW * bi;
      if (blk >= 10 || !outs) break;
      const int bt = tri_i(blk), bs = tri_j(blk);
      bf16x8 pk[4], pq[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        pk[ks] = tile_frag(Kb, bs * 4 + ks, lane);
        pq[ks] = tile_frag(Qb, bt * 4 + ks, lane);
      }
      sched_fence();
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
      acc0 = mfma16x16x32(pk[0], pq[0], acc0);
      acc1 = mfma16x16x32(pk[1], pq[1], acc1);
      acc0 = mfma16x16x32(pk[2], pq[2], acc0);
      acc1 = mfma16x16x32(pk[3], pq[3], acc1);
      sched_fence();
      const f32x4 acc = acc0 + acc1;
      const float Gt = sc[1][16 * bt + n16] + log2_scale;  // P carries the output scale
      const f32x4 Gs = *(const f32x4*)&sc[1][16 * bs + 4 * gq];
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float val = __builtin_amdgcn_exp2f(Gt - Gs[r]) * acc[r];
        v[r] = 16 * bt + n16 >= 16 * bs + 4 * gq + r ? val : 0.f;
      }
      const int f = bt * 2 + (bs >> 1);
      *(u32x2*)&sm.Pf[(f * 64 + lane) * 8 + 4 * (bs & 1)] = u32x2{f2bf2(v[0], v[1]), f2bf2(v[2], v[3])};
    }
    // K^T fragments (k block mk = f/2, t-step ks = f%2).  With 8 waves only
    // waves 0-3 take them (on each SIMD the older wave w of the pair w, w + 4
    // wins issue, so waves 4-7 set the pace and get less of this work), and
    // waves 0-1 take six each against two for waves 2-3, which carry the o
    // stores and the two extra P blocks: f = w, w + 4 for every such wave,
    // then 8 + w, 12 + w, 10 + w, 14 + w for w < 2.  A K fragment times the
    // 0/1 operand ksel[mk%2] leaves, in lane (i, g), the accumulator rows
    // K[16mt + 4g + r][state_k(mk, i/4) + i%4] -- the k of lane i's A-operand
    // row, 4 consecutive t (exact: one product by 1).
#pragma unroll
    for (int i = 0; i < (NW == 8 ? 6 : 16 / NW); ++i) {
      if (NW == 8 && (wid >= 4 || (i >= 2 && wid >= 2))) break;
      const int f = NW != 8 ? wid + NW * i
                  : i < 2   ? wid + 4 * i
                  : i < 4   ? 8 + wid + 4 * (i - 2)
                            : 10 + wid + 4 * (i - 4);
      const int mk = f >> 1, ks = f & 1;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 c1 = mfma16x16x32(tile_frag(Kb, (2 * ks) * 4 + (mk >> 1), lane), ksel[mk & 1], zero);
      const f32x4 c2 = mfma16x16x32(tile_frag(Kb, (2 * ks + 1) * 4 + (mk >> 1), lane), ksel[mk & 1], zero);
      *(u32x4*)&sm.Ktf[(f * 64 + lane) * 8] =
          u32x4{f2bf2(c1[0], c1[1]), f2bf2(c1[2], c1[3]), f2bf2(c2[0], c2[1]), f2bf2(c2[2], c2[3])};
    }
    // E rounded to bf16 for P E (an output-only product, like Z: the bf16
    // output rounding dominates its error) and (dec E) split hi/lo for the
    // state update, beside the P and K^T products above
    bf16x8 Ehi[2], Dhi[2], Dlo[2];
    {
      Ehi[0] = round_rows(E, 0);
      Ehi[1] = round_rows(E, 1);
      f32x4 Ed[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 dc = *(const f32x4*)&sc[3][16 * mt + 4 * gq];
#pragma unroll
        for (int r = 0; r < 4; ++r) Ed[mt][r] = dc[r] * E[mt][r];
      }
      split_rows(Ed, 0, Dhi[0], Dlo[0]);
      split_rows(Ed, 1, Dhi[1], Dlo[1]);
    }
    __syncthreads();  // P and K^T complete; every wave is past its V reads
    if constexpr (NW == 8) {
      if (more && wid < 4 && !vzero) load_tile<4, OUT>(sm.Vb, vsrc, v_stride, off_v, p.zero_row, s, n0 + kChunk, 4 * wid, lane);
    } else if (more && !vzero) {
      load_tile<16 / NW, OUT>(sm.Vb, vsrc, v_stride, off_v, p.zero_row, s, n0 + kChunk, wid * (16 / NW), lane);
    }

    // O^T = scale (S Q^T diag(gamma) + E^T P^T), by 16-token blocks: the
    // state fragments and E act as A operands, Q and P fragments as B, so a
    // lane ends up with 4 adjacent v of one token (one 8-byte LDS store)
    if (outs) {
      bf16x8 pfr[6];
      // P fragments (mt, ks) with mt >= 2 or ks == 0: 0, 2, 4, 5, 6, 7
#pragma unroll
      for (int i = 0; i < 6; ++i) pfr[i] = lds_frag(sm.Pf, i < 2 ? 2 * i : i + 2, lane);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int mt = ks ? 2 : 0; mt < 4; ++mt) z[mt] = mfma16x16x32(Ehi[ks], pfr[t_slot(mt, ks)], z[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        *(u32x2*)&sm.Os[16 * mt + n16][16 * wid + 4 * gq] =
            u32x2{f2bf2(z[mt][0], z[mt][1]), f2bf2(z[mt][2], z[mt][3])};
    }

    // Checkpoints after rows r inside the chunk, from the start state S:
    // S_r = gamma_r S + (dec_r E)^T K with dec_r = exp(G_r - G_t) on rows
    // t <= r and 0 after them (the state update truncated at row r); then the
    // decay of S postponed above.
    if (ck_inside) {
      while (ck_next < a_end && ck_next <= pre + s.L) {
        const int r = ck_next - (a_end - kChunk) - 1;
        const int64_t row = ld_index(p.ckpt_idx, ck_base + ck_j, p.ckpt_idx64);
        ++ck_j;
        ck_next += p.ckpt_every;
        if (row < 0) continue;
        const float Gr = sc[1][r], gr = sc[2][r];
        f32x4 Er[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 Gt = *(const f32x4*)&sc[1][16 * mt + 4 * gq];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            Er[mt][j] = 16 * mt + 4 * gq + j <= r ? __builtin_amdgcn_exp2f(Gr - Gt[j]) * E[mt][j] : 0.f;
        }
        bf16x8 rh[2], rl[2];
        split_rows(Er, 0, rh[0], rl[0]);
        split_rows(Er, 1, rh[1], rl[1]);
        f32x4 acc[8];
#pragma unroll
        for (int mk = 0; mk < 8; ++mk) acc[mk] = accS[mk] * gr;
#pragma unroll
        for (int f = 0; f < 16; ++f) {
          const bf16x8 kt = lds_frag(sm.Ktf, f, lane);  // k block f/2, t-step f%2
          acc[f >> 1] = mfma16x16x32(kt, rh[f & 1], acc[f >> 1]);
          acc[f >> 1] = mfma16x16x32(kt, rl[f & 1], acc[f >> 1]);
        }
        store_state_buf(p.ckpt, row * p.ckpt_stride + head_off, acc, gq, p.state_bf16);
      }
      const float gC = sc[2][kChunk - 1];
#pragma unroll
      for (int mk = 0; mk < 8; ++mk) accS[mk] = accS[mk] * gC;
    }

    // S <- gamma_last S + (dec E)^T K (the decay was applied beside Y); 4
    // groups (ks, mk/4) of 4 K^T fragments, the next group read while this
    // one multiplies (hi pass over the group's 4 blocks, then lo pass)
    {
      bf16x8 ktf[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ktf[0][i] = lds_frag(sm.Ktf, i * 2, lane);
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int ks = gi >> 1, mk0 = 4 * (gi & 1);
        if (gi < 3) {
          const int nks = (gi + 1) >> 1, nmk0 = 4 * ((gi + 1) & 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) ktf[(gi + 1) & 1][i] = lds_frag(sm.Ktf, (nmk0 + i) * 2 + nks, lane);
        }
        sched_fence();
#pragma unroll
        for (int i = 0; i < 4; ++i) accS[mk0 + i] = mfma16x16x32(ktf[gi & 1][i], Dhi[ks], accS[mk0 + i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) accS[mk0 + i] = mfma16x16x32(ktf[gi & 1][i], Dlo[ks], accS[mk0 + i]);
        sched_fence();
      }
    }

    // checkpoint at this chunk's end: stored before the wait below, which
    // then covers the stores too (the state registers are free again before
    // the next chunk's decay overwrites them)
    if (a_end == ck_next && ck_next <= pre + s.L) {
      const int64_t row = ld_index(p.ckpt_idx, ck_base + ck_j, p.ckpt_idx64);
      ++ck_j;
      ck_next += p.ckpt_every;
      if (row >= 0) store_state_buf(p.ckpt, row * p.ckpt_stride + head_off, accS, gq, p.state_bf16);
    }
    wait_loads();     // the next chunk's tiles have landed (this wave's part)
    __syncthreads();  // ... and every wave's; this chunk's LDS operands are free
  }
  if constexpr (OUT) {
    if constexpr (NW == 8) write_o<2>(p, sm, s, nbase + kChunk * (nch - 1), 2 * wid, lane);
    else write_o_tile<NW>(p, sm, s, nbase + kChunk * (nch - 1), 16 * NW * vt, tid);
  }
  if (wr >= 0 && p.out) store_state_buf(p.out, (int64_t)wr * p.out_stride + head_off, accS, gq, p.state_bf16);
  if (wr <= -2) store_state<false>(p.ws_state + (int64_t)(-2 - wr) * p.ws_state_stride + head_off, accS, gq);
}

// With 8 waves the pairs (0, 1), (2, 3), (4, 5), (6, 7) have different work
// (loads, o stores, P blocks, K^T fragments), so each pair runs its own copy
// of the body, compiled with the pair known: its role tests fold away and
// its block and fragment offsets become constants, which takes vector
// compares, address arithmetic and scalar spills out of every chunk (4
// copies; one copy per wave, twice the code, measured slower).
template <int NW, bool OUT>
__global__ __launch_bounds__(NW * 64) void rec_kernel(const PrefillParams p) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (NW == 8) {
    switch (w >> 1) {
      case 0: rec_body<NW, OUT, 0>(p, w & 1); break;
      case 1: rec_body<NW, OUT, 1>(p, w & 1); break;
      case 2: rec_body<NW, OUT, 2>(p, w & 1); break;
      default: rec_body<NW, OUT, 3>(p, w & 1); break;
    }
  } else {
    rec_body<NW, OUT, -1>(p, w);
  }
}

// Launch plan, one workgroup: the longest-first order of the sequences (by
// chunk count; ties by index), the chunk-slot table and the zero row that
// padding rows read.  Sequences are staged through LDS a tile at a time: the
// rank of a sequence counts the longer (or equally long, earlier) ones tile by
// tile, and each chunk slot finds its sequence by binary search over the
// tile's chunk starts (ascending: an exclusive scan of the chunk counts).
constexpr int kPlanTile = 1024;
struct PlanSmem {
  int cnt[kPlanTile];     // chunk count
  int cs[kPlanTile + 1];  // first chunk slot; cs[n] = the tile's end
  int len[kPlanTile];     // new tokens
  int tok0[kPlanTile];    // first token
  int nbase[kPlanTile];   // new-token index of chunk 0's row 0
};

__device__ void plan_body(const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
                          const int32_t* __restrict__ chunk_start, int B, int nslots,
                          int32_t* __restrict__ order, int4* __restrict__ tab,
                          uint32_t* __restrict__ zero_row) {
  __shared__ PlanSmem sm;
  const int tid = threadIdx.x;
  if (tid < 64) zero_row[tid] = 0u;
  for (int c = tid; c < nslots; c += kPlanTile) tab[c] = int4{-1, 0, 0, 0};
  int my_cnt = 0, my_rank = 0;  // of sequence base + tid, for the tile being ranked
  for (int base = 0; base < B; base += kPlanTile) {
    const int b = base + tid;
    if (b < B) my_cnt = chunks_of(prefix[b], cu[b + 1] - cu[b]);
    my_rank = 0;
    for (int t0 = 0; t0 < B; t0 += kPlanTile) {
      const int n = min(kPlanTile, B - t0);
      __syncthreads();
      if (tid < n) {
        const int o = t0 + tid;
        const int pre = prefix[o], L = cu[o + 1] - cu[o];
        sm.cnt[tid] = chunks_of(pre, L);
        sm.cs[tid] = chunk_start[o];
        sm.len[tid] = L;
        sm.tok0[tid] = cu[o];
        sm.nbase[tid] = (pre & ~(kChunk - 1)) - pre;
        if (tid == n - 1) sm.cs[n] = chunk_start[o] + sm.cnt[tid];
      }
      __syncthreads();
      if (b < B) {
        for (int i = 0; i < n; ++i) {
          const int no = sm.cnt[i];
          my_rank += (no > my_cnt) || (no == my_cnt && t0 + i < b);
        }
      }
      // the table for this tile's chunks, once (during the first rank pass)
      if (base == 0) {
        const int c0 = max(sm.cs[0], 0), c1 = min(sm.cs[n], nslots);
        for (int c = c0 + tid; c < c1; c += kPlanTile) {
          int lo = 0, hi = n;  // last i with cs[i] <= c
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sm.cs[mid] <= c) lo = mid;
            else hi = mid;
          }
          const int j = c - sm.cs[lo];
          if (j >= 0 && j < sm.cnt[lo]) tab[c] = int4{t0 + lo, sm.nbase[lo] + kChunk * j, sm.len[lo], sm.tok0[lo]};
        }
      }
    }
    if (b < B) order[my_rank] = b;
  }
}

// Sequence-parallel plan, one workgroup.  Sequence b is cut into G segments
// of s chunks (the last one shorter): s = m when m is forced, the balanced
// length ceil(c / ceil(c / m)) under the auto plan; segment g starts at new
// token lo_g, an absolute multiple of 64 for g >= 1.  It gets, when G >= 2:
//   first pass:  for g = 0 .. G-2 the segment from the zero state (its offset
//                N_g) and from the identity with v = 0 (its transition M_g),
//                so that S_end = S_start M_g + N_g;
//   scan:        start_0 = the sequence's initial state, copied into the
//                workspace; start_{g+1} = start_g M_g + N_g, g = 0 .. G-2;
//   second pass: segments 0 .. G-1 for real from start_g, the last one
//                writing the final state.
// Workspace state rows of b, from row0: start_0 .. start_{G-1}, then
// N_0 .. N_{G-2}, then M_0 .. M_{G-2} (3G - 2 rows).  No launch both reads and
// writes a caller row: the first pass reads none, the scan reads the
// initial state and writes only workspace rows, and the second pass reads
// only workspace rows (segment 0 too) while it stores checkpoints and final
// states -- so an in-place update (write row = read row) or a prefix page
// that a later segment checkpoints never depends on the order in which the
// second pass's workgroups run.  A sequence with G = 1 runs whole in the
// second pass from its own read row, in one workgroup per (sequence, head,
// V-tile) that reads before it writes.

// Auto plan: the segment length m (or none) that minimises an estimate of
// the recurrence's time, in chunk-steps of one recurrence workgroup.  A
// sequence of c chunks is cut into G = ceil(c / s) segments of s =
// ceil(c / ceil(c / m)) chunks (balanced: no short tail segment).  Each pass
// is a list of (sequence, head) runs dealt longest first to the P that are
// resident at once (one recurrence workgroup per compute unit); for N runs
// of total length W and longest p its time is taken as p when N <= P, else
// max(p, W / P + W / N) (the longest-first bound W / P + p_(P+1) with the
// mean length standing in for the (P+1)-th longest).  Per plan:
//   whole sequences:  runs(c, H each)
//   cut:  a1 * first pass (2 (G - 1) H runs of s)
//       + a_s * scan ((G_max - 1) steps, 8 workgroups a pair, in rounds of the CUs)
//       + second pass (G H runs of at most s) + a_l (the two extra launches)
// a1 = 1.0, a_s = 0.75 and a_l = 2 fit the measured times of the 8-sequence
// 16-head ragged batch and the 32-head single prompt over segment lengths
// 6 .. 32 (a first-pass chunk, without outputs, takes about as long as a
// full one: the chunk's dependency chain, not its output work, sets it).
constexpr float kCostPass1 = 1.0f;
constexpr float kCostScanStep = 0.75f;
constexpr float kCostLaunches = 2.0f;

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sumf(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// time of N runs of total length W, the longest p, P resident at once
__device__ __forceinline__ float pass_time(float N, float W, float pmax, float P) {
  if (N <= P) return pmax;
  return fmaxf(pmax, W / P + W / N);
}

// segment length (chunks) of a sequence of c chunks under the auto plan's m
__device__ __forceinline__ int balanced_len(int c, int m) {
  const int G = (c + m - 1) / m;
  return (c + G - 1) / G;
}

// Segment length of the auto plan (0: whole sequences), the same in every
// thread.  B <= 256 (the host enables the auto plan only when B H <= 256).
// Lane j of every wave evaluates candidate j (the longest sequence in j + 2
// segments) over the wave's share of the sequences; the shares meet once in
// LDS, where wave 0 prices the 64 candidates and picks the cheapest.
// The first pass's cost follows the negligible-transition rule: from 16
// sampled g of every (sequence, head) the plan estimates each sequence's
// decay per chunk (its weakest head's, in log2), with which an offset run
// covers only the chunks the rest of the segment does not wipe out and a
// transition run of a segment that decays below 2^-330 costs nothing (a
// margin over the kernels' 2^-300 for the sampling).  Without g, or with the
// key-norm term the sample cannot see, the estimate only misprices the plan;
// the kernels decide exactly.
constexpr int kAutoWaves = 4;
constexpr int kDecaySamples = 16;
constexpr float kPlanSkipLog2 = 330.f;
__device__ int auto_split_m(const PrefillParams& p) {
  __shared__ int cnt[256];
  __shared__ int dec_bits[256];  // per sequence: decay per chunk (log2, >= 0) as float bits
  __shared__ int part_i[kAutoWaves][6][64];
  __shared__ float part_f[kAutoWaves][64];
  __shared__ int chosen;
  const int B = p.num_seqs, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (B > 256) return 0;
  if (tid < B) cnt[tid] = chunks_of(p.slots.prefix[tid], p.cu_seqlens[tid + 1] - p.cu_seqlens[tid]);
  if (tid < 256) dec_bits[tid] = __float_as_int(3.0e38f);
  __syncthreads();
  if (tid < B * p.H) {  // one (sequence, head) pair a thread
    const int i = tid / p.H, h = tid - i * p.H;
    const int t0 = p.cu_seqlens[i], L = p.cu_seqlens[i + 1] - t0;
    float d = 0.f;
    if (p.g && L > 0) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < kDecaySamples; ++j) {
        const int t = t0 + (int)((int64_t)L * (2 * j + 1) / (2 * kDecaySamples));
        sum += p.g[(int64_t)t * p.H + h];
      }
      d = fmaxf(0.f, -sum * (float)kChunk * kLog2e / kDecaySamples);  // NaN -> 0
    }
    atomicMin(&dec_bits[i], __float_as_int(d));  // non-negative floats order as their bits
  }
  __syncthreads();
  if (wid < kAutoWaves) {
    int cmax = 0;
    for (int i = lane; i < B; i += 64) cmax = max(cmax, cnt[i]);
    cmax = wave_max(cmax);
    const int m = max(kSplitMinChunks, (cmax + lane + 1) / (lane + 2));  // candidate lane: lane + 2 segments
    int sg = 0, sg1 = 0, gmax = 0, p1 = 0, p2 = 0;
    float w1 = 0.f;
    for (int i = wid; i < B; i += kAutoWaves) {
      const int c = cnt[i];  // the same address in every lane: one broadcast read
      if (c <= 0) continue;
      const float d = __int_as_float(dec_bits[i]);
      const int sl = balanced_len(c, m);
      const int g = (c + sl - 1) / sl;
      sg += g;
      sg1 += g - 1;
      gmax = max(gmax, g);
      p2 = max(p2, sl);
      if (g > 1) {
        // first-pass run lengths: the offset's tail, the transition's whole segment or nothing
        const int koff = d > 1.f ? min(sl, (int)ceilf(kPlanSkipLog2 / d) + 1) : sl;
        const int kmap = d * sl > kPlanSkipLog2 ? 0 : sl;
        p1 = max(p1, max(koff, kmap));
        w1 += (float)((g - 1) * (koff + kmap));
      }
    }
    part_i[wid][0][lane] = sg;
    part_i[wid][1][lane] = sg1;
    part_i[wid][2][lane] = gmax;
    part_i[wid][3][lane] = p1;
    part_i[wid][4][lane] = p2;
    part_i[wid][5][lane] = cmax;
    part_f[wid][lane] = w1;
  }
  __syncthreads();
  if (wid == 0) {
    int sg = 0, sg1 = 0, gmax = 0, p1 = 0, p2 = 0, csum = 0, nact = 0;
    float w1 = 0.f;
#pragma unroll
    for (int w = 0; w < kAutoWaves; ++w) {
      sg += part_i[w][0][lane];
      sg1 += part_i[w][1][lane];
      gmax = max(gmax, part_i[w][2][lane]);
      p1 = max(p1, part_i[w][3][lane]);
      p2 = max(p2, part_i[w][4][lane]);
      w1 += part_f[w][lane];
    }
    const int cmax = part_i[0][5][lane];
    for (int i = lane; i < B; i += 64) {
      csum += cnt[i];
      nact += cnt[i] > 0;
    }
    csum = wave_sum(csum);
    nact = wave_sum(nact);
    const int m = max(kSplitMinChunks, (cmax + lane + 1) / (lane + 2));
    const float P = fmaxf(1.f, (float)(p.num_cus * p.tile_waves / 8));
    const float H = (float)p.H;
    const float rounds_scan = ceilf(8.f * B * p.H / fmaxf(1.f, (float)p.num_cus));
    const float whole = pass_time(H * nact, H * csum, (float)cmax, P);
    float cost = whole;
    if (m < cmax && sg <= p.seg_cap2 && 2 * sg1 <= p.seg_cap1)
      cost = kCostPass1 * pass_time(2.f * H * sg1, H * w1, (float)p1, P) +
             kCostScanStep * (gmax - 1) * rounds_scan + pass_time(H * sg, H * csum, (float)p2, P) +
             kCostLaunches;
    // cheapest candidate (ties: the longer segments), whole sequences unless one beats them
    float best = cost < whole ? cost : whole;
    int bm = cost < whole ? m : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ob = __shfl_xor(best, off, 64);
      const int om = __shfl_xor(bm, off, 64);
      if (ob < best || (ob == best && om > bm)) {
        best = ob;
        bm = om;
      }
    }
    if (lane == 0) chosen = bm;
  }
  __syncthreads();
  return chosen;
}

__device__ void split_plan(const PrefillParams& p) {
  const int m = p.split_mode == kSplitAuto ? auto_split_m(p) : p.split_m;
  const int B = p.num_seqs;
  int carry1 = 0, carry2 = 0, carry_row = 0;
  for (int base = 0; base < B; base += blockDim.x) {
    const int b = base + (int)threadIdx.x;
    int L = 0, pre = 0, G = 0, mm = 1;  // mm: this sequence's segment length (chunks)
    if (b < B) {
      L = p.cu_seqlens[b + 1] - p.cu_seqlens[b];
      pre = p.slots.prefix[b];
      const int c = chunks_of(pre, L);
      if (m > 0 && c > 0) mm = p.split_mode == kSplitAuto ? balanced_len(c, m) : m;
      G = L <= 0 ? 0 : m > 0 ? (c + mm - 1) / mm : 1;
    }
    const int n1 = G > 1 ? G - 1 : 0, n2 = G, nrow = G > 1 ? 3 * G - 2 : 0;
    int t1, t2, trow;
    const int o1 = carry1 + block_exclusive_scan(n1, &t1);
    const int o2 = carry2 + block_exclusive_scan(n2, &t2);
    const int row0 = carry_row + block_exclusive_scan(nrow, &trow);
    if (b < B) {
      p.seg_scan[b] = int4{G, row0, 0, 0};
      const int tok0 = p.cu_seqlens[b], cs = p.slots.chunk_start[b];
      const int rd = p.slots.read[b], wr = p.slots.write[b];
      const int ckb = p.ckpt_idx ? p.slots.ckpt_start[b] : 0;
      const int nbase = (pre & ~(kChunk - 1)) - pre;
      auto lo = [&](int g) { return g == 0 ? 0 : nbase + kChunk * mm * g; };
      auto hi = [&](int g) { return G == 1 ? L : min(L, nbase + kChunk * mm * (g + 1)); };
      auto put = [](int32_t* d, int a, int b_, int c, int e, int f, int g_, int h, int i) {
        d[0] = a; d[1] = b_; d[2] = c; d[3] = e; d[4] = f; d[5] = g_; d[6] = h; d[7] = i;
      };
      // offset runs in the first half of the first pass's records, transition
      // runs in the second: the offsets, which do the work, are dispatched first
      const int half = p.seg_cap1 / 2;
      for (int g = 0; g <= G - 2; ++g) {
        const int a = lo(g), n = hi(g) - a;
        put(p.seg1 + kSegWords * (o1 + g), tok0 + a, n, pre + a, cs + g * mm, -1,
            -2 - (row0 + G + g), 0, kSegOffset);
        put(p.seg1 + kSegWords * (half + o1 + g), tok0 + a, n, pre + a, cs + g * mm, -1,
            -2 - (row0 + 2 * G - 1 + g), 0, kSegMap);
      }
      for (int g = 0; g <= G - 1; ++g) {
        const int a = lo(g), n = hi(g) - a;
        const int ck = p.ckpt_idx ? ckb + (pre + a) / p.ckpt_every - pre / p.ckpt_every : 0;
        put(p.seg2 + kSegWords * (o2 + g), tok0 + a, n, pre + a, cs + g * mm,
            G == 1 ? rd : -2 - (row0 + g), g == G - 1 ? wr : -1, ck, kSegNormal);
      }
    }
    carry1 += t1;
    carry2 += t2;
    carry_row += trow;
  }
  if (threadIdx.x == 0) {
    p.seg_counts[0] = carry1;
    p.seg_counts[1] = carry2;
  }
}

// The launch plan, and with the sequence-parallel recurrence its segment
// plan too (the two read the slot rows only, not each other's output): one
// workgroup of kPlanTile threads, one launch.
__global__ __launch_bounds__(kPlanTile) void plan_kernel(const PrefillParams p) {
  if (guarded(p.guard)) return;
  plan_body(p.cu_seqlens, p.slots.prefix, p.slots.chunk_start, p.num_seqs, p.num_chunk_slots,
            p.order, p.chunk_tab, (uint32_t*)p.zero_row);
  if (p.split_mode != kSplitOff) split_plan(p);
}

// start_{g+1} = start_g M_g + N_g for g = 0 .. G-2, 16 state rows of one
// (sequence, v-head) per workgroup: rows of a state evolve independently, so
// the 8 row blocks of a head run in parallel.  The transitions M_g (64 KiB
// each) stream into LDS straight from global memory, double-buffered (the
// next one lands while this one multiplies); the current rows stay in LDS.
// M_g as row pairs (2 x 128 floats, one global-to-LDS load each) 16 bytes
// apart from the next pair, so that the four lane groups of an operand read
// (rows 8 apart) fall in different banks; double-buffered by step parity.
constexpr int kPairPitch = 2 * kDim + 4;
struct ScanSmem {
  float M[2][kDim / 2][kPairPitch];
  float S[16][kDim + 4];  // the workgroup's 16 rows of start_g
};

// Workgroup (sequence, v-head, rb) composes rows 16 rb .. 16 rb + 15 of the
// segment start states: start_{g+1} = start_g M_g + N_g, g = 0 .. G - 2.  The
// product runs on MFMA with fp32 operands split hi/lo (3 passes, ~2^-16
// relative): wave w produces columns 32 w .. 32 w + 31 (two 16 x 16 tiles),
// the output's lane (n, q) holding rows 4q .. 4q + 3 of column n.  The 8
// workgroups of a (sequence, v-head) sit 8 block indices apart -- the same
// XCD -- so that 7 of the 8 reads of each M_g hit in that XCD's L2.
__global__ __launch_bounds__(256) void seg_scan_kernel(const PrefillParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  ScanSmem& sm = *reinterpret_cast<ScanSmem*>(smem_raw);
  if (guarded(p.guard)) return;
  const int j = blockIdx.x;
  const int rb = (j >> 3) & 7, bh = 8 * (j >> 6) + (j & 7);
  if (bh >= p.num_seqs * p.H) return;  // the last group of 8 heads may be partial
  const int b = bh / p.H, h = bh - b * p.H;
  const int4 sc = p.seg_scan[b];
  const int G = sc.x, row0 = sc.y;
  if (G < 2) return;  // a whole sequence: nothing to compose
  const int rd = p.slots.read[b];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, gq = lane >> 4;
  const int r = tid >> 4, c0 = 4 * (tid & 15);
  const int64_t hoff = (int64_t)h * kDim * kDim;
  auto state = [&](int row) { return p.ws_state + (int64_t)row * p.ws_state_stride + hoff; };
  // M_g into buffer X: 64 row pairs of 1 KiB, 16 per wave
  auto fetch = [&](int g, int X) {
    const char* src = uniform_ptr(state(row0 + 2 * G - 1 + g));
    const uint32_t dst = lds_addr(&sm.M[X][0][0]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int blk = 16 * wid + i;
      lds_load16_at<false>(dst + blk * (kPairPitch * 4), src + blk * 1024, lane * 16);
    }
  };
  fetch(0, 0);
  // start_0: the sequence's initial state (a row of the caller's buffer or zero)
  f32x4 i0 = {0.f, 0.f, 0.f, 0.f}, i1 = i0;
  if (rd >= 0 && p.init) {
    const int64_t off = (int64_t)rd * p.init_stride + hoff + (int64_t)(16 * rb + r) * kDim;
    if (p.state_bf16) {
      const u16* s0 = (const u16*)p.init + off;
      const u32x2 w0 = *(const u32x2*)(s0 + c0), w1 = *(const u32x2*)(s0 + 64 + c0);
      i0 = f32x4{__uint_as_float(w0.x << 16), __uint_as_float(w0.x & 0xffff0000u),
                 __uint_as_float(w0.y << 16), __uint_as_float(w0.y & 0xffff0000u)};
      i1 = f32x4{__uint_as_float(w1.x << 16), __uint_as_float(w1.x & 0xffff0000u),
                 __uint_as_float(w1.y << 16), __uint_as_float(w1.y & 0xffff0000u)};
    } else {
      const float* s0 = (const float*)p.init + off;
      i0 = *(const f32x4*)(s0 + c0);
      i1 = *(const f32x4*)(s0 + 64 + c0);
    }
  }
  *(f32x4*)&sm.S[r][c0] = i0;
  *(f32x4*)&sm.S[r][64 + c0] = i1;
  // start_0 into the workspace: the second pass reads it there, never the
  // caller's row, which that pass may overwrite
  {
    float* s0 = state(row0) + (int64_t)(16 * rb + r) * kDim;
    *(f32x4*)(s0 + c0) = i0;
    *(f32x4*)(s0 + 64 + c0) = i1;
  }
  wait_loads();
  __syncthreads();
  for (int g = 0; g <= G - 2; ++g) {
    const int X = g & 1;
    if (g + 1 <= G - 2) fetch(g + 1, X ^ 1);
    // this lane's outputs: rows 4 gq + i, columns 32 wid + 16 t + n16; N_g is
    // added after the product, so its loads are in flight meanwhile
    const float* Ng = state(row0 + G + g) + (int64_t)(16 * rb) * kDim + 32 * wid + n16;
    float nv[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) nv[t][i] = Ng[(4 * gq + i) * kDim + 16 * t];
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 32 * ks + 8 * gq;  // this lane's 8 k of the step
      float av[8];
      *(f32x4*)&av[0] = *(const f32x4*)&sm.S[n16][k0];
      *(f32x4*)&av[4] = *(const f32x4*)&sm.S[n16][k0 + 4];
      bf16x8 ahi, alo;
      split8(av, ahi, alo);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int n = 32 * wid + 16 * t + n16;
        float bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = sm.M[X][(k0 + j) >> 1][((k0 + j) & 1) * kDim + n];
        bf16x8 bhi, blo;
        split8(bv, bhi, blo);
        acc[t] = mfma16x16x32(ahi, bhi, acc[t]);
        acc[t] = mfma16x16x32(ahi, blo, acc[t]);
        acc[t] = mfma16x16x32(alo, bhi, acc[t]);
      }
    }
    float* out = state(row0 + g + 1) + (int64_t)(16 * rb) * kDim + 32 * wid + n16;  // start_{g+1}
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[t][i] += nv[t][i];
        out[(4 * gq + i) * kDim + 16 * t] = acc[t][i];
      }
    __syncthreads();  // every wave is done reading S and M[X]
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.S[4 * gq + i][32 * wid + 16 * t + n16] = acc[t][i];
    wait_loads();     // this wave's part of the next M has landed
    __syncthreads();  // ... and every wave's; the new rows are in place
  }
}

}  // namespace

// The dynamic-LDS limit of a kernel is raised once per device (the
// attribute belongs to the device's copy of the kernel); idempotent if two
// threads race.
// Once per kernel and device (threads that race here both set it: harmless).
static bool raise_lds_limit(const void* fn, int bytes, std::atomic<bool> (&done)[kMaxDevices],
                            hipError_t* err) {
  const int dev = current_device();
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire)) return true;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) {
    *err = e;
    return false;
  }
  if (dev >= 0 && dev < kMaxDevices) done[dev].store(true, std::memory_order_release);
  return true;
}

template <int NW, bool OUT>
hipError_t launch_rec(const PrefillParams& p, int64_t blocks, hipStream_t s) {
  static std::atomic<bool> done[kMaxDevices];
  hipError_t e = hipSuccess;
  if (!raise_lds_limit((const void*)rec_kernel<NW, OUT>, (int)sizeof(RecSmem), done, &e)) return e;
  rec_kernel<NW, OUT><<<(unsigned)blocks, NW * 64, sizeof(RecSmem), s>>>(p);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int64_t num_chunk_slots, hipStream_t s) {
  const int64_t blocks = (int64_t)p.num_seqs * p.H;
  if (blocks <= 0 || num_chunk_slots <= 0) return hipSuccess;
  const bool split = p.split_mode != kSplitOff;
  if (split && (p.seg_cap1 <= 0 || p.seg_cap2 <= 0)) return hipErrorInvalidValue;
  plan_kernel<<<1, kPlanTile, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  wy_kernel<<<(unsigned)((num_chunk_slots + 7) / 8 * 8 * p.H), kWyThreads, 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Whole heads per workgroup (8 waves) by default.  Narrower V-tiles (4, 2
  // or 1 waves) add workgroups but not speed: each still walks every chunk of
  // its sequence, and the per-chunk time is set by the chunk's dependency
  // chain, which fewer waves only lengthen (measured: a 32k-token single
  // sequence, 32 heads, takes 2.28 / 2.32 / 2.68 / 3.69 ms with 8 / 4 / 2 / 1
  // waves).
  const int nw = p.tile_waves;
  auto rec = [&](const PrefillParams& q, int64_t items, bool out) {
    switch (nw * 2 + out) {
      case 17: return launch_rec<8, true>(q, items * p.H, s);
      case 16: return launch_rec<8, false>(q, items * p.H, s);
      case 9: return launch_rec<4, true>(q, items * p.H * 2, s);
      case 8: return launch_rec<4, false>(q, items * p.H * 2, s);
      case 5: return launch_rec<2, true>(q, items * p.H * 4, s);
      case 4: return launch_rec<2, false>(q, items * p.H * 4, s);
      case 3: return launch_rec<1, true>(q, items * p.H * 8, s);
      case 2: return launch_rec<1, false>(q, items * p.H * 8, s);
      default: return hipErrorInvalidValue;
    }
  };
  if (!split) return rec(p, p.num_seqs, true);
  // sequence-parallel (its segment plan came with the launch plan): first
  // pass, scan of the segment maps, second pass
  PrefillParams p1 = p;
  p1.vseq = p.seg1;
  p1.vcount = p.seg_counts;
  p1.vhalf = p.seg_cap1 / 2;
  if ((e = rec(p1, p.seg_cap1, false)) != hipSuccess) return e;
  {
    static std::atomic<bool> done[kMaxDevices];
    if (!raise_lds_limit((const void*)seg_scan_kernel, (int)sizeof(ScanSmem), done, &e)) return e;
  }
  seg_scan_kernel<<<(unsigned)(((int64_t)p.num_seqs * p.H + 7) / 8 * 64), 256, sizeof(ScanSmem), s>>>(p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  PrefillParams p2 = p;
  p2.vseq = p.seg2;
  p2.vcount = p.seg_counts + 1;
  return rec(p2, p.seg_cap2, true);
}

}  // namespace gdn
