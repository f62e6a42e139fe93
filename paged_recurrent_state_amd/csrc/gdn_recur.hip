// Inter-chunk state recurrence of chunked Gated Delta-Rule prefill.
//
// One wave per (sequence, v-head, 16-row slice of the state).  Rows of S
// evolve independently (every update multiplies S on the right), so a slice
// needs only its own rows.  The fp32 slice S[16, 128] stays in the MFMA
// accumulators for the whole sequence, stored transposed (lane holds column v,
// rows k), which is exactly the layout the next chunk needs as a B operand.
//
// Per chunk, with T, P, beta, gamma, dec = exp(G_last - G) from the
// intra-chunk kernel:
//   Y = K S^T, Z = Q S^T                 (bf16 K, Q exact; S split hi + lo)
//   R = diag(beta) (V - diag(gamma) Y)
//   E = T R                              (both split: 3 MFMA passes)
//   O = scale (diag(gamma) Z + P E)      (3 passes)
//   S <- gamma_last S + (diag(dec) E)^T K   (K exact; E split)
// then the state is stored when the chunk ends on a checkpoint position
// (pages: flashinfer.gdn_paged "Page table"; checkpoints: "Slot arguments",
// checkpoint_state_indices / prefix_lens) and after the last chunk to the
// write row.  A read row of -1 starts from literal zeros.
//
// Operands that come out of an accumulator are used in place: accumulator
// rows 4*gq + r of two consecutive 16-row blocks form one 32-deep k-step, and
// the operand loaded from memory uses the same row order (perm_row).
#include "gdn_internal.h"

namespace gdn {

namespace {

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

__global__ __launch_bounds__(64) void recur_kernel(const RecurParams p) {
  const int lane = threadIdx.x;
  const int n16 = lane & 15;
  const int gq = lane >> 4;
  // blockIdx -> (pair, slice): the 8 slices of one (sequence, head) pair share
  // the pair's low 3 bits, i.e. land on the same XCD and share its L2.
  const int bid = blockIdx.x;
  const int slice = (bid >> 3) & (kVSlices - 1);
  const int pair = ((bid >> 6) << 3) | (bid & 7);
  if (pair >= p.num_seqs * p.H) return;
  const int b = pair / p.H;
  const int h = pair - b * p.H;
  const int tok0 = p.cu_seqlens[b];
  const int L = p.cu_seqlens[b + 1] - tok0;
  if (L <= 0) return;  // a zero-length sequence writes nothing
  const int pre = p.slots.prefix[b];
  const int nch = ((pre & (kChunk - 1)) + L + kChunk - 1) / kChunk;
  const int cs0 = p.slots.chunk_start[b];
  const int rd = p.slots.read[b];
  const int wr = p.slots.write[b];
  const int hq = h / p.group;
  const int vrow = slice * kVSlice + n16;
  const int64_t head_off = ((int64_t)h * kDim + vrow) * kDim + 4 * gq;

  f32x4 accS[8];
  if (rd >= 0 && p.init) {
    const float* src = p.init + (int64_t)rd * p.init_stride + head_off;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) accS[mb] = *(const f32x4*)(src + 16 * mb);
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) accS[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int ci = 0; ci < nch; ++ci) {
    const int c = cs0 + ci;
    const int n0 = (pre & ~(kChunk - 1)) + kChunk * ci - pre;  // new-token index of row 0
    const int64_t ch = (int64_t)c * p.H + h;
    const float* sc = p.ws.scal + ch * kScal;
    const u16* Tw = p.ws.T + ch * kMatWords;
    const u16* Pw = p.ws.P + ch * kMatWords;
    const u16* Kw = p.ws.Kt + ((int64_t)c * p.Hqk + hq) * kKtWords;

    // ---- loads that do not depend on the state, issued up front.  Rows
    // outside the sequence read token 0 of the sequence (always in bounds)
    // and are zeroed by select, so no load sits behind a branch.
    u32x4 ka[4][4], qa[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int n = n0 + 16 * mt + n16;
      const bool valid = (unsigned)n < (unsigned)L;
      const int64_t off = (((int64_t)tok0 + (valid ? n : 0)) * p.Hqk + hq) * kDim + 4 * gq;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x2 k0 = *(const u32x2*)(p.k + off + 32 * ks);
        const u32x2 k1 = *(const u32x2*)(p.k + off + 32 * ks + 16);
        const u32x2 q0 = *(const u32x2*)(p.q + off + 32 * ks);
        const u32x2 q1 = *(const u32x2*)(p.q + off + 32 * ks + 16);
        const u32x4 z = {0u, 0u, 0u, 0u};
        ka[mt][ks] = valid ? u32x4{k0.x, k0.y, k1.x, k1.y} : z;
        qa[mt][ks] = valid ? u32x4{q0.x, q0.y, q1.x, q1.y} : z;
      }
    }
    float vv[4][4];
    f32x4 bet[4], gam[4], dec[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      bet[mt] = *(const f32x4*)(sc + 16 * mt + 4 * gq);
      gam[mt] = *(const f32x4*)(sc + kChunk + 16 * mt + 4 * gq);
      dec[mt] = *(const f32x4*)(sc + 2 * kChunk + 16 * mt + 4 * gq);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 16 * mt + 4 * gq + r;
        const bool valid = (unsigned)n < (unsigned)L;
        const float x = bf2f(p.v[(((int64_t)tok0 + (valid ? n : 0)) * p.H + h) * kDim + vrow]);
        vv[mt][r] = valid ? x : 0.f;
      }
    }
    const float gC = sc[kChunk + kChunk - 1];
    bf16x8 th[8], tl[8], ph[8], pl[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      th[f] = *(const bf16x8*)(Tw + (f * 64 + lane) * 8);
      tl[f] = *(const bf16x8*)(Tw + kTFragsPerMat * kFragElems + (f * 64 + lane) * 8);
      ph[f] = *(const bf16x8*)(Pw + (f * 64 + lane) * 8);
      pl[f] = *(const bf16x8*)(Pw + kTFragsPerMat * kFragElems + (f * 64 + lane) * 8);
    }

    // ---- Y = K S^T, Z = Q S^T
    bf16x8 Shi[4], Slo[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = accS[2 * ks + (j >> 2)][j & 3];
      split8(v, Shi[ks], Slo[ks]);
    }
    f32x4 accY[4], accZ[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      accY[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accZ[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ak = as_bf16x8(ka[mt][ks]), aq = as_bf16x8(qa[mt][ks]);
        accY[mt] = mfma16x16x32(ak, Shi[ks], accY[mt]);
        accY[mt] = mfma16x16x32(ak, Slo[ks], accY[mt]);
        accZ[mt] = mfma16x16x32(aq, Shi[ks], accZ[mt]);
        accZ[mt] = mfma16x16x32(aq, Slo[ks], accZ[mt]);
      }
    }

    // ---- R = beta (V - gamma Y), O = gamma Z
    f32x4 R[4], O[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        R[mt][r] = bet[mt][r] * (vv[mt][r] - gam[mt][r] * accY[mt][r]);
        O[mt][r] = gam[mt][r] * accZ[mt][r];
      }

    // ---- E = T R
    bf16x8 Rhi[2], Rlo[2];
    split_rows(R, 0, Rhi[0], Rlo[0]);
    split_rows(R, 1, Rhi[1], Rlo[1]);
    f32x4 E[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      E[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int f = mt * 2 + ks;
        E[mt] = mfma16x16x32(th[f], Rhi[ks], E[mt]);
        E[mt] = mfma16x16x32(th[f], Rlo[ks], E[mt]);
        E[mt] = mfma16x16x32(tl[f], Rhi[ks], E[mt]);
      }
    }

    // ---- O += P E, store o
    bf16x8 Ehi[2], Elo[2];
    split_rows(E, 0, Ehi[0], Elo[0]);
    split_rows(E, 1, Ehi[1], Elo[1]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int f = mt * 2 + ks;
        O[mt] = mfma16x16x32(ph[f], Ehi[ks], O[mt]);
        O[mt] = mfma16x16x32(ph[f], Elo[ks], O[mt]);
        O[mt] = mfma16x16x32(pl[f], Ehi[ks], O[mt]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 16 * mt + 4 * gq + r;
        if ((unsigned)n < (unsigned)L)
          p.o[(((int64_t)tok0 + n) * p.H + h) * kDim + vrow] = f2bf(p.scale * O[mt][r]);
      }
    }

    // ---- S <- gamma_last S + (dec E)^T K
    f32x4 Ed[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Ed[mt][r] = dec[mt][r] * E[mt][r];
    bf16x8 Dhi[2], Dlo[2];
    split_rows(Ed, 0, Dhi[0], Dlo[0]);
    split_rows(Ed, 1, Dhi[1], Dlo[1]);
#pragma unroll
    for (int mk = 0; mk < 8; ++mk) {
      accS[mk] = accS[mk] * gC;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int f = mk * 2 + ks;
        const bf16x8 kt = *(const bf16x8*)(Kw + (f * 64 + lane) * 8);
        accS[mk] = mfma16x16x32(kt, Dhi[ks], accS[mk]);
        accS[mk] = mfma16x16x32(kt, Dlo[ks], accS[mk]);
      }
    }

    // ---- checkpoint at this chunk's end?
    if (p.ckpt_idx) {
      const int pos = (pre & ~(kChunk - 1)) + kChunk * (ci + 1);
      if (pos % p.ckpt_every == 0 && pos > pre && pos <= pre + L) {
        const int j = pos / p.ckpt_every - pre / p.ckpt_every - 1;
        const int64_t row = ld_index(p.ckpt_idx, p.slots.ckpt_start[b] + j, p.ckpt_idx64);
        if (row >= 0) store_state(p.ckpt + row * p.ckpt_stride + head_off, accS);
      }
    }
  }
  if (wr >= 0 && p.out) store_state(p.out + (int64_t)wr * p.out_stride + head_off, accS);
}

}  // namespace

hipError_t launch_recur(const RecurParams& p, hipStream_t s) {
  const int64_t pairs = (int64_t)p.num_seqs * p.H;
  if (pairs <= 0) return hipSuccess;
  const int64_t blocks = ((pairs + 7) / 8) * 8 * kVSlices;
  recur_kernel<<<(unsigned)blocks, 64, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace gdn
