// Internal definitions shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kDim = 128;    // K = V

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Per-sequence rows every prefill kernel consumes (device arrays, [B] int32).
struct SlotsDev {
  const int32_t* read;        // initial-state row, -1 = zero state
  const int32_t* write;       // final-state row, -1 = no store
  const int32_t* ckpt_start;  // offset of this call's first checkpoint row
  const int32_t* prefix;      // tokens before the call (chunk alignment)
  const int32_t* chunk_start; // exclusive scan of chunk counts
};

constexpr int kFragElems = 64 * 8;  // one 16x16x32 MFMA operand fragment, bf16 elements

// Per (chunk slot, v-head) record the intra-chunk kernel hands to the
// recurrence: T diag(beta), T = (I + A)^-1, as 5 hi and 5 lo bf16 operand
// fragments (its 6 nonzero ones, two half-empty ones sharing one), and the
// per-row scalars beta, G (log2 units), gamma = 2^G, exp(G_last - G).
constexpr int kRecWords = 2 * 5 * kFragElems;  // bf16 elements (10 KiB)
constexpr int kRecScal = 4 * kChunk;           // floats (1 KiB)

// Sequence-parallel recurrence (long sequences in batches too small to fill
// the chip): every sequence's chunks are cut into segments of m chunks, and
// the recurrence runs over segment records of kSegWords int32 each
// {first token, tokens, prefix (absolute position of the segment's start),
// first chunk slot, read row, write row, first checkpoint index, mode}.
// Rows: >= 0 a row of the caller's state buffers, -1 none (zero state / no
// store), <= -2 row (-2 - r) of the workspace's segment states.
// split_mode: off (whole sequences, one recurrence launch), forced (segments
// of split_m chunks) or auto (the plan kernel picks m, or no split, from the
// batch's chunk counts).
constexpr int kSplitOff = 0;
constexpr int kSplitForced = 1;
constexpr int kSplitAuto = 2;
constexpr int kSplitMinChunks = 4;  // shortest segment the auto plan considers
constexpr int kSplitMaxPerHead = 512;  // auto plan: segments <= kSplitMaxPerHead / H + B
constexpr int kSegWords = 8;
constexpr int kSegNormal = 0;  // a real run: outputs, checkpoints, final state
constexpr int kSegOffset = 1;  // from the zero state, no outputs: the segment's offset N
constexpr int kSegMap = 2;     // from the identity with v = 0, no outputs: its transition M

struct PrefillParams {
  const u16* q;
  const u16* k;
  const u16* v;
  const float* g;
  const float* beta;
  u16* o;
  const int32_t* cu_seqlens;
  SlotsDev slots;
  int32_t* order;  // [B] workspace: sequences longest first
  int4* chunk_tab; // [chunk slots] workspace: {sequence (-1: unused), new-token index of row 0, L, first token}
  int num_chunk_slots;
  u16* ws_T;       // [chunk slots][H][kRecWords]
  float* ws_scal;  // [chunk slots][H][kRecScal]
  u16* zero_row;   // 256 bytes (workspace), zeroed by the order kernel; read for padding rows
  int num_seqs;
  int H;
  int Hqk;
  int group;  // H / Hqk
  float scale;
  // state buffers: fp32, or bf16 when state_bf16 (strides in elements)
  int state_bf16;
  const void* init;
  int64_t init_stride;
  void* out;
  int64_t out_stride;
  void* ckpt;
  int64_t ckpt_stride;
  const void* ckpt_idx;
  int ckpt_idx64;
  int ckpt_every;
  // sequence-parallel recurrence
  int split_mode;          // kSplitOff / kSplitForced / kSplitAuto
  int split_m;             // forced segment length (chunks)
  int num_cus;             // compute units of the device (auto plan's cost model)
  int tile_waves;          // waves per recurrence workgroup (8: whole heads)
  int seg_cap1, seg_cap2;  // segment records the two passes have room for
  int32_t* seg1;           // [seg_cap1][kSegWords] first pass (workspace)
  int32_t* seg2;           // [seg_cap2][kSegWords] second pass (workspace)
  int4* seg_scan;          // [B] {segments, first workspace state row, -, -}
  int32_t* seg_counts;     // [2] first pass: offset runs (as many transition runs); second pass: runs
  float* ws_state;         // workspace states, rows of H * V * K floats
  float* ws_bound;         // [chunk slots][H] log2 bound on the norm of each chunk's transition
                           // (sequence-parallel calls; null otherwise)
  int64_t ws_state_stride;
  const int32_t* vseq;     // the records this launch walks (null: whole sequences)
  const int32_t* vcount;   // how many of them are real
  int vhalf;               // > 0: the records are two halves of vhalf (offset runs, then
                           // transition runs), each with *vcount real ones at its start
  const int32_t* guard;    // debug check word (null: none); nonzero error bits: return at once
};

struct DecodeParams {
  const u16* q;
  const u16* k;
  const u16* v;
  const float* g;
  const float* beta;
  u16* o;
  int num_seqs;
  int H;
  int Hqk;
  int group;
  float scale;
  // Rows: mode 0 = explicit index arrays (may be null: row b / the read row),
  // mode 1 = derived from the page table inside the kernel.
  int mode;
  const void* rd_idx;
  const void* wr_idx;
  int idx64;
  const int32_t* page_indices;
  const int32_t* page_indptr;
  const int32_t* last_page_len;
  // state buffers: fp32, or bf16 when state_bf16 (strides in elements)
  int state_bf16;
  const void* init;
  int64_t init_stride;
  void* out;
  int64_t out_stride;
  const int32_t* guard;  // debug check word (null: none); nonzero error bits: return at once
};

// Launchers (return hipError_t of the launch).
hipError_t launch_prefill_slots(const int32_t* cu, const int32_t* idx, const int32_t* ptr,
                                const int32_t* lpl, int B, int page_size, int32_t* read,
                                int32_t* write, int32_t* ckpt, int32_t* prefix,
                                int32_t* chunk_start, const int32_t* guard, hipStream_t s);
hipError_t launch_decode_slots(const int32_t* idx, const int32_t* ptr, const int32_t* lpl,
                               int B, int32_t* read, int32_t* write, hipStream_t s);
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t s);
hipError_t launch_check_paged(const int32_t* cu, const int32_t* idx, const int32_t* ptr,
                              const int32_t* lpl, int B, int page_size, int num_pages,
                              int32_t* word, hipStream_t s);
hipError_t launch_general_slots(const int32_t* cu, int B, const void* sidx, const void* oidx,
                                const void* cstart, const void* plen, int idx64, int has_init,
                                int write_final, int32_t* read, int32_t* write, int32_t* ckpt,
                                int32_t* prefix, int32_t* chunk_start, hipStream_t s);
hipError_t launch_block_table_to_csr(const int32_t* table, int64_t row_stride, const int32_t* ctx,
                                     int B, int max_blocks, int ps, int32_t* indptr,
                                     int32_t* indices, int32_t* lpl, int32_t* bad,
                                     hipStream_t s);
hipError_t launch_csr_to_block_table(const int32_t* indptr, const int32_t* indices,
                                     const int32_t* lpl, int B, int ps, int max_blocks,
                                     int32_t* table, int64_t row_stride, int32_t* ctx,
                                     int32_t* bad, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, int64_t num_chunk_slots, hipStream_t s);
// Decode launch shape (all 0: the default; see gdn_options_t).
struct DecodeShape {
  int waves;       // one-pair kernel width (2, 4, 8, 16), 0 = default
  int stream_per_cu;  // streaming workgroups per compute unit, 0 = default, -1 = off
  int stream_grid;    // streaming grid, 0 = from stream_per_cu
};
hipError_t launch_decode(const DecodeParams& p, const DecodeShape& shape, hipStream_t s);

// Compute units of the current device (queried once per device).
int device_cus();
// Index of the current device, or -1 (for per-device caches of size kMaxDevices).
constexpr int kMaxDevices = 64;
int current_device();

// ---------------------------------------------------------------- device helpers
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float(uint32_t(b) << 16); }

// A debug check word holding an error (any bit but "not checked", 32): the
// kernels of a checked call then return before touching memory.
__device__ __forceinline__ bool guarded(const int32_t* g) { return g && (*g & ~32) != 0; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ u16 f2bf(float x) { return __builtin_bit_cast(u16, (__bf16)x); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ uint32_t pack2(u16 lo, u16 hi) {
  return uint32_t(lo) | (uint32_t(hi) << 16);
}

// Split 8 fp32 values into bf16 hi + lo parts (x ~= hi + lo to ~2^-17).
// x = hi + lo with hi = bf16(x) (round to nearest) and lo = bf16(x - hi);
// x - hi is exact in fp32.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = f2bf2(x[2 * i], x[2 * i + 1]);
    h[i] = w;
    l[i] = f2bf2(x[2 * i] - __uint_as_float(w << 16), x[2 * i + 1] - __uint_as_float(w & 0xffff0000u));
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

// Round 8 fp32 values to bf16 (single part).
__device__ __forceinline__ bf16x8 round8(const float* x) {
  u32x4 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = f2bf2(x[2 * i], x[2 * i + 1]);
  return as_bf16x8(h);
}

// Workgroup-wide exclusive scan of one int per thread (blockDim.x a multiple of
// 64, at most 1024); *total receives the workgroup's sum.  Every thread must
// call it (it synchronizes the workgroup).
__device__ inline int block_exclusive_scan(int x, int* total) {
  __shared__ int wsum[16];
  __shared__ int tot;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = wsum[w];
      wsum[w] = run;
      run += t;
    }
    tot = run;
  }
  __syncthreads();
  const int out = wsum[wid] + incl - x;
  *total = tot;
  __syncthreads();  // wsum / tot are reused by the next call
  return out;
}

// Row index, within a 64-row operand, of slot j (0..7) of lane group gq (0..3)
// at k-step ks (0..1 for 64, 0..3 for 128) under the permuted reduction order
// shared by every operand that comes out of an accumulator: row blocks
// 2ks and 2ks+1, four consecutive rows at 4*gq.
__device__ __forceinline__ int perm_row(int ks, int gq, int j) {
  return 32 * ks + 16 * (j >> 2) + 4 * gq + (j & 3);
}

#endif

}  // namespace gdn
