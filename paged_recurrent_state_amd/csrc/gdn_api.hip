// C-ABI entry points: argument checks, workspace carving and launches.
// Every host-checkable error returns before any launch; nothing here
// synchronizes with the device or allocates memory.
#include "gdn_paged.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "gdn_internal.h"

using namespace gdn;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return GDN_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GDN_ELAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return GDN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: the per-sequence rows (5 x [B] int32), the launch order ([B]),
// 256 bytes of zeros (read for padding rows), the chunk-slot table ([slots]
// x 16 bytes) and, per (chunk slot, v-head), the intra-chunk record (T
// fragments + scalars).
// A sequence with L new tokens spans ceil(((prefix mod 64) + L) / 64) <=
// (L + 126) / 64 chunks, so a batch never has more than T / 64 + 2 B of them.
// With the sequence-parallel recurrence it also holds the segment records of
// both passes, the per-sequence scan records and the segment states (a
// sequence of G >= 2 segments keeps 3 G - 2 states: its G start states and
// the offset and transition of every segment but the last; rows of H * V * K
// floats), room for `segs` segments.
struct WsLayout {
  int64_t nc;
  int split_mode, split_m;
  int64_t cap1, cap2, rows;
  size_t slots, order, zero, tab, T, scal, seg1, seg2, scan, counts, states, bound, total;
};

// Launch choices of a call, from dims->options (NULL: all defaults).
struct Opts {
  int split;   // gdn_options_t.prefill_split_chunks
  int waves;   // recurrence workgroup width
  DecodeShape dec;
  int32_t* check;  // debug check word (null: no check)
  int check_pages;
};

Opts get_opts(const gdn_dims_t* d) {
  Opts o{0, 8, DecodeShape{0, 0, 0}, nullptr, 0};
  if (d && d->options) {
    const gdn_options_t* x = d->options;
    o.split = x->prefill_split_chunks;
    o.waves = x->prefill_tile_waves ? x->prefill_tile_waves : 8;
    o.dec = DecodeShape{x->decode_waves, x->decode_stream_per_cu, x->decode_stream_grid};
    o.check = x->check_error_word;
    o.check_pages = x->check_num_pages;
  }
  return o;
}

// The auto plan is possible when the batch's (sequence, head) pairs fill the
// compute units at most once and there are enough tokens for a sequence of
// 16 chunks; its segments are bounded by kSplitMaxPerHead / H + B (beyond
// that, the second pass alone would take several rounds of the chip) and by
// chunks / kSplitMinChunks + B.
constexpr int64_t kAutoMinTokens = 16 * kChunk;
bool auto_allowed(int64_t T, int64_t B, int H) {
  return B >= 1 && B * H <= 256 && T >= kAutoMinTokens;
}
int64_t auto_segments(int64_t T, int64_t B, int H) {
  const int64_t nc = T / kChunk + 2 * B + 1;
  return std::min<int64_t>(nc / kSplitMinChunks + B, kSplitMaxPerHead / H + B);
}

// Workspace regions for a call of T tokens in B sequences.  With `bound`,
// the sequence-parallel regions are sized for every call of at most T tokens
// and B sequences (the size query: one workspace serves every smaller call);
// without, for this call's own plan (the layout a call uses).
WsLayout ws_layout(int64_t T, int B, int H, int split_opt, bool bound = false) {
  WsLayout w;
  w.nc = T / kChunk + 2 * (int64_t)B + 1;
  int64_t segs = 0;
  w.split_m = 0;
  if (split_opt > 0) {  // forced: a sequence of c chunks has ceil(c / m) <= c / m + 1 segments
    w.split_mode = kSplitForced;
    w.split_m = split_opt;
    segs = w.nc / split_opt + B;
  } else if (split_opt == 0 && auto_allowed(T, B, H)) {
    w.split_mode = kSplitAuto;
    segs = auto_segments(T, B, H);
  } else {
    w.split_mode = kSplitOff;
  }
  if (bound && split_opt == 0) {
    // every call of T' <= T tokens in B' <= B sequences that takes the auto
    // plan has B' <= min(B, 256 / H) and T' >= 16 chunks; its room grows with
    // T' and B', so the largest such call bounds them all
    const int64_t bmax = std::min<int64_t>(B, 256 / H);
    if (bmax >= 1 && T >= kAutoMinTokens) segs = std::max(segs, auto_segments(T, bmax, H));
  }
  w.cap1 = 2 * segs;
  w.cap2 = segs;
  w.rows = 3 * segs;
  size_t off = 0;
  w.slots = off;
  off += align256((size_t)5 * B * sizeof(int32_t));
  w.order = off;
  off += align256((size_t)B * sizeof(int32_t));
  w.zero = off;
  off += 256;
  w.tab = off;
  off += align256((size_t)w.nc * 4 * sizeof(int32_t));
  w.T = off;
  off += align256((size_t)w.nc * H * kRecWords * sizeof(u16));
  w.scal = off;
  off += align256((size_t)w.nc * H * kRecScal * sizeof(float));
  w.seg1 = w.seg2 = w.scan = w.counts = w.states = w.bound = off;
  if (segs > 0) {
    w.seg1 = off;
    off += align256((size_t)w.cap1 * kSegWords * sizeof(int32_t));
    w.seg2 = off;
    off += align256((size_t)w.cap2 * kSegWords * sizeof(int32_t));
    w.scan = off;
    off += align256((size_t)B * 4 * sizeof(int32_t));
    w.counts = off;
    off += 256;
    w.states = off;
    off += align256((size_t)w.rows * H * kDim * kDim * sizeof(float));
    w.bound = off;  // one float per (chunk slot, v-head)
    off += align256((size_t)w.nc * H * sizeof(float));
  }
  w.total = off;
  return w;
}

int check_opts(const gdn_dims_t* d) {
  if (!d->options) return GDN_OK;
  const gdn_options_t* x = d->options;
  if (x->prefill_split_chunks < -1)
    return fail(GDN_EINVAL, "options.prefill_split_chunks must be -1, 0 or positive (got %d)",
                x->prefill_split_chunks);
  const int w = x->prefill_tile_waves;
  if (w != 0 && w != 1 && w != 2 && w != 4 && w != 8)
    return fail(GDN_EINVAL, "options.prefill_tile_waves must be 0, 1, 2, 4 or 8 (got %d)", w);
  const int dw = x->decode_waves;
  if (dw != 0 && dw != 2 && dw != 4 && dw != 8 && dw != 16)
    return fail(GDN_EINVAL, "options.decode_waves must be 0, 2, 4, 8 or 16 (got %d)", dw);
  if (x->decode_stream_per_cu < -1 || x->decode_stream_grid < 0)
    return fail(GDN_EINVAL, "options.decode_stream_per_cu must be >= -1 and decode_stream_grid >= 0");
  if (x->check_error_word && x->check_num_pages < 1)
    return fail(GDN_EINVAL, "options.check_error_word needs check_num_pages >= 1");
  return GDN_OK;
}

int check_dims(const gdn_dims_t* d) {
  if (!d) return fail(GDN_EINVAL, "dims is NULL");
  if (d->num_qk_heads <= 0 || d->num_v_heads <= 0)
    return fail(GDN_EINVAL, "head counts must be positive (Hqk=%d, H=%d)", d->num_qk_heads,
                d->num_v_heads);
  if (d->head_dim_k != kDim || d->head_dim_v != kDim)
    return fail(GDN_EUNSUPPORTED, "only K = V = 128 is built (K=%d, V=%d)", d->head_dim_k,
                d->head_dim_v);
  if (d->num_v_heads % d->num_qk_heads != 0)
    return fail(GDN_EUNSUPPORTED, "v-heads (%d) must be a multiple of q/k heads (%d)",
                d->num_v_heads, d->num_qk_heads);
  if (d->state_dtype != GDN_STATE_F32 && d->state_dtype != GDN_STATE_BF16)
    return fail(GDN_EINVAL, "state_dtype must be GDN_STATE_F32 or GDN_STATE_BF16 (got %d)",
                d->state_dtype);
  return check_opts(d);
}

float eff_scale(const gdn_dims_t* d) {
  return d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->head_dim_k);
}

int64_t state_block(const gdn_dims_t* d) { return (int64_t)d->num_v_heads * kDim * kDim; }

int check_tokens(const void* q, const void* k, const void* v, const int32_t* cu, const void* o) {
  if (!q || !k || !v) return fail(GDN_EINVAL, "q, k and v must not be NULL");
  if (!cu) return fail(GDN_EINVAL, "cu_seqlens must not be NULL");
  if (!o) return fail(GDN_EINVAL, "o must not be NULL");
  return GDN_OK;
}

int check_page_size(int32_t ps) {
  if (ps <= 0 || ps % kChunk != 0)
    return fail(GDN_EINVAL, "page_size must be a positive multiple of 64 (got %d)", ps);
  return GDN_OK;
}

SlotsDev carve_slots(void* ws, const WsLayout& L, int B) {
  int32_t* base = (int32_t*)((char*)ws + L.slots);
  return SlotsDev{base, base + B, base + 2 * B, base + 3 * B, base + 4 * B};
}

// Launch the fused prefill once the rows are on the device.
int run_prefill(const gdn_dims_t* d, const void* q, const void* k, const void* v,
                const float* g, const float* beta, const int32_t* cu, int B,
                const SlotsDev& sd, const WsLayout& L, void* ws, const void* init,
                int64_t init_stride, void* out, int64_t out_stride, void* ckpt,
                int64_t ckpt_stride, const void* ckpt_idx, int ckpt_idx64, int ckpt_every,
                void* o, hipStream_t stream, const int32_t* guard = nullptr) {
  PrefillParams pp;
  pp.q = (const u16*)q;
  pp.k = (const u16*)k;
  pp.v = (const u16*)v;
  pp.g = g;
  pp.beta = beta;
  pp.o = (u16*)o;
  pp.cu_seqlens = cu;
  pp.slots = sd;
  pp.order = (int32_t*)((char*)ws + L.order);
  pp.chunk_tab = (int4*)((char*)ws + L.tab);
  pp.num_chunk_slots = (int)L.nc;
  pp.ws_T = (u16*)((char*)ws + L.T);
  pp.ws_scal = (float*)((char*)ws + L.scal);
  pp.zero_row = (u16*)((char*)ws + L.zero);
  pp.num_seqs = B;
  pp.H = d->num_v_heads;
  pp.Hqk = d->num_qk_heads;
  pp.group = d->num_v_heads / d->num_qk_heads;
  pp.scale = eff_scale(d);
  pp.state_bf16 = d->state_dtype == GDN_STATE_BF16;
  pp.init = init;
  pp.init_stride = init_stride;
  pp.out = out;
  pp.out_stride = out_stride;
  pp.ckpt = ckpt;
  pp.ckpt_stride = ckpt_stride;
  pp.ckpt_idx = ckpt_idx;
  pp.ckpt_idx64 = ckpt_idx64;
  pp.ckpt_every = ckpt_every;
  pp.split_mode = L.split_mode;
  pp.split_m = L.split_m;
  pp.num_cus = device_cus();
  pp.tile_waves = get_opts(d).waves;
  pp.seg_cap1 = (int)L.cap1;
  pp.seg_cap2 = (int)L.cap2;
  pp.seg1 = (int32_t*)((char*)ws + L.seg1);
  pp.seg2 = (int32_t*)((char*)ws + L.seg2);
  pp.seg_scan = (int4*)((char*)ws + L.scan);
  pp.seg_counts = (int32_t*)((char*)ws + L.counts);
  pp.ws_state = (float*)((char*)ws + L.states);
  pp.ws_state_stride = (int64_t)d->num_v_heads * kDim * kDim;
  pp.ws_bound = L.split_mode != kSplitOff ? (float*)((char*)ws + L.bound) : nullptr;
  pp.vseq = nullptr;
  pp.vcount = nullptr;
  pp.vhalf = 0;
  pp.guard = guard;
  if (int rc = launched(launch_prefill(pp, L.nc, stream), "prefill kernels")) return rc;
  return ok();
}

// Scratch of gdn_prefill_paged_noalloc: the workspace of calls that may not
// allocate, one copy per device, held from the library's load until the
// process ends.  Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(256) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ELAUNCH, "no current HIP device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(GDN_ELAUNCH, "device address of the fixed scratch: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

// The paged prefill; with `fixed_scratch` its workspace is the device's
// fixed scratch instead of the caller's.
int prefill_paged_impl(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const int32_t* cu_seqlens,
                       int32_t num_seqs, int64_t total_tokens, void* state_pool,
                       int64_t pool_row_stride, const int32_t* page_indices,
                       const int32_t* page_indptr, const int32_t* last_page_len,
                       int32_t page_size, const gdn_prefill_slots_t* slots, void* o,
                       void* workspace, size_t workspace_bytes, bool fixed_scratch,
                       hipStream_t stream) {
  if (int rc = check_dims(dims)) return rc;
  if (num_seqs < 0 || total_tokens < 0)
    return fail(GDN_EINVAL, "num_seqs and total_tokens must be >= 0");
  if (int rc = check_page_size(page_size)) return rc;
  if (!cu_seqlens) return fail(GDN_EINVAL, "cu_seqlens must not be NULL");
  if (!state_pool) return fail(GDN_EINVAL, "state_pool must not be NULL");
  if (!page_indices || !page_indptr || !last_page_len)
    return fail(GDN_EINVAL, "page table must not be NULL");
  if (pool_row_stride < state_block(dims))
    return fail(GDN_EINVAL, "pool_row_stride %lld < H*V*K", (long long)pool_row_stride);
  if (num_seqs == 0) return ok();
  if (total_tokens > 0)
    if (int rc = check_tokens(q, k, v, cu_seqlens, o)) return rc;
  if (slots && (!slots->state_indices || !slots->output_state_indices ||
                !slots->checkpoint_cu_starts || !slots->prefix_lens || !slots->chunk_starts))
    return fail(GDN_EINVAL, "every slot array must be given");
  const WsLayout L = ws_layout(total_tokens, num_seqs, dims->num_v_heads, get_opts(dims).split);
  if (fixed_scratch) {
    if (L.total > kScratchBytes)
      return fail(GDN_EWORKSPACE,
                  "this call needs %zu bytes of workspace; the fixed scratch holds %zu "
                  "(use gdn_prefill_paged with a workspace)", L.total, kScratchBytes);
    if (int rc = scratch_for_current_device(&workspace)) return rc;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 255))
    return fail(GDN_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", L.total,
                workspace_bytes);
  const Opts opt = get_opts(dims);
  if (opt.check &&
      launched(launch_check_paged(cu_seqlens, page_indices, page_indptr, last_page_len, num_seqs,
                                  page_size, opt.check_pages, opt.check, stream),
               "check kernel"))
    return GDN_ELAUNCH;
  SlotsDev sd;
  if (slots) {
    sd = SlotsDev{slots->state_indices, slots->output_state_indices, slots->checkpoint_cu_starts,
                  slots->prefix_lens, slots->chunk_starts};
  } else {
    sd = carve_slots(workspace, L, num_seqs);
    if (int rc = launched(launch_prefill_slots(cu_seqlens, page_indices, page_indptr,
                                               last_page_len, num_seqs, page_size,
                                               (int32_t*)sd.read, (int32_t*)sd.write,
                                               (int32_t*)sd.ckpt_start, (int32_t*)sd.prefix,
                                               (int32_t*)sd.chunk_start, opt.check, stream),
                          "prefill slot kernel"))
      return rc;
  }
  if (total_tokens == 0) return ok();
  // The paged call is the slot-argument call with one pool for all three
  // buffers and a checkpoint every page_size tokens into page_indices.
  return run_prefill(dims, q, k, v, g, beta, cu_seqlens, num_seqs, sd, L, workspace, state_pool,
                     pool_row_stride, state_pool, pool_row_stride, state_pool, pool_row_stride,
                     page_indices, 0, page_size, o, stream, opt.check);
}

}  // namespace

namespace gdn {

int current_device() {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}

int device_cus() {
  static std::atomic<int> cus[kMaxDevices];  // 0 until first asked (threads may race: same value)
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c <= 0) {
    int n = 0;
    c = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0
            ? n : 256;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

}  // namespace gdn

extern "C" {

const char* gdn_last_error(void) { return g_err.c_str(); }

const char* gdn_version(void) { return "gdn_paged 0.2.0 (gfx950)"; }

size_t gdn_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs, const gdn_dims_t* dims) {
  if (check_dims(dims) != GDN_OK || total_tokens < 0 || num_seqs < 0) return 0;
  return ws_layout(total_tokens, num_seqs, dims->num_v_heads, get_opts(dims).split, true).total;
}

int gdn_prefill_slots(const int32_t* cu_seqlens, const int32_t* page_indices,
                      const int32_t* page_indptr, const int32_t* last_page_len,
                      int32_t num_seqs, int32_t page_size, const gdn_prefill_slots_t* out,
                      hipStream_t stream) {
  if (num_seqs < 0) return fail(GDN_EINVAL, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (int rc = check_page_size(page_size)) return rc;
  if (!cu_seqlens || !page_indices || !page_indptr || !last_page_len)
    return fail(GDN_EINVAL, "page table and cu_seqlens must not be NULL");
  if (!out || !out->state_indices || !out->output_state_indices || !out->checkpoint_cu_starts ||
      !out->prefix_lens || !out->chunk_starts)
    return fail(GDN_EINVAL, "every output slot array must be given");
  if (int rc = launched(launch_prefill_slots(cu_seqlens, page_indices, page_indptr, last_page_len,
                                             num_seqs, page_size, out->state_indices,
                                             out->output_state_indices,
                                             out->checkpoint_cu_starts, out->prefix_lens,
                                             out->chunk_starts, nullptr, stream),
                        "prefill slot kernel"))
    return rc;
  return ok();
}

int gdn_decode_slots(const int32_t* page_indices, const int32_t* page_indptr,
                     const int32_t* last_page_len, int32_t num_seqs,
                     const gdn_decode_slots_t* out, hipStream_t stream) {
  if (num_seqs < 0) return fail(GDN_EINVAL, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (!page_indices || !page_indptr || !last_page_len)
    return fail(GDN_EINVAL, "page table must not be NULL");
  if (!out || !out->initial_state_indices || !out->output_state_indices)
    return fail(GDN_EINVAL, "both output slot arrays must be given");
  if (int rc = launched(launch_decode_slots(page_indices, page_indptr, last_page_len, num_seqs,
                                            out->initial_state_indices,
                                            out->output_state_indices, stream),
                        "decode slot kernel"))
    return rc;
  return ok();
}

int gdn_block_table_to_csr(const int32_t* block_tables, int64_t row_stride,
                           const int32_t* ctx_lens, int32_t num_seqs, int32_t max_blocks,
                           int32_t page_size, int32_t* page_indptr, int32_t* page_indices,
                           int32_t* last_page_len, int32_t* bad_rows, hipStream_t stream) {
  if (num_seqs < 0) return fail(GDN_EINVAL, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (page_size <= 0) return fail(GDN_EINVAL, "page_size must be positive (got %d)", page_size);
  if (max_blocks < 0 || row_stride < max_blocks)
    return fail(GDN_EINVAL, "need 0 <= max_blocks <= row_stride (got %d, %lld)", max_blocks,
                (long long)row_stride);
  if (!block_tables || !ctx_lens || !page_indptr || !page_indices || !last_page_len)
    return fail(GDN_EINVAL, "block table, lengths and CSR outputs must not be NULL");
  if (int rc = launched(launch_block_table_to_csr(block_tables, row_stride, ctx_lens, num_seqs,
                                                  max_blocks, page_size, page_indptr,
                                                  page_indices, last_page_len, bad_rows, stream),
                        "block table to CSR"))
    return rc;
  return ok();
}

int gdn_csr_to_block_table(const int32_t* page_indptr, const int32_t* page_indices,
                           const int32_t* last_page_len, int32_t num_seqs, int32_t page_size,
                           int32_t max_blocks, int32_t* block_tables, int64_t row_stride,
                           int32_t* ctx_lens, int32_t* bad_rows, hipStream_t stream) {
  if (num_seqs < 0) return fail(GDN_EINVAL, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (page_size <= 0) return fail(GDN_EINVAL, "page_size must be positive (got %d)", page_size);
  if (max_blocks < 0 || row_stride < max_blocks)
    return fail(GDN_EINVAL, "need 0 <= max_blocks <= row_stride (got %d, %lld)", max_blocks,
                (long long)row_stride);
  if (!page_indptr || !page_indices || !last_page_len || !block_tables || !ctx_lens)
    return fail(GDN_EINVAL, "CSR table and block-table outputs must not be NULL");
  if (int rc = launched(launch_csr_to_block_table(page_indptr, page_indices, last_page_len,
                                                  num_seqs, page_size, max_blocks, block_tables,
                                                  row_stride, ctx_lens, bad_rows, stream),
                        "CSR to block table"))
    return rc;
  return ok();
}

int gdn_check_paged(const int32_t* cu_seqlens, const int32_t* page_indices,
                    const int32_t* page_indptr, const int32_t* last_page_len, int32_t num_seqs,
                    int32_t page_size, int32_t num_pages, int32_t* error_word,
                    hipStream_t stream) {
  if (num_seqs < 1) return fail(GDN_EINVAL, "num_seqs must be >= 1 (got %d)", num_seqs);
  if (int rc = check_page_size(page_size)) return rc;
  if (num_pages < 1) return fail(GDN_EINVAL, "num_pages must be >= 1 (got %d)", num_pages);
  if (!page_indices || !page_indptr || !last_page_len || !error_word)
    return fail(GDN_EINVAL, "page table and error_word must not be NULL");
  if (int rc = launched(launch_check_paged(cu_seqlens, page_indices, page_indptr, last_page_len,
                                           num_seqs, page_size, num_pages, error_word, stream),
                        "check kernel"))
    return rc;
  return ok();
}

int gdn_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  if (bytes < 0 || bytes % 16)
    return fail(GDN_EINVAL, "bytes must be a non-negative multiple of 16 (got %lld)", (long long)bytes);
  if (bytes == 0) return ok();
  if (!dst || !src) return fail(GDN_EINVAL, "dst and src must not be NULL");
  if ((uintptr_t)dst % 16 || (uintptr_t)src % 16)
    return fail(GDN_EINVAL, "dst and src must be 16-byte aligned");
  const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
  if (d < s + (uintptr_t)bytes && s < d + (uintptr_t)bytes) return fail(GDN_EINVAL, "dst and src overlap");
  if (int rc = launched(launch_stream_copy(dst, src, bytes, stream), "copy kernel")) return rc;
  return ok();
}

int gdn_prefill_paged(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const int32_t* cu_seqlens,
                      int32_t num_seqs, int64_t total_tokens, void* state_pool,
                      int64_t pool_row_stride, const int32_t* page_indices,
                      const int32_t* page_indptr, const int32_t* last_page_len,
                      int32_t page_size, const gdn_prefill_slots_t* slots, void* o,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_paged_impl(dims, q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens,
                            state_pool, pool_row_stride, page_indices, page_indptr,
                            last_page_len, page_size, slots, o, workspace, workspace_bytes,
                            false, stream);
}

int gdn_prefill_paged_noalloc(const gdn_dims_t* dims, const void* q, const void* k,
                              const void* v, const float* g, const float* beta,
                              const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                              void* state_pool, int64_t pool_row_stride,
                              const int32_t* page_indices, const int32_t* page_indptr,
                              const int32_t* last_page_len, int32_t page_size,
                              const gdn_prefill_slots_t* slots, void* o, hipStream_t stream) {
  return prefill_paged_impl(dims, q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens,
                            state_pool, pool_row_stride, page_indices, page_indptr,
                            last_page_len, page_size, slots, o, nullptr, 0, true, stream);
}

int gdn_decode_paged(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                     const float* g, const float* beta, int32_t num_seqs, void* state_pool,
                     int64_t pool_row_stride, const int32_t* page_indices,
                     const int32_t* page_indptr, const int32_t* last_page_len,
                     int32_t page_size, const gdn_decode_slots_t* slots, void* o,
                     hipStream_t stream) {
  if (int rc = check_dims(dims)) return rc;
  if (num_seqs < 0) return fail(GDN_EINVAL, "num_seqs must be >= 0");
  if (int rc = check_page_size(page_size)) return rc;
  if (!state_pool) return fail(GDN_EINVAL, "state_pool must not be NULL");
  if (pool_row_stride < state_block(dims))
    return fail(GDN_EINVAL, "pool_row_stride %lld < H*V*K", (long long)pool_row_stride);
  if (num_seqs == 0) return ok();
  if (!q || !k || !v || !o) return fail(GDN_EINVAL, "q, k, v and o must not be NULL");
  DecodeParams dp{};
  dp.q = (const u16*)q;
  dp.k = (const u16*)k;
  dp.v = (const u16*)v;
  dp.g = g;
  dp.beta = beta;
  dp.o = (u16*)o;
  dp.num_seqs = num_seqs;
  dp.H = dims->num_v_heads;
  dp.Hqk = dims->num_qk_heads;
  dp.group = dims->num_v_heads / dims->num_qk_heads;
  dp.scale = eff_scale(dims);
  dp.state_bf16 = dims->state_dtype == GDN_STATE_BF16;
  dp.init = state_pool;
  dp.init_stride = pool_row_stride;
  dp.out = state_pool;
  dp.out_stride = pool_row_stride;
  const Opts opt = get_opts(dims);
  if (opt.check) {
    if (!page_indices || !page_indptr || !last_page_len)
      return fail(GDN_EINVAL, "the check needs the page table");
    if (launched(launch_check_paged(nullptr, page_indices, page_indptr, last_page_len, num_seqs,
                                    page_size, opt.check_pages, opt.check, stream),
                 "check kernel"))
      return GDN_ELAUNCH;
    dp.guard = opt.check;
  }
  if (slots) {
    if (!slots->initial_state_indices || !slots->output_state_indices)
      return fail(GDN_EINVAL, "both slot arrays must be given");
    dp.mode = 0;
    dp.rd_idx = slots->initial_state_indices;
    dp.wr_idx = slots->output_state_indices;
    dp.idx64 = 0;
  } else {
    if (!page_indices || !page_indptr || !last_page_len)
      return fail(GDN_EINVAL, "page table must not be NULL");
    dp.mode = 1;
    dp.page_indices = page_indices;
    dp.page_indptr = page_indptr;
    dp.last_page_len = last_page_len;
  }
  if (int rc = launched(launch_decode(dp, get_opts(dims).dec, stream), "decode kernel")) return rc;
  return ok();
}

int gdn_prefill(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                const float* g, const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                int64_t total_tokens, const void* initial_state, int64_t initial_row_stride,
                const void* state_indices, void* output_state, int64_t output_row_stride,
                const void* output_state_indices, int32_t output_final_state,
                void* state_checkpoints, int64_t checkpoint_row_stride,
                const void* checkpoint_state_indices, const void* checkpoint_cu_starts,
                const void* prefix_lens, int32_t checkpoint_every_n_tokens, int32_t index_dtype,
                void* o, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (int rc = check_dims(dims)) return rc;
  if (num_seqs < 0 || total_tokens < 0)
    return fail(GDN_EINVAL, "num_seqs and total_tokens must be >= 0");
  if (!cu_seqlens) return fail(GDN_EINVAL, "cu_seqlens must not be NULL");
  if (index_dtype != GDN_INDEX_INT32 && index_dtype != GDN_INDEX_INT64)
    return fail(GDN_EINVAL, "index_dtype must be GDN_INDEX_INT32 or GDN_INDEX_INT64");
  const int64_t blk = state_block(dims);
  if (initial_state && initial_row_stride < blk)
    return fail(GDN_EINVAL, "initial_row_stride < H*V*K");
  if (output_state_indices && (!output_final_state || !output_state))
    return fail(GDN_EINVAL,
                "output_state_indices needs output_state and output_final_state");
  if (output_final_state && !output_state)
    return fail(GDN_EINVAL, "output_final_state needs output_state");
  if (output_state && output_row_stride < blk)
    return fail(GDN_EINVAL, "output_row_stride < H*V*K");
  if (checkpoint_state_indices) {
    if (checkpoint_every_n_tokens <= 0 || !prefix_lens || !checkpoint_cu_starts ||
        !state_checkpoints)
      return fail(GDN_EINVAL,
                  "checkpoint_state_indices needs checkpoint_every_n_tokens > 0, prefix_lens, "
                  "checkpoint_cu_starts and state_checkpoints");
    if (checkpoint_row_stride < blk) return fail(GDN_EINVAL, "checkpoint_row_stride < H*V*K");
  }
  if (num_seqs == 0 || total_tokens == 0) return ok();
  if (int rc = check_tokens(q, k, v, cu_seqlens, o)) return rc;
  const WsLayout L = ws_layout(total_tokens, num_seqs, dims->num_v_heads, get_opts(dims).split);
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 255))
    return fail(GDN_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", L.total,
                workspace_bytes);
  const int idx64 = index_dtype == GDN_INDEX_INT64;
  const SlotsDev sd = carve_slots(workspace, L, num_seqs);
  if (int rc = launched(
          launch_general_slots(cu_seqlens, num_seqs, state_indices, output_state_indices,
                               checkpoint_state_indices ? checkpoint_cu_starts : nullptr,
                               prefix_lens, idx64, initial_state != nullptr,
                               output_final_state != 0, (int32_t*)sd.read, (int32_t*)sd.write,
                               (int32_t*)sd.ckpt_start, (int32_t*)sd.prefix,
                               (int32_t*)sd.chunk_start, stream),
          "slot-argument kernel"))
    return rc;
  return run_prefill(dims, q, k, v, g, beta, cu_seqlens, num_seqs, sd, L, workspace,
                     initial_state, initial_row_stride, output_state, output_row_stride,
                     state_checkpoints, checkpoint_row_stride, checkpoint_state_indices, idx64,
                     checkpoint_every_n_tokens, o, stream);
}

int gdn_decode(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
               const float* g, const float* beta, int32_t num_seqs, const void* initial_state,
               int64_t initial_row_stride, const void* initial_state_indices,
               void* output_state, int64_t output_row_stride, const void* output_state_indices,
               int32_t index_dtype, void* o, hipStream_t stream) {
  if (int rc = check_dims(dims)) return rc;
  if (num_seqs < 0) return fail(GDN_EINVAL, "num_seqs must be >= 0");
  if (index_dtype != GDN_INDEX_INT32 && index_dtype != GDN_INDEX_INT64)
    return fail(GDN_EINVAL, "index_dtype must be GDN_INDEX_INT32 or GDN_INDEX_INT64");
  const int64_t blk = state_block(dims);
  if (initial_state && initial_row_stride < blk)
    return fail(GDN_EINVAL, "initial_row_stride < H*V*K");
  if (output_state && output_row_stride < blk)
    return fail(GDN_EINVAL, "output_row_stride < H*V*K");
  if (output_state_indices && !output_state)
    return fail(GDN_EINVAL, "output_state_indices needs output_state");
  if (num_seqs == 0) return ok();
  if (!q || !k || !v || !o) return fail(GDN_EINVAL, "q, k, v and o must not be NULL");
  DecodeParams dp{};
  dp.q = (const u16*)q;
  dp.k = (const u16*)k;
  dp.v = (const u16*)v;
  dp.g = g;
  dp.beta = beta;
  dp.o = (u16*)o;
  dp.num_seqs = num_seqs;
  dp.H = dims->num_v_heads;
  dp.Hqk = dims->num_qk_heads;
  dp.group = dims->num_v_heads / dims->num_qk_heads;
  dp.scale = eff_scale(dims);
  dp.mode = 0;
  dp.rd_idx = initial_state_indices;
  dp.wr_idx = output_state_indices;
  dp.idx64 = index_dtype == GDN_INDEX_INT64;
  dp.state_bf16 = dims->state_dtype == GDN_STATE_BF16;
  dp.init = initial_state;
  dp.init_stride = initial_row_stride;
  dp.out = output_state;
  dp.out_stride = output_row_stride;
  if (int rc = launched(launch_decode(dp, get_opts(dims).dec, stream), "decode kernel")) return rc;
  return ok();
}

}  // extern "C"
