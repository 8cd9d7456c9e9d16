// The C ABI (include/decstep.h): host-side validation, workspace layout, launches
// and graph helpers.  No entry point allocates, synchronises or reads device data.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "../../include/decstep.h"
#include "dec_common.h"
#include "dec_kernels.h"
#include "probe.h"

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = static_cast<int>(e);
  return DEC_E_HIP;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Workspace of an attention call, used when a launch spreads the chunks of a sequence
// over several workgroups: two regions of per-sequence arrival tickets (the call's first
// segment, then its second; zero between calls), then each segment's chunk states at
// `chunk` keys per chunk.  The tickets sit at the same places whatever chunk a call
// uses, so the chunk states of one call never land on another's tickets.  Capacities
// that fit one chunk need none.
struct WsLayout {
  size_t ticket_bytes = 0;  // one ticket region
  size_t part_off[2] = {0, 0};
  size_t bytes = 0;
};

WsLayout ws_layout(int NL, int B, int H, int hd, const int (&L_cap)[2], int chunk) {
  WsLayout w;
  int nck[2];
  bool any = false;
  for (int s = 0; s < 2; ++s) {
    nck[s] = L_cap[s] > 0 ? (L_cap[s] + chunk - 1) / chunk : 0;
    any = any || nck[s] > 1;
  }
  if (!any) return w;
  const size_t nseq = (size_t)NL * B * H;
  w.ticket_bytes = align_up(nseq * sizeof(int32_t), 256);
  size_t off = 2 * w.ticket_bytes;
  for (int s = 0; s < 2; ++s) {
    w.part_off[s] = off;
    if (nck[s] > 1) off += align_up(nseq * nck[s] * dec::attn_part_stride(hd) * sizeof(float), 256);
  }
  w.bytes = off;
  return w;
}

// The no-allocation entry point's workspace: one array per GPU, of a fixed size, held
// until the process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address is taken with hipGetSymbolAddress, once per device,
// and only that address is ever passed to kernels or fills.
constexpr size_t kScratchBytes = DEC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// This device's address of `scratch` (looked up on the first call on the device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // every thread finds the same
  }
  *out = ptr;
  return hipSuccess;
}

// After the layout: one first-tile record per wave of up to kAttnRecGroups workgroups
// (the next launch requests those tiles while it derives its schedule).  Optional: a
// workspace without room for it runs without.
constexpr size_t kRecBytes = (size_t)dec::kAttnRecGroups * dec::kAttnWaves * sizeof(dec::TileRec);
static_assert(kRecBytes % 256 == 0, "whole 256-byte blocks");

bool hd_ok(int hd) { return hd == dec::kAttnHeadDim || hd == dec::kAttnHeadDimWide; }

bool sizes_ok(int NL, int B, int H, int L_cap, int hd) {
  if (NL < 1 || B < 1 || H < 1 || L_cap < 1) return false;
  const long long nseq = (long long)NL * B * H;
  if (nseq > (1LL << 30)) return false;
  const long long elems = nseq * L_cap * hd;
  return elems < (1LL << 46);
}

// Launch-policy overrides of the calling thread (dec_tuning_set); all zero by default.
thread_local dec_tuning g_tuning{};

struct SegArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* len;
  void* out;
  int L_cap;
  // paged cache: k, v are block pools; L_cap = table_stride * block_size
  const int32_t* table = nullptr;
  int table_stride = 0;
  int n_blocks = 0;
  int block_size = 0;
  // key bitmask [B, mask_words] (bit j % 32 of word j / 32: key j attended), or none
  const uint32_t* mask = nullptr;
  int mask_words = 0;
  int out_bf16 = 0;
  // the current token's rows, appended at slot len[b] - 1 of k / v in the launch
  const void* k_new = nullptr;
  const void* v_new = nullptr;
};

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// clear_bytes > 0: the first clear_bytes of the workspace (its arrival counters) are
// zeroed by a fill kernel on `stream` after every host check has passed, right before
// the attention launch.
int attn_common(const SegArgs* segs, int nseg, int NL, int B, int H, int hd, int dtype,
                float scale, void* ws, size_t ws_bytes, hipStream_t stream,
                size_t clear_bytes = 0) {
  for (int s = 0; s < nseg; ++s) {
    if (!segs[s].q || !segs[s].k || !segs[s].v || !segs[s].len || !segs[s].out) return DEC_E_NULL;
  }
  if (dtype != DEC_BF16 && dtype != DEC_F32) return DEC_E_DTYPE;
  for (int s = 0; s < nseg; ++s) {
    if (!sizes_ok(NL, B, H, segs[s].L_cap, hd > 0 ? hd : 1)) return DEC_E_SHAPE;
  }
  for (int s = 0; s < nseg; ++s) {
    const SegArgs& a = segs[s];
    if (a.table == nullptr) continue;
    const long long row = (long long)hd * (dtype == DEC_BF16 ? 2 : 4);
    if (a.n_blocks < 1 || a.table_stride < 1) return DEC_E_SHAPE;
    if ((long long)NL * a.n_blocks * H * a.block_size * row > (1LL << 46)) return DEC_E_SHAPE;
    if ((long long)B * a.table_stride > (1LL << 30)) return DEC_E_SHAPE;
    if (!is_pow2(a.block_size) || a.block_size < dec::kAttnMinBlockKeys ||
        a.block_size > (1 << 20))
      return DEC_E_UNSUPPORTED;
    if (!aligned(a.table, 4)) return DEC_E_ALIGN;
  }
  if (!hd_ok(hd)) return DEC_E_UNSUPPORTED;
  if (nseg * B > dec::kAttnMaxGroups) return DEC_E_UNSUPPORTED;
  for (int s = 0; s < nseg; ++s) {  // one sequence's static cache (and one tile past its
    // end, where no-traffic loads are addressed): 32-bit byte offsets
    const long long seq_bytes = (long long)segs[s].L_cap * hd * (dtype == DEC_BF16 ? 2 : 4);
    if (segs[s].table == nullptr && seq_bytes + 65536 > 0x7FFFFFFFLL) return DEC_E_UNSUPPORTED;
  }
  for (int s = 0; s < nseg; ++s) {
    if (!aligned(segs[s].q, 16) || !aligned(segs[s].k, 16) || !aligned(segs[s].v, 16) ||
        !aligned(segs[s].len, 4) || !aligned(segs[s].out, segs[s].out_bf16 ? 2 : 4))
      return DEC_E_ALIGN;
    if (segs[s].mask != nullptr) {
      // whole 64-bit words per 64 keys: a tile never reads past the row
      const long long need = 2LL * ((segs[s].L_cap + 63) / 64);
      if (segs[s].mask_words < need || segs[s].mask_words % 2 != 0) return DEC_E_SHAPE;
      if (segs[s].table != nullptr) return DEC_E_UNSUPPORTED;  // masks go with static caches
      if (!aligned(segs[s].mask, 8)) return DEC_E_ALIGN;
    }
  }
  // required: the chunk states at 1024-key chunks; a workspace that also holds them at
  // the smallest chunk lets a launch with few sequences cut its chunks smaller
  const int caps[2] = {segs[0].L_cap, nseg > 1 ? segs[1].L_cap : 0};
  const WsLayout lay_max = ws_layout(NL, B, H, hd, caps, dec::kAttnChunk);
  const WsLayout lay_min = ws_layout(NL, B, H, hd, caps, dec::kAttnMinChunk);
  if (lay_max.bytes > 0) {
    if (ws == nullptr) return DEC_E_NULL;
    if (!aligned(ws, 16)) return DEC_E_ALIGN;
    if (ws_bytes < lay_max.bytes) return DEC_E_WORKSPACE;
  }
  const bool small_ok =
      lay_min.bytes > 0 && ws != nullptr && aligned(ws, 16) && ws_bytes >= lay_min.bytes;
  const WsLayout& lay = small_ok ? lay_min : lay_max;
  const int min_log2 = dec::attn_log2(small_ok ? dec::kAttnMinChunk : dec::kAttnChunk);
  int chunk_log2 = 0;  // the launcher chooses
  const int chunk_keys = g_tuning.attn_chunk_keys;
  if (chunk_keys != 0) {  // a fixed chunk (tests of every cut, measurements)
    if (!is_pow2(chunk_keys) || chunk_keys > dec::kAttnChunk || chunk_keys < (1 << min_log2))
      return DEC_E_UNSUPPORTED;
    chunk_log2 = dec::attn_log2(chunk_keys);
  }

  dec::AttnParams p{};
  if (ws != nullptr && aligned(ws, 16) && ws_bytes >= lay.bytes + kRecBytes) {
    p.rec = reinterpret_cast<dec::TileRec*>(static_cast<char*>(ws) + lay.bytes);
    p.rec_groups = dec::kAttnRecGroups;
  }
  p.balance = g_tuning.attn_no_halves ? 0 : 1;
  if (g_tuning.attn_no_records) p.rec = nullptr;
  p.nseg = nseg;
  p.NL = NL;
  p.B = B;
  p.H = H;
  p.hd = hd;
  p.qscale = scale * 1.4426950408889634f;  // log2(e)
  p.chunk_log2 = chunk_log2;
  p.min_chunk_log2 = min_log2;
  for (int s = 0; s < nseg; ++s) {
    dec::AttnSeg& g = p.seg[s];
    g.q = segs[s].q;
    g.k = segs[s].k;
    g.v = segs[s].v;
    g.len = segs[s].len;
    g.out = segs[s].out;
    g.L_cap = segs[s].L_cap;
    g.table = segs[s].table;
    g.table_stride = segs[s].table_stride;
    g.n_blocks = segs[s].n_blocks;
    g.bs_log2 = segs[s].table ? __builtin_ctz((unsigned)segs[s].block_size) : 0;
    g.mask = segs[s].mask;
    g.mask_words = segs[s].mask_words;
    g.out_bf16 = segs[s].out_bf16;
    g.k_new = segs[s].k_new;
    g.v_new = segs[s].v_new;
    if (lay.bytes > 0) {  // nck_cap follows the chunk the launcher settles on
      char* base = static_cast<char*>(ws);
      g.ticket = reinterpret_cast<int32_t*>(base + s * lay.ticket_bytes);
      g.part = reinterpret_cast<float*>(base + lay.part_off[s]);
    }
  }
  // Few sequences: every chunk is its own work item, so the CUs get equal bytes;
  // otherwise one workgroup owns a whole sequence (no cross-workgroup traffic).
  const long long seqs = (long long)NL * B * H * nseg;
  const int split = g_tuning.attn_schedule == 0 ? (seqs < dec::kAttnSplitBelow ? 1 : 0)
                                                 : (g_tuning.attn_schedule == 1 ? 1 : 0);
  p.cpi = split ? 1 : (1 << 24);  // whole mode: every chunk of a sequence in one item
  if (nseg == 1) p.seg[1] = p.seg[0];
  if (clear_bytes > 0 && lay.bytes > 0) {
    const hipError_t ez = dec::fill_zero_launch(ws, clear_bytes, stream);
    if (ez != hipSuccess) return hip_fail(ez);
  }
  const hipError_t e = dec::attn_launch(p, dtype, g_tuning.attn_blocks, stream);
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int dec_attn_chunk_keys(void) { return dec::kAttnChunk; }

size_t dec_attn_workspace_bytes(int n_layers, int B, int H, int hd, int L_cap_self,
                                int L_cap_cross) {
  if (!hd_ok(hd) || n_layers < 1 || B < 1 || H < 1 || L_cap_self < 0 || L_cap_cross < 0)
    return 0;
  const int caps[2] = {L_cap_self, L_cap_cross};
  return ws_layout(n_layers, B, H, hd, caps, dec::kAttnMinChunk).bytes + kRecBytes;
}

int dec_attn_workspace_init(void* workspace, size_t ws_bytes, dec_stream_t stream) {
  if (ws_bytes == 0) return DEC_OK;
  if (workspace == nullptr) return DEC_E_NULL;
  if (!aligned(workspace, 16)) return DEC_E_ALIGN;
  const hipError_t e = dec::fill_zero_launch(workspace, ws_bytes, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_attn_self(const void* q, const void* k, const void* v, const int32_t* len, float* out,
                  int n_layers, int B, int H, int L_cap, int hd, int dtype, float scale,
                  void* workspace, size_t ws_bytes, dec_stream_t stream) {
  const SegArgs s{q, k, v, len, out, L_cap};
  return attn_common(&s, 1, n_layers, B, H, hd, dtype, scale, workspace, ws_bytes,
                     reinterpret_cast<hipStream_t>(stream));
}

int dec_attn_cross(const void* q, const void* k, const void* v, const int32_t* enc_len,
                   float* out, int n_layers, int B, int H, int L_cap, int hd, int dtype,
                   float scale, void* workspace, size_t ws_bytes, dec_stream_t stream) {
  const SegArgs s{q, k, v, enc_len, out, L_cap};
  return attn_common(&s, 1, n_layers, B, H, hd, dtype, scale, workspace, ws_bytes,
                     reinterpret_cast<hipStream_t>(stream));
}

int dec_attn_step(const void* q_self, const void* k_self, const void* v_self, const int32_t* len,
                  int L_cap_self, float* out_self, const void* q_cross, const void* k_cross,
                  const void* v_cross, const int32_t* enc_len, int L_cap_cross, float* out_cross,
                  int n_layers, int B, int H, int hd, int dtype, float scale, void* workspace,
                  size_t ws_bytes, dec_stream_t stream) {
  const SegArgs s[2] = {{q_self, k_self, v_self, len, out_self, L_cap_self},
                        {q_cross, k_cross, v_cross, enc_len, out_cross, L_cap_cross}};
  return attn_common(s, 2, n_layers, B, H, hd, dtype, scale, workspace, ws_bytes,
                     reinterpret_cast<hipStream_t>(stream));
}

int dec_attn_step_append(const void* q_self, void* k_self, void* v_self, const int32_t* len,
                         int L_cap_self, float* out_self, const void* k_new, const void* v_new,
                         const void* q_cross, const void* k_cross, const void* v_cross,
                         const int32_t* enc_len, int L_cap_cross, float* out_cross, int n_layers,
                         int B, int H, int hd, int dtype, float scale, void* workspace,
                         size_t ws_bytes, dec_stream_t stream) {
  if (k_new == nullptr || v_new == nullptr) return DEC_E_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return DEC_E_ALIGN;
  SegArgs s[2] = {{q_self, k_self, v_self, len, out_self, L_cap_self},
                  {q_cross, k_cross, v_cross, enc_len, out_cross, L_cap_cross}};
  s[0].k_new = k_new;
  s[0].v_new = v_new;
  return attn_common(s, 2, n_layers, B, H, hd, dtype, scale, workspace, ws_bytes,
                     reinterpret_cast<hipStream_t>(stream));
}

int dec_attn_step_noalloc(const void* q_self, const void* k_self, const void* v_self,
                          const int32_t* len, int L_cap_self, float* out_self,
                          const void* q_cross, const void* k_cross, const void* v_cross,
                          const int32_t* enc_len, int L_cap_cross, float* out_cross,
                          int n_layers, int B, int H, int hd, int dtype, float scale,
                          dec_stream_t stream) {
  // host checks first: nothing is looked up or enqueued for a call that fails them
  if (!q_self || !k_self || !v_self || !len || !out_self || !q_cross || !k_cross || !v_cross ||
      !enc_len || !out_cross)
    return DEC_E_NULL;
  if (dtype != DEC_BF16 && dtype != DEC_F32) return DEC_E_DTYPE;
  if (!hd_ok(hd) || n_layers < 1 || B < 1 || H < 1 || L_cap_self < 1 || L_cap_cross < 1)
    return hd_ok(hd) ? DEC_E_SHAPE : DEC_E_UNSUPPORTED;
  const int caps[2] = {L_cap_self, L_cap_cross};
  if (!sizes_ok(n_layers, B, H, L_cap_self, hd) || !sizes_ok(n_layers, B, H, L_cap_cross, hd))
    return DEC_E_SHAPE;
  const WsLayout lay_max = ws_layout(n_layers, B, H, hd, caps, dec::kAttnChunk);
  const WsLayout lay_min = ws_layout(n_layers, B, H, hd, caps, dec::kAttnMinChunk);
  if (lay_max.bytes > kScratchBytes) return DEC_E_WORKSPACE;
  const SegArgs s[2] = {{q_self, k_self, v_self, len, out_self, L_cap_self},
                        {q_cross, k_cross, v_cross, enc_len, out_cross, L_cap_cross}};
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e);
  // both layouts start with the same two arrival-counter regions
  return attn_common(s, 2, n_layers, B, H, hd, dtype, scale, ws, kScratchBytes,
                     reinterpret_cast<hipStream_t>(stream), 2 * lay_min.ticket_bytes);
}

int dec_attn_step_ex(const void* q_self, const void* k_self, const void* v_self,
                     const int32_t* len, int L_cap_self, void* out_self, const void* q_cross,
                     const void* k_cross, const void* v_cross, const int32_t* enc_len,
                     const uint32_t* cross_mask, int mask_words, int L_cap_cross,
                     void* out_cross, int n_layers, int B, int H, int hd, int dtype,
                     int out_dtype, float scale, void* workspace, size_t ws_bytes,
                     dec_stream_t stream) {
  if (out_dtype != DEC_BF16 && out_dtype != DEC_F32) return DEC_E_DTYPE;
  SegArgs s[2] = {{q_self, k_self, v_self, len, out_self, L_cap_self},
                  {q_cross, k_cross, v_cross, enc_len, out_cross, L_cap_cross}};
  s[1].mask = cross_mask;
  s[1].mask_words = mask_words;
  s[0].out_bf16 = s[1].out_bf16 = out_dtype == DEC_BF16 ? 1 : 0;
  return attn_common(s, 2, n_layers, B, H, hd, dtype, scale, workspace, ws_bytes,
                     reinterpret_cast<hipStream_t>(stream));
}

int dec_attn_self_paged(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, const int32_t* len, float* out,
                        int n_layers, int B, int H, int hd, int block_size, int n_blocks,
                        int max_blocks, int dtype, float scale, void* workspace,
                        size_t ws_bytes, dec_stream_t stream) {
  if (!block_table) return DEC_E_NULL;
  if (max_blocks < 1 || block_size < 1 || (long long)max_blocks * block_size > (1LL << 30))
    return DEC_E_SHAPE;
  SegArgs a{q, k_pool, v_pool, len, out, max_blocks * block_size};
  a.table = block_table;
  a.table_stride = max_blocks;
  a.n_blocks = n_blocks;
  a.block_size = block_size;
  return attn_common(&a, 1, n_layers, B, H, hd, dtype, scale, workspace, ws_bytes,
                     reinterpret_cast<hipStream_t>(stream));
}

int dec_attn_step_paged(const void* q_self, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, const int32_t* len, int block_size,
                        int n_blocks, int max_blocks, float* out_self, const void* q_cross,
                        const void* k_cross, const void* v_cross, const int32_t* enc_len,
                        int L_cap_cross, float* out_cross, int n_layers, int B, int H, int hd,
                        int dtype, float scale, void* workspace, size_t ws_bytes,
                        dec_stream_t stream) {
  if (!block_table) return DEC_E_NULL;
  if (max_blocks < 1 || block_size < 1 || (long long)max_blocks * block_size > (1LL << 30))
    return DEC_E_SHAPE;
  SegArgs s[2] = {{q_self, k_pool, v_pool, len, out_self, max_blocks * block_size},
                  {q_cross, k_cross, v_cross, enc_len, out_cross, L_cap_cross}};
  s[0].table = block_table;
  s[0].table_stride = max_blocks;
  s[0].n_blocks = n_blocks;
  s[0].block_size = block_size;
  return attn_common(s, 2, n_layers, B, H, hd, dtype, scale, workspace, ws_bytes,
                     reinterpret_cast<hipStream_t>(stream));
}

int dec_attn_step_paged_ex(const void* q_self, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const int32_t* len, int block_size,
                           int n_blocks, int max_blocks, void* out_self, const void* q_cross,
                           const void* k_cross, const void* v_cross, const int32_t* enc_len,
                           const uint32_t* cross_mask, int mask_words, int L_cap_cross,
                           void* out_cross, int n_layers, int B, int H, int hd, int dtype,
                           int out_dtype, float scale, void* workspace, size_t ws_bytes,
                           dec_stream_t stream) {
  if (!block_table) return DEC_E_NULL;
  if (out_dtype != DEC_BF16 && out_dtype != DEC_F32) return DEC_E_DTYPE;
  if (max_blocks < 1 || block_size < 1 || (long long)max_blocks * block_size > (1LL << 30))
    return DEC_E_SHAPE;
  SegArgs s[2] = {{q_self, k_pool, v_pool, len, out_self, max_blocks * block_size},
                  {q_cross, k_cross, v_cross, enc_len, out_cross, L_cap_cross}};
  s[0].table = block_table;
  s[0].table_stride = max_blocks;
  s[0].n_blocks = n_blocks;
  s[0].block_size = block_size;
  s[1].mask = cross_mask;
  s[1].mask_words = mask_words;
  s[0].out_bf16 = s[1].out_bf16 = out_dtype == DEC_BF16 ? 1 : 0;
  return attn_common(s, 2, n_layers, B, H, hd, dtype, scale, workspace, ws_bytes,
                     reinterpret_cast<hipStream_t>(stream));
}

int dec_sample_topk(const float* logits, int B, int n_cb, int V_valid, int V_stride,
                    const float* temperature, int top_k, const float* uniforms,
                    const int32_t* step, int32_t fill_token, int32_t* tokens, int32_t* topk_idx,
                    float* topk_prob, dec_stream_t stream) {
  if (!logits || !temperature || !uniforms || !tokens) return DEC_E_NULL;
  if (B < 1 || n_cb < 1 || V_valid < 1 || V_stride < V_valid) return DEC_E_SHAPE;
  if ((long long)B * n_cb > (1LL << 30) || (long long)B * n_cb * V_stride > (1LL << 46))
    return DEC_E_SHAPE;
  if (top_k < 1 || top_k > 64) return DEC_E_SHAPE;
  if (V_valid > dec::kSampMaxVocab) return DEC_E_UNSUPPORTED;
  if (!aligned(logits, 4) || !aligned(temperature, 4) || !aligned(uniforms, 4) ||
      !aligned(step, 4) || !aligned(tokens, 4) || !aligned(topk_idx, 4) || !aligned(topk_prob, 4))
    return DEC_E_ALIGN;
  dec::SampleParams p{};
  p.logits = logits;
  p.temperature = temperature;
  p.uniforms = uniforms;
  p.step = step;
  p.tokens = tokens;
  p.topk_idx = topk_idx;
  p.topk_prob = topk_prob;
  p.B = B;
  p.n_cb = n_cb;
  p.V_valid = V_valid;
  p.V_stride = V_stride;
  p.top_k = top_k;
  p.fill = fill_token;
  const hipError_t e = dec::sample_launch(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_sample_topk_philox(const float* logits, int B, int n_cb, int V_valid, int V_stride,
                           const float* temperature, int top_k, uint64_t seed,
                           const int32_t* step, int32_t fill_token, int32_t* tokens,
                           int32_t* topk_idx, float* topk_prob, dec_stream_t stream) {
  if (!logits || !temperature || !tokens) return DEC_E_NULL;
  if (B < 1 || n_cb < 1 || V_valid < 1 || V_stride < V_valid) return DEC_E_SHAPE;
  if ((long long)B * n_cb > (1LL << 30) || (long long)B * n_cb * V_stride > (1LL << 46))
    return DEC_E_SHAPE;
  if (top_k < 1 || top_k > 64) return DEC_E_SHAPE;
  if (V_valid > dec::kSampMaxVocab) return DEC_E_UNSUPPORTED;
  if (!aligned(logits, 4) || !aligned(temperature, 4) || !aligned(step, 4) ||
      !aligned(tokens, 4) || !aligned(topk_idx, 4) || !aligned(topk_prob, 4))
    return DEC_E_ALIGN;
  dec::SampleParams p{};
  p.logits = logits;
  p.temperature = temperature;
  p.uniforms = nullptr;
  p.step = step;
  p.tokens = tokens;
  p.topk_idx = topk_idx;
  p.topk_prob = topk_prob;
  p.seed = seed;
  p.rng = 1;
  p.B = B;
  p.n_cb = n_cb;
  p.V_valid = V_valid;
  p.V_stride = V_stride;
  p.top_k = top_k;
  p.fill = fill_token;
  const hipError_t e = dec::sample_launch(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

// The widened sampler's checks and launch, with the optional in-launch advance.
static int sample_ex(const void* logits, int logits_dtype, int B, int n_cb, int V_valid, int V_stride,
              const float* temperature, int top_k, const float* uniforms, uint64_t seed,
              const int32_t* step, int32_t* step_inc, int32_t* len_inc, int32_t fill_token,
              int32_t* tokens, int32_t* topk_idx, float* topk_prob, dec_stream_t stream) {
  if (!logits || !temperature || !tokens) return DEC_E_NULL;
  if (logits_dtype != DEC_BF16 && logits_dtype != DEC_F32) return DEC_E_DTYPE;
  if (B < 1 || n_cb < 1 || V_valid < 1 || V_stride < V_valid) return DEC_E_SHAPE;
  if ((long long)B * n_cb > (1LL << 30) || (long long)B * n_cb * V_stride > (1LL << 46))
    return DEC_E_SHAPE;
  if (top_k < 1 || top_k > dec::kSampMaxVocab) return DEC_E_SHAPE;
  if ((long long)B * n_cb * top_k > (1LL << 46)) return DEC_E_SHAPE;
  if (V_valid > dec::kSampMaxVocab) return DEC_E_UNSUPPORTED;
  if (!aligned(logits, logits_dtype == DEC_F32 ? 4 : 2) || !aligned(temperature, 4) ||
      !aligned(uniforms, 4) || !aligned(step, 4) || !aligned(len_inc, 4) || !aligned(tokens, 4) ||
      !aligned(topk_idx, 4) || !aligned(topk_prob, 4))
    return DEC_E_ALIGN;
  dec::SampleParams p{};
  p.logits = logits;
  p.logits_bf16 = logits_dtype == DEC_BF16;
  p.step_inc = step_inc;
  p.len_inc = len_inc;
  p.temperature = temperature;
  p.uniforms = uniforms;
  p.rng = uniforms == nullptr;
  p.seed = seed;
  p.step = step;
  p.tokens = tokens;
  p.topk_idx = topk_idx;
  p.topk_prob = topk_prob;
  p.B = B;
  p.n_cb = n_cb;
  p.V_valid = V_valid;
  p.V_stride = V_stride;
  p.top_k = top_k;
  p.fill = fill_token;
  const hipError_t e = dec::sample_launch(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_sample_topk_ex(const void* logits, int logits_dtype, int B, int n_cb, int V_valid,
                       int V_stride, const float* temperature, int top_k, const float* uniforms,
                       uint64_t seed, const int32_t* step, int32_t fill_token, int32_t* tokens,
                       int32_t* topk_idx, float* topk_prob, dec_stream_t stream) {
  return sample_ex(logits, logits_dtype, B, n_cb, V_valid, V_stride, temperature, top_k,
                   uniforms, seed, step, nullptr, nullptr, fill_token, tokens, topk_idx,
                   topk_prob, stream);
}

int dec_sample_topk_advance(const void* logits, int logits_dtype, int B, int n_cb, int V_valid,
                            int V_stride, const float* temperature, int top_k,
                            const float* uniforms, uint64_t seed, int32_t* step, int32_t* len,
                            int32_t fill_token, int32_t* tokens, int32_t* topk_idx,
                            float* topk_prob, dec_stream_t stream) {
  if (step == nullptr) return DEC_E_NULL;
  return sample_ex(logits, logits_dtype, B, n_cb, V_valid, V_stride, temperature, top_k,
                   uniforms, seed, step, step, len, fill_token, tokens, topk_idx, topk_prob,
                   stream);
}

int dec_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* len, int n_layers, int B, int H, int L_cap, int hd, int dtype,
                  dec_stream_t stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !len) return DEC_E_NULL;
  if (dtype != DEC_BF16 && dtype != DEC_F32) return DEC_E_DTYPE;
  if (n_layers < 1 || B < 1 || H < 1 || L_cap < 1 || hd < 1) return DEC_E_SHAPE;
  const long long row_bytes = (long long)hd * (dtype == DEC_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0) return DEC_E_UNSUPPORTED;
  if ((long long)n_layers * B * H * L_cap * row_bytes > (1LL << 46)) return DEC_E_SHAPE;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(len, 4))
    return DEC_E_ALIGN;
  dec::AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.len = len;
  p.NL = n_layers;
  p.B = B;
  p.H = H;
  p.L_cap = L_cap;
  p.row16 = (int)(row_bytes / 16);
  const hipError_t e = dec::append_launch(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_lm_head(const void* h, const void* W, float* logits, int B, int D, int n_cb,
                int V_valid, int V_stride, dec_stream_t stream) {
  if (!h || !W || !logits) return DEC_E_NULL;
  if (B < 1 || n_cb < 1 || V_valid < 1 || V_stride < V_valid || D < 1) return DEC_E_SHAPE;
  if ((long long)B * n_cb * V_stride > (1LL << 40) || (long long)n_cb * V_stride > (1 << 24))
    return DEC_E_SHAPE;
  if (D != 512 && D != 768 && D != 1024 && D != 1536 && D != 2048) return DEC_E_UNSUPPORTED;
  if ((long long)(V_valid + 64) * D * 2 > (1LL << 31) - 1) return DEC_E_UNSUPPORTED;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(logits, 4)) return DEC_E_ALIGN;
  dec::HeadParams p{};
  p.h = static_cast<const uint16_t*>(h);
  p.W = static_cast<const uint16_t*>(W);
  p.logits = logits;
  p.B = B;
  p.D = D;
  p.n_cb = n_cb;
  p.V_valid = V_valid;
  p.V_stride = V_stride;
  // B <= 2 is a matrix-vector product: the vector ALU (measured faster at B = 1 and equal
  // at B = 2); larger batches on MFMA, which stores 4 logits at a time and addresses h
  // with 32-bit offsets
  const bool mfma_ok = aligned(logits, 16) && V_stride % 4 == 0 &&
                       (long long)(B + 32) * D * 2 <= (1LL << 31) - 1;
  const int kernel = g_tuning.head_kernel;  // 0: by shape, 1: vector ALU, 2: MFMA if it can
  p.force_gemv = !mfma_ok || kernel == 1 || (kernel == 0 && B <= 2);
  p.mfma_cfg = g_tuning.head_mfma_cfg;  // 0: the measured policy
  const hipError_t e = dec::lm_head_launch(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_embed_sum(const int32_t* tokens, const void* E, float* x, int B, int n_cb, int V_emb,
                  int D, dec_stream_t stream) {
  if (!tokens || !E || !x) return DEC_E_NULL;
  if (B < 1 || B > 65535 || n_cb < 1 || V_emb < 1 || D < 1) return DEC_E_SHAPE;
  if ((long long)n_cb * V_emb * D > (1LL << 40)) return DEC_E_SHAPE;
  if (D % 8 != 0) return DEC_E_UNSUPPORTED;
  if (!aligned(tokens, 4) || !aligned(E, 16) || !aligned(x, 16)) return DEC_E_ALIGN;
  dec::EmbedParams p{};
  p.tokens = tokens;
  p.E = static_cast<const uint16_t*>(E);
  p.x = x;
  p.B = B;
  p.n_cb = n_cb;
  p.V_emb = V_emb;
  p.D = D;
  const hipError_t e = dec::embed_sum_launch(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_philox_uniforms(uint64_t seed, int step0, int n_steps, int B, int n_cb, float* out,
                        dec_stream_t stream) {
  if (out == nullptr) return DEC_E_NULL;
  if (n_steps < 1 || B < 1 || n_cb < 1 || step0 < 0) return DEC_E_SHAPE;
  if ((long long)step0 + n_steps > 0x7FFFFFFFLL || (long long)n_steps * B * n_cb > 0x7FFFFFFFLL)
    return DEC_E_SHAPE;
  if (!aligned(out, 4)) return DEC_E_ALIGN;
  const hipError_t e = dec::uniforms_launch(seed, step0, B, n_cb, n_steps * B * n_cb, out,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_step_advance(int32_t* len, int32_t* step, int B, dec_stream_t stream) {
  if (B < 1) return DEC_E_SHAPE;
  if (len == nullptr && step == nullptr) return DEC_E_NULL;
  if (!aligned(len, 4) || !aligned(step, 4)) return DEC_E_ALIGN;
  const hipError_t e = dec::advance_launch(len, step, B, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_probe_read(const void* buf, size_t bytes, uint32_t* sink, dec_stream_t stream) {
  if (buf == nullptr || sink == nullptr) return DEC_E_NULL;
  if (bytes == 0 || bytes % 16 != 0) return DEC_E_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return DEC_E_ALIGN;
  if ((bytes - 1) / (4 * (size_t)dec::kProbeWaveBytes) >= 0x7FFFFFFF) return DEC_E_UNSUPPORTED;
  const hipError_t e = dec::probe_read_launch(buf, bytes, sink, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_probe_empty(dec_stream_t stream) {
  const hipError_t e = dec::probe_empty_launch(reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_probe_clock(uint64_t* clocks, dec_stream_t stream) {
  static_assert(dec::kProbeClockSlots == DEC_PROBE_CLOCK_SLOTS, "header and kernel agree");
  if (clocks == nullptr) return DEC_E_NULL;
  if (!aligned(clocks, 8)) return DEC_E_ALIGN;
  const hipError_t e = dec::probe_clock_launch(clocks, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_graph_begin(dec_stream_t stream) {
  if (stream == nullptr) return DEC_E_NULL;
  const hipError_t e =
      hipStreamBeginCapture(reinterpret_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal);
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_graph_end(dec_stream_t stream, void** exec) {
  if (stream == nullptr || exec == nullptr) return DEC_E_NULL;
  *exec = nullptr;
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(reinterpret_cast<hipStream_t>(stream), &graph);
  if (e != hipSuccess) return hip_fail(e);
  hipGraphExec_t ge = nullptr;
  e = hipGraphInstantiate(&ge, graph, nullptr, nullptr, 0);
  const hipError_t e2 = hipGraphDestroy(graph);
  if (e != hipSuccess) return hip_fail(e);
  if (e2 != hipSuccess) {
    (void)hipGraphExecDestroy(ge);
    return hip_fail(e2);
  }
  *exec = ge;
  return DEC_OK;
}

int dec_graph_launch(void* exec, dec_stream_t stream) {
  if (exec == nullptr) return DEC_E_NULL;
  const hipError_t e =
      hipGraphLaunch(static_cast<hipGraphExec_t>(exec), reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_graph_destroy(void* exec) {
  if (exec == nullptr) return DEC_E_NULL;
  const hipError_t e = hipGraphExecDestroy(static_cast<hipGraphExec_t>(exec));
  return e == hipSuccess ? DEC_OK : hip_fail(e);
}

int dec_tuning_set(const dec_tuning* t) {
  if (t == nullptr) {
    g_tuning = dec_tuning{};
    return DEC_OK;
  }
  const int ck = t->attn_chunk_keys;
  if (ck != 0 && (!is_pow2(ck) || ck < 128 || ck > dec::kAttnChunk)) return DEC_E_SHAPE;
  if (t->attn_schedule < 0 || t->attn_schedule > 2 || t->attn_blocks < 0 ||
      t->attn_no_halves < 0 || t->attn_no_halves > 1 || t->attn_no_records < 0 ||
      t->attn_no_records > 1 || t->head_kernel < 0 || t->head_kernel > 2)
    return DEC_E_SHAPE;
  const int mc = t->head_mfma_cfg;  // the MFMA kernel's instantiated tilings
  if (mc != 0 && mc != 11 && mc != 12 && mc != 22 && mc != 42) return DEC_E_SHAPE;
  g_tuning = *t;
  return DEC_OK;
}

int dec_tuning_get(dec_tuning* t) {
  if (t == nullptr) return DEC_E_NULL;
  *t = g_tuning;
  return DEC_OK;
}

int dec_last_hip_error(void) { return g_last_hip; }

const char* dec_strerror(int status) {
  switch (status) {
    case DEC_OK: return "DEC_OK: success";
    case DEC_E_NULL: return "DEC_E_NULL: a required pointer is NULL";
    case DEC_E_SHAPE: return "DEC_E_SHAPE: a size is out of range or sizes disagree";
    case DEC_E_DTYPE: return "DEC_E_DTYPE: unknown dtype code";
    case DEC_E_WORKSPACE: return "DEC_E_WORKSPACE: workspace too small";
    case DEC_E_UNSUPPORTED: return "DEC_E_UNSUPPORTED: a legal but unimplemented case (e.g. head_dim other than 64 or 128)";
    case DEC_E_HIP: return "DEC_E_HIP: a HIP runtime call failed (see dec_last_hip_error)";
    case DEC_E_ALIGN: return "DEC_E_ALIGN: pointer not aligned as required";
    default: return "unknown dec_status";
  }
}

void dec_order_keys_host(const float* x, uint32_t* keys, size_t n) {
  if (x == nullptr || keys == nullptr) return;
  for (size_t i = 0; i < n; ++i) keys[i] = dec::order_key(x[i]);
}

}  // extern "C"
