// Kernel parameter blocks and launchers shared by the kernel sources and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dec {

// ---- attention (split-K flash-decode over the valid prefix) ----------------------

#ifndef DEC_ATTN_WAVES
#define DEC_ATTN_WAVES 4
#endif
constexpr int kAttnWaves = DEC_ATTN_WAVES;          // waves per workgroup
constexpr int kAttnThreads = 64 * kAttnWaves;
#ifndef DEC_ATTN_TILE_KEYS
#define DEC_ATTN_TILE_KEYS 32
#endif
constexpr int kAttnKeysPerTile = DEC_ATTN_TILE_KEYS;  // keys one wave loads per tile at head
                                                    // dim 64 (at 128: half, same bytes)
constexpr int kAttnMinBlockKeys = 64;               // paged cache: smallest block (keys)
static_assert(kAttnKeysPerTile <= kAttnMinBlockKeys, "a tile never crosses a paged block");
#ifndef DEC_ATTN_CHUNK
#define DEC_ATTN_CHUNK 1024
#endif
constexpr int kAttnChunk = DEC_ATTN_CHUNK;          // keys per chunk (the largest chunk)
constexpr int kAttnHeadDim = 64;                   // the model's head dim; 128 is also built
constexpr int kAttnHeadDimWide = 128;
// keys per tile and tiles per chunk at head dim HD
constexpr int attn_keys_per_tile(int hd) { return kAttnKeysPerTile * kAttnHeadDim / hd; }
constexpr int attn_tiles_per_chunk(int hd) { return kAttnChunk / (kAttnWaves * attn_keys_per_tile(hd)); }
static_assert(attn_tiles_per_chunk(kAttnHeadDim) * kAttnWaves * kAttnKeysPerTile == kAttnChunk,
              "a chunk is a whole number of workgroup tile rounds");
static_assert(attn_tiles_per_chunk(kAttnHeadDimWide) * kAttnWaves *
                      attn_keys_per_tile(kAttnHeadDimWide) == kAttnChunk,
              "a chunk is a whole number of workgroup tile rounds");
// Launches with few sequences may cut chunks smaller, down to this many keys, so that
// every CU gets a work item; a power of two and a whole number of tile rounds.
constexpr int kAttnMinChunk = kAttnWaves * kAttnKeysPerTile > 128 ? kAttnWaves * kAttnKeysPerTile : 128;
static_assert((kAttnMinChunk & (kAttnMinChunk - 1)) == 0 && kAttnMinChunk <= kAttnChunk &&
                  kAttnMinChunk % (kAttnWaves * kAttnKeysPerTile) == 0 &&
                  kAttnMinChunk % (kAttnWaves * attn_keys_per_tile(kAttnHeadDimWide)) == 0,
              "the smallest chunk is a whole number of workgroup tile rounds");
constexpr int attn_log2(int x) { return x <= 1 ? 0 : 1 + attn_log2(x / 2); }
// floats per chunk partial: m, l, pad, pad, acc[hd]
constexpr int attn_part_stride(int hd) { return 4 + hd; }
constexpr int kAttnMaxGroups = 4096;                // (segments x batch) handled per launch
constexpr int kAttnSortMax = 1024;                  // groups ordered longest-first up to this count
constexpr int kAttnSplitBelow = 512;                // below this many sequences per launch, every
                                                    // chunk is its own work item (balance)

// Division by a launch constant d >= 1, exact for every 32-bit x: a multiply-high, an add
// and two shifts (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994; the case whose multiplier needs 33 bits, applied as
// t + ((x - t) >> 1)).  Keeps runtime integer divisions off the work-item decode.
struct DivMagic {
  uint32_t m;
  int s1, s2;
};
constexpr DivMagic div_magic(uint32_t d) {
  int l = 0;
  while ((1ull << l) < d) ++l;  // 2^(l-1) < d <= 2^l
  DivMagic r{};
  r.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  r.s1 = l < 1 ? l : 1;
  r.s2 = l > 1 ? l - 1 : 0;
  return r;
}
__device__ __forceinline__ uint32_t udiv(uint32_t x, const DivMagic& d) {
  const uint32_t t = __umulhi(x, d.m);
  return (t + ((x - t) >> d.s1)) >> d.s2;
}
// The same arithmetic on the host, checked against division at compile time below.
constexpr uint32_t udiv_host(uint32_t x, DivMagic d) {
  const uint32_t t = (uint32_t)(((uint64_t)x * d.m) >> 32);
  return (t + ((x - t) >> d.s1)) >> d.s2;
}
constexpr bool div_magic_ok(uint32_t d) {
  const uint32_t xs[] = {0u, 1u, d - 1u, d, d + 1u, 2u * d - 1u, 2u * d, 12345u, 0x7FFFFFFFu,
                         0x80000000u, 0xFFFFFFFEu, 0xFFFFFFFFu};
  for (uint32_t x : xs)
    if (udiv_host(x, div_magic(d)) != x / d) return false;
  return true;
}
static_assert(div_magic_ok(1) && div_magic_ok(2) && div_magic_ok(3) && div_magic_ok(5) &&
                  div_magic_ok(7) && div_magic_ok(16) && div_magic_ok(24) && div_magic_ok(384) &&
                  div_magic_ok(1000) && div_magic_ok(4095) && div_magic_ok(65537) &&
                  div_magic_ok(0x7FFFFFFFu) && div_magic_ok(0xFFFFFFFFu),
              "multiply-high division agrees with division");
static_assert((kAttnWaves & (kAttnWaves - 1)) == 0, "waves per workgroup: a power of two");

// One attention problem ("segment"): self-attention or cross-attention of a step.
struct AttnSeg {
  const void* q;          // [NL, B, H, hd]
  const void* k;          // [NL, B, H, L_cap, hd]
  const void* v;          // [NL, B, H, L_cap, hd]
  const int32_t* len;     // [B] valid slots
  void* out;              // [NL, B, H, hd] fp32, or bf16 when out_bf16
  float* part;            // [NL*B*H, nck_cap, attn_part_stride(hd)] chunk partials (split mode)
  int32_t* ticket;        // [NL*B*H] chunk arrival counters (split mode), zero between calls
  int L_cap;              // keys a sequence can hold (paged: table_stride << bs_log2)
  int nck_cap;            // ceil(L_cap / chunk), the chunk of this launch
  // paged cache (table != nullptr): k, v are pools [NL, n_blocks, H, 1 << bs_log2, hd]
  const int32_t* table;   // [B, table_stride] physical block of each logical block
  int table_stride;
  int n_blocks;           // physical blocks per layer
  int bs_log2;            // log2(keys per block), at least log2(64)
  // key mask (mask != nullptr): bit j % 32 of word j / 32 of row b set = key j attended
  const uint32_t* mask;   // [B, mask_words], mask_words even
  int mask_words;
  int out_bf16;
  // the current token's rows (static caches): when k_new != nullptr, a sequence with
  // 1 <= len <= L_cap attends with k_new / v_new as its key len - 1 and the launch writes
  // them to that slot of k / v
  const void* k_new;      // [NL, B, H, hd]
  const void* v_new;
};

// One wave's first tile of a launch: the next launch requests the same bytes before it
// has derived its own schedule, and keeps them when its first tile is that one.
struct TileRec {
  int tag;                // bit 0: valid; bit 1: segment 1
  int row;                // (layer, b, head) row of the sequence
  int key0;               // first key of the tile
  int n;                  // valid keys of the sequence (rows of the load's buffer range)
};
constexpr int kAttnRecGroups = 4096;   // workgroups a workspace keeps first-tile records for
constexpr int kAttnRecLdsPerWave = 8192;  // LDS bytes that hold one wave's requested tile

struct AttnParams {
  AttnSeg seg[2];
  int nseg;
  int NL, B, H;
  int hd;                 // 64 or 128 (selects the instantiation)
  int cpi;                // chunks per work item (>= nck_cap of every segment: no split),
                          // a power of two
  int cpi_log2;           // log2(cpi), set by the launcher
  DivMagic div_nlh, div_h;  // division by NL * H and by H, set by the launcher
  int chunk_log2;         // log2(keys per chunk); 0: the launcher chooses
  int min_chunk_log2;     // the smallest chunk the workspace holds partials for
  float qscale;           // scale * log2(e): scores are formed in base 2
  int cus;                // compute units of the device (set by the launcher)
  int balance;            // whole-sequence launches: cut the heavy excess in halves
  TileRec* rec;           // [rec_groups][kAttnWaves] first tiles of the last launch, or null
  int rec_groups;
};

// Upper bound on the work items of a launch (every sequence at full capacity).
long long attn_items_cap(const AttnParams& p);
// Enqueue the attention kernel; `blocks` <= 0 picks the occupancy-sized persistent grid.
hipError_t attn_launch(const AttnParams& p, int dtype, int blocks, hipStream_t stream);

// ---- sampler ---------------------------------------------------------------------

constexpr int kSampWaves = 4;                       // rows (one per wave) per workgroup
constexpr int kSampMaxVocab = 4096;
constexpr int kSampNarrowK = 64;                    // top_k up to this: kept set one per lane

struct SampleParams {
  const void* logits;     // [B, n_cb, V_stride] fp32, or bf16 when logits_bf16
  const float* temperature;
  const float* uniforms;  // [B, n_cb], or unused when rng != 0
  const int32_t* step;
  int32_t* tokens;
  int32_t* topk_idx;
  float* topk_prob;
  unsigned long long seed;  // Philox key word 0 when rng != 0
  int B, n_cb, V_valid, V_stride, top_k, fill;
  int rng;                  // 1: uniforms from Philox4x64-10 at counter (step, b, c, 0)
  int logits_bf16;
  // advance in the same launch: step is then [B, n_cb] (one counter per row) and row r
  // writes step[r] + 1 back; row (b, 0) adds one to len[b] when len_inc is not null
  int32_t* step_inc;
  int32_t* len_inc;
};

hipError_t sample_launch(const SampleParams& p, hipStream_t stream);

// ---- merged LM head and embedding sum ----------------------------------------------------

constexpr int kHeadWaves = 4;   // 8-row groups (one per wave) per workgroup

struct HeadParams {
  const uint16_t* h;      // [B, D] bf16
  const uint16_t* W;      // [n_cb, V_stride, D] bf16
  float* logits;          // [B, n_cb, V_stride]; columns >= V_valid untouched
  int B, D, n_cb, V_valid, V_stride;
  int force_gemv;         // 1: the vector-ALU kernel at every batch size (tests)
  int mfma_cfg;           // MFMA path: 10 * row tiles + batch tiles per workgroup, 0: by B
};

struct EmbedParams {
  const int32_t* tokens;  // [B, n_cb]
  const uint16_t* E;      // [n_cb, V_emb, D] bf16
  float* x;               // [B, D]
  int B, n_cb, V_emb, D;
};

hipError_t lm_head_launch(const HeadParams& p, hipStream_t stream);
hipError_t embed_sum_launch(const EmbedParams& p, hipStream_t stream);

// ---- small utility kernels ------------------------------------------------------------

hipError_t fill_zero_launch(void* ptr, size_t bytes, hipStream_t stream);

// ---- cache append: the current token's K/V rows into slot len[b] - 1 --------------------

struct AppendParams {
  const void* k_new;      // [NL, B, H, row_bytes]
  const void* v_new;
  void* k_cache;          // [NL, B, H, L_cap, row_bytes]
  void* v_cache;
  const int32_t* len;     // [B]
  int NL, B, H, L_cap;
  int row16;              // 16-byte pieces per row
};

hipError_t append_launch(const AppendParams& p, hipStream_t stream);
hipError_t advance_launch(int32_t* len, int32_t* step, int B, hipStream_t stream);

// ---- uniforms of several steps in one launch -----------------------------------------

// out[(s * B + b) * n_cb + c] = the Philox4x64-10 uniform of row (b, c) at step step0 + s
// (the value the sampler draws for that row and step); total = n_steps * B * n_cb.
hipError_t uniforms_launch(uint64_t seed, int step0, int B, int n_cb, int total, float* out,
                           hipStream_t stream);

}  // namespace dec
