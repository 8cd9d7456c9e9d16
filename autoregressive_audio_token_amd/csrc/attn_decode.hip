// Single-token attention over the valid prefix of static KV caches (gfx950).
//
// "Optimized Parler TTS", "Analysis and improvements": with static caches the
// attention kernel moved the whole preallocated cache every step and became
// several times slower than the dynamic-cache one.  This kernel reads only the
// first len[b] slots of each sequence, so its HBM traffic is the valid K/V
// bytes plus a few hundred bytes per sequence.
//
// Split-K flash-decode, arranged for CDNA4:
//   * A sequence of n valid keys is cut into chunks of 1024 keys (a launch with
//     too few chunks to give every CU one cuts them smaller, down to 128).  A
//     workgroup of kAttnWaves wavefronts streams a chunk in tile rounds: in
//     each round every wave reads a 32-key tile (a key row of 64 bf16 is 128 B
//     = 8 lanes x 16 B, so one dwordx4 load instruction covers 8 consecutive
//     keys, 1 KiB, fully coalesced; at head dim 128 a tile is 16 keys of 256 B,
//     the same bytes), and the next tile's K and V loads are in flight while
//     the current tile is computed (double buffering).  Tiles of this size keep
//     the bf16 static kernel at four waves per SIMD (128 VGPRs) and the other
//     variants at three.  There is no MFMA: the work is a GEMV, bound by HBM.
//   * Scores reduce across the 8 lanes of a key with DPP moves.  Each group of
//     8 lanes keeps its own online-softmax state across the tiles (base 2, q
//     pre-scaled by scale * log2 e, fp32), so a tile needs no cross-lane max.
//     At the end of a chunk the groups merge with DPP/shuffle butterflies and
//     the waves merge through LDS, in a fixed order, into one chunk state.
//   * Chunk states of a sequence fold in chunk order.  When a launch has many
//     sequences, one workgroup owns every chunk of its sequence and folds in
//     registers: nothing crosses workgroups.  When it has few, every chunk is
//     its own work item (so the CUs get equal bytes): the chunk's workgroup
//     writes its state with agent-coherent (write-through) stores, waits for
//     them, and takes a ticket with an agent-scope atomic; the last to arrive
//     reads every chunk state with agent-coherent loads, folds them in chunk
//     order and resets the ticket.  No L2 write-back or invalidate is needed,
//     and both modes fold the same fp32 chunk states in the same order, so
//     results are bitwise equal either way and independent of the grid.
//   * Short sequences are packed several to a workgroup (one or two waves
//     each).  The work list is derived on the device from len[] (device
//     resident, so a captured graph stays valid as lengths change), longest
//     sequences first; a persistent, occupancy-sized grid walks it.
//   * A launch whose sequences each get one workgroup cuts the excess of its
//     heaviest sequences (beyond a multiple of the CU count) in halves, so every
//     CU carries nearly the same bytes.
//   * Each wave records in the workspace the tile it read first; the next launch
//     on the workspace requests that tile into LDS before deriving its schedule
//     and uses it only when its own first tile is the same one.

#include "dec_common.h"
#include "dec_kernels.h"

namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor word 3 for raw (untyped) buffer access on the gfx9 family,
// and the cache-policy bit of a non-temporal access.
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufNonTemporal = 2;

// A raw buffer over `rows` rows of `row_bytes` bytes starting at `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int rows,
                                                            int row_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, rows * row_bytes,
                                           kBufWord3);
}

template <typename T>
struct KvTraits;
template <>
struct KvTraits<uint16_t> {  // bfloat16 bit patterns
  static constexpr int kElemsPerLoad = 8;
};
template <>
struct KvTraits<float> {
  static constexpr int kElemsPerLoad = 4;
};

__device__ __forceinline__ void unpack(const u32x4& w, float (&x)[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void unpack(const u32x4& w, float (&x)[4]) {
  // element values, not element lvalues: bit-casting a vector-element lvalue
  // miscompiles to element 0 with this compiler
  x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
  x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// A 32-bit word as two packed bf16.  Taken by value: bit-casting a vector-element
// lvalue directly miscompiles to element 0 with this compiler.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// <q, k> over one 16-byte slice.  bf16: four packed bf16 pairs, each a
// v_dot2c_f32_bf16 (products exact, fp32 accumulation); q stays packed bf16.
// fp32: four fmas on q pre-converted to fp32.
__device__ __forceinline__ float dot_slice(const u32x4& q, const u32x4& k) {
  float s = 0.f;
  s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.x), as_bf16x2(k.x), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.y), as_bf16x2(k.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.z), as_bf16x2(k.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w), as_bf16x2(k.w), s, false);
  return s;
}
__device__ __forceinline__ float dot_slice(const float (&q)[4], const u32x4& w) {
  float x[4];
  unpack(w, x);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s = fmaf(q[e], x[e], s);
  return s;
}

// This lane's 16-byte slice of the query, and how a score is finished.
template <typename T>
struct QSlice;
template <>
struct QSlice<uint16_t> {  // packed bf16; the scale is applied to the finished score
  u32x4 q;
  float scale;
  __device__ __forceinline__ void load(const uint16_t* qp, float qscale) {
    q = *reinterpret_cast<const u32x4*>(qp);
    scale = qscale;
  }
  __device__ __forceinline__ float dot(const u32x4& k) const { return dot_slice(q, k); }
  __device__ __forceinline__ float finish(float s) const { return s * scale; }
};
template <>
struct QSlice<float> {  // fp32, pre-scaled
  float q[4];
  __device__ __forceinline__ void load(const float* qp, float qscale) {
    unpack(*reinterpret_cast<const u32x4*>(qp), q);
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] *= qscale;
  }
  __device__ __forceinline__ float dot(const u32x4& k) const { return dot_slice(q, k); }
  __device__ __forceinline__ float finish(float s) const { return s; }
};

// 2^x by the hardware exponential (results below the fp32 normal range flush to 0,
// a relative weight under 1e-38 that no output can show).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int EPL>
__device__ __forceinline__ void accum_slice(float (&acc)[EPL], float p, const u32x4& w) {
  float x[EPL];
  unpack(w, x);
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, x[e], acc[e]);
}

// Chunks of 1 << clog keys covering n keys.
__device__ __forceinline__ int nchunks(int n, int clog) {
  return n > 0 ? ((n - 1) >> clog) + 1 : 0;
}

// Work items per (layer, head) of a sequence with n valid keys (1 << cpi_log2 chunks each).
__device__ __forceinline__ int items_per_lh(int n, int cpi_log2, int clog) {
  const int c = nchunks(n, clog);
  return c > (1 << cpi_log2) ? ((c - 1) >> cpi_log2) + 1 : 1;
}

// Waves that share one sequence: the smallest power of two covering n keys in one
// round, or every wave of the workgroup (then the sequence runs in chunk rounds).
// Shorter sequences are packed kAttnWaves / S to a work item.  At least HD / 64
// waves: the workgroup's threads combine kAttnThreads / HD sequences at a time.
template <int HD>
__device__ __forceinline__ int waves_per_seq(int n) {
  int s = HD / kAttnHeadDim < kAttnWaves ? HD / kAttnHeadDim : kAttnWaves;
  while (s < kAttnWaves && s * attn_keys_per_tile(HD) < n) s <<= 1;
  return s;
}

// Work items of a (segment, b) group with n valid keys.
template <int HD>
__device__ __forceinline__ int group_items(int n, int NLH, int cpi_log2, int clog) {
  const int S = waves_per_seq<HD>(n);  // a power of two
  if (S < kAttnWaves) {
    const int pl = __builtin_ctz(kAttnWaves) - __builtin_ctz(S);  // log2(sequences per item)
    return (NLH + (1 << pl) - 1) >> pl;
  }
  return NLH * items_per_lh(n, cpi_log2, clog);
}

// Fold chunk state (mc, lc, ac) into the running state (m, l, a); the first
// chunk initialises it.  Shared by both fold sites so they agree bit for bit.
// EX (key masks): a chunk may have no attended key (mc = -inf) and is skipped.
template <bool EX>
__device__ __forceinline__ void fold_chunk(bool first, float mc, float lc, float ac, float& m,
                                           float& l, float& a) {
  if (first) {
    m = mc;
    l = lc;
    a = ac;
    return;
  }
  if (EX && mc == -INFINITY) return;
  const float mn = fmaxf(m, mc);
  const float fa = exp2_hw(m - mn);
  const float fc = exp2_hw(mc - mn);
  l = fmaf(lc, fc, l * fa);
  a = fmaf(ac, fc, a * fa);
  m = mn;
}

// One wave's view of a tile of KPT keys: NLD loads per operand, each covering KPL keys.
// A tile holds the same bytes at either head dim (32 keys of 64, 16 keys of 128).
template <typename T, int HD>
struct Tile {
  static constexpr int EPL = KvTraits<T>::kElemsPerLoad;  // elements per lane per load
  static constexpr int LPK = HD / EPL;                    // lanes per key row: 8 / 16 (bf16),
                                                          // 16 / 32 (f32) at HD 64 / 128
  static constexpr int KPL = kWave / LPK;                 // keys per wave-wide load
  static constexpr int KPT = attn_keys_per_tile(HD);      // keys per tile
  static constexpr int NLD = KPT / KPL;                   // loads per operand per tile
  u32x4 k[NLD], v[NLD];

  // Buffer loads through a descriptor that spans exactly the sequence's valid
  // prefix (n rows): rows at or past n fall outside the descriptor's range and
  // return zero without touching memory (their scores are masked to -inf in
  // consume).  lane_off is this lane's byte offset inside a wave-wide load.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                       int base, int lane_off) {
    constexpr int kRowBytes = HD * (int)sizeof(T);
    const int tile_off = base * kRowBytes + lane_off;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int off = tile_off + i * KPL * kRowBytes;
      // K and V are read once: non-temporal
      k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kBufNonTemporal);
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kBufNonTemporal);
    }
  }

  // The same requests with the data landing in LDS instead of registers (8 KiB per wave:
  // NLD wave-wide loads of K, then of V, each 1 KiB in lane order).
  static __device__ __forceinline__ void load_lds_static(__amdgpu_buffer_rsrc_t rk,
                                                         __amdgpu_buffer_rsrc_t rv, int base,
                                                         int lane_off, u32x4* lds) {
    constexpr int kRowBytes = HD * (int)sizeof(T);
    const int tile_off = base * kRowBytes + lane_off;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int off = tile_off + i * KPL * kRowBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(lds + i * kWave), 16, off, 0, 0,
          kBufNonTemporal);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)(lds + (NLD + i) * kWave), 16, off, 0, 0,
          kBufNonTemporal);
    }
  }
  // Registers from a completed load_lds (the caller has waited for it).
  __device__ __forceinline__ void from_lds(const u32x4* lds, int lane) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      k[i] = lds[i * kWave + lane];
      v[i] = lds[(NLD + i) * kWave + lane];
    }
  }

  // The key `row` of the sequence, if this tile holds it, becomes the lanes' slices kn, vn
  // (the current token's rows, which the cache does not hold yet); the lanes holding it
  // also write them to that row of the sequence's cache (kseq, vseq; this lane's slice at
  // element offset `slice`).  Uniform test: one tile per sequence takes the branch.
  __device__ __forceinline__ void put_row(int base, int row, int kg, const u32x4& kn,
                                          const u32x4& vn, const T* kseq, const T* vseq,
                                          int slice) {
    const int j = row - base;
    if ((unsigned)j >= (unsigned)KPT) return;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const bool mine = j == i * KPL + kg;
      k[i] = mine ? kn : k[i];
      v[i] = mine ? vn : v[i];
    }
    if (j % KPL == kg) {
      const size_t off = (size_t)row * HD + slice;
      *reinterpret_cast<u32x4*>(const_cast<T*>(kseq) + off) = kn;
      *reinterpret_cast<u32x4*>(const_cast<T*>(vseq) + off) = vn;
    }
  }

  // Online-softmax update of this lane group's state (m, l, acc) with the tile.
  // MASK: bit j of `keep` says whether key base + j is attended (a boolean key mask).
  template <bool MASK = false>
  __device__ __forceinline__ void consume(const QSlice<T>& qs, int base, int n, int kg,
                                          float& m, float& l, float (&acc)[EPL],
                                          uint64_t keep = ~0ull) const {
    float s[NLD];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      s[i] = qs.finish(group_sum<LPK>(qs.dot(k[i])));
      if (base + i * KPL + kg >= n) s[i] = -INFINITY;
      if (MASK && ((keep >> (i * KPL + kg)) & 1ull) == 0ull) s[i] = -INFINITY;
      tmax = fmaxf(tmax, s[i]);
    }
    if (tmax == -INFINITY) return;  // no valid key of this group in the tile
    const float mn = fmaxf(m, tmax);
    const float corr = exp2_hw(m - mn);  // 0 while m is still -inf
    l *= corr;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= corr;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const float pj = exp2_hw(s[i] - mn);
      l += pj;
      accum_slice(acc, pj, v[i]);
    }
    m = mn;
  }
};

// Buffer descriptors for one tile's K and V rows, the tile's first row inside them,
// and (key masks) which of its keys are attended.
struct TileAddr {
  __amdgpu_buffer_rsrc_t k, v;
  int row0;
  uint64_t keep;
};

// An output element a / l.  EX: fp32 or bfloat16 (rounded to nearest even), and zero
// for a sequence with no attended key (l == 0, only under a key mask).
template <bool EX>
__device__ __forceinline__ void store_out(const AttnSeg& S, size_t i, float a, float l) {
  if (!EX) {
    static_cast<float*>(S.out)[i] = a / l;
    return;
  }
  const float v = l > 0.f ? a / l : 0.f;
  if (S.out_bf16) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    static_cast<uint16_t*>(S.out)[i] = (uint16_t)r;
  } else {
    static_cast<float*>(S.out)[i] = v;
  }
}

// PAGED: segments with a block table read each tile through a descriptor over its block of
// the pool (a tile of at most 64 keys never crosses a block); other segments read the
// static layout.  EX: the widened entry point -- segments with a key bitmask skip the
// keys whose bit is clear, and outputs may be bf16.  HD: head dim, 64 or 128.
// Waves per SIMD the compiler is held to: four (128 VGPRs) for the bf16 kernels of static
// or paged caches, which fit there; the masked, appending and fp32 kernels need more
// registers and get what their code needs (three, two).
template <typename T, bool PAGED, bool EX, bool APP>
constexpr int attn_waves_per_eu() { return (sizeof(T) == 2 && !EX && !APP) ? 4 : 1; }

template <typename T, bool PAGED, bool EX, int HD, bool APP = false>
__global__ __launch_bounds__(kAttnThreads) __attribute__((
    amdgpu_waves_per_eu(attn_waves_per_eu<T, PAGED, EX, APP>()))) void attn_decode_kernel(AttnParams p) {
  using TileT = Tile<T, HD>;
  constexpr int EPL = TileT::EPL;
  constexpr int LPK = TileT::LPK;
  constexpr int KPT = TileT::KPT;
  constexpr int PS = attn_part_stride(HD);
  static_assert(kAttnThreads % HD == 0, "whole sequences per combining pass");
  static_assert(sizeof(T) != 2 || 2 * TileT::NLD * kWave * 16 == kAttnRecLdsPerWave,
                "a requested bf16 tile is kAttnRecLdsPerWave bytes per wave");
  static_assert(!EX || KPT == 16 || KPT == 32 || KPT == 64, "a tile's mask bits lie in whole words");

  extern __shared__ __align__(16) int s_dyn[];  // layout below
  __shared__ float s_acc[kAttnWaves][HD];
  __shared__ float s_m[kAttnWaves];
  __shared__ float s_l[kAttnWaves];
  __shared__ int s_wsum[kAttnWaves];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // uniform per wave; said explicitly so the sequence, its pointers and its buffer
  // descriptors stay in scalar registers (a descriptor the compiler must treat as
  // per-lane turns every buffer load into a readfirstlane loop)
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int B = p.B;
  const int G = p.nseg * B;
  const int NLH = p.NL * p.H;
  const int cpl = p.cpi_log2;      // chunks per work item: 1 << cpl
  const int clog = p.chunk_log2;  // keys per chunk: 1 << clog, whole tile rounds
  // dynamic LDS: [the waves' requested tiles, when records are kept][G] lengths, [G]
  // order, [G+1] item prefix
  const int rec_ints = p.rec != nullptr ? kAttnWaves * kAttnRecLdsPerWave / 4 : 0;
  int* s_n = s_dyn + rec_ints;
  int* s_order = s_n + G;
  int* s_pref = s_n + 2 * G;

  const int kg = lane / LPK;  // key slot within a wave-wide load (lane group)
  const int dl = lane % LPK;  // which 16-byte slice of the row this lane reads
  constexpr int kRowBytes = HD * (int)sizeof(T);
  const int lane_off = kg * kRowBytes + dl * 16;

  // The lengths (up to 64 groups: lane g loads group g's) go out first: a wave's loads
  // return in order, so a length load issued after the requested tile would wait for it.
  int len_raw = 0;
  if (G <= kWave) {  // every lane loads (lanes past G re-read group 0): no divergent branch
    const int gl = lane < G ? lane : 0;
    const bool cross = gl >= B;
    len_raw = (cross ? p.seg[1].len : p.seg[0].len)[cross ? gl - B : gl];
  }

  // ---- the last launch's first tile of this wave, requested at once ------------------
  // Deriving the schedule takes microseconds at the start of a launch (the instruction
  // cache starts cold), so a wave first requests the tile it read first in the last
  // launch that used this workspace.  The address comes from this call's own arguments
  // and is checked against them, so a stale record can only cost bytes; the data is used
  // only when this launch's first tile is exactly that one (same bytes requested).
  constexpr bool REC = !PAGED && !EX && sizeof(T) == 2;
  // (the dynamic LDS holds the waves' requested tiles first when records are kept)
  u32x4* const s_spec = reinterpret_cast<u32x4*>(s_dyn) + wave * 2 * TileT::NLD * kWave;
  TileRec spec{0, 0, 0, 0};
  bool spec_live = false;
  const bool use_rec = REC && p.rec != nullptr && (int)blockIdx.x < p.rec_groups;
  TileRec r{0, 0, 0, 0};
  if (use_rec) r = p.rec[blockIdx.x * kAttnWaves + wave];
  // both small loads are in flight together and have landed here, before any tile request
  asm volatile("" ::"v"(len_raw), "v"(r.tag), "v"(r.row), "v"(r.key0), "v"(r.n));
  if (use_rec) {
    spec.tag = __builtin_amdgcn_readfirstlane(r.tag);
    spec.row = __builtin_amdgcn_readfirstlane(r.row);
    spec.key0 = __builtin_amdgcn_readfirstlane(r.key0);
    spec.n = __builtin_amdgcn_readfirstlane(r.n);
    const int sseg = (spec.tag >> 1) & 1;
    const int cap = sseg ? p.seg[1].L_cap : p.seg[0].L_cap;
    if ((spec.tag & 1) && sseg < p.nseg && spec.row >= 0 && spec.row < B * NLH &&
        spec.key0 >= 0 && spec.key0 < spec.n && spec.n <= cap) {
      const T* kb = static_cast<const T*>(sseg ? p.seg[1].k : p.seg[0].k);
      const T* vb = static_cast<const T*>(sseg ? p.seg[1].v : p.seg[0].v);
      const size_t off = (size_t)spec.row * cap * HD;
      TileT::load_lds_static(rows_rsrc(kb + off, spec.n, kRowBytes),
                             rows_rsrc(vb + off, spec.n, kRowBytes), spec.key0, lane_off, s_spec);
      spec_live = true;
    }
  }
  bool rec_pending = REC && p.rec != nullptr && (int)blockIdx.x < p.rec_groups;

  // ---- item list: groups (segment, b) longest first; group_items(n) each -------------
  // Up to 64 groups: every wave derives the list in registers (lane r holds the group of
  // rank r and the inclusive item prefix), so no wave waits on another.  More groups:
  // the list is built in LDS and searched.
  const bool in_regs = G <= kWave;
  int r_n = 0, r_order = 0, r_items = 0, r_incl = 0, total = 0;
  int half_E = 0, half_g = -1;  // balance: E sequences of group half_g cut in halves
  if (in_regs) {
    int n = 0, items = 0;
    {
      const int cap = lane >= B ? p.seg[1].L_cap : p.seg[0].L_cap;
      n = lane < G ? (len_raw < 0 ? 0 : (len_raw > cap ? cap : len_raw)) : 0;
      items = lane < G ? group_items<HD>(n, NLH, cpl, clog) : 0;
    }
    int rank = 0;  // stable rank by descending length
    for (int j = 0; j < G; ++j) {
      const int nj = __builtin_amdgcn_readlane(n, j);
      rank += (nj > n || (nj == n && j < lane)) ? 1 : 0;
    }
    // lane `rank` receives the group and its item count (a permutation of lanes < G)
    const int dst = (lane < G ? rank : lane) * 4;
    r_n = n;
    r_order = __builtin_amdgcn_ds_permute(dst, lane);
    r_items = __builtin_amdgcn_ds_permute(dst, items);
    // balance (whole-sequence launches): the heavy class -- every sequence of the longest
    // length, each a whole one-chunk item -- lands two to a CU on some CUs and one on
    // others when its count is not a multiple of the CU count.  Its excess E (when at
    // least a quarter of the CUs) is cut in halves, the last E sequences of the longest
    // group; the 2E halves come first in the list, so they take the older workgroup slot
    // of 2E CUs and fold while the CU's whole sequence still streams.
    if (p.balance) {
      const int g_top = __builtin_amdgcn_readlane(r_order, 0);
      const int n_top = __builtin_amdgcn_readlane(n, g_top);
      if (waves_per_seq<HD>(n_top) == kAttnWaves && nchunks(n_top, clog) == 1 &&
          n_top > (1 << (clog - 1))) {
        const int heavy = __popcll(__ballot(lane < G && n == n_top)) * NLH;
        const int E = heavy % p.cus;
        if (4 * E >= p.cus && E <= NLH) {
          half_E = E;
          half_g = g_top;
        }
      }
      if (lane == 0) r_items += half_E;
    }
    r_incl = wave_inclusive_sum_int(lane < G ? r_items : 0, lane);
    total = __builtin_amdgcn_readlane(r_incl, G - 1);
  } else {
    for (int g = tid; g < G; g += kAttnThreads) {
      const bool cross = g >= B;
      const int32_t* len = cross ? p.seg[1].len : p.seg[0].len;
      const int cap = cross ? p.seg[1].L_cap : p.seg[0].L_cap;
      int n = len[cross ? g - B : g];
      s_n[g] = n < 0 ? 0 : (n > cap ? cap : n);
    }
    __syncthreads();
    for (int g = tid; g < G; g += kAttnThreads) {
      int rank = g;
      if (G <= kAttnSortMax) {  // stable rank by descending length
        const int ng = s_n[g];
        rank = 0;
        for (int j = 0; j < G; ++j) {
          const int nj = s_n[j];
          rank += (nj > ng || (nj == ng && j < g)) ? 1 : 0;
        }
      }
      s_order[rank] = g;
    }
    __syncthreads();
    const int per = (G + kAttnThreads - 1) / kAttnThreads;
    const int lo = min(G, tid * per);
    const int hi = min(G, lo + per);
    int local = 0;
    for (int i = lo; i < hi; ++i) local += group_items<HD>(s_n[s_order[i]], NLH, cpl, clog);
    int ex = wave_inclusive_sum_int(local, lane) - local;
    if (lane == kWave - 1) s_wsum[wave] = ex + local;
    __syncthreads();
    for (int w = 0; w < kAttnWaves; ++w) {
      if (w < wave) ex += s_wsum[w];
      total += s_wsum[w];
    }
    for (int i = lo; i < hi; ++i) {
      s_pref[i] = ex;
      ex += group_items<HD>(s_n[s_order[i]], NLH, cpl, clog);
    }
    if (tid == 0) s_pref[G] = total;
    __syncthreads();
  }

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // locate the group of this item and the item's index within the group
    int g, n, r;
    if (in_regs) {  // sorted position: the number of groups whose items end at or before it
      const int pos = __popcll(__ballot(lane < G && r_incl <= item));
      g = __builtin_amdgcn_readlane(r_order, pos);
      r = item - (__builtin_amdgcn_readlane(r_incl, pos) - __builtin_amdgcn_readlane(r_items, pos));
      n = __builtin_amdgcn_readlane(r_n, g);
    } else {  // the largest position with s_pref[pos] <= item
      int lo = 0, hi = G - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] <= item) lo = mid; else hi = mid - 1;
      }
      g = s_order[lo];
      n = s_n[g];
      r = item - s_pref[lo];
    }
    const bool cross = g >= B;
    const AttnSeg& S = cross ? p.seg[1] : p.seg[0];
    const int b = cross ? g - B : g;
    // a half of a cut heavy sequence (chunks of half the launch's keys, two of them)
    int half_r = -1;
    if (g == half_g) {
      if (r < 2 * half_E) half_r = r;
      else r -= 2 * half_E;
    }
    const int iclog = half_r >= 0 ? clog - 1 : clog;  // keys per chunk of this item: 1 << iclog
    const int nck = nchunks(n, iclog);
    const int spw = waves_per_seq<HD>(n);        // waves per sequence, a power of two
    const int spw_l = __builtin_ctz(spw);
    const bool packed = spw < kAttnWaves;        // several sequences share this item
    const int P = kAttnWaves >> spw_l;           // sequences in this item (packed)

    // this wave's sequence and its first key within each chunk.  Unpacked items of a group
    // run chunk-major: item r holds chunk group r / NLH of (layer, head) r % NLH.
    int wave_lh, wave_part, c0, c1;
    bool whole;
    if (packed) {  // one tile per wave, one chunk
      wave_lh = r * P + (wave >> spw_l);
      wave_part = wave & (spw - 1);
      c0 = 0;
      c1 = nck;
      whole = true;
    } else if (half_r >= 0) {
      wave_lh = NLH - half_E + (half_r >> 1);
      wave_part = wave;
      c0 = half_r & 1;
      c1 = c0 + 1;
      whole = false;
    } else {
      const int ipl = items_per_lh(n, cpl, clog);
      const int k = ipl == 1 ? 0 : (int)udiv((uint32_t)r, p.div_nlh);
      wave_lh = r - k * NLH;
      wave_part = wave;
      c0 = k << cpl;
      c1 = min(nck, c0 + (1 << cpl));
      whole = ipl == 1;
    }
    const bool wave_ok = wave_lh < NLH;  // the last packed item may have empty slots
    const int wlh = wave_ok ? wave_lh : 0;
    const int wl = (int)udiv((uint32_t)wlh, p.div_h);  // layer, and head wlh - wl * H
    const int wh = wlh - wl * p.H;
    const size_t wave_sidx = ((size_t)wl * B + b) * p.H + wh;

    // the combining threads: sequence slot `slot`, head dimension `d`
    const int slot = tid / HD;
    const int d = tid % HD;
    const int nslot = packed ? P : 1;
    const int slot_lh = packed ? r * P + slot : wave_lh;
    const bool slot_ok = slot < nslot && slot_lh < NLH;
    const int slh = slot_ok ? slot_lh : 0;
    const int sl = (int)udiv((uint32_t)slh, p.div_h);
    const size_t slot_sidx = ((size_t)sl * B + b) * p.H + (slh - sl * p.H);

    // this launch's first tile of the wave: compared with the requested one, and recorded
    // for the next launch (waves without a tile record none)
    bool spec_hit = false;
    if (REC && rec_pending) {
      const int key0 = (c0 << iclog) + wave_part * KPT;
      const bool has = wave_ok && key0 < n;
      // an appending launch takes key n - 1 of a self sequence from the new rows, never
      // from the cache, so a record one key shorter (the last step's) holds every row
      // this launch reads from memory (records exist only with the list in registers, so
      // lane b holds sequence b's length as given)
      const bool grown = APP && !cross && S.k_new != nullptr && n == spec.n + 1 &&
                         __builtin_amdgcn_readlane(len_raw, b) <= S.L_cap;
      spec_hit = spec_live && has && spec.tag == (1 | (cross ? 2 : 0)) &&
                 spec.row == (int)wave_sidx && spec.key0 == key0 &&
                 (spec.n == n || key0 + KPT <= min(n, spec.n) || grown);
      if (lane == 0)
        p.rec[blockIdx.x * kAttnWaves + wave] =
            has ? TileRec{1 | (cross ? 2 : 0), (int)wave_sidx, key0, n} : TileRec{0, 0, 0, 0};
      rec_pending = false;
    }

    if (n == 0) {  // no valid key: defined output of zeros
      if (slot_ok) {
        if (EX) store_out<EX>(S, slot_sidx * HD + d, 0.f, 0.f);
        else static_cast<float*>(S.out)[slot_sidx * HD + d] = 0.f;
      }
      continue;
    }

    constexpr int kStep = kAttnWaves * KPT;  // keys between a wave's tiles
    const int tpc = (1 << iclog) / kStep;    // a wave's tiles per chunk
    // chunk states per sequence in the workspace at this item's chunk
    const int nck_cap = iclog == clog ? S.nck_cap : ((S.L_cap - 1) >> iclog) + 1;
    const bool paged = PAGED && S.table != nullptr;  // uniform: per segment
    const T* kp = static_cast<const T*>(S.k);
    const T* vp = static_cast<const T*>(S.v);
    size_t head_off = 0;  // paged: offset of (layer, head) inside a block, before the block term
    if (paged) {
      head_off = (size_t)wl * S.n_blocks;  // layer's first block
    } else {
      kp += wave_sidx * (size_t)S.L_cap * HD;
      vp += wave_sidx * (size_t)S.L_cap * HD;
    }
    // static: one descriptor over the whole valid prefix (paged: none, so no rows).  A
    // tile that must move no bytes is addressed at row `none`, the end of that range:
    // every lane is out of range, reads zero and makes no memory request.
    const __amdgpu_buffer_rsrc_t rk_seq = rows_rsrc(kp, paged ? 0 : n, kRowBytes);
    const __amdgpu_buffer_rsrc_t rv_seq = rows_rsrc(vp, paged ? 0 : n, kRowBytes);
    const int none = paged ? 0 : n;
    float fm = 0.f, fl = 0.f, fa = 0.f;  // running fold (combining threads)
    const T* qp = static_cast<const T*>(S.q) + wave_sidx * HD + dl * EPL;
    // the current token's rows (static caches): key n - 1 is taken from k_new / v_new and
    // written to the cache by the lanes that hold it; a length past the capacity appends
    // nothing (the cache's rows are read as they are)
    int app_row = -1;
    u32x4 kn = {0u, 0u, 0u, 0u}, vn = {0u, 0u, 0u, 0u};
    if (APP && S.k_new != nullptr) {  // uniform: the self segment of an appending launch
      if (S.len[b] <= S.L_cap) app_row = n - 1;
      const size_t src = wave_sidx * HD + dl * EPL;
      kn = *reinterpret_cast<const u32x4*>(static_cast<const T*>(S.k_new) + src);
      vn = *reinterpret_cast<const u32x4*>(static_cast<const T*>(S.v_new) + src);
    }

    for (int c = c0; c < c1; ++c) {
      // tile t of this wave starts at key cb + t * kStep; packed items read one tile
      const int cb = (c << iclog) + wave_part * KPT;
      float m_g = -INFINITY, l_g = 0.f;  // this lane group's online state
      float acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
      if (wave_ok && cb < n) {  // uniform across the wave
        const int nt = packed ? 1 : min(tpc, (n - cb + kStep - 1) / kStep);
        // paged: lane i < nt holds the physical block of the wave's tile i in this chunk
        int blk_of = 0;
        if (paged && lane < nt)
          blk_of = S.table[(size_t)b * S.table_stride + ((cb + lane * kStep) >> S.bs_log2)];
        // key masks: lane i < nt holds the mask bits of the wave's tile i in this chunk, so
        // a tile's bits are a register read, not a load on its address path
        uint32_t mask_lo = ~0u, mask_hi = ~0u;
        if (EX && S.mask != nullptr && lane < nt) {
          const int base_i = cb + lane * kStep;
          const uint32_t* mw = S.mask + (size_t)b * S.mask_words + (base_i >> 5);
          if (KPT == 64) {
            mask_lo = mw[0];
            mask_hi = mw[1];
          } else {
            mask_lo = (mw[0] >> (base_i & 31)) & (KPT == 32 ? 0xFFFFFFFFu : 0xFFFFu);
          }
        }
        auto addr = [&](int t) -> TileAddr {
          const int base = cb + t * kStep;
          // past this wave's tiles of the chunk: out of range, so the pipeline's last
          // prefetch moves no bytes (the next chunk loads its own)
          if (t >= nt) return {rk_seq, rv_seq, none, 0ull};
          uint64_t keep = ~0ull;
          if (EX && S.mask != nullptr) {  // the tile's KPT mask bits (uniform)
            keep = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mask_lo, t);
            if (KPT == 64) keep |= (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mask_hi, t) << 32;
            // no attended key in the tile: nothing to read (every score is masked)
            if (keep == 0ull) return {rk_seq, rv_seq, none, 0ull};
          }
          if (!paged) return {rk_seq, rv_seq, base, keep};
          const int bs = 1 << S.bs_log2;
          const int row = base & (bs - 1);
          const int blk = __builtin_amdgcn_readlane(blk_of, t);
          // rows of this tile inside its block; none past n or for an entry outside the pool
          int rows = base < n ? min(bs - row, n - base) : 0;
          if (blk < 0 || blk >= S.n_blocks) rows = 0;
          const size_t off = (((head_off + (size_t)(unsigned)blk) * p.H + wh) * bs + row) * HD;
          return {rows_rsrc(kp + off, rows, kRowBytes), rows_rsrc(vp + off, rows, kRowBytes), 0,
                  keep};
        };
        TileT ta, tb;
        const TileAddr a0 = addr(0);
        if (spec_hit && c == c0) {  // the requested tile is this one: wait for it in LDS
          __builtin_amdgcn_s_waitcnt(0);
          ta.from_lds(s_spec, lane);
        } else {
          ta.load(a0.k, a0.v, a0.row0, lane_off);
        }
        uint64_t keep_a = a0.keep;
        QSlice<T> qs;  // after the first tile's loads, so K/V requests leave first
        qs.load(qp, p.qscale);
        // ping-pong: the next tile is in flight while one is consumed (past n the
        // prefetch lies wholly outside its descriptor: no traffic)
#pragma nounroll
        for (int t = 0; t < nt; t += 2) {
          const int base = cb + t * kStep;
          const TileAddr a1 = addr(t + 1);
          tb.load(a1.k, a1.v, a1.row0, lane_off);
          if constexpr (APP) ta.put_row(base, app_row, kg, kn, vn, kp, vp, dl * EPL);
          ta.template consume<EX>(qs, base, n, kg, m_g, l_g, acc, keep_a);
          if (t + 1 >= nt) break;
          const TileAddr a2 = addr(t + 2);
          ta.load(a2.k, a2.v, a2.row0, lane_off);
          if constexpr (APP) tb.put_row(base + kStep, app_row, kg, kn, vn, kp, vp, dl * EPL);
          tb.template consume<EX>(qs, base + kStep, n, kg, m_g, l_g, acc, a1.keep);
          keep_a = a2.keep;
        }
      }
      // merge the lane groups of the wave, in butterfly order
      const float m_w = xor_max_from<LPK>(m_g);
      const float f = (m_g == -INFINITY) ? 0.f : exp2_hw(m_g - m_w);
      const float l_w = xor_sum_from<LPK>(l_g * f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = xor_sum_from<LPK>(acc[e] * f);
      if (kg == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_acc[wave][dl * EPL + e] = acc[e];
      }
      if (lane == 0) {
        s_m[wave] = m_w;
        s_l[wave] = l_w;
      }
      __syncthreads();
      if (slot_ok) {  // the chunk's state: the sequence's waves in wave order
        const int w0 = packed ? slot * spw : 0;
        const int w1 = packed ? w0 + spw : kAttnWaves;
        float mc = s_m[w0];
        for (int w = w0 + 1; w < w1; ++w) mc = fmaxf(mc, s_m[w]);
        float lc = 0.f, ac = 0.f;
        for (int w = w0; w < w1; ++w) {
          const float fw = (s_m[w] == -INFINITY) ? 0.f : exp2_hw(s_m[w] - mc);
          lc = fmaf(fw, s_l[w], lc);
          ac = fmaf(fw, s_acc[w][d], ac);
        }
        if (whole) {
          fold_chunk<EX>(c == c0, mc, lc, ac, fm, fl, fa);
        } else {  // publish the chunk state, write-through
          float* pp = S.part + (slot_sidx * nck_cap + c) * PS;
          __hip_atomic_store(pp + 4 + d, ac, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (d == 0) {
            __hip_atomic_store(pp, mc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pp + 1, lc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      __syncthreads();  // LDS is rewritten by the next chunk
    }
    if (whole) {
      if (slot_ok) store_out<EX>(S, slot_sidx * HD + d, fa, fl);
      continue;
    }
    // split mode (one chunk per item): every thread's stores have completed before
    // the ticket is taken; the last chunk to arrive folds them all in chunk order
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const int prev =
          __hip_atomic_fetch_add(S.ticket + slot_sidx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == nck - 1;
    }
    __syncthreads();
    if (s_last) {
      if (slot_ok) {
        // the states of up to 8 chunks are in flight at once (a load past the last chunk
        // re-reads it and is not folded), then folded in chunk order
        constexpr int kFoldBatch = 8;
        const float* pp = S.part + slot_sidx * nck_cap * PS;
        for (int cf = 0; cf < nck; cf += kFoldBatch) {
          float mc[kFoldBatch], lc[kFoldBatch], ac[kFoldBatch];
#pragma unroll
          for (int j = 0; j < kFoldBatch; ++j) {
            const float* q = pp + min(cf + j, nck - 1) * PS;
            mc[j] = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            lc[j] = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ac[j] = __hip_atomic_load(q + 4 + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
#pragma unroll
          for (int j = 0; j < kFoldBatch; ++j)
            if (cf + j < nck) fold_chunk<EX>(cf + j == 0, mc[j], lc[j], ac[j], fm, fl, fa);
        }
        store_out<EX>(S, slot_sidx * HD + d, fa, fl);
      }
      if (tid == 0)
        __hip_atomic_store(S.ticket + slot_sidx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // s_last is rewritten by the next item
  }
}

long long attn_items_cap(const AttnParams& p) {
  long long total = 0;
  for (int s = 0; s < p.nseg; ++s) {
    const long long nck = p.seg[s].nck_cap;
    const long long ipl = nck > p.cpi ? (nck + p.cpi - 1) / p.cpi : 1;
    total += (long long)p.NL * p.B * p.H * ipl;
  }
  return total;
}

namespace {
// Per-device launch facts, filled on a thread's first launch on the device: each thread
// keeps its own copy, so no state is shared between threads.  0 = not yet queried.
struct Occupancy {
  size_t lds;  // the dynamic LDS bytes it was queried for
  int wgs;     // resident workgroups per CU
};
struct DevInfo {
  int cus = 0;
  Occupancy occ[2][2][5] = {};  // [dtype][head dim 64/128][variant]
};
constexpr int kDevInfoSlots = 64;
thread_local DevInfo t_dev[kDevInfoSlots];

// variant: 0 static, 1 paged, 2 widened (key masks / bf16 outputs, static caches), 3 static
// with the current token's rows appended, 4 widened with a paged self cache
template <typename T, int HD>
void* attn_kernel_ptr(int variant) {
  return variant == 4   ? reinterpret_cast<void*>(&attn_decode_kernel<T, true, true, HD>)
         : variant == 3 ? reinterpret_cast<void*>(&attn_decode_kernel<T, false, false, HD, true>)
         : variant == 2 ? reinterpret_cast<void*>(&attn_decode_kernel<T, false, true, HD>)
         : variant == 1 ? reinterpret_cast<void*>(&attn_decode_kernel<T, true, false, HD>)
                        : reinterpret_cast<void*>(&attn_decode_kernel<T, false, false, HD>);
}

template <typename T, int HD>
void attn_kernel_go(int variant, int blocks, size_t lds, hipStream_t stream, const AttnParams& p) {
  if (variant == 4)
    hipLaunchKernelGGL((attn_decode_kernel<T, true, true, HD>), dim3(blocks), dim3(kAttnThreads),
                       lds, stream, p);
  else if (variant == 3)
    hipLaunchKernelGGL((attn_decode_kernel<T, false, false, HD, true>), dim3(blocks),
                       dim3(kAttnThreads), lds, stream, p);
  else if (variant == 2)
    hipLaunchKernelGGL((attn_decode_kernel<T, false, true, HD>), dim3(blocks), dim3(kAttnThreads),
                       lds, stream, p);
  else if (variant == 1)
    hipLaunchKernelGGL((attn_decode_kernel<T, true, false, HD>), dim3(blocks), dim3(kAttnThreads),
                       lds, stream, p);
  else
    hipLaunchKernelGGL((attn_decode_kernel<T, false, false, HD>), dim3(blocks), dim3(kAttnThreads),
                       lds, stream, p);
}
}  // namespace

// Work items of a launch at chunk 1 << clog, every sequence at full capacity.
static long long items_at(const AttnParams& p, int clog) {
  AttnParams q = p;
  for (int s = 0; s < q.nseg; ++s) q.seg[s].nck_cap = ((q.seg[s].L_cap - 1) >> clog) + 1;
  return attn_items_cap(q);
}

hipError_t attn_launch(const AttnParams& p_in, int dtype, int blocks, hipStream_t stream) {
  AttnParams p = p_in;
  const int G = p.nseg * p.B;
  const bool paged = p.seg[0].table != nullptr || (p.nseg > 1 && p.seg[1].table != nullptr);
  const bool ex = p.seg[0].mask != nullptr || p.seg[0].out_bf16 ||
                  (p.nseg > 1 && (p.seg[1].mask != nullptr || p.seg[1].out_bf16));
  const bool app = p.seg[0].k_new != nullptr;  // static, plain: the ABI allows no other
  const int variant = ex ? (paged ? 4 : 2) : paged ? 1 : app ? 3 : 0;
  // first-tile records: bf16 static caches without key masks, the in-register list, and
  // kAttnRecLdsPerWave bytes of LDS per wave
  if (G > kWave || paged || ex || dtype != 0) p.rec = nullptr;
  const size_t lds = (size_t)(3 * G + 1) * sizeof(int) +
                     (p.rec != nullptr ? (size_t)kAttnWaves * kAttnRecLdsPerWave : 0);
  const int wide = p.hd == kAttnHeadDimWide ? 1 : 0;
  if (!wide && p.hd != kAttnHeadDim) return hipErrorInvalidValue;
  void* fn = dtype == 0 ? (wide ? attn_kernel_ptr<uint16_t, kAttnHeadDimWide>(variant)
                                : attn_kernel_ptr<uint16_t, kAttnHeadDim>(variant))
                        : (wide ? attn_kernel_ptr<float, kAttnHeadDimWide>(variant)
                                : attn_kernel_ptr<float, kAttnHeadDim>(variant));
  const bool choose_chunk = p.chunk_log2 == 0;
  int dev = 0, cus = 0;
  {
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kDevInfoSlots;
    cus = cached ? t_dev[dev].cus : 0;
    if (cus == 0) {
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      if (cached) t_dev[dev].cus = cus;
    }
  }
  if (choose_chunk) {
    // 1024-key chunks; a split launch with fewer items than a quarter of the CUs halves
    // them (down to the smallest chunk the workspace holds partials for), so more CUs
    // share its bytes.  Measured on 16 sequences of 1024 keys: 64 items of 256 keys beat
    // 128 of 128 (each item pays a prologue and a fold) and 16 or 32 larger ones.
    p.chunk_log2 = attn_log2(kAttnChunk);
    if (p.cpi == 1)
      while (p.chunk_log2 > p.min_chunk_log2 && items_at(p, p.chunk_log2) * 4 < cus)
        --p.chunk_log2;
  }
  for (int s = 0; s < 2; ++s)
    p.seg[s].nck_cap = p.seg[s].L_cap > 0 ? ((p.seg[s].L_cap - 1) >> p.chunk_log2) + 1 : 0;
  if (p.cpi < 1 || (p.cpi & (p.cpi - 1)) != 0) return hipErrorInvalidValue;
  p.cpi_log2 = attn_log2(p.cpi);
  p.div_nlh = div_magic((uint32_t)(p.NL * p.H));
  p.div_h = div_magic((uint32_t)p.H);
  p.cus = cus;
  // halves need the chunk states at half the launch's chunk and the in-register list
  if (p.cpi == 1 || p.min_chunk_log2 >= p.chunk_log2 || G > kWave) p.balance = 0;
  if (blocks <= 0) {
    hipError_t e = hipSuccess;
    Occupancy* slot = dev >= 0 && dev < kDevInfoSlots ? &t_dev[dev].occ[dtype][wide][variant]
                                                      : nullptr;
    int occ = slot != nullptr && slot->lds == lds ? slot->wgs : 0;
    if (occ == 0) {
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kAttnThreads, lds);
      if (e != hipSuccess) return e;
      if (occ < 1) occ = 1;
      if (slot != nullptr) *slot = Occupancy{lds, occ};
    }
    const long long cap = attn_items_cap(p);
    const long long want = (long long)cus * occ;
    blocks = (int)(want < cap ? want : cap);
  }
  if (blocks < 1) blocks = 1;
  if (dtype == 0) {
    if (wide) attn_kernel_go<uint16_t, kAttnHeadDimWide>(variant, blocks, lds, stream, p);
    else attn_kernel_go<uint16_t, kAttnHeadDim>(variant, blocks, lds, stream, p);
  } else {
    if (wide) attn_kernel_go<float, kAttnHeadDimWide>(variant, blocks, lds, stream, p);
    else attn_kernel_go<float, kAttnHeadDim>(variant, blocks, lds, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dec
