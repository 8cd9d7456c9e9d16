// Fused temperature / top-k / softmax / inverse-CDF sampling with the codebook
// delay mask, one wavefront per (sequence, codebook) row (gfx950).
//
// "Optimized Parler TTS", "Future work", item 2: sampling was more than ten
// kernels (temperature, top-k, softmax) with global-memory round trips between
// them.  Here one kernel reads each row of logits once and writes the token.
// "Analysis and improvements": logits exist for the last position only (one
// row per codebook) and the vocabulary is padded to a multiple of 8 -- the
// padding columns are never read.  Random numbers arrive as per-row uniforms,
// so nothing waits on the host.  "A rough architecture of Parler TTS": 9
// codebooks per step under a delay pattern; codebook c emits the fill token
// until the sequence has taken c steps.
//
// Per row (64 lanes):
//   1. Each lane loads entries lane, lane + 64, lane + 128, ... (every load
//      instruction is one coalesced 256-byte row segment; all are in flight at
//      once).  Vocabulary order is (slot, lane) order.  Values map to
//      order-preserving uint32 keys.
//   2. Prune: the kk-th largest of the 64 per-lane maxima is a lower bound L0
//      on the kk-th largest key (at least kk keys reach it), so keys below L0
//      are never kept.  The survivors (typically under a tenth of the row) are
//      compacted through LDS, still in vocabulary order, to at most kSurvSlots
//      per lane; if more survive, the full row is searched instead.
//   3. Exact threshold: a radix search for the kk-th largest key, 8 bits per
//      pass (a 256-bucket LDS histogram of the keys that still match the
//      resolved prefix, a wave scan and a ballot), stopping once exactly kk keys
//      reach the prefix.  Keys above it are kept, plus the lowest-index keys
//      equal to it; ranks in vocabulary order come from ballots and mbcnt, and
//      the kept entries are compacted through LDS so lane t holds the t-th kept
//      entry in ascending vocabulary order (kk <= 64).
//   4. e_t = exp((x_t - max) / T) and their sum in float64; p_t = e_t / sum,
//      rounded once to float32 (the exported probability); the CDF is the
//      float64 running sum of those p_t, and the token is the first kept entry
//      with u < C_t (the last one if rounding leaves u >= C_last).  T <= 0:
//      greedy.
//
// Wide variant (top_k > 64): the lane maxima bound only the 64th largest key,
// so up to top_k 256 a wider bound prunes the row (the WIDE branch below); the
// radix search then runs over the compacted survivors, or over the whole row.
// The kept entries stay where they were loaded: slot j of every lane holds
// entries 64 j .. 64 j + 63 (of the row or of its survivors, in vocabulary
// order), so the CDF in vocabulary order is one wave scan per slot plus the
// running total of the slots before it.  Logits may be bf16: each value widens
// exactly to fp32 before its key is formed.
#include "dec_common.h"
#include "dec_kernels.h"

namespace dec {

// Entry slots per lane that every row given to the VPL-slot instantiation fills on every lane:
// sample_launch picks the smallest VPL in {4, 8, 16, 18, 32, 64} that covers the row, so the
// row is longer than the next smaller size's slots.
constexpr int samp_full_slots(int vpl) {
  return vpl == 8 ? 4 : vpl == 16 ? 8 : vpl == 18 ? 16 : vpl == 32 ? 18 : vpl == 64 ? 32 : 0;
}

constexpr int kSurvSlots = 3;                   // survivor slots per lane after pruning
constexpr int kSurvCap = kSurvSlots * kWave;     // survivors that fit
// Wide variant: top_k up to kWidePruneK is pruned to at most kWideSlots per lane (the
// bound below, for t = ceil(top_k / 64) and t + 1, so each lane keeps its kWideMaxT
// largest keys).
constexpr int kWidePruneK = 4 * kWave;
constexpr int kWideMaxT = 5;
constexpr int kWideSlots = 8;
constexpr int kWideSurvCap = kWideSlots * kWave;

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(mask), 0u));
}

// Inverse of order_key (-0 comes back as +0; NaN payloads survive).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

// Largest key in the wave: DPP within 16-lane rows, then the four row results.
__device__ __forceinline__ uint32_t wave_max_key(uint32_t v) {
  auto step = [](uint32_t x, int y) { const uint32_t u = static_cast<uint32_t>(y); return x > u ? x : u; };
  v = step(v, __builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor1, 0xF, 0xF, false));
  v = step(v, __builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor2, 0xF, 0xF, false));
  v = step(v, __builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xF, 0xF, false));
  v = step(v, __builtin_amdgcn_update_dpp(0, (int)v, kDppRowMirror, 0xF, 0xF, false));
  const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
  const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// Count of keys >= t over NS slots, across the wave.
template <int NS>
__device__ __forceinline__ int count_ge(const uint32_t (&key)[NS], uint32_t t) {
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) cnt += __popcll(__ballot(key[j] >= t));
  return cnt;
}

// Search step over two bits below `bit` + 1 of tau: the three candidates are
// counted independently, so a step costs one dependency chain for two bits.
// Keeps the invariant #(key >= tau) >= kk; returns true once exactly kk keys are >= tau.
template <int NS>
__device__ __forceinline__ bool search2(const uint32_t (&key)[NS], int kk, int lowbit, uint32_t& tau) {
  const uint32_t c1 = tau | (1u << lowbit), c2 = tau | (2u << lowbit), c3 = tau | (3u << lowbit);
  const int n1 = count_ge(key, c1), n2 = count_ge(key, c2), n3 = count_ge(key, c3);
  if (n3 >= kk) { tau = c3; return n3 == kk; }
  if (n2 >= kk) { tau = c2; return n2 == kk; }
  if (n1 >= kk) { tau = c1; return n1 == kk; }
  return false;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Per wave: 256 histogram buckets, then one private word per lane that absorbs the
// counts of keys outside the current prefix, so no atomic is predicated (a branch
// around each one costs more than the add).
constexpr int kHistWords = 256 + kWave;

// Radix search for tau over NS slots per lane (absent slots: idx -1).  Every present
// key lies in [lo, hi], so the bits above the highest bit where lo and hi differ are
// shared and known.  Each pass resolves the next 8 bits: the keys that still match
// the resolved prefix are counted into 256 LDS buckets (stored in descending bucket
// order, so lane l holds buckets 255-4l..252-4l in one 16-byte read), a wave scan
// turns the counts into "keys at or above this bucket", and a ballot picks the bucket
// that holds the kk-th largest key.  Returns tau such that either exactly
// kk keys are >= tau (an exact cut was found), or tau is the kk-th largest key; both
// give the same kept set under the tie rule of select_kept.  hist: kHistWords words.
template <int NS>
__device__ __forceinline__ uint32_t radix_tau(const uint32_t (&key)[NS], const int (&idx)[NS],
                                              int kk, uint32_t lo, uint32_t hi, uint32_t* hist) {
  const uint32_t diff = lo ^ hi;
  if (diff == 0u) return hi;
  const int lane = static_cast<int>(__lane_id());
  int top = 31 - __builtin_clz(diff);                          // highest unresolved bit
  uint32_t prefix = top == 31 ? 0u : (hi & ~((2u << top) - 1u));
  int above = 0;                                               // keys above the prefix range
  u32x4_t* h4 = reinterpret_cast<u32x4_t*>(hist);
  uint32_t* const dummy = hist + 256 + lane;
  for (;;) {
    const int sh = top >= 7 ? top - 7 : 0;
    const uint32_t high = top == 31 ? 0u : ~((2u << top) - 1u);  // resolved bits
    h4[lane] = u32x4_t{0u, 0u, 0u, 0u};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const bool in = idx[j] >= 0 && (key[j] & high) == prefix;
      atomicAdd(in ? &hist[255 - ((key[j] >> sh) & 0xFFu)] : dummy, 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4_t c4 = h4[lane];
    const int a0 = (int)c4.x, a1 = a0 + (int)c4.y, a2 = a1 + (int)c4.z, a3 = a2 + (int)c4.w;
    const int base = wave_exclusive_sum_int(a3, lane);
    const int need = kk - above;
    const unsigned long long reach = __ballot(base + a3 >= need);
    const int L = __ffsll((long long)reach) - 1;   // a lane reaches need: candidates >= need
    const int bL = __builtin_amdgcn_readlane(base, L);
    const int r0 = bL + __builtin_amdgcn_readlane(a0, L);
    const int r1 = bL + __builtin_amdgcn_readlane(a1, L);
    const int r2 = bL + __builtin_amdgcn_readlane(a2, L);
    const int r3 = bL + __builtin_amdgcn_readlane(a3, L);
    const int i = r0 >= need ? 0 : r1 >= need ? 1 : r2 >= need ? 2 : 3;
    const int cum_at = i == 0 ? r0 : i == 1 ? r1 : i == 2 ? r2 : r3;
    const int cum_before = i == 0 ? bL : i == 1 ? r0 : i == 2 ? r1 : r2;
    // bits above `top` inside the 8-bit digit (only when sh == 0) equal the prefix's
    prefix |= (uint32_t)(255 - (4 * L + i)) << sh;
    if (cum_at == need) return prefix;  // exactly kk keys are >= prefix
    above += cum_before;
    if (sh == 0) return prefix;         // every bit resolved: the kk-th largest key
    top = sh - 1;
  }
}

// Exact top-kk over NS slots per lane whose slot-major order is vocabulary order.
// Absent slots carry key 0 and idx -1.  Every present key is at least `lo`, and
// the largest is `hi`.  Writes the kept (value, index) pairs in vocabulary order to
// cval/cidx[0..kk) (lanes outside the kept set write a dummy slot, so no store is
// predicated).  hist: kHistWords words of this wave's LDS, 16-byte aligned.
template <int NS>
__device__ __forceinline__ void select_kept(const uint32_t (&key)[NS], const int (&idx)[NS], int kk,
                                            uint32_t lo, uint32_t hi, float* cval, int* cidx,
                                            uint32_t* hist) {
  const uint32_t tau = radix_tau(key, idx, kk, lo, hi, hist);
  int cnt_gt = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) cnt_gt += __popcll(__ballot(key[j] > tau));
  const int need = kk - cnt_gt;  // entries equal to tau to keep, lowest index first
  int eq_before = 0, kept_before = 0;
  const int lane = static_cast<int>(__lane_id());
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const bool eq = idx[j] >= 0 && key[j] == tau;
    const unsigned long long eqm = __ballot(eq);
    const bool kept = key[j] > tau || (eq && eq_before + lanes_below(eqm) < need);
    const unsigned long long km = __ballot(kept);
    const int pos = kept ? kept_before + lanes_below(km) : kWave + lane;
    cval[pos] = key_value(key[j]);
    cidx[pos] = idx[j];
    eq_before += __popcll(eqm);
    kept_before += __popcll(km);
  }
}

// Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC 2011); returns output word 0 for counter c and key k.
__device__ __forceinline__ uint64_t philox4x64_10_w0(uint64_t c0, uint64_t c1, uint64_t c2,
                                                     uint64_t c3, uint64_t k0, uint64_t k1) {
  constexpr uint64_t kMulA = 0xD2E7470EE14C6C93ull, kMulB = 0xCA5A826395121157ull;
  constexpr uint64_t kWeylA = 0x9E3779B97F4A7C15ull, kWeylB = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t ha = __umul64hi(kMulA, c0), la = kMulA * c0;
    const uint64_t hb = __umul64hi(kMulB, c2), lb = kMulB * c2;
    const uint64_t n0 = hb ^ c1 ^ k0, n2 = ha ^ c3 ^ k1;
    c0 = n0;
    c1 = lb;
    c2 = n2;
    c3 = la;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  return c0;
}

// The uniform of row (b, c) at step st: counter (st, b, c, 0), key (seed, 0), the top 24
// bits of word 0 scaled by 2^-24 (exact in float32, in [0, 1)).
__device__ __forceinline__ float philox_uniform(int st, int b, int c, uint64_t seed) {
  const uint64_t w = philox4x64_10_w0((uint64_t)(int64_t)st, (uint64_t)b, (uint64_t)c, 0ull, seed,
                                      0ull);
  return (float)(uint32_t)(w >> 40) * 0x1p-24f;
}

__device__ __forceinline__ float logit_at(const float* x, int i) { return x[i]; }
__device__ __forceinline__ float logit_at(const uint16_t* x, int i) {
  return __uint_as_float(static_cast<uint32_t>(x[i]) << 16);
}

// Wide variant, steps 3 and 4 over the loaded slots (see the file comment).  The
// kept set is {key > tau} plus the lowest-index entries equal to tau; its t-th
// entry in vocabulary order goes to output position t.
template <int VPL>
__device__ __forceinline__ void sample_wide(const SampleParams& p, int row, const uint32_t (&key)[VPL],
                                            const int (&idx)[VPL], int kk, uint32_t lo,
                                            uint32_t kmax, float T, float u, int started,
                                            uint32_t* hist) {
  const int lane = static_cast<int>(__lane_id());
  const uint32_t tau = radix_tau(key, idx, kk, lo, kmax, hist);
  int cnt_gt = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) cnt_gt += __popcll(__ballot(key[j] > tau));
  const int need = kk - cnt_gt;  // entries equal to tau to keep, lowest index first
  const float m = key_value(kmax);
  const bool greedy = T <= 0.f;
  // weights e = exp((x - m) / T) in float64, each rounded once to float32 and held; their
  // sum Z in float64 (per lane in slot order, then across the wave); p = e / Z rounded
  // once to float32 (the exported value).  The CDF the uniform is compared with is the
  // float64 running sum of the exported probabilities in vocabulary order (one wave scan
  // per slot plus the total of the slots before it).  Each p is within 3 x 2^-24 of the
  // exact probability, so the CDF is within 3 x 2^-24 of the exact one.
  const double md = (double)m, Td = (double)T;
  double e[VPL];
  int pos[VPL];
  int eq_before = 0, kept_before = 0;
  double zl = 0.0;  // this lane's share of Z
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const bool eq = idx[j] >= 0 && key[j] == tau;
    const unsigned long long eqm = __ballot(eq);
    const bool kept = key[j] > tau || (eq && eq_before + lanes_below(eqm) < need);
    const unsigned long long km = __ballot(kept);
    pos[j] = kept ? kept_before + lanes_below(km) : -1;
    e[j] = kept && !greedy ? exp(((double)key_value(key[j]) - md) / Td) : 0.0;
    zl += e[j];
    eq_before += __popcll(eqm);
    kept_before += __popcll(km);
  }
  const double Zd = readlane_f64(wave_inclusive_sum_f64(zl), kWave - 1);
  float pr[VPL];
  int token = -1;  // the sampled index, before the delay mask
  double run = 0.0;  // sum of the probabilities over the slots before j
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    pr[j] = (float)(e[j] / Zd);
    const double C = run + wave_inclusive_sum_f64((double)pr[j]);
    run = readlane_f64(C, kWave - 1);
    // slots hold entries in vocabulary order (the whole row, or its compacted survivors):
    // the first slot with a hit wins, and the token is that entry's index (greedy: the
    // lowest index holding the largest key)
    const unsigned long long hit = greedy ? __ballot(idx[j] >= 0 && key[j] == kmax)
                                          : __ballot(pos[j] >= 0 && (double)u < C);
    if (token < 0 && hit) token = __builtin_amdgcn_readlane(idx[j], __ffsll(hit) - 1);
  }
  if (token < 0) {  // rounding left u >= C_last: the last kept entry
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const unsigned long long mk = __ballot(pos[j] == kk - 1);
      if (mk) token = __builtin_amdgcn_readlane(idx[j], __ffsll(mk) - 1);
    }
  }
  if (lane == 0) p.tokens[row] = started ? token : p.fill;
  int32_t* oi = p.topk_idx != nullptr ? p.topk_idx + (size_t)row * p.top_k : nullptr;
  float* op = p.topk_prob != nullptr ? p.topk_prob + (size_t)row * p.top_k : nullptr;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    if (pos[j] < 0) continue;
    if (oi != nullptr) oi[pos[j]] = idx[j];
    if (op != nullptr) op[pos[j]] = greedy ? (idx[j] == token ? 1.f : 0.f) : pr[j];
  }
  for (int t = kk + lane; t < p.top_k; t += kWave) {
    if (oi != nullptr) oi[t] = -1;
    if (op != nullptr) op[t] = 0.f;
  }
}

template <int VPL, typename LT, bool WIDE>
__global__ __launch_bounds__(kSampWaves * kWave) void sample_topk_kernel(SampleParams p) {
  // per wave: kept entries [0, 64) plus one dummy slot per lane; survivors
  // [0, kSurvCap) plus one dummy slot per lane
  __shared__ float s_val[kSampWaves][2 * kWave];
  __shared__ int s_idx[kSampWaves][2 * kWave];
  __shared__ uint2 s_surv[kSampWaves][(WIDE ? kWideSurvCap : kSurvCap) + kWave];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kSampWaves][kHistWords];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
  const int rows = p.B * p.n_cb;
  const int row = blockIdx.x * kSampWaves + wave;
  if (row >= rows) return;  // uniform per wave; waves never wait on each other
  const int kk = p.top_k < p.V_valid ? p.top_k : p.V_valid;

  // per-row scalars first, so their latency overlaps the logits' and the selection
  const int b = row / p.n_cb;
  const int c = row - b * p.n_cb;
  const float T = p.temperature[b];
  const int st = p.step != nullptr ? p.step[p.step_inc != nullptr ? row : b] : 0;
  if (p.step_inc != nullptr && lane == 0) {  // every counter is read by its own row only
    p.step_inc[row] = st + 1;
    if (c == 0 && p.len_inc != nullptr) p.len_inc[b] += 1;  // nothing here reads len
  }
  const int started = p.step != nullptr ? (st >= c) : 1;
  const float u = p.rng ? philox_uniform(st, b, c, p.seed) : p.uniforms[row];

  // Slots below samp_full_slots(VPL) hold valid entries on every lane (the launcher picks VPL
  // only for rows longer than that many slots), so they load at fixed offsets from one base,
  // with no clamp and no mask; the others clamp their index, so every load stays in the row.
  constexpr int kFull = samp_full_slots(VPL);
  const LT* x = static_cast<const LT*>(p.logits) + (size_t)row * p.V_stride;
  float v[VPL];
  uint32_t key[VPL];
  int idx[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {  // no branches
    const int i = j * kWave + lane;
    v[j] = logit_at(x, j < kFull || i < p.V_valid ? i : p.V_valid - 1);
  }
  uint32_t lmax = 0u;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int i = j * kWave + lane;
    const bool ok = j < kFull || i < p.V_valid;
    key[j] = order_key(v[j]) & (ok ? 0xFFFFFFFFu : 0u);  // absent: below every candidate
    idx[j] = ok ? i : -1;
    lmax = key[j] > lmax ? key[j] : lmax;
  }
  const uint32_t kmax = wave_max_key(lmax);
  if constexpr (WIDE) {
    if constexpr (VPL > kWideSlots) {
      // Pruning: for any t with c = ceil(kk / t) <= 64, each lane holds t keys at least as
      // large as its t-th largest a_l, so at least t * c >= kk keys reach the c-th largest
      // a_l: that bounds the kk-th largest key from below, and so does the larger of the
      // bounds for t = ceil(kk / 64) and t + 1 (the second is often the tighter: at the
      // first, c is often 64, the smallest a_l).  Every entry the kept set can hold, ties
      // included, survives.
      const int t0 = (kk + kWave - 1) / kWave;
      if (kk <= kWidePruneK) {
        uint32_t top[kWideMaxT];  // this lane's largest keys, descending
#pragma unroll
        for (int i = 0; i < kWideMaxT; ++i) top[i] = 0u;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          uint32_t x = key[j];
#pragma unroll
          for (int i = 0; i < kWideMaxT; ++i) {
            const uint32_t hi = top[i] > x ? top[i] : x;
            x = top[i] > x ? x : top[i];
            top[i] = hi;
          }
        }
        // a_l for t0 and t0 + 1 (t0 is 2, 3 or 4 here); both searches run interleaved, to
        // 18 leading bits (independent chains)
        const uint32_t lm1[1] = {t0 == 2 ? top[1] : (t0 == 3 ? top[2] : top[3])};
        const uint32_t lm2[1] = {t0 == 2 ? top[2] : (t0 == 3 ? top[3] : top[4])};
        const int c1 = (kk + t0 - 1) / t0, c2 = (kk + t0) / (t0 + 1);
        uint32_t b1 = 0u, b2 = 0u;
#pragma unroll
        for (int bit = 31; bit > 14; bit -= 2) {
          (void)search2(lm1, c1, bit - 1, b1);
          (void)search2(lm2, c2, bit - 1, b2);
        }
        const uint32_t l0 = b1 > b2 ? b1 : b2;
        const uint32_t thr = uniform(l0 > 1u ? l0 : 1u);  // absent entries (key 0) never survive
        uint2* surv = s_surv[wave];
        int nsurv = 0;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {  // survivors in vocabulary order, as in the narrow path
          const bool sv = key[j] >= thr;
          const unsigned long long m = __ballot(sv);
          const int pos = nsurv + lanes_below(m);
          const int dummy = kWideSurvCap + lane;
          surv[sv ? min(pos, dummy) : dummy] = make_uint2(key[j], (uint32_t)idx[j]);
          nsurv += __popcll(m);
        }
        if (nsurv <= kWideSurvCap) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          uint32_t sk[kWideSlots];
          int si[kWideSlots];
#pragma unroll
          for (int j = 0; j < kWideSlots; ++j) {
            const int q = j * kWave + lane;
            const uint2 e = surv[q < nsurv ? q : kWideSurvCap + lane];
            sk[j] = q < nsurv ? e.x : 0u;
            si[j] = q < nsurv ? (int)e.y : -1;
          }
          sample_wide(p, row, sk, si, kk, thr, kmax, T, u, started, s_hist[wave]);
          return;
        }
      }
    }
    sample_wide(p, row, key, idx, kk, 0u, kmax, T, u, started, s_hist[wave]);
    return;
  }
  // L0: the kk-th largest lane maximum, to its 10 leading bits (a lower bound on
  // the kk-th largest key either way: at least kk lanes hold a key >= L0)
  uint32_t l0 = 0u;
  {
    const uint32_t lm[1] = {lmax};
    for (int bit = 31; bit > 22; bit -= 2) (void)search2(lm, kk, bit - 1, l0);
  }
  // compact the survivors (key >= L0) in vocabulary order, as long as they fit;
  // absent entries have key 0, so a threshold of at least 1 leaves them out
  const uint32_t thr = uniform(l0 > 1u ? l0 : 1u);
  uint2* surv = s_surv[wave];
  int nsurv = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const bool sv = key[j] >= thr;
    const unsigned long long m = __ballot(sv);
    const int pos = nsurv + lanes_below(m);
    // past the capacity (the full-row search is taken then) or not a survivor:
    // a dummy slot, never read
    const int dummy = kSurvCap + lane;
    surv[sv ? min(pos, dummy) : dummy] = make_uint2(key[j], (uint32_t)idx[j]);
    nsurv += __popcll(m);
  }
  if (nsurv >= kk && nsurv <= kSurvCap) {  // (fewer than kk only if L0 found nothing)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t sk[kSurvSlots];
    int si[kSurvSlots];
#pragma unroll
    for (int j = 0; j < kSurvSlots; ++j) {
      const int q = j * kWave + lane;
      const uint2 e = surv[q < nsurv ? q : kSurvCap + lane];
      sk[j] = q < nsurv ? e.x : 0u;
      si[j] = q < nsurv ? (int)e.y : -1;
    }
    select_kept(sk, si, kk, thr, kmax, s_val[wave], s_idx[wave], s_hist[wave]);
  } else {  // too many survivors (heavy ties or a flat row): search the whole row
    select_kept(key, idx, kk, 0u, kmax, s_val[wave], s_idx[wave], s_hist[wave]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const bool act = lane < kk;
  const float xv = act ? s_val[wave][lane] : -INFINITY;
  const int xi = act ? s_idx[wave][lane] : -1;
  const float m = key_value(kmax);  // the row maximum is always kept
  int sel;
  float prob;
  if (T <= 0.f) {
    const unsigned long long mk = __ballot(act && xv == m);
    sel = mk ? __ffsll(mk) - 1 : 0;
    prob = lane == sel ? 1.f : 0.f;
  } else {
    // weights and their sum in fp64; each probability is rounded once to fp32 (the
    // exported value), and the CDF the uniform is compared with is the fp64 running sum
    // of those exported probabilities in vocabulary order, so it differs from the exact
    // one by at most 2^-24 (the roundings of the probabilities) at any k
    const double ed = act ? exp(((double)xv - (double)m) / (double)T) : 0.0;
    const double Zd = readlane_f64(wave_inclusive_sum_f64(ed), kk - 1);
    prob = act ? (float)(ed / Zd) : 0.f;
    const double C = wave_inclusive_sum_f64((double)prob);
    const unsigned long long mk = __ballot(act && (double)u < C);
    sel = mk ? __ffsll(mk) - 1 : kk - 1;
  }
  int token = __builtin_amdgcn_readlane(xi, sel);
  if (!started) token = p.fill;
  if (lane == 0) p.tokens[row] = token;
  if (lane < p.top_k) {
    if (p.topk_idx != nullptr) p.topk_idx[(size_t)row * p.top_k + lane] = act ? xi : -1;
    if (p.topk_prob != nullptr) p.topk_prob[(size_t)row * p.top_k + lane] = act ? prob : 0.f;
  }
}

template <int VPL>
static hipError_t sample_launch_vpl(const SampleParams& p, hipStream_t stream) {
  // the kernel reads slots below samp_full_slots(VPL) without a bound: the row must be longer
  if (p.V_valid <= samp_full_slots(VPL) * kWave || p.V_valid > VPL * kWave) return hipErrorInvalidValue;
  const int rows = p.B * p.n_cb;
  const dim3 grid((rows + kSampWaves - 1) / kSampWaves), block(kSampWaves * kWave);
  const bool wide = p.top_k > kSampNarrowK;
  if (p.logits_bf16) {
    if (wide) hipLaunchKernelGGL((sample_topk_kernel<VPL, uint16_t, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((sample_topk_kernel<VPL, uint16_t, false>), grid, block, 0, stream, p);
  } else {
    if (wide) hipLaunchKernelGGL((sample_topk_kernel<VPL, float, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((sample_topk_kernel<VPL, float, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t sample_launch(const SampleParams& p, hipStream_t stream) {
  const int need = (p.V_valid + kWave - 1) / kWave;  // entries per lane
  if (need <= 4) return sample_launch_vpl<4>(p, stream);
  if (need <= 8) return sample_launch_vpl<8>(p, stream);
  if (need <= 16) return sample_launch_vpl<16>(p, stream);
  if (need <= 18) return sample_launch_vpl<18>(p, stream);
  if (need <= 32) return sample_launch_vpl<32>(p, stream);
  return sample_launch_vpl<64>(p, stream);
}

// ---- utilities ------------------------------------------------------------------------

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t fill_zero_launch(void* ptr, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ptr), n);
  return hipGetLastError();
}

__global__ void advance_kernel(int32_t* len, int32_t* step, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    if (len != nullptr) len[b] += 1;
    if (step != nullptr) step[b] += 1;
  }
}

__global__ void append_kernel(AppendParams p) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const long long rows = (long long)p.NL * p.B * p.H;
  const long long n = rows * p.row16;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const long long row = i / p.row16;
    const int piece = (int)(i - row * p.row16);
    const int b = (int)((row / p.H) % p.B);
    const int len = p.len[b];
    if (len < 1 || len > p.L_cap) continue;  // nothing to write for this sequence
    const u32x4_t* kn = static_cast<const u32x4_t*>(p.k_new) + row * p.row16 + piece;
    const u32x4_t* vn = static_cast<const u32x4_t*>(p.v_new) + row * p.row16 + piece;
    const long long dst = (row * p.L_cap + (len - 1)) * p.row16 + piece;
    static_cast<u32x4_t*>(p.k_cache)[dst] = *kn;
    static_cast<u32x4_t*>(p.v_cache)[dst] = *vn;
  }
}

hipError_t append_launch(const AppendParams& p, hipStream_t stream) {
  const long long n = (long long)p.NL * p.B * p.H * p.row16;
  if (n == 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

__global__ void uniforms_kernel(uint64_t seed, int step0, int B, int n_cb, int total, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int rows = B * n_cb;
  const int s = i / rows;
  const int row = i - s * rows;
  const int b = row / n_cb;
  out[i] = philox_uniform(step0 + s, b, row - b * n_cb, seed);
}

hipError_t uniforms_launch(uint64_t seed, int step0, int B, int n_cb, int total, float* out,
                           hipStream_t stream) {
  hipLaunchKernelGGL(uniforms_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     seed, step0, B, n_cb, total, out);
  return hipGetLastError();
}

hipError_t advance_launch(int32_t* len, int32_t* step, int B, hipStream_t stream) {
  hipLaunchKernelGGL(advance_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, len, step, B);
  return hipGetLastError();
}

}  // namespace dec
