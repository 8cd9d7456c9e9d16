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
//   3. Exact threshold: MSB-first bisection for the kk-th largest key; each step
//      counts keys >= candidate with wave ballots and stops once exactly kk
//      remain.  Keys above it are kept, plus the lowest-index keys equal to it;
//      ranks in vocabulary order come from ballots and mbcnt, and the kept
//      entries are compacted through LDS so lane t holds the t-th kept entry in
//      ascending vocabulary order (kk <= 64).
//   4. e_t = exp((x_t - max) / T); wave inclusive scan; C_t = S_t / S_last;
//      the token is the first kept entry with u < C_t.  T <= 0: greedy.
#include "dec_common.h"
#include "dec_kernels.h"

namespace dec {

constexpr int kSurvSlots = 3;  // survivor slots per lane after pruning

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(mask), 0u));
}

// Exact top-kk over NS slots per lane, slot-major order = vocabulary order.
// Absent slots carry key 0 and ok = false.  Writes the kept (value, index)
// pairs, in order, to cval/cidx[0..kk).
template <int NS>
__device__ __forceinline__ void select_kept(const uint32_t (&key)[NS], const float (&val)[NS],
                                            const int (&idx)[NS], int kk, float* cval,
                                            int* cidx) {
  // the largest t with #(key >= t) >= kk, i.e. the kk-th largest key; stop early
  // once exactly kk keys are >= t
  uint32_t tau = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) cnt += __popcll(__ballot(key[j] >= cand));
    if (cnt >= kk) {
      tau = cand;
      if (cnt == kk) break;
    }
  }
  int cnt_gt = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) cnt_gt += __popcll(__ballot(key[j] > tau));
  const int need = kk - cnt_gt;  // entries equal to tau to keep, lowest index first
  int eq_before = 0, kept_before = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const bool eq = idx[j] >= 0 && key[j] == tau;
    const unsigned long long eqm = __ballot(eq);
    const bool kept = key[j] > tau || (eq && eq_before + lanes_below(eqm) < need);
    const unsigned long long km = __ballot(kept);
    if (kept) {
      const int pos = kept_before + lanes_below(km);
      cval[pos] = val[j];
      cidx[pos] = idx[j];
    }
    eq_before += __popcll(eqm);
    kept_before += __popcll(km);
  }
}

template <int VPL>
__global__ __launch_bounds__(kSampWaves * kWave) void sample_topk_kernel(SampleParams p) {
  __shared__ float s_val[kSampWaves][kWave];
  __shared__ int s_idx[kSampWaves][kWave];
  __shared__ uint32_t s_skey[kSampWaves][kSurvSlots * kWave];
  __shared__ float s_sval[kSampWaves][kSurvSlots * kWave];
  __shared__ int s_sidx[kSampWaves][kSurvSlots * kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int rows = p.B * p.n_cb;
  const int row = blockIdx.x * kSampWaves + wave;
  const bool active = row < rows;  // uniform per wave; inactive waves still reach the barrier
  const int kk = p.top_k < p.V_valid ? p.top_k : p.V_valid;

  // per-row scalars first, so their latency overlaps the logits' and the selection
  const int b = active ? row / p.n_cb : 0;
  const int c = active ? row - b * p.n_cb : 0;
  const float T = active ? p.temperature[b] : 1.f;
  const float u = active ? p.uniforms[row] : 0.f;
  const int started = (active && p.step != nullptr) ? (p.step[b] >= c) : 1;

  if (active) {
    const float* x = p.logits + (size_t)row * p.V_stride;
    float v[VPL];
    uint32_t key[VPL];
    int idx[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {  // clamped index: every load is in bounds, no branches
      const int i = j * kWave + lane;
      v[j] = x[i < p.V_valid ? i : p.V_valid - 1];
    }
    uint32_t lmax = 0u;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int i = j * kWave + lane;
      const bool ok = i < p.V_valid;
      key[j] = ok ? order_key(v[j]) : 0u;  // absent entries: below every candidate
      idx[j] = ok ? i : -1;
      lmax = key[j] > lmax ? key[j] : lmax;
    }
    // L0: the kk-th largest lane maximum, to its 10 leading bits (a lower bound either way)
    uint32_t l0 = 0u;
    for (int bit = 31; bit >= 22; --bit) {
      const uint32_t cand = l0 | (1u << bit);
      if (__popcll(__ballot(lmax >= cand)) >= kk) l0 = cand;
    }
    // compact the survivors in vocabulary order (as long as they fit)
    int nsurv = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const bool sv = idx[j] >= 0 && key[j] >= l0;
      const unsigned long long m = __ballot(sv);
      const int pos = nsurv + lanes_below(m);
      if (sv && pos < kSurvSlots * kWave) {
        s_skey[wave][pos] = key[j];
        s_sval[wave][pos] = v[j];
        s_sidx[wave][pos] = idx[j];
      }
      nsurv += __popcll(m);
    }
    if (nsurv <= kSurvSlots * kWave) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      uint32_t sk[kSurvSlots];
      float sv[kSurvSlots];
      int si[kSurvSlots];
#pragma unroll
      for (int j = 0; j < kSurvSlots; ++j) {
        const int q = j * kWave + lane;
        const bool ok = q < nsurv;
        sk[j] = ok ? s_skey[wave][q] : 0u;
        sv[j] = ok ? s_sval[wave][q] : 0.f;
        si[j] = ok ? s_sidx[wave][q] : -1;
      }
      select_kept(sk, sv, si, kk, s_val[wave], s_idx[wave]);
    } else {  // too many survivors (heavy ties or a flat row): search the whole row
      select_kept(key, v, idx, kk, s_val[wave], s_idx[wave]);
    }
  }
  __syncthreads();

  if (active) {
    const bool act = lane < kk;
    const float xv = act ? s_val[wave][lane] : -INFINITY;
    const int xi = act ? s_idx[wave][lane] : -1;
    const float m = wave_max(xv);
    int sel;
    float prob;
    if (T <= 0.f) {
      const unsigned long long mk = __ballot(act && xv == m);
      sel = mk ? __ffsll(mk) - 1 : 0;
      prob = lane == sel ? 1.f : 0.f;
    } else {
      const float e = act ? expf((xv - m) / T) : 0.f;
      const float S = wave_inclusive_sum(e, lane);
      const float Z = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, S), kk - 1));
      const float C = S / Z;
      const unsigned long long mk = __ballot(act && u < C);
      sel = mk ? __ffsll(mk) - 1 : kk - 1;
      prob = e / Z;
    }
    int token = __builtin_amdgcn_readlane(xi, sel);
    if (!started) token = p.fill;
    if (lane == 0) p.tokens[row] = token;
    if (lane < p.top_k) {
      if (p.topk_idx != nullptr) p.topk_idx[(size_t)row * p.top_k + lane] = act ? xi : -1;
      if (p.topk_prob != nullptr) p.topk_prob[(size_t)row * p.top_k + lane] = act ? prob : 0.f;
    }
  }
}

template <int VPL>
static hipError_t sample_launch_vpl(const SampleParams& p, hipStream_t stream) {
  const int rows = p.B * p.n_cb;
  const int blocks = (rows + kSampWaves - 1) / kSampWaves;
  hipLaunchKernelGGL(sample_topk_kernel<VPL>, dim3(blocks), dim3(kSampWaves * kWave), 0, stream, p);
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

hipError_t advance_launch(int32_t* len, int32_t* step, int B, hipStream_t stream) {
  hipLaunchKernelGGL(advance_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, len, step, B);
  return hipGetLastError();
}

}  // namespace dec
