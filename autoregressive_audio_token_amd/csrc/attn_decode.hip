// Single-token attention over the valid prefix of static KV caches (gfx950).
//
// "Optimized Parler TTS", "Analysis and improvements": with static caches the
// attention kernel moved the whole preallocated cache every step and became
// several times slower than the dynamic-cache one.  This kernel reads only the
// first len[b] slots of each sequence, so its HBM traffic is the valid K/V
// bytes plus a few hundred bytes per sequence.
//
// Split-K flash-decode, arranged for CDNA4:
//   * A sequence of n valid keys is cut into chunks of kAttnChunk keys.  One
//     workgroup of kAttnWaves wavefronts reads a whole chunk in one round: each
//     wave owns 64 keys and issues all of its K and V loads at once (a key row
//     of 64 bf16 is 128 B = 8 lanes x 16 B, so one dwordx4 load instruction
//     covers 8 consecutive keys, 1 KiB, fully coalesced).  There is no MFMA:
//     the work is a GEMV.
//   * Scores reduce across the 8 lanes of a key with DPP moves; softmax is in
//     base 2 (q pre-scaled by scale * log2 e) and fp32 throughout.
//   * The waves' partial states (max, sum, acc[64]) combine through LDS in
//     wave order into one state per chunk; the chunk states of a sequence then
//     fold in chunk order.  Normally one workgroup owns every chunk of its
//     sequence, so nothing crosses workgroups (no atomics, no fences).  When a
//     launch has few sequences, chunks are spread over workgroups, written to
//     the workspace, and a second kernel performs the same fold; both paths
//     execute identical arithmetic, so results are bitwise equal either way
//     and independent of the grid.
//   * The list of work items is derived on the device from len[] (device
//     resident, so a captured graph stays valid as lengths change), longest
//     sequences first; a persistent grid of one workgroup per CU walks it.
#include "dec_common.h"
#include "dec_kernels.h"

namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

template <int EPL>
__device__ __forceinline__ float dot_slice(const float (&q)[EPL], const u32x4& w) {
  float x[EPL];
  unpack(w, x);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) s = fmaf(q[e], x[e], s);
  return s;
}

template <int EPL>
__device__ __forceinline__ void accum_slice(float (&acc)[EPL], float p, const u32x4& w) {
  float x[EPL];
  unpack(w, x);
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, x[e], acc[e]);
}

__device__ __forceinline__ int nchunks(int n) { return n > 0 ? (n + kAttnChunk - 1) / kAttnChunk : 0; }

// Work items per (layer, head) of a sequence with n valid keys.
__device__ __forceinline__ int items_per_lh(int n, int cpi) {
  const int c = nchunks(n);
  return c > cpi ? (c + cpi - 1) / cpi : 1;
}

// Waves that share one sequence: the smallest power of two covering n keys in one
// round, or every wave of the workgroup (then the sequence runs in chunk rounds).
// Shorter sequences are packed kAttnWaves / S to a work item.
__device__ __forceinline__ int waves_per_seq(int n) {
  int s = 1;
  while (s < kAttnWaves && s * kAttnKeysPerWave < n) s <<= 1;
  return s;
}

// Work items of a (segment, b) group with n valid keys.
__device__ __forceinline__ int group_items(int n, int NLH, int cpi) {
  const int S = waves_per_seq(n);
  if (S < kAttnWaves) {
    const int P = kAttnWaves / S;
    return (NLH + P - 1) / P;
  }
  return NLH * items_per_lh(n, cpi);
}

// Fold chunk state (mc, lc, ac) into the running state (m, l, a); the first
// chunk initialises it.  Shared by both fold sites so they agree bit for bit.
__device__ __forceinline__ void fold_chunk(bool first, float mc, float lc, float ac, float& m,
                                           float& l, float& a) {
  if (first) {
    m = mc;
    l = lc;
    a = ac;
    return;
  }
  const float mn = fmaxf(m, mc);
  const float fa = exp2f(m - mn);
  const float fc = exp2f(mc - mn);
  l = fmaf(lc, fc, l * fa);
  a = fmaf(ac, fc, a * fa);
  m = mn;
}

template <typename T>
__global__ __launch_bounds__(kAttnThreads) void attn_decode_kernel(AttnParams p) {
  constexpr int HD = kAttnHeadDim;
  constexpr int EPL = KvTraits<T>::kElemsPerLoad;  // elements per lane per load
  constexpr int LPK = HD / EPL;                     // lanes per key row: 8 (bf16), 16 (f32)
  constexpr int KPL = kWave / LPK;                  // keys per wave-wide load
  constexpr int NLD = kAttnKeysPerWave / KPL;       // loads per operand per round

  extern __shared__ int s_dyn[];  // [G] lengths, [G] order, [G+1] item prefix
  __shared__ float s_acc[kAttnWaves][HD];
  __shared__ float s_m[kAttnWaves];
  __shared__ float s_l[kAttnWaves];
  __shared__ int s_wsum[kAttnWaves];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int B = p.B;
  const int G = p.nseg * B;
  const int NLH = p.NL * p.H;
  const int cpi = p.cpi;
  int* s_n = s_dyn;
  int* s_order = s_dyn + G;
  int* s_pref = s_dyn + 2 * G;

  // ---- item list: groups (segment, b) longest first; group_items(n) each -------------
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
  {
    const int per = (G + kAttnThreads - 1) / kAttnThreads;
    const int lo = min(G, tid * per);
    const int hi = min(G, lo + per);
    int local = 0;
    for (int i = lo; i < hi; ++i) local += group_items(s_n[s_order[i]], NLH, cpi);
    int ex = wave_exclusive_sum_int(local, lane);
    if (lane == kWave - 1) s_wsum[wave] = ex + local;
    __syncthreads();
    int total = 0;
    for (int w = 0; w < kAttnWaves; ++w) {
      if (w < wave) ex += s_wsum[w];
      total += s_wsum[w];
    }
    for (int i = lo; i < hi; ++i) {
      s_pref[i] = ex;
      ex += group_items(s_n[s_order[i]], NLH, cpi);
    }
    if (tid == 0) s_pref[G] = total;
    __syncthreads();
  }
  const int total = s_pref[G];

  const int kg = lane / LPK;  // key slot within a wave-wide load
  const int dl = lane % LPK;  // which 16-byte slice of the row this lane reads

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // locate the group: the largest position with s_pref[pos] <= item
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int g = s_order[lo];
    const bool cross = g >= B;
    const AttnSeg& S = cross ? p.seg[1] : p.seg[0];
    const int b = cross ? g - B : g;
    const int n = s_n[g];
    const int r = item - s_pref[lo];
    const int nck = nchunks(n);
    const int spw = waves_per_seq(n);            // waves per sequence
    const bool packed = spw < kAttnWaves;        // several sequences share this item
    const int P = kAttnWaves / spw;              // sequences in this item (packed)

    // this wave's sequence and which 64-key slice of each round it reads
    int wave_lh, wave_part, c0, c1;
    bool whole;
    if (packed) {
      wave_lh = r * P + wave / spw;
      wave_part = wave % spw;
      c0 = 0;
      c1 = nck;  // at most one chunk
      whole = true;
    } else {
      const int ipl = items_per_lh(n, cpi);
      const int k = r % ipl;
      wave_lh = r / ipl;
      wave_part = wave;
      c0 = k * cpi;
      c1 = min(nck, c0 + cpi);
      whole = ipl == 1;
    }
    const bool wave_ok = wave_lh < NLH;  // the last packed item may have empty slots
    const int wlh = wave_ok ? wave_lh : 0;
    const size_t wave_sidx = ((size_t)(wlh / p.H) * B + b) * p.H + (wlh % p.H);

    // the combining threads: sequence slot `slot`, head dimension `d`
    const int slot = tid / HD;
    const int d = tid % HD;
    const int nslot = packed ? P : 1;
    const int slot_lh = packed ? r * P + slot : wave_lh;
    const bool slot_ok = slot < nslot && slot_lh < NLH;
    const int slh = slot_ok ? slot_lh : 0;
    const size_t slot_sidx = ((size_t)(slh / p.H) * B + b) * p.H + (slh % p.H);

    if (n == 0) {  // no valid key: defined output of zeros
      if (slot_ok) S.out[slot_sidx * HD + d] = 0.f;
      continue;
    }

    const T* qp = static_cast<const T*>(S.q) + wave_sidx * HD;
    const T* kp = static_cast<const T*>(S.k) + wave_sidx * (size_t)S.L_cap * HD;
    const T* vp = static_cast<const T*>(S.v) + wave_sidx * (size_t)S.L_cap * HD;
    float fm = 0.f, fl = 0.f, fa = 0.f;  // running fold (combining threads)

    for (int c = c0; c < c1; ++c) {
      const int base = c * kAttnChunk + wave_part * kAttnKeysPerWave;
      float m_w = -INFINITY, l_w = 0.f;
      float acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
      if (wave_ok && base < n) {  // uniform across the wave
        u32x4 kr[NLD], vr[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int j = base + i * KPL + kg;
          if (j < n) {  // K and V are read once: non-temporal loads
            kr[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(kp + (size_t)j * HD + dl * EPL));
            vr[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(vp + (size_t)j * HD + dl * EPL));
          } else {
            kr[i] = u32x4{0u, 0u, 0u, 0u};
            vr[i] = u32x4{0u, 0u, 0u, 0u};
          }
        }
        float qf[EPL];
        {
          const u32x4 w = *reinterpret_cast<const u32x4*>(qp + dl * EPL);
          unpack(w, qf);
#pragma unroll
          for (int e = 0; e < EPL; ++e) qf[e] *= p.qscale;
        }
        float s[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          s[i] = group_sum<LPK>(dot_slice(qf, kr[i]));
          if (base + i * KPL + kg >= n) s[i] = -INFINITY;
          m_w = fmaxf(m_w, s[i]);
        }
        m_w = xor_max_from<LPK>(m_w);  // finite: key `base` is valid
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const float pj = exp2f(s[i] - m_w);
          l_w += pj;
          accum_slice(acc, pj, vr[i]);
        }
        // sum the key groups of the wave (they share the wave max)
        l_w = xor_sum_from<LPK>(l_w);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = xor_sum_from<LPK>(acc[e]);
      }
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
          const float f = (s_m[w] == -INFINITY) ? 0.f : exp2f(s_m[w] - mc);
          lc = fmaf(f, s_l[w], lc);
          ac = fmaf(f, s_acc[w][d], ac);
        }
        if (whole) {
          fold_chunk(c == c0, mc, lc, ac, fm, fl, fa);
        } else {
          float* pp = S.part + (slot_sidx * S.nck_cap + c) * kAttnPartStride;
          pp[4 + d] = ac;
          if (d == 0) {
            pp[0] = mc;
            pp[1] = lc;
          }
        }
      }
      __syncthreads();  // LDS is rewritten by the next chunk
    }
    if (whole && slot_ok) S.out[slot_sidx * HD + d] = fa / fl;
  }
}

// Split mode only: fold the chunk states of every sequence that spans several
// work items, in chunk order (one 64-thread workgroup per sequence).
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnParams p) {
  const int nseq = p.NL * p.B * p.H;
  int sid = blockIdx.x;
  const AttnSeg& S = sid >= nseq ? p.seg[1] : p.seg[0];
  if (sid >= nseq) sid -= nseq;
  const int b = (sid / p.H) % p.B;
  int n = S.len[b];
  n = n < 0 ? 0 : (n > S.L_cap ? S.L_cap : n);
  const int nck = nchunks(n);
  if (nck <= p.cpi) return;  // written whole by the attention kernel
  const int d = threadIdx.x;
  const float* pp = S.part + (size_t)sid * S.nck_cap * kAttnPartStride;
  float fm = 0.f, fl = 0.f, fa = 0.f;
  for (int c = 0; c < nck; ++c) {
    const float* q = pp + (size_t)c * kAttnPartStride;
    fold_chunk(c == 0, q[0], q[1], q[4 + d], fm, fl, fa);
  }
  S.out[(size_t)sid * kAttnHeadDim + d] = fa / fl;
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
struct DevInfo {
  int cus = 0;
  int occ[2] = {0, 0};  // resident workgroups per CU, per dtype, at the small-LDS size
};
DevInfo g_dev[64];
}  // namespace

template <typename T>
static void* attn_kernel_ptr() {
  return reinterpret_cast<void*>(&attn_decode_kernel<T>);
}

hipError_t attn_launch(const AttnParams& p, int dtype, int blocks, hipStream_t stream) {
  const int G = p.nseg * p.B;
  const size_t lds = (size_t)(3 * G + 1) * sizeof(int);
  void* fn = dtype == 0 ? attn_kernel_ptr<uint16_t>() : attn_kernel_ptr<float>();
  if (blocks <= 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    DevInfo& di = g_dev[dev & 63];
    if (di.cus == 0) {
      int cus = 0;
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      di.cus = cus;
    }
    int occ = di.occ[dtype];
    if (occ == 0 || G > 64) {
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kAttnThreads, lds);
      if (e != hipSuccess) return e;
      if (occ < 1) occ = 1;
      if (G <= 64) di.occ[dtype] = occ;
    }
    const long long cap = attn_items_cap(p);
    const long long want = (long long)di.cus * occ;
    blocks = (int)(want < cap ? want : cap);
  }
  if (blocks < 1) blocks = 1;
  if (dtype == 0) {
    hipLaunchKernelGGL(attn_decode_kernel<uint16_t>, dim3(blocks), dim3(kAttnThreads), lds, stream, p);
  } else {
    hipLaunchKernelGGL(attn_decode_kernel<float>, dim3(blocks), dim3(kAttnThreads), lds, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bool split = false;
  for (int s = 0; s < p.nseg; ++s) split = split || p.seg[s].nck_cap > p.cpi;
  if (split) {
    const int nseq = p.NL * p.B * p.H * p.nseg;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(nseq), dim3(64), 0, stream, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace dec
