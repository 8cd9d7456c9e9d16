// Single-token attention over the valid prefix of static KV caches (gfx950).
//
// "Optimized Parler TTS", "Analysis and improvements": with static caches the
// attention kernel moved the whole preallocated cache every step and became
// several times slower than the dynamic-cache one.  This kernel reads only the
// first len[b] slots of each sequence, so its HBM traffic is the valid K/V
// bytes plus a few hundred bytes per sequence.
//
// Design (one launch serves every layer, and optionally self- and
// cross-attention together):
//   * Work item = (segment, layer, batch, head, chunk of kAttnChunk keys).  The
//     item list is derived on the device from len[] (device-resident, so a
//     captured graph stays valid as lengths change); a persistent grid walks it.
//   * Inside an item each of the 4 waves owns 64-key tiles.  A key row of 64
//     bf16 is 128 B = 8 lanes x 16 B, so one wave-wide dwordx4 load covers 8
//     consecutive keys (1 KiB, fully coalesced); K and V of a tile are 16
//     loads in flight per wave.  There is no MFMA: the work is a GEMV.
//   * The dot product reduces across the 8 lanes of a key with DPP moves; the
//     tile max and the final sums reduce across key groups with DPP/shuffles.
//     Softmax is online, in base 2 (q pre-scaled by scale*log2 e), fp32.
//   * Waves combine through LDS in wave order; chunks of one sequence combine
//     through a workspace in chunk order, performed by whichever workgroup
//     arrives last (an arrival counter that the combiner resets to zero).
//     The split depends on len only, so results are bitwise reproducible and
//     independent of the grid size.
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
  x[0] = __builtin_bit_cast(float, w.x); x[1] = __builtin_bit_cast(float, w.y);
  x[2] = __builtin_bit_cast(float, w.z); x[3] = __builtin_bit_cast(float, w.w);
}

template <typename T, int EPL>
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

__device__ __forceinline__ int nchunks(int n) { return n > 0 ? (n + kAttnChunk - 1) / kAttnChunk : 1; }

template <typename T>
__global__ __launch_bounds__(kAttnThreads) void attn_decode_kernel(AttnParams p) {
  constexpr int HD = kAttnHeadDim;
  constexpr int EPL = KvTraits<T>::kElemsPerLoad;  // elements per lane per load
  constexpr int LPK = HD / EPL;                     // lanes per key row: 8 (bf16), 16 (f32)
  constexpr int KPL = kWave / LPK;                  // keys per wave-wide load
  constexpr int NLD = kAttnKeysPerWaveTile / KPL;   // loads per operand per tile

  extern __shared__ int s_dyn[];                    // [G] clamped lengths, [G+1] item prefix
  __shared__ float s_acc[kAttnWaves][HD];
  __shared__ float s_m[kAttnWaves];
  __shared__ float s_l[kAttnWaves];
  __shared__ int s_wsum[kAttnWaves];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int B = p.B;
  const int G = p.nseg * B;
  const int NLH = p.NL * p.H;
  int* s_n = s_dyn;
  int* s_pref = s_dyn + G;

  // ---- item list: per (segment, b) group, NL*H*nchunks(len) items -------------------
  {
    const int per = (G + kAttnThreads - 1) / kAttnThreads;
    const int lo = min(G, tid * per);
    const int hi = min(G, lo + per);
    int local = 0;
    for (int g = lo; g < hi; ++g) {
      const bool cross = g >= B;
      const int32_t* len = cross ? p.seg[1].len : p.seg[0].len;
      const int cap = cross ? p.seg[1].L_cap : p.seg[0].L_cap;
      int n = len[cross ? g - B : g];
      n = n < 0 ? 0 : (n > cap ? cap : n);
      s_n[g] = n;
      local += NLH * nchunks(n);
    }
    int ex = wave_exclusive_sum_int(local, lane);
    if (lane == kWave - 1) s_wsum[wave] = ex + local;
    __syncthreads();
    for (int w = 0; w < wave; ++w) ex += s_wsum[w];
    for (int g = lo; g < hi; ++g) {
      s_pref[g] = ex;
      ex += NLH * nchunks(s_n[g]);
    }
    if (tid == 0) s_pref[G] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
  }
  const int total = s_pref[G];

  const int kg = lane / LPK;  // key slot within a wave-wide load
  const int dl = lane % LPK;  // which 16-byte slice of the row this lane reads

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    __syncthreads();  // LDS of the previous item is free

    // locate the group: the largest g with s_pref[g] <= item
    int glo = 0, ghi = G - 1;
    while (glo < ghi) {
      const int mid = (glo + ghi + 1) >> 1;
      if (s_pref[mid] <= item) glo = mid; else ghi = mid - 1;
    }
    const int g = glo;
    const bool cross = g >= B;
    const AttnSeg& S = cross ? p.seg[1] : p.seg[0];
    const int b = cross ? g - B : g;
    const int n = s_n[g];
    const int nck = nchunks(n);
    const int r = item - s_pref[g];
    const int c = r % nck;
    const int lh = r / nck;
    const int h = lh % p.H;
    const int layer = lh / p.H;
    const size_t sidx = ((size_t)layer * B + b) * p.H + h;
    float* out = S.out + sidx * HD;

    if (n == 0) {  // no valid key: defined output of zeros
      if (tid < HD) out[tid] = 0.f;
      continue;
    }

    const T* qp = static_cast<const T*>(S.q) + sidx * HD;
    const T* kp = static_cast<const T*>(S.k) + sidx * (size_t)S.L_cap * HD;
    const T* vp = static_cast<const T*>(S.v) + sidx * (size_t)S.L_cap * HD;

    float qf[EPL];
    {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qp + dl * EPL);
      unpack(w, qf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[e] *= p.qscale;
    }

    float m_run = -INFINITY, l_run = 0.f;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

    const int chunk_start = c * kAttnChunk;
#pragma unroll
    for (int t = 0; t < kAttnTiles; ++t) {
      const int base = chunk_start + (t * kAttnWaves + wave) * kAttnKeysPerWaveTile;
      if (base >= n) break;  // uniform across the wave
      u32x4 kr[NLD], vr[NLD];
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int j = base + i * KPL + kg;
        if (j < n) {
          kr[i] = *reinterpret_cast<const u32x4*>(kp + (size_t)j * HD + dl * EPL);
          vr[i] = *reinterpret_cast<const u32x4*>(vp + (size_t)j * HD + dl * EPL);
        } else {
          kr[i] = u32x4{0u, 0u, 0u, 0u};
          vr[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      float s[NLD];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        s[i] = group_sum<LPK>(dot_slice<T, EPL>(qf, kr[i]));
        if (base + i * KPL + kg >= n) s[i] = -INFINITY;
        mt = fmaxf(mt, s[i]);
      }
      mt = xor_max_from<LPK>(mt);
      const float m_new = fmaxf(m_run, mt);  // finite: key `base` is valid
      const float corr = exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= corr;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const float pj = exp2f(s[i] - m_new);
        l_run += pj;
        accum_slice(acc, pj, vr[i]);
      }
      m_run = m_new;
    }

    // sum the key groups of the wave (all share the wave's running max)
    l_run = xor_sum_from<LPK>(l_run);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = xor_sum_from<LPK>(acc[e]);
    if (kg == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][dl * EPL + e] = acc[e];
    }
    if (lane == 0) {
      s_m[wave] = m_run;
      s_l[wave] = l_run;
    }
    __syncthreads();

    if (tid < HD) {  // combine the waves in wave order
      float M = s_m[0];
#pragma unroll
      for (int w = 1; w < kAttnWaves; ++w) M = fmaxf(M, s_m[w]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = (s_m[w] == -INFINITY) ? 0.f : exp2f(s_m[w] - M);
        L = fmaf(f, s_l[w], L);
        A = fmaf(f, s_acc[w][tid], A);
      }
      if (nck == 1) {
        out[tid] = A / L;
      } else {
        float* pp = S.part + (sidx * S.nck_cap + c) * kAttnPartStride;
        pp[4 + tid] = A;
        if (tid == 0) {
          pp[0] = M;
          pp[1] = L;
        }
      }
    }
    if (nck == 1) continue;

    // split-K: the last chunk to arrive combines all chunks in chunk order
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(S.ticket + sidx, 1) == nck - 1);
    __syncthreads();
    if (s_last) {
      __threadfence();
      if (tid < HD) {
        const float* pp = S.part + sidx * S.nck_cap * kAttnPartStride;
        float M = -INFINITY;
        for (int cc = 0; cc < nck; ++cc) M = fmaxf(M, pp[cc * kAttnPartStride]);
        float L = 0.f, A = 0.f;
        for (int cc = 0; cc < nck; ++cc) {
          const float* q = pp + cc * kAttnPartStride;
          const float f = exp2f(q[0] - M);
          L = fmaf(f, q[1], L);
          A = fmaf(f, q[4 + tid], A);
        }
        out[tid] = A / L;
      }
      if (tid == 0) __hip_atomic_store(S.ticket + sidx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

long long attn_items_cap(const AttnParams& p) {
  long long total = 0;
  for (int s = 0; s < p.nseg; ++s) {
    const long long nck = p.seg[s].L_cap > 0 ? (p.seg[s].L_cap + kAttnChunk - 1) / kAttnChunk : 1;
    total += (long long)p.NL * p.B * p.H * nck;
  }
  return total;
}

namespace {
struct DevInfo {
  int cus = 0;
  int occ[2] = {0, 0};  // blocks per CU, per dtype, at the small-LDS size
};
DevInfo g_dev[64];
}  // namespace

template <typename T>
static void* attn_kernel_ptr() {
  return reinterpret_cast<void*>(&attn_decode_kernel<T>);
}

hipError_t attn_launch(const AttnParams& p, int dtype, int blocks, hipStream_t stream) {
  const int G = p.nseg * p.B;
  const size_t lds = (size_t)(2 * G + 1) * sizeof(int);
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
    long long want = (long long)di.cus * occ;
    blocks = (int)(want < cap ? want : cap);
  }
  if (blocks < 1) blocks = 1;
  if (dtype == 0) {
    hipLaunchKernelGGL(attn_decode_kernel<uint16_t>, dim3(blocks), dim3(kAttnThreads), lds, stream, p);
  } else {
    hipLaunchKernelGGL(attn_decode_kernel<float>, dim3(blocks), dim3(kAttnThreads), lds, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dec
