// The merged 9-codebook LM head on the last position and the merged 9-codebook
// embedding sum (gfx950).
//
// "Optimized Parler TTS", "Analysis and improvements": logits are produced for
// the last position only, the nine LM heads are merged into one weight matrix,
// and the nine embedding lookups into one gather.  "A rough architecture of
// Parler TTS": the decoder takes the nine tokens of a step at once, so its
// input is the sum of the nine codebooks' embedding rows.
//
// LM head: logits[b, c, v] = <h[b], W[c, v]> for v < V_valid.  At decode batch sizes
// the product is bound by reading W once (~20 MB at 9 x 1089 x 1024 bf16).  At B <= 2 it
// is a matrix-vector product and runs on the vector ALU (lm_head_kernel,
// v_dot2c_f32_bf16); larger batches run on MFMA (lm_head_mfma_kernel), where each load of
// h serves many rows of W.  Both read W in whole 128-byte lines in the same order: a
// workgroup owns 16 rows of one codebook, its 4 waves split D into quarters, and 8
// consecutive lanes read one line.  A buffer descriptor spans the codebook's V_valid
// rows, so the padding rows of a partial last group are never read.
#include "dec_common.h"
#include "dec_kernels.h"

namespace dec {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float s) {
  s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), s, false);
  return s;
}

constexpr int kBufWord3 = 0x00020000;
constexpr int kBufNonTemporal = 2;

}  // namespace

// Small batches: the product on the vector ALU (v_dot2c_f32_bf16), with W read exactly as
// the MFMA kernel below reads it.  A workgroup owns 16 rows of one codebook and its 4
// waves split D into quarters; load t gives lane l row (l >> 3) + 8 (t & 1), columns
// (t >> 1) * 64 + (l & 7) * 8 .. + 8 of the wave's quarter, so 8 consecutive lanes read
// one whole 128-byte line.  Per batch row, a lane dots its slices with the same columns
// of h (read straight from memory: 16 bytes per 64 columns), the 8 lanes of a row add
// with DPP, and the four quarter sums meet in LDS in wave order.  Rows of W at or past
// V_valid read as zero through the descriptor and are not stored.
template <int NSEG>
__global__ __launch_bounds__(kHeadWaves * kWave) void lm_head_kernel(HeadParams p) {
  constexpr int D = NSEG * 64;
  constexpr int Q = D / kHeadWaves;        // columns per wave
  constexpr int LT = 2 * Q / 64;           // loads per wave: two row halves per 64 columns
  __shared__ float s_q[2][kHeadWaves][16];  // quarter sums, double-buffered over b
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  const int rgpc = (p.V_valid + 15) / 16;  // 16-row groups per codebook
  const int c = blockIdx.x / rgpc;
  const int v0 = (blockIdx.x - c * rgpc) * 16;
  const int col = wave * Q + (lane & 7) * 8;  // this lane's first column

  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.W + (size_t)c * p.V_stride * D), 0, p.V_valid * D * 2, kBufWord3);
  u32x4 w[LT];
#pragma unroll
  for (int t = 0; t < LT; ++t)
    w[t] = __builtin_amdgcn_raw_buffer_load_b128(
        rw, ((v0 + (lane >> 3) + 8 * (t & 1)) * D + col + (t >> 1) * 64) * 2, 0, kBufNonTemporal);
  for (int b = 0; b < p.B; ++b) {
    const u32x4* hb = reinterpret_cast<const u32x4*>(p.h + (size_t)b * D + col);
    float acc0 = 0.f, acc1 = 0.f;  // rows (l >> 3) and (l >> 3) + 8
#pragma unroll
    for (int j = 0; j < LT / 2; ++j) {
      const u32x4 hv = hb[j * 8];  // columns j * 64 + (l & 7) * 8 .. + 8 of the quarter
      acc0 = dot8(w[2 * j], hv, acc0);
      acc1 = dot8(w[2 * j + 1], hv, acc1);
    }
    acc0 = group_sum<8>(acc0);
    acc1 = group_sum<8>(acc1);
    float* const q = s_q[b & 1][wave];
    if ((lane & 7) == 0) {
      q[lane >> 3] = acc0;
      q[(lane >> 3) + 8] = acc1;
    }
    __syncthreads();  // (double buffering: the other half is rewritten only after the next)
    if (wave == 0 && lane < 16 && v0 + lane < p.V_valid) {
      const float (*qs)[16] = s_q[b & 1];
      p.logits[((size_t)b * p.n_cb + c) * p.V_stride + v0 + lane] =
          ((qs[0][lane] + qs[1][lane]) + qs[2][lane]) + qs[3][lane];
    }
  }
}

// Orders one wave's LDS writes before its later LDS reads (and reads before later
// writes) of lanes other than its own; LDS executes a wave's operations in order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Batches of several rows: the same product on MFMA (v_mfma_f32_16x16x32_bf16).  A
// workgroup owns RT tiles of 16 rows of one codebook; its 4 waves split D into
// quarters, so a wave holds RT x 16 rows x D/4 of W (T k-steps of 32 per tile), read in
// whole cache lines and rearranged through LDS.  The A operand is W (lane l: row
// l % 16, k (l / 16) * 8 .. + 8 of each 32-wide step), the B operand h^T for 16 batch
// rows (lane l: batch row l % 16, the same k), so C holds rows (l / 16) * 4 + i of
// batch row l % 16.  The k order inside a step is the same for A
// and B, so the product is the plain dot product.  A pass covers NBT tiles of 16 batch
// rows whose B fragments are all loaded with W, up front; the next pass's fragments are
// in flight while a pass is reduced.  Rows of W at or past V_valid and rows of h at or
// past B read as zero through their descriptors.  The four quarter sums of each output
// tile meet in LDS and are added in wave order.
template <int T, int RT, int NBT>
__global__ __launch_bounds__(kHeadWaves * kWave) void lm_head_mfma_kernel(HeadParams p) {
  constexpr int D = kHeadWaves * 32 * T;
  constexpr int NT = RT * NBT;  // output tiles of 16 x 16 per pass
  __shared__ f32x4 s_c[kHeadWaves][NT][kWave];
  __shared__ u32x4 s_w[kHeadWaves][T / 2][128];  // per wave: 16 rows x 8 chunks per step pair
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  constexpr int ROWS = 16 * RT;
  const int rgpc = (p.V_valid + ROWS - 1) / ROWS;  // row groups per codebook
  const int c = blockIdx.x / rgpc;
  const int v0 = (blockIdx.x - c * rgpc) * ROWS;
  const int r = lane & 15;    // A row / B column within a tile
  const int q = lane >> 4;    // 8-element k slice within a 32-wide step
  const int k0 = wave * (D / kHeadWaves) + q * 8;

  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.W + (size_t)c * p.V_stride * D), 0, p.V_valid * D * 2, kBufWord3);
  // W is read in whole 128-byte lines, 8 consecutive lanes to a line: load t gives lane
  // l row (l >> 3) + 8 * (t & 1), columns (t >> 1) * 64 + (l & 7) * 8 .. + 8 of the
  // wave's quarter.  Each tile of 16 rows then passes through the wave's own slice of
  // LDS into the A layout.  A pair of loads covers 16 rows x 8 chunks of 16 bytes; the
  // chunk of row R sits at position chunk ^ swz(R), which puts the 8 chunks of a row
  // (the writes) and one chunk of 16 rows (the reads) in distinct bank groups.
  static_assert(T % 2 == 0, "W loads come in pairs of 32-wide steps");
  const int wl = (lane >> 3) * D + wave * (D / kHeadWaves) + (lane & 7) * 8;
  u32x4 a[RT][T];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < T; ++t)
      a[rt][t] = __builtin_amdgcn_raw_buffer_load_b128(
          rw, ((v0 + rt * 16 + 8 * (t & 1)) * D + wl + (t >> 1) * 64) * 2, 0, kBufNonTemporal);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.h), 0, p.B * D * 2, kBufWord3);
  u32x4 hq[NBT][T];
#pragma unroll
  for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
    for (int t = 0; t < T; ++t)
      hq[bt][t] = __builtin_amdgcn_raw_buffer_load_b128(rh, ((bt * 16 + r) * D + k0 + t * 32) * 2,
                                                        0, 0);
  u32x4* const tile = &s_w[wave][0][0];
  auto swz = [](int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; };
  int put[2], get[2];  // chunk slots within a pair: written by load parity, read by step parity
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int wr = (lane >> 3) + 8 * h;
    put[h] = wr * 8 + ((lane & 7) ^ swz(wr));
    get[h] = r * 8 + ((h * 4 + q) ^ swz(r));
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (rt > 0) wave_lds_sync();  // the previous tile's reads are done before the writes
#pragma unroll
    for (int t = 0; t < T; ++t) tile[(t >> 1) * 128 + put[t & 1]] = a[rt][t];
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < T; ++t) a[rt][t] = tile[(t >> 1) * 128 + get[t & 1]];
  }
  for (int b0 = 0; b0 < p.B; b0 += 16 * NBT) {
    f32x4 acc[NBT][RT];
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        acc[bt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < T; ++t)
          acc[bt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, a[rt][t]), __builtin_bit_cast(bf16x8, hq[bt][t]),
              acc[bt][rt], 0, 0, 0);
      }
    if (b0 + 16 * NBT < p.B) {  // the next pass's fragments (uniform branch)
#pragma unroll
      for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
        for (int t = 0; t < T; ++t)
          hq[bt][t] = __builtin_amdgcn_raw_buffer_load_b128(
              rh, ((b0 + (NBT + bt) * 16 + r) * D + k0 + t * 32) * 2, 0, 0);
    }
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s_c[wave][bt * RT + rt][lane] = acc[bt][rt];
    __syncthreads();
    for (int tile = wave; tile < NT; tile += kHeadWaves) {  // wave w reduces tiles w, w + 4, ..
      const f32x4 sum = ((s_c[0][tile][lane] + s_c[1][tile][lane]) + s_c[2][tile][lane]) +
                        s_c[3][tile][lane];
      const int b = b0 + (tile / RT) * 16 + r;
      const int v = v0 + (tile % RT) * 16 + q * 4;  // rows v .. v + 3 of codebook c
      if (b < p.B) {
        float* out = p.logits + ((size_t)b * p.n_cb + c) * p.V_stride + v;
        if (v + 3 < p.V_valid) {
          *reinterpret_cast<f32x4*>(out) = sum;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v + i < p.V_valid) out[i] = sum[i];
        }
      }
    }
    __syncthreads();  // s_c is rewritten by the next pass
  }
}

template <int T, int RT, int NBT>
static void lm_head_mfma_go(const HeadParams& p, hipStream_t stream) {
  const int blocks = p.n_cb * ((p.V_valid + 16 * RT - 1) / (16 * RT));
  hipLaunchKernelGGL((lm_head_mfma_kernel<T, RT, NBT>), dim3(blocks), dim3(kHeadWaves * kWave), 0,
                     stream, p);
}

template <int NSEG>
static hipError_t lm_head_launch_n(const HeadParams& p, hipStream_t stream) {
  if (!p.force_gemv) {
    constexpr int T = NSEG * 64 / (kHeadWaves * 32);
    // Row tiles x batch tiles per workgroup, from measurement at every width: one 16-row
    // tile up to 12 batch rows (the most workgroups, which is what a weight-bound
    // product needs); beyond, four row tiles and two batch tiles per pass, so each load
    // of h serves 64 rows of W.  The MFMA kernel is the faster one from B = 1 on (W is
    // read once either way; its loads are whole lines).
    int cfg = p.mfma_cfg;
    if (cfg == 0) cfg = p.B <= 12 ? 11 : 42;
    switch (cfg) {
      case 11: lm_head_mfma_go<T, 1, 1>(p, stream); break;
      case 12: lm_head_mfma_go<T, 1, 2>(p, stream); break;
      case 22: lm_head_mfma_go<T, 2, 2>(p, stream); break;
      default: lm_head_mfma_go<T, 4, 2>(p, stream); break;
    }
    return hipGetLastError();
  }
  const int blocks = p.n_cb * ((p.V_valid + 15) / 16);
  hipLaunchKernelGGL(lm_head_kernel<NSEG>, dim3(blocks), dim3(kHeadWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

hipError_t lm_head_launch(const HeadParams& p, hipStream_t stream) {
  switch (p.D) {
    case 512: return lm_head_launch_n<8>(p, stream);
    case 768: return lm_head_launch_n<12>(p, stream);
    case 1024: return lm_head_launch_n<16>(p, stream);
    case 1536: return lm_head_launch_n<24>(p, stream);
    case 2048: return lm_head_launch_n<32>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// x[b, :] = sum_c E[c, tokens[b, c], :]; tokens outside [0, V_emb) add nothing.
// One workgroup per (sequence, 16-byte column slice block); fp32 accumulation in
// codebook order.
__global__ __launch_bounds__(256) void embed_sum_kernel(EmbedParams p) {
  const int b = blockIdx.y;
  const int col = (blockIdx.x * blockDim.x + threadIdx.x) * 8;  // bf16 element
  if (col >= p.D) return;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int c = 0; c < p.n_cb; ++c) {
    const int t = p.tokens[(size_t)b * p.n_cb + c];
    if (t < 0 || t >= p.V_emb) continue;  // uniform across the workgroup
    const u32x4 r = *reinterpret_cast<const u32x4*>(p.E + ((size_t)c * p.V_emb + t) * p.D + col);
    acc[0] += bf16_lo(r.x); acc[1] += bf16_hi(r.x);
    acc[2] += bf16_lo(r.y); acc[3] += bf16_hi(r.y);
    acc[4] += bf16_lo(r.z); acc[5] += bf16_hi(r.z);
    acc[6] += bf16_lo(r.w); acc[7] += bf16_hi(r.w);
  }
  float4* out = reinterpret_cast<float4*>(p.x + (size_t)b * p.D + col);
  out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

hipError_t embed_sum_launch(const EmbedParams& p, hipStream_t stream) {
  const int threads = 128;
  const int per_b = (p.D / 8 + threads - 1) / threads;
  hipLaunchKernelGGL(embed_sum_kernel, dim3(per_b, p.B), dim3(threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dec
