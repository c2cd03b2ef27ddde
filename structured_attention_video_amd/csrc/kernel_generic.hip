// Plain grouped-attention kernel: fp32 VALU arithmetic, any problem length.
//
// This is the fp32 path (fp32 products keep the 1e-5 bound that reduced-
// precision matrix cores would break) and the reference-shaped fallback for
// shapes the MFMA kernels do not cover. A query row is shared by D/16 lanes
// of one wave, each holding 16 of its channels (query slice and output
// accumulator in registers): a score is 16 FMAs per lane and a butterfly sum
// over the row's lanes, and every lane then has the row's full softmax state.
// Keys and values are staged through LDS in chunks of KC rows, row-major, so
// a lane reads its 16 channels of a key as four 16-byte reads (the lanes of
// one row read one contiguous row, the rows of a wave read the same one).
// Softmax is online (running max and sum per row, exp2 with the scale folded
// in), with one rescale of the accumulator per chunk. Sixteen channels per
// lane keep the registers few and a workgroup at four waves even for short
// problems, which are latency-bound.
#include "internal.h"

#include <math.h>

namespace monarch {
namespace {

constexpr int KC = 32;    // keys per LDS chunk
constexpr int PART = 16;  // channels per lane

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, ElemType t) {
  if (t == kF32) return static_cast<const float*>(base)[idx];
  return static_cast<float>(static_cast<const __bf16*>(base)[idx]);
}

__device__ __forceinline__ void store_elem(void* base, int64_t idx, float x, ElemType t) {
  if (t == kF32)
    static_cast<float*>(base)[idx] = x;
  else
    static_cast<__bf16*>(base)[idx] = static_cast<__bf16>(x);
}

// sum of x over the SPLIT consecutive lanes of one row (SPLIT a power of two <= 8)
template <int SPLIT>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = SPLIT / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, SPLIT);
  return x;
}

template <int D>
__global__ void __launch_bounds__(256) generic_kernel(GroupedArgs a, int rows_per_wg, int chunks) {
  constexpr int SPLIT = D / PART;
  __shared__ __attribute__((aligned(16))) float ks[KC][D];
  __shared__ __attribute__((aligned(16))) float vs[KC][D];

  const int64_t wg = blockIdx.x;
  const int chunk = static_cast<int>(wg % chunks);
  const int64_t rest = wg / chunks;
  const int p = static_cast<int>(rest % a.problems);
  const int h = static_cast<int>(rest / a.problems);

  const int64_t head_off = static_cast<int64_t>(h) * a.head_elems;
  const int64_t base = static_cast<int64_t>(p / a.inner) * a.outer + (p % a.inner);

  const int tid = threadIdx.x;
  const int part = tid % SPLIT;
  const int qr0 = chunk * rows_per_wg + tid / SPLIT;  // within the query rows
  const int row = a.q_row0 + qr0;
  const bool row_ok = (tid / SPLIT) < rows_per_wg && qr0 < a.Lq;

  float qr[PART];
  float acc[PART];
  const int64_t qrow = head_off + (base + static_cast<int64_t>(row_ok ? row : 0) * a.row_stride) * D;
#pragma unroll
  for (int e = 0; e < PART; ++e) {
    qr[e] = row_ok ? load_elem(a.q, qrow + part * PART + e, a.qk_type) * a.scale_log2 : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f, wsum = 0.f;
  const int64_t rows_off = static_cast<int64_t>(h) * (a.head_elems / D);
  const float* kb = a.kbias ? a.kbias + rows_off + base : nullptr;

  for (int k0 = 0; k0 < a.L; k0 += KC) {
    const int nk = min(KC, a.L - k0);
    __syncthreads();
    for (int idx = tid; idx < KC * D; idx += blockDim.x) {
      const int key = idx / D, e = idx % D;
      float kv = 0.f, vv = 0.f;
      if (key < nk) {
        const int64_t g = head_off + (base + static_cast<int64_t>(k0 + key) * a.row_stride) * D + e;
        kv = load_elem(a.k, g, a.qk_type);
        vv = load_elem(a.v, g, a.v_type);
      }
      ks[key][e] = kv;
      vs[key][e] = vv;
    }
    __syncthreads();

    float sc[KC];
    float cmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const float4* kr = reinterpret_cast<const float4*>(&ks[j][part * PART]);
      float s = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < PART / 4; ++c4) {
        const float4 k4 = kr[c4];
        s = fmaf(qr[4 * c4 + 0], k4.x, s);
        s = fmaf(qr[4 * c4 + 1], k4.y, s);
        s = fmaf(qr[4 * c4 + 2], k4.z, s);
        s = fmaf(qr[4 * c4 + 3], k4.w, s);
      }
      s = row_sum<SPLIT>(s);
      if (kb && j < nk) s += kb[static_cast<int64_t>(k0 + j) * a.row_stride];
      sc[j] = (j < nk) ? s : -INFINITY;
      cmax = fmaxf(cmax, sc[j]);
    }
    const float m_new = fmaxf(m, cmax);
    const float alpha = exp2f(m - m_new);
    // wsum: sum of p * (logit - running max) in bits, moved to the new maximum
    wsum = l > 0.f ? alpha * fmaf(m - m_new, l, wsum) : 0.f;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < PART; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const float z = sc[j] - m_new;
      const float pj = exp2f(z);
      l += pj;
      if (pj > 0.f) wsum = fmaf(pj, z, wsum);
      const float4* vr = reinterpret_cast<const float4*>(&vs[j][part * PART]);
#pragma unroll
      for (int c4 = 0; c4 < PART / 4; ++c4) {
        const float4 v4 = vr[c4];
        acc[4 * c4 + 0] = fmaf(pj, v4.x, acc[4 * c4 + 0]);
        acc[4 * c4 + 1] = fmaf(pj, v4.y, acc[4 * c4 + 1]);
        acc[4 * c4 + 2] = fmaf(pj, v4.z, acc[4 * c4 + 2]);
        acc[4 * c4 + 3] = fmaf(pj, v4.w, acc[4 * c4 + 3]);
      }
    }
    m = m_new;
  }

  if (row_ok) {
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < PART; ++e) store_elem(a.o, qrow + part * PART + e, acc[e] * inv, a.o_type);
    if (a.ent && part == 0)
      a.ent[rows_off + base + static_cast<int64_t>(row) * a.row_stride] = log2f(l) - wsum * inv;
  }
}

}  // namespace

hipError_t launch_generic(const GroupedArgs& a, hipStream_t stream) {
  const int split = a.D / PART;
  int threads = 256;
  const int need = a.Lq * split;
  if (need < threads) threads = ((need + 63) / 64) * 64;
  const int rows_per_wg = threads / split;
  const int chunks = (a.Lq + rows_per_wg - 1) / rows_per_wg;
  const int64_t grid = static_cast<int64_t>(chunks) * a.problems * a.heads;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.D == 64)
    hipLaunchKernelGGL(generic_kernel<64>, dim3(static_cast<unsigned>(grid)), dim3(threads), 0, stream,
                       a, rows_per_wg, chunks);
  else if (a.D == 128)
    hipLaunchKernelGGL(generic_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(threads), 0, stream,
                       a, rows_per_wg, chunks);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace monarch
