// Plain grouped-attention kernel: fp32 VALU arithmetic, any problem length.
//
// This is the fp32 path (fp32 products keep the 1e-5 bound that reduced-
// precision matrix cores would break) and the reference-shaped fallback for
// shapes the MFMA kernels do not cover. One thread holds 64 of the D
// channels of one query row (D/64 threads per row) with its output
// accumulator in registers; keys and values are staged through LDS in chunks
// of KC rows, converted to fp32. Softmax is online (running max and sum per
// row, exp2 with the scale folded in), with one rescale of the accumulator per
// chunk.
#include "internal.h"

#include <math.h>

namespace monarch {
namespace {

constexpr int KC = 32;          // keys per LDS chunk
constexpr int PART = 64;        // channels per thread
constexpr int PSTRIDE = PART + 1;

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

template <int D>
__global__ void __launch_bounds__(256) generic_kernel(GroupedArgs a, int rows_per_wg, int chunks) {
  constexpr int SPLIT = D / PART;
  // [part][key][PSTRIDE]: the two halves of a row sit 32 banks apart
  __shared__ float ks[SPLIT][KC][PSTRIDE];
  __shared__ float vs[SPLIT][KC][PSTRIDE];

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
      ks[e / PART][key][e % PART] = kv;
      vs[e / PART][key][e % PART] = vv;
    }
    __syncthreads();

    float sc[KC];
    float cmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < PART; ++e) s = fmaf(qr[e], ks[part][j][e], s);
      if (SPLIT == 2) s += __shfl_xor(s, 1);
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
#pragma unroll
      for (int e = 0; e < PART; ++e) acc[e] = fmaf(pj, vs[part][j][e], acc[e]);
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
