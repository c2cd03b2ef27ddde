// Grouped attention for very small problems (L <= 8 rows): the tiled Monarch
// variant's stage 2 (groups of m_tau = 3 blocks inside a tile, gist.science
// explainer section 2.B) and any block or group of a handful of tokens.
//
// Pure streaming work (per token: read Q, K, V/Y rows, write one row), so the
// kernel is built for coalescing, not arithmetic: D/8 lanes own one problem
// (8 channels each), so one problem's row is one contiguous 256-byte access
// and a wave covers the same row of 64*8/D adjacent problems (adjacent tokens
// in stage 2). Dot products are lane-partial and reduced with DPP inside a
// 16-lane row; softmax and the value sum run in fp32 on every lane.
#include "internal.h"

#include <math.h>

namespace monarch {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t tiny_base(const GroupedArgs& a, int p) {
  return static_cast<int64_t>(p / a.inner) * a.outer + (p % a.inner);
}

// 8 consecutive channels starting at element `idx` as fp32
__device__ __forceinline__ void load8(float (&x)[8], const void* base, int64_t idx, ElemType t) {
  if (t == kF32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + idx);
    const u32x4 lo = p[0], hi = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = __uint_as_float(lo[e]);
      x[4 + e] = __uint_as_float(hi[e]);
    }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(base) + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
}

__device__ __forceinline__ void store8(void* base, int64_t idx, const float (&x)[8], ElemType t) {
  if (t == kF32) {
    u32x4* p = reinterpret_cast<u32x4*>(static_cast<float*>(base) + idx);
    p[0] = u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    p[1] = u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])};
  } else {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(x[e]);
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(base) + idx) = v;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// sum over the LP lanes of one problem (LP = 8 or 16, aligned inside a DPP row)
template <int LP>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of the half row
  if (LP == 16) x += dpp<0x140>(x);  // row_mirror: the other half row
  return x;
}

template <int D, int LMAX>
__global__ void __launch_bounds__(256) tiny_kernel(GroupedArgs a, int64_t total) {
  constexpr int LP = D / 8;        // lanes per problem
  constexpr int PPB = 256 / LP;    // problems per workgroup
  const int sub = threadIdx.x % LP;
  const int64_t gp = static_cast<int64_t>(blockIdx.x) * PPB + threadIdx.x / LP;
  const bool ok = gp < total;
  const int64_t g = ok ? gp : total - 1;  // idle lanes mirror a real problem (DPP needs them active)
  const int hd = static_cast<int>(g / a.problems);
  const int p = static_cast<int>(g % a.problems);
  const int64_t head = static_cast<int64_t>(hd) * a.head_elems;
  const int64_t base = tiny_base(a, p);
  const int L = a.L;
  const int ch = sub * 8;

  float k[LMAX][8], v[LMAX][8];
#pragma unroll
  for (int r = 0; r < LMAX; ++r) {
    if (r < L) {
      const int64_t e = head + (base + r * a.row_stride) * D + ch;
      load8(k[r], a.k, e, a.qk_type);
      load8(v[r], a.v, e, a.v_type);
    }
  }
  const float c = a.scale_log2;
#pragma unroll
  for (int i = 0; i < LMAX; ++i) {
    if (i >= L) break;
    if (i < a.q_row0 || i >= a.q_row0 + a.Lq) continue;
    const int64_t row = head + (base + i * a.row_stride) * D + ch;
    float q[8];
    load8(q, a.q, row, a.qk_type);
    float s[LMAX];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < LMAX; ++j) {
      if (j < L) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(q[e], k[j][e], part);
        s[j] = group_sum<LP>(part) * c;
        if (a.kbias) s[j] += a.kbias[hd * (a.head_elems / D) + base + j * a.row_stride];
        mx = fmaxf(mx, s[j]);
      }
    }
    float sum = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < LMAX; ++j) {
      if (j < L) {
        const float w = __builtin_amdgcn_exp2f(s[j] - mx);
        sum += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(w, v[j][e], o[e]);
      }
    }
    const float inv = 1.f / sum;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv;
    if (ok) store8(a.o, row, o, a.o_type);
    if (ok && a.lse && sub == 0) a.lse[hd * (a.head_elems / D) + base + i * a.row_stride] = mx + __builtin_amdgcn_logf(sum);
  }
}

template <int D>
hipError_t launch_tiny_d(const GroupedArgs& a, hipStream_t s) {
  constexpr int PPB = 256 / (D / 8);
  const int64_t total = static_cast<int64_t>(a.problems) * a.heads;
  const int64_t grid = (total + PPB - 1) / PPB;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.L <= 4)
    hipLaunchKernelGGL((tiny_kernel<D, 4>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a, total);
  else
    hipLaunchKernelGGL((tiny_kernel<D, 8>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

}  // namespace

bool tiny_supported(const GroupedArgs& a) {
  return (a.D == 64 || a.D == 128) && a.L >= 1 && a.L <= 8 && !a.ent;
}

hipError_t launch_tiny(const GroupedArgs& a, hipStream_t s) {
  if (!tiny_supported(a)) return hipErrorInvalidValue;
  return a.D == 128 ? launch_tiny_d<128>(a, s) : launch_tiny_d<64>(a, s);
}

}  // namespace monarch
