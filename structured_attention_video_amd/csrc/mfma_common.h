// Device helpers shared by the bf16 MFMA grouped-attention kernels (gfx950).
//
// Matrix-core layout used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand: lane l holds A[l%32][8*(l/32) + e], e = 0..7
//   B operand: lane l holds B[8*(l/32) + e][l%32]
//   C/D:       lane l, register i holds D[8*(i/4) + 4*(l/32) + i%4][l%32]
//
// Scores are computed transposed, S^T = K Q^T (M = keys, N = queries, K = d):
// each lane then owns one query column and 16 of every 32 keys, so row max
// and row sum are in-lane reductions plus one swap between the two lane
// halves. The probabilities P^T leave the accumulator in exactly the B-operand
// layout of the second product O^T = V^T P^T, with the key order inside each
// 16-key step permuted: lane half h, element e holds key
// 8*(e/4) + 4*h + e%4. V^T is stored in LDS with the same permutation of its
// key slots, so both operands agree and no register shuffle is needed.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace monarch {
namespace mfma {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum of x over the two lanes l and l^32 (v_permlane32_swap)
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// key (0..n-1 inside a tile) -> V^T slot: inside every 16 keys the groups of
// four keys 4..7 and 8..11 trade places (an involution)
__device__ __forceinline__ int key_slot(int k) {
  const int g = (k >> 2) & 3;
  const int sg = g == 1 ? 2 : (g == 2 ? 1 : g);
  return (k & ~15) | (sg << 2) | (k & 3);
}

// key index of accumulator register i for lane half h, in a 32-key tile
__device__ __forceinline__ int acc_key(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// LDS geometry: K rows (d contiguous) and V^T rows (keys contiguous), each
// padded by 16 bytes so that 16 consecutive rows start in distinct banks.
template <int D>
struct KRow { static constexpr int bytes = D * 2 + 16; };
template <int BN>
struct VRow { static constexpr int bytes = BN * 2 + 16; };

// Interleave two packed bf16 pairs: low halves (sel 0x05040100) or high halves
// (sel 0x07060302) of lo and hi into one dword [lo.x, hi.x].
__device__ __forceinline__ uint32_t pack_lo(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// Write four keys x eight channels (four 16-byte rows r0..r3 = keys k..k+3,
// channels d0..d0+7) into V^T: eight 8-byte writes, one per channel.
template <int BN>
__device__ __forceinline__ void store_vt4(char* vt, int d0, int slot, const u32x4& r0, const u32x4& r1,
                                          const u32x4& r2, const u32x4& r3) {
  constexpr int VR = VRow<BN>::bytes;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t a0 = r0[w], a1 = r1[w], a2 = r2[w], a3 = r3[w];
    u32x2 lo, hi;
    lo[0] = pack_lo(a0, a1);
    lo[1] = pack_lo(a2, a3);
    hi[0] = pack_hi(a0, a1);
    hi[1] = pack_hi(a2, a3);
    *reinterpret_cast<u32x2*>(vt + (d0 + 2 * w) * VR + slot * 2) = lo;
    *reinterpret_cast<u32x2*>(vt + (d0 + 2 * w + 1) * VR + slot * 2) = hi;
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ bf16x8 ld_bf16x8(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

// S^T for one 32-key tile of K in LDS (rows key0..key0+31) against a wave's
// query fragment qf (B operand, one bf16x8 per 16 channels).
template <int D>
__device__ __forceinline__ f32x16 scores_tile(const char* kl, int key0, const bf16x8 (&qf)[D / 16], int lane) {
  constexpr int KR = KRow<D>::bytes;
  const char* row = kl + (key0 + (lane & 31)) * KR + (lane >> 5) * 16;
  f32x16 s = {};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) s = mma(ld_bf16x8(row + ks * 32), qf[ks], s);
  return s;
}

// O^T[32*mt .. +32) += V^T P^T over one 16-key step (slots 16*step ..)
template <int BN>
__device__ __forceinline__ f32x16 pv_step(const char* vt, int mt, int step, bf16x8 p, f32x16 o, int lane) {
  constexpr int VR = VRow<BN>::bytes;
  const char* row = vt + (32 * mt + (lane & 31)) * VR + step * 32 + (lane >> 5) * 16;
  return mma(ld_bf16x8(row), p, o);
}

// bf16 B operand for PV step `step` from probabilities held as accumulator
// tiles (registers 8*(step%2) .. +7 of tile step/2)
__device__ __forceinline__ bf16x8 p_operand(const f32x16& p, int half) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<bf16>(p[8 * half + e]);
  return r;
}

// Write one lane's share of O (query row `row`, all D channels) from O^T
// accumulators; channel of register i in tile mt is 32*mt + acc_key(i, h).
template <int D, bool OUT_F32>
__device__ __forceinline__ void store_out(void* out, int64_t row_elem, const f32x16 (&o)[D / 32], float inv,
                                          int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * mt + 8 * g + 4 * h;
      if (OUT_F32) {
        float4 v = make_float4(o[mt][4 * g] * inv, o[mt][4 * g + 1] * inv, o[mt][4 * g + 2] * inv,
                               o[mt][4 * g + 3] * inv);
        *reinterpret_cast<float4*>(static_cast<float*>(out) + row_elem + d) = v;
      } else {
        typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(o[mt][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(out) + row_elem + d) = v;
      }
    }
  }
}

}  // namespace mfma
}  // namespace monarch
