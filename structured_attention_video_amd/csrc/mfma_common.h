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
// 16-key step permuted: lane half h, element e holds key 8*(e/4) + 4*h + e%4.
// V stays row-major in LDS, like K; the V^T A operand is gathered with two
// transposing reads (ds_read_b64_tr_b16) whose source rows follow the same
// key permutation, so both operands agree and no register shuffle is needed.
//
// ds_read_b64_tr_b16 lane map (measured on gfx950): inside each group of 16
// lanes, lane i receives element i%4 of the 8-byte segment addressed by lane
// 4*e + i/4, for e = 0..3. If lane j of the group addresses row key0 + j/4 at
// channels c0 + 4*(j%4), lane i receives channel c0 + i of rows key0..key0+3.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace monarch {
namespace mfma {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

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

// key index of accumulator register i for lane half h, in a 32-key tile
__device__ __forceinline__ int acc_key(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

__device__ __forceinline__ bf16x8 ld_bf16x8(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

// ---------------------------------------------------------------- global access
// Buffer descriptor over one problem's rows: base = its first token, size =
// up to the end of its last row. Rows past the end read as zero and stores
// to them are dropped, so tails need no clamp or branch. The fields are
// wave-uniform; readfirstlane tells the compiler so (otherwise it keeps them
// in vector registers and serialises every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t problem_rsrc(const void* head, int64_t base_token, int64_t rs,
                                                               int L, int D, int esize) {
  const uint64_t addr = reinterpret_cast<uint64_t>(static_cast<const char*>(head) + base_token * D * esize);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr >> 32));
  const uint32_t bytes =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(((static_cast<int64_t>(L) - 1) * rs + 1) * D * esize));
  void* p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, static_cast<short>(0), static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}

// One 32-row query fragment as MFMA B operands: lane l reads row l%32,
// channels 16*ks + 8*(l/32) .. +8 (rows past the end read as zero).
template <int D>
__device__ __forceinline__ void load_qfrag(bf16x8 (&qf)[D / 16], __amdgpu_buffer_rsrc_t rq, int row0, int64_t rs,
                                           int lane) {
  const uint32_t off = static_cast<uint32_t>(((row0 + (lane & 31)) * rs * D + (lane >> 5) * 8) * 2);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, bload16(rq, off + ks * 32));
}

// ---------------------------------------------------------------- matrix products
// bf16 B operand for PV step `step` from probabilities held as accumulator
// tiles (registers 8*(step%2) .. +7 of tile step/2)
__device__ __forceinline__ bf16x8 p_operand(const f32x16& p, int half) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<bf16>(p[8 * half + e]);
  return r;
}

// Write one lane's share of O (query row `row` of the problem, all D
// channels) from O^T accumulators through the problem's descriptor (rows past
// the end are dropped). Channel of register i in tile mt is 32*mt + acc_key(i, h).
// Cache-policy operand of buffer instructions: SC1 (bit 4) makes an access
// coherent at device scope on gfx950 (a store is written through the
// per-XCD L2, a load does not use a possibly stale L2 line).
constexpr int kPolicyDevice = 16;

template <int D, bool OUT_F32, int POLICY = 0>
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t ro, int row, int64_t rs, const f32x16 (&o)[D / 32],
                                          float inv, int lane) {
  const int h = lane >> 5;
  const uint32_t esz = OUT_F32 ? 4 : 2;
  const uint32_t rowoff = static_cast<uint32_t>(row * rs * D) * esz;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = rowoff + (32 * mt + 8 * g + 4 * h) * esz;
      if (OUT_F32) {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(o[mt][4 * g + e] * inv);
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, static_cast<int>(off), 0, POLICY);
      } else {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(o[mt][4 * g + e] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), ro, static_cast<int>(off), 0, POLICY);
      }
    }
  }
}

}  // namespace mfma
}  // namespace monarch
