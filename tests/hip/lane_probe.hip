// Lane-layout probe: one wave64 runs one cross-lane or matrix-core operation
// of the kind the library's MFMA kernels use, on inputs given per lane, and
// writes every lane's result. A GPU test compares the results with the CPU
// wave model of the tests (wave64.py), which the CPU lane-mapping tests use.
//
// Every entry point takes device pointers and a stream, launches one
// 64-thread workgroup and returns the launch status (0 = success). Sizes:
//   swap:     x, y [64] u32 -> out [2][64] u32 (the builtin's results 0, 1)
//   bpermute: addr, data [64] i32 -> out [64] i32
//   tr16:     init [4096] u16 (the 8 KiB LDS array), addr [64] i32 byte
//             addresses (taken modulo 8 KiB, rounded down to 8 bytes) ->
//             out [64][4] u16
//   mfma:     a, b [64][8] bf16 bits, c [64][16] f32 -> d [64][16] f32
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kLdsBytes = 8192;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__global__ void __launch_bounds__(64) swap_kernel(const uint32_t* x, const uint32_t* y, uint32_t* out) {
  const int l = threadIdx.x;
  auto r = __builtin_amdgcn_permlane32_swap(x[l], y[l], false, false);
  out[l] = r[0];
  out[64 + l] = r[1];
}

__global__ void __launch_bounds__(64) bpermute_kernel(const int* addr, const int* data, int* out) {
  const int l = threadIdx.x;
  out[l] = __builtin_amdgcn_ds_bpermute(addr[l], data[l]);
}

__global__ void __launch_bounds__(64) tr16_kernel(const uint16_t* init, const int* addr, uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsBytes / 2];
  const int l = threadIdx.x;
  for (int i = l; i < kLdsBytes / 2; i += 64) lds[i] = init[i];
  __syncthreads();
  const int a = addr[l] & (kLdsBytes - 8);
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(reinterpret_cast<char*>(lds) + a));
  for (int e = 0; e < 4; ++e) out[4 * l + e] = static_cast<uint16_t>(v[e]);
}

__global__ void __launch_bounds__(64) mfma_kernel(const uint16_t* a, const uint16_t* b, const float* c, float* d) {
  const int l = threadIdx.x;
  bf16x8 av, bv;
  f32x16 cv;
  for (int e = 0; e < 8; ++e) {
    av[e] = __builtin_bit_cast(__bf16, a[8 * l + e]);
    bv[e] = __builtin_bit_cast(__bf16, b[8 * l + e]);
  }
  for (int i = 0; i < 16; ++i) cv[i] = c[16 * l + i];
  cv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, cv, 0, 0, 0);
  for (int i = 0; i < 16; ++i) d[16 * l + i] = cv[i];
}

int status(hipStream_t) { return static_cast<int>(hipGetLastError()); }

}  // namespace

extern "C" int lane_probe_swap(const void* x, const void* y, void* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(swap_kernel, dim3(1), dim3(64), 0, s, static_cast<const uint32_t*>(x),
                     static_cast<const uint32_t*>(y), static_cast<uint32_t*>(out));
  return status(s);
}

extern "C" int lane_probe_bpermute(const void* addr, const void* data, void* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(bpermute_kernel, dim3(1), dim3(64), 0, s, static_cast<const int*>(addr),
                     static_cast<const int*>(data), static_cast<int*>(out));
  return status(s);
}

extern "C" int lane_probe_tr16(const void* init, const void* addr, void* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(tr16_kernel, dim3(1), dim3(64), 0, s, static_cast<const uint16_t*>(init),
                     static_cast<const int*>(addr), static_cast<uint16_t*>(out));
  return status(s);
}

extern "C" int lane_probe_mfma(const void* a, const void* b, const void* c, void* d, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(mfma_kernel, dim3(1), dim3(64), 0, s, static_cast<const uint16_t*>(a),
                     static_cast<const uint16_t*>(b), static_cast<const float*>(c), static_cast<float*>(d));
  return status(s);
}
