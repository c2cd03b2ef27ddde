// Hardware probes behind the flash kernel's design: in-kernel cycle counts
// (s_memtime, the shader clock) of
//   (1) the 32x32x16 bf16 MFMA issue interval: one dependent chain or two or
//       four independent chains, one or two waves per SIMD;
//   (2) LDS read bandwidth of 16-byte reads (swizzled, conflict free) and of
//       the transposing 8-byte reads, alone and feeding MFMAs, at 4 and 8
//       waves per CU;
//   (3) VALU throughput (FMA, exp2) and its co-issue with MFMAs.
// A standalone program (python tests/hip/build.py builds it): each probe runs
// 256 workgroups three times and prints per-wave averages. Figures are
// cycles of the shader clock, whatever frequency it runs at.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---------------------------------------------------------------- (1) MFMA issue
// MFMA 32x32x16 bf16 issue rate per wave, dependent chain vs independent chains,
// one or two waves per SIMD. Output per wave: cycles (s_memtime) and 100 MHz ticks.

template <int MODE>
__global__ void __launch_bounds__(512) mfma_probe(float* out, uint64_t* times, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) { a[e] = (__bf16)(0.001f * (lane + e)); b[e] = (__bf16)(0.002f * (lane - e)); }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if (MODE == 0) {  // one dependent chain of 8
#pragma unroll
      for (int k = 0; k < 8; ++k) c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    } else if (MODE == 1) {  // four independent chains, 8 MFMAs
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      }
    } else {  // two chains
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      }
    }
  }
  // wait for the results before the closing timestamps
  float s = 0.f;
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  asm volatile("" :: "v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;
  out[gw * 64 + lane] = s;
  if (lane == 0) { times[2 * gw] = t1 - t0; times[2 * gw + 1] = r1 - r0; }
}

static int run_mfma() {
  const int iters = 4096;
  for (int mode = 0; mode < 3; ++mode)
    for (int waves = 4; waves <= 8; waves += 4) {
      const int wgs = 256;
      const int nw = wgs * waves;
      float* out; uint64_t* times;
      if (hipMalloc(&out, sizeof(float) * nw * 64) != hipSuccess) return 1;
      if (hipMalloc(&times, sizeof(uint64_t) * 2 * nw) != hipSuccess) return 1;
      dim3 g(wgs), blk(64 * waves);
      for (int rep = 0; rep < 3; ++rep) {
        if (mode == 0) hipLaunchKernelGGL(mfma_probe<0>, g, blk, 0, 0, out, times, iters);
        if (mode == 1) hipLaunchKernelGGL(mfma_probe<1>, g, blk, 0, 0, out, times, iters);
        if (mode == 2) hipLaunchKernelGGL(mfma_probe<2>, g, blk, 0, 0, out, times, iters);
      }
      if (hipDeviceSynchronize() != hipSuccess) return 2;
      uint64_t* h = (uint64_t*)malloc(sizeof(uint64_t) * 2 * nw);
      if (hipMemcpy(h, times, sizeof(uint64_t) * 2 * nw, hipMemcpyDeviceToHost) != hipSuccess) return 3;
      double cyc = 0, rt = 0;
      for (int i = 0; i < nw; ++i) { cyc += h[2 * i]; rt += h[2 * i + 1]; }
      cyc /= nw; rt /= nw;
      const double mfmas = 8.0 * iters;
      printf("mode %d (%s) waves/WG %d: %.1f memtime/MFMA, %.1f ns/MFMA (100 MHz clock), memtime rate %.2f GHz\n",
             mode, mode == 0 ? "1 chain" : mode == 1 ? "4 chains" : "2 chains", waves, cyc / mfmas,
             rt * 10.0 / mfmas, cyc / (rt * 10.0));
      free(h);
      if (hipFree(out) != hipSuccess || hipFree(times) != hipSuccess) return 4;
    }
  return 0;
}

// ---------------------------------------------------------------- (2) LDS reads
// LDS read bandwidth alone and MFMA rate when each MFMA (or each pair) takes
// its A operand from LDS, 8 waves per CU (2 per SIMD).

template <int MODE>
__global__ void __launch_bounds__(512) lds_probe(float* out, uint64_t* times, int iters) {
  __shared__ __attribute__((aligned(1024))) char lds[64 * 1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 64 * 1024 / 4; i += blockDim.x) reinterpret_cast<float*>(lds)[i] = 0.001f * (i & 255);
  __syncthreads();
  // lane reads 16 B at row lane%32 (256 B rows), chunk 2*k + lane/32 with a 4-bit swizzle: conflict free
  const int r = lane & 31, h = lane >> 5;
  const int swz = ((r & 3) << 2) | ((r >> 2) & 3);
  uint32_t off[8];
  for (int k = 0; k < 8; ++k) off[k] = r * 256 + 16 * ((2 * k + h) ^ swz) + (wave & 1) * 8192;
  bf16x8 b;
  for (int e = 0; e < 8; ++e) b[e] = (__bf16)(0.002f * (lane - e));
  f32x16 c0 = {}, c1 = {};
  float acc = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    const char* base = lds + (it & 3) * 16384;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + off[k]);
      if (MODE == 0) {  // LDS reads only
        acc += (float)a[0] + (float)a[7];
      } else if (MODE == 1) {  // one MFMA per LDS read
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      } else if (MODE == 2) {  // two MFMAs per LDS read
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      }
    }
  }
  float s = acc;
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e];
  asm volatile("" :: "v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;
  out[gw * 64 + lane] = s;
  if (lane == 0) times[gw] = t1 - t0;
}

template <int MODE>
__global__ void __launch_bounds__(512) lds_probe_tr(float* out, uint64_t* times, int iters) {
  __shared__ __attribute__((aligned(1024))) char lds[64 * 1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 64 * 1024 / 4; i += blockDim.x) reinterpret_cast<float*>(lds)[i] = 0.001f * (i & 255);
  __syncthreads();
  const int j = lane & 15, g = lane >> 4;
  uint32_t off[4][2];
  for (int mt = 0; mt < 4; ++mt)
    for (int sec = 0; sec < 2; ++sec) {
      const int row = 4 * (g >> 1) + (j >> 2) + 8 * sec;
      const int ch = 32 * mt + 16 * (g & 1) + 4 * (j & 3);
      const int swz = ((row & 3) << 2) | ((row >> 2) & 3);
      off[mt][sec] = row * 256 + 16 * ((ch / 8) ^ swz) + (ch % 8) * 2;
    }
  bf16x8 b;
  for (int e = 0; e < 8; ++e) b[e] = (__bf16)(0.002f * (lane - e));
  f32x16 c[4] = {};
  float acc = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    const char* base = lds + (it & 3) * 16384 + (it & 1) * 4096;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + st * 4096 + off[mt][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + st * 4096 + off[mt][1]));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        if (MODE == 0) acc += (float)a[0] + (float)a[7];
        else c[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[mt], 0, 0, 0);
      }
  }
  float s = acc;
  for (int mt = 0; mt < 4; ++mt) for (int e = 0; e < 16; ++e) s += c[mt][e];
  asm volatile("" :: "v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;
  out[gw * 64 + lane] = s;
  if (lane == 0) times[gw] = t1 - t0;
}

static int run_lds() {
  const int iters = 2048, wgs = 256;
  const char* names[] = {"b128 reads only", "b128 read + 1 MFMA", "b128 read + 2 MFMA", "tr reads only", "tr reads + 1 MFMA per 2 reads"};
  for (int waves = 4; waves <= 8; waves += 4)
    for (int mode = 0; mode < 5; ++mode) {
      const int nw = wgs * waves;
      float* out; uint64_t* times;
      if (hipMalloc(&out, sizeof(float) * nw * 64) != hipSuccess) return 1;
      if (hipMalloc(&times, sizeof(uint64_t) * nw) != hipSuccess) return 1;
      for (int rep = 0; rep < 3; ++rep) {
        dim3 g(wgs), blk(64 * waves);
        switch (mode) {
          case 0: hipLaunchKernelGGL(lds_probe<0>, g, blk, 0, 0, out, times, iters); break;
          case 1: hipLaunchKernelGGL(lds_probe<1>, g, blk, 0, 0, out, times, iters); break;
          case 2: hipLaunchKernelGGL(lds_probe<2>, g, blk, 0, 0, out, times, iters); break;
          case 3: hipLaunchKernelGGL(lds_probe_tr<0>, g, blk, 0, 0, out, times, iters); break;
          case 4: hipLaunchKernelGGL(lds_probe_tr<1>, g, blk, 0, 0, out, times, iters); break;
        }
      }
      if (hipDeviceSynchronize() != hipSuccess) return 2;
      uint64_t* h = (uint64_t*)malloc(sizeof(uint64_t) * nw);
      if (hipMemcpy(h, times, sizeof(uint64_t) * nw, hipMemcpyDeviceToHost) != hipSuccess) return 3;
      double cyc = 0;
      for (int i = 0; i < nw; ++i) cyc += h[i];
      cyc /= nw;
      const double reads = (mode < 3 ? 8.0 : 16.0) * iters;        // LDS instructions per wave
      const double bytes = (mode < 3 ? 1024.0 : 512.0) * reads;    // per wave
      const double mfma = mode == 1 ? 8.0 * iters : mode == 2 ? 16.0 * iters : mode == 4 ? 8.0 * iters : 0;
      printf("waves/CU %d %-30s: LDS %.0f B/clk/CU", waves, names[mode], bytes * waves / cyc);
      if (mfma > 0) printf(", %.1f cycles per MFMA per SIMD", cyc / (mfma * waves / 4));
      printf("\n");
      free(h);
      if (hipFree(out) != hipSuccess || hipFree(times) != hipSuccess) return 4;
    }
  return 0;
}

// ---------------------------------------------------------------- (3) VALU and MFMA
// VALU throughput (fma, exp) per SIMD and its co-execution with MFMA.

// MODE 0: fma only; 1: exp only; 2: waves of even index MFMA-only, odd VALU(fma)-only;
// 3: every wave 1 MFMA + 4 fma interleaved; 4: every wave 1 MFMA + 8 fma; 5: 1 MFMA + 4 exp
template <int MODE>
__global__ void __launch_bounds__(512) valu_probe(float* out, uint64_t* times, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = 0.001f * (lane + i);
  const float y = 0.999f, z = 0.0001f;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) { a[e] = (__bf16)(0.001f * (lane + e)); b[e] = (__bf16)(0.002f * (lane - e)); }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const bool mf = (MODE != 2) || ((wave >> 2) & 1) == 0;   // wave w and w+4 share a SIMD
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    if (MODE == 0 || (MODE == 2 && !mf)) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], y, z);
    } else if (MODE == 1) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) * y;
    } else if (MODE == 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
      }
    } else {
      constexpr int NV = MODE == 4 ? 8 : 4;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          if (MODE == 5) x[i] = __builtin_amdgcn_exp2f(x[i]);
          else x[i] = fmaf(x[i], y, z);
        }
      }
    }
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  asm volatile("" :: "v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;
  out[gw * 64 + lane] = s;
  if (lane == 0) times[gw] = t1 - t0;
}

static int run_valu() {
  const int iters = 2048, wgs = 256, waves = 8;
  const char* names[] = {"fma only", "exp(+mul) only", "MFMA waves + fma waves", "1 MFMA + 4 fma per wave",
                         "1 MFMA + 8 fma per wave", "1 MFMA + 4 exp per wave"};
  for (int mode = 0; mode < 6; ++mode) {
    const int nw = wgs * waves;
    float* out; uint64_t* times;
    if (hipMalloc(&out, sizeof(float) * nw * 64) != hipSuccess) return 1;
    if (hipMalloc(&times, sizeof(uint64_t) * nw) != hipSuccess) return 1;
    for (int rep = 0; rep < 3; ++rep) {
      dim3 g(wgs), blk(64 * waves);
      switch (mode) {
        case 0: hipLaunchKernelGGL(valu_probe<0>, g, blk, 0, 0, out, times, iters); break;
        case 1: hipLaunchKernelGGL(valu_probe<1>, g, blk, 0, 0, out, times, iters); break;
        case 2: hipLaunchKernelGGL(valu_probe<2>, g, blk, 0, 0, out, times, iters); break;
        case 3: hipLaunchKernelGGL(valu_probe<3>, g, blk, 0, 0, out, times, iters); break;
        case 4: hipLaunchKernelGGL(valu_probe<4>, g, blk, 0, 0, out, times, iters); break;
        case 5: hipLaunchKernelGGL(valu_probe<5>, g, blk, 0, 0, out, times, iters); break;
      }
    }
    if (hipDeviceSynchronize() != hipSuccess) return 2;
    uint64_t* h = (uint64_t*)malloc(sizeof(uint64_t) * nw);
    if (hipMemcpy(h, times, sizeof(uint64_t) * nw, hipMemcpyDeviceToHost) != hipSuccess) return 3;
    double c_m = 0, c_v = 0; int n_m = 0, n_v = 0;
    for (int i = 0; i < nw; ++i) {
      const int w = i % waves;
      if (mode == 2 && ((w >> 2) & 1)) { c_v += h[i]; ++n_v; } else { c_m += h[i]; ++n_m; }
    }
    c_m /= (n_m ? n_m : 1); c_v /= (n_v ? n_v : 1);
    if (mode == 0) printf("%-26s: %.2f cycles per VALU instruction per wave (2 waves/SIMD)\n", names[mode], c_m / (32.0 * iters));
    if (mode == 1) printf("%-26s: %.2f cycles per exp+mul pair per wave (2 waves/SIMD)\n", names[mode], c_m / (32.0 * iters));
    if (mode == 2) printf("%-26s: MFMA wave %.1f cycles/MFMA; fma wave %.2f cycles/fma\n", names[mode], c_m / (8.0 * iters), c_v / (32.0 * iters));
    if (mode >= 3) printf("%-26s: %.1f cycles per MFMA step per wave (2 waves/SIMD)\n", names[mode], c_m / (8.0 * iters));
    free(h);
    if (hipFree(out) != hipSuccess || hipFree(times) != hipSuccess) return 4;
  }
  return 0;
}

int main() {
  int rc = run_mfma();
  if (rc == 0) rc = run_lds();
  if (rc == 0) rc = run_valu();
  printf("probes done (status %d)\n", rc);
  return rc;
}
