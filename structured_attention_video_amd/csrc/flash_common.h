// Device pieces shared by the flash-style kernels (forward and backward):
// problem geometry, XCD-aware ordering, the swizzled LDS tile layout, the
// asynchronous global -> LDS copy and the MFMA operand reads from LDS tiles.
// See mfma_common.h for the matrix-core register layouts.
#pragma once
#include "mfma_common.h"

namespace monarch {
namespace {

using namespace mfma;

constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ int64_t problem_base(const GroupedArgs& a, int p) {
  return static_cast<int64_t>(p / a.inner) * a.outer + (p % a.inner);
}

// Map the hardware workgroup id to a logical id so that consecutive logical
// ids run on the same XCD (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_order(int w, int nwg) {
  const int q = nwg >> 3, r = nwg & 7, x = w & 7, slot = w >> 3;
  return x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

// ---------------------------------------------------------------- flash
constexpr int FBM = 128;  // query rows per four-wave workgroup
constexpr int FBN = 64;   // keys per LDS tile
constexpr int FNT = 256;  // threads of a four-wave workgroup

// LDS tiles of the flash kernel: 64 rows x D channels, rows unpadded, the
// 16-byte chunks of row r permuted by c -> c ^ swz(r). Tiles are filled by
// buffer loads that write LDS directly (64 lanes x 16 bytes = one contiguous
// kilobyte per instruction; lane i fetches the global chunk that belongs in
// slot i). The swizzle keeps every 16-lane phase of the 16-byte K reads and
// every 32-lane phase of the transposing V reads on distinct banks: a
// transposing read touches rows 4q..4q+3 of one 16-row step, and the low two
// row bits pick the high chunk bits (D = 128, 16 chunks: a 4x4 bit transpose
// of r mod 16; D = 64, 8 chunks, two rows per 256-byte bank line: row bit 1
// picks the top chunk bit). The previous choice, which XORed 2r into the
// chunk index, left pairs of those rows on one bank group and doubled the
// transposing reads' LDS cycles (measured with SQ_LDS_BANK_CONFLICT).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// byte offset of 16-byte chunk c of row r in a swizzled tile of unpadded rows
template <int D>
__device__ __forceinline__ int swoff(int r, int c) {
  return r * D * 2 + 16 * (c ^ swz<D>(r));
}

template <int D>
struct SwTile {
  static constexpr int ROWB = D * 2;          // bytes per row
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int bytes = FBN * ROWB;    // one tile
  static constexpr int RPI = 1024 / ROWB;     // rows per load instruction
  static constexpr int IPW = FBN / 4 / RPI;   // load instructions per wave per tile
  static constexpr int total = 4 * bytes;     // two-slot rings for K and V
};

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer straight into LDS (lane i -> lds + 16*i).
// Only the device pass sees the builtin: instantiating it in the host pass
// silently drops the host launch stub of the kernel that uses it, and device
// functions never run on the host.
template <int POLICY = 0>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t src, char* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)lds, 16, voff, 0, 0, POLICY);
#else
  (void)src; (void)lds; (void)voff;
#endif
}


// Per-lane byte offsets: DMA source chunks (tile 0) and LDS read addresses.
template <int D>
struct FlashOffsets {
  using T = SwTile<D>;
  uint32_t src_off[T::IPW];  // global, relative to the tile's first row
  uint32_t k[D / 16];     // K read, k-step ks, rows 0..31 (+32 rows = +32*ROWB)
  uint32_t v[D / 32][2];  // V^T reads, channel tile mt, keys +0..3 / +8..11 (+16*step rows)
  __device__ __forceinline__ FlashOffsets(int wave, int lane, int64_t rs) {
#pragma unroll
    for (int i = 0; i < T::IPW; ++i) {
      const int row = 16 * wave + T::RPI * i + lane / T::CPR;
      const int c = (lane % T::CPR) ^ swz<D>(row);
      src_off[i] = static_cast<uint32_t>((row * rs * D + c * 8) * 2);
    }
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) k[ks] = r * T::ROWB + 16 * ((2 * ks + h) ^ swz<D>(r));
    const int j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int row = 4 * (g >> 1) + (j >> 2) + 8 * sec;
        const int ch = 32 * mt + 16 * (g & 1) + 4 * (j & 3);
        v[mt][sec] = row * T::ROWB + 16 * ((ch / 8) ^ swz<D>(row)) + (ch % 8) * 2;
      }
  }
  // Issue this wave's share (16 rows) of one tile's global -> LDS copy.
  __device__ __forceinline__ void dma(char* tile, __amdgpu_buffer_rsrc_t src, uint32_t tile_off, int wave) const {
#pragma unroll
    for (int i = 0; i < T::IPW; ++i)
      lds_dma16(src, tile + (16 * wave + T::RPI * i) * T::ROWB, src_off[i] + tile_off);
  }
};

// One wave's share of a 64-row tile copy when NW waves split it: rows
// RW*wave .. +RW, 16 bytes per lane per instruction (the same slot mapping
// as FlashOffsets::dma, which is the NW = 4 case).
template <int D, int NW>
struct TileDma {
  using T = SwTile<D>;
  static constexpr int RW = FBN / NW;      // rows per wave
  static constexpr int IPW = RW / T::RPI;  // copy instructions per wave per tile
  static_assert(IPW >= 1 && RW % T::RPI == 0, "tile rows must split evenly over the waves");
  uint32_t src_off[IPW];  // global, relative to the tile's first row
  __device__ __forceinline__ TileDma(int wave, int lane, int64_t rs) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int row = RW * wave + T::RPI * i + lane / T::CPR;
      const int c = (lane % T::CPR) ^ swz<D>(row);
      src_off[i] = static_cast<uint32_t>((row * rs * D + c * 8) * 2);
    }
  }
  // copy instruction i of this wave's share alone
  __device__ __forceinline__ void dma1(char* tile, __amdgpu_buffer_rsrc_t src, uint32_t tile_off, int wave,
                                       int i) const {
    lds_dma16(src, tile + (RW * wave + T::RPI * i) * T::ROWB, src_off[i] + tile_off);
  }
  __device__ __forceinline__ void dma(char* tile, __amdgpu_buffer_rsrc_t src, uint32_t tile_off, int wave) const {
#pragma unroll
    for (int i = 0; i < IPW; ++i) lds_dma16(src, tile + (RW * wave + T::RPI * i) * T::ROWB, src_off[i] + tile_off);
  }
};

// wait for this wave's outstanding global -> LDS copies
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ __forceinline__ void mask_tail(f32x16 (&s)[2], int nvalid, int h) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (32 * t + acc_key(i, h) >= nvalid) s[t][i] = -INFINITY;
}

template <int D>
__device__ __forceinline__ bf16x8 k_operand(const char* kl, const FlashOffsets<D>& fo, int ks, int t) {
  return ld_bf16x8(kl + fo.k[ks] + t * 32 * SwTile<D>::ROWB);
}

template <int D>
__device__ __forceinline__ bf16x8 v_operand(const char* vl, const FlashOffsets<D>& fo, int mt, int st) {
  const char* base = vl + st * 16 * SwTile<D>::ROWB;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + fo.v[mt][0]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + fo.v[mt][1]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S^T for a 64-key tile (two independent 32-key accumulator chains)
// ---------------------------------------------------------------- staged row stores
// One wave stores its 32 rows of x^T accumulators (lane: row lane % 32,
// channels 32 mt + 8 (i / 4) + 4 h + i % 4), scaled by mul, as whole rows
// through LDS: written into the wave's dead tiles, read back 16 bytes per lane
// (fp32 rows: two or four per instruction; bf16 rows: four or eight), stored
// with one instruction per 1 KB. fp32 rows go to t0 (rows 0..15) and t1
// (rows 16..31), 16-byte chunk c of row r at c ^ (r % 16); bf16 rows to t0
// in the tile swizzle. Rows past the problem's end are dropped by ro.
template <int D, bool F32>
__device__ __forceinline__ void stage_rows(char* t0, char* t1, const f32x16 (&x)[D / 32], float mul,
                                           __amdgpu_buffer_rsrc_t ro, int64_t rs, int lane) {
  const int h = lane >> 5;
  int r = lane & 31;
  asm volatile("" : "+v"(r));
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): earlier reads of the tiles are done
  __builtin_amdgcn_wave_barrier();
  if constexpr (F32) {
    constexpr int RB = D * 4, CH = D / 4, RPI = 64 / CH;
    char* t = r < 16 ? t0 : t1;
    const int rr = r & 15;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 v = {__float_as_uint(x[mt][4 * g] * mul), __float_as_uint(x[mt][4 * g + 1] * mul),
                         __float_as_uint(x[mt][4 * g + 2] * mul), __float_as_uint(x[mt][4 * g + 3] * mul)};
        *reinterpret_cast<u32x4*>(t + rr * RB + 16 * ((8 * mt + 2 * g + h) ^ rr)) = v;
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    const uint32_t row_bytes = static_cast<uint32_t>(rs * D * 4);
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + lane / CH, chk = lane % CH;
      const char* tr = row < 16 ? t0 : t1;
      const u32x4 v = *reinterpret_cast<const u32x4*>(tr + (row & 15) * RB + 16 * (chk ^ (row & 15)));
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, static_cast<int>(row * row_bytes + chk * 16), 0, 0);
    }
  } else {
    constexpr int CPR = D / 8, RPI = 64 / CPR;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(x[mt][4 * g + e] * mul);
        *reinterpret_cast<bf16x4*>(t0 + swoff<D>(r, 4 * mt + g) + 8 * h) = v;
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    const uint32_t row_bytes = static_cast<uint32_t>(rs * D * 2);
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + lane / CPR, chk = lane % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(t0 + swoff<D>(row, chk));
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, static_cast<int>(row * row_bytes + chk * 16), 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // the read-backs are done before the tiles are reused
  __builtin_amdgcn_wave_barrier();
}

// As stage_rows for fp32 rows, but the stored rows are bf16 and, when
// has_add, the fp32 rows of ra are added before the rounding (one rounding
// of the sum): rows are staged in fp32, read back 16 bytes (4 channels) per
// lane, the matching 16 bytes of ra loaded (consecutive lanes, consecutive
// bytes), and 8 bytes per lane stored.
template <int D>
__device__ __forceinline__ void stage_rows_add(char* t0, char* t1, const f32x16 (&x)[D / 32], float mul,
                                               __amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t ra, bool has_add,
                                               int64_t rs, int lane) {
  constexpr int RB = D * 4, CH = D / 4, RPI = 64 / CH;
  const int h = lane >> 5;
  int r = lane & 31;
  asm volatile("" : "+v"(r));
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): earlier reads of the tiles are done
  __builtin_amdgcn_wave_barrier();
  char* t = r < 16 ? t0 : t1;
  const int rr = r & 15;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4 v = {__float_as_uint(x[mt][4 * g] * mul), __float_as_uint(x[mt][4 * g + 1] * mul),
                       __float_as_uint(x[mt][4 * g + 2] * mul), __float_as_uint(x[mt][4 * g + 3] * mul)};
      *reinterpret_cast<u32x4*>(t + rr * RB + 16 * ((8 * mt + 2 * g + h) ^ rr)) = v;
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  const uint32_t row_el = static_cast<uint32_t>(rs * D);
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + lane / CH, chk = lane % CH;
    const char* tr = row < 16 ? t0 : t1;
    const u32x4 v = *reinterpret_cast<const u32x4*>(tr + (row & 15) * RB + 16 * (chk ^ (row & 15)));
    const uint32_t el = row * row_el + chk * 4;
    float f[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
    if (has_add) {
      const u32x4 ad = bload16(ra, el * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] += __uint_as_float(ad[e]);
    }
    bf16x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = static_cast<bf16>(f[e]);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, w), ro, static_cast<int>(el * 2), 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // the read-backs are done before the tiles are reused
  __builtin_amdgcn_wave_barrier();
}

// fp32 rows as stage_rows<D, true>, through one region of 16 rows (rows 0..15
// first, then 16..31), stored base_off bytes into ro: for a wave that has only
// half the room.
template <int D>
__device__ __forceinline__ void stage_rows_f32_halves(char* t, const f32x16 (&x)[D / 32], float mul,
                                                      __amdgpu_buffer_rsrc_t ro, int64_t rs, int lane,
                                                      uint32_t base_off) {
  constexpr int RB = D * 4, CH = D / 4, RPI = 64 / CH;
  const int h = lane >> 5;
  int r = lane & 31;
  asm volatile("" : "+v"(r));
  const int rr = r & 15;
  const uint32_t row_bytes = static_cast<uint32_t>(rs * D * 4);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // earlier reads of the region are done
    __builtin_amdgcn_wave_barrier();
    if ((r >> 4) == half) {
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 v = {__float_as_uint(x[mt][4 * g] * mul), __float_as_uint(x[mt][4 * g + 1] * mul),
                           __float_as_uint(x[mt][4 * g + 2] * mul), __float_as_uint(x[mt][4 * g + 3] * mul)};
          *reinterpret_cast<u32x4*>(t + rr * RB + 16 * ((8 * mt + 2 * g + h) ^ rr)) = v;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
      const int row = RPI * i + lane / CH, chk = lane % CH;
      const u32x4 v = *reinterpret_cast<const u32x4*>(t + row * RB + 16 * (chk ^ row));
      __builtin_amdgcn_raw_buffer_store_b128(
          v, ro, static_cast<int>(base_off + (16 * half + row) * row_bytes + chk * 16), 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // the read-backs are done before the region is reused
  __builtin_amdgcn_wave_barrier();
}

}  // namespace
}  // namespace monarch
