// bf16 MFMA grouped-attention kernels for gfx950.
//
// flash: problems longer than 128 rows (stage-1 frame blocks, stage-2 groups
//   of many blocks, dense attention). A workgroup of four waves owns 128
//   query rows of one problem (32 per wave, kept as MFMA B operands in
//   registers) and streams the problem's keys and values in tiles of 64 rows
//   through double-buffered LDS: the next tile's global loads are in flight
//   while the current tile is multiplied. Softmax is online with a lazy
//   rescale: the running maximum only moves when a tile's maximum exceeds it
//   by more than 8 (log2 units), so the unnormalised weights stay <= 2^8 and
//   the accumulator is rescaled rarely. Workgroups are ordered so that the
//   query tiles of one problem land on the same XCD and share its L2.
//
// group: problems of at most 128 rows (stage-2 groups of a few blocks,
//   stage-1 row blocks). One pass: a workgroup loads whole problems (K and
//   V^T) into LDS once; each wave owns 32 query rows of one problem.
//
// The softmax follows the "SRAM reduction" design the MonarchRT pages
// describe for their kernels (gist.science explainer, section 2.C): scores
// never leave the chip and memory stays linear in N.
#include "mfma_common.h"

namespace monarch {
namespace {

using namespace mfma;

constexpr float kRescaleThreshold = 8.0f;

struct Rows {
  int64_t head_elems;
  int64_t base;   // first token of the problem
  int64_t rs;     // token stride between rows
};

__device__ __forceinline__ int64_t problem_base(const GroupedArgs& a, int p) {
  return static_cast<int64_t>(p / a.inner) * a.outer + (p % a.inner);
}

// Map the hardware workgroup id to a logical id so that consecutive logical
// ids run on the same XCD (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_order(int w, int nwg) {
  const int q = nwg >> 3, r = nwg & 7, x = w & 7, slot = w >> 3;
  return x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

// Load one 32-row query fragment (rows row0 .. row0+31, clamped to L) as
// MFMA B operands.
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[D / 16], const bf16* q, const Rows& r, int row0, int L,
                                       int lane) {
  // rows past the end are clamped to the last row; their outputs are never stored
  const int row = min(row0 + (lane & 31), L - 1);
  const bf16* src = q + (r.base + static_cast<int64_t>(row) * r.rs) * D + (lane >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(src + ks * 16));
}

// ---------------------------------------------------------------- flash
constexpr int FBM = 128;  // query rows per workgroup
constexpr int FBN = 64;   // keys per LDS tile
constexpr int FNT = 256;  // threads

// LDS: two-slot rings for K tiles and V^T tiles. Iteration j multiplies
// Q K_{j+1}^T (scores one tile ahead) and V_j^T P_j^T, while tile K_{j+2} and
// V_{j+1} are in flight from global memory into registers; they are written
// into the slots of K_j and V_{j-1}, which no wave reads any more.
template <int D>
struct FlashLds {
  static constexpr int kbytes = FBN * KRow<D>::bytes;
  static constexpr int vbytes = D * VRow<FBN>::bytes;
  static constexpr int total = 2 * kbytes + 2 * vbytes;
  static constexpr int kchunks = FBN * D / 8 / FNT;  // 16-byte K chunks per thread
  static constexpr int vunits = 16 * (D / 8);        // (4 keys x 8 channels) units per tile
};

// Global loads go through buffer descriptors that cover exactly one
// problem's rows (base = its first token, size = up to the end of its last
// row): a row past the end of the problem reads as zeros, so tail tiles need
// no clamp or branch. Keys beyond the end are masked out of the softmax and
// zero values add nothing.
// The descriptor fields are wave-uniform; readfirstlane tells the compiler so
// (otherwise it may keep them in vector registers and serialise each load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t problem_rsrc(const bf16* head, const Rows& r, int L, int D) {
  const uint64_t addr = reinterpret_cast<uint64_t>(head + r.base * D);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr >> 32));
  const uint32_t bytes = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(((static_cast<int64_t>(L) - 1) * r.rs + 1) * D * 2));
  void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(off), 0, 0));
}

// Per-thread byte offsets of the 16-byte K chunks inside a tile (tile 0)
template <int D>
struct KOffsets {
  uint32_t off[FlashLds<D>::kchunks];
  __device__ __forceinline__ KOffsets(int tid, int64_t rs) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int c = 0; c < FlashLds<D>::kchunks; ++c) {
      const int id = tid + FNT * c;
      off[c] = static_cast<uint32_t>(((id / CPR) * rs * D + (id % CPR) * 8) * 2);
    }
  }
};

template <int D>
__device__ __forceinline__ void load_k(u32x4 (&g)[FlashLds<D>::kchunks], __amdgpu_buffer_rsrc_t rk,
                                       const KOffsets<D>& ko, uint32_t tile_off) {
#pragma unroll
  for (int c = 0; c < FlashLds<D>::kchunks; ++c) g[c] = bload16(rk, ko.off[c] + tile_off);
}

template <int D>
__device__ __forceinline__ void store_k(char* kl, const u32x4 (&g)[FlashLds<D>::kchunks], int tid) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int c = 0; c < FlashLds<D>::kchunks; ++c) {
    const int id = tid + FNT * c;
    *reinterpret_cast<u32x4*>(kl + (id / CPR) * KRow<D>::bytes + (id % CPR) * 16) = g[c];
  }
}

// V: thread (kg, dc) loads keys 4kg..4kg+3, channels 8dc..8dc+7
template <int D>
__device__ __forceinline__ uint32_t v_offset(int tid, int64_t rs) {
  const int kg = tid & 15, dc = tid >> 4;
  return static_cast<uint32_t>((4 * kg * rs * D + dc * 8) * 2);
}

template <int D>
__device__ __forceinline__ void load_v(u32x4 (&g)[4], __amdgpu_buffer_rsrc_t rv, uint32_t voff, uint32_t row_bytes,
                                       uint32_t tile_off, int tid) {
  if (tid < FlashLds<D>::vunits) {
#pragma unroll
    for (int j = 0; j < 4; ++j) g[j] = bload16(rv, voff + tile_off + j * row_bytes);
  }
}

template <int D>
__device__ __forceinline__ void store_v(char* vt, const u32x4 (&g)[4], int tid) {
  if (tid < FlashLds<D>::vunits) {
    const int kg = tid & 15, dc = tid >> 4;
    store_vt4<FBN>(vt, dc * 8, key_slot(4 * kg), g[0], g[1], g[2], g[3]);
  }
}

// S^T for a 64-key tile: two independent 32-key accumulator chains
template <int D>
__device__ __forceinline__ void scores64(f32x16 (&s)[2], const char* kl, const bf16x8 (&qf)[D / 16], int lane) {
  constexpr int KR = KRow<D>::bytes;
  const char* r0 = kl + (lane & 31) * KR + (lane >> 5) * 16;
  const char* r1 = r0 + 32 * KR;
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    s[0] = mma(ld_bf16x8(r0 + ks * 32), qf[ks], s[0]);
    s[1] = mma(ld_bf16x8(r1 + ks * 32), qf[ks], s[1]);
  }
}

__device__ __forceinline__ void mask_tail(f32x16 (&s)[2], int nvalid, int h) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (32 * t + acc_key(i, h) >= nvalid) s[t][i] = -INFINITY;
}

// Running max update with lazy rescale of the accumulator.
template <int D>
__device__ __forceinline__ void update_max(const f32x16 (&s)[2], f32x16 (&o)[D / 32], float& m, float& l, float c) {
  float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[0][i], s[1][i]));
  mx = halves_max(mx) * c;
  if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleThreshold)) {
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    l *= alpha;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) o[mt] *= alpha;
    m = mn;
  }
}

// exp2(s*c - m) as bf16 B operands for the four 16-key PV steps; adds the
// unnormalised weights to l.
__device__ __forceinline__ void probs(const f32x16 (&s)[2], bf16x8 (&pb)[4], float& l, float c, float m) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fast_exp2(fmaf(s[st >> 1][8 * (st & 1) + e], c, -m));
      l += p;
      pb[st][e] = static_cast<bf16>(p);
    }
  }
}

template <int D>
__device__ __forceinline__ void pv64(f32x16 (&o)[D / 32], const char* vt, const bf16x8 (&pb)[4], int steps, int lane) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if (st < steps) {
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) o[mt] = pv_step<FBN>(vt, mt, st, pb[st], o[mt], lane);
    }
  }
}

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(FNT, 2) flash_kernel(GroupedArgs a, int qtiles, int nwg) {
  using FL = FlashLds<D>;
  __shared__ __attribute__((aligned(16))) char smem[FL::total];
  char* const kring = smem;
  char* const vring = smem + 2 * FL::kbytes;

  const int id = xcd_order(blockIdx.x, nwg);
  const int qt = id % qtiles;
  const int rest = id / qtiles;
  const int p = rest % a.problems;
  const int hd = rest / a.problems;

  Rows r;
  r.head_elems = a.head_elems;
  r.base = problem_base(a, p);
  r.rs = a.row_stride;
  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const bf16* qp = static_cast<const bf16*>(a.q) + hoff;
  const bf16* kp = static_cast<const bf16*>(a.k) + hoff;
  const bf16* vp = static_cast<const bf16*>(a.v) + hoff;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int L = a.L;
  const int row0 = qt * FBM + wave * 32;
  const bool active = row0 < L;
  const int n = (L + FBN - 1) / FBN;
  const int nv_last = L - (n - 1) * FBN;
  const float c = a.scale_log2;

  bf16x8 qf[D / 16];
  load_q<D>(qf, qp, r, row0, L, lane);
  f32x16 o[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const __amdgpu_buffer_rsrc_t rk = problem_rsrc(kp, r, L, D);
  const __amdgpu_buffer_rsrc_t rv = problem_rsrc(vp, r, L, D);
  const KOffsets<D> ko(tid, r.rs);
  const uint32_t voff = v_offset<D>(tid, r.rs);
  const uint32_t row_bytes = static_cast<uint32_t>(r.rs * D * 2);
  const uint32_t tile_bytes = static_cast<uint32_t>(FBN * r.rs * D * 2);

  u32x4 gk[FL::kchunks], gv[4];
  load_k<D>(gk, rk, ko, 0);
  load_v<D>(gv, rv, voff, row_bytes, 0, tid);
  store_k<D>(kring, gk, tid);
  store_v<D>(vring, gv, tid);
  if (n > 1) {
    load_k<D>(gk, rk, ko, tile_bytes);
    store_k<D>(kring + FL::kbytes, gk, tid);
  }
  __syncthreads();

  f32x16 s[2];
  if (active) scores64<D>(s, kring, qf, lane);

  // steady state: every iteration has a next tile
  for (int j = 0; j + 1 < n; ++j) {
    if (j + 2 < n) load_k<D>(gk, rk, ko, (j + 2) * tile_bytes);
    load_v<D>(gv, rv, voff, row_bytes, (j + 1) * tile_bytes, tid);
    if (active) {
      update_max<D>(s, o, m, l, c);
      f32x16 sn[2];
      scores64<D>(sn, kring + ((j + 1) & 1) * FL::kbytes, qf, lane);
      bf16x8 pb[4];
      probs(s, pb, l, c, m);
      pv64<D>(o, vring + (j & 1) * FL::vbytes, pb, 4, lane);
      s[0] = sn[0];
      s[1] = sn[1];
    }
    if (j + 2 < n) store_k<D>(kring + (j & 1) * FL::kbytes, gk, tid);
    store_v<D>(vring + ((j + 1) & 1) * FL::vbytes, gv, tid);
    __syncthreads();
  }

  if (!active) return;
  // last tile: mask keys past the end, skip the empty half of the PV product
  if (nv_last < FBN) mask_tail(s, nv_last, h);
  update_max<D>(s, o, m, l, c);
  bf16x8 pb[4];
  probs(s, pb, l, c, m);
  pv64<D>(o, vring + ((n - 1) & 1) * FL::vbytes, pb, nv_last > 32 ? 4 : 2, lane);

  const float inv = 1.f / halves_sum(l);  // both lane halves of a row are active together
  const int row = row0 + (lane & 31);
  if (row < L) store_out<D, OUT_F32>(a.o, hoff + (r.base + static_cast<int64_t>(row) * r.rs) * D, o, inv, lane);
}

// ---------------------------------------------------------------- group
template <int D, int QT>
struct GroupLds {
  static constexpr int BN = 32 * QT;
  static constexpr int PPW = QT == 1 ? 4 : (QT == 2 ? 2 : 1);
  static constexpr int NT = 64 * QT * PPW;
  static constexpr int kbytes = BN * KRow<D>::bytes;
  static constexpr int vbytes = D * VRow<BN>::bytes;
  static constexpr int prob = kbytes + vbytes;
};

template <int D, int QT, bool OUT_F32>
__global__ void __launch_bounds__((GroupLds<D, QT>::NT), 2) group_kernel(GroupedArgs a, int wg_per_head) {
  using G = GroupLds<D, QT>;
  constexpr int BN = G::BN, PPW = G::PPW, NT = G::NT, CPR = D / 8;
  __shared__ __attribute__((aligned(16))) char smem[PPW * G::prob];

  const int hd = blockIdx.x / wg_per_head;
  const int p0 = (blockIdx.x % wg_per_head) * PPW;
  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const bf16* qp = static_cast<const bf16*>(a.q) + hoff;
  const bf16* kp = static_cast<const bf16*>(a.k) + hoff;
  const bf16* vp = static_cast<const bf16*>(a.v) + hoff;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = a.L;

  // K rows: PPW problems x BN rows x CPR chunks
  for (int id = tid; id < PPW * BN * CPR; id += NT) {
    const int pl = id / (BN * CPR), row = (id / CPR) % BN, ch = id % CPR;
    const int p = p0 + pl;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (p < a.problems && row < L)
      v = ld16(kp + (problem_base(a, p) + static_cast<int64_t>(row) * a.row_stride) * D + ch * 8);
    *reinterpret_cast<u32x4*>(smem + pl * G::prob + row * KRow<D>::bytes + ch * 16) = v;
  }
  // V^T: units of 4 keys x 8 channels; channel chunk fastest so that 16
  // lanes read one 256-byte row
  for (int id = tid; id < PPW * (BN / 4) * CPR; id += NT) {
    const int dc = id % CPR, kg = (id / CPR) % (BN / 4), pl = id / (CPR * (BN / 4));
    const int p = p0 + pl;
    u32x4 rows[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 4 * kg + j;
      rows[j] = (p < a.problems && key < L)
                    ? ld16(vp + (problem_base(a, p) + static_cast<int64_t>(key) * a.row_stride) * D + dc * 8)
                    : u32x4{0u, 0u, 0u, 0u};
    }
    store_vt4<BN>(smem + pl * G::prob + G::kbytes, dc * 8, key_slot(4 * kg), rows[0], rows[1], rows[2], rows[3]);
  }
  __syncthreads();

  const int pl = wave / QT, qt = wave % QT;
  const int p = p0 + pl;
  const int row0 = qt * 32;
  if (p >= a.problems || row0 >= L) return;
  Rows r;
  r.head_elems = a.head_elems;
  r.base = problem_base(a, p);
  r.rs = a.row_stride;
  bf16x8 qf[D / 16];
  load_q<D>(qf, qp, r, row0, L, lane);
  const char* kl = smem + pl * G::prob;
  const char* vt = kl + G::kbytes;
  const int h = lane >> 5;
  const float c = a.scale_log2;

  f32x16 s[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) s[t] = scores_tile<D>(kl, 32 * t, qf, lane);
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < QT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (32 * t + acc_key(i, h) >= L) s[t][i] = -INFINITY;
      mx = fmaxf(mx, s[t][i]);
    }
  mx = halves_max(mx) * c;
  float l = 0.f;
#pragma unroll
  for (int t = 0; t < QT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[t][i] = fast_exp2(fmaf(s[t][i], c, -mx));
      l += s[t][i];
    }
  f32x16 o[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};
#pragma unroll
  for (int st = 0; st < 2 * QT; ++st) {
    const bf16x8 pb = p_operand(s[st >> 1], st & 1);
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) o[mt] = pv_step<BN>(vt, mt, st, pb, o[mt], lane);
  }
  const float inv = 1.f / halves_sum(l);
  const int row = row0 + (lane & 31);
  if (row < L) store_out<D, OUT_F32>(a.o, hoff + (r.base + static_cast<int64_t>(row) * r.rs) * D, o, inv, lane);
}

bool mfma_types_ok(const GroupedArgs& a) {
  return (a.D == 64 || a.D == 128) && a.qk_type == kBF16 && a.v_type == kBF16;
}

template <int D, bool F32>
hipError_t launch_flash_t(const GroupedArgs& a, hipStream_t s) {
  const int qtiles = (a.L + FBM - 1) / FBM;
  const int64_t nwg = static_cast<int64_t>(qtiles) * a.problems * a.heads;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((flash_kernel<D, F32>), dim3(static_cast<unsigned>(nwg)), dim3(FNT), 0, s, a, qtiles,
                     static_cast<int>(nwg));
  return hipGetLastError();
}

template <int D, int QT, bool F32>
hipError_t launch_group_t(const GroupedArgs& a, hipStream_t s) {
  using G = GroupLds<D, QT>;
  const int wg_per_head = (a.problems + G::PPW - 1) / G::PPW;
  const int64_t nwg = static_cast<int64_t>(wg_per_head) * a.heads;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((group_kernel<D, QT, F32>), dim3(static_cast<unsigned>(nwg)), dim3(G::NT), 0, s, a,
                     wg_per_head);
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_group_d(const GroupedArgs& a, hipStream_t s) {
  const int qt = (a.L + 31) / 32;
  switch (qt) {
    case 1: return launch_group_t<D, 1, F32>(a, s);
    case 2: return launch_group_t<D, 2, F32>(a, s);
    case 3: return launch_group_t<D, 3, F32>(a, s);
    case 4: return launch_group_t<D, 4, F32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// 32-bit buffer offsets must reach one tile past the end of a problem
bool flash_supported(const GroupedArgs& a) {
  return mfma_types_ok(a) && a.L > 128 &&
         (static_cast<int64_t>(a.L) + FBN) * a.row_stride * a.D * 2 < (int64_t{1} << 31);
}

hipError_t launch_flash(const GroupedArgs& a, hipStream_t s) {
  if (!flash_supported(a)) return hipErrorInvalidValue;
  const bool f32 = a.o_type == kF32;
  if (a.D == 128) return f32 ? launch_flash_t<128, true>(a, s) : launch_flash_t<128, false>(a, s);
  return f32 ? launch_flash_t<64, true>(a, s) : launch_flash_t<64, false>(a, s);
}

bool small_supported(const GroupedArgs& a) { return mfma_types_ok(a) && a.L >= 2 && a.L <= 128; }

hipError_t launch_small(const GroupedArgs& a, hipStream_t s) {
  if (!small_supported(a)) return hipErrorInvalidValue;
  const bool f32 = a.o_type == kF32;
  if (a.D == 128) return f32 ? launch_group_d<128, true>(a, s) : launch_group_d<128, false>(a, s);
  return f32 ? launch_group_d<64, true>(a, s) : launch_group_d<64, false>(a, s);
}

}  // namespace monarch
