// bf16 MFMA grouped-attention kernels for gfx950.
//
// flash: problems longer than 128 rows (stage-1 frame blocks, stage-2 groups
//   of many blocks, dense attention). A workgroup of four waves owns 128
//   query rows of one problem (32 per wave, kept as MFMA B operands in
//   registers) and streams the problem's keys and values in tiles of 64 rows
//   through LDS. K and V tiles live in two-slot rings: iteration j computes
//   the scores of tile j+1 while the softmax of tile j runs, then the value
//   product of tile j, with tile j+2's keys and tile j+1's values in flight
//   from global memory. Softmax is online with a lazy rescale: the running
//   maximum only moves when a tile's maximum exceeds it by more than 8 (log2
//   units), so unnormalised weights stay <= 2^8 and the accumulator is rarely
//   rescaled. Workgroups are ordered so that the query tiles of one problem
//   run on one XCD and share its L2.
//
// group: problems of at most 128 rows (stage-2 groups of a few blocks,
//   stage-1 row blocks). One problem per workgroup, one wave per 32 query
//   rows, all keys and values in LDS at once, a single pass.
//
// Scores never leave the chip and memory stays linear in N, the "SRAM
// reduction" design the MonarchRT pages describe for their kernels
// (gist.science explainer, section 2.C).
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

// Per-thread byte offsets of the 16-byte chunks a cooperative tile load
// covers: chunk id = tid + NT*c -> row id/CPR, channels 8*(id%CPR).. (16
// consecutive lanes read one 256-byte row).
template <int D, int ROWS, int NT>
struct TileOffsets {
  static constexpr int CPR = D / 8;
  static constexpr int N = ROWS * CPR / NT;
  uint32_t g[N];  // global, relative to row 0 of the tile
  uint32_t s[N];  // LDS
  __device__ __forceinline__ TileOffsets(int tid, int64_t rs) {
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const int id = tid + NT * c;
      g[c] = static_cast<uint32_t>(((id / CPR) * rs * D + (id % CPR) * 8) * 2);
      s[c] = static_cast<uint32_t>((id / CPR) * KRow<D>::bytes + (id % CPR) * 16);
    }
  }
  __device__ __forceinline__ void load(u32x4* r, __amdgpu_buffer_rsrc_t src, uint32_t tile_off) const {
#pragma unroll
    for (int c = 0; c < N; ++c) r[c] = bload16(src, g[c] + tile_off);
  }
  __device__ __forceinline__ void store(char* lds, const u32x4* r) const {
#pragma unroll
    for (int c = 0; c < N; ++c) *reinterpret_cast<u32x4*>(lds + s[c]) = r[c];
  }
};

// ---------------------------------------------------------------- flash
constexpr int FBM = 128;  // query rows per workgroup
constexpr int FBN = 64;   // keys per LDS tile
constexpr int FNT = 256;  // threads

template <int D>
struct FlashLds {
  static constexpr int tile = FBN * KRow<D>::bytes;  // one K or V tile
  static constexpr int total = 4 * tile;             // two-slot rings for K and V
};

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
__device__ __forceinline__ void pv64(f32x16 (&o)[D / 32], const char* vl, const bf16x8 (&pb)[4], int steps, int lane) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if (st < steps) {
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) o[mt] = pv_step<D>(vl, mt, st, pb[st], o[mt], lane);
    }
  }
}

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(FNT, 2) flash_kernel(GroupedArgs a, int qtiles, int nwg) {
  using FL = FlashLds<D>;
  using TO = TileOffsets<D, FBN, FNT>;
  __shared__ __attribute__((aligned(16))) char smem[FL::total];
  char* const kring = smem;
  char* const vring = smem + 2 * FL::tile;

  const int id = xcd_order(blockIdx.x, nwg);
  const int qt = id % qtiles;
  const int rest = id / qtiles;
  const int p = rest % a.problems;
  const int hd = rest / a.problems;

  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L;
  const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, base, rs, L, D, 2);
  const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
  const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
  const auto ro = problem_rsrc(static_cast<const char*>(a.o) + hoff * (OUT_F32 ? 4 : 2), base, rs, L, D,
                               OUT_F32 ? 4 : 2);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int row0 = qt * FBM + wave * 32;
  const bool active = row0 < L;
  const int n = (L + FBN - 1) / FBN;
  const int nv_last = L - (n - 1) * FBN;
  const float c = a.scale_log2;
  const TO to(tid, rs);
  const uint32_t tile_bytes = static_cast<uint32_t>(FBN * rs * D * 2);

  bf16x8 qf[D / 16];
  load_qfrag<D>(qf, rq, row0, rs, lane);
  f32x16 o[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};
  float m = -INFINITY, l = 0.f;

  u32x4 gk[TO::N], gv[TO::N];
  to.load(gk, rk, 0);
  to.load(gv, rv, 0);
  to.store(kring, gk);
  to.store(vring, gv);
  if (n > 1) {
    to.load(gk, rk, tile_bytes);
    to.store(kring + FL::tile, gk);
  }
  __syncthreads();

  f32x16 s[2];
  if (active) scores64<D>(s, kring, qf, lane);
  // iteration 0 overwrites K ring slot 0 (tile 0) with tile 2: every wave
  // must be done reading it
  __syncthreads();

  // steady state: every iteration has a next tile
  for (int j = 0; j + 1 < n; ++j) {
    if (j + 2 < n) to.load(gk, rk, (j + 2) * tile_bytes);
    to.load(gv, rv, (j + 1) * tile_bytes);
    if (active) {
      update_max<D>(s, o, m, l, c);
      f32x16 sn[2];
      scores64<D>(sn, kring + ((j + 1) & 1) * FL::tile, qf, lane);
      bf16x8 pb[4];
      probs(s, pb, l, c, m);
      pv64<D>(o, vring + (j & 1) * FL::tile, pb, 4, lane);
      s[0] = sn[0];
      s[1] = sn[1];
    }
    if (j + 2 < n) to.store(kring + (j & 1) * FL::tile, gk);
    to.store(vring + ((j + 1) & 1) * FL::tile, gv);
    __syncthreads();
  }

  if (!active) return;
  // last tile: mask keys past the end, skip the empty half of the PV product
  if (nv_last < FBN) mask_tail(s, nv_last, h);
  update_max<D>(s, o, m, l, c);
  bf16x8 pb[4];
  probs(s, pb, l, c, m);
  pv64<D>(o, vring + ((n - 1) & 1) * FL::tile, pb, nv_last > 32 ? 4 : 2, lane);

  const float inv = 1.f / halves_sum(l);  // both lane halves of a row are active together
  store_out<D, OUT_F32>(ro, row0 + (lane & 31), rs, o, inv, lane);
}

// ---------------------------------------------------------------- group
template <int D, int QT>
struct GroupCfg {
  static constexpr int BN = 32 * QT;  // keys (padded to whole 32-key tiles)
  static constexpr int NT = 64 * QT;  // one wave per 32 query rows
  static constexpr int lds = 2 * BN * KRow<D>::bytes;
};

template <int D, int QT, bool OUT_F32>
__global__ void __launch_bounds__((GroupCfg<D, QT>::NT), 2) group_kernel(GroupedArgs a) {
  using G = GroupCfg<D, QT>;
  using TO = TileOffsets<D, G::BN, G::NT>;
  __shared__ __attribute__((aligned(16))) char smem[G::lds];
  char* const kl = smem;
  char* const vl = smem + G::BN * KRow<D>::bytes;

  const int p = blockIdx.x % a.problems;
  const int hd = blockIdx.x / a.problems;
  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L;
  const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, base, rs, L, D, 2);
  const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
  const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
  const auto ro = problem_rsrc(static_cast<const char*>(a.o) + hoff * (OUT_F32 ? 4 : 2), base, rs, L, D,
                               OUT_F32 ? 4 : 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int row0 = wave * 32;

  bf16x8 qf[D / 16];
  load_qfrag<D>(qf, rq, row0, rs, lane);
  const TO to(tid, rs);
  {
    u32x4 gk[TO::N], gv[TO::N];
    to.load(gk, rk, 0);
    to.load(gv, rv, 0);
    to.store(kl, gk);
    to.store(vl, gv);
  }
  __syncthreads();

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
    for (int mt = 0; mt < D / 32; ++mt) o[mt] = pv_step<D>(vl, mt, st, pb, o[mt], lane);
  }
  const float inv = 1.f / halves_sum(l);
  store_out<D, OUT_F32>(ro, row0 + (lane & 31), rs, o, inv, lane);
}

bool mfma_types_ok(const GroupedArgs& a) {
  return (a.D == 64 || a.D == 128) && a.qk_type == kBF16 && a.v_type == kBF16;
}

// 32-bit buffer offsets must reach a whole key tile past the end of a problem
// (bytes counted at the widest output element, 4)
bool offsets_fit(const GroupedArgs& a, int pad_rows) {
  return (static_cast<int64_t>(a.L) + pad_rows) * a.row_stride * a.D * 4 < (int64_t{1} << 31);
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
  const int64_t nwg = static_cast<int64_t>(a.problems) * a.heads;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((group_kernel<D, QT, F32>), dim3(static_cast<unsigned>(nwg)), dim3(GroupCfg<D, QT>::NT), 0,
                     s, a);
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_group_d(const GroupedArgs& a, hipStream_t s) {
  switch ((a.L + 31) / 32) {
    case 1: return launch_group_t<D, 1, F32>(a, s);
    case 2: return launch_group_t<D, 2, F32>(a, s);
    case 3: return launch_group_t<D, 3, F32>(a, s);
    case 4: return launch_group_t<D, 4, F32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool flash_supported(const GroupedArgs& a) { return mfma_types_ok(a) && a.L > 128 && offsets_fit(a, FBN); }

hipError_t launch_flash(const GroupedArgs& a, hipStream_t s) {
  if (!flash_supported(a)) return hipErrorInvalidValue;
  const bool f32 = a.o_type == kF32;
  if (a.D == 128) return f32 ? launch_flash_t<128, true>(a, s) : launch_flash_t<128, false>(a, s);
  return f32 ? launch_flash_t<64, true>(a, s) : launch_flash_t<64, false>(a, s);
}

bool small_supported(const GroupedArgs& a) {
  return mfma_types_ok(a) && a.L >= 2 && a.L <= 128 && offsets_fit(a, 32);
}

hipError_t launch_small(const GroupedArgs& a, hipStream_t s) {
  if (!small_supported(a)) return hipErrorInvalidValue;
  const bool f32 = a.o_type == kF32;
  if (a.D == 128) return f32 ? launch_group_d<128, true>(a, s) : launch_group_d<128, false>(a, s);
  return f32 ? launch_group_d<64, true>(a, s) : launch_group_d<64, false>(a, s);
}

}  // namespace monarch
