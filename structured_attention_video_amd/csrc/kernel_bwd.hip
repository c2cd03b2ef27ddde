// Backward of one grouped-attention stage on the matrix cores (bf16 inputs,
// fp32 accumulation), by recomputation from the forward's per-row log-sum-
// exp statistic, in two kernels that share no accumulator, so no atomics:
//
// bwd_dq: a workgroup of 4 waves owns 128 query rows of one problem (as the
//   forward's flash kernel) and streams the problem's K and V in 64-row
//   tiles through LDS. Per tile: S^T = K Q^T and dP^T = V G^T (V rows are
//   read exactly like K rows, G is held like Q), P^T = exp2(c S^T - lse),
//   dS^T = P^T * (dP^T - delta), and dQ^T += K^T dS^T, where the K^T operand
//   is gathered by the transposing LDS reads the forward uses for V^T and
//   dS^T leaves the accumulator already in B-operand layout (as P^T does in
//   the forward).
// bwd_dkdv (launched twice: dV, then dK): a workgroup owns 128 key rows of
//   one problem (32 per wave, K and V held as B operands) and streams the
//   problem's Q and G in 64-row tiles through LDS, with lse and delta of
//   those rows. Per 32-query step: S = Q K^T and dP = G V^T (lane = key), P
//   and dS as above, then dV^T += G^T P or dK^T += Q^T dS with G^T and Q^T
//   gathered by transposing reads, P and dS again straight from the
//   accumulators.
//
// Rows past the end of a problem read as zero through the buffer
// descriptors; keys past the end get score -inf in the last tile of
// bwd_dq; queries past the end have zero Q and G rows and delta 0, so their
// terms in dK and dV vanish. (The chain rule itself: explainer section 2.C
// ships forward and backward kernels; the formulas are those of softmax
// attention, applied to each Monarch stage.)
#include "flash_common.h"

namespace monarch {
namespace {

// P = exp2(c s - lse) and dS = P * (dp - delta), in place (s -> P, dp -> dS)
__device__ __forceinline__ void probs_grads(f32x16& s, f32x16& dp, const float (&lse)[16], const float (&del)[16],
                                            float c) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s[i] = fast_exp2(fmaf(s[i], c, -lse[i]));
    dp[i] = s[i] * (dp[i] - del[i]);
  }
}

// Store a lane's share of X^T accumulators (channels in registers, rows in
// lanes: row `row` of the problem) scaled by `mul`, plus the fp32 `add` rows.
template <int D>
__device__ __forceinline__ void store_rows(__amdgpu_buffer_rsrc_t ro, bool out_f32, __amdgpu_buffer_rsrc_t ra,
                                           bool has_add, int row, int64_t rs, const f32x16 (&x)[D / 32], float mul,
                                           int lane) {
  const int h = lane >> 5;
  const uint32_t rowel = static_cast<uint32_t>(row * rs * D);
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t ch = 32 * mt + 8 * g + 4 * h;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = x[mt][4 * g + e] * mul;
      if (has_add) {
        const u32x4 a = bload16(ra, (rowel + ch) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += __uint_as_float(a[e]);
      }
      if (out_f32) {
        const u32x4 w = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, static_cast<int>((rowel + ch) * 4), 0, 0);
      } else {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = static_cast<bf16>(v[e]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, w), ro, static_cast<int>((rowel + ch) * 2), 0, 0);
      }
    }
  }
}

// S^T (or dP^T) of one 64-row tile against a wave's fragment f: two 32-row
// accumulator chains from the row-major tile t
template <int D>
__device__ __forceinline__ void tile_products(f32x16 (&s)[2], const char* t, const FlashOffsets<D>& fo,
                                              const bf16x8 (&f)[D / 16]) {
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    s[0] = mma(k_operand<D>(t, fo, ks, 0), f[ks], s[0]);
    s[1] = mma(k_operand<D>(t, fo, ks, 1), f[ks], s[1]);
  }
}

template <int D>
__global__ void __launch_bounds__(FNT, 2) bwd_dq_kernel(BwdArgs b, int qtiles, int nwg) {
  using T = SwTile<D>;
  __shared__ __attribute__((aligned(1024))) char k0[T::bytes];
  __shared__ __attribute__((aligned(1024))) char k1[T::bytes];
  __shared__ __attribute__((aligned(1024))) char v0[T::bytes];
  __shared__ __attribute__((aligned(1024))) char v1[T::bytes];
  const GroupedArgs& a = b.g;
  const int id = xcd_order(blockIdx.x, nwg);
  // uniform per workgroup: readfirstlane keeps the decode and the addresses derived from it
  // in scalar registers
  const int qt = __builtin_amdgcn_readfirstlane(id % qtiles), rest = id / qtiles;
  const int p = __builtin_amdgcn_readfirstlane(rest % a.problems);
  const int hd = __builtin_amdgcn_readfirstlane(rest / a.problems);
  const int64_t ntok = a.head_elems / D;
  const int64_t hoff = hd * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L;
  const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, base, rs, L, D, 2);
  const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
  const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
  const auto rg = problem_rsrc(static_cast<const bf16*>(b.go) + hoff, base, rs, L, D, 2);
  const bool f32 = b.dq_type == kF32;
  const auto ro = problem_rsrc(static_cast<const char*>(b.dq) + hoff * (f32 ? 4 : 2), base, rs, L, D, f32 ? 4 : 2);
  const auto ra = problem_rsrc(b.dq_in ? b.dq_in + hoff : b.delta, base, rs, L, D, 4);

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: copy addresses stay scalar
  const int row0 = qt * FBM + wave * 32;
  const int r = row0 + (lane & 31);
  const int n = (L + FBN - 1) / FBN;
  const int nv_last = L - (n - 1) * FBN;
  const float c = a.scale_log2;
  const FlashOffsets<D> fo(wave, lane, rs);
  const uint32_t tile_bytes = static_cast<uint32_t>(FBN * rs * D * 2);

  fo.dma(k0, rk, 0, wave);
  fo.dma(v0, rv, 0, wave);
  bf16x8 qf[D / 16], gf[D / 16];
  load_qfrag<D>(qf, rq, row0, rs, lane);
  load_qfrag<D>(gf, rg, row0, rs, lane);
  const float lse_r = r < L ? b.lse[hd * ntok + base + r * rs] : 0.f;
  const float del_r = r < L ? b.delta[hd * ntok + base + r * rs] : 0.f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dq[mt] = f32x16{};
  wait_dma();
  __syncthreads();

  auto step = [&](int j, const char* kc, const char* vc, char* kn, char* vn) {
    if (j + 1 < n) {
      fo.dma(kn, rk, (j + 1) * tile_bytes, wave);
      fo.dma(vn, rv, (j + 1) * tile_bytes, wave);
    }
    f32x16 s[2], dp[2];
    tile_products<D>(s, kc, fo, qf);
    tile_products<D>(dp, vc, fo, gf);
    if (j == n - 1 && nv_last < FBN) mask_tail(s, nv_last, h);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[t][i] = fast_exp2(fmaf(s[t][i], c, -lse_r));
        dp[t][i] = s[t][i] * (dp[t][i] - del_r);
      }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8 pb = p_operand(dp[st >> 1], st & 1);
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) dq[mt] = mma(v_operand<D>(kc, fo, mt, st), pb, dq[mt]);
    }
    wait_dma();
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < n; j += 2) {
    step(j, k0, v0, k1, v1);
    step(j + 1, k1, v1, k0, v0);
  }
  if (j < n) step(j, k0, v0, k1, v1);

  // dQ = s * dS K, where s = scale_log2 / log2(e)
  store_rows<D>(ro, f32, ra, b.dq_in != nullptr, r, rs, dq, c * 0.6931471805599453f, lane);
}

// A per-query bias as one more 16-channel K-step of a product with lane =
// key: the A operand (rows = queries) carries x of this lane's query row in
// channels 0 and 1 as two bf16 parts (x = hi + lo to ~2^-18 relative), the
// B operand (bias_ones) ones in channels 0 and 1, so the accumulator gains x
// for every key. Lanes of the upper half hold channels 8..15: zeros.
__device__ __forceinline__ bf16x8 bias_operand(float x, int h) {
  const bf16 hi = static_cast<bf16>(x);
  const bf16 lo = static_cast<bf16>(x - static_cast<float>(hi));
  bf16x8 r = {};
  r[0] = h == 0 ? hi : static_cast<bf16>(0.f);
  r[1] = h == 0 ? lo : static_cast<bf16>(0.f);
  return r;
}
__device__ __forceinline__ bf16x8 bias_ones(int h) {
  bf16x8 r = {};
  r[0] = static_cast<bf16>(h == 0 ? 1.f : 0.f);
  r[1] = r[0];
  return r;
}

// MODE 0: dV only (S -> P; dV^T += G^T P). MODE 1: dK only (S, dP -> dS;
// dK^T += Q^T dS). MODE 1 raises the wave's priority over its matrix-product
// phases (s_setprio 1), so the two waves sharing a SIMD tend to alternate
// between products and exponentials (measured -4.5% at the frame shape; the
// same change slowed bwd_dq by as much and left MODE 0 unchanged). In MODE 1 the per-query lse and delta enter the products
// as a bias K-step (c S - lse and dP - delta come out of the accumulators),
// so a lane needs only its own query's two values, not one per accumulator
// register: without it the kernel spilled 25 VGPRs (measured 693 -> 628 us at
// the frame shape). MODE 0 has registers to spare and reads lse per register
// (the extra MFMA at the end of its short chain measured slower there). One kernel holding both accumulators, K and V would need
// more registers than two waves per SIMD have; recomputing S in both costs
// a quarter more matrix work instead.
template <int D, int MODE>
__global__ void __launch_bounds__(FNT, 2) bwd_dkdv_kernel(BwdArgs b, int ktiles, int nwg) {
  using T = SwTile<D>;
  __shared__ __attribute__((aligned(1024))) char q0[T::bytes];
  __shared__ __attribute__((aligned(1024))) char q1[T::bytes];
  __shared__ __attribute__((aligned(1024))) char g0[T::bytes];
  __shared__ __attribute__((aligned(1024))) char g1[T::bytes];
  __shared__ __attribute__((aligned(16))) float st_lse[2][FBN];
  __shared__ __attribute__((aligned(16))) float st_del[2][FBN];
  const GroupedArgs& a = b.g;
  const int id = xcd_order(blockIdx.x, nwg);
  // uniform per workgroup (as in bwd_dq_kernel)
  const int kt = __builtin_amdgcn_readfirstlane(id % ktiles), rest = id / ktiles;
  const int p = __builtin_amdgcn_readfirstlane(rest % a.problems);
  const int hd = __builtin_amdgcn_readfirstlane(rest / a.problems);
  const int64_t ntok = a.head_elems / D;
  const int64_t hoff = hd * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L;
  const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, base, rs, L, D, 2);
  const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
  const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
  const auto rg = problem_rsrc(static_cast<const bf16*>(b.go) + hoff, base, rs, L, D, 2);
  const bool kf32 = b.dk_type == kF32, vf32 = b.dv_type == kF32;
  const auto rdk = problem_rsrc(static_cast<const char*>(b.dk) + hoff * (kf32 ? 4 : 2), base, rs, L, D, kf32 ? 4 : 2);
  const auto ra = problem_rsrc(b.dk_in ? b.dk_in + hoff : b.delta, base, rs, L, D, 4);

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: copy addresses stay scalar
  const int key0 = kt * FBM + wave * 32;
  const int n = (L + FBN - 1) / FBN;
  const float c = a.scale_log2;
  const FlashOffsets<D> fo(wave, lane, rs);
  const uint32_t tile_bytes = static_cast<uint32_t>(FBN * rs * D * 2);
  const float* lse_h = b.lse + hd * ntok + base;
  const float* del_h = b.delta + hd * ntok + base;

  // per-row statistics of query tile j (rows past the end: 0), loaded into
  // registers early and stored to LDS slot s just before the barrier
  float nl = 0.f, nd = 0.f;
  const float inv_c = 1.f / c;
  auto stats_load = [&](int j) {
    if (tid < FBN) {
      const int q = j * FBN + tid;
      nl = q < L ? lse_h[q * rs] : 0.f;
      nd = q < L ? del_h[q * rs] : 0.f;
    }
  };
  auto stats_store = [&](int s) {
    if (tid < FBN) {
      st_lse[s][tid] = nl;
      st_del[s][tid] = nd;
    }
  };
  fo.dma(q0, rq, 0, wave);
  fo.dma(g0, rg, 0, wave);
  stats_load(0);
  stats_store(0);
  bf16x8 kf[D / 16], vf[D / 16];
  load_qfrag<D>(kf, rk, key0, rs, lane);
  if (MODE == 1) load_qfrag<D>(vf, rv, key0, rs, lane);
  const bf16x8 ones = bias_ones(h);  // MODE 1 only
  f32x16 acc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) acc[mt] = f32x16{};
  wait_dma();
  __syncthreads();

  auto step = [&](int j, const char* qc, const char* gc, char* qn, char* gn, int sc) {
    if (j + 1 < n) {
      fo.dma(qn, rq, (j + 1) * tile_bytes, wave);
      fo.dma(gn, rg, (j + 1) * tile_bytes, wave);
      stats_load(j + 1);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // S = Q K^T, dP = G V^T for 32 queries: lane = key, register i = query
      // 32*sub + 8*(i/4) + 4*h + i%4 of the tile
      f32x16 s = {}, dp = {};
      if (MODE == 1) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s = mma(k_operand<D>(qc, fo, ks, sub), kf[ks], s);
        if (MODE == 1) dp = mma(k_operand<D>(gc, fo, ks, sub), vf[ks], dp);
      }
      if (MODE == 1) {
        // s -= lse / c and dp -= delta (the bias K-step, lane = this query row)
        const int qrow = 32 * sub + (lane & 31);
        s = mma(bias_operand(-st_lse[sc][qrow] * inv_c, h), ones, s);
        dp = mma(bias_operand(-st_del[sc][qrow], h), ones, dp);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] = fast_exp2(s[i] * c);  // P
          dp[i] *= s[i];               // dS = P (dP - delta)
        }
      } else {
        // P = exp2(c s - lse) with lse of each register's query
        float lse[16], del[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int q = 32 * sub + 8 * g + 4 * h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lse[4 * g + e] = st_lse[sc][q + e];
            del[4 * g + e] = 0.f;
          }
        }
        probs_grads(s, dp, lse, del, c);
      }
      // dV^T += G^T P (MODE 0) or dK^T += Q^T dS (MODE 1), two 16-query steps
      if (MODE == 1) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 pb = p_operand(MODE == 1 ? dp : s, st);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
          acc[mt] = mma(v_operand<D>(MODE == 1 ? qc : gc, fo, mt, 2 * sub + st), pb, acc[mt]);
      }
      if (MODE == 1) __builtin_amdgcn_s_setprio(0);
    }
    if (j + 1 < n) stats_store(sc ^ 1);
    wait_dma();
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < n; j += 2) {
    step(j, q0, g0, q1, g1, 0);
    step(j + 1, q1, g1, q0, g0, 1);
  }
  if (j < n) step(j, q0, g0, q1, g1, 0);

  const int r = key0 + (lane & 31);
  if constexpr (MODE == 1) {
    store_rows<D>(rdk, kf32, ra, b.dk_in != nullptr, r, rs, acc, c * 0.6931471805599453f, lane);
  } else if (key0 < L) {
    // dV rows leave whole, staged through this wave's own (dead) Q or G slot:
    // measured 2.4% (frame) and 6.5% (row layout, rows 52 tokens apart)
    // faster than 8-byte pieces of 32 rows; for the dK and dQ kernels the
    // same change measured slower at the frame shape
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    char* t = wv == 0 ? q0 : wv == 1 ? q1 : wv == 2 ? g0 : g1;
    const int64_t wb = base + key0 * rs;
    const auto rw = problem_rsrc(static_cast<const char*>(b.dv) + hoff * (vf32 ? 4 : 2), wb, rs, L - key0, D,
                                 vf32 ? 4 : 2);
    if (vf32)
      stage_rows<D, true>(t, t + 64 * D, acc, 1.f, rw, rs, lane);
    else
      stage_rows<D, false>(t, t, acc, 1.f, rw, rs, lane);
  }
}

// ---------------------------------------------------------------- small problems, one pass
// One wave per problem of at most 32 rows (the frame layout's stage-2 groups,
// m = 21), everything in one launch. Q, K, V (the stage's values) and G rows
// are copied whole into four swizzled 32-row LDS tiles; every product is one
// 32x32 tile. The wave
//   (a) recomputes the forward with lane = query: S^T = K Q^T, its row max
//       and sum (so lse) and P^T; dP^T = V G^T; delta = rowsum(G * O) as the
//       sum over keys of P dP; dS^T = P^T (dP^T - delta); dQ^T = K^T dS^T;
//   (b) with lane = key, taking lse and delta of each query from LDS:
//       S = Q K^T, dP = G V^T, P, dS, dV^T = G^T P and dK^T = Q^T dS, and
//       the next stage's delta of each key row, rowsum(dV * V) with dV
//       rounded as stored.
// Recomputing S and dP in the second layout costs 16 MFMAs per problem,
// nothing against its memory traffic; the launch replaces the stage's
// forward recompute, both row-dot launches and the three tiled backward
// launches.
// Rows past the end read as zero (keys masked in (a); queries have zero G,
// so zero dS; results of rows past the end are dropped at the store).
// Sum over this lane's channels of x^T (register i of tile mt: channel
// 32 mt + 8 (i / 4) + 4 h + i % 4), scaled by mul and optionally rounded to
// bf16, times the same channels of row r of a bf16 tile.
template <int D>
__device__ __forceinline__ float row_dot_acc(const f32x16 (&x)[D / 32], float mul, bool round_bf16,
                                             const char* tile, int r, int h) {
  constexpr int ROWB = D * 2;
  float acc = 0.f;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(tile + r * ROWB + 16 * ((4 * mt + g) ^ swz<D>(r)) + 8 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
        float xv = x[mt][4 * g + e] * mul;
        if (round_bf16) xv = static_cast<float>(static_cast<bf16>(xv));
        acc = fmaf(xv, __uint_as_float(bits), acc);
      }
    }
  return acc;
}

template <int D>
__global__ void __launch_bounds__(64, 2) bwd_small_kernel(BwdArgs b) {
  constexpr int ROWB = D * 2, CPR = D / 8, RPI = 1024 / ROWB, IPW = 32 / RPI, TILE = 32 * ROWB;
  __shared__ __attribute__((aligned(1024))) char qt[TILE];
  __shared__ __attribute__((aligned(1024))) char kt[TILE];
  __shared__ __attribute__((aligned(1024))) char vt[TILE];
  __shared__ __attribute__((aligned(1024))) char gt[TILE];
  const GroupedArgs& a = b.g;
  const int p = blockIdx.x % a.problems, hd = blockIdx.x / a.problems;
  const int64_t ntok = a.head_elems / D;
  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L;
  const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, base, rs, L, D, 2);
  const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
  const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
  const auto rg = problem_rsrc(static_cast<const bf16*>(b.go) + hoff, base, rs, L, D, 2);
  const auto rdq = problem_rsrc(static_cast<const char*>(b.dq) + hoff * 4, base, rs, L, D, 4);
  const auto rdk = problem_rsrc(static_cast<const char*>(b.dk) + hoff * 4, base, rs, L, D, 4);
  const auto rdv = problem_rsrc(static_cast<const char*>(b.dv) + hoff * 2, base, rs, L, D, 2);
  const int lane = threadIdx.x, h = lane >> 5, r = lane & 31;
  const float c = a.scale_log2;

#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = RPI * i + lane / CPR;
    const int ch = (lane % CPR) ^ swz<D>(row);
    const uint32_t goff = static_cast<uint32_t>((row * rs * D + ch * 8) * 2);
    const int dst = RPI * i * ROWB;
    lds_dma16(rq, qt + dst, goff);
    lds_dma16(rk, kt + dst, goff);
    lds_dma16(rv, vt + dst, goff);
    lds_dma16(rg, gt + dst, goff);
  }
  wait_dma();
  __syncthreads();
  const FlashOffsets<D> fo(0, lane, rs);  // LDS read offsets of a tile's first 32 rows

  // per-query statistics handed from (a) (lane = query) to (b) (register =
  // query) by lane permutes, which need no LDS allocation: the four tiles
  // alone (32 KB at d = 128) let five workgroups share a CU
  float q_lse = 0.f, q_del = 0.f;
  bf16x8 dsb[2];
  // (a) lane = query r
  {
    bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = ld_bf16x8(qt + swoff<D>(r, 2 * ks + h));
      gf[ks] = ld_bf16x8(gt + swoff<D>(r, 2 * ks + h));
    }
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = mma(k_operand<D>(kt, fo, ks, 0), qf[ks], s);
      dp = mma(k_operand<D>(vt, fo, ks, 0), gf[ks], dp);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (acc_key(i, h) >= L) s[i] = -INFINITY;
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = halves_max(mx) * c;
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = fast_exp2(fmaf(s[i], c, -mx));
      l += s[i];
    }
    l = halves_sum(l);
    const float inv = 1.f / l;
    // delta = rowsum(G * O) = sum over keys of P dP, taken from the fp32 P and
    // dP in registers: dS = P (dP - delta) then sums to zero over the keys up
    // to fp32 rounding (G * O with O built from bf16 weights misses that by a
    // bf16 rounding of P, which the subtraction amplifies)
    float pd = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) pd = fmaf(s[i], dp[i], pd);
    const float del = halves_sum(pd) * inv;
    q_lse = mx + __builtin_amdgcn_logf(l);
    q_del = del;
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] = s[i] * inv * (dp[i] - del);
    // dS^T as bf16 operands: dQ^T = K^T dS^T comes last, once the other
    // tiles are free to stage the outputs
    dsb[0] = p_operand(dp, 0);
    dsb[1] = p_operand(dp, 1);
  }

  // (b) lane = key r
  {
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = ld_bf16x8(kt + swoff<D>(r, 2 * ks + h));
      vf[ks] = ld_bf16x8(vt + swoff<D>(r, 2 * ks + h));
    }
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = mma(k_operand<D>(qt, fo, ks, 0), kf[ks], s);
      dp = mma(k_operand<D>(gt, fo, ks, 0), vf[ks], dp);
    }
    float lse[16], del[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // lane acc_key(i, h) holds that query's values (both lane halves do)
      const int src = 4 * acc_key(i, h);
      lse[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(q_lse)));
      del[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(q_del)));
    }
    probs_grads(s, dp, lse, del, c);
    const bf16x8 pp[2] = {p_operand(s, 0), p_operand(s, 1)};
    const bf16x8 ps[2] = {p_operand(dp, 0), p_operand(dp, 1)};
    // dV, then dK: one 64-register accumulator at a time (two waves per SIMD)
    {
      f32x16 dv[D / 32];
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) dv[mt] = f32x16{};
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) dv[mt] = mma(v_operand<D>(gt, fo, mt, st), pp[st], dv[mt]);
      const float d1 = halves_sum(row_dot_acc<D>(dv, 1.f, true, vt, r, h));
      if (h == 0 && r < L) b.dv_delta[hd * ntok + base + r * rs] = d1;
      stage_rows<D, false>(vt, vt, dv, 1.f, rdv, rs, lane);  // V and G are dead now
    }
    {
      f32x16 dk[D / 32];
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) dk[mt] = f32x16{};
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) dk[mt] = mma(v_operand<D>(qt, fo, mt, st), ps[st], dk[mt]);
      stage_rows<D, true>(gt, vt, dk, c * 0.6931471805599453f, rdk, rs, lane);
    }
  }

  // (a, end) dQ^T = K^T dS^T, lane = query r
  {
    f32x16 dq[D / 32];
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) dq[mt] = f32x16{};
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) dq[mt] = mma(v_operand<D>(kt, fo, mt, st), dsb[st], dq[mt]);
    stage_rows<D, true>(qt, gt, dq, c * 0.6931471805599453f, rdq, rs, lane);
  }
}

// ---------------------------------------------------------------- mid-size problems, one pass
// One workgroup of W = ceil(L / 32) waves per problem of up to 128 rows (the
// long layout's stage-2 groups, m = 81; the row layout's stage-1 blocks, b =
// 52), the multi-wave form of bwd_small_kernel. Two roles: partial (FINAL
// false, a stage-2 backward feeding stage 1: dQ, dK in fp32, dV in bf16 and
// dv_delta, as bwd_small_kernel) and final (FINAL true, the last stage: dQ
// and dK in bf16 with the fp32 dq_in and dk_in added before the rounding, dV
// in bf16). In both, lse and delta are recomputed, not read. Q, K, V (the stage's
// values) and G rows are copied whole into four swizzled 32W-row LDS tiles;
// wave w owns rows 32w .. 32w+31.
//   (a) lane = query: S^T and dP^T against every 32-key block, the row max,
//       sum, lse and delta = sum over keys of P dP (fp32, in registers),
//       dS^T as bf16 operands, and dQ^T = K^T dS^T, kept in registers; lse
//       and delta of each query go to LDS;
//   (b) lane = key: S and dP against every 32-query block with lse and delta
//       read per register, dV^T = G^T P and dK^T = Q^T dS in one sweep, and
//       the next stage's delta of each key row, rowsum(dV * V) with dV
//       rounded as stored.
// The tiles (up to 128 KB at d = 128) leave room for one workgroup per CU,
// so each wave has a SIMD to itself and the register budget of a lone wave:
// the three accumulators need not take turns. Outputs leave as whole rows
// through the tiles once every wave is done with them.
template <int D, int W, bool FINAL>
__global__ void __launch_bounds__(64 * W, 1) bwd_group_kernel(BwdArgs b) {
  constexpr int ROWB = D * 2, CPR = D / 8, RPI = 1024 / ROWB, IPW = 32 / RPI, TILE = 32 * W * ROWB;
  __shared__ __attribute__((aligned(1024))) char qt[TILE];
  __shared__ __attribute__((aligned(1024))) char kt[TILE];
  __shared__ __attribute__((aligned(1024))) char vt[TILE];
  __shared__ __attribute__((aligned(1024))) char gt[TILE];
  __shared__ __attribute__((aligned(16))) float xl[32 * W];
  __shared__ __attribute__((aligned(16))) float xd[32 * W];
  const GroupedArgs& a = b.g;
  const int p = blockIdx.x % a.problems, hd = blockIdx.x / a.problems;
  const int64_t ntok = a.head_elems / D;
  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int own = 32 * wave;  // first row of this wave
  const float c = a.scale_log2;
  {
    const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, base, rs, L, D, 2);
    const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
    const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
    const auto rg = problem_rsrc(static_cast<const bf16*>(b.go) + hoff, base, rs, L, D, 2);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int row = own + RPI * i + lane / CPR;
      const int ch = (lane % CPR) ^ swz<D>(row);
      const uint32_t goff = static_cast<uint32_t>((row * rs * D + ch * 8) * 2);
      const int dst = (own + RPI * i) * ROWB;
      lds_dma16(rq, qt + dst, goff);
      lds_dma16(rk, kt + dst, goff);
      lds_dma16(rv, vt + dst, goff);
      lds_dma16(rg, gt + dst, goff);
    }
  }
  wait_dma();
  __syncthreads();
  const FlashOffsets<D> fo(0, lane, rs);  // LDS read offsets of a 32-row block

  // (a) lane = query own + r
  f32x16 dq[D / 32];
  {
    bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = ld_bf16x8(qt + swoff<D>(own + r, 2 * ks + h));
      gf[ks] = ld_bf16x8(gt + swoff<D>(own + r, 2 * ks + h));
    }
    f32x16 s[W], dp[W];
#pragma unroll
    for (int kb = 0; kb < W; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s[kb] = mma(k_operand<D>(kt, fo, ks, kb), qf[ks], s[kb]);
        dp[kb] = mma(k_operand<D>(vt, fo, ks, kb), gf[ks], dp[kb]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < W; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (32 * kb + acc_key(i, h) >= L) s[kb][i] = -INFINITY;
        mx = fmaxf(mx, s[kb][i]);
      }
    mx = halves_max(mx) * c;
    float l = 0.f, pd = 0.f;
#pragma unroll
    for (int kb = 0; kb < W; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = fast_exp2(fmaf(s[kb][i], c, -mx));
        l += s[kb][i];
        pd = fmaf(s[kb][i], dp[kb][i], pd);
      }
    l = halves_sum(l);
    const float inv = 1.f / l;
    // delta from the fp32 P and dP in registers (as bwd_small_kernel)
    const float del = halves_sum(pd) * inv;
    if (h == 0) {
      xl[own + r] = mx + __builtin_amdgcn_logf(l);
      xd[own + r] = del;
    }
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) dq[mt] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < W; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dp[kb][i] = s[kb][i] * inv * (dp[kb][i] - del);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 ds = p_operand(dp[kb], st);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) dq[mt] = mma(v_operand<D>(kt, fo, mt, 2 * kb + st), ds, dq[mt]);
      }
    }
  }
  __syncthreads();  // lse and delta of every query are in LDS

  // (b) lane = key own + r
  f32x16 dv[D / 32], dk[D / 32];
  {
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = ld_bf16x8(kt + swoff<D>(own + r, 2 * ks + h));
      vf[ks] = ld_bf16x8(vt + swoff<D>(own + r, 2 * ks + h));
    }
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) {
      dv[mt] = f32x16{};
      dk[mt] = f32x16{};
    }
#pragma unroll
    for (int qb = 0; qb < W; ++qb) {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s = mma(k_operand<D>(qt, fo, ks, qb), kf[ks], s);
        dp = mma(k_operand<D>(gt, fo, ks, qb), vf[ks], dp);
      }
      float lse[16], del[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        lse[i] = xl[32 * qb + acc_key(i, h)];
        del[i] = xd[32 * qb + acc_key(i, h)];
      }
      probs_grads(s, dp, lse, del, c);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 pp = p_operand(s, st), ps = p_operand(dp, st);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          dv[mt] = mma(v_operand<D>(gt, fo, mt, 2 * qb + st), pp, dv[mt]);
          dk[mt] = mma(v_operand<D>(qt, fo, mt, 2 * qb + st), ps, dk[mt]);
        }
      }
    }
    if constexpr (!FINAL) {
      const float d1 = halves_sum(row_dot_acc<D>(dv, 1.f, true, vt, own + r, h));
      if (h == 0 && own + r < L) b.dv_delta[hd * ntok + base + (own + r) * rs] = d1;
    }
  }
  __syncthreads();  // every wave is done with every tile

  // this wave's rows leave through its own rows of the (now dead) tiles
  const int64_t wbase = base + own * rs;
  const int wl = L - own;  // >= 1: W = ceil(L / 32)
  const auto rdv = problem_rsrc(static_cast<const char*>(b.dv) + hoff * 2, wbase, rs, wl, D, 2);
  stage_rows<D, false>(qt + own * ROWB, qt + own * ROWB, dv, 1.f, rdv, rs, lane);
  const float sc = c * 0.6931471805599453f;  // dQ, dK = scale * dS K, dS^T Q
  if constexpr (FINAL) {
    const auto rdk = problem_rsrc(static_cast<const char*>(b.dk) + hoff * 2, wbase, rs, wl, D, 2);
    const auto rka = problem_rsrc(b.dk_in ? b.dk_in + hoff : b.dq, wbase, rs, wl, D, 4);
    stage_rows_add<D>(kt + own * ROWB, vt + own * ROWB, dk, sc, rdk, rka, b.dk_in != nullptr, rs, lane);
    const auto rdq = problem_rsrc(static_cast<const char*>(b.dq) + hoff * 2, wbase, rs, wl, D, 2);
    const auto rqa = problem_rsrc(b.dq_in ? b.dq_in + hoff : b.dk, wbase, rs, wl, D, 4);
    stage_rows_add<D>(gt + own * ROWB, qt + own * ROWB, dq, sc, rdq, rqa, b.dq_in != nullptr, rs, lane);
  } else {
    const auto rdk = problem_rsrc(static_cast<const char*>(b.dk) + hoff * 4, wbase, rs, wl, D, 4);
    stage_rows<D, true>(kt + own * ROWB, vt + own * ROWB, dk, sc, rdk, rs, lane);
    const auto rdq = problem_rsrc(static_cast<const char*>(b.dq) + hoff * 4, wbase, rs, wl, D, 4);
    stage_rows<D, true>(gt + own * ROWB, qt + own * ROWB, dq, sc, rdq, rs, lane);
  }
}

// Final-role form for problems of at most 64 rows (the row layout's stage-1
// blocks, b = 52) with half the LDS: two 32W-row tiles instead of four, and
// 256 registers, so that four workgroups (two waves per SIMD) share a CU.
// Phase (a) (lane = query) runs with K and V in the tiles and this wave's Q
// and G rows loaded straight into registers; dQ (bf16, plus dq_in) leaves
// through the tiles once every wave has read its own K and V rows into
// registers; Q and G are then copied into the same tiles (this wave's rows
// come back from L2) for phase (b) (lane = key), where lse and delta enter as
// a bias K-step (as bwd_dkdv MODE 1) and dV and dK take one sweep each (S is
// computed twice: the accumulators do not fit together). Measured at the row
// layout: 321 us against 433 us for bwd_group_kernel.
template <int D, int W>
__global__ void __launch_bounds__(64 * W, 2) bwd_group2_kernel(BwdArgs b) {
  constexpr int ROWB = D * 2, CPR = D / 8, RPI = 1024 / ROWB, IPW = 32 / RPI, TILE = 32 * W * ROWB;
  __shared__ __attribute__((aligned(1024))) char ta[TILE];
  __shared__ __attribute__((aligned(1024))) char tb[TILE];
  __shared__ __attribute__((aligned(16))) float xl[32 * W];
  __shared__ __attribute__((aligned(16))) float xd[32 * W];
  const GroupedArgs& a = b.g;
  const int p = blockIdx.x % a.problems, hd = blockIdx.x / a.problems;
  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int own = 32 * wave;
  const float c = a.scale_log2;
  const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, base, rs, L, D, 2);
  const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
  const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
  const auto rg = problem_rsrc(static_cast<const bf16*>(b.go) + hoff, base, rs, L, D, 2);
  auto copy = [&](char* t, __amdgpu_buffer_rsrc_t src) {  // this wave's 32 rows of a tile
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int row = own + RPI * i + lane / CPR;
      const int ch = (lane % CPR) ^ swz<D>(row);
      lds_dma16(src, t + (own + RPI * i) * ROWB, static_cast<uint32_t>((row * rs * D + ch * 8) * 2));
    }
  };
  copy(ta, rk);
  copy(tb, rv);
  bf16x8 kf[D / 16], vf[D / 16];
  {
    bf16x8 qf[D / 16], gf[D / 16];
    load_qfrag<D>(qf, rq, own, rs, lane);
    load_qfrag<D>(gf, rg, own, rs, lane);
    wait_dma();
    __syncthreads();
    const FlashOffsets<D> fo(0, lane, rs);

    // (a) lane = query own + r
    f32x16 s[W], dp[W];
#pragma unroll
    for (int kb = 0; kb < W; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s[kb] = mma(k_operand<D>(ta, fo, ks, kb), qf[ks], s[kb]);
        dp[kb] = mma(k_operand<D>(tb, fo, ks, kb), gf[ks], dp[kb]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < W; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (32 * kb + acc_key(i, h) >= L) s[kb][i] = -INFINITY;
        mx = fmaxf(mx, s[kb][i]);
      }
    mx = halves_max(mx) * c;
    float l = 0.f, pd = 0.f;
#pragma unroll
    for (int kb = 0; kb < W; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = fast_exp2(fmaf(s[kb][i], c, -mx));
        l += s[kb][i];
        pd = fmaf(s[kb][i], dp[kb][i], pd);
      }
    l = halves_sum(l);
    const float inv = 1.f / l;
    const float del = halves_sum(pd) * inv;
    if (h == 0) {
      xl[own + r] = mx + __builtin_amdgcn_logf(l);
      xd[own + r] = del;
    }
    f32x16 dq[D / 32];
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) dq[mt] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < W; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dp[kb][i] = s[kb][i] * inv * (dp[kb][i] - del);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 ds = p_operand(dp[kb], st);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) dq[mt] = mma(v_operand<D>(ta, fo, mt, 2 * kb + st), ds, dq[mt]);
      }
    }
    // this wave's K and V rows for (b), then the tiles are free
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = ld_bf16x8(ta + swoff<D>(own + r, 2 * ks + h));
      vf[ks] = ld_bf16x8(tb + swoff<D>(own + r, 2 * ks + h));
    }
    __syncthreads();
    const int64_t wbase = base + own * rs;
    const int wl = L - own;  // >= 1: W = ceil(L / 32)
    const auto rdq = problem_rsrc(static_cast<const char*>(b.dq) + hoff * 2, wbase, rs, wl, D, 2);
    const auto rqa = problem_rsrc(b.dq_in ? b.dq_in + hoff : b.dk, wbase, rs, wl, D, 4);
    stage_rows_add<D>(ta + own * ROWB, tb + own * ROWB, dq, c * 0.6931471805599453f, rdq, rqa,
                      b.dq_in != nullptr, rs, lane);
  }
  __syncthreads();  // every wave's staging reads are done: refill the tiles
  copy(ta, rq);
  copy(tb, rg);
  wait_dma();
  __syncthreads();

  // (b) lane = key own + r, in two sweeps over the query blocks (S again in
  // the second): dV (stored directly, the tiles are still in use), then dK;
  // S - lse/c and dP - delta come straight from the accumulators (bias K-step:
  // lane r of the A operand carries query 32qb + r)
  const int64_t wbase = base + own * rs;
  const int wl = L - own;
  const FlashOffsets<D> fo(0, lane, rs);
  const bf16x8 ones = bias_ones(h);
  const float inv_c = 1.f / c;
  {
    f32x16 dv[D / 32];
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) dv[mt] = f32x16{};
#pragma unroll
    for (int qb = 0; qb < W; ++qb) {
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) s = mma(k_operand<D>(ta, fo, ks, qb), kf[ks], s);
      s = mma(bias_operand(-xl[32 * qb + r] * inv_c, h), ones, s);
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = fast_exp2(s[i] * c);  // P
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 pp = p_operand(s, st);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) dv[mt] = mma(v_operand<D>(tb, fo, mt, 2 * qb + st), pp, dv[mt]);
      }
    }
    const auto rdv = problem_rsrc(static_cast<const char*>(b.dv) + hoff * 2, wbase, rs, wl, D, 2);
    store_rows<D>(rdv, false, rdv, false, r, rs, dv, 1.f, lane);
  }
  f32x16 dk[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dk[mt] = f32x16{};
#pragma unroll
  for (int qb = 0; qb < W; ++qb) {
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = mma(k_operand<D>(ta, fo, ks, qb), kf[ks], s);
      dp = mma(k_operand<D>(tb, fo, ks, qb), vf[ks], dp);
    }
    s = mma(bias_operand(-xl[32 * qb + r] * inv_c, h), ones, s);
    dp = mma(bias_operand(-xd[32 * qb + r], h), ones, dp);
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] *= fast_exp2(s[i] * c);  // dS = P (dP - delta)
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bf16x8 ps = p_operand(dp, st);
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) dk[mt] = mma(v_operand<D>(ta, fo, mt, 2 * qb + st), ps, dk[mt]);
    }
  }
  __syncthreads();  // every wave is done with both tiles
  const auto rdk = problem_rsrc(static_cast<const char*>(b.dk) + hoff * 2, wbase, rs, wl, D, 2);
  const auto rka = problem_rsrc(b.dk_in ? b.dk_in + hoff : b.dq, wbase, rs, wl, D, 4);
  stage_rows_add<D>(ta + own * ROWB, tb + own * ROWB, dk, c * 0.6931471805599453f, rdk, rka, b.dk_in != nullptr,
                    rs, lane);
}

// 8 consecutive elements of a row as floats (one 16-byte load for bf16, two
// for fp32)
template <bool F32>
__device__ __forceinline__ void load8(const void* base, int64_t e0, float (&x)[8]) {
  if constexpr (F32) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + e0);
    const u32x4 b = *reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + e0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = __uint_as_float(a[e]);
      x[4 + e] = __uint_as_float(b[e]);
    }
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(base) + e0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(a[e] << 16);
      x[2 * e + 1] = __uint_as_float(a[e] & 0xffff0000u);
    }
  }
}

// out[row] = sum over the D channels of a[row] * b[row]: D/8 lanes per row,
// 8 channels each (16-byte loads), reduced across the row's lanes
template <int D, bool FA, bool FB>
__global__ void __launch_bounds__(256) rowdot_kernel(const void* a, const void* bp, float* out, int64_t rows) {
  constexpr int LP = D / 8;
  const int64_t row = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / LP;
  const int sub = threadIdx.x % LP;
  const int64_t rr = row < rows ? row : rows - 1;
  const int64_t e0 = rr * D + sub * 8;
  float x[8], y[8];
  load8<FA>(a, e0, x);
  load8<FB>(bp, e0, y);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(x[e], y[e], acc);
#pragma unroll
  for (int off = LP / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LP);
  if (sub == 0 && row < rows) out[row] = acc;
}

}  // namespace

bool bwd_supported(const GroupedArgs& g) {
  return (g.D == 64 || g.D == 128) && g.qk_type == kBF16 && g.v_type == kBF16 && g.L >= 1 && g.q_row0 == 0 &&
         g.Lq == g.L &&
         (static_cast<int64_t>(g.L) + FBN) * g.row_stride * g.D * 4 < (int64_t{1} << 31);
}

hipError_t launch_bwd(const BwdArgs& b, hipStream_t s) {
  const GroupedArgs& g = b.g;
  if (!bwd_supported(g) || !b.go || !b.lse || !b.delta || !b.dq || !b.dk || !b.dv) return hipErrorInvalidValue;
  const int tiles = (g.L + FBM - 1) / FBM;
  const int64_t nwg = static_cast<int64_t>(tiles) * g.problems * g.heads;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  const unsigned grid = static_cast<unsigned>(nwg);
  if (g.D == 128) {
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(grid), dim3(FNT), 0, s, b, tiles, static_cast<int>(nwg));
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, 0>), dim3(grid), dim3(FNT), 0, s, b, tiles, static_cast<int>(nwg));
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, 1>), dim3(grid), dim3(FNT), 0, s, b, tiles, static_cast<int>(nwg));
  } else {
    hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(grid), dim3(FNT), 0, s, b, tiles, static_cast<int>(nwg));
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, 0>), dim3(grid), dim3(FNT), 0, s, b, tiles, static_cast<int>(nwg));
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, 1>), dim3(grid), dim3(FNT), 0, s, b, tiles, static_cast<int>(nwg));
  }
  return hipGetLastError();
}

bool bwd_small_supported(const GroupedArgs& g) {
  return (g.D == 64 || g.D == 128) && g.qk_type == kBF16 && g.v_type == kBF16 && g.L >= 1 && g.L <= 32 &&
         g.q_row0 == 0 && g.Lq == g.L && (static_cast<int64_t>(32) + 32) * g.row_stride * g.D * 4 < (int64_t{1} << 31);
}

hipError_t launch_bwd_small(const BwdArgs& b, hipStream_t s) {
  const GroupedArgs& g = b.g;
  if (!bwd_small_supported(g) || !b.go || !b.dq || !b.dk || !b.dv || !b.dv_delta) return hipErrorInvalidValue;
  const int64_t nwg = static_cast<int64_t>(g.problems) * g.heads;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (g.D == 128)
    hipLaunchKernelGGL(bwd_small_kernel<128>, dim3(static_cast<unsigned>(nwg)), dim3(64), 0, s, b);
  else
    hipLaunchKernelGGL(bwd_small_kernel<64>, dim3(static_cast<unsigned>(nwg)), dim3(64), 0, s, b);
  return hipGetLastError();
}

bool bwd_group_supported(const GroupedArgs& g) {
  return (g.D == 64 || g.D == 128) && g.qk_type == kBF16 && g.v_type == kBF16 && g.L >= 1 && g.L <= 128 &&
         g.q_row0 == 0 && g.Lq == g.L && (static_cast<int64_t>(128) + 32) * g.row_stride * g.D * 4 < (int64_t{1} << 31);
}

template <int D, bool FINAL>
hipError_t launch_bwd_group_t(const BwdArgs& b, hipStream_t s) {
  const GroupedArgs& g = b.g;
  const int64_t nwg = static_cast<int64_t>(g.problems) * g.heads;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(nwg));
  if constexpr (FINAL) {
    if (g.L <= 64) {
      if (g.L <= 32) hipLaunchKernelGGL((bwd_group2_kernel<D, 1>), grid, dim3(64), 0, s, b);
      else hipLaunchKernelGGL((bwd_group2_kernel<D, 2>), grid, dim3(128), 0, s, b);
      return hipGetLastError();
    }
  }
  switch ((g.L + 31) / 32) {
    case 1: hipLaunchKernelGGL((bwd_group_kernel<D, 1, FINAL>), grid, dim3(64), 0, s, b); break;
    case 2: hipLaunchKernelGGL((bwd_group_kernel<D, 2, FINAL>), grid, dim3(128), 0, s, b); break;
    case 3: hipLaunchKernelGGL((bwd_group_kernel<D, 3, FINAL>), grid, dim3(192), 0, s, b); break;
    default: hipLaunchKernelGGL((bwd_group_kernel<D, 4, FINAL>), grid, dim3(256), 0, s, b); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_group(const BwdArgs& b, hipStream_t s) {
  const GroupedArgs& g = b.g;
  if (!bwd_group_supported(g) || !b.go || !b.dq || !b.dk || !b.dv || b.dv_type != kBF16) return hipErrorInvalidValue;
  const bool final_role = b.dq_type == kBF16 && b.dk_type == kBF16;
  const bool partial_role = b.dq_type == kF32 && b.dk_type == kF32 && b.dv_delta && !b.dq_in && !b.dk_in;
  if (!final_role && !partial_role) return hipErrorInvalidValue;
  if (g.D == 128) return final_role ? launch_bwd_group_t<128, true>(b, s) : launch_bwd_group_t<128, false>(b, s);
  return final_role ? launch_bwd_group_t<64, true>(b, s) : launch_bwd_group_t<64, false>(b, s);
}

hipError_t launch_rowdot(const void* a, ElemType ta, const void* bp, ElemType tb, float* out, int64_t rows, int D,
                         hipStream_t s) {
  if (rows <= 0 || (D != 64 && D != 128)) return hipErrorInvalidValue;
  const int64_t threads = rows * (D / 8);
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 g(static_cast<unsigned>(grid)), blk(256);
  const bool fa = ta == kF32, fb = tb == kF32;
#define MONARCH_ROWDOT(DD, A, B) hipLaunchKernelGGL((rowdot_kernel<DD, A, B>), g, blk, 0, s, a, bp, out, rows)
  if (D == 128) {
    if (fa) { if (fb) MONARCH_ROWDOT(128, true, true); else MONARCH_ROWDOT(128, true, false); }
    else { if (fb) MONARCH_ROWDOT(128, false, true); else MONARCH_ROWDOT(128, false, false); }
  } else {
    if (fa) { if (fb) MONARCH_ROWDOT(64, true, true); else MONARCH_ROWDOT(64, true, false); }
    else { if (fb) MONARCH_ROWDOT(64, false, true); else MONARCH_ROWDOT(64, false, false); }
  }
#undef MONARCH_ROWDOT
  return hipGetLastError();
}

}  // namespace monarch
