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
#include "flash_common.h"

namespace monarch {
namespace {

using namespace mfma;

// max of three (one v_max3_f32)
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Fold a lane's tile maximum mx (raw scores) into the running maximum m
// (scaled), with lazy rescale of the accumulator and the row sum: m only moves
// when the tile's maximum exceeds it by more than the threshold.
template <int D>
__device__ __forceinline__ void fold_max(float mx, f32x16 (&o)[D / 32], float& m, float& l, float c) {
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

// Running max update with lazy rescale of the accumulator. The tile maximum
// is a max3 tree over the lane's 32 scores (16 instructions).
template <int D>
__device__ __forceinline__ void update_max(const f32x16 (&s)[2], f32x16 (&o)[D / 32], float& m, float& l, float c) {
  float t[12];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int a = 3 * i, b = 3 * i + 1, e = 3 * i + 2;
    t[i] = max3(s[a >> 4][a & 15], s[b >> 4][b & 15], s[e >> 4][e & 15]);
  }
  t[10] = s[1][14];
  t[11] = s[1][15];
  const float mx4 = max3(max3(t[0], t[1], t[2]), max3(t[3], t[4], t[5]), max3(t[6], t[7], t[8]));
  fold_max<D>(fmaxf(mx4, max3(t[9], t[10], t[11])), o, m, l, c);
}

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));

// l += a + b over a pair of bf16 weights (one v_dot2c_f32_bf16): the row sum
// then adds exactly the rounded weights the value product uses.
__device__ __forceinline__ float sum2(bf16x2 p, float l) {
  const bf16x2 one = {static_cast<bf16>(1.0f), static_cast<bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(p, one, l, false);
}

template <int D>
__device__ __forceinline__ void scores64(f32x16 (&s)[2], const char* kl, const FlashOffsets<D>& fo,
                                         const bf16x8 (&qf)[D / 16]) {
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    s[0] = mma(k_operand<D>(kl, fo, ks, 0), qf[ks], s[0]);
    s[1] = mma(k_operand<D>(kl, fo, ks, 1), qf[ks], s[1]);
  }
}

// Scores of the next tile interleaved with the probabilities of the current
// one: each 16-channel step (two MFMAs, K read one step ahead) carries a
// slice of the exponentials; sched_barrier keeps the steps apart so the
// compiler does not regroup all MFMAs first. hook(ks) runs after step ks's
// MFMAs are issued (the caller's tile copies go there).
template <int D, bool PIN, typename Hook, int NP = 32>
__device__ __forceinline__ void scores_with_probs(f32x16 (&sn)[2], const char* kl, const FlashOffsets<D>& fo,
                                                  const bf16x8 (&qf)[D / 16], const f32x16 (&s)[2],
                                                  bf16x8 (&pb)[4], float& l, float c, float m, Hook&& hook) {
  // NP: weights (of the lane's 32) computed here, the first NP; the rest in the value product
  constexpr int KS = D / 16;
  constexpr int PER = NP / KS;  // weights per step, even
  static_assert(PER % 2 == 0 && NP % 8 == 0, "whole weight pairs per step, whole PV steps");
  sn[0] = f32x16{};
  sn[1] = f32x16{};
  bf16x2 pp[16];
  bf16x8 a0 = k_operand<D>(kl, fo, 0, 0), a1 = k_operand<D>(kl, fo, 0, 1);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 n0 = a0, n1 = a1;
    if (ks + 1 < KS) {
      n0 = k_operand<D>(kl, fo, ks + 1, 0);
      n1 = k_operand<D>(kl, fo, ks + 1, 1);
    }
    sn[0] = mma(a0, qf[ks], sn[0]);
    sn[1] = mma(a1, qf[ks], sn[1]);
    hook(ks);
#pragma unroll
    for (int e = 0; e < PER; e += 2) {
      const int i = ks * PER + e;
      const float z0 = fmaf(s[i >> 4][i & 15], c, -m), z1 = fmaf(s[(i + 1) >> 4][(i + 1) & 15], c, -m);
      const float p0 = fast_exp2(z0);
      const float p1 = fast_exp2(z1);
      pp[i >> 1] = bf16x2{static_cast<bf16>(p0), static_cast<bf16>(p1)};
      l = sum2(pp[i >> 1], l);
      // pin the weights to this step: without it the compiler sinks every
      // exponential of the tile below the last score MFMA in one of the two
      // unrolled steps, and that step loses its MFMA/VALU overlap (left out
      // where the extra register pressure would spill)
      if constexpr (PIN) asm volatile("" : "+v"(pp[i >> 1]));
    }
    __builtin_amdgcn_sched_barrier(0);
    a0 = n0;
    a1 = n1;
  }
#pragma unroll
  for (int st = 0; st < NP / 8; ++st)
    pb[st] = __builtin_shufflevector(__builtin_shufflevector(pp[4 * st], pp[4 * st + 1], 0, 1, 2, 3),
                                     __builtin_shufflevector(pp[4 * st + 2], pp[4 * st + 3], 0, 1, 2, 3), 0, 1, 2,
                                     3, 4, 5, 6, 7);
}

// exp2(s*c - m) as bf16 B operands for the four 16-key PV steps (last tile)
__device__ __forceinline__ void probs(const f32x16 (&s)[2], bf16x8 (&pb)[4], float& l, float c, float m) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    bf16x2 pp[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float z0 = fmaf(s[st >> 1][8 * (st & 1) + e], c, -m);
      const float z1 = fmaf(s[st >> 1][8 * (st & 1) + e + 1], c, -m);
      const float p0 = fast_exp2(z0);
      const float p1 = fast_exp2(z1);
      pp[e >> 1] = bf16x2{static_cast<bf16>(p0), static_cast<bf16>(p1)};
      l = sum2(pp[e >> 1], l);
    }
    pb[st] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                     __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// O^T += V^T P^T over `steps` 16-key steps, next step's V^T read one step ahead
template <int D>
__device__ __forceinline__ void pv64(f32x16 (&o)[D / 32], const char* vl, const FlashOffsets<D>& fo,
                                     const bf16x8 (&pb)[4], int steps) {
  constexpr int MT = D / 32;
  bf16x8 v[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) v[mt] = v_operand<D>(vl, fo, mt, 0);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if (st < steps) {
      bf16x8 nv[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) nv[mt] = (st + 1 < 4) ? v_operand<D>(vl, fo, mt, st + 1) : v[mt];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] = mma(v[mt], pb[st], o[mt]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) v[mt] = nv[mt];
    }
  }
}

// pv64 over all four steps with the maximum of the next tile's raw scores sm
// taken on the side: each step's four MFMAs carry a max over 8 of the lane's
// 32 scores (5 VALU instructions), so the max tree runs while the matrix core
// works instead of in front of the next tile's exponentials.
// NP < 32: the weights NP..31 of the current tile (scores s) are computed here,
// 8 per step in the first steps, each just before the PV step that takes them.
template <int D, int NP = 32>
__device__ __forceinline__ void pv64_max(f32x16 (&o)[D / 32], const char* vl, const FlashOffsets<D>& fo,
                                         bf16x8 (&pb)[4], const f32x16 (&sm)[2], float& mx, const f32x16 (&s)[2],
                                         float& l, float c, float m) {
  constexpr int MT = D / 32;
  bf16x8 v[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) v[mt] = v_operand<D>(vl, fo, mt, 0);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    bf16x8 nv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) nv[mt] = (st + 1 < 4) ? v_operand<D>(vl, fo, mt, st + 1) : v[mt];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = mma(v[mt], pb[st], o[mt]);
    if (NP / 8 + st < 4) {
      // weights of PV step NP / 8 + st
      const int ps = NP / 8 + st;
      bf16x2 pp[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float z0 = fmaf(s[ps >> 1][8 * (ps & 1) + e], c, -m);
        const float z1 = fmaf(s[ps >> 1][8 * (ps & 1) + e + 1], c, -m);
        pp[e >> 1] = bf16x2{static_cast<bf16>(fast_exp2(z0)), static_cast<bf16>(fast_exp2(z1))};
        l = sum2(pp[e >> 1], l);
      }
      pb[ps] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                       __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    }
    const int t = st >> 1, b = 8 * (st & 1);
    const float q = max3(max3(sm[t][b], sm[t][b + 1], sm[t][b + 2]), max3(sm[t][b + 3], sm[t][b + 4], sm[t][b + 5]),
                         fmaxf(sm[t][b + 6], sm[t][b + 7]));
    mx = st == 0 ? q : fmaxf(mx, q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) v[mt] = nv[mt];
  }
}

// Key biases (refinement step): the 64 biases of a key tile (bits, fp32) come
// into LDS beside the tile's values, one 4-byte copy per lane issued by wave 0;
// each lane then turns its raw scores into logits in bits, c s + bias, for its
// keys 32 t + acc_key(i, h) (four consecutive keys per 16-byte read).
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t src, float* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)lds, 4, voff, 0, 0, 0);
#else
  (void)src; (void)lds; (void)voff;
#endif
}

__device__ __forceinline__ void add_kbias(f32x16 (&s)[2], const float* kb, int h, float c) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 b = *reinterpret_cast<const float4*>(kb + 32 * t + 8 * g + 4 * h);
      s[t][4 * g + 0] = fmaf(s[t][4 * g + 0], c, b.x);
      s[t][4 * g + 1] = fmaf(s[t][4 * g + 1], c, b.y);
      s[t][4 * g + 2] = fmaf(s[t][4 * g + 2], c, b.z);
      s[t][4 * g + 3] = fmaf(s[t][4 * g + 3], c, b.w);
    }
}

// Weights of a tile (of a lane's 32) computed beside the next tile's score
// MFMAs; the other 16 are computed beside the first two value-product steps,
// which balances the VALU work between the two MFMA phases (ABBA on one box,
// all 32 beside the scores -> 16: frame stage 1 -0.6%, row stage 2 -1.5%,
// dense -0.3%; bitwise the same results)
constexpr int kScoreWeights = 16;

// Wave priority while issuing MFMA-heavy phases (MONARCH_PRIO): 0 = never
// raised; 1 = raised for the value product; 2 = raised for scores + values
// (measured best: the two waves sharing a SIMD then tend to alternate
// between their MFMA and softmax phases instead of colliding).
#ifndef MONARCH_PRIO
#define MONARCH_PRIO 2
#endif

// Mutable per-wave state of the flash loop (the raw scores of the current
// tile alternate between two register sets, sa and sb, so that no copy is
// needed between iterations).
template <int D>
struct FlashState {
  f32x16 o[D / 32];  // O^T accumulators
  float m, l;        // running max (scaled) and partial sum
};

// Query tile qt (rows qt*qrows .. +qrows, qrows a multiple of 32 and at most
// 32*NW) of problem p of head hd, computed by NW waves: wave w owns rows
// 32w .. 32w+31 of the tile and all NW waves share the tile copies. The LDS
// slots are four separate __shared__ arrays of the calling kernel (not
// fields of one): the compiler then proves that reads of one slot never
// alias the asynchronous copy into another and waits for the copies only at
// the barriers. Every copy it issues has completed when it returns; waves
// whose rows lie outside the tile or past the end of the problem only copy,
// and return early (after the last barrier).
//
// KB (key biases, bf16 output only): logits are c <q, k> + kbias[key] in bits;
// kb0 / kb1 are two 64-float LDS slots that alternate like v0 / v1.
template <int D, bool OUT_F32, int POLICY = 0, int NW = 4, bool DELTA = false, bool ENT = false, bool KB = false>
__device__ __forceinline__ void flash_tile(const GroupedArgs& a, int hd, int p, int qt, int qrows, char* k0,
                                           char* k1, char* v0, char* v1, int tid, float* kb0 = nullptr,
                                           float* kb1 = nullptr) {
  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L;
  // query rows: q_row0 .. q_row0 + Lq - 1 of the problem (qbase is the first)
  const int64_t qbase = base + a.q_row0 * rs;
  const int Lq = a.Lq;
  const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, qbase, rs, Lq, D, 2);
  const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
  const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
  const auto ro = problem_rsrc(static_cast<const char*>(a.o) + hoff * (OUT_F32 ? 4 : 2), qbase, rs, Lq, D,
                               OUT_F32 ? 4 : 2);

  const int lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: copy addresses stay scalar
  const int row0 = qt * qrows + wave * 32;
  const bool active = wave * 32 < qrows && row0 < Lq;
  const int n = (L + FBN - 1) / FBN;
  const int nv_last = L - (n - 1) * FBN;
  const float c = a.scale_log2;
  // with key biases the scores are logits in bits once the biases are added,
  // so the softmax below runs with scale 1
  const float cs = KB ? 1.f : c;
  const FlashOffsets<D> fo(wave, lane, rs);  // LDS read offsets
  const TileDma<D, NW> td(wave, lane, rs);
  const uint32_t tile_bytes = static_cast<uint32_t>(FBN * rs * D * 2);
  const auto rb = problem_rsrc(KB ? static_cast<const void*>(a.kbias + hd * (a.head_elems / D)) : a.k, base, rs,
                               L, 1, 4);  // key biases (unused without KB)
  const uint32_t kb_lane = static_cast<uint32_t>(lane * rs * 4);
  const uint32_t kb_tile = static_cast<uint32_t>(FBN * rs * 4);

  // prologue: K tiles 0 and 1, V tile 0 (and its key biases)
  td.dma(k0, rk, 0, wave);
  td.dma(v0, rv, 0, wave);
  if constexpr (KB) {
    if (wave == 0) lds_dma4(rb, kb0, kb_lane);
  }
  if (n > 1) td.dma(k1, rk, tile_bytes, wave);
  bf16x8 qf[D / 16];
  load_qfrag<D>(qf, rq, row0, rs, lane);
  FlashState<D> st;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) st.o[mt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  wait_dma();
  __syncthreads();

  // EM: the maximum of each tile's scores is taken during the previous tile's
  // value product (pv64_max; measured 1-2% faster than a max tree at the start
  // of the tile's own step); with key biases it must wait for the biases, so
  // it is taken at the start of the tile's own step
  constexpr bool EM = !KB;
  f32x16 sa[2], sb[2];
  if (active) scores64<D>(sa, k0, fo, qf);
  if (EM && active) update_max<D>(sa, st.o, st.m, st.l, cs);
  // iteration 0 refills K slot 0 (tile 0): every wave must be done with it
  __syncthreads();

  // Iteration j: copy K_{j+2} into kdma and V_{j+1} into vdma (global ->
  // LDS, asynchronous), then the scores of tile j+1 (into sn) from kread
  // while the softmax of tile j (scores s) runs, then its value product from
  // vread. The four LDS slots are distinct fields so the compiler can see
  // that the reads never touch the tiles being copied and does not wait for
  // the copies first.
  auto step = [&](int j, char* kdma, char* vdma, const char* kread, const char* vread, float* kbdma,
                  const float* kbread, f32x16 (&s)[2], f32x16 (&sn)[2]) {
    // copies of V_{j+1} and K_{j+2}: waves without rows issue them here,
    // the others between their score steps (below)
    const bool kc = j + 2 < n;
    if constexpr (KB) {
      if (wave == 0) lds_dma4(rb, kbdma, (j + 1) * kb_tile + kb_lane);
    }
    if (!active) td.dma(vdma, rv, (j + 1) * tile_bytes, wave);
    if (!active && kc) td.dma(kdma, rk, (j + 2) * tile_bytes, wave);
    if (active) {
      if constexpr (KB) add_kbias(s, kbread, h, c);
      if constexpr (!EM) update_max<D>(s, st.o, st.m, st.l, cs);
      bf16x8 pb[4];
#if MONARCH_PRIO == 2
      __builtin_amdgcn_s_setprio(1);
#endif
      // the wave's copy instructions go one per score step (V's first, then
      // K's) instead of back to back before them: stage 1 at the frame shape
      // measured 1.7% faster
      auto copy_hook = [&](int ks) {
        constexpr int IPW = TileDma<D, NW>::IPW;
        static_assert(2 * IPW <= D / 16, "one copy instruction per score step");
        if (ks < IPW) td.dma1(vdma, rv, (j + 1) * tile_bytes, wave, ks);
        if (ks >= IPW && ks < 2 * IPW && kc) td.dma1(kdma, rk, (j + 2) * tile_bytes, wave, ks - IPW);
      };
      scores_with_probs<D, !OUT_F32 && !DELTA && !KB && POLICY == 0, decltype(copy_hook)&, EM ? kScoreWeights : 32>(
          sn, kread, fo, qf, s, pb, st.l, cs, st.m, copy_hook);

#if MONARCH_PRIO == 1
      __builtin_amdgcn_s_setprio(1);
#endif
      if constexpr (EM) {
        // the last tile's keys past the end are masked before its maximum is taken
        if (j + 2 == n && nv_last < FBN) mask_tail(sn, nv_last, h);
        float mx;
        pv64_max<D, kScoreWeights>(st.o, vread, fo, pb, sn, mx, s, st.l, cs, st.m);
#if MONARCH_PRIO
        __builtin_amdgcn_s_setprio(0);
#endif
        fold_max<D>(mx, st.o, st.m, st.l, cs);
      } else {
        pv64<D>(st.o, vread, fo, pb, 4);
#if MONARCH_PRIO
        __builtin_amdgcn_s_setprio(0);
#endif
      }
    }
    wait_dma();
    __syncthreads();
  };

  // steady state, two iterations per trip so every slot is a fixed array:
  // even j copies into (k0, v1) and reads (k1, v0), scores sa -> sb; odd j
  // the reverse
  int j = 0;
  for (; j + 2 < n; j += 2) {
    step(j, k0, v1, k1, v0, kb1, kb0, sa, sb);
    step(j + 1, k1, v0, k0, v1, kb0, kb1, sb, sa);
  }
  const bool odd = j + 1 < n;
  if (odd) step(j, k0, v1, k1, v0, kb1, kb0, sa, sb);

  if (!active) return;
  // last tile: mask keys past the end, skip the empty half of the PV product
  f32x16 sl[2] = {odd ? sb[0] : sa[0], odd ? sb[1] : sa[1]};
  if constexpr (!EM) {
    if constexpr (KB) add_kbias(sl, ((n - 1) & 1) ? kb1 : kb0, h, c);
    if (nv_last < FBN) mask_tail(sl, nv_last, h);
    update_max<D>(sl, st.o, st.m, st.l, cs);
  }
  bf16x8 pb[4];
  probs(sl, pb, st.l, cs, st.m);
  pv64<D>(st.o, ((n - 1) & 1) ? v1 : v0, fo, pb, nv_last > 32 ? 4 : 2);

  const float lsum = halves_sum(st.l);  // both lane halves of a row are active together
  // lane-derived indices made opaque here, so that no address below is
  // computed before the loop and kept live across it (that spilled)
  int r = lane & 31;
  asm volatile("" : "+v"(r));
  if (a.lse && h == 0 && row0 + r < Lq)
    a.lse[hd * (a.head_elems / D) + qbase + (row0 + r) * rs] = st.m + __builtin_amdgcn_logf(lsum);
  if constexpr (ENT) {
    // Entropy in bits of the row's weights p_k = 2^(c s_k - m) / l: log2 l minus the
    // weighted mean of (c s_k - m). The values of this pass are the keys (flash_supported),
    // so sum_k p_k s_k = <q, sum_k p_k k_k> = <q, O_acc>: the weighted sum is
    // c <q, O_acc> - m l, one dot product per row at the end instead of a term per score
    // in the loop. q is read in the accumulator layout (register i of tile mt: channel
    // 32 mt + 8 (i / 4) + 4 h + i % 4), 4 channels (8 bytes) at a time.
    const uint32_t rowel = static_cast<uint32_t>(row0 + r) * static_cast<uint32_t>(rs * D);
    float acc = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 qv = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rq, static_cast<int>((rowel + 32 * mt + 8 * g + 4 * h) * 2), 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t bits = (e & 1) ? (qv[e >> 1] & 0xffff0000u) : (qv[e >> 1] << 16);
          acc = fmaf(st.o[mt][4 * g + e], __uint_as_float(bits), acc);
        }
      }
    const float w = fmaf(c, halves_sum(acc), -st.m * lsum);
    if (h == 0 && row0 + r < Lq)
      a.ent[hd * (a.head_elems / D) + qbase + (row0 + r) * rs] = __builtin_amdgcn_logf(lsum) - w / lsum;
  }
  if constexpr (DELTA) {
    // delta of this lane's query row instead of O: the sum over channels of G
    // times O (fp32, before any rounding); register i of tile mt holds channel
    // 32 mt + 8 (i / 4) + 4 h + i % 4, read from G 4 channels (8 bytes) at a time
    const auto rg = problem_rsrc(static_cast<const bf16*>(a.dg) + hoff, qbase, rs, Lq, D, 2);
    const uint32_t rowel = static_cast<uint32_t>(row0 + r) * static_cast<uint32_t>(rs * D);
    const float inv = 1.f / lsum;
    float acc = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 gv = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, static_cast<int>((rowel + 32 * mt + 8 * g + 4 * h) * 2), 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t bits = (e & 1) ? (gv[e >> 1] & 0xffff0000u) : (gv[e >> 1] << 16);
          acc = fmaf(st.o[mt][4 * g + e] * inv, __uint_as_float(bits), acc);
        }
      }
    const float d = halves_sum(acc);
    if (h == 0 && row0 + r < Lq) a.delta[hd * (a.head_elems / D) + qbase + (row0 + r) * rs] = d;
  } else if constexpr (OUT_F32) {
    // fp32 rows (4 D bytes each) staged 16 at a time through this wave's
    // half of a K slot, then stored whole
    char* stage = (wave < 2 ? k0 : k1) + (wave & 1) * 32 * (D * 2);
    const uint32_t row_bytes = static_cast<uint32_t>(rs * D * 4);  // offsets fit 32 bits (offsets_fit)
    if constexpr (POLICY == 0)
      stage_rows_f32_halves<D>(stage, st.o, 1.f / lsum, ro, rs, lane, static_cast<uint32_t>(row0) * row_bytes);
    else
      store_out<D, true, POLICY>(ro, row0 + r, rs, st.o, 1.f / lsum, lane);
  } else {
    // Stage this wave's 32 rows in its own half of a K slot (no wave reads K
    // after the loop), swizzled, then store whole rows (16-byte pieces of
    // 256-byte rows, four rows per instruction) instead of 8-byte pieces of 32
    // rows. Only this wave touches its half: the LDS ops of one wave run in
    // order, the wait and the wave barrier keep the compiler from moving the
    // reads above the writes.
    constexpr int ROWB = D * 2, CPR = D / 8, RPI = 64 / CPR;
    char* stage = (wave < 2 ? k0 : k1) + (wave & 1) * 32 * ROWB;
    int lr = lane / CPR;
    asm volatile("" : "+v"(lr));
    const float inv = 1.f / lsum;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(st.o[mt][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(stage + swoff<D>(r, 4 * mt + g) + 8 * h) = v;
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    const uint32_t row_bytes = static_cast<uint32_t>(rs * D * 2);  // offsets fit 32 bits (offsets_fit)
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int rr = RPI * i + lr, chk = lane % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + swoff<D>(rr, chk));
      const uint32_t off = static_cast<uint32_t>(row0 + rr) * row_bytes + static_cast<uint32_t>(chk * 16);
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, static_cast<int>(off), 0, POLICY);
    }
  }
}

// Waves per workgroup of the flash kernel: four (two workgroups per CU).
// Eight-wave workgroups halve the tile copies per CU but measured slower:
// the two waves sharing a SIMD then belong to one workgroup and meet at
// every barrier, so their MFMA and softmax phases stop overlapping.
constexpr int kFlashWaves = 4;

template <int D, bool OUT_F32, bool DELTA = false, bool ENT = false, bool KB = false>
__global__ void __launch_bounds__(64 * kFlashWaves, 2) flash_kernel(GroupedArgs a, int qtiles, int qrows, int nwg) {
  using T = SwTile<D>;
  __shared__ __attribute__((aligned(1024))) char k0[T::bytes];
  __shared__ __attribute__((aligned(1024))) char k1[T::bytes];
  __shared__ __attribute__((aligned(1024))) char v0[T::bytes];
  __shared__ __attribute__((aligned(1024))) char v1[T::bytes];
  const int id = xcd_order(blockIdx.x, nwg);
  // the workgroup's tile, problem and head are uniform: readfirstlane keeps them and the
  // addresses derived from them in scalar registers (the integer divisions run on the vector
  // unit, and vector copies of these values were spilled across the loop)
  const int qt = __builtin_amdgcn_readfirstlane(id % qtiles);
  const int rest = id / qtiles;
  const int p = __builtin_amdgcn_readfirstlane(rest % a.problems);
  const int hd = __builtin_amdgcn_readfirstlane(rest / a.problems);
  if constexpr (KB) {
    __shared__ __attribute__((aligned(256))) float kb0[FBN];
    __shared__ __attribute__((aligned(256))) float kb1[FBN];
    flash_tile<D, OUT_F32, 0, kFlashWaves, DELTA, ENT, true>(a, hd, p, qt, qrows, k0, k1, v0, v1, threadIdx.x, kb0,
                                                             kb1);
  } else {
    flash_tile<D, OUT_F32, 0, kFlashWaves, DELTA, ENT>(a, hd, p, qt, qrows, k0, k1, v0, v1, threadIdx.x);
  }
}

// ---------------------------------------------------------------- group
// One problem (at most 128 rows) per workgroup, one wave per 32 query rows.
// Q, K and V rows are copied global -> LDS whole (each DMA instruction moves
// four 256-byte rows), scores and values run from LDS, and O goes back
// through LDS so that it leaves as whole 256-byte rows too. Every global
// access is a full-row, coalesced 16-byte-per-lane access: for stage-2
// groups (rows a block apart) this is what keeps the L2 request count down.
template <int D, int QT>
struct GroupCfg {
  static constexpr int BN = 32 * QT;       // rows per tile (keys = queries)
  static constexpr int NT = 64 * QT;       // one wave per 32 query rows
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int tile = BN * ROWB;
  static constexpr int RPI = 1024 / ROWB;  // rows per DMA instruction
  static constexpr int IPW = 32 / RPI;     // DMA instructions per wave per tile
  // waves per SIMD the register budget aims at: two unless the three tiles
  // already keep a second workgroup off the CU (128-row tiles at d = 128)
  static constexpr int MINW = 3 * tile <= 80 * 1024 ? 2 : 1;
};

// SR = 0: each tile holds 32 QT rows. SR = 24 (one wave, problems of at most
// 24 rows): the three tiles hold 24 rows each and sit back to back, followed
// by 8 zero rows, so the MFMAs' 32-row reads of a tile run into the next
// tile's first rows (finite values: keys past the end are masked, query rows
// past the end are not stored) and, for the values, into the zero rows (keys
// past the end have weight 0). The smaller footprint (20 KB instead of 24 KB
// at d = 128) lets eight workgroups share a CU instead of six.
template <int D, int QT, bool OUT_F32, int SR>
__device__ __forceinline__ void group_body(const GroupedArgs& a, char* ql, char* kl, char* vl) {
  using G = GroupCfg<D, QT>;
  static_assert(SR == 0 || QT == 1, "short tiles: one wave");
  constexpr int IPW = (SR ? SR : 32) / G::RPI;  // DMA instructions per tile of this wave
  const int p = blockIdx.x % a.problems;
  const int hd = blockIdx.x / a.problems;
  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L;
  // queries (and outputs): rows q_row0 .. q_row0 + Lq - 1; keys, values: rows 0 .. L - 1
  const int64_t qbase = base + a.q_row0 * rs;
  const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, qbase, rs, a.Lq, D, 2);
  const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
  const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
  const auto ro = problem_rsrc(static_cast<const char*>(a.o) + hoff * (OUT_F32 ? 4 : 2), qbase, rs, a.Lq, D,
                               OUT_F32 ? 4 : 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;

  // wave w copies rows 32w .. 32w+31 of Q, K and V (rows past L read as zero;
  // short tiles: rows 0 .. SR-1)
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = 32 * wave + G::RPI * i + lane / G::CPR;
    const int c = (lane % G::CPR) ^ swz<D>(row);
    const uint32_t goff = static_cast<uint32_t>((row * rs * D + c * 8) * 2);
    const int dst = (32 * wave + G::RPI * i) * G::ROWB;
    lds_dma16(rq, ql + dst, goff);
    lds_dma16(rk, kl + dst, goff);
    lds_dma16(rv, vl + dst, goff);
  }
  wait_dma();
  __syncthreads();

  const int r = 32 * wave + (lane & 31);  // this lane's query row
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = ld_bf16x8(ql + swoff<D>(r, 2 * ks + h));

  float c = a.scale_log2;
  f32x16 s[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    s[t] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      s[t] = mma(ld_bf16x8(kl + swoff<D>(32 * t + (lane & 31), 2 * ks + h)), qf[ks], s[t]);
  }
  const int64_t rows_off = static_cast<int64_t>(hd) * (a.head_elems / D);
  if (a.kbias) {
    // logits in bits with the per-key bias added; the scale is then already applied
    const float* kb = a.kbias + rows_off + base;
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * t + acc_key(i, h);
        if (key < L) s[t][i] = fmaf(s[t][i], c, kb[key * rs]);
      }
    c = 1.f;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < QT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (32 * t + acc_key(i, h) >= L) s[t][i] = -INFINITY;
      mx = fmaxf(mx, s[t][i]);
    }
  mx = halves_max(mx) * c;
  // l: the softmax denominator; wsum: sum of p * (logit - max) in bits (for the entropy)
  float l = 0.f, wsum = 0.f;
  const bool want_ent = a.ent != nullptr;
#pragma unroll
  for (int t = 0; t < QT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float z = fmaf(s[t][i], c, -mx);
      s[t][i] = fast_exp2(z);
      l += s[t][i];
      if (want_ent && s[t][i] > 0.f) wsum = fmaf(s[t][i], z, wsum);
    }
  f32x16 o[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};
  const int j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int st = 0; st < 2 * QT; ++st) {
    const bf16x8 pb = p_operand(s[st >> 1], st & 1);
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) {
      // V^T operand: keys 16*st + 4*(g/2) + j/4 (+8), channels 32*mt + 16*(g%2) + 4*(j%4) + 0..3
      const int row = 16 * st + 4 * (g >> 1) + (j >> 2);
      const int ch = 32 * mt + 16 * (g & 1) + 4 * (j & 3);
      const char* p0 = vl + swoff<D>(row, ch / 8) + (ch % 8) * 2;
      const char* p1 = vl + swoff<D>(row + 8, ch / 8) + (ch % 8) * 2;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
      o[mt] = mma(__builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)), pb, o[mt]);
    }
  }
  const float lsum = halves_sum(l);
  const float inv = 1.f / lsum;
  if (a.lse && h == 0 && r < a.Lq) a.lse[rows_off + qbase + r * rs] = mx + __builtin_amdgcn_logf(lsum);
  if (want_ent) {
    const float w = halves_sum(wsum);
    if (h == 0 && r < a.Lq) a.ent[rows_off + qbase + r * rs] = __builtin_amdgcn_logf(lsum) - w * inv;
  }
  if constexpr (OUT_F32) {
    store_out<D, true>(ro, r, rs, o, inv, lane);
  } else {
    // stage O in this wave's own Q rows (row-major, swizzled), then write
    // whole rows: 16 lanes x 16 bytes per 256-byte row
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(o[mt][4 * gg + e] * inv);
        *reinterpret_cast<bf16x4*>(ql + swoff<D>(r, 4 * mt + gg) + 8 * h) = v;
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32 * G::CPR / 64; ++i) {
      const int idx = 64 * i + lane;
      const int row = 32 * wave + idx / G::CPR, chk = idx % G::CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ql + swoff<D>(row, chk));
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, static_cast<int>((row * rs * D + chk * 8) * 2), 0, 0);
    }
  }
}

template <int D, int QT, bool OUT_F32>
__global__ void __launch_bounds__((GroupCfg<D, QT>::NT), (GroupCfg<D, QT>::MINW)) group_kernel(GroupedArgs a) {
  using G = GroupCfg<D, QT>;
  __shared__ __attribute__((aligned(1024))) char ql[G::tile];
  __shared__ __attribute__((aligned(1024))) char kl[G::tile];
  __shared__ __attribute__((aligned(1024))) char vl[G::tile];
  group_body<D, QT, OUT_F32, 0>(a, ql, kl, vl);
}

constexpr int kShortRows = 24;

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(64, 2) group_short_kernel(GroupedArgs a) {
  constexpr int ROWB = D * 2, TB = kShortRows * ROWB, PADB = 8 * ROWB;
  __shared__ __attribute__((aligned(1024))) char lds[3 * TB + PADB];
  // the 8 rows after the value tile read as zero
  const int lane = threadIdx.x;
#pragma unroll
  for (int i = 0; i < PADB / 1024; ++i)
    *reinterpret_cast<u32x4*>(lds + 3 * TB + 1024 * i + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
  group_body<D, 1, OUT_F32, kShortRows>(a, lds, lds + TB, lds + 2 * TB);
}

// ---------------------------------------------------------------- fused
// Both stages in one launch (fused_grid_kernel below): stage-1 query tiles
// (as flash_kernel) and stage-2 chunks of kFusedGroups groups (m_tau <= 32
// rows each).
//
// Y crosses XCDs, whose L2 caches are not coherent with one another. It is
// written with device-scope stores (written through the L2) and read with
// device-scope loads, so no L2 writeback or invalidation is needed (each
// costs a whole-L2 operation).
//
// Control block (ints): [0, 16) the per-XCD claim words (8 x 64 bits),
// [16] error, [32, ...) ready counters, one per (head, tile), 32 ints apart.
constexpr int kFusedXcds = 8;
constexpr int kFusedGroups = 16;  // stage-2 groups per work item, 4 per wave
constexpr int kCtlError = 2 * kFusedXcds;
constexpr int kCtlReady = 2 * kFusedXcds + 16;

__global__ void __launch_bounds__(256) fused_reset(int* ctl, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) ctl[i] = 0;
}

// One stage-2 group (2 <= L <= 32 rows) by one wave: K and Y rows copied into
// this wave's LDS (two swizzled 32-row tiles), the Q fragment read directly,
// one pass, O written directly.
template <int D>
__device__ __forceinline__ void group_wave(const GroupedArgs& a, int hd, int p, char* kl, char* vl,
                                           const FlashOffsets<D>& fo, int lane, bool poison) {
  constexpr int ROWB = D * 2, CPR = D / 8, RPI = 1024 / ROWB;
  const int64_t hoff = static_cast<int64_t>(hd) * a.head_elems;
  const int64_t base = problem_base(a, p);
  const int64_t rs = a.row_stride;
  const int L = a.L, h = lane >> 5;
  const auto rq = problem_rsrc(static_cast<const bf16*>(a.q) + hoff, base, rs, L, D, 2);
  const auto rk = problem_rsrc(static_cast<const bf16*>(a.k) + hoff, base, rs, L, D, 2);
  const auto rv = problem_rsrc(static_cast<const bf16*>(a.v) + hoff, base, rs, L, D, 2);
  const auto ro = problem_rsrc(static_cast<const bf16*>(a.o) + hoff, base, rs, L, D, 2);
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + lane / CPR;
    const int c = (lane % CPR) ^ swz<D>(row);
    const uint32_t goff = static_cast<uint32_t>((row * rs * D + c * 8) * 2);
    lds_dma16(rk, kl + RPI * i * ROWB, goff);
    lds_dma16<kPolicyDevice>(rv, vl + RPI * i * ROWB, goff);  // Y, written by other XCDs
  }
  bf16x8 qf[D / 16];
  load_qfrag<D>(qf, rq, 0, rs, lane);
  wait_dma();
  f32x16 s = {};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) s = mma(ld_bf16x8(kl + fo.k[ks]), qf[ks], s);
  const float c = a.scale_log2;
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (acc_key(i, h) >= L) s[i] = -INFINITY;
    mx = fmaxf(mx, s[i]);
  }
  mx = halves_max(mx) * c;
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s[i] = fast_exp2(fmaf(s[i], c, -mx));
    l += s[i];
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const bf16x8 pb = p_operand(s, st);
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) o[mt] = mma(v_operand<D>(vl, fo, mt, st), pb, o[mt]);
  }
  // poison: the wait for this group's Y timed out, so its rows are written as NaN (a quiet
  // NaN bit pattern the compiler cannot see through: kernels build without NaN semantics)
  float inv = 1.f / halves_sum(l);
  if (poison) {
    uint32_t nan_bits = 0x7fc00000u;
    asm volatile("" : "+v"(nan_bits));
    inv = __uint_as_float(nan_bits);
  }
  store_out<D, false>(ro, lane & 31, rs, o, inv, lane);
}

// Both stages in one launch of n1 + n2 workgroups: n1
// stage-1 query tiles, then n2 stage-2 chunks in head order.
//
// Stage-1 tiles are claimed, not indexed by workgroup id: the blocks (problems
// of all heads, in head order) are dealt to the XCDs round-robin, block B to
// list B mod nxcd, each list holding its blocks' query tiles in order. A
// workgroup claims the next tile from the front of its own XCD's list; when
// that list is used up it claims from the back of another list. So all query
// tiles of a block run on one XCD (shared L2) except for a few at the end,
// and the XCDs work through the blocks, hence the heads, together: the first
// heads' Y is complete while the last tiles still run, and their stage-2
// chunks (dispatched once every stage-1 workgroup has been) fill the
// workgroup slots the last tiles leave free. A list's front and back counts
// share one 64-bit word, so every claim sees all earlier ones: a claim is
// valid iff fewer than the list's length were taken before it, and every
// stage-1 workgroup finds a tile (there are as many tiles as workgroups).
//
// Each tile counts itself in ready[head, tile] (one 128-byte line per
// counter) once its written-through Y stores have completed; a stage-2 chunk
// waits for its count and reads Y with device-scope loads. Workgroups start
// in index order on each XCD, so every stage-1 tile has started before any
// stage-2 chunk of its XCD and never waits: the wait ends (the spin bound and
// the error word remain as a guard).
constexpr int kCtlClaims = 0;  // nxcd 64-bit words: front count (low half), back count (high half)
constexpr int kReadyStride = 32;

__device__ __forceinline__ bool claim_tile(int* ctl, int list, bool back, int nb, int nxcd, int qtiles, int& blk,
                                           int& qt) {
  const int nblk = (nb - list + nxcd - 1) / nxcd;  // blocks list, list + nxcd, ...
  const int len = nblk * qtiles;
  unsigned long long* w = reinterpret_cast<unsigned long long*>(ctl + kCtlClaims) + list;
  const unsigned long long old =
      __hip_atomic_fetch_add(w, back ? (1ull << 32) : 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int front = static_cast<int>(old & 0xffffffffu), taken_back = static_cast<int>(old >> 32);
  if (front + taken_back >= len) return false;
  const int j = back ? len - 1 - taken_back : front;
  blk = list + nxcd * (j / qtiles);
  qt = j % qtiles;
  return true;
}

template <int D>
__global__ void __launch_bounds__(FNT, 2) fused_grid_kernel(FusedArgs f, int qtiles, int nchunks, int n1, int nxcd) {
  using T = SwTile<D>;
  __shared__ __attribute__((aligned(1024))) char k0[T::bytes];
  __shared__ __attribute__((aligned(1024))) char k1[T::bytes];
  __shared__ __attribute__((aligned(1024))) char v0[T::bytes];
  __shared__ __attribute__((aligned(1024))) char v1[T::bytes];
  __shared__ int item[2];
  __shared__ int timed_out;
  const int tid = threadIdx.x;
  int* ready = f.ctl + kCtlReady;
  if (static_cast<int>(blockIdx.x) < n1) {
    if (tid == 0) {
      // hardware XCD of this workgroup (HW_REG_XCC_ID, bits 3:0)
      const int xcd = static_cast<int>(__builtin_amdgcn_s_getreg((3 << 11) | 20)) % nxcd;
      const int nb = f.s1.problems * f.s1.heads;
      int blk = -1, qt = 0;
      if (!claim_tile(f.ctl, xcd, false, nb, nxcd, qtiles, blk, qt))
        for (int d = 1; d < nxcd && blk < 0; ++d)
          if (!claim_tile(f.ctl, (xcd + d) % nxcd, true, nb, nxcd, qtiles, blk, qt)) blk = -1;
      item[0] = blk;
      item[1] = qt;
    }
    __syncthreads();
    const int blk = item[0], qt = item[1];
    if (blk < 0) return;  // cannot happen (as many tiles as workgroups); no counter waits on it
    const int p = blk % f.s1.problems, hd = blk / f.s1.problems;
    flash_tile<D, false, kPolicyDevice>(f.s1, hd, p, qt, FBM, k0, k1, v0, v1, tid);
    wait_dma();  // this wave's written-through Y stores have completed
    __syncthreads();
    if (tid == 0)
      __hip_atomic_fetch_add(ready + kReadyStride * (hd * f.tiles + p / f.m_tau), 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int id = static_cast<int>(blockIdx.x) - n1;
  const int chunk = id % nchunks, rest = id / nchunks;
  const int u = rest % f.tiles, hd = rest / f.tiles;
  const int key = hd * f.tiles + u;
  const int target = f.m_tau * qtiles;
  if (tid == 0) {
    int spins = 0, late = 0;
    while (__hip_atomic_load(ready + kReadyStride * key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(32);
      if (++spins > (1 << 18)) {
        __hip_atomic_store(f.ctl + kCtlError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        late = 1;
        break;
      }
    }
    timed_out = late;
  }
  __syncthreads();  // Y is read below with device-coherent loads only
  const bool poison = timed_out != 0;
  const int w = tid >> 6;
  char* const lds_wave = w == 0 ? k0 : w == 1 ? k1 : w == 2 ? v0 : v1;
  const FlashOffsets<D> fo(w, tid & 63, f.s2.row_stride);
  const int j0 = chunk * kFusedGroups;
#pragma unroll 1
  for (int g = w; g < kFusedGroups; g += 4) {
    const int j = j0 + g;
    if (j >= f.b) break;
    group_wave<D>(f.s2, hd, u * f.b + j, lds_wave, lds_wave + 32 * 2 * D, fo, tid & 63, poison);
  }
}

bool mfma_types_ok(const GroupedArgs& a) {
  return (a.D == 64 || a.D == 128) && a.qk_type == kBF16 && a.v_type == kBF16;
}

// 32-bit buffer offsets must reach a whole key tile past the end of a problem
// (bytes counted at the widest output element, 4)
bool offsets_fit(const GroupedArgs& a, int pad_rows) {
  return (static_cast<int64_t>(a.L) + pad_rows) * a.row_stride * a.D * 4 < (int64_t{1} << 31);
}

template <int D, bool F32, bool DELTA = false, bool ENT = false, bool KB = false>
hipError_t launch_flash_t(const GroupedArgs& a, hipStream_t s) {
  // query rows in units of one wave's 32, spread evenly over the fewest
  // tiles of at most kFlashWaves units (a 1560-row block: 49 units, 13 tiles
  // of 128 rows, the last holding 24)
  const int units = (a.Lq + 31) / 32;
  if (units <= 0) return hipErrorInvalidConfiguration;
  const int qtiles = (units + kFlashWaves - 1) / kFlashWaves;
  const int qrows = 32 * ((units + qtiles - 1) / qtiles);
  const int64_t nwg = static_cast<int64_t>(qtiles) * a.problems * a.heads;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((flash_kernel<D, F32, DELTA, ENT, KB>), dim3(static_cast<unsigned>(nwg)), dim3(64 * kFlashWaves), 0,
                     s, a, qtiles, qrows, static_cast<int>(nwg));
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
  if (a.L <= kShortRows) {
    const int64_t nwg = static_cast<int64_t>(a.problems) * a.heads;
    if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((group_short_kernel<D, F32>), dim3(static_cast<unsigned>(nwg)), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  switch ((a.L + 31) / 32) {
    case 1: return launch_group_t<D, 1, F32>(a, s);
    case 2: return launch_group_t<D, 2, F32>(a, s);
    case 3: return launch_group_t<D, 3, F32>(a, s);
    case 4: return launch_group_t<D, 4, F32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool flash_supported(const GroupedArgs& a) {
  return mfma_types_ok(a) && a.L > 128 && offsets_fit(a, FBN) &&
         !(a.kbias && (a.ent || a.delta || a.o_type != kBF16)) &&
         !(a.ent && (a.delta || a.o_type != kBF16 || a.v != a.k));
}

hipError_t launch_flash(const GroupedArgs& a, hipStream_t s) {
  if (!flash_supported(a)) return hipErrorInvalidValue;
  if (a.delta) {  // row sums of G * O instead of O
    if (!a.dg) return hipErrorInvalidValue;
    return a.D == 128 ? launch_flash_t<128, true, true>(a, s) : launch_flash_t<64, true, true>(a, s);
  }
  if (a.kbias)  // per-key biases of the logits (bf16 output only)
    return a.D == 128 ? launch_flash_t<128, false, false, false, true>(a, s)
                      : launch_flash_t<64, false, false, false, true>(a, s);
  if (a.ent)  // entropies of the rows (bf16 output only)
    return a.D == 128 ? launch_flash_t<128, false, false, true>(a, s) : launch_flash_t<64, false, false, true>(a, s);
  const bool f32 = a.o_type == kF32;
  if (a.D == 128) return f32 ? launch_flash_t<128, true>(a, s) : launch_flash_t<128, false>(a, s);
  return f32 ? launch_flash_t<64, true>(a, s) : launch_flash_t<64, false>(a, s);
}

bool fused_supported(const GroupedArgs& s1, const GroupedArgs& s2) {
  return flash_supported(s1) && s1.o_type == kBF16 && mfma_types_ok(s2) && s2.o_type == kBF16 && s2.D == s1.D &&
         s2.L >= 2 && s2.L <= 32 && offsets_fit(s2, 32) && s1.q_row0 == 0 && s1.Lq == s1.L && s2.q_row0 == 0 &&
         s2.Lq == s2.L;
}

int64_t fused_ctl_ints(int64_t heads, int64_t tiles) { return kCtlReady + 32 * heads * tiles; }
int64_t fused_ctl_error_index() { return kCtlError; }

hipError_t launch_fused(const FusedArgs& f, hipStream_t s) {
  if (!fused_supported(f.s1, f.s2) || !f.ctl) return hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // XCDs of 32 CUs each on this part (8 on the full device)
  const int nxcd = cus >= 32 * kFusedXcds ? kFusedXcds : (cus >= 32 ? cus / 32 : 1);
  const int qtiles = (f.s1.L + FBM - 1) / FBM;
  const int nchunks = (f.b + kFusedGroups - 1) / kFusedGroups;
  const int64_t nctl = fused_ctl_ints(f.s1.heads, f.tiles);
  hipLaunchKernelGGL(fused_reset, dim3(1), dim3(256), 0, s, f.ctl, static_cast<int>(nctl));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n1 = static_cast<int64_t>(qtiles) * f.s1.problems * f.s1.heads;
  const int64_t n2 = static_cast<int64_t>(nchunks) * f.tiles * f.s2.heads;
  if (n1 + n2 > 0x7fffffff) return hipErrorInvalidConfiguration;
  const unsigned grid = static_cast<unsigned>(n1 + n2);
  if (f.s1.D == 128)
    hipLaunchKernelGGL((fused_grid_kernel<128>), dim3(grid), dim3(FNT), 0, s, f, qtiles, nchunks, static_cast<int>(n1),
                       nxcd);
  else
    hipLaunchKernelGGL((fused_grid_kernel<64>), dim3(grid), dim3(FNT), 0, s, f, qtiles, nchunks, static_cast<int>(n1),
                       nxcd);
  return hipGetLastError();
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
