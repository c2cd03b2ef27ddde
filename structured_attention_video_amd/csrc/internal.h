// Internal launch interface between the C-ABI layer and the kernels.
//
// Both Monarch stages are instances of one primitive, "grouped attention":
// a head is split into `problems` independent softmax-attention problems of L
// rows each. Problem p owns the tokens
//     base(p) + r * row_stride,  r = 0..L-1,
//     base(p) = (p / inner) * outer + (p % inner),
// and every row attends to every row of its own problem (keys = the same
// tokens). Stage 1 (contiguous blocks): inner = 1, outer = b, row_stride = 1,
// L = b. Stage 2 (stride-b groups inside tile u): inner = b, outer = tau,
// row_stride = b, L = m_tau. Dense attention is stage 1 with b = N.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace monarch {

enum ElemType : int32_t { kBF16 = 0, kF32 = 1 };

struct GroupedArgs {
  const void* q;
  const void* k;
  const void* v;      // values (V in stage 1, Y in stage 2)
  void* o;            // output (Y in stage 1, O in stage 2)
  int64_t head_elems; // elements between consecutive heads (N * D)
  int32_t heads;      // batch * heads
  int32_t problems;   // problems per head
  int32_t inner;
  int64_t outer;
  int64_t row_stride; // in tokens
  int32_t L;          // rows per problem (keys and values: rows 0..L-1)
  int32_t q_row0;     // first query row inside each problem (0 when every row queries)
  int32_t Lq;         // query rows per problem, q_row0 + Lq <= L (L when every row queries);
                      // outputs (and lse) are written for the query rows only
  int32_t D;          // head dim
  float scale_log2;   // softmax scale * log2(e)
  ElemType qk_type;
  ElemType v_type;
  ElemType o_type;
  float* lse;         // optional (bf16 MFMA and tiny kernels): per query row, log2 of the
                      // softmax denominator in the exp2 domain, i.e. the row's probabilities
                      // are exp2(scale_log2 * <q,k> - lse); indexed [head][token]
  const void* dg;     // optional, flash kernel only, with delta: bf16 rows G (layout of q);
  float* delta;       // then, instead of O, delta[row] = sum over channels of G * O with O in
                      // fp32 before any rounding, indexed [head][token] (o is not written)
  float* ent;         // optional (flash when the values are the keys, group and generic
                      // kernels): per query row, the Shannon entropy in bits of the row's
                      // softmax weights, [head][token]
  const float* kbias; // optional (flash with bf16 output, group, tiny and generic kernels): per key row, a bias in
                      // bits added to the row's logits, i.e. weights ~ exp2(scale_log2 * <q,k>
                      // + kbias[key]); indexed [head][token]
};

// Backward of one grouped-attention stage (the chain rule of O = P V with
// P = rowsoftmax(s Q K^T)): dQ = s dS K, dK = s dS^T Q, dV = P^T G with
// dS = P * (G V^T - delta). g: the forward's problem geometry and inputs
// (v = the stage's values); go: G, the gradient of the stage output, same
// layout as q; lse: the forward's per-row statistic (see GroupedArgs::lse);
// delta: per row, the sum over channels of G * O. Outputs are written in
// their element types; dq_in / dk_in (optional, fp32, same layout) are added
// before the store. Per-row arrays are indexed [head][token].
struct BwdArgs {
  GroupedArgs g;
  const void* go;
  const float* lse;
  const float* delta;
  void* dq;
  void* dk;
  void* dv;
  const float* dq_in;
  const float* dk_in;
  ElemType dq_type, dk_type, dv_type;
  float* dv_delta;  // one-pass small-problem backward only: per row, sum over channels of
                    // the stored (rounded) dV times the stage's values v
};
bool bwd_supported(const GroupedArgs& g);
hipError_t launch_bwd(const BwdArgs& b, hipStream_t stream);
// One-pass backward of a stage whose problems have at most 32 rows (the frame
// stage-2 groups): one wave per problem recomputes the forward (its own lse and
// fp32 output, so lse and delta are not inputs), forms dQ, dK (fp32) and dV
// (bf16), and writes dv_delta for the next stage's backward. Needs go, dq, dk,
// dv, dv_delta; lse, delta, dq_in and dk_in are not used.
bool bwd_small_supported(const GroupedArgs& g);
hipError_t launch_bwd_small(const BwdArgs& b, hipStream_t stream);
// One-pass backward of a stage whose problems have at most 128 rows: one
// workgroup of ceil(L / 32) waves per problem, lse and delta recomputed. Two
// roles, picked by the output types: partial (dq, dk fp32; dv bf16; dv_delta;
// as launch_bwd_small: the long layout's stage-2 groups) and final (dq, dk,
// dv bf16, with the fp32 dq_in and dk_in added when given: the row layout's
// stage-1 blocks). lse and delta are not used.
bool bwd_group_supported(const GroupedArgs& g);
hipError_t launch_bwd_group(const BwdArgs& b, hipStream_t stream);
// out[r] = sum_c a[r][c] * b[r][c] over rows x D (bf16 or fp32 elements)
hipError_t launch_rowdot(const void* a, ElemType ta, const void* b, ElemType tb, float* out, int64_t rows, int D,
                         hipStream_t stream);

// Kernel variant ids (reported through the plan info).
enum KernelId : int32_t {
  kKernelNone = 0,
  kKernelGeneric = 1,   // plain VALU, fp32 arithmetic, any L
  kKernelFlash = 2,     // bf16 MFMA, LDS-staged K/V tiles, online softmax, large L
  kKernelSmall = 3,     // bf16 MFMA, one wavefront per problem, L <= 32
  kKernelTiny = 4,      // VALU, D/8 lanes per problem, L <= 8, any element types
  kKernelFused = 5,     // bf16 MFMA, both stages in one persistent launch
};

const char* kernel_name(int32_t id);

// Both stages in one launch. s1: stage 1 (Q, K, V -> Y), s2: stage 2
// (Q, K, Y -> O) of the same plan; ctl: device control block of
// fused_ctl_ints(...) ints inside the workspace (reset by the launch).
struct FusedArgs {
  GroupedArgs s1, s2;
  int* ctl;
  int32_t tiles;  // U
  int32_t m_tau;  // blocks per tile
  int32_t b;      // block size
};
bool fused_supported(const GroupedArgs& s1, const GroupedArgs& s2);
int64_t fused_ctl_ints(int64_t heads, int64_t tiles);
int64_t fused_ctl_error_index();  // int index of the error word in the control block
hipError_t launch_fused(const FusedArgs& f, hipStream_t stream);

// Each launcher returns hipSuccess or the launch error.
hipError_t launch_generic(const GroupedArgs& a, hipStream_t stream);
bool flash_supported(const GroupedArgs& a);
hipError_t launch_flash(const GroupedArgs& a, hipStream_t stream);
bool small_supported(const GroupedArgs& a);
hipError_t launch_small(const GroupedArgs& a, hipStream_t stream);
bool tiny_supported(const GroupedArgs& a);
hipError_t launch_tiny(const GroupedArgs& a, hipStream_t stream);

}  // namespace monarch
