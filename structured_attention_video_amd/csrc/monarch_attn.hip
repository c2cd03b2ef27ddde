// C-ABI layer: plan validation, workspace sizing, pointer checks and kernel
// dispatch for the two Monarch stages. Everything before a launch is plain
// host arithmetic, so every error path runs without a GPU.
#include "monarch_attn.h"

#include <math.h>
#include <string.h>
#include <mutex>
#include <new>

#include "internal.h"

using namespace monarch;

struct monarch_plan {
  monarch_plan_info info;
};

namespace {

constexpr uint32_t kKnownFlags = MONARCH_FLAG_Y_FP32 | MONARCH_FLAG_ALLOW_UNALIGNED | MONARCH_FLAG_GENERIC |
                                  MONARCH_FLAG_FUSED | MONARCH_FLAG_REFINE;


size_t elem_bytes(int32_t dt) { return dt == MONARCH_FP32 ? 4 : 2; }

int64_t tensor_bytes(const monarch_plan_info& p, int32_t dt) {
  return p.batch * p.heads * p.N * p.head_dim * static_cast<int64_t>(elem_bytes(dt));
}

ElemType as_elem(int32_t dt) { return dt == MONARCH_FP32 ? kF32 : kBF16; }

// The fused control block follows Y in the workspace, 256-byte aligned.
int64_t ctl_offset(const monarch_plan_info& p) { return (tensor_bytes(p, p.y_dtype) + 255) / 256 * 256; }

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Refinement-step workspace: Y (y_dtype), the mixed keys Kbar (input dtype) and the
// stage-1 row entropies (fp32), each section 256-aligned.
struct RefineLayout {
  int64_t y, kbar, ent, total;
};
RefineLayout refine_layout(const monarch_plan_info& p) {
  RefineLayout l{};
  l.y = 0;
  l.kbar = align256(tensor_bytes(p, p.y_dtype));
  l.ent = l.kbar + align256(tensor_bytes(p, p.dtype));
  l.total = l.ent + align256(p.batch * p.heads * p.N * 4);
  return l;
}

// Backward workspace: Y and dY (bf16), the stage-2 partial dQ and dK (fp32),
// then per-row lse and delta of both stages (fp32), each section 256-aligned.
struct BwdLayout {
  int64_t y, dy, dq2, dk2, lse1, lse2, del1, del2, total;
};
BwdLayout bwd_layout(const monarch_plan_info& p) {
  const int64_t t2 = tensor_bytes(p, MONARCH_BF16), t4 = tensor_bytes(p, MONARCH_FP32);
  const int64_t rows = align256(p.batch * p.heads * p.N * 4);
  BwdLayout l{};
  l.y = 0;
  l.dy = align256(t2);
  l.dq2 = l.dy + align256(t2);
  l.dk2 = l.dq2 + align256(t4);
  l.lse1 = l.dk2 + align256(t4);
  l.lse2 = l.lse1 + rows;
  l.del1 = l.lse2 + rows;
  l.del2 = l.del1 + rows;
  l.total = l.del2 + rows;
  return l;
}


// Grouped-attention description of stage 1 (contiguous blocks of b tokens).
GroupedArgs stage1_args(const monarch_plan_info& p, const void* q, const void* k, const void* v,
                        void* out, int32_t out_dtype) {
  GroupedArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = out;
  a.head_elems = p.N * p.head_dim;
  a.heads = static_cast<int32_t>(p.batch * p.heads);
  a.problems = static_cast<int32_t>(p.N / p.b);
  a.inner = 1;
  a.outer = p.b;
  a.row_stride = 1;
  a.L = static_cast<int32_t>(p.b);
  a.q_row0 = 0;
  a.Lq = a.L;
  a.D = static_cast<int32_t>(p.head_dim);
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.qk_type = as_elem(p.dtype);
  a.v_type = as_elem(p.dtype);
  a.o_type = as_elem(out_dtype);
  return a;
}

// Stage 2: the group of (tile u, position j) is u*tau + i*b + j, i < m_tau.
GroupedArgs stage2_args(const monarch_plan_info& p, const void* q, const void* k, const void* y,
                        int32_t y_dtype, void* out) {
  GroupedArgs a{};
  a.q = q; a.k = k; a.v = y; a.o = out;
  a.head_elems = p.N * p.head_dim;
  a.heads = static_cast<int32_t>(p.batch * p.heads);
  a.problems = static_cast<int32_t>(p.tiles * p.b);
  a.inner = static_cast<int32_t>(p.b);
  a.outer = p.tau;
  a.row_stride = p.b;
  a.L = static_cast<int32_t>(p.m_tau);
  a.q_row0 = 0;
  a.Lq = a.L;
  a.D = static_cast<int32_t>(p.head_dim);
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.qk_type = as_elem(p.dtype);
  a.v_type = as_elem(y_dtype);
  a.o_type = as_elem(p.dtype);
  return a;
}

// Stand-in target of the refinement fields when a kernel is chosen at plan time:
// the choice only tests them for null; no kernel is launched with it.
float g_choice_marker = 0.f;

GroupedArgs with_refine_fields(GroupedArgs a, bool ent, bool kbias) {
  if (ent) a.ent = &g_choice_marker;
  if (kbias) a.kbias = &g_choice_marker;
  return a;
}

int32_t choose_kernel(const GroupedArgs& a, uint32_t flags) {
  if (!(flags & MONARCH_FLAG_GENERIC)) {
    if (tiny_supported(a)) return kKernelTiny;
    if (small_supported(a)) return kKernelSmall;
    if (flash_supported(a)) return kKernelFlash;
  }
  return kKernelGeneric;
}

hipError_t launch(int32_t kernel, const GroupedArgs& a, hipStream_t s) {
  switch (kernel) {
    case kKernelFlash: return launch_flash(a, s);
    case kKernelSmall: return launch_small(a, s);
    case kKernelTiny: return launch_tiny(a, s);
    default: return launch_generic(a, s);
  }
}

bool bwd_plan_ok(const monarch_plan_info& p) {
  if (p.dtype != MONARCH_BF16 || (p.flags & MONARCH_FLAG_GENERIC) || p.refine_steps) return false;
  const bool has1 = p.b > 1, has2 = p.m_tau > 1;
  if (has1 || !has2) {
    GroupedArgs a = stage1_args(p, nullptr, nullptr, nullptr, nullptr, MONARCH_BF16);
    if (!bwd_supported(a) || choose_kernel(a, p.flags) == kKernelGeneric) return false;
  }
  if (has2) {
    GroupedArgs a = stage2_args(p, nullptr, nullptr, nullptr, MONARCH_BF16, nullptr);
    if (!bwd_supported(a) || choose_kernel(a, p.flags) == kKernelGeneric) return false;
  }
  return true;
}

// bit-level test, independent of floating-point compile flags
bool finite_nonnegative(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u) return false;  // inf or nan
  return (u >> 31) == 0 || (u & 0x7fffffffu) == 0;      // +x, or -0
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

// ---------------------------------------------------------------- static scratch
// Device memory of monarch_attn_forward_noalloc: the forward's workspace (Y, and a fused plan's
// control block) for callers that cannot allocate. Each GPU the library runs on holds its own
// copy of this array from the time the code object is loaded there until the process ends. In
// host code `scratch` names a host-side stand-in, not device memory: its device address is
// taken once per device with hipGetSymbolAddress (with that device current) and only that
// address is ever passed on.
constexpr int64_t kScratchBytes = MONARCH_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch array (the stream, when given, must belong to
// the current device).
monarch_status scratch_address(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MONARCH_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return MONARCH_ERR_HIP;
    if (sdev != dev) return MONARCH_ERR_INVALID_ARG;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return MONARCH_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MONARCH_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MONARCH_OK;
}

}  // namespace

extern "C" {

monarch_status monarch_attn_plan(monarch_plan** out, int32_t batch, int32_t heads, int32_t head_dim,
                                 int32_t T, int32_t H, int32_t W, int32_t align, int64_t custom_b,
                                 int64_t tile_tokens, int32_t dtype, float scale, uint32_t flags) {
  if (!out) return MONARCH_ERR_INVALID_ARG;
  *out = nullptr;
  if (batch < 1 || heads < 1 || head_dim < 1 || T < 1 || H < 1 || W < 1) return MONARCH_ERR_INVALID_ARG;
  if (dtype != MONARCH_BF16 && dtype != MONARCH_FP32) return MONARCH_ERR_INVALID_ARG;
  if (align < MONARCH_ALIGN_FRAME || align > MONARCH_ALIGN_CUSTOM) return MONARCH_ERR_INVALID_ARG;
  if (flags & ~kKnownFlags) return MONARCH_ERR_INVALID_ARG;
  if (!finite_nonnegative(scale)) return MONARCH_ERR_INVALID_ARG;
  if (tile_tokens < 0) return MONARCH_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return MONARCH_ERR_UNSUPPORTED;

  const int64_t N = static_cast<int64_t>(T) * H * W;
  if (N >= (int64_t{1} << 31)) return MONARCH_ERR_INVALID_ARG;
  const int64_t BH = static_cast<int64_t>(batch) * heads;
  if (BH >= (int64_t{1} << 31) || BH * N * head_dim >= (int64_t{1} << 56)) return MONARCH_ERR_INVALID_ARG;

  int64_t b = 0;
  switch (align) {
    case MONARCH_ALIGN_FRAME: b = static_cast<int64_t>(H) * W; break;
    case MONARCH_ALIGN_ROW: b = W; break;
    case MONARCH_ALIGN_DENSE: b = N; break;
    case MONARCH_ALIGN_TOKEN: b = 1; break;
    default:
      if (custom_b < 1) return MONARCH_ERR_INVALID_ARG;
      b = custom_b;
  }
  if (N % b) return MONARCH_ERR_UNALIGNED;
  // with (t,h,w) row-major tokens the contiguous splits that keep every axis
  // inside one block dimension are b in {1, W, H*W, N}
  const bool axis_aligned = b == 1 || b == W || b == static_cast<int64_t>(H) * W || b == N;
  if (!axis_aligned && !(flags & MONARCH_FLAG_ALLOW_UNALIGNED)) return MONARCH_ERR_UNALIGNED;
  const int64_t tau = tile_tokens ? tile_tokens : N;
  if (tau % b || N % tau) return MONARCH_ERR_UNALIGNED;

  monarch_plan* p = new (std::nothrow) monarch_plan;
  if (!p) return MONARCH_ERR_INVALID_ARG;
  monarch_plan_info& i = p->info;
  i = monarch_plan_info{};
  i.batch = batch; i.heads = heads; i.head_dim = head_dim;
  i.T = T; i.H = H; i.W = W; i.N = N;
  i.b = b; i.tau = tau; i.m_tau = tau / b; i.tiles = N / tau;
  i.dtype = dtype;
  i.y_dtype = (dtype == MONARCH_FP32 || (flags & MONARCH_FLAG_Y_FP32)) ? MONARCH_FP32 : MONARCH_BF16;
  i.scale = scale != 0.f ? scale : 1.0f / sqrtf(static_cast<float>(head_dim));
  i.flags = flags;
  const bool has1 = b > 1, has2 = i.m_tau > 1;
  i.refine_steps = (flags & MONARCH_FLAG_REFINE) && has1 && has2 ? 1 : 0;
  i.fused_error_offset = -1;
  i.workspace_bytes = (has1 && has2) ? tensor_bytes(i, i.y_dtype) : 0;
  if (i.refine_steps) i.workspace_bytes = refine_layout(i).total;
  i.flops_stage1 = has1 || !has2 ? 4 * BH * N * b * head_dim : 0;
  i.flops_stage2 = has2 ? 4 * BH * N * i.m_tau * head_dim : 0;
  // kernel choice is a function of the problem geometry only (no device query)
  i.stage1_kernel = kKernelNone;
  i.stage2_kernel = kKernelNone;
  if (has1 || !has2) {
    GroupedArgs a = stage1_args(i, nullptr, nullptr, nullptr, nullptr, has2 ? i.y_dtype : dtype);
    i.stage1_kernel = choose_kernel(a, flags);
  }
  if (has2) {
    GroupedArgs a = stage2_args(i, nullptr, nullptr, nullptr, has1 ? i.y_dtype : dtype, nullptr);
    i.stage2_kernel = choose_kernel(with_refine_fields(a, false, i.refine_steps > 0), flags);
  }
  i.fused = 0;
  if ((flags & MONARCH_FLAG_FUSED) && !(flags & MONARCH_FLAG_GENERIC) && has1 && has2 && !i.refine_steps) {
    const GroupedArgs a1 = stage1_args(i, nullptr, nullptr, nullptr, nullptr, i.y_dtype);
    const GroupedArgs a2 = stage2_args(i, nullptr, nullptr, nullptr, i.y_dtype, nullptr);
    if (fused_supported(a1, a2)) {
      i.fused = 1;
      i.workspace_bytes = ctl_offset(i) + fused_ctl_ints(BH, i.tiles) * static_cast<int64_t>(sizeof(int));
      i.fused_error_offset = ctl_offset(i) + fused_ctl_error_index() * static_cast<int64_t>(sizeof(int));
    }
  }
  *out = p;
  return MONARCH_OK;
}

void monarch_attn_destroy(monarch_plan* plan) { delete plan; }

size_t monarch_attn_workspace_size(const monarch_plan* plan) {
  return plan ? static_cast<size_t>(plan->info.workspace_bytes) : 0;
}

monarch_status monarch_attn_plan_info(const monarch_plan* plan, monarch_plan_info* info) {
  if (!plan || !info) return MONARCH_ERR_INVALID_ARG;
  *info = plan->info;
  return MONARCH_OK;
}

static monarch_status run_stage1(const monarch_plan_info& p, const void* q, const void* k, const void* v,
                                 void* y, int32_t y_dtype, hipStream_t s) {
  GroupedArgs a = stage1_args(p, q, k, v, y, y_dtype);
  return launch(p.stage1_kernel, a, s) == hipSuccess ? MONARCH_OK : MONARCH_ERR_HIP;
}

static monarch_status run_stage2(const monarch_plan_info& p, const void* q, const void* k, const void* y,
                                 int32_t y_dtype, void* o, hipStream_t s) {
  GroupedArgs a = stage2_args(p, q, k, y, y_dtype, o);
  return launch(p.stage2_kernel, a, s) == hipSuccess ? MONARCH_OK : MONARCH_ERR_HIP;
}

// Argument checks of the forward that need no workspace (plain host arithmetic).
static monarch_status forward_io_checks(const monarch_plan* plan, const void* q, const void* k, const void* v,
                                        const void* o) {
  if (!plan || !q || !k || !v || !o) return MONARCH_ERR_INVALID_ARG;
  const monarch_plan_info& p = plan->info;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o)) return MONARCH_ERR_UNALIGNED;
  const int64_t io = tensor_bytes(p, p.dtype);
  if (overlap(o, io, q, io) || overlap(o, io, k, io) || overlap(o, io, v, io)) return MONARCH_ERR_ALIAS;
  return MONARCH_OK;
}

// The forward's launches, once every argument has been checked.
static monarch_status forward_launch(const monarch_plan_info& p, const void* q, const void* k, const void* v,
                                     void* o, void* workspace, hipStream_t s) {
  const bool has1 = p.b > 1, has2 = p.m_tau > 1;
  if (!has2) return run_stage1(p, q, k, v, o, p.dtype, s);  // second factor is the identity
  if (!has1) return run_stage2(p, q, k, v, p.dtype, o, s);  // first factor is the identity: Y = V
  if (p.refine_steps) {
    // one refinement step: Y = R V, Kbar = R K with the entropies of R's rows, then
    // stage 2 against Kbar with the entropies as key biases
    const RefineLayout lay = refine_layout(p);
    char* w = static_cast<char*>(workspace);
    void* y = w + lay.y;
    void* kbar = w + lay.kbar;
    float* ent = reinterpret_cast<float*>(w + lay.ent);
    monarch_status st = run_stage1(p, q, k, v, y, p.y_dtype, s);
    if (st != MONARCH_OK) return st;
    GroupedArgs a1 = stage1_args(p, q, k, k, kbar, p.dtype);
    a1.ent = ent;
    if (launch(choose_kernel(a1, p.flags), a1, s) != hipSuccess) return MONARCH_ERR_HIP;
    GroupedArgs a2 = stage2_args(p, q, kbar, y, p.y_dtype, o);
    a2.kbias = ent;
    return launch(p.stage2_kernel, a2, s) == hipSuccess ? MONARCH_OK : MONARCH_ERR_HIP;
  }
  if (p.fused) {
    FusedArgs f{};
    f.s1 = stage1_args(p, q, k, v, workspace, p.y_dtype);
    f.s2 = stage2_args(p, q, k, workspace, p.y_dtype, o);
    f.ctl = reinterpret_cast<int*>(static_cast<char*>(workspace) + ctl_offset(p));
    f.tiles = static_cast<int32_t>(p.tiles);
    f.m_tau = static_cast<int32_t>(p.m_tau);
    f.b = static_cast<int32_t>(p.b);
    return launch_fused(f, s) == hipSuccess ? MONARCH_OK : MONARCH_ERR_HIP;
  }
  monarch_status st = run_stage1(p, q, k, v, workspace, p.y_dtype, s);
  if (st != MONARCH_OK) return st;
  return run_stage2(p, q, k, workspace, p.y_dtype, o, s);
}

monarch_status monarch_attn_forward(const monarch_plan* plan, const void* q, const void* k,
                                    const void* v, void* o, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  const monarch_status chk = forward_io_checks(plan, q, k, v, o);
  if (chk != MONARCH_OK) return chk;
  const monarch_plan_info& p = plan->info;
  const int64_t io = tensor_bytes(p, p.dtype);
  const int64_t ws = p.workspace_bytes;
  if (ws > 0) {
    if (!workspace || static_cast<int64_t>(workspace_bytes) < ws) return MONARCH_ERR_WORKSPACE;
    if (misaligned(workspace)) return MONARCH_ERR_UNALIGNED;
    if (overlap(o, io, workspace, ws) || overlap(workspace, ws, q, io) || overlap(workspace, ws, k, io) ||
        overlap(workspace, ws, v, io))
      return MONARCH_ERR_ALIAS;
  }
  return forward_launch(p, q, k, v, o, workspace, static_cast<hipStream_t>(stream));
}

monarch_status monarch_attn_forward_noalloc(const monarch_plan* plan, const void* q, const void* k,
                                            const void* v, void* o, void* stream) {
  const monarch_status chk = forward_io_checks(plan, q, k, v, o);
  if (chk != MONARCH_OK) return chk;
  const monarch_plan_info& p = plan->info;
  if (p.workspace_bytes > kScratchBytes) return MONARCH_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (p.workspace_bytes > 0) {
    const monarch_status st = scratch_address(stream, &ws);
    if (st != MONARCH_OK) return st;
  }
  return forward_launch(p, q, k, v, o, ws, static_cast<hipStream_t>(stream));
}

monarch_status monarch_attn_stage1(const monarch_plan* plan, const void* q, const void* k,
                                   const void* v, void* y, size_t y_bytes, void* stream) {
  if (!plan || !q || !k || !v || !y) return MONARCH_ERR_INVALID_ARG;
  const monarch_plan_info& p = plan->info;
  if (p.b == 1) return MONARCH_ERR_INVALID_ARG;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(y)) return MONARCH_ERR_UNALIGNED;
  const int32_t ydt = p.m_tau > 1 ? p.y_dtype : p.dtype;
  const int64_t need = tensor_bytes(p, ydt), io = tensor_bytes(p, p.dtype);
  if (static_cast<int64_t>(y_bytes) < need) return MONARCH_ERR_WORKSPACE;
  if (overlap(y, need, q, io) || overlap(y, need, k, io) || overlap(y, need, v, io)) return MONARCH_ERR_ALIAS;
  return run_stage1(p, q, k, v, y, ydt, static_cast<hipStream_t>(stream));
}

monarch_status monarch_attn_stage2(const monarch_plan* plan, const void* q, const void* k,
                                   const void* y, void* o, void* stream) {
  if (!plan || !q || !k || !y || !o) return MONARCH_ERR_INVALID_ARG;
  const monarch_plan_info& p = plan->info;
  if (p.m_tau == 1) return MONARCH_ERR_INVALID_ARG;
  if (p.refine_steps) return MONARCH_ERR_UNSUPPORTED;  // needs the mixed keys and entropies
  if (misaligned(q) || misaligned(k) || misaligned(y) || misaligned(o)) return MONARCH_ERR_UNALIGNED;
  const int32_t ydt = p.b > 1 ? p.y_dtype : p.dtype;
  const int64_t io = tensor_bytes(p, p.dtype), ny = tensor_bytes(p, ydt);
  if (overlap(o, io, q, io) || overlap(o, io, k, io) || overlap(o, io, y, ny)) return MONARCH_ERR_ALIAS;
  return run_stage2(p, q, k, y, ydt, o, static_cast<hipStream_t>(stream));
}

monarch_status monarch_attn_chunk_forward(const monarch_plan* plan, int32_t t0, int32_t t1, const void* q,
                                          const void* k, const void* v, void* y, void* o, void* stream) {
  if (!plan || !q || !k || !v || !o) return MONARCH_ERR_INVALID_ARG;
  const monarch_plan_info& p = plan->info;
  if (t0 < 0 || t1 <= t0 || t1 > p.T) return MONARCH_ERR_INVALID_ARG;
  if (p.refine_steps) return MONARCH_ERR_UNSUPPORTED;
  const int64_t frame = p.H * p.W;
  // chunks must consist of whole blocks, and stage 2 must span the whole video
  if (p.tiles != 1 || frame % p.b != 0) return MONARCH_ERR_UNSUPPORTED;
  const bool has1 = p.b > 1, has2 = p.m_tau > 1;
  if (!has2) return MONARCH_ERR_UNSUPPORTED;  // b = N: the one block is the whole video
  if (has1 && !y) return MONARCH_ERR_INVALID_ARG;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || (y && misaligned(y)))
    return MONARCH_ERR_UNALIGNED;
  const int64_t io = tensor_bytes(p, p.dtype), ny = tensor_bytes(p, p.y_dtype);
  if (overlap(o, io, q, io) || overlap(o, io, k, io) || overlap(o, io, v, io)) return MONARCH_ERR_ALIAS;
  if (y && has1 && (overlap(y, ny, o, io) || overlap(y, ny, q, io) || overlap(y, ny, k, io) ||
                    overlap(y, ny, v, io)))
    return MONARCH_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t bpf = frame / p.b;  // blocks per frame
  const int64_t r0 = t0 * bpf, r1 = t1 * bpf;  // block rows of the chunk
  if (has1) {
    // stage 1 on the chunk's blocks only: the same problems, shifted
    const int64_t shift = r0 * p.b * p.head_dim;
    const size_t e = elem_bytes(p.dtype), ey = elem_bytes(p.y_dtype);
    GroupedArgs a = stage1_args(p, static_cast<const char*>(q) + shift * e, static_cast<const char*>(k) + shift * e,
                                static_cast<const char*>(v) + shift * e, static_cast<char*>(y) + shift * ey,
                                p.y_dtype);
    a.problems = static_cast<int32_t>(r1 - r0);
    if (launch(choose_kernel(a, p.flags), a, s) != hipSuccess) return MONARCH_ERR_HIP;
  }
  // stage 2: every group keeps the rows of blocks 0 .. r1-1 as keys and values
  // (earlier chunks' Y from the cache), and only the chunk's rows query
  GroupedArgs a = stage2_args(p, q, k, has1 ? y : v, has1 ? p.y_dtype : p.dtype, o);
  a.L = static_cast<int32_t>(r1);
  a.q_row0 = static_cast<int32_t>(r0);
  a.Lq = static_cast<int32_t>(r1 - r0);
  return launch(choose_kernel(a, p.flags), a, s) == hipSuccess ? MONARCH_OK : MONARCH_ERR_HIP;
}

size_t monarch_attn_backward_workspace_size(const monarch_plan* plan) {
  if (!plan || !bwd_plan_ok(plan->info)) return 0;
  return static_cast<size_t>(bwd_layout(plan->info).total);
}

// Training forward: the launches of the backward's forward recompute (stage 1
// into the workspace's Y with its per-row statistics, bf16 Y), then stage 2
// into O, so that a backward from the saved state skips the recompute.
monarch_status monarch_attn_forward_train(const monarch_plan* plan, const void* q, const void* k, const void* v,
                                          void* o, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !q || !k || !v || !o || !workspace) return MONARCH_ERR_INVALID_ARG;
  const monarch_plan_info& p = plan->info;
  if (!bwd_plan_ok(p)) return MONARCH_ERR_UNSUPPORTED;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(workspace))
    return MONARCH_ERR_UNALIGNED;
  const BwdLayout lay = bwd_layout(p);
  if (static_cast<int64_t>(workspace_bytes) < lay.total) return MONARCH_ERR_WORKSPACE;
  const int64_t io = tensor_bytes(p, p.dtype);
  const void* ins[] = {q, k, v};
  for (const void* x : ins)
    if (overlap(o, io, x, io) || overlap(workspace, lay.total, x, io)) return MONARCH_ERR_ALIAS;
  if (overlap(o, io, workspace, lay.total)) return MONARCH_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  void* y = w + lay.y;
  const bool has1 = p.b > 1, has2 = p.m_tau > 1;
  if (has1 || !has2) {
    GroupedArgs f1 = stage1_args(p, q, k, v, has2 ? y : o, MONARCH_BF16);
    f1.lse = reinterpret_cast<float*>(w + lay.lse1);
    if (launch(choose_kernel(f1, p.flags), f1, s) != hipSuccess) return MONARCH_ERR_HIP;
  }
  if (has2) return run_stage2(p, q, k, has1 ? y : v, MONARCH_BF16, o, s);
  return MONARCH_OK;
}

namespace {

monarch_status backward_impl(const monarch_plan* plan, const void* q, const void* k, const void* v, const void* o,
                             const void* grad_o, void* grad_q, void* grad_k, void* grad_v, void* workspace,
                             size_t workspace_bytes, void* stream, bool saved) {
  if (!plan || !q || !k || !v || !o || !grad_o || !grad_q || !grad_k || !grad_v || !workspace)
    return MONARCH_ERR_INVALID_ARG;
  const monarch_plan_info& p = plan->info;
  if (!bwd_plan_ok(p)) return MONARCH_ERR_UNSUPPORTED;
  const void* ins[] = {q, k, v, o, grad_o};
  void* outs[] = {grad_q, grad_k, grad_v};
  for (const void* x : ins)
    if (misaligned(x)) return MONARCH_ERR_UNALIGNED;
  for (const void* x : outs)
    if (misaligned(x)) return MONARCH_ERR_UNALIGNED;
  if (misaligned(workspace)) return MONARCH_ERR_UNALIGNED;
  const BwdLayout lay = bwd_layout(p);
  if (static_cast<int64_t>(workspace_bytes) < lay.total) return MONARCH_ERR_WORKSPACE;
  const int64_t io = tensor_bytes(p, p.dtype);
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], io, workspace, lay.total)) return MONARCH_ERR_ALIAS;
    for (const void* x : ins)
      if (overlap(outs[i], io, x, io)) return MONARCH_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], io, outs[j], io)) return MONARCH_ERR_ALIAS;
  }
  for (const void* x : ins)
    if (overlap(workspace, lay.total, x, io)) return MONARCH_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  void* y = w + lay.y;
  void* dy = w + lay.dy;
  float* dq2 = reinterpret_cast<float*>(w + lay.dq2);
  float* dk2 = reinterpret_cast<float*>(w + lay.dk2);
  float* lse1 = reinterpret_cast<float*>(w + lay.lse1);
  float* lse2 = reinterpret_cast<float*>(w + lay.lse2);
  float* del1 = reinterpret_cast<float*>(w + lay.del1);
  float* del2 = reinterpret_cast<float*>(w + lay.del2);
  const int64_t rows = p.batch * p.heads * p.N;
  const int D = static_cast<int>(p.head_dim);
  const bool has1 = p.b > 1, has2 = p.m_tau > 1;
  auto ok = [](hipError_t e) { return e == hipSuccess; };
  // stage-2 problems of at most 128 rows (frame and long layouts): one launch
  // does the stage-2 forward recompute, its backward and stage 1's delta
  const GroupedArgs g2 = stage2_args(p, q, k, y, MONARCH_BF16, nullptr);
  const bool one32 = has1 && has2 && bwd_small_supported(g2);
  const bool one128 = has1 && has2 && !one32 && g2.L > 32 && bwd_group_supported(g2);
  const bool small2 = one32 || one128;
  // the last stage's problems of at most 128 rows (the row layout's stage 1;
  // stage 1 or stage 2 alone): one final-role launch recomputes its softmax
  // and replaces the row-dot and the three tiled launches
  const bool small1 = (has1 || !has2) && bwd_group_supported(stage1_args(p, q, k, v, y, MONARCH_BF16));
  const bool solo2 = !has1 && has2 && bwd_group_supported(stage2_args(p, q, k, v, MONARCH_BF16, nullptr));

  // forward again, keeping Y and the per-row statistics (or, from a training
  // forward's saved state, only the argument set-up); a lone stage 1 done in
  // one pass needs neither
  GroupedArgs f1{}, f2{};
  if (has1 || !has2) {
    f1 = stage1_args(p, q, k, v, y, MONARCH_BF16);
    f1.lse = lse1;
    if (!saved && (has2 || !small1) && !ok(launch(choose_kernel(f1, p.flags), f1, s))) return MONARCH_ERR_HIP;
  }
  if (small2) {
    BwdArgs b2{};
    b2.g = stage2_args(p, q, k, y, MONARCH_BF16, nullptr);
    b2.go = grad_o;
    b2.dq = dq2; b2.dq_type = kF32;
    b2.dk = dk2; b2.dk_type = kF32;
    b2.dv = dy; b2.dv_type = kBF16;
    b2.dv_delta = del1;
    if (!ok(one32 ? launch_bwd_small(b2, s) : launch_bwd_group(b2, s))) return MONARCH_ERR_HIP;
  }
  if (solo2) {
    BwdArgs b2{};
    b2.g = stage2_args(p, q, k, v, MONARCH_BF16, nullptr);
    b2.go = grad_o;
    b2.dq = grad_q; b2.dq_type = kBF16;
    b2.dk = grad_k; b2.dk_type = kBF16;
    b2.dv = grad_v; b2.dv_type = kBF16;
    if (!ok(launch_bwd_group(b2, s))) return MONARCH_ERR_HIP;
  }
  bool delta2_done = false;
  if (has2 && !small2 && !solo2) {
    // values: Y (or V when stage 1 is the identity). delta = rowsum(G * O)
    // uses O before its bf16 rounding, which matters because dS = P * (dP -
    // delta) subtracts two nearly equal numbers: the flash kernel forms it in
    // its epilogue from the fp32 O in registers; otherwise the recomputed
    // output is kept in fp32 (in the dQ2 section, free until the stage-2
    // backward) for a row-dot launch.
    f2 = stage2_args(p, q, k, has1 ? y : v, MONARCH_BF16, dq2);
    f2.o_type = kF32;
    f2.lse = lse2;
    const int32_t k2 = choose_kernel(f2, p.flags);
    if (k2 == kKernelFlash) {
      f2.dg = grad_o;
      f2.delta = del2;
      delta2_done = true;
    }
    if (!ok(launch(k2, f2, s))) return MONARCH_ERR_HIP;
    f2.dg = nullptr;
    f2.delta = nullptr;
  }
  if (has2 && !small2 && !solo2) {
    BwdArgs b2{};
    b2.g = f2;
    b2.go = grad_o;
    b2.lse = lse2;
    b2.delta = del2;
    if (!delta2_done && !ok(launch_rowdot(grad_o, kBF16, dq2, kF32, del2, rows, D, s))) return MONARCH_ERR_HIP;
    if (has1) {  // partial dQ, dK in fp32; dY (bf16) feeds stage 1
      b2.dq = dq2; b2.dq_type = kF32;
      b2.dk = dk2; b2.dk_type = kF32;
      b2.dv = dy; b2.dv_type = kBF16;
    } else {     // stage 2 alone: final gradients
      b2.dq = grad_q; b2.dq_type = kBF16;
      b2.dk = grad_k; b2.dk_type = kBF16;
      b2.dv = grad_v; b2.dv_type = kBF16;
    }
    if (!ok(launch_bwd(b2, s))) return MONARCH_ERR_HIP;
  }
  if (has1 || !has2) {
    BwdArgs b1{};
    b1.g = f1;
    b1.go = has2 ? dy : grad_o;
    b1.lse = lse1;
    b1.delta = del1;
    if (!small2 && !small1 && !ok(launch_rowdot(b1.go, kBF16, has2 ? y : o, kBF16, del1, rows, D, s)))
      return MONARCH_ERR_HIP;
    b1.dq = grad_q; b1.dq_type = kBF16;
    b1.dk = grad_k; b1.dk_type = kBF16;
    b1.dv = grad_v; b1.dv_type = kBF16;
    if (has2) {
      b1.dq_in = dq2;
      b1.dk_in = dk2;
    }
    if (!ok(small1 ? launch_bwd_group(b1, s) : launch_bwd(b1, s))) return MONARCH_ERR_HIP;
  }
  return MONARCH_OK;
}

}  // namespace

monarch_status monarch_attn_backward(const monarch_plan* plan, const void* q, const void* k, const void* v,
                                     const void* o, const void* grad_o, void* grad_q, void* grad_k, void* grad_v,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(plan, q, k, v, o, grad_o, grad_q, grad_k, grad_v, workspace, workspace_bytes, stream, false);
}

monarch_status monarch_attn_backward_saved(const monarch_plan* plan, const void* q, const void* k, const void* v,
                                           const void* o, const void* grad_o, void* grad_q, void* grad_k,
                                           void* grad_v, void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(plan, q, k, v, o, grad_o, grad_q, grad_k, grad_v, workspace, workspace_bytes, stream, true);
}

const char* monarch_status_string(int32_t status) {
  switch (status) {
    case MONARCH_OK: return "ok";
    case MONARCH_ERR_INVALID_ARG: return "invalid argument";
    case MONARCH_ERR_UNSUPPORTED: return "unsupported head_dim or dtype";
    case MONARCH_ERR_UNALIGNED: return "block, tile or pointer alignment violated";
    case MONARCH_ERR_WORKSPACE: return "workspace missing or too small";
    case MONARCH_ERR_ALIAS: return "output overlaps an input or the workspace";
    case MONARCH_ERR_HIP: return "HIP launch failed";
    case MONARCH_ERR_TOO_LARGE: return "workspace exceeds the library's static scratch (no-allocation forward)";
  }
  return "unknown status";
}

const char* monarch_attn_kernel_name(int32_t kernel_id) { return kernel_name(kernel_id); }

int32_t monarch_attn_abi_version(void) { return MONARCH_ABI_VERSION; }

}  // extern "C"

namespace monarch {
const char* kernel_name(int32_t id) {
  switch (id) {
    case kKernelNone: return "none";
    case kKernelGeneric: return "generic_valu_fp32";
    case kKernelFlash: return "flash_mfma_bf16";
    case kKernelSmall: return "small_group_mfma_bf16";
    case kKernelTiny: return "tiny_group_valu";
    case kKernelFused: return "fused_mfma_bf16";
  }
  return "unknown";
}
}  // namespace monarch
