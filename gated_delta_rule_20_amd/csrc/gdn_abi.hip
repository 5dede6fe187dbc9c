// gdn_abi.hip -- host side of the C ABI declared in include/gdn.h.
//
// Validates every argument on the host, chooses the kernel configuration, carves
// the caller's workspace and launches on the caller's stream.  Nothing here
// allocates, copies or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_kernels.h"

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool gate_ok(int g) {
  return g == GDN_GATE_NONE || g == GDN_GATE_HEAD || g == GDN_GATE_KEY || g == GDN_GATE_HEAD_CONST;
}
bool write_ok(int w) { return w == GDN_WRITE_DELTA || w == GDN_WRITE_ADD; }
// Kernel gate of an ABI gate: the constant per-head gate is the scalar gate read
// with a token stride of 0.
int kernel_gate(int g) { return g == GDN_GATE_HEAD_CONST ? gdn::GATE_HEAD : g; }
// beta is given exactly for the delta write, log_alpha exactly for a gate.
bool operands_ok(int gate, int write, const void *beta, const void *log_alpha) {
  return (beta != nullptr) == (write == GDN_WRITE_DELTA) && (log_alpha != nullptr) == (gate != GDN_GATE_NONE);
}

// Value columns per workgroup: 64, or 32 when there are too few (sequence, head)
// streams to give every compute unit a workgroup.
int choose_dvb(int N, int H, int dv) {
  const long wg64 = (long)N * H * (dv / 64);
  return wg64 >= 256 ? 64 : 32;
}

int check_fwd(const gdn_fwd_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  if (a->B < 0 || a->T < 0 || a->H <= 0 || a->N < 0) return GDN_ERR_INVALID_ARG;
  if (a->dtype != GDN_F32 && a->dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (!gate_ok(a->gate) || !write_ok(a->write)) return GDN_ERR_INVALID_ARG;
  if (a->chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (!head_dim_ok(a->d_k) || !head_dim_ok(a->d_v)) return GDN_ERR_UNSUPPORTED;
  if (a->dtype == GDN_F32 && a->d_k != 64) return GDN_ERR_UNSUPPORTED;
  if (a->cu_seqlens) {
    if (a->B != 1 || a->N < 1) return GDN_ERR_INVALID_ARG;
  } else if (a->N != a->B) {
    return GDN_ERR_INVALID_ARG;
  }
  if ((long)a->B * a->T > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  const bool tokens = (long)a->B * a->T > 0;
  if (tokens && (!a->q || !a->k || !a->v || !a->o)) return GDN_ERR_INVALID_ARG;
  if (tokens && !operands_ok(a->gate, a->write, a->beta, a->log_alpha)) return GDN_ERR_INVALID_ARG;
  if (a->gate == GDN_GATE_NONE && a->log_alpha) return GDN_ERR_INVALID_ARG;
  if (a->write == GDN_WRITE_ADD && a->beta) return GDN_ERR_INVALID_ARG;
  const void *p16[] = {a->q, a->k, a->v, a->o, a->initial_state, a->final_state};
  for (const void *p : p16)
    if (p && !aligned(p, 16)) return GDN_ERR_INVALID_ARG;
  const size_t la_align = a->gate == GDN_GATE_KEY ? 16 : 4;
  if ((a->beta && !aligned(a->beta, 4)) || (a->log_alpha && !aligned(a->log_alpha, la_align)) ||
      (a->cu_seqlens && !aligned(a->cu_seqlens, 4)))
    return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t order_bytes(const gdn_fwd_args *a) {
  if (!a->cu_seqlens || a->N > 8192) return 0;
  return align256((size_t)a->N * sizeof(int32_t));
}

// The pipelined kernel takes bf16 with d_k = 128; everything else runs on the fused
// kernel.
bool use_pipe(const gdn_fwd_args *a) { return a->dtype == GDN_BF16 && a->d_k == 128; }
// The per-key-channel gate on the pipelined kernel: a first pass prepares every
// chunk's operands in the workspace.
bool key_pipe(const gdn_fwd_args *a) { return a->gate == GDN_GATE_KEY && use_pipe(a); }
struct KeyLayout {
  long slots;
  size_t kq, tp, eg;  // bytes of one pre-scaled K/Q array, the T/P images, e^{g_C}
  size_t total() const { return 3 * kq + tp + eg; }
};
KeyLayout key_layout(const gdn_fwd_args *a) {
  KeyLayout L{0, 0, 0, 0};
  if (!key_pipe(a)) return L;
  const long tokens = (long)a->B * a->T;
  L.slots = gdn::key_slots(tokens, a->N);
  L.kq = align256((size_t)tokens * a->H * 128 * 2);
  L.tp = align256((size_t)L.slots * a->H * 16384);
  L.eg = align256((size_t)L.slots * a->H * 128 * 4);
  return L;
}

int check_step(const gdn_step_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  if (a->N < 0 || a->H <= 0) return GDN_ERR_INVALID_ARG;
  if (a->dtype != GDN_F32 && a->dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (!gate_ok(a->gate) || !write_ok(a->write)) return GDN_ERR_INVALID_ARG;
  if (!head_dim_ok(a->d_k) || !head_dim_ok(a->d_v)) return GDN_ERR_UNSUPPORTED;
  if (a->N == 0) return GDN_OK;
  if (!a->q || !a->k || !a->v || !a->state || !a->o) return GDN_ERR_INVALID_ARG;
  if (!operands_ok(a->gate, a->write, a->beta, a->log_alpha)) return GDN_ERR_INVALID_ARG;
  if (!aligned(a->state, 16) || !aligned(a->q, 4) || !aligned(a->k, 4) || !aligned(a->v, 4) ||
      !aligned(a->o, 4) || !aligned(a->beta, 4) || (a->log_alpha && !aligned(a->log_alpha, 4)))
    return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

int check_decode(const gdn_decode_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  if (a->N < 0 || a->L < 1 || a->H <= 0 || a->pool_size < 1) return GDN_ERR_INVALID_ARG;
  if ((long long)a->N * a->H > INT32_MAX || (long long)a->N * a->L > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  if (a->dtype != GDN_F32 && a->dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (!gate_ok(a->gate) || !write_ok(a->write)) return GDN_ERR_INVALID_ARG;
  if (!head_dim_ok(a->d_k) || !head_dim_ok(a->d_v)) return GDN_ERR_UNSUPPORTED;
  if (a->N == 0) return GDN_OK;
  if (!a->q || !a->k || !a->v || !a->state_pool || !a->src_slots || !a->dst_slots || !a->o)
    return GDN_ERR_INVALID_ARG;
  if (!operands_ok(a->gate, a->write, a->beta, a->log_alpha)) return GDN_ERR_INVALID_ARG;
  if (!aligned(a->state_pool, 16) || !aligned(a->q, 4) || !aligned(a->k, 4) || !aligned(a->v, 4) ||
      !aligned(a->o, 4) || !aligned(a->beta, 4) || (a->log_alpha && !aligned(a->log_alpha, 4)) ||
      !aligned(a->src_slots, 4) || !aligned(a->dst_slots, 4))
    return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

// The forward arguments of a backward call, for the shared checks.
gdn_fwd_args fwd_of(const gdn_bwd_args *a) {
  gdn_fwd_args f{};
  f.B = a->B; f.T = a->T; f.H = a->H; f.d_k = a->d_k; f.d_v = a->d_v; f.chunk = a->chunk; f.N = a->N;
  f.dtype = a->dtype; f.gate = a->gate; f.write = a->write;
  f.q = a->q; f.k = a->k; f.v = a->v; f.beta = a->beta; f.log_alpha = a->log_alpha;
  f.initial_state = a->initial_state; f.cu_seqlens = a->cu_seqlens;
  f.o = const_cast<void *>(a->dout);  // checked like o (present, aligned); never written
  f.final_state = nullptr;
  return f;
}

int check_bwd(const gdn_bwd_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  const gdn_fwd_args f = fwd_of(a);
  const int st = check_fwd(&f);
  if (st != GDN_OK) return st;
  if (a->gate == GDN_GATE_KEY) return GDN_ERR_UNSUPPORTED;
  const bool tokens = (long)a->B * a->T > 0;
  if (tokens && (!a->dq || !a->dk || !a->dv)) return GDN_ERR_INVALID_ARG;
  // dbeta exactly for the delta write; dlog_alpha exactly for a gate (the constant
  // per-head decay's gradient is [H], written even without tokens)
  if ((tokens || a->dbeta) && ((a->write == GDN_WRITE_DELTA) != (a->dbeta != nullptr))) return GDN_ERR_INVALID_ARG;
  if ((tokens || a->gate == GDN_GATE_HEAD_CONST || a->dlog_alpha) &&
      ((a->gate != GDN_GATE_NONE) != (a->dlog_alpha != nullptr)))
    return GDN_ERR_INVALID_ARG;
  const void *p16[] = {a->dq, a->dk, a->dv, a->dfinal_state, a->dinitial_state};
  for (const void *p : p16)
    if (p && !aligned(p, 16)) return GDN_ERR_INVALID_ARG;
  if ((a->dbeta && !aligned(a->dbeta, 4)) || (a->dlog_alpha && !aligned(a->dlog_alpha, 4)))
    return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

int check_dplr(const gdn_dplr_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  gdn_fwd_args f{};
  f.B = a->B; f.T = a->T; f.H = a->H; f.d_k = a->d_k; f.d_v = a->d_v; f.chunk = a->chunk; f.N = a->N;
  f.dtype = a->dtype; f.gate = a->gate; f.write = GDN_WRITE_ADD;
  f.q = a->q; f.k = a->k; f.v = a->v; f.beta = nullptr; f.log_alpha = a->log_alpha;
  f.initial_state = a->initial_state; f.cu_seqlens = a->cu_seqlens; f.o = a->o; f.final_state = a->final_state;
  const int st = check_fwd(&f);
  if (st != GDN_OK) return st;
  if (a->gate != GDN_GATE_NONE && a->gate != GDN_GATE_HEAD) return GDN_ERR_UNSUPPORTED;
  if ((long)a->B * a->T > 0 && (!a->a || !a->b)) return GDN_ERR_INVALID_ARG;
  if ((a->a && !aligned(a->a, 16)) || (a->b && !aligned(a->b, 16))) return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

int check_dplr_step(const gdn_dplr_step_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  if (a->N < 0 || a->H <= 0) return GDN_ERR_INVALID_ARG;
  if (a->dtype != GDN_F32 && a->dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (!gate_ok(a->gate)) return GDN_ERR_INVALID_ARG;
  if (!head_dim_ok(a->d_k) || !head_dim_ok(a->d_v)) return GDN_ERR_UNSUPPORTED;
  if (a->N == 0) return GDN_OK;
  if (!a->q || !a->k || !a->a || !a->b || !a->v || !a->state || !a->o) return GDN_ERR_INVALID_ARG;
  if ((a->log_alpha != nullptr) != (a->gate != GDN_GATE_NONE)) return GDN_ERR_INVALID_ARG;
  const void *p4[] = {a->q, a->k, a->a, a->b, a->v, a->o, a->log_alpha};
  for (const void *p : p4)
    if (p && !aligned(p, 4)) return GDN_ERR_INVALID_ARG;
  if (!aligned(a->state, 16)) return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

int check_dplr_decode(const gdn_dplr_decode_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  if (a->N < 0 || a->L < 1 || a->H <= 0 || a->pool_size < 1) return GDN_ERR_INVALID_ARG;
  if ((long long)a->N * a->H > INT32_MAX || (long long)a->N * a->L > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  if (a->dtype != GDN_F32 && a->dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (!gate_ok(a->gate)) return GDN_ERR_INVALID_ARG;
  if (!head_dim_ok(a->d_k) || !head_dim_ok(a->d_v)) return GDN_ERR_UNSUPPORTED;
  if (a->N == 0) return GDN_OK;
  if (!a->q || !a->k || !a->a || !a->b || !a->v || !a->state_pool || !a->src_slots || !a->dst_slots || !a->o)
    return GDN_ERR_INVALID_ARG;
  if ((a->log_alpha != nullptr) != (a->gate != GDN_GATE_NONE)) return GDN_ERR_INVALID_ARG;
  const void *p4[] = {a->q, a->k, a->a, a->b, a->v, a->o, a->log_alpha, a->src_slots, a->dst_slots};
  for (const void *p : p4)
    if (p && !aligned(p, 4)) return GDN_ERR_INVALID_ARG;
  if (!aligned(a->state_pool, 16)) return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

struct BwdLayout {
  long slots;
  size_t states, tmat, part, dla;
  size_t total() const { return states + tmat + part + dla; }
};
BwdLayout bwd_layout(const gdn_bwd_args *a) {
  BwdLayout L{0, 0, 0, 0, 0};
  const long tokens = (long)a->B * a->T;
  L.slots = gdn::key_slots(tokens, a->N);
  L.states = align256((size_t)L.slots * a->H * a->d_k * a->d_v * 4);
  if (a->write == GDN_WRITE_DELTA) L.tmat = align256((size_t)L.slots * a->H * 64 * 64 * 4);  // T per chunk
  L.part = align256((size_t)L.slots * a->H * (a->d_v / 32) * gdn::bwd_part_floats(a->d_k) * 4);
  // the constant per-head decay: per-token gradients, summed per head afterwards
  if (a->gate == GDN_GATE_HEAD_CONST) L.dla = align256((size_t)tokens * a->H * 4);
  return L;
}

}  // namespace

extern "C" {

size_t gdn_bwd_workspace_size(const gdn_bwd_args *a) {
  if (check_bwd(a) != GDN_OK) return 0;
  return bwd_layout(a).total();
}

int gdn_bwd_chunked(const gdn_bwd_args *a, void *hip_stream) {
  const int st = check_bwd(a);
  if (st != GDN_OK) return st;
  const BwdLayout L = bwd_layout(a);
  if (!a->workspace || a->workspace_bytes < L.total() || !aligned(a->workspace, 256)) return GDN_ERR_WORKSPACE;
  const long tokens = (long)a->B * a->T;
  if (a->N == 0 || tokens == 0) {
    // no tokens: the initial-state gradient is the final-state gradient (or zero), and a
    // constant decay's gradient is zero
    if (a->gate == GDN_GATE_HEAD_CONST &&
        gdn::launch_sum_tokens(nullptr, 0, a->H, a->dlog_alpha, (hipStream_t)hip_stream) != hipSuccess)
      return GDN_ERR_HIP;
    if (a->dinitial_state && a->N > 0) {
      const size_t bytes = (size_t)a->N * a->H * a->d_k * a->d_v * 4;
      hipError_t e = a->dfinal_state
                         ? hipMemcpyAsync(a->dinitial_state, a->dfinal_state, bytes, hipMemcpyDeviceToDevice,
                                          (hipStream_t)hip_stream)
                         : hipMemsetAsync(a->dinitial_state, 0, bytes, (hipStream_t)hip_stream);
      if (e != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
  }
  hipStream_t stream = (hipStream_t)hip_stream;
  char *ws = (char *)a->workspace;
  // 1. forward recomputation: every chunk's entering state
  gdn::FwdParams fp;
  fp.q = a->q;
  fp.k = a->k;
  fp.v = a->v;
  fp.beta = a->beta;
  fp.log_alpha = a->log_alpha;
  fp.init_state = a->initial_state;
  fp.final_state = nullptr;
  fp.o = nullptr;
  fp.cu_seqlens = a->cu_seqlens;
  fp.order = nullptr;
  fp.k_hat = nullptr;
  fp.tp_img = nullptr;
  fp.egc = nullptr;
  fp.N = a->N;
  fp.H = a->H;
  fp.T = a->T;
  fp.dv = a->d_v;
  const bool add = a->write == GDN_WRITE_ADD;
  const int la_stride = a->gate == GDN_GATE_HEAD_CONST ? 0 : a->H;
  fp.la_stride = la_stride;
  fp.chunk_states = (float *)ws;
  const gdn_fwd_args f = fwd_of(a);
  if (use_pipe(&f)) {  // bf16, d_k = 128: the pipelined kernel, chunk states instead of o
    fp.nb = a->d_v / 64;
    if (gdn::launch_fwd_pipe(fp, (int)a->gate, add, stream) != hipSuccess) return GDN_ERR_HIP;
  } else {
    const int dvb = choose_dvb(a->N, a->H, a->d_v);
    fp.nb = a->d_v / dvb;
    if (gdn::launch_fwd_fused(fp, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, dvb, kernel_gate(a->gate), add, stream) !=
        hipSuccess)
      return GDN_ERR_HIP;
  }
  // 2. reverse state pass and 3. per-chunk gradients
  gdn::BwdParams bp;
  bp.q = a->q;
  bp.k = a->k;
  bp.v = a->v;
  bp.dout = a->dout;
  bp.beta = a->beta;
  bp.log_alpha = a->log_alpha;
  bp.dfinal = a->dfinal_state;
  bp.cu_seqlens = a->cu_seqlens;
  bp.states = (const float *)ws;
  bp.tmat = (float *)(ws + L.states);
  bp.part = (float *)(ws + L.states + L.tmat);
  bp.dq = a->dq;
  bp.dk = a->dk;
  bp.dv_out = a->dv;
  bp.dbeta = a->dbeta;
  float *const dla_tok = (float *)(ws + L.states + L.tmat + L.part);
  bp.dlog_alpha = a->gate == GDN_GATE_HEAD_CONST ? dla_tok : a->dlog_alpha;
  bp.la_stride = la_stride;
  bp.dinit = a->dinitial_state;
  bp.N = a->N;
  bp.H = a->H;
  bp.T = a->T;
  bp.dv = a->d_v;
  bp.slots = L.slots;
  if (gdn::launch_bwd(bp, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, kernel_gate(a->gate), add, stream) != hipSuccess)
    return GDN_ERR_HIP;
  if (a->gate == GDN_GATE_HEAD_CONST &&
      gdn::launch_sum_tokens(dla_tok, tokens, a->H, a->dlog_alpha, stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

size_t gdn_fwd_workspace_size(const gdn_fwd_args *a) {
  if (check_fwd(a) != GDN_OK) return 0;
  return order_bytes(a) + key_layout(a).total();
}

int gdn_fwd_chunked(const gdn_fwd_args *a, void *hip_stream) {
  const int st = check_fwd(a);
  if (st != GDN_OK) return st;
  const size_t obytes = order_bytes(a);
  const KeyLayout L = key_layout(a);
  const size_t need = obytes + L.total();
  if (need && (!a->workspace || a->workspace_bytes < need || !aligned(a->workspace, 256)))
    return GDN_ERR_WORKSPACE;
  if (a->N == 0) return GDN_OK;
  hipStream_t stream = (hipStream_t)hip_stream;
  gdn::FwdParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.beta = a->beta;
  p.log_alpha = a->log_alpha;
  p.init_state = a->initial_state;
  p.final_state = a->final_state;
  p.o = a->o;
  p.cu_seqlens = a->cu_seqlens;
  p.order = obytes ? (const int32_t *)a->workspace : nullptr;
  p.k_hat = nullptr;
  p.tp_img = nullptr;
  p.egc = nullptr;
  p.N = a->N;
  p.H = a->H;
  p.T = a->T;
  p.dv = a->d_v;
  p.la_stride = a->gate == GDN_GATE_HEAD_CONST ? 0 : a->H;
  p.chunk_states = nullptr;
  if (obytes) {
    if (gdn::launch_seq_order(a->cu_seqlens, a->N, (int32_t *)a->workspace, stream) != hipSuccess)
      return GDN_ERR_HIP;
  }
  if (L.slots) {
    char *ws = (char *)a->workspace + obytes;
    gdn::KeyPrepParams kp;
    kp.q = a->q;
    kp.k = a->k;
    kp.beta = a->beta;
    kp.log_alpha = a->log_alpha;
    kp.cu_seqlens = a->cu_seqlens;
    kp.k_g = ws;
    kp.q_g = ws + L.kq;
    kp.k_hat = ws + 2 * L.kq;
    kp.tp_img = ws + 3 * L.kq;
    kp.egc = (float *)(ws + 3 * L.kq + L.tp);
    kp.N = a->N;
    kp.H = a->H;
    kp.T = a->T;
    if (gdn::launch_key_prep(kp, L.slots, a->write == GDN_WRITE_ADD, stream) != hipSuccess) return GDN_ERR_HIP;
    p.k = kp.k_g;  // the pipelined kernel then reads the pre-scaled operands
    p.q = kp.q_g;
    p.k_hat = kp.k_hat;
    p.tp_img = kp.tp_img;
    p.egc = kp.egc;
  }
  if (use_pipe(a)) {
    p.nb = a->d_v / 64;
    if (gdn::launch_fwd_pipe(p, (int)a->gate, a->write == GDN_WRITE_ADD, stream) != hipSuccess)
      return GDN_ERR_HIP;
    return GDN_OK;
  }
  const int dvb = choose_dvb(a->N, a->H, a->d_v);
  p.nb = a->d_v / dvb;
  if (gdn::launch_fwd_fused(p, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, dvb, kernel_gate(a->gate),
                            a->write == GDN_WRITE_ADD, stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_fwd_recurrent_step(const gdn_step_args *a, void *hip_stream) {
  const int st = check_step(a);
  if (st != GDN_OK) return st;
  if (a->N == 0) return GDN_OK;
  gdn::StepParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.beta = a->beta;
  p.log_alpha = a->log_alpha;
  p.state = a->state;
  p.o = a->o;
  p.N = a->N;
  p.H = a->H;
  p.la_stride = a->gate == GDN_GATE_HEAD_CONST ? 0 : a->H;
  if (gdn::launch_recurrent_step(p, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, a->d_v, kernel_gate(a->gate),
                                 a->write == GDN_WRITE_ADD, (hipStream_t)hip_stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_fwd_decode(const gdn_decode_args *a, void *hip_stream) {
  const int st = check_decode(a);
  if (st != GDN_OK) return st;
  if (a->N == 0) return GDN_OK;
  gdn::DecodeParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.beta = a->beta;
  p.log_alpha = a->log_alpha;
  p.pool = a->state_pool;
  p.src = a->src_slots;
  p.dst = a->dst_slots;
  p.o = a->o;
  p.N = a->N;
  p.L = a->L;
  p.H = a->H;
  p.P = a->pool_size;
  p.la_stride = a->gate == GDN_GATE_HEAD_CONST ? 0 : a->H;
  if (gdn::launch_decode(p, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, a->d_v, kernel_gate(a->gate),
                         a->write == GDN_WRITE_ADD, (hipStream_t)hip_stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_fwd_dplr(const gdn_dplr_args *a, void *hip_stream) {
  const int st = check_dplr(a);
  if (st != GDN_OK) return st;
  if (a->N == 0) return GDN_OK;
  gdn::DplrParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.a = a->a;
  p.b = a->b;
  p.log_alpha = a->log_alpha;
  p.init_state = a->initial_state;
  p.final_state = a->final_state;
  p.o = a->o;
  p.cu_seqlens = a->cu_seqlens;
  p.N = a->N;
  p.H = a->H;
  p.T = a->T;
  p.dv = a->d_v;
  if (gdn::launch_dplr(p, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, (int)a->gate, (hipStream_t)hip_stream) !=
      hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_fwd_dplr_step(const gdn_dplr_step_args *a, void *hip_stream) {
  const int st = check_dplr_step(a);
  if (st != GDN_OK) return st;
  if (a->N == 0) return GDN_OK;
  gdn::DplrStepParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.a = a->a;
  p.b = a->b;
  p.log_alpha = a->log_alpha;
  p.state = a->state;
  p.o = a->o;
  p.N = a->N;
  p.H = a->H;
  p.la_stride = a->gate == GDN_GATE_HEAD_CONST ? 0 : a->H;
  if (gdn::launch_dplr_step(p, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, a->d_v, kernel_gate(a->gate),
                            (hipStream_t)hip_stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_fwd_dplr_decode(const gdn_dplr_decode_args *a, void *hip_stream) {
  const int st = check_dplr_decode(a);
  if (st != GDN_OK) return st;
  if (a->N == 0) return GDN_OK;
  gdn::DplrDecodeParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.a = a->a;
  p.b = a->b;
  p.log_alpha = a->log_alpha;
  p.pool = a->state_pool;
  p.src = a->src_slots;
  p.dst = a->dst_slots;
  p.o = a->o;
  p.N = a->N;
  p.L = a->L;
  p.H = a->H;
  p.P = a->pool_size;
  p.la_stride = a->gate == GDN_GATE_HEAD_CONST ? 0 : a->H;
  if (gdn::launch_dplr_decode(p, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, a->d_v, kernel_gate(a->gate),
                              (hipStream_t)hip_stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

const char *gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported shape or mode";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int gdn_version(void) { return 200; }

}  // extern "C"
