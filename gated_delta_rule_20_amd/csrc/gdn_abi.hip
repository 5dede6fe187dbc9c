// gdn_abi.hip -- host side of the C ABI declared in include/gdn.h.
//
// Validates every argument on the host, chooses the kernel configuration, carves
// the caller's workspace and launches on the caller's stream.  Nothing here
// allocates, copies or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "gdn.h"
#include "gdn_kernels.h"

// Scratch memory of gdn_fwd_chunked_static: one array per GPU, alive until the process
// ends.  Its name is a host-side stand-in, never a device address: host code uses only
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[GDN_STATIC_SCRATCH_BYTES];

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool gate_ok(int g) {
  return g == GDN_GATE_NONE || g == GDN_GATE_HEAD || g == GDN_GATE_KEY || g == GDN_GATE_HEAD_CONST;
}
bool write_ok(int w) { return w == GDN_WRITE_DELTA || w == GDN_WRITE_ADD; }
// The integer a caller stored in an enum field, read without loading the enum type (a
// value outside the enumerators must be rejected, not loaded: that load is undefined
// in C++).
template <class En> int raw(const En &e) {
  static_assert(sizeof(En) == sizeof(int), "enum fields are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}
bool dtype_ok(int t) { return t == GDN_F32 || t == GDN_BF16; }
// Kernel gate of an ABI gate: the constant per-head gate is the scalar gate read
// with a token stride of 0.
int kernel_gate(int g) { return g == GDN_GATE_HEAD_CONST ? gdn::GATE_HEAD : g; }
// beta is given exactly for the delta write, log_alpha exactly for a gate.
bool operands_ok(int gate, int write, const void *beta, const void *log_alpha) {
  return (beta != nullptr) == (write == GDN_WRITE_DELTA) && (log_alpha != nullptr) == (gate != GDN_GATE_NONE);
}

// Value columns per workgroup of the fused kernel: 64, or 32 when there are too few
// (sequence, head) streams to give every compute unit a workgroup; always 32 for fp32
// I/O with d_k = 128, whose tiles leave LDS room for 32 columns only.
int choose_dvb(int N, int H, int dv, int dtype, int dk) {
  if (dtype == GDN_F32 && dk == 128) return 32;
  const long wg64 = (long)N * H * (dv / 64);
  return wg64 >= 256 ? 64 : 32;
}

int check_fwd(const gdn_fwd_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  if (a->B < 0 || a->T < 0 || a->H <= 0 || a->N < 0) return GDN_ERR_INVALID_ARG;
  if (!dtype_ok(raw(a->dtype)) || !gate_ok(raw(a->gate)) || !write_ok(raw(a->write))) return GDN_ERR_INVALID_ARG;
  if (a->chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (!head_dim_ok(a->d_k) || !head_dim_ok(a->d_v)) return GDN_ERR_UNSUPPORTED;
  // every offset inside one 64-token chunk of q, k or v must fit 32 bits
  if ((long)a->H * 64 * 256 > (long)UINT32_MAX) return GDN_ERR_UNSUPPORTED;
  if (a->cu_seqlens) {
    if (a->B != 1 || a->N < 1) return GDN_ERR_INVALID_ARG;
  } else if (a->N != a->B) {
    return GDN_ERR_INVALID_ARG;
  }
  if ((long)a->B * a->T > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  // every launch grid must fit a signed 32-bit count: per-stream grids have at most
  // d_v / 16 workgroups per (sequence, head); per-chunk grids one per (chunk slot, head),
  // with fewer than B T / 64 + N + 1 slots
  {
    const long long streams = (long long)a->N * a->H;
    const long long slots = ((long long)a->B * a->T + 63) / 64 + a->N + 1;
    if (streams * (a->d_v / 16) > INT32_MAX || slots * a->H > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  }
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
// The windowed per-key-channel forward: long batch-mode sequences run as consecutive
// windows of chunks, each launch preparing the next window's operands (N H items per
// chunk, one item at a time per CU) on the CUs that the state pass of the current one
// leaves free.  A window is the shortest of at least 16 chunks whose items fill whole
// rounds of those CUs (as nearly as whole chunks allow): a last, partial round would
// leave the state pass waiting for a few CUs.  At N = 2, H = 16, d_v = 128 (192 free
// CUs, 6 chunks per round) that is 18 chunks: 0.64 ms per forward call, against 0.66
// at 24 chunks, 0.69 at 20 and 0.78 at 32.
constexpr int KEY_WINDOW_MIN = 16;
int key_window_len(const gdn_fwd_args *a, int free_cus) {
  const double per_round = (double)free_cus / ((double)a->N * a->H);  // chunks per round
  const double rounds = std::ceil(KEY_WINDOW_MIN / per_round);
  return std::max(KEY_WINDOW_MIN, (int)std::floor(rounds * per_round));
}
int key_windows(const gdn_fwd_args *a, int len) {
  const int nchunks = (a->T + 63) / 64;
  return (!a->cu_seqlens && nchunks >= 2 * len) ? (nchunks + len - 1) / len : 1;
}
struct KeyLayout {
  long slots;
  size_t kq, tp, eg, carry;  // bytes of one pre-scaled K/Q array, the T/P images, e^{g_C},
                             // the state between windows
  size_t total() const { return 3 * kq + tp + eg + carry; }
};
KeyLayout key_layout(const gdn_fwd_args *a) {
  KeyLayout L{0, 0, 0, 0, 0};
  if (!key_pipe(a)) return L;
  const long tokens = (long)a->B * a->T;
  L.slots = gdn::key_slots(tokens, a->N);
  L.kq = align256((size_t)tokens * a->H * 128 * 2);
  L.tp = align256((size_t)L.slots * a->H * 16384);
  L.eg = align256((size_t)L.slots * a->H * 128 * 4);
  if (key_windows(a, KEY_WINDOW_MIN) > 1)  // every window length is at least the minimum
    L.carry = align256((size_t)a->N * a->H * 128 * a->d_v * 4);
  return L;
}

int check_step(const gdn_step_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  if (a->N < 0 || a->H <= 0) return GDN_ERR_INVALID_ARG;
  if ((long long)a->N * a->H > INT32_MAX) return GDN_ERR_UNSUPPORTED;  // one workgroup per (stream, head)
  if (!dtype_ok(raw(a->dtype)) || !gate_ok(raw(a->gate)) || !write_ok(raw(a->write))) return GDN_ERR_INVALID_ARG;
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
  if (!dtype_ok(raw(a->dtype)) || !gate_ok(raw(a->gate)) || !write_ok(raw(a->write))) return GDN_ERR_INVALID_ARG;
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
  if (!dtype_ok(raw(a->dtype)) || !gate_ok(raw(a->gate)) || !write_ok(raw(a->write))) return GDN_ERR_INVALID_ARG;
  const gdn_fwd_args f = fwd_of(a);
  const int st = check_fwd(&f);
  if (st != GDN_OK) return st;
  // fp32 I/O at d_k = 128 has gradients only with the per-key-channel gate
  if (a->dtype == GDN_F32 && a->d_k != 64 && a->gate != GDN_GATE_KEY) return GDN_ERR_UNSUPPORTED;
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
  if (!dtype_ok(raw(a->dtype)) || !gate_ok(raw(a->gate))) return GDN_ERR_INVALID_ARG;
  gdn_fwd_args f{};
  f.B = a->B; f.T = a->T; f.H = a->H; f.d_k = a->d_k; f.d_v = a->d_v; f.chunk = a->chunk; f.N = a->N;
  f.dtype = a->dtype; f.gate = a->gate; f.write = GDN_WRITE_ADD;
  f.q = a->q; f.k = a->k; f.v = a->v; f.beta = nullptr; f.log_alpha = a->log_alpha;
  f.initial_state = a->initial_state; f.cu_seqlens = a->cu_seqlens; f.o = a->o; f.final_state = a->final_state;
  const int st = check_fwd(&f);
  if (st != GDN_OK) return st;
  if (a->dtype == GDN_F32 && a->d_k != 64) return GDN_ERR_UNSUPPORTED;
  if ((long)a->B * a->T > 0 && (!a->a || !a->b)) return GDN_ERR_INVALID_ARG;
  if ((a->a && !aligned(a->a, 16)) || (a->b && !aligned(a->b, 16))) return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

int check_dplr_step(const gdn_dplr_step_args *a) {
  if (!a) return GDN_ERR_INVALID_ARG;
  if (a->N < 0 || a->H <= 0) return GDN_ERR_INVALID_ARG;
  if ((long long)a->N * a->H > INT32_MAX) return GDN_ERR_UNSUPPORTED;  // one workgroup per (stream, head)
  if (!dtype_ok(raw(a->dtype)) || !gate_ok(raw(a->gate))) return GDN_ERR_INVALID_ARG;
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
  if (!dtype_ok(raw(a->dtype)) || !gate_ok(raw(a->gate))) return GDN_ERR_INVALID_ARG;
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

// The per-key-channel gate of the diagonal-plus-low-rank forward: the arrays of
// DplrKeyParams, in this order (tm, aak, pqb, pqk, at, qg, bhT, khT, gam)
struct DplrKeyLayout {
  long slots;
  size_t sz[9];
  size_t total() const {
    size_t t = 0;
    for (size_t x : sz) t += x;
    return t;
  }
};
DplrKeyLayout dplr_key_layout(const gdn_dplr_args *a) {
  DplrKeyLayout L{};
  if (a->gate != GDN_GATE_KEY) return L;
  L.slots = gdn::key_slots((long)a->B * a->T, a->N);
  const size_t sh = (size_t)L.slots * a->H, dk = a->d_k;
  const size_t sizes[9] = {sh * 4096 * 4, sh * 4096 * 4, sh * 4096 * 4, sh * 4096 * 4, sh * 64 * dk * 4,
                           sh * 64 * dk * 4, sh * dk * 64 * 4, sh * dk * 64 * 4, sh * dk * 4};
  for (int i = 0; i < 9; ++i) L.sz[i] = align256(sizes[i]);
  return L;
}

// The backward's workspace: the fp32 arrays of BwdKeyParams / BwdParams, in this order,
// then the constant decay's per-token gradients
struct BwdLayout {
  long slots;
  size_t sz[13];
  size_t total() const {
    size_t t = 0;
    for (size_t x : sz) t += x;
    return t;
  }
};
BwdLayout bwd_layout(const gdn_bwd_args *a) {
  BwdLayout L{};
  const long tokens = (long)a->B * a->T;
  L.slots = gdn::key_slots(tokens, a->N);
  const size_t sh = (size_t)L.slots * a->H, dk = a->d_k, dv = a->d_v;
  const bool delta = a->write == GDN_WRITE_DELTA, key = a->gate == GDN_GATE_KEY;
  const size_t es = a->dtype == GDN_BF16 ? 2 : 4;  // the scalar gates' Q^T and K^T: I/O dtype
  const size_t sizes[13] = {
      sh * dk * dv * 4,                              // states
      sh * dk * dv * 4,                              // chunk-end state gradients
      sh * 64 * dv * 4,                              // dDelta
      delta ? sh * 4096 * 4 : 0,                     // T
      delta ? sh * 4096 * 4 : 0,                     // T^T
      sh * 4096 * 4,                                 // P^T
      key && delta ? sh * 64 * dk * 4 : 0,           // K e^G (per key channel)
      key ? sh * 64 * dk * 4 : sh * 128 * 4,         // K e^{g_C - G}; scalar gates: e^g, e^{g_C - g} rows
      delta ? sh * dk * 64 * (key ? 4 : es) : 0,     // (K e^G)^T; scalar gates: K^T
      sh * dk * 64 * (key ? 4 : es),                 // (Q e^G)^T; scalar gates: Q^T
      key ? sh * dk * 64 * 4 : 0,                    // (K e^{g_C - G})^T (per key channel)
      sh * dk * 4,                                   // e^{g_C}
      a->gate == GDN_GATE_HEAD_CONST ? (size_t)tokens * a->H * 4 : 0};  // per-token decay gradients
  for (int i = 0; i < 13; ++i) L.sz[i] = align256(sizes[i]);
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
  const size_t need = L.total();
  if (!a->workspace || a->workspace_bytes < need || !aligned(a->workspace, 256)) return GDN_ERR_WORKSPACE;
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
                         : gdn::launch_fill_zero(a->dinitial_state, bytes / 4, (hipStream_t)hip_stream);
      if (e != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
  }
  hipStream_t stream = (hipStream_t)hip_stream;
  char *ws = (char *)a->workspace;
  float *arr[13];
  {
    size_t off = 0;
    for (int i = 0; i < 13; ++i) {
      arr[i] = (float *)(ws + off);
      off += L.sz[i];
    }
  }
  if (a->gate == GDN_GATE_KEY) {
    gdn::BwdKeyParams kp;
    kp.q = a->q;
    kp.k = a->k;
    kp.v = a->v;
    kp.dout = a->dout;
    kp.beta = a->beta;
    kp.log_alpha = a->log_alpha;
    kp.init_state = a->initial_state;
    kp.dfinal = a->dfinal_state;
    kp.cu_seqlens = a->cu_seqlens;
    kp.states = arr[0];
    kp.dmc = arr[1];
    kp.dd = arr[2];
    kp.tm = arr[3];
    kp.tmT = arr[4];
    kp.pmT = arr[5];
    kp.kt = arr[6];
    kp.kh = arr[7];
    kp.ktT = arr[8];
    kp.qtT = arr[9];
    kp.khT = arr[10];
    kp.gam = arr[11];
    kp.dq = a->dq;
    kp.dk = a->dk;
    kp.dv_out = a->dv;
    kp.dbeta = a->dbeta;
    kp.dlog_alpha = a->dlog_alpha;
    kp.dinit = a->dinitial_state;
    kp.N = a->N;
    kp.H = a->H;
    kp.T = a->T;
    kp.dv = a->d_v;
    kp.slots = L.slots;
    kp.states_ready = 0;
    const gdn_fwd_args f = fwd_of(a);
    const KeyLayout FL = key_layout(&f);
    if (FL.slots && FL.total() <= L.sz[1] + L.sz[2]) {
      // bf16 with d_k = 128: the forward's own per-channel path recomputes the chunk
      // states (its preparation's operands go to the chunk-end-gradient and dDelta
      // arrays, which the reverse pass writes only afterwards)
      char *fw = (char *)arr[1];
      gdn::KeyPrepParams pp;
      pp.q = a->q;
      pp.k = a->k;
      pp.beta = a->beta;
      pp.log_alpha = a->log_alpha;
      pp.cu_seqlens = a->cu_seqlens;
      pp.k_g = fw;
      pp.q_g = fw + FL.kq;
      pp.k_hat = fw + 2 * FL.kq;
      pp.tp_img = fw + 3 * FL.kq;
      pp.egc = (float *)(fw + 3 * FL.kq + FL.tp);
      pp.N = a->N;
      pp.H = a->H;
      pp.T = a->T;
      const bool add = a->write == GDN_WRITE_ADD;
      const int ns = a->N * a->H * (a->d_v / 64), free_cus = gdn::device_cus() - ns;
      const int wlen = free_cus > 0 ? key_window_len(&f, free_cus) : 0;
      const int windows = free_cus > 0 ? key_windows(&f, wlen) : 1;
      const bool windowed = windows > 1;
      if (windowed) {  // this launch prepares window 0 only
        pp.c_lo = 0;
        pp.c_hi = wlen;
        pp.win_items = 1;
      }
      if (gdn::launch_key_prep(pp, FL.slots, add, stream) != hipSuccess) return GDN_ERR_HIP;
      gdn::FwdParams fp;
      fp.q = pp.q_g;
      fp.k = pp.k_g;
      fp.v = a->v;
      fp.beta = a->beta;
      fp.log_alpha = a->log_alpha;
      fp.init_state = a->initial_state;
      fp.final_state = nullptr;
      fp.o = nullptr;
      fp.cu_seqlens = a->cu_seqlens;
      fp.order = nullptr;
      fp.k_hat = pp.k_hat;
      fp.tp_img = pp.tp_img;
      fp.egc = pp.egc;
      fp.N = a->N;
      fp.H = a->H;
      fp.T = a->T;
      fp.dv = a->d_v;
      fp.nb = a->d_v / 64;
      fp.la_stride = a->H;
      fp.chunk_states = arr[0];
      if (windowed) {
        // as in the forward: window w's state pass shares a launch with window w + 1's
        // preparation
        float *carry = (float *)(fw + 3 * FL.kq + FL.tp + FL.eg);
        for (int w = 0; w < windows; ++w) {
          fp.c_lo = w * wlen;
          fp.c_hi = (w + 1) * wlen;
          fp.init_state = w == 0 ? a->initial_state : carry;
          fp.final_state = w == windows - 1 ? nullptr : carry;
          pp.c_lo = (w + 1) * wlen;
          pp.c_hi = (w + 2) * wlen;
          if (gdn::launch_key_window(fp, pp, FL.slots, w + 1 < windows ? free_cus : 0, add, stream) != hipSuccess)
            return GDN_ERR_HIP;
        }
      } else if (gdn::launch_fwd_pipe(fp, gdn::GATE_KEY, add, stream) != hipSuccess) {
        return GDN_ERR_HIP;
      }
      kp.states_ready = 1;
    }
    if (gdn::launch_bwd_key(kp, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, a->write == GDN_WRITE_ADD, stream) !=
        hipSuccess)
      return GDN_ERR_HIP;
    return GDN_OK;
  }
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
  fp.chunk_states = arr[0];
  const gdn_fwd_args f = fwd_of(a);
  if (use_pipe(&f)) {  // bf16, d_k = 128: the pipelined kernel, chunk states instead of o
    fp.nb = a->d_v / 64;
    if (gdn::launch_fwd_pipe(fp, (int)a->gate, add, stream) != hipSuccess) return GDN_ERR_HIP;
  } else {
    const int dvb = choose_dvb(a->N, a->H, a->d_v, a->dtype, a->d_k);
    fp.nb = a->d_v / dvb;
    if (gdn::launch_fwd_fused(fp, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, dvb, kernel_gate(a->gate), add, stream) !=
        hipSuccess)
      return GDN_ERR_HIP;
  }
  // 2. operands, 3. reverse state pass, 4. per-chunk gradients
  gdn::BwdParams bp;
  bp.q = a->q;
  bp.k = a->k;
  bp.v = a->v;
  bp.dout = a->dout;
  bp.beta = a->beta;
  bp.log_alpha = a->log_alpha;
  bp.dfinal = a->dfinal_state;
  bp.cu_seqlens = a->cu_seqlens;
  bp.states = arr[0];
  bp.dmc = arr[1];
  bp.dd = arr[2];
  bp.tm = arr[3];
  bp.tmT = arr[4];
  bp.pmT = arr[5];
  bp.egr = arr[7];
  bp.etr = arr[7] + (size_t)L.slots * a->H * 64;
  bp.kT = arr[8];
  bp.qT = arr[9];
  bp.gam = arr[11];
  bp.dq = a->dq;
  bp.dk = a->dk;
  bp.dv_out = a->dv;
  bp.dbeta = a->dbeta;
  float *const dla_tok = arr[12];
  bp.dlog_alpha = a->gate == GDN_GATE_HEAD_CONST ? dla_tok : a->dlog_alpha;
  bp.la_stride = la_stride;
  bp.dinit = a->dinitial_state;
  bp.N = a->N;
  bp.H = a->H;
  bp.T = a->T;
  bp.dv = a->d_v;
  bp.slots = L.slots;
  // the constant decay's per-token gradients are summed over every token of the call:
  // tokens that no valid sequence covers (outside [cu[0], cu[N]), or in a sequence
  // skipped for malformed offsets) must contribute zero
  if (a->gate == GDN_GATE_HEAD_CONST && gdn::launch_fill_zero(dla_tok, (size_t)tokens * a->H, stream) != hipSuccess)
    return GDN_ERR_HIP;
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

}  // extern "C"

namespace {

// The forward on a checked argument set, with its scratch memory at `ws` (need bytes,
// 256-aligned; may be NULL when need is 0).
int fwd_chunked_launch(const gdn_fwd_args *a, void *ws_base, void *hip_stream);

// Device address of this process's scratch array on the current device, looked up once
// per device (NULL if the lookup fails).
void *static_scratch() {
  static std::mutex mu;
  static void *ptr[256];
  static bool done[256];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = p;
    done[dev] = true;
  }
  return ptr[dev];
}

}  // namespace

extern "C" {

int gdn_fwd_chunked_static(const gdn_fwd_args *a, void *hip_stream) {
  const int st = check_fwd(a);
  if (st != GDN_OK) return st;
  const size_t need = order_bytes(a) + key_layout(a).total();
  if (need > GDN_STATIC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
  if (a->N == 0) return GDN_OK;
  void *ws = nullptr;
  if (need) {
    ws = static_scratch();
    if (!ws) return GDN_ERR_HIP;
  }
  return fwd_chunked_launch(a, ws, hip_stream);
}

int gdn_fwd_chunked(const gdn_fwd_args *a, void *hip_stream) {
  const int st = check_fwd(a);
  if (st != GDN_OK) return st;
  const size_t need = order_bytes(a) + key_layout(a).total();
  if (need && (!a->workspace || a->workspace_bytes < need || !aligned(a->workspace, 256)))
    return GDN_ERR_WORKSPACE;
  if (a->N == 0) return GDN_OK;
  return fwd_chunked_launch(a, a->workspace, hip_stream);
}

}  // extern "C"

namespace {

int fwd_chunked_launch(const gdn_fwd_args *a, void *ws_base, void *hip_stream) {
  const size_t obytes = order_bytes(a);
  const KeyLayout L = key_layout(a);
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
  p.order = obytes ? (const int32_t *)ws_base : nullptr;
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
    if (gdn::launch_seq_order(a->cu_seqlens, a->N, (int32_t *)ws_base, stream) != hipSuccess)
      return GDN_ERR_HIP;
  }
  if (L.slots) {
    char *ws = (char *)ws_base + obytes;
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
    p.k = kp.k_g;  // the pipelined kernel then reads the pre-scaled operands
    p.q = kp.q_g;
    p.k_hat = kp.k_hat;
    p.tp_img = kp.tp_img;
    p.egc = kp.egc;
    const bool add = a->write == GDN_WRITE_ADD;
    const int ns = a->N * a->H * (a->d_v / 64), free_cus = gdn::device_cus() - ns;
    const int wlen = free_cus > 0 ? key_window_len(a, free_cus) : 0;
    const int windows = free_cus > 0 ? key_windows(a, wlen) : 1;
    if (windows > 1) {
      // window w's state pass shares a launch with window w + 1's preparation
      float *carry = (float *)(ws + 3 * L.kq + L.tp + L.eg);
      p.nb = a->d_v / 64;
      kp.c_lo = 0;
      kp.c_hi = wlen;
      kp.win_items = 1;
      if (gdn::launch_key_prep(kp, L.slots, add, stream) != hipSuccess) return GDN_ERR_HIP;
      for (int w = 0; w < windows; ++w) {
        p.c_lo = w * wlen;
        p.c_hi = (w + 1) * wlen;
        p.init_state = w == 0 ? a->initial_state : carry;
        p.final_state = w == windows - 1 ? a->final_state : carry;
        kp.c_lo = (w + 1) * wlen;
        kp.c_hi = (w + 2) * wlen;
        if (gdn::launch_key_window(p, kp, L.slots, w + 1 < windows ? free_cus : 0, add, stream) != hipSuccess)
          return GDN_ERR_HIP;
      }
      return GDN_OK;
    }
    if (gdn::launch_key_prep(kp, L.slots, add, stream) != hipSuccess) return GDN_ERR_HIP;
  }
  if (use_pipe(a)) {
    p.nb = a->d_v / 64;
    if (gdn::launch_fwd_pipe(p, (int)a->gate, a->write == GDN_WRITE_ADD, stream) != hipSuccess)
      return GDN_ERR_HIP;
    return GDN_OK;
  }
  const int dvb = choose_dvb(a->N, a->H, a->d_v, a->dtype, a->d_k);
  p.nb = a->d_v / dvb;
  if (gdn::launch_fwd_fused(p, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, dvb, kernel_gate(a->gate),
                            a->write == GDN_WRITE_ADD, stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

}  // namespace

extern "C" {

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

size_t gdn_dplr_workspace_size(const gdn_dplr_args *a) {
  if (check_dplr(a) != GDN_OK) return 0;
  return dplr_key_layout(a).total();
}

int gdn_fwd_dplr(const gdn_dplr_args *a, void *hip_stream) {
  const int st = check_dplr(a);
  if (st != GDN_OK) return st;
  if (a->gate == GDN_GATE_KEY) {
    const DplrKeyLayout L = dplr_key_layout(a);
    const size_t need = L.total();
    if (need && (!a->workspace || a->workspace_bytes < need || !aligned(a->workspace, 256)))
      return GDN_ERR_WORKSPACE;
    if (a->N == 0) return GDN_OK;
    gdn::DplrKeyParams p;
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
    __bf16 **arr[8] = {&p.tm, &p.aak, &p.pqb, &p.pqk, &p.at, &p.qg, &p.bhT, &p.khT};
    char *ws = (char *)a->workspace;
    for (int i = 0; i < 8; ++i) {
      *arr[i] = (__bf16 *)ws;
      ws += L.sz[i];
    }
    p.gam = (float *)ws;
    p.N = a->N;
    p.H = a->H;
    p.T = a->T;
    p.dv = a->d_v;
    p.slots = (long)a->B * a->T > 0 ? L.slots : 0;
    if (gdn::launch_dplr_key(p, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, (hipStream_t)hip_stream) != hipSuccess)
      return GDN_ERR_HIP;
    return GDN_OK;
  }
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
  p.la_stride = a->gate == GDN_GATE_HEAD_CONST ? 0 : a->H;
  if (gdn::launch_dplr(p, a->dtype == GDN_BF16 ? 1 : 0, a->d_k, kernel_gate(a->gate), (hipStream_t)hip_stream) !=
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
