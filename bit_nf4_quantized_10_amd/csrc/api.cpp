// C ABI of the QLoRA NF4 library: argument validation, workspace carving and
// dispatch onto the caller's stream.  No allocation, no synchronisation
// (except nf4_status_read and qlora_timer_read, which exist to wait).
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/qlora_nf4.h"
#include "kernels.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

void counts(int64_t P, int64_t* n1, int64_t* n2) {
  *n1 = (P + NF4_BLOCK1 - 1) / NF4_BLOCK1;
  *n2 = (*n1 + NF4_BLOCK2 - 1) / NF4_BLOCK2;
}

// The encoder and decoders move packed codes and second-level codes as
// 32-bit words and the scales as fp32, so those buffers must be aligned.
bool state_ok(const nf4_state_t* s) {
  if (s == nullptr || s->numel < 1 || s->codes == nullptr || !aligned16(s->codes)) return false;
  if (s->absmax != nullptr) return (reinterpret_cast<uintptr_t>(s->absmax) & 3u) == 0;   // single level
  return s->qabsmax != nullptr && s->absmax2 != nullptr && s->offset != nullptr && aligned16(s->qabsmax) &&
         (reinterpret_cast<uintptr_t>(s->absmax2) & 3u) == 0 && (reinterpret_cast<uintptr_t>(s->offset) & 3u) == 0;
}

qn::NF4View view_of(const nf4_state_t* s) { return qn::NF4View{s->codes, s->qabsmax, s->absmax2, s->offset, s->absmax}; }

bool dtype_ok(int d) { return d == NF4_COMPUTE_BF16 || d == NF4_COMPUTE_F16; }

// Kernels address operands with 32-bit buffer offsets and mark masked lanes
// with offset 2^31; keeping every bf16 operand (X, G, Y, dX, A, B and the
// dequantized weight) under 1 GiB, and so every fp32 M x N buffer under
// 2 GiB, keeps all real offsets below 2^31.
constexpr int64_t kMaxOperandElems = int64_t(1) << 29;

bool layer_shape_ok(int64_t M, int64_t K, int64_t N, int64_t r) {
  return M >= 1 && K >= 1 && N >= 1 && r >= 1 && N % NF4_BLOCK1 == 0 && K % 8 == 0 && r % 8 == 0 &&
         r <= 256 && M <= (int64_t(1) << 20) && K <= (int64_t(1) << 24) && N <= (int64_t(1) << 24) &&
         M * K < kMaxOperandElems && M * N < kMaxOperandElems && K * N < kMaxOperandElems &&
         K * r < kMaxOperandElems && r * N < kMaxOperandElems;
}

// ---------------------------------------------------------------- timers
struct TimerSlot {
  bool enabled = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  std::vector<hipEvent_t> pool;
};
std::mutex g_timer_mu;
TimerSlot g_timers[QK_NUM_KERNELS];

// Events a timer slot holds once enabled: enough for 4096 timed launches
// between two reads.  They are created by qlora_timer_enable, never on the
// launch path; a launch that finds the pool empty is simply not timed (it
// is then not counted either, so the average stays right).
constexpr size_t kTimerEvents = 8192;

hipEvent_t take_event(TimerSlot& s) {
  if (s.pool.empty()) return nullptr;
  hipEvent_t e = s.pool.back();
  s.pool.pop_back();
  return e;
}

// ------------------------------------------------- no-allocation forward
// Scratch of qlora_linear_fwd_noalloc: one file-scope device array, which
// every GPU the library runs on holds (its own copy, at its own address)
// until the process ends.  Host code never passes the array's name to a
// kernel: that name is a host-side stand-in.  The device address comes from
// hipGetSymbolAddress, once per device with that device current, and is
// kept per device below.
static __device__ __align__(256) char scratch[NF4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device (looked up on the first call).
hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace qn {

Timer::Timer(int kernel_id, hipStream_t stream, bool packet)
    : id_(kernel_id), stream_(stream), stop_event_(nullptr), start_event_(nullptr), packet_stop_(nullptr) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  TimerSlot& s = g_timers[id_];
  if (!s.enabled) return;
  if (s.pool.size() < 2) return;
  hipEvent_t a = take_event(s), b = take_event(s);
  s.pending.emplace_back(a, b);
  if (packet) {
    start_event_ = a;
    packet_stop_ = b;
    return;
  }
  (void)hipEventRecord(a, stream_);
  stop_event_ = b;
}

void Timer::stop() {
  if (stop_event_ != nullptr) (void)hipEventRecord(static_cast<hipEvent_t>(stop_event_), stream_);
  stop_event_ = nullptr;
}

}  // namespace qn

extern "C" {

int nf4_sizes(int64_t numel, int64_t* code_bytes, int64_t* n1, int64_t* n2, int64_t* quant_workspace_bytes) {
  if (numel < 1) return NF4_EINVAL;
  int64_t a, b;
  counts(numel, &a, &b);
  if (code_bytes) *code_bytes = (numel + 1) / 2;
  if (n1) *n1 = a;
  if (n2) *n2 = b;
  if (quant_workspace_bytes) *quant_workspace_bytes = align256(4 * a) + align256(8 * b) + align256(4 * b);
  return NF4_OK;
}

int nf4_quantize(const float* W, const nf4_state_t* out, void* workspace, int64_t workspace_bytes,
                 int32_t* status, void* stream) {
  if (W == nullptr || !state_ok(out) || workspace == nullptr || status == nullptr) return NF4_EINVAL;
  if (!aligned16(W) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return NF4_EINVAL;
  int64_t n1, n2, need;
  nf4_sizes(out->numel, nullptr, &n1, &n2, &need);
  if (workspace_bytes < need) return NF4_EINVAL;
  if (out->numel >= (int64_t(1) << 29)) return NF4_EINVAL;   // fp32 input under 2 GiB (32-bit buffer offsets)
  char* ws = static_cast<char*>(workspace);
  float* ws_absmax = reinterpret_cast<float*>(ws);
  double* ws_gsum = reinterpret_cast<double*>(ws + align256(4 * n1));
  int32_t* ws_flags = reinterpret_cast<int32_t*>(ws + align256(4 * n1) + align256(8 * n2));
  hipError_t e = qn::launch_quantize(W, out->numel, out->codes, out->qabsmax, out->absmax2, out->offset, out->absmax,
                                     ws_absmax, ws_gsum, ws_flags, status, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4_OK : NF4_EHIP;
}

int nf4_dequantize(const nf4_state_t* state, void* out, int out_dtype, int32_t* status, void* stream) {
  if (!state_ok(state) || out == nullptr || !aligned16(out)) return NF4_EINVAL;
  if (out_dtype != NF4_OUT_F32 && out_dtype != NF4_OUT_BF16 && out_dtype != NF4_OUT_F16) return NF4_EINVAL;
  hipError_t e = qn::launch_dequantize(view_of(state), state->numel, out, out_dtype, status,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4_OK : NF4_EHIP;
}

int qlora_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t r, int64_t* fwd_bytes, int64_t* bwd_bytes) {
  if (!layer_shape_ok(M, K, N, r)) return NF4_EINVAL;
  if (fwd_bytes) *fwd_bytes = qn::fwd_workspace_bytes(M, K, N, r);
  if (bwd_bytes) *bwd_bytes = qn::bwd_workspace_bytes(M, K, N, r);
  return NF4_OK;
}

int qlora_linear_fwd_dt(int compute_dtype, int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X,
                        const nf4_state_t* W,
                     const uint16_t* A, const uint16_t* B, float c, uint16_t* Y, uint16_t* Z, void* workspace,
                     int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(compute_dtype) || !layer_shape_ok(M, K, N, r) || !state_ok(W) || W->numel != K * N) return NF4_EINVAL;
  if (!X || !A || !B || !Y || !workspace) return NF4_EINVAL;   // Z may be NULL
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y) || (Z && !aligned16(Z)) ||
      !aligned16(W->codes) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return NF4_EINVAL;
  if (workspace_bytes < qn::fwd_workspace_bytes(M, K, N, r)) return NF4_EINVAL;
  const qn::NF4View v = view_of(W);
  hipError_t e =
      qn::launch_fwd(M, K, N, r, X, v, A, B, c, Y, Z, workspace, static_cast<hipStream_t>(stream), compute_dtype);
  return e == hipSuccess ? NF4_OK : NF4_EHIP;
}

int qlora_linear_fwd_noalloc(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, const nf4_state_t* W,
                             const uint16_t* A, const uint16_t* B, float c, uint16_t* Y, uint16_t* Z, void* stream) {
  if (!layer_shape_ok(M, K, N, r) || !state_ok(W) || W->numel != K * N) return NF4_EINVAL;
  if (!X || !A || !B || !Y) return NF4_EINVAL;
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y) || (Z && !aligned16(Z))) return NF4_EINVAL;
  if (qn::fwd_workspace_bytes(M, K, N, r) > NF4_NOALLOC_SCRATCH_BYTES) return NF4_EINVAL;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return NF4_EHIP;
  // the forward's kernels need no zeroed scratch: every region they read
  // was written earlier in the same call
  hipError_t e = qn::launch_fwd(M, K, N, r, X, view_of(W), A, B, c, Y, Z, ws, static_cast<hipStream_t>(stream),
                                NF4_COMPUTE_BF16);
  return e == hipSuccess ? NF4_OK : NF4_EHIP;
}

int qlora_linear_fwd(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, const nf4_state_t* W,
                     const uint16_t* A, const uint16_t* B, float c, uint16_t* Y, uint16_t* Z, void* workspace,
                     int64_t workspace_bytes, void* stream) {
  return qlora_linear_fwd_dt(NF4_COMPUTE_BF16, M, K, N, r, X, W, A, B, c, Y, Z, workspace, workspace_bytes, stream);
}

int qlora_linear_bwd_dt(int compute_dtype, int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G,
                        const uint16_t* X,
                     const uint16_t* Z, const nf4_state_t* W, const uint16_t* A, const uint16_t* B, float c,
                     uint16_t* dX, float* dA, float* dB, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  if (!dtype_ok(compute_dtype) || !layer_shape_ok(M, K, N, r) || !state_ok(W) || W->numel != K * N) return NF4_EINVAL;
  if (!G || !X || !A || !B || !dA || !dB || !workspace) return NF4_EINVAL;   // Z may be NULL
  if (!aligned16(G) || !aligned16(X) || (Z && !aligned16(Z)) || !aligned16(A) || !aligned16(B) || !aligned16(dA) ||
      !aligned16(dB) || (dX && !aligned16(dX)) || !aligned16(W->codes) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return NF4_EINVAL;
  if (workspace_bytes < qn::bwd_workspace_bytes(M, K, N, r)) return NF4_EINVAL;
  const qn::NF4View v = view_of(W);
  hipError_t e = qn::launch_bwd(M, K, N, r, G, X, Z, v, A, B, c, dX, dA, dB, workspace,
                                static_cast<hipStream_t>(stream), compute_dtype);
  return e == hipSuccess ? NF4_OK : NF4_EHIP;
}

int qlora_linear_bwd(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G, const uint16_t* X,
                     const uint16_t* Z, const nf4_state_t* W, const uint16_t* A, const uint16_t* B, float c,
                     uint16_t* dX, float* dA, float* dB, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  return qlora_linear_bwd_dt(NF4_COMPUTE_BF16, M, K, N, r, G, X, Z, W, A, B, c, dX, dA, dB, workspace,
                             workspace_bytes, stream);
}

// Each member's rank must itself be a multiple of 8: the kernels move Z,
// (c B)ᵀ and the dB partials in 8-element chunks along the concatenated
// rank axis, and a chunk must never straddle two members.
static bool grouped_shape_ok(int64_t M, int64_t K, int g, const int64_t* N, int64_t r, int64_t* Ntot) {
  if (g < 1 || g > qn::kMaxGroupMembers || N == nullptr || r < 8 || r % 8 != 0) return false;
  int64_t tot = 0;
  for (int i = 0; i < g; ++i) {
    if (N[i] < 256 || N[i] % 256 != 0 || N[i] > (int64_t(1) << 24)) return false;
    tot += N[i];
  }
  *Ntot = tot;
  return layer_shape_ok(M, K, tot, g * r);
}

static bool grouped_states_ok(const nf4_state_t* W, int g, int64_t K, const int64_t* N, qn::NF4View* views) {
  if (W == nullptr) return false;
  for (int i = 0; i < g; ++i) {
    if (!state_ok(&W[i]) || W[i].numel != K * N[i]) return false;
    views[i] = view_of(&W[i]);
  }
  return true;
}

int qlora_grouped_workspace_bytes(int64_t M, int64_t K, int g, const int64_t* N, int64_t r, int64_t* fwd_bytes,
                                  int64_t* bwd_bytes) {
  int64_t Ntot;
  if (!grouped_shape_ok(M, K, g, N, r, &Ntot)) return NF4_EINVAL;
  if (fwd_bytes) *fwd_bytes = qn::grouped_fwd_workspace_bytes(M, K, g, N, r);
  if (bwd_bytes) *bwd_bytes = qn::grouped_bwd_workspace_bytes(M, K, g, N, r);
  return NF4_OK;
}

int qlora_grouped_fwd_dt(int compute_dtype, int64_t M, int64_t K, int g, const int64_t* N, int64_t r,
                         const uint16_t* X, const nf4_state_t* W, const uint16_t* A, const uint16_t* B, float c,
                         uint16_t* Y, uint16_t* Z, void* workspace, int64_t workspace_bytes, void* stream) {
  int64_t Ntot;
  qn::NF4View views[qn::kMaxGroupMembers];
  if (!dtype_ok(compute_dtype)) return NF4_EINVAL;
  if (!grouped_shape_ok(M, K, g, N, r, &Ntot) || !grouped_states_ok(W, g, K, N, views)) return NF4_EINVAL;
  if (!X || !A || !B || !Y || !Z || !workspace) return NF4_EINVAL;
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y) || !aligned16(Z) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return NF4_EINVAL;
  if (workspace_bytes < qn::grouped_fwd_workspace_bytes(M, K, g, N, r)) return NF4_EINVAL;
  hipError_t e = qn::launch_grouped_fwd(M, K, g, N, r, X, views, A, B, c, Y, Z, workspace,
                                        static_cast<hipStream_t>(stream), compute_dtype);
  return e == hipSuccess ? NF4_OK : NF4_EHIP;
}

int qlora_grouped_fwd(int64_t M, int64_t K, int g, const int64_t* N, int64_t r, const uint16_t* X,
                      const nf4_state_t* W, const uint16_t* A, const uint16_t* B, float c, uint16_t* Y, uint16_t* Z,
                      void* workspace, int64_t workspace_bytes, void* stream) {
  return qlora_grouped_fwd_dt(NF4_COMPUTE_BF16, M, K, g, N, r, X, W, A, B, c, Y, Z, workspace, workspace_bytes,
                              stream);
}

int qlora_grouped_bwd_dt(int compute_dtype, int64_t M, int64_t K, int g, const int64_t* N, int64_t r,
                         const uint16_t* G, const uint16_t* X, const uint16_t* Z, const nf4_state_t* W,
                         const uint16_t* A, const uint16_t* B, float c, uint16_t* dX, float* dA, float* dB,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  int64_t Ntot;
  qn::NF4View views[qn::kMaxGroupMembers];
  if (!dtype_ok(compute_dtype)) return NF4_EINVAL;
  if (!grouped_shape_ok(M, K, g, N, r, &Ntot) || !grouped_states_ok(W, g, K, N, views)) return NF4_EINVAL;
  if (!G || !X || !Z || !A || !B || !dA || !dB || !workspace) return NF4_EINVAL;
  if (!aligned16(G) || !aligned16(X) || !aligned16(Z) || !aligned16(A) || !aligned16(B) || !aligned16(dA) ||
      !aligned16(dB) || (dX && !aligned16(dX)) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return NF4_EINVAL;
  if (workspace_bytes < qn::grouped_bwd_workspace_bytes(M, K, g, N, r)) return NF4_EINVAL;
  hipError_t e = qn::launch_grouped_bwd(M, K, g, N, r, G, X, Z, views, A, B, c, dX, dA, dB, workspace,
                                        static_cast<hipStream_t>(stream), compute_dtype);
  return e == hipSuccess ? NF4_OK : NF4_EHIP;
}

int qlora_grouped_bwd(int64_t M, int64_t K, int g, const int64_t* N, int64_t r, const uint16_t* G, const uint16_t* X,
                      const uint16_t* Z, const nf4_state_t* W, const uint16_t* A, const uint16_t* B, float c,
                      uint16_t* dX, float* dA, float* dB, void* workspace, int64_t workspace_bytes, void* stream) {
  return qlora_grouped_bwd_dt(NF4_COMPUTE_BF16, M, K, g, N, r, G, X, Z, W, A, B, c, dX, dA, dB, workspace,
                              workspace_bytes, stream);
}

int qlora_merge(int64_t K, int64_t N, int64_t r, const nf4_state_t* W, const void* A, const void* B, int ab_dtype,
                float c, float* W_merged, void* stream) {
  if (K < 1 || N < 1 || r < 1 || r > 65536 || !state_ok(W) || W->numel != K * N) return NF4_EINVAL;
  if (K * N >= kMaxOperandElems || K * r >= kMaxOperandElems || r * N >= kMaxOperandElems) return NF4_EINVAL;
  if (ab_dtype != NF4_AB_BF16 && ab_dtype != NF4_AB_F32 && ab_dtype != NF4_AB_F16) return NF4_EINVAL;
  if (A == nullptr || B == nullptr || W_merged == nullptr || !aligned16(W_merged)) return NF4_EINVAL;
  const uintptr_t elem_mask = ab_dtype == NF4_AB_F32 ? 3u : 1u;
  if ((reinterpret_cast<uintptr_t>(A) & elem_mask) != 0 || (reinterpret_cast<uintptr_t>(B) & elem_mask) != 0)
    return NF4_EINVAL;
  const qn::NF4View v = view_of(W);
  hipError_t e = qn::launch_merge(K, N, r, v, A, B, ab_dtype, c, W_merged,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4_OK : NF4_EHIP;
}

int qlora_sgd_step(int64_t K, int64_t N, int64_t r, uint16_t* A, uint16_t* B, const float* dA, const float* dB,
                   float lr, float* A_master, float* B_master, void* stream) {
  return qlora_sgd_step_dt(NF4_COMPUTE_BF16, K, N, r, A, B, dA, dB, lr, A_master, B_master, stream);
}

int qlora_sgd_step_dt(int param_dtype, int64_t K, int64_t N, int64_t r, uint16_t* A, uint16_t* B, const float* dA,
                      const float* dB, float lr, float* A_master, float* B_master, void* stream) {
  if (!dtype_ok(param_dtype)) return NF4_EINVAL;
  if (K < 1 || N < 1 || r < 1 || K * r >= kMaxOperandElems || r * N >= kMaxOperandElems) return NF4_EINVAL;
  if (A == nullptr || B == nullptr || dA == nullptr || dB == nullptr) return NF4_EINVAL;
  if ((A_master == nullptr) != (B_master == nullptr)) return NF4_EINVAL;
  if ((reinterpret_cast<uintptr_t>(A) & 1u) || (reinterpret_cast<uintptr_t>(B) & 1u) ||
      (reinterpret_cast<uintptr_t>(dA) & 3u) || (reinterpret_cast<uintptr_t>(dB) & 3u) ||
      (reinterpret_cast<uintptr_t>(A_master) & 3u) || (reinterpret_cast<uintptr_t>(B_master) & 3u))
    return NF4_EINVAL;
  hipError_t e =
      qn::launch_sgd(K, N, r, A, B, dA, dB, lr, A_master, B_master, static_cast<hipStream_t>(stream), param_dtype);
  return e == hipSuccess ? NF4_OK : NF4_EHIP;
}

int nf4_status_read(const int32_t* status, int32_t* host_value, void* stream) {
  if (status == nullptr || host_value == nullptr) return NF4_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return NF4_EHIP;
  if (hipMemcpy(host_value, status, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return NF4_EHIP;
  return NF4_OK;
}

int qlora_timer_enable(int kernel_id, int enable) {
  if (kernel_id < 0 || kernel_id >= QK_NUM_KERNELS) return NF4_EINVAL;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  TimerSlot& s = g_timers[kernel_id];
  if (enable != 0) {
    // the slot's events are created here, once; they stay with the slot
    // (the library's only held state, and only once a timer was enabled)
    const size_t have = s.pool.size() + 2 * s.pending.size();
    for (size_t i = have; i < kTimerEvents; ++i) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return NF4_EHIP;
      s.pool.push_back(e);
    }
  }
  s.enabled = enable != 0;
  return NF4_OK;
}

int qlora_timer_read(int kernel_id, double* total_ms, int64_t* launches) {
  if (kernel_id < 0 || kernel_id >= QK_NUM_KERNELS || total_ms == nullptr || launches == nullptr)
    return NF4_EINVAL;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  TimerSlot& s = g_timers[kernel_id];
  double total = 0.0;
  int64_t n = 0;
  int rc = NF4_OK;
  for (auto& pr : s.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(pr.second) != hipSuccess || hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess)
      rc = NF4_EHIP;
    total += ms;
    ++n;
    s.pool.push_back(pr.first);
    s.pool.push_back(pr.second);
  }
  s.pending.clear();
  *total_ms = total;
  *launches = n;
  return rc;
}

const char* nf4_error_string(int code) {
  switch (code) {
    case NF4_OK: return "ok";
    case NF4_EINVAL: return "invalid argument";
    case NF4_ENONFINITE: return "non-finite weight or reconstruction";
    case NF4_EPADDING: return "pad nibble of an odd-length payload is not code 7";
    case NF4_EHIP: return "HIP runtime error";
    default: return "several status bits set";
  }
}

}  // extern "C"
