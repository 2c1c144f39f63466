// Host-side declarations shared by the kernel translation units and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "side_jobs.hpp"

namespace qn {

// Optional per-kernel event timer (see qlora_timer_enable).  Construct right
// before a launch, call stop() right after it; a no-op unless enabled.
// Per-kernel timing for qlora_timer_*: when kernel_id's timer is enabled,
// an event pair brackets the launches between construction and stop().  With
// packet = true the pair is instead handed to one launch through start() /
// end() (hipExtLaunchKernelGGL records it in the dispatch packet itself, so
// it measures that kernel alone); stop() then does nothing.
class Timer {
 public:
  Timer(int kernel_id, hipStream_t stream, bool packet = false);
  void stop();
  hipEvent_t start() const { return static_cast<hipEvent_t>(start_event_); }
  hipEvent_t end() const { return static_cast<hipEvent_t>(packet_stop_); }

 private:
  int id_;
  hipStream_t stream_;
  void* stop_event_;
  void* start_event_;
  void* packet_stop_;
};

// The layer's 16-bit compute type: 0 = bf16, 1 = fp16 (the kDtype of the
// Bf16 / F16 tags); activations, adapters, outputs and the dequantized weight use it.
constexpr int kDtypeBf16 = 0;
constexpr int kDtypeF16 = 1;

// Most member linears in one grouped call (e.g. q, k, v or gate, up).
constexpr int kMaxGroupMembers = 8;

// The read-only view of a stored weight the kernels decode.  With absmax
// non-null the state has no second level: â = absmax[block] (fp32); else
// â = fl32(fl32(fl32(q / 127) * absmax2[block / 256]) + offset).
struct NF4View {
  const uint8_t* codes;
  const int8_t* qabsmax;
  const float* absmax2;
  const float* offset;
  const float* absmax;
};

// absmax_out non-null: single-level encoding (the fp32 first-level scales are
// the stored state; qabsmax, absmax2 and offset are not written).
hipError_t launch_quantize(const float* W, int64_t P, uint8_t* codes, int8_t* qabsmax,
                           float* absmax2, float* offset, float* absmax_out, float* ws_absmax, double* ws_gsum,
                           int32_t* ws_flags, int32_t* status, hipStream_t stream);

// ncols != 0: W is K x ncols and goes to columns 0 .. ncols-1 of an output
// with row stride out_ld (ncols a multiple of 8).
hipError_t launch_dequantize(NF4View W, int64_t P, void* out, int out_dtype, int32_t* status, hipStream_t stream,
                             int64_t ncols = 0, int64_t out_ld = 0);

// W' = fl32(ŵ + c A B) (fp64 accumulation; A, B of element type ab_dtype,
// one of NF4_AB_BF16 / NF4_AB_F32 / NF4_AB_F16).
hipError_t launch_merge(int64_t K, int64_t N, int64_t r, NF4View W, const void* A, const void* B, int ab_dtype,
                        float c, float* out, hipStream_t stream);
// One SGD step on A (K x r) and B (r x N) of the 16-bit type dtype,
// optionally through fp32 masters.
hipError_t launch_sgd(int64_t K, int64_t N, int64_t r, uint16_t* A, uint16_t* B, const float* dA, const float* dB,
                      float lr, float* A_master, float* B_master, hipStream_t stream, int dtype = 0);

// Grouped linears sharing X (see layer.hip).
int64_t grouped_fwd_workspace_bytes(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r);
int64_t grouped_bwd_workspace_bytes(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r);
hipError_t launch_grouped_fwd(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r, const uint16_t* X,
                              const NF4View* W, const uint16_t* A, const uint16_t* B, float c, uint16_t* Y,
                              uint16_t* Z, void* ws, hipStream_t stream, int dtype = kDtypeBf16);
hipError_t launch_grouped_bwd(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r, const uint16_t* G,
                              const uint16_t* X, const uint16_t* Z, const NF4View* W, const uint16_t* A,
                              const uint16_t* B, float c, uint16_t* dX, float* dA, float* dB, void* ws,
                              hipStream_t stream, int dtype = kDtypeBf16);

// Workspace needs (bytes) of the layer kernels; the C ABI adds them up.
int64_t fwd_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t r);
int64_t bwd_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t r);

// Split plans of the rank-r products and of the small-M GEMV (sizes in bytes).
struct SkinnyPlan {
  int64_t z_splits, z_per, dz_splits, dz_per, da_splits, da_per, db_splits, db_per;
  int64_t at_bytes, z_part, dz_part, da_part, db_part;
  int64_t gv_rows_per_wave, gv_splits, gv_part, gv_zpart;
};
void plan_gemv(int64_t M, int64_t K, int64_t N, int64_t r, SkinnyPlan* p);
SkinnyPlan plan_skinny(int64_t M, int64_t K, int64_t N, int64_t r);

// The transposes Z = X A needs (Aᵀ into At) and, with cbt != nullptr, the
// forward's LoRA extension operand cbt = RNE_16(c B)ᵀ (N x r).
void lora_transposes(int64_t K, int64_t r, const uint16_t* A, uint16_t* At, int64_t N, const uint16_t* B, float c,
                     uint16_t* cbt, int64_t rb, int dtype, TJob out[2]);
// Z = X A: the transposes above (one launch, unless pre_transposed: another
// launch already ran them), then the split partials and their sum.
hipError_t launch_lora_down(int64_t M, int64_t K, int64_t r, const uint16_t* X, const uint16_t* A, uint16_t* Z,
                            const SkinnyPlan& p, void* at_ws, void* part_ws, hipStream_t stream, int64_t N = 0,
                            const uint16_t* B = nullptr, float c = 1.0f, uint16_t* cbt = nullptr, int64_t rb = 0,
                            int dtype = 0, bool pre_transposed = false);

// Split plans of a group of g linears sharing X (column counts Ns[i], rank r
// each); zp covers Z = X A over all g r columns.
struct GroupPlan {
  SkinnyPlan zp;
  int64_t dz_splits[kMaxGroupMembers], dz_per[kMaxGroupMembers], dz_part, dz_off[kMaxGroupMembers];
  int64_t cs_splits, cs_per, da_part, db_part_total, db_off[kMaxGroupMembers];
};
GroupPlan plan_grouped(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r);
hipError_t launch_dz_grouped(int64_t M, int g, const int64_t* Ns, int64_t Ntot, int64_t r, const uint16_t* G,
                             const uint16_t* B, float c, uint16_t* dZ, const GroupPlan& gp, void* part_ws,
                             hipStream_t stream, int dtype = 0, RdJob* defer = nullptr);
hipError_t launch_colsums_grouped(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t Ntot, int64_t r,
                                  const uint16_t* X, const uint16_t* G, const uint16_t* Z, const uint16_t* dZ, float c,
                                  float* dA, float* dB, const GroupPlan& gp, void* da_ws, void* db_ws,
                                  hipStream_t stream, int dtype = 0);
// Small-M forward (M <= 16) in two launches: the split-K partials of X Ŵ and
// of Z = X A (extra workgroups of the same launch), then their fixed-order
// sums, Z (written out) and Y = X Ŵ + c Z B.  part_ws: gv_part + gv_zpart.
hipError_t launch_gemv(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W, const uint16_t* A,
                       const uint16_t* B, float c, uint16_t* Y, uint16_t* Z, const SkinnyPlan& p, void* part_ws,
                       hipStream_t stream, int dtype = 0);
// dZ = c G Bᵀ: split partials, then their sum (with defer != nullptr that sum
// is not launched but returned, for the caller to run in a later launch).
hipError_t launch_dz(int64_t M, int64_t N, int64_t r, const uint16_t* G, const uint16_t* B, float c, uint16_t* dZ,
                     const SkinnyPlan& p, void* part_ws, hipStream_t stream, int dtype = 0, RdJob* defer = nullptr);
hipError_t launch_colsums(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, const uint16_t* G,
                          const uint16_t* Z, const uint16_t* dZ, float c, float* dA, float* dB, const SkinnyPlan& p,
                          void* da_ws, void* db_ws, hipStream_t stream, int dtype = 0);

hipError_t launch_fwd(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W,
                      const uint16_t* A, const uint16_t* B, float c, uint16_t* Y, uint16_t* Z,
                      void* ws, hipStream_t stream, int dtype = 0);

hipError_t launch_bwd(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G,
                      const uint16_t* X, const uint16_t* Z, NF4View W, const uint16_t* A,
                      const uint16_t* B, float c, uint16_t* dX, float* dA, float* dB, void* ws,
                      hipStream_t stream, int dtype = 0);

// Split-K plan of the 256 x 256-tile GEMMs for an M x cols output reduced
// over red: splits (1: none), elements per split, fp32 partial bytes.
struct SplitPlan {
  int64_t splits, k_per, part_bytes;
};
SplitPlan plan_split(int64_t M, int64_t cols, int64_t red);

// The GEMMs below split their reduction per plan_split when split_ws (at
// least part_bytes, 16-byte aligned) is given, then sum the partials in
// split order into the 16-bit output (a second launch).
// cBt: RNE_bf16(c B)ᵀ, N x r
hipError_t launch_fwd_big(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W,
                          const uint16_t* Z, const uint16_t* cBt, uint16_t* Y, hipStream_t stream, int dtype = 0,
                          void* split_ws = nullptr);

hipError_t launch_dx_big(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G, NF4View W,
                         const uint16_t* dZ, const uint16_t* A, uint16_t* dX, hipStream_t stream, int dtype = 0,
                         void* split_ws = nullptr);

hipError_t launch_fwd_dense(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, const uint16_t* WhatT,
                            const uint16_t* Z, const uint16_t* cBt, uint16_t* Y, hipStream_t stream, int dtype = 0,
                            void* split_ws = nullptr);
// Forward over g members' concatenated columns (Ntot in all, member i ending
// at column gend[i], every member a multiple of 256 columns): Zcat is M x g r,
// member i's Z in columns i r .. +r; WhatT and cBt are the members' Ŵᵀ and
// (c B)ᵀ stacked row-wise (Ntot x K and Ntot x r).
hipError_t launch_fwd_dense_grouped(int64_t M, int64_t K, int64_t Ntot, int64_t r, const uint16_t* X,
                                    const uint16_t* WhatT, const uint16_t* Zcat, int g, const int64_t* gend,
                                    const uint16_t* cBt, uint16_t* Y, hipStream_t stream, int dtype = 0,
                                    void* split_ws = nullptr);
hipError_t launch_dx_dense(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G, const uint16_t* What,
                           const uint16_t* dZ, const uint16_t* A, uint16_t* dX, hipStream_t stream, int dtype = 0,
                           void* split_ws = nullptr);

// Dequantize a K x N weight to the 16-bit compute type (dtype), either as
// stored (K x N) or transposed (N x K).
// out_ld: row stride of the untransposed output (0: N).
// Side jobs run as extra workgroups of the same launch: side_t (two
// transposes, transposed output only), side_r (one split sum, untransposed
// output only).
hipError_t launch_dequant_bf16(NF4View W, int64_t K, int64_t N, bool transposed, uint16_t* out, hipStream_t stream,
                               int64_t out_ld = 0, int dtype = 0, const TJob* side_t = nullptr,
                               const RdJob* side_r = nullptr);

}  // namespace qn
