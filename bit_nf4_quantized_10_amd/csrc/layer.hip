// Orchestration of the layer entry points: workspace carving and the kernel
// sequence of the forward and backward passes.
//   forward : M <= 16: dequant-GEMV and Z = X A split-K partials (one
//                      launch), then their sums and c Z B;
//             M < 192: Aᵀ and (c B)ᵀ in bf16 (one launch); Z = X A (split
//                      rows/K, fixed-order reduce); fused dequant-GEMM with
//                      the LoRA extension;
//             else   : Ŵᵀ dequantized to bf16 with Aᵀ and (c B)ᵀ in the same
//                      launch; Z = X A; dense GEMM.
//   backward: dZ = c G Bᵀ; dA = Xᵀ dZ; dB = c Zᵀ G; dX = G Ŵᵀ + dZ Aᵀ
//             (M >= 192: Ŵ dequantized to bf16, with dZ's split sum in the
//             same launch, before dA and dB; then a dense GEMM).
// Either GEMM splits its reduction when its output has too few 256 x 256
// tiles to occupy the device (plan_split), with a fixed-order sum after.
#include "common.hpp"
#include "kernels.hpp"

namespace qn {

namespace {
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// From this many tokens on, the weight is dequantized once to bf16 and the
// product runs as a dense bf16 GEMM; below, the fused kernel decodes the
// packed codes inside its k-loop (each weight tile is then decoded by fewer
// row-tiles, so the one-off decode pass does not pay for itself).  Both
// give bit-identical outputs; with split reductions, the measured layer
// step (4096 x 4096, r = 64) crosses over between M = 176 and 192.
#ifndef QN_DENSE_MIN_M
#define QN_DENSE_MIN_M 192
#endif
constexpr int64_t kDenseMinM = QN_DENSE_MIN_M;
bool use_dense(int64_t M) { return M >= kDenseMinM; }
int64_t dense_bytes(int64_t M, int64_t K, int64_t N) { return use_dense(M) ? align256(K * N * 2) : 0; }
}  // namespace

// (c B)ᵀ in bf16 for the GEMM kernels' LoRA extension
int64_t cbt_bytes(int64_t M, int64_t N, int64_t r) { return M > 16 ? align256(N * r * 2) : 0; }

// Workspace layouts: the kernels' scratch, then a Z buffer for calls that do
// not pass Z (the forward computes Z there; the backward recomputes it there
// from X and A, with its own Aᵀ and split partials in front of it).
int64_t fwd_core_bytes(int64_t M, int64_t K, int64_t N, int64_t r) {
  const SkinnyPlan p = plan_skinny(M, K, N, r);
  if (M <= 16) return p.gv_part + p.gv_zpart;
  return p.at_bytes + p.z_part + cbt_bytes(M, N, r) + dense_bytes(M, K, N) + plan_split(M, N, K).part_bytes;
}

int64_t bwd_core_bytes(int64_t M, int64_t K, int64_t N, int64_t r) {
  const SkinnyPlan p = plan_skinny(M, K, N, r);
  return p.dz_part + align256(M * r * 2) + p.da_part + p.db_part + dense_bytes(M, K, N) +
         plan_split(M, K, N).part_bytes;
}

int64_t fwd_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t r) {
  return fwd_core_bytes(M, K, N, r) + align256(M * r * 2);
}

int64_t bwd_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t r) {
  const SkinnyPlan p = plan_skinny(M, K, N, r);
  return bwd_core_bytes(M, K, N, r) + p.at_bytes + p.z_part + align256(M * r * 2);
}

hipError_t launch_fwd(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W, const uint16_t* A,
                      const uint16_t* B, float c, uint16_t* Y, uint16_t* Z, void* ws, hipStream_t stream,
                      int dtype) {
  const SkinnyPlan p = plan_skinny(M, K, N, r);
  char* base = static_cast<char*>(ws);
  char* after_z = base + p.at_bytes + p.z_part;
  if (Z == nullptr) Z = reinterpret_cast<uint16_t*>(base + fwd_core_bytes(M, K, N, r));
  hipError_t e;
  if (M <= 16) return launch_gemv(M, K, N, r, X, W, A, B, c, Y, Z, p, base, stream, dtype);
  uint16_t* cbt = reinterpret_cast<uint16_t*>(after_z);
  uint16_t* wt = reinterpret_cast<uint16_t*>(after_z + cbt_bytes(M, N, r));
  void* split_ws = reinterpret_cast<char*>(wt) + dense_bytes(M, K, N);
  uint16_t* at = reinterpret_cast<uint16_t*>(base);
  if (use_dense(M)) {
    // Aᵀ and (c B)ᵀ ride along in the launch that dequantizes Ŵᵀ
    TJob tj[2];
    lora_transposes(K, r, A, at, N, B, c, cbt, 0, dtype, tj);
    if ((e = launch_dequant_bf16(W, K, N, true, wt, stream, 0, dtype, tj)) != hipSuccess) return e;
    if ((e = launch_lora_down(M, K, r, X, A, Z, p, base, base + p.at_bytes, stream, N, B, c, cbt, 0, dtype, true)) !=
        hipSuccess)
      return e;
    return launch_fwd_dense(M, K, N, r, X, wt, Z, cbt, Y, stream, dtype, split_ws);
  }
  if ((e = launch_lora_down(M, K, r, X, A, Z, p, base, base + p.at_bytes, stream, N, B, c, cbt, 0, dtype)) != hipSuccess)
    return e;
  return launch_fwd_big(M, K, N, r, X, W, Z, cbt, Y, stream, dtype, split_ws);
}

hipError_t launch_bwd(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G, const uint16_t* X,
                      const uint16_t* Z, NF4View W, const uint16_t* A, const uint16_t* B, float c, uint16_t* dX,
                      float* dA, float* dB, void* ws, hipStream_t stream, int dtype) {
  const SkinnyPlan p = plan_skinny(M, K, N, r);
  char* base = static_cast<char*>(ws);
  void* dz_part = base;
  uint16_t* dz16 = reinterpret_cast<uint16_t*>(base + p.dz_part);
  void* da_part = base + p.dz_part + align256(M * r * 2);
  void* db_part = static_cast<char*>(da_part) + p.da_part;
  uint16_t* wd = reinterpret_cast<uint16_t*>(static_cast<char*>(db_part) + p.db_part);
  void* split_ws = reinterpret_cast<char*>(wd) + dense_bytes(M, K, N);
  hipError_t e;
  if (Z == nullptr) {
    // recompute Z = X A (for M > 16 the forward's own kernels, so the same bits)
    char* zr = base + bwd_core_bytes(M, K, N, r);
    uint16_t* zbuf = reinterpret_cast<uint16_t*>(zr + p.at_bytes + p.z_part);
    if ((e = launch_lora_down(M, K, r, X, A, zbuf, p, zr, zr + p.at_bytes, stream, 0, nullptr, 1.0f, nullptr, 0,
                              dtype)) != hipSuccess)
      return e;
    Z = zbuf;
  }
  if (dX != nullptr && use_dense(M)) {
    // the fixed-order sum of dZ rides along in the launch that dequantizes Ŵ
    RdJob jz;
    if ((e = launch_dz(M, N, r, G, B, c, dz16, p, dz_part, stream, dtype, &jz)) != hipSuccess) return e;
    if ((e = launch_dequant_bf16(W, K, N, false, wd, stream, 0, dtype, nullptr, &jz)) != hipSuccess) return e;
    if ((e = launch_colsums(M, K, N, r, X, G, Z, dz16, c, dA, dB, p, da_part, db_part, stream, dtype)) != hipSuccess)
      return e;
    return launch_dx_dense(M, K, N, r, G, wd, dz16, A, dX, stream, dtype, split_ws);
  }
  if ((e = launch_dz(M, N, r, G, B, c, dz16, p, dz_part, stream, dtype)) != hipSuccess) return e;
  if ((e = launch_colsums(M, K, N, r, X, G, Z, dz16, c, dA, dB, p, da_part, db_part, stream, dtype)) != hipSuccess) return e;
  if (dX == nullptr) return hipGetLastError();
  return launch_dx_big(M, K, N, r, G, W, dz16, A, dX, stream, dtype, split_ws);
}

// ------------------------------------------------------------ grouped linears
// g members sharing X with their outputs side by side (Y, G: M x Ntot;
// A, dA: K x g r; B, dB: r x Ntot; Z: M x g r).  Every member is
// dequantized to the compute type (bf16 or fp16) into one stacked weight and the product runs as one
// dense GEMM over all Ntot columns (forward) or over all Ntot reduction
// columns (dX), with one Z = X A over all g r columns.  The transposes ride
// in the first member's dequantize launch, each member's dZ sum in its own
// dequantize launch, and dA with every member's dB is one column-sum launch
// (up to three members).
int64_t grouped_fwd_workspace_bytes(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r) {
  const GroupPlan gp = plan_grouped(M, K, g, Ns, r);
  int64_t Ntot = 0;
  for (int i = 0; i < g; ++i) Ntot += Ns[i];
  return gp.zp.at_bytes + gp.zp.z_part + align256(Ntot * r * 2) + align256(Ntot * K * 2) +
         plan_split(M, Ntot, K).part_bytes;
}

int64_t grouped_bwd_workspace_bytes(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r) {
  const GroupPlan gp = plan_grouped(M, K, g, Ns, r);
  int64_t Ntot = 0;
  for (int i = 0; i < g; ++i) Ntot += Ns[i];
  return gp.dz_part + align256(M * g * r * 2) + gp.da_part + gp.db_part_total + align256(K * Ntot * 2) +
         plan_split(M, K, Ntot).part_bytes;
}

hipError_t launch_grouped_fwd(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r, const uint16_t* X,
                              const NF4View* W, const uint16_t* A, const uint16_t* B, float c, uint16_t* Y,
                              uint16_t* Z, void* ws, hipStream_t stream, int dtype) {
  const GroupPlan gp = plan_grouped(M, K, g, Ns, r);
  int64_t Ntot = 0;
  for (int i = 0; i < g; ++i) Ntot += Ns[i];
  char* base = static_cast<char*>(ws);
  char* zpart = base + gp.zp.at_bytes;
  uint16_t* cbt = reinterpret_cast<uint16_t*>(zpart + gp.zp.z_part);
  uint16_t* wt = reinterpret_cast<uint16_t*>(zpart + gp.zp.z_part + align256(Ntot * r * 2));
  // Aᵀ and (c B)ᵀ of all members ride along in the first member's dequantize launch
  TJob tj[2];
  lora_transposes(K, g * r, A, reinterpret_cast<uint16_t*>(base), Ntot, B, c, cbt, r, dtype, tj);
  hipError_t e;
  int64_t gend[kMaxGroupMembers];
  int64_t off = 0;
  for (int i = 0; i < g; ++i) {
    if ((e = launch_dequant_bf16(W[i], K, Ns[i], true, wt + off * K, stream, 0, dtype, i == 0 ? tj : nullptr)) !=
        hipSuccess)
      return e;
    off += Ns[i];
    gend[i] = off;
  }
  if ((e = launch_lora_down(M, K, g * r, X, A, Z, gp.zp, base, zpart, stream, Ntot, B, c, cbt, r, dtype, true)) !=
      hipSuccess)
    return e;
  return launch_fwd_dense_grouped(M, K, Ntot, r, X, wt, Z, g, gend, cbt, Y, stream, dtype,
                                  reinterpret_cast<char*>(wt) + align256(Ntot * K * 2));
}

hipError_t launch_grouped_bwd(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r, const uint16_t* G,
                              const uint16_t* X, const uint16_t* Z, const NF4View* W, const uint16_t* A,
                              const uint16_t* B, float c, uint16_t* dX, float* dA, float* dB, void* ws,
                              hipStream_t stream, int dtype) {
  const GroupPlan gp = plan_grouped(M, K, g, Ns, r);
  int64_t Ntot = 0;
  for (int i = 0; i < g; ++i) Ntot += Ns[i];
  char* base = static_cast<char*>(ws);
  uint16_t* dz16 = reinterpret_cast<uint16_t*>(base + gp.dz_part);
  char* da_ws = base + gp.dz_part + align256(M * g * r * 2);
  char* db_ws = da_ws + gp.da_part;
  uint16_t* wd = reinterpret_cast<uint16_t*>(db_ws + gp.db_part_total);
  // with dX wanted, member i's dZ sum rides along in member i's dequantize launch
  RdJob jz[kMaxGroupMembers];
  hipError_t e = launch_dz_grouped(M, g, Ns, Ntot, r, G, B, c, dz16, gp, base, stream, dtype,
                                   dX != nullptr ? jz : nullptr);
  if (e != hipSuccess) return e;
  if (dX != nullptr) {
    int64_t off = 0;
    for (int i = 0; i < g; ++i) {
      if ((e = launch_dequant_bf16(W[i], K, Ns[i], false, wd + off, stream, Ntot, dtype, nullptr, &jz[i])) !=
          hipSuccess)
        return e;
      off += Ns[i];
    }
  }
  if ((e = launch_colsums_grouped(M, K, g, Ns, Ntot, r, X, G, Z, dz16, c, dA, dB, gp, da_ws, db_ws, stream, dtype)) !=
      hipSuccess)
    return e;
  if (dX == nullptr) return hipGetLastError();
  return launch_dx_dense(M, K, Ntot, g * r, G, wd, dz16, A, dX, stream, dtype,
                         reinterpret_cast<char*>(wd) + align256(K * Ntot * 2));
}

}  // namespace qn
