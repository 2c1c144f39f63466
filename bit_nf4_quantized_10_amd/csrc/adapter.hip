// Adapter-side operations around the frozen NF4 base, for gfx950.
//
// Merge (page "QLoRA：冻结的 4-bit 权重怎样参与一次微调", section
// "Merge 后还是不是训练时的函数"): the trained function is Ŵ + c A B; its
// high-precision merge is
//   W'[k][n] = fl32(ŵ[k][n] + c * sum_t A[k][t] B[t][n])
// with the sum accumulated in fp64 over t = 0 .. r-1 in order, then c * sum
// and the addition of ŵ (the fp32 reconstruction fl32(C[j] * â)) in fp64, and
// one rounding to fp32.  Every product of two fp32 (or bf16) values is exact
// in fp64, so an fp64 fused multiply-add of a product and the running sum
// rounds exactly like the separate product and sum.  Re-quantizing W' is a
// separate nf4_quantize call (the section treats it as a new step).
//
// SGD step (section "一次完整反向与有限差分": only the adapter is updated,
// v <- v - lr g): p' = fl32(p - fl32(lr * g)) on the fp32 master copy when
// one is kept, else on the 16-bit parameter read as fp32; the bf16 (or fp16)
// parameter becomes RNE(p').
#include "common.hpp"
#include "kernels.hpp"

namespace qn {

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kMgTile = 64;   // output tile: 64 rows k x 64 columns n
constexpr int kMgStep = 32;   // rank steps staged in LDS at a time

// kAB: NF4_AB_BF16, NF4_AB_F32 or NF4_AB_F16 (the adapter's element type).
template <int kAB>
__device__ __forceinline__ double ab_value(const void* p, int64_t i) {
  if (kAB == NF4_AB_F32) return static_cast<double>(static_cast<const float*>(p)[i]);
  if (kAB == NF4_AB_F16) return static_cast<double>(F16::widen(static_cast<const uint16_t*>(p)[i]));
  return static_cast<double>(bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]));
}

// Workgroup = one 64 x 64 output tile; thread (tk, tn) owns rows
// k0 + tk + 16 i and columns n0 + tn + 16 l (i, l < 4), so that the lanes of
// a wave read 4 distinct A values and 16 consecutive B values per rank step.
template <int kAB>
__global__ __launch_bounds__(256) void qlora_merge_kernel(int64_t K, int64_t N, int64_t r, NF4View W,
                                                          const void* __restrict__ A, const void* __restrict__ B,
                                                          float c, float* __restrict__ out) {
  __shared__ double sA[kMgTile][kMgStep + 1];
  __shared__ double sB[kMgStep][kMgTile];
  const int t = threadIdx.x, tk = t >> 4, tn = t & 15;
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * kMgTile, n0 = static_cast<int64_t>(blockIdx.x) * kMgTile;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int l = 0; l < 4; ++l) acc[i][l] = 0.0;
  for (int64_t t0 = 0; t0 < r; t0 += kMgStep) {
    // stage A[k0.., t0..] and B[t0.., n0..] as fp64 (zeros outside)
#pragma unroll
    for (int j = 0; j < (kMgTile * kMgStep) / 256; ++j) {
      const int idx = t + 256 * j;
      const int kk = idx / kMgStep, tt = idx % kMgStep;
      const int64_t k = k0 + kk, tr = t0 + tt;
      sA[kk][tt] = (k < K && tr < r) ? ab_value<kAB>(A, k * r + tr) : 0.0;
      const int tb = idx / kMgTile, nn = idx % kMgTile;
      const int64_t trb = t0 + tb, n = n0 + nn;
      sB[tb][nn] = (trb < r && n < N) ? ab_value<kAB>(B, trb * N + n) : 0.0;
    }
    __syncthreads();
    const int steps = static_cast<int>(r - t0 < kMgStep ? r - t0 : kMgStep);
    for (int tt = 0; tt < steps; ++tt) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[tk + 16 * i][tt];
#pragma unroll
      for (int l = 0; l < 4; ++l) b[l] = sB[tt][tn + 16 * l];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int l = 0; l < 4; ++l) acc[i][l] = __fma_rn(a[i], b[l], acc[i][l]);
    }
    __syncthreads();
  }
  const bool single = W.absmax != nullptr;   // no second level: â = absmax[block]
  const float off = single ? 0.0f : W.offset[0];
  const double cd = static_cast<double>(c);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t k = k0 + tk + 16 * i;
    if (k >= K) continue;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int64_t n = n0 + tn + 16 * l;
      if (n >= N) continue;
      const int64_t e = k * N + n;
      const uint32_t byte = W.codes[e >> 1];
      const uint32_t code = (e & 1) ? (byte & 15u) : (byte >> 4);
      const float ahat = single ? W.absmax[e >> 6] : absmax_hat(W.qabsmax[e >> 6], W.absmax2[e >> 14], off);
      const float w = __fmul_rn(kNF4[code], ahat);
      out[e] = __double2float_rn(__dadd_rn(static_cast<double>(w), __dmul_rn(cd, acc[i][l])));
    }
  }
}

struct SgdJob {
  uint16_t* param;
  const float* grad;
  float* master;   // may be null
  int64_t count;
  int64_t nblk;
  int f16;         // parameters are fp16 (else bf16)
};

__global__ __launch_bounds__(256) void sgd_kernel(SgdJob j0, SgdJob j1, float lr) {
  const bool second = blockIdx.x >= j0.nblk;
  const SgdJob& J = second ? j1 : j0;
  const int64_t blk = second ? blockIdx.x - j0.nblk : blockIdx.x;
  for (int64_t i = blk * 256 + threadIdx.x; i < J.count; i += J.nblk * 256) {
    const float base =
        J.master != nullptr ? J.master[i] : (J.f16 ? F16::widen(J.param[i]) : Bf16::widen(J.param[i]));
    const float v = __fsub_rn(base, __fmul_rn(lr, J.grad[i]));
    if (J.master != nullptr) J.master[i] = v;
    J.param[i] = static_cast<uint16_t>((J.f16 ? F16::pack2(v, 0.0f) : Bf16::pack2(v, 0.0f)) & 0xffffu);
  }
}

SgdJob sgd_job(uint16_t* param, const float* grad, float* master, int64_t count, int dtype) {
  int64_t blocks = cdiv(count, 256);
  if (blocks > 4096) blocks = 4096;
  return SgdJob{param, grad, master, count, blocks, dtype == kDtypeF16 ? 1 : 0};
}

}  // namespace

hipError_t launch_merge(int64_t K, int64_t N, int64_t r, NF4View W, const void* A, const void* B, int ab_dtype,
                        float c, float* out, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(cdiv(N, kMgTile)), static_cast<unsigned>(cdiv(K, kMgTile)));
  Timer tm(QK_MERGE, stream);
  if (ab_dtype == NF4_AB_F32)
    hipLaunchKernelGGL(qlora_merge_kernel<NF4_AB_F32>, grid, dim3(256), 0, stream, K, N, r, W, A, B, c, out);
  else if (ab_dtype == NF4_AB_F16)
    hipLaunchKernelGGL(qlora_merge_kernel<NF4_AB_F16>, grid, dim3(256), 0, stream, K, N, r, W, A, B, c, out);
  else
    hipLaunchKernelGGL(qlora_merge_kernel<NF4_AB_BF16>, grid, dim3(256), 0, stream, K, N, r, W, A, B, c, out);
  tm.stop();
  return hipGetLastError();
}

hipError_t launch_sgd(int64_t K, int64_t N, int64_t r, uint16_t* A, uint16_t* B, const float* dA, const float* dB,
                      float lr, float* A_master, float* B_master, hipStream_t stream, int dtype) {
  const SgdJob ja = sgd_job(A, dA, A_master, K * r, dtype), jb = sgd_job(B, dB, B_master, r * N, dtype);
  Timer tm(QK_SGD, stream);
  hipLaunchKernelGGL(sgd_kernel, dim3(static_cast<unsigned>(ja.nblk + jb.nblk)), dim3(256), 0, stream, ja, jb, lr);
  tm.stop();
  return hipGetLastError();
}

}  // namespace qn
