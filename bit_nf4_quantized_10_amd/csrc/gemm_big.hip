// Large-M fused dequant-GEMM kernels for gfx950: the forward Y = X Ŵ + c Z B
// and the backward dX = G Ŵᵀ + dZ Aᵀ (page "QLoRA：冻结的 4-bit 权重怎样参与一次微调",
// sections "量化基座与可训练支路怎样相加" and "冻结权重为什么仍然需要输入梯度").
//
// Workgroup: 256 threads (4 waves, 2 x 2), output tile 256 x 256, each wave
// 128 x 128 as 8 x 8 tiles of v_mfma_f32_16x16x32_bf16 (256 fp32 accumulators
// per lane, one wave per SIMD).  The reduction advances 64 elements per LDS
// stage with two stages in flight: while the MFMAs consume stage s, the
// global loads of stage s+1 are outstanding; the loaded codes are then decoded
// to bf16 and written to the other LDS buffer.
//
// LDS layout of one operand stage: 256 rows x 64 bf16 (128 bytes per row), the
// eight 16-byte chunks of row r stored at chunk ^ ((r ^ r >> 3) & 7).  The
// swizzle keeps both the 16-byte fragment reads (16 consecutive rows, one
// chunk) and the decoder's writes (rows 8 apart, one chunk) free of bank
// conflicts within each group of 8 lanes.
//
// Weight operand:
//  - forward (reduction over k, codes packed along n): each thread loads one
//    32-bit code word (8 consecutive n) from each of 8 consecutive k-rows,
//    transposes the 8 x 8 nibble matrix in registers (three byte/nibble
//    butterfly stages), and decodes each column's 8 k-values with their 8
//    row scales into one 16-byte LDS chunk;
//  - backward dX (reduction over n, the packed direction): each thread owns
//    one k-row and decodes its 64 consecutive n (exactly one 64-weight block,
//    one scale) into 8 LDS chunks.
// Decoding is ŵ = RNE_bf16(fl32(C[code] * â)), bit-identical to nf4_dequantize.
//
// The MFMA is issued as D = Ŵ-fragment x activation-fragment, so each lane
// holds 4 consecutive output columns of one output row: 8-byte bf16 stores.
#include "common.hpp"
#include "kernels.hpp"

namespace qn {

namespace {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kTileBytes = 256 * 128;
constexpr int kLutOffset = 4 * kTileBytes;
constexpr int kQ2Offset = kLutOffset + 16 * 4;
constexpr int kLdsBytes = kQ2Offset + 256 * 4;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 8 x 8 nibble transpose: afterwards r[j] holds, at bits 4i..4i+3, what r[i]
// held at bits 4j..4j+3.
__device__ __forceinline__ void transpose8x8_nibbles(uint32_t (&r)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // swap the off-diagonal 4 x 4 blocks (16-bit halves)
    const uint32_t a = r[i], b = r[i + 4];
    r[i] = perm(b, a, 0x05040100u);
    r[i + 4] = perm(b, a, 0x07060302u);
  }
#pragma unroll
  for (int h = 0; h < 8; h += 4)   // swap the off-diagonal 2 x 2 blocks (bytes)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t a = r[h + i], b = r[h + i + 2];
      r[h + i] = perm(b, a, 0x06020400u);
      r[h + i + 2] = perm(b, a, 0x07030501u);
    }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {  // swap single nibbles
    const uint32_t a = r[i], b = r[i + 1];
    r[i] = (a & 0x0F0F0F0Fu) | ((b & 0x0F0F0F0Fu) << 4);
    r[i + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
}

__device__ __forceinline__ float lut_mul(const float* lut, uint32_t d, int shift, float s) {
  return __fmul_rn(lut[(d >> shift) & 15u], s);
}

struct BigArgs {
  const uint16_t* act;     // X (forward) or G (backward): rows m, reduction contiguous
  int64_t act_ld;          // K (forward) or N (backward)
  NF4View W;
  const uint16_t* ext_a;   // Z (forward) or dZ (backward), M x r bf16
  const uint16_t* ext_b;   // B (forward, r x N) or A (backward, K x r)
  float c;                 // forward: LoRA scale
  uint16_t* out;           // Y (M x N) or dX (M x K)
  int64_t M, K, N, r;
};

struct StageRegs {
  uint4 x[8];
  uint32_t w[8];
  int q[8];
  float s2[8];
};

// Activation operand of one stage: 256 rows x 64 reduction elements, row-major
// source.  Thread t loads chunk t&7 of rows t/8 + 32i.
__device__ __forceinline__ void load_act(StageRegs& R, const uint16_t* __restrict__ src, int64_t ld, int64_t rows,
                                         int64_t red, int64_t m0, int64_t k0, int t) {
  const int c = t & 7;
  const int64_t k = k0 + 8 * c;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + (t >> 3) + 32 * i;
    R.x[i] = (m < rows && k < red) ? *reinterpret_cast<const uint4*>(src + m * ld + k) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_act(const StageRegs& R, char* sA, int t) {
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(sA + lds_off((t >> 3) + 32 * i, c)) = R.x[i];
}

// Forward weight stage: rows k0 + 8*rg + i, columns n0 + 8*cg .. +7.
__device__ __forceinline__ void load_w_fwd(StageRegs& R, const BigArgs& a, int64_t n0, int64_t k0, int t) {
  const int rg = t >> 5, cg = t & 31;
  const int64_t n = n0 + 8 * cg;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t k = k0 + 8 * rg + i;
    if (k < a.K && n < a.N) {
      const int64_t e = k * a.N + n;
      R.w[i] = *reinterpret_cast<const uint32_t*>(a.W.codes + (e >> 1));
      R.q[i] = a.W.qabsmax[e >> 6];
      R.s2[i] = a.W.absmax2[e >> 14];
    } else {
      R.w[i] = 0x77777777u;  // code 7 decodes to 0
      R.q[i] = 0;
      R.s2[i] = 0.0f;
    }
  }
}

__device__ __forceinline__ void store_w_fwd(StageRegs& R, char* sB, const float* lut, const float* q2t, float off,
                                            int t) {
  const int rg = t >> 5, cg = t & 31;
  float sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sc[i] = __fadd_rn(__fmul_rn(q2t[R.q[i] + 128], R.s2[i]), off);
  uint32_t r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = R.w[i];
  transpose8x8_nibbles(r);
  // input nibble position p holds column p^1 (first code of a byte in the
  // high nibble), so column tc now sits in r[tc ^ 1], nibble i = row i.
#pragma unroll
  for (int tc = 0; tc < 8; ++tc) {
    const uint32_t d = r[tc ^ 1];
    uint4 o;
    o.x = pack_bf16x2(lut_mul(lut, d, 0, sc[0]), lut_mul(lut, d, 4, sc[1]));
    o.y = pack_bf16x2(lut_mul(lut, d, 8, sc[2]), lut_mul(lut, d, 12, sc[3]));
    o.z = pack_bf16x2(lut_mul(lut, d, 16, sc[4]), lut_mul(lut, d, 20, sc[5]));
    o.w = pack_bf16x2(lut_mul(lut, d, 24, sc[6]), lut_mul(lut, d, 28, sc[7]));
    *reinterpret_cast<uint4*>(sB + lds_off(8 * cg + tc, rg)) = o;
  }
}

// Backward weight stage (Ŵᵀ): row k = kc0 + t, reduction n0 .. n0+63 (one block).
__device__ __forceinline__ void load_w_bwd(StageRegs& R, const BigArgs& a, int64_t kc0, int64_t n0, int t) {
  const int64_t k = kc0 + t;
  if (k < a.K) {
    const int64_t e = k * a.N + n0;
    const uint4 lo = *reinterpret_cast<const uint4*>(a.W.codes + (e >> 1));
    const uint4 hi = *reinterpret_cast<const uint4*>(a.W.codes + (e >> 1) + 16);
    R.w[0] = lo.x; R.w[1] = lo.y; R.w[2] = lo.z; R.w[3] = lo.w;
    R.w[4] = hi.x; R.w[5] = hi.y; R.w[6] = hi.z; R.w[7] = hi.w;
    R.q[0] = a.W.qabsmax[e >> 6];
    R.s2[0] = a.W.absmax2[e >> 14];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) R.w[i] = 0x77777777u;
    R.q[0] = 0;
    R.s2[0] = 0.0f;
  }
}

__device__ __forceinline__ void store_w_bwd(const StageRegs& R, char* sB, const float* lut, const float* q2t,
                                            float off, int t) {
  const float s = __fadd_rn(__fmul_rn(q2t[R.q[0] + 128], R.s2[0]), off);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t d = R.w[c];
    uint4 o;  // byte b: high nibble = element 2b, low nibble = element 2b+1
    o.x = pack_bf16x2(lut_mul(lut, d, 4, s), lut_mul(lut, d, 0, s));
    o.y = pack_bf16x2(lut_mul(lut, d, 12, s), lut_mul(lut, d, 8, s));
    o.z = pack_bf16x2(lut_mul(lut, d, 20, s), lut_mul(lut, d, 16, s));
    o.w = pack_bf16x2(lut_mul(lut, d, 28, s), lut_mul(lut, d, 24, s));
    *reinterpret_cast<uint4*>(sB + lds_off(t, c)) = o;
  }
}

__device__ __forceinline__ void compute_stage(const char* sA, const char* sB, f32x4 (&acc)[8][8], int wm, int wn,
                                              int lane) {
  const int q = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 af[8], bw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(sA + lds_off(wm * 128 + 16 * i + q, ks * 4 + g));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      bw[j] = *reinterpret_cast<const bf16x8*>(sB + lds_off(wn * 128 + 16 * j + q, ks * 4 + g));
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mfma16x16x32(bw[j], af[i], acc[i][j]);
  }
}

// Lane (q, g) holds, for tile (i, j), output row 16i+q and columns 16j+4g..+3.
__device__ __forceinline__ void store_out(const f32x4 (&acc)[8][8], uint16_t* out, int64_t ld, int64_t rows,
                                          int64_t cols, int64_t m0, int64_t c0, int wm, int wn, int lane) {
  const int q = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + wm * 128 + 16 * i + q;
    if (m >= rows) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = c0 + wn * 128 + 16 * j + 4 * g;
      if (n < cols) {
        uint2 v;
        v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<uint2*>(out + m * ld + n) = v;
      }
    }
  }
}

__device__ __forceinline__ void stage_tables(char* smem) {
  float* lut = reinterpret_cast<float*>(smem + kLutOffset);
  float* q2t = reinterpret_cast<float*>(smem + kQ2Offset);
  const int t = threadIdx.x;
  q2t[t] = q2_value(t - 128);
  if (t < 16) lut[t] = kNF4[t];
}

template <bool kForward>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void qlora_big_kernel(BigArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // stage buffer b: activation tile at 2b*T, weight tile at (2b+1)*T
  auto sA = [&](int b) { return smem + (2 * b) * kTileBytes; };
  auto sB = [&](int b) { return smem + (2 * b + 1) * kTileBytes; };
  const float* lut = reinterpret_cast<const float*>(smem + kLutOffset);
  const float* q2t = reinterpret_cast<const float*>(smem + kQ2Offset);
  stage_tables(smem);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kBN;   // n0 (forward) or k0 (backward)
  const int64_t red = kForward ? a.K : a.N;
  const int64_t nst = (red + kBK - 1) / kBK;
  const float off = a.W.offset[0];

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  StageRegs R;
  load_act(R, a.act, a.act_ld, a.M, red, m0, 0, t);
  if (kForward)
    load_w_fwd(R, a, c0, 0, t);
  else
    load_w_bwd(R, a, c0, 0, t);
  __syncthreads();  // tables staged
  store_act(R, sA(0), t);
  if (kForward)
    store_w_fwd(R, sB(0), lut, q2t, off, t);
  else
    store_w_bwd(R, sB(0), lut, q2t, off, t);
  __syncthreads();

  for (int64_t s = 0; s < nst; ++s) {
    const int cur = static_cast<int>(s & 1);
    const bool more = s + 1 < nst;
    if (more) {
      const int64_t k0 = (s + 1) * kBK;
      load_act(R, a.act, a.act_ld, a.M, red, m0, k0, t);
      if (kForward)
        load_w_fwd(R, a, c0, k0, t);
      else
        load_w_bwd(R, a, c0, k0, t);
    }
    compute_stage(sA(cur), sB(cur), acc, wm, wn, lane);
    if (more) {
      store_act(R, sA(cur ^ 1), t);
      if (kForward)
        store_w_fwd(R, sB(cur ^ 1), lut, q2t, off, t);
      else
        store_w_bwd(R, sB(cur ^ 1), lut, q2t, off, t);
    }
    __syncthreads();
  }

  // LoRA extension: r more reduction steps with (Z, c·B) or (dZ, A).
  for (int64_t j0 = 0; j0 < a.r; j0 += kBK) {
    load_act(R, a.ext_a, a.r, a.M, a.r, m0, j0, t);
    store_act(R, sA(0), t);
    if (kForward) {
      // B tile row n = c0 + t, chunk jc holds c*B[j0 + 8jc + e][n]
      const int64_t n = c0 + t;
#pragma unroll
      for (int jc = 0; jc < 8; ++jc) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t j = j0 + 8 * jc + e;
          v[e] = (j < a.r && n < a.N) ? a.c * bf16_bits_to_f32(a.ext_b[j * a.N + n]) : 0.0f;
        }
        uint4 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        o.z = pack_bf16x2(v[4], v[5]);
        o.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(sB(0) + lds_off(t, jc)) = o;
      }
    } else {
      // A-matrix row k = c0 + t, reduction j contiguous
      const int64_t k = c0 + t;
#pragma unroll
      for (int jc = 0; jc < 8; ++jc) {
        const int64_t j = j0 + 8 * jc;
        const uint4 v = (k < a.K && j < a.r) ? *reinterpret_cast<const uint4*>(a.ext_b + k * a.r + j)
                                             : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(sB(0) + lds_off(t, jc)) = v;
      }
    }
    __syncthreads();
    compute_stage(sA(0), sB(0), acc, wm, wn, lane);
    __syncthreads();
  }

  store_out(acc, a.out, kForward ? a.N : a.K, a.M, kForward ? a.N : a.K, m0, c0, wm, wn, lane);
}

template <bool kForward>
hipError_t launch_big(const BigArgs& a, hipStream_t stream) {
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qlora_big_kernel<kForward>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int64_t cols = kForward ? a.N : a.K;
  dim3 grid(static_cast<unsigned>((cols + kBN - 1) / kBN), static_cast<unsigned>((a.M + kBM - 1) / kBM), 1);
  hipLaunchKernelGGL((qlora_big_kernel<kForward>), grid, dim3(kThreads), kLdsBytes, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_big(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W,
                          const uint16_t* Z, const uint16_t* B, float c, uint16_t* Y, hipStream_t stream) {
  BigArgs a{X, K, W, Z, B, c, Y, M, K, N, r};
  Timer t(QK_FWD_GEMM, stream);
  hipError_t e = launch_big<true>(a, stream);
  t.stop();
  return e;
}

hipError_t launch_dx_big(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G, NF4View W,
                         const uint16_t* dZ, const uint16_t* A, uint16_t* dX, hipStream_t stream) {
  BigArgs a{G, N, W, dZ, A, 1.0f, dX, M, K, N, r};
  Timer t(QK_BWD_DX, stream);
  hipError_t e = launch_big<false>(a, stream);
  t.stop();
  return e;
}

}  // namespace qn
