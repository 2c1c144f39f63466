// Layer kernels for gfx950: the fused dequant-GEMM forward with the LoRA
// branch as a reduction extension, the transposed-dequant dX kernel, and the
// skinny rank-r products (Z, dZ, dA, dB) with fixed-order split reductions.
//
// Layer (page "QLoRA：冻结的 4-bit 权重怎样参与一次微调", sections
// "量化基座与可训练支路怎样相加" and "冻结权重为什么仍然需要输入梯度"):
//   Z = X A,  Y = X Ŵ + c Z B,  dZ = c G Bᵀ,  dA = Xᵀ dZ,  dB = c Zᵀ G,
//   dX = G Ŵᵀ + dZ Aᵀ.
//
// Every product runs on v_mfma_f32_16x16x32_bf16 from LDS tiles stored as
// [row][32 reduction elements] (+8 pad): lane l of a wave reads row l%16 and
// the 8 reduction elements 8*(l/16)..+7 of both operands; lane l holds rows
// 4*(l/16)..+3 of output column l%16.
#include "common.hpp"
#include "kernels.hpp"

namespace qn {

namespace {

constexpr int BK = 32;
constexpr int PITCH = BK + 8;  // bf16 elements per LDS tile row (80 bytes)

struct Tables {
  float lut[16];   // NF4 values
  float q2[256];   // fl32(q/127) for q = -128..127 at index q+128
};

__device__ __forceinline__ void stage_tables(Tables& t) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    t.q2[i] = q2_value(i - 128);
    if (i < 16) t.lut[i] = kNF4[i];
  }
}

__device__ __forceinline__ float ahat_of(const Tables& t, const NF4View& w, int64_t block, float off) {
  return __fadd_rn(__fmul_rn(t.q2[w.qabsmax[block] + 128], w.absmax2[block / kBlock2]), off);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// Tile [ROWS][BK] from src[row][red] (reduction contiguous, ld elements per
// row).  Requires red_len % 8 == 0 and 16-byte aligned rows.
template <int ROWS, int NT>
__device__ __forceinline__ void load_rowmajor(uint16_t* sT, const uint16_t* __restrict__ src, int64_t ld,
                                              int64_t nrows, int64_t row0, int64_t red_len, int64_t red0) {
  constexpr int CH = ROWS * (BK / 8);
  for (int id = threadIdx.x; id < CH; id += NT) {
    const int row = id >> 2, c = id & 3;
    const int64_t gr = row0 + row, gk = red0 + c * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (gr < nrows && gk < red_len) v = *reinterpret_cast<const uint4*>(src + gr * ld + gk);
    *reinterpret_cast<uint4*>(sT + row * PITCH + c * 8) = v;
  }
}

// Tile [ROWS][BK] from src[red][row] (rows contiguous): a transposing copy,
// optionally scaling each value by `scale` (rounded back to bf16).
// Requires nrows % 8 == 0 and 16-byte aligned rows of src.
template <int ROWS, int NT, bool SCALE>
__device__ __forceinline__ void load_transposed(uint16_t* sT, const uint16_t* __restrict__ src, int64_t ld,
                                                int64_t nrows, int64_t row0, int64_t red_len, int64_t red0,
                                                float scale) {
  constexpr int CPR = ROWS / 8;
  constexpr int CH = BK * CPR;
  for (int id = threadIdx.x; id < CH; id += NT) {
    const int rr = id / CPR, c = id % CPR;
    const int64_t gk = red0 + rr, gr = row0 + c * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (gk < red_len && gr < nrows) v = *reinterpret_cast<const uint4*>(src + gk * ld + gr);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t e = static_cast<uint16_t>(w4[i >> 1] >> (16 * (i & 1)));
      if (SCALE) e = to_bf16(scale * bf16_bits_to_f32(e));
      sT[(c * 8 + i) * PITCH + rr] = e;
    }
  }
}

// Forward weight operand: tile rows are output columns n, reduction is k.
// Decodes 8 consecutive n of one k-row per code word and writes them
// transposed.  Out-of-range weights are zero.
template <int ROWS, int NT>
__device__ __forceinline__ void load_nf4_fwd(uint16_t* sT, const NF4View& w, const Tables& tb, float off,
                                             int64_t K, int64_t N, int64_t n0, int64_t k0) {
  constexpr int WPR = ROWS / 8;
  constexpr int CH = BK * WPR;
  for (int id = threadIdx.x; id < CH; id += NT) {
    const int kk = id / WPR, wc = id % WPR;
    const int64_t gk = k0 + kk, gn = n0 + wc * 8;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (gk < K && gn < N) {
      const int64_t e0 = gk * N + gn;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(w.codes + e0 / 2);
      decode8(word, ahat_of(tb, w, e0 / kBlock1, off), tb.lut, v);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sT[(wc * 8 + i) * PITCH + kk] = to_bf16(v[i]);
  }
}

// Backward weight operand (Ŵᵀ): tile rows are k, reduction is n, which is the
// packed direction, so each code word lands as one 16-byte LDS row chunk.
template <int ROWS, int NT>
__device__ __forceinline__ void load_nf4_bwd(uint16_t* sT, const NF4View& w, const Tables& tb, float off,
                                             int64_t K, int64_t N, int64_t k0, int64_t n0) {
  constexpr int CH = ROWS * (BK / 8);
  for (int id = threadIdx.x; id < CH; id += NT) {
    const int row = id >> 2, c = id & 3;
    const int64_t gk = k0 + row, gn = n0 + c * 8;
    uint4 out = make_uint4(0, 0, 0, 0);
    if (gk < K && gn < N) {
      const int64_t e0 = gk * N + gn;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(w.codes + e0 / 2);
      float v[8];
      decode8(word, ahat_of(tb, w, e0 / kBlock1, off), tb.lut, v);
      out.x = pack_bf16x2(v[0], v[1]);
      out.y = pack_bf16x2(v[2], v[3]);
      out.z = pack_bf16x2(v[4], v[5]);
      out.w = pack_bf16x2(v[6], v[7]);
    }
    *reinterpret_cast<uint4*>(sT + row * PITCH + c * 8) = out;
  }
}

template <int TM, int TN>
__device__ __forceinline__ void mma_tile(const uint16_t* sA, const uint16_t* sB, f32x4 (&acc)[TM][TN],
                                         int arow0, int brow0, int lane) {
  const int q = lane & 15, g = lane >> 4;
  bf16x8 af[TM], bfr[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
    af[i] = *reinterpret_cast<const bf16x8*>(sA + (arow0 + i * 16 + q) * PITCH + g * 8);
#pragma unroll
  for (int j = 0; j < TN; ++j)
    bfr[j] = *reinterpret_cast<const bf16x8*>(sB + (brow0 + j * 16 + q) * PITCH + g * 8);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
}

// Writes the accumulators of one wave: bf16 (out_bf16 != null) or fp32.
template <int TM, int TN>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[TM][TN], int64_t row0, int64_t col0,
                                           int64_t nrows, int64_t ncols, int64_t ld, uint16_t* out_bf16,
                                           float* out_f32, int lane) {
  const int q = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = row0 + i * 16 + g * 4 + e, col = col0 + j * 16 + q;
        if (row < nrows && col < ncols) {
          if (out_bf16)
            out_bf16[row * ld + col] = to_bf16(acc[i][j][e]);
          else
            out_f32[row * ld + col] = acc[i][j][e];
        }
      }
}

struct FwdArgs {
  const uint16_t* X;
  NF4View W;
  const uint16_t* Z;
  const uint16_t* B;
  float c;
  uint16_t* Y;        // bf16 output when part == nullptr
  float* part;        // [splits][M][N] fp32 partials otherwise
  int64_t M, K, N, r;
  int64_t k_per_split;
};

// Y tile = X·Ŵ over the split's k-range, plus (split 0 only) Z·(c B).
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void qlora_fwd_kernel(FwdArgs a) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  __shared__ Tables tb;
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * PITCH];
  stage_tables(tb);
  __syncthreads();
  const float off = a.W.offset[0];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM, n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * a.k_per_split;
  const int64_t kend = min(a.K, kbeg + a.k_per_split);
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    load_rowmajor<BM, NT>(sA, a.X, a.K, a.M, m0, kend, k0);
    load_nf4_fwd<BN, NT>(sB, a.W, tb, off, kend, a.N, n0, k0);
    __syncthreads();
    mma_tile<TM, TN>(sA, sB, acc, wm * TM * 16, wn * TN * 16, lane);
    __syncthreads();
  }
  if (blockIdx.z == 0) {
    for (int64_t j0 = 0; j0 < a.r; j0 += BK) {
      load_rowmajor<BM, NT>(sA, a.Z, a.r, a.M, m0, a.r, j0);
      load_transposed<BN, NT, true>(sB, a.B, a.N, a.N, n0, a.r, j0, a.c);
      __syncthreads();
      mma_tile<TM, TN>(sA, sB, acc, wm * TM * 16, wn * TN * 16, lane);
      __syncthreads();
    }
  }
  const int64_t row0 = m0 + wm * TM * 16, col0 = n0 + wn * TN * 16;
  if (a.part == nullptr)
    store_tile<TM, TN>(acc, row0, col0, a.M, a.N, a.N, a.Y, nullptr, lane);
  else
    store_tile<TM, TN>(acc, row0, col0, a.M, a.N, a.N, nullptr,
                       a.part + static_cast<int64_t>(blockIdx.z) * a.M * a.N, lane);
}

struct DxArgs {
  const uint16_t* G;
  NF4View W;
  const uint16_t* dZ;   // bf16 M x r
  const uint16_t* A;    // bf16 K x r
  uint16_t* dX;
  int64_t M, K, N, r;
};

// dX tile (rows m, cols k) = G·Ŵᵀ over all n, then dZ·Aᵀ over r.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void qlora_dx_kernel(DxArgs a) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  __shared__ Tables tb;
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * PITCH];
  stage_tables(tb);
  __syncthreads();
  const float off = a.W.offset[0];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM, kc0 = static_cast<int64_t>(blockIdx.x) * BN;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  for (int64_t n0 = 0; n0 < a.N; n0 += BK) {
    load_rowmajor<BM, NT>(sA, a.G, a.N, a.M, m0, a.N, n0);
    load_nf4_bwd<BN, NT>(sB, a.W, tb, off, a.K, a.N, kc0, n0);
    __syncthreads();
    mma_tile<TM, TN>(sA, sB, acc, wm * TM * 16, wn * TN * 16, lane);
    __syncthreads();
  }
  for (int64_t j0 = 0; j0 < a.r; j0 += BK) {
    load_rowmajor<BM, NT>(sA, a.dZ, a.r, a.M, m0, a.r, j0);
    load_rowmajor<BN, NT>(sB, a.A, a.r, a.K, kc0, a.r, j0);
    __syncthreads();
    mma_tile<TM, TN>(sA, sB, acc, wm * TM * 16, wn * TN * 16, lane);
    __syncthreads();
  }
  store_tile<TM, TN>(acc, m0 + wm * TM * 16, kc0 + wn * TN * 16, a.M, a.K, a.K, a.dX, nullptr, lane);
}

struct SkinnyArgs {
  const uint16_t* srcA;  // operand A source
  const uint16_t* srcB;  // operand B source
  int64_t ldA, ldB;
  int64_t rows, cols, red;
  int64_t red_per_split;
  float* part;  // [splits][rows][cols]
};

// Generic rank-r product with a split reduction.  TA/TB select a transposed
// source ([red][row]) instead of a row-major one ([row][red]).
template <int BM, int BN, int WM, int WN, bool TA, bool TB>
__global__ __launch_bounds__(WM* WN * 64) void skinny_kernel(SkinnyArgs a) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * PITCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * BM, c0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * a.red_per_split;
  const int64_t kend = min(a.red, kbeg + a.red_per_split);
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    if (TA)
      load_transposed<BM, NT, false>(sA, a.srcA, a.ldA, a.rows, r0, kend, k0, 1.0f);
    else
      load_rowmajor<BM, NT>(sA, a.srcA, a.ldA, a.rows, r0, kend, k0);
    if (TB)
      load_transposed<BN, NT, false>(sB, a.srcB, a.ldB, a.cols, c0, kend, k0, 1.0f);
    else
      load_rowmajor<BN, NT>(sB, a.srcB, a.ldB, a.cols, c0, kend, k0);
    __syncthreads();
    mma_tile<TM, TN>(sA, sB, acc, wm * TM * 16, wn * TN * 16, lane);
    __syncthreads();
  }
  store_tile<TM, TN>(acc, r0 + wm * TM * 16, c0 + wn * TN * 16, a.rows, a.cols, a.cols, nullptr,
                     a.part + static_cast<int64_t>(blockIdx.z) * a.rows * a.cols, lane);
}

// out[i] = scale * sum_{s=0..S-1} part[s][i] in that order; writes fp32
// and/or bf16.
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int splits,
                                                            int64_t count, float scale,
                                                            float* __restrict__ out_f32,
                                                            uint16_t* __restrict__ out_bf16) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float s = 0.0f;
    for (int k = 0; k < splits; ++k) s += part[k * count + i];
    s *= scale;
    if (out_f32) out_f32[i] = s;
    if (out_bf16) out_bf16[i] = to_bf16(s);
  }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Splits of a reduction of length red so that tiles*splits reaches ~target
// workgroups; every split but the last covers a multiple of BK.
void choose_split(int64_t tiles, int64_t red, int64_t target, int64_t* splits, int64_t* per_split) {
  int64_t s = ceil_div(target, tiles);
  const int64_t max_s = ceil_div(red, BK);
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  int64_t per = align_up(ceil_div(red, s), BK);
  *per_split = per;
  *splits = ceil_div(red, per);
}

hipError_t launch_reduce(const float* part, int64_t splits, int64_t count, float scale, float* out_f32,
                         uint16_t* out_bf16, hipStream_t stream) {
  int64_t blocks = ceil_div(count, 256);
  if (blocks > 8192) blocks = 8192;
  Timer t(QK_REDUCE, stream);
  hipLaunchKernelGGL(reduce_splits_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, part,
                     static_cast<int>(splits), count, scale, out_f32, out_bf16);
  t.stop();
  return hipGetLastError();
}

// Tile shapes.
constexpr int kTallBM = 128, kTallBN = 64;          // rows large, cols = r
constexpr int kWideBM = 64, kWideBN = 128;          // rows = r, cols large
constexpr int kGemvBM = 16, kGemvBN = 256;          // M <= 16 forward
constexpr int64_t kSplitTarget = 1024;

struct FwdPlan {
  bool gemv;
  int64_t z_splits, z_per;
  int64_t y_splits, y_per;
  int64_t z_part_bytes, y_part_bytes;
};

FwdPlan plan_fwd(int64_t M, int64_t K, int64_t N, int64_t r) {
  FwdPlan p{};
  p.gemv = M <= 16;
  choose_split(ceil_div(M, kTallBM) * ceil_div(r, kTallBN), K, kSplitTarget, &p.z_splits, &p.z_per);
  p.z_part_bytes = align_up(p.z_splits * M * r * 4, 256);
  if (p.gemv) {
    choose_split(ceil_div(N, kGemvBN), K, kSplitTarget, &p.y_splits, &p.y_per);
    p.y_part_bytes = align_up(p.y_splits * M * N * 4, 256);
  } else {
    p.y_splits = 1;
    p.y_per = align_up(K, BK);
    p.y_part_bytes = 0;
  }
  return p;
}

struct BwdPlan {
  int64_t dz_splits, dz_per, da_splits, da_per, db_splits, db_per;
  int64_t dz_part, dz_bf16, da_part, db_part;
};

BwdPlan plan_bwd(int64_t M, int64_t K, int64_t N, int64_t r) {
  BwdPlan p{};
  choose_split(ceil_div(M, kTallBM) * ceil_div(r, kTallBN), N, kSplitTarget, &p.dz_splits, &p.dz_per);
  choose_split(ceil_div(K, kTallBM) * ceil_div(r, kTallBN), M, kSplitTarget, &p.da_splits, &p.da_per);
  choose_split(ceil_div(r, kWideBM) * ceil_div(N, kWideBN), M, kSplitTarget, &p.db_splits, &p.db_per);
  p.dz_part = align_up(p.dz_splits * M * r * 4, 256);
  p.dz_bf16 = align_up(M * r * 2, 256);
  p.da_part = align_up(p.da_splits * K * r * 4, 256);
  p.db_part = align_up(p.db_splits * r * N * 4, 256);
  return p;
}

}  // namespace

int64_t fwd_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t r) {
  const FwdPlan p = plan_fwd(M, K, N, r);
  return p.z_part_bytes + p.y_part_bytes;
}

int64_t bwd_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t r) {
  const BwdPlan p = plan_bwd(M, K, N, r);
  return p.dz_part + p.dz_bf16 + p.da_part + p.db_part;
}

hipError_t launch_fwd(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W,
                      const uint16_t* A, const uint16_t* B, float c, uint16_t* Y, uint16_t* Z, void* ws,
                      hipStream_t stream) {
  const FwdPlan p = plan_fwd(M, K, N, r);
  char* base = static_cast<char*>(ws);
  float* zpart = reinterpret_cast<float*>(base);
  float* ypart = reinterpret_cast<float*>(base + p.z_part_bytes);

  // Z = X A (split over K), reduced in fixed order to bf16.
  {
    SkinnyArgs s{X, A, K, r, M, r, K, p.z_per, zpart};
    dim3 grid(static_cast<unsigned>(ceil_div(r, kTallBN)), static_cast<unsigned>(ceil_div(M, kTallBM)),
              static_cast<unsigned>(p.z_splits));
    Timer t(QK_LORA_DOWN, stream);
    hipLaunchKernelGGL((skinny_kernel<kTallBM, kTallBN, 4, 1, false, true>), grid, dim3(256), 0, stream, s);
    t.stop();
    hipError_t e = launch_reduce(zpart, p.z_splits, M * r, 1.0f, nullptr, Z, stream);
    if (e != hipSuccess) return e;
  }
  if (p.gemv) {
    FwdArgs f{X, W, Z, B, c, nullptr, ypart, M, K, N, r, p.y_per};
    dim3 grid(static_cast<unsigned>(ceil_div(N, kGemvBN)), 1, static_cast<unsigned>(p.y_splits));
    Timer t(QK_FWD_GEMV, stream);
    hipLaunchKernelGGL((qlora_fwd_kernel<kGemvBM, kGemvBN, 1, 4>), grid, dim3(256), 0, stream, f);
    t.stop();
    return launch_reduce(ypart, p.y_splits, M * N, 1.0f, nullptr, Y, stream);
  }
  return launch_fwd_big(M, K, N, r, X, W, Z, B, c, Y, stream);
}

hipError_t launch_bwd(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G, const uint16_t* X,
                      const uint16_t* Z, NF4View W, const uint16_t* A, const uint16_t* B, float c,
                      uint16_t* dX, float* dA, float* dB, void* ws, hipStream_t stream) {
  const BwdPlan p = plan_bwd(M, K, N, r);
  char* base = static_cast<char*>(ws);
  float* dzpart = reinterpret_cast<float*>(base);
  uint16_t* dz16 = reinterpret_cast<uint16_t*>(base + p.dz_part);
  float* dapart = reinterpret_cast<float*>(base + p.dz_part + p.dz_bf16);
  float* dbpart = reinterpret_cast<float*>(base + p.dz_part + p.dz_bf16 + p.da_part);
  hipError_t e;

  // dZ = c G Bᵀ (split over N) -> bf16
  {
    SkinnyArgs s{G, B, N, N, M, r, N, p.dz_per, dzpart};
    dim3 grid(static_cast<unsigned>(ceil_div(r, kTallBN)), static_cast<unsigned>(ceil_div(M, kTallBM)),
              static_cast<unsigned>(p.dz_splits));
    Timer t(QK_BWD_DZ, stream);
    hipLaunchKernelGGL((skinny_kernel<kTallBM, kTallBN, 4, 1, false, false>), grid, dim3(256), 0, stream, s);
    t.stop();
    if ((e = launch_reduce(dzpart, p.dz_splits, M * r, c, nullptr, dz16, stream)) != hipSuccess) return e;
  }
  // dB = c Zᵀ G (split over M)
  {
    SkinnyArgs s{Z, G, r, N, r, N, M, p.db_per, dbpart};
    dim3 grid(static_cast<unsigned>(ceil_div(N, kWideBN)), static_cast<unsigned>(ceil_div(r, kWideBM)),
              static_cast<unsigned>(p.db_splits));
    Timer t(QK_BWD_DB, stream);
    hipLaunchKernelGGL((skinny_kernel<kWideBM, kWideBN, 1, 4, true, true>), grid, dim3(256), 0, stream, s);
    t.stop();
    if ((e = launch_reduce(dbpart, p.db_splits, r * N, c, dB, nullptr, stream)) != hipSuccess) return e;
  }
  // dA = Xᵀ dZ (split over M)
  {
    SkinnyArgs s{X, dz16, K, r, K, r, M, p.da_per, dapart};
    dim3 grid(static_cast<unsigned>(ceil_div(r, kTallBN)), static_cast<unsigned>(ceil_div(K, kTallBM)),
              static_cast<unsigned>(p.da_splits));
    Timer t(QK_BWD_DA, stream);
    hipLaunchKernelGGL((skinny_kernel<kTallBM, kTallBN, 4, 1, true, true>), grid, dim3(256), 0, stream, s);
    t.stop();
    if ((e = launch_reduce(dapart, p.da_splits, K * r, 1.0f, dA, nullptr, stream)) != hipSuccess) return e;
  }
  // dX = G Ŵᵀ + dZ Aᵀ
  if (dX != nullptr) {
    if ((e = launch_dx_big(M, K, N, r, G, W, dz16, A, dX, stream)) != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace qn
