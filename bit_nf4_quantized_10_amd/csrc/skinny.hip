// Rank-r products of the layer and the small-M dequant-GEMV, for gfx950.
//
// Layer (page "QLoRA：冻结的 4-bit 权重怎样参与一次微调", sections
// "量化基座与可训练支路怎样相加" and "冻结权重为什么仍然需要输入梯度"):
//   Z = X A (M x r), dZ = c G Bᵀ (M x r): "row sums" - each output row reduces
//     one activation row against r weight rows; both operands are contiguous
//     along the reduction, so MFMA fragments are loaded straight from global
//     memory (A is transposed once, r x K, so that it is too).
//   dA = Xᵀ dZ (K x r), dB = c Zᵀ G (r x N): "column sums" over the M tokens;
//     both operands are strided along the reduction, so 32-token tiles are
//     transposed through LDS.
//   The small-M forward (M <= 16): each wave streams a 128-column slab of the
//     packed weight over a k-range with 8 code words per lane per 32 rows,
//     transposes the nibbles in registers and feeds 8 MFMAs whose A operand is
//     the (zero-padded) 16-row activation block; the four waves of a workgroup
//     cover consecutive k-ranges and are summed in LDS in a fixed order; the
//     split-K partials and the LoRA term c Z B are added by a final kernel.
// Every reduction is in a fixed order, so results are run-to-run identical.
#include "common.hpp"
#include "kernels.hpp"

namespace qn {

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

__device__ __forceinline__ uint16_t bf16_of(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.0f) & 0xffffu);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ------------------------------------------------------------ transpose
// dst[c][r] = RNE_bf16(scale * src[r][c]) for a rows x cols bf16 matrix
// (32 x 32 LDS tiles; scale 1 copies the bits).  One launch serves two such
// jobs: Aᵀ for the rank-r products and, in the forward, the LoRA extension
// operand (c B)ᵀ, rounded once to bf16.
struct TJob {
  const uint16_t* src;
  uint16_t* dst;
  int64_t rows, cols;
  float scale;
  int64_t bx, nblk;   // 32-column tiles per tile row, tiles in this job
};

__global__ __launch_bounds__(256) void transpose_bf16_kernel(TJob j0, TJob j1) {
  __shared__ uint16_t tile[32][33];
  const bool second = blockIdx.x >= j0.nblk;
  const TJob j = second ? j1 : j0;
  const int64_t b = second ? blockIdx.x - j0.nblk : blockIdx.x;
  const int64_t r0 = (b / j.bx) * 32, c0 = (b % j.bx) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int64_t r = r0 + i, c = c0 + tx;
    uint16_t v = (r < j.rows && c < j.cols) ? j.src[r * j.cols + c] : 0;
    if (j.scale != 1.0f) v = bf16_of(j.scale * bf16_bits_to_f32(v));
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < j.cols && r < j.rows) j.dst[c * j.rows + r] = tile[tx][i];
  }
}

TJob tjob(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols, float scale) {
  const int64_t bx = cdiv(cols, 32);
  return TJob{src, dst, rows, cols, scale, bx, bx * cdiv(rows, 32)};
}

// ------------------------------------------------------------ row sums
// out[row][j] = sum_red act[row][red] * wt[j][red] over this wave's split.
// One wave per (16-row tile, split); r <= 16 * RT.  The reduction runs in
// chunks of U steps of 32; the next chunk's fragments are loaded before the
// current chunk's MFMAs so that memory latency overlaps the math.
template <int RT, int U>
struct RowFrag {
  uint4 a[U];
  uint4 w[U][RT];
};

template <int RT, int U>
__device__ __forceinline__ void rowsum_load(RowFrag<RT, U>& f, Rsrc ra, int64_t arow_off, bool row_ok, Rsrc rw,
                                            int64_t ld_wt, int64_t r, int64_t kc, int64_t end, int q, int g) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t k = kc + 32 * u + 8 * g;
    const bool k_ok = k < end;
    f.a[u] = ld_b128(ra, (row_ok && k_ok) ? static_cast<uint32_t>((arow_off + k) * 2) : kMasked);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int64_t j = 16 * t + q;
      f.w[u][t] = ld_b128(rw, (j < r && k_ok) ? static_cast<uint32_t>((j * ld_wt + k) * 2) : kMasked);
    }
  }
}

template <int RT, int U>
__global__ __launch_bounds__(64) void rowsum_kernel(const uint16_t* __restrict__ act, int64_t ld_act,
                                                    const uint16_t* __restrict__ wt, int64_t ld_wt,
                                                    int64_t rows, int64_t r, int64_t red, int64_t per_split,
                                                    int64_t row_tiles, float* __restrict__ part) {
  const int lane = threadIdx.x, q = lane & 15, g = lane >> 4;
  const int64_t tile = blockIdx.x % row_tiles, split = blockIdx.x / row_tiles;
  const int64_t row = tile * 16 + q;
  const int64_t beg = split * per_split, end = min(red, beg + per_split);
  const bool row_ok = row < rows;
  const Rsrc ra = make_rsrc(act, rows * ld_act * 2), rw = make_rsrc(wt, r * ld_wt * 2);
  const int64_t arow_off = row * ld_act;
  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0, 0, 0, 0};
  RowFrag<RT, U> cur, nxt;
  rowsum_load<RT, U>(cur, ra, arow_off, row_ok, rw, ld_wt, r, beg, end, q, g);
  for (int64_t kc = beg; kc < end; kc += 32 * U) {
    const int64_t kn = kc + 32 * U;
    rowsum_load<RT, U>(nxt, ra, arow_off, row_ok, rw, ld_wt, r, kn, end, q, g);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < RT; ++t)
        acc[t] = mfma16x16x32(__builtin_bit_cast(bf16x8, cur.a[u]), __builtin_bit_cast(bf16x8, cur.w[u][t]), acc[t]);
    cur = nxt;
  }
  // lane holds rows 4g+e of column 16t+q
  float* out = part + split * rows * r;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int64_t j = 16 * t + q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t orow = tile * 16 + 4 * g + e;
      if (orow < rows && j < r) out[orow * r + j] = acc[t][e];
    }
  }
}

// ------------------------------------------------------------ column sums
// out[col][j] = sum_m act[m][col] * v[m][j] over this workgroup's token split;
// 64 columns x r (<= 64) per workgroup, 32 tokens per LDS step.
constexpr int kCsPitch = 40;  // 32 tokens + 8 pad (bf16)

__global__ __launch_bounds__(256) void colsum_kernel(const uint16_t* __restrict__ act, int64_t ld_act,
                                                     const uint16_t* __restrict__ v, int64_t r, int64_t j0,
                                                     int64_t M, int64_t cols, int64_t per_split, int64_t col_tiles,
                                                     float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t sAct[64 * kCsPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sV[64 * kCsPitch];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, q = lane & 15, g = lane >> 4;
  const int64_t ctile = blockIdx.x % col_tiles, split = blockIdx.x / col_tiles;
  const int64_t c0 = ctile * 64;
  const int64_t beg = split * per_split, end = min(M, beg + per_split);
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0, 0, 0, 0};
  const int lr = t >> 3, lc = t & 7;  // loader: token row lr (0..31), 8-wide chunk lc
  const Rsrc ra = make_rsrc(act, M * ld_act * 2), rv = make_rsrc(v, M * r * 2);
  auto load = [&](int64_t m0, uint4& a4, uint4& v4) {
    const int64_t m = m0 + lr;
    const bool ok = m < end;
    a4 = ld_b128(ra, (ok && c0 + 8 * lc < cols) ? static_cast<uint32_t>((m * ld_act + c0 + 8 * lc) * 2) : kMasked);
    v4 = ld_b128(rv, (ok && j0 + 8 * lc < r) ? static_cast<uint32_t>((m * r + j0 + 8 * lc) * 2) : kMasked);
  };
  uint4 a4, v4;
  load(beg, a4, v4);
  for (int64_t m0 = beg; m0 < end; m0 += 32) {
    const uint32_t aw[4] = {a4.x, a4.y, a4.z, a4.w}, vw[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sAct[(8 * lc + e) * kCsPitch + lr] = static_cast<uint16_t>(aw[e >> 1] >> (16 * (e & 1)));
      sV[(8 * lc + e) * kCsPitch + lr] = static_cast<uint16_t>(vw[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
    load(m0 + 32, a4, v4);
    const bf16x8 af = *reinterpret_cast<const bf16x8*>(sAct + (16 * wave + q) * kCsPitch + 8 * g);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sV + (16 * jt + q) * kCsPitch + 8 * g);
      acc[jt] = mfma16x16x32(af, vf, acc[jt]);
    }
    __syncthreads();
  }
  // wave covers columns 16*wave + 4g + e, j = 16*jt + q
  float* out = part + split * cols * r;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const int64_t j = j0 + 16 * jt + q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t col = c0 + 16 * wave + 4 * g + e;
      if (col < cols && j < r) out[col * r + j] = acc[jt][e];
    }
  }
}

// out = scale * sum_s part[s] (fixed order), optionally transposed from
// [rows][cols] to [cols][rows]; fp32 and/or bf16 outputs.
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, int splits, int64_t rows,
                                                     int64_t cols, float scale, bool transpose,
                                                     float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16) {
  const int64_t count = rows * cols;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float s = 0.0f;
    int k = 0;
    for (; k + 8 <= splits; k += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(k + u) * count + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; k < splits; ++k) s += part[k * count + i];
    s *= scale;
    const int64_t o = transpose ? (i % cols) * rows + i / cols : i;
    if (out_f32) out_f32[o] = s;
    if (out_bf16) out_bf16[o] = bf16_of(s);
  }
}

// ------------------------------------------------------------ small-M GEMV
constexpr int kGvWaves = 4;
constexpr int kGvCols = 256;    // columns per workgroup slab (16 per lane)
constexpr int kGvTab = 32 * 4 * 16;  // bf16 entries of one wave's tables for one 32-row step

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// 8 x 8 bf16 transpose: out[t] holds column t of the 8 input rows.
__device__ __forceinline__ void transpose8x8_bf16(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
    uint32_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) d[p] = perm(word_of(in[2 * p + 1], t >> 1), word_of(in[2 * p], t >> 1), sel);
    out[t] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// Nibble of column t (0..7) in a code word: byte t/2, high nibble for even t.
__device__ __forceinline__ uint32_t nib(uint32_t w, int t) { return (w >> (8 * (t >> 1) + ((t & 1) ? 0 : 4))) & 15u; }

struct GvStep {
  uint2 w[8];   // code words of rows 8g..8g+7 (16 columns each)
  uint4 x;      // activation fragment
  int q[2];     // second-level codes of the two tables this lane builds
  float s2[2];
};

// Workgroup (4 waves) = one 256-column slab; wave w covers rows
// [(split*4 + w) * rpw, +rpw) in steps of 32.  Lane (q, g): columns
// n0 + 16q .. +15, rows 8g .. 8g+7 of each step.  Per step, each wave first
// writes the 128 block tables (32 rows x 4 blocks, 16 bf16 each) of the NEXT
// step to its LDS ring, then decodes the current step by table lookups, so no
// per-weight multiply or conversion is needed; column t of the lane feeds the
// MFMA of tile t.  part[split][m][n] = sum of the 4 waves (fixed order).
__global__ __launch_bounds__(256) void gemv_kernel(const uint16_t* __restrict__ X, int64_t M, NF4View W, int64_t K,
                                                   int64_t N, int64_t rpw, int64_t slabs, float* __restrict__ part) {
  __shared__ float q2t[256];
  __shared__ __attribute__((aligned(16))) uint16_t tabs[kGvWaves * 2 * kGvTab];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, q = lane & 15, g = lane >> 4;
  q2t[t] = q2_value(t - 128);
  const int64_t slab = blockIdx.x % slabs, split = blockIdx.x / slabs;
  const int64_t n0 = slab * kGvCols;
  const int64_t kw0 = (split * kGvWaves + wave) * rpw;
  const int64_t P = K * N;
  const Rsrc rc = make_rsrc(W.codes, (P + 1) / 2);
  const Rsrc rq = make_rsrc(W.qabsmax, (P + 63) / 64);
  const Rsrc rs = make_rsrc(W.absmax2, ((P + 16383) / 16384) * 4);
  const Rsrc rx = make_rsrc(X, M * K * 2);
  const float off = W.offset[0];
  const int64_t n = n0 + 16 * q;
  const bool n_ok = n < N;
  const int blk = q >> 2;
  uint16_t* my_tabs = tabs + wave * 2 * kGvTab;

  auto load = [&](GvStep& S, int64_t kk) {
    const int64_t kb = kw0 + kk + 8 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t k = kb + i;
      S.w[i] = ld_b64(rc, (k < K && n_ok) ? static_cast<uint32_t>((k * N + n) >> 1) : kMasked);
    }
    S.x = ld_b128(rx, (q < M && kb < K) ? static_cast<uint32_t>((q * K + kb) * 2) : kMasked);
    const int64_t kt = kw0 + kk + (lane >> 1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t nb = n0 + 64 * (2 * (lane & 1) + u);
      const bool ok = kt < K && nb < N;
      const int64_t e = kt * N + nb;
      S.q[u] = ld_i8(rq, ok ? static_cast<uint32_t>(e >> 6) : kMasked);
      S.s2[u] = ld_f32(rs, ok ? static_cast<uint32_t>((e >> 14) * 4) : kMasked);
    }
  };
  auto build = [&](const GvStep& S, int buf) {
    uint16_t* tb = my_tabs + buf * kGvTab + ((lane >> 1) * 4 + 2 * (lane & 1)) * 16;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      write_block_table(tb + 16 * u, __fadd_rn(__fmul_rn(q2t[S.q[u] + 128], S.s2[u]), off));
  };

  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0, 0, 0, 0};
  __syncthreads();  // q2t
  GvStep cur, nxt;
  load(cur, 0);
  build(cur, 0);
  __syncthreads();
  int buf = 0;
  for (int64_t kk = 0; kk < rpw; kk += 32) {
    const bool more = kk + 32 < rpw;
    if (more) load(nxt, kk + 32);
    const uint16_t* tb = my_tabs + buf * kGvTab + (8 * g * 4 + blk) * 16;  // table of row 8g, this lane's block
    const bf16x8 xf = __builtin_bit_cast(bf16x8, cur.x);
#pragma unroll
    for (int tile = 0; tile < 16; ++tile) {
      uint32_t fw[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t w0 = (tile < 8) ? cur.w[2 * p].x : cur.w[2 * p].y;
        const uint32_t w1 = (tile < 8) ? cur.w[2 * p + 1].x : cur.w[2 * p + 1].y;
        const uint32_t lo = tb[(2 * p) * 64 + nib(w0, tile & 7)];
        const uint32_t hi = tb[(2 * p + 1) * 64 + nib(w1, tile & 7)];
        fw[p] = lo | (hi << 16);
      }
      acc[tile] = mfma16x16x32(xf, __builtin_bit_cast(bf16x8, make_uint4(fw[0], fw[1], fw[2], fw[3])), acc[tile]);
    }
    if (more) build(nxt, buf ^ 1);
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }
  // lane holds Y[m = 4g+e][n + tile]; fixed-order sum: (w0 + w2) + (w1 + w3)
  float* red = reinterpret_cast<float*>(tabs);   // 2 waves x 64 floats x 64 lanes = 32 KB
  if (wave >= 2) {
#pragma unroll
    for (int tile = 0; tile < 16; ++tile)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave - 2) * 64 + tile * 4 + e) * 64 + lane] = acc[tile][e];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int tile = 0; tile < 16; ++tile)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[tile][e] += red[(wave * 64 + tile * 4 + e) * 64 + lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int tile = 0; tile < 16; ++tile)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(tile * 4 + e) * 64 + lane] = acc[tile][e];
  }
  __syncthreads();
  if (wave == 0) {
    float* out = part + split * M * N;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t m = 4 * g + e;
      float v[16];
#pragma unroll
      for (int tile = 0; tile < 16; ++tile) v[tile] = acc[tile][e] + red[(tile * 4 + e) * 64 + lane];
      if (m < M && n_ok) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          *reinterpret_cast<float4*>(out + m * N + n + 4 * h) = make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
      }
    }
  }
}

// Y = sum_s part[s] + c Z B for M <= 16: one wave per 128 columns; lane
// (q, g) holds rows 4g..4g+3 of columns n0+8q..+7; the LoRA product runs on
// MFMA with B transposed in registers.
__global__ __launch_bounds__(64) void gemv_finish_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                         int64_t N, const uint16_t* __restrict__ Z,
                                                         const uint16_t* __restrict__ B, int64_t r, float c,
                                                         uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x, q = lane & 15, g = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 128, n = n0 + 8 * q;
  const bool n_ok = n < N;
  const Rsrc rz = make_rsrc(Z, M * r * 2), rb = make_rsrc(B, r * N * 2);
  f32x4 accl[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) accl[i] = f32x4{0, 0, 0, 0};
  for (int64_t j0 = 0; j0 < r; j0 += 32) {
    const int64_t jb = j0 + 8 * g;
    const uint4 zv = ld_b128(rz, (q < M && jb < r) ? static_cast<uint32_t>((q * r + jb) * 2) : kMasked);
    uint4 rows8[8], cols8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rows8[i] = ld_b128(rb, (jb + i < r && n_ok) ? static_cast<uint32_t>(((jb + i) * N + n) * 2) : kMasked);
    transpose8x8_bf16(rows8, cols8);
#pragma unroll
    for (int tc = 0; tc < 8; ++tc)
      accl[tc] = mfma16x16x32(__builtin_bit_cast(bf16x8, zv), __builtin_bit_cast(bf16x8, cols8[tc]), accl[tc]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t m = 4 * g + e;
    if (m >= M || !n_ok) continue;
    float v[8];
#pragma unroll
    for (int tc = 0; tc < 8; ++tc) v[tc] = 0.0f;
    for (int s = 0; s < splits; ++s) {
      const float* src = part + (s * M + m) * N + n;
      const float4 a = *reinterpret_cast<const float4*>(src), b = *reinterpret_cast<const float4*>(src + 4);
      v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w; v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
    }
    uint4 o;
    o.x = pack_bf16x2(v[0] + c * accl[0][e], v[1] + c * accl[1][e]);
    o.y = pack_bf16x2(v[2] + c * accl[2][e], v[3] + c * accl[3][e]);
    o.z = pack_bf16x2(v[4] + c * accl[4][e], v[5] + c * accl[5][e]);
    o.w = pack_bf16x2(v[6] + c * accl[6][e], v[7] + c * accl[7][e]);
    *reinterpret_cast<uint4*>(Y + m * N + n) = o;
  }
}

void split_plan(int64_t tiles, int64_t red, int64_t target, int64_t quantum, int64_t* splits, int64_t* per) {
  int64_t s = cdiv(target, tiles);
  const int64_t max_s = cdiv(red, quantum);
  s = s < 1 ? 1 : (s > max_s ? max_s : s);
  *per = round_up(cdiv(red, s), quantum);
  *splits = cdiv(red, *per);
}

hipError_t launch_reduce2(const float* part, int64_t splits, int64_t rows, int64_t cols, float scale, bool transpose,
                          float* out_f32, uint16_t* out_bf16, hipStream_t stream) {
  int64_t blocks = cdiv(rows * cols, 256);
  if (blocks > 4096) blocks = 4096;
  Timer tm(QK_REDUCE, stream);
  hipLaunchKernelGGL(reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, part,
                     static_cast<int>(splits), rows, cols, scale, transpose, out_f32, out_bf16);
  tm.stop();
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------ plans
#ifndef QN_ROWSUM_WAVES
#define QN_ROWSUM_WAVES 512   // target number of row-sum waves (row tiles x splits)
#endif
SkinnyPlan plan_skinny(int64_t M, int64_t K, int64_t N, int64_t r) {
  SkinnyPlan p{};
  const int64_t row_tiles = cdiv(M, 16);
  split_plan(row_tiles, K, QN_ROWSUM_WAVES, 128, &p.z_splits, &p.z_per);
  split_plan(row_tiles, N, QN_ROWSUM_WAVES, 128, &p.dz_splits, &p.dz_per);
  split_plan(cdiv(K, 64), M, 512, 32, &p.da_splits, &p.da_per);
  split_plan(cdiv(N, 64), M, 512, 32, &p.db_splits, &p.db_per);
  p.at_bytes = round_up(r * K * 2, 256);
  p.z_part = round_up(p.z_splits * M * r * 4, 256);
  p.dz_part = round_up(p.dz_splits * M * r * 4, 256);
  p.da_part = round_up(p.da_splits * K * r * 4, 256);
  p.db_part = round_up(p.db_splits * N * r * 4, 256);
  // GEMV: 4 waves x rows_per_wave rows per workgroup, ~1400 waves in total
  const int64_t slabs = cdiv(N, kGvCols);
  const int64_t groups = cdiv(1400, slabs * kGvWaves);
  int64_t rpw = round_up(cdiv(K, groups * kGvWaves), 32);
  if (rpw < 64) rpw = 64;
  p.gv_rows_per_wave = rpw;
  p.gv_splits = cdiv(K, rpw * kGvWaves);
  p.gv_part = round_up(p.gv_splits * M * N * 4, 256);
  return p;
}

hipError_t launch_lora_down(int64_t M, int64_t K, int64_t r, const uint16_t* X, const uint16_t* A, uint16_t* Z,
                            const SkinnyPlan& p, void* at_ws, void* part_ws, hipStream_t stream, int64_t N,
                            const uint16_t* B, float c, uint16_t* cbt) {
  uint16_t* At = static_cast<uint16_t*>(at_ws);
  const TJob ja = tjob(A, At, K, r, 1.0f);
  TJob jb = cbt != nullptr ? tjob(B, cbt, r, N, c) : ja;
  if (cbt == nullptr) jb.nblk = 0;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(static_cast<unsigned>(ja.nblk + jb.nblk)), dim3(256), 0, stream, ja,
                     jb);
  float* part = static_cast<float*>(part_ws);
  const int64_t row_tiles = cdiv(M, 16);
  Timer tm(QK_LORA_DOWN, stream);
  if (r <= 64)
    hipLaunchKernelGGL((rowsum_kernel<4, 4>), dim3(static_cast<unsigned>(row_tiles * p.z_splits)), dim3(64), 0, stream, X,
                       K, At, K, M, r, K, p.z_per, row_tiles, part);
  else
    hipLaunchKernelGGL((rowsum_kernel<16, 1>), dim3(static_cast<unsigned>(row_tiles * p.z_splits)), dim3(64), 0, stream,
                       X, K, At, K, M, r, K, p.z_per, row_tiles, part);
  tm.stop();
  return launch_reduce2(part, p.z_splits, M, r, 1.0f, false, nullptr, Z, stream);
}

hipError_t launch_gemv(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W, const uint16_t* Z,
                       const uint16_t* B, float c, uint16_t* Y, const SkinnyPlan& p, void* part_ws,
                       hipStream_t stream) {
  const int64_t slabs = cdiv(N, kGvCols);
  float* part = static_cast<float*>(part_ws);
  Timer tm(QK_FWD_GEMV, stream);
  hipLaunchKernelGGL(gemv_kernel, dim3(static_cast<unsigned>(slabs * p.gv_splits)), dim3(kGvWaves * 64), 0, stream, X,
                     M, W, K, N, p.gv_rows_per_wave, slabs, part);
  tm.stop();
  Timer te(QK_REDUCE, stream);
  hipLaunchKernelGGL(gemv_finish_kernel, dim3(static_cast<unsigned>(cdiv(N, 128))), dim3(64), 0, stream, part,
                     static_cast<int>(p.gv_splits), M, N, Z, B, r, c, Y);
  te.stop();
  return hipGetLastError();
}

hipError_t launch_dz(int64_t M, int64_t N, int64_t r, const uint16_t* G, const uint16_t* B, float c, uint16_t* dZ,
                     const SkinnyPlan& p, void* part_ws, hipStream_t stream) {
  float* part = static_cast<float*>(part_ws);
  const int64_t row_tiles = cdiv(M, 16);
  Timer tm(QK_BWD_DZ, stream);
  if (r <= 64)
    hipLaunchKernelGGL((rowsum_kernel<4, 4>), dim3(static_cast<unsigned>(row_tiles * p.dz_splits)), dim3(64), 0, stream,
                       G, N, B, N, M, r, N, p.dz_per, row_tiles, part);
  else
    hipLaunchKernelGGL((rowsum_kernel<16, 1>), dim3(static_cast<unsigned>(row_tiles * p.dz_splits)), dim3(64), 0, stream,
                       G, N, B, N, M, r, N, p.dz_per, row_tiles, part);
  tm.stop();
  return launch_reduce2(part, p.dz_splits, M, r, c, false, nullptr, dZ, stream);
}

// dA = Xᵀ dZ (K x r) and dB = c Zᵀ G (r x N).
hipError_t launch_colsums(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, const uint16_t* G,
                          const uint16_t* Z, const uint16_t* dZ, float c, float* dA, float* dB, const SkinnyPlan& p,
                          void* da_ws, void* db_ws, hipStream_t stream) {
  hipError_t e;
  {
    const int64_t tiles = cdiv(K, 64);
    Timer tm(QK_BWD_DA, stream);
    for (int64_t j0 = 0; j0 < r; j0 += 64)
      hipLaunchKernelGGL(colsum_kernel, dim3(static_cast<unsigned>(tiles * p.da_splits)), dim3(256), 0, stream, X, K,
                         dZ, r, j0, M, K, p.da_per, tiles, static_cast<float*>(da_ws));
    tm.stop();
    if ((e = launch_reduce2(static_cast<float*>(da_ws), p.da_splits, K, r, 1.0f, false, dA, nullptr, stream)) !=
        hipSuccess)
      return e;
  }
  {
    const int64_t tiles = cdiv(N, 64);
    Timer tm(QK_BWD_DB, stream);
    for (int64_t j0 = 0; j0 < r; j0 += 64)
      hipLaunchKernelGGL(colsum_kernel, dim3(static_cast<unsigned>(tiles * p.db_splits)), dim3(256), 0, stream, G, N,
                         Z, r, j0, M, N, p.db_per, tiles, static_cast<float*>(db_ws));
    tm.stop();
    if ((e = launch_reduce2(static_cast<float*>(db_ws), p.db_splits, N, r, c, true, dB, nullptr, stream)) !=
        hipSuccess)
      return e;
  }
  return hipGetLastError();
}

}  // namespace qn
