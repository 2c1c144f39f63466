// Small-M forward (M <= 16) for gfx950: Y = X Ŵ + c Z B as a dequant-GEMV
// (page "QLoRA：冻结的 4-bit 权重怎样参与一次微调", section "量化基座与可训练支路怎样相加";
// the decode is the one of section "Double Quantization 压缩的是 Scale").
//
// Workgroup (4 waves) = one 256-column slab; wave w covers a contiguous range
// of 32-row steps.  Lane (q, g) owns columns n0 + 16q .. +15 and rows
// 8g .. 8g+7 of each step.  Per step each wave writes the 128 block tables
// (32 rows x 4 blocks, 16 bf16 RNE(fl32(C[j] * â)) each) of the step to its
// own LDS area and decodes by table lookups: one byte-select add and one
// 16-bit LDS read per weight, pairs packed with v_perm; column t of the lane
// feeds the MFMA of tile t with the zero-padded 16-row activation block.
// Three steps of code loads are in flight per wave (per-wave buffer
// descriptors, so rows past the wave's range read as zeros and meet zero
// activations).  The four waves are added in LDS in a fixed order; the
// split-K partials and the LoRA term are added by gemv_finish_kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace qn {

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

constexpr int kGvWaves = 4;
constexpr int kGvCols = 256;    // columns per workgroup slab (16 per lane)
// One wave's block tables for one 32-row step: row r (4 tables of 16 bf16,
// 128 bytes) at byte r * 128 + 128 * (r / 8), so that the four rows 8g + c
// (g = 0..3) that one lookup instruction touches fall on both halves of the
// 64 LDS banks.
constexpr int kGvTabBytes = 32 * 128 + 4 * 128;
#ifndef QN_GV_DEPTH
#define QN_GV_DEPTH 3
#endif
constexpr int kGvDepth = QN_GV_DEPTH;   // 32-row steps of code loads in flight per wave
__device__ __forceinline__ int gv_row(int r) { return r * 128 + 128 * (r >> 3); }

// base + byte b of w, one VALU instruction (SDWA byte select on the second operand)
__device__ __forceinline__ uint32_t add_byte(uint32_t base, uint32_t w, int b) {
  uint32_t r;
  switch (b) {
    case 0: asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(base), "v"(w)); break;
    case 1: asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(base), "v"(w)); break;
    case 2: asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(base), "v"(w)); break;
    default: asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(base), "v"(w)); break;
  }
  return r;
}

// 16-bit LDS load from a byte address
__device__ __forceinline__ uint32_t lds_u16(uint32_t addr) {
  typedef __attribute__((address_space(3))) const uint16_t* lp;
  return *reinterpret_cast<lp>(static_cast<uintptr_t>(addr));
}

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

// Split-K partial of Z = X A for M <= 16 over rows [split * 4 rpw, +4 rpw),
// each wave over the rows its GEMV counterpart streams.  A is read row-major
// (8 rows of 8 columns per lane, transposed in registers), X rows feed the
// MFMA as the 16-row operand; lane (q, g) accumulates columns j0 + 8q .. +7.
// The four waves are added in LDS in a fixed order: (w0 + w2) + (w1 + w3).
// zpart[split][m][j], fp32.  red: 16 KB of LDS.
template <class T>
__device__ void gemv_zpart(const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t rpw,
                           const uint16_t* __restrict__ A, int64_t r, float* __restrict__ zpart, int64_t split,
                           float* red) {
  const int t = threadIdx.x, lane = t & 63, q = lane & 15, g = lane >> 4;
  const int wave = t >> 6;
  const int64_t kw0 = (split * kGvWaves + wave) * rpw;
  const int64_t kend = min(K, kw0 + rpw);
  const Rsrc rx = make_rsrc(X, M * K * 2), ra = make_rsrc(A, K * r * 2);
  for (int64_t j0 = 0; j0 < r; j0 += 128) {
    const int64_t j = j0 + 8 * q;
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0, 0, 0, 0};
    for (int64_t kb = kw0; kb < kend; kb += 32) {
      const int64_t k = kb + 8 * g;
      const uint4 xv = ld_b128(rx, (q < M && k < kend) ? static_cast<uint32_t>((q * K + k) * 2) : kMasked);
      uint4 rows8[8], cols8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rows8[i] = ld_b128(ra, (k + i < kend && j < r) ? static_cast<uint32_t>(((k + i) * r + j) * 2) : kMasked);
      transpose8x8_bf16(rows8, cols8);
#pragma unroll
      for (int tc = 0; tc < 8; ++tc)
        acc[tc] = T::mfma16(__builtin_bit_cast(typename T::v8, xv), __builtin_bit_cast(typename T::v8, cols8[tc]), acc[tc]);
    }
    // lane holds Z[m = 4g + e][j + tc]
    __syncthreads();
    if (wave >= 2) {
#pragma unroll
      for (int tc = 0; tc < 8; ++tc)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((wave - 2) * 32 + tc * 4 + e) * 64 + lane] = acc[tc][e];
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
      for (int tc = 0; tc < 8; ++tc)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tc][e] += red[(wave * 32 + tc * 4 + e) * 64 + lane];
    }
    __syncthreads();
    if (wave == 1) {
#pragma unroll
      for (int tc = 0; tc < 8; ++tc)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(tc * 4 + e) * 64 + lane] = acc[tc][e];
    }
    __syncthreads();
    if (wave == 0 && j < r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = 4 * g + e;
        if (m >= M) continue;
        float v[8];
#pragma unroll
        for (int tc = 0; tc < 8; ++tc) v[tc] = acc[tc][e] + red[(tc * 4 + e) * 64 + lane];
        float* o = zpart + (split * M + m) * r + j;
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
}

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
template <class T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemv_kernel(const uint16_t* __restrict__ X, int64_t M, NF4View W, int64_t K,
                                                   int64_t N, int64_t rpw, int64_t slabs, float* __restrict__ part,
                                                   const uint16_t* __restrict__ A, int64_t r,
                                                   float* __restrict__ zpart) {
  __shared__ float q2t[256];
  __shared__ __attribute__((aligned(16))) char tabs[kGvWaves * 2 * kGvTabBytes];
  const int t = threadIdx.x, lane = t & 63, q = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t splits = (K + kGvWaves * rpw - 1) / (kGvWaves * rpw);
  if (blockIdx.x >= slabs * splits) {
    // the last `splits` workgroups: Z partials over the same row ranges
    gemv_zpart<T>(X, M, K, rpw, A, r, zpart, blockIdx.x - slabs * splits, reinterpret_cast<float*>(tabs));
    return;
  }
  q2t[t] = q2_value(t - 128);
  const int64_t slab = blockIdx.x % slabs, split = blockIdx.x / slabs;
  const int64_t n0 = slab * kGvCols;
  const int64_t kw0 = (split * kGvWaves + wave) * rpw;
  const int64_t kend = min(K, kw0 + rpw);   // this wave's rows; nothing past them is fetched
  const int64_t rows = kend > kw0 ? kend - kw0 : 0;
  const int64_t P = K * N;
  // descriptors over this wave's rows only: rows past kend read zeros, and the
  // step advance is a scalar offset (N is a multiple of 64)
  const int64_t kb0 = kend > kw0 ? kw0 : 0;
  const Rsrc rc = make_rsrc(W.codes + kb0 * N / 2, rows * N / 2);
  // a state without a second level stores one fp32 scale per block: â = that
  const bool single = W.absmax != nullptr;
  const Rsrc rq = single ? make_rsrc(nullptr, 0) : make_rsrc(W.qabsmax + kb0 * N / 64, rows * N / 64);
  const Rsrc rs = single ? make_rsrc(W.absmax, ((P + 63) / 64) * 4) : make_rsrc(W.absmax2, ((P + 16383) / 16384) * 4);
  const int s_shift = single ? 6 : 14;
  const Rsrc rx = make_rsrc(X, M * K * 2);
  const float off = single ? 0.0f : W.offset[0];
  const int64_t n = n0 + 16 * q;
  const bool n_ok = n < N;
  const int blk = q >> 2;
  char* my_tabs = tabs + wave * 2 * kGvTabBytes;
  uint32_t voff_w[8], voff_q[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) voff_w[i] = n_ok ? static_cast<uint32_t>(((8 * g + i) * N + n) >> 1) : kMasked;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t nb = n0 + 64 * (2 * (lane & 1) + u);
    voff_q[u] = nb < N ? static_cast<uint32_t>(((lane >> 1) * N + nb) >> 6) : kMasked;
  }
  const uint32_t voff_x = q < M ? static_cast<uint32_t>((q * K + kw0 + 8 * g) * 2) : kMasked;

  auto load = [&](GvStep& S, int64_t kk) {
    const uint32_t sw = static_cast<uint32_t>((kk * N) >> 1);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      S.w[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, voff_w[i], sw, 0));
    // zero activations past this wave's rows (their codes read as 0, a finite weight)
    S.x = ld_b128(rx, (kw0 + kk + 8 * g < kend) ? voff_x + static_cast<uint32_t>(kk * 2) : kMasked);
    const uint32_t sq = static_cast<uint32_t>((kk * N) >> 6);
    const uint32_t kt = static_cast<uint32_t>(kw0 + kk + (lane >> 1));
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      S.q[u] = static_cast<int>(static_cast<int8_t>(__builtin_amdgcn_raw_buffer_load_b8(rq, voff_q[u], sq, 0)));
      const uint32_t nb = static_cast<uint32_t>(n0 + 64 * (2 * (lane & 1) + u));
      const bool ok = kt < kend && nb < N;
      S.s2[u] = ld_f32(rs, ok ? ((kt * static_cast<uint32_t>(N) + nb) >> s_shift) * 4 : kMasked);
    }
  };
  auto build = [&](const GvStep& S, int buf) {
    char* tb = my_tabs + buf * kGvTabBytes + gv_row(lane >> 1) + 64 * (lane & 1);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      write_block_table<T>(reinterpret_cast<uint16_t*>(tb + 32 * u),
                        single ? S.s2[u] : __fadd_rn(__fmul_rn(q2t[S.q[u] + 128], S.s2[u]), off));
  };

  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0, 0, 0, 0};
  __syncthreads();  // q2t
  // kGvDepth steps of loads in flight per wave: set u holds step D j + u and
  // is refilled with step D (j+1) + u as soon as it has been decoded.  Each
  // wave's tables live in its own LDS ring, so no workgroup barrier is needed
  // (LDS operations of one wave complete in order).
  GvStep R[kGvDepth];
#pragma unroll
  for (int u = 0; u < kGvDepth; ++u) load(R[u], 32 * u);
  build(R[0], 0);
  for (int64_t kk = 0; kk < rpw; kk += 32 * kGvDepth) {
#pragma unroll
    for (int u = 0; u < kGvDepth; ++u) {
      const int64_t ks = kk + 32 * u;
      if (ks >= rpw) break;
      const int buf = static_cast<int>((ks >> 5) & 1);   // tables alternate per 32-row step
      // table of row 8g + i (i < 8) for this lane's block: tb + 128 i
      const char* tb = my_tabs + buf * kGvTabBytes + gv_row(8 * g) + 32 * blk;
      // doubled codes: byte b of ev = 2 * code of column 2b, of od = 2 * code of
      // column 2b + 1 (x word: columns 0..7, y word: columns 8..15)
      uint32_t ev[8][2], od[8][2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ev[i][0] = (R[u].w[i].x >> 3) & 0x1e1e1e1eu;
        od[i][0] = (R[u].w[i].x << 1) & 0x1e1e1e1eu;
        ev[i][1] = (R[u].w[i].y >> 3) & 0x1e1e1e1eu;
        od[i][1] = (R[u].w[i].y << 1) & 0x1e1e1e1eu;
      }
      const uint32_t tbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tb));
      const typename T::v8 xf = __builtin_bit_cast(typename T::v8, R[u].x);
#pragma unroll
      for (int tile = 0; tile < 16; ++tile) {
        const int h = tile >> 3, col = tile & 7;
        uint32_t fw[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t a0 = add_byte(tbase, (col & 1) ? od[2 * p][h] : ev[2 * p][h], col >> 1);
          const uint32_t a1 = add_byte(tbase, (col & 1) ? od[2 * p + 1][h] : ev[2 * p + 1][h], col >> 1);
          const uint32_t lo = lds_u16(a0 + 2 * p * 128);
          const uint32_t hi = lds_u16(a1 + (2 * p + 1) * 128);
          fw[p] = perm(hi, lo, 0x05040100u);
        }
        acc[tile] = T::mfma16(xf, __builtin_bit_cast(typename T::v8, make_uint4(fw[0], fw[1], fw[2], fw[3])), acc[tile]);
      }
      if (ks + 32 < rpw) build(R[(u + 1) % kGvDepth], buf ^ 1);
      load(R[u], ks + 32 * kGvDepth);   // past the k-range: masked, reads zeros
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
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

// Y = sum_s part[s] + c Z B for M <= 16: one wave per 128 columns and row
// phase e (blockIdx.y); lane (q, g) owns columns n0+8q..+7 and row 4g+e.
// The LoRA product runs on MFMA with B transposed in registers (every phase
// computes it; only row 4g+e is kept).  Z = RNE_bf16(sum_s zpart[s]) in a
// fixed order; workgroup (0, 0) writes it.  The split loops request 8
// partials at a time before adding them in order.
template <class T>
__global__ __launch_bounds__(64) void gemv_finish_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                         int64_t N, const float* __restrict__ zpart,
                                                         uint16_t* __restrict__ Z, const uint16_t* __restrict__ B,
                                                         int64_t r, float c, uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x, q = lane & 15, g = lane >> 4;
  const int e = blockIdx.y;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 128, n = n0 + 8 * q;
  const bool n_ok = n < N;
  const Rsrc rb = make_rsrc(B, r * N * 2);
  const Rsrc rzp = make_rsrc(zpart, static_cast<int64_t>(splits) * M * r * 4);
  const Rsrc rp = make_rsrc(part, static_cast<int64_t>(splits) * M * N * 4);
  f32x4 accl[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) accl[i] = f32x4{0, 0, 0, 0};
  for (int64_t j0 = 0; j0 < r; j0 += 32) {
    const int64_t jb = j0 + 8 * g;
    const bool zok = q < M && jb < r;
    uint4 rows8[8], cols8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rows8[i] = ld_b128(rb, (jb + i < r && n_ok) ? static_cast<uint32_t>(((jb + i) * N + n) * 2) : kMasked);
    float zs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) zs[i] = 0.0f;
    for (int s0 = 0; s0 < splits; s0 += 8) {
      uint4 za[8], zb[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t off = (zok && s0 + k < splits) ? static_cast<uint32_t>((((s0 + k) * M + q) * r + jb) * 4) : kMasked;
        za[k] = ld_b128(rzp, off);
        zb[k] = ld_b128(rzp, off == kMasked ? kMasked : off + 16);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (s0 + k >= splits) break;
        zs[0] += __builtin_bit_cast(float, za[k].x); zs[1] += __builtin_bit_cast(float, za[k].y);
        zs[2] += __builtin_bit_cast(float, za[k].z); zs[3] += __builtin_bit_cast(float, za[k].w);
        zs[4] += __builtin_bit_cast(float, zb[k].x); zs[5] += __builtin_bit_cast(float, zb[k].y);
        zs[6] += __builtin_bit_cast(float, zb[k].z); zs[7] += __builtin_bit_cast(float, zb[k].w);
      }
    }
    uint4 zv = make_uint4(0, 0, 0, 0);
    if (zok) {
      zv = make_uint4(T::pack2(zs[0], zs[1]), T::pack2(zs[2], zs[3]), T::pack2(zs[4], zs[5]),
                      T::pack2(zs[6], zs[7]));
      if (blockIdx.x == 0 && e == 0) *reinterpret_cast<uint4*>(Z + q * r + jb) = zv;
    }
    transpose8x8_bf16(rows8, cols8);
#pragma unroll
    for (int tc = 0; tc < 8; ++tc)
      accl[tc] = T::mfma16(__builtin_bit_cast(typename T::v8, zv), __builtin_bit_cast(typename T::v8, cols8[tc]), accl[tc]);
  }
  const int64_t m = 4 * g + e;
  if (m >= M || !n_ok) return;
  float v[8];
#pragma unroll
  for (int tc = 0; tc < 8; ++tc) v[tc] = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += 8) {
    uint4 pa[8], pb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t off = (s0 + k < splits) ? static_cast<uint32_t>((((s0 + k) * M + m) * N + n) * 4) : kMasked;
      pa[k] = ld_b128(rp, off);
      pb[k] = ld_b128(rp, off == kMasked ? kMasked : off + 16);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (s0 + k >= splits) break;
      v[0] += __builtin_bit_cast(float, pa[k].x); v[1] += __builtin_bit_cast(float, pa[k].y);
      v[2] += __builtin_bit_cast(float, pa[k].z); v[3] += __builtin_bit_cast(float, pa[k].w);
      v[4] += __builtin_bit_cast(float, pb[k].x); v[5] += __builtin_bit_cast(float, pb[k].y);
      v[6] += __builtin_bit_cast(float, pb[k].z); v[7] += __builtin_bit_cast(float, pb[k].w);
    }
  }
  uint4 o;
  o.x = T::pack2(v[0] + c * accl[0][e], v[1] + c * accl[1][e]);
  o.y = T::pack2(v[2] + c * accl[2][e], v[3] + c * accl[3][e]);
  o.z = T::pack2(v[4] + c * accl[4][e], v[5] + c * accl[5][e]);
  o.w = T::pack2(v[6] + c * accl[6][e], v[7] + c * accl[7][e]);
  *reinterpret_cast<uint4*>(Y + m * N + n) = o;
}

}  // namespace

#ifndef QN_GV_WAVES
#define QN_GV_WAVES 1400
#endif

void plan_gemv(int64_t M, int64_t K, int64_t N, int64_t r, SkinnyPlan* p_) {
  SkinnyPlan& p = *p_;
  // 4 waves x rows_per_wave rows per workgroup, ~1400 waves in total
  const int64_t slabs = cdiv(N, kGvCols);
  const int64_t groups = cdiv(QN_GV_WAVES, slabs * kGvWaves);
  int64_t rpw = round_up(cdiv(K, groups * kGvWaves), 32);
  if (rpw < 64) rpw = 64;
  p.gv_rows_per_wave = rpw;
  p.gv_splits = cdiv(K, rpw * kGvWaves);
  p.gv_part = round_up(p.gv_splits * M * N * 4, 256);
  p.gv_zpart = round_up(p.gv_splits * M * r * 4, 256);
}

hipError_t launch_gemv(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W, const uint16_t* A,
                       const uint16_t* B, float c, uint16_t* Y, uint16_t* Z, const SkinnyPlan& p, void* part_ws,
                       hipStream_t stream, int dtype) {
  const int64_t slabs = cdiv(N, kGvCols);
  float* part = static_cast<float*>(part_ws);
  float* zpart = reinterpret_cast<float*>(static_cast<char*>(part_ws) + p.gv_part);
  Timer tm(QK_FWD_GEMV, stream);
  hipLaunchKernelGGL(dtype == kDtypeF16 ? gemv_kernel<F16> : gemv_kernel<Bf16>, dim3(static_cast<unsigned>((slabs + 1) * p.gv_splits)), dim3(kGvWaves * 64), 0,
                     stream, X, M, W, K, N, p.gv_rows_per_wave, slabs, part, A, r, zpart);
  tm.stop();
  Timer te(QK_REDUCE, stream);
  const unsigned phases = static_cast<unsigned>(M < 4 ? M : 4);   // rows 4g + e, e < phases
  hipLaunchKernelGGL(dtype == kDtypeF16 ? gemv_finish_kernel<F16> : gemv_finish_kernel<Bf16>, dim3(static_cast<unsigned>(cdiv(N, 128)), phases), dim3(64), 0, stream,
                     static_cast<const float*>(part), static_cast<int>(p.gv_splits), M, N,
                     static_cast<const float*>(zpart), Z, B, r, c, Y);
  te.stop();
  return hipGetLastError();
}

}  // namespace qn
