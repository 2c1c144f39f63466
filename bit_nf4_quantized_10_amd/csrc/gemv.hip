// Small-M forward (M <= 16) for gfx950: Y = X Ŵ + c Z B as a dequant-GEMV
// (page "QLoRA：冻结的 4-bit 权重怎样参与一次微调", section "量化基座与可训练支路怎样相加";
// the decode is the one of section "Double Quantization 压缩的是 Scale").
//
// Workgroup (4 waves) = two neighbouring 128-column strips x two row ranges;
// each wave streams one strip over its own contiguous range of 32-row steps,
// so the two waves of a row range read the two halves of every 128-byte line
// at about the same time.  Lane (q, g) owns columns n0 + 8q .. +7 and rows
// 8g .. 8g+7 of each step.  Per step a wave stages its codes in LDS (16-byte
// loads of whole 64-byte row pieces), builds the step's 64 block tables
// (32 rows x 2 blocks, 16 RNE(fl32(C[j] * â)) each; one per lane) and
// decodes by table lookups: one byte-select add and one 16-bit LDS read per
// weight, pairs packed with v_perm; column t of the lane feeds the MFMA of
// tile t with the zero-padded 16-row activation block.  A lookup instruction
// touches eight tables that together fill the 64 LDS banks once.  Three
// steps of loads are in flight per wave (per-wave buffer descriptors, so rows
// past the wave's range read as zeros and meet zero activations).  The two
// row ranges of a strip are added in LDS in a fixed order; the split-K
// partials and the LoRA term are added by gemv_finish_kernel.
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
constexpr int kGvCols = 128;    // columns per workgroup strip (8 per lane)
// Per wave, for one 32-row step: the 64 block tables (32 rows x 2 blocks, 16
// bf16 each) and the step's codes (32 rows x 64 bytes).  The table of row
// 8g + i, block b sits at byte (4i + g) * 64 + 32b, and code row 8g + i at
// (4i + g) * 64, so the 64 lanes of one lookup (rows 8g + i, g < 4, both
// blocks) or of one code read cover the 64 LDS banks once.
constexpr int kGvTabBytes = 32 * 2 * 32;
constexpr int kGvStageBytes = 32 * 64;
constexpr int kGvWaveLds = kGvTabBytes + kGvStageBytes;
#ifndef QN_GV_DEPTH
#define QN_GV_DEPTH 3
#endif
constexpr int kGvDepth = QN_GV_DEPTH;   // 32-row steps of code loads in flight per wave
__device__ __forceinline__ int gv_pos(int row) { return 4 * (row & 7) + (row >> 3); }   // row 8g + i -> 4i + g

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
  uint4 c[2];   // 16 code bytes of one row per load (row order of the LDS stage)
  uint4 x;      // activation fragment X[q][k + 8g .. k + 8g + 7]
  int q;        // second-level code of the table this lane builds
  float s2;
};

// Workgroup (4 waves) = one 128-column strip; wave w covers rows
// [(split*4 + w) * rpw, +rpw) in steps of 32.  Lane (q, g): columns
// n0 + 8q .. +7, rows 8g .. 8g+7 of each step.  Per step a wave copies its
// 2 KB of codes (two 16-byte loads per lane, whole 64-byte row pieces) into
// its LDS stage, each lane builds one of the step's 64 block tables, and the
// lane reads its eight 4-byte code words back in MFMA order.  Each weight is
// one byte-select add and one 16-bit table lookup, pairs packed with v_perm;
// column t of the lane feeds the MFMA of tile t.  part[split][m][n] = sum of
// the 4 waves (fixed order).
template <class T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void gemv_kernel(const uint16_t* __restrict__ X, int64_t M, NF4View W, int64_t K,
                                                   int64_t N, int64_t rpw, int64_t pairs, float* __restrict__ part,
                                                   const uint16_t* __restrict__ A, int64_t r,
                                                   float* __restrict__ zpart) {
  __shared__ float q2t[256];
  __shared__ __attribute__((aligned(16))) char lds[kGvWaves * kGvWaveLds];
  const int t = threadIdx.x, lane = t & 63, q = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t splits = (K + 2 * rpw - 1) / (2 * rpw);
  const int64_t gv = pairs * splits;
  if (blockIdx.x >= gv) {
    // the last `splits` workgroups: Z partials over the same row ranges
    gemv_zpart<T>(X, M, K, rpw / 2, A, r, zpart, blockIdx.x - gv, reinterpret_cast<float*>(lds));
    return;
  }
  q2t[t] = q2_value(t - 128);
  // Workgroup ids are dealt to the 8 XCDs in turn.  Logical workgroup L
  // (pair L % pairs of row range L / pairs) is placed so that each XCD runs a
  // contiguous run of L: neighbouring pairs of one row range share an XCD,
  // whose L2 then fetches the lines of int8 scale codes they share once.
  const int64_t per = gv / 8, rem = gv % 8, xcd = blockIdx.x % 8;
  const int64_t L = xcd * per + min(xcd, rem) + blockIdx.x / 8;
  const int64_t split = L / pairs;
  const int64_t n0 = (2 * (L % pairs) + (wave & 1)) * kGvCols;
  const int64_t kw0 = (split * 2 + (wave >> 1)) * rpw;
  const int64_t kend = min(K, kw0 + rpw);   // this wave's rows; nothing past them is fetched
  const int64_t rows = kend > kw0 ? kend - kw0 : 0;
  const int64_t kb0 = kend > kw0 ? kw0 : 0;
  // descriptors over this wave's rows only: rows past kend read zeros
  const Rsrc rc = make_rsrc(W.codes + kb0 * N / 2, rows * N / 2);
  // a state without a second level stores one fp32 scale per block: â = that
  const bool single = W.absmax != nullptr;
  const int64_t P = K * N;
  const Rsrc rq = single ? make_rsrc(nullptr, 0) : make_rsrc(W.qabsmax + kb0 * N / 64, rows * N / 64);
  const Rsrc rs = single ? make_rsrc(W.absmax, ((P + 63) / 64) * 4) : make_rsrc(W.absmax2, ((P + 16383) / 16384) * 4);
  const int s_shift = single ? 6 : 14;
  const Rsrc rx = make_rsrc(X, M * K * 2);
  const float off = single ? 0.0f : W.offset[0];
  char* tabs = lds + wave * kGvWaveLds;
  char* stage = tabs + kGvTabBytes;

  // code load j, lane l: stage position p = 16j + l/4 (row 8(p & 3) + p/4),
  // bytes 16(l & 3) .. +15 of that row's 64-byte piece
  uint32_t voff_c[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = 16 * j + (lane >> 2), row = 8 * (p & 3) + (p >> 2);
    const int64_t cb = n0 + 32 * (lane & 3);
    voff_c[j] = cb < N ? static_cast<uint32_t>((row * N + cb) >> 1) : kMasked;
  }
  // the table this lane builds: row trow, block tblk of the step
  const int trow = lane >> 1, tblk = lane & 1;
  const int64_t tcol = n0 + 64 * tblk;
  const uint32_t voff_q = tcol < N ? static_cast<uint32_t>((trow * N + tcol) >> 6) : kMasked;
  char* my_tab = tabs + gv_pos(trow) * 64 + 32 * tblk;
  const uint32_t voff_x = q < M ? static_cast<uint32_t>((q * K + kw0 + 8 * g) * 2) : kMasked;

  auto load = [&](GvStep& S, int64_t kk) {
    // offsets past this wave's rows (or masked) are out of the descriptor: zeros
    const uint32_t sw = static_cast<uint32_t>((kk * N) >> 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) S.c[j] = ld_b128(rc, voff_c[j] + sw);
    // zero activations past this wave's rows (their codes read as 0, a finite weight)
    S.x = ld_b128(rx, (kw0 + kk + 8 * g < kend) ? voff_x + static_cast<uint32_t>(kk * 2) : kMasked);
    const int64_t kt = kw0 + kk + trow;
    const bool ok = kt < kend && tcol < N;
    S.q = ld_i8(rq, ok ? voff_q + static_cast<uint32_t>((kk * N) >> 6) : kMasked);
    S.s2 = ld_f32(rs, ok ? static_cast<uint32_t>(((kt * N + tcol) >> s_shift) * 4) : kMasked);
  };

  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0, 0, 0, 0};
  __syncthreads();  // q2t
  // kGvDepth steps of loads in flight per wave: set u holds step D j + u and
  // is refilled with step D (j+1) + u as soon as it has been staged.  Each
  // wave's stage and tables are its own, so no workgroup barrier is needed
  // (LDS operations of one wave complete in order).
  GvStep R[kGvDepth];
#pragma unroll
  for (int u = 0; u < kGvDepth; ++u) load(R[u], 32 * u);
  // lookups of row 8g + i go to tbase + 256 i + 2 code
  const uint32_t tbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tabs + g * 64 + 32 * (q >> 3)));
  for (int64_t kk = 0; kk < rpw; kk += 32 * kGvDepth) {
#pragma unroll
    for (int u = 0; u < kGvDepth; ++u) {
      const int64_t ks = kk + 32 * u;
      if (ks >= rpw) break;
#pragma unroll
      for (int j = 0; j < 2; ++j) *reinterpret_cast<uint4*>(stage + j * 1024 + lane * 16) = R[u].c[j];
      write_block_table<T>(reinterpret_cast<uint16_t*>(my_tab),
                           single ? R[u].s2 : __fadd_rn(__fmul_rn(q2t[R[u].q + 128], R[u].s2), off));
      const typename T::v8 xf = __builtin_bit_cast(typename T::v8, R[u].x);
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = *reinterpret_cast<const uint32_t*>(stage + (4 * i + g) * 64 + 4 * q);
      load(R[u], ks + 32 * kGvDepth);   // past the k-range: masked, reads zeros
      // doubled codes: byte b of ev = 2 * code of column 2b, of od = 2 * code
      // of column 2b + 1
      uint32_t ev[8], od[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ev[i] = (w[i] >> 3) & 0x1e1e1e1eu;
        od[i] = (w[i] << 1) & 0x1e1e1e1eu;
      }
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) {
        uint32_t fw[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t a0 = add_byte(tbase, (tile & 1) ? od[2 * p] : ev[2 * p], tile >> 1);
          const uint32_t a1 = add_byte(tbase, (tile & 1) ? od[2 * p + 1] : ev[2 * p + 1], tile >> 1);
          const uint32_t lo = lds_u16(a0 + 2 * p * 256);
          const uint32_t hi = lds_u16(a1 + (2 * p + 1) * 256);
          fw[p] = perm(hi, lo, 0x05040100u);
        }
        acc[tile] = T::mfma16(xf, __builtin_bit_cast(typename T::v8, make_uint4(fw[0], fw[1], fw[2], fw[3])), acc[tile]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // lane holds Y[m = 4g+e][n0 + 8q + tile]; the two row ranges of a strip
  // are added in a fixed order: wave w (w < 2) + wave w + 2
  float* red = reinterpret_cast<float*>(lds);   // 2 waves x 32 floats x 64 lanes = 16 KB
  if (wave >= 2) {
#pragma unroll
    for (int tile = 0; tile < 8; ++tile)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave - 2) * 32 + tile * 4 + e) * 64 + lane] = acc[tile][e];
  }
  __syncthreads();
  if (wave < 2) {
    float* out = part + split * M * N;
    const int64_t n = n0 + 8 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t m = 4 * g + e;
      float v[8];
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) v[tile] = acc[tile][e] + red[(wave * 32 + tile * 4 + e) * 64 + lane];
      if (m < M && n < N) {
        *reinterpret_cast<float4*>(out + m * N + n) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(out + m * N + n + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
}

// Y = sum_s part[s] + c Z B for M <= 16.  Workgroup (4 waves) = 512
// columns and row phase e (blockIdx.y); lane (q, g) of wave w owns columns
// n0 + 128w + 8q .. +7 and row 4g + e.  A workgroup requests at its start
// the first 8 split partials of its outputs, the first 64 rows of B and the
// first 8 split partials of Z, so that the common case (splits <= 8,
// M r <= 1024, r <= 64) waits for memory once.  The workgroup forms
// Z = RNE_T(sum_s zpart[s]) in LDS, and workgroup (0, 0) writes it out; the
// LoRA product runs on MFMA with Z from LDS and B transposed in registers
// (every phase computes all 16 rows; only row 4g + e is kept).  Partials past
// the last split read as +0 and are added all the same: the running sums
// start at +0 and can never be -0, so adding +0 leaves them unchanged.
constexpr int kFinCols = 512;
__device__ __forceinline__ void fin_add4(float (&s)[4], const uint4 (&v)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    s[0] += __builtin_bit_cast(float, v[k].x); s[1] += __builtin_bit_cast(float, v[k].y);
    s[2] += __builtin_bit_cast(float, v[k].z); s[3] += __builtin_bit_cast(float, v[k].w);
  }
}
__device__ __forceinline__ void fin_add8(float (&s)[8], const uint4 (&a)[8], const uint4 (&b)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    s[0] += __builtin_bit_cast(float, a[k].x); s[1] += __builtin_bit_cast(float, a[k].y);
    s[2] += __builtin_bit_cast(float, a[k].z); s[3] += __builtin_bit_cast(float, a[k].w);
    s[4] += __builtin_bit_cast(float, b[k].x); s[5] += __builtin_bit_cast(float, b[k].y);
    s[6] += __builtin_bit_cast(float, b[k].z); s[7] += __builtin_bit_cast(float, b[k].w);
  }
}
template <class T>
__global__ __launch_bounds__(256) void gemv_finish_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                          int64_t N, const float* __restrict__ zpart,
                                                          uint16_t* __restrict__ Z, const uint16_t* __restrict__ B,
                                                          int64_t r, float c, uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint16_t zl[16 * 256];   // Z, M x r (M <= 16, r <= 256)
  const int t = threadIdx.x, lane = t & 63, q = lane & 15, g = lane >> 4, wave = t >> 6;
  const int e = blockIdx.y;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kFinCols + 128 * wave + 8 * q;
  const bool n_ok = n < N;
  const int64_t m = 4 * g + e;
  const bool out_ok = m < M && n_ok;
  const int64_t MR = M * r;
  const Rsrc rb = make_rsrc(B, r * N * 2);
  const Rsrc rzp = make_rsrc(zpart, static_cast<int64_t>(splits) * MR * 4);
  const Rsrc rp = make_rsrc(part, static_cast<int64_t>(splits) * M * N * 4);
  auto load_b = [&](int64_t j0, uint4 (&rows8)[8]) {
    const int64_t jb = j0 + 8 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rows8[i] = ld_b128(rb, (jb + i < r && n_ok) ? static_cast<uint32_t>(((jb + i) * N + n) * 2) : kMasked);
  };
  auto load_part = [&](int s0, uint4 (&pa)[8], uint4 (&pb)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t off = (out_ok && s0 + k < splits) ? static_cast<uint32_t>((((s0 + k) * M + m) * N + n) * 4) : kMasked;
      pa[k] = ld_b128(rp, off);
      pb[k] = ld_b128(rp, off == kMasked ? kMasked : off + 16);
    }
  };
  // thread t sums elements idx .. idx+3 of the row-major M x r matrix Z
  // (r % 8 == 0, so a group of 4 never leaves its row)
  auto load_z = [&](int s0, int64_t idx, uint4 (&za)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      za[k] = ld_b128(rzp, (idx < MR && s0 + k < splits) ? static_cast<uint32_t>(((s0 + k) * MR + idx) * 4) : kMasked);
  };
  auto store_z = [&](int64_t idx, const float (&zs)[4]) {
    if (idx >= MR) return;
    const uint2 zv = make_uint2(T::pack2(zs[0], zs[1]), T::pack2(zs[2], zs[3]));
    *reinterpret_cast<uint2*>(zl + idx) = zv;
    if (blockIdx.x == 0 && e == 0) *reinterpret_cast<uint2*>(Z + idx) = zv;
  };
  uint4 pa[8], pb[8], b0[8], b1[8], za[8];
  load_part(0, pa, pb);
  load_b(0, b0);
  load_b(32, b1);
  load_z(0, 4 * t, za);
  {
    float zs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    fin_add4(zs, za);
    for (int s0 = 8; s0 < splits; s0 += 8) {
      load_z(s0, 4 * t, za);
      fin_add4(zs, za);
    }
    store_z(4 * t, zs);
  }
  for (int64_t base = 1024; base < MR; base += 1024) {
    float zs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < splits; s0 += 8) {
      load_z(s0, base + 4 * t, za);
      fin_add4(zs, za);
    }
    store_z(base + 4 * t, zs);
  }
  __syncthreads();
  f32x4 accl[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) accl[i] = f32x4{0, 0, 0, 0};
  auto lora_step = [&](int64_t j0, const uint4 (&rows8)[8]) {
    const int64_t jb = j0 + 8 * g;
    const uint4 zv = (q < M && jb < r) ? *reinterpret_cast<const uint4*>(zl + q * r + jb) : make_uint4(0, 0, 0, 0);
    uint4 cols8[8];
    transpose8x8_bf16(rows8, cols8);
#pragma unroll
    for (int tc = 0; tc < 8; ++tc)
      accl[tc] = T::mfma16(__builtin_bit_cast(typename T::v8, zv), __builtin_bit_cast(typename T::v8, cols8[tc]), accl[tc]);
  };
  lora_step(0, b0);
  if (r > 32) lora_step(32, b1);
  for (int64_t j0 = 64; j0 < r; j0 += 32) {
    load_b(j0, b0);
    lora_step(j0, b0);
  }
  if (!out_ok) return;
  float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  fin_add8(v, pa, pb);
  for (int s0 = 8; s0 < splits; s0 += 8) {
    load_part(s0, pa, pb);
    fin_add8(v, pa, pb);
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
#define QN_GV_WAVES 2752
#endif

void plan_gemv(int64_t M, int64_t K, int64_t N, int64_t r, SkinnyPlan* p_) {
  SkinnyPlan& p = *p_;
  // workgroup = 2 strips x 2 row ranges of rows_per_wave rows, about
  // QN_GV_WAVES waves in total; rows_per_wave is a multiple of 64 so that the Z
  // workgroups' four waves split a row range in 32-row steps
  const int64_t pairs = cdiv(N, 2 * kGvCols);
  const int64_t groups = cdiv(QN_GV_WAVES, pairs * kGvWaves);
  int64_t rpw = round_up(cdiv(K, groups * 2), 64);
  p.gv_rows_per_wave = rpw;
  p.gv_splits = cdiv(K, 2 * rpw);
  p.gv_part = round_up(p.gv_splits * M * N * 4, 256);
  p.gv_zpart = round_up(p.gv_splits * M * r * 4, 256);
}

hipError_t launch_gemv(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W, const uint16_t* A,
                       const uint16_t* B, float c, uint16_t* Y, uint16_t* Z, const SkinnyPlan& p, void* part_ws,
                       hipStream_t stream, int dtype) {
  const int64_t pairs = cdiv(N, 2 * kGvCols);
  float* part = static_cast<float*>(part_ws);
  float* zpart = reinterpret_cast<float*>(static_cast<char*>(part_ws) + p.gv_part);
  Timer tm(QK_FWD_GEMV, stream);
  hipLaunchKernelGGL(dtype == kDtypeF16 ? gemv_kernel<F16> : gemv_kernel<Bf16>, dim3(static_cast<unsigned>((pairs + 1) * p.gv_splits)), dim3(kGvWaves * 64), 0,
                     stream, X, M, W, K, N, p.gv_rows_per_wave, pairs, part, A, r, zpart);
  tm.stop();
  Timer te(QK_REDUCE, stream);
  const unsigned phases = static_cast<unsigned>(M < 4 ? M : 4);   // rows 4g + e, e < phases
  hipLaunchKernelGGL(dtype == kDtypeF16 ? gemv_finish_kernel<F16> : gemv_finish_kernel<Bf16>, dim3(static_cast<unsigned>(cdiv(N, kFinCols)), phases), dim3(256), 0, stream,
                     static_cast<const float*>(part), static_cast<int>(p.gv_splits), M, N,
                     static_cast<const float*>(zpart), Z, B, r, c, Y);
  te.stop();
  return hipGetLastError();
}

}  // namespace qn
