// Large-M GEMM kernels for gfx950: the forward Y = X Ŵ + c Z B and the
// backward dX = G Ŵᵀ + dZ Aᵀ (page "QLoRA：冻结的 4-bit 权重怎样参与一次微调",
// sections "量化基座与可训练支路怎样相加" and "冻结权重为什么仍然需要输入梯度").
//
// Both kernels: workgroup of 256 threads (4 waves, 2 x 2), output tile
// 256 x 256, each wave 128 x 128 as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16
// (256 fp32 accumulators per lane in AGPRs, one wave per SIMD).  The LoRA
// term is r more reduction steps over (Z, (c B)ᵀ) or (dZ, A) after the main
// loop; the bf16 tile is then stored through LDS as whole rows.
//
// qlora_big_kernel (17 <= M < 192) decodes the packed weight inside its
// reduction loop.  Per 64-element stage the workgroup
//   - copies the activation tile of stage s+1 from global memory straight into
//     LDS (buffer loads with the LDS destination, no registers involved);
//   - loads the code words and block scales of stage s+2 into registers;
//   - builds the bf16 block tables of stage s+1 (16 entries RNE(fl32(C[j]*â))
//     per 64-weight block row) and decodes stage s+1 into the other weight
//     buffer by table lookups (no per-weight multiply or conversion);
//   - runs the 64 MFMAs of stage s;
// then waits for its loads and synchronises once.  LDS layout of one operand
// stage: 256 rows x 64 bf16 (128 bytes per row), the eight 16-byte chunks of
// row r stored at chunk ^ ((r ^ r >> 3) & 7), which keeps the fragment reads
// and the decoder's writes free of bank conflicts per 8 lanes.
//  - forward weight (reduction over k, codes packed along n): thread (rg, cg)
//    owns k-rows 8rg..8rg+7 and columns 8cg..8cg+7 of the stage; it builds the
//    table of one (row, block) pair that the 8 threads of its group share
//    and writes each column's 8 k-values as one chunk;
//  - backward weight (reduction over n, the packed direction): thread t owns
//    k-row t and the stage's 64 n, exactly one block and one table.
// Rows at or past K get an all-zero table and the matching activation
// chunks are masked, so tails add exact zeros.
//
// qlora_dense_kernel (M >= 192) reads a weight dequantized beforehand to bf16
// (bit-identical to the fused decode) and streams both operands through two
// LDS slots of 64-element stages, whole cache lines per copy (see Dense).
//
// Every global load is a raw buffer load, so masked lanes need no branches:
// a lane whose row, column or reduction index lies outside its operand
// (tails, and the prefetches that run past the last stage) gets a per-lane
// offset past the buffer's size, whatever the scalar stage offset added.
// The MFMA is issued as D = Ŵ-fragment x activation-fragment, so each lane
// holds 4 consecutive output columns of one output row.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace qn {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kTileBytes = 256 * 128;
constexpr int kTabBytes = 256 * 32;
constexpr int kOffA = 0;                           // 2 stages of activation tiles
constexpr int kOffB = 2 * kTileBytes;              // 2 stages of weight tiles
constexpr int kOffT = 4 * kTileBytes;              // 2 stages of block tables
constexpr int kOffQ = kOffT + 2 * kTabBytes;       // fl32(q/127) table
constexpr int kLdsBytes = kOffQ + 256 * 4;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }


struct BigArgs {
  const uint16_t* act;     // X (forward) or G (backward): rows m, reduction contiguous
  int64_t act_ld;          // K (forward) or N (backward)
  NF4View W;
  const uint16_t* ext_a;   // Z (forward) or dZ (backward), M x r bf16
  const uint16_t* ext_b;   // (c B)ᵀ in bf16 (forward, N x r) or A (backward, K x r)
  uint16_t* out;           // Y (M x N) or dX (M x K)
  int64_t M, K, N, r;
  const uint16_t* wdense;  // dense path: Ŵᵀ (N x K, forward) or Ŵ (K x N, backward), bf16
  // Forward over the concatenated columns of a group of linears sharing X:
  // ext_a is then M x (ngroups r) (row stride ext_a_ld) and output columns
  // c >= gend[i] (member i+1 onwards) take their Z from column block i+1.
  // Zero / unset: one linear, ext_a row stride r.
  int64_t ext_a_ld;
  int ngroups;
  int64_t gend[kMaxGroupMembers];
  // Split-K (part non-null): workgroup z reduces elements [z k_per,
  // (z+1) k_per) and writes its fp32 tile to part + z M cols (row-major);
  // only z = 0 adds the LoRA extension.  The sum over z in order then gives
  // the output.
  float* part;
  int64_t k_per;
};

// Reduction stages [beg, end) of this workgroup.
template <bool kSplit>
__device__ __forceinline__ void stage_range(const BigArgs& a, int64_t red, int64_t step, int64_t& beg, int64_t& end) {
  const int64_t all = (red + step - 1) / step;
  beg = 0;
  end = all;
  if (kSplit) {
    beg = static_cast<int64_t>(blockIdx.z) * (a.k_per / step);
    end = beg + a.k_per / step < all ? beg + a.k_per / step : all;
  }
}

#ifndef QN_TILE_GROUP
#define QN_TILE_GROUP 4
#endif
constexpr int64_t kGroup = QN_TILE_GROUP;

// Workgroup -> output tile origin.  Workgroups are dealt to the 8 XCDs
// round-robin (id % 8); XCD x takes the x-th contiguous run of tile numbers,
// and tile numbers walk groups of kGroup row-tiles column by column, so the
// tiles of one XCD form a compact block whose activation rows and weight
// columns are shared in that XCD's L2.  A bijection for any grid.
__device__ __forceinline__ void tile_origin(int64_t& m0, int64_t& c0) {
  const int64_t ntx = gridDim.x, nty = gridDim.y, total = ntx * nty;
  const int64_t id = static_cast<int64_t>(blockIdx.y) * ntx + blockIdx.x;
  const int64_t t = (total % 8 == 0) ? (id % 8) * (total / 8) + id / 8 : id;
  const int64_t g = t / (kGroup * ntx), first = g * kGroup;
  const int64_t gm = nty - first < kGroup ? nty - first : kGroup;
  const int64_t w = t - g * kGroup * ntx;
  m0 = (first + w % gm) * kBM;
  c0 = (w / gm) * kBN;
}

// Registers carried from the load of a stage to its decode.
struct WRegs {
  uint32_t w[8];
  int q;
  float s2;
};

__device__ __forceinline__ uint32_t nib(uint32_t w, int t) { return (w >> (8 * (t >> 1) + ((t & 1) ? 0 : 4))) & 15u; }


__device__ __forceinline__ uint32_t ld32s(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint4 ld128s(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <class T, bool kForward, bool kKTail>
struct Big {
  const BigArgs& a;
  char* smem;
  int t, lane, wave;            // wave is wave-uniform (scalar)
  int64_t m0, c0, red;
  Rsrc r_act, r_codes, r_q, r_s2;
  float off;
  bool single;   // state without a second level: â = absmax[block]
  int s_shift;   // flat weight index -> index of its stored scale
  uint32_t act_voff[8];         // byte offset of this lane's activation chunk, stage 0
  int act_lim[8];               // forward tail: chunk valid while k0 < act_lim
  uint32_t w_voff[8];           // forward: code word of row i at stage 0; backward: [0] = row start
  uint32_t q_voff;              // second-level code of this thread's table at stage 0
  int64_t tab_e0;               // flat weight index of this thread's table block at stage 0
  int tab_row, tab_blk;
  bool tab_ok;

  __device__ Big(const BigArgs& args, char* s) : a(args), smem(s) {
    t = threadIdx.x;
    lane = t & 63;
    wave = __builtin_amdgcn_readfirstlane(t >> 6);
    tile_origin(m0, c0);
    red = kForward ? a.K : a.N;
    const int64_t P = a.K * a.N;
    r_act = make_rsrc(a.act, a.M * a.act_ld * 2);
    r_codes = make_rsrc(a.W.codes, (P + 1) / 2);
    single = a.W.absmax != nullptr;
    r_q = make_rsrc(a.W.qabsmax, single ? 0 : (P + 63) / 64);
    r_s2 = single ? make_rsrc(a.W.absmax, ((P + 63) / 64) * 4) : make_rsrc(a.W.absmax2, ((P + 16383) / 16384) * 4);
    s_shift = single ? 6 : 14;
    off = single ? 0.0f : a.W.offset[0];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // row = wave*64 + 8j + lane/8, whose swizzle is (lane/8) ^ j
      const int chunk = (lane & 7) ^ (lane >> 3) ^ j;
      const int64_t m = m0 + wave * 64 + 8 * j + (lane >> 3);
      act_voff[j] = m < a.M ? static_cast<uint32_t>((m * a.act_ld + 8 * chunk) * 2) : kMasked;
      act_lim[j] = static_cast<int>(red - 8 * chunk);
    }
    if (kForward) {
      const int rg = t >> 5, cg = t & 31;
      const int64_t col = c0 + 8 * cg;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w_voff[i] = col < a.N ? static_cast<uint32_t>(((8 * rg + i) * a.N + col) >> 1) : kMasked;
      tab_row = 8 * rg + (cg & 7);
      tab_blk = cg >> 3;
      tab_ok = c0 + 64 * tab_blk < a.N;
      tab_e0 = tab_row * a.N + c0 + 64 * tab_blk;
    } else {
      const int64_t k = c0 + t;
      w_voff[0] = k < a.K ? static_cast<uint32_t>((k * a.N) >> 1) : kMasked;
      tab_row = t;
      tab_blk = 0;
      tab_ok = k < a.K;
      tab_e0 = k * a.N;
    }
    q_voff = tab_ok ? static_cast<uint32_t>(tab_e0 >> 6) : kMasked;
  }

  __device__ char* sA(int b) const { return smem + kOffA + b * kTileBytes; }
  __device__ char* sB(int b) const { return smem + kOffB + b * kTileBytes; }
  __device__ uint16_t* tabs(int b) const { return reinterpret_cast<uint16_t*>(smem + kOffT + b * kTabBytes); }
  __device__ const float* q2t() const { return reinterpret_cast<const float*>(smem + kOffQ); }

  // Activation stage s -> LDS buffer b, straight from global memory.
  __device__ void copy_act(int64_t s, int b) const {
    const int64_t k0 = s * kBK;
    const uint32_t soff = static_cast<uint32_t>(k0 * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t v = k0 < act_lim[j] ? act_voff[j] : kMasked;
      char* dst = sA(b) + (wave * 64 + 8 * j) * 128;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_act, (lds_ptr_t)(dst), 16, v, soff, 0, 0);
    }
  }

  // Code words and the table's second-level code / scale of stage s.
  __device__ void load_w(WRegs& R, int64_t s) const {
    const int64_t k0 = s * kBK;
    if (kForward) {
      const uint32_t soff = static_cast<uint32_t>((k0 * a.N) >> 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = kKTail ? k0 + 8 * (t >> 5) + i < a.K : k0 < a.K;
        R.w[i] = ld32s(r_codes, ok ? w_voff[i] : kMasked, soff);
      }
      R.q = static_cast<int>(static_cast<int8_t>(__builtin_amdgcn_raw_buffer_load_b8(
          r_q, k0 + tab_row < a.K ? q_voff : kMasked, static_cast<uint32_t>((k0 * a.N) >> 6), 0)));
      const int64_t e = tab_e0 + k0 * a.N;
      R.s2 = ld_f32(r_s2, tab_ok ? static_cast<uint32_t>((e >> s_shift) * 4) : kMasked);
    } else {
      const uint32_t soff = static_cast<uint32_t>(k0 >> 1);
      const uint32_t wv = k0 < a.N ? w_voff[0] : kMasked;
      const uint4 lo = ld128s(r_codes, wv, soff);
      const uint4 hi = ld128s(r_codes, wv, soff + 16);
      R.w[0] = lo.x; R.w[1] = lo.y; R.w[2] = lo.z; R.w[3] = lo.w;
      R.w[4] = hi.x; R.w[5] = hi.y; R.w[6] = hi.z; R.w[7] = hi.w;
      R.q = static_cast<int>(static_cast<int8_t>(
          __builtin_amdgcn_raw_buffer_load_b8(r_q, k0 < a.N ? q_voff : kMasked, static_cast<uint32_t>(k0 >> 6), 0)));
      const int64_t e = tab_e0 + k0;
      R.s2 = ld_f32(r_s2, tab_ok ? static_cast<uint32_t>((e >> s_shift) * 4) : kMasked);
    }
  }

  // Build this thread's table for stage s into table buffer b.
  __device__ void build_table(const WRegs& R, int64_t s, int b) const {
    const int64_t krow = kForward ? s * kBK + tab_row : c0 + tab_row;
    float ahat = single ? R.s2 : __fadd_rn(__fmul_rn(q2t()[R.q + 128], R.s2), off);
    if (krow >= a.K) ahat = 0.0f;   // rows past K decode to zero
    write_block_table<T>(tabs(b) + (kForward ? (tab_row * 4 + tab_blk) : tab_row) * 16, ahat);
  }

  // Split code words into byte-wise doubled nibbles: ix[2c] holds 2*code of
  // the even (high-nibble) elements of word c in its 4 bytes, ix[2c+1] those
  // of the odd (low-nibble) elements, so a lookup address is table + 1 byte.
  __device__ void split_codes(const WRegs& R, uint32_t (&ix)[16]) const {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      ix[2 * c] = (R.w[c] >> 3) & 0x1E1E1E1Eu;
      ix[2 * c + 1] = (R.w[c] << 1) & 0x1E1E1E1Eu;
    }
  }

  // Decode part `part` (0..7) of this thread's share of a stage into weight
  // buffer b: forward column `part` of the thread's 8 columns (8 rows, one
  // table each); backward chunk `part` of its row (8 elements, one table).
  __device__ void decode_part(const uint32_t (&ix)[16], int b, int part) const {
    const char* tb = reinterpret_cast<const char*>(tabs(b));
    char* dst = sB(b);
    uint32_t d[4];
    if (kForward) {
      const int rg = t >> 5, cg = t & 31;
      const char* trow = tb + ((8 * rg) * 4 + (cg >> 3)) * 32;   // table of row 8rg + i at trow + 128 i
      const int sh = 8 * (part >> 1);
      const int odd = part & 1;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t i0 = (ix[2 * (2 * p) + odd] >> sh) & 0xFFu;
        const uint32_t i1 = (ix[2 * (2 * p + 1) + odd] >> sh) & 0xFFu;
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(trow + (2 * p) * 128 + i0);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(trow + (2 * p + 1) * 128 + i1);
        d[p] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(dst + lds_off(8 * cg + part, rg)) = make_uint4(d[0], d[1], d[2], d[3]);
    } else {
      const char* tr = tb + tab_row * 32;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // elements 2p (high nibble of byte p) and 2p+1 (low nibble)
        const uint32_t i0 = (ix[2 * part] >> (8 * p)) & 0xFFu;
        const uint32_t i1 = (ix[2 * part + 1] >> (8 * p)) & 0xFFu;
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(tr + i0);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(tr + i1);
        d[p] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(dst + lds_off(t, part)) = make_uint4(d[0], d[1], d[2], d[3]);
    }
  }

  // One stage of MFMAs from buffer b: 4 substeps of 16 reduction elements,
  // each 4 activation x 4 weight fragments (32 rows x 16 values; lane l holds
  // row l%32, values 8*(l/32)..+7) and 16 v_mfma_f32_32x32x16_bf16.
  struct Frags {
    typename T::v8 a[4], w[4];
  };
  __device__ void load_frags(int b, int ks, Frags& F) const {
    const int r32 = lane & 31, h = lane >> 5, wm = wave >> 1, wn = wave & 1;
    const char* A = sA(b);
    const char* Bt = sB(b);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      F.a[i] = *reinterpret_cast<const typename T::v8*>(A + lds_off(wm * 128 + 32 * i + r32, 2 * ks + h));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      F.w[j] = *reinterpret_cast<const typename T::v8*>(Bt + lds_off(wn * 128 + 32 * j + r32, 2 * ks + h));
  }
  __device__ static void mma(const Frags& F, f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = T::mfma32(F.w[j], F.a[i], acc[i][j]);
  }
  __device__ void compute(int b, f32x16 (&acc)[4][4]) const {
    Frags F;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      load_frags(b, ks, F);
      mma(F, acc);
    }
  }
};

// Dense core: both operands are 16-bit matrices with the reduction
// contiguous (activations M x red and the dequantized weight, rows x red).
// 64-element stages alternate between two LDS slots; a slot holds 256
// activation rows and 256 weight rows of 128 bytes in the fused kernel's
// layout (chunk c of row R at c ^ ((R ^ R >> 3) & 7)).  Copies are buffer
// loads straight into LDS, each instruction 8 rows x 128 bytes, i.e. whole
// cache lines: issuing the same bytes as 16 half-line rows per instruction
// cost about 10% more time.  Stage s+2's 16 copies per wave go out in the
// last substep of stage s and the first of stage s+1, one per two MFMAs (in
// bursts they fill the TA command FIFO and stall the MFMA stream); the one
// barrier per stage sits before the last substep, whose fragments are
// already in registers.
constexpr int kDenseSlot = 2 * kTileBytes;
constexpr int kDenseLds = 2 * kDenseSlot;   // 128 KB

template <class T, bool kForward, bool kKTail>
struct Dense {
  const BigArgs& a;
  char* smem;
  int t, lane, wave;
  int64_t m0, c0, red;
  Rsrc r_act, r_w;
  uint32_t act_voff[8], w_voff[8];   // copy j: row wave*64 + 8j + lane/8, chunk (lane&7)^(lane>>3)^j
  int lim[8];                        // reduction tail: copy j's chunk valid while k0 < lim[j]
  int fA[4], fW[4];                  // fragment offsets within a slot at substep 0
  // Stages: n_main of the product (from s_beg), then the LoRA extension's
  // ceil(r_ext / 64) over (Z, (c B)ᵀ) or (dZ, A), copied like the others.
  int64_t s_beg, n_main, r_ext, lda, cols;
  Rsrc r_ea, r_eb;

  __device__ Dense(const BigArgs& args, char* s) : a(args), smem(s) {
    t = threadIdx.x;
    lane = t & 63;
    wave = __builtin_amdgcn_readfirstlane(t >> 6);
    tile_origin(m0, c0);
    red = kForward ? a.K : a.N;
    const int64_t wrows = kForward ? a.N : a.K;
    r_act = make_rsrc(a.act, a.M * red * 2);
    r_w = make_rsrc(a.wdense, wrows * red * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // row = wave*64 + 8j + lane/8, whose swizzle is (lane/8) ^ j
      const int chunk = (lane & 7) ^ (lane >> 3) ^ j;
      const int row = wave * 64 + 8 * j + (lane >> 3);
      const int64_t m = m0 + row, n = c0 + row;
      act_voff[j] = m < a.M ? static_cast<uint32_t>((m * red + 8 * chunk) * 2) : kMasked;
      w_voff[j] = n < wrows ? static_cast<uint32_t>((n * red + 8 * chunk) * 2) : kMasked;
      lim[j] = static_cast<int>(red - 8 * chunk);
    }
    const int r32 = lane & 31, h = lane >> 5, wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fA[i] = lds_off(wm * 128 + 32 * i + r32, h);
      fW[i] = kTileBytes + lds_off(wn * 128 + 32 * i + r32, h);
    }
    cols = wrows;
    lda = a.ext_a_ld ? a.ext_a_ld : a.r;
    int64_t zoff = 0;   // grouped forward: this tile's member's block of Z columns
    if (kForward)
      for (int i = 0; i < a.ngroups; ++i) zoff += c0 >= a.gend[i] ? a.r : 0;
    r_ea = make_rsrc(a.ext_a + zoff, (a.M * lda - zoff) * 2);
    r_eb = make_rsrc(a.ext_b, cols * a.r * 2);
  }
  // this workgroup's stages (with_ext: it also adds the LoRA extension)
  __device__ int64_t set_stages(int64_t beg, int64_t end, bool with_ext) {
    s_beg = beg;
    n_main = end - beg;
    r_ext = with_ext ? a.r : 0;
    return n_main + (r_ext + kBK - 1) / kBK;
  }

  // slot 0 in the fused kernel's names, for the LoRA extension after the loop
  __device__ char* sA(int) const { return smem; }
  __device__ char* sB(int) const { return smem + kTileBytes; }

  // Copy q (0..15) of stage u (counted from s_beg) into slot b: the
  // activation (even q) or weight (odd q) rows wave*64 + 8(q/2) .. +7.
  // Past the reduction end and the extension: masked.  kMix: u may be an
  // extension stage (else u < n_main, known to the caller).
  template <bool kMix>
  __device__ void copy_one(int64_t u, int b, int q) const {
    const int j = q >> 1;
    char* dst = smem + b * kDenseSlot + (q & 1) * kTileBytes + (wave * 64 + 8 * j) * 128;
    if (!kMix || u < n_main) {
      const int64_t k0 = (s_beg + u) * kBK;
      const uint32_t soff = static_cast<uint32_t>(k0 * 2);
      const bool ok = kKTail ? k0 < lim[j] : k0 < red;
      if ((q & 1) == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_act, (lds_ptr_t)(dst), 16, ok ? act_voff[j] : kMasked, soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_w, (lds_ptr_t)(dst), 16, ok ? w_voff[j] : kMasked, soff, 0, 0);
    } else {
      const int row = wave * 64 + 8 * j + (lane >> 3);
      const int64_t e = (u - n_main) * kBK + 8 * ((lane & 7) ^ (lane >> 3) ^ j);
      if ((q & 1) == 0) {
        const int64_t m = m0 + row;
        const uint32_t v = (m < a.M && e < r_ext) ? static_cast<uint32_t>((m * lda + e) * 2) : kMasked;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_ea, (lds_ptr_t)(dst), 16, v, 0, 0, 0);
      } else {
        const int64_t n = c0 + row;
        const uint32_t v = (n < cols && e < r_ext) ? static_cast<uint32_t>((n * a.r + e) * 2) : kMasked;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_eb, (lds_ptr_t)(dst), 16, v, 0, 0, 0);
      }
    }
  }

  struct Frags {
    typename T::v8 a[4], w[4];
  };
  // Fragment q (activation q/2 for even q, weight q/2 for odd q) of
  // substep ks of slot b: chunk 2ks + h of its row, i.e. the substep-0
  // offset with bits 5-6 flipped by ks.
  __device__ void read_one(int b, int ks, int q, Frags& F) const {
    const char* base = smem + b * kDenseSlot;
    if ((q & 1) == 0)
      F.a[q >> 1] = *reinterpret_cast<const typename T::v8*>(base + (fA[q >> 1] ^ (ks << 5)));
    else
      F.w[q >> 1] = *reinterpret_cast<const typename T::v8*>(base + (fW[q >> 1] ^ (ks << 5)));
  }
  __device__ void load_frags(int b, int ks, Frags& F) const {
#pragma unroll
    for (int q = 0; q < 8; ++q) read_one(b, ks, q, F);
  }

  // 16 MFMAs from Fc; in their shadow the 8 reads of substep ksn of slot bn
  // into Fn (within the first 8 MFMAs, so the last 8 cover their latency)
  // and, when nc > 0, copies q0 .. q0+nc-1 of stage cs into slot cb, one
  // per 16/nc MFMAs.  The order is pinned with scheduling barriers.
  template <bool kMix>
  __device__ void sub_step(const Frags& Fc, Frags& Fn, int bn, int ksn, int64_t cs, int cb, int q0, int nc,
                           f32x16 (&acc)[4][4]) const {
    const int sp = 16 / (nc > 0 ? nc : 1);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int m = 4 * g + u;
        acc[g][u] = T::mfma32(Fc.w[u], Fc.a[g], acc[g][u]);
        __builtin_amdgcn_sched_barrier(0);
        if (m < 8) {
          read_one(bn, ksn, m, Fn);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (nc > 0 && m % sp == (sp > 1 ? 1 : 0)) {
          copy_one<kMix>(cs, cb, q0 + m / sp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // Stage u from slot b, with the next stages' fragment reads and copies
  // in its shadow (see qlora_dense_kernel).
  template <bool kMix>
  __device__ void stage(int64_t u, int b, Frags& F0, Frags& F1, f32x16 (&acc)[4][4]) const {
    sub_step<kMix>(F0, F1, b, 1, u + 1, b ^ 1, 8, 8, acc);
    sub_step<kMix>(F1, F0, b, 2, 0, 0, 0, 0, acc);
    sub_step<kMix>(F0, F1, b, 3, 0, 0, 0, 0, acc);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    sub_step<kMix>(F1, F0, b ^ 1, 0, u + 2, b, 0, 8, acc);
  }

  // finish() is called without the extension (it ran as the last stages).
  __device__ void compute(int, f32x16 (&)[4][4]) const {}
};

// LoRA extension: r more reduction steps over (Z, (c B)ᵀ) in the forward or
// (dZ, A) in the backward; both operands are row-major with r contiguous
// (M x r and cols x r), staged into the 64-wide LDS layout of the main loop.
// Then the bf16 store: the tile goes through LDS (row-major, 512 bytes per
// row, 16-byte chunk q of row R at q ^ (R & 31)) so that every global store
// writes whole 512-byte row segments.  Shared by the fused and dense kernels;
// the main loop has released LDS when this starts.
template <class T, bool kForward, bool kSplit, bool kExt, class Core>
__device__ __forceinline__ void finish(const Core& k, const BigArgs& a, f32x16 (&acc)[4][4]) {
  const int lane = k.lane, t = k.t;
  const int64_t cols = kForward ? a.N : a.K;
  const int64_t lda = a.ext_a_ld ? a.ext_a_ld : a.r;
  int64_t zoff = 0;   // grouped forward: this tile's member's block of Z columns
  if (kForward)
    for (int i = 0; i < a.ngroups; ++i) zoff += k.c0 >= a.gend[i] ? a.r : 0;
  const Rsrc re = make_rsrc(a.ext_a + zoff, (a.M * lda - zoff) * 2);
  const Rsrc rb = make_rsrc(a.ext_b, cols * a.r * 2);
  const int64_t r_ext = kExt && (!kSplit || blockIdx.z == 0) ? a.r : 0;
  for (int64_t j0 = 0; j0 < r_ext; j0 += kBK) {
    const int c = t & 7;
    const int64_t j = j0 + 8 * c;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (t >> 3) + 32 * i;
      const int64_t m = k.m0 + row, n = k.c0 + row;
      const uint4 v = ld_b128(re, (m < a.M && j < a.r) ? static_cast<uint32_t>((m * lda + j) * 2) : kMasked);
      const uint4 w = ld_b128(rb, (n < cols && j < a.r) ? static_cast<uint32_t>((n * a.r + j) * 2) : kMasked);
      *reinterpret_cast<uint4*>(k.sA(0) + lds_off(row, c)) = v;
      *reinterpret_cast<uint4*>(k.sB(0) + lds_off(row, c)) = w;
    }
    __syncthreads();
    k.compute(0, acc);
    __syncthreads();
  }

  // Lane l holds, for tile (i, j), output row 32i + l%32 and, for each jj,
  // the 4 columns 32j + 8jj + 4(l/32) .. +3.
  if constexpr (kSplit) {
    // split-K: the fp32 tile, 16 bytes per buffer store; rows past M and
    // columns past cols (cols % 8 == 0) are masked.
    const int r32 = lane & 31, h = lane >> 5, wm = k.wave >> 1, wn = k.wave & 1;
    const Rsrc rp = make_rsrc(a.part + (static_cast<int64_t>(blockIdx.z) * a.M + k.m0) * cols + k.c0,
                              ((a.M - k.m0) * cols - k.c0) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + 32 * i + r32;
      const bool row_ok = k.m0 + row < a.M;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int col = wn * 128 + 32 * j + 8 * jj + 4 * h;
          const uint32_t voff =
              (row_ok && k.c0 + col < cols) ? static_cast<uint32_t>((row * cols + col) * 4) : kMasked;
          const f32x4 v = {acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2], acc[i][j][4 * jj + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp, voff, 0, 0);
        }
    }
    return;
  }
  char* st = k.sA(0);
  {
    const int r32 = lane & 31, h = lane >> 5, wm = k.wave >> 1, wn = k.wave & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int R = wm * 128 + 32 * i + r32;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int q = wn * 16 + 4 * j + jj;
          uint2 v;
          v.x = T::pack2(acc[i][j][4 * jj], acc[i][j][4 * jj + 1]);
          v.y = T::pack2(acc[i][j][4 * jj + 2], acc[i][j][4 * jj + 3]);
          *reinterpret_cast<uint2*>(st + R * 512 + ((q ^ r32) << 4) + 8 * h) = v;
        }
    }
  }
  __syncthreads();
  {
    const int q = lane & 31;
    const int64_t n = k.c0 + 8 * q;
#pragma unroll 4
    for (int u = 0; u < 32; ++u) {
      const int R = k.wave * 64 + 2 * u + (lane >> 5);
      const int64_t m = k.m0 + R;
      const uint4 v = *reinterpret_cast<const uint4*>(st + R * 512 + ((q ^ (R & 31)) << 4));
      // non-temporal: the output streams out during the epilogue instead of
      // waiting, dirty in L2, for the end-of-kernel release (1-2 us per launch)
      if (m < a.M && n < cols)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(a.out + m * cols + n));
    }
  }
}

template <class T, bool kForward, bool kKTail, bool kSplit>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void qlora_big_kernel(BigArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Big<T, kForward, kKTail> k(a, smem);
  {
    float* q2t = reinterpret_cast<float*>(smem + kOffQ);
    q2t[k.t] = q2_value(k.t - 128);
  }
  int64_t s_beg, s_end;
  stage_range<kSplit>(a, k.red, kBK, s_beg, s_end);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // prologue: the first stage into buffer 0, the next one's weights into registers
  WRegs cur, nxt;
  k.copy_act(s_beg, 0);
  k.load_w(cur, s_beg);
  k.load_w(nxt, s_beg + 1);
  __syncthreads();                 // q2t staged
  k.build_table(cur, s_beg, 0);
  {
    uint32_t ix[16];
    k.split_codes(cur, ix);
#pragma unroll
    for (int p = 0; p < 8; ++p) k.decode_part(ix, 0, p);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  cur = nxt;

  for (int64_t s = s_beg; s < s_end; ++s) {
    const int b = static_cast<int>((s - s_beg) & 1);
    // (stage s+1 and s+2 accesses past the range are masked or never read)
    k.copy_act(s + 1, b ^ 1);
    k.load_w(nxt, s + 2);
    k.build_table(cur, s + 1, b ^ 1);
    uint32_t ix[16];
    k.split_codes(cur, ix);
    // MFMAs of stage s, with the fragments of substep ks+1 and two decode
    // parts of stage s+1 issued in the shadow of substep ks.
    typename Big<T, kForward, kKTail>::Frags F0, F1;
    k.load_frags(b, 0, F0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) k.load_frags(b, ks + 1, F1);
      k.decode_part(ix, b ^ 1, 2 * ks);
      k.decode_part(ix, b ^ 1, 2 * ks + 1);
      Big<T, kForward, kKTail>::mma(F0, acc);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);     // DS write
      if (ks < 3) F0 = F1;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    cur = nxt;
  }

  finish<T, kForward, kSplit, true>(k, a, acc);
}

template <class T, bool kForward, bool kKTail, bool kSplit>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void qlora_dense_kernel(BigArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Dense<T, kForward, kKTail> k(a, smem);
  int64_t s_beg, s_end;
  stage_range<kSplit>(a, k.red, kBK, s_beg, s_end);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  // Stage u (counted from the first of this workgroup's range; the LoRA
  // extension's stages follow the product's) lives in slot u & 1.  The
  // barrier of stage u, before its last substep, says: every wave has read
  // all of slot u & 1 (its last substep's fragments are in registers) and
  // stage u+1 has landed in the other slot.  Stage u+2's copies into slot
  // u & 1 follow it.  Copies past the end are masked or land in a slot that
  // is never read.
  const int64_t total = k.set_stages(s_beg, s_end, !kSplit || blockIdx.z == 0);
#pragma unroll
  for (int q = 0; q < 16; ++q) k.template copy_one<true>(0, 0, q);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  typename Dense<T, kForward, kKTail>::Frags F0, F1;
  k.load_frags(0, 0, F0);
#pragma unroll
  for (int q = 0; q < 8; ++q) k.template copy_one<true>(1, 1, q);
  int b = 0;
  int64_t u = 0;
  // stages whose copies (of u+1 and u+2) are all of the product, then the rest
  for (; u + 2 < k.n_main; ++u, b ^= 1) k.template stage<false>(u, b, F0, F1, acc);
  for (; u < total; ++u, b ^= 1) k.template stage<true>(u, b, F0, F1, acc);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  finish<T, kForward, kSplit, false>(k, a, acc);
}

template <class T, bool kForward, bool kKTail, bool kSplit>
hipError_t launch_big_t(const BigArgs& a, hipStream_t stream, const Timer& tm) {
  // raised once per process; the initialisation of a function-local static
  // is thread-safe, so concurrent first calls do not race
  static const hipError_t lds_limit = hipFuncSetAttribute(reinterpret_cast<const void*>(&qlora_big_kernel<T, kForward, kKTail, kSplit>),
                                                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (lds_limit != hipSuccess) return lds_limit;
  const int64_t cols = kForward ? a.N : a.K, red = kForward ? a.K : a.N;
  const unsigned zs = kSplit ? static_cast<unsigned>((red + a.k_per - 1) / a.k_per) : 1u;
  dim3 grid(static_cast<unsigned>((cols + kBN - 1) / kBN), static_cast<unsigned>((a.M + kBM - 1) / kBM), zs);
  hipExtLaunchKernelGGL((qlora_big_kernel<T, kForward, kKTail, kSplit>), grid, dim3(kThreads), kLdsBytes, stream,
                        tm.start(), tm.end(), 0, a);
  return hipGetLastError();
}

template <class T, bool kForward, bool kKTail, bool kSplit>
hipError_t launch_dense_t(const BigArgs& a, hipStream_t stream, const Timer& tm) {
  // raised once per process; the initialisation of a function-local static
  // is thread-safe, so concurrent first calls do not race
  static const hipError_t lds_limit = hipFuncSetAttribute(reinterpret_cast<const void*>(&qlora_dense_kernel<T, kForward, kKTail, kSplit>),
                                                          hipFuncAttributeMaxDynamicSharedMemorySize, kDenseLds);
  if (lds_limit != hipSuccess) return lds_limit;
  const int64_t cols = kForward ? a.N : a.K, red = kForward ? a.K : a.N;
  const unsigned zs = kSplit ? static_cast<unsigned>((red + a.k_per - 1) / a.k_per) : 1u;
  dim3 grid(static_cast<unsigned>((cols + kBN - 1) / kBN), static_cast<unsigned>((a.M + kBM - 1) / kBM), zs);
  hipExtLaunchKernelGGL((qlora_dense_kernel<T, kForward, kKTail, kSplit>), grid, dim3(kThreads), kDenseLds, stream,
                        tm.start(), tm.end(), 0, a);
  return hipGetLastError();
}

// Instantiation by compute type, reduction tail and split.
template <bool kForward, bool kDense, class T, bool kKTail>
hipError_t launch_gemm_s(const BigArgs& a, hipStream_t stream, const Timer& tm) {
  if (kDense)
    return a.part != nullptr ? launch_dense_t<T, kForward, kKTail, true>(a, stream, tm)
                             : launch_dense_t<T, kForward, kKTail, false>(a, stream, tm);
  return a.part != nullptr ? launch_big_t<T, kForward, kKTail, true>(a, stream, tm)
                           : launch_big_t<T, kForward, kKTail, false>(a, stream, tm);
}
template <bool kForward, bool kDense, class T>
hipError_t launch_gemm_t(const BigArgs& a, hipStream_t stream, const Timer& tm) {
  const int64_t red = kForward ? a.K : a.N;
  return (red % kBK) ? launch_gemm_s<kForward, kDense, T, true>(a, stream, tm)
                     : launch_gemm_s<kForward, kDense, T, false>(a, stream, tm);
}
template <bool kForward, bool kDense>
hipError_t launch_gemm(const BigArgs& a, hipStream_t stream, const Timer& tm, int dtype) {
  return dtype == F16::kDtype ? launch_gemm_t<kForward, kDense, F16>(a, stream, tm)
                              : launch_gemm_t<kForward, kDense, Bf16>(a, stream, tm);
}

// out = the 16-bit rounding of sum_z part[z] (z in order, fp32), 8 elements
// per thread and step; count % 8 == 0.
template <class T>
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, int64_t splits, int64_t count,
                                                        uint16_t* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * 8;
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8; i < count; i += stride) {
    f32x4 lo = *reinterpret_cast<const f32x4*>(part + i);
    f32x4 hi = *reinterpret_cast<const f32x4*>(part + i + 4);
#pragma unroll 4
    for (int64_t z = 1; z < splits; ++z) {
      const float* p = part + z * count + i;
      lo += *reinterpret_cast<const f32x4*>(p);
      hi += *reinterpret_cast<const f32x4*>(p + 4);
    }
    *reinterpret_cast<uint4*>(out + i) =
        make_uint4(T::pack2(lo[0], lo[1]), T::pack2(lo[2], lo[3]), T::pack2(hi[0], hi[1]), T::pack2(hi[2], hi[3]));
  }
}

// Attach the split plan of an M x cols output over a reduction of red to a
// (part_ws null: no split).
void attach_split(BigArgs& a, int64_t cols, int64_t red, void* part_ws) {
  const SplitPlan sp = plan_split(a.M, cols, red);
  if (part_ws == nullptr || sp.splits < 2) return;
  a.part = static_cast<float*>(part_ws);
  a.k_per = sp.k_per;
}

// After a split GEMM: the fixed-order sum into the 16-bit output.
hipError_t split_sum(const BigArgs& a, int64_t cols, hipStream_t stream, int dtype) {
  if (a.part == nullptr) return hipGetLastError();
  const int64_t red = cols == a.N ? a.K : a.N;
  const int64_t splits = (red + a.k_per - 1) / a.k_per, count = a.M * cols;
  int64_t blocks = (count / 8 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  Timer tm(QK_REDUCE, stream);
  if (dtype == F16::kDtype)
    hipLaunchKernelGGL(split_sum_kernel<F16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a.part,
                       splits, count, a.out);
  else
    hipLaunchKernelGGL(split_sum_kernel<Bf16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a.part,
                       splits, count, a.out);
  tm.stop();
  return hipGetLastError();
}

#ifndef QN_SPLIT_TARGET
#define QN_SPLIT_TARGET 256
#endif
#ifndef QN_SPLIT_MIN_STAGES
#define QN_SPLIT_MIN_STAGES 4
#endif
#ifndef QN_SPLIT_BUDGET_MB
#define QN_SPLIT_BUDGET_MB 32
#endif

}  // namespace

// One 256 x 256 tile per workgroup and one workgroup per CU: with fewer
// tiles than about 256 the reduction is split so that splits x tiles stays
// within 256 workgroups, each split at least QN_SPLIT_MIN_STAGES 64-element
// stages long, and the fp32 partials (written once, read once) within
// QN_SPLIT_BUDGET_MB: past that their traffic costs more than the idle CUs.
SplitPlan plan_split(int64_t M, int64_t cols, int64_t red) {
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((cols + kBN - 1) / kBN);
  int64_t s = QN_SPLIT_TARGET / tiles;
  const int64_t max_s = red / (kBK * QN_SPLIT_MIN_STAGES);
  const int64_t budget_s = (static_cast<int64_t>(QN_SPLIT_BUDGET_MB) << 20) / (M * cols * 4);
  if (s > max_s) s = max_s;
  if (s > budget_s) s = budget_s;
  if (s < 2) return SplitPlan{1, red, 0};
  const int64_t per = ((red + s - 1) / s + kBK - 1) / kBK * kBK;
  const int64_t splits = (red + per - 1) / per;
  if (splits < 2) return SplitPlan{1, red, 0};
  return SplitPlan{splits, per, (splits * M * cols * 4 + 255) / 256 * 256};
}

hipError_t launch_fwd_dense(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, const uint16_t* WhatT,
                            const uint16_t* Z, const uint16_t* cBt, uint16_t* Y, hipStream_t stream, int dtype,
                            void* split_ws) {
  BigArgs a{X, K, NF4View{}, Z, cBt, Y, M, K, N, r, WhatT};
  attach_split(a, N, K, split_ws);
  hipError_t e;
  {
    const Timer t(QK_FWD_GEMM, stream, true);
    if ((e = launch_gemm<true, true>(a, stream, t, dtype)) != hipSuccess) return e;
  }
  return split_sum(a, N, stream, dtype);
}

hipError_t launch_fwd_dense_grouped(int64_t M, int64_t K, int64_t Ntot, int64_t r, const uint16_t* X,
                                    const uint16_t* WhatT, const uint16_t* Zcat, int g, const int64_t* gend,
                                    const uint16_t* cBt, uint16_t* Y, hipStream_t stream, int dtype, void* split_ws) {
  BigArgs a{X, K, NF4View{}, Zcat, cBt, Y, M, K, Ntot, r, WhatT};
  a.ext_a_ld = g * r;
  a.ngroups = g - 1;
  for (int i = 0; i + 1 < g; ++i) a.gend[i] = gend[i];
  attach_split(a, Ntot, K, split_ws);
  hipError_t e;
  {
    const Timer t(QK_FWD_GEMM, stream, true);
    if ((e = launch_gemm<true, true>(a, stream, t, dtype)) != hipSuccess) return e;
  }
  return split_sum(a, Ntot, stream, dtype);
}

hipError_t launch_dx_dense(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G, const uint16_t* What,
                           const uint16_t* dZ, const uint16_t* A, uint16_t* dX, hipStream_t stream, int dtype,
                           void* split_ws) {
  BigArgs a{G, N, NF4View{}, dZ, A, dX, M, K, N, r, What};
  attach_split(a, K, N, split_ws);
  hipError_t e;
  {
    const Timer t(QK_BWD_DX, stream, true);
    if ((e = launch_gemm<false, true>(a, stream, t, dtype)) != hipSuccess) return e;
  }
  return split_sum(a, K, stream, dtype);
}

hipError_t launch_fwd_big(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, NF4View W,
                          const uint16_t* Z, const uint16_t* cBt, uint16_t* Y, hipStream_t stream, int dtype,
                          void* split_ws) {
  BigArgs a{X, K, W, Z, cBt, Y, M, K, N, r, nullptr};
  attach_split(a, N, K, split_ws);
  hipError_t e;
  {
    const Timer t(QK_FWD_GEMM, stream, true);
    if ((e = launch_gemm<true, false>(a, stream, t, dtype)) != hipSuccess) return e;
  }
  return split_sum(a, N, stream, dtype);
}

hipError_t launch_dx_big(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G, NF4View W,
                         const uint16_t* dZ, const uint16_t* A, uint16_t* dX, hipStream_t stream, int dtype,
                         void* split_ws) {
  BigArgs a{G, N, W, dZ, A, dX, M, K, N, r, nullptr};
  attach_split(a, K, N, split_ws);
  hipError_t e;
  {
    const Timer t(QK_BWD_DX, stream, true);
    if ((e = launch_gemm<false, false>(a, stream, t, dtype)) != hipSuccess) return e;
  }
  return split_sum(a, K, stream, dtype);
}

}  // namespace qn
