// Rank-r products of the layer and the small-M dequant-GEMV, for gfx950.
//
// Layer (page "QLoRA：冻结的 4-bit 权重怎样参与一次微调", sections
// "量化基座与可训练支路怎样相加" and "冻结权重为什么仍然需要输入梯度"):
//   Z = X A (M x r), dZ = c G Bᵀ (M x r): "row sums" - each output row reduces
//     one activation row against r weight rows; both operands are contiguous
//     along the reduction, so MFMA fragments are loaded straight from global
//     memory (A is transposed once, r x K, so that it is too).
//   dA = Xᵀ dZ (K x r), dB = c Zᵀ G (r x N): "column sums" over the M tokens;
//     both operands are strided along the reduction, so 16-token steps are
//     transposed by LDS reads.  With a single token split the column sums
//     write dA and dB themselves; otherwise a reduce kernel adds the splits.
// (The small-M dequant-GEMV is in gemv.hip.)
// Every reduction is in a fixed order, so results are run-to-run identical.
#include "common.hpp"
#include "kernels.hpp"
#include "side_jobs.hpp"

namespace qn {

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// ------------------------------------------------------------ transpose
// Two TJobs per launch (side_jobs.hpp): Aᵀ and, in the forward, (c B)ᵀ.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(TJob j0, TJob j1) {
  __shared__ uint16_t tile[32][33];
  const bool second = blockIdx.x >= j0.nblk;
  transpose_block(second ? j1 : j0, second ? blockIdx.x - j0.nblk : blockIdx.x, tile);
}

TJob tjob(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols, float scale, int dtype = kDtypeBf16) {
  return make_tjob(src, dst, rows, cols, scale, dtype == kDtypeF16 ? 1 : 0);
}

// ------------------------------------------------------------ row sums
// part[split][m][j] = sum, over this split's share of the reduction, of
// act[m][k] * wt[j][k]; both operands contiguous along k.  A workgroup owns a
// 128-row x 64-column output block (columns j0 .. j0+63): eight waves of 16
// rows x 4 tiles of v_mfma_f32_16x16x32_bf16.  64-wide stages flow through a
// ring of kRsSlots LDS slots (128 activation rows, then 64 weight rows, 128
// bytes each, 16-byte chunk c of row R at c ^ (R & 7)), filled by buffer loads
// with the LDS destination three stages ahead; one barrier per stage.  The
// weight rows are shared by the eight waves, so each weight slice is fetched
// once per 128 activation rows.  One such workgroup per CU (96 KB of LDS)
// streams faster than two of half the size.
#ifndef QN_RS_SLOTS
#define QN_RS_SLOTS 4
#endif
#ifndef QN_RS_WAVES
#define QN_RS_WAVES 8
#endif
constexpr int kRsSlots = QN_RS_SLOTS;
constexpr int kRsWaves = QN_RS_WAVES;   // 16 activation rows each
static_assert(kRsWaves == 4 || kRsWaves == 8, "row sums: 4 or 8 waves");
constexpr int kRsRows = 16 * kRsWaves;
constexpr int kRsActBytes = kRsRows * 128;
constexpr int kRsSlot = kRsActBytes + 64 * 128;
constexpr int kRsLds = kRsSlots * kRsSlot;
constexpr int kRsWtCopies = 8 / kRsWaves;   // 8-row weight copies per wave and stage

struct RsArgs {
  const uint16_t* act;
  const uint16_t* wt;
  int64_t M, r, red, per_split, row_blocks, j_chunks;
  float* part;   // [splits][M][r]
  int64_t act_ld, wt_ld;   // row strides of act (M x red) and wt (r x red)
};

__device__ __forceinline__ int rs_off(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <class T>
__global__ __launch_bounds__(64 * kRsWaves) void rowsum_kernel(RsArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int t = threadIdx.x, lane = t & 63, q = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t rb = blockIdx.x % a.row_blocks, rest = blockIdx.x / a.row_blocks;
  const int64_t m0 = rb * kRsRows, j0 = (rest % a.j_chunks) * 64, split = rest / a.j_chunks;
  const int64_t beg = split * a.per_split;
  const int64_t len = min(a.red, beg + a.per_split) - beg;
  const int64_t nst = (len + 63) / 64;
  const Rsrc ra = make_rsrc(a.act, ((a.M - 1) * a.act_ld + a.red) * 2);
  const Rsrc rw = make_rsrc(a.wt, ((a.r - 1) * a.wt_ld + a.red) * 2);
  // activation copy i (0..1) fills slot rows 16*wave + 8i .. +7; weight copy
  // i fills weight rows 8 (kRsWtCopies wave + i) .. +7; lane -> row + lane/8,
  // slot position lane & 7, global chunk (lane & 7) ^ (row & 7)
  uint32_t av[2], wv[kRsWtCopies];
  int alim[2], wlim[kRsWtCopies];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int R = 16 * wave + 8 * i + (lane >> 3), c = (lane & 7) ^ (R & 7);
    const int64_t m = m0 + R;
    av[i] = m < a.M ? static_cast<uint32_t>((m * a.act_ld + beg + 8 * c) * 2) : kMasked;
    alim[i] = static_cast<int>(len - 8 * c);
  }
#pragma unroll
  for (int i = 0; i < kRsWtCopies; ++i) {
    const int R = 8 * (kRsWtCopies * wave + i) + (lane >> 3), c = (lane & 7) ^ (R & 7);
    const int64_t j = j0 + R;
    wv[i] = j < a.r ? static_cast<uint32_t>((j * a.wt_ld + beg + 8 * c) * 2) : kMasked;
    wlim[i] = static_cast<int>(len - 8 * c);
  }
  auto copy = [&](int64_t s, int b) {
    const int64_t k0 = s * 64;
    const uint32_t soff = static_cast<uint32_t>(k0 * 2);
    char* slot = smem + b * kRsSlot;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + (16 * wave + 8 * i) * 128), 16,
                                               k0 < alim[i] ? av[i] : kMasked, soff, 0, 0);
#pragma unroll
    for (int i = 0; i < kRsWtCopies; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(slot + kRsActBytes + 8 * (kRsWtCopies * wave + i) * 128),
                                               16, k0 < wlim[i] ? wv[i] : kMasked, soff, 0, 0);
  };
  f32x4 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x4{0, 0, 0, 0};
  // Stage x goes to slot x % S, S - 1 stages ahead (2 + kRsWtCopies copies
  // per wave per stage); no copies are issued past the last stage.
  constexpr int S = kRsSlots, kCopies = 2 + kRsWtCopies;
  for (int x = 0; x < S - 1; ++x)
    if (x < nst) copy(x, x);
  int b = 0;
  for (int64_t s = 0; s < nst; ++s) {
    // own copies of stage s landed (later stages may still be in flight)
    if (s + S - 2 < nst) __builtin_amdgcn_s_waitcnt(waitcnt_imm(kCopies * (S - 2), 0));
    else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();   // everyone's; slot of stage s-1 released
    if (s + S - 1 < nst) copy(s + S - 1, b == 0 ? S - 1 : b - 1);
    const char* slot = smem + b * kRsSlot;
    b = b == S - 1 ? 0 : b + 1;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const typename T::v8 af = *reinterpret_cast<const typename T::v8*>(slot + rs_off(16 * wave + q, 4 * st + g));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const typename T::v8 wf = *reinterpret_cast<const typename T::v8*>(slot + kRsActBytes + rs_off(16 * u + q, 4 * st + g));
        acc[u] = T::mfma16(af, wf, acc[u]);
      }
    }
  }
  // lane holds rows 4g + e of column 16u + q
  float* out = a.part + split * a.M * a.r;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = j0 + 16 * u + q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t m = m0 + 16 * wave + 4 * g + e;
      if (m < a.M && j < a.r) out[m * a.r + j] = acc[u][e];
    }
  }
}

// ------------------------------------------------------------ column sums
// part[split][c][j] = sum, over this split's tokens, of act[m][c] * v[m][j]
// (both token-major).  A workgroup owns a 64-column x 64-j block; its tokens
// are divided among its 4 waves, and each wave streams 16-token steps
// (16 activation rows of 64 columns and 16 rows of v, 128 bytes each) through
// its own ring of kCsSlots LDS slots, so waves never wait for each other.
// Rings of four slots (64 KB per workgroup) let two workgroups share a CU,
// which streams these 128-byte row pieces faster than deeper rings.  Within a
// slot, 16-byte chunk c of row R sits at c ^ (((R >> 1) & 1) << 2), which
// keeps the transposing reads below free of bank conflicts.  The MFMA
// operands (8 consecutive tokens of one column per lane) come from
// ds_read_b64_tr_b16: in each 16-lane group, lane L names the 4 values of
// row L/4, columns 4(L%4) .. +3 of a 4 x 16 block, and receives column L of
// that block.  The waves' sums are added in LDS in a fixed order.
#ifndef QN_CS_SLOTS
#define QN_CS_SLOTS 4
#endif
#ifndef QN_CS_WGS
#define QN_CS_WGS 256
#endif
constexpr int kCsSlots = QN_CS_SLOTS;
constexpr int kCsSlot = 2 * 16 * 128;
constexpr int kCsRing = kCsSlots * kCsSlot;
constexpr int kCsBlock = 64 * 64 * 4;   // one wave's 64 x 64 fp32 sums, for the epilogue
static_assert(kCsRing >= kCsBlock, "column sums: each wave's epilogue block lives in its own ring");
constexpr int kCsLds = 4 * kCsRing;

struct CsJob {
  const uint16_t* act;   // M x cols, leading dimension ld
  int64_t ld, cols;
  const uint16_t* v;     // M x r, leading dimension v_ld
  float* part;           // [splits][cols][r]; with `transposed`, the final r x cols result
  int64_t col_blocks, j_chunks, per_split, nblk;
  int64_t r, v_ld;
  // a job with one split may write its final result: scale * sum, stored
  // r x cols (row j, column c) instead of as a partial
  int transposed = 0;
  float scale = 1.0f;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int cs_off(int row, int chunk) { return row * 128 + ((chunk ^ (((row >> 1) & 1) << 2)) << 4); }

template <class T>
__device__ __forceinline__ typename T::v8 tr_read2(const char* p0, const char* p1) {
  typedef __attribute__((address_space(3))) v4i16* lp;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p1));
  const v4i16 both[2] = {lo, hi};
  return __builtin_bit_cast(typename T::v8, both);
}

// Up to kCsJobs jobs per launch, their workgroups one after another.
constexpr int kCsJobs = 4;
struct CsJobs {
  CsJob j[kCsJobs];
};

// A wave's 64 x 64 fp32 sums in an epilogue block.  Lane (h = lane/32,
// c = 32 ci + lane%32) holds j = 32 vj + 8 jj + 4 h + e.
// - Partials, [c][j]: groups of 4 j are stored as 16-byte words, the group
//   index XORed with c % 16 so that the lanes' words spread over the banks.
// - Transposed, [j][c]: single floats, bit 5 of c flipped on every other
//   group of 4 rows, so that the two half-waves' stores fall on different banks.
__device__ __forceinline__ int cs_pos_part(int c, int j) { return c * 64 + (j ^ (4 * (c & 15))); }
__device__ __forceinline__ int cs_pos_tr(int j, int c) { return j * 64 + (c ^ (((j >> 2) & 1) << 5)); }

// this lane's sums into a wave's epilogue block
__device__ __forceinline__ void cs_block(float* blk, bool tr, const f32x16 (&acc)[2][2], int lane) {
  const int h = lane >> 5, cl = lane & 31;
#pragma unroll
  for (int vj = 0; vj < 2; ++vj)
#pragma unroll
    for (int ci = 0; ci < 2; ++ci)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int c = 32 * ci + cl, j = 32 * vj + 8 * jj + 4 * h;
        if (tr) {
#pragma unroll
          for (int e = 0; e < 4; ++e) blk[cs_pos_tr(j + e, c)] = acc[vj][ci][4 * jj + e];
        } else {
          *reinterpret_cast<f32x4*>(blk + cs_pos_part(c, j)) =
              f32x4{acc[vj][ci][4 * jj], acc[vj][ci][4 * jj + 1], acc[vj][ci][4 * jj + 2], acc[vj][ci][4 * jj + 3]};
        }
      }
}

template <class T>
__global__ __launch_bounds__(256) void colsum_kernel(CsJobs jobs, int64_t M) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int64_t blk = blockIdx.x;
  CsJob J = jobs.j[0];
#pragma unroll
  for (int i = 1; i < kCsJobs; ++i)
    if (blk >= J.nblk) {
      blk -= J.nblk;
      J = jobs.j[i];
    }
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t cb = blk % J.col_blocks, rest = blk / J.col_blocks;
  const int64_t c0 = cb * 64, jb = (rest % J.j_chunks) * 64, split = rest / J.j_chunks;
  const int64_t mb = split * J.per_split, me = min(M, mb + J.per_split);
  const int64_t share = (((me - mb) + 63) / 64) * 16;   // tokens per wave, a multiple of 16
  const int64_t wb = mb + wave * share, we = min(me, wb + share);
  const int64_t nsteps = we > wb ? (we - wb + 15) / 16 : 0;
  char* ring = smem + wave * kCsRing;
  const int64_t r = J.r;
  const Rsrc ra = make_rsrc(J.act, ((M - 1) * J.ld + J.cols) * 2), rv = make_rsrc(J.v, ((M - 1) * J.v_ld + r) * 2);
  // copy i (0..1) of each operand fills slot rows 8i .. 8i+7: lane -> row
  // 8i + lane/8, slot position lane & 7, global chunk (lane & 7) ^ swizzle
  uint32_t av[2], vv[2];
  int lim[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int R = 8 * i + (lane >> 3), c = (lane & 7) ^ (((R >> 1) & 1) << 2);
    const int64_t m = wb + R;
    av[i] = c0 + 8 * c < J.cols ? static_cast<uint32_t>((m * J.ld + c0 + 8 * c) * 2) : kMasked;
    vv[i] = jb + 8 * c < r ? static_cast<uint32_t>((m * J.v_ld + jb + 8 * c) * 2) : kMasked;
    lim[i] = static_cast<int>(we - wb - R);   // row valid in step s iff 16 s < lim
  }
  auto copy = [&](int64_t s, int b) {
    const uint32_t sa = static_cast<uint32_t>(s * 16 * J.ld * 2), sv = static_cast<uint32_t>(s * 16 * J.v_ld * 2);
    char* slot = ring + b * kCsSlot;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool ok = 16 * s < lim[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + 8 * i * 128), 16, ok ? av[i] : kMasked, sa, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(slot + 2048 + 8 * i * 128), 16, ok ? vv[i] : kMasked, sv,
                                               0, 0);
    }
  };
  // transposing-read addresses within a slot: group G = lane/16 reads rows
  // 8(G>>1) + 4 half + L/4 and columns 16(G&1) + 4(L&3) of 32-column tile ti
  const int G = lane >> 4, L = lane & 15;
  int toff[2][2];   // [tile][half], byte offsets
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int R = 8 * (G >> 1) + 4 * h + (L >> 2);
      const int col = 32 * ti + 16 * (G & 1) + 4 * (L & 3);
      toff[ti][h] = cs_off(R, col >> 3) + 2 * (col & 7);
    }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  constexpr int S = kCsSlots;
  for (int x = 0; x < S - 1; ++x)
    if (x < nsteps) copy(x, x);
  for (int64_t s = 0; s < nsteps; ++s) {
    const int b = static_cast<int>(s % S);
    if (s + S - 1 < nsteps) {
      copy(s + S - 1, static_cast<int>((s + S - 1) % S));   // slot of step s-1, read in full already
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * (S - 1), 15));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    }
    const char* slot = ring + b * kCsSlot;
    typename T::v8 fa[2], fv[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      fa[ti] = tr_read2<T>(slot + toff[ti][0], slot + toff[ti][1]);
      fv[ti] = tr_read2<T>(slot + 2048 + toff[ti][0], slot + 2048 + toff[ti][1]);
    }
    // D[j][c]: each lane holds column c = 32 ci + lane%32 and j = 32 vj + 8jj + 4(lane/32) + e
#pragma unroll
    for (int vj = 0; vj < 2; ++vj)
#pragma unroll
      for (int ci = 0; ci < 2; ++ci) acc[vj][ci] = T::mfma32(fv[vj], fa[ci], acc[vj][ci]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  // Each wave's 64 x 64 sums go to the start of its own ring (its last reads
  // of the ring are done); the final sum is block 0 + 1 + 2 + 3.
  const bool tr = J.transposed != 0;
  float* blocks = reinterpret_cast<float*>(smem);
  cs_block(reinterpret_cast<float*>(ring), tr, acc, lane);
  __syncthreads();
  // thread t: row t / 4 of the 64 x 64 block, four groups of 4 along it
  const int row = t >> 2, q0 = 16 * (t & 3);
  if (tr) {
    // row = j; the scaled sum is stored along the columns of the r x cols result
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = q0 + 4 * u, pos = cs_pos_tr(row, c);
      f32x4 s4 = *reinterpret_cast<const f32x4*>(blocks + pos);
#pragma unroll
      for (int w = 1; w < 4; ++w) s4 += *reinterpret_cast<const f32x4*>(blocks + w * (kCsRing / 4) + pos);
      s4 *= J.scale;
      if (c0 + c < J.cols && jb + row < r) *reinterpret_cast<f32x4*>(J.part + (jb + row) * J.cols + c0 + c) = s4;
    }
    return;
  }
  {
    // row = c; the split's partial, [c][j]
    float* out = J.part + split * J.cols * r;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = q0 + 4 * u, pos = cs_pos_part(row, j);
      f32x4 s4 = *reinterpret_cast<const f32x4*>(blocks + pos);
#pragma unroll
      for (int w = 1; w < 4; ++w) s4 += *reinterpret_cast<const f32x4*>(blocks + w * (kCsRing / 4) + pos);
      if (c0 + row < J.cols && jb + j < r) *reinterpret_cast<f32x4*>(out + (c0 + row) * r + jb + j) = s4;
    }
  }
}

// Two RdJobs per launch (side_jobs.hpp).
__global__ __launch_bounds__(256) void reduce_kernel(RdJob j0, RdJob j1) {
  const bool second = blockIdx.x >= j0.nblk;
  reduce_block(second ? j1 : j0, second ? blockIdx.x - j0.nblk : blockIdx.x);
}

void split_plan(int64_t tiles, int64_t red, int64_t target, int64_t quantum, int64_t* splits, int64_t* per) {
  int64_t s = cdiv(target, tiles);
  const int64_t max_s = cdiv(red, quantum);
  s = s < 1 ? 1 : (s > max_s ? max_s : s);
  *per = round_up(cdiv(red, s), quantum);
  *splits = cdiv(red, *per);
}

RdJob rdjob(const float* part, int64_t splits, int64_t rows, int64_t cols, float scale, bool transpose, float* out_f32,
            uint16_t* out_bf16, int dtype = kDtypeBf16) {
  return make_rdjob(part, splits, rows, cols, scale, transpose, out_f32, out_bf16, dtype == kDtypeF16 ? 1 : 0);
}

hipError_t launch_reduce(const RdJob& ja, const RdJob* jb, hipStream_t stream) {
  RdJob second = jb != nullptr ? *jb : ja;
  if (jb == nullptr) second.nblk = 0;
  Timer tm(QK_REDUCE, stream);
  hipLaunchKernelGGL(reduce_kernel, dim3(static_cast<unsigned>(ja.nblk + second.nblk)), dim3(256), 0, stream, ja,
                     second);
  tm.stop();
  return hipGetLastError();
}

template <class T>
hipError_t rowsum_launch_t(const RsArgs& a, int64_t splits, hipStream_t stream) {
  // raised once per process; the initialisation of a function-local static
  // is thread-safe, so concurrent first calls do not race
  static const hipError_t lds_limit = hipFuncSetAttribute(reinterpret_cast<const void*>(&rowsum_kernel<T>),
                                                          hipFuncAttributeMaxDynamicSharedMemorySize, kRsLds);
  if (lds_limit != hipSuccess) return lds_limit;
  hipLaunchKernelGGL(rowsum_kernel<T>, dim3(static_cast<unsigned>(a.row_blocks * a.j_chunks * splits)), dim3(64 * kRsWaves),
                     kRsLds, stream, a);
  return hipGetLastError();
}

hipError_t launch_rowsum(const uint16_t* act, const uint16_t* wt, int64_t M, int64_t r, int64_t red, int64_t splits,
                         int64_t per, float* part, hipStream_t stream, int64_t act_ld = 0, int64_t wt_ld = 0,
                         int dtype = kDtypeBf16) {
  const RsArgs a{act, wt, M, r, red, per, cdiv(M, kRsRows), cdiv(r, 64), part, act_ld ? act_ld : red, wt_ld ? wt_ld : red};
  return dtype == kDtypeF16 ? rowsum_launch_t<F16>(a, splits, stream) : rowsum_launch_t<Bf16>(a, splits, stream);
}

template <class T>
hipError_t colsum_launch_t(const CsJobs& jobs, int64_t M, hipStream_t stream) {
  // raised once per process; the initialisation of a function-local static
  // is thread-safe, so concurrent first calls do not race
  static const hipError_t lds_limit = hipFuncSetAttribute(reinterpret_cast<const void*>(&colsum_kernel<T>),
                                                          hipFuncAttributeMaxDynamicSharedMemorySize, kCsLds);
  if (lds_limit != hipSuccess) return lds_limit;
  int64_t blocks = 0;
  for (int i = 0; i < kCsJobs; ++i) blocks += jobs.j[i].nblk;
  hipLaunchKernelGGL(colsum_kernel<T>, dim3(static_cast<unsigned>(blocks)), dim3(256), kCsLds, stream, jobs, M);
  return hipGetLastError();
}

// jobs[0 .. n-1] (n <= kCsJobs) in one launch.
hipError_t launch_colsum(const CsJob* jobs, int n, int64_t M, hipStream_t stream, int dtype) {
  CsJobs js{};
  for (int i = 0; i < n; ++i) js.j[i] = jobs[i];
  return dtype == kDtypeF16 ? colsum_launch_t<F16>(js, M, stream) : colsum_launch_t<Bf16>(js, M, stream);
}

}  // namespace

// ------------------------------------------------------------ plans
#ifndef QN_ROWSUM_WAVES
#define QN_ROWSUM_WAVES 256   // target number of row-sum workgroups
#endif
SkinnyPlan plan_skinny(int64_t M, int64_t K, int64_t N, int64_t r) {
  SkinnyPlan p{};
  // row sums: 128-row blocks x 64-wide column chunks, split along the
  // reduction into multiples of 256 until ~256 workgroups (1 per CU)
  const int64_t rs_tiles = cdiv(M, kRsRows) * cdiv(r, 64);
  split_plan(rs_tiles, K, QN_ROWSUM_WAVES, 256, &p.z_splits, &p.z_per);
  split_plan(rs_tiles, N, QN_ROWSUM_WAVES, 256, &p.dz_splits, &p.dz_per);
  // column sums: 64-column blocks of dA and dB together, split along the
  // tokens (multiples of 64) until ~256 workgroups (1 per CU)
  const int64_t cs_tiles = (cdiv(K, 64) + cdiv(N, 64)) * cdiv(r, 64);
  int64_t cs_splits, cs_per;
  split_plan(cs_tiles, M, QN_CS_WGS, 64, &cs_splits, &cs_per);
  p.da_splits = p.db_splits = cs_splits;
  p.da_per = p.db_per = cs_per;
  p.at_bytes = round_up(r * K * 2, 256);
  p.z_part = round_up(p.z_splits * M * r * 4, 256);
  p.dz_part = round_up(p.dz_splits * M * r * 4, 256);
  p.da_part = round_up(p.da_splits * K * r * 4, 256);
  p.db_part = round_up(p.db_splits * N * r * 4, 256);
  plan_gemv(M, K, N, r, &p);
  return p;
}

void lora_transposes(int64_t K, int64_t r, const uint16_t* A, uint16_t* At, int64_t N, const uint16_t* B, float c,
                     uint16_t* cbt, int64_t rb, int dtype, TJob out[2]) {
  out[0] = tjob(A, At, K, r, 1.0f, dtype);
  out[1] = cbt != nullptr ? tjob(B, cbt, rb ? rb : r, N, c, dtype) : out[0];
  if (cbt == nullptr) out[1].nblk = 0;
}

hipError_t launch_lora_down(int64_t M, int64_t K, int64_t r, const uint16_t* X, const uint16_t* A, uint16_t* Z,
                            const SkinnyPlan& p, void* at_ws, void* part_ws, hipStream_t stream, int64_t N,
                            const uint16_t* B, float c, uint16_t* cbt, int64_t rb, int dtype, bool pre_transposed) {
  uint16_t* At = static_cast<uint16_t*>(at_ws);
  if (!pre_transposed) {
    TJob tj[2];
    lora_transposes(K, r, A, At, N, B, c, cbt, rb, dtype, tj);
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3(static_cast<unsigned>(tj[0].nblk + tj[1].nblk)), dim3(256), 0,
                       stream, tj[0], tj[1]);
  }
  float* part = static_cast<float*>(part_ws);
  Timer tm(QK_LORA_DOWN, stream);
  hipError_t e = launch_rowsum(X, At, M, r, K, p.z_splits, p.z_per, part, stream, 0, 0, dtype);
  tm.stop();
  if (e != hipSuccess) return e;
  const RdJob jz = rdjob(part, p.z_splits, M, r, 1.0f, false, nullptr, Z, dtype);
  return launch_reduce(jz, nullptr, stream);
}

hipError_t launch_dz(int64_t M, int64_t N, int64_t r, const uint16_t* G, const uint16_t* B, float c, uint16_t* dZ,
                     const SkinnyPlan& p, void* part_ws, hipStream_t stream, int dtype, RdJob* defer) {
  float* part = static_cast<float*>(part_ws);
  Timer tm(QK_BWD_DZ, stream);
  hipError_t e = launch_rowsum(G, B, M, r, N, p.dz_splits, p.dz_per, part, stream, 0, 0, dtype);
  tm.stop();
  if (e != hipSuccess) return e;
  const RdJob jz = rdjob(part, p.dz_splits, M, r, c, false, nullptr, dZ, dtype);
  if (defer != nullptr) {
    *defer = jz;
    return hipSuccess;
  }
  return launch_reduce(jz, nullptr, stream);
}

// dA = Xᵀ dZ (K x r) and dB = c Zᵀ G (r x N).
hipError_t launch_colsums(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X, const uint16_t* G,
                          const uint16_t* Z, const uint16_t* dZ, float c, float* dA, float* dB, const SkinnyPlan& p,
                          void* da_ws, void* db_ws, hipStream_t stream, int dtype) {
  const int64_t jc = cdiv(r, 64);
  CsJob ja{X, K, K, dZ, static_cast<float*>(da_ws), cdiv(K, 64), jc, p.da_per, 0, r, r};
  CsJob jb{G, N, N, Z, static_cast<float*>(db_ws), cdiv(N, 64), jc, p.db_per, 0, r, r};
  ja.nblk = ja.col_blocks * jc * p.da_splits;
  jb.nblk = jb.col_blocks * jc * p.db_splits;
  // with one token split the sums are final: dA is written in place, dB
  // scaled and transposed, and no reduce launch follows
  const bool direct = p.da_splits == 1 && p.db_splits == 1;
  if (direct) {
    ja.part = dA;
    jb.part = dB;
    jb.transposed = 1;
    jb.scale = c;
  }
  const CsJob both[2] = {ja, jb};
  Timer tm(QK_BWD_COLSUM, stream);
  hipError_t e = launch_colsum(both, 2, M, stream, dtype);
  tm.stop();
  if (e != hipSuccess || direct) return e;
  const RdJob ra = rdjob(static_cast<float*>(da_ws), p.da_splits, K, r, 1.0f, false, dA, nullptr);
  const RdJob rb = rdjob(static_cast<float*>(db_ws), p.db_splits, N, r, c, true, dB, nullptr);
  return launch_reduce(ra, &rb, stream);
}

}  // namespace qn

namespace qn {

// ------------------------------------------------------------ grouped linears
// g members sharing X, concatenated: member i owns columns off_i .. off_i + N_i
// of G (M x Ntot) and B (r x Ntot), and columns i r .. i r + r of Z, dZ (M x g r)
// and A, dA (K x g r).
GroupPlan plan_grouped(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t r) {
  GroupPlan gp{};
  int64_t Ntot = 0;
  for (int i = 0; i < g; ++i) Ntot += Ns[i];
  const int64_t rt = g * r;
  gp.zp = plan_skinny(M, K, Ntot, rt);
  int64_t cs_tiles = cdiv(K, 64) * cdiv(rt, 64);
  for (int i = 0; i < g; ++i) {
    const SkinnyPlan pi = plan_skinny(M, K, Ns[i], r);
    gp.dz_splits[i] = pi.dz_splits;
    gp.dz_per[i] = pi.dz_per;
    gp.dz_off[i] = gp.dz_part;   // every member's partials kept until its sum runs
    gp.dz_part += pi.dz_part;
    cs_tiles += cdiv(Ns[i], 64) * cdiv(r, 64);
  }
  // the jobs run kCsJobs to a launch (all of them for up to three members)
  // (the jobs run kCsJobs to a launch: all of them for up to three members)
  split_plan(cs_tiles, M, QN_CS_WGS, 64, &gp.cs_splits, &gp.cs_per);
  gp.da_part = round_up(gp.cs_splits * K * rt * 4, 256);
  gp.db_part_total = 0;
  for (int i = 0; i < g; ++i) {
    gp.db_off[i] = gp.db_part_total;
    gp.db_part_total += round_up(gp.cs_splits * Ns[i] * r * 4, 256);
  }
  return gp;
}

// dZ_i = c G_i B_iᵀ for every member: a row-sum over member i's columns of G
// and B (row stride Ntot), reduced into column block i of dZ (row stride g r).
// With defer != nullptr the g sums are not launched but returned there.
hipError_t launch_dz_grouped(int64_t M, int g, const int64_t* Ns, int64_t Ntot, int64_t r, const uint16_t* G,
                             const uint16_t* B, float c, uint16_t* dZ, const GroupPlan& gp, void* part_ws,
                             hipStream_t stream, int dtype, RdJob* defer) {
  int64_t off = 0;
  for (int i = 0; i < g; ++i) {
    float* part = reinterpret_cast<float*>(static_cast<char*>(part_ws) + gp.dz_off[i]);
    Timer tm(QK_BWD_DZ, stream);
    hipError_t e =
        launch_rowsum(G + off, B + off, M, r, Ns[i], gp.dz_splits[i], gp.dz_per[i], part, stream, Ntot, Ntot, dtype);
    tm.stop();
    if (e != hipSuccess) return e;
    RdJob jz = rdjob(part, gp.dz_splits[i], M, r, c, false, nullptr, dZ + i * r, dtype);
    jz.out_ld = g * r;
    if (defer != nullptr) defer[i] = jz;
    else if ((e = launch_reduce(jz, nullptr, stream)) != hipSuccess) return e;
    off += Ns[i];
  }
  return hipSuccess;
}

// dA = Xᵀ dZ (K x g r, all members at once) and, per member, dB_i = c Z_iᵀ G_i
// into columns off_i .. of dB (r x Ntot); two column-sum jobs per launch.
hipError_t launch_colsums_grouped(int64_t M, int64_t K, int g, const int64_t* Ns, int64_t Ntot, int64_t r,
                                  const uint16_t* X, const uint16_t* G, const uint16_t* Z, const uint16_t* dZ, float c,
                                  float* dA, float* dB, const GroupPlan& gp, void* da_ws, void* db_ws,
                                  hipStream_t stream, int dtype) {
  const int64_t rt = g * r;
  CsJob jobs[kMaxGroupMembers + 1];
  RdJob rds[kMaxGroupMembers + 1];
  jobs[0] = CsJob{X, K, K, dZ, static_cast<float*>(da_ws), cdiv(K, 64), cdiv(rt, 64), gp.cs_per, 0, rt, rt};
  rds[0] = rdjob(static_cast<float*>(da_ws), gp.cs_splits, K, rt, 1.0f, false, dA, nullptr);
  int64_t off = 0;
  for (int i = 0; i < g; ++i) {
    float* part = reinterpret_cast<float*>(static_cast<char*>(db_ws) + gp.db_off[i]);
    jobs[i + 1] = CsJob{G + off, Ntot, Ns[i], Z + i * r, part, cdiv(Ns[i], 64), cdiv(r, 64), gp.cs_per, 0, r, rt};
    rds[i + 1] = rdjob(part, gp.cs_splits, Ns[i], r, c, true, dB + off, nullptr);
    rds[i + 1].out_ld = Ntot;
    off += Ns[i];
  }
  for (int j = 0; j <= g; ++j) jobs[j].nblk = jobs[j].col_blocks * jobs[j].j_chunks * gp.cs_splits;
  for (int j = 0; j <= g; j += kCsJobs) {
    const int n = g + 1 - j < kCsJobs ? g + 1 - j : kCsJobs;
    Timer tm(QK_BWD_COLSUM, stream);
    hipError_t e = launch_colsum(jobs + j, n, M, stream, dtype);
    tm.stop();
    if (e != hipSuccess) return e;
  }
  for (int j = 0; j <= g; j += 2) {
    hipError_t e = launch_reduce(rds[j], j + 1 <= g ? &rds[j + 1] : nullptr, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qn
