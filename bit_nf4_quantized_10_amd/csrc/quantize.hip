// NF4 encoder and decoder kernels for gfx950.
//
// Encoding follows the page "QLoRA：冻结的 4-bit 权重怎样参与一次微调":
// per 64-weight block the absmax a (scale 1 for an all-zero block), the NF4
// code nearest to w / a with ties to the smaller index, two codes per byte
// with the first in the high nibble and code 7 as odd-length padding
// (sections "NF4 保存的是索引而不是均匀整数值", "从 NF4 索引打包成字节");
// then the double quantization of the absmax values: global mean offset,
// centred values coded in 8 bits per group of 256 with an fp32 scale
// (section "Double Quantization 压缩的是 Scale").
//
// Exactness: the nearest code is decided without dividing.  With m_j the
// midpoint of codes j and j+1 (exact in double) the code is the number of
// midpoints strictly below w / a, and "w > m_j * a" is decided exactly in
// double because m_j has at most 26 significant bits and a at most 24, so
// the product is exact.  A 256-bin table indexed by an fp32 estimate of
// w / a names the one midpoint that can lie near it (bins are 1/128 wide and
// padded by 2^-12, far below the 0.08 gap between midpoints), so each weight
// costs one double comparison.  The same argument, with the 255 midpoints of
// the linear 8-bit code, decides the second-level codes.
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "side_jobs.hpp"

namespace qn {

namespace {

constexpr int kQuantThreads = 256;
constexpr double kBinPad = 0x1p-12;

__device__ __forceinline__ float dpp_max_row8(float x) {
  // max over each aligned group of 8 lanes: xor 1, xor 2 (quad_perm), then
  // the half-row mirror pairs quads {0..3} <-> {7..4}.
  int v = __builtin_bit_cast(int, x);
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false)));
  v = __builtin_bit_cast(int, x);
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false)));
  v = __builtin_bit_cast(int, x);
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false)));
  return x;
}

// One bin of the encoder's lookup: the midpoint m_L it may straddle and L.
struct __attribute__((aligned(16))) BinEntry {
  double mid;
  int L;
  int pad;
};

// Midpoint between NF4 codes j and j+1, exact in double; +4 for j = 15 so a
// comparison against it is always false.
__device__ __forceinline__ double nf4_midpoint(int j) {
  return j < 15 ? 0.5 * (static_cast<double>(kNF4[j]) + static_cast<double>(kNF4[j + 1])) : 4.0;
}

}  // namespace

#ifndef QN_P1_DEPTH
#define QN_P1_DEPTH 3
#endif
constexpr int kP1Depth = QN_P1_DEPTH;

// Pass 1: one workgroup per group of 256 blocks (16384 weights).  Each lane
// owns 8 consecutive weights; 8 lanes form a block.  Writes the packed codes,
// the exact fp32 absmax per block and the fp64 stride-halving sum of the
// group's absmax values.
__global__ __launch_bounds__(kQuantThreads) void nf4_quant_pass1_kernel(
    const float* __restrict__ W, int64_t P, uint8_t* __restrict__ codes,
    float* __restrict__ absmax, double* __restrict__ group_sum, int32_t* __restrict__ flags,
    int32_t* __restrict__ status) {
  __shared__ BinEntry s_tab[256];
  __shared__ float s_abs[kBlock2];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  {
    // bin b covers estimates in [b/128 - 1, (b+1)/128 - 1); its entry holds
    // L, the number of midpoints below the padded lower edge, and m_L.
    const double lo = static_cast<double>(tid) / 128.0 - 1.0 - kBinPad;
    int cnt = 0;
    for (int j = 0; j < 15; ++j) cnt += nf4_midpoint(j) < lo ? 1 : 0;
    s_tab[tid] = BinEntry{nf4_midpoint(cnt), cnt, 0};
  }
  __syncthreads();

  const int64_t n1 = (P + kBlock1 - 1) / kBlock1;
  const int64_t code_bytes = (P + 1) / 2;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane & 7;
  bool bad = false;

  // The thread's 8 steps of 8 weights are loaded kP1Depth steps ahead of
  // their use, so the encoding of early steps overlaps the later loads (raw
  // buffer loads: elements past P read as +0).
  const Rsrc rw = make_rsrc(W, P * 4);
  uint4 raw[16];
  auto load_step = [&](int it) {
    const int64_t block = static_cast<int64_t>(blockIdx.x) * kBlock2 + wave * 64 + it * 8 + (lane >> 3);
    const uint32_t off = static_cast<uint32_t>((block * kBlock1 + sub * 8) * 4);
    raw[2 * it] = ld_b128(rw, off);
    raw[2 * it + 1] = ld_b128(rw, off + 16);
  };
#pragma unroll
  for (int it = 0; it < kP1Depth; ++it) load_step(it);

#pragma unroll
  for (int it = 0; it < 8; ++it) {
    if (kP1Depth < 8) {
      __builtin_amdgcn_sched_barrier(0);
      if (it + kP1Depth < 8) load_step(it + kP1Depth);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int bl = wave * 64 + it * 8 + (lane >> 3);   // block within the group
    const int64_t block = static_cast<int64_t>(blockIdx.x) * kBlock2 + bl;
    const int64_t e0 = block * kBlock1 + sub * 8;
    float w[8];
    {
      const uint4 v0 = raw[2 * it], v1 = raw[2 * it + 1];
      w[0] = __builtin_bit_cast(float, v0.x); w[1] = __builtin_bit_cast(float, v0.y);
      w[2] = __builtin_bit_cast(float, v0.z); w[3] = __builtin_bit_cast(float, v0.w);
      w[4] = __builtin_bit_cast(float, v1.x); w[5] = __builtin_bit_cast(float, v1.y);
      w[6] = __builtin_bit_cast(float, v1.z); w[7] = __builtin_bit_cast(float, v1.w);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bad |= !is_finite_bits(w[i]);
      m = fmaxf(m, fabsf(w[i]));
    }
    m = dpp_max_row8(m);
    const float a = (m == 0.0f) ? 1.0f : m;
    // fp32 estimate of w / a, used only to pick the bin (its error, a few
    // ulp, is far inside the bin padding).  Scales outside [2^-100, 2^100]
    // are first brought inside by an exact power of two, so that the
    // reciprocal is a normal number.
    const float lift = (a < 0x1p-100f) ? 0x1p64f : ((a > 0x1p100f) ? 0x1p-64f : 1.0f);
    const float inv = __builtin_amdgcn_rcpf(a * lift);
    const double ad = static_cast<double>(a);
    int bin[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // truncation, then the clamp, gives the floor's bin for every estimate
      // in [-1 - 2^-20, 1 + 2^-20]
      const int b = static_cast<int>(fmaf((w[i] * lift) * inv, 128.0f, 128.0f));
      bin[i] = min(max(b, 0), 255);
    }
    BinEntry ent[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ent[i] = s_tab[bin[i]];
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int code = ent[i].L + ((static_cast<double>(w[i]) > ent[i].mid * ad) ? 1 : 0);
      // byte i/2 of the little-endian word: even i -> high nibble
      word |= static_cast<uint32_t>(code) << (8 * (i >> 1) + ((i & 1) ? 0 : 4));
    }
    if (e0 + 8 <= P) {
      *reinterpret_cast<uint32_t*>(codes + e0 / 2) = word;
    } else if (e0 < P) {
      for (int b = 0; b < 4; ++b) {
        const int64_t byte_idx = e0 / 2 + b;
        if (byte_idx < code_bytes) codes[byte_idx] = static_cast<uint8_t>(word >> (8 * b));
      }
    }
    if (sub == 0) {
      if (block < n1) absmax[block] = a;
      s_abs[bl] = (block < n1) ? a : 0.0f;
    }
  }
  if (bad) s_bad = 1;
  __syncthreads();
  // This group's non-finite flag, for pass 2 to report; the status word is
  // cleared here (pass 2, the only writer, runs after this kernel).
  if (tid == 0) {
    flags[blockIdx.x] = s_bad ? NF4_ENONFINITE : 0;
    if (blockIdx.x == 0) status[0] = 0;
  }

  if (wave == 0) {
    // stride-halving fp64 sum of the 256 values (pairs i, i+128; i, i+64; ...)
    const double s0 = static_cast<double>(s_abs[lane]) + static_cast<double>(s_abs[lane + 128]);
    const double s1 = static_cast<double>(s_abs[lane + 64]) + static_cast<double>(s_abs[lane + 192]);
    double t = s0 + s1;
    for (int h = 32; h >= 1; h >>= 1) t = t + __shfl_down(t, h, 64);
    if (lane == 0) group_sum[blockIdx.x] = t;
  }
}

// The offset is the mean of the n1 first-level scales: the stride-halving
// fp64 sum of the n2 group sums (zero-padded to a power of two L; pass 1
// summed each group's 256 values the same way), divided by n1 in fp64 and
// rounded to fp32.  With T threads, thread t holds x[t + T s] for
// s < S = L / T and combines them with strides S/2, ..., 1 in registers;
// the levels T/2, ..., 1 then pair threads t and t + h.  Zero padding adds
// +0 exactly, so any power of two T gives the same sum.
constexpr int kMaxSumPerThread = 32;

template <int T>
__device__ __forceinline__ double tree_partial(const double* __restrict__ group_sum, int64_t n2, int t) {
  int64_t L = 1;
  while (L < n2) L <<= 1;
  const int S = L > T ? static_cast<int>(L / T) : 1;   // <= kMaxSumPerThread
  double v[kMaxSumPerThread];
#pragma unroll
  for (int i = 0; i < kMaxSumPerThread; ++i) {
    const int64_t idx = t + static_cast<int64_t>(i) * T;
    v[i] = (i < S && idx < n2) ? group_sum[idx] : 0.0;
  }
#pragma unroll
  for (int h = kMaxSumPerThread / 2; h >= 1; h >>= 1)
    if (h < S)
#pragma unroll
      for (int i = 0; i < h; ++i) v[i] = v[i] + v[i + h];
  return v[0];
}

__device__ __forceinline__ float offset_of(double total, int64_t n1) {
  return __double2float_rn(__ddiv_rn(total, static_cast<double>(n1)));
}

// One wave computes the whole sum (n2 <= 64 * kMaxSumPerThread); every
// lane receives it.
__device__ __forceinline__ double tree_sum_wave(const double* __restrict__ group_sum, int64_t n2, int lane) {
  double x = tree_partial<64>(group_sum, n2, lane);
  for (int h = 32; h >= 1; h >>= 1) x = x + __shfl_down(x, h, 64);
  return __shfl(x, 0, 64);
}

constexpr int kMeanThreads = 1024;

// Separate offset kernel for n2 > 64 * kMaxSumPerThread groups (one
// workgroup of 1024 threads; n2 <= 1024 * kMaxSumPerThread).
__global__ __launch_bounds__(kMeanThreads) void nf4_quant_mean_kernel(
    const double* __restrict__ group_sum, int64_t n2, int64_t n1, float* __restrict__ offset) {
  __shared__ double s_x[kMeanThreads];
  const int tid = threadIdx.x;
  s_x[tid] = tree_partial<kMeanThreads>(group_sum, n2, tid);
  __syncthreads();
  for (int h = kMeanThreads / 2; h >= 64; h >>= 1) {
    if (tid < h) s_x[tid] = s_x[tid] + s_x[tid + h];
    __syncthreads();
  }
  if (tid < 64) {
    double x = s_x[tid];
    for (int h = 32; h >= 1; h >>= 1) x = x + __shfl_down(x, h, 64);
    if (tid == 0) offset[0] = offset_of(x, n1);
  }
}

// Up to this many groups every pass-2 wave sums the group sums itself (the
// values are in L2) instead of waiting for a separate launch.
constexpr int64_t kSelfMeanGroups = 64 * kMaxSumPerThread;

// Pass 2: one wave per group of 256 first-level scales, 4 groups per
// workgroup; lane l holds scales 4l .. 4l+3 of its group.  c = a - offset
// (fp32), s2 = max |c| (1 if zero), q = nearest fl32(q/127) to c / s2 with
// ties to the smaller q.  Also checks that each reconstructed scale is
// finite and reports pass 1's non-finite flag of the group.
constexpr int kPass2Groups = 4;

__global__ __launch_bounds__(64 * kPass2Groups) void nf4_quant_pass2_kernel(
    const float* __restrict__ absmax, int64_t n1, const double* __restrict__ group_sum, int64_t n2,
    float* __restrict__ offset, int8_t* __restrict__ qabsmax, float* __restrict__ absmax2,
    const int32_t* __restrict__ flags, int32_t* __restrict__ status) {
  // s_mid[k + 127] = midpoint between codes k and k+1, exact in double
  __shared__ double s_mid[2 * kLevels2];
  for (int k = threadIdx.x; k < 2 * kLevels2; k += blockDim.x)
    s_mid[k] = 0.5 * (static_cast<double>(q2_value(k - kLevels2)) + static_cast<double>(q2_value(k - kLevels2 + 1)));
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kPass2Groups + (threadIdx.x >> 6);
  if (g >= n2) return;   // whole waves only
  const Rsrc ra = make_rsrc(absmax, n1 * 4);
  const int64_t i0 = g * kBlock2 + 4 * lane;
  const uint4 raw = ld_b128(ra, static_cast<uint32_t>(i0 * 4));   // scales past n1 read as 0
  float off;
  if (n2 <= kSelfMeanGroups) {
    off = offset_of(tree_sum_wave(group_sum, n2, lane), n1);
    if (g == 0 && lane == 0) offset[0] = off;
  } else {
    off = offset[0];   // written by nf4_quant_mean_kernel
  }
  const float a[4] = {__builtin_bit_cast(float, raw.x), __builtin_bit_cast(float, raw.y),
                      __builtin_bit_cast(float, raw.z), __builtin_bit_cast(float, raw.w)};
  float c[4];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = (i0 + i < n1) ? __fsub_rn(a[i], off) : 0.0f;
    m = fmaxf(m, fabsf(c[i]));
  }
  for (int h = 32; h >= 1; h >>= 1) m = fmaxf(m, __shfl_xor(m, h, 64));
  const float s2 = (m == 0.0f) ? 1.0f : m;
  const double sd = s2;
  auto mid = [&](int k) { return s_mid[k + kLevels2]; };
  uint32_t packed = 0;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // estimate, then the exact corrections against the neighbouring midpoints
    const float est = __fdiv_rn(c[i], s2);
    int q = static_cast<int>(rintf(est * static_cast<float>(kLevels2)));
    q = min(max(q, -kLevels2), kLevels2);
    const double cd = c[i];
    for (int it = 0; it < 2; ++it)
      if (q > -kLevels2 && cd <= mid(q - 1) * sd) --q;
    for (int it = 0; it < 2; ++it)
      if (q < kLevels2 && cd > mid(q) * sd) ++q;
    if (i0 + i < n1 && !is_finite_bits(absmax_hat(q, s2, off))) bad = true;
    packed |= (static_cast<uint32_t>(q) & 0xffu) << (8 * i);
  }
  if (i0 + 4 <= n1) {
    *reinterpret_cast<uint32_t*>(qabsmax + i0) = packed;
  } else {
    for (int i = 0; i < 4; ++i)
      if (i0 + i < n1) qabsmax[i0 + i] = static_cast<int8_t>(packed >> (8 * i));
  }
  const bool any_bad = __any(bad);
  if (lane == 0) {
    absmax2[g] = s2;
    if (any_bad || flags[g] != 0) atomicOr(status, NF4_ENONFINITE);
  }
}

// Single-level encoding: OR the groups' non-finite flags (pass 1) into the
// status word that pass 1 cleared.  One workgroup.
__global__ __launch_bounds__(kQuantThreads) void nf4_quant_flags_kernel(const int32_t* __restrict__ flags, int64_t n2,
                                                                        int32_t* __restrict__ status) {
  int f = 0;
  for (int64_t g = threadIdx.x; g < n2; g += kQuantThreads) f |= flags[g];
  if (__syncthreads_or(f)) {
    if (threadIdx.x == 0) atomicOr(status, NF4_ENONFINITE);
  }
}

// Decoder.  The whole code words (8 weights each) are cut into tiles of
// 256 * U words; thread t handles words tile * 256 * U + t + 256 * u, u < U,
// so every load and every 16-byte store of a wave is contiguous.  Workgroups
// stride over the tiles and request the next tile's codes and scales before
// decoding and storing the current one.  The decoded second-level values
// fl32(q / 127) come from a table in LDS, one division per thread at start.
// A final partial word (P % 8 != 0) is decoded by one thread on its own.
// Words per thread per tile, and the most workgroups a launch uses (8 per
// CU; larger tensors loop over their tiles).
#ifndef QN_DQ_U
#define QN_DQ_U 4
#endif
#ifndef QN_DQ_GRID
#define QN_DQ_GRID 2048
#endif

template <int U>
struct DqTile {
  uint32_t wd[U];
  int q[U];
  float s2[U];
};

// sshift: word index -> index of its scale (11: one per 256 blocks of 8
// words; 3: one per block, for a state without a second level).
template <int U, bool kSingle>
__device__ __forceinline__ void dq_load(DqTile<U>& t, int64_t tile, int64_t words, Rsrc rc, Rsrc rq, Rsrc rs,
                                        int sshift) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t wi = tile * (kQuantThreads * U) + threadIdx.x + static_cast<int64_t>(u) * kQuantThreads;
    const bool in = wi < words;
    t.wd[u] = ld_b32(rc, in ? static_cast<uint32_t>(wi * 4) : kMasked);
    t.q[u] = kSingle ? 0 : ld_i8(rq, in ? static_cast<uint32_t>(wi >> 3) : kMasked);
    t.s2[u] = ld_f32(rs, in ? static_cast<uint32_t>((wi >> sshift) * 4) : kMasked);
  }
}

// O: float (fp32 output) or the 16-bit tag (Bf16 / F16) of the output.
template <class O>
__device__ __forceinline__ void dq_store(void* out, int64_t e0, const float v[8]) {
  if constexpr (!std::is_same<O, float>::value) {
    uint4 pk;
    pk.x = O::pack2(v[0], v[1]);
    pk.y = O::pack2(v[2], v[3]);
    pk.z = O::pack2(v[4], v[5]);
    pk.w = O::pack2(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + e0) = pk;
  } else {
    float* o = static_cast<float*>(out) + e0;
    *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// ncols = 0: the output is the flat P-element tensor; else the weight is
// K x ncols and lands in columns 0 .. ncols-1 of an output with row stride
// out_ld (ncols a multiple of 8, so a word never straddles two rows).
template <int U, class O, bool kSingle, bool kStrided>
__device__ __forceinline__ void dq_decode(const DqTile<U>& t, int64_t tile, int64_t words, const float* s_lut,
                                          const float* s_q2, float off, void* out, uint32_t ncols,
                                          int64_t out_ld) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t wi = tile * (kQuantThreads * U) + threadIdx.x + static_cast<int64_t>(u) * kQuantThreads;
    if (wi < words) {
      const float ahat = kSingle ? t.s2[u] : __fadd_rn(__fmul_rn(s_q2[t.q[u] + kLevels2], t.s2[u]), off);
      float v[8];
      decode8(t.wd[u], ahat, s_lut, v);
      int64_t dst = wi * 8;
      if (kStrided) {
        const uint32_t e0 = static_cast<uint32_t>(wi * 8), k = e0 / ncols;
        dst = static_cast<int64_t>(k) * out_ld + (e0 - k * ncols);
      }
      dq_store<O>(out, dst, v);
    }
  }
}

// Workgroups dq_blocks and up run the side job (a split sum) instead.
template <int U, class O, bool kSingle, bool kStrided>
__global__ __launch_bounds__(kQuantThreads) void nf4_dequant_kernel(NF4View W, int64_t P, void* __restrict__ out,
                                                                    int32_t* __restrict__ status, uint32_t ncols,
                                                                    int64_t out_ld, int64_t dq_blocks, RdJob side) {
  if (blockIdx.x >= dq_blocks) {
    reduce_block(side, blockIdx.x - dq_blocks);
    return;
  }
  __shared__ float s_lut[16];
  __shared__ float s_q2[2 * kLevels2 + 2];
  const int tid = threadIdx.x;
  const int64_t n1 = (P + kBlock1 - 1) / kBlock1;
  const int64_t code_bytes = (P + 1) / 2;
  const int64_t words = P >> 3;   // whole words
  const uint8_t* __restrict__ codes = W.codes;
  constexpr bool single = kSingle;   // no second level: â = absmax[block]
  const Rsrc rc = make_rsrc(codes, words * 4);
  const Rsrc rq = make_rsrc(W.qabsmax, single ? 0 : n1);
  const Rsrc rs = single ? make_rsrc(W.absmax, n1 * 4) : make_rsrc(W.absmax2, ((n1 + kBlock2 - 1) / kBlock2) * 4);
  const int sshift = single ? 3 : 11;
  const int64_t tiles = (words + kQuantThreads * U - 1) / (kQuantThreads * U);
  int64_t tile = blockIdx.x;
  DqTile<U> cur;
  dq_load<U, kSingle>(cur, tile, words, rc, rq, rs, sshift);
  if (tid < 16) s_lut[tid] = kNF4[tid];
  if (tid <= 2 * kLevels2) s_q2[tid] = q2_value(tid - kLevels2);
  const float off = single ? 0.0f : W.offset[0];
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0 && (P & 7)) {
    uint32_t word = 0;
    for (int b = 0; b < 4; ++b)
      if (words * 4 + b < code_bytes) word |= static_cast<uint32_t>(codes[words * 4 + b]) << (8 * b);
    // odd P: the pad nibble (low half of the last byte) must be code 7
    if ((P & 1) && status && (codes[code_bytes - 1] & 15u) != 7u) atomicOr(status, NF4_EPADDING);
    float v[8];
    decode8(word, single ? W.absmax[n1 - 1] : absmax_hat(W.qabsmax[n1 - 1], W.absmax2[(n1 - 1) / kBlock2], off),
            s_lut, v);
    for (int i = 0; i < 8; ++i) {
      const int64_t e = words * 8 + i;
      if (e >= P) break;
      if constexpr (!std::is_same<O, float>::value) static_cast<uint16_t*>(out)[e] = static_cast<uint16_t>(O::pack2(v[i], 0.0f) & 0xffffu);
      else static_cast<float*>(out)[e] = v[i];
    }
  }
  // two register tiles in turn, so no copy waits on loads still in flight
  DqTile<U> nxt;
  for (; tile < tiles; tile += 2 * dq_blocks) {
    dq_load<U, kSingle>(nxt, tile + dq_blocks, words, rc, rq, rs, sshift);
    dq_decode<U, O, kSingle, kStrided>(cur, tile, words, s_lut, s_q2, off, out, ncols, out_ld);
    if (tile + dq_blocks >= tiles) break;
    dq_load<U, kSingle>(cur, tile + 2 * dq_blocks, words, rc, rq, rs, sshift);
    dq_decode<U, O, kSingle, kStrided>(nxt, tile + dq_blocks, words, s_lut, s_q2, off, out, ncols, out_ld);
  }
}

// Transposed decoder for a K x N weight: out[n][k] = RNE_bf16(fl32(C[j] * â))
// (the same values nf4_dequant_kernel writes at [k][n]).  Workgroup tile:
// 64 k x 128 n, staged through LDS so both the code reads (along n) and the
// bf16 writes (along k) are row-contiguous.
constexpr int kTPad = 66;  // bf16 per LDS row (64 k + 2): 132-byte rows

// Tile rows blockIdx.y >= ceil(K / 64) run the side jobs (two transposes)
// instead, one 32 x 32 tile per workgroup.
template <class T>
__global__ __launch_bounds__(256) void nf4_dequant_t_kernel(NF4View W, int64_t K, int64_t N,
                                                            uint16_t* __restrict__ out, TJob t0, TJob t1) {
  __shared__ float s_lut[16];
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * kTPad];
  const int64_t ky = (K + 63) / 64;
  if (blockIdx.y >= ky) {
    const int64_t id = (static_cast<int64_t>(blockIdx.y) - ky) * gridDim.x + blockIdx.x;
    uint16_t(*tt)[33] = reinterpret_cast<uint16_t(*)[33]>(tile);
    if (id < t0.nblk) transpose_block(t0, id, tt);
    else if (id - t0.nblk < t1.nblk) transpose_block(t1, id - t0.nblk, tt);
    return;
  }
  const int t = threadIdx.x;
  if (t < 16) s_lut[t] = kNF4[t];
  __syncthreads();
  // Workgroups are dealt to the 8 XCDs round-robin by linear id.  Within each
  // complete group of 16 ids, tiles 2m and 2m+1 (neighbours along n, whose
  // 64-byte code rows share 128-byte lines) go to ids q and q + 8, i.e. to
  // one XCD, so that its L2 serves the second half of every line.
  const int64_t nx = gridDim.x, L = static_cast<int64_t>(blockIdx.y) * nx + blockIdx.x;
  int64_t id = L;
  if ((L | 15) < nx * ky) id = (L & ~static_cast<int64_t>(15)) + ((L & 7) << 1) + ((L >> 3) & 1);
  const int64_t k0 = (id / nx) * 64, n0 = (id % nx) * 128;
  const bool single = W.absmax != nullptr;   // no second level: â = absmax[block]
  const float off = single ? 0.0f : W.offset[0];
  {
    const int kk = t >> 2, part = t & 3;           // row k0+kk, columns n0 + 32*part .. +31 (one block)
    const int64_t k = k0 + kk, nb = n0 + 32 * part;
    const bool ok = k < K && nb < N;
    float ahat = 0.0f;
    uint32_t w[4] = {0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
    if (ok) {
      const int64_t e0 = k * N + nb;
      ahat = single ? W.absmax[e0 >> 6] : absmax_hat(W.qabsmax[e0 >> 6], W.absmax2[e0 >> 14], off);
      const uint4 v = *reinterpret_cast<const uint4*>(W.codes + (e0 >> 1));
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v[8];
      decode8(w[c], ahat, s_lut, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[(32 * part + 8 * c + e) * kTPad + kk] = static_cast<uint16_t>(T::pack2(v[e], 0.0f));
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = t + 256 * i, nn = id >> 3, c = id & 7;
    const int64_t n = n0 + nn, k = k0 + 8 * c;
    if (n < N && k < K) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(tile + nn * kTPad + 8 * c);
      *reinterpret_cast<uint4*>(out + n * K + k) = make_uint4(src[0], src[1], src[2], src[3]);
    }
  }
}


// ----------------------------------------------------------------- launchers
hipError_t launch_quantize(const float* W, int64_t P, uint8_t* codes, int8_t* qabsmax,
                           float* absmax2, float* offset, float* absmax_out, float* ws_absmax, double* ws_gsum,
                           int32_t* ws_flags, int32_t* status, hipStream_t stream) {
  const int64_t n1 = (P + kBlock1 - 1) / kBlock1;
  const int64_t n2 = (n1 + kBlock2 - 1) / kBlock2;
  Timer t1(QK_QUANT_PASS1, stream);
  hipLaunchKernelGGL(nf4_quant_pass1_kernel, dim3(static_cast<unsigned>(n2)), dim3(kQuantThreads), 0,
                     stream, W, P, codes, absmax_out != nullptr ? absmax_out : ws_absmax, ws_gsum, ws_flags, status);
  t1.stop();
  if (absmax_out != nullptr) {
    // single-level state: the exact absmax values are the stored scales; only
    // the groups' non-finite flags remain to be reported
    Timer t3(QK_QUANT_PASS2, stream);
    hipLaunchKernelGGL(nf4_quant_flags_kernel, dim3(1), dim3(kQuantThreads), 0, stream, ws_flags, n2, status);
    t3.stop();
    return hipGetLastError();
  }
  if (n2 > kSelfMeanGroups) {
    if (n2 > static_cast<int64_t>(kMeanThreads) * kMaxSumPerThread) return hipErrorInvalidValue;
    Timer t2(QK_QUANT_MEAN, stream);
    hipLaunchKernelGGL(nf4_quant_mean_kernel, dim3(1), dim3(kMeanThreads), 0, stream, ws_gsum, n2, n1, offset);
    t2.stop();
  }
  Timer t3(QK_QUANT_PASS2, stream);
  hipLaunchKernelGGL(nf4_quant_pass2_kernel, dim3(static_cast<unsigned>((n2 + kPass2Groups - 1) / kPass2Groups)),
                     dim3(64 * kPass2Groups), 0, stream, ws_absmax, n1, ws_gsum, n2, offset, qabsmax, absmax2,
                     ws_flags, status);
  t3.stop();
  return hipGetLastError();
}

template <class O>
hipError_t dequant_launch_t(NF4View W, int64_t P, void* out, int32_t* status, hipStream_t stream, int64_t ncols,
                            int64_t out_ld, const RdJob* side) {
  constexpr int U = QN_DQ_U;
  const int64_t tiles = (P / 8 + kQuantThreads * U - 1) / (kQuantThreads * U);
  const int64_t blocks = tiles < 1 ? 1 : (tiles < QN_DQ_GRID ? tiles : QN_DQ_GRID);
  RdJob sj{};
  if (side != nullptr) sj = *side;
  const Timer t(QK_DEQUANT, stream, true);
  const dim3 grid(static_cast<unsigned>(blocks + sj.nblk)), block(kQuantThreads);
  const uint32_t nc = static_cast<uint32_t>(ncols);
  if (W.absmax != nullptr) {
    if (ncols != 0)
      hipExtLaunchKernelGGL((nf4_dequant_kernel<U, O, true, true>), grid, block, 0, stream, t.start(), t.end(), 0, W,
                            P, out, status, nc, out_ld, blocks, sj);
    else
      hipExtLaunchKernelGGL((nf4_dequant_kernel<U, O, true, false>), grid, block, 0, stream, t.start(), t.end(), 0, W,
                            P, out, status, nc, out_ld, blocks, sj);
  } else {
    if (ncols != 0)
      hipExtLaunchKernelGGL((nf4_dequant_kernel<U, O, false, true>), grid, block, 0, stream, t.start(), t.end(), 0, W,
                            P, out, status, nc, out_ld, blocks, sj);
    else
      hipExtLaunchKernelGGL((nf4_dequant_kernel<U, O, false, false>), grid, block, 0, stream, t.start(), t.end(), 0,
                            W, P, out, status, nc, out_ld, blocks, sj);
  }
  return hipGetLastError();
}

static hipError_t dequantize_with(NF4View W, int64_t P, void* out, int out_dtype, int32_t* status, hipStream_t stream,
                           int64_t ncols, int64_t out_ld, const RdJob* side) {
  if (out_dtype == NF4_OUT_BF16) return dequant_launch_t<Bf16>(W, P, out, status, stream, ncols, out_ld, side);
  if (out_dtype == NF4_OUT_F16) return dequant_launch_t<F16>(W, P, out, status, stream, ncols, out_ld, side);
  return dequant_launch_t<float>(W, P, out, status, stream, ncols, out_ld, side);
}

hipError_t launch_dequantize(NF4View W, int64_t P, void* out, int out_dtype, int32_t* status, hipStream_t stream,
                             int64_t ncols, int64_t out_ld) {
  return dequantize_with(W, P, out, out_dtype, status, stream, ncols, out_ld, nullptr);
}

hipError_t launch_dequant_bf16(NF4View W, int64_t K, int64_t N, bool transposed, uint16_t* out, hipStream_t stream,
                               int64_t out_ld, int dtype, const TJob* side_t, const RdJob* side_r) {
  if (!transposed)
    return dequantize_with(W, K * N, out, dtype == kDtypeF16 ? NF4_OUT_F16 : NF4_OUT_BF16, nullptr, stream,
                           out_ld != 0 && out_ld != N ? N : 0, out_ld, side_r);
  TJob t0{}, t1{};
  if (side_t != nullptr) {
    t0 = side_t[0];
    t1 = side_t[1];
  }
  const int64_t gx = (N + 127) / 128, ky = (K + 63) / 64;
  const int64_t side_rows = (t0.nblk + t1.nblk + gx - 1) / gx;
  Timer t(QK_DEQUANT_BF16, stream);
  dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(ky + side_rows));
  hipLaunchKernelGGL(dtype == kDtypeF16 ? nf4_dequant_t_kernel<F16> : nf4_dequant_t_kernel<Bf16>, grid, dim3(256), 0,
                     stream, W, K, N, out, t0, t1);
  t.stop();
  return hipGetLastError();
}

}  // namespace qn
