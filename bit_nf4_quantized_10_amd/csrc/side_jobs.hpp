// Two small jobs of the layer that run either as launches of their own or as
// extra workgroups of another launch (the dequantize launches of the
// two-pass GEMM path), which saves a launch and its ramp:
//   - TJob: dst[c][r] = RNE_16(scale * src[r][c]) for a rows x cols matrix of
//     the layer's 16-bit type, in 32 x 32 LDS tiles (scale 1 copies the bits);
//     it produces Aᵀ for the rank-r products and the forward's LoRA extension
//     operand (c B)ᵀ, rounded once.
//   - RdJob: out = scale * sum_s part[s] over the split partials in split
//     order, optionally transposed from [rows][cols] to [cols][rows]; fp32
//     and/or 16-bit outputs.
// Both are plain data; a workgroup of 256 threads runs one block of a job.
#pragma once

#include "common.hpp"

namespace qn {

// RNE to the layer's 16-bit type (f16: fp16, else bf16) and back to fp32.
__device__ __forceinline__ uint16_t half_of(float x, int f16) {
  return static_cast<uint16_t>((f16 ? F16::pack2(x, 0.0f) : Bf16::pack2(x, 0.0f)) & 0xffffu);
}
__device__ __forceinline__ float widen_of(uint32_t bits16, int f16) {
  return f16 ? F16::widen(bits16) : Bf16::widen(bits16);
}

struct TJob {
  const uint16_t* src;
  uint16_t* dst;
  int64_t rows, cols;
  float scale;
  int64_t bx, nblk;   // 32-column tiles per tile row, tiles in this job
  int f16;            // elements are fp16 (else bf16)
};

inline TJob make_tjob(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols, float scale, int f16) {
  const int64_t bx = (cols + 31) / 32;
  return TJob{src, dst, rows, cols, scale, bx, bx * ((rows + 31) / 32), f16};
}

// Tile b of job j; `tile` is 32 x 33 uint16 of LDS.  All 256 threads call it.
__device__ __forceinline__ void transpose_block(const TJob& j, int64_t b, uint16_t (*tile)[33]) {
  const int64_t r0 = (b / j.bx) * 32, c0 = (b % j.bx) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int64_t r = r0 + i, c = c0 + tx;
    uint16_t v = (r < j.rows && c < j.cols) ? j.src[r * j.cols + c] : 0;
    if (j.scale != 1.0f) v = half_of(j.scale * widen_of(v, j.f16), j.f16);
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < j.cols && r < j.rows) j.dst[c * j.rows + r] = tile[tx][i];
  }
}

struct RdJob {
  const float* part;
  int64_t splits, rows, cols;
  float scale;
  int transpose;
  float* out_f32;
  uint16_t* out_bf16;
  int64_t nblk;
  int64_t out_ld;   // row stride of the output (cols, or rows when transposed, for a dense result)
  int f16;          // the 16-bit output is fp16 (else bf16)
};

inline RdJob make_rdjob(const float* part, int64_t splits, int64_t rows, int64_t cols, float scale, bool transpose,
                        float* out_f32, uint16_t* out_16, int f16) {
  int64_t blocks = (rows * cols + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  return RdJob{part, splits, rows, cols, scale, transpose ? 1 : 0, out_f32, out_16, blocks, transpose ? rows : cols,
               f16};
}

// Block blk of job J (grid-stride over J.nblk blocks).
__device__ __forceinline__ void reduce_block(const RdJob& J, int64_t blk) {
  const int64_t count = J.rows * J.cols;
  for (int64_t i = blk * 256 + threadIdx.x; i < count; i += J.nblk * 256) {
    float s = 0.0f;
    int64_t k = 0;
    for (; k + 8 <= J.splits; k += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = J.part[(k + u) * count + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; k < J.splits; ++k) s += J.part[k * count + i];
    s *= J.scale;
    const int64_t o = J.transpose ? (i % J.cols) * J.out_ld + i / J.cols : (i / J.cols) * J.out_ld + i % J.cols;
    if (J.out_f32) J.out_f32[o] = s;
    if (J.out_bf16) J.out_bf16[o] = half_of(s, J.f16);
  }
}

}  // namespace qn
