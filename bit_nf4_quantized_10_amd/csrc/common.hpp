// Device-side building blocks shared by the gfx950 kernels of the QLoRA NF4
// library: the NF4 codebook, scale reconstruction, bf16 packing and the MFMA
// fragment types.  Nothing here is used by the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlora_nf4.h"

namespace qn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock1 = NF4_BLOCK1;   // weights per first-level block
constexpr int kBlock2 = NF4_BLOCK2;   // first-level scales per second-level block
constexpr int kLevels2 = NF4_LEVELS2;

// The sixteen NF4 reconstruction values in ascending order (7 negative, an
// exact zero at code 7, 8 positive), as exact fp32 numbers; the table printed
// in section "从 NF4 索引打包成字节" of the page
// "QLoRA：冻结的 4-bit 权重怎样参与一次微调".
__constant__ static const float kNF4[16] = {
    -0x1p+0f,        -0x1.647362p-1f, -0x1.0cd66p-1f,  -0x1.94654p-2f,
    -0x1.23449ap-2f, -0x1.7a6a7ep-3f, -0x1.74f0e2p-4f, 0.0f,
    0x1.45f5fep-4f,  0x1.4995c6p-3f,  0x1.f809bap-3f,  0x1.5a0674p-2f,
    0x1.c3497p-2f,   0x1.200f56p-1f,  0x1.722766p-1f,  0x1p+0f,
};

// Second-level code value fl32(q / 127): one correctly rounded fp32 divide.
__device__ __forceinline__ float q2_value(int q) {
  return __fdiv_rn(static_cast<float>(q), static_cast<float>(kLevels2));
}

// Reconstructed first-level scale: decode the 8-bit code, then add the
// offset back, as two separately rounded fp32 operations (no FMA).
__device__ __forceinline__ float absmax_hat(int q, float s2, float offset) {
  return __fadd_rn(__fmul_rn(q2_value(q), s2), offset);
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ bool is_finite_bits(float x) {
  return (__builtin_bit_cast(uint32_t, x) & 0x7f800000u) != 0x7f800000u;
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


// Decode the 8 nibbles of one little-endian code word (byte i holds codes
// 2i in the high nibble and 2i+1 in the low nibble) with a per-block scale
// held in `ahat`, into 8 fp32 reconstructions fl32(C[j] * ahat).  `lut` is
// the NF4 table staged in LDS.
__device__ __forceinline__ void decode8(uint32_t w, float ahat, const float* lut, float out[8]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t byte = (w >> (8 * b)) & 0xffu;
    out[2 * b] = __fmul_rn(lut[byte >> 4], ahat);
    out[2 * b + 1] = __fmul_rn(lut[byte & 15u], ahat);
  }
}

// ---- raw buffer access: loads whose offset is at or past the byte count
// return zeros, so masked loads need no branches (an offset of 0x80000000
// marks a masked lane; every tensor is smaller than 2 GiB).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kMasked = 0x80000000u;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0x7fffffff ? bytes : 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(n),
                                           0x00020000);
}
__device__ __forceinline__ uint4 ld_b128(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 ld_b64(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t ld_b32(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
__device__ __forceinline__ float ld_f32(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ int ld_i8(Rsrc r, uint32_t off) {
  return static_cast<int>(static_cast<int8_t>(__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0)));
}

// s_waitcnt immediate for gfx9: vmcnt split over bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; an all-ones field does not wait.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// ---- the two 16-bit compute types of the layer (page "SFT（四）：QLoRA的4-bit量化与LoRA微调原理" §20: BF16, or FP16
// where BF16 is not wanted).  Each tag gives the MFMA operand vector, the
// 16x16x32 and 32x32x16 MFMAs with fp32 accumulation, the fp32 -> 16-bit
// round-to-nearest-even packing of two values, and the widening to fp32.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct Bf16 {
  typedef bf16x8 v8;
  static constexpr int kDtype = 0;
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
  __device__ static __forceinline__ float widen(uint32_t bits16) { return bf16_bits_to_f32(bits16); }
  __device__ static __forceinline__ f32x4 mfma16(const v8& a, const v8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x16 mfma32(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

struct F16 {
  typedef f16x8 v8;
  static constexpr int kDtype = 1;
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float widen(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
  }
  __device__ static __forceinline__ f32x4 mfma16(const v8& a, const v8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x16 mfma32(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// The 16 reconstructions RNE_T(fl32(C[j] * ahat)) of one block, written as
// 32 bytes (entry j at byte 2j) to 16-byte aligned LDS.
template <class T = Bf16>
__device__ __forceinline__ void write_block_table(uint16_t* tab, float ahat) {
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = T::pack2(__fmul_rn(kNF4[2 * j], ahat), __fmul_rn(kNF4[2 * j + 1], ahat));
  reinterpret_cast<uint4*>(tab)[0] = make_uint4(w[0], w[1], w[2], w[3]);
  reinterpret_cast<uint4*>(tab)[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

}  // namespace qn
