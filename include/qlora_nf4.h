/*
 * qlora_nf4.h - C ABI of the MI355X (gfx950) QLoRA NF4 linear-layer library.
 *
 * The library computes, on one GPU, the frozen-base encoding and the layer of
 * the page "QLoRA：冻结的 4-bit 权重怎样参与一次微调" (charlestar.github.io):
 *   - NF4 encoding of a weight in blocks of 64 with an fp32 absmax per block,
 *     nearest code with ties to the smaller index, two codes per byte with the
 *     first code in the high nibble and code 7 padding an odd length
 *     (sections "NF4 保存的是索引而不是均匀整数值", "从 NF4 索引打包成字节");
 *   - double quantization of those absmax values: mean offset, 8-bit codes in
 *     blocks of 256 with one fp32 scale per block (section
 *     "Double Quantization 压缩的是 Scale");
 *   - the layer Y = X Ŵ + c (X A) B and its gradients dX, dA, dB, with the
 *     packed weight frozen (sections "量化基座与可训练支路怎样相加",
 *     "冻结权重为什么仍然需要输入梯度").
 *
 * Conventions for every entry point:
 *   - Pointers named as device buffers are device pointers (HIP), owned by
 *     the caller; the library never allocates, frees or keeps them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns without synchronising.
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, dense.
 *   - Argument errors are returned synchronously (NF4_EINVAL) before any
 *     launch; nothing is enqueued then.  Errors found by the GPU (non-finite
 *     weights, a bad pad nibble) are OR-ed into the caller's device status
 *     word; read it with nf4_status_read().  Outputs are undefined when a
 *     call returns non-zero or leaves a non-zero status.
 *   - Weight layout: W is K x N row-major (index k*N + n).  Blocks of 64 run
 *     over that flat index, so the layer entry points require N % 64 == 0 so
 *     that a block never straddles two rows.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return / status codes. */
#define NF4_OK          0
#define NF4_EINVAL      1  /* bad argument (NULL, size, alignment, workspace) */
#define NF4_ENONFINITE  2  /* status bit: a weight or a reconstruction is not finite */
#define NF4_EPADDING    4  /* status bit: odd length whose pad nibble is not code 7 */
#define NF4_EHIP        8  /* a HIP runtime call or kernel launch failed */

/* 16-bit compute types of the layer (see qlora_linear_fwd_dt). */
#define NF4_COMPUTE_BF16 0
#define NF4_COMPUTE_F16  1

/* Output dtypes of nf4_dequantize. */
#define NF4_OUT_F32   0
#define NF4_OUT_BF16  1
#define NF4_OUT_F16   2   /* round-to-nearest-even fp16 (overflow gives inf) */

/* Fixed format constants: 64 weights per first-level block, 256 first-level
 * scales per second-level block, second-level codes q in [-127, 127] standing
 * for fl32(q / 127) (a signed linear 8-bit code; the page names an 8-bit
 * codebook without printing it). */
#define NF4_BLOCK1  64
#define NF4_BLOCK2  256
#define NF4_LEVELS2 127

/* The stored, frozen state of one weight tensor (all device pointers).
 * Double-quantized (absmax == NULL): codes, qabsmax, absmax2 and offset are
 * used; codes and qabsmax 16-byte aligned, absmax2 and offset 4-byte aligned.
 * Single-level (absmax != NULL; the pages' configuration with double
 * quantization switched off): codes and absmax are used, one fp32 scale per
 * 64-block, â = absmax; qabsmax, absmax2 and offset are ignored (may be NULL).
 * Any other combination makes every entry point taking the state return
 * NF4_EINVAL. */
typedef struct nf4_state {
  int64_t  numel;    /* P, the logical number of weights (>= 1)            */
  uint8_t* codes;    /* ceil(P/2) bytes, packed NF4 codes                  */
  int8_t*  qabsmax;  /* n1 = ceil(P/64) second-level codes                 */
  float*   absmax2;  /* n2 = ceil(n1/256) fp32 second-level scales         */
  float*   offset;   /* 1 fp32, the mean of the first-level absmax values  */
  float*   absmax;   /* NULL, or n1 fp32 first-level scales (no second level) */
} nf4_state_t;

/* Host only.  Sizes of the state of a P-weight tensor (closed forms of the
 * storage bill in "Double Quantization 压缩的是 Scale") and the workspace
 * nf4_quantize needs.  Any output pointer may be NULL.  NF4_EINVAL if P < 1. */
int nf4_sizes(int64_t numel, int64_t* code_bytes, int64_t* n1, int64_t* n2,
              int64_t* quant_workspace_bytes);

/* Encode P fp32 weights (device, 16-byte aligned) into `out` (all buffers
 * sized per nf4_sizes; out->numel must equal P).  With out->absmax non-NULL
 * the encoding stops at the first level: the exact per-block absmax values
 * are written there and nothing else is (storage 8*ceil(P/2) + 32*n1 bits,
 * page section "Double Quantization 压缩的是 Scale").  `workspace` is device
 * memory of at least quant_workspace_bytes, 256-byte aligned.  `status` is a
 * device int32 that the call first sets to 0; the GPU ORs NF4_ENONFINITE into
 * it if a weight is NaN/Inf or a reconstructed scale overflows (the page
 * rejects both).  Codes use the exact first-level absmax; the offset is the
 * fp64 fixed-tree mean rounded to fp32.  P must be below 2^29 (the fp32
 * input under 2 GiB); NF4_EINVAL otherwise. */
int nf4_quantize(const float* W, const nf4_state_t* out, void* workspace,
                 int64_t workspace_bytes, int32_t* status, void* stream);

/* Decode a state to P weights: ŵ = fl32(C[j] * â) with
 * â = fl32(fl32(fl32(q/127) * s2) + offset) (or â = absmax for a
 * single-level state), written as fp32
 * (NF4_OUT_F32) or round-to-nearest-even bf16 (NF4_OUT_BF16).  `out` is
 * device memory of P elements, 16-byte aligned.  `status` (device int32,
 * may be NULL) receives NF4_EPADDING if P is odd and the last pad nibble is
 * not 7 (the page's unpack check); it is not cleared first. */
int nf4_dequantize(const nf4_state_t* state, void* out, int out_dtype,
                   int32_t* status, void* stream);

/* Host only.  Workspace sizes (bytes) of qlora_linear_fwd and
 * qlora_linear_bwd for the given shape; NF4_EINVAL for a shape the layer
 * entry points reject. */
int qlora_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t r,
                          int64_t* fwd_bytes, int64_t* bwd_bytes);

/* Forward of one QLoRA linear (page section "量化基座与可训练支路怎样相加"):
 *   Z = X A            (M x r, bf16 output, fp32 accumulation)
 *   Y = X Ŵ + c Z B    (M x N, bf16 output, fp32 accumulation)
 * X: M x K bf16, W: state of the K x N weight (W->numel == K*N), A: K x r
 * bf16, B: r x N bf16, c = alpha / r.  Ŵ is exactly the bf16 weight that
 * nf4_dequantize(W, NF4_OUT_BF16) returns.  Z is written for the backward
 * pass; with Z = NULL it is computed in the workspace and not returned.
 * Requirements: M, K, N, r >= 1, N % 64 == 0, K % 8 == 0, r % 8 == 0,
 * r <= 256, M <= 2^20, K, N <= 2^24, each of M*K, M*N, K*N, K*r and r*N
 * below 2^29 elements (every bf16 operand under 1 GiB, so that 32-bit
 * buffer offsets suffice), all pointers 16-byte aligned, workspace >= fwd_bytes.  The
 * state is only read.  M <= 16 runs the memory-bound dequant-GEMV kernels;
 * M >= 192 dequantizes Ŵ to bf16 in the workspace and runs a dense GEMM. */
int qlora_linear_fwd(int64_t M, int64_t K, int64_t N, int64_t r,
                     const uint16_t* X, const nf4_state_t* W,
                     const uint16_t* A, const uint16_t* B, float c,
                     uint16_t* Y, uint16_t* Z,
                     void* workspace, int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): qlora_linear_fwd
 * (bf16 compute) with its scratch taken from a device array of
 * NF4_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on,
 * instead of a workspace argument.  The call allocates nothing.  Shapes
 * whose forward workspace (qlora_workspace_bytes' fwd_bytes) exceeds that
 * size return NF4_EINVAL: in practice the small-M (dequant-GEMV) and
 * fused-decode forwards, not the M >= 192 one, whose workspace holds the
 * dequantized weight.  Z may be NULL (then it is computed in the scratch).
 * The scratch keeps the last call's contents; calls that overlap on one GPU
 * (two streams, or two host threads) race on it and must be serialised by
 * the caller.  The stream must belong to the current device.  Results are
 * bit-identical to qlora_linear_fwd's. */
#define NF4_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
int qlora_linear_fwd_noalloc(int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X,
                             const nf4_state_t* W, const uint16_t* A, const uint16_t* B, float c,
                             uint16_t* Y, uint16_t* Z, void* stream);

/* Backward of the same linear given G = dL/dY (page section
 * "冻结权重为什么仍然需要输入梯度"):
 *   dZ = c G Bᵀ,  dA = Xᵀ dZ (K x r fp32),  dB = c Zᵀ G (r x N fp32),
 *   dX = G Ŵᵀ + dZ Aᵀ (M x K bf16; skipped when dX is NULL).
 * Z is the forward's Z, or NULL: then Z = X A is recomputed in the
 * workspace (one more read of X; for M > 16 with the forward's own kernels,
 * so the same bits).  The frozen state receives no gradient and is only
 * read.  Same requirements as the forward; workspace >= bwd_bytes.  dA and
 * dB are computed with deterministic (fixed-order) split reductions. */
int qlora_linear_bwd(int64_t M, int64_t K, int64_t N, int64_t r,
                     const uint16_t* G, const uint16_t* X, const uint16_t* Z,
                     const nf4_state_t* W, const uint16_t* A, const uint16_t* B,
                     float c, uint16_t* dX, float* dA, float* dB,
                     void* workspace, int64_t workspace_bytes, void* stream);

/* Element types of the adapter matrices passed to qlora_merge. */
#define NF4_AB_BF16 0
#define NF4_AB_F32  1
#define NF4_AB_F16  2

/* Merge the adapter into the frozen base for re-export (page section
 * "Merge 后还是不是训练时的函数": the trained function is Ŵ + cAB, merged in
 * high precision; re-quantizing the result is a separate step, done by
 * passing W_merged to nf4_quantize):
 *   W_merged[k][n] = fl32(ŵ[k][n] + c * sum_t A[k][t] B[t][n])
 * with ŵ the fp32 reconstruction nf4_dequantize(W, NF4_OUT_F32) returns, the
 * sum accumulated in fp64 for t = 0 .. r-1 in order, c * sum and the addition
 * in fp64, and one rounding to fp32.  A: K x r, B: r x N, row-major, of
 * element type ab_dtype (NF4_AB_BF16 or NF4_AB_F32, e.g. fp32 master copies),
 * (NF4_AB_F16: fp16) aligned to their element size; W_merged: K x N fp32, 16-byte aligned,
 * caller-owned.  Requirements: K, N, r >= 1, r <= 65536, W->numel == K*N,
 * K*N, K*r and r*N below 2^29.  Any N is allowed (blocks run over the flat
 * index).  NF4_EINVAL otherwise.  The state is only read. */
int qlora_merge(int64_t K, int64_t N, int64_t r, const nf4_state_t* W, const void* A, const void* B,
                int ab_dtype, float c, float* W_merged, void* stream);

/* One plain SGD step on the adapter after qlora_linear_bwd (page section
 * "一次完整反向与有限差分": only A and B move, v <- v - lr * g):
 *   p' = fl32(p - fl32(lr * g)),  bf16 parameter <- RNE_bf16(p')
 * where p is the fp32 master copy when A_master / B_master are given (both
 * or neither; they are updated to p'), else the bf16 parameter itself.
 * A, B: bf16 K x r and r x N (updated in place); dA, dB: fp32 gradients of
 * the same shapes (as qlora_linear_bwd returns them).  Requirements: K, N,
 * r >= 1, K*r and r*N below 2^29, each pointer aligned to its element size.
 * NF4_EINVAL otherwise. */
int qlora_sgd_step(int64_t K, int64_t N, int64_t r, uint16_t* A, uint16_t* B, const float* dA, const float* dB,
                   float lr, float* A_master, float* B_master, void* stream);
/* The same step for parameters of the 16-bit type param_dtype
 * (NF4_COMPUTE_BF16 or NF4_COMPUTE_F16). */
int qlora_sgd_step_dt(int param_dtype, int64_t K, int64_t N, int64_t r, uint16_t* A, uint16_t* B,
                      const float* dA, const float* dB, float lr, float* A_master, float* B_master,
                      void* stream);

/* Grouped linears sharing one input (e.g. the q, k, v projections, or gate
 * and up: adapters on several projections of one layer, page
 * "qlora-4bit-quantization-finetune" section "训练全流程" (Q and V) and page
 * "SFT（四）" §22.1 (all linear layers); each member is the layer of page
 * "QLoRA：冻结的 4-bit 权重怎样参与一次微调" section "量化基座与可训练支路怎样相加").  g members (1 <= g <= 8),
 * member i a K x N[i] weight (state W[i]) with its own rank-r adapter; the
 * members' outputs and adapters are stored side by side:
 *   Y = [Y_1 .. Y_g] (M x Ntot, Ntot = sum N[i]),  Z = [Z_1 .. Z_g] (M x g r),
 *   A = [A_1 .. A_g] (K x g r),                   B = [B_1 .. B_g] (r x Ntot),
 * and Y_i = X Ŵ_i + c Z_i B_i, Z_i = X A_i, i.e. the layer above per member,
 * with X read once.  Every N[i] must be a multiple of 256 and r a multiple
 * of 8 (so no 8-element chunk of Z, A or B straddles two members); the concatenated
 * shape (M, K, Ntot, g r) must meet qlora_linear_fwd's requirements; W is a
 * host array of g states.  All members are dequantized to a 16-bit workspace
 * and multiplied by one dense GEMM for any M (fp16: qlora_grouped_fwd_dt
 * below).  Host only: */
int qlora_grouped_workspace_bytes(int64_t M, int64_t K, int g, const int64_t* N, int64_t r,
                                  int64_t* fwd_bytes, int64_t* bwd_bytes);
int qlora_grouped_fwd(int64_t M, int64_t K, int g, const int64_t* N, int64_t r, const uint16_t* X,
                      const nf4_state_t* W, const uint16_t* A, const uint16_t* B, float c,
                      uint16_t* Y, uint16_t* Z, void* workspace, int64_t workspace_bytes, void* stream);
/* Backward of the grouped forward given G = dL/dY (M x Ntot, side by side):
 * dZ_i = c G_i B_iᵀ, dA = Xᵀ [dZ_1 .. dZ_g] (K x g r fp32), dB = [c Z_iᵀ G_i]
 * (r x Ntot fp32), dX = sum_i (G_i Ŵ_iᵀ + dZ_i A_iᵀ) (skipped when NULL). */
int qlora_grouped_bwd(int64_t M, int64_t K, int g, const int64_t* N, int64_t r, const uint16_t* G,
                      const uint16_t* X, const uint16_t* Z, const nf4_state_t* W, const uint16_t* A,
                      const uint16_t* B, float c, uint16_t* dX, float* dA, float* dB,
                      void* workspace, int64_t workspace_bytes, void* stream);

/* The 16-bit compute type of the layer (page "SFT（四）：QLoRA的4-bit量化与LoRA微调原理" §20: BF16 where supported,
 * else FP16).  The _dt entry points take it as their first argument; X, A,
 * B, G, Y, Z and dX are then of that type (uint16_t bit patterns), the
 * dequantized weight is RNE_T(ŵ) (fp16: overflow past 65504 gives inf), and
 * every product accumulates in fp32.  qlora_linear_fwd / _bwd are the
 * NF4_COMPUTE_BF16 case; requirements and results are otherwise the same. */
int qlora_linear_fwd_dt(int compute_dtype, int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* X,
                        const nf4_state_t* W, const uint16_t* A, const uint16_t* B, float c, uint16_t* Y,
                        uint16_t* Z, void* workspace, int64_t workspace_bytes, void* stream);
int qlora_linear_bwd_dt(int compute_dtype, int64_t M, int64_t K, int64_t N, int64_t r, const uint16_t* G,
                        const uint16_t* X, const uint16_t* Z, const nf4_state_t* W, const uint16_t* A,
                        const uint16_t* B, float c, uint16_t* dX, float* dA, float* dB, void* workspace,
                        int64_t workspace_bytes, void* stream);
/* The grouped calls (qlora_grouped_fwd / _bwd above) in the compute type
 * compute_dtype (page "SFT（四）：QLoRA的4-bit量化与LoRA微调原理" §20): X, A, B, G, Y, Z and dX
 * of that type, the stacked weight RNE_T(ŵ), dA and dB fp32, fp32
 * accumulation.  qlora_grouped_fwd / _bwd are the NF4_COMPUTE_BF16 case;
 * requirements, errors and results are otherwise the same. */
int qlora_grouped_fwd_dt(int compute_dtype, int64_t M, int64_t K, int g, const int64_t* N, int64_t r,
                         const uint16_t* X, const nf4_state_t* W, const uint16_t* A, const uint16_t* B, float c,
                         uint16_t* Y, uint16_t* Z, void* workspace, int64_t workspace_bytes, void* stream);
int qlora_grouped_bwd_dt(int compute_dtype, int64_t M, int64_t K, int g, const int64_t* N, int64_t r,
                         const uint16_t* G, const uint16_t* X, const uint16_t* Z, const nf4_state_t* W,
                         const uint16_t* A, const uint16_t* B, float c, uint16_t* dX, float* dA, float* dB,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* Synchronise `stream`, then copy the device status word to *host_value.
 * Returns NF4_EHIP if the copy fails, else NF4_OK. */
int nf4_status_read(const int32_t* status, int32_t* host_value, void* stream);

/* Instrumentation.  Kernel ids for the timer below. */
#define QK_QUANT_PASS1  0
#define QK_QUANT_MEAN   1
#define QK_QUANT_PASS2  2
#define QK_DEQUANT      3
#define QK_LORA_DOWN    4   /* Z = X A (split-K partials)               */
#define QK_FWD_GEMM     5   /* fused dequant-GEMM + LoRA epilogue       */
#define QK_FWD_GEMV     6   /* small-M dequant-GEMV                     */
#define QK_BWD_DZ       7   /* dZ = c G Bᵀ partials                     */
#define QK_BWD_DX       8   /* dX = G Ŵᵀ + dZ Aᵀ                        */
#define QK_BWD_COLSUM   9   /* dA = Xᵀ dZ and dB = c Zᵀ G partials      */
#define QK_DEQUANT_BF16 10  /* Ŵ (or Ŵᵀ) to bf16 for the M >= 192 GEMMs */
#define QK_REDUCE       11  /* fixed-order split reductions             */
#define QK_MERGE        12  /* adapter merge W' = fl32(ŵ + cAB)          */
#define QK_SGD          13  /* adapter SGD step                          */
#define QK_NUM_KERNELS  14

/* When enabled, the library records a pair of hipEvents on the launch
 * stream around every launch of kernel `kernel_id`.  qlora_timer_read
 * waits for the recorded events, returns the summed elapsed milliseconds
 * and the launch count since the last read, and resets them.  Host-side
 * only; meant for benchmarks (it adds two event records per launch).
 * qlora_timer_enable creates the slot's pool of 8192 events the first time
 * (NF4_EHIP if that fails); the pool is the library's only held state and
 * stays until the process ends.  Launches never create events: beyond 4096
 * launches between two reads, further launches are neither timed nor
 * counted. */
int qlora_timer_enable(int kernel_id, int enable);
int qlora_timer_read(int kernel_id, double* total_ms, int64_t* launches);

/* Short English text for a return code or status bit set. */
const char* nf4_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
