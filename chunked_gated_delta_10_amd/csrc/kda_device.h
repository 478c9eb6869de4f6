// kda_device.h -- device-side building blocks shared by the KDA kernels
// (gfx950 / CDNA4, wave64).
//
// Matrix-core conventions (checked on the hardware for the gfx950 builtins):
//   v_mfma_f32_16x16x32_{f16,bf16}: lane l holds A[l%16][8*(l/16)+e] and
//   B[8*(l/16)+e][l%16] for e = 0..7, and C[4*(l/16)+j][l%16] for j = 0..3.
// Because a contraction is a sum, the contraction index may be permuted as
// long as both operands use the same permutation.  The recurrence uses the
// permutation "slice s, lane group g, element e -> index
// 32s + 4g + e (e < 4) or 32s + 16 + 4g + (e - 4) (e >= 4)", which makes the
// C layout of two stacked 16-row output tiles directly usable as a B operand
// without moving data between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int HD = 128;       // head dimension (K = V = 128)
constexpr int CH = 64;        // chunk length (tokens)
constexpr int SUB = 16;       // sub-chunk length (decay reference span)
constexpr int NSUB = CH / SUB;

// ---------------------------------------------------------------------------
// Chunk record: everything the sequential recurrence needs from one
// (chunk, head), produced by the chunk-local kernel.  All matrices are stored
// as 1 KiB MFMA operand fragments (64 lanes x 8 fp16) in the exact register
// order the consumer loads, so every fragment read is one contiguous 16-byte
// load per lane.
//   wneg[t][s]  -W = -(T diag(b) Khat)   A operand, token tile t, key slice s
//   qhat[t][s]  Qhat = exp(Gamma) . qn     A operand, token tile t, key slice s
//   kbar[kb][s] Kbar^T                     A operand, key tile kb, token slice s
//   m[t][s]     M (decayed q.k, i <= r)    A operand, token tile t, token slice s
//   tb[t][s]    T diag(b)                  A operand, token tile t, token slice s
//   gl[k]       exp(Gamma_last)[k], fp32
// Scalar gate with value heads grouped on q/k heads (one decay per
// token-head, so exp(Gamma) scales whole rows): qhat holds qn and kbar holds
// kn^T, both written only in the record of the group's first value head and
// read by all heads of the group, and gl holds exp(Gamma_r) (r < 64)
// followed by exp(Gamma_last - Gamma_r); exp(Gamma_last) = gl[63], since
// rows past a chunk's end carry no decay.
// ---------------------------------------------------------------------------
constexpr int FRAG_HALVES = 64 * 8;                   // fp16 elements per fragment
constexpr int FRAG_BYTES = FRAG_HALVES * 2;           // 1024
constexpr int REC_WNEG = 0;                           // 16 fragments
constexpr int REC_QHAT = REC_WNEG + 16 * FRAG_BYTES;  // 16 fragments
constexpr int REC_KBAR = REC_QHAT + 16 * FRAG_BYTES;  // 16 fragments
constexpr int REC_M = REC_KBAR + 16 * FRAG_BYTES;     // 8 fragments (t, s) = t*2+s
constexpr int REC_TB = REC_M + 8 * FRAG_BYTES;        // 8 fragments
constexpr int REC_GL = REC_TB + 8 * FRAG_BYTES;       // 128 floats
constexpr int REC_BYTES = REC_GL + HD * 4;            // 66048
// Records of the fused kernel add the low parts (x - fp16(x)) of Kbar^T and
// T diag(b), in the same fragment order, and a copy of the chunk's value
// rows (bf16 [64][128], rows past the chunk's end undefined), so that the
// consumers read nothing but records.
constexpr int REC_KBAR_LO = REC_BYTES;                   // 16 fragments
constexpr int REC_TB_LO = REC_KBAR_LO + 16 * FRAG_BYTES;  // 8 fragments
constexpr int REC_V = REC_TB_LO + 8 * FRAG_BYTES;         // 64 rows x 256 bytes
constexpr int REC2_BYTES = REC_V + CH * HD * 2;           // 107008

// Chunk schedule entry (int4): x = sequence, y = first token (flattened
// token index), z = valid tokens (0 = unused entry), w = chunk index within
// the sequence.
// Sequence entry (int4): x = first token, y = length, z = first chunk entry,
// w = unused.

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // round to nearest even (one v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& w, float* out) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(a[i] << 16);
    out[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ f16x8 to_f16x8(const float* x) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (f16)x[i];
  return r;
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}

// x = hi + lo with hi, lo in bf16 (about 16 significant bits together).
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)x[i];
    hi[i] = h;
    lo[i] = (__bf16)(x[i] - (float)h);
  }
}

// ---------------------------------------------------------------------------
// matrix-core wrappers
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 16x16x4: lane l holds A[l%16][l/16], B[l/16][l%16]; C as above.
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Sum over the 4 consecutive lanes l, l^1, l^2, l^3.
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}
// Sum over an aligned row of 16 lanes with DPP row rotations (no LDS traffic):
// after rotating by 8, 4, 2, 1 every lane of the row holds the row sum.
__device__ __forceinline__ float dpp_ror(float x, int n) {
  // DPP control 0x120 + n: row_ror:n (rotate right within a row of 16 lanes)
  switch (n) {
    case 8: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
    case 4: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
    case 2: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x122, 0xF, 0xF, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x121, 0xF, 0xF, false));
  }
}
__device__ __forceinline__ float rowsum16(float x) {
  x += dpp_ror(x, 8);
  x += dpp_ror(x, 4);
  x += dpp_ror(x, 2);
  x += dpp_ror(x, 1);
  return x;
}

// Sum over aligned groups of 16 lanes.
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}
__device__ __forceinline__ float sum64(float x) {
  x = sum16(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Per-token decay factor exp(g) with g = -a * softplus(x), and g itself.
// softplus(x) = ln2 * log2(1 + 2^(x log2 e)); for large x it is x to within
// 2^-28 relative, which avoids the overflow of 2^(x log2 e).
__device__ __forceinline__ void gate_decay(float x, float a, float& d, float& g) {
  constexpr float LOG2E = 1.4426950408889634f;
  constexpr float LN2 = 0.6931471805599453f;
  // v_exp_f32 / v_log_f32 directly (no denormal range handling is needed:
  // 1 + 2^y >= 1, and a decay below 2^-126 may flush to zero)
  float t2;  // softplus(x) / ln 2
  if (x > 20.f) t2 = x * LOG2E;
  else t2 = __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(x * LOG2E));
  d = __builtin_amdgcn_exp2f(-a * t2);
  g = -a * LN2 * t2;
}

// log2 of the decay factor: -a * softplus(x) / ln 2 (same evaluation as
// above, without a branch: for x > 20 the select drops the log-exp side,
// which may then be +inf but never NaN for a finite x).
__device__ __forceinline__ float gate_log2(float x, float a) {
  constexpr float LOG2E = 1.4426950408889634f;
  const float y = x * LOG2E;
  const float t = __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(y));
  return -a * (x > 20.f ? y : t);
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

}  // namespace kda
