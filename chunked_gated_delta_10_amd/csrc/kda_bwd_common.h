// kda_bwd_common.h -- pieces shared by the backward kernels of both gate
// modes (kda_bwd.hip: one decay per token-head; kda_bwd_pc.hip: one decay per
// key channel): LDS matrix strides, the per-(chunk, head) record layout,
// operand-fragment loads, the schedule entry of a job and the fp32 solve of
// T = (I + A)^-1.
#pragma once

#include "kda_bwd.h"
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int NTH = 512;              // threads of the chunk-parallel kernels (8 waves)
constexpr int LDW = HD + 8;           // halves per row: fp16 matrices of 128 columns
constexpr int LDN = CH + 8;           // halves per row: fp16 matrices of 64 columns
constexpr int LDF = CH + 4;           // floats per row: fp32 64 x 64 matrices
constexpr int MAT_W = CH * LDW * 2;   // bytes of a 64 x 128 fp16 matrix
constexpr int MAT_N = CH * LDN * 2;   // 64 x 64 fp16
constexpr int MAT_NT = HD * LDN * 2;  // 128 x 64 fp16
constexpr int MAT_F = CH * LDF * 4;   // 64 x 64 fp32
constexpr int BR_PHI = 0;             // record: Phi fragments [8 row tiles][4 slices]
constexpr int BR_BC = 32 * FRAG_BYTES;  // Bc fragments [8 row tiles][2 slices]
constexpr int BR_T = BR_BC + 16 * FRAG_BYTES;  // T, fp16 [64][64]
constexpr int BR_PHIT = BR_T + CH * CH * 2;    // Phi^T fragments [8 row tiles][4 slices]
constexpr int BR_GC = BR_PHIT + 32 * FRAG_BYTES;  // Gc fragments [8 row tiles][2 slices]
static_assert(BR_GC + 16 * FRAG_BYTES == BREC_BYTES, "record size");
// per-channel gate only: M (fp16 [64][64], lower with the diagonal) and the
// decay-masked key Gram matrix H (fp16 [64][64], strictly lower) with A = diag(b) H
constexpr int BR_M = BR_GC + 16 * FRAG_BYTES;
constexpr int BR_HK = BR_M + CH * CH * 2;
static_assert(BR_HK + CH * CH * 2 == BREC_PC_BYTES, "per-channel record size");

__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float softplus_(float x) { return x > 20.f ? x : log1pf(expf(x)); }
__device__ __forceinline__ float sigmoid_(float x) { return 1.f / (1.f + expf(-x)); }

// Operand fragments (lane l: row r0 + l % 16, contraction index k0 + 8 (l / 16) + e).
// Contraction index contiguous in X (row-major X[row][k]): one 16-byte read.
__device__ __forceinline__ f16x8 frag_rm(const f16* X, int ld, int r0, int k0, int lane) {
  return *reinterpret_cast<const f16x8*>(X + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
// Contraction index strided (X stored [k][row]).
__device__ __forceinline__ f16x8 frag_cm(const f16* X, int ld, int r0, int k0, int lane) {
  const f16* p = X + (k0 + 8 * (lane >> 4)) * ld + r0 + (lane & 15);
  f16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = p[e * ld];
  return v;
}
// Strided fragment of a row-scaled matrix: element e is s[k] X[k][r0 + l % 16], k = k0 + 8 (l / 16) + e.
__device__ __forceinline__ f16x8 frag_cm_scaled(const f16* X, int ld, const float* s, int r0, int k0, int lane) {
  const int k = k0 + 8 * (lane >> 4);
  const f16* p = X + k * ld + r0 + (lane & 15);
  f16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (f16)(s[k + e] * (float)p[e * ld]);
  return v;
}

// (first token, length) of schedule entry e
__device__ __forceinline__ int2 entry_of(const BwdParams& p, int e) {
  if (p.dense_T >= 0) {
    const int T = p.dense_T, nc = (T + CH - 1) / CH, b = e / nc, c = e - b * nc;
    return make_int2(b * T + c * CH, min(CH, T - c * CH));
  }
  const int4 ce = p.chunks[e];
  return make_int2(ce.y, ce.z);
}

// (I + N)^-1 of a strictly lower 16 x 16 block on fp32 matrix cores: blocked
// forward substitution with block sizes doubling 1 -> 2 -> 4 -> 8 -> 16
// (D_2k = D_k - D_k M_k D_k, every intermediate a block of the inverse or of
// N).  Nc, NT: N and N^T in C layout; result in C layout.
__device__ __forceinline__ f32x4 mul_cc_(const f32x4& XT, const f32x4& Y) {
  f32x4 z = mma_f32(XT[0], Y[0], zero4());
  z = mma_f32(XT[1], Y[1], z);
  z = mma_f32(XT[2], Y[2], z);
  return mma_f32(XT[3], Y[3], z);
}
__device__ __forceinline__ f32x4 lower_inverse16(const f32x4& Nc, const f32x4& NT, int l16, int lg) {
  f32x4 D, DT;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * lg + j, c = l16;
    const float eye = r == c ? 1.f : 0.f;
    const bool in1 = (r >> 1) == (c >> 1) && r != c;
    D[j] = eye - (in1 ? Nc[j] : 0.f);
    DT[j] = eye - (in1 ? NT[j] : 0.f);
  }
#pragma unroll
  for (int k = 2; k < SUB; k *= 2) {
    f32x4 MT;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * lg + j, c = l16;
      MT[j] = ((r / (2 * k)) == (c / (2 * k)) && (r / k) != (c / k)) ? NT[j] : 0.f;
    }
    const f32x4 P = mul_cc_(MT, D);
    const f32x4 Q = mul_cc_(DT, P);
    if (2 * k < SUB) DT = DT - mul_cc_(P, DT);
    D = D - Q;
  }
  return D;
}

// Off-diagonal 16 x 16 blocks of T in block column a: T_ba = -T_bb sum_{a<=j<b} A_bj T_ja.
// The contraction index of product jj is 4 lg + jj, so C layout is the B operand in place.
template <int A>
__device__ __forceinline__ void t_column(const float* AF, float* TF, f32x4 Td, int l16, int lg) {
  f32x4 Tc[NSUB];
  Tc[A] = Td;
#pragma unroll
  for (int b = A + 1; b < NSUB; ++b) {
    f32x4 X = zero4();
#pragma unroll
    for (int j = A; j < b; ++j) {
      const float4 av = *reinterpret_cast<const float4*>(&AF[(SUB * b + l16) * LDF + SUB * j + 4 * lg]);
      X = mma_f32(av.x, Tc[j][0], X);
      X = mma_f32(av.y, Tc[j][1], X);
      X = mma_f32(av.z, Tc[j][2], X);
      X = mma_f32(av.w, Tc[j][3], X);
    }
    const float4 tb = *reinterpret_cast<const float4*>(&TF[(SUB * b + l16) * LDF + SUB * b + 4 * lg]);
    f32x4 Y = mma_f32(tb.x, X[0], zero4());
    Y = mma_f32(tb.y, X[1], Y);
    Y = mma_f32(tb.z, X[2], Y);
    Y = mma_f32(tb.w, X[3], Y);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      Tc[b][jj] = -Y[jj];
      TF[(SUB * b + 4 * lg + jj) * LDF + SUB * A + l16] = -Y[jj];
    }
  }
}

// T = (I + A)^-1 from A (fp32, strictly lower, complete in AF: the caller
// synchronises first) into TF (fp32) and T16 (fp16 row-major, zero above the
// diagonal blocks); ends with a barrier.  Diagonal 16 x 16 blocks by
// lower_inverse16, then one wave per block column.
__device__ void solve_T(const float* AF, float* TF, f16* T16) {
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l16 = lane & 15, lg = lane >> 4;
  f32x4 Td = zero4();
  if (w < NSUB) {  // diagonal blocks
    const int n = w;
    f32x4 Nc, NT;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Nc[j] = AF[(SUB * n + 4 * lg + j) * LDF + SUB * n + l16];
      NT[j] = AF[(SUB * n + l16) * LDF + SUB * n + 4 * lg + j];
    }
    Td = lower_inverse16(Nc, NT, l16, lg);
#pragma unroll
    for (int j = 0; j < 4; ++j) TF[(SUB * n + 4 * lg + j) * LDF + SUB * n + l16] = Td[j];
  }
  __syncthreads();
  if (w == 0) t_column<0>(AF, TF, Td, l16, lg);
  else if (w == 1) t_column<1>(AF, TF, Td, l16, lg);
  else if (w == 2) t_column<2>(AF, TF, Td, l16, lg);
  __syncthreads();
  for (int i = t; i < CH * CH; i += NTH) {
    const int r = i >> 6, c = i & 63;
    T16[r * LDN + c] = (f16)((r >> 4) >= (c >> 4) ? TF[r * LDF + c] : 0.f);
  }
  __syncthreads();
}

}  // namespace
}  // namespace kda
