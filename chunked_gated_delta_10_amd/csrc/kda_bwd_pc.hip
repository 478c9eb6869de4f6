// kda_bwd_pc.hip -- backward pass with one decay per key channel (the KDA
// gate of the cuLA / FlashKDA pages): the coefficient and gradient stages.
// The chains over chunks are the scalar-gate ones (kda_bwd.hip), fed with
// this file's records.
//
// Per chunk, with Gamma the per-channel cumulative log-decay (every exponent
// below is <= 0 where it is evaluated), Qhat = exp(Gamma) . qn,
// Khat = exp(Gamma) . kn, Kbar = exp(Gamma_L - Gamma) . kn and the
// decay-masked Gram matrices
//   M[r][i] = sum_c qn_rc kn_ic exp(Gamma_rc - Gamma_ic)  (i <= r)
//   H[r][i] = sum_c kn_rc kn_ic exp(Gamma_rc - Gamma_ic)  (i < r),  A = diag(b) H,
// the chunk is S_c+1 = Phi^T S_c + Gc V_c and its adjoint dS_c = Phi dS' + Bc dO'
// with
//   Phi^T = D_L - Kbar^T T diag(b) Khat,  Gc = Kbar^T T diag(b),
//   Bc = Qhat^T - Khat^T diag(b) T^T M^T,  D_L = Diag(exp(Gamma_L)).
// The gradients of one chunk, from S_c and dS' (R = V - Khat S_c,
// U = T diag(b) R):
//   dU = M^T dO' + Kbar dS',  Y = T^T dU,  dV = diag(b) Y,
//   dQhat = dO' S_c^T,  dKhat = -dV S_c^T,  dKbar = U dS'^T,
//   dM = lower(dO' U^T),  dT = dU (b R)^T,  dA = strict_lower(-T^T dT T^T),
//   dH = diag(b) dA,  db = rowsum(Y . R) + rowsum(dA . H),
// and through the masks, with E_ric = exp(Gamma_rc - Gamma_ic):
//   Yq_rc = sum_i dM_ri kn_ic E_ric,  X_rc = sum_i dH_ri kn_ic E_ric,
//   Z_ic  = sum_r (dH_ri kn_rc + dM_ri qn_rc) E_ric,
//   dqn = exp(Gamma) . dQhat + Yq,
//   dkn = exp(Gamma) . dKhat + exp(Gamma_L - Gamma) . dKbar + X + Z,
//   dGamma = qn . dqn + kn . (exp(Gamma) . dKhat - exp(Gamma_L - Gamma) . dKbar + X - Z),
// plus, on the chunk's last token, sum_r Kbar . dKbar + exp(Gamma_L) . rowsum(S_c . dS')
// (per key channel); dg is the reverse cumulative sum of dGamma over the chunk.
//
// Decay masks: the chunk is cut into four 16-token blocks.  For r in block
// rb and i in an earlier block, with p = 16 rb - 1 (the last token before
// block rb),
//   E_ric = exp(Gamma_rc - Gamma_pc) * exp(Gamma_pc - Gamma_ic),
// both factors <= 1, so those blocks are fp16 matrix-core products with the
// factors folded into the operands.  Inside a block every E_ric is one
// exponential of a non-positive number, evaluated exactly in fp32 (no range
// limit for harsh gates).
#include "kda_bwd_common.h"

namespace kda {

namespace {

constexpr int LGS = HD + 4;          // floats per row of the fp32 64 x 128 gate matrix
constexpr int MAT_G = CH * LGS * 4;  // bytes of it

// per-token and per-channel values of a job
struct __attribute__((aligned(16))) PcRows {
  float b[CH], nq[CH], nk[CH];
  float lgl[HD];  // Gamma_L log2(e) per key channel
  float el[HD];   // exp(Gamma_L) per key channel
};

__device__ __forceinline__ void load_f16x16(const f16* src, float* x) {
  const f16x8 a = *reinterpret_cast<const f16x8*>(src), b = *reinterpret_cast<const f16x8*>(src + 8);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = (float)a[j];
    x[8 + j] = (float)b[j];
  }
}
__device__ __forceinline__ void load_f32x16(const float* src, float* x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 v = reinterpret_cast<const float4*>(src)[j];
    x[4 * j] = v.x;
    x[4 * j + 1] = v.y;
    x[4 * j + 2] = v.z;
    x[4 * j + 3] = v.w;
  }
}

// Prologue of both kernels.  Thread t -> row r = t / 8, key channels
// c0 = 16 (t % 8) .. c0 + 15.  Normalised k rows to KN (fp16) and kv, q's raw
// entries to qraw (normalised later by the caller with R.nq), the gates'
// log2 cumulative sums along the chunk to LG (rows past the chunk's end
// repeat the last one), b, the norms, Gamma_L.  part: 2 KB of scratch.
// Contains barriers; LG and R are complete on return.
__device__ void load_pc(const BwdParams& p, int tok0, int len, int h, int hq, f16* KN, float* LG, float* part,
                        PcRows& R, uint4 (&qraw)[2], float (&kv)[16]) {
  const int t = threadIdx.x, r = t >> 3, c0 = (t & 7) * 16;
  const bool live = r < len;
  const int tr = tok0 + min(r, len - 1);  // loads clamped, values selected
  const size_t base = ((size_t)tr * p.H_qk + hq) * HD + c0;
  qraw[0] = *reinterpret_cast<const uint4*>(p.q + base);
  qraw[1] = *reinterpret_cast<const uint4*>(p.q + base + 8);
  const uint4 k0 = *reinterpret_cast<const uint4*>(p.k + base), k1 = *reinterpret_cast<const uint4*>(p.k + base + 8);
  const size_t gb = ((size_t)tr * p.H + h) * HD + c0;
  const uint4 g0 = *reinterpret_cast<const uint4*>(p.g_raw + gb), g1 = *reinterpret_cast<const uint4*>(p.g_raw + gb + 8);
  const float a = expf(p.A_log[h]), m = live ? 1.f : 0.f;
  float qv[16], gv[16];
  unpack_bf16x8(qraw[0], qv);
  unpack_bf16x8(qraw[1], qv + 8);
  unpack_bf16x8(k0, kv);
  unpack_bf16x8(k1, kv + 8);
  unpack_bf16x8(g0, gv);
  unpack_bf16x8(g1, gv + 8);
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    qv[j] *= m;
    kv[j] *= m;
    sq += qv[j] * qv[j];
    sk += kv[j] * kv[j];
    gv[j] = m * gate_log2(gv[j], a);
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    sq += __shfl_xor(sq, o);
    sk += __shfl_xor(sk, o);
  }
  const float nq = sqrtf(sq + 1e-6f), nk = sqrtf(sk + 1e-6f), ik = 1.f / nk;
#pragma unroll
  for (int j = 0; j < 16; ++j) kv[j] *= ik;
  *reinterpret_cast<f16x8*>(KN + r * LDW + c0) = to_f16x8(kv);
  *reinterpret_cast<f16x8*>(KN + r * LDW + c0 + 8) = to_f16x8(kv + 8);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    reinterpret_cast<float4*>(LG + r * LGS + c0)[j] = make_float4(gv[4 * j], gv[4 * j + 1], gv[4 * j + 2], gv[4 * j + 3]);
  if ((t & 7) == 0) {
    R.nq[r] = nq;
    R.nk[r] = nk;
  }
  if (t < CH) R.b[t] = t < len ? sigmoid_(p.beta[(size_t)(tok0 + t) * p.H + h]) : 0.f;
  __syncthreads();
  // cumulative sums down the rows: thread -> channel c, rows 16 qd .. 16 qd + 15
  const int c = t & (HD - 1), qd = t >> 7;
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = LG[(16 * qd + j) * LGS + c];
#pragma unroll
  for (int j = 1; j < 16; ++j) x[j] += x[j - 1];
  part[qd * HD + c] = x[15];
  __syncthreads();
  float before = 0.f;
  for (int q2 = 0; q2 < qd; ++q2) before += part[q2 * HD + c];
#pragma unroll
  for (int j = 0; j < 16; ++j) LG[(16 * qd + j) * LGS + c] = x[j] + before;
  if (qd == 3) {
    R.lgl[c] = x[15] + before;
    R.el[c] = exp2f(x[15] + before);
  }
  __syncthreads();
}

// Operand fragment (8 contraction indices k = k0 + 8 (lane / 16) + e over key
// channels, row r) of exp2(LG[r][k] - LG[p][k]) X[r][k] (sign = +1: r after p)
// or of exp2(LG[p][k] - LG[r][k]) X[r][k] (sign = -1: r at or before p); the
// exponent is <= 0 on those sides and clamped at 0 against rounding.
__device__ __forceinline__ f16x8 frag_decay_rm(const f16* X, const float* LG, int r, int p, int k0, float sign) {
  const f16x8 x = *reinterpret_cast<const f16x8*>(X + r * LDW + k0);
  const float4 a0 = *reinterpret_cast<const float4*>(LG + r * LGS + k0);
  const float4 a1 = *reinterpret_cast<const float4*>(LG + r * LGS + k0 + 4);
  const float4 b0 = *reinterpret_cast<const float4*>(LG + p * LGS + k0);
  const float4 b1 = *reinterpret_cast<const float4*>(LG + p * LGS + k0 + 4);
  const float la[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  const float lb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  f16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (f16)(exp2f(fminf(sign * (la[e] - lb[e]), 0.f)) * (float)x[e]);
  return o;
}
// The same along a column: contraction index k = row of X (k0 + 8 (lane / 16) + e), key channel c;
// factor exp2(LG[p][c] - LG[k][c]) for k <= p (before) or exp2(LG[k][c] - LG[p][c]) for k > p (after).
__device__ __forceinline__ f16x8 frag_decay_cm(const f16* X, const float* LG, int c, int p, int k0, bool after) {
  const float lp = LG[p * LGS + c];
  f16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = k0 + e;
    const float d = LG[k * LGS + c] - lp;
    const bool live = after ? k > p : k <= p;
    o[e] = (f16)((live ? exp2f(fminf(after ? d : -d, 0.f)) : 0.f) * (float)X[k * LDW + c]);
  }
  return o;
}

}  // namespace

// ---------------------------------------------------------------------------
// coef_pc_kernel: per (chunk, head), the masked Gram matrices M and H, T, and
// the records of both chains (Phi, Bc, Phi^T, Gc as fp16 A-operand fragments
// in the chain's contraction order, T, M, H).  Two workgroups per CU (72 KB of
// LDS): qn, kn and the gates live only through the Gram products; A and T in
// fp32 for the solve, then M and T (fp16), take their space; Khat and Kbar are
// formed after the solve from registers, over the solve's space; Qhat waits in
// Bc's record slot until the last product reads it.
// ---------------------------------------------------------------------------
namespace {
// Gram products: qn, kn, the gates; the prologue's scan scratch after them
constexpr int C_QN = 0, C_KN = C_QN + MAT_W, C_LG = C_KN + MAT_W, C_PART = C_LG + MAT_G;
// solve: A and T in fp32, M and T in fp16
constexpr int C_AF = 0, C_TF = C_AF + MAT_F, C_M = C_TF + MAT_F, C_T = C_M + MAT_N;
// operators: Khat, Kbar over A and T (fp32); M, T kept; Y1^T, then Z1^T, after them
constexpr int C_KH = 0, C_KB = C_KH + MAT_W, C_YZ = C_T + MAT_N, C_END = C_YZ + MAT_NT;
static_assert(C_PART + 4 * HD * 4 <= C_END, "scan scratch (4 x 128 floats) inside the layout");
static_assert(C_KB + MAT_W <= C_M, "Khat, Kbar over the fp32 solve");
static_assert(2 * (C_END + (int)sizeof(PcRows)) <= 160 * 1024, "two workgroups per CU");
}  // namespace

// two workgroups per CU: at least four waves per SIMD
__global__ __launch_bounds__(NTH, 4) void bwd_coef_pc_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C_END];
  __shared__ PcRows R;
  f16* QN = reinterpret_cast<f16*>(smem + C_QN);
  f16* KN = reinterpret_cast<f16*>(smem + C_KN);
  float* LG = reinterpret_cast<float*>(smem + C_LG);
  float* AF = reinterpret_cast<float*>(smem + C_AF);
  float* TF = reinterpret_cast<float*>(smem + C_TF);
  f16* M16 = reinterpret_cast<f16*>(smem + C_M);
  f16* T16 = reinterpret_cast<f16*>(smem + C_T);
  f16* KH = reinterpret_cast<f16*>(smem + C_KH);
  f16* KB = reinterpret_cast<f16*>(smem + C_KB);
  f16* YZt = reinterpret_cast<f16*>(smem + C_YZ);

  const int job = blockIdx.x, e = job / p.H, h = job - e * p.H, hq = h / (p.H / p.H_qk);
  const int2 ce = entry_of(p, e);
  const int tok0 = ce.x, len = ce.y;
  if (len <= 0) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l16 = lane & 15, lg = lane >> 4;
  uint8_t* rec = p.brec + (size_t)job * p.rec_bytes;
  f16* HKg = reinterpret_cast<f16*>(rec + BR_HK);
  f16* QHg = reinterpret_cast<f16*>(rec + BR_BC);  // Qhat rows until Bc replaces them

  uint4 qraw[2];
  float kv[16], lr[16];
  load_pc(p, tok0, len, h, hq, KN, LG, reinterpret_cast<float*>(smem + C_PART), R, qraw, kv);
  const int r = t >> 3, c0 = (t & 7) * 16;
  float qv[16];
  {  // qn rows to LDS, Qhat rows to the record
    unpack_bf16x8(qraw[0], qv);
    unpack_bf16x8(qraw[1], qv + 8);
    const float iq = r < len ? 1.f / R.nq[r] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) qv[j] *= iq;
    *reinterpret_cast<f16x8*>(QN + r * LDW + c0) = to_f16x8(qv);
    *reinterpret_cast<f16x8*>(QN + r * LDW + c0 + 8) = to_f16x8(qv + 8);
    load_f32x16(LG + r * LGS + c0, lr);
    float qh[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) qh[j] = exp2f(lr[j]) * qv[j];
    *reinterpret_cast<f16x8*>(QHg + r * HD + c0) = to_f16x8(qh);
    *reinterpret_cast<f16x8*>(QHg + r * HD + c0 + 8) = to_f16x8(qh + 8);
  }
  __syncthreads();  // qn complete
  // ---- diagonal blocks, exactly: thread (r, 16 channels), partners i of r's block in two groups of 8;
  // the sums over the 8 lanes of the row (channel groups) halve the partners at every step, so lane
  // cg = t % 8 ends with the full sums of partner 8 g + cg of group g
  const int b0 = r & ~15, cg = t & 7;
  float q1[2], k1[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float hq[8], hk[8];
#pragma unroll
    for (int jl = 0; jl < 8; ++jl) {
      const int i = b0 + 8 * g + jl;
      float li[16], ki[16];
      load_f32x16(LG + i * LGS + c0, li);
      load_f16x16(KN + i * LDW + c0, ki);
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float E = exp2f(fminf(lr[j] - li[j], 0.f)) * ki[j];
        sq += qv[j] * E;
        sk += kv[j] * E;
      }
      hq[jl] = sq;
      hk[jl] = sk;
    }
    float q4[4], k4[4], q2[2], k2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool hi = cg & 4;
      q4[j] = (hi ? hq[4 + j] : hq[j]) + __shfl_xor(hi ? hq[j] : hq[4 + j], 4);
      k4[j] = (hi ? hk[4 + j] : hk[j]) + __shfl_xor(hi ? hk[j] : hk[4 + j], 4);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool hi = cg & 2;
      q2[j] = (hi ? q4[2 + j] : q4[j]) + __shfl_xor(hi ? q4[j] : q4[2 + j], 2);
      k2[j] = (hi ? k4[2 + j] : k4[j]) + __shfl_xor(hi ? k4[j] : k4[2 + j], 2);
    }
    const bool hi = cg & 1;
    q1[g] = (hi ? q2[1] : q2[0]) + __shfl_xor(hi ? q2[0] : q2[1], 1);
    k1[g] = (hi ? k2[1] : k2[0]) + __shfl_xor(hi ? k2[0] : k2[1], 1);
  }
  f16x8 khb[4];  // this row's Khat, Kbar entries (fp16), kept until the solve's space is free
  {
    float kh[16], kb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      kh[j] = exp2f(lr[j]) * kv[j];
      kb[j] = exp2f(R.lgl[c0 + j] - lr[j]) * kv[j];
    }
    khb[0] = to_f16x8(kh);
    khb[1] = to_f16x8(kh + 8);
    khb[2] = to_f16x8(kb);
    khb[3] = to_f16x8(kb + 8);
  }
  // ---- off-diagonal 16 x 16 blocks (waves 0..5; in registers until the gates are dead)
  f32x4 HQ = zero4(), HK = zero4();
  const int rt = w < 1 ? 1 : (w < 3 ? 2 : 3), ct = w < 1 ? 0 : (w < 3 ? w - 1 : w - 3);
  if (w < 6) {
    const int pr = 16 * rt - 1;
#pragma unroll
    for (int s = 0; s < HD / 32; ++s) {
      const int k0 = 32 * s + 8 * lg;
      const f16x8 bk = frag_decay_rm(KN, LG, 16 * ct + l16, pr, k0, -1.f);
      HQ = mma_f16(frag_decay_rm(QN, LG, 16 * rt + l16, pr, k0, 1.f), bk, HQ);
      HK = mma_f16(frag_decay_rm(KN, LG, 16 * rt + l16, pr, k0, 1.f), bk, HK);
    }
  }
  __syncthreads();  // qn, kn and the gates read for the last time: A and M take their space
  if (w < 6) {
    const int i = 16 * ct + l16;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int rr = 16 * rt + 4 * lg + jj;
      M16[rr * LDN + i] = (f16)HQ[jj];
      AF[rr * LDF + i] = R.b[rr] * HK[jj];
      HKg[rr * CH + i] = (f16)HK[jj];
    }
  } else {  // zero blocks above the diagonal
#pragma unroll
    for (int q3 = 0; q3 < 3; ++q3) {
      const int blk = 3 * (w - 6) + q3;  // (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
      const int zr = blk < 3 ? 0 : (blk < 5 ? 1 : 2), zc = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
      const int i = 16 * zc + l16;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int rr = 16 * zr + 4 * lg + jj;
        M16[rr * LDN + i] = (f16)0.f;
        AF[rr * LDF + i] = 0.f;
        HKg[rr * CH + i] = (f16)0.f;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {  // the diagonal blocks' entries of this lane
    const int i = b0 + 8 * g + cg;
    M16[r * LDN + i] = (f16)(i <= r ? q1[g] : 0.f);
    AF[r * LDF + i] = i < r ? R.b[r] * k1[g] : 0.f;
    HKg[r * CH + i] = (f16)(i < r ? k1[g] : 0.f);
  }
  __syncthreads();  // A, M complete
  solve_T(AF, TF, T16);
  // T and M (fp16 rows) for the gradient kernel: thread -> row t / 8, columns 8 (t % 8) ..
  __builtin_nontemporal_store(*reinterpret_cast<const f16x8*>(T16 + (t >> 3) * LDN + 8 * (t & 7)), reinterpret_cast<f16x8*>(rec + BR_T + t * 16));
  __builtin_nontemporal_store(*reinterpret_cast<const f16x8*>(M16 + (t >> 3) * LDN + 8 * (t & 7)), reinterpret_cast<f16x8*>(rec + BR_M + t * 16));
  // Khat, Kbar rows over the solve's fp32 space (dead: solve_T ended with a barrier)
  *reinterpret_cast<f16x8*>(KH + r * LDW + c0) = khb[0];
  *reinterpret_cast<f16x8*>(KH + r * LDW + c0 + 8) = khb[1];
  *reinterpret_cast<f16x8*>(KB + r * LDW + c0) = khb[2];
  *reinterpret_cast<f16x8*>(KB + r * LDW + c0 + 8) = khb[3];
  __syncthreads();  // Khat, Kbar complete

  const int d = 16 * w + l16;  // this lane's key column of the 128-wide results
  // Y1 = T^T Kbar: rows i (4 tiles), columns d (tile w); K = 64
  {
    f32x4 Y1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Y1[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 bk = frag_cm(KB, LDW, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) Y1[i] = mma_f16(frag_cm(T16, LDN, 16 * i, 32 * s, lane), bk, Y1[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f16x4*>(YZt + d * LDN + 16 * i + 4 * lg) =
          f16x4{(f16)Y1[i][0], (f16)Y1[i][1], (f16)Y1[i][2], (f16)Y1[i][3]};
    // Gc = Kbar^T T diag(b): its transpose is diag(b) Y1, rows i, columns d
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f16x8 o;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) o[4 * hh + jj] = (f16)(R.b[32 * s + 16 * hh + 4 * lg + jj] * Y1[2 * s + hh][jj]);
      __builtin_nontemporal_store(o, reinterpret_cast<f16x8*>(rec + BR_GC + (w * 2 + s) * FRAG_BYTES + lane * 16));
    }
  }
  __syncthreads();
  // Phi^T = D_L - Y1^T diag(b) Khat: rows d' (8 tiles), columns d (tile w); K = 64 over tokens
  {
    f32x4 A[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 bb = frag_cm_scaled(KH, LDW, R.b, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) A[i] = mma_f16(frag_rm(YZt, LDN, 16 * i, 32 * s, lane), bb, A[i]);
    }
    const float eL = R.el[d];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 o;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * s + 4 * lg + jj, d1 = d0 + 16;
        o[jj] = (f16)((d0 == d ? eL : 0.f) - A[2 * s][jj]);
        o[4 + jj] = (f16)((d1 == d ? eL : 0.f) - A[2 * s + 1][jj]);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<f16x8*>(rec + BR_PHI + (w * 4 + s) * FRAG_BYTES + lane * 16));
    }
  }
  // Phi = D_L - (diag(b) Khat)^T Y1: rows d (8 tiles), columns d' (tile w); its C layout is the
  // fragment order of Phi^T, the forward chain's operator
  {
    const f16x8 by0 = frag_rm(YZt, LDN, 16 * w, 0, lane), by1 = frag_rm(YZt, LDN, 16 * w, 32, lane);
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // row tiles 4 half .. 4 half + 3: slices 2 half, 2 half + 1
      f32x4 A[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i] = mma_f16(frag_cm_scaled(KH, LDW, R.b, 16 * (4 * half + i), 0, lane), by0, zero4());
        A[i] = mma_f16(frag_cm_scaled(KH, LDW, R.b, 16 * (4 * half + i), 32, lane), by1, A[i]);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int s = 2 * half + s2;
        f16x8 o;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d0 = 32 * s + 4 * lg + jj, d1 = d0 + 16;
          o[jj] = (f16)((d0 == d ? R.el[d0] : 0.f) - A[2 * s2][jj]);
          o[4 + jj] = (f16)((d1 == d ? R.el[d1] : 0.f) - A[2 * s2 + 1][jj]);
        }
        __builtin_nontemporal_store(o, reinterpret_cast<f16x8*>(rec + BR_PHIT + (w * 4 + s) * FRAG_BYTES + lane * 16));
      }
    }
  }
  // this lane's Qhat entries (rows i = 32 s + 16 hh + 4 lg + jj, column d), read back now and
  // used after the next product
  f16 qh[2][2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) qh[s][hh][jj] = QHg[(32 * s + 16 * hh + 4 * lg + jj) * HD + d];
  __syncthreads();  // Y1^T read for the last time
  // Z1 = T diag(b) Khat
  {
    f32x4 Z1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Z1[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 bb = frag_cm_scaled(KH, LDW, R.b, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) Z1[i] = mma_f16(frag_rm(T16, LDN, 16 * i, 32 * s, lane), bb, Z1[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f16x4*>(YZt + d * LDN + 16 * i + 4 * lg) =
          f16x4{(f16)Z1[i][0], (f16)Z1[i][1], (f16)Z1[i][2], (f16)Z1[i][3]};
  }
  __syncthreads();  // Z1 complete; every lane's Qhat entries are in registers: Bc may replace them
  // Bc^T = Qhat - M Z1: rows i (4 tiles), columns d (tile w); K = 64
  {
    f32x4 B[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) B[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 bz = frag_rm(YZt, LDN, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) B[i] = mma_f16(frag_rm(M16, LDN, 16 * i, 32 * s, lane), bz, B[i]);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f16x8 o;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) o[4 * hh + jj] = (f16)((float)qh[s][hh][jj] - B[2 * s + hh][jj]);
      __builtin_nontemporal_store(o, reinterpret_cast<f16x8*>(rec + BR_BC + (w * 2 + s) * FRAG_BYTES + lane * 16));
    }
  }
}

// ---------------------------------------------------------------------------
// grad_pc_kernel: per (chunk, head), every gradient of the chunk's inputs.
// Eight waves, one workgroup per CU.  64 x 128 results: wave w holds column
// tile w (16 key or value columns), all 64 rows, in matrix-core C layout, from
// product to product; 64 x 64 ones: row tile w / 2, column tiles 2 (w % 2) + j.
// The exact diagonal-block terms are formed by thread (row, 16 channels) and
// added to the C-layout sums through one fp32 exchange matrix.
// ---------------------------------------------------------------------------
namespace {
constexpr int P_KN = 0, P_LG = P_KN + MAT_W, P_MT = P_LG + MAT_G, P_T = P_MT + MAT_N, P_DO = P_T + MAT_N,
              P_BR = P_DO + MAT_W, P_U = P_BR + MAT_W, P_DU = P_U + MAT_W, P_DR = P_DU + MAT_W,
              P_END = P_DR + MAT_W;
constexpr int P_KH = P_U, P_KB = P_DU;  // Khat, Kbar until R and Kbar dS' are formed
constexpr int P_PART = P_DR;            // scan scratch of the prologue
// after the last reads of dO', bR, U, dU, dR: the 64 x 64 results
constexpr int P_DH = P_DO, P_DM = P_DH + MAT_N, P_DHT = P_DM + MAT_N, P_DMT = P_DHT + MAT_N, P_DT = P_DMT + MAT_N,
              P_X1 = P_DT + MAT_N;
constexpr int P_XB = P_DT;  // fp32 exchange matrix, over dT and X1^T once dA is formed
constexpr int P_QN = P_MT;  // qn, over M^T and T once dA is formed
static_assert(P_XB + MAT_G <= P_END && P_X1 + MAT_N <= P_END, "64 x 64 results fit");
static_assert(MAT_W <= 2 * MAT_N, "qn fits over M^T and T");

// Per-row and per-channel sums over the waves are formed in a fixed order (each wave's partial sum
// stored, then added up wave by wave), so that a call's results do not depend on the order in which the
// waves finish.
struct __attribute__((aligned(16))) PcRed {
  float db[CH], qd[CH], kd[CH];
  float dgl[HD];  // sum_r Kbar . dKbar per key channel
  float sdl[HD];  // sum_v S_c . dS' per key channel
  float part[8][CH];  // the waves' partial row sums
  float dalw[8];      // the waves' partial sums of dA_log
};
}  // namespace

__global__ __launch_bounds__(NTH) void bwd_grad_pc_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[P_END];
  __shared__ PcRows R;
  __shared__ PcRed red;
  f16* KN = reinterpret_cast<f16*>(smem + P_KN);
  float* LG = reinterpret_cast<float*>(smem + P_LG);
  f16* Mt = reinterpret_cast<f16*>(smem + P_MT);
  f16* T16 = reinterpret_cast<f16*>(smem + P_T);
  f16* DO = reinterpret_cast<f16*>(smem + P_DO);
  f16* BR = reinterpret_cast<f16*>(smem + P_BR);
  f16* U = reinterpret_cast<f16*>(smem + P_U);
  f16* DU = reinterpret_cast<f16*>(smem + P_DU);
  f16* DR = reinterpret_cast<f16*>(smem + P_DR);
  f16* KH = reinterpret_cast<f16*>(smem + P_KH);
  f16* KB = reinterpret_cast<f16*>(smem + P_KB);
  f16* DH = reinterpret_cast<f16*>(smem + P_DH);
  f16* DMm = reinterpret_cast<f16*>(smem + P_DM);
  f16* DHt = reinterpret_cast<f16*>(smem + P_DHT);
  f16* DMt = reinterpret_cast<f16*>(smem + P_DMT);
  f16* DT = reinterpret_cast<f16*>(smem + P_DT);
  f16* X1t = reinterpret_cast<f16*>(smem + P_X1);
  float* XB = reinterpret_cast<float*>(smem + P_XB);
  f16* QN = reinterpret_cast<f16*>(smem + P_QN);

  const int job = blockIdx.x, G = p.H / p.H_qk;
  const int e = job / p.H, h = job - e * p.H, hq = h / G;
  const int2 ce = entry_of(p, e);
  const int tok0 = ce.x, len = ce.y;
  if (len <= 0) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l16 = lane & 15, lg = lane >> 4;
  const f16* Sg = reinterpret_cast<const f16*>(p.states) + (size_t)job * HD * HD;    // [V][K]
  const f16* dSg = reinterpret_cast<const f16*>(p.dstates) + (size_t)job * HD * HD;  // [V][K]
  const uint8_t* rec = p.brec + (size_t)job * p.rec_bytes;
  const size_t vrow = (size_t)p.H * HD;
  const uint16_t* vbase = p.v + (size_t)tok0 * vrow + (size_t)h * HD;
  const int vc = 16 * w + l16;  // this lane's column of the 64 x 128 results
  const int rt = w >> 1, ct0 = 2 * (w & 1);

  // global operands issued first: S_c and dS' as B operands (rows d of kn-type products, columns v),
  // this lane's value entries, T and M rows, this lane's entries of H
  f16x8 sfr[4], dsfr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    sfr[s] = *reinterpret_cast<const f16x8*>(Sg + (size_t)vc * HD + 32 * s + 8 * lg);
    dsfr[s] = *reinterpret_cast<const f16x8*>(dSg + (size_t)vc * HD + 32 * s + 8 * lg);
  }
  uint16_t vraw[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) vraw[i][jj] = vbase[(size_t)min(16 * i + 4 * lg + jj, len - 1) * vrow + vc];
  const f16x8 trow = *reinterpret_cast<const f16x8*>(rec + BR_T + t * 16);
  const f16x8 mrow = *reinterpret_cast<const f16x8*>(rec + BR_M + t * 16);
  const f16* HKg = reinterpret_cast<const f16*>(rec + BR_HK);
  f16 hkv[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) hkv[j][jj] = HKg[(16 * rt + 4 * lg + jj) * CH + 16 * (ct0 + j) + l16];
  {  // T and M^T: thread -> row t / 8, columns 8 (t % 8) ..
    const int r = t >> 3, c0 = 8 * (t & 7);
    *reinterpret_cast<f16x8*>(T16 + r * LDN + c0) = trow;
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) Mt[(c0 + e2) * LDN + r] = mrow[e2];
  }
  {  // dO' rows (fp16, zero past the chunk's end): thread -> row t / 8, 16 columns
    const int r = t >> 3, c0 = (t & 7) * 16;
    float x[16];
    const uint16_t* src = p.dout + (size_t)(tok0 + min(r, len - 1)) * vrow + (size_t)h * HD + c0;
    unpack_bf16x8(*reinterpret_cast<const uint4*>(src), x);
    unpack_bf16x8(*reinterpret_cast<const uint4*>(src + 8), x + 8);
    const float sc = r < len ? p.scale : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] *= sc;
    *reinterpret_cast<f16x8*>(DO + r * LDW + c0) = to_f16x8(x);
    *reinterpret_cast<f16x8*>(DO + r * LDW + c0 + 8) = to_f16x8(x + 8);
  }
  uint4 qraw[2];
  float kv[16];
  load_pc(p, tok0, len, h, hq, KN, LG, reinterpret_cast<float*>(smem + P_PART), R, qraw, kv);
  const int r8 = t >> 3, c0 = (t & 7) * 16;  // the row-and-channels mapping
  {  // Khat, Kbar rows
    float lr[16], kh[16], kb[16];
    load_f32x16(LG + r8 * LGS + c0, lr);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      kh[j] = exp2f(lr[j]) * kv[j];
      kb[j] = exp2f(R.lgl[c0 + j] - lr[j]) * kv[j];
    }
    *reinterpret_cast<f16x8*>(KH + r8 * LDW + c0) = to_f16x8(kh);
    *reinterpret_cast<f16x8*>(KH + r8 * LDW + c0 + 8) = to_f16x8(kh + 8);
    *reinterpret_cast<f16x8*>(KB + r8 * LDW + c0) = to_f16x8(kb);
    *reinterpret_cast<f16x8*>(KB + r8 * LDW + c0 + 8) = to_f16x8(kb + 8);
  }
  // sum_v S_c . dS' per key channel d = 32 s + 8 lg + e (v = this lane's column); the waves' partial
  // sums in dR's space (free until dR is formed, several barriers later)
  float* psdl = reinterpret_cast<float*>(smem + P_DR);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) {
      const float x = rowsum16((float)sfr[s][e2] * (float)dsfr[s][e2]);
      if (l16 == 0) psdl[w * HD + 32 * s + 8 * lg + e2] = x;
    }
  __syncthreads();  // Khat, Kbar complete
  if (t < HD) {
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) a += psdl[q * HD + t];
    red.sdl[t] = a;
  }
  // ---- KS = Khat S (rows r, columns v); R = V - KS; bR;  KD = Kbar dS' ------
  f32x4 RR[4], KD[4];
  {
    f32x4 KS[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) KS[i] = KD[i] = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        KS[i] = mma_f16(frag_rm(KH, LDW, 16 * i, 32 * s, lane), sfr[s], KS[i]);
        KD[i] = mma_f16(frag_rm(KB, LDW, 16 * i, 32 * s, lane), dsfr[s], KD[i]);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * i + 4 * lg + jj;
        const float vv = bf(vraw[i][jj]) * (r < len ? 1.f : 0.f);
        RR[i][jj] = vv - KS[i][jj];
        BR[r * LDW + vc] = (f16)(R.b[r] * RR[i][jj]);
      }
  }
  __syncthreads();  // bR complete; Khat, Kbar read for the last time
  // ---- U^T = (b R)^T T^T -> U row-major;  dU = KD + M^T dO' -----------------
  {
    f32x4 UT[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) UT[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 a = frag_cm(BR, LDW, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) UT[i] = mma_f16(a, frag_rm(T16, LDN, 16 * i, 32 * s, lane), UT[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f16x4*>(U + (16 * i + l16) * LDW + 16 * w + 4 * lg) =
          f16x4{(f16)UT[i][0], (f16)UT[i][1], (f16)UT[i][2], (f16)UT[i][3]};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 b = frag_cm(DO, LDW, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) KD[i] = mma_f16(frag_rm(Mt, LDN, 16 * i, 32 * s, lane), b, KD[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) DU[(16 * i + 4 * lg + jj) * LDW + vc] = (f16)KD[i][jj];
  }
  __syncthreads();  // U, dU complete
  // ---- Y = T^T dU; dV = diag(b) Y; db += rowsum(Y . R) ------------------------
  {
    f32x4 Y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Y[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 b = frag_cm(DU, LDW, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[i] = mma_f16(frag_cm(T16, LDN, 16 * i, 32 * s, lane), b, Y[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * i + 4 * lg + jj;
        const float dv = R.b[r] * Y[i][jj];
        if (r < len) __builtin_nontemporal_store(dv, p.dv + (size_t)(tok0 + r) * vrow + (size_t)h * HD + vc);
        DR[r * LDW + vc] = (f16)dv;
        const float db = rowsum16(Y[i][jj] * RR[i][jj]);
        if (l16 == 0) red.part[w][r] = db;
      }
  }
  __syncthreads();  // dR complete
  if (t < CH) {
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) a += red.part[q][t];
    red.db[t] = a;
  }
  // ---- dQhat = dO' S^T, dKhat = -dR S^T, dKbar = U dS'^T (rows r, key columns: tile w)
  f32x4 dqn[4], dkn[4], dgk[4];
  {
    f32x4 SD[4], DRS[4], UD[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) SD[i] = DRS[i] = UD[i] = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 bs, bd;  // S^T and dS'^T operands: element e = X[v = 32 s + 8 lg + e][d]
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const size_t o = (size_t)(32 * s + 8 * lg + e2) * HD + vc;
        bs[e2] = Sg[o];
        bd[e2] = dSg[o];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        SD[i] = mma_f16(frag_rm(DO, LDW, 16 * i, 32 * s, lane), bs, SD[i]);
        DRS[i] = mma_f16(frag_rm(DR, LDW, 16 * i, 32 * s, lane), bs, DRS[i]);
        UD[i] = mma_f16(frag_rm(U, LDW, 16 * i, 32 * s, lane), bd, UD[i]);
      }
    }
    const float lgl = R.lgl[vc];
    float kbd = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * i + 4 * lg + jj;
        const float l = LG[r * LGS + vc], ee = exp2f(l), ff = exp2f(lgl - l);
        dqn[i][jj] = ee * SD[i][jj];
        dkn[i][jj] = ff * UD[i][jj] - ee * DRS[i][jj];
        dgk[i][jj] = -ff * UD[i][jj] - ee * DRS[i][jj];
        kbd += (float)KN[r * LDW + vc] * ff * UD[i][jj];
      }
    kbd += __shfl_xor(kbd, 16);
    kbd += __shfl_xor(kbd, 32);
    if (lg == 0) red.dgl[vc] = kbd;  // column vc belongs to this wave alone
  }
  // ---- dM = dO' U^T, dT = dU (b R)^T (64 x 64 tiles of this wave) -------------
  f32x4 DM[2];
  {
    f32x4 DTa[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) DM[j] = DTa[j] = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 ado = frag_rm(DO, LDW, 16 * rt, 32 * s, lane), adu = frag_rm(DU, LDW, 16 * rt, 32 * s, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        DM[j] = mma_f16(ado, frag_rm(U, LDW, 16 * (ct0 + j), 32 * s, lane), DM[j]);
        DTa[j] = mma_f16(adu, frag_rm(BR, LDW, 16 * (ct0 + j), 32 * s, lane), DTa[j]);
      }
    }
    __syncthreads();  // last reads of dO', bR, U, dU, dR: their space now holds the 64 x 64 results
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) DT[(16 * rt + 4 * lg + jj) * LDN + 16 * (ct0 + j) + l16] = (f16)DTa[j][jj];
  }
  __syncthreads();
  // ---- X1 = dT T^T -> X1t -----------------------------------------------------
  {
    f32x4 X[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) X[j] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 a = frag_rm(DT, LDN, 16 * rt, 32 * s, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) X[j] = mma_f16(a, frag_rm(T16, LDN, 16 * (ct0 + j), 32 * s, lane), X[j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *reinterpret_cast<f16x4*>(X1t + (16 * (ct0 + j) + l16) * LDN + 16 * rt + 4 * lg) =
          f16x4{(f16)X[j][0], (f16)X[j][1], (f16)X[j][2], (f16)X[j][3]};
  }
  __syncthreads();
  // ---- dA = -T^T X1; dH = diag(b) dA; db += rowsum(dA . H); dM, dH and their transposes
  {
    f32x4 DA[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) DA[j] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 a = frag_cm(T16, LDN, 16 * rt, 32 * s, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) DA[j] = mma_f16(a, frag_rm(X1t, LDN, 16 * (ct0 + j), 32 * s, lane), DA[j]);
    }
    float db2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = 16 * (ct0 + j) + l16;
      f16x4 mc, hc;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * rt + 4 * lg + jj;
        const float dm = r >= c ? DM[j][jj] : 0.f;
        const float da = r > c ? -DA[j][jj] : 0.f;
        const float dh = R.b[r] * da;
        DMm[r * LDN + c] = (f16)dm;
        DH[r * LDN + c] = (f16)dh;
        mc[jj] = (f16)dm;
        hc[jj] = (f16)dh;
        db2[jj] += rowsum16(da * (float)hkv[j][jj]);
      }
      *reinterpret_cast<f16x4*>(DMt + c * LDN + 16 * rt + 4 * lg) = mc;
      *reinterpret_cast<f16x4*>(DHt + c * LDN + 16 * rt + 4 * lg) = hc;
    }
    if (l16 == 0) {  // this row tile's two waves: column tiles 0, 1 and 2, 3
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) red.part[w & 1][16 * rt + 4 * lg + jj] = db2[jj];
    }
  }
  __syncthreads();  // dM, dH complete; M^T, T, dT, X1^T dead
  if (t < CH) red.db[t] += red.part[0][t] + red.part[1][t];
  {  // qn rows over M^T and T
    float qv[16];
    unpack_bf16x8(qraw[0], qv);
    unpack_bf16x8(qraw[1], qv + 8);
    const float iq = r8 < len ? 1.f / R.nq[r8] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) qv[j] *= iq;
    *reinterpret_cast<f16x8*>(QN + r8 * LDW + c0) = to_f16x8(qv);
    *reinterpret_cast<f16x8*>(QN + r8 * LDW + c0 + 8) = to_f16x8(qv + 8);
  }
  __syncthreads();
  // ---- masked products over earlier blocks on matrix cores (key column c = vc) -----------
  //   rows r of block rb, partners i < 16 rb:    Yq, X += exp2(LG[r] - LG[p]) (dM, dH) (exp2(LG[p] - LG[i]) kn_i)
  //   rows i of block ib, partners r > 16 ib + 15: Z += exp2(LG[p] - LG[i]) (dH^T (a kn) + dM^T (a qn)),
  //   a = exp2(LG[r] - LG[p]);  p = the block boundary before the later block
#pragma unroll 1
  for (int rb = 1; rb < NSUB; ++rb) {
    const int pb = 16 * rb - 1;
    f32x4 X = zero4(), Yq = zero4();
#pragma unroll
    for (int s = 0; s < (rb == 3 ? 2 : 1); ++s) {
      const f16x8 bk = frag_decay_cm(KN, LG, vc, pb, 32 * s + 8 * lg, false);
      X = mma_f16(frag_rm(DH, LDN, 16 * rb, 32 * s, lane), bk, X);
      Yq = mma_f16(frag_rm(DMm, LDN, 16 * rb, 32 * s, lane), bk, Yq);
    }
    const float lp = LG[pb * LGS + vc];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * rb + 4 * lg + jj;
      const float a = exp2f(fminf(LG[r * LGS + vc] - lp, 0.f));
      dqn[rb][jj] += a * Yq[jj];
      dkn[rb][jj] += a * X[jj];
      dgk[rb][jj] += a * X[jj];
    }
  }
#pragma unroll 1
  for (int ib = 0; ib < NSUB - 1; ++ib) {
    const int pb = 16 * ib + 15;
    f32x4 Z = zero4();
#pragma unroll
    for (int s = (ib == 0 ? 0 : 1); s < 2; ++s) {
      const f16x8 bk = frag_decay_cm(KN, LG, vc, pb, 32 * s + 8 * lg, true);
      const f16x8 bq = frag_decay_cm(QN, LG, vc, pb, 32 * s + 8 * lg, true);
      Z = mma_f16(frag_rm(DHt, LDN, 16 * ib, 32 * s, lane), bk, Z);
      Z = mma_f16(frag_rm(DMt, LDN, 16 * ib, 32 * s, lane), bq, Z);
    }
    const float lp = LG[pb * LGS + vc];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = 16 * ib + 4 * lg + jj;
      const float bfac = exp2f(fminf(lp - LG[i * LGS + vc], 0.f));
      dkn[ib][jj] += bfac * Z[jj];
      dgk[ib][jj] -= bfac * Z[jj];
    }
  }
  // ---- the diagonal blocks, exactly: thread -> block bb = t / 128, key channel c = t % 128, every pair
  // i < r of the block once (E = exp2(LG[r][c] - LG[i][c]) <= 1), row sums X, Yq for r and column
  // sums Z for i in registers; then through one fp32 exchange matrix into the C layout:
  // X + Z -> dkn, Yq -> dqn, X - Z -> dgk.  The pairs i = r (dH's diagonal is zero, E = 1) add
  // dM_rr kn_r to dqn_r and dM_rr qn_r to dkn_r, and nothing to dGamma: in dGamma's qn . Yq - kn . Z
  // they cancel exactly, so they are added to dqn, dkn only after dGamma is formed (under harsh decays
  // their rounding would otherwise swamp dGamma's small true value)
  {
    const int bb = t >> 7, c = t & (HD - 1), rb0 = 16 * bb;
    float lgc[16], knc[16], qnc[16], Xd[16], Yd[16], Zd[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      lgc[j] = LG[(rb0 + j) * LGS + c];
      knc[j] = (float)KN[(rb0 + j) * LDW + c];
      qnc[j] = (float)QN[(rb0 + j) * LDW + c];
      Xd[j] = Yd[j] = Zd[j] = 0.f;
    }
#pragma unroll
    for (int rl = 0; rl < 16; ++rl) {
      // row rb0 + rl of dH and dM, columns rb0 .. rb0 + 15 (the same for every thread of the block)
      const f16x8 h0 = *reinterpret_cast<const f16x8*>(DH + (rb0 + rl) * LDN + rb0);
      const f16x8 h1 = *reinterpret_cast<const f16x8*>(DH + (rb0 + rl) * LDN + rb0 + 8);
      const f16x8 m0 = *reinterpret_cast<const f16x8*>(DMm + (rb0 + rl) * LDN + rb0);
      const f16x8 m1 = *reinterpret_cast<const f16x8*>(DMm + (rb0 + rl) * LDN + rb0 + 8);
#pragma unroll
      for (int il = 0; il < rl; ++il) {
        const float hv = (float)(il < 8 ? h0[il & 7] : h1[il & 7]), mv = (float)(il < 8 ? m0[il & 7] : m1[il & 7]);
        const float E = exp2f(fminf(lgc[rl] - lgc[il], 0.f));
        const float ke = knc[il] * E;
        Xd[rl] += hv * ke;
        Yd[rl] += mv * ke;
        Zd[il] += (hv * knc[rl] + mv * qnc[rl]) * E;
      }
    }
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        XB[(rb0 + j) * LGS + c] = pass == 0 ? Xd[j] + Zd[j] : (pass == 1 ? Yd[j] : Xd[j] - Zd[j]);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float x = XB[(16 * i + 4 * lg + jj) * LGS + vc];
          if (pass == 0) dkn[i][jj] += x;
          else if (pass == 1) dqn[i][jj] += x;
          else dgk[i][jj] += x;
        }
      __syncthreads();
    }
  }
  // ---- row dots qn . dqn, kn . dkn; dGamma; dg (reverse cumulative sum over the chunk's rows)
  float dgm[4][4];
  float* pqk = reinterpret_cast<float*>(smem + P_DHT);  // the waves' partial row dots (dH^T, dM^T are dead)
  uint4 graw[2];  // g_raw of row r8, channels c0 .. c0 + 15 (issued now, used last)
  {
    const size_t o = ((size_t)(tok0 + min(r8, len - 1)) * p.H + h) * HD + c0;
    graw[0] = *reinterpret_cast<const uint4*>(p.g_raw + o);
    graw[1] = *reinterpret_cast<const uint4*>(p.g_raw + o + 8);
  }
  {
    const float dglc = red.dgl[vc] + R.el[vc] * red.sdl[vc];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * i + 4 * lg + jj;
        const float qx = (float)QN[r * LDW + vc], kx = (float)KN[r * LDW + vc];
        dgm[i][jj] = r < len ? qx * dqn[i][jj] + kx * dgk[i][jj] + (r == len - 1 ? dglc : 0.f) : 0.f;
        const float dmrr = (float)DMm[r * LDN + r];  // the pair i = r
        dqn[i][jj] += dmrr * kx;
        dkn[i][jj] += dmrr * qx;
        const float qd = rowsum16(qx * dqn[i][jj]), kd = rowsum16(kx * dkn[i][jj]);
        if (l16 == 0) {
          pqk[w * CH + r] = qd;
          pqk[(8 + w) * CH + r] = kd;
        }
      }
    // reverse inclusive sum over rows 16 i + 4 lg + jj of column vc (lanes lg = 0..3 share the column)
    float tot_after = 0.f;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      float loc[4];
      loc[3] = dgm[i][3];
#pragma unroll
      for (int jj = 2; jj >= 0; --jj) loc[jj] = loc[jj + 1] + dgm[i][jj];
      const float s = loc[0];
      const float a1 = __shfl_down(s, 16), a2 = __shfl_down(s, 32), a3 = __shfl_down(s, 48);
      const float after = (lg < 3 ? a1 : 0.f) + (lg < 2 ? a2 : 0.f) + (lg < 1 ? a3 : 0.f);
      float tile = s + __shfl_xor(s, 16);
      tile += __shfl_xor(tile, 32);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dgm[i][jj] = loc[jj] + after + tot_after;
      tot_after += tile;
    }
    // dg to the exchange matrix: dg_raw and dA_log follow in the row-and-channels mapping
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) XB[(16 * i + 4 * lg + jj) * LGS + vc] = dgm[i][jj];
  }
  __syncthreads();
  if (t < 2 * CH) {  // the row dots, wave by wave
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) a += pqk[((t >> 6) * 8 + q) * CH + (t & (CH - 1))];
    (t < CH ? red.qd : red.kd)[t & (CH - 1)] = a;
  }
  __syncthreads();
  // dq, dk through the normalisation: (dxn - xn (xn . dxn)) / |x|
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * i + 4 * lg + jj;
      if (r < len) {
        const size_t o = ((size_t)(tok0 + r) * p.H_qk + hq) * HD + vc;
        const float qx = (float)QN[r * LDW + vc], kx = (float)KN[r * LDW + vc];
        const float gq = (dqn[i][jj] - qx * red.qd[r]) / R.nq[r];
        const float gk = (dkn[i][jj] - kx * red.kd[r]) / R.nk[r];
        if (G == 1) {
          __builtin_nontemporal_store(gq, p.dq + o);
          __builtin_nontemporal_store(gk, p.dk + o);
        } else {
          atomicAdd(p.dq + o, gq);
          atomicAdd(p.dk + o, gk);
        }
      }
    }
  {  // dg_raw = dg (-exp(A_log)) sigmoid(g_raw), dA_log = sum dg g: thread -> row r8, channels c0 ..
    float dg[16], x[16], o[16];
    load_f32x16(XB + r8 * LGS + c0, dg);
    unpack_bf16x8(graw[0], x);
    unpack_bf16x8(graw[1], x + 8);
    const float a = expf(p.A_log[h]);
    float dal = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      // sigmoid and softplus from one exponential e = exp(-|x|) <= 1
      const float ex = __expf(-fabsf(x[j])), inv = 1.f / (1.f + ex);
      const float sg = x[j] >= 0.f ? inv : ex * inv, sp = fmaxf(x[j], 0.f) + __logf(1.f + ex);
      o[j] = dg[j] * (-a) * sg;
      dal += dg[j] * (-a * sp);  // dg = 0 past the chunk's end
    }
    if (r8 < len) {
      f32x4* dst = reinterpret_cast<f32x4*>(p.dg_raw + ((size_t)(tok0 + r8) * p.H + h) * HD + c0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        __builtin_nontemporal_store(f32x4{o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]}, dst + j);
    }
    dal = sum64(dal);
    if (lane == 0) red.dalw[w] = dal;
  }
  if (t < len) {
    const float b = R.b[t];
    p.dbeta[(size_t)(tok0 + t) * p.H + h] = red.db[t] * b * (1.f - b);
  }
  __syncthreads();
  if (t == 0) {
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) a += red.dalw[q];
    atomicAdd(p.dA_log + h, a);
  }
}

void launch_coef_pc(const BwdParams& p, hipStream_t stream) {
  const int jobs = p.n_entries * p.H;
  if (jobs > 0) bwd_coef_pc_kernel<<<jobs, NTH, 0, stream>>>(p);
}

void launch_grad_pc(const BwdParams& p, hipStream_t stream) {
  const int jobs = p.n_entries * p.H;
  if (jobs > 0) bwd_grad_pc_kernel<<<jobs, NTH, 0, stream>>>(p);
}

}  // namespace kda
