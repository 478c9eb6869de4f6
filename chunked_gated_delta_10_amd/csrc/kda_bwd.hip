// kda_bwd.hip -- backward pass of the chunked forward with one decay per
// token-head (the gated delta rule; the FlashQLA H200 results page,
// "BACKWARD BENCHMARKS" table).
//
// L = sum(dout * out) + sum(dfinal * final_state).  With a scalar decay per
// token every decay factor of a 64-token chunk is a row scaling by
// e_r = exp(G_r) or f_r = exp(G_L - G_r) (G: the gate's cumulative sum in the
// chunk, L: its last token) or the mask Lam[r][i] = exp(G_r - G_i), r >= i,
// on a 64 x 64 Gram matrix; all of them are <= 1.  With P = qn kn^T,
// Gm = kn kn^T, M = lower(P . Lam), A = strict_lower(diag(b) (Gm . Lam)),
// T = (I + A)^-1, R = V - diag(e) kn S_c and U = T diag(b) R, one chunk is
//   O = scale (diag(e) qn S_c + M U),  S_c+1 = e_L S_c + kn^T diag(f) U.
// Its adjoint, with dO' = scale dO and dS' the gradient of S_c+1:
//   dU   = M^T dO' + diag(f) kn dS'
//   dS_c = qn^T diag(e) dO' - kn^T diag(b e) T^T dU + e_L dS'
// and the gradients of the chunk's own inputs follow from dU, dS', S_c by
// 64 x 64 and 64 x 128 algebra (grad_kernel below).
//
// Kernels, in launch order (the forward's chunk-local kernel and a
// recurrence that stores the state entering every chunk run first):
//   prep_kernel     per (chunk, head): qn, kn, the gate rows, P, Gm, M, T
//   adjoint_kernel  per (chain, 16 value columns): the adjoint over chunks,
//                   last to first; stores dS' of every chunk and dS_0
//   grad_kernel     per (chunk, head): every input gradient of the chunk
// All arithmetic is fp32 (vector ALU, LDS-tiled products).
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

constexpr int BT = 256;                 // threads per workgroup
constexpr int MM = CH * CH;             // floats of a 64 x 64 block
constexpr int MK = CH * HD;             // floats of a 64 x 128 block
// prep block of one (chunk, head), floats
constexpr int P_QN = 0, P_KN = P_QN + MK, P_M = P_KN + MK, P_T = P_M + MM, P_GM = P_T + MM, P_P = P_GM + MM;
constexpr int P_ROWS = P_P + MM;
constexpr int R_E = 0, R_F = CH, R_B = 2 * CH, R_GAM = 3 * CH, R_G = 4 * CH, R_NQ = 5 * CH, R_NK = 6 * CH,
              R_EL = 7 * CH;  // e, f, b, Gamma, g, |q|, |k| per row; e_L and the live length after
constexpr int PREP_FLOATS_ = P_ROWS + 8 * CH;
static_assert(PREP_FLOATS_ == PREP_FLOATS, "prep block size");
// grad-kernel scratch of one job, floats
constexpr int S_DO = 0, S_R = S_DO + MK, S_KS = S_R + MK, S_SDO = S_KS + MK, S_KDS = S_SDO + MK, S_BR = S_KDS + MK,
              S_U = S_BR + MK, S_UDS = S_U + MK, S_DU = S_UDS + MK, S_DR = S_DU + MK, S_DRS = S_DR + MK,
              S_DQN = S_DRS + MK, S_DKN = S_DQN + MK, S_DM = S_DKN + MK, S_DT = S_DM + MM, S_X1 = S_DT + MM,
              S_DA = S_X1 + MM, S_DG2 = S_DA + MM, S_DP = S_DG2 + MM, S_ROWS = S_DP + MM;
constexpr int SLOT_FLOATS_ = S_ROWS + 8 * CH;
static_assert(SLOT_FLOATS_ == BWD_SLOT_FLOATS, "scratch slot size");

__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float softplus_(float x) { return x > 20.f ? x : log1pf(expf(x)); }
__device__ __forceinline__ float sigmoid_(float x) { return 1.f / (1.f + expf(-x)); }

// (sequence, first token, length, chunk index) of schedule entry e
__device__ __forceinline__ int4 entry_of(const BwdParams& p, int e) {
  if (p.dense_T >= 0) {
    const int T = p.dense_T, nc = (T + CH - 1) / CH, b = e / nc, c = e - b * nc;
    return make_int4(b, b * T + c * CH, min(CH, T - c * CH), c);
  }
  return p.chunks[e];
}

// C = alpha op(A) op(B) (+ C when ACC) for the whole workgroup; fp32, row-major,
// C with leading dimension N.  op(A) is M x K (TA: A is stored K x M), op(B) is
// K x N (TB: B is stored N x K).  sh: LDS of 16 (M + N) floats.
template <int M, int N, int K, bool TA, bool TB, bool ACC>
__device__ void wg_gemm(float* __restrict__ C, const float* __restrict__ A, int lda, const float* __restrict__ B,
                        int ldb, float alpha, float* sh) {
  constexpr int TM = M / 16, TN = N / 16;
  const int t = threadIdx.x, tr = t >> 4, tc = t & 15;
  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;
  float* As = sh;           // [16][M]
  float* Bs = sh + 16 * M;  // [16][N]
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = t; i < M * 16; i += BT) {
      if (TA) {
        const int m = i % M, kk = i / M;
        As[kk * M + m] = A[(size_t)(k0 + kk) * lda + m];
      } else {
        const int kk = i & 15, m = i >> 4;
        As[kk * M + m] = A[(size_t)m * lda + k0 + kk];
      }
    }
    for (int i = t; i < N * 16; i += BT) {
      if (TB) {
        const int kk = i & 15, n = i >> 4;
        Bs[kk * N + n] = B[(size_t)n * ldb + k0 + kk];
      } else {
        const int n = i % N, kk = i / N;
        Bs[kk * N + n] = B[(size_t)(k0 + kk) * ldb + n];
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < 16; ++kk) {
      float a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = As[kk * M + tr * TM + i];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = Bs[kk * N + tc * TN + j];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      float* c = C + (size_t)(tr * TM + i) * N + tc * TN + j;
      *c = ACC ? *c + alpha * acc[i][j] : alpha * acc[i][j];
    }
  __syncthreads();  // C complete for the next product
}

}  // namespace

// ---------------------------------------------------------------------------
// Per (chunk, head): normalised rows, gate rows, Gram matrices, M and T.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BT) void bwd_prep_kernel(BwdParams p) {
  __shared__ float sQ[CH][HD + 1], sK[CH][HD + 1];
  __shared__ float sA[CH][CH + 1], sT[CH][CH + 1];
  __shared__ float sRow[8 * CH];
  const int job = blockIdx.x, e = job / p.H, h = job - e * p.H, hq = h / (p.H / p.H_qk);
  const int4 ce = entry_of(p, e);
  const int len = ce.z, tok0 = ce.y;
  float* blk = p.prep + (size_t)job * PREP_FLOATS;
  const int t = threadIdx.x, r = t >> 2, qd = t & 3;
  // rows: load, normalise (4 threads per row, 32 channels each)
  {
    float qv[32], kv[32], sq = 0.f, sk = 0.f;
    const bool live = r < len;
    const size_t row = (size_t)(tok0 + (live ? r : 0)) * p.H_qk + hq;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      qv[i] = live ? bf(p.q[row * HD + 32 * qd + i]) : 0.f;
      kv[i] = live ? bf(p.k[row * HD + 32 * qd + i]) : 0.f;
      sq += qv[i] * qv[i];
      sk += kv[i] * kv[i];
    }
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    sk += __shfl_xor(sk, 1);
    sk += __shfl_xor(sk, 2);
    const float nq = sqrtf(sq + 1e-6f), nk = sqrtf(sk + 1e-6f);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      sQ[r][32 * qd + i] = qv[i] / nq;
      sK[r][32 * qd + i] = kv[i] / nk;
      blk[P_QN + r * HD + 32 * qd + i] = qv[i] / nq;
      blk[P_KN + r * HD + 32 * qd + i] = kv[i] / nk;
    }
    if (qd == 0) {
      sRow[R_NQ + r] = nq;
      sRow[R_NK + r] = nk;
    }
  }
  if (t < CH) {  // gate and write strength of row t
    const bool live = t < len;
    const size_t th = (size_t)(tok0 + (live ? t : 0)) * p.H + h;
    sRow[R_G + t] = live ? -expf(p.A_log[h]) * softplus_(bf(p.g_raw[th])) : 0.f;
    sRow[R_B + t] = live ? sigmoid_(p.beta[th]) : 0.f;
  }
  __syncthreads();
  if (t == 0) {  // cumulative gate and the chunk-end factors
    float G = 0.f;
    for (int i = 0; i < CH; ++i) {
      G += sRow[R_G + i];
      sRow[R_GAM + i] = G;
    }
    const float GL = sRow[R_GAM + max(len, 1) - 1];
    sRow[R_EL] = expf(GL);
    sRow[R_EL + 1] = (float)len;
  }
  __syncthreads();
  if (t < CH) {
    sRow[R_E + t] = expf(sRow[R_GAM + t]);
    sRow[R_F + t] = expf(sRow[R_GAM + max(len, 1) - 1] - sRow[R_GAM + t]);
  }
  // P = qn kn^T, Gm = kn kn^T; M = lower(P . Lam), A = strict_lower(b (Gm . Lam))
  {
    const int r0 = (t >> 4) * 4, c0 = (t & 15) * 4;
    float pp[4][4] = {}, gg[4][4] = {};
    for (int k = 0; k < HD; ++k) {
      float a[4], b[4], c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = sQ[r0 + i][k];
        b[i] = sK[r0 + i][k];
        c[i] = sK[c0 + i][k];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pp[i][j] += a[i] * c[j];
          gg[i][j] += b[i] * c[j];
        }
    }
    __syncthreads();  // sRow e, f written
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ri = r0 + i, cj = c0 + j;
        const float lam = ri >= cj ? expf(fminf(sRow[R_GAM + ri] - sRow[R_GAM + cj], 0.f)) : 0.f;
        blk[P_P + ri * CH + cj] = pp[i][j];
        blk[P_GM + ri * CH + cj] = gg[i][j];
        blk[P_M + ri * CH + cj] = pp[i][j] * lam;
        sA[ri][cj] = ri > cj ? sRow[R_B + ri] * gg[i][j] * lam : 0.f;
      }
  }
  __syncthreads();
  if (t < CH) {  // T = (I + A)^-1 by forward substitution, thread t owns column t
    const int j = t;
    for (int i = 0; i < CH; ++i) {
      float v = 0.f;
      if (i == j) {
        v = 1.f;
      } else if (i > j) {
        for (int m = j; m < i; ++m) v -= sA[i][m] * sT[m][j];
      }
      sT[i][j] = v;
    }
  }
  __syncthreads();
  for (int i = t; i < MM; i += BT) blk[P_T + i] = sT[i / CH][i % CH];
  for (int i = t; i < 8 * CH; i += BT) blk[P_ROWS + i] = sRow[i];
}

// ---------------------------------------------------------------------------
// Per (chain, 16 value columns): the adjoint of the chunk recurrence, last
// chunk first.  dS (128 x 16) lives in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BT) void bwd_adjoint_kernel(BwdParams p) {
  __shared__ float sQ[CH][HD + 1], sK[CH][HD + 1];
  __shared__ float sM[CH][CH + 1], sT[CH][CH + 1];
  __shared__ float sdS[HD][17], sdO[CH][17], sdU[CH][17], sZ[CH][17];
  __shared__ float sRow[8 * CH];
  const int x = blockIdx.x, vt = x & 7, ch = x >> 3;
  const int h = ch % p.H;
  int n, tok0, len, chunk0;
  if (p.dense_T >= 0) {
    n = ch / p.H;
    tok0 = n * p.dense_T;
    len = p.dense_T;
    chunk0 = n * ((p.dense_T + CH - 1) / CH);
  } else {
    n = p.order[ch / p.H];
    const int4 sq = p.seqs[n];
    tok0 = sq.x;
    len = max(0, sq.y);
    chunk0 = sq.z;
  }
  const int nch = max(0, min((len + CH - 1) / CH, p.n_entries - chunk0));
  const int v0 = 16 * vt, t = threadIdx.x;
  const size_t sbase = ((size_t)n * p.H + h) * HD * HD;
  // dS <- dfinal (columns v0 .. v0 + 15): thread -> column t / 16, keys 8 (t % 16) .. + 7
  const int cv = t >> 4, k8 = (t & 15) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    sdS[k8 + i][cv] = p.dfinal ? p.dfinal[sbase + (size_t)(v0 + cv) * HD + k8 + i] : 0.f;
  for (int c = nch - 1; c >= 0; --c) {
    const size_t e = (size_t)(chunk0 + c);
    const float* blk = p.prep + (e * p.H + h) * PREP_FLOATS;
    __syncthreads();  // the previous chunk's dS is complete
    // dS' of this chunk (the gradient of the state leaving it)
    float* ds = p.dstates + (e * p.H + h) * HD * HD + (size_t)(v0 + cv) * HD + k8;
#pragma unroll
    for (int i = 0; i < 8; ++i) ds[i] = sdS[k8 + i][cv];
    for (int i = t; i < MK; i += BT) {
      sQ[i / HD][i % HD] = blk[P_QN + i];
      sK[i / HD][i % HD] = blk[P_KN + i];
    }
    for (int i = t; i < MM; i += BT) {
      sM[i / CH][i % CH] = blk[P_M + i];
      sT[i / CH][i % CH] = blk[P_T + i];
    }
    for (int i = t; i < 8 * CH; i += BT) sRow[i] = blk[P_ROWS + i];
    const int L = min(CH, len - c * CH);
    for (int i = t; i < CH * 16; i += BT) {
      const int r = i >> 4, v = i & 15;
      sdO[r][v] = r < L ? p.scale * bf(p.dout[((size_t)(tok0 + c * CH + r) * p.H + h) * HD + v0 + v]) : 0.f;
    }
    __syncthreads();
    // dU = M^T dO' + diag(f) kn dS     (thread: row r, columns 4 cq .. + 3)
    {
      const int r = t >> 2, c4 = (t & 3) * 4;
      float x[4] = {}, m[4] = {};
      for (int k = 0; k < HD; ++k) {
        const float a = sK[r][k];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] += a * sdS[k][c4 + j];
      }
      for (int i = 0; i < CH; ++i) {
        const float a = sM[i][r];
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] += a * sdO[i][c4 + j];
      }
      const float f = sRow[R_F + r];
#pragma unroll
      for (int j = 0; j < 4; ++j) sdU[r][c4 + j] = m[j] + f * x[j];
    }
    __syncthreads();
    // Z = diag(b e) T^T dU;  dO' rows scaled by e for the next product
    {
      const int r = t >> 2, c4 = (t & 3) * 4;
      float z[4] = {};
      for (int i = 0; i < CH; ++i) {
        const float a = sT[i][r];
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] += a * sdU[i][c4 + j];
      }
      const float be = sRow[R_B + r] * sRow[R_E + r], er = sRow[R_E + r];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sZ[r][c4 + j] = be * z[j];
        sdO[r][c4 + j] *= er;
      }
    }
    __syncthreads();
    // dS <- qn^T diag(e) dO' - kn^T Z + e_L dS     (thread: key k, columns 8 cw .. + 7)
    {
      const int k = t >> 1, c8 = (t & 1) * 8;
      float a8[8] = {};
      for (int r = 0; r < CH; ++r) {
        const float qa = sQ[r][k], ka = sK[r][k];
#pragma unroll
        for (int j = 0; j < 8; ++j) a8[j] += qa * sdO[r][c8 + j] - ka * sZ[r][c8 + j];
      }
      const float eL = sRow[R_EL];
#pragma unroll
      for (int j = 0; j < 8; ++j) sdS[k][c8 + j] = a8[j] + eL * sdS[k][c8 + j];
    }
  }
  __syncthreads();
  if (p.dinit) {
#pragma unroll
    for (int i = 0; i < 8; ++i) p.dinit[sbase + (size_t)(v0 + cv) * HD + k8 + i] = sdS[k8 + i][cv];
  }
}

// ---------------------------------------------------------------------------
// Per (chunk, head): every gradient of the chunk's inputs.  Intermediates of
// the job live in its scratch slot (L2), products through wg_gemm.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BT) void bwd_grad_kernel(BwdParams p) {
  __shared__ float sh[16 * (CH + HD)];
  __shared__ float red[BT];
  const int job = p.job0 + blockIdx.x, e = job / p.H, h = job - e * p.H, G = p.H / p.H_qk, hq = h / G;
  const int4 ce = entry_of(p, e);
  const int len = ce.z, tok0 = ce.y;
  if (len <= 0) return;  // uniform over the workgroup
  const float* blk = p.prep + (size_t)job * PREP_FLOATS;
  float* sc = p.scratch + (size_t)blockIdx.x * BWD_SLOT_FLOATS;
  const float* QN = blk + P_QN;
  const float* KN = blk + P_KN;
  const float* rows = blk + P_ROWS;
  const float* St = p.states + ((size_t)e * p.H + h) * HD * HD;    // [V][K]: S^T
  const float* dSt = p.dstates + ((size_t)e * p.H + h) * HD * HD;  // [V][K]: dS'^T
  const int t = threadIdx.x;
  // dO' and V (zero past the chunk's end)
  for (int i = t; i < MK; i += BT) {
    const int r = i / HD, c = i % HD;
    const size_t at = ((size_t)(tok0 + min(r, len - 1)) * p.H + h) * HD + c;
    sc[S_DO + i] = r < len ? p.scale * bf(p.dout[at]) : 0.f;
    sc[S_R + i] = r < len ? bf(p.v[at]) : 0.f;
  }
  __syncthreads();
  wg_gemm<CH, HD, HD, false, true, false>(sc + S_KS, KN, HD, St, HD, 1.f, sh);     // kn S
  wg_gemm<CH, HD, HD, false, false, false>(sc + S_SDO, sc + S_DO, HD, St, HD, 1.f, sh);  // dO' S^T
  wg_gemm<CH, HD, HD, false, true, false>(sc + S_KDS, KN, HD, dSt, HD, 1.f, sh);   // kn dS'
  for (int i = t; i < MK; i += BT) {  // R = V - diag(e) kn S;  b R
    const int r = i / HD;
    const float R = sc[S_R + i] - rows[R_E + r] * sc[S_KS + i];
    sc[S_R + i] = R;
    sc[S_BR + i] = rows[R_B + r] * R;
  }
  __syncthreads();
  wg_gemm<CH, HD, CH, false, false, false>(sc + S_U, blk + P_T, CH, sc + S_BR, HD, 1.f, sh);    // U = T b R
  wg_gemm<CH, HD, HD, false, false, false>(sc + S_UDS, sc + S_U, HD, dSt, HD, 1.f, sh);         // U dS'^T
  for (int i = t; i < MK; i += BT) sc[S_DU + i] = rows[R_F + i / HD] * sc[S_KDS + i];
  __syncthreads();
  wg_gemm<CH, HD, CH, true, false, true>(sc + S_DU, blk + P_M, CH, sc + S_DO, HD, 1.f, sh);     // += M^T dO'
  wg_gemm<CH, HD, CH, true, false, false>(sc + S_DR, blk + P_T, CH, sc + S_DU, HD, 1.f, sh);    // Y = T^T dU
  // dR = diag(b) Y (= dV), and db1 = rowsum(Y . R)
  float* srow = sc + S_ROWS;  // de, df, db, dG
  {
    const int r = t >> 2, qd = t & 3;
    float db = 0.f;
    const float b = rows[R_B + r];
    for (int c = 32 * qd; c < 32 * qd + 32; ++c) {
      const float y = sc[S_DR + r * HD + c];
      db += y * sc[S_R + r * HD + c];
      sc[S_DR + r * HD + c] = b * y;
    }
    db += __shfl_xor(db, 1);
    db += __shfl_xor(db, 2);
    if (qd == 0) srow[2 * CH + r] = db;
  }
  __syncthreads();
  wg_gemm<CH, HD, HD, false, false, false>(sc + S_DRS, sc + S_DR, HD, St, HD, 1.f, sh);   // dR S^T
  wg_gemm<CH, CH, HD, false, true, false>(sc + S_DM, sc + S_DO, HD, sc + S_U, HD, 1.f, sh);   // dO' U^T
  wg_gemm<CH, CH, HD, false, true, false>(sc + S_DT, sc + S_DU, HD, sc + S_BR, HD, 1.f, sh);  // dU (b R)^T
  wg_gemm<CH, CH, CH, false, true, false>(sc + S_X1, sc + S_DT, CH, blk + P_T, CH, 1.f, sh);  // dT T^T
  wg_gemm<CH, CH, CH, true, false, false>(sc + S_DA, blk + P_T, CH, sc + S_X1, CH, -1.f, sh); // -T^T (dT T^T)
  // 64 x 64 elementwise: dM, dA masked; dGm + dGm^T, dP; the rows and columns of dLam . Lam
  const float* GM = blk + P_GM;
  const float* PP = blk + P_P;
  for (int i = t; i < MM; i += BT) {
    const int r = i / CH, c = i % CH;
    const float lam = r >= c ? expf(fminf(rows[R_GAM + r] - rows[R_GAM + c], 0.f)) : 0.f;
    const float dm = r >= c ? sc[S_DM + i] : 0.f;
    const float da = r > c ? sc[S_DA + i] : 0.f;
    const float b = rows[R_B + r];
    sc[S_DM + i] = (da * GM[i] * lam);            // db2 terms (row sums below)
    sc[S_X1 + i] = (b * da * GM[i] + dm * PP[i]) * lam;  // W = dLam . Lam
    sc[S_DP + i] = dm * lam;                      // dP
    sc[S_DT + i] = b * da * lam;                  // dGm
  }
  __syncthreads();
  for (int i = t; i < MM; i += BT) {
    const int r = i / CH, c = i % CH;
    sc[S_DG2 + i] = sc[S_DT + i] + sc[S_DT + c * CH + r];  // dGm + dGm^T
  }
  __syncthreads();
  // dqn = diag(e) (dO' S^T) + dP kn;  dkn = diag(f) (U dS'^T) - diag(e) (dR S^T) + (dGm + dGm^T) kn + dP^T qn
  for (int i = t; i < MK; i += BT) {
    const int r = i / HD;
    sc[S_DQN + i] = rows[R_E + r] * sc[S_SDO + i];
    sc[S_DKN + i] = rows[R_F + r] * sc[S_UDS + i] - rows[R_E + r] * sc[S_DRS + i];
  }
  __syncthreads();
  wg_gemm<CH, HD, CH, false, false, true>(sc + S_DQN, sc + S_DP, CH, KN, HD, 1.f, sh);
  wg_gemm<CH, HD, CH, false, false, true>(sc + S_DKN, sc + S_DG2, CH, KN, HD, 1.f, sh);
  wg_gemm<CH, HD, CH, true, false, true>(sc + S_DKN, sc + S_DP, CH, QN, HD, 1.f, sh);
  // row terms: de = rowsum(qn . dO'S^T) - rowsum(dR . kn S), df = rowsum(kn . U dS'^T), db2, rows and
  // columns of W;  deL = sum(dS' . S)
  float deL = 0.f;
  for (int i = t; i < HD * HD; i += BT) deL += dSt[i] * St[i];
  red[t] = deL;
  {
    const int r = t >> 2, qd = t & 3;
    float de = 0.f, df = 0.f;
    for (int c = 32 * qd; c < 32 * qd + 32; ++c) {
      de += QN[r * HD + c] * sc[S_SDO + r * HD + c] - sc[S_DR + r * HD + c] * sc[S_KS + r * HD + c];
      df += KN[r * HD + c] * sc[S_UDS + r * HD + c];
    }
    float db2 = 0.f, wr = 0.f, wc = 0.f;
    for (int c = 16 * qd; c < 16 * qd + 16; ++c) {
      db2 += sc[S_DM + r * CH + c];
      wr += sc[S_X1 + r * CH + c];
      wc += sc[S_X1 + c * CH + r];
    }
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
      de += __shfl_xor(de, o);
      df += __shfl_xor(df, o);
      db2 += __shfl_xor(db2, o);
      wr += __shfl_xor(wr, o);
      wc += __shfl_xor(wc, o);
    }
    __syncthreads();  // red[] complete
    if (qd == 0) {
      srow[r] = de;
      srow[CH + r] = df;
      srow[2 * CH + r] += db2;
      srow[3 * CH + r] = wr - wc + de * rows[R_E + r] - df * rows[R_F + r];  // dG without the chunk-end terms
    }
  }
  __syncthreads();
  if (t == 0) {  // chunk-end terms on the last live row, then dg = reverse cumulative sum of dG
    float tot = 0.f;
    for (int i = 0; i < BT; ++i) tot += red[i];
    float dfs = 0.f;
    for (int r = 0; r < len; ++r) dfs += srow[CH + r] * rows[R_F + r];
    srow[3 * CH + len - 1] += dfs + tot * rows[R_EL];
    float acc = 0.f, dal = 0.f;
    for (int r = len - 1; r >= 0; --r) {
      acc += srow[3 * CH + r];
      srow[3 * CH + r] = acc;                       // dg_r
      dal += acc * rows[R_G + r];
    }
    atomicAdd(p.dA_log + h, dal);
  }
  __syncthreads();
  // per-token outputs: dv, dg_raw, dbeta; dq, dk through the L2 normalisation (summed over the group)
  for (int i = t; i < len * HD; i += BT) {
    const int r = i / HD, c = i % HD;
    p.dv[((size_t)(tok0 + r) * p.H + h) * HD + c] = sc[S_DR + i];
  }
  if (t < len) {
    const size_t th = (size_t)(tok0 + t) * p.H + h;
    const float graw = bf(p.g_raw[th]), b = rows[R_B + t];
    p.dg_raw[th] = srow[3 * CH + t] * (-expf(p.A_log[h])) * sigmoid_(graw);
    p.dbeta[th] = srow[2 * CH + t] * b * (1.f - b);
  }
  {
    const int r = t >> 2, qd = t & 3;
    if (r < len) {
      float dq = 0.f, dk = 0.f;  // qn . dqn, kn . dkn
      for (int c = 32 * qd; c < 32 * qd + 32; ++c) {
        dq += QN[r * HD + c] * sc[S_DQN + r * HD + c];
        dk += KN[r * HD + c] * sc[S_DKN + r * HD + c];
      }
      dq += __shfl_xor(dq, 1);
      dq += __shfl_xor(dq, 2);
      dk += __shfl_xor(dk, 1);
      dk += __shfl_xor(dk, 2);
      const float nq = rows[R_NQ + r], nk = rows[R_NK + r];
      const size_t at = ((size_t)(tok0 + r) * p.H_qk + hq) * HD;
      for (int c = 32 * qd; c < 32 * qd + 32; ++c) {
        // d/dq of q / n(q): (dqn - qn (qn . dqn)) / n
        const float gq = (sc[S_DQN + r * HD + c] - QN[r * HD + c] * dq) / nq;
        const float gk = (sc[S_DKN + r * HD + c] - KN[r * HD + c] * dk) / nk;
        if (G == 1) {
          p.dq[at + c] = gq;
          p.dk[at + c] = gk;
        } else {
          atomicAdd(p.dq + at + c, gq);
          atomicAdd(p.dk + at + c, gk);
        }
      }
    }
  }
}

__global__ __launch_bounds__(BT) void bwd_fill_kernel(float* a, size_t n) {
  for (size_t i = (size_t)blockIdx.x * BT + threadIdx.x; i < n; i += (size_t)gridDim.x * BT) a[i] = 0.f;
}

void launch_bwd(const BwdParams& p0, size_t qk_floats, size_t slots, hipStream_t stream) {
  BwdParams p = p0;
  const int jobs = p.n_entries * p.H;
  if (p.H != p.H_qk) {  // dq, dk are accumulated over each group's value heads
    bwd_fill_kernel<<<1024, BT, 0, stream>>>(p.dq, qk_floats);
    bwd_fill_kernel<<<1024, BT, 0, stream>>>(p.dk, qk_floats);
  }
  bwd_fill_kernel<<<1, BT, 0, stream>>>(p.dA_log, (size_t)p.H);
  if (jobs > 0) bwd_prep_kernel<<<jobs, BT, 0, stream>>>(p);
  if (p.n_chains > 0) bwd_adjoint_kernel<<<p.n_chains * 8, BT, 0, stream>>>(p);
  for (int j0 = 0; j0 < jobs; j0 += (int)slots) {
    p.job0 = j0;
    bwd_grad_kernel<<<(int)std::min<size_t>(slots, (size_t)(jobs - j0)), BT, 0, stream>>>(p);
  }
}

}  // namespace kda
