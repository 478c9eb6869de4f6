// kda_bwd.hip -- backward pass of the chunked forward with one decay per
// token-head (the gated delta rule whose backward the FlashQLA H200 results
// page times, "BACKWARD BENCHMARKS" table).
//
// L = sum(dout * out) + sum(dfinal * final_state).  With a scalar decay per
// token every decay factor of a 64-token chunk is a row scaling by
// e_r = exp(G_r) or f_r = exp(G_L - G_r) (G: the gate's cumulative sum in the
// chunk, L: its last token) or the mask Lam[r][i] = exp(G_r - G_i), r >= i,
// on a 64 x 64 Gram matrix; all of them are <= 1.  With P = qn kn^T,
// Gm = kn kn^T, M = lower(P . Lam), A = strict_lower(diag(b) (Gm . Lam)),
// T = (I + A)^-1, R = V - diag(e) kn S_c and U = T diag(b) R, one chunk is
//   O = scale (diag(e) qn S_c + M U),  S_c+1 = e_L S_c + kn^T diag(f) U.
// Its adjoint, with dO' = scale dO and dS' the gradient of S_c+1, is linear:
//   dS_c = Phi dS' + Bc dO'
//   Phi = e_L I - kn^T diag(b e) T^T diag(f) kn         (128 x 128)
//   Bc  = qn^T diag(e) - kn^T diag(b e) T^T M^T          (128 x 64)
// so the chain over chunks (last to first) is one matrix-core step per
// chunk, like the forward recurrence, and everything else is chunk-parallel:
//   dU = M^T dO' + diag(f) kn dS',  Y = T^T dU,  dV = diag(b) Y,
//   dT = dU (b R)^T,  dA = strict_lower(-T^T dT T^T),
//   dP = lower(dO' U^T) . Lam,  dGm = diag(b) dA . Lam,
//   dqn = diag(e) dO' S_c^T + dP kn,
//   dkn = diag(f) U dS'^T - diag(e) dV S_c^T + (dGm + dGm^T) kn + dP^T qn,
//   d(Lam) . Lam = (diag(b) dA . Gm + lower(dO' U^T) . P) . Lam, whose row and
//   column sums, with the e, f and e_L terms, give dG and dg = its reverse
//   cumulative sum; then the prologue (norms, gate, sigmoid) in reverse.
//
// The forward is linear in the state as well: S_c+1 = Phi^T S_c + Gc V with
// Gc = kn^T diag(f) T diag(b), so both chains are the same kernel.  Kernels:
//   coef_kernel   per (chunk, head): Phi, Phi^T, Bc, Gc as fp16 operand
//                 fragments, and T
//   chain_kernel  per (chain, value-column tile), both chains in one launch:
//                 the state entering every chunk (fp16); dS' of every chunk
//                 (fp16, last chunk first) and dS_0 (fp32)
//   grad_kernel   per (chunk, head): every input gradient of the chunk
// Products run on fp16 matrix cores with fp32 accumulation (the precision of
// the forward's chunk path); T = (I + A)^-1 is formed in fp32.
#include <algorithm>

#include "kda_bwd_common.h"

namespace kda {

namespace {

struct __attribute__((aligned(16))) RowsLds {
  float e[CH], f[CH], b[CH], gam[CH], g[CH], nq[CH], nk[CH];
  float eL;
  int len;
};
// per-row sums collected across waves (grad kernel); each wave stores its partial sums and they are added
// up wave by wave after a barrier, so a call's results do not depend on the order in which waves finish
struct __attribute__((aligned(16))) RedLds {
  float de[CH], df[CH], db[CH], wr[CH], wc[CH], qd[CH], kd[CH];
  float deL[NTH / 64];
  float part[4][NTH / 64][CH];
};

// Gate rows and normalised q, k rows (fp16, rows past the chunk's end zero).
__device__ void load_chunk(const BwdParams& p, int tok0, int len, int h, int hq, f16* QN, f16* KN, RowsLds& R) {
  const int t = threadIdx.x;
  if (t < CH) {
    const bool live = t < len;
    const size_t th = (size_t)(tok0 + min(t, len - 1)) * p.H + h;  // loads clamped, values selected
    const float graw = bf(p.g_raw[th]), blog = p.beta[th];
    const float m = live ? 1.f : 0.f;
    const float g = m * (-expf(p.A_log[h]) * softplus_(graw));
    const float b = m * sigmoid_(blog);
    float G = g;  // inclusive scan over the 64 lanes
#pragma unroll
    for (int o = 1; o < CH; o <<= 1) {
      const float y = __shfl_up(G, o);
      if (t >= o) G += y;
    }
    const float GL = __shfl(G, max(len, 1) - 1);
    R.g[t] = g;
    R.b[t] = b;
    R.gam[t] = G;
    R.e[t] = expf(G);
    R.f[t] = expf(GL - G);
    if (t == 0) {
      R.eL = expf(GL);
      R.len = len;
    }
  }
  // thread -> row t / 8, channels 16 (t % 8) .. + 15
  const int r = t >> 3, c0 = (t & 7) * 16;
  float qv[16], kv[16];
  {
    const size_t base = ((size_t)(tok0 + min(r, len - 1)) * p.H_qk + hq) * HD + c0;
    unpack_bf16x8(*reinterpret_cast<const uint4*>(p.q + base), qv);
    unpack_bf16x8(*reinterpret_cast<const uint4*>(p.q + base + 8), qv + 8);
    unpack_bf16x8(*reinterpret_cast<const uint4*>(p.k + base), kv);
    unpack_bf16x8(*reinterpret_cast<const uint4*>(p.k + base + 8), kv + 8);
    const float m = r < len ? 1.f : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      qv[i] *= m;
      kv[i] *= m;
    }
  }
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sq += qv[i] * qv[i];
    sk += kv[i] * kv[i];
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    sq += __shfl_xor(sq, o);
    sk += __shfl_xor(sk, o);
  }
  const float nq = sqrtf(sq + 1e-6f), nk = sqrtf(sk + 1e-6f), iq = 1.f / nq, ik = 1.f / nk;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    qv[i] *= iq;
    kv[i] *= ik;
  }
  *reinterpret_cast<f16x8*>(QN + r * LDW + c0) = to_f16x8(qv);
  *reinterpret_cast<f16x8*>(QN + r * LDW + c0 + 8) = to_f16x8(qv + 8);
  *reinterpret_cast<f16x8*>(KN + r * LDW + c0) = to_f16x8(kv);
  *reinterpret_cast<f16x8*>(KN + r * LDW + c0 + 8) = to_f16x8(kv + 8);
  if ((t & 7) == 0) {
    R.nq[r] = nq;
    R.nk[r] = nk;
  }
}

// P = qn kn^T and Gm = kn kn^T on this wave's tiles (row tile w / 2, column
// tiles 2 (w % 2) + j), kept in registers; M = lower(P . Lam) to Mt
// (transposed) and/or Mr (row-major); A = strict_lower(b Gm . Lam) to AF;
// then (SOLVE) T = (I + A)^-1 into T16 (fp16, row-major), ending with a
// barrier.  Without SOLVE only the Gram products and M.
template <bool SOLVE>
__device__ void gram_and_T(const f16* QN, const f16* KN, const RowsLds& R, f16* Mt, f16* Mr, float* AF, float* TF,
                           f16* T16, f32x4 (&P)[2], f32x4 (&Gm)[2]) {
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l16 = lane & 15, lg = lane >> 4;
  const int rt = w >> 1, ct0 = 2 * (w & 1);
#pragma unroll
  for (int j = 0; j < 2; ++j) P[j] = Gm[j] = zero4();
#pragma unroll
  for (int s = 0; s < HD / 32; ++s) {
    const f16x8 aq = frag_rm(QN, LDW, 16 * rt, 32 * s, lane), ak = frag_rm(KN, LDW, 16 * rt, 32 * s, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f16x8 bk = frag_rm(KN, LDW, 16 * (ct0 + j), 32 * s, lane);
      P[j] = mma_f16(aq, bk, P[j]);
      Gm[j] = mma_f16(ak, bk, Gm[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = 16 * (ct0 + j) + l16;
    f16x4 mcol;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * rt + 4 * lg + jj;
      const float lam = r >= c ? expf(fminf(R.gam[r] - R.gam[c], 0.f)) : 0.f;
      const float m = P[j][jj] * lam;
      mcol[jj] = (f16)m;
      if (Mr) Mr[r * LDN + c] = (f16)m;
      if (SOLVE) AF[r * LDF + c] = r > c ? R.b[r] * Gm[j][jj] * lam : 0.f;
    }
    if (Mt) *reinterpret_cast<f16x4*>(Mt + c * LDN + 16 * rt + 4 * lg) = mcol;
  }
  if (!SOLVE) return;
  __syncthreads();
  solve_T(AF, TF, T16);
}

}  // namespace

// ---------------------------------------------------------------------------
// coef_kernel: per (chunk, head), Phi and Bc as A-operand fragments of the
// adjoint's products.  A fragment (row tile m, slice s) holds, for lane l,
// row 16 m + l % 16 and contraction indices 32 s + 4 (l / 16) + e (e < 4) and
// 32 s + 16 + 4 (l / 16) + e - 4 (e >= 4): the order in which the C layout of
// two stacked 16-row tiles is a B operand (kda_device.h).  Computed as
//   Y1 = T^T diag(f) kn,  Phi^T = e_L I - Y1^T diag(b e) kn,
//   Z1 = T diag(b e) kn,  Bc^T = diag(e) qn - M Z1,
// so that the C layout of Phi^T and Bc^T is the fragment order of Phi and Bc.
// ---------------------------------------------------------------------------
// two workgroups per CU: at least four waves per SIMD
__global__ __launch_bounds__(NTH, 4) void bwd_coef_kernel(BwdParams p) {
  // 72 KB, two workgroups per CU: the fp32 T solve uses QN's space (qn is
  // read from the inputs after the Gram products) and one 128 x 64 buffer
  // holds Y1^T, then Z1^T
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * MAT_W + 2 * MAT_N + MAT_NT];
  __shared__ RowsLds R;
  __shared__ float be[CH];
  f16* QN = reinterpret_cast<f16*>(smem);
  f16* KN = reinterpret_cast<f16*>(smem + MAT_W);
  f16* M16 = reinterpret_cast<f16*>(smem + 2 * MAT_W);
  f16* T16 = reinterpret_cast<f16*>(smem + 2 * MAT_W + MAT_N);
  uint8_t* X = smem + 2 * MAT_W + 2 * MAT_N;
  float* AF = reinterpret_cast<float*>(X);
  float* TF = reinterpret_cast<float*>(smem);  // over QN
  f16* YZt = reinterpret_cast<f16*>(X);        // Y1^T, then Z1^T
  static_assert(MAT_F <= MAT_W && MAT_F <= MAT_NT, "fp32 solve fits");

  const int job = blockIdx.x, e = job / p.H, h = job - e * p.H, hq = h / (p.H / p.H_qk);
  const int2 ce = entry_of(p, e);
  const int tok0 = ce.x, len = ce.y;
  if (len <= 0) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l16 = lane & 15, lg = lane >> 4;
  const int d = 16 * w + l16;  // this lane's key column of the 128-wide results
  // e_i qn[i][d] for Bc^T's rows i = 32 s + 4 lg + jj (+ 16): raw q entries, loaded first
  uint16_t qraw[2][2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i = 32 * s + 16 * hh + 4 * lg + jj;
        qraw[s][hh][jj] = p.q[((size_t)(tok0 + min(i, len - 1)) * p.H_qk + hq) * HD + d];
      }
  load_chunk(p, tok0, len, h, hq, QN, KN, R);
  __syncthreads();
  if (t < CH) be[t] = R.b[t] * R.e[t];
  f32x4 P[2], Gm[2];
  gram_and_T<true>(QN, KN, R, nullptr, M16, AF, TF, T16, P, Gm);
  uint8_t* rec = p.brec + (size_t)job * p.rec_bytes;
  // T (fp16 rows) for the gradient kernel: thread -> row t / 8, columns 8 (t % 8) ..
  __builtin_nontemporal_store(*reinterpret_cast<const f16x8*>(T16 + (t >> 3) * LDN + 8 * (t & 7)),
                              reinterpret_cast<f16x8*>(rec + BR_T + t * 16));

  // Y1 = T^T diag(f) kn: rows i (4 tiles), columns d (tile w); K = 64
  {
    f32x4 Y1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Y1[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 bf_ = frag_cm_scaled(KN, LDW, R.f, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) Y1[i] = mma_f16(frag_cm(T16, LDN, 16 * i, 32 * s, lane), bf_, Y1[i]);
    }
    // (the solve's fp32 scratch is dead: gram_and_T ended with a barrier)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f16x4*>(YZt + d * LDN + 16 * i + 4 * lg) =
          f16x4{(f16)Y1[i][0], (f16)Y1[i][1], (f16)Y1[i][2], (f16)Y1[i][3]};
    // Gc = kn^T diag(f) T diag(b): its transpose is diag(b) Y1, rows i, columns d
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
  // Phi^T = e_L I - Y1^T diag(b e) kn: rows d' (8 tiles), columns d (tile w); K = 64 over tokens
  {
    f32x4 A[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 bb = frag_cm_scaled(KN, LDW, be, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) A[i] = mma_f16(frag_rm(YZt, LDN, 16 * i, 32 * s, lane), bb, A[i]);
    }
    const float eL = R.eL;
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
  // Phi = e_L I - (diag(b e) kn)^T Y1: rows d (8 tiles), columns d' (tile w); its C layout is the
  // fragment order of Phi^T, the forward chain's operator
  {
    const f16x8 by0 = frag_rm(YZt, LDN, 16 * w, 0, lane), by1 = frag_rm(YZt, LDN, 16 * w, 32, lane);
    const float eL = R.eL;
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // row tiles 4 half .. 4 half + 3: slices 2 half, 2 half + 1
      f32x4 A[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i] = mma_f16(frag_cm_scaled(KN, LDW, be, 16 * (4 * half + i), 0, lane), by0, zero4());
        A[i] = mma_f16(frag_cm_scaled(KN, LDW, be, 16 * (4 * half + i), 32, lane), by1, A[i]);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int s = 2 * half + s2;
        f16x8 o;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d0 = 32 * s + 4 * lg + jj, d1 = d0 + 16;
          o[jj] = (f16)((d0 == d ? eL : 0.f) - A[2 * s2][jj]);
          o[4 + jj] = (f16)((d1 == d ? eL : 0.f) - A[2 * s2 + 1][jj]);
        }
        __builtin_nontemporal_store(o, reinterpret_cast<f16x8*>(rec + BR_PHIT + (w * 4 + s) * FRAG_BYTES + lane * 16));
      }
    }
  }
  __syncthreads();  // Y1^T read for the last time
  // Z1 = T diag(b e) kn
  {
    f32x4 Z1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Z1[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 bb = frag_cm_scaled(KN, LDW, be, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) Z1[i] = mma_f16(frag_rm(T16, LDN, 16 * i, 32 * s, lane), bb, Z1[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f16x4*>(YZt + d * LDN + 16 * i + 4 * lg) =
          f16x4{(f16)Z1[i][0], (f16)Z1[i][1], (f16)Z1[i][2], (f16)Z1[i][3]};
  }
  __syncthreads();
  // Bc^T = diag(e) qn - M Z1: rows i (4 tiles), columns d (tile w); K = 64
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
        for (int jj = 0; jj < 4; ++jj) {
          const int i = 32 * s + 16 * hh + 4 * lg + jj;
          const float qn = i < len ? bf(qraw[s][hh][jj]) / R.nq[i] : 0.f;
          o[4 * hh + jj] = (f16)(R.e[i] * qn - B[2 * s + hh][jj]);
        }
      __builtin_nontemporal_store(o, reinterpret_cast<f16x8*>(rec + BR_BC + (w * 2 + s) * FRAG_BYTES + lane * 16));
    }
  }
}

// ---------------------------------------------------------------------------
// chain_kernel: the two chains over a sequence's chunks, which do not depend
// on each other, in one launch: the first half of the grid runs the forward
// chain, the second half the adjoint; one workgroup per (chain, 16 NCT value
// columns).
//   forward: S_c+1 = Phi^T S_c + Gc V_c, first chunk first, from the initial
//            state; stores S_c (the state entering chunk c, fp16).
//   adjoint: dS_c = Phi dS' + Bc dO', last chunk first, from dfinal; stores
//            dS' (the gradient of the state leaving chunk c, fp16) and dS_0
//            (fp32).
// Wave w holds rows 32 w .. 32 w + 31 of the state for every column tile in
// C layout (fp32); the four waves' rows, converted to fp16, are the B operand
// of the next step, and the token-row fragments (V or dO', loaded once per
// workgroup, a share per wave) go the same way: both through LDS, two
// barriers per chunk.  The next chunk's operator fragments and token rows are
// loaded while the current chunk is processed.
// ---------------------------------------------------------------------------
template <int NCT>
__global__ __launch_bounds__(256, 2) void bwd_chain_kernel(BwdParams p) {  // two workgroups per CU
  constexpr int NW = 8 / NCT;       // workgroups per chain
  constexpr int NF = 2 * NCT;       // token-row fragments per chunk (column tile, token slice)
  constexpr int FPW = (NF + 3) / 4;  // of which each wave loads up to FPW
  __shared__ __attribute__((aligned(16))) f16x8 sB[NCT][4][64];
  __shared__ __attribute__((aligned(16))) f16x8 sD[NF][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lg = lane >> 4;
  const int half = gridDim.x / 2;
  const bool fwd = (int)blockIdx.x < half;  // uniform over the workgroup
  const int off_a = fwd ? BR_PHIT : BR_PHI, off_b = fwd ? BR_GC : BR_BC;
  // the workgroups of a chain share an XCD (blocks are dealt to XCDs round robin; half is a multiple of 8)
  const int x = fwd ? blockIdx.x : blockIdx.x - half, xcd = x & 7, y = x >> 3, vt = y % NW,
            ch = (y / NW) * 8 + xcd;
  if (ch >= p.n_chains) return;
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
  const int v0 = 16 * NCT * vt;
  const size_t sbase = ((size_t)n * p.H + h) * HD * HD;
  const float* s_in = fwd ? p.s0 : p.dfinal;
  f32x4 S[NCT][2];
#pragma unroll
  for (int j = 0; j < NCT; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const size_t o = sbase + (size_t)(v0 + 16 * j + l16) * HD + 32 * w + 16 * i + 4 * lg;
      if (s_in) {
        const float4 x4 = *reinterpret_cast<const float4*>(s_in + o);
        S[j][i] = f32x4{x4.x, x4.y, x4.z, x4.w};
      } else {
        S[j][i] = zero4();
      }
    }
  const size_t vstride = (size_t)p.H * HD;
  const uint16_t* rows = fwd ? p.v : p.dout;
  const float rscale = fwd ? 1.f : p.scale;
  f16* st_base = reinterpret_cast<f16*>(fwd ? p.states : p.dstates);
  // raw token-row values are kept as loaded and converted in step(): a load's
  // result used right away would make the wait cover the prefetches issued
  // before it (the memory counter drains in order)
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));  // two raw values in one register
  struct Frags {
    f16x8 a[2][4], b[2][2];
    us2 d[FPW][4];
  };
  auto load = [&](Frags& F, int c) {
    // token rows first: tokens of slice s in fragment order (rows past the chunk's end clamped here,
    // zeroed in step)
    const int L = min(CH, len - c * CH);
    const uint16_t* rb = rows + ((size_t)tok0 + (size_t)c * CH) * vstride + (size_t)h * HD + v0 + l16;
#pragma unroll
    for (int q = 0; q < FPW; ++q) {
      const int f = w + 4 * q;
      if (f < NF) {
        const int j = f >> 1, s = f & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tk = 32 * s + (e < 4 ? 4 * lg + e : 16 + 4 * lg + e - 4);
          F.d[q][e >> 1][e & 1] = rb[(size_t)min(tk, L - 1) * vstride + 16 * j];
        }
      }
    }
    const uint8_t* rec = p.brec + ((size_t)(chunk0 + c) * p.H + h) * p.rec_bytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        F.a[i][s] = *reinterpret_cast<const f16x8*>(rec + off_a + ((2 * w + i) * 4 + s) * FRAG_BYTES + lane * 16);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        F.b[i][s] = *reinterpret_cast<const f16x8*>(rec + off_b + ((2 * w + i) * 2 + s) * FRAG_BYTES + lane * 16);
    }
  };
  auto step = [&](const Frags& F, int c) {
    f16* st = st_base + ((size_t)(chunk0 + c) * p.H + h) * HD * HD;
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
#pragma unroll
      for (int i = 0; i < 2; ++i)  // the state entering (forward) or the gradient leaving this chunk
        *reinterpret_cast<f16x4*>(st + (size_t)(v0 + 16 * j + l16) * HD + 32 * w + 16 * i + 4 * lg) =
            f16x4{(f16)S[j][i][0], (f16)S[j][i][1], (f16)S[j][i][2], (f16)S[j][i][3]};
      sB[j][w][lane] = f16x8{(f16)S[j][0][0], (f16)S[j][0][1], (f16)S[j][0][2], (f16)S[j][0][3],
                             (f16)S[j][1][0], (f16)S[j][1][1], (f16)S[j][1][2], (f16)S[j][1][3]};
    }
    const int L = min(CH, len - c * CH);
#pragma unroll
    for (int q = 0; q < FPW; ++q) {
      const int f = w + 4 * q;
      if (f < NF) {
        f16x8 dv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tk = 32 * (f & 1) + (e < 4 ? 4 * lg + e : 16 + 4 * lg + e - 4);
          dv[e] = (f16)(bf(F.d[q][e >> 1][e & 1]) * (tk < L ? rscale : 0.f));
        }
        sD[f][lane] = dv;
      }
    }
    __syncthreads();  // every wave's rows of the state and every token-row fragment published
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      f16x8 sb[4], sd[2];
#pragma unroll
      for (int s = 0; s < 4; ++s) sb[s] = sB[j][s][lane];
#pragma unroll
      for (int s = 0; s < 2; ++s) sd[s] = sD[2 * j + s][lane];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        f32x4 a = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) a = mma_f16(F.a[i][s], sb[s], a);
#pragma unroll
        for (int s = 0; s < 2; ++s) a = mma_f16(F.b[i][s], sd[s], a);
        S[j][i] = a;
      }
    }
    __syncthreads();  // every wave has read the published operands
  };
  // chunk k-th in processing order
  auto at = [&](int k) { return fwd ? min(k, nch - 1) : max(nch - 1 - k, 0); };
  Frags f0, f1;
  if (nch > 0) load(f0, at(0));
  for (int k = 0; k < nch; k += 2) {
    load(f1, at(k + 1));
    step(f0, at(k));
    if (k + 1 >= nch) break;
    load(f0, at(k + 2));
    step(f1, at(k + 1));
  }
  if (!fwd && p.dinit) {
#pragma unroll
    for (int j = 0; j < NCT; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<float4*>(p.dinit + sbase + (size_t)(v0 + 16 * j + l16) * HD + 32 * w + 16 * i + 4 * lg) =
            make_float4(S[j][i][0], S[j][i][1], S[j][i][2], S[j][i][3]);
  }
}

// ---------------------------------------------------------------------------
// grad_kernel: per (chunk, head), every gradient of the chunk's inputs.
// Eight waves; 64 x 128 results are split by 16-column tiles (wave w: tile
// w, all 64 rows), 64 x 64 ones by tiles (row tile w / 2, column tiles
// 2 (w % 2) + j), so a wave's registers hold the same elements from product
// to product.  S_c and dS' are read from global memory (fp16) as operands.
// ---------------------------------------------------------------------------
namespace {
// LDS of the grad kernel, bytes
constexpr int G_QN = 0, G_KN = G_QN + MAT_W, G_MT = G_KN + MAT_W, G_T16 = G_MT + MAT_N, G_TT = G_T16 + MAT_N,
              G_DO = G_TT + MAT_N,
              G_X = G_DO + MAT_W,             // bR + U
              G_DU = G_X + 2 * MAT_W, G_DR = G_DU + MAT_W, G_END = G_DR + MAT_W;
// after the last reads of dO', bR, U, dU, dR: the 64 x 64 results
constexpr int G_DT = G_DO, G_X1 = G_DT + MAT_N, G_DP = G_X1 + MAT_N, G_DPT = G_DP + MAT_N, G_DG = G_DPT + MAT_N,
              G_DGT = G_DG + MAT_N;
static_assert(G_DGT + MAT_N <= G_END, "64 x 64 results fit");
}  // namespace

__global__ __launch_bounds__(NTH) void bwd_grad_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[G_END];
  __shared__ RowsLds R;
  __shared__ RedLds red;
  f16* QN = reinterpret_cast<f16*>(smem + G_QN);
  f16* KN = reinterpret_cast<f16*>(smem + G_KN);
  f16* Mt = reinterpret_cast<f16*>(smem + G_MT);
  f16* T16 = reinterpret_cast<f16*>(smem + G_T16);
  f16* Tt16 = reinterpret_cast<f16*>(smem + G_TT);  // T^T, row-major
  f16* DO = reinterpret_cast<f16*>(smem + G_DO);
  f16* BR = reinterpret_cast<f16*>(smem + G_X);
  f16* U = reinterpret_cast<f16*>(smem + G_X + MAT_W);
  f16* DU = reinterpret_cast<f16*>(smem + G_DU);
  f16* DR = reinterpret_cast<f16*>(smem + G_DR);
  f16* DT = reinterpret_cast<f16*>(smem + G_DT);
  f16* X1t = reinterpret_cast<f16*>(smem + G_X1);
  f16* DP = reinterpret_cast<f16*>(smem + G_DP);
  f16* DPt = reinterpret_cast<f16*>(smem + G_DPT);
  f16* DG = reinterpret_cast<f16*>(smem + G_DG);
  f16* DGt = reinterpret_cast<f16*>(smem + G_DGT);

  const int job = blockIdx.x, G = p.H / p.H_qk;
  const int e = job / p.H, h = job - e * p.H, hq = h / G;
  const int2 ce = entry_of(p, e);
  const int tok0 = ce.x, len = ce.y;
  if (len <= 0) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, l16 = lane & 15, lg = lane >> 4;
  const f16* Sg = reinterpret_cast<const f16*>(p.states) + (size_t)job * HD * HD;    // [V][K]
  const f16* dSg = reinterpret_cast<const f16*>(p.dstates) + (size_t)job * HD * HD;  // [V][K]
  const size_t vrow = (size_t)p.H * HD;
  const uint16_t* vbase = p.v + (size_t)tok0 * vrow + (size_t)h * HD;

  const int vc = 16 * w + l16;  // this lane's column of the 64 x 128 results
  // Operands read from global memory, issued first so that their latency
  // overlaps the prologue: S_c and dS' as the B operands of kn S and kn dS'
  // (together they cover each block once, which also gives sum(dS' . S)),
  // and this lane's value entries.
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
  const f16x8 trow = *reinterpret_cast<const f16x8*>(p.brec + (size_t)job * p.rec_bytes + BR_T + t * 16);
  load_chunk(p, tok0, len, h, hq, QN, KN, R);
  {  // T (from the coefficient kernel) and T^T: thread -> row t / 8, columns 8 (t % 8) ..
    const int r = t >> 3, c0 = 8 * (t & 7);
    *reinterpret_cast<f16x8*>(T16 + r * LDN + c0) = trow;
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) Tt16[(c0 + e2) * LDN + r] = trow[e2];
  }
  // dO' rows (fp16, zero past the chunk's end): thread -> row t / 8, 16 columns
  {
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
  __syncthreads();
  f32x4 P[2], Gm[2];
  gram_and_T<false>(QN, KN, R, Mt, nullptr, nullptr, nullptr, nullptr, P, Gm);
  {  // sum(dS' . S) over the 128 x 128 block
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) a += (float)sfr[s][j] * (float)dsfr[s][j];
    a = sum64(a);
    if (lane == 0) red.deL[w] = a;
  }
  // ---- KS = kn S (rows r, columns v); R = V - diag(e) KS; bR -------------
  f32x4 KS[4], RR[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) KS[i] = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) KS[i] = mma_f16(frag_rm(KN, LDW, 16 * i, 32 * s, lane), sfr[s], KS[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * i + 4 * lg + jj;
      const float vv = bf(vraw[i][jj]) * (r < len ? 1.f : 0.f);
      RR[i][jj] = vv - R.e[r] * KS[i][jj];
      BR[r * LDW + vc] = (f16)(R.b[r] * RR[i][jj]);
    }
  __syncthreads();  // bR complete
  // ---- U^T = (b R)^T T^T (rows v: tile w, columns r: 4 tiles) -> U row-major
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
  }
  // ---- dU = diag(f) kn dS' + M^T dO' (rows r, columns v) -----------------
  {
    f32x4 D[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) D[i] = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) D[i] = mma_f16(frag_rm(KN, LDW, 16 * i, 32 * s, lane), dsfr[s], D[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) D[i][jj] *= R.f[16 * i + 4 * lg + jj];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 b = frag_cm(DO, LDW, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) D[i] = mma_f16(frag_rm(Mt, LDN, 16 * i, 32 * s, lane), b, D[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) DU[(16 * i + 4 * lg + jj) * LDW + vc] = (f16)D[i][jj];
  }
  __syncthreads();  // U, dU complete
  // ---- Y = T^T dU; dV = diag(b) Y; db += rowsum(Y . R); de -= rowsum(dV . KS)
  {
    f32x4 Y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Y[i] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 b = frag_cm(DU, LDW, 16 * w, 32 * s, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[i] = mma_f16(frag_rm(Tt16, LDN, 16 * i, 32 * s, lane), b, Y[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * i + 4 * lg + jj;
        const float dv = R.b[r] * Y[i][jj];
        // outputs are written once and not read again: non-temporal, so they do not evict inputs from L2
        if (r < len) __builtin_nontemporal_store(dv, p.dv + (size_t)(tok0 + r) * vrow + (size_t)h * HD + vc);
        DR[r * LDW + vc] = (f16)dv;
        const float db = rowsum16(Y[i][jj] * RR[i][jj]), de = rowsum16(dv * KS[i][jj]);
        if (l16 == 0) {
          red.part[0][w][r] = db;
          red.part[1][w][r] = -de;
        }
      }
  }
  __syncthreads();  // dR complete
  if (t < CH) {
    float db = 0.f, de = 0.f;
#pragma unroll
    for (int q = 0; q < NTH / 64; ++q) {
      db += red.part[0][q][t];
      de += red.part[1][q][t];
    }
    red.db[t] = db;
    red.de[t] = de;
  }
  // ---- [dO'; dR] S^T and U dS'^T (rows r, columns d: tile w) ------------------
  f32x4 dqn[4], dkn[4];
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
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * i + 4 * lg + jj;
        dqn[i][jj] = R.e[r] * SD[i][jj];
        dkn[i][jj] = R.f[r] * UD[i][jj] - R.e[r] * DRS[i][jj];
        const float de = rowsum16((float)QN[r * LDW + vc] * SD[i][jj]);
        const float df = rowsum16((float)KN[r * LDW + vc] * UD[i][jj]);
        if (l16 == 0) {
          red.part[2][w][r] = de;
          red.part[3][w][r] = df;
        }
      }
  }
  // ---- dM = dO' U^T, dT = dU (b R)^T (64 x 64 tiles of this wave) -------------
  const int rt = w >> 1, ct0 = 2 * (w & 1);
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
    if (t < CH) {
      float de = 0.f, df = 0.f;
#pragma unroll
      for (int q = 0; q < NTH / 64; ++q) {
        de += red.part[2][q][t];
        df += red.part[3][q][t];
      }
      red.de[t] += de;
      red.df[t] = df;
    }
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
  // ---- dA = -T^T X1 and the 64 x 64 elementwise terms ----------------------
  {
    f32x4 DA[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) DA[j] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 a = frag_rm(Tt16, LDN, 16 * rt, 32 * s, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) DA[j] = mma_f16(a, frag_rm(X1t, LDN, 16 * (ct0 + j), 32 * s, lane), DA[j]);
    }
    float db2[4] = {0.f, 0.f, 0.f, 0.f}, wr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = 16 * (ct0 + j) + l16;
      f16x4 pc, gc;
      float wcol = 0.f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * rt + 4 * lg + jj;
        const float lam = r >= c ? expf(fminf(R.gam[r] - R.gam[c], 0.f)) : 0.f;
        const float dm = r >= c ? DM[j][jj] : 0.f;
        const float da = r > c ? -DA[j][jj] : 0.f;
        const float dp = dm * lam, dgm = R.b[r] * da * lam;
        // W's diagonal (dM_rr P_rr) enters its row sum and its column sum alike and cancels in dG exactly;
        // left out, its rounding cannot swamp dG when harsh decays make dG small
        const float wv = r != c ? (R.b[r] * da * Gm[j][jj] + dm * P[j][jj]) * lam : 0.f;
        DP[r * LDN + c] = (f16)dp;
        DG[r * LDN + c] = (f16)dgm;
        pc[jj] = (f16)dp;
        gc[jj] = (f16)dgm;
        wcol += wv;
        db2[jj] += rowsum16(da * Gm[j][jj] * lam);
        wr[jj] += rowsum16(wv);
      }
      *reinterpret_cast<f16x4*>(DPt + c * LDN + 16 * rt + 4 * lg) = pc;
      *reinterpret_cast<f16x4*>(DGt + c * LDN + 16 * rt + 4 * lg) = gc;
      wcol += __shfl_xor(wcol, 16);
      wcol += __shfl_xor(wcol, 32);
      if (lg == 0) red.part[1][rt][c] = wcol;  // column c's share from row tile rt
    }
    if (l16 == 0) {  // row tile rt's two waves: column tiles 0, 1 and 2, 3
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        red.part[0][w & 1][16 * rt + 4 * lg + jj] = db2[jj];
        red.part[0][2 + (w & 1)][16 * rt + 4 * lg + jj] = wr[jj];
      }
    }
  }
  __syncthreads();
  if (t < CH) {
    red.db[t] += red.part[0][0][t] + red.part[0][1][t];
    red.wr[t] = red.part[0][2][t] + red.part[0][3][t];
    red.wc[t] = (red.part[1][0][t] + red.part[1][1][t]) + (red.part[1][2][t] + red.part[1][3][t]);
  }
  // ---- dqn += dP kn;  dkn += (dGm + dGm^T) kn + dP^T qn ---------------------
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const f16x8 bk = frag_cm(KN, LDW, 16 * w, 32 * s, lane), bq = frag_cm(QN, LDW, 16 * w, 32 * s, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x8 ag = frag_rm(DG, LDN, 16 * i, 32 * s, lane) + frag_rm(DGt, LDN, 16 * i, 32 * s, lane);
      dqn[i] = mma_f16(frag_rm(DP, LDN, 16 * i, 32 * s, lane), bk, dqn[i]);
      dkn[i] = mma_f16(ag, bk, dkn[i]);
      dkn[i] = mma_f16(frag_rm(DPt, LDN, 16 * i, 32 * s, lane), bq, dkn[i]);
    }
  }
  // row dots qn . dqn, kn . dkn
  float qf[4][4], kf[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * i + 4 * lg + jj;
      const float qx = (float)QN[r * LDW + vc], kx = (float)KN[r * LDW + vc];
      qf[i][jj] = qx;
      kf[i][jj] = kx;
      const float qd = rowsum16(qx * dqn[i][jj]), kd = rowsum16(kx * dkn[i][jj]);
      if (l16 == 0) {
        red.part[2][w][r] = qd;
        red.part[3][w][r] = kd;
      }
    }
  __syncthreads();
  if (t < 2 * CH) {  // the row dots, wave by wave
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < NTH / 64; ++q) a += red.part[2 + (t >> 6)][q][t & (CH - 1)];
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
        const float gq = (dqn[i][jj] - qf[i][jj] * red.qd[r]) / R.nq[r];
        const float gk = (dkn[i][jj] - kf[i][jj] * red.kd[r]) / R.nk[r];
        if (G == 1) {
          __builtin_nontemporal_store(gq, p.dq + o);
          __builtin_nontemporal_store(gk, p.dk + o);
        } else {
          atomicAdd(p.dq + o, gq);
          atomicAdd(p.dk + o, gk);
        }
      }
    }
  // ---- dG, dg (reverse cumulative sum), dg_raw, dbeta, dA_log --------------
  if (t < CH) {
    const bool live = t < len;
    float deL = 0.f;
#pragma unroll
    for (int i = 0; i < NTH / 64; ++i) deL += red.deL[i];
    const float dff = live ? red.df[t] * R.f[t] : 0.f;
    const float sum_df = sum64(dff);
    float dG = live ? red.wr[t] - red.wc[t] + red.de[t] * R.e[t] - dff : 0.f;
    if (t == len - 1) dG += sum_df + deL * R.eL;
    float acc = dG;  // reverse inclusive scan over the 64 lanes
#pragma unroll
    for (int o = 1; o < CH; o <<= 1) {
      const float y = __shfl_down(acc, o);
      if (t + o < CH) acc += y;
    }
    const float dal = sum64(live ? acc * R.g[t] : 0.f);
    if (live) {
      const size_t th = (size_t)(tok0 + t) * p.H + h;
      const float b = R.b[t];
      p.dg_raw[th] = acc * (-expf(p.A_log[h])) * sigmoid_(bf(p.g_raw[th]));
      p.dbeta[th] = red.db[t] * b * (1.f - b);
    }
    if (t == 0) atomicAdd(p.dA_log + h, dal);
  }
}

__global__ __launch_bounds__(256) void bwd_fill_kernel(float* a, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) a[i] = 0.f;
}

void launch_chains(const BwdParams& p, hipStream_t stream) {
  if (p.n_chains <= 0) return;
  // the narrowest column tiles that keep every workgroup of both chains resident (two per CU)
  const int slots = 2 * device_cu_count(), g8 = (p.n_chains + 7) / 8 * 8;
  if (2 * g8 * 8 <= slots) bwd_chain_kernel<1><<<2 * g8 * 8, 256, 0, stream>>>(p);
  else if (2 * g8 * 4 <= slots) bwd_chain_kernel<2><<<2 * g8 * 4, 256, 0, stream>>>(p);
  else if (2 * g8 * 2 <= slots) bwd_chain_kernel<4><<<2 * g8 * 2, 256, 0, stream>>>(p);
  else bwd_chain_kernel<8><<<2 * g8, 256, 0, stream>>>(p);
}

void launch_bwd(const BwdParams& p, size_t qk_floats, int stage, hipStream_t stream) {
  const int jobs = p.n_entries * p.H;
  if (stage == 0) {
    if (p.H != p.H_qk && qk_floats > 0) {  // dq, dk are accumulated over each group's value heads
      bwd_fill_kernel<<<1024, 256, 0, stream>>>(p.dq, qk_floats);
      bwd_fill_kernel<<<1024, 256, 0, stream>>>(p.dk, qk_floats);
    }
    bwd_fill_kernel<<<1, 256, 0, stream>>>(p.dA_log, (size_t)p.H);
    if (jobs > 0) {
      if (p.per_channel) launch_coef_pc(p, stream);
      else bwd_coef_kernel<<<jobs, NTH, 0, stream>>>(p);
    }
  } else if (stage == 1) {
    launch_chains(p, stream);
  } else if (jobs > 0) {
    if (p.per_channel) launch_grad_pc(p, stream);
    else bwd_grad_kernel<<<jobs, NTH, 0, stream>>>(p);
  }
}

}  // namespace kda
