// kda_chunk.hip -- chunk-local kernel: everything about one (64-token chunk,
// value head) that does not depend on the state entering the chunk.
//
// For a chunk of L <= 64 tokens with normalised keys/queries kn, qn, gates g
// (<= 0) and betas b, write Gamma_r = sum_{j<=r} g_j (per key channel).  With
// S0 the state entering the chunk, the chunk's effect is the WY/UT form of
// the gated delta rule:
//   A[r][i] = b_r sum_c kn_rc kn_ic exp(Gamma_rc - Gamma_ic)   (i < r)
//   M[r][i] =     sum_c qn_rc kn_ic exp(Gamma_rc - Gamma_ic)   (i <= r)
//   T = (I + A)^-1,  W = T diag(b) Khat,  Khat = exp(Gamma) . kn
//   U = T diag(b) V - W S0
//   O = scale * (Qhat S0 + M U),  Qhat = exp(Gamma) . qn
//   S_L = Diag(exp(Gamma_L)) S0 + Kbar^T U,  Kbar = exp(Gamma_L - Gamma) . kn
// This kernel computes A, M, T, W, Qhat, Kbar, T diag(b) and exp(Gamma_L)
// and stores them as MFMA fragments (kda_device.h) for the recurrence.
//
// Decay factoring (per key channel): the chunk is cut into four 16-token
// sub-chunks; d_j is token j's decay exp(g_j) and D_n the product of d over
// sub-chunk n.
//   rho_r = prod_{16n <= j <= r} d_j  (<= 1),  kappa_i = prod_{i < j < 16n+16} d_j (<= 1)
// For r in sub-chunk b and i in sub-chunk a < b:
//   exp(Gamma_r - Gamma_i) = rho_r * (prod_{a<m<b} D_m) * kappa_i, every factor <= 1,
// so those blocks use fp16 operands without overflow.  Diagonal blocks use
//   exp(Gamma_r - Gamma_i) = (rho_r / D_b) * kappa_i
// whose first factor can reach 1/D_b; they run with split-bf16 operands
// (three bf16 products, ~16 significant bits) while D_b >= 2^-100, and fall
// back to an exact per-channel evaluation in the log domain otherwise.
// In scalar-gate mode exp(Gamma_r - Gamma_i) is one number per (r, i) and is
// applied after the Gram products.
//
// Work layout: 512 threads (8 waves, two per SIMD so one wave's LDS and
// transcendental latency hides behind the other's work).  The kernel is
// persistent: each workgroup walks (chunk, head) jobs with a stride of the
// grid size and prefetches the next job's q, k, gate and beta into
// registers while it computes the current one.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

constexpr int NT = 512;  // threads per workgroup
constexpr int LS = 132;  // row stride (floats) of the [64][128] operand arrays
constexpr int MS = 68;   // row stride (floats) of the [64][64] matrices
constexpr float LOG2E = 1.4426950408889634f;
constexpr float TINY_D = 0x1p-100f;  // smallest sub-chunk decay the fast diagonal path takes

// LDS layout (bytes)
constexpr int L_KR = 0;                          // kn*rho (kn in scalar mode), fp32 [64][LS]
constexpr int L_QR = L_KR + CH * LS * 4;         // qn*rho (qn)
constexpr int L_YS = L_QR + CH * LS * 4;         // raw gates, then kn*kappa (unused in scalar mode)
constexpr int L_AM = L_YS + CH * LS * 4;         // A [64][MS]; after the inverse: Khat^T fragments
constexpr int L_TM = L_AM + CH * MS * 4;         // T [64][MS]; before the inverse: fallback scratch
constexpr int L_EP = L_TM + CH * MS * 4;         // exp(Gamma before sub-chunk n)[c]      [4][128]
constexpr int L_EG = L_EP + NSUB * HD * 4;       // exp(Gamma_L - Gamma_end(n))[c]         [4][128]
constexpr int L_LAM = L_EG + NSUB * HD * 4;      // pair factors for blocks (b, a <= b)    [10][128]
constexpr int L_DS = L_LAM + 10 * HD * 4;        // D_n[c]                                 [4][128]
constexpr int L_MX = L_DS + NSUB * HD * 4;       // M fragment halves handed between waves [2][64] f16x4
constexpr int L_ROW = L_MX + 2 * 64 * 8;         // beta, exp(Gamma), exp(Gamma_L-Gamma), Gamma, 1/|k|, 1/|q|
constexpr int L_FLAG = L_ROW + 6 * CH * 4;       // unsafe[4], any
constexpr int LDS_BYTES = L_FLAG + 8 * 4;
static_assert(16 * 64 * 16 <= CH * MS * 4, "Khat^T fragments must fit in the A region");
static_assert(3328 * 4 <= CH * MS * 4, "fallback scratch must fit in the T region");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// ROW sub-arrays
constexpr int R_BETA = 0, R_EG = CH, R_EGL = 2 * CH, R_G = 3 * CH, R_RK = 4 * CH, R_RQ = 5 * CH;

__device__ __forceinline__ int pair_index(int b, int a) { return b * (b + 1) / 2 + a; }

__device__ __forceinline__ void store_frag(uint8_t* rec, int off, int frag, int lane, const float* v) {
  *reinterpret_cast<f16x8*>(rec + off + frag * FRAG_BYTES + lane * 16) = to_f16x8(v);
}

__device__ __forceinline__ void ld8(const float* p, float* x) {
  *reinterpret_cast<float4*>(x) = *reinterpret_cast<const float4*>(p);
  *reinterpret_cast<float4*>(x + 4) = *reinterpret_cast<const float4*>(p + 4);
}
__device__ __forceinline__ void ld4(const float* p, float* x) {
  *reinterpret_cast<float4*>(x) = *reinterpret_cast<const float4*>(p);
}

// Registers prefetched for one job: row tid/8, channels 16*(tid%8) .. +15.
struct Pref {
  uint4 q[2], k[2], g[2];  // bf16; g only in per-channel mode
  uint32_t gs;             // scalar gate of row tid%64, bf16 in the low half
  float beta;              // logit of row tid/8
};

template <bool PER_CHANNEL>
__device__ __forceinline__ void prefetch(Pref& P, const ChunkParams& p, int4 ce, int h, int tid) {
  // Loads are unconditional (rows past the chunk end are clamped to its last
  // row and zeroed when used) so they issue back to back without waits.
  const int len = ce.z, tok0 = ce.y;
  if (len <= 0) return;
  const int hq = h / (p.H / p.H_qk);
  const int last = len - 1;
  const int r = min(tid >> 3, last), c0 = (tid & 7) * 16;
  const size_t base = ((size_t)(tok0 + r) * p.H_qk + hq) * HD + c0;
  const uint4* qp = reinterpret_cast<const uint4*>(p.q + base);
  const uint4* kp = reinterpret_cast<const uint4*>(p.k + base);
  P.q[0] = qp[0];
  P.q[1] = qp[1];
  P.k[0] = kp[0];
  P.k[1] = kp[1];
  P.beta = p.beta[(size_t)(tok0 + r) * p.H + h];
  if (PER_CHANNEL) {
    const uint4* gp = reinterpret_cast<const uint4*>(p.g_raw + ((size_t)(tok0 + r) * p.H + h) * HD + c0);
    P.g[0] = gp[0];
    P.g[1] = gp[1];
  } else {
    P.gs = p.g_raw[(size_t)(tok0 + min(tid & 63, last)) * p.H + h];
  }
}

// One A block (b, a) (fp32, to LDS) and its M^T block (returned in C layout:
// lane holds M[16b + l16][16a + 4lg + j]).  K = 128 key channels, 4 slices.
template <bool PER_CHANNEL>
__device__ __forceinline__ void ablock(int b, int a, const float* KR, const float* QR, const float* YSrc,
                                       const float* LAM, const float* ROW, float* AM, int l16, int lg,
                                       f32x4& accM) {
  const int r = SUB * b + l16, i = SUB * a + l16;
  const bool diag = (a == b);
  f32x4 accA = zero4();
  accM = zero4();
#pragma unroll 1
  for (int s = 0; s < 4; ++s) {
    const int c0 = 32 * s + 8 * lg;
    float xk[8], xq[8], y[8];
    ld8(&KR[r * LS + c0], xk);
    ld8(&QR[r * LS + c0], xq);
    ld8(&YSrc[i * LS + c0], y);
    if (PER_CHANNEL) {
      float lam[8];
      ld8(&LAM[pair_index(b, a) * HD + c0], lam);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        xk[q] *= lam[q];
        xq[q] *= lam[q];
      }
    }
    if (PER_CHANNEL && diag) {
      bf16x8 xkh, xkl, xqh, xql, yh, yl;
      split_bf16x8(xk, xkh, xkl);
      split_bf16x8(xq, xqh, xql);
      split_bf16x8(y, yh, yl);
      accA = mma_bf16(xkh, yh, accA);
      accA = mma_bf16(xkh, yl, accA);
      accA = mma_bf16(xkl, yh, accA);
      accM = mma_bf16(yh, xqh, accM);
      accM = mma_bf16(yl, xqh, accM);
      accM = mma_bf16(yh, xql, accM);
    } else {
      const f16x8 yf = to_f16x8(y);
      accA = mma_f16(to_f16x8(xk), yf, accA);
      accM = mma_f16(yf, to_f16x8(xq), accM);
    }
  }
  // A block: lane holds A[16b + 4lg + j][16a + l16]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = SUB * b + 4 * lg + j, ii = SUB * a + l16;
    float v = 0.f;
    if (ii < rr) {
      v = accA[j];
      if (!PER_CHANNEL) v *= exp2f((ROW[R_G + rr] - ROW[R_G + ii]) * LOG2E);
      v *= ROW[R_BETA + rr];
    }
    AM[rr * MS + ii] = v;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = SUB * b + l16, ii = SUB * a + 4 * lg + j;
    float v = 0.f;
    if (ii <= rr) {
      v = accM[j];
      if (!PER_CHANNEL) v *= exp2f((ROW[R_G + rr] - ROW[R_G + ii]) * LOG2E);
    }
    accM[j] = v;
  }
}

}  // namespace

template <bool PER_CHANNEL>
__global__ __launch_bounds__(NT) void chunk_local_kernel(const ChunkParams p, const int n_jobs) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* KR = reinterpret_cast<float*>(smem + L_KR);
  float* QR = reinterpret_cast<float*>(smem + L_QR);
  float* YS = reinterpret_cast<float*>(smem + L_YS);
  float* AM = reinterpret_cast<float*>(smem + L_AM);
  f16x8* KH = reinterpret_cast<f16x8*>(smem + L_AM);
  float* TM = reinterpret_cast<float*>(smem + L_TM);
  float* EP = reinterpret_cast<float*>(smem + L_EP);
  float* EG = reinterpret_cast<float*>(smem + L_EG);
  float* LAM = reinterpret_cast<float*>(smem + L_LAM);
  float* DS = reinterpret_cast<float*>(smem + L_DS);
  f16x4* MX = reinterpret_cast<f16x4*>(smem + L_MX);
  float* ROW = reinterpret_cast<float*>(smem + L_ROW);
  int* FLAG = reinterpret_cast<int*>(smem + L_FLAG);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const float* YSrc = PER_CHANNEL ? YS : KR;

  // Job indices are wave-uniform; the schedule and A_log are read through
  // the constant address space so these loads go to the scalar unit and
  // waiting for them never waits on the vector-memory counter that the
  // prefetch and the record stores share.
  const int H = p.H;
  typedef __attribute__((address_space(4))) const int cint;
  typedef __attribute__((address_space(4))) const float cfloat;
  cint* chunks = (cint*)p.chunks;
  cfloat* A_log = (cfloat*)p.A_log;
  auto entry = [&](int i) {
    return make_int4(chunks[4 * i], chunks[4 * i + 1], chunks[4 * i + 2], chunks[4 * i + 3]);
  };
  int job = __builtin_amdgcn_readfirstlane(blockIdx.x);
  if (job >= n_jobs) return;
  int4 ce = entry(__builtin_amdgcn_readfirstlane(job / H));
  float alog = A_log[__builtin_amdgcn_readfirstlane(job % H)];
  Pref nxt;
  prefetch<PER_CHANNEL>(nxt, p, ce, job % H, tid);

  for (;;) {
    const Pref cur = nxt;
    const int4 ce_cur = ce;
    const float alog_cur = alog;
    const int e = __builtin_amdgcn_readfirstlane(job / H), h = __builtin_amdgcn_readfirstlane(job % H);
    const int nj = __builtin_amdgcn_readfirstlane(job + (int)gridDim.x);
    if (nj < n_jobs) {
      ce = entry(__builtin_amdgcn_readfirstlane(nj / H));
      alog = A_log[__builtin_amdgcn_readfirstlane(nj % H)];
      prefetch<PER_CHANNEL>(nxt, p, ce, nj % H, tid);
    }
    const int len = ce_cur.z;
    if (len > 0) {  // uniform over the workgroup
      uint8_t* rec = p.rec + ((size_t)e * p.H + h) * REC_BYTES;
      if (tid < 8) FLAG[tid] = 0;

      // ---- A: L2-normalise q, k rows; beta; stage raw gates -----------------
      {
        const int r = tid >> 3, c0 = (tid & 7) * 16;
        const bool live = r < len;
        float qv[16], kv[16];
        unpack_bf16x8(cur.q[0], qv);
        unpack_bf16x8(cur.q[1], qv + 8);
        unpack_bf16x8(cur.k[0], kv);
        unpack_bf16x8(cur.k[1], kv + 8);
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          qv[i] = live ? qv[i] : 0.f;
          kv[i] = live ? kv[i] : 0.f;
          sq += qv[i] * qv[i];
          sk += kv[i] * kv[i];
        }
        sq += __shfl_xor(sq, 1);
        sk += __shfl_xor(sk, 1);
        sq += __shfl_xor(sq, 2);
        sk += __shfl_xor(sk, 2);
        sq += __shfl_xor(sq, 4);
        sk += __shfl_xor(sk, 4);
        const float rq = 1.f / sqrtf(sq + 1e-6f), rk = 1.f / sqrtf(sk + 1e-6f);
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          *reinterpret_cast<float4*>(&QR[r * LS + c0 + i]) =
              make_float4(qv[i] * rq, qv[i + 1] * rq, qv[i + 2] * rq, qv[i + 3] * rq);
          *reinterpret_cast<float4*>(&KR[r * LS + c0 + i]) =
              make_float4(kv[i] * rk, kv[i + 1] * rk, kv[i + 2] * rk, kv[i + 3] * rk);
        }
        if (PER_CHANNEL) {
          float gv[16];
          unpack_bf16x8(cur.g[0], gv);
          unpack_bf16x8(cur.g[1], gv + 8);
#pragma unroll
          for (int i = 0; i < 16; i += 4)
            *reinterpret_cast<float4*>(&YS[r * LS + c0 + i]) = make_float4(gv[i], gv[i + 1], gv[i + 2], gv[i + 3]);
        }
        if ((tid & 7) == 0) {
          ROW[R_BETA + r] = live ? sigmoidf_(cur.beta) : 0.f;
          ROW[R_RK + r] = rk;
          ROW[R_RQ + r] = rq;
        }
      }
      __syncthreads();

      // ---- B: gates -> decay factors ----------------------------------------
      const float a_h = __expf(alog_cur);
      if (PER_CHANNEL) {
        // thread (key channel c, sub-chunk n)
        const int c = tid & 127, n = tid >> 7;
        float d[SUB];
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
          const int r = n * SUB + i;
          float dd, g;
          gate_decay(YS[r * LS + c], a_h, dd, g);
          d[i] = (r < len) ? dd : 1.f;
        }
        float kap = 1.f;
#pragma unroll
        for (int i = SUB - 1; i >= 0; --i) {
          const int r = n * SUB + i;
          YS[r * LS + c] = KR[r * LS + c] * kap;
          kap *= d[i];
        }
        float rho = 1.f;
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
          const int r = n * SUB + i;
          rho *= d[i];
          KR[r * LS + c] *= rho;
          QR[r * LS + c] *= rho;
        }
        DS[n * HD + c] = rho;
        if (!(rho >= TINY_D)) {
          FLAG[n] = 1;
          FLAG[4] = 1;
        }
      } else if (wave == 0) {
        float d = 1.f, g = 0.f;
        if (lane < len) gate_decay(bf16_to_f32((uint16_t)cur.gs), a_h, d, g);
        float G = g;  // inclusive prefix sum over the 64 tokens
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(G, off);
          if (lane >= off) G += y;
        }
        const float GL = __shfl(G, 63);
        ROW[R_EG + lane] = exp2f(G * LOG2E);
        ROW[R_EGL + lane] = exp2f((GL - G) * LOG2E);
        ROW[R_G + lane] = G;
      }
      __syncthreads();

      // ---- B2: per-channel factor vectors; exp(Gamma_L) ----------------------
      if (PER_CHANNEL) {
        if (tid < HD) {
          const int c = tid;
          const float Dn[4] = {DS[c], DS[HD + c], DS[2 * HD + c], DS[3 * HD + c]};
          EP[c] = 1.f;
          EP[HD + c] = Dn[0];
          EP[2 * HD + c] = Dn[0] * Dn[1];
          EP[3 * HD + c] = Dn[0] * Dn[1] * Dn[2];
          EG[c] = Dn[1] * Dn[2] * Dn[3];
          EG[HD + c] = Dn[2] * Dn[3];
          EG[2 * HD + c] = Dn[3];
          EG[3 * HD + c] = 1.f;
#pragma unroll
          for (int b = 0; b < NSUB; ++b) {
#pragma unroll
            for (int a = 0; a <= b; ++a) {
              float f = 1.f;
              if (a == b) f = Dn[b] >= TINY_D ? 1.f / Dn[b] : 0.f;
              else {
#pragma unroll
                for (int m = a + 1; m < b; ++m) f *= Dn[m];
              }
              LAM[pair_index(b, a) * HD + c] = f;
            }
          }
          *reinterpret_cast<float*>(rec + REC_GL + 4 * c) = Dn[0] * Dn[1] * Dn[2] * Dn[3];
        }
        __syncthreads();
      } else if (tid < HD) {
        *reinterpret_cast<float*>(rec + REC_GL + 4 * tid) = ROW[R_EG + CH - 1];
      }

      // ---- D: A and M blocks on the matrix cores -----------------------------
      // Waves 0..3 take the diagonal blocks (b, b) (split-bf16, the costliest);
      // waves 4..7 the off-diagonal ones.  M fragment (t, s) covers blocks
      // (t, 2s) and (t, 2s+1); halves computed by different waves meet in MX.
      //   w0 (0,0) -> M(0,0)        w4 (1,0) + half from w1 -> M(1,0)
      //   w1 (1,1) -> MX[0]         w5 (3,2) + half from w3 -> M(3,1)
      //   w2 (2,2) -> M(2,1)        w6 (2,0),(2,1) -> M(2,0)
      //   w3 (3,3) -> MX[1]         w7 (3,0),(3,1) -> M(3,0)
      f32x4 m0 = zero4(), m1 = zero4();
      if (wave < 4) {
        ablock<PER_CHANNEL>(wave, wave, KR, QR, YSrc, LAM, ROW, AM, l16, lg, m0);
      } else if (wave == 4) {
        ablock<PER_CHANNEL>(1, 0, KR, QR, YSrc, LAM, ROW, AM, l16, lg, m0);
      } else if (wave == 5) {
        ablock<PER_CHANNEL>(3, 2, KR, QR, YSrc, LAM, ROW, AM, l16, lg, m0);
      } else if (wave == 6) {
        ablock<PER_CHANNEL>(2, 0, KR, QR, YSrc, LAM, ROW, AM, l16, lg, m0);
        ablock<PER_CHANNEL>(2, 1, KR, QR, YSrc, LAM, ROW, AM, l16, lg, m1);
      } else {
        ablock<PER_CHANNEL>(3, 0, KR, QR, YSrc, LAM, ROW, AM, l16, lg, m0);
        ablock<PER_CHANNEL>(3, 1, KR, QR, YSrc, LAM, ROW, AM, l16, lg, m1);
      }

      // ---- D': exact diagonal blocks when a sub-chunk's decay span is huge ---
      // Rare (a channel decays by more than 2^-100 within 16 tokens).  Runs
      // before anything consumes A or M: the unsafe diagonal blocks of A are
      // overwritten and the affected M values replaced in m0 of waves 0..3.
      // Scratch lives in the (not yet used) T region: normalised k, q rows of
      // the sub-chunk and the running log-decay for 64 key channels at a time.
      if (PER_CHANNEL && FLAG[4]) {
        const int hq = h / (p.H / p.H_qk);
        float* SK = TM;         // [16][64]
        float* SQ = TM + 1024;  // [16][64]
        float* SG = TM + 2048;  // [16][64]
        float* FM = TM + 3072;  // [16][16] M sums
#pragma unroll 1
        for (int b = 0; b < NSUB; ++b) {
          if (!FLAG[b]) continue;
          const int rr = (tid >> 4) & 15, ii = tid & 15;
          float accA = 0.f, accM = 0.f;
#pragma unroll 1
          for (int half = 0; half < 2; ++half) {
            __syncthreads();
            if (tid < 64) {
              const int c = half * 64 + tid;
              float run = 0.f;
#pragma unroll 1
              for (int i = 0; i < SUB; ++i) {
                const int r = SUB * b + i;
                float kk = 0.f, qq = 0.f, g = 0.f, dd;
                if (r < len) {
                  const size_t t = (size_t)(ce_cur.y + r);
                  kk = bf16_to_f32(p.k[(t * p.H_qk + hq) * HD + c]) * ROW[R_RK + r];
                  qq = bf16_to_f32(p.q[(t * p.H_qk + hq) * HD + c]) * ROW[R_RQ + r];
                  gate_decay(bf16_to_f32(p.g_raw[(t * p.H + h) * HD + c]), a_h, dd, g);
                }
                run += g;
                SK[i * 64 + tid] = kk;
                SQ[i * 64 + tid] = qq;
                SG[i * 64 + tid] = run;
              }
            }
            __syncthreads();
            if (tid < SUB * SUB && ii <= rr) {
#pragma unroll 4
              for (int c = 0; c < 64; ++c) {
                const float dec = exp2f((SG[rr * 64 + c] - SG[ii * 64 + c]) * LOG2E);
                accA += SK[rr * 64 + c] * SK[ii * 64 + c] * dec;
                accM += SQ[rr * 64 + c] * SK[ii * 64 + c] * dec;
              }
            }
          }
          if (tid < SUB * SUB) {
            AM[(SUB * b + rr) * MS + SUB * b + ii] = ii < rr ? accA * ROW[R_BETA + SUB * b + rr] : 0.f;
            FM[rr * SUB + ii] = ii <= rr ? accM : 0.f;
          }
          __syncthreads();
          if (wave == b) {
#pragma unroll
            for (int j = 0; j < 4; ++j) m0[j] = FM[l16 * SUB + 4 * lg + j];
          }
        }
        __syncthreads();
      }

      // hand over M halves computed by waves 1 and 3
      if (wave == 1) MX[lane] = f16x4{(f16)m0[0], (f16)m0[1], (f16)m0[2], (f16)m0[3]};
      if (wave == 3) MX[64 + lane] = f16x4{(f16)m0[0], (f16)m0[1], (f16)m0[2], (f16)m0[3]};
      __syncthreads();  // A complete, M halves visible

      // ---- E1 (waves 0..3): inverse of diagonal block w of I + A ---------------
      // ---- G  (waves 4..7): M, Qhat and Kbar^T fragments -----------------------
      if (wave < 4) {
        if (wave == 0 || wave == 2) {  // complete M fragments (0,0) and (2,1)
          float v[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = m0[j];
            v[4 + j] = 0.f;
          }
          store_frag(rec, REC_M, wave == 0 ? 0 : 5, lane, v);
        }
        if (lane < SUB) {
          const int b = wave, c = lane;
          float x[SUB];
#pragma unroll
          for (int i = 0; i < SUB; ++i) {
            float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) acc -= AM[(SUB * b + i) * MS + SUB * b + j] * x[j];
            x[i] = acc;
          }
#pragma unroll
          for (int i = 0; i < SUB; ++i) TM[(SUB * b + i) * MS + SUB * b + c] = x[i];
        }
      } else {
        {
          float v[8];
          if (wave == 4 || wave == 5) {  // (1,0) or (3,1): own half + handed half
            const f16x4 hx = MX[(wave == 4 ? 0 : 64) + lane];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[j] = m0[j];
              v[4 + j] = (float)hx[j];
            }
            store_frag(rec, REC_M, wave == 4 ? 2 : 7, lane, v);
          } else {  // (2,0) or (3,0): both halves computed here
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[j] = m0[j];
              v[4 + j] = m1[j];
            }
            store_frag(rec, REC_M, wave == 6 ? 4 : 6, lane, v);
          }
        }
#pragma unroll 1
        for (int job2 = wave - 4; job2 < 32; job2 += 4) {
          float v[8];
          if (job2 < 16) {  // Qhat (t, s): lane (row r, key channels perm(s, lg))
            const int t = job2 >> 2, s = job2 & 3;
            const int r = SUB * t + l16, n = t;
            const int c0 = 32 * s + 4 * lg, c1 = c0 + 16;
            ld4(&QR[r * LS + c0], v);
            ld4(&QR[r * LS + c1], v + 4);
            float f[8];
            if (PER_CHANNEL) {
              ld4(&EP[n * HD + c0], f);
              ld4(&EP[n * HD + c1], f + 4);
            } else {
#pragma unroll
              for (int q = 0; q < 8; ++q) f[q] = ROW[R_EG + r];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] *= f[q];
            store_frag(rec, REC_QHAT, job2, lane, v);
          } else {  // Kbar^T (kb, s): lane (key channel k, tokens perm(s, lg))
            const int f = job2 - 16, kb = f >> 1, s = f & 1;
            const int k = SUB * kb + l16;
            const int j0 = 32 * s + 4 * lg, j1 = j0 + 16;
            const float f0 = PER_CHANNEL ? EG[(j0 / SUB) * HD + k] : 0.f;
            const float f1 = PER_CHANNEL ? EG[(j1 / SUB) * HD + k] : 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              v[q] = YSrc[(j0 + q) * LS + k] * (PER_CHANNEL ? f0 : ROW[R_EGL + j0 + q]);
              v[4 + q] = YSrc[(j1 + q) * LS + k] * (PER_CHANNEL ? f1 : ROW[R_EGL + j1 + q]);
            }
            store_frag(rec, REC_KBAR, f, lane, v);
          }
        }
      }
      __syncthreads();

      // ---- E2: off-diagonal blocks of T, level by level (fp32 matrix cores) --
      //   T_ba = -T_bb * sum_{a<=j<b} A_bj T_ja
#pragma unroll
      for (int lev = 1; lev < NSUB; ++lev) {
        if (wave < NSUB - lev) {
          const int a = wave, b = wave + lev;
          f32x4 X = zero4();
          for (int j = a; j < b; ++j) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const float av = AM[(SUB * b + l16) * MS + SUB * j + 4 * s + lg];
              const float tv = TM[(SUB * j + 4 * s + lg) * MS + SUB * a + l16];
              X = mma_f32(av, tv, X);
            }
          }
          // contraction order permuted so that X's own C layout is the B operand
          f32x4 Y = zero4();
#pragma unroll
          for (int s = 0; s < 4; ++s) Y = mma_f32(TM[(SUB * b + l16) * MS + SUB * b + 4 * lg + s], X[s], Y);
#pragma unroll
          for (int j = 0; j < 4; ++j) TM[(SUB * b + 4 * lg + j) * MS + SUB * a + l16] = -Y[j];
        }
        __syncthreads();
      }

      // ---- F0: Khat^T fragments into LDS (A is dead now) ----------------------
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int f = wave * 2 + q2, kb = f >> 1, s = f & 1;
        const int k = SUB * kb + l16;
        const int j0 = 32 * s + 8 * lg;
        const float fe = PER_CHANNEL ? EP[(j0 / SUB) * HD + k] : 0.f;
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = KR[(j0 + q) * LS + k] * (PER_CHANNEL ? fe : ROW[R_EG + j0 + q]);
        KH[f * 64 + lane] = to_f16x8(v);
      }
      __syncthreads();

      // ---- F: W^T = Khat^T (T diag(b))^T; T diag(b) fragments -----------------
      // wave w: token tile t = w % 4, key slices sp = 2 (w / 4) .. +1
      {
        const int t = wave & 3;
        const int r = SUB * t + l16;
        const int ns = (t >> 1) + 1;  // token slices with nonzero T entries for this tile
        f16x8 tbB[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          float v[8], bb[8];
          ld8(&TM[r * MS + 32 * s + 8 * lg], v);
          ld8(&ROW[R_BETA + 32 * s + 8 * lg], bb);
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = (32 * s + 8 * lg + q <= r) ? v[q] * bb[q] : 0.f;
          tbB[s] = to_f16x8(v);
        }
#pragma unroll
        for (int sq = 0; sq < 2; ++sq) {
          const int sp = 2 * (wave >> 2) + sq;
          float v[8];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int kb = 2 * sp + hh;
            f32x4 acc = zero4();
            acc = mma_f16(KH[(kb * 2) * 64 + lane], tbB[0], acc);
            if (ns > 1) acc = mma_f16(KH[(kb * 2 + 1) * 64 + lane], tbB[1], acc);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[hh * 4 + j] = -acc[j];
          }
          store_frag(rec, REC_WNEG, t * 4 + sp, lane, v);
        }
        const int s = wave >> 2;  // T diag(b) fragment (t, s), if nonzero
        if (s < ns) {
          const int j0 = 32 * s + 4 * lg, j1 = j0 + 16;
          float v[8], bb[8];
          ld4(&TM[r * MS + j0], v);
          ld4(&TM[r * MS + j1], v + 4);
          ld4(&ROW[R_BETA + j0], bb);
          ld4(&ROW[R_BETA + j1], bb + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[q] = (j0 + q <= r) ? v[q] * bb[q] : 0.f;
            v[4 + q] = (j1 + q <= r) ? v[4 + q] * bb[4 + q] : 0.f;
          }
          store_frag(rec, REC_TB, t * 2 + s, lane, v);
        }
      }
      __syncthreads();  // LDS is reused by the next job
    }
    job = nj;
    if (job >= n_jobs) break;
  }
}

void launch_chunk_local(const ChunkParams& p, int n_entries, bool per_channel, hipStream_t stream) {
  const int n_jobs = n_entries * p.H;
  if (n_jobs <= 0) return;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const int grid = n_jobs < cus ? n_jobs : cus;  // one resident workgroup per CU (LDS-bound)
  static bool attr_set[2] = {false, false};
  if (per_channel) {
    if (!attr_set[1]) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_local_kernel<true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
      attr_set[1] = true;
    }
    chunk_local_kernel<true><<<grid, NT, LDS_BYTES, stream>>>(p, n_jobs);
  } else {
    if (!attr_set[0]) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_local_kernel<false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
      attr_set[0] = true;
    }
    chunk_local_kernel<false><<<grid, NT, LDS_BYTES, stream>>>(p, n_jobs);
  }
}

}  // namespace kda
