// kda_chunk.hip -- chunk-local kernel: everything about one (64-token chunk,
// value head) that does not depend on the state entering the chunk.
//
// For a chunk of L <= 64 tokens with normalised keys/queries kn, qn, gates g
// (<= 0) and betas b, write Gamma_r = sum_{j<=r} g_j (per key channel).  The
// state entering the chunk is S0; the chunk's effect is (derivation in the
// project's design notes; it is the standard WY/UT form of the delta rule
// with a decay):
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
// sub-chunks; D_n = prod of the per-token decays over sub-chunk n.
//   rho_r = prod_{16n <= j <= r} d_j  (<= 1),  kappa_i = prod_{i < j < 16n+16} d_j (<= 1)
// For r in sub-chunk b and i in sub-chunk a < b:
//   exp(Gamma_r - Gamma_i) = rho_r * (prod_{a<m<b} D_m) * kappa_i, every factor <= 1,
// so those blocks use fp16 operands without overflow.  Diagonal blocks use
//   exp(Gamma_r - Gamma_i) = (rho_r / D_b) * kappa_i
// whose first factor can reach 1/D_b; they run with split-bf16 operands
// (three bf16 products, ~16 significant bits) while D_b >= 2^-100, and fall
// back to an exact elementwise evaluation otherwise.
// In scalar-gate mode exp(Gamma_r - Gamma_i) is one number per (r, i) and is
// applied after the Gram products.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

constexpr int LS = 132;  // row stride (floats) of the [64][128] operand arrays
constexpr int MS = 68;   // row stride (floats) of the [64][64] matrices
constexpr float LOG2E = 1.4426950408889634f;

// Product of D_m[c] over a < m < b.
__device__ __forceinline__ float dprod(const float* DS, int a, int b, int c) {
  float p = 1.f;
  for (int m = a + 1; m < b; ++m) p *= DS[m * HD + c];
  return p;
}

__device__ __forceinline__ void store_frag(uint8_t* rec, int off, int frag, int lane, const float* v) {
  f16x8 h = to_f16x8(v);
  *reinterpret_cast<f16x8*>(rec + off + frag * FRAG_BYTES + lane * 16) = h;
}

}  // namespace

template <bool PER_CHANNEL>
__global__ __launch_bounds__(256) void chunk_local_kernel(ChunkParams p) {
  __shared__ __attribute__((aligned(16))) float KR[CH * LS];  // kn*rho (kn in scalar mode)
  __shared__ __attribute__((aligned(16))) float QR[CH * LS];  // qn*rho (qn)
  __shared__ __attribute__((aligned(16))) float YS[CH * LS];  // kn*kappa (unused in scalar mode)
  __shared__ __attribute__((aligned(16))) float AM[CH * MS];  // A, strictly lower
  __shared__ __attribute__((aligned(16))) float TM[CH * MS];  // T = (I + A)^-1
  __shared__ __attribute__((aligned(16))) f16x8 KH[16 * 64]; // Khat^T fragments [kb][s][lane]
  __shared__ float DS[NSUB * HD];                             // D_n[c]
  __shared__ float rowf[4][CH];  // beta_r, exp(Gamma_r), exp(Gamma_L - Gamma_r), Gamma_r (scalar mode)
  __shared__ float nrm[2][CH];   // 1/|k_r|, 1/|q_r|
  __shared__ int unsafe[NSUB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int e = blockIdx.x, h = blockIdx.y;
  const int4 ce = p.chunks[e];
  const int len = ce.z;
  if (len <= 0) return;  // unused schedule entry (uniform over the workgroup)
  const int tok0 = ce.y;
  const int hq = h / (p.H / p.H_qk);
  uint8_t* rec = p.rec + ((size_t)e * p.H + h) * REC_BYTES;

  if (tid < NSUB) unsafe[tid] = 0;

  // ---- A: load q, k rows; L2-normalise; beta --------------------------------
  {
    const int r = tid >> 2, c0 = (tid & 3) * 32;
    float qv[32], kv[32];
    if (r < len) {
      const size_t base = ((size_t)(tok0 + r) * p.H_qk + hq) * HD + c0;
      const uint4* qp = reinterpret_cast<const uint4*>(p.q + base);
      const uint4* kp = reinterpret_cast<const uint4*>(p.k + base);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        unpack_bf16x8(qp[i], qv + 8 * i);
        unpack_bf16x8(kp[i], kv + 8 * i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) qv[i] = kv[i] = 0.f;
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      sq += qv[i] * qv[i];
      sk += kv[i] * kv[i];
    }
    sq = sum4(sq);
    sk = sum4(sk);
    const float rq = 1.f / sqrtf(sq + 1e-6f), rk = 1.f / sqrtf(sk + 1e-6f);
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      *reinterpret_cast<float4*>(&QR[r * LS + c0 + i]) =
          make_float4(qv[i] * rq, qv[i + 1] * rq, qv[i + 2] * rq, qv[i + 3] * rq);
      *reinterpret_cast<float4*>(&KR[r * LS + c0 + i]) =
          make_float4(kv[i] * rk, kv[i + 1] * rk, kv[i + 2] * rk, kv[i + 3] * rk);
    }
    if ((tid & 3) == 0) {
      rowf[0][r] = r < len ? sigmoidf_(p.beta[(size_t)(tok0 + r) * p.H + h]) : 0.f;
      nrm[0][r] = rk;
      nrm[1][r] = rq;
    }
  }
  __syncthreads();

  // ---- B: gates -> decay factors --------------------------------------------
  const float a_h = __expf(p.A_log[h]);
  if (PER_CHANNEL) {
    const int c = tid & 127, half = tid >> 7;
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const int n = half * 2 + nn;
      float d[SUB];
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const int r = n * SUB + i;
        if (r < len) {
          float g;
          gate_decay(bf16_to_f32(p.g_raw[((size_t)(tok0 + r) * p.H + h) * HD + c]), a_h, d[i], g);
        } else {
          d[i] = 1.f;
        }
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
      if (!(rho >= 0x1p-100f)) atomicOr(&unsafe[n], 1);
    }
  } else {
    if (wave == 0) {
      const int r = lane;
      float d = 1.f, g = 0.f;
      if (r < len) gate_decay(bf16_to_f32(p.g_raw[(size_t)(tok0 + r) * p.H + h]), a_h, d, g);
      // inclusive prefix sum of g over the 64 tokens
      float G = g;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(G, off);
        if (lane >= off) G += y;
      }
      const float GL = __shfl(G, 63);
      rowf[1][r] = exp2f(G * LOG2E);
      rowf[2][r] = exp2f((GL - G) * LOG2E);
      rowf[3][r] = G;
    }
  }
  __syncthreads();

  const float* YSrc = PER_CHANNEL ? YS : KR;

  // ---- D: A and M blocks on the matrix cores -------------------------------
  // Wave b owns row block b: A[b][a] (a <= b) and the M fragments of token tile b.
  float mfr[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) mfr[s][j] = 0.f;
  {
    const int b = wave;
    const int r = SUB * b + l16;
    for (int a = 0; a <= b; ++a) {
      const int i = SUB * a + l16;
      const bool diag = (a == b);
      f32x4 accA = zero4(), accM = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c0 = 32 * s + 8 * lg;
        float xk[8], xq[8], y[8];
        *reinterpret_cast<float4*>(xk) = *reinterpret_cast<const float4*>(&KR[r * LS + c0]);
        *reinterpret_cast<float4*>(xk + 4) = *reinterpret_cast<const float4*>(&KR[r * LS + c0 + 4]);
        *reinterpret_cast<float4*>(xq) = *reinterpret_cast<const float4*>(&QR[r * LS + c0]);
        *reinterpret_cast<float4*>(xq + 4) = *reinterpret_cast<const float4*>(&QR[r * LS + c0 + 4]);
        *reinterpret_cast<float4*>(y) = *reinterpret_cast<const float4*>(&YSrc[i * LS + c0]);
        *reinterpret_cast<float4*>(y + 4) = *reinterpret_cast<const float4*>(&YSrc[i * LS + c0 + 4]);
        if (PER_CHANNEL) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float lam = diag ? 1.f / DS[b * HD + c0 + q] : dprod(DS, a, b, c0 + q);
            xk[q] *= lam;
            xq[q] *= lam;
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
          if (!PER_CHANNEL) v *= exp2f((rowf[3][rr] - rowf[3][ii]) * LOG2E);
          v *= rowf[0][rr];
        }
        AM[rr * MS + ii] = v;
      }
      // M^T block: lane holds M[16b + l16][16a + 4lg + j]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = SUB * b + l16, ii = SUB * a + 4 * lg + j;
        float v = 0.f;
        if (ii <= rr) {
          v = accM[j];
          if (!PER_CHANNEL) v *= exp2f((rowf[3][rr] - rowf[3][ii]) * LOG2E);
        }
        mfr[a >> 1][(a & 1) * 4 + j] = v;
      }
    }
  }
  __syncthreads();  // AM complete; unsafe[] visible

  // ---- D': exact fallback for diagonal blocks with a very large decay span ---
  if (PER_CHANNEL && unsafe[wave]) {
    const int b = wave;
    float kk[SUB][2], qq[SUB][2], dd[SUB][2];
    for (int i = 0; i < SUB; ++i) {
      const int r = SUB * b + i;
      for (int u = 0; u < 2; ++u) {
        const int c = lane + 64 * u;
        if (r < len) {
          const size_t t = (size_t)(tok0 + r);
          kk[i][u] = bf16_to_f32(p.k[(t * p.H_qk + hq) * HD + c]) * nrm[0][r];
          qq[i][u] = bf16_to_f32(p.q[(t * p.H_qk + hq) * HD + c]) * nrm[1][r];
          float g;
          gate_decay(bf16_to_f32(p.g_raw[(t * p.H + h) * HD + c]), a_h, dd[i][u], g);
        } else {
          kk[i][u] = qq[i][u] = 0.f;
          dd[i][u] = 1.f;
        }
      }
    }
    for (int ii = 0; ii < SUB; ++ii) {
      float pr0 = 1.f, pr1 = 1.f;
      for (int rr = ii; rr < SUB; ++rr) {
        if (rr > ii) {
          pr0 *= dd[rr][0];
          pr1 *= dd[rr][1];
        }
        const float sK = sum64(kk[rr][0] * kk[ii][0] * pr0 + kk[rr][1] * kk[ii][1] * pr1);
        const float sQ = sum64(qq[rr][0] * kk[ii][0] * pr0 + qq[rr][1] * kk[ii][1] * pr1);
        if (rr > ii && lane == 0) AM[(SUB * b + rr) * MS + SUB * b + ii] = sK * rowf[0][SUB * b + rr];
        if (l16 == rr && lg == (ii >> 2)) mfr[b >> 1][(b & 1) * 4 + (ii & 3)] = sQ;
      }
    }
  }
  // M fragments of token tile `wave`
  for (int s = 0; s <= (wave >> 1); ++s) store_frag(rec, REC_M, wave * 2 + s, lane, mfr[s]);
  __syncthreads();

  // ---- E1 (wave 0): inverse of the diagonal 16x16 blocks of I + A ----------
  //      G (waves 1..3): Qhat, Kbar fragments, Khat^T fragments, exp(Gamma_L)
  if (wave == 0) {
    const int b = lane >> 4, c = l16;
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
  } else {
    // 48 fragment jobs + gl, spread over waves 1..3
    for (int job = wave - 1; job < 48; job += 3) {
      float v[8];
      if (job < 16) {  // Qhat fragment (t, s)
        const int t = job >> 2, s = job & 3;
        const int r = SUB * t + l16;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int c = 32 * s + (q < 4 ? 4 * lg + q : 16 + 4 * lg + q - 4);
          float f = PER_CHANNEL ? dprod(DS, -1, r / SUB, c) : rowf[1][r];
          v[q] = QR[r * LS + c] * f;
        }
        store_frag(rec, REC_QHAT, job, lane, v);
      } else if (job < 32) {  // Kbar^T fragment (kb, s)
        const int f = job - 16, kb = f >> 1, s = f & 1;
        const int kc = SUB * kb + l16;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = 32 * s + (q < 4 ? 4 * lg + q : 16 + 4 * lg + q - 4);
          const float fac = PER_CHANNEL ? dprod(DS, j / SUB, NSUB, kc) : rowf[2][j];
          v[q] = YSrc[j * LS + kc] * fac;
        }
        store_frag(rec, REC_KBAR, f, lane, v);
      } else {  // Khat^T fragment (kb, s) into LDS, standard contraction order
        const int f = job - 32, kb = f >> 1, s = f & 1;
        const int kc = SUB * kb + l16;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = 32 * s + 8 * lg + q;
          const float fac = PER_CHANNEL ? dprod(DS, -1, j / SUB, kc) : rowf[1][j];
          v[q] = KR[j * LS + kc] * fac;
        }
        KH[f * 64 + lane] = to_f16x8(v);
      }
    }
    if (tid >= 64 && tid < 64 + HD) {
      const int c = tid - 64;
      const float gl = PER_CHANNEL ? dprod(DS, -1, NSUB, c) : rowf[1][CH - 1];
      *reinterpret_cast<float*>(rec + REC_GL + 4 * c) = gl;
    }
  }
  __syncthreads();

  // ---- E2: off-diagonal blocks of T, level by level (fp32 matrix cores) ----
  //   T_ba = -T_bb * sum_{a<=j<b} A_bj T_ja
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
      for (int s = 0; s < 4; ++s) {
        const float tv = TM[(SUB * b + l16) * MS + SUB * b + 4 * lg + s];
        Y = mma_f32(tv, X[s], Y);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) TM[(SUB * b + 4 * lg + j) * MS + SUB * a + l16] = -Y[j];
    }
    __syncthreads();
  }

  // ---- F: W^T = Khat^T (T diag(b))^T per token tile; T diag(b) fragments ----
  {
    const int t = wave;
    const int r = SUB * t + l16;
    f16x8 tbB[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = 32 * s + 8 * lg + q;
        v[q] = (j <= r) ? TM[r * MS + j] * rowf[0][j] : 0.f;
      }
      tbB[s] = to_f16x8(v);
    }
    const int ns = (t >> 1) + 1;  // token slices with nonzero T entries for this tile
    for (int sp = 0; sp < 4; ++sp) {
      float v[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kb = 2 * sp + half;
        f32x4 acc = zero4();
        for (int s = 0; s < ns; ++s) acc = mma_f16(KH[(kb * 2 + s) * 64 + lane], tbB[s], acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[half * 4 + j] = -acc[j];
      }
      store_frag(rec, REC_WNEG, t * 4 + sp, lane, v);
    }
    for (int s = 0; s < ns; ++s) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = 32 * s + (q < 4 ? 4 * lg + q : 16 + 4 * lg + q - 4);
        v[q] = (j <= r) ? TM[r * MS + j] * rowf[0][j] : 0.f;
      }
      store_frag(rec, REC_TB, t * 2 + s, lane, v);
    }
  }
}

void launch_chunk_local(const ChunkParams& p, int n_entries, bool per_channel, hipStream_t stream) {
  dim3 grid(n_entries, p.H);
  if (per_channel) chunk_local_kernel<true><<<grid, 256, 0, stream>>>(p);
  else chunk_local_kernel<false><<<grid, 256, 0, stream>>>(p);
}

}  // namespace kda
