// kda_chunk_job.h -- one chunk-local job: everything about one (64-token
// chunk, value head) that does not depend on the state entering the chunk.
// Shared by the chunk-local kernel (kda_chunk.hip) and the fused persistent
// kernel (kda_fused.hip).
//
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
//   exp(Gamma_r - Gamma_i) = (kn_r / kappa_r) . (kn_i kappa_i)
// whose first factor can reach 1/D_b.
// The per-token log2-decays are scanned along the sub-chunk (prefix and
// suffix sums) and every factor is one exp2 of a scan value.  Diagonal blocks
// run on bf16 matrix cores with every operand split into hi + lo parts (about
// 16 significant bits, and bf16 keeps the range of 1/D_b) while
// D_b >= 2^-100 and fall back to an exact per-channel evaluation in the log
// domain otherwise.
// In scalar-gate mode exp(Gamma_r - Gamma_i) is one number per (r, i) and is
// applied after the Gram products.  With value heads grouped on q/k heads a
// separate kernel (chunk_group_kernel below) forms the head-independent part
// once per q/k head and writes records that keep the group's qn and kn^T once.
//
// Work layout: 4 waves, wave n owns sub-chunk n.  Lane (l16, g) of wave n
// holds token 16n + l16 and the 32 key channels 32s + 8g + e (e < 8,
// s = 0..3): one 16-byte load per slice and tensor, and the natural key
// order of a 16x16x32 matrix-core operand, so the Gram products and the
// decay scans (DPP shifts along the 16 token lanes of a row) run on registers
// loaded straight from memory.  Products with 0/1 selection matrices give the
// transposed (key-major) operands Khat^T and Kbar^T and put Qhat into the
// record's key order (32s + 4g + e, then 32s + 16 + 4g + e).  Only the fp16 Y operands, the sub-chunk decay
// products and the 64 x 64 matrices A and T go through LDS (~65 KB), so two
// workgroups share a CU and hide each other's latencies (one waits on its
// loads while the other computes).  One workgroup per (chunk, head); the
// schedule entry comes from the schedule table for packed sequences and by
// arithmetic for B rows of T tokens.
//
// Decay-only linear attention (DELTA = false) writes the same records with
// the UT transform reduced to the identity: no q/k normalisation, b = 1,
// A = 0 (T = I) and W = 0.
#pragma once

#include <type_traits>

#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

constexpr int NT = 256;  // threads per workgroup (4 waves)
constexpr int MS = 68;   // row stride (floats) of the 64 x 64 matrices
constexpr float LOG2E = 1.4426950408889634f;
constexpr float TINY_D = 7.888609052210118e-31f;  // 2^-100: the smallest sub-chunk decay the fast diagonal path takes

// LDS layout (bytes)
constexpr int L_YB = 0;                          // Y = kn*kappa (fp16) of sub-chunks 0..2 [3][4 slices][64] f16x8
constexpr int L_KH = L_YB + 3 * 4 * 64 * 16;     // Khat^T fragments [8 key tiles][2 token slices][64] f16x8
constexpr int L_AM = L_KH + 16 * 64 * 16;        // A [64][MS] fp32 (upper blocks: exact diagonal M scratch)
constexpr int L_TM = L_AM + CH * MS * 4;         // T [64][MS] fp32 (upper blocks: exact diagonal A scratch)
constexpr int L_DS = L_TM + CH * MS * 4;         // D_n[key] [4][128]
constexpr int L_ROW = L_DS + NSUB * HD * 4;      // per-token values, see R_*
constexpr int L_FLAG = L_ROW + (5 * CH + 8) * 4;  // exact-fallback flags of the 4 sub-chunks
constexpr int LDS_BYTES = L_FLAG + 8 * 4;
static_assert(3 * 16 * 64 * 4 <= 16 * 64 * 16, "fallback scratch must fit in the Khat^T region");
static_assert(2 * LDS_BYTES <= 160 * 1024, "two workgroups per CU");

// Decay-only linear attention with one decay per token-head touches only YB
// and ROW (no A, no inverse, no K-hat, no per-channel decay products, no
// exact fallback), so it gets a compact layout and more jobs per CU.
template <bool PER_CHANNEL, bool DELTA>
struct Lds {
  static constexpr bool COMPACT = !PER_CHANNEL && !DELTA;
  static constexpr int YB = L_YB;
  static constexpr int ROW = COMPACT ? L_KH : L_ROW;
  static constexpr int FLAG = COMPACT ? ROW + (5 * CH + 8) * 4 : L_FLAG;
  static constexpr int BYTES = COMPACT ? FLAG + 8 * 4 : LDS_BYTES;
  static constexpr int JOBS_PER_CU = COMPACT ? 3 : 2;  // by registers (and LDS in the full layout)
};

// ROW sub-arrays (floats)
constexpr int R_BETA = 0, R_RK = CH, R_RQ = 2 * CH, R_GP = 3 * CH, R_GS = 5 * CH;

// Upper (never used) 16x16 blocks of A and T that hold the exact diagonal
// blocks of sub-chunk b when the fallback runs.
__device__ __forceinline__ int upper_block(int b) { return b < 3 ? b + 1 : 6; }  // (0,1) (0,2) (0,3) (1,2)
__device__ __forceinline__ int upper_off(int b) {
  const int rb = b < 3 ? 0 : 1, cb = b < 3 ? b + 1 : 2;
  return (SUB * rb) * MS + SUB * cb;
}

// Sums along the 16 token lanes of a DPP row.  Lanes whose source lies
// outside the row read 0 (bound_ctrl), so each step is one v_add_f32_dpp.
template <int CTRL>
__device__ __forceinline__ float dpp0(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// inclusive prefix sum over the lanes up to this one
__device__ __forceinline__ float row_prefix_sum(float x) {
  x += dpp0<0x111>(x);  // row_shr:1
  x += dpp0<0x112>(x);
  x += dpp0<0x114>(x);
  x += dpp0<0x118>(x);
  return x;
}
// Sum over the lanes after this one (0 for the last lane of the row), from
// the inclusive prefix sum: the row total (lane 15's prefix, broadcast with
// row_newbcast:15) minus this lane's prefix, one v_sub_f32_dpp.
__device__ __forceinline__ float row_suffix_from_prefix(float prefix) {
  const float total =
      __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, prefix), 0x15F, 0xF, 0xF, false));
  return total - prefix;
}

__device__ __forceinline__ void unpack4(uint2 w, float* out) {
  out[0] = __uint_as_float(w.x << 16);
  out[1] = __uint_as_float(w.x & 0xFFFF0000u);
  out[2] = __uint_as_float(w.y << 16);
  out[3] = __uint_as_float(w.y & 0xFFFF0000u);
}

// X Y for 16 x 16 fp32 blocks in matrix-core C layout (lane (l16, lg) holds
// rows 4 lg .. 4 lg + 3 of column l16), given X^T and Y in C layout: product
// jj contracts over index 4 lg + jj, so both operands are read in place.
__device__ __forceinline__ f32x4 mul_cc(const f32x4& XT, const f32x4& Y) {
  f32x4 z = mma_f32(XT[0], Y[0], zero4());
  z = mma_f32(XT[1], Y[1], z);
  z = mma_f32(XT[2], Y[2], z);
  return mma_f32(XT[3], Y[3], z);
}

// (I + N)^-1 for a strictly lower triangular 16 x 16 block N: blocked
// forward substitution with block sizes doubling 1 -> 2 -> 4 -> 8 -> 16.
// With D_k the block-diagonal part of the inverse made of its k x k diagonal
// blocks (D_1 = I) and M_k the part of N inside the 2k x 2k diagonal blocks
// but outside the k x k ones, every 2k x 2k diagonal block of the inverse is
// [[T11, 0], [-T22 N21 T11, T22]], that is D_2k = D_k - D_k M_k D_k.  Every
// intermediate is a block of the inverse or of N (no powers of N, which
// reach ~3e3 for nearly parallel keys and would cancel in fp32), so the
// rounding is that of forward substitution.  Eight block products on fp32
// matrix cores, all in registers; D and D^T are both carried in C layout so
// every product reads its operands in place.
// Nc, NT: N and N^T in C layout; result in C layout.
__device__ __forceinline__ f32x4 unit_lower_inverse(const f32x4& Nc, const f32x4& NT, int l16, int lg) {
  f32x4 D, DT;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // D_2 = I - M_1
    const int r = 4 * lg + j, c = l16;
    const float eye = r == c ? 1.f : 0.f;
    const bool in1 = (r >> 1) == (c >> 1) && r != c;
    D[j] = eye - (in1 ? Nc[j] : 0.f);
    DT[j] = eye - (in1 ? NT[j] : 0.f);
  }
#pragma unroll
  for (int k = 2; k < SUB; k *= 2) {
    f32x4 MT;  // M_k^T (the mask is symmetric in row and column)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * lg + j, c = l16;
      MT[j] = ((r / (2 * k)) == (c / (2 * k)) && (r / k) != (c / k)) ? NT[j] : 0.f;
    }
    const f32x4 P = mul_cc(MT, D);   // M_k D_k
    const f32x4 Q = mul_cc(DT, P);   // D_k M_k D_k
    if (2 * k < SUB) DT = DT - mul_cc(P, DT);  // (D_k M_k D_k)^T = P^T D_k^T
    D = D - Q;
  }
  return D;
}

// Store an A-operand fragment held in natural key order (this lane: keys
// 32s + 8 lg + e of token l16) in the record's order (keys 32s + 4 lg + e,
// then 32s + 16 + 4 lg + e): sel[h] x' picks keys 32s + 16h + 4 lg + j of
// token l16 into the C layout, exactly (0/1 products, fp32 accumulation).
// Record stores.  In the two-kernel path a record is read back by the
// recurrence only after the whole chunk-local grid has written its records
// (hundreds of MB), so they are written non-temporally (NT) and do not evict
// lines from L2 (measured on the dense workload: recurrence 0.297 -> 0.286 ms,
// chunk-local unchanged).  The fused kernel's records are read from L2 by
// another workgroup right away, so they use ordinary stores.
template <bool NT, typename V>
__device__ __forceinline__ void st_rec(uint8_t* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  else *reinterpret_cast<V*>(p) = v;
}

template <bool NT>
__device__ __forceinline__ void store_reordered(uint8_t* frag, f16x8 x, const f16x8* sel, int lane) {
  const f32x4 lo = mma_f16(sel[0], x, zero4()), hi = mma_f16(sel[1], x, zero4());
  const f16x8 o = {(f16)lo[0], (f16)lo[1], (f16)lo[2], (f16)lo[3], (f16)hi[0], (f16)hi[1], (f16)hi[2], (f16)hi[3]};
  st_rec<NT>(frag + lane * 16, o);
}

template <bool NT>
__device__ __forceinline__ void store_frag(uint8_t* rec, int off, int frag, int lane, const float* v) {
  st_rec<NT>(rec + off + frag * FRAG_BYTES + lane * 16, to_f16x8(v));
}

// One job's inputs for this lane: token 16*wave + lane%16, key channels of
// slice s: 32s + 8g .. +3 (half 0) and 32s + 8g + 4 .. +7 (half 1).
struct Pref {
  uint2 q[8], k[8], g[8];  // [2s + half], bf16; g only in per-channel mode
  uint32_t gs;             // scalar gate of the token, bf16 in the low half
  float beta;              // logit of the token
};

template <bool PER_CHANNEL, bool DELTA>
__device__ __forceinline__ void load_rows(Pref& P, const ChunkParams& p, int4 ce, int h, int wave, int lane) {
  // Loads are unconditional (rows past the chunk end are clamped to its last
  // row and zeroed when used) so they issue back to back without waits.
  const int len = ce.z, tok0 = ce.y;
  if (len <= 0) return;
  const int hq = h / (p.H / p.H_qk);
  const int r = min(SUB * wave + (lane & 15), len - 1), g8 = 8 * (lane >> 4);
  const size_t t = (size_t)(tok0 + r);
  const uint16_t* qp = p.q + (t * p.H_qk + hq) * HD + g8;
  const uint16_t* kp = p.k + (t * p.H_qk + hq) * HD + g8;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint4 a = *reinterpret_cast<const uint4*>(qp + 32 * s);
    const uint4 b = *reinterpret_cast<const uint4*>(kp + 32 * s);
    P.q[2 * s] = make_uint2(a.x, a.y);
    P.q[2 * s + 1] = make_uint2(a.z, a.w);
    P.k[2 * s] = make_uint2(b.x, b.y);
    P.k[2 * s + 1] = make_uint2(b.z, b.w);
  }
  P.beta = DELTA ? p.beta[t * p.H + h] : 0.f;  // no write strength without the delta rule
  if (PER_CHANNEL) {
    const uint16_t* gp = p.g_raw + (t * p.H + h) * HD + g8;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 c = *reinterpret_cast<const uint4*>(gp + 32 * s);
      P.g[2 * s] = make_uint2(c.x, c.y);
      P.g[2 * s + 1] = make_uint2(c.z, c.w);
    }
  } else {
    P.gs = p.g_raw[t * p.H + h];
  }
}


// DELTA = false: decay-only linear attention.  The same chunk records with
// the UT transform reduced to the identity: no q/k normalisation, write
// strength 1, A = 0 (so T = I) and W = 0 (K-hat is not formed), which makes
// the recurrence's U equal to V.
//
// PRECISE = true also stores the low parts of the fp16 Kbar^T and T diag(b)
// fragments (x - fp16(x), fp16), which the fused kernel's state path adds
// back: with nearly parallel keys, strong writes and little decay, the
// rows of U telescope inside a chunk, and a single fp16 rounding of Kbar or
// T diag(b) is amplified into the state.
template <bool PER_CHANNEL, bool DELTA, bool PRECISE>
__device__ __forceinline__ void chunk_job(const ChunkParams& p, uint8_t* smem, const int4 ce_cur, const int h,
                                          uint8_t* rec) {
  using LD = Lds<PER_CHANNEL, DELTA>;
  f16x8* YB = reinterpret_cast<f16x8*>(smem + LD::YB);
  uint8_t* KHb = smem + L_KH;
  const f16x8* KH = reinterpret_cast<const f16x8*>(smem + L_KH);
  float* AM = reinterpret_cast<float*>(smem + L_AM);
  float* TM = reinterpret_cast<float*>(smem + L_TM);
  float* DS = reinterpret_cast<float*>(smem + L_DS);
  float* ROW = reinterpret_cast<float*>(smem + LD::ROW);
  int* FLAG = reinterpret_cast<int*>(smem + LD::FLAG);

  // In the fused kernel's persistent loop (PRECISE) the thread index goes
  // through an empty asm statement, so that nothing derived from it is
  // hoisted out of the loop and kept live across jobs (which would push the
  // job past 256 registers).  The one-shot kernel keeps the plain index (the
  // barrier costs it 12 registers and 4% of its time).
  int tid_opaque = threadIdx.x;
  if (PRECISE) asm volatile("" : "+v"(tid_opaque));
  const int tid = tid_opaque, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int n = wave;              // sub-chunk of this wave
  const int r = SUB * n + l16;     // this lane's token row in the chunk

  // 0/1 selection operands: sel[h] picks key 32s + 16h + l16 out of slice s
  // (this lane's element e of a slice is key 32s + 8 lg + e)
  f16x8 sel[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[hh][e] = (8 * lg + e == 16 * hh + l16) ? (f16)1.f : (f16)0.f;

  // A_log is read through the constant address space (a scalar load).
  typedef __attribute__((address_space(4))) const float cfloat;
  cfloat* A_log = (cfloat*)p.A_log;
  {
    const int len = ce_cur.z;
    if (len > 0) {  // uniform over the workgroup
      // PRECISE (fused kernel): the chunk's value rows are copied into the
      // record; issued first, so waiting for them does not wait for q, k, g
      u32x4 vr0, vr1, vr2, vr3;  // four named vectors (an array of them ended up on the stack)
      if (PRECISE) {
        const int rr = min(SUB * wave + (lane & 15), len - 1);
        const u32x4* vsrc = reinterpret_cast<const u32x4*>(p.v + ((size_t)(ce_cur.y + rr) * p.H + h) * HD +
                                                           8 * (lane >> 4));
        vr0 = vsrc[0];
        vr1 = vsrc[4];
        vr2 = vsrc[8];
        vr3 = vsrc[12];
      }
      Pref cur;
      load_rows<PER_CHANNEL, DELTA>(cur, p, ce_cur, h, wave, lane);
      // keep every input load ahead of the first use, so the three streams
      // (q, k, g) are in flight together rather than g after q and k arrive
      __builtin_amdgcn_sched_barrier(0);
      if (PRECISE) {
        u32x4* vdst = reinterpret_cast<u32x4*>(rec + REC_V + (SUB * wave + (lane & 15)) * (HD * 2) +
                                               16 * (lane >> 4));
        vdst[0] = vr0;
        vdst[4] = vr1;
        vdst[8] = vr2;
        vdst[12] = vr3;
      }
      const float alog_cur = A_log[h];
      const bool live = r < len;
      const float a_h = __expf(alog_cur);

      // ---- 1. normalise; gates -> decay scans; diagonal block ---------------
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float x[4], y[4];
        unpack4(cur.q[i], x);
        unpack4(cur.k[i], y);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sq += x[j] * x[j];
          sk += y[j] * y[j];
        }
      }
      sq += __shfl_xor(sq, 16);
      sk += __shfl_xor(sk, 16);
      sq += __shfl_xor(sq, 32);
      sk += __shfl_xor(sk, 32);
      const float rq = live ? (DELTA ? 1.f / sqrtf(sq + 1e-6f) : 1.f) : 0.f;
      const float rk = live ? (DELTA ? 1.f / sqrtf(sk + 1e-6f) : 1.f) : 0.f;
      const float beta = live ? (DELTA ? sigmoidf_(cur.beta) : 1.f) : 0.f;
      if (lg == 0) {
        ROW[R_BETA + r] = beta;
        ROW[R_RK + r] = rk;
        ROW[R_RQ + r] = rq;
      }

      float X[32], Q[32], Y[32];  // kn*rho, qn*rho, kn*kappa (scalar mode: kn, qn, -)
      f32x4 accA_d = zero4(), accM_d = zero4();
      float Gloc = 0.f;           // scalar mode: gate prefix within the sub-chunk
      if (PER_CHANNEL) {
        bool tiny = false;
        f32x4 accA2 = zero4(), accM2 = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float kn[8], qn[8], gx[8];
          unpack4(cur.k[2 * s], kn);
          unpack4(cur.k[2 * s + 1], kn + 4);
          unpack4(cur.q[2 * s], qn);
          unpack4(cur.q[2 * s + 1], qn + 4);
          unpack4(cur.g[2 * s], gx);
          unpack4(cur.g[2 * s + 1], gx + 4);
          float P[8], S[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            kn[q] *= rk;
            qn[q] *= rq;
            const float l2d = gate_log2(gx[q], a_h);  // log2 of the token's decay
            P[q] = live ? l2d : 0.f;
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            P[q] = row_prefix_sum(P[q]);           // log2 rho
            S[q] = row_suffix_from_prefix(P[q]);  // log2 kappa
          }
          float Dv[8], kik[8], qik[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float rho = __builtin_amdgcn_exp2f(P[q]);
            const float kap = __builtin_amdgcn_exp2f(S[q]);
            const float ikap = __builtin_amdgcn_exp2f(-S[q]);
            const int v = 8 * s + q;
            X[v] = kn[q] * rho;
            Q[v] = qn[q] * rho;
            Y[v] = kn[q] * kap;
            Dv[q] = rho * kap;
            tiny |= !(Dv[q] >= TINY_D);
            kik[q] = kn[q] * ikap;
            qik[q] = qn[q] * ikap;
          }
          // diagonal block on bf16 matrix cores with hi + lo splits of every
          // operand (about 16 significant bits; bf16 keeps the range of the
          // row factor 1/kappa, which reaches 2^100)
          {
            bf16x8 yh, yl, qh, ql;
            split_bf16x8(&Y[8 * s], yh, yl);
            split_bf16x8(qik, qh, ql);
            if (DELTA) {
              bf16x8 kh, kl;
              split_bf16x8(kik, kh, kl);
              accA_d = mma_bf16(kh, yh, accA_d);
              accA2 = mma_bf16(kh, yl, accA2);
              accA2 = mma_bf16(kl, yh, accA2);
            }
            accM_d = mma_bf16(yh, qh, accM_d);
            accM2 = mma_bf16(yh, ql, accM2);
            accM2 = mma_bf16(yl, qh, accM2);
          }
          if (l16 == 0) {  // D_n of this lane group's 8 keys
            *reinterpret_cast<float4*>(&DS[n * HD + 32 * s + 8 * lg]) = make_float4(Dv[0], Dv[1], Dv[2], Dv[3]);
            *reinterpret_cast<float4*>(&DS[n * HD + 32 * s + 8 * lg + 4]) = make_float4(Dv[4], Dv[5], Dv[6], Dv[7]);
          }
          if (n < 3) {
            f16x8 yh;
#pragma unroll
            for (int q = 0; q < 8; ++q) yh[q] = (f16)Y[8 * s + q];
            YB[(n * 4 + s) * 64 + lane] = yh;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          accA_d[j] += accA2[j];
          accM_d[j] += accM2[j];
        }
        const bool any_tiny = __ballot(tiny && l16 == 0) != 0;
        if (lane == 0) FLAG[n] = any_tiny ? 1 : 0;
      } else {
        float g = 0.f;
        if (live) {
          float d;
          gate_decay(bf16_to_f32((uint16_t)cur.gs), a_h, d, g);
        }
        Gloc = row_prefix_sum(g);
        if (lg == 0) ROW[R_GP + r] = Gloc;
        if (lane == 15) ROW[R_GS + n] = Gloc;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float kn[8], qn[8];
          unpack4(cur.k[2 * s], kn);
          unpack4(cur.k[2 * s + 1], kn + 4);
          unpack4(cur.q[2 * s], qn);
          unpack4(cur.q[2 * s + 1], qn + 4);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            X[8 * s + q] = kn[q] * rk;
            Q[8 * s + q] = qn[q] * rq;
          }
          if (n < 3) YB[(n * 4 + s) * 64 + lane] = to_f16x8(&X[8 * s]);
        }
      }
      __syncthreads();  // Y operands, D_n, per-token values and flags visible

      // ---- 1'. exact diagonal blocks when a sub-chunk's decay span is huge -----
      // Rare (a channel decays by more than 2^-100 within 16 tokens).  Results
      // go to upper (unused) blocks of T (A values) and A (M values); scratch
      // lives in the Khat^T region, which is written only afterwards.
      const bool flagged = PER_CHANNEL && FLAG[n];
      if (PER_CHANNEL && (FLAG[0] | FLAG[1] | FLAG[2] | FLAG[3])) {
        const int hq = h / (p.H / p.H_qk);
        float* SK = reinterpret_cast<float*>(KHb);  // [16][64]
        float* SQ = SK + 1024;                      // [16][64]
        float* SG = SK + 2048;                      // [16][64]
        const int rr = tid >> 4, ii = tid & 15;
#pragma unroll 1
        for (int b = 0; b < NSUB; ++b) {
          if (!FLAG[b]) continue;
          float accA = 0.f, accM = 0.f;
#pragma unroll 1
          for (int half = 0; half < 2; ++half) {
            __syncthreads();
            if (tid < 64) {
              const int c = half * 64 + tid;
              float run = 0.f;
#pragma unroll 1
              for (int i = 0; i < SUB; ++i) {
                const int rw = SUB * b + i;
                float kk = 0.f, qq = 0.f, g = 0.f, dd;
                if (rw < len) {
                  const size_t t = (size_t)(ce_cur.y + rw);
                  kk = bf16_to_f32(p.k[(t * p.H_qk + hq) * HD + c]) * ROW[R_RK + rw];
                  qq = bf16_to_f32(p.q[(t * p.H_qk + hq) * HD + c]) * ROW[R_RQ + rw];
                  gate_decay(bf16_to_f32(p.g_raw[(t * p.H + h) * HD + c]), a_h, dd, g);
                }
                run += g;
                SK[i * 64 + tid] = kk;
                SQ[i * 64 + tid] = qq;
                SG[i * 64 + tid] = run;
              }
            }
            __syncthreads();
            if (ii <= rr) {
#pragma unroll 4
              for (int c = 0; c < 64; ++c) {
                const float dec = exp2f((SG[rr * 64 + c] - SG[ii * 64 + c]) * LOG2E);
                accA += SK[rr * 64 + c] * SK[ii * 64 + c] * dec;
                accM += SQ[rr * 64 + c] * SK[ii * 64 + c] * dec;
              }
            }
          }
          TM[upper_off(b) + rr * MS + ii] = ii < rr ? accA * ROW[R_BETA + SUB * b + rr] : 0.f;
          AM[upper_off(b) + rr * MS + ii] = ii <= rr ? accM : 0.f;
        }
        __syncthreads();  // scratch free for Khat^T; exact blocks visible
      }

      // ---- 2. off-diagonal blocks; Qhat, Kbar^T (record) and Khat^T (LDS) -----
      f32x4 accA[3], accM[3];
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        accA[a] = zero4();
        accM[a] = zero4();
      }
      float Gr = 0.f, GL = 0.f;  // scalar mode: Gamma of this token, Gamma_L
      if (!PER_CHANNEL) {
        float below = 0.f;
#pragma unroll
        for (int m = 0; m < NSUB; ++m) {
          const float gs = ROW[R_GS + m];
          if (m < n) below += gs;
          GL += gs;
        }
        Gr = Gloc + below;
      }
      const float EGr = PER_CHANNEL ? 0.f : exp2f(Gr * LOG2E);
      const float EGLr = PER_CHANNEL ? 0.f : exp2f((GL - Gr) * LOG2E);
      // The slice loop is instantiated per sub-chunk index N (wave-uniform), so
      // the decay products and the (N, a < N) blocks resolve at compile time.
      auto step2 = [&](auto Nc) {
        constexpr int N = decltype(Nc)::value;
  #pragma unroll
        for (int s = 0; s < 4; ++s) {
          float ep[8], eg[8], lam[8];
          float Dm[4][8];
          if (PER_CHANNEL) {
  #pragma unroll
            for (int m = 0; m < NSUB; ++m) {
              const float4 lo = *reinterpret_cast<const float4*>(&DS[m * HD + 32 * s + 8 * lg]);
              const float4 hi = *reinterpret_cast<const float4*>(&DS[m * HD + 32 * s + 8 * lg + 4]);
              Dm[m][0] = lo.x; Dm[m][1] = lo.y; Dm[m][2] = lo.z; Dm[m][3] = lo.w;
              Dm[m][4] = hi.x; Dm[m][5] = hi.y; Dm[m][6] = hi.z; Dm[m][7] = hi.w;
            }
  #pragma unroll
            for (int q = 0; q < 8; ++q) {
              float a1 = 1.f, a2 = 1.f;
  #pragma unroll
              for (int m = 0; m < NSUB; ++m) {
                if (m < N) a1 *= Dm[m][q];
                if (m > N) a2 *= Dm[m][q];
              }
              ep[q] = a1;
              eg[q] = a2;
              lam[q] = 1.f;
            }
          } else {
  #pragma unroll
            for (int q = 0; q < 8; ++q) {
              ep[q] = EGr;
              eg[q] = EGLr;
              lam[q] = 1.f;
            }
          }
          // Qhat fragment (N, s), put into the record's key order
          {
            float v[8];
  #pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = Q[8 * s + q] * ep[q];
            store_reordered<!PRECISE>(rec + REC_QHAT + (N * 4 + s) * FRAG_BYTES, to_f16x8(v), sel, lane);
          }
          // Khat and Kbar of this sub-chunk, transposed by selection products
          {
            f16x8 kh, kb, kbl;
  #pragma unroll
            for (int q = 0; q < 8; ++q) {
              kh[q] = DELTA ? (f16)(X[8 * s + q] * ep[q]) : (f16)0.f;
              const float kbv = (PER_CHANNEL ? Y[8 * s + q] : X[8 * s + q]) * eg[q];
              kb[q] = (f16)kbv;
              kbl[q] = PRECISE ? (f16)(kbv - (float)kb[q]) : (f16)0.f;
            }
  #pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int kt = 2 * s + hh;  // key tile
              if (DELTA) {  // K-hat^T feeds only W
                const f32x4 th = mma_f16(kh, sel[hh], zero4());
                const f16x4 th4 = {(f16)th[0], (f16)th[1], (f16)th[2], (f16)th[3]};
                *reinterpret_cast<f16x4*>(KHb + ((kt * 2 + (N >> 1)) * 64 + lane) * 16 + (N & 1) * 8) = th4;
              }
              const f32x4 tb = mma_f16(kb, sel[hh], zero4());
              const f16x4 tb4 = {(f16)tb[0], (f16)tb[1], (f16)tb[2], (f16)tb[3]};
              // half-fragment pieces from two waves: an ordinary store, so L2 merges them into whole
              // lines (non-temporal, they reach memory as 571 instead of 508 MB of writes)
              *reinterpret_cast<f16x4*>(rec + REC_KBAR + (kt * 2 + (N >> 1)) * FRAG_BYTES + lane * 16 + (N & 1) * 8) = tb4;
              if (PRECISE) {
                const f32x4 tl = mma_f16(kbl, sel[hh], zero4());
                const f16x4 tl4 = {(f16)tl[0], (f16)tl[1], (f16)tl[2], (f16)tl[3]};
                *reinterpret_cast<f16x4*>(rec + REC_KBAR_LO + (kt * 2 + (N >> 1)) * FRAG_BYTES + lane * 16 +
                                          (N & 1) * 8) = tl4;
              }
            }
          }
          // blocks (N, a), a < N: (X lam) Y_a^T and Y_a (Q lam)^T
  #pragma unroll
          for (int a = 2; a >= 0; --a) {
            if (a < N) {
              if (PER_CHANNEL && a + 1 < N) {
  #pragma unroll
                for (int q = 0; q < 8; ++q) lam[q] *= Dm[a + 1][q];
              }
              f16x8 xl, ql;
  #pragma unroll
              for (int q = 0; q < 8; ++q) {
                xl[q] = (f16)(X[8 * s + q] * lam[q]);
                ql[q] = (f16)(Q[8 * s + q] * lam[q]);
              }
              const f16x8 ya = YB[(a * 4 + s) * 64 + lane];
              if (DELTA) accA[a] = mma_f16(xl, ya, accA[a]);
              accM[a] = mma_f16(ya, ql, accM[a]);
            }
          }
          if (!PER_CHANNEL) {  // scalar mode: the diagonal block is an fp16 Gram block too
            const f16x8 xh = to_f16x8(&X[8 * s]);
            if (DELTA) accA_d = mma_f16(xh, xh, accA_d);
            accM_d = mma_f16(xh, to_f16x8(&Q[8 * s]), accM_d);
          }
        }
      };
      switch (n) {
        case 0: step2(std::integral_constant<int, 0>()); break;
        case 1: step2(std::integral_constant<int, 1>()); break;
        case 2: step2(std::integral_constant<int, 2>()); break;
        default: step2(std::integral_constant<int, 3>()); break;
      }
      if (tid < HD) {  // exp(Gamma_L) per key
        const float gl = PER_CHANNEL ? DS[tid] * DS[HD + tid] * DS[2 * HD + tid] * DS[3 * HD + tid]
                                     : exp2f(GL * LOG2E);
        *reinterpret_cast<float*>(rec + REC_GL + 4 * tid) = gl;
      }

      // Steps 3 to 6 are instantiated per sub-chunk index N like step 2 (the
      // same barriers in every instantiation).
      auto steps3to6 = [&](auto Nc) {
        constexpr int N = decltype(Nc)::value;
        f32x4 Ncl = zero4();  // the diagonal block A_nn in C layout
        // ---- 3. A rows of this sub-chunk -> LDS; M fragments -> record ----------
        {
          // scalar mode: Gamma_x from the per-token prefix within its sub-chunk
          // plus the totals of the sub-chunks before it
          float gbase[NSUB];
          if (!PER_CHANNEL) {
            float acc = 0.f;
  #pragma unroll
            for (int m = 0; m < NSUB; ++m) {
              gbase[m] = acc;
              acc += ROW[R_GS + m];
            }
          }
          auto gam = [&](int x) { return ROW[R_GP + x] + gbase[x >> 4]; };
          float brow[4], grow[4];
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int rr = SUB * N + 4 * lg + j;
            brow[j] = ROW[R_BETA + rr];
            grow[j] = PER_CHANNEL ? 0.f : gam(rr);
          }
          // diagonal block: lane holds A[16n + 4lg + j][16n + l16]
          // (no A without the delta rule: T = I, steps 4 and 5 are skipped)
          if (DELTA) {
          float dv[4];
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int rl = 4 * lg + j, il = l16;
            float v = 0.f;
            if (il < rl) {
              if (flagged) v = TM[upper_off(N) + rl * MS + il];
              else {
                v = accA_d[j] * brow[j];
                if (!PER_CHANNEL) v *= exp2f((grow[j] - gam(SUB * N + il)) * LOG2E);
              }
            }
            dv[j] = v;
            AM[(SUB * N + rl) * MS + SUB * N + il] = v;
          }
          Ncl = f32x4{dv[0], dv[1], dv[2], dv[3]};
  #pragma unroll
          for (int a = 0; a < 3; ++a) {
            if (a < N) {
              const float gi = PER_CHANNEL ? 0.f : gam(SUB * a + l16);
  #pragma unroll
              for (int j = 0; j < 4; ++j) {
                float v = accA[a][j] * brow[j];
                if (!PER_CHANNEL) v *= exp2f((grow[j] - gi) * LOG2E);
                AM[(SUB * N + 4 * lg + j) * MS + SUB * a + l16] = v;
              }
            }
          }
          }
          // M^T blocks: lane holds M[16n + l16][16a + 4lg + j]
          const float gr = PER_CHANNEL ? 0.f : gam(r);
          float md[4], mo[3][4];
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int il = 4 * lg + j;
            float v = 0.f;
            if (il <= l16) {
              if (flagged) v = AM[upper_off(N) + l16 * MS + il];
              else {
                v = accM_d[j];
                if (!PER_CHANNEL) v *= exp2f((gr - gam(SUB * N + il)) * LOG2E);
              }
            }
            md[j] = v;
          }
  #pragma unroll
          for (int a = 0; a < 3; ++a)
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              float v = accM[a][j];
              if (!PER_CHANNEL && a < N) v *= exp2f((gr - gam(SUB * a + 4 * lg + j)) * LOG2E);
              mo[a][j] = v;
            }
          float v[8];
          // fragment (n, 0): blocks (n, 0), (n, 1)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = N == 0 ? md[j] : mo[0][j];
            v[4 + j] = N == 0 ? 0.f : (N == 1 ? md[j] : mo[1][j]);
          }
          store_frag<!PRECISE>(rec, REC_M, N * 2, lane, v);
          if (N >= 2) {  // fragment (n, 1): blocks (n, 2), (n, 3)
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[j] = N == 2 ? md[j] : mo[2][j];
              v[4 + j] = N == 3 ? md[j] : 0.f;
            }
            store_frag<!PRECISE>(rec, REC_M, N * 2 + 1, lane, v);
          }
        }

        // ---- 4. T_nn = (I + A_nn)^-1 on fp32 matrix cores (blocked substitution) -
        // A_nn^T in C layout is one row read of the A rows this wave wrote just
        // above (no barrier needed within a wave).
        f32x4 Tnn = zero4();
        if (DELTA) {
          const float4 nt = *reinterpret_cast<const float4*>(&AM[(SUB * N + l16) * MS + SUB * N + 4 * lg]);
          Tnn = unit_lower_inverse(Ncl, f32x4{nt.x, nt.y, nt.z, nt.w}, l16, lg);
  #pragma unroll
          for (int j = 0; j < 4; ++j) TM[(SUB * N + 4 * lg + j) * MS + SUB * N + l16] = Tnn[j];
          __syncthreads();  // A rows, diagonal T blocks and Khat^T visible
        }

        // ---- 5. off-diagonal blocks of T by block column (fp32 matrix cores) ----
        //   T_ba = -T_bb * sum_{a<=j<b} A_bj T_ja
        // Block column a depends only on A, the diagonal blocks and its own
        // earlier blocks, so wave a computes it alone, holding its blocks in
        // registers in C layout; the contraction index is permuted (4 lg + jj
        // in product jj) so that C layout is the B operand and every A operand
        // is one 16-byte row read.
        if (DELTA) {
          constexpr int a = N;
          if (a < NSUB - 1) {
            f32x4 Tc[NSUB];
            Tc[a] = Tnn;
  #pragma unroll
            for (int b = a + 1; b < NSUB; ++b) {
              f32x4 Xs = zero4();
  #pragma unroll
              for (int j = a; j < b; ++j) {
                const float4 av = *reinterpret_cast<const float4*>(&AM[(SUB * b + l16) * MS + SUB * j + 4 * lg]);
                Xs = mma_f32(av.x, Tc[j][0], Xs);
                Xs = mma_f32(av.y, Tc[j][1], Xs);
                Xs = mma_f32(av.z, Tc[j][2], Xs);
                Xs = mma_f32(av.w, Tc[j][3], Xs);
              }
              const float4 tb = *reinterpret_cast<const float4*>(&TM[(SUB * b + l16) * MS + SUB * b + 4 * lg]);
              f32x4 Ys = mma_f32(tb.x, Xs[0], zero4());
              Ys = mma_f32(tb.y, Xs[1], Ys);
              Ys = mma_f32(tb.z, Xs[2], Ys);
              Ys = mma_f32(tb.w, Xs[3], Ys);
  #pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                Tc[b][jj] = -Ys[jj];
                TM[(SUB * b + 4 * lg + jj) * MS + SUB * a + l16] = -Ys[jj];
              }
            }
          }
          __syncthreads();  // every block of T visible
        }

        // ---- 6. -W^T = -Khat^T (T diag(b))^T and T diag(b) fragments -----------
        {
          const int t = N, rt = SUB * t + l16;
          const int ns = (t >> 1) + 1;  // token slices with nonzero T entries for this tile
          f16x8 tbB[2];
  #pragma unroll
          for (int s = 0; s < 2; ++s) {
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (s < ns) {
              const int j0 = 32 * s + 4 * lg, j1 = j0 + 16;
              float tv[8], bb[8];
              if (DELTA) {
                *reinterpret_cast<float4*>(&tv[0]) = *reinterpret_cast<const float4*>(&TM[rt * MS + j0]);
                *reinterpret_cast<float4*>(&tv[4]) = *reinterpret_cast<const float4*>(&TM[rt * MS + j1]);
              } else {  // T = I
  #pragma unroll
                for (int q = 0; q < 4; ++q) {
                  tv[q] = j0 + q == rt ? 1.f : 0.f;
                  tv[4 + q] = j1 + q == rt ? 1.f : 0.f;
                }
              }
              *reinterpret_cast<float4*>(&bb[0]) = *reinterpret_cast<const float4*>(&ROW[R_BETA + j0]);
              *reinterpret_cast<float4*>(&bb[4]) = *reinterpret_cast<const float4*>(&ROW[R_BETA + j1]);
  #pragma unroll
              for (int q = 0; q < 4; ++q) {
                v[q] = (j0 + q <= rt) ? tv[q] * bb[q] : 0.f;
                v[4 + q] = (j1 + q <= rt) ? tv[4 + q] * bb[4 + q] : 0.f;
              }
              store_frag<!PRECISE>(rec, REC_TB, t * 2 + s, lane, v);
              if (PRECISE) {
                float lo[8];
  #pragma unroll
                for (int q = 0; q < 8; ++q) lo[q] = v[q] - (float)(f16)v[q];
                store_frag<!PRECISE>(rec, REC_TB_LO, t * 2 + s, lane, lo);
              }
            }
            tbB[s] = to_f16x8(v);
          }
  #pragma unroll
          for (int sp = 0; sp < 4; ++sp) {
            float v[8];
  #pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int kt = 2 * sp + hh;
              f32x4 acc = zero4();
              if (DELTA) {  // W = 0 for decay-only attention
                acc = mma_f16(KH[(kt * 2) * 64 + lane], tbB[0], acc);
                if (ns > 1) acc = mma_f16(KH[(kt * 2 + 1) * 64 + lane], tbB[1], acc);
              }
  #pragma unroll
              for (int j = 0; j < 4; ++j) v[hh * 4 + j] = -acc[j];
            }
            store_frag<!PRECISE>(rec, REC_WNEG, t * 4 + sp, lane, v);
          }
        }
      };
      switch (n) {
        case 0: steps3to6(std::integral_constant<int, 0>()); break;
        case 1: steps3to6(std::integral_constant<int, 1>()); break;
        case 2: steps3to6(std::integral_constant<int, 2>()); break;
        default: steps3to6(std::integral_constant<int, 3>()); break;
      }
    }
  }
}


}  // namespace

}  // namespace kda
