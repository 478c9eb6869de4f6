// kda_chunk.hip -- the chunk-local kernels: one workgroup per (chunk, value
// head) job (chunk_local_kernel, the job itself in kda_chunk_job.h) or per
// (chunk, q/k head) for grouped value heads with a scalar gate
// (chunk_group_kernel).
#include "kda_chunk_job.h"

namespace kda {

template <bool PER_CHANNEL, bool DELTA>
__global__ __launch_bounds__(NT, (Lds<PER_CHANNEL, DELTA>::JOBS_PER_CU)) void chunk_local_kernel(const ChunkParams p,
                                                                                                 const int n_jobs) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // Job indices are wave-uniform; the schedule is read through the constant
  // address space so these loads go to the scalar unit.
  typedef __attribute__((address_space(4))) const int cint;
  cint* chunks = (cint*)p.chunks;
  const int job = blockIdx.x;
  const int e = __builtin_amdgcn_readfirstlane(job / p.H), h = __builtin_amdgcn_readfirstlane(job % p.H);
  int4 ce;
  if (p.dense_T > 0) {  // B rows of T tokens: entry e is chunk e % NC of row e / NC
    const int T = p.dense_T, nc = (T + CH - 1) / CH, b = e / nc, c = e - b * nc;
    ce = make_int4(b, b * T + c * CH, min(CH, T - c * CH), c);
  } else {
    ce = make_int4(chunks[4 * e], chunks[4 * e + 1], chunks[4 * e + 2], chunks[4 * e + 3]);
  }
  chunk_job<PER_CHANNEL, DELTA, false>(p, smem, ce, h, p.rec + ((size_t)e * p.H + h) * REC_BYTES);
}

// ---------------------------------------------------------------------------
// Scalar gate with value heads grouped on q/k heads: one workgroup per
// (chunk, q/k head).  With one decay per token-head the normalised rows, the
// Gram products kn kn^T and qn kn^T and the transposes kn^T do not depend on
// the value head, so they are formed once; the workgroup then walks the G
// value heads of the group, each with its own gates and write strengths:
// decays applied to the Gram blocks, A and M, T = (I + A)^-1 and the record
// fragments.  The records have the shared-q/k format: qn, kn^T and (delta
// rule) kn in the group's first record, the per-token factors exp(Gamma_r),
// exp(Gamma_L - Gamma_r), M and T diag(b) in every record, and no W (the
// recurrence forms W S as T diag(b) diag(exp(Gamma)) (kn S)).
// ---------------------------------------------------------------------------
// LDS of the grouped kernel: Y blocks, A, T and the per-token rows; no K-hat^T
// (no W is formed) and no exact-fallback scratch (with one decay per
// token-head every decay factor is applied after the products and is <= 1).
// 48 KB, so three jobs share a CU.
template <bool DELTA>
struct GroupLds {
  static constexpr int YB = L_YB;
  static constexpr int AM = L_YB + 3 * 4 * 64 * 16;
  static constexpr int TM = AM + (DELTA ? CH * MS * 4 : 0);
  static constexpr int ROW = TM + (DELTA ? CH * MS * 4 : 0);
  static constexpr int BYTES = ROW + (5 * CH + 8) * 4;
  static constexpr int JOBS_PER_CU = 3;
};
static_assert(3 * GroupLds<true>::BYTES <= 160 * 1024, "three grouped jobs per CU");

template <bool DELTA>
__global__ __launch_bounds__(NT, 3) void chunk_group_kernel(const ChunkParams p, const int n_jobs) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  using LD = GroupLds<DELTA>;
  f16x8* YB = reinterpret_cast<f16x8*>(smem + LD::YB);
  float* AM = reinterpret_cast<float*>(smem + LD::AM);
  float* TM = reinterpret_cast<float*>(smem + LD::TM);
  float* ROW = reinterpret_cast<float*>(smem + LD::ROW);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int n = wave, r = SUB * n + l16;

  f16x8 sel[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[hh][e] = (8 * lg + e == 16 * hh + l16) ? (f16)1.f : (f16)0.f;

  const int H = p.H, HQ = p.H_qk, G = H / HQ;
  typedef __attribute__((address_space(4))) const int cint;
  typedef __attribute__((address_space(4))) const float cfloat;
  cint* chunks = (cint*)p.chunks;
  cfloat* A_log = (cfloat*)p.A_log;
  const int job = blockIdx.x;
  const int e = __builtin_amdgcn_readfirstlane(job / HQ), hq = __builtin_amdgcn_readfirstlane(job % HQ);
  int4 ce;
  if (p.dense_T > 0) {  // B rows of T tokens: entry e is chunk e % NC of row e / NC
    const int T = p.dense_T, nc = (T + CH - 1) / CH, b = e / nc, c = e - b * nc;
    ce = make_int4(b, b * T + c * CH, min(CH, T - c * CH), c);
  } else {
    ce = make_int4(chunks[4 * e], chunks[4 * e + 1], chunks[4 * e + 2], chunks[4 * e + 3]);
  }
  const int len = ce.z, tok0 = ce.y;
  if (len <= 0) return;  // uniform over the workgroup
  const bool live = r < len;
  const size_t t = (size_t)(tok0 + min(r, len - 1));  // rows past the end are clamped and zeroed when used
  const int h_first = hq * G;

  // inputs: this lane's q/k row slices, and the gate and write strength of the group's first head
  uint2 qv[8], kv[8];
  {
    const uint16_t* qp = p.q + (t * HQ + hq) * HD + 8 * lg;
    const uint16_t* kp = p.k + (t * HQ + hq) * HD + 8 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 a = *reinterpret_cast<const uint4*>(qp + 32 * s);
      const uint4 b = *reinterpret_cast<const uint4*>(kp + 32 * s);
      qv[2 * s] = make_uint2(a.x, a.y);
      qv[2 * s + 1] = make_uint2(a.z, a.w);
      kv[2 * s] = make_uint2(b.x, b.y);
      kv[2 * s + 1] = make_uint2(b.z, b.w);
    }
  }
  uint32_t gs_next = p.g_raw[t * H + h_first];
  float bl_next = DELTA ? p.beta[t * H + h_first] : 0.f;
  __builtin_amdgcn_sched_barrier(0);

  // ---- shared part: normalised rows, qn and kn^T fragments, Gram blocks ------
  float X[32], Q[32];  // kn, qn
  {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x[4], y[4];
      unpack4(qv[i], x);
      unpack4(kv[i], y);
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
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float kn[8], qn[8];
      unpack4(kv[2 * s], kn);
      unpack4(kv[2 * s + 1], kn + 4);
      unpack4(qv[2 * s], qn);
      unpack4(qv[2 * s + 1], qn + 4);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        X[8 * s + q] = kn[q] * rk;
        Q[8 * s + q] = qn[q] * rq;
      }
    }
  }
  uint8_t* rec0 = p.rec + ((size_t)e * H + h_first) * REC_BYTES;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f16x8 xh = to_f16x8(&X[8 * s]);
    if (n < 3) YB[(n * 4 + s) * 64 + lane] = xh;
    store_reordered<true>(rec0 + REC_QHAT + (n * 4 + s) * FRAG_BYTES, to_f16x8(&Q[8 * s]), sel, lane);
    // the delta rule's W S is formed in the recurrence from kn S (W = T diag(b) diag(exp(Gamma)) kn):
    // kn goes to the first head's W slot in the A-operand order of Qhat, and no head stores W
    if (DELTA) store_reordered<true>(rec0 + REC_WNEG + (n * 4 + s) * FRAG_BYTES, xh, sel, lane);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {  // kn^T by selection products
      const int kt = 2 * s + hh;
      const f32x4 tb = mma_f16(xh, sel[hh], zero4());
      const f16x4 tb4 = {(f16)tb[0], (f16)tb[1], (f16)tb[2], (f16)tb[3]};
      // half-fragment pieces from two waves: an ordinary store, so L2 merges them into whole lines
      // (measured: a non-temporal store here took the kernel from 0.30 to 0.35 ms)
      *reinterpret_cast<f16x4*>(rec0 + REC_KBAR + (kt * 2 + (n >> 1)) * FRAG_BYTES + lane * 16 + (n & 1) * 8) = tb4;
    }
  }
  __syncthreads();  // Y operands visible

  f32x4 accA[3], accM[3], accA_d = zero4(), accM_d = zero4();
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    accA[a] = zero4();
    accM[a] = zero4();
  }

  // Everything below is instantiated per sub-chunk index N (wave-uniform);
  // every instantiation passes the same barriers.
  auto body = [&](auto Nc) {
    constexpr int N = decltype(Nc)::value;
    // Gram blocks (N, a <= N), shared by the group's value heads
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 xh = to_f16x8(&X[8 * s]), qh = to_f16x8(&Q[8 * s]);
#pragma unroll
      for (int a = 2; a >= 0; --a) {
        if (a < N) {
          const f16x8 ya = YB[(a * 4 + s) * 64 + lane];
          if (DELTA) accA[a] = mma_f16(xh, ya, accA[a]);
          accM[a] = mma_f16(ya, qh, accM[a]);
        }
      }
      if (DELTA) accA_d = mma_f16(xh, xh, accA_d);
      accM_d = mma_f16(xh, qh, accM_d);
    }

#pragma unroll 1
    for (int gi = 0; gi < G; ++gi) {
      const int h = h_first + gi;
      const uint32_t gs = gs_next;
      const float bl = bl_next;
      {  // the next head's gate and write strength (clamped, so the loads are unconditional)
        const int hn = h_first + min(gi + 1, G - 1);
        gs_next = p.g_raw[t * H + hn];
        if (DELTA) bl_next = p.beta[t * H + hn];
      }
      const float a_h = __expf(A_log[h]);
      float g = 0.f;
      if (live) {
        float d;
        gate_decay(bf16_to_f32((uint16_t)gs), a_h, d, g);
      }
      const float beta = live ? (DELTA ? sigmoidf_(bl) : 1.f) : 0.f;
      const float Gloc = row_prefix_sum(g);  // gate prefix within the sub-chunk
      if (lg == 0) {
        ROW[R_BETA + r] = beta;
        ROW[R_GP + r] = Gloc;
      }
      if (lane == 15) ROW[R_GS + n] = Gloc;
      __syncthreads();  // this head's per-token values visible

      float gbase[NSUB], GL = 0.f;
#pragma unroll
      for (int m = 0; m < NSUB; ++m) {
        gbase[m] = GL;
        GL += ROW[R_GS + m];
      }
      auto gam = [&](int x) { return ROW[R_GP + x] + gbase[x >> 4]; };
      const float Gr = Gloc + gbase[N];
      const float EGr = exp2f(Gr * LOG2E), EGLr = exp2f((GL - Gr) * LOG2E);
      uint8_t* rec = p.rec + ((size_t)e * H + h) * REC_BYTES;
      if (lg == 0) {
        float* glp = reinterpret_cast<float*>(rec + REC_GL);
        glp[r] = EGr;
        glp[CH + r] = EGLr;
      }

      // ---- A rows of this sub-chunk -> LDS; M fragments -> record ------------
      float brow[4], grow[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = SUB * N + 4 * lg + j;
        brow[j] = ROW[R_BETA + rr];
        grow[j] = gam(rr);
      }
      f32x4 Ncl = zero4();  // the diagonal block A_nn in C layout
      if (DELTA) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rl = 4 * lg + j, il = l16;
          float v = 0.f;
          if (il < rl) v = accA_d[j] * brow[j] * exp2f((grow[j] - gam(SUB * N + il)) * LOG2E);
          Ncl[j] = v;
          AM[(SUB * N + rl) * MS + SUB * N + il] = v;
        }
#pragma unroll
        for (int a = 0; a < 3; ++a) {
          if (a < N) {
            const float gi_ = gam(SUB * a + l16);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              AM[(SUB * N + 4 * lg + j) * MS + SUB * a + l16] = accA[a][j] * brow[j] * exp2f((grow[j] - gi_) * LOG2E);
          }
        }
      }
      {
        const float gr = gam(r);
        float md[4], mo[3][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int il = 4 * lg + j;
          md[j] = il <= l16 ? accM_d[j] * exp2f((gr - gam(SUB * N + il)) * LOG2E) : 0.f;
        }
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            mo[a][j] = a < N ? accM[a][j] * exp2f((gr - gam(SUB * a + 4 * lg + j)) * LOG2E) : 0.f;
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // fragment (n, 0): blocks (n, 0), (n, 1)
          v[j] = N == 0 ? md[j] : mo[0][j];
          v[4 + j] = N == 0 ? 0.f : (N == 1 ? md[j] : mo[1][j]);
        }
        store_frag<true>(rec, REC_M, N * 2, lane, v);
        if (N >= 2) {  // fragment (n, 1): blocks (n, 2), (n, 3)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = N == 2 ? md[j] : mo[2][j];
            v[4 + j] = N == 3 ? md[j] : 0.f;
          }
          store_frag<true>(rec, REC_M, N * 2 + 1, lane, v);
        }
      }

      if (DELTA) {
        // ---- T_nn = (I + A_nn)^-1 on fp32 matrix cores (as in chunk_local_kernel) --
        const float4 nt = *reinterpret_cast<const float4*>(&AM[(SUB * N + l16) * MS + SUB * N + 4 * lg]);
        const f32x4 Tnn = unit_lower_inverse(Ncl, f32x4{nt.x, nt.y, nt.z, nt.w}, l16, lg);
#pragma unroll
        for (int j = 0; j < 4; ++j) TM[(SUB * N + 4 * lg + j) * MS + SUB * N + l16] = Tnn[j];
        __syncthreads();  // A rows and diagonal T blocks visible

        // ---- off-diagonal blocks of T by block column (as in chunk_local_kernel) --
        {
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

        // ---- T diag(b) fragments ------------------------------------------------
        {
          const int rt = SUB * N + l16;
          constexpr int ns = (N >> 1) + 1;  // token slices with nonzero T entries for this tile
#pragma unroll
          for (int s = 0; s < ns; ++s) {
            const int j0 = 32 * s + 4 * lg, j1 = j0 + 16;
            float v[8], tv[8], bb[8];
            *reinterpret_cast<float4*>(&tv[0]) = *reinterpret_cast<const float4*>(&TM[rt * MS + j0]);
            *reinterpret_cast<float4*>(&tv[4]) = *reinterpret_cast<const float4*>(&TM[rt * MS + j1]);
            *reinterpret_cast<float4*>(&bb[0]) = *reinterpret_cast<const float4*>(&ROW[R_BETA + j0]);
            *reinterpret_cast<float4*>(&bb[4]) = *reinterpret_cast<const float4*>(&ROW[R_BETA + j1]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              v[q] = (j0 + q <= rt) ? tv[q] * bb[q] : 0.f;
              v[4 + q] = (j1 + q <= rt) ? tv[4 + q] * bb[4 + q] : 0.f;
            }
            store_frag<true>(rec, REC_TB, N * 2 + s, lane, v);
          }
        }
      }
      __syncthreads();  // this head's per-token values, A and T consumed before the next head
    }
  };
  switch (n) {
    case 0: body(std::integral_constant<int, 0>()); break;
    case 1: body(std::integral_constant<int, 1>()); break;
    case 2: body(std::integral_constant<int, 2>()); break;
    default: body(std::integral_constant<int, 3>()); break;
  }
}

namespace {
// The dynamic LDS size above 64 KB is a per-device kernel attribute.
template <bool PER_CHANNEL, bool DELTA>
hipError_t launch_chunk_variant(const ChunkParams& p, int n_jobs, hipStream_t stream) {
  static std::atomic<int> attr_set[MAX_DEVICES];
  const hipError_t e = once_per_device(attr_set, [] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_local_kernel<PER_CHANNEL, DELTA>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, Lds<PER_CHANNEL, DELTA>::BYTES);
  });
  if (e != hipSuccess) return e;
  // one job per workgroup; two (full layout, LDS-bound) or three (compact) per CU
  chunk_local_kernel<PER_CHANNEL, DELTA><<<n_jobs, NT, Lds<PER_CHANNEL, DELTA>::BYTES, stream>>>(p, n_jobs);
  return hipSuccess;
}

// one job per (chunk, q/k head), three per CU
template <bool DELTA>
hipError_t launch_group_variant(const ChunkParams& p, int n_jobs, hipStream_t stream) {
  static std::atomic<int> attr_set[MAX_DEVICES];
  const hipError_t e = once_per_device(attr_set, [] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_group_kernel<DELTA>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, GroupLds<DELTA>::BYTES);
  });
  if (e != hipSuccess) return e;
  chunk_group_kernel<DELTA><<<n_jobs, NT, GroupLds<DELTA>::BYTES, stream>>>(p, n_jobs);
  return hipSuccess;
}
}  // namespace

hipError_t launch_chunk_local(const ChunkParams& p, int n_entries, bool per_channel, bool delta,
                              hipStream_t stream) {
  const int n_jobs = n_entries * p.H;
  if (n_jobs <= 0) return hipSuccess;
  if (shares_qk_fragments(per_channel, p.H, p.H_qk, n_entries)) {  // one workgroup per (chunk, q/k head)
    if (delta) return launch_group_variant<true>(p, n_entries * p.H_qk, stream);
    return launch_group_variant<false>(p, n_entries * p.H_qk, stream);
  }
  if (delta) {
    if (per_channel) return launch_chunk_variant<true, true>(p, n_jobs, stream);
    return launch_chunk_variant<false, true>(p, n_jobs, stream);
  }
  if (per_channel) return launch_chunk_variant<true, false>(p, n_jobs, stream);
  return launch_chunk_variant<false, false>(p, n_jobs, stream);
}

}  // namespace kda
