// kda_recur.hip -- the sequential part of the chunked forward pass.
//
// A workgroup owns one (sequence, value head) chain and one, two or four
// adjacent 16-column value tiles: the columns of the state evolve
// independently, so a chain's 128 value columns are spread over 8, 4 or 2
// workgroups that never communicate (four tiles only for decay-only linear
// attention over many chains).  Per chunk, with the chunk record produced by the chunk-local
// kernel and the 128 x 16 state tiles S (fp32, held in registers in
// matrix-core C layout):
//   U  = T diag(b) V - W S
//   O  = scale * (Qhat S + M U)          -> out (bf16)
//   S <- Diag(exp(Gamma_L)) S + Kbar^T U
// Eight waves split the work by role: four run the chain S -> U -> S' and
// four the output products, so the output of chunk c overlaps the chain of
// chunk c+1.  The fp16 copies of S and U travel between waves through LDS.
//
// Workgroups of one chain are given ids congruent mod 8 so they land on the
// same XCD and share its L2 for the chunk records.  In the one-tile form
// (eight workgroups per chain) each of them also warms its share of the
// record two chunks ahead in that L2; with two tiles per workgroup (many
// chains, the grid runs in rounds) the touches only add HBM requests and are
// left out (measured: grouped-head recurrence 0.93 -> 0.83 ms without them).
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

constexpr int VT = 16;        // value columns per workgroup
constexpr int NVT = HD / VT;  // value tiles per chain
constexpr int VS = CH + 8;    // row stride (fp16) of the transposed value tile

constexpr int PF_AHEAD = 2;                          // chunks the L2 touches run ahead of the loads
constexpr int LINE = 128;                            // L2 line bytes
constexpr int REC_LINES = (REC_BYTES + LINE - 1) / LINE;

template <typename StT>
struct StateIO;

template <>
struct StateIO<float> {
  __device__ static f32x4 load(const void* base, size_t off) {
    const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    return f32x4{x.x, x.y, x.z, x.w};
  }
  __device__ static void store(void* base, size_t off, f32x4 v) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

template <>
struct StateIO<uint16_t> {  // bf16 state
  __device__ static f32x4 load(const void* base, size_t off) {
    const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
    return f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u),
                 __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xFFFF0000u)};
  }
  __device__ static void store(void* base, size_t off, f32x4 v) {
    uint2 x;
    x.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    x.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + off) = x;
  }
};

__device__ __forceinline__ f16x8 ldfrag(const uint8_t* rec, int off, int frag, int lane) {
  return *reinterpret_cast<const f16x8*>(rec + off + frag * FRAG_BYTES + lane * 16);
}

}  // namespace

// ---------------------------------------------------------------------------
// Eight waves, one workgroup per CU (about 230 registers per lane).  The
// chunk-to-chunk chain is S -> U -> S'; the output products (Qhat S, M U)
// and the stores hang off it.  Waves 0..3 run only the chain (token tile w of
// U, key tiles 2w, 2w+1 of S) and waves 4..7 only the output (token tile
// w-4), so the output work of chunk c overlaps the chain of chunk c+1.  Each
// role streams its own fragments through three register sets, two chunks
// ahead; in the one-tile form the chain waves also issue the L2 touches.
// Both roles meet at the same two barriers per chunk.
//
// A workgroup owns NCT adjacent 16-column tiles.  Every fragment of the
// chunk record is loaded once per workgroup and used for all NCT tiles, so
// the record bytes a CU pulls per value column drop by NCT.  A CU takes in
// records at a roughly fixed rate (its outstanding L2 misses times the L2
// latency), so two tiles per workgroup give the better throughput, and one
// tile spreads few chains over more CUs for the shorter chain latency.
// ---------------------------------------------------------------------------
template <int NCT>
struct Bf16Row {  // 4 NCT bf16 of a value row (NCT >= 2)
  uint4 q[NCT / 2];
};
template <int NCT>
using ValueRow = typename std::conditional<NCT == 1, uint2, Bf16Row<NCT>>::type;

template <int NCT>
struct ChainFrags {
  f16x8 w[4], t[2], k[4];  // w: -W, or kn for shared q/k records with the delta rule
  float4 gl[2];
  float4 eg;  // shared q/k records with the delta rule: exp(Gamma_r) of this lane's four U rows
  ValueRow<NCT> v;  // 4 NCT bf16 of the value tile
  uint32_t touch;
};
struct OutFrags {
  f16x8 q[4], m[2];
  float4 eg;  // scalar gate: exp(Gamma_r) of this lane's four output rows
};

__device__ __forceinline__ void unpack_bf16(uint2 x, f16* o) {
  o[0] = (f16)__uint_as_float(x.x << 16);
  o[1] = (f16)__uint_as_float(x.x & 0xFFFF0000u);
  o[2] = (f16)__uint_as_float(x.y << 16);
  o[3] = (f16)__uint_as_float(x.y & 0xFFFF0000u);
}

// DELTA = false (decay-only linear attention): the chunk records carry
// T diag(b) = I and W = 0, so U = V is read straight from the value tile and
// neither W nor T diag(b) is loaded.
//
// PC = false (one decay per token-head, value heads grouped on q/k heads,
// records with shared q/k fragments): Qhat = diag(exp(Gamma)) qn and
// Kbar^T = kn^T diag(exp(Gamma_L - Gamma)), so the record of the first value
// head of each q/k group holds qn and kn^T for the whole group and every
// record holds the two per-token factors.  The output waves scale the rows of
// qn S by exp(Gamma_r); the chain waves scale U's rows by
// exp(Gamma_L - Gamma_r) (a second LDS copy, since M U needs U itself) and
// decay S by the single exp(Gamma_L).  With the delta rule these records hold
// no W either: W = T diag(b) diag(exp(Gamma)) kn, so the chain forms
//   U = T diag(b) (V - diag(exp(Gamma)) (kn S))
// from the group's kn fragments (stored once per group, in the first head's W
// slot): kn S is a product of the same shape as W S, the residual
// V - exp(Gamma_r) (kn S)_r is formed in fp32 and passed through LDS as the
// B operand of T diag(b), at the cost of one more barrier per chunk.
template <typename StT, int NCT, bool DELTA, bool PC>
__global__ __launch_bounds__(512) void recur_split_kernel(RecurParams p) {
  constexpr int VC = VT * NCT;       // value columns per workgroup
  constexpr int NW = NVT / NCT;      // workgroups per chain
  constexpr int T_REC = (REC_LINES + NW - 1) / NW;  // record lines touched per workgroup
  constexpr int T_V = 2 * CH / NW;                 // value-row lines touched per workgroup
  static_assert(NCT != 1 || T_REC + T_V <= 256, "one touch per chain thread");
  __shared__ __attribute__((aligned(16))) f16x8 sbuf[NCT][4 * 64];  // S slices (B operand)
  __shared__ __attribute__((aligned(16))) f16x4 ubuf[NCT][4 * 64];  // U tiles (C layout)
  __shared__ __attribute__((aligned(16))) f16x4 ubuf2[PC ? 1 : NCT][4 * 64];  // scalar gate: decayed U tiles
  constexpr bool KN = DELTA && !PC;  // U from kn S (records without W)
  __shared__ __attribute__((aligned(16))) f16x4 rbuf[KN ? NCT : 1][4 * 64];   // V - exp(Gamma) kn S (C layout)
  __shared__ __attribute__((aligned(16))) f16 vsT[VC * VS];         // value tile, [column][token]

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int tw = wave & 3;
  const int x = blockIdx.x, xcd = x & 7, y = x >> 3;
  if (x == 0 && tid == 0 && p.err) *p.err = 0;
  const int G = PC ? 1 : p.H / p.H_qk;  // value heads per q/k head
  const int vt = y % NW, ch = (y / NW) * 8 + xcd;
  if (ch >= p.n_chains) return;
  const int h = ch % p.H, h0 = h - h % G;  // h0: the group's first value head
  int n;
  int4 sq;
  if (p.dense_T >= 0) {  // B rows of T tokens, in row order
    const int T = p.dense_T;
    n = ch / p.H;
    sq = make_int4(n * T, T, n * ((T + CH - 1) / CH), 0);
  } else {
    n = p.order[ch / p.H];
    sq = p.seqs[n];
  }
  const int tok0 = sq.x, len = sq.y, chunk0 = sq.z;
  // never walk past the schedule, whatever cu_seqlens held
  const int nch = max(0, min((len + CH - 1) / CH, p.n_entries - chunk0));
  const int last = nch - 1;
  const int v0 = vt * VC;
  auto record = [&](int c) { return p.rec + ((size_t)(chunk0 + c) * p.H + h) * REC_BYTES; };
  auto shared_record = [&](int c) { return p.rec + ((size_t)(chunk0 + c) * p.H + h0) * REC_BYTES; };

  // Each role is instantiated per token tile TW (wave-uniform), so the
  // lower-triangular blocks each tile needs resolve at compile time.
  if (wave < 4) {
    // ---- chain waves ---------------------------------------------------------
    auto chain_role = [&](auto TWc) {
      constexpr int TW = decltype(TWc)::value;
      // S[j][i]: column tile j, key tile 2 tw + i; lane (column l16, keys 4lg..4lg+3)
      const size_t sbase = ((size_t)n * p.H + h) * HD * HD + (size_t)(v0 + l16) * HD;
      f32x4 S[NCT][2];
#pragma unroll
      for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int k0 = SUB * (2 * TW + i) + 4 * lg;
          S[j][i] = p.s0 ? StateIO<StT>::load(p.s0, sbase + (size_t)VT * j * HD + k0) : zero4();
        }
      const size_t vstride = (size_t)p.H * HD;
      const int vq = tid & 3;  // this thread's value columns: v0 + 4 NCT vq ..
      const uint16_t* vchain = p.v + ((size_t)tok0 * p.H + h) * HD + v0 + 4 * NCT * vq;
      const int tl = tid < T_REC + T_V ? tid : 0;
      const bool trec = tl < T_REC;
      const int rec_line = min(vt * T_REC + (trec ? tl : 0), REC_LINES - 1);
      const int vrow = (vt * T_V + (trec ? 0 : tl - T_REC)) >> 1, vhalf = (tl - T_REC) & 1;
      auto load = [&](ChainFrags<NCT>& F, int c) {
        const uint8_t* R = record(c);
        const uint8_t* RK = PC ? R : shared_record(c);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          F.w[s2] = ldfrag(KN ? RK : R, REC_WNEG, TW * 4 + s2, lane);
          F.k[s2] = ldfrag(RK, REC_KBAR, (2 * TW + (s2 >> 1)) * 2 + (s2 & 1), lane);
        }
        if constexpr (KN) F.eg = *reinterpret_cast<const float4*>(R + REC_GL + 4 * (SUB * TW + 4 * lg));
        F.t[0] = ldfrag(R, REC_TB, TW * 2, lane);
        F.t[1] = ldfrag(R, REC_TB, TW * 2 + (TW >= 2 ? 1 : 0), lane);
        if (PC) {  // exp(Gamma_L) of this lane's state rows
#pragma unroll
          for (int i = 0; i < 2; ++i)
            F.gl[i] = *reinterpret_cast<const float4*>(R + REC_GL + 4 * (SUB * (2 * TW + i) + 4 * lg));
        } else {   // exp(Gamma_L - Gamma_r) of this lane's U rows; exp(Gamma_L) = exp(Gamma) of the last row
          F.gl[0] = *reinterpret_cast<const float4*>(R + REC_GL + 4 * (CH + SUB * TW + 4 * lg));
          F.gl[1] = *reinterpret_cast<const float4*>(R + REC_GL + 4 * (CH - 4));
        }
        // rows past the chunk's end are clamped here and zeroed at use
        const int Lc = min(CH, len - c * CH);
        F.v = *reinterpret_cast<const decltype(F.v)*>(vchain + (size_t)c * CH * vstride +
                                                        (size_t)min(tid >> 2, Lc - 1) * vstride);
        if constexpr (NCT == 1) {
          const int ct = min(c + PF_AHEAD, last);
          const uint32_t* tp;
          if (trec) {
            tp = reinterpret_cast<const uint32_t*>(record(ct) + (size_t)rec_line * LINE);
          } else {
            const int Lt = min(CH, len - ct * CH);
            tp = reinterpret_cast<const uint32_t*>(p.v + ((size_t)(tok0 + ct * CH + min(vrow, Lt - 1)) * p.H + h) *
                                                       HD + vhalf * (LINE / 2));
          }
          F.touch = *tp;
        } else {
          F.touch = 0u;
        }
      };
      uint32_t sink = 0;
      auto step = [&](const ChainFrags<NCT>& F, int c) {
        sink ^= F.touch;
        const int L = min(CH, len - c * CH);
        {
#pragma unroll
          for (int j = 0; j < NCT; ++j) {
            f16x8 sb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sb[e] = (f16)S[j][0][e];
              sb[4 + e] = (f16)S[j][1][e];
            }
            sbuf[j][TW * 64 + lane] = sb;
          }
          const int r = tid >> 2;
          f16 vh[4 * NCT];
          if constexpr (NCT == 1) {
            unpack_bf16(r < L ? F.v : make_uint2(0u, 0u), vh);
          } else {
#pragma unroll
            for (int i = 0; i < NCT / 2; ++i) {
              const uint4 vv = r < L ? F.v.q[i] : make_uint4(0u, 0u, 0u, 0u);
              unpack_bf16(make_uint2(vv.x, vv.y), vh + 8 * i);
              unpack_bf16(make_uint2(vv.z, vv.w), vh + 8 * i + 4);
            }
          }
#pragma unroll
          for (int e = 0; e < 4 * NCT; ++e) vsT[(4 * NCT * vq + e) * VS + r] = vh[e];
        }
        __syncthreads();  // A
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          if (!DELTA) {  // U = V: rows 16 tw + 4 lg .. +3 of column 16 j + l16
            const f16x4 u = *reinterpret_cast<const f16x4*>(&vsT[(VT * j + l16) * VS + SUB * TW + 4 * lg]);
            ubuf[j][TW * 64 + lane] = u;
            if (!PC)
              ubuf2[j][TW * 64 + lane] = f16x4{(f16)((float)u[0] * F.gl[0].x), (f16)((float)u[1] * F.gl[0].y),
                                               (f16)((float)u[2] * F.gl[0].z), (f16)((float)u[3] * F.gl[0].w)};
            continue;
          }
          f16x8 sB[4];
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) sB[s2] = sbuf[j][s2 * 64 + lane];
          f32x4 U = zero4(), U2 = zero4();
          if constexpr (KN) {
            // residual rows 16 tw + 4 lg .. +3 of column 16 j + l16: V - exp(Gamma_r) (kn S)_r
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
              if (s2 & 1) U2 = mma_f16(F.w[s2], sB[s2], U2);
              else U = mma_f16(F.w[s2], sB[s2], U);
            }
            const f16x4 vr = *reinterpret_cast<const f16x4*>(&vsT[(VT * j + l16) * VS + SUB * TW + 4 * lg]);
            rbuf[j][TW * 64 + lane] = f16x4{(f16)((float)vr[0] - F.eg.x * (U[0] + U2[0])),
                                            (f16)((float)vr[1] - F.eg.y * (U[1] + U2[1])),
                                            (f16)((float)vr[2] - F.eg.z * (U[2] + U2[2])),
                                            (f16)((float)vr[3] - F.eg.w * (U[3] + U2[3]))};
            continue;
          }
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 <= (TW >> 1)) {
              const f16* vr = &vsT[(VT * j + l16) * VS + 32 * s2 + 4 * lg];
              const f16x4 lo = *reinterpret_cast<const f16x4*>(vr);
              const f16x4 hi = *reinterpret_cast<const f16x4*>(vr + 16);
              const f16x8 vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              if (s2 == 0) U = mma_f16(F.t[0], vb, U);
              else U2 = mma_f16(F.t[1], vb, U2);
            }
          }
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            if (s2 & 1) U2 = mma_f16(F.w[s2], sB[s2], U2);
            else U = mma_f16(F.w[s2], sB[s2], U);
          }
          const f32x4 Us = {U[0] + U2[0], U[1] + U2[1], U[2] + U2[2], U[3] + U2[3]};
          ubuf[j][TW * 64 + lane] = f16x4{(f16)Us[0], (f16)Us[1], (f16)Us[2], (f16)Us[3]};
          if (!PC)
            ubuf2[j][TW * 64 + lane] = f16x4{(f16)(Us[0] * F.gl[0].x), (f16)(Us[1] * F.gl[0].y),
                                             (f16)(Us[2] * F.gl[0].z), (f16)(Us[3] * F.gl[0].w)};
        }
        if constexpr (KN) {
          __syncthreads();  // A2: residual tiles published
#pragma unroll
          for (int j = 0; j < NCT; ++j) {
            f32x4 U = zero4(), U2 = zero4();
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              if (s2 <= (TW >> 1)) {  // tokens 32 s2 + 4 lg + e, then 32 s2 + 16 + 4 lg + e (T's slice order)
                const f16x4 a = rbuf[j][(2 * s2) * 64 + lane], b = rbuf[j][(2 * s2 + 1) * 64 + lane];
                const f16x8 rb = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
                if (s2 == 0) U = mma_f16(F.t[0], rb, U);
                else U2 = mma_f16(F.t[1], rb, U2);
              }
            }
            const f32x4 Us = {U[0] + U2[0], U[1] + U2[1], U[2] + U2[2], U[3] + U2[3]};
            ubuf[j][TW * 64 + lane] = f16x4{(f16)Us[0], (f16)Us[1], (f16)Us[2], (f16)Us[3]};
            ubuf2[j][TW * 64 + lane] = f16x4{(f16)(Us[0] * F.gl[0].x), (f16)(Us[1] * F.gl[0].y),
                                             (f16)(Us[2] * F.gl[0].z), (f16)(Us[3] * F.gl[0].w)};
          }
        }
        __syncthreads();  // B
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          f16x8 uB[2];
          const f16x4* ub = PC ? ubuf[j] : ubuf2[PC ? 0 : j];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const f16x4 a = ub[(2 * s2) * 64 + lane], b = ub[(2 * s2 + 1) * 64 + lane];
            uB[s2] = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
          }
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const float4 d = PC ? F.gl[i] : make_float4(F.gl[1].w, F.gl[1].w, F.gl[1].w, F.gl[1].w);
            const f32x4 a = mma_f16(F.k[2 * i], uB[0],
                                    f32x4{d.x * S[j][i][0], d.y * S[j][i][1], d.z * S[j][i][2], d.w * S[j][i][3]});
            const f32x4 b = mma_f16(F.k[2 * i + 1], uB[1], zero4());
            S[j][i] = f32x4{a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
          }
        }
      };
      ChainFrags<NCT> f0, f1, f2;
      if (nch > 0) {
        load(f0, 0);
        load(f1, min(1, last));
      }
      __builtin_amdgcn_s_waitcnt(0);
      for (int c = 0; c < nch; c += 3) {
        load(f2, min(c + 2, last));
        step(f0, c);
        if (c + 1 >= nch) break;
        load(f0, min(c + 3, last));
        step(f1, c + 1);
        if (c + 2 >= nch) break;
        load(f1, min(c + 4, last));
        step(f2, c + 2);
      }
      asm volatile("" ::"v"(sink));
      if (p.s1) {
#pragma unroll
        for (int j = 0; j < NCT; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int k0 = SUB * (2 * TW + i) + 4 * lg;
            StateIO<StT>::store(p.s1, sbase + (size_t)VT * j * HD + k0, S[j][i]);
          }
      }
    };
    switch (tw) {
      case 0: chain_role(std::integral_constant<int, 0>()); break;
      case 1: chain_role(std::integral_constant<int, 1>()); break;
      case 2: chain_role(std::integral_constant<int, 2>()); break;
      default: chain_role(std::integral_constant<int, 3>()); break;
    }
    return;
  }


  // ---- output waves ----------------------------------------------------------
  auto out_role = [&](auto TWc) {
    constexpr int TW = decltype(TWc)::value;
    const size_t row_step = (size_t)p.H * HD;
    uint16_t* orow = p.out + ((size_t)(tok0 + SUB * TW + 4 * lg) * p.H + h) * HD + v0 + l16;
    auto load = [&](OutFrags& F, int c) {
      const uint8_t* R = record(c);
      const uint8_t* RQ = PC ? R : shared_record(c);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) F.q[s2] = ldfrag(RQ, REC_QHAT, TW * 4 + s2, lane);
      F.m[0] = ldfrag(R, REC_M, TW * 2, lane);
      F.m[1] = ldfrag(R, REC_M, TW * 2 + (TW >= 2 ? 1 : 0), lane);
      if (!PC) F.eg = *reinterpret_cast<const float4*>(R + REC_GL + 4 * (SUB * TW + 4 * lg));
    };
    auto step = [&](const OutFrags& F, int c) {
      const int L = min(CH, len - c * CH);
      __syncthreads();  // A: S_c slices published
      f32x4 OQ[NCT];
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        f16x8 sB[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) sB[s2] = sbuf[j][s2 * 64 + lane];
        f32x4 a = zero4(), b = zero4();
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          if (s2 & 1) b = mma_f16(F.q[s2], sB[s2], b);
          else a = mma_f16(F.q[s2], sB[s2], a);
        }
        OQ[j] = f32x4{a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
        if (!PC) OQ[j] = f32x4{OQ[j][0] * F.eg.x, OQ[j][1] * F.eg.y, OQ[j][2] * F.eg.z, OQ[j][3] * F.eg.w};
      }
      if constexpr (KN) __syncthreads();  // A2 (the chain waves' residual exchange)
      __syncthreads();  // B: U_c published
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        f16x8 uB[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const f16x4 a = ubuf[j][(2 * s2) * 64 + lane], b = ubuf[j][(2 * s2 + 1) * 64 + lane];
          uB[s2] = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        }
        f32x4 O = mma_f16(F.m[0], uB[0], OQ[j]);
        if (TW >= 2) O = mma_f16(F.m[1], uB[1], O);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = SUB * TW + 4 * lg + e;
          // rows past the chunk's end go to a sink, keeping the store unconditional
          uint16_t* dst = r < L ? orow + (size_t)e * row_step + VT * j : p.sink + lane;
          *dst = f32_to_bf16(p.scale * O[e]);
        }
      }
      orow += (size_t)CH * row_step;
    };
    OutFrags f0, f1, f2;
    if (nch > 0) {
      load(f0, 0);
      load(f1, min(1, last));
    }
    __builtin_amdgcn_s_waitcnt(0);
    for (int c = 0; c < nch; c += 3) {
      load(f2, min(c + 2, last));
      step(f0, c);
      if (c + 1 >= nch) break;
      load(f0, min(c + 3, last));
      step(f1, c + 1);
      if (c + 2 >= nch) break;
      load(f1, min(c + 4, last));
      step(f2, c + 2);
    }
  };
  switch (tw) {
    case 0: out_role(std::integral_constant<int, 0>()); break;
    case 1: out_role(std::integral_constant<int, 1>()); break;
    case 2: out_role(std::integral_constant<int, 2>()); break;
    default: out_role(std::integral_constant<int, 3>()); break;
  }
}

namespace {
// workgroups for n_chains chains with `tiles` workgroups per chain
int grid_for(int n_chains, int tiles) { return ((n_chains + 7) / 8) * 8 * tiles; }

int cu_count() { return device_cu_count(); }
}  // namespace

int device_cu_count() {
  static std::atomic<int> cus[MAX_DEVICES];
  const int d = current_device();
  int v = cus[d].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess || v <= 0) v = 256;
    cus[d].store(v, std::memory_order_relaxed);
  }
  return v;
}

bool shares_qk_fragments(bool per_channel, int H, int H_qk, int n_entries) {
  // the grouped chunk-local kernel walks a group's heads in series, so it
  // needs enough (chunk, q/k head) jobs to fill the chip; below that the
  // per-head kernel and its records are faster
  return !per_channel && H != H_qk && (long)n_entries * H_qk >= GROUP_MIN_JOBS;
}

int recur_grid(int n_chains) {
  const int g = grid_for(n_chains, NVT);
  return g <= cu_count() ? g : grid_for(n_chains, NVT / 2);
}

namespace {
template <bool DELTA, bool PC>
void launch_recur_variant(const RecurParams& p, bool bf16_state, hipStream_t stream) {
  if (grid_for(p.n_chains, NVT) <= cu_count()) {  // few chains: one column tile per workgroup, all on CUs of their own
    const int g = grid_for(p.n_chains, NVT);
    if (bf16_state) recur_split_kernel<uint16_t, 1, DELTA, PC><<<g, 512, 0, stream>>>(p);
    else recur_split_kernel<float, 1, DELTA, PC><<<g, 512, 0, stream>>>(p);
    return;
  }
  const int g2 = grid_for(p.n_chains, NVT / 2);  // two column tiles per workgroup
  if constexpr (!DELTA) {
    if (g2 > 2 * cu_count()) {
      // decay-only linear attention over many chains: its chain step has no
      // W S product, so four column tiles per workgroup cost little compute
      // and halve again the record bytes each column pulls
      const int g4 = grid_for(p.n_chains, NVT / 4);
      if (bf16_state) recur_split_kernel<uint16_t, 4, false, PC><<<g4, 512, 0, stream>>>(p);
      else recur_split_kernel<float, 4, false, PC><<<g4, 512, 0, stream>>>(p);
      return;
    }
  }
  if (bf16_state) recur_split_kernel<uint16_t, 2, DELTA, PC><<<g2, 512, 0, stream>>>(p);
  else recur_split_kernel<float, 2, DELTA, PC><<<g2, 512, 0, stream>>>(p);
}
}  // namespace

void launch_recur(const RecurParams& p, bool bf16_state, bool per_channel, bool delta, hipStream_t stream) {
  // records without shared q/k fragments carry Qhat, Kbar^T and exp(Gamma_L) per key
  if (!shares_qk_fragments(per_channel, p.H, p.H_qk, p.n_entries)) per_channel = true;
  if (delta) {
    if (per_channel) launch_recur_variant<true, true>(p, bf16_state, stream);
    else launch_recur_variant<true, false>(p, bf16_state, stream);
  } else {
    if (per_channel) launch_recur_variant<false, true>(p, bf16_state, stream);
    else launch_recur_variant<false, false>(p, bf16_state, stream);
  }
}

}  // namespace kda
