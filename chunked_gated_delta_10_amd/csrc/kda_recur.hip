// kda_recur.hip -- the sequential part of the chunked forward pass.
//
// One workgroup owns one (sequence, value head, 16-column value tile): the
// columns of the state evolve independently, so a chain's 128 value columns
// are spread over 8 workgroups that never communicate.  Per chunk, with the
// chunk record produced by the chunk-local kernel and the 128 x 16 state tile
// S (fp32, held in registers in matrix-core C layout):
//   U  = T diag(b) V - W S
//   O  = scale * (Qhat S + M U)          -> out (bf16)
//   S <- Diag(exp(Gamma_L)) S + Kbar^T U
// Wave w owns token tile w of U and O and key tiles 2w, 2w+1 of S; the fp16
// copies of S and U travel between waves through LDS (4 KiB + 2 KiB).  The
// chunk records stream through two or three register sets.  Grids of at most
// one workgroup per CU use an eight-wave variant that gives the chain
// S -> U -> S' and the output products to different waves.
//
// Workgroups of one chain are given ids congruent mod 8 so they land on the
// same XCD and share its L2 for the chunk records, and each of them warms a
// later record's eighth in that L2.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

constexpr int VT = 16;        // value columns per workgroup
constexpr int NVT = HD / VT;  // value tiles per chain
constexpr int VS = CH + 8;    // row stride (fp16) of the transposed value tile

constexpr int PF_AHEAD = 3;                          // chunks the L2 touches run ahead of the loads
constexpr int LINE = 128;                            // L2 line bytes
constexpr int REC_LINES = (REC_BYTES + LINE - 1) / LINE;
constexpr int TOUCH_REC = (REC_LINES + NVT - 1) / NVT;  // record lines touched per value tile (65)
constexpr int TOUCH_V = 2 * CH / NVT;                // value-row lines touched per value tile (16)
static_assert(TOUCH_REC + TOUCH_V <= 256, "one touch per thread");

struct Frags {
  f16x8 w[4], q[4], k[4], m[2], t[2];
  float4 gl[2];
  uint2 v;         // 4 bf16 of the value tile (token tid/4, columns 4*(tid%4)..)
  uint32_t touch;  // word of a later chunk's record or value row, loaded only to pull its line into L2
};

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

__device__ __forceinline__ void load_frags(Frags& F, const uint8_t* R, int wave, int lane, int tid,
                                           const uint16_t* vsrc, int L, size_t vstride) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    F.w[s] = ldfrag(R, REC_WNEG, wave * 4 + s, lane);
    F.q[s] = ldfrag(R, REC_QHAT, wave * 4 + s, lane);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) F.k[i] = ldfrag(R, REC_KBAR, (2 * wave + (i >> 1)) * 2 + (i & 1), lane);
  F.m[0] = ldfrag(R, REC_M, wave * 2, lane);
  F.t[0] = ldfrag(R, REC_TB, wave * 2, lane);
  if (wave >= 2) {
    F.m[1] = ldfrag(R, REC_M, wave * 2 + 1, lane);
    F.t[1] = ldfrag(R, REC_TB, wave * 2 + 1, lane);
  }
  const int lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    F.gl[i] = *reinterpret_cast<const float4*>(R + REC_GL + 4 * (SUB * (2 * wave + i) + 4 * lg));
  // rows past the chunk's end are clamped here (L >= 1) and zeroed at use, so
  // the load is unconditional
  F.v = *reinterpret_cast<const uint2*>(vsrc + (size_t)min(tid >> 2, L - 1) * vstride);
}

}  // namespace

template <typename StT, int NSTAGE>
__global__ __launch_bounds__(256) void recur_kernel(RecurParams p) {
  __shared__ __attribute__((aligned(16))) f16x8 sbuf[4 * 64];  // S slices (B operand)
  __shared__ __attribute__((aligned(16))) f16x4 ubuf[4 * 64];  // U tiles (C layout)
  __shared__ __attribute__((aligned(16))) f16 vsT[VT * VS];    // value tile, [column][token]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int x = blockIdx.x, xcd = x & 7, y = x >> 3;
  const int vt = y % NVT, ch = (y / NVT) * 8 + xcd;
  if (ch >= p.n_chains) return;
  const int n = p.order[ch / p.H], h = ch % p.H;
  const int4 sq = p.seqs[n];
  const int tok0 = sq.x, len = sq.y, chunk0 = sq.z;
  // never walk past the schedule, whatever cu_seqlens held
  const int nch = max(0, min((len + CH - 1) / CH, p.n_entries - chunk0));
  const int v0 = vt * VT;

  // state tile: wave holds key tiles 2w, 2w+1; lane (column l16, key rows 4lg..4lg+3)
  const size_t sbase = ((size_t)n * p.H + h) * HD * HD + (size_t)(v0 + l16) * HD;
  f32x4 S[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int k0 = SUB * (2 * wave + i) + 4 * lg;
    S[i] = p.s0 ? StateIO<StT>::load(p.s0, sbase + k0) : zero4();
  }

  const size_t vstride = (size_t)p.H * HD;
  const int vcol = v0 + 4 * (tid & 3);
  const uint16_t* vchain = p.v + ((size_t)tok0 * p.H + h) * HD + vcol;
  // L2 warm-up: value tile vt's workgroup touches record lines
  // [vt*TOUCH_REC, ...) and value-row lines [vt*TOUCH_V, ...) of chunk
  // c + PF_AHEAD, so the eight workgroups of a chain together bring each
  // record into their XCD's L2 before any of them loads it.  Threads past
  // the share repeat a valid address.
  const int tl = tid < TOUCH_REC + TOUCH_V ? tid : 0;
  const bool trec = tl < TOUCH_REC;
  const int rec_line = min(vt * TOUCH_REC + (trec ? tl : 0), REC_LINES - 1);
  const int vrow = (vt * TOUCH_V + (trec ? 0 : tl - TOUCH_REC)) >> 1, vhalf = (tl - TOUCH_REC) & 1;
  auto load_chunk = [&](Frags& F, int c) {
    const uint8_t* R = p.rec + ((size_t)(chunk0 + c) * p.H + h) * REC_BYTES;
    load_frags(F, R, wave, lane, tid, vchain + (size_t)c * CH * vstride, min(CH, len - c * CH), vstride);
    const int ct = min(c + PF_AHEAD, nch - 1);
    const uint32_t* tp;
    if (trec) {
      tp = reinterpret_cast<const uint32_t*>(p.rec + ((size_t)(chunk0 + ct) * p.H + h) * REC_BYTES + (size_t)rec_line * LINE);
    } else {
      const int L = min(CH, len - ct * CH);
      tp = reinterpret_cast<const uint32_t*>(p.v + ((size_t)(tok0 + ct * CH + min(vrow, L - 1)) * p.H + h) * HD +
                                             vhalf * (LINE / 2));
    }
    F.touch = *tp;
  };

  uint32_t sink = 0;  // keeps the L2 touches alive; consumed NSTAGE-1 steps after issue
  // one chunk of the recurrence on fragments F
  auto step = [&](const Frags& F, int c) {
    sink ^= F.touch;
    const int L = min(CH, len - c * CH);
    // 1. publish this wave's fp16 slice of S and the value tile
    {
      f16x8 sb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sb[j] = (f16)S[0][j];
        sb[4 + j] = (f16)S[1][j];
      }
      sbuf[wave * 64 + lane] = sb;
      const int r = tid >> 2, c4 = 4 * (tid & 3);
      const uint2 vv = r < L ? F.v : make_uint2(0u, 0u);
      vsT[(c4 + 0) * VS + r] = (f16)__uint_as_float(vv.x << 16);
      vsT[(c4 + 1) * VS + r] = (f16)__uint_as_float(vv.x & 0xFFFF0000u);
      vsT[(c4 + 2) * VS + r] = (f16)__uint_as_float(vv.y << 16);
      vsT[(c4 + 3) * VS + r] = (f16)__uint_as_float(vv.y & 0xFFFF0000u);
    }
    __syncthreads();
    // 2. U = T diag(b) V - W S ;  OQ = Qhat S      (token tile `wave`)
    //    (two accumulators each, halving the dependent matrix-core chains)
    f16x8 sB[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) sB[s] = sbuf[s * 64 + lane];
    f32x4 U = zero4(), U2 = zero4(), OQ = zero4(), OQ2 = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s <= (wave >> 1)) {
        const f16x4 lo = *reinterpret_cast<const f16x4*>(&vsT[l16 * VS + 32 * s + 4 * lg]);
        const f16x4 hi = *reinterpret_cast<const f16x4*>(&vsT[l16 * VS + 32 * s + 16 + 4 * lg]);
        const f16x8 vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (s == 0) U = mma_f16(F.t[s], vb, U);
        else U2 = mma_f16(F.t[s], vb, U2);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s & 1) {
        U2 = mma_f16(F.w[s], sB[s], U2);
        OQ2 = mma_f16(F.q[s], sB[s], OQ2);
      } else {
        U = mma_f16(F.w[s], sB[s], U);
        OQ = mma_f16(F.q[s], sB[s], OQ);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      U[j] += U2[j];
      OQ[j] += OQ2[j];
    }
    // 3. publish U (fp16, C layout of token tile `wave`)
    {
      const f16x4 u4 = {(f16)U[0], (f16)U[1], (f16)U[2], (f16)U[3]};
      ubuf[wave * 64 + lane] = u4;
    }
    __syncthreads();
    // 4. O = scale (OQ + M U) ; S <- Diag(exp(Gamma_L)) S + Kbar^T U
    f16x8 uB[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x4 a = ubuf[(2 * s) * 64 + lane], b = ubuf[(2 * s + 1) * 64 + lane];
      uB[s] = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    f32x4 O = OQ;
    O = mma_f16(F.m[0], uB[0], O);
    if (wave >= 2) O = mma_f16(F.m[1], uB[1], O);
    {
      const size_t orow0 = (size_t)(tok0 + c * CH) * p.H + h;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = SUB * wave + 4 * lg + j;
        // rows past the chunk's end go to a sink, keeping the store unconditional
        // (a conditional store would make later waits cover all stores)
        uint16_t* dst = r < L ? p.out + (orow0 + (size_t)r * p.H) * HD + v0 + l16 : p.sink + lane;
        *dst = f32_to_bf16(p.scale * O[j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float4 gl = F.gl[i];
      f32x4 acc = {gl.x * S[i][0], gl.y * S[i][1], gl.z * S[i][2], gl.w * S[i][3]};
      acc = mma_f16(F.k[2 * i], uB[0], acc);
      acc = mma_f16(F.k[2 * i + 1], uB[1], acc);
      S[i] = acc;
    }
  };

  // NSTAGE fragment sets in rotation: chunk c + NSTAGE - 1 loads while chunk
  // c computes.  Loads past the last chunk re-read the last chunk (clamped),
  // so every load is unconditional and the wait counts inside the loop are
  // exact.  Three sets give a record two chunk steps to arrive but take ~300
  // registers (one workgroup per CU); two sets fit two workgroups per CU,
  // which suits grids with many short chains.
  const int last = nch - 1;
  if (NSTAGE == 3) {
    Frags f0, f1, f2;
    if (nch > 0) {
      load_chunk(f0, 0);
      load_chunk(f1, min(1, last));
    }
    // Drain the first loads here, so the loop header carries no pending-load
    // state on the fragments and each wait inside the loop only covers the
    // oldest set.
    __builtin_amdgcn_s_waitcnt(0);
    for (int c = 0; c < nch; c += 3) {
      load_chunk(f2, min(c + 2, last));
      step(f0, c);
      if (c + 1 >= nch) break;
      load_chunk(f0, min(c + 3, last));
      step(f1, c + 1);
      if (c + 2 >= nch) break;
      load_chunk(f1, min(c + 4, last));
      step(f2, c + 2);
    }
  } else {
    Frags f0, f1;
    if (nch > 0) load_chunk(f0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    for (int c = 0; c < nch; c += 2) {
      load_chunk(f1, min(c + 1, last));
      step(f0, c);
      if (c + 1 >= nch) break;
      load_chunk(f0, min(c + 2, last));
      step(f1, c + 1);
    }
  }
  asm volatile("" ::"v"(sink));
  if (p.s1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k0 = SUB * (2 * wave + i) + 4 * lg;
      StateIO<StT>::store(p.s1, sbase + k0, S[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Split-role variant (eight waves) for grids of at most one workgroup per CU.
// The chunk-to-chunk chain is S -> U -> S'; the output products (Qhat S,
// M U) and the stores hang off it.  Waves 0..3 run only the chain (token
// tile w of U, key tiles 2w, 2w+1 of S) and waves 4..7 only the output
// (token tile w-4), so the output work of chunk c overlaps the chain of chunk
// c+1.  Each role streams its own fragments through three register sets, two
// chunks ahead; the chain waves also issue the L2 touches.  Both roles meet
// at the same two barriers per chunk.
//
// A workgroup owns NCT adjacent 16-column tiles.  Every fragment of the
// chunk record is loaded once per workgroup and used for all NCT tiles, so
// the record bytes a CU pulls per value column drop by NCT; two tiles per
// workgroup suit grids with many chains (grouped value heads), one tile
// spreads few chains over more CUs.
// ---------------------------------------------------------------------------
template <int NCT>
struct ChainFrags {
  f16x8 w[4], t[2], k[4];
  float4 gl[2];
  typename std::conditional<NCT == 1, uint2, uint4>::type v;  // 4 NCT bf16 of the value tile
  uint32_t touch;
};
struct OutFrags {
  f16x8 q[4], m[2];
};

__device__ __forceinline__ void unpack_bf16(uint2 x, f16* o) {
  o[0] = (f16)__uint_as_float(x.x << 16);
  o[1] = (f16)__uint_as_float(x.x & 0xFFFF0000u);
  o[2] = (f16)__uint_as_float(x.y << 16);
  o[3] = (f16)__uint_as_float(x.y & 0xFFFF0000u);
}

template <typename StT, int NCT>
__global__ __launch_bounds__(512) void recur_split_kernel(RecurParams p) {
  constexpr int VC = VT * NCT;       // value columns per workgroup
  constexpr int NW = NVT / NCT;      // workgroups per chain
  constexpr int T_REC = (REC_LINES + NW - 1) / NW;  // record lines touched per workgroup
  constexpr int T_V = 2 * CH / NW;                 // value-row lines touched per workgroup
  static_assert(T_REC + T_V <= 256, "one touch per chain thread");
  __shared__ __attribute__((aligned(16))) f16x8 sbuf[NCT][4 * 64];  // S slices (B operand)
  __shared__ __attribute__((aligned(16))) f16x4 ubuf[NCT][4 * 64];  // U tiles (C layout)
  __shared__ __attribute__((aligned(16))) f16 vsT[VC * VS];         // value tile, [column][token]

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int tw = wave & 3;
  const int x = blockIdx.x, xcd = x & 7, y = x >> 3;
  const int vt = y % NW, ch = (y / NW) * 8 + xcd;
  if (ch >= p.n_chains) return;
  const int n = p.order[ch / p.H], h = ch % p.H;
  const int4 sq = p.seqs[n];
  const int tok0 = sq.x, len = sq.y, chunk0 = sq.z;
  // never walk past the schedule, whatever cu_seqlens held
  const int nch = max(0, min((len + CH - 1) / CH, p.n_entries - chunk0));
  const int last = nch - 1;
  const int v0 = vt * VC;
  auto record = [&](int c) { return p.rec + ((size_t)(chunk0 + c) * p.H + h) * REC_BYTES; };

  if (wave < 4) {
    // ---- chain waves ---------------------------------------------------------
    // S[j][i]: column tile j, key tile 2 tw + i; lane (column l16, keys 4lg..4lg+3)
    const size_t sbase = ((size_t)n * p.H + h) * HD * HD + (size_t)(v0 + l16) * HD;
    f32x4 S[NCT][2];
#pragma unroll
    for (int j = 0; j < NCT; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int k0 = SUB * (2 * tw + i) + 4 * lg;
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
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        F.w[s2] = ldfrag(R, REC_WNEG, tw * 4 + s2, lane);
        F.k[s2] = ldfrag(R, REC_KBAR, (2 * tw + (s2 >> 1)) * 2 + (s2 & 1), lane);
      }
      F.t[0] = ldfrag(R, REC_TB, tw * 2, lane);
      F.t[1] = ldfrag(R, REC_TB, tw * 2 + (tw >= 2 ? 1 : 0), lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        F.gl[i] = *reinterpret_cast<const float4*>(R + REC_GL + 4 * (SUB * (2 * tw + i) + 4 * lg));
      // rows past the chunk's end are clamped here and zeroed at use
      const int Lc = min(CH, len - c * CH);
      F.v = *reinterpret_cast<const decltype(F.v)*>(vchain + (size_t)c * CH * vstride +
                                                      (size_t)min(tid >> 2, Lc - 1) * vstride);
      const int ct = min(c + PF_AHEAD, last);
      const uint32_t* tp;
      if (trec) {
        tp = reinterpret_cast<const uint32_t*>(record(ct) + (size_t)rec_line * LINE);
      } else {
        const int Lt = min(CH, len - ct * CH);
        tp = reinterpret_cast<const uint32_t*>(p.v + ((size_t)(tok0 + ct * CH + min(vrow, Lt - 1)) * p.H + h) * HD +
                                               vhalf * (LINE / 2));
      }
      F.touch = *tp;
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
          sbuf[j][tw * 64 + lane] = sb;
        }
        const int r = tid >> 2;
        f16 vh[4 * NCT];
        if constexpr (NCT == 1) {
          unpack_bf16(r < L ? F.v : make_uint2(0u, 0u), vh);
        } else {
          const uint4 vv = r < L ? F.v : make_uint4(0u, 0u, 0u, 0u);
          unpack_bf16(make_uint2(vv.x, vv.y), vh);
          unpack_bf16(make_uint2(vv.z, vv.w), vh + 4);
        }
#pragma unroll
        for (int e = 0; e < 4 * NCT; ++e) vsT[(4 * NCT * vq + e) * VS + r] = vh[e];
      }
      __syncthreads();  // A
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        f16x8 sB[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) sB[s2] = sbuf[j][s2 * 64 + lane];
        f32x4 U = zero4(), U2 = zero4();
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (s2 <= (tw >> 1)) {
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
        ubuf[j][tw * 64 + lane] =
            f16x4{(f16)(U[0] + U2[0]), (f16)(U[1] + U2[1]), (f16)(U[2] + U2[2]), (f16)(U[3] + U2[3])};
      }
      __syncthreads();  // B
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        f16x8 uB[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const f16x4 a = ubuf[j][(2 * s2) * 64 + lane], b = ubuf[j][(2 * s2 + 1) * 64 + lane];
          uB[s2] = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const f32x4 a = mma_f16(F.k[2 * i], uB[0],
                                  f32x4{F.gl[i].x * S[j][i][0], F.gl[i].y * S[j][i][1], F.gl[i].z * S[j][i][2],
                                        F.gl[i].w * S[j][i][3]});
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
          const int k0 = SUB * (2 * tw + i) + 4 * lg;
          StateIO<StT>::store(p.s1, sbase + (size_t)VT * j * HD + k0, S[j][i]);
        }
    }
    return;
  }

  // ---- output waves ----------------------------------------------------------
  const size_t row_step = (size_t)p.H * HD;
  uint16_t* orow = p.out + ((size_t)(tok0 + SUB * tw + 4 * lg) * p.H + h) * HD + v0 + l16;
  auto load = [&](OutFrags& F, int c) {
    const uint8_t* R = record(c);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) F.q[s2] = ldfrag(R, REC_QHAT, tw * 4 + s2, lane);
    F.m[0] = ldfrag(R, REC_M, tw * 2, lane);
    F.m[1] = ldfrag(R, REC_M, tw * 2 + (tw >= 2 ? 1 : 0), lane);
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
    }
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
      if (tw >= 2) O = mma_f16(F.m[1], uB[1], O);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = SUB * tw + 4 * lg + e;
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
}

namespace {
// workgroups for n_chains chains with `tiles` workgroups per chain
int grid_for(int n_chains, int tiles) { return ((n_chains + 7) / 8) * 8 * tiles; }
}  // namespace

int recur_grid(int n_chains) { return grid_for(n_chains, NVT); }

void launch_recur(const RecurParams& p, bool bf16_state, hipStream_t stream) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    cus = (hipGetDevice(&dev) == hipSuccess &&
           hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ? v : 256;
  }
  const int g = grid_for(p.n_chains, NVT);
  if (g <= cus) {  // one workgroup per CU: chain and output waves, one column tile each
    if (bf16_state) recur_split_kernel<uint16_t, 1><<<g, 512, 0, stream>>>(p);
    else recur_split_kernel<float, 1><<<g, 512, 0, stream>>>(p);
    return;
  }
  const int g2 = grid_for(p.n_chains, NVT / 2);
  if (g2 <= cus) {  // still one workgroup per CU with two column tiles each
    if (bf16_state) recur_split_kernel<uint16_t, 2><<<g2, 512, 0, stream>>>(p);
    else recur_split_kernel<float, 2><<<g2, 512, 0, stream>>>(p);
    return;
  }
  const bool deep = g <= 4 * cus;  // few chains: latency per chain matters most
  if (bf16_state) {
    if (deep) recur_kernel<uint16_t, 3><<<g, 256, 0, stream>>>(p);
    else recur_kernel<uint16_t, 2><<<g, 256, 0, stream>>>(p);
  } else {
    if (deep) recur_kernel<float, 3><<<g, 256, 0, stream>>>(p);
    else recur_kernel<float, 2><<<g, 256, 0, stream>>>(p);
  }
}

}  // namespace kda
