// kda_fused.hip -- the chunked forward pass of KDA (per-channel gate, delta
// rule) as ONE persistent kernel, with the chunk records passed from
// producer to consumer workgroups through the L2 of the XCD they share
// instead of through HBM.
//
// Teams.  Workgroups are spread over the 8 XCDs by id (id mod 8), and the
// workgroups of an XCD form `tpx` teams.  A team owns a list of chains (a
// batch row or packed sequence, and a value head) and walks their 64-token
// chunks in order: item i of the team is one (chain, chunk).  A team has
//   - NCW consumer workgroups: consumer w keeps value columns
//     CVC w .. CVC w + CVC - 1 of the state S (fp32, in registers; CVC = 16
//     NCT) and runs the sequential recurrence over every item of the team;
//   - P producer workgroups: producer p computes the chunk-local job of items
//     p, p + P, p + 2P, ... (the same job as the chunk-local kernel, in
//     kda_chunk_job.h) and writes its record into ring slot i mod R (R = P).
// Records are written and read on one XCD, so they travel through its L2.
//
// Protocol (every flag is a 32-bit word in its own 128-byte line; flag
// stores and loads are device-scope, so they bypass the CU's L1; record
// loads bypass it too):
//   producer, item i:  wait until every consumer's progress >= i - R + 1
//                      (slot i mod R is free); compute the job into the slot;
//                      wait for its own stores to complete (s_waitcnt), barrier;
//                      ready[slot] = i + 1.
//   consumer, item i:  wait until ready[slot] == i + 1; read the record;
//                      after every wave of the workgroup has read it,
//                      progress = i + 1.
// A consumer waits for item i + 1 before it finishes item i (it reads the
// next record a phase ahead), so its progress can lag one item behind the
// item it waits for.
// Forward progress (R >= 2): let m be the smallest unproduced item.  Every
// earlier item is produced, so every consumer can finish items up to m - 2
// and wait at m - 1 with progress >= m - 1 >= m - R + 1, which frees slot
// m mod R; the producer of m has finished all its earlier items, so it can
// start m.  (With one slot the producer of m would wait for item m - 1 to be
// finished while the consumer waits for m: the layout never uses fewer than
// two.)  This needs every workgroup resident at once: the kernel is launched
// cooperatively.  Every wait is bounded (about 0.2 s); on a timeout the
// wave records an error bit in the workspace header and skips its later
// waits, so every wave still meets the same barriers and the grid drains.
// A workgroup that finds itself on an XCD other than its id says records an
// error the same way (the exchange relies on one L2).  tests/
// test_fused_protocol.py models the protocol on the CPU.
//
// Selected by KDA_PRECISE=1.  Measured on the dense workload (B=2, T=16384,
// H=16) it takes 0.79-0.82 ms against 0.52 ms for the two-kernel path: a
// consumer needs 1.8-2.2 us per chunk even with every record ready (its two
// barriers, LDS round trips and dependent matrix-core chains per chunk), and
// the producers' jobs run ~12 us each, so the sequential chain, not HBM,
// bounds it.  What it buys is precision (below).
//
// Precision of the state path: the records carry the low parts of Kbar^T and
// T diag(b) (x - fp16(x)) and U is split the same way, so
//   U   = (T diag(b))_hi V + (T diag(b))_lo V - W S
//   S' <- Diag(exp(Gamma_L)) S + Kbar_hi^T (U_hi + U_lo) + Kbar_lo^T U_hi
//   O   = scale * (Qhat S + M (U_hi + U_lo))
// (fp16 operands, fp32 accumulation).  With nearly parallel keys, strong
// writes and little decay the rows of U telescope within a chunk, and a
// single fp16 rounding of Kbar, T diag(b) or U is amplified into the state.
#include "kda_chunk_job.h"

namespace kda {

namespace {

constexpr int NCT = 1;             // 16-column value tiles per consumer workgroup
constexpr int NCW = 8 / NCT;       // consumer workgroups per team
constexpr int CVC = 16 * NCT;      // value columns per consumer
constexpr int FVS = CH + 8;   // row stride (fp16) of the transposed value tile
constexpr int FLAG_STRIDE = 32;  // ints: one flag per 128-byte line
constexpr int MAX_POLLS = 1 << 18;  // polls of about 1 us each: a wait gives up after ~0.3 s

constexpr int ERR_XCD = 1, ERR_CONSUMER_WAIT = 2, ERR_PRODUCER_WAIT = 4;

// LDS of a consumer workgroup (bytes)
constexpr int C_SBUF = 0;                            // S (fp16) slices [NCT tiles][4][64] f16x8
constexpr int C_UHI = C_SBUF + NCT * 4 * 64 * 16;    // U_hi [NCT][4][64] f16x4
constexpr int C_ULO = C_UHI + NCT * 4 * 64 * 8;      // U_lo
constexpr int C_VST = C_ULO + NCT * 4 * 64 * 8;      // value tile [CVC columns][FVS] fp16
constexpr int C_BYTES = C_VST + CVC * FVS * 2;
static_assert(C_BYTES <= LDS_BYTES, "consumer LDS fits in the producer's");

__device__ __forceinline__ int ld_flag(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void set_err(int* err, int bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Record reads: device-scope buffer loads (sc1), so a CU never serves them
// from a stale L1 line of the slot's previous record.
struct RecReader {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ RecReader(const uint8_t* base, int bytes) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
  }
  __device__ __forceinline__ f16x8 frag(int off, int frag_idx, int lane) const {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + frag_idx * FRAG_BYTES + lane * 16, 0, 16);
    return __builtin_bit_cast(f16x8, v);
  }
  __device__ __forceinline__ void row(int off, uint2& x) const {
    x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, off, 0, 16));
  }
  __device__ __forceinline__ void row(int off, uint4& x) const {
    x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 16));
  }
  __device__ __forceinline__ uint4 u4(int off) const {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 16);
    return __builtin_bit_cast(uint4, v);
  }
  __device__ __forceinline__ float4 f4(int off) const {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 16);
    return __builtin_bit_cast(float4, v);
  }
};

template <typename StT>
struct FStateIO;
template <>
struct FStateIO<float> {
  __device__ static f32x4 load(const void* base, size_t off) {
    const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    return f32x4{x.x, x.y, x.z, x.w};
  }
  __device__ static void store(void* base, size_t off, f32x4 v) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct FStateIO<uint16_t> {  // bf16 state: converted on load and on store only
  __device__ static f32x4 load(const void* base, size_t off) {
    const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
    return f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u), __uint_as_float(x.y << 16),
                 __uint_as_float(x.y & 0xFFFF0000u)};
  }
  __device__ static void store(void* base, size_t off, f32x4 v) {
    uint2 x;
    x.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    x.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + off) = x;
  }
};

// One chain of a team: sequence, head, first token, length, chunks.
struct Chain {
  int seq, h, tok0, len, nch;
};

__device__ __forceinline__ Chain chain_at(const FusedParams& p, int pos) {
  Chain c;
  c.h = pos % p.cp.H;
  if (p.dense_T >= 0) {
    c.seq = pos / p.cp.H;
    c.tok0 = c.seq * p.dense_T;
    c.len = p.dense_T;
  } else {
    c.seq = p.order[pos / p.cp.H];
    const int4 sq = p.seqs[c.seq];
    c.tok0 = sq.x;
    c.len = max(0, sq.y);
  }
  c.nch = (c.len + CH - 1) / CH;
  return c;
}

// Walks the items (chain, chunk) of one team in order, skipping empty chains.
struct ItemIter {
  int pos, j;  // chain position (team, team + n_teams, ...) and chunk within it
  Chain c;
  int valid;  // an int, not a bool: a struct copy then has no padding bytes to carry
  __device__ void settle(const FusedParams& p) {
    while (pos < p.n_chains) {
      c = chain_at(p, pos);
      if (j < c.nch) {
        valid = 1;
        return;
      }
      j -= c.nch;
      pos += p.n_teams;
    }
    valid = 0;
  }
  __device__ void begin(const FusedParams& p, int team, int skip) {
    pos = team;
    j = skip;
    settle(p);
  }
  __device__ void advance(const FusedParams& p, int by) {
    j += by;
    settle(p);
  }
};

__device__ __forceinline__ void unpack_bf16x4_to_f16(uint32_t a, uint32_t b, f16* o) {
  o[0] = (f16)__uint_as_float(a << 16);
  o[1] = (f16)__uint_as_float(a & 0xFFFF0000u);
  o[2] = (f16)__uint_as_float(b << 16);
  o[3] = (f16)__uint_as_float(b & 0xFFFF0000u);
}
// bf16 value-row entries to fp16 (zero for rows past the chunk's end)
__device__ __forceinline__ void unpack_row(uint2 v, bool live, f16* o) {
  unpack_bf16x4_to_f16(live ? v.x : 0u, live ? v.y : 0u, o);
}
__device__ __forceinline__ void unpack_row(uint4 v, bool live, f16* o) {
  unpack_bf16x4_to_f16(live ? v.x : 0u, live ? v.y : 0u, o);
  unpack_bf16x4_to_f16(live ? v.z : 0u, live ? v.w : 0u, o + 4);
}

// ---------------------------------------------------------------------------
// Producer role: the chunk-local jobs of items p, p + P, ... of the team.
// ---------------------------------------------------------------------------
__device__ void producer_role(const FusedParams& p, uint8_t* smem, int team, int prod, int P) {
  const int tid = threadIdx.x;
  uint8_t* ring = p.ring + (size_t)team * p.R * REC2_BYTES;
  int* ready = p.ready + (size_t)team * p.R * FLAG_STRIDE;
  const int* prog = p.prog + (size_t)team * NCW * FLAG_STRIDE;
  ItemIter it;
  it.begin(p, team, prod);
  // A timed-out wait records an error and makes every later wait of this
  // wave a no-op: the workgroup keeps executing the same barriers in every
  // wave and finishes (with garbage) in bounded time.
  bool dead = false;
  for (int i = prod; it.valid; i += P) {
    const int slot = i % p.R;
    if (i >= p.R && !dead) {  // slot free once every consumer has finished item i - R
      const int need = i - p.R + 1;
      int polls = 0;
      for (;;) {
        int lo = ld_flag(prog);
#pragma unroll
        for (int w = 1; w < NCW; ++w) lo = min(lo, ld_flag(prog + w * FLAG_STRIDE));
        if (__builtin_amdgcn_readfirstlane(lo) >= need) break;
        if (++polls > MAX_POLLS) {
          if ((tid & 63) == 0) set_err(p.err, ERR_PRODUCER_WAIT);
          dead = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    const int4 ce = make_int4(it.c.seq, it.c.tok0 + it.j * CH, min(CH, it.c.len - it.j * CH), it.j);
    chunk_job<true, true, true>(p.cp, smem, ce, it.c.h, ring + (size_t)slot * REC2_BYTES);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's record stores have reached the L2
    __syncthreads();                // ... and every wave's; the job's LDS is free again
    if (tid == 0) st_flag(ready + slot * FLAG_STRIDE, i + 1);
    it.advance(p, P);
  }
}

// ---------------------------------------------------------------------------
// Consumer role: value columns c0 .. c0 + CVC - 1 of every chain of the team.
// Four waves; wave TW owns token tile TW of U and O and key tiles 2TW, 2TW+1
// of S.  The fragments of an item are read in two halves, each into one
// register set and one phase ahead of its use: the U half (W, T diag(b)
// hi/lo, Qhat) of item i+1 once item i's U half is consumed, the S half
// (Kbar^T hi/lo, M, exp(Gamma_L)) of item i+1 once item i's S half is.  The
// ready flag of item i+1 is polled at the top of item i.  The value rows come
// with the record (the producer copies them), so every load a consumer waits
// on is an L2 hit: a wait for a flag waits for every earlier load (loads
// complete in issue order), and an HBM load in flight would hold it up.
// ---------------------------------------------------------------------------
// this thread's 4 NCT value-row entries (bf16)
using VRow = typename std::conditional<NCT == 1, uint2, uint4>::type;
struct UFrags {
  f16x8 w[4], t[2], tl[2], q[4];
  VRow v;
};
struct SFrags {
  f16x8 k[4], kl[4], m[2];
  float4 g[2];
};

template <typename StT>
__device__ void consumer_role(const FusedParams& p, uint8_t* smem, int team, int cw) {
  f16x8* sbuf = reinterpret_cast<f16x8*>(smem + C_SBUF);
  f16x4* uhi = reinterpret_cast<f16x4*>(smem + C_UHI);
  f16x4* ulo = reinterpret_cast<f16x4*>(smem + C_ULO);
  f16* vsT = reinterpret_cast<f16*>(smem + C_VST);
  const int tid = threadIdx.x, lane = tid & 63, TW = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int c0 = CVC * cw;
  const int H = p.cp.H;
  const size_t row_step = (size_t)H * HD;
  const uint8_t* ring = p.ring + (size_t)team * p.R * REC2_BYTES;
  const int* ready = p.ready + (size_t)team * p.R * FLAG_STRIDE;
  int* my_prog = p.prog + ((size_t)team * NCW + cw) * FLAG_STRIDE;
  const int vr = tid >> 2, vq = tid & 3;  // value-row loader: token row vr, columns c0 + 4 NCT vq ..

  // A timed-out wait records an error and makes every later wait of this
  // wave a no-op, so all waves keep meeting at the same barriers and the
  // workgroup finishes (with garbage) in bounded time.
  bool dead = false;
  auto wait_ready = [&](int i) {
    const int* f = ready + (i % p.R) * FLAG_STRIDE;
    int polls = 0;
    while (!dead && __builtin_amdgcn_readfirstlane(ld_flag(f)) != i + 1) {
      if (++polls > MAX_POLLS) {
        if (lane == 0) set_err(p.err, ERR_CONSUMER_WAIT);
        dead = true;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  };
  auto load_u = [&](UFrags& F, int i) {
    const RecReader R(ring + (size_t)(i % p.R) * REC2_BYTES, REC2_BYTES);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      F.w[s2] = R.frag(REC_WNEG, TW * 4 + s2, lane);
      F.q[s2] = R.frag(REC_QHAT, TW * 4 + s2, lane);
    }
    const int t1 = TW * 2 + (TW >= 2 ? 1 : 0);
    F.t[0] = R.frag(REC_TB, TW * 2, lane);
    F.t[1] = R.frag(REC_TB, t1, lane);
    F.tl[0] = R.frag(REC_TB_LO, TW * 2, lane);
    F.tl[1] = R.frag(REC_TB_LO, t1, lane);
    R.row(REC_V + vr * (HD * 2) + (c0 + 4 * NCT * vq) * 2, F.v);
  };
  auto load_s = [&](SFrags& F, int i) {
    const RecReader R(ring + (size_t)(i % p.R) * REC2_BYTES, REC2_BYTES);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int f = (2 * TW + (s2 >> 1)) * 2 + (s2 & 1);
      F.k[s2] = R.frag(REC_KBAR, f, lane);
      F.kl[s2] = R.frag(REC_KBAR_LO, f, lane);
    }
    F.m[0] = R.frag(REC_M, TW * 2, lane);
    F.m[1] = R.frag(REC_M, TW * 2 + (TW >= 2 ? 1 : 0), lane);
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) F.g[i2] = R.f4(REC_GL + 4 * (SUB * (2 * TW + i2) + 4 * lg));
  };
  // Empty chains pass their state through (or write zero when there is none).
  auto pass_through = [&](int pos_from, int pos_to) {
    for (int pos = pos_from; pos < pos_to; pos += p.n_teams) {
      const Chain c = chain_at(p, pos);
      if (c.nch != 0 || !p.s1) continue;
      const size_t sb = ((size_t)c.seq * H + c.h) * HD * HD + (size_t)(c0 + l16) * HD;
#pragma unroll
      for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const size_t off = sb + (size_t)16 * j * HD + SUB * (2 * TW + i2) + 4 * lg;
          FStateIO<StT>::store(p.s1, off, p.s0 ? FStateIO<StT>::load(p.s0, off) : zero4());
        }
    }
  };

  ItemIter cur;
  cur.begin(p, team, 0);
  pass_through(team, cur.valid ? cur.pos : p.n_chains);
  UFrags fu;
  SFrags fs;
  if (cur.valid) {
    wait_ready(0);
    load_u(fu, 0);
    load_s(fs, 0);
  }
  f32x4 S[NCT][2];
  for (int i = 0; cur.valid; ++i) {
    const Chain c = cur.c;
    const int L = min(CH, c.len - cur.j * CH);
    const size_t sbase = ((size_t)c.seq * H + c.h) * HD * HD + (size_t)(c0 + l16) * HD;
    ItemIter nxt = cur;
    nxt.advance(p, 1);
    if (nxt.valid) wait_ready(i + 1);   // the loads of item i + 1 are issued below
    if (cur.j == 0) {  // chain start: the initial state (or zero)
#pragma unroll
      for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
          S[j][i2] = p.s0 ? FStateIO<StT>::load(p.s0, sbase + (size_t)16 * j * HD + SUB * (2 * TW + i2) + 4 * lg)
                          : zero4();
    }
    // ---- publish S (fp16) and the value tile -----------------------------------
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      f16x8 sb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sb[e] = (f16)S[j][0][e];
        sb[4 + e] = (f16)S[j][1][e];
      }
      sbuf[j * 256 + TW * 64 + lane] = sb;
    }
    {
      f16 vh[4 * NCT];
      unpack_row(fu.v, vr < L, vh);
#pragma unroll
      for (int e = 0; e < 4 * NCT; ++e) vsT[(4 * NCT * vq + e) * FVS + vr] = vh[e];
    }
    __syncthreads();  // A: S slices and value tile visible; every wave is done with item i - 1
    if (i > 0 && tid == 0) st_flag(my_prog, i);  // item i - 1 fully read by this workgroup

    // ---- U = T diag(b) V - W S (hi + lo T), and Qhat S -------------------------
    f32x4 OQ[NCT];
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      f16x8 sB[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) sB[s2] = sbuf[j * 256 + s2 * 64 + lane];
      f32x4 U = zero4(), U2 = zero4();
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        if (s2 <= (TW >> 1)) {
          const f16* vp = &vsT[(16 * j + l16) * FVS + 32 * s2 + 4 * lg];
          const f16x4 a = *reinterpret_cast<const f16x4*>(vp);
          const f16x4 b = *reinterpret_cast<const f16x4*>(vp + 16);
          const f16x8 vb = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
          U2 = mma_f16(fu.tl[s2], vb, U2);
          U = mma_f16(fu.t[s2], vb, U);
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        if (s2 & 1) U2 = mma_f16(fu.w[s2], sB[s2], U2);
        else U = mma_f16(fu.w[s2], sB[s2], U);
      }
      f32x4 qa = zero4(), qb = zero4();
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        if (s2 & 1) qb = mma_f16(fu.q[s2], sB[s2], qb);
        else qa = mma_f16(fu.q[s2], sB[s2], qa);
      }
      OQ[j] = qa + qb;
      const f32x4 Us = U + U2;
      f16x4 h4, l4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h4[e] = (f16)Us[e];
        l4[e] = (f16)(Us[e] - (float)h4[e]);
      }
      uhi[j * 256 + TW * 64 + lane] = h4;
      ulo[j * 256 + TW * 64 + lane] = l4;
    }
    if (nxt.valid) load_u(fu, i + 1);  // item i's U half is consumed
    __syncthreads();  // B: U visible

    // ---- O = scale (Qhat S + M U);  S <- Diag(exp(Gamma_L)) S + Kbar^T U ---------
    uint16_t* orow = p.out + ((size_t)(c.tok0 + cur.j * CH + SUB * TW + 4 * lg) * H + c.h) * HD + c0 + l16;
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      f16x8 uH[2], uL[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const f16x4 a = uhi[j * 256 + (2 * s2) * 64 + lane], b = uhi[j * 256 + (2 * s2 + 1) * 64 + lane];
        const f16x4 x = ulo[j * 256 + (2 * s2) * 64 + lane], y = ulo[j * 256 + (2 * s2 + 1) * 64 + lane];
        uH[s2] = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        uL[s2] = f16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
      }
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const float4 d = fs.g[i2];
        f32x4 small = mma_f16(fs.kl[2 * i2], uH[0], zero4());
        small = mma_f16(fs.kl[2 * i2 + 1], uH[1], small);
        small = mma_f16(fs.k[2 * i2], uL[0], small);
        small = mma_f16(fs.k[2 * i2 + 1], uL[1], small);
        f32x4 a = mma_f16(fs.k[2 * i2], uH[0], f32x4{d.x * S[j][i2][0], d.y * S[j][i2][1], d.z * S[j][i2][2],
                                                     d.w * S[j][i2][3]});
        a = mma_f16(fs.k[2 * i2 + 1], uH[1], a);
        S[j][i2] = a + small;
      }
      f32x4 O = mma_f16(fs.m[0], uL[0], OQ[j]);
      O = mma_f16(fs.m[0], uH[0], O);
      if (TW >= 2) {
        O = mma_f16(fs.m[1], uL[1], O);
        O = mma_f16(fs.m[1], uH[1], O);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = SUB * TW + 4 * lg + e;
        uint16_t* dst = r < L ? orow + (size_t)e * row_step + 16 * j : p.sink + lane;
        *dst = f32_to_bf16(p.scale * O[e]);
      }
    }
    if (nxt.valid) load_s(fs, i + 1);  // item i's S half is consumed
    if (cur.j == c.nch - 1 && p.s1) {  // chain end: the final state
#pragma unroll
      for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
          FStateIO<StT>::store(p.s1, sbase + (size_t)16 * j * HD + SUB * (2 * TW + i2) + 4 * lg, S[j][i2]);
    }
    const int pos_before = cur.pos;
    cur = nxt;
    pass_through(pos_before + p.n_teams, cur.valid ? cur.pos : p.n_chains);
    if (!cur.valid) {
      __syncthreads();  // every wave has read the last item
      if (tid == 0) st_flag(my_prog, i + 1);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Zeroes the flags and the error word of a fused launch (one workgroup).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fused_prep_kernel(int* flags, int n_flags, int* err) {
  for (int i = threadIdx.x; i < n_flags; i += 256) flags[i] = 0;
  if (threadIdx.x == 0) *err = 0;
}

template <typename StT>
__global__ __launch_bounds__(256, 2) void fused_kernel(FusedParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int x = blockIdx.x, xcd = x & 7, y = x >> 3;
  if (__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) != xcd) {  // hwreg(HW_REG_XCC_ID, 0, 4)
    if (threadIdx.x == 0) set_err(p.err, ERR_XCD);
  }
  // Consumers take the first `cons` local slots of the XCD.  Workgroups are
  // dispatched one per CU before any CU gets a second (local slots y and
  // y + 32 share a CU as placed on the hardware), so with cons <= 32 every
  // consumer shares its CU with a producer, never with another consumer
  // (two consumers on one CU were measured 15% slower).
  const int cons = p.tpx * NCW;  // consumer workgroups per XCD
  if (y < cons) {
    const int team = xcd + 8 * (y / NCW);
    consumer_role<StT>(p, smem, team, y % NCW);
    return;
  }
  const int pi = y - cons;
  const int P = p.P;
  if (pi >= p.tpx * P) return;  // no team for it
  producer_role(p, smem, xcd + 8 * (pi / P), pi % P, P);
}

namespace {
std::atomic<int> g_fused_state[MAX_DEVICES];  // 0 unknown, 1 available, 2 unavailable

template <typename StT>
hipError_t set_fused_attr() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_kernel<StT>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
}
}  // namespace

FusedLayout fused_layout(int n_chains) {
  FusedLayout L;
  const int cus = device_cu_count();
  L.grid = 2 * cus;
  const int wpx = L.grid / 8;  // workgroups per XCD
  L.tpx = max(1, min(4, (n_chains + 7) / 8));
  L.P = (wpx - L.tpx * NCW) / L.tpx;  // producers per team (>= 2 wherever the path is taken)
  L.R = L.P;                           // ring slots per team
  L.n_teams = 8 * L.tpx;
  L.ring_bytes = (size_t)L.n_teams * L.R * REC2_BYTES;
  L.n_flags = L.n_teams * (L.R + NCW) * FLAG_STRIDE;
  return L;
}

bool fused_available() {
  const int d = current_device();
  int st = g_fused_state[d].load(std::memory_order_acquire);
  if (st == 0) {
    int coop = 0, occ32 = 0, occ16 = 0;
    const int cus = device_cu_count();
    // 2 workgroups per CU; four teams of NCW consumers per XCD and at least
    // two producers (ring slots) per team need 2 cus / 8 >= 4 (NCW + 2).
    bool okay = cus % 8 == 0 && 2 * cus / 8 >= 4 * (NCW + 2) &&
                hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, d) == hipSuccess && coop &&
                set_fused_attr<float>() == hipSuccess && set_fused_attr<uint16_t>() == hipSuccess &&
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ32, fused_kernel<float>, 256, LDS_BYTES) ==
                    hipSuccess &&
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ16, fused_kernel<uint16_t>, 256, LDS_BYTES) ==
                    hipSuccess &&
                occ32 >= 2 && occ16 >= 2;
    (void)hipGetLastError();
    st = okay ? 1 : 2;
    g_fused_state[d].store(st, std::memory_order_release);
  }
  return st == 1;
}

hipError_t launch_fused(const FusedParams& p, int grid, bool bf16_state, hipStream_t stream) {
  fused_prep_kernel<<<1, 256, 0, stream>>>(p.ready, p.n_flags_total, p.err);
  void* args[] = {const_cast<FusedParams*>(&p)};
  const void* f = bf16_state ? reinterpret_cast<const void*>(&fused_kernel<uint16_t>)
                             : reinterpret_cast<const void*>(&fused_kernel<float>);
  return hipLaunchCooperativeKernel(f, dim3(grid), dim3(256), args, LDS_BYTES, stream);
}

}  // namespace kda
