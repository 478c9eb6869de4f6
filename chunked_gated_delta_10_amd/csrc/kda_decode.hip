// kda_decode.hip -- one decode step for every (batch row, value head).
//
// With the state stored [V, K] (row v is the 128-float key vector s_v), one
// token advances each row independently:
//   s'_v = exp(g) . s_v                 (per key channel)
//   a_v  = kn . s'_v,   c_v = qn . s'_v  (one fused pass, two dot products)
//   u_v  = b (v_v - a_v)
//   o_v  = scale (c_v + u_v (qn . kn))   (since S_t^T qn = S'^T qn + (qn.kn) u)
//   s_v  = s'_v + u_v kn
// so the state streams through once: read 512 B, write 512 B per row.
// Decay-only linear attention drops the normalisation, b and the erase:
// u_v = v_v.
//
// Workgroup = one (batch row, head), 256 threads; a group of 16 lanes owns
// one state row per step (8 key channels per lane, two 16-byte accesses that
// each cover half a row contiguously across the 16 lanes),
// 16 rows are in flight per pass and each lane walks 8 rows.  All loads of a
// lane are issued before any arithmetic so 16 x 16-byte requests per lane
// are outstanding.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

// A lane holds key channels 4ks .. 4ks+3 and 64+4ks .. 64+4ks+3 of a row, so
// each 16-byte access instruction of 16 lanes covers 256 contiguous bytes.
template <typename StT>
struct RowIO;

template <>
struct RowIO<float> {
  __device__ static void load(const void* base, size_t row, int ks, float* x) {
    const float* r = reinterpret_cast<const float*>(base) + row;
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r + 4 * ks));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r + 64 + 4 * ks));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = a[j];
      x[4 + j] = b[j];
    }
  }
  __device__ static void store(void* base, size_t row, int ks, const float* x) {
    float* r = reinterpret_cast<float*>(base) + row;
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(r + 4 * ks));
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(r + 64 + 4 * ks));
  }
};

template <>
struct RowIO<uint16_t> {
  __device__ static void load(const void* base, size_t row, int ks, float* x) {
    const uint16_t* r = reinterpret_cast<const uint16_t*>(base) + row;
    const uint2 a = *reinterpret_cast<const uint2*>(r + 4 * ks);
    const uint2 b = *reinterpret_cast<const uint2*>(r + 64 + 4 * ks);
    unpack_bf16x8(make_uint4(a.x, a.y, b.x, b.y), x);
  }
  __device__ static void store(void* base, size_t row, int ks, const float* x) {
    uint16_t* r = reinterpret_cast<uint16_t*>(base) + row;
    uint2 a, b;
    a.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    a.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    b.x = (uint32_t)f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
    b.y = (uint32_t)f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
    *reinterpret_cast<uint2*>(r + 4 * ks) = a;
    *reinterpret_cast<uint2*>(r + 64 + 4 * ks) = b;
  }
};

// 8 bf16 values of a vector at this lane's channels
__device__ __forceinline__ void load_vec8(const uint16_t* base, int ks, float* x) {
  const uint2 a = *reinterpret_cast<const uint2*>(base + 4 * ks);
  const uint2 b = *reinterpret_cast<const uint2*>(base + 64 + 4 * ks);
  unpack_bf16x8(make_uint4(a.x, a.y, b.x, b.y), x);
}

}  // namespace

// DELTA = false: decay-only linear attention, s_v = exp(g) . s_v + v_v k with
// q and k as given (u_v = v_v: no erase, no write strength, no normalisation).
template <typename StT, bool PER_CHANNEL, bool DELTA>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  constexpr int ROWS = 8;  // rows per lane
  const int tid = threadIdx.x;
  const int ks = tid & 15;   // key slice: channels 4ks .. 4ks+3 and 64+4ks .. 64+4ks+3
  const int rg = tid >> 4;   // row group: rows rg + 16 i
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh - b * p.H;
  const int hq = h / (p.H / p.H_qk);
  const size_t sbase = (size_t)bh * HD * HD;

  float s[ROWS][8];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) RowIO<StT>::load(p.state, sbase + (size_t)(rg + 16 * i) * HD, ks, s[i]);

  float qv[8], kv[8], d[8];
  {
    const size_t qoff = ((size_t)b * p.H_qk + hq) * HD;
    load_vec8(p.q + qoff, ks, qv);
    load_vec8(p.k + qoff, ks, kv);
    const float a = __expf(p.A_log[h]);
    if (PER_CHANNEL) {
      float gr[8];
      load_vec8(p.g_raw + (size_t)bh * HD, ks, gr);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float g;
        gate_decay(gr[j], a, d[j], g);
      }
    } else {
      float dd, g;
      gate_decay(bf16_to_f32(p.g_raw[bh]), a, dd, g);
#pragma unroll
      for (int j = 0; j < 8; ++j) d[j] = dd;
    }
  }
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sq += qv[j] * qv[j];
    sk += kv[j] * kv[j];
  }
  sq = rowsum16(sq);
  sk = rowsum16(sk);
  const float rq = DELTA ? 1.f / sqrtf(sq + 1e-6f) : 1.f, rk = DELTA ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
  float qk = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    qv[j] *= rq;
    kv[j] *= rk;
    qk += qv[j] * kv[j];
  }
  qk = rowsum16(qk);
  const float beta = DELTA ? sigmoidf_(p.beta[bh]) : 1.f;
  float vrow[ROWS];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) vrow[i] = bf16_to_f32(p.v[(size_t)bh * HD + rg + 16 * i]);

#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    float a = 0.f, c = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s[i][j] *= d[j];
      a += kv[j] * s[i][j];
      c += qv[j] * s[i][j];
    }
    a = rowsum16(a);
    c = rowsum16(c);
    const float u = DELTA ? beta * (vrow[i] - a) : vrow[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[i][j] += u * kv[j];
    RowIO<StT>::store(p.state, sbase + (size_t)(rg + 16 * i) * HD, ks, s[i]);
    if (ks == 0) p.out[(size_t)bh * HD + rg + 16 * i] = f32_to_bf16(p.scale * (c + u * qk));
  }
}

namespace {
template <typename StT, bool DELTA>
void launch_decode_state(const DecodeParams& p, dim3 grid, bool per_channel, hipStream_t stream) {
  if (per_channel) decode_kernel<StT, true, DELTA><<<grid, 256, 0, stream>>>(p);
  else decode_kernel<StT, false, DELTA><<<grid, 256, 0, stream>>>(p);
}
}  // namespace

void launch_decode(const DecodeParams& p, int B, bool bf16_state, bool per_channel, bool delta, hipStream_t stream) {
  dim3 grid((unsigned)(B * p.H));
  if (bf16_state) {
    if (delta) launch_decode_state<uint16_t, true>(p, grid, per_channel, stream);
    else launch_decode_state<uint16_t, false>(p, grid, per_channel, stream);
  } else {
    if (delta) launch_decode_state<float, true>(p, grid, per_channel, stream);
    else launch_decode_state<float, false>(p, grid, per_channel, stream);
  }
}

}  // namespace kda
