// kda_api.hip -- the C ABI of libkda.so (declared in include/kda.h).
//
// Host side only: argument validation (before anything touches the device),
// workspace layout, and the launch sequence
//   schedule (kda_table) -> chunk-local (kda_chunk) -> recurrence (kda_recur)
// for the chunked forward pass, and the single decode kernel for decode.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_bwd.h"
#include "kda_device.h"
#include "kda_kernels.h"

// Scratch of kda_fwd_noalloc (file scope, one copy per device).
static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kda_status ok() {
  g_last_error.clear();
  return KDA_OK;
}

bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] == '1';
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t ALIGN = 256;
size_t round_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
  size_t seqs, chunks, order, sink, rec, flags, total;
  bool fused;
  kda::FusedLayout F;
};

int cdiv(long a, long b);

// Workspace: a 256-byte header (word 0: the error bits of the last forward
// call), the schedule (sequence table, chunk table, order), a small sink for
// output rows past a chunk's end, then either the chunk records of every
// (chunk, head) (two-kernel path) or the fused kernel's record rings and
// flags.
Layout layout(int n_seqs, int n_entries, int H, bool fused) {
  Layout L;
  L.fused = fused;
  L.seqs = ALIGN;
  L.chunks = L.seqs + round_up((size_t)n_seqs * sizeof(int4));
  L.order = L.chunks + round_up((size_t)n_entries * sizeof(int4));
  L.sink = L.order + round_up((size_t)n_seqs * sizeof(int));
  L.rec = L.sink + round_up(64 * sizeof(uint16_t));
  if (fused) {
    L.F = kda::fused_layout(n_seqs * H);
    L.flags = L.rec + round_up(L.F.ring_bytes);
    L.total = L.flags + round_up((size_t)L.F.n_flags * sizeof(int));
  } else {
    L.flags = 0;
    L.total = L.rec + round_up((size_t)n_entries * H * kda::REC_BYTES);
  }
  return L;
}

int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// KDA_PRECISE=1 selects the fused persistent kernel for the per-channel
// delta-rule forward (split-precision state path; see include/kda.h) when
// the device supports it; otherwise the two-kernel path runs.
bool takes_fused(bool delta, int gate_per_channel) {
  return delta && gate_per_channel == 1 && env_flag("KDA_PRECISE") && kda::fused_available();
}

// ---- per-kernel event timing (diagnostics) --------------------------------
enum {
  K_TABLE = 0, K_CHUNK = 1, K_RECUR = 2, K_DECODE = 3, K_FUSED = 4, K_BWD_COEF = 5, K_BWD_CHAINS = 6, K_BWD_GRAD = 7,
  K_COUNT = 8
};
const char* const kKernelNames[K_COUNT] = {"kda_table", "kda_chunk_local", "kda_recur",      "kda_decode",
                                           "kda_fused", "kda_bwd_coef",    "kda_bwd_chains", "kda_bwd_grad"};

struct Timing {
  bool on = false;
  struct Rec { int id; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local Timing g_timing;

// Brackets one launch with events when timing is on.
struct Timed {
  int id;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  Timed(int id_, hipStream_t s_, bool allowed = true) : id(id_), s(s_) {
    if (!g_timing.on || !allowed) return;
    a = g_timing.get();
    b = g_timing.get();
    if (a && b) (void)hipEventRecord(a, s);
  }
  ~Timed() {
    if (!a || !b) return;
    (void)hipEventRecord(b, s);
    g_timing.pending.push_back({id, a, b});
  }
};

kda_status check_state_dtypes(const void* init, kda_state_dtype idt, const void* fin, kda_state_dtype fdt,
                               bool* bf16) {
  auto valid = [](kda_state_dtype d) { return d == KDA_STATE_BF16 || d == KDA_STATE_FP32; };
  if (init && !valid(idt)) return fail(KDA_ERR_DTYPE, "initial_state dtype %d is not bf16 (1) or fp32 (2)", (int)idt);
  if (fin && !valid(fdt)) return fail(KDA_ERR_DTYPE, "final_state dtype %d is not bf16 (1) or fp32 (2)", (int)fdt);
  if (init && fin && idt != fdt)
    return fail(KDA_ERR_STATE_DTYPE_MISMATCH, "initial_state and final_state dtypes differ (%d vs %d)", (int)idt,
                (int)fdt);
  *bf16 = (init ? idt : fdt) == KDA_STATE_BF16;
  return KDA_OK;
}

struct FwdArgs {
  const void *q, *k, *v, *g_raw;
  const float *beta, *A_log;
  float scale;
  int gate_per_channel;
  const void* s0;
  kda_state_dtype s0_dt;
  void* out;
  void* s1;
  kda_state_dtype s1_dt;
  const int32_t* cu;  // null for dense
  int n_seqs;         // B (dense) or N (packed)
  int T;              // tokens per row (dense) or total tokens
  int rows;           // B for dense, 1 for packed
  int H_qk, H, K, V;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  bool delta;         // false: decay-only linear attention (beta unused)
  bool noalloc = false;  // the allocation-free entry point: the workspace is the static scratch array
};

kda_status validate_common(const FwdArgs& a) {
  if (a.n_seqs < 0 || a.T < 0 || a.H_qk <= 0 || a.H <= 0)
    return fail(KDA_ERR_SHAPE, "sizes must be non-negative with H, H_qk > 0 (got seqs=%d T=%d H_qk=%d H=%d)",
                a.n_seqs, a.T, a.H_qk, a.H);
  if (a.K != kda::HD || a.V != kda::HD)
    return fail(KDA_ERR_SHAPE, "only K = V = 128 is supported (got K=%d V=%d)", a.K, a.V);
  if (a.H % a.H_qk != 0) return fail(KDA_ERR_SHAPE, "H (%d) must be a multiple of H_qk (%d)", a.H, a.H_qk);
  if (a.gate_per_channel != 0 && a.gate_per_channel != 1)
    return fail(KDA_ERR_SHAPE, "gate_per_channel must be 0 or 1 (got %d)", a.gate_per_channel);
  if ((long)a.rows * a.T >= (1L << 31) || (long)a.n_seqs * a.H >= (1L << 31))
    return fail(KDA_ERR_SHAPE, "problem too large (tokens and sequences x heads must fit in int32)");
  return KDA_OK;
}

struct FwdPlan {
  bool bf16_state = false;
  int n_entries = 0;
  Layout L{};
};

// Host-only validation of a forward call (no device access).  KDA_OK with
// plan->n_entries < 0 means a successful no-op (no sequences).
kda_status validate_forward(const FwdArgs& a, FwdPlan* plan = nullptr) {
  FwdPlan local;
  FwdPlan& P = plan ? *plan : local;
  P.n_entries = -1;
  kda_status st = validate_common(a);
  if (st != KDA_OK) return st;
  st = check_state_dtypes(a.s0, a.s0_dt, a.s1, a.s1_dt, &P.bf16_state);
  if (st != KDA_OK) return st;
  if (a.n_seqs == 0) return ok();
  const long tokens = (long)a.rows * a.T;
  if (tokens > 0) {
    const void* req[] = {a.q, a.k, a.v, a.g_raw, a.A_log, a.out, a.beta};
    const char* names[] = {"q", "k", "v", "g_raw", "A_log", "out", "beta_logits"};
    const int n_req = a.delta ? 7 : 6;
    for (int i = 0; i < n_req; ++i)
      if (!req[i]) return fail(KDA_ERR_NULL, "%s is NULL", names[i]);
    for (int i = 0; i < n_req; ++i)
      if (!aligned16(req[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  if (a.s0 && !aligned16(a.s0)) return fail(KDA_ERR_ALIGN, "initial_state is not 16-byte aligned");
  if (a.s1 && !aligned16(a.s1)) return fail(KDA_ERR_ALIGN, "final_state is not 16-byte aligned");
  if (a.cu && (reinterpret_cast<uintptr_t>(a.cu) & 3u)) return fail(KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
  const int n_entries = a.cu ? cdiv(a.T, kda::CH) + a.n_seqs : a.n_seqs * cdiv(a.T, kda::CH);
  if ((long)n_entries * a.H >= (1L << 31))
    return fail(KDA_ERR_SHAPE, "problem too large (chunks x heads must fit in int32)");
  const Layout L = layout(a.n_seqs, n_entries, a.H, takes_fused(a.delta, a.gate_per_channel));
  if (a.noalloc && L.total > KDA_NOALLOC_SCRATCH_BYTES)
    return fail(KDA_ERR_WORKSPACE,
                "kda_fwd_noalloc: these sizes need %zu bytes of scratch, the static scratch array holds %zu "
                "(the two-kernel path keeps about %d (chunk, head) records); call kda_fwd with a workspace instead",
                L.total, (size_t)KDA_NOALLOC_SCRATCH_BYTES, (int)(KDA_NOALLOC_SCRATCH_BYTES / kda::REC_BYTES) - 1);
  if (!a.ws) return fail(KDA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
  if (a.ws_bytes < L.total)
    return fail(KDA_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", a.ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(a.ws) & (ALIGN - 1)) return fail(KDA_ERR_ALIGN, "workspace is not 256-byte aligned");
  P.n_entries = n_entries;
  P.L = L;
  return ok();
}

kda_status run_forward(const FwdArgs& a) {
  FwdPlan P;
  kda_status st = validate_forward(a, &P);
  if (st != KDA_OK || P.n_entries < 0) return st;
  const bool bf16_state = P.bf16_state;
  const int n_entries = P.n_entries;
  const Layout L = P.L;
  const long tokens = (long)a.rows * a.T;

  if (a.cu && env_flag("KDA_DEBUG")) {
    std::vector<int32_t> h(a.n_seqs + 1);
    if (hipMemcpyAsync(h.data(), a.cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, a.stream) != hipSuccess ||
        hipStreamSynchronize(a.stream) != hipSuccess)
      return fail(KDA_ERR_HIP, "KDA_DEBUG: could not read cu_seqlens: %s", hipGetErrorString(hipGetLastError()));
    if (h[0] != 0) return fail(KDA_ERR_SHAPE, "KDA_DEBUG: cu_seqlens[0] = %d, expected 0", h[0]);
    for (int n = 0; n < a.n_seqs; ++n)
      if (h[n + 1] < h[n]) return fail(KDA_ERR_SHAPE, "KDA_DEBUG: cu_seqlens decreases at %d", n);
    if (h[a.n_seqs] != a.T) return fail(KDA_ERR_SHAPE, "KDA_DEBUG: cu_seqlens[N] = %d, expected T = %d", h[a.n_seqs], a.T);
  }

  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  int4* seqs = reinterpret_cast<int4*>(ws + L.seqs);
  int4* chunks = reinterpret_cast<int4*>(ws + L.chunks);
  int* order = reinterpret_cast<int*>(ws + L.order);

  (void)hipGetLastError();  // clear any stale error before launching
  // Packed sequences need the device schedule (sequence starts, chunk entries,
  // longest-first order) built from cu_seqlens; B rows of T tokens do not:
  // the kernels derive their schedule arithmetically.
  if (a.cu) {
    kda::TableParams tp{a.cu, a.n_seqs, a.T, n_entries, seqs, chunks, order};
    Timed t(K_TABLE, a.stream, !a.noalloc);
    kda::launch_table(tp, a.stream);
  }
  const kda::ChunkParams cp{static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                            static_cast<const uint16_t*>(a.g_raw), a.beta, a.A_log, chunks, a.H, a.H_qk,
                            L.fused ? nullptr : ws + L.rec, a.cu ? 0 : a.T, static_cast<const uint16_t*>(a.v)};
  int* err = reinterpret_cast<int*>(ws);
  uint16_t* sink = reinterpret_cast<uint16_t*>(ws + L.sink);
  if (L.fused) {
    int* flags = reinterpret_cast<int*>(ws + L.flags);
    const kda::FusedParams fp{cp, static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.out), a.s0, a.s1,
                              a.scale, seqs, order, a.cu ? -1 : a.T, a.n_seqs * a.H, L.F.n_teams, L.F.tpx, L.F.R, L.F.P,
                              ws + L.rec, flags, flags + (size_t)L.F.n_teams * L.F.R * 32, L.F.n_flags, err, sink};
    Timed t(K_FUSED, a.stream, !a.noalloc);
    const hipError_t e = kda::launch_fused(fp, L.F.grid, bf16_state, a.stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "fused kernel launch failed: %s", hipGetErrorString(e));
  } else {
    if (n_entries > 0 && tokens > 0) {
      Timed t(K_CHUNK, a.stream, !a.noalloc);
      const hipError_t e = kda::launch_chunk_local(cp, n_entries, a.gate_per_channel == 1, a.delta, a.stream);
      if (e != hipSuccess) return fail(KDA_ERR_HIP, "kernel setup failed: %s", hipGetErrorString(e));
    }
    kda::RecurParams rp{ws + L.rec, seqs, order, a.n_seqs * a.H, n_entries, a.H, a.H_qk,
                        static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.out), a.s0, a.s1, a.scale, sink,
                        a.cu ? -1 : a.T, err};
    Timed t(K_RECUR, a.stream, !a.noalloc);
    kda::launch_recur(rp, bf16_state, a.gate_per_channel == 1, a.delta, a.stream);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  if (env_flag("KDA_LOG"))
    std::fprintf(stderr, "[kda] fwd seqs=%d T=%d H=%d H_qk=%d entries=%d path=%s state=%s\n", a.n_seqs, a.T, a.H,
                 a.H_qk, n_entries, L.fused ? "fused" : "split", bf16_state ? "bf16" : "fp32");
  return ok();
}

// ---- static scratch of the allocation-free entry point ---------------------
// One copy per device, held until the process ends.  Host code never uses
// the array's name as an address: the per-device address comes from
// hipGetSymbolAddress, called once per device with that device current.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kda::MAX_DEVICES];

kda_status scratch_address(void** out) {
  int dev = 0;
  const hipError_t e0 = hipGetDevice(&dev);
  if (e0 != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e0));
  if (dev < 0 || dev >= kda::MAX_DEVICES) return fail(KDA_ERR_HIP, "device %d beyond the supported %d", dev,
                                                      kda::MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

kda_status run_decode(const void* q, const void* k, const void* v, const void* g_raw, const float* beta_logits,
                      const float* A_log, float scale, int gate_per_channel, void* state, kda_state_dtype state_dtype,
                      void* out, int B, int H_qk, int H, int K, int V, hipStream_t stream, bool delta) {
  if (B < 0 || H_qk <= 0 || H <= 0)
    return fail(KDA_ERR_SHAPE, "sizes must be non-negative with H, H_qk > 0 (got B=%d H_qk=%d H=%d)", B, H_qk, H);
  if (K != kda::HD || V != kda::HD) return fail(KDA_ERR_SHAPE, "only K = V = 128 is supported (got K=%d V=%d)", K, V);
  if (H % H_qk != 0) return fail(KDA_ERR_SHAPE, "H (%d) must be a multiple of H_qk (%d)", H, H_qk);
  if (gate_per_channel != 0 && gate_per_channel != 1)
    return fail(KDA_ERR_SHAPE, "gate_per_channel must be 0 or 1 (got %d)", gate_per_channel);
  if (state_dtype != KDA_STATE_BF16 && state_dtype != KDA_STATE_FP32)
    return fail(KDA_ERR_DTYPE, "state dtype %d is not bf16 (1) or fp32 (2)", (int)state_dtype);
  if ((long)B * H >= (1L << 31)) return fail(KDA_ERR_SHAPE, "problem too large");
  if (B == 0) return ok();
  const void* req[] = {q, k, v, g_raw, A_log, state, out, beta_logits};
  const char* names[] = {"q", "k", "v", "g_raw", "A_log", "state", "out", "beta_logits"};
  const int n_req = delta ? 8 : 7;
  for (int i = 0; i < n_req; ++i)
    if (!req[i]) return fail(KDA_ERR_NULL, "%s is NULL", names[i]);
  for (int i = 0; i < n_req; ++i)
    if (!aligned16(req[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  (void)hipGetLastError();
  kda::DecodeParams p{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(g_raw), beta_logits, A_log,
                      state, static_cast<uint16_t*>(out), H, H_qk, scale};
  {
    Timed t(K_DECODE, stream);
    kda::launch_decode(p, B, state_dtype == KDA_STATE_BF16, gate_per_channel == 1, delta, stream);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  if (env_flag("KDA_LOG"))
    std::fprintf(stderr, "[kda] %s decode B=%d H=%d H_qk=%d grid=%d state=%s\n", delta ? "delta-rule" : "linear",
                 B, H, H_qk, B * H, state_dtype == KDA_STATE_BF16 ? "bf16" : "fp32");
  return ok();
}

// ---- backward ----------------------------------------------------------------
// Workspace: a 256-byte header, the schedule (sequence table, chunk table,
// order), then the state entering every (chunk, head) and the gradient of
// the state leaving it (fp16, 32 KiB each), and the chains' operator records
// (sized for the per-channel gate's kda::BREC_PC_BYTES each; the scalar gate
// uses kda::BREC_BYTES of each slot).
struct BwdLayout {
  size_t seqs, chunks, order, states, dstates, brec, total;
};

BwdLayout bwd_layout(int n_seqs, int n_entries, int H) {
  BwdLayout L;
  const size_t jobs = (size_t)n_entries * H;
  L.seqs = ALIGN;
  L.chunks = L.seqs + round_up((size_t)n_seqs * sizeof(int4));
  L.order = L.chunks + round_up((size_t)n_entries * sizeof(int4));
  L.states = L.order + round_up((size_t)n_seqs * sizeof(int));
  L.dstates = L.states + round_up(jobs * kda::HD * kda::HD * sizeof(uint16_t));
  L.brec = L.dstates + round_up(jobs * kda::HD * kda::HD * sizeof(uint16_t));
  L.total = L.brec + round_up(jobs * kda::BREC_PC_BYTES);
  return L;
}

struct BwdArgs {
  const void *q, *k, *v, *g_raw;
  const float *beta, *A_log;
  float scale;
  int gate_per_channel;
  const float* s0;
  const void* dout;
  const float* dfinal;
  float *dq, *dk, *dv, *dg_raw, *dbeta, *dA_log, *dinit;
  const int32_t* cu;
  int n_seqs, T, rows, H_qk, H, K, V;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
};

kda_status run_backward(const BwdArgs& a) {
  FwdArgs f{a.q, a.k, a.v, a.g_raw, a.beta, a.A_log, a.scale, a.gate_per_channel, nullptr, KDA_STATE_NONE,
            nullptr, nullptr, KDA_STATE_NONE, a.cu, a.n_seqs, a.T, a.rows, a.H_qk, a.H, a.K, a.V, nullptr, 0,
            a.stream, true};
  kda_status st = validate_common(f);
  if (st != KDA_OK) return st;
  if (a.n_seqs == 0) return ok();
  const long tokens = (long)a.rows * a.T;
  if (tokens > 0) {
    const void* req[] = {a.q, a.k, a.v, a.g_raw, a.beta, a.A_log, a.dout, a.dq, a.dk, a.dv, a.dg_raw, a.dbeta};
    const char* names[] = {"q", "k", "v", "g_raw", "beta_logits", "A_log", "dout", "dq", "dk", "dv", "dg_raw",
                           "dbeta_logits"};
    for (int i = 0; i < 12; ++i)
      if (!req[i]) return fail(KDA_ERR_NULL, "%s is NULL", names[i]);
    for (int i = 0; i < 12; ++i)
      if (!aligned16(req[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  if (!a.dA_log) return fail(KDA_ERR_NULL, "dA_log is NULL");
  const void* opt[] = {a.s0, a.dfinal, a.dinit, a.dA_log};
  const char* onames[] = {"initial_state", "dfinal", "dinitial_state", "dA_log"};
  for (int i = 0; i < 4; ++i)
    if (opt[i] && !aligned16(opt[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", onames[i]);
  if (a.cu && (reinterpret_cast<uintptr_t>(a.cu) & 3u)) return fail(KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
  const int n_entries = a.cu ? cdiv(a.T, kda::CH) + a.n_seqs : a.n_seqs * cdiv(a.T, kda::CH);
  if ((long)n_entries * a.H >= (1L << 31))
    return fail(KDA_ERR_SHAPE, "problem too large (chunks x heads must fit in int32)");
  const BwdLayout L = bwd_layout(a.n_seqs, n_entries, a.H);
  if (!a.ws) return fail(KDA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
  if (a.ws_bytes < L.total)
    return fail(KDA_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", a.ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(a.ws) & (ALIGN - 1)) return fail(KDA_ERR_ALIGN, "workspace is not 256-byte aligned");

  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  int4* seqs = reinterpret_cast<int4*>(ws + L.seqs);
  int4* chunks = reinterpret_cast<int4*>(ws + L.chunks);
  int* order = reinterpret_cast<int*>(ws + L.order);
  (void)hipGetLastError();
  if (a.cu) {
    kda::TableParams tp{a.cu, a.n_seqs, a.T, n_entries, seqs, chunks, order};
    Timed t(K_TABLE, a.stream);
    kda::launch_table(tp, a.stream);
  }
  kda::BwdParams bp{static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                    static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.g_raw), a.beta, a.A_log,
                    static_cast<const uint16_t*>(a.dout), a.dfinal, a.s0, a.scale, a.gate_per_channel != 0 ? 1 : 0,
                    a.gate_per_channel != 0 ? kda::BREC_PC_BYTES : kda::BREC_BYTES, a.H, a.H_qk, a.cu ? -1 : a.T,
                    chunks, seqs, order, tokens > 0 ? n_entries : 0, a.n_seqs * a.H,
                    reinterpret_cast<uint16_t*>(ws + L.states), reinterpret_cast<uint16_t*>(ws + L.dstates),
                    ws + L.brec, a.dq, a.dk, a.dv, a.dg_raw, a.dbeta, a.dA_log, a.dinit};
  // coefficients; both chains (chunk states and their gradients); the gradients
  const int ids[3] = {K_BWD_COEF, K_BWD_CHAINS, K_BWD_GRAD};
  for (int stage = 0; stage < 3; ++stage) {
    Timed t(ids[stage], a.stream);
    kda::launch_bwd(bp, (size_t)tokens * a.H_qk * kda::HD, stage, a.stream);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  if (env_flag("KDA_LOG"))
    std::fprintf(stderr, "[kda] bwd seqs=%d T=%d H=%d H_qk=%d entries=%d\n", a.n_seqs, a.T, a.H, a.H_qk,
                 n_entries);
  return ok();
}

}  // namespace

extern "C" {

size_t kda_fwd_workspace_bytes(int B, int T, int H_qk, int H, int N) {
  if (B < 0 || T < 0 || H_qk <= 0 || H <= 0 || N < 0 || H % H_qk != 0) return 0;
  if (N > 0 && B != 1) return 0;
  const int n_seqs = N > 0 ? N : B;
  const int n_entries = N > 0 ? cdiv(T, kda::CH) + N : B * cdiv(T, kda::CH);
  const size_t split = layout(n_seqs, n_entries, H, false).total;
  return kda::fused_available() ? std::max(split, layout(n_seqs, n_entries, H, true).total) : split;
}

kda_status kda_fwd(const void* q, const void* k, const void* v, const void* g_raw, const float* beta_logits,
                   const float* A_log, float scale, int gate_per_channel, const void* initial_state,
                   kda_state_dtype init_dtype, void* out, void* final_state, kda_state_dtype final_dtype, int B,
                   int T, int H_qk, int H, int K, int V, void* workspace, size_t workspace_bytes, void* stream) {
  FwdArgs a{q, k, v, g_raw, beta_logits, A_log, scale, gate_per_channel, initial_state, init_dtype, out,
            final_state, final_dtype, nullptr, B, T, B, H_qk, H, K, V, workspace, workspace_bytes,
            static_cast<hipStream_t>(stream), true};
  return run_forward(a);
}

kda_status kda_fwd_noalloc(const void* q, const void* k, const void* v, const void* g_raw,
                           const float* beta_logits, const float* A_log, float scale, int gate_per_channel,
                           const void* initial_state, kda_state_dtype init_dtype, void* out, void* final_state,
                           kda_state_dtype final_dtype, int B, int T, int H_qk, int H, int K, int V, void* stream) {
  FwdArgs a{q, k, v, g_raw, beta_logits, A_log, scale, gate_per_channel, initial_state, init_dtype, out,
            final_state, final_dtype, nullptr, B, T, B, H_qk, H, K, V, nullptr, 0,
            static_cast<hipStream_t>(stream), true, true};
  // Validate everything that needs no device first (sizes against the scratch
  // capacity included), then look up this device's copy of the scratch.
  FwdArgs probe = a;
  probe.ws = reinterpret_cast<void*>(ALIGN);  // stands in for the scratch address during validation only
  probe.ws_bytes = KDA_NOALLOC_SCRATCH_BYTES;
  FwdPlan plan;
  kda_status st = validate_forward(probe, &plan);
  if (st != KDA_OK || plan.n_entries < 0) return st;
  st = scratch_address(&a.ws);
  if (st != KDA_OK) return st;
  a.ws_bytes = KDA_NOALLOC_SCRATCH_BYTES;
  return run_forward(a);
}

kda_status kda_fwd_varlen(const void* q, const void* k, const void* v, const void* g_raw, const float* beta_logits,
                          const float* A_log, float scale, int gate_per_channel, const void* initial_state,
                          kda_state_dtype init_dtype, void* out, void* final_state, kda_state_dtype final_dtype,
                          const int32_t* cu_seqlens, int N, int T, int H_qk, int H, int K, int V, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (N > 0 && !cu_seqlens) return fail(KDA_ERR_NULL, "cu_seqlens is NULL");
  FwdArgs a{q, k, v, g_raw, beta_logits, A_log, scale, gate_per_channel, initial_state, init_dtype, out,
            final_state, final_dtype, cu_seqlens, N, T, 1, H_qk, H, K, V, workspace, workspace_bytes,
            static_cast<hipStream_t>(stream), true};
  return run_forward(a);
}

kda_status kda_la_fwd(const void* q, const void* k, const void* v, const void* g_raw, const float* A_log, float scale,
                      int gate_per_channel, const void* initial_state, kda_state_dtype init_dtype, void* out,
                      void* final_state, kda_state_dtype final_dtype, int B, int T, int H_qk, int H, int K, int V,
                      void* workspace, size_t workspace_bytes, void* stream) {
  FwdArgs a{q, k, v, g_raw, nullptr, A_log, scale, gate_per_channel, initial_state, init_dtype, out,
            final_state, final_dtype, nullptr, B, T, B, H_qk, H, K, V, workspace, workspace_bytes,
            static_cast<hipStream_t>(stream), false};
  return run_forward(a);
}

kda_status kda_la_fwd_varlen(const void* q, const void* k, const void* v, const void* g_raw, const float* A_log,
                             float scale, int gate_per_channel, const void* initial_state, kda_state_dtype init_dtype,
                             void* out, void* final_state, kda_state_dtype final_dtype, const int32_t* cu_seqlens,
                             int N, int T, int H_qk, int H, int K, int V, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (N > 0 && !cu_seqlens) return fail(KDA_ERR_NULL, "cu_seqlens is NULL");
  FwdArgs a{q, k, v, g_raw, nullptr, A_log, scale, gate_per_channel, initial_state, init_dtype, out,
            final_state, final_dtype, cu_seqlens, N, T, 1, H_qk, H, K, V, workspace, workspace_bytes,
            static_cast<hipStream_t>(stream), false};
  return run_forward(a);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g_raw, const float* beta_logits,
                           const float* A_log, float scale, int gate_per_channel, void* state,
                           kda_state_dtype state_dtype, void* out, int B, int H_qk, int H, int K, int V,
                           void* stream) {
  return run_decode(q, k, v, g_raw, beta_logits, A_log, scale, gate_per_channel, state, state_dtype, out, B, H_qk, H,
                    K, V, static_cast<hipStream_t>(stream), true);
}

kda_status kda_la_decode_step(const void* q, const void* k, const void* v, const void* g_raw, const float* A_log,
                              float scale, int gate_per_channel, void* state, kda_state_dtype state_dtype, void* out,
                              int B, int H_qk, int H, int K, int V, void* stream) {
  return run_decode(q, k, v, g_raw, nullptr, A_log, scale, gate_per_channel, state, state_dtype, out, B, H_qk, H, K,
                    V, static_cast<hipStream_t>(stream), false);
}

kda_status kda_fwd_check(const void* workspace, void* stream) {
  const void* word = workspace;
  if (!word) {
    void* scratch_ptr = nullptr;
    const kda_status st = scratch_address(&scratch_ptr);
    if (st != KDA_OK) return st;
    word = scratch_ptr;
  }
  int bits = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipMemcpy(&bits, word, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(KDA_ERR_HIP, "kda_fwd_check: %s", hipGetErrorString(hipGetLastError()));
  if (bits == 0) return ok();
  return fail(KDA_ERR_HIP, "the last forward call on this workspace reported error bits 0x%x (%s%s%s)", bits,
              (bits & 1) ? "a workgroup ran on an unexpected XCD; " : "",
              (bits & 2) ? "a consumer's bounded wait for a record timed out; " : "",
              (bits & 4) ? "a producer's bounded wait for a free ring slot timed out" : "");
}

size_t kda_bwd_workspace_bytes(int B, int T, int H_qk, int H, int N) {
  if (B < 0 || T < 0 || H_qk <= 0 || H <= 0 || N < 0 || H % H_qk != 0) return 0;
  if (N > 0 && B != 1) return 0;
  const int n_seqs = N > 0 ? N : B;
  const int n_entries = N > 0 ? cdiv(T, kda::CH) + N : B * cdiv(T, kda::CH);
  return bwd_layout(n_seqs, n_entries, H).total;
}

kda_status kda_bwd(const void* q, const void* k, const void* v, const void* g_raw, const float* beta_logits,
                   const float* A_log, float scale, int gate_per_channel, const float* initial_state,
                   const void* dout, const float* dfinal, float* dq, float* dk, float* dv, float* dg_raw,
                   float* dbeta_logits, float* dA_log, float* dinitial_state, int B, int T, int H_qk, int H, int K,
                   int V, void* workspace, size_t workspace_bytes, void* stream) {
  BwdArgs a{q, k, v, g_raw, beta_logits, A_log, scale, gate_per_channel, initial_state, dout, dfinal, dq, dk, dv,
            dg_raw, dbeta_logits, dA_log, dinitial_state, nullptr, B, T, B, H_qk, H, K, V, workspace,
            workspace_bytes, static_cast<hipStream_t>(stream)};
  return run_backward(a);
}

kda_status kda_bwd_varlen(const void* q, const void* k, const void* v, const void* g_raw, const float* beta_logits,
                          const float* A_log, float scale, int gate_per_channel, const float* initial_state,
                          const void* dout, const float* dfinal, float* dq, float* dk, float* dv, float* dg_raw,
                          float* dbeta_logits, float* dA_log, float* dinitial_state, const int32_t* cu_seqlens,
                          int N, int T, int H_qk, int H, int K, int V, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (N > 0 && !cu_seqlens) return fail(KDA_ERR_NULL, "cu_seqlens is NULL");
  BwdArgs a{q, k, v, g_raw, beta_logits, A_log, scale, gate_per_channel, initial_state, dout, dfinal, dq, dk, dv,
            dg_raw, dbeta_logits, dA_log, dinitial_state, cu_seqlens, N, T, 1, H_qk, H, K, V, workspace,
            workspace_bytes, static_cast<hipStream_t>(stream)};
  return run_backward(a);
}

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE";
    case KDA_ERR_STATE_DTYPE_MISMATCH: return "KDA_ERR_STATE_DTYPE_MISMATCH";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_UNKNOWN_STATUS";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

void kda_kernel_timing_enable(int enable) { g_timing.on = enable != 0; }

int kda_kernel_timing_read(double* total_ms, int* launches, int max_kernels) {
  for (int i = 0; i < max_kernels && i < K_COUNT; ++i) {
    if (total_ms) total_ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  int rc = K_COUNT;
  for (auto& r : g_timing.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) rc = -1;
    if (r.id < max_kernels) {
      if (total_ms) total_ms[r.id] += ms;
      if (launches) launches[r.id] += 1;
    }
    g_timing.pool.push_back(r.a);
    g_timing.pool.push_back(r.b);
  }
  g_timing.pending.clear();
  return rc;
}

const char* kda_kernel_name(int id) { return (id >= 0 && id < K_COUNT) ? kKernelNames[id] : ""; }

}  // extern "C"
