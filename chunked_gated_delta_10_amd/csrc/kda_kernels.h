// kda_kernels.h -- launch interface between the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace kda {

// ---- host-side, per-device setup ---------------------------------------------
constexpr int MAX_DEVICES = 64;

// The calling thread's current device (0 if it cannot be read).
inline int current_device() {
  int d = 0;
  return (hipGetDevice(&d) == hipSuccess && d >= 0 && d < MAX_DEVICES) ? d : 0;
}

// Runs set() on the current device until it has once succeeded there
// (e.g. a kernel attribute, which is per device).  Concurrent first calls
// may both run set(), which is harmless for idempotent settings.  Returns
// set()'s error, or hipSuccess once done.
template <typename F>
hipError_t once_per_device(std::atomic<int> (&done)[MAX_DEVICES], F set) {
  const int d = current_device();
  if (done[d].load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = set();
  if (e == hipSuccess) done[d].store(1, std::memory_order_release);
  return e;
}

// Compute units of the current device (cached per device).
int device_cu_count();

// Chunk-local kernel (kda_chunk.hip): one workgroup per (schedule entry, head).
struct ChunkParams {
  const uint16_t* q;      // bf16 [tokens, H_qk, 128]
  const uint16_t* k;      // bf16 [tokens, H_qk, 128]
  const uint16_t* g_raw;  // bf16 [tokens, H, 128] or [tokens, H]
  const float* beta;      // fp32 [tokens, H] (logits)
  const float* A_log;     // fp32 [H]
  const int4* chunks;     // schedule entries
  int H, H_qk;
  uint8_t* rec;           // [entries][H] chunk records
  int dense_T;            // > 0: B rows of dense_T tokens, schedule by arithmetic; 0: read `chunks`
  const uint16_t* v;      // bf16 [tokens, H, 128]: copied into the fused kernel's records (else unused)
};

// Recurrence kernel (kda_recur.hip): one workgroup per (chain, value tile).
struct RecurParams {
  const uint8_t* rec;
  const int4* seqs;       // per sequence: first token, length, first schedule entry
  const int* order;       // sequences in processing order (longest first)
  int n_chains;           // sequences * H
  int n_entries;          // schedule entries (records per head)
  int H, H_qk;
  const uint16_t* v;      // bf16 [tokens, H, 128]
  uint16_t* out;          // bf16 [tokens, H, 128]
  const void* s0;         // [seqs, H, 128, 128] fp32 or bf16, or null
  void* s1;               // same layout, or null
  float scale;
  uint16_t* sink;         // 64 scratch values: destination of output rows past a chunk's end
  int dense_T;            // >= 0: B rows of dense_T tokens, schedule by arithmetic; -1: read `seqs`/`order`
  int* err;               // error word of the workspace header: cleared (this path reports no errors)
};

// Fused persistent forward (kda_fused.hip): per-channel gate, delta rule.
struct FusedParams {
  ChunkParams cp;         // producer inputs: q, k, g_raw, beta, A_log, H, H_qk (rec, chunks unused)
  const uint16_t* v;      // bf16 [tokens, H, 128]
  uint16_t* out;          // bf16 [tokens, H, 128]
  const void* s0;         // [seqs, H, 128, 128] fp32 or bf16, or null
  void* s1;               // same layout, or null
  float scale;
  const int4* seqs;       // packed sequences: first token, length (dense_T < 0)
  const int* order;       // packed sequences in processing order (longest first)
  int dense_T;            // >= 0: B rows of dense_T tokens
  int n_chains;           // sequences * H
  int n_teams, tpx, R, P;  // teams (8 * tpx), teams per XCD, ring slots and producers per team
  uint8_t* ring;          // [n_teams][R] records of REC2_BYTES
  int* ready;             // [n_teams][R] ready flags, then prog [n_teams][NCW]; one per 128 bytes
  int* prog;
  int n_flags_total;      // ints covered by ready and prog
  int* err;               // error bits of the launch (0 = fine)
  uint16_t* sink;         // 64 scratch values for output rows past a chunk's end
};
struct FusedLayout {
  int grid, tpx, R, P, n_teams, n_flags;
  size_t ring_bytes;
};
// Team layout and ring size for n_chains chains on the current device.
FusedLayout fused_layout(int n_chains);
// Cooperative launches, two fused workgroups per CU and a CU count divisible
// by 8 on the current device (checked once per device).
bool fused_available();
// Clears the flags and the error word, then launches the cooperative kernel.
hipError_t launch_fused(const FusedParams& p, int grid, bool bf16_state, hipStream_t stream);

// Decode kernel (kda_decode.hip): one workgroup per (batch row, head).
struct DecodeParams {
  const uint16_t* q;      // bf16 [B, H_qk, 128]
  const uint16_t* k;
  const uint16_t* v;      // bf16 [B, H, 128]
  const uint16_t* g_raw;  // bf16 [B, H, 128] or [B, H]
  const float* beta;      // fp32 [B, H]
  const float* A_log;     // fp32 [H]
  void* state;            // [B, H, 128, 128], in place
  uint16_t* out;          // bf16 [B, H, 128]
  int H, H_qk;
  float scale;
};

// Schedule kernel (kda_table.hip): one workgroup.
struct TableParams {
  const int32_t* cu;      // device offsets [N + 1], or null for B rows of T tokens
  int N;                  // sequences (B when cu is null)
  int T;                  // tokens per row (dense) or total tokens (packed)
  int n_entries;          // capacity of `chunks`
  int4* seqs;             // [N]
  int4* chunks;           // [n_entries]
  int* order;             // [N]
};

void launch_table(const TableParams& p, hipStream_t stream);
// delta = false: decay-only linear attention (no erase, no write strength, no q/k normalisation).
// Returns the error of the kernel's one-time attribute setup on this device (launch errors are
// read by the caller with hipGetLastError).
hipError_t launch_chunk_local(const ChunkParams& p, int n_entries, bool per_channel, bool delta, hipStream_t stream);
void launch_recur(const RecurParams& p, bool bf16_state, bool per_channel, bool delta, hipStream_t stream);
// Scalar gate with value heads grouped on q/k heads and at least
// GROUP_MIN_JOBS (schedule entry, q/k head) jobs: the value heads of a group
// share one copy of the qn and kn^T record fragments, written by the grouped
// chunk-local kernel.  Fewer jobs take the per-head kernel and records.
constexpr int GROUP_MIN_JOBS = 256;
bool shares_qk_fragments(bool per_channel, int H, int H_qk, int n_entries);
int recur_grid(int n_chains);
void launch_decode(const DecodeParams& p, int B, bool bf16_state, bool per_channel, bool delta, hipStream_t stream);

}  // namespace kda
