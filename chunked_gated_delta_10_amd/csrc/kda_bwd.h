// kda_bwd.h -- launch interface of the backward pass (kda_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Backward pass of the delta rule: one decay per token-head (kda_bwd.hip) or per key channel
// (kda_bwd_pc.hip); the chains are shared.
constexpr int BREC_BYTES = 104 * 1024;     // per (entry, head): operand fragments of both chains, and T
constexpr int BREC_PC_BYTES = 120 * 1024;  // per-channel gate: the same, and M and the masked key Gram matrix
struct BwdParams {
  const uint16_t* q;      // bf16 [tokens, H_qk, 128]
  const uint16_t* k;
  const uint16_t* v;      // bf16 [tokens, H, 128]
  const uint16_t* g_raw;  // bf16 [tokens, H] (per_channel: [tokens, H, 128])
  const float* beta;      // fp32 [tokens, H] (logits)
  const float* A_log;     // fp32 [H]
  const uint16_t* dout;   // bf16 [tokens, H, 128]
  const float* dfinal;    // fp32 [seqs, H, 128, 128] ([V][K]) or null
  const float* s0;        // fp32 initial state, same layout, or null
  float scale;
  int per_channel;        // 0: one decay per token-head; 1: one per key channel
  int rec_bytes;          // BREC_BYTES or BREC_PC_BYTES
  int H, H_qk;
  int dense_T;            // >= 0: B rows of dense_T tokens; -1: read chunks / seqs / order
  const int4* chunks;
  const int4* seqs;
  const int* order;
  int n_entries, n_chains;
  uint16_t* states;        // fp16 [entries][H][V][K]: the state entering every chunk
  uint16_t* dstates;       // fp16 [entries][H][V][K]: the gradient of the state leaving every chunk
  uint8_t* brec;           // [entries][H][rec_bytes]
  float* dq;              // fp32 [tokens, H_qk, 128]
  float* dk;
  float* dv;              // fp32 [tokens, H, 128]
  float* dg_raw;          // fp32, the layout of g_raw
  float* dbeta;           // fp32 [tokens, H]
  float* dA_log;          // fp32 [H]
  float* dinit;           // fp32 [seqs, H, 128, 128] or null
};
// Stages, in this order: 0 the coefficient records (after clearing dA_log, and dq, dk when value heads
// share q/k heads; qk_floats: elements of dq), 1 both chains (the chunk states and their gradients),
// 2 the gradients.
void launch_bwd(const BwdParams& p, size_t qk_floats, int stage, hipStream_t stream);
// per-channel gate: the coefficient and gradient stages (kda_bwd_pc.hip)
void launch_coef_pc(const BwdParams& p, hipStream_t stream);
void launch_grad_pc(const BwdParams& p, hipStream_t stream);

}  // namespace kda
