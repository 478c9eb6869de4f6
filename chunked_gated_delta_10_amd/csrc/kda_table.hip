// kda_table.hip -- chunk schedule built on the device from cu_seqlens (or
// from B rows of T tokens), so the host never reads the offsets.
//
// Every sequence is cut into 64-token chunks starting at its first token
// (chunking restarts at each sequence start; the last chunk may be short).
// Entries past the real chunk count are marked unused (z = 0).  Offsets are
// clamped into [0, T] so a malformed cu_seqlens cannot send a later kernel
// outside the token tensors.  Sequences are also ranked by length, longest
// first, so the recurrence starts the longest chains first.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

constexpr int TB = 1024;
constexpr int MAX_RANKED = 4096;

__global__ __launch_bounds__(TB) void table_kernel(TableParams p) {
  __shared__ int scan[TB];
  __shared__ int carry;
  __shared__ int lens[MAX_RANKED];
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < p.N; base += TB) {
    const int n = base + tid;
    int tok0 = 0, len = 0;
    if (n < p.N) {
      if (p.cu) {
        tok0 = min(max(p.cu[n], 0), p.T);
        const int end = min(max(p.cu[n + 1], tok0), p.T);
        len = end - tok0;
      } else {
        tok0 = n * p.T;
        len = p.T;
      }
    }
    const int nch = (len + CH - 1) / CH;
    scan[tid] = nch;
    __syncthreads();
    for (int off = 1; off < TB; off <<= 1) {
      const int y = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += y;
      __syncthreads();
    }
    const int first = carry + scan[tid] - nch;
    if (n < p.N) {
      p.seqs[n] = make_int4(tok0, len, first, 0);
      if (n < MAX_RANKED) lens[n] = len;
      for (int c = 0; c < nch; ++c) {
        const int e = first + c;
        if (e < p.n_entries) p.chunks[e] = make_int4(n, tok0 + c * CH, min(CH, len - c * CH), c);
      }
    }
    __syncthreads();
    if (tid == TB - 1) carry += scan[TB - 1];
    __syncthreads();
  }
  for (int e = carry + tid; e < p.n_entries; e += TB) p.chunks[e] = make_int4(0, 0, 0, 0);
  if (p.N <= MAX_RANKED) {
    for (int n = tid; n < p.N; n += TB) {
      const int ln = lens[n];
      int rank = 0;
      for (int m = 0; m < p.N; ++m) {
        const int lm = lens[m];
        rank += (lm > ln) || (lm == ln && m < n);
      }
      p.order[rank] = n;
    }
  } else {
    for (int n = tid; n < p.N; n += TB) p.order[n] = n;
  }
}

void launch_table(const TableParams& p, hipStream_t stream) {
  table_kernel<<<1, TB, 0, stream>>>(p);
}

}  // namespace kda
