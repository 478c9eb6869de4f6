// kda_table.hip -- chunk schedule built on the device from cu_seqlens (or
// from B rows of T tokens), so the host never reads the offsets.  The
// forward pass launches it for packed sequences; for B rows of T tokens the
// other kernels derive the same schedule arithmetically.
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
  __shared__ int scan[TB];   // inclusive scan of chunk counts within the current block of sequences
  __shared__ int tok0s[TB];
  __shared__ int lens_blk[TB];
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
    tok0s[tid] = tok0;
    lens_blk[tid] = len;
    __syncthreads();
    for (int off = 1; off < TB; off <<= 1) {
      const int y = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += y;
      __syncthreads();
    }
    const int c0 = carry;
    if (n < p.N) {
      p.seqs[n] = make_int4(tok0, len, c0 + scan[tid] - nch, 0);
      if (n < MAX_RANKED) lens[n] = len;
    }
    // chunk entries of this block, written cooperatively: entry j belongs to
    // the first sequence i of the block whose inclusive scan exceeds j
    const int blk_total = scan[TB - 1];
    for (int j = tid; j < blk_total; j += TB) {
      int lo = 0, hi = TB - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (scan[mid] > j) hi = mid;
        else lo = mid + 1;
      }
      const int c = j - (scan[lo] - (lens_blk[lo] + CH - 1) / CH);
      const int e = c0 + j;
      if (e < p.n_entries)
        p.chunks[e] = make_int4(base + lo, tok0s[lo] + c * CH, min(CH, lens_blk[lo] - c * CH), c);
    }
    __syncthreads();
    if (tid == 0) carry = c0 + blk_total;
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
