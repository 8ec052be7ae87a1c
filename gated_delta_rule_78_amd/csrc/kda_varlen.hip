// kda_varlen.hip -- chunk table of a packed variable-length batch (two-pass forward).
//
// N sequences lie back to back along T at offsets cu[0..N].  Every sequence is cut
// into its own 64-token chunks (the last one masked), so a chunk never straddles two
// sequences; the record pass runs over the global list of those chunks and the state
// pass walks each (sequence, head) chain.  This kernel (one workgroup) writes into the
// workspace:
//   cs[N + 1]      the offsets, clamped to [0, T] and made non-decreasing (so that no
//                  kernel can index outside the token arrays, whatever cu holds)
//   ctab[gmax][2]  (sequence, chunk of that sequence) of every global chunk
//   cbase[N]       the first global chunk of each sequence
//   ctotal[1]      the number of chunks (<= gmax = ceil(T / 64) + N)
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int NTB = 1024;

__global__ __launch_bounds__(NTB) void varlen_table_kernel(const int* __restrict__ cu, int nseq, int T,
                                                           int* __restrict__ cs, int* __restrict__ ctab,
                                                           int* __restrict__ cbase, int* __restrict__ ctotal,
                                                           int gmax) {
  __shared__ int part[NTB];
  const int tid = threadIdx.x;
  const int per = (nseq + NTB - 1) / NTB;
  const int s0 = min(nseq, tid * per), s1 = min(nseq, s0 + per);
  // 1. clamped offsets cu[1..N]: running maximum (exclusive scan of block maxima)
  int mx = 0;
  for (int i = s0; i < s1; ++i) mx = max(mx, min(max(cu[i + 1], 0), T));
  part[tid] = mx;
  __syncthreads();
  for (int off = 1; off < NTB; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] = max(part[tid], v);
    __syncthreads();
  }
  int run = tid ? part[tid - 1] : 0;
  __syncthreads();
  if (tid == 0) cs[0] = 0;
  for (int i = s0; i < s1; ++i) {
    run = max(run, min(max(cu[i + 1], 0), T));
    cs[i + 1] = run;
  }
  __syncthreads();
  // 2. chunks per sequence, exclusive scan -> first global chunk, then the table
  int sum = 0;
  for (int i = s0; i < s1; ++i) sum += (cs[i + 1] - cs[i] + 63) / 64;
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < NTB; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int base = tid ? part[tid - 1] : 0;
  for (int i = s0; i < s1; ++i) {
    const int nc = (cs[i + 1] - cs[i] + 63) / 64;
    cbase[i] = base;
    for (int c = 0; c < nc; ++c) {
      if (base + c < gmax) {
        ctab[2 * (base + c)] = i;
        ctab[2 * (base + c) + 1] = c;
      }
    }
    base += nc;
  }
  if (tid == NTB - 1) *ctotal = min(part[NTB - 1], gmax);
}

}  // namespace

hipError_t launch_varlen_table(const ChunkArgs& a, int* cs, int* ctab, int* cbase, int* ctotal) {
  hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(NTB), 0, (hipStream_t)a.stream, a.cu, a.n_seqs, a.T, cs,
                     ctab, cbase, ctotal, a.gmax);
  return hipGetLastError();
}

}  // namespace kda
