// Sequence tables of a packed batch of independent sequences of different lengths.
//
// Each sequence keeps its own fixed-size state from its own initial state ("Gated DeltaNet-2:
// decoupling erase and write in linear attention", sections "The attention bottleneck" and
// "Why this matters": one constant-size state per sequence, constant-memory decoding).  The
// sequences lie one after another on the token axis, delimited by nseq + 1 int32 offsets on
// the device.  One workgroup turns the offsets into
//   seqs[n]   = {first token, tokens, H * (chunks before sequence n), chunks of sequence n}
//   chunks[g] = {first token, tokens (1 .. chunk), H * (chunks before its sequence) + its index
//                in the sequence, chunks of its sequence}           for every chunk g, in order
//   *total    = number of chunks.
// The offsets are first clamped into [0, T] and replaced by their running maximum, so the
// tables address only tokens of the packed arrays whatever the offsets hold; valid offsets
// (0 = cu[0] <= cu[1] <= ... <= cu[nseq] = T) pass through unchanged.

#include "dr_internal.h"

namespace dr {
namespace {

constexpr int kSetupThreads = 1024;

// In-place inclusive scan of x[0 .. kSetupThreads) in LDS with `op`; every thread takes part.
template <typename Op>
__device__ void block_scan(int* x, int tid, Op op) {
  for (int off = 1; off < kSetupThreads; off <<= 1) {
    const int y = tid >= off ? x[tid - off] : 0;
    __syncthreads();
    if (tid >= off) x[tid] = op(x[tid], y);
    __syncthreads();
  }
}

__global__ __launch_bounds__(kSetupThreads) void varlen_setup_kernel(const int* __restrict__ cu, int nseq, int T,
                                                                     int H, int chunk, int4* __restrict__ seqs,
                                                                     int4* __restrict__ chunks,
                                                                     int* __restrict__ total) {
  __shared__ int sb[kSetupThreads + 1];  // boundaries of this tile's sequences
  __shared__ int sc[kSetupThreads];      // inclusive prefix sums of their chunk counts
  const int tid = threadIdx.x;
  auto clamp_t = [&](int x) { return x < 0 ? 0 : (x > T ? T : x); };
  auto imax = [](int a, int b) { return a > b ? a : b; };
  int bcarry = 0, ccarry = 0;  // last boundary and chunk count of the earlier tiles
  for (int base = 0; base < nseq; base += kSetupThreads) {
    // boundaries base .. base + kSetupThreads: clamped, then their running maximum
    const int i = base + tid;
    sb[tid] = imax(i <= nseq ? clamp_t(cu[i]) : T, bcarry);
    if (tid == 0) {
      const int i2 = base + kSetupThreads;
      sb[kSetupThreads] = i2 <= nseq ? clamp_t(cu[i2]) : T;
    }
    __syncthreads();
    block_scan(sb, tid, imax);
    if (tid == 0) sb[kSetupThreads] = imax(sb[kSetupThreads], sb[kSetupThreads - 1]);
    __syncthreads();

    const int bos = sb[tid];
    const int len = i < nseq ? sb[tid + 1] - bos : 0;
    const int nch = (len + chunk - 1) / chunk;
    sc[tid] = nch;
    __syncthreads();
    block_scan(sc, tid, [](int a, int b) { return a + b; });
    const int cb = ccarry + sc[tid] - nch;  // chunks before sequence i
    if (i < nseq) seqs[i] = make_int4(bos, len, H * cb, nch);
    const int tile = sc[kSetupThreads - 1];
    if (chunks != nullptr) {
      // The tile's chunks over all threads: chunk g belongs to the first sequence j of the tile
      // whose inclusive prefix sum exceeds g.
      for (int g = tid; g < tile; g += kSetupThreads) {
        int lo = 0, hi = kSetupThreads - 1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (sc[mid] > g)
            hi = mid;
          else
            lo = mid + 1;
        }
        const int nj = sc[lo] - (lo > 0 ? sc[lo - 1] : 0);
        const int cj = ccarry + sc[lo] - nj;  // chunks before sequence base + lo
        const int c = g - (sc[lo] - nj);      // index of chunk g in its sequence
        const int bj = sb[lo], lenj = sb[lo + 1] - bj;
        const int rest = lenj - chunk * c;
        chunks[ccarry + g] = make_int4(bj + chunk * c, rest < chunk ? rest : chunk, H * cj + c, nj);
      }
    }
    bcarry = sb[kSetupThreads];
    ccarry += tile;
    __syncthreads();  // the next tile overwrites sb and sc
  }
  if (tid == 0) *total = ccarry;
}

}  // namespace

hipError_t launch_varlen_setup(const int* cu, int nseq, int T, int H, int chunk, int4* seqs, int4* chunks,
                               int* total, hipStream_t stream) {
  hipLaunchKernelGGL(varlen_setup_kernel, dim3(1), dim3(kSetupThreads), 0, stream, cu, nseq, T, H, chunk, seqs,
                     chunks, total);
  return hipGetLastError();
}

}  // namespace dr
