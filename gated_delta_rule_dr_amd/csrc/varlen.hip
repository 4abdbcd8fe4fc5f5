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
//   *total    = number of chunks
//   order[r]  = the sequences by chunk count, longest first (when `order` is not null): exact
//               counts below 128 chunks, eight classes per octave above, so that the longest
//               sequences' scan workgroups start first and the short ones fill in behind them.
// The offsets are first clamped into [0, T] and replaced by their running maximum, so the
// tables address only tokens of the packed arrays whatever the offsets hold; valid offsets
// (0 = cu[0] <= cu[1] <= ... <= cu[nseq] = T) pass through unchanged.

#include "dr_internal.h"

namespace dr {
namespace {

constexpr int kSetupThreads = 1024;
constexpr int kOrderKeys = 320;

// Nondecreasing key of a chunk count, < kOrderKeys: the count itself below 128, else its octave
// and the three bits below the leading one.
__device__ __forceinline__ int order_key(int nch) {
  if (nch < 128) return nch;
  const int e = 31 - __builtin_clz(unsigned(nch));
  return 128 + (e - 7) * 8 + ((nch >> (e - 3)) & 7);
}

// Inclusive scan of one value per thread over the workgroup with `op` (identity 0 for the
// nonnegative values here): within each wave by lane shifts, then across the waves through
// `wtot` (LDS, one slot per wave).  Every thread takes part; `wtot` is free again on return.
template <typename Op>
__device__ int block_scan(int x, int* wtot, int tid, Op op) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x = op(x, y);
  }
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre = op(pre, wtot[w]);
  __syncthreads();
  return op(pre, x);
}

__global__ __launch_bounds__(kSetupThreads) void varlen_setup_kernel(const int* __restrict__ cu, int nseq, int T,
                                                                     int H, int chunk, int4* __restrict__ seqs,
                                                                     int4* __restrict__ chunks,
                                                                     int* __restrict__ total,
                                                                     int* __restrict__ order) {
  __shared__ int sb[kSetupThreads + 1];  // boundaries of this tile's sequences
  __shared__ int sc[kSetupThreads];      // inclusive prefix sums of their chunk counts
  __shared__ int hist[kOrderKeys];       // sequences per order key, then each key's next slot
  __shared__ int wtot[kSetupThreads / 64];
  const int tid = threadIdx.x;
  auto clamp_t = [&](int x) { return x < 0 ? 0 : (x > T ? T : x); };
  auto imax = [](int a, int b) { return a > b ? a : b; };
  auto iadd = [](int a, int b) { return a + b; };
  for (int i = tid; i < kOrderKeys; i += kSetupThreads) hist[i] = 0;
  __syncthreads();
  int bcarry = 0, ccarry = 0;  // last boundary and chunk count of the earlier tiles
  for (int base = 0; base < nseq; base += kSetupThreads) {
    // boundaries base .. base + kSetupThreads: clamped, then their running maximum
    const int i = base + tid;
    const int bnd = block_scan(imax(i <= nseq ? clamp_t(cu[i]) : T, bcarry), wtot, tid, imax);
    sb[tid] = bnd;
    if (tid == kSetupThreads - 1) {
      const int i2 = base + kSetupThreads;
      sb[kSetupThreads] = imax(i2 <= nseq ? clamp_t(cu[i2]) : T, bnd);
    }
    __syncthreads();

    const int len = i < nseq ? sb[tid + 1] - bnd : 0;
    const int nch = (len + chunk - 1) / chunk;
    const int incl = block_scan(nch, wtot, tid, iadd);
    sc[tid] = incl;
    const int cb = ccarry + incl - nch;  // chunks before sequence i
    if (i < nseq) {
      seqs[i] = make_int4(bnd, len, H * cb, nch);
      if (order != nullptr) atomicAdd(&hist[order_key(nch)], 1);
    }
    __syncthreads();
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
  if (order == nullptr) return;

  // Longest first: each sequence goes after every sequence of a larger key (in any order within
  // its key).  The key's first slot is an inclusive scan over the keys in descending order less
  // the key's own count.
  const int cnt = tid < kOrderKeys ? hist[kOrderKeys - 1 - tid] : 0;
  const int excl = block_scan(cnt, wtot, tid, iadd) - cnt;
  if (tid < kOrderKeys) hist[kOrderKeys - 1 - tid] = excl;
  __syncthreads();
  // each thread places the sequences whose table entries it wrote itself
  for (int n = tid; n < nseq; n += kSetupThreads) order[atomicAdd(&hist[order_key(seqs[n].w)], 1)] = n;
}

}  // namespace

hipError_t launch_varlen_setup(const int* cu, int nseq, int T, int H, int chunk, int4* seqs, int4* chunks,
                               int* total, int* order, hipStream_t stream) {
  hipLaunchKernelGGL(varlen_setup_kernel, dim3(1), dim3(kSetupThreads), 0, stream, cu, nseq, T, H, chunk, seqs,
                     chunks, total, order);
  return hipGetLastError();
}

}  // namespace dr
