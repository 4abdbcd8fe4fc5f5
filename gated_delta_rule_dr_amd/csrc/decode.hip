// Single-token decode for dk == dv == 128: the fp32 state streams through HBM exactly once
// (read once, written once) and is updated in place.
//
// Constant-memory decode is the point of the fixed-size state ("Gated DeltaNet-2 ...", the
// attention bottleneck: decoding uses constant memory; "KronLSTM ...", The problem).  The step
// is the general one:  S' = Diag(a) S,  S_new = S' - (e*k) m^T + k (w*v)^T with m = S'^T k,
// o = S_new^T q (FG2's per-channel rate beta scales k and v by sqrt(beta) instead, with unit
// erase and write gates).  Expanding the read of the new state avoids a second pass over S:
//   o = S'^T q - m (u . q) + (w*v) (k . q),   u = e * k,
// so both column reductions over dk (m = S'^T k and p = S'^T q) come from one read of S.
//
// Mapping: one 256-thread workgroup per (sequence, head).  Thread = 4-column quad (32) x row
// group (8); each thread keeps 16 rows x 4 columns (rows rg + 8 i) in registers.  Every wave
// load / store instruction covers two full 512-byte rows (128-bit per lane, coalesced).
// Reductions over the 8 row groups: one cross-lane step inside the wave (lanes l and l ^ 32)
// and one exchange of the four waves' partial sums through LDS.

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int D = 128;
constexpr int kThreads = 256;
constexpr int kRows = 16;  // rows per thread

template <bool kBf16, bool kDecayCh, bool kEraseCh, bool kWriteCh>
__global__ __launch_bounds__(kThreads) void decode128_kernel(Problem p) {
  __shared__ float s_k[D], s_q[D], s_a[D], s_u[D], s_wv[D];
  __shared__ float s_red[4][32][10];

  const int tid = threadIdx.x;
  const int cq = tid & 31;   // column quad: columns 4 cq .. 4 cq + 3
  const int rg = tid >> 5;   // row group: rows rg + 8 i
  const int wave = tid >> 6;
  const int64_t nh = blockIdx.x;  // (sequence, head) = token index for T == 1
  float* S = p.S_T + nh * D * D;

  // Issue the whole state read first so it overlaps the small vector loads below.
  f32x4 s[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (rg + 8 * i) * D) + cq);

  if (tid < D) {
    const int i = tid;
    const int64_t o = nh * D + i;
    float kk = load_qkv(p.k, o, kBf16);
    float e = kEraseCh ? p.erase[o] : p.erase[nh];
    if (kEraseCh && p.rate_sqrt) {  // FG2's rate: k~ = sqrt(beta) k, unit erase
      kk *= sqrtf(e);
      e = 1.f;
    }
    s_k[i] = kk;
    s_q[i] = load_qkv(p.q, o, kBf16);
    s_a[i] = expf(kDecayCh ? p.log_decay[o] : p.log_decay[nh]);
    s_u[i] = e * kk;
  } else {
    const int j = tid - D;
    const int64_t o = nh * D + j;
    float w = kWriteCh ? p.write[o] : p.write[nh];
    if (kWriteCh && p.rate_sqrt) w = sqrtf(w);  // v~ = sqrt(beta) v, unit write
    s_wv[j] = w * load_qkv(p.v, o, kBf16);
  }
  __syncthreads();

  // One pass: S' = a * S, partial m = S'^T k and p = S'^T q over this thread's rows, plus
  // the partial dot products k.q and u.q.
  float m[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f, uq = 0.f;
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = rg + 8 * i;
    const float a = s_a[r], kr = s_k[r], qr = s_q[r];
    s[i].x *= a;
    s[i].y *= a;
    s[i].z *= a;
    s[i].w *= a;
    m[0] = fmaf(kr, s[i].x, m[0]);
    m[1] = fmaf(kr, s[i].y, m[1]);
    m[2] = fmaf(kr, s[i].z, m[2]);
    m[3] = fmaf(kr, s[i].w, m[3]);
    pq[0] = fmaf(qr, s[i].x, pq[0]);
    pq[1] = fmaf(qr, s[i].y, pq[1]);
    pq[2] = fmaf(qr, s[i].z, pq[2]);
    pq[3] = fmaf(qr, s[i].w, pq[3]);
    kq = fmaf(kr, qr, kq);
    uq = fmaf(s_u[r], qr, uq);
  }
  float part[10] = {m[0], m[1], m[2], m[3], pq[0], pq[1], pq[2], pq[3], kq, uq};
#pragma unroll
  for (int x = 0; x < 10; ++x) part[x] += __shfl_xor(part[x], 32);
  if ((tid & 32) == 0) {
#pragma unroll
    for (int x = 0; x < 10; ++x) s_red[wave][cq][x] = part[x];
  }
  __syncthreads();
  float tot[10];
#pragma unroll
  for (int x = 0; x < 10; ++x)
    tot[x] = s_red[0][cq][x] + s_red[1][cq][x] + s_red[2][cq][x] + s_red[3][cq][x];

  const float kqt = tot[8], uqt = tot[9];
  float wv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) wv[c] = s_wv[4 * cq + c];

  if (rg == 0) {
    float out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = fmaf(wv[c], kqt, fmaf(-tot[c], uqt, tot[4 + c]));
    const int64_t ob = nh * D + 4 * cq;
    if (p.o_bf16) {
      uint2 packed;
      packed.x = uint32_t(f32_to_bf16(out[0])) | (uint32_t(f32_to_bf16(out[1])) << 16);
      packed.y = uint32_t(f32_to_bf16(out[2])) | (uint32_t(f32_to_bf16(out[3])) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + ob) = packed;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.o) + ob) =
          make_float4(out[0], out[1], out[2], out[3]);
    }
  }

  // S_new = S' - u m^T + k (w v)^T, written back in place.
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = rg + 8 * i;
    const float u = s_u[r], kr = s_k[r];
    f32x4 x = s[i];
    x.x = fmaf(-u, tot[0], fmaf(kr, wv[0], x.x));
    x.y = fmaf(-u, tot[1], fmaf(kr, wv[1], x.y));
    x.z = fmaf(-u, tot[2], fmaf(kr, wv[2], x.z));
    x.w = fmaf(-u, tot[3], fmaf(kr, wv[3], x.w));
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(S + r * D) + cq);
  }
}

template <bool kBf16, bool kDecayCh, bool kEraseCh>
hipError_t launch_w(const Problem& p, hipStream_t stream) {
  dim3 grid(unsigned(int64_t(p.B) * p.H));
  if (p.write_channel)
    hipLaunchKernelGGL((decode128_kernel<kBf16, kDecayCh, kEraseCh, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode128_kernel<kBf16, kDecayCh, kEraseCh, false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool kBf16, bool kDecayCh>
hipError_t launch_e(const Problem& p, hipStream_t stream) {
  return p.erase_channel ? launch_w<kBf16, kDecayCh, true>(p, stream)
                         : launch_w<kBf16, kDecayCh, false>(p, stream);
}

template <bool kBf16>
hipError_t launch_d(const Problem& p, hipStream_t stream) {
  return p.decay_channel ? launch_e<kBf16, true>(p, stream) : launch_e<kBf16, false>(p, stream);
}

}  // namespace

hipError_t launch_decode128(const Problem& p, hipStream_t stream) {
  return p.qkv_bf16 ? launch_d<true>(p, stream) : launch_d<false>(p, stream);
}

}  // namespace dr
