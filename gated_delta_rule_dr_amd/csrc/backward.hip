// Gradients of the gated delta-rule recurrence: the adjoint of the token loop, in fp32.
//
// Training runs the recurrence forward and needs its gradients ("FG2-GDN ...", sections 2-3:
// chunk-parallel training of the update).  For L = sum(o * dO) + sum(S_T * dS_T), walking the
// tokens backwards with the state's adjoint G = dL/dS_t (from dS_T), token t of
//     S' = Diag(a) S_{t-1},  m = S'^T k,  u = e * k,  v~ = w * v,
//     S_t = S' - u m^T + k v~^T,  o_t = S_t^T q_t
// gives (in this order)
//     G += q dO^T;  dq = S_t dO;  dm = -G^T u;  du = -G m;  dv~ = G^T k;
//     dk = G v~ + S' dm + e * du;  de = k * du;  dw = v * dv~;  dv = w * dv~;
//     G' = G + k dm^T;  d(log a) = a * rowsum(G' * S_{t-1});  G = Diag(a) G'
// and dS0 is G after token 0.
//
// Kernel 1, one wave per (b, h, group of 16 value columns), with the token kernel's mapping
// (lane = column (16) x row group (4), dk / 4 rows of one column per lane):
//   pass 1 runs the forward and stores the state at the start of every 64-token chunk;
//   pass 2 takes the chunks backwards: it recomputes the chunk's states from its checkpoint
//   into a scratch area of its own, then walks the chunk's tokens backwards through the adjoint
//   above.  Column sums (m, dm, dv~) are lane sums plus two cross-lane steps; row sums (the
//   per-row parts of dq, du, dk and d(log a), summed over this wave's 16 columns) are reduced
//   over the 16 column lanes and stored per column group.
// Kernel 2 sums the column groups' row parts, applies the per-row factors (e, k, a) and forms
// the gate gradients (summed over channels for a per-head gate; the erase and write parts added
// for a shared gate).
// Every state value is read and written by the lane that owns it, so neither pass needs a
// barrier; the two kernels are ordered by the stream.

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int kCols = 16;   // value columns per wave
constexpr int kGroups = 4;  // row groups per wave
constexpr int CK = 64;      // tokens per checkpoint

__device__ __forceinline__ float group_sum(float x) {  // over the 4 lanes of one column
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float column_sum(float x) {  // over the 16 lanes of one row group
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

// Workspace layout of the backward (offsets in floats).
struct BwdLayout {
  int64_t nslice, nck, bth;
  int64_t ckpt, states, parts, tmp_dw, total;
  __host__ __device__ BwdLayout(const Problem& p) {
    nslice = p.dv / kCols;
    nck = (int64_t(p.T) + CK - 1) / CK;
    bth = int64_t(p.B) * p.T * p.H;
    const int64_t waves = int64_t(p.B) * p.H * nslice;
    ckpt = 0;                                             // [waves][nck][dk][16]
    states = ckpt + waves * nck * p.dk * kCols;           // [waves][CK][dk][16]
    parts = states + waves * CK * p.dk * kCols;           // [4][nslice][bth][dk]
    tmp_dw = parts + 4 * nslice * bth * p.dk;             // [bth][dv]: v * dv~
    total = tmp_dw + bth * p.dv;
  }
};

template <int DK>
__global__ __launch_bounds__(64) void bwd_token_kernel(Problem p, BwdArgs g, float* __restrict__ ws) {
  constexpr int RPL = DK / kGroups;
  const int lane = threadIdx.x;
  const int c = lane & (kCols - 1);
  const int grp = lane >> 4;
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh - b * p.H;
  const int dv = p.dv;
  const int slice = blockIdx.y;
  const int j = slice * kCols + c;
  const int row0 = grp * RPL;
  const bool bf = p.qkv_bf16;
  const int T = p.T;
  const BwdLayout L(p);
  const int64_t wave_id = int64_t(bh) * L.nslice + slice;
  float* ck = ws + L.ckpt + wave_id * L.nck * DK * kCols;
  float* st = ws + L.states + wave_id * CK * DK * kCols;
  auto at = [&](int r) { return (row0 + r) * kCols + c; };  // this lane's element of a state slice

  struct Tok {
    float k[RPL], a[RPL], e[RPL];
    float v, w;
  };
  auto load_tok = [&](Tok& x, int64_t tok) {
    float la[RPL];
    load_rows<RPL>(p.k, tok * DK + row0, bf, x.k);
    if (p.decay_channel) {
      load_f32_rows<RPL>(p.log_decay, tok * DK + row0, la);
    } else {
      const float l = p.log_decay[tok];
#pragma unroll
      for (int r = 0; r < RPL; ++r) la[r] = l;
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r) x.a[r] = expf(la[r]);
    if (p.erase_channel) {
      load_f32_rows<RPL>(p.erase, tok * DK + row0, x.e);
    } else {
      const float e = p.erase[tok];
#pragma unroll
      for (int r = 0; r < RPL; ++r) x.e[r] = e;
    }
    x.v = load_qkv(p.v, tok * dv + j, bf);
    x.w = p.write_channel ? p.write[tok * dv + j] : p.write[tok];
  };
  // one forward token: s <- S_t from s = S_{t-1}
  auto step = [&](float (&s)[RPL], const Tok& x) {
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      s[r] *= x.a[r];
      m = fmaf(x.k[r], s[r], m);
    }
    m = group_sum(m);
    const float wv = x.w * x.v;
#pragma unroll
    for (int r = 0; r < RPL; ++r) s[r] = fmaf(-x.e[r] * x.k[r], m, fmaf(x.k[r], wv, s[r]));
  };
  auto token = [&](int t) { return (int64_t(b) * T + t) * p.H + h; };

  // ---- pass 1: forward, checkpoint every CK tokens -------------------------------------------
  float s[RPL];
  const int64_t sbase = int64_t(bh) * DK * dv + j;
#pragma unroll
  for (int r = 0; r < RPL; ++r) s[r] = p.S0 ? p.S0[sbase + int64_t(row0 + r) * dv] : 0.f;
  for (int t = 0; t < T; ++t) {
    if (t % CK == 0) {
      float* dst = ck + int64_t(t / CK) * DK * kCols;
#pragma unroll
      for (int r = 0; r < RPL; ++r) dst[at(r)] = s[r];
    }
    Tok x;
    load_tok(x, token(t));
    step(s, x);
  }

  // ---- pass 2: the adjoint, chunk by chunk from the last ----------------------------------------
  float G[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) G[r] = g.dS_T ? g.dS_T[sbase + int64_t(row0 + r) * dv] : 0.f;
  float* parts = ws + L.parts;
  const int64_t pstride = L.nslice * L.bth * DK;  // between the four row-part arrays
  for (int64_t ci = L.nck - 1; ci >= 0; --ci) {
    const int t0 = int(ci * CK), t1 = t0 + CK < T ? t0 + CK : T;
    const float* src = ck + ci * DK * kCols;
#pragma unroll
    for (int r = 0; r < RPL; ++r) s[r] = src[at(r)];
    for (int t = t0; t < t1; ++t) {  // S_{t-1} of every token of the chunk
      float* dst = st + int64_t(t - t0) * DK * kCols;
#pragma unroll
      for (int r = 0; r < RPL; ++r) dst[at(r)] = s[r];
      Tok x;
      load_tok(x, token(t));
      step(s, x);
    }
    for (int t = t1 - 1; t >= t0; --t) {
      const int64_t tok = token(t);
      Tok x;
      load_tok(x, tok);
      float qr[RPL], sp[RPL];
      load_rows<RPL>(p.q, tok * DK + row0, bf, qr);
      const float* prv = st + int64_t(t - t0) * DK * kCols;
#pragma unroll
      for (int r = 0; r < RPL; ++r) sp[r] = prv[at(r)];
      const float dO = g.dO[tok * dv + j];
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < RPL; ++r) m = fmaf(x.k[r], x.a[r] * sp[r], m);
      m = group_sum(m);
      const float vw = x.w * x.v;
      // row parts, summed over this wave's 16 columns; lane c stores rows r = c (mod 16)
      float* pbase = parts + (int64_t(slice) * L.bth + tok) * DK + row0;
      auto put = [&](int r, int which, float val) {
        const float sum = column_sum(val);
        if ((r & (kCols - 1)) == c) pbase[which * pstride + r] = sum;
      };
      float dm = 0.f, dvw = 0.f;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const float Sp = x.a[r] * sp[r];
        const float St = fmaf(-x.e[r] * x.k[r], m, fmaf(x.k[r], vw, Sp));
        G[r] = fmaf(qr[r], dO, G[r]);
        put(r, 0, St * dO);    // dq
        put(r, 1, -G[r] * m);  // du
        dm = fmaf(-G[r] * x.e[r], x.k[r], dm);
        dvw = fmaf(G[r], x.k[r], dvw);
      }
      dm = group_sum(dm);
      dvw = group_sum(dvw);
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const float Sp = x.a[r] * sp[r];
        put(r, 2, fmaf(G[r], vw, Sp * dm));  // dk, less the erase part
        const float Gp = fmaf(x.k[r], dm, G[r]);
        put(r, 3, Gp * sp[r]);  // d(log a) / a
        G[r] = x.a[r] * Gp;
      }
      if (grp == 0) {
        g.dv[tok * dv + j] = x.w * dvw;
        ws[L.tmp_dw + tok * dv + j] = x.v * dvw;
      }
    }
  }
  if (g.dS0) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) g.dS0[sbase + int64_t(row0 + r) * dv] = G[r];
  }
}

// Sum over the workgroup (128 threads).
__device__ float block_sum128(float x, float* red) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  if ((tid & 63) == 0) red[tid >> 6] = x;
  __syncthreads();
  const float s = red[0] + red[1];
  __syncthreads();
  return s;
}

// One workgroup of 128 threads per token (b, t, h); thread i < dk is row i, i < dv column i.
__global__ __launch_bounds__(128) void bwd_reduce_kernel(Problem p, BwdArgs g, const float* __restrict__ ws) {
  __shared__ float red[2];
  const BwdLayout L(p);
  const int64_t tok = blockIdx.x;
  const int i = threadIdx.x;
  const int dk = p.dk, dv = p.dv;
  const float* parts = ws + L.parts;
  const int64_t pstride = L.nslice * L.bth * dk;
  float sq = 0.f, sdu = 0.f, skw = 0.f, sda = 0.f;
  float de = 0.f, dla = 0.f, dwv = 0.f;
  if (i < dk) {
    for (int64_t s = 0; s < L.nslice; ++s) {
      const float* pb = parts + (s * L.bth + tok) * dk + i;
      sq += pb[0];
      sdu += pb[pstride];
      skw += pb[2 * pstride];
      sda += pb[3 * pstride];
    }
    const float k = load_qkv(p.k, tok * dk + i, p.qkv_bf16);
    const float e = p.erase_channel ? p.erase[tok * dk + i] : p.erase[tok];
    const float a = expf(p.decay_channel ? p.log_decay[tok * dk + i] : p.log_decay[tok]);
    g.dq[tok * dk + i] = sq;
    g.dk[tok * dk + i] = fmaf(e, sdu, skw);
    de = k * sdu;
    dla = a * sda;
  }
  if (i < dv) dwv = ws[L.tmp_dw + tok * dv + i];
  // decay
  if (p.decay_channel) {
    if (i < dk) g.dlog_decay[tok * dk + i] = dla;
  } else {
    const float s = block_sum128(dla, red);
    if (i == 0) g.dlog_decay[tok] = s;
  }
  // erase and write (a shared gate takes both parts; dk == dv when it is per channel)
  const bool shared = g.dwrite == nullptr;
  if (p.erase_channel) {
    if (i < dk) g.derase[tok * dk + i] = shared ? de + dwv : de;
  } else {
    const float s = block_sum128(shared ? de + dwv : de, red);
    if (i == 0) g.derase[tok] = s;
  }
  if (!shared) {
    if (p.write_channel) {
      if (i < dv) g.dwrite[tok * dv + i] = dwv;
    } else {
      const float s = block_sum128(dwv, red);
      if (i == 0) g.dwrite[tok] = s;
    }
  }
}

}  // namespace

size_t bwd_workspace_bytes(const Problem& p) { return size_t(BwdLayout(p).total) * 4; }

hipError_t launch_bwd(const Problem& p, const BwdArgs& g, void* workspace, hipStream_t stream) {
  float* ws = static_cast<float*>(workspace);
  dim3 grid(unsigned(p.B * p.H), unsigned(p.dv / kCols));
  switch (p.dk) {
    case 16: hipLaunchKernelGGL(bwd_token_kernel<16>, grid, dim3(64), 0, stream, p, g, ws); break;
    case 32: hipLaunchKernelGGL(bwd_token_kernel<32>, grid, dim3(64), 0, stream, p, g, ws); break;
    case 64: hipLaunchKernelGGL(bwd_token_kernel<64>, grid, dim3(64), 0, stream, p, g, ws); break;
    case 128: hipLaunchKernelGGL(bwd_token_kernel<128>, grid, dim3(64), 0, stream, p, g, ws); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t bth = int64_t(p.B) * p.T * p.H;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(unsigned(bth)), dim3(128), 0, stream, p, g, ws);
  return hipGetLastError();
}

}  // namespace dr
