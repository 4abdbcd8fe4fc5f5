// fp32 token-by-token gated delta-rule recurrence (any supported width, fp32 or bf16 q/k/v).
//
// This is the plain definition of one token step, evaluated in fp32 on the GPU:
//   S' = Diag(a_t) S,  m = S'^T k_t,  S = S' - (e_t * k_t) m^T + k_t (w_t * v_t)^T,  o_t = S^T q_t
// ("Gated DeltaNet-2: decoupling erase and write in linear attention", gate table: erase on
// the key side, write on the value side, channel decay from KDA; "FG2-GDN ...", section 2,
// update rule).  It serves the fp32 workloads, widths the matrix-core path does not cover,
// chunk == 1, and decode steps of other widths (in place: every state element is read and
// written by the same lane).  FG2's per-channel rate beta ("FG2-GDN ...", section 2, update
// rule) scales k and v by sqrt(beta) as they are loaded and leaves unit erase and write gates.  Over packed sequences of different lengths each workgroup takes
// its sequence's first token and length from the sequence table.
//
// Mapping: one wave per (b, h, group of 16 value columns).  Lane = column c (16) x row group
// (4); each lane keeps dk/4 rows of its column in registers, so the two reductions over dk per
// token (k^T S' and q^T S) are a register sum plus two cross-lane steps.

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int kCols = 16;
constexpr int kGroups = 4;

__device__ __forceinline__ float group_sum(float x) {
  // Sum over the 4 lanes that share a column: lanes c, c+16, c+32, c+48.
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <int DK>
__global__ __launch_bounds__(64) void recurrent_kernel(Problem p) {
  constexpr int RPL = DK / kGroups;
  const int lane = threadIdx.x;
  const int c = lane & (kCols - 1);
  const int grp = lane >> 4;
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh - b * p.H;
  const int dv = p.dv;
  const int j = blockIdx.y * kCols + c;
  const int row0 = grp * RPL;
  const bool bf = p.qkv_bf16;

  const int64_t sbase = int64_t(bh) * DK * dv + j;
  float s[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) s[r] = p.S0 ? p.S0[sbase + int64_t(row0 + r) * dv] : 0.f;

  // Token rows of sequence b: a dense batch row, or a packed sequence from the table.
  int64_t tok0 = int64_t(b) * p.T;
  int len = p.T;
  if (p.seqs) {
    const int4 e = p.seqs[b];
    tok0 = e.x;
    len = e.y;
  }
  for (int t = 0; t < len; ++t) {
    const int64_t tok = (tok0 + t) * p.H + h;
    float kr[RPL], qr[RPL], ar[RPL], er[RPL];
    load_rows<RPL>(p.k, tok * DK + row0, bf, kr);
    load_rows<RPL>(p.q, tok * DK + row0, bf, qr);
    if (p.decay_channel) {
      load_f32_rows<RPL>(p.log_decay, tok * DK + row0, ar);
    } else {
      const float la = p.log_decay[tok];
#pragma unroll
      for (int r = 0; r < RPL; ++r) ar[r] = la;
    }
    if (p.erase_channel) {
      load_f32_rows<RPL>(p.erase, tok * DK + row0, er);
    } else {
      const float e = p.erase[tok];
#pragma unroll
      for (int r = 0; r < RPL; ++r) er[r] = e;
    }
    const float vj = load_qkv(p.v, tok * dv + j, bf);
    float wj = p.write_channel ? p.write[tok * dv + j] : p.write[tok];
    if (p.rate_sqrt) {
      // FG2's per-channel rate: key and value scaled by sqrt(beta), unit erase and write
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        kr[r] *= sqrtf(er[r]);
        er[r] = 1.f;
      }
      wj = sqrtf(wj);
    }

    float m = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      s[r] *= expf(ar[r]);   // S' = Diag(a_t) S
      m = fmaf(kr[r], s[r], m);
    }
    m = group_sum(m);  // (S'^T k_t)_j
    const float wv = wj * vj;
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      s[r] = fmaf(-er[r] * kr[r], m, fmaf(kr[r], wv, s[r]));
      o = fmaf(qr[r], s[r], o);
    }
    o = group_sum(o);
    if (grp == 0) store_o(p.o, tok * dv + j, o, p.o_bf16);
  }
  if (p.S_T) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) p.S_T[sbase + int64_t(row0 + r) * dv] = s[r];
  }
}

__global__ __launch_bounds__(256) void state_copy_kernel(const float4* src, float4* dst, int64_t n4) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride)
    dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_recurrent(const Problem& p, hipStream_t stream) {
  dim3 grid(p.B * p.H, p.dv / kCols);
  switch (p.dk) {
    case 16: hipLaunchKernelGGL(recurrent_kernel<16>, grid, dim3(64), 0, stream, p); break;
    case 32: hipLaunchKernelGGL(recurrent_kernel<32>, grid, dim3(64), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(recurrent_kernel<64>, grid, dim3(64), 0, stream, p); break;
    case 128: hipLaunchKernelGGL(recurrent_kernel<128>, grid, dim3(64), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t recurrent_varlen_workspace_bytes(int nseq) {
  return size_t((int64_t(nseq) * 16 + 255) / 256 * 256 + 256);
}

hipError_t launch_recurrent_varlen(Problem p, const int* cu, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  int4* seqs = reinterpret_cast<int4*>(ws);
  int* total = reinterpret_cast<int*>(ws + (int64_t(p.B) * 16 + 255) / 256 * 256);
  hipError_t e = launch_varlen_setup(cu, p.B, p.T, p.H, 64, seqs, nullptr, total, nullptr, stream);
  if (e != hipSuccess) return e;
  p.seqs = seqs;
  return launch_recurrent(p, stream);
}

hipError_t launch_state_copy(const float* S0, float* S_T, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;  // state sizes are multiples of 16 x 16 floats
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(state_copy_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(S0), reinterpret_cast<float4*>(S_T), n4);
  return hipGetLastError();
}

}  // namespace dr
