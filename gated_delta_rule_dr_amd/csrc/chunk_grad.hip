// Gradients through the matrix-core chunk path, chunk by chunk on the matrix cores.
//
// Training runs the chunked forward and needs its gradients ("FG2-GDN ...", sections 2-3: the WY
// form keeps a chunk of rank-1 updates a set of dense products, which is what makes chunk-parallel
// training possible; "Linearized 2-Simplicial Attention", method: the backward is a second scan
// over the chunks).  With general gates (erase e, write w; u = e * k, Vt = w * v) a chunk with
// incoming state S computes
//   M = (I + A_ku)^{-1} (K+ S + A_kk Vt),  O = Q+ S + A_qk Vt - A_qu M,
//   S_C = Diag(e^{g_C}) S + K^end^T Vt - U^end^T M,
// and for the adjoint G of S_C and dO of O, reverse mode through these products gives
//   Z     = -(I + A_ku)^{-T} (A_qu^T dO + U^end G)                 (the adjoint scan)
//   dK+   = Z S^T,   dQ+ = dO S^T,   dK^end = Vt G^T,   dU^end = -M G^T,   dGamma = rowsum(S * G)
//   dA_kk = strict(Z Vt^T),  dA_ku = -strict(Z M^T),  dA_qk = lower(dO Vt^T),  dA_qu = -lower(dO M^T)
//   dVt   = A_kk^T Z + A_qk^T dO + K^end G.
// One scalar gate per head (u = beta k, Vt = beta v) is the same algebra, so those problems run
// the general-gate forward and adjoint scans here.  With FG2's rate (u = k~, unit gates) A_ku =
// A_kk, A_qu = A_qk and U^end = K^end, so the adjoints merge: dA_kk = strict(Z Delta^T), dA_qk =
// lower(dO Delta^T), dK^end = Delta G^T with Delta = Vt - M (the symmetric scan's delta), and
// dVt = -Z.
//
// Kernel 1 (one workgroup of eight waves per chunk): the products above, from the chunk's
// incoming state (stored by the forward scan), its end adjoint and Z (stored by the adjoint
// scan), M (forward scan), dO, Vt and the packet's A_kk, A_qk, K^end; fp16 operands, fp32
// results into the workspace.
//
// Kernel 2 (one workgroup of four waves per chunk): the adjoints of the Gram matrices
// A_xy[t, i] = sum_d x_t,d y_i,d e^{g_t,d - g_i,d}:
//   dx_t = sum_i dA[t, i] y_i e^{g_t - g_i},   dy_i = sum_t dA[t, i] x_t e^{g_t - g_i},
// with g's adjoint taking x * dx on the row side and -y * dy on the column side.  An off-diagonal
// 16-token block (I, J), J < I, is one product dA_IJ Y~_J (and dA_IJ^T X~_I) of operands
// referenced inside their own block -- Y~ = y e^{g_r - g} with r the last token of J, X~ =
// x e^{g - g_s} with s the last token before I -- scaled by e^{g_s - g_r} per channel and by the
// row's own factor, so every factor is e^{x} with x <= 0 (no decay in (0, 1] overflows); the
// diagonal blocks are summed element by element in fp32 with the exact factor.  Then the chain
// rule through the decayed operands (K+ = k e^{g}: g takes K+ * dK+, and so on; e^{g_C} and the
// end-referenced operands add their share at the chunk's last token) and the gates, and the
// log-decay's adjoint as the reverse prefix sum of g's over the chunk.  Channels are taken 32 at a
// time (the Gram adjoints are independent per channel); per-head gate gradients are summed over
// channels in a fixed order, so the results are deterministic.

#include "chunk_layout.h"
#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int kG1Threads = 512;
constexpr int kG2Threads = 512;
constexpr int P1 = 136;  // row stride (halves) of fp16 [*][128] LDS tiles
constexpr int P2 = 72;   // row stride (halves) of fp16 [*][64] LDS tiles
constexpr float kLog2e = 1.4426950408889634f;

// Kernel-1 results per chunk: five fp32 [C][D] matrices dK+, dQ+, dK^end, dU^end, dVt; four fp16
// [C][C] matrices dA_kk, dA_ku, dA_qk, dA_qu (kernel 2 multiplies them as fp16 operands);
// dGamma [D] fp32.
constexpr int64_t kGkFloats = 5 * C * D;
constexpr int64_t kGaHalves = 4 * C * C;
enum { GK_KP = 0, GK_QP = 1, GK_KE = 2, GK_UE = 3, GK_VT = 4 };
enum { GA_KK = 0, GA_KU = 1, GA_QK = 2, GA_QU = 3 };

struct GradWork {
  float* gk;  // [chunks][5][C][D]
  _Float16* ga;  // [chunks][4][C][C]
  float* gd;  // [chunks][D]
};

// A[row][k] = base[k][row] from a row-major tile of row stride `stride` (halves), as frag():
// lane 16 g + l16 receives base[k0 + 8 g + 0..7][r0 + l16] (r0 % 4 == 0, stride % 4 == 0).
__device__ __forceinline__ half8 fragT(const _Float16* base, int stride, int r0, int k0, int lane) {
  const int m = lane & 15;
  const int k = k0 + 8 * (lane >> 4) + (m >> 2), r = r0 + 4 * (m & 3);
  const half4v lo = ld_tr16(base + k * stride + r);
  const half4v hi = ld_tr16(base + (k + 4) * stride + r);
  return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Operands of v_mfma_f32_16x16x16_f16: lane l supplies A[row = l % 16][k = 4 (l / 16) + 0..3].
__device__ __forceinline__ half4v frag4N(const _Float16* base, int stride, int r0, int k0, int lane) {
  return *reinterpret_cast<const half4v*>(base + (r0 + (lane & 15)) * stride + k0 + 4 * (lane >> 4));
}
// ... and the same of A[row][k] = base[k][row]: lane 16 g + l16 receives base[k0 + 4 g + 0..3][r0 + l16].
__device__ __forceinline__ half4v frag4T(const _Float16* base, int stride, int r0, int k0, int lane) {
  const int m = lane & 15;
  return ld_tr16(base + (k0 + 4 * (lane >> 4) + (m >> 2)) * stride + r0 + 4 * (m & 3));
}

__device__ __forceinline__ half4v h4(float4 x) {
  return half4v{(_Float16)x.x, (_Float16)x.y, (_Float16)x.z, (_Float16)x.w};
}

// ------------------------------------------------------------------------------------------
// Kernel 1: the products with the state and its adjoint, and the Gram matrices' adjoints.
// ------------------------------------------------------------------------------------------
// MODE: general gates (the general-gate packet and M from the forward scan); one per-head gate
// (the symmetric packet, A_kk from the prep's side buffer, delta from the forward scan, and
// M = K+ S + A_kk delta formed here); FG2's rate (delta only, merged adjoints).
enum { kModeGen = 0, kModeSym = 1, kModeFg2 = 2 };

template <int MODE, bool DCH>
__global__ __launch_bounds__(kG1Threads) void chunk_grad_state_kernel(Problem p, const char* __restrict__ ws,
                                                                      const float* __restrict__ dO, GradWork gw) {
  constexpr bool FG2 = MODE == kModeFg2, SYM = MODE == kModeSym;
  constexpr bool SCAL = SYM && !DCH;  // plain k tiles with per-row factors in the packet
  using PK = Packet<SYM ? DCH : true, !SYM>;
  __shared__ __attribute__((aligned(16))) _Float16 SG[D * P1];  // S, then G: [d][j]
  __shared__ __attribute__((aligned(16))) _Float16 ZZ[C * P1];  // Z [t][j]
  __shared__ __attribute__((aligned(16))) _Float16 MM[C * P1];  // M (FG2: Delta; one gate: Delta, then M)
  __shared__ __attribute__((aligned(16))) _Float16 DO[C * P1];  // dO [t][j]
  __shared__ __attribute__((aligned(16))) _Float16 VV[C * P1];  // Vt [t][j]
  __shared__ __attribute__((aligned(16))) _Float16 AK[FG2 ? 8 : C * P2];  // A_kk [t][i]
  __shared__ __attribute__((aligned(16))) _Float16 AQ[FG2 ? 8 : C * P2];  // A_qk [t][i]
  __shared__ __attribute__((aligned(16))) _Float16 KE[FG2 ? 8 : C * P1];  // K^end [t][d] (one gate: K+ first)
  __shared__ float FAC[SCAL ? 2 * C : 1];  // one gate, per-head decay: e^{g_t}, e^{g_C - g_t}

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t pkt = blockIdx.x;
  const int nck = (p.T + C - 1) / C;
  const int bh = int(pkt / nck), ci = int(pkt - int64_t(bh) * nck);
  const int b = bh / p.H, h = bh - b * p.H;
  const int tlen = p.T - ci * C < C ? p.T - ci * C : C;
  const int64_t tok0 = (int64_t(b) * p.T + int64_t(ci) * C) * p.H + h;
  auto tok = [&](int t) { return tok0 + int64_t(t) * p.H; };
  const _Float16* Sg = static_cast<const _Float16*>(p.ck_S) + pkt * D * D;
  const _Float16* Gg = static_cast<const _Float16*>(p.ck_G) + pkt * D * D;
  const _Float16* Zg = static_cast<const _Float16*>(p.ck_Z) + pkt * C * D;
  const _Float16* Mg = static_cast<const _Float16*>(p.ck_M) + pkt * C * D;
  float* out_k = gw.gk + pkt * kGkFloats;
  _Float16* out_a = gw.ga + pkt * kGaHalves;

  // ---- loads ----------------------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // S: 2048 units of 8 halves
    const int u = tid + kG1Threads * i, d = u >> 4, j = (u & 15) * 8;
    *reinterpret_cast<uint4*>(SG + d * P1 + j) = *reinterpret_cast<const uint4*>(Sg + d * D + j);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // Z, M: 1024 units of 8 halves each
    const int u = tid + kG1Threads * i, t = u >> 4, j = (u & 15) * 8;
    *reinterpret_cast<uint4*>(ZZ + t * P1 + j) = *reinterpret_cast<const uint4*>(Zg + t * D + j);
    *reinterpret_cast<uint4*>(MM + t * P1 + j) = *reinterpret_cast<const uint4*>(Mg + t * D + j);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // dO: 2048 float4, zero past the last token
    const int f = tid + kG1Threads * i, t = f >> 5, j = (f & 31) * 4;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < tlen) x = *reinterpret_cast<const float4*>(dO + tok(t) * D + j);
    *reinterpret_cast<half4v*>(DO + t * P1 + j) = h4(x);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // Vt = w * v (FG2: sqrt(beta) v): 1024 units of 8 values
    const int u = tid + kG1Threads * i, t = u >> 4, j = (u & 15) * 8;
    float vf[8];
    for (int e = 0; e < 8; ++e) vf[e] = 0.f;
    if (t < tlen) {
      const int64_t x = tok(t);
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) + x * D + j), vf);
      if (FG2) {
        for (int e = 0; e < 8; ++e) vf[e] *= sqrtf(p.erase[x * D + j + e]);
      } else if (p.write_channel) {
        for (int e = 0; e < 8; ++e) vf[e] *= p.write[x * D + j + e];
      } else {
        const float w = p.write[x];
        for (int e = 0; e < 8; ++e) vf[e] *= w;
      }
    }
    *reinterpret_cast<half8*>(VV + t * P1 + j) = cvt8(vf);
  }
  if constexpr (!FG2) {
    const char* pk = ws + pkt * PK::bytes;
    // A_kk (packet matrix 2; one gate: the prep's side buffer) and A_qk (matrix 1): six stored
    // 16 x 32 blocks of 1 KB each
    const char* akk = SYM ? static_cast<const char*>(p.ck_A) + pkt * (6 * 1024) : pk + PK::mat + 2 * PK::matb;
    for (int u = tid; u < 768; u += kG1Threads) {
      const int m = u / 384, k = (u % 384) / 64, w64 = u % 64, r = w64 >> 2;
      const int lu = (w64 & 3) ^ ((r >> 2) & 3);
      const int I = k < 2 ? k : 2 + ((k - 2) >> 1), Hh = k < 2 ? 0 : ((k - 2) & 1);
      const char* src = m ? pk + PK::mat + PK::matb : akk;
      const uint4 x = *reinterpret_cast<const uint4*>(src + 1024 * k + 16 * w64);
      *reinterpret_cast<uint4*>((m ? AQ : AK) + (16 * I + r) * P2 + 32 * Hh + 8 * lu) = x;
    }
    if (tid < 256) {  // the upper blocks that the packet does not store
      const int m = tid >> 7, r = (tid >> 2) & 31, c8 = 32 + 8 * (tid & 3);
      *reinterpret_cast<uint4*>((m ? AQ : AK) + r * P2 + c8) = make_uint4(0, 0, 0, 0);
    }
    // K^end (one gate: K+ first): swizzled [64][128] tile
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + kG1Threads * i, t = u >> 4, pos = u & 15;
      *reinterpret_cast<uint4*>(KE + t * P1 + 8 * (pos ^ swz_key<16>(t))) =
          *reinterpret_cast<const uint4*>(pk + (SYM ? PK::kp : PK::kmt) + 16 * u);
    }
    if constexpr (SCAL) {
      if (tid < C) {
        const float* gv = reinterpret_cast<const float*>(pk + PK::gate);
        FAC[tid] = gv[GV_FP + tid];
        FAC[C + tid] = gv[GV_FM + tid];
      }
    }
  }
  __syncthreads();

  if constexpr (SYM) {
    // M = K+ S + A_kk delta (the in-chunk reads), transposed as below; then into MM
    f32x4 mt[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int n = wave + 8 * k, tm = n >> 3, tn = n & 7;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(fragT(SG, P1, 16 * tn, 32 * ks, lane), frag(KE, P1, 16 * tm, 32 * ks, lane), acc);
      if constexpr (SCAL) acc = acc * FAC[16 * tm + l16];  // K+ = Diag(e^{g}) k
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        acc = mfma16x16x32(fragT(MM, P1, 16 * tn, 32 * ks, lane), frag(AK, P2, 16 * tm, 32 * ks, lane), acc);
      mt[k] = acc;
    }
    __syncthreads();  // every read of delta and K+ is done
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int n = wave + 8 * k, tm = n >> 3, tn = n & 7;
      *reinterpret_cast<half4v*>(MM + (16 * tm + l16) * P1 + 16 * tn + 4 * lg) = cvt4(mt[k]);
    }
    // K^end: DCH, the packet's tile; per-head decay, plain k (the row factor goes on the product)
    if constexpr (DCH) {
      const char* pk = ws + pkt * PK::bytes;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = tid + kG1Threads * i, t = u >> 4, pos = u & 15;
        *reinterpret_cast<uint4*>(KE + t * P1 + 8 * (pos ^ swz_key<16>(t))) =
            *reinterpret_cast<const uint4*>(pk + PK::kmt + 16 * u);
      }
    }
    __syncthreads();
  }

  // One 16 x 16 output tile of out[m][n] = sum_k A[m][k] Bm[n][k] over k = 0 .. 32 NK - 1 of two
  // row-major tiles, computed transposed so that lane holds out[m0 + l16][n0 + 4 lg + 0..3].
  auto tileNN = [&](const _Float16* A, const _Float16* Bm, int m0, int n0, int NK) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < NK; ++ks)
      acc = mfma16x16x32(frag(Bm, P1, n0, 32 * ks, lane), frag(A, P1, m0, 32 * ks, lane), acc);
    return acc;
  };
  auto store4 = [&](float* dst, f32x4 x) { *reinterpret_cast<f32x4*>(dst) = x; };

  // ---- products with S, and the Gram adjoints ---------------------------------------------
  // tasks: 32 dK+ tiles, 32 dQ+ tiles, then 16 tiles of each Gram adjoint (upper ones zero)
  constexpr int NA = FG2 ? 2 : 4;
  for (int n = wave; n < 64 + 16 * NA; n += 8) {
    if (n < 64) {
      const int q = n >> 5, tm = (n >> 3) & 3, tn = n & 7;
      const f32x4 acc = tileNN(q ? DO : ZZ, SG, 16 * tm, 16 * tn, 4);
      store4(out_k + ((q ? GK_QP : GK_KP) * C + 16 * tm + l16) * D + 16 * tn + 4 * lg, acc);
    } else {
      const int a = (n - 64) >> 4, tm = ((n - 64) >> 2) & 3, tn = (n - 64) & 3;
      // FG2: dA_kk = Z Delta^T, dA_qk = dO Delta^T; general: Z Vt^T, -Z M^T, dO Vt^T, -dO M^T
      const int which = FG2 ? (a ? GA_QK : GA_KK) : a == 0 ? GA_KK : a == 1 ? GA_KU : a == 2 ? GA_QK : GA_QU;
      const bool rowz = which == GA_KK || which == GA_KU;
      const bool colm = FG2 || which == GA_KU || which == GA_QU;
      const float sgn = (!FG2 && colm) ? -1.f : 1.f;
      const bool strict = which == GA_KK || which == GA_KU;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (tn <= tm) {
        acc = tileNN(rowz ? ZZ : DO, colm ? MM : VV, 16 * tm, 16 * tn, 4);
        const int t = 16 * tm + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * tn + 4 * lg + r;
          acc[r] = (i < t || (!strict && i == t)) ? sgn * acc[r] : 0.f;
        }
      }
      *reinterpret_cast<half4v*>(out_a + (which * C + 16 * tm + l16) * C + 16 * tn + 4 * lg) = cvt4(acc);
    }
  }
  // dVt's tiles are kept by their wave across the load of G: wave w owns tiles w, w + 8, ...
  f32x4 dvt[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) dvt[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (!FG2) {
    // A_kk^T Z + A_qk^T dO: out[t][j] = sum_i A[i][t] X[i][j], transposed as above
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int n = wave + 8 * k, tm = n >> 3, tn = n & 7;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        acc = mfma16x16x32(fragT(ZZ, P1, 16 * tn, 32 * ks, lane), fragT(AK, P2, 16 * tm, 32 * ks, lane), acc);
        acc = mfma16x16x32(fragT(DO, P1, 16 * tn, 32 * ks, lane), fragT(AQ, P2, 16 * tm, 32 * ks, lane), acc);
      }
      dvt[k] = acc;
    }
  }
  __syncthreads();

  // ---- G, and dGamma = rowsum(S * G) in fp32 -----------------------------------------------
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + kG1Threads * i, d = u >> 4, j = (u & 15) * 8;
    const half8 g8 = *reinterpret_cast<const half8*>(Gg + d * D + j);
    const half8 s8 = *reinterpret_cast<const half8*>(SG + d * P1 + j);
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) x = fmaf(float(g8[e]), float(s8[e]), x);
    // the 16 threads of row d are lanes 16 (lane / 16) .. + 15 of one wave
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    if (l16 == 0) gw.gd[pkt * D + d] = x;
  }
  __syncthreads();  // every S read above is done
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + kG1Threads * i, d = u >> 4, j = (u & 15) * 8;
    *reinterpret_cast<uint4*>(SG + d * P1 + j) = *reinterpret_cast<const uint4*>(Gg + d * D + j);
  }
  __syncthreads();

  // ---- products with G ------------------------------------------------------------------
  for (int n = wave; n < (FG2 ? 32 : 64); n += 8) {
    const int q = n >> 5, tm = (n >> 3) & 3, tn = n & 7;
    // dK^end = Vt G^T (FG2: Delta G^T); dU^end = -M G^T
    f32x4 acc = tileNN((q || FG2) ? MM : VV, SG, 16 * tm, 16 * tn, 4);
    if (q) acc = -acc;
    store4(out_k + ((q ? GK_UE : GK_KE) * C + 16 * tm + l16) * D + 16 * tn + 4 * lg, acc);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = wave + 8 * k, tm = n >> 3, tn = n & 7;
    f32x4 acc = dvt[k];
    if constexpr (FG2) {
      // dVt = -Z
      const _Float16* z = ZZ + (16 * tm + l16) * P1 + 16 * tn + 4 * lg;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = -float(z[r]);
    } else {
      // + K^end G: out[t][j] = sum_d KE[t][d] G[d][j]
      f32x4 kg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kg = mfma16x16x32(fragT(SG, P1, 16 * tn, 32 * ks, lane), frag(KE, P1, 16 * tm, 32 * ks, lane), kg);
      if constexpr (SCAL) kg = kg * FAC[C + 16 * tm + l16];  // K^end = Diag(e^{g_C - g}) k
      acc += kg;
    }
    store4(out_k + (GK_VT * C + 16 * tm + l16) * D + 16 * tn + 4 * lg, acc);
  }
}

// ------------------------------------------------------------------------------------------
// Kernel 2: the Gram adjoints with their decays, the chain rule, the outputs.
// ------------------------------------------------------------------------------------------
template <bool DCH, bool FG2>
__global__ __launch_bounds__(kG2Threads) void chunk_grad_gram_kernel(Problem p, BwdArgs g, GradWork gw) {
  constexpr int NA = FG2 ? 2 : 4;      // Gram adjoints held: kk, qk (, ku, qu)
  constexpr int GS = D + 4;            // row stride (floats) of the per-channel g table
  __shared__ __attribute__((aligned(16))) _Float16 DA[4][C * P2];      // dA_kk, dA_ku, dA_qk, dA_qu [t][i]
  __shared__ __attribute__((aligned(16))) float GL[DCH ? C * GS : C];  // g log2(e) [t][c] (or [t])
  __shared__ __attribute__((aligned(16))) _Float16 XK[C * P1];         // k (FG2: k~) [t][c]
  __shared__ __attribute__((aligned(16))) _Float16 XQ[C * P1];         // q
  __shared__ __attribute__((aligned(16))) _Float16 XU[FG2 ? 8 : C * P1];  // u = e * k
  __shared__ __attribute__((aligned(16))) float BT[4][D];   // per block: g-adjoint totals, then shares
  __shared__ __attribute__((aligned(16))) float GNS[4][D];  // per block: end-referenced shares
  __shared__ float RED[3][2][C];                            // per-head sums (decay, erase, write)
  __shared__ float MISC[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int blk = wave & 3, hc = wave >> 2;  // this wave's 16 tokens and 64 channels
  const int64_t pkt = blockIdx.x;
  const int nck = (p.T + C - 1) / C;
  const int bh = int(pkt / nck), ci = int(pkt - int64_t(bh) * nck);
  const int b = bh / p.H, h = bh - b * p.H;
  const int tlen = p.T - ci * C < C ? p.T - ci * C : C;
  const int64_t tok0 = (int64_t(b) * p.T + int64_t(ci) * C) * p.H + h;
  auto tok = [&](int t) { return tok0 + int64_t(t) * p.H; };
  const float* gk = gw.gk + pkt * kGkFloats;
  const _Float16* ga = gw.ga + pkt * kGaHalves;
  const bool shared_gate = g.dwrite == nullptr;  // write gate == erase gate
  const int t_own = 16 * blk + l16;
  const bool own_ok = t_own < tlen;
  const int64_t x_own = tok(own_ok ? t_own : 0) * D;  // row of this lane's token (token 0 when padded)

  // the Gram adjoints, fp16
  for (int f = tid; f < NA * C * C / 4; f += kG2Threads) {
    const int m = f / (C * C / 4), r = f % (C * C / 4), t = r >> 4, i = (r & 15) * 4;
    const int which = FG2 ? (m ? GA_QK : GA_KK) : m;
    *reinterpret_cast<half4v*>(DA[which] + t * P2 + i) = *reinterpret_cast<const half4v*>(ga + (which * C + t) * C + i);
  }
  // k, q, u of every channel, fp16
  {
    const int t = tid >> 3, c16 = (tid & 7) * 16;
    float kf[16], qf[16], uf[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) kf[e] = qf[e] = uf[e] = 0.f;
    if (t < tlen) {
      const int64_t x = tok(t) * D + c16;
      const uint16_t* kp = static_cast<const uint16_t*>(p.k) + x;
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + x;
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(kp), kf);
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(kp + 8), kf + 8);
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(qp), qf);
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(qp + 8), qf + 8);
      if (FG2 || p.erase_channel) {
        float ef[16];
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(p.erase + x + e);
          ef[e] = v4.x; ef[e + 1] = v4.y; ef[e + 2] = v4.z; ef[e + 3] = v4.w;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (FG2) kf[e] *= sqrtf(ef[e]);
          else uf[e] = kf[e] * ef[e];
        }
      } else {
        const float e1 = p.erase[tok(t)];
#pragma unroll
        for (int e = 0; e < 16; ++e) uf[e] = kf[e] * e1;
      }
    }
    *reinterpret_cast<half8*>(XK + t * P1 + c16) = cvt8(kf);
    *reinterpret_cast<half8*>(XK + t * P1 + c16 + 8) = cvt8(kf + 8);
    *reinterpret_cast<half8*>(XQ + t * P1 + c16) = cvt8(qf);
    *reinterpret_cast<half8*>(XQ + t * P1 + c16 + 8) = cvt8(qf + 8);
    if constexpr (!FG2) {
      *reinterpret_cast<half8*>(XU + t * P1 + c16) = cvt8(uf);
      *reinterpret_cast<half8*>(XU + t * P1 + c16 + 8) = cvt8(uf + 8);
    }
  }
  // g: the chunk-local inclusive prefix sum of the log-decay, in log2 units
  if constexpr (DCH) {
    const int c = tid & 127, seg = tid >> 7;  // tokens 16 seg .. + 15 of channel c
    float gl[16], acc = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = 16 * seg + e;
      acc += t < tlen ? p.log_decay[tok(t) * D + c] : 0.f;
      gl[e] = acc;
    }
    BT[seg][c] = acc;
    __syncthreads();
    float base = 0.f;
    for (int s2 = 0; s2 < seg; ++s2) base += BT[s2][c];
#pragma unroll
    for (int e = 0; e < 16; ++e) GL[(16 * seg + e) * GS + c] = (base + gl[e]) * kLog2e;
  } else {
    if (wave == 0) {
      float x = lane < tlen ? p.log_decay[tok(lane)] : 0.f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      GL[lane] = x * kLog2e;
    }
  }
  __syncthreads();

  auto gl = [&](int t, int c) { return DCH ? GL[t * GS + c] : GL[t]; };
  // Operand fragment (rows c0 + l16, contraction over tokens tb + 4 lg + 0..3) of x e^{g_t - g_ref}
  // (inv = false) or x e^{g_ref - g_t} (inv = true).
  auto opfrag = [&](const _Float16* X, int c0, int tb, int ref, bool inv) {
    const int c = c0 + l16;
    const float gr = gl(ref, c);
    half4v f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tb + 4 * lg + j;
      const float d = gl(t, c) - gr;
      f[j] = (_Float16)(float(X[t * P1 + c]) * exp2f(inv ? -d : d));
    }
    return f;
  };
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int m_ref = 16 * blk + 7;  // the diagonal block's reference token
  constexpr float kSpan = 6.f * kLog2e;

  float s_e = 0.f, s_w = 0.f, s_g = 0.f;  // per-head sums over this lane's channels
  f32x4 dgv[4], gnv[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int c0 = 64 * hc + 16 * ct;   // channel tile
    const int cq = c0 + 4 * lg;         // this lane's output channels cq .. + 3
    // this lane's kernel-1 products and the raw inputs of the chain rule, issued before the
    // products of this tile
    f32x4 pk[5];
#pragma unroll
    for (int q = 0; q < 5; ++q)
      pk[q] = (FG2 && q == GK_UE) ? z4 : *reinterpret_cast<const f32x4*>(gk + (q * C + t_own) * D + cq);
    uint2 vb = make_uint2(0, 0), kb = make_uint2(0, 0);
    f32x4 e4 = {1.f, 1.f, 1.f, 1.f}, w4 = {1.f, 1.f, 1.f, 1.f};
    if (own_ok) {
      vb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.v) + x_own + cq);
      if (FG2) {
        kb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.k) + x_own + cq);
        e4 = *reinterpret_cast<const f32x4*>(p.erase + x_own + cq);
      } else {
        if (p.erase_channel) e4 = *reinterpret_cast<const f32x4*>(p.erase + x_own + cq);
        else e4 = f32x4{1.f, 1.f, 1.f, 1.f} * p.erase[x_own / D];
        if (p.write_channel) w4 = *reinterpret_cast<const f32x4*>(p.write + x_own + cq);
        else w4 = f32x4{1.f, 1.f, 1.f, 1.f} * p.write[x_own / D];
      }
    }

    // ---- row side (this block's tokens as rows): earlier blocks J, then the diagonal -------
    f32x4 rk = z4, rq = z4, ck = z4, cu = z4;
    for (int J = 0; J < blk; ++J) {
      const int r = 16 * J + 15, s = 16 * blk - 1;
      const half4v yk = opfrag(XK, c0, 16 * J, r, true);
      f32x4 tk = mfma16(yk, frag4N(DA[GA_KK], P2, 16 * blk, 16 * J, lane), z4);
      f32x4 tq = mfma16(yk, frag4N(DA[GA_QK], P2, 16 * blk, 16 * J, lane), z4);
      if constexpr (!FG2) {
        const half4v yu = opfrag(XU, c0, 16 * J, r, true);
        tk = mfma16(yu, frag4N(DA[GA_KU], P2, 16 * blk, 16 * J, lane), tk);
        tq = mfma16(yu, frag4N(DA[GA_QU], P2, 16 * blk, 16 * J, lane), tq);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float F = r == s ? 1.f : exp2f(gl(s, cq + e) - gl(r, cq + e));
        rk[e] = fmaf(F, tk[e], rk[e]);
        rq[e] = fmaf(F, tq[e], rq[e]);
      }
    }
    // ---- column side (this block's tokens as columns): later blocks I ----------------------
    for (int I = blk + 1; I < 4; ++I) {
      const int s = 16 * I - 1, r = 16 * blk + 15;
      const half4v xk = opfrag(XK, c0, 16 * I, s, false), xq = opfrag(XQ, c0, 16 * I, s, false);
      f32x4 tk = mfma16(xk, frag4T(DA[GA_KK], P2, 16 * blk, 16 * I, lane), z4);
      tk = mfma16(xq, frag4T(DA[GA_QK], P2, 16 * blk, 16 * I, lane), tk);
      f32x4 tu = z4;
      if constexpr (!FG2) {
        tu = mfma16(xk, frag4T(DA[GA_KU], P2, 16 * blk, 16 * I, lane), z4);
        tu = mfma16(xq, frag4T(DA[GA_QU], P2, 16 * blk, 16 * I, lane), tu);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float F = r == s ? 1.f : exp2f(gl(s, cq + e) - gl(r, cq + e));
        ck[e] = fmaf(F, tk[e], ck[e]);
        cu[e] = fmaf(F, tu[e], cu[e]);
      }
    }
    // the rows' own factors (to their reference: the token before the block, the block's last)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gt = gl(t_own, cq + e);
      const float fr = blk > 0 ? exp2f(gt - gl(16 * blk - 1, cq + e)) : 0.f;
      const float fc = blk < 3 ? exp2f(gl(16 * blk + 15, cq + e) - gt) : 0.f;
      rk[e] *= fr;
      rq[e] *= fr;
      ck[e] *= fc;
      cu[e] *= fc;
    }
    // ---- the diagonal block: referenced at its 8th token when every factor stays within
    // e^{+-6} and the operands below 80 (fp16 range), else element by element in fp32 ---------
    bool ok = true;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = gl(t_own, cq + e) - gl(m_ref, cq + e);
      const float ax = fmaxf(fabsf(float(XK[t_own * P1 + cq + e])), fabsf(float(XQ[t_own * P1 + cq + e])));
      const float au = FG2 ? 0.f : fabsf(float(XU[t_own * P1 + cq + e]));
      ok = ok && fabsf(d) <= kSpan && fmaxf(ax, au) <= 80.f;
    }
    if (__all(ok)) {
      const half4v yk = opfrag(XK, c0, 16 * blk, m_ref, true);
      const half4v xk = opfrag(XK, c0, 16 * blk, m_ref, false), xq = opfrag(XQ, c0, 16 * blk, m_ref, false);
      f32x4 tk = mfma16(yk, frag4N(DA[GA_KK], P2, 16 * blk, 16 * blk, lane), z4);
      f32x4 tq = mfma16(yk, frag4N(DA[GA_QK], P2, 16 * blk, 16 * blk, lane), z4);
      f32x4 sk = mfma16(xk, frag4T(DA[GA_KK], P2, 16 * blk, 16 * blk, lane), z4);
      sk = mfma16(xq, frag4T(DA[GA_QK], P2, 16 * blk, 16 * blk, lane), sk);
      f32x4 su = z4;
      if constexpr (!FG2) {
        const half4v yu = opfrag(XU, c0, 16 * blk, m_ref, true);
        tk = mfma16(yu, frag4N(DA[GA_KU], P2, 16 * blk, 16 * blk, lane), tk);
        tq = mfma16(yu, frag4N(DA[GA_QU], P2, 16 * blk, 16 * blk, lane), tq);
        su = mfma16(xk, frag4T(DA[GA_KU], P2, 16 * blk, 16 * blk, lane), z4);
        su = mfma16(xq, frag4T(DA[GA_QU], P2, 16 * blk, 16 * blk, lane), su);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = gl(t_own, cq + e) - gl(m_ref, cq + e);
        const float fr = exp2f(d), fc = exp2f(-d);
        rk[e] = fmaf(fr, tk[e], rk[e]);
        rq[e] = fmaf(fr, tq[e], rq[e]);
        ck[e] = fmaf(fc, sk[e], ck[e]);
        cu[e] = fmaf(fc, su[e], cu[e]);
      }
    } else {
#pragma unroll 1
      for (int i2 = 0; i2 < 16; ++i2) {
        const int o = 16 * blk + i2;
        const bool row_ok = i2 <= l16, col_ok = i2 >= l16;
        const float r_kk = float(DA[GA_KK][t_own * P2 + o]), r_qk = float(DA[GA_QK][t_own * P2 + o]);
        const float c_kk = float(DA[GA_KK][o * P2 + t_own]), c_qk = float(DA[GA_QK][o * P2 + t_own]);
        float r_ku = 0.f, r_qu = 0.f, c_ku = 0.f, c_qu = 0.f;
        if constexpr (!FG2) {
          r_ku = float(DA[GA_KU][t_own * P2 + o]);
          r_qu = float(DA[GA_QU][t_own * P2 + o]);
          c_ku = float(DA[GA_KU][o * P2 + t_own]);
          c_qu = float(DA[GA_QU][o * P2 + t_own]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float go = gl(o, cq + e), gt = gl(t_own, cq + e);
          const float ko = float(XK[o * P1 + cq + e]), qo = float(XQ[o * P1 + cq + e]);
          const float uo = FG2 ? 0.f : float(XU[o * P1 + cq + e]);
          const float er = row_ok ? exp2f(gt - go) : 0.f;
          const float ec = col_ok ? exp2f(go - gt) : 0.f;
          rk[e] = fmaf(er, fmaf(r_kk, ko, r_ku * uo), rk[e]);
          rq[e] = fmaf(er, fmaf(r_qk, ko, r_qu * uo), rq[e]);
          ck[e] = fmaf(ec, fmaf(c_kk, ko, c_qk * qo), ck[e]);
          cu[e] = fmaf(ec, fmaf(c_ku, ko, c_qu * qo), cu[e]);
        }
      }
    }

    // ---- chain rule, outputs ------------------------------------------------------------
    const f32x4 dkp = pk[GK_KP], dqp = pk[GK_QP], dke = pk[GK_KE], due = pk[GK_UE], dvt = pk[GK_VT];
    float vv[4], kraw[4];
    vv[0] = __uint_as_float(vb.x << 16);
    vv[1] = __uint_as_float(vb.x & 0xffff0000u);
    vv[2] = __uint_as_float(vb.y << 16);
    vv[3] = __uint_as_float(vb.y & 0xffff0000u);
    kraw[0] = __uint_as_float(kb.x << 16);
    kraw[1] = __uint_as_float(kb.x & 0xffff0000u);
    kraw[2] = __uint_as_float(kb.y << 16);
    kraw[3] = __uint_as_float(kb.y & 0xffff0000u);
    f32x4 o_dq, o_dk, o_dv, o_de, o_dw = z4, dgt, gnt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = cq + e;
      const float gt = gl(t_own, c);
      const float eg = exp2f(gt), egn = exp2f(gl(C - 1, c) - gt);
      const float kk = float(XK[t_own * P1 + c]), qq = float(XQ[t_own * P1 + c]);
      const float uu = FG2 ? 0.f : float(XU[t_own * P1 + c]);
      const float a_kp = eg * dkp[e], a_qp = eg * dqp[e], a_ke = egn * dke[e], a_ue = egn * due[e];
      const float dkap = a_kp + a_ke + rk[e] + ck[e];
      const float du = a_ue + cu[e];
      o_dq[e] = a_qp + rq[e];
      dgt[e] = kk * (a_kp - a_ke + rk[e] - ck[e]) + qq * (a_qp + rq[e]) - uu * (a_ue + cu[e]);
      gnt[e] = kk * a_ke + uu * a_ue;
      if (FG2) {
        const float rt = sqrtf(e4[e]);
        o_dk[e] = rt * dkap;
        o_dv[e] = rt * dvt[e];
        o_de[e] = own_ok ? (kraw[e] * dkap + vv[e] * dvt[e]) / (2.f * rt) : 0.f;
      } else {
        // k's adjoint with the erase gate's share (u = e * k); the fp16 table holds k exactly
        o_dk[e] = fmaf(e4[e], du, dkap);
        o_de[e] = kk * du;
        o_dv[e] = w4[e] * dvt[e];
        o_dw[e] = vv[e] * dvt[e];
        if (shared_gate) o_de[e] += o_dw[e];
      }
      s_e += o_de[e];
      s_w += o_dw[e];
      s_g += dgt[e];
    }
    dgv[ct] = dgt;
    gnv[ct] = gnt;
    if (own_ok) {
      *reinterpret_cast<f32x4*>(g.dq + x_own + cq) = o_dq;
      *reinterpret_cast<f32x4*>(g.dk + x_own + cq) = o_dk;
      *reinterpret_cast<f32x4*>(g.dv + x_own + cq) = o_dv;
      if (FG2 || p.erase_channel) *reinterpret_cast<f32x4*>(g.derase + x_own + cq) = o_de;
      if (!FG2 && !shared_gate && p.write_channel) *reinterpret_cast<f32x4*>(g.dwrite + x_own + cq) = o_dw;
    }
  }

  // ---- g's adjoint: suffix sums within the block (lanes of one lane group are its 16 tokens),
  // block totals and the end-referenced shares through LDS --------------------------------------
  __syncthreads();  // BT held the prefix-sum totals
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = dgv[ct][e];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float y = __shfl_down(v, o, 16);
        if (l16 + o < 16) v += y;
      }
      dgv[ct][e] = v;
      float n = gnv[ct][e];
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) n += __shfl_xor(n, o);
      const int c = 64 * hc + 16 * ct + 4 * lg + e;
      if (l16 == 0) {
        BT[blk][c] = v;
        GNS[blk][c] = n;
      }
    }
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    s_e += __shfl_xor(s_e, o);
    s_w += __shfl_xor(s_w, o);
    s_g += __shfl_xor(s_g, o);
  }
  if (lg == 0) {
    RED[0][hc][t_own] = s_g;
    RED[1][hc][t_own] = s_e;
    RED[2][hc][t_own] = s_w;
  }
  __syncthreads();
  if constexpr (DCH) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int cq = 64 * hc + 16 * ct + 4 * lg;
      f32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = cq + e;
        float later = 0.f;
        for (int b2 = blk + 1; b2 < 4; ++b2) later += BT[b2][c];
        const float dgn = exp2f(gl(C - 1, c)) * gw.gd[pkt * D + c] + GNS[0][c] + GNS[1][c] + GNS[2][c] + GNS[3][c];
        out[e] = dgv[ct][e] + later + dgn;
      }
      if (own_ok) *reinterpret_cast<f32x4*>(g.dlog_decay + x_own + cq) = out;
    }
  } else {
    // g_C's share summed over channels (waves 0 and 1: one channel per thread)
    if (wave < 2) {
      const int c = tid;
      float n = exp2f(gl(C - 1, c)) * gw.gd[pkt * D + c] + GNS[0][c] + GNS[1][c] + GNS[2][c] + GNS[3][c];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o);
      if (lane == 0) MISC[wave] = n;
    }
    __syncthreads();
    if (tid < C) {
      float s = MISC[0] + MISC[1];
      for (int t2 = C - 1; t2 >= tid; --t2) s += RED[0][0][t2] + RED[0][1][t2];
      if (tid < tlen) g.dlog_decay[tok(tid)] = s;
    }
  }
  if (tid < tlen) {
    if (!FG2 && !p.erase_channel) g.derase[tok(tid)] = RED[1][0][tid] + RED[1][1][tid];
    if (!FG2 && !shared_gate && !p.write_channel) g.dwrite[tok(tid)] = RED[2][0][tid] + RED[2][1][tid];
  }
}

template <int MODE, bool DCH>
void launch_state(const Problem& p, const char* ws, const float* dO, GradWork gw, int64_t nchunks,
                  hipStream_t stream) {
  hipLaunchKernelGGL((chunk_grad_state_kernel<MODE, DCH>), dim3(unsigned(nchunks)), dim3(kG1Threads), 0, stream, p,
                     ws, dO, gw);
}

template <bool DCH, bool FG2>
void launch_gram(const Problem& p, const BwdArgs& g, GradWork gw, int64_t nchunks, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_grad_gram_kernel<DCH, FG2>), dim3(unsigned(nchunks)), dim3(kG2Threads), 0, stream, p, g,
                     gw);
}

}  // namespace

size_t chunk_grad_work_bytes(const Problem& p) {
  const int64_t nchunks = int64_t(p.B) * p.H * ((int64_t(p.T) + C - 1) / C);
  return size_t(nchunks * ((kGkFloats + D) * 4 + kGaHalves * 2));
}

hipError_t launch_chunk_grad(const Problem& p, const BwdArgs& g, const void* packets, void* work,
                             hipStream_t stream) {
  const int64_t nchunks = int64_t(p.B) * p.H * ((int64_t(p.T) + C - 1) / C);
  if (nchunks == 0) return hipSuccess;
  float* w = static_cast<float*>(work);
  GradWork gw{w, reinterpret_cast<_Float16*>(w + nchunks * (kGkFloats + D)), w + nchunks * kGkFloats};
  const char* ws = static_cast<const char*>(packets);
  if (p.rate_sqrt) {
    launch_state<kModeFg2, false>(p, ws, g.dO, gw, nchunks, stream);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    if (p.decay_channel) launch_gram<true, true>(p, g, gw, nchunks, stream);
    else launch_gram<false, true>(p, g, gw, nchunks, stream);
  } else {
    if (!p.symmetric) launch_state<kModeGen, false>(p, ws, g.dO, gw, nchunks, stream);
    else if (p.decay_channel) launch_state<kModeSym, true>(p, ws, g.dO, gw, nchunks, stream);
    else launch_state<kModeSym, false>(p, ws, g.dO, gw, nchunks, stream);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    if (p.decay_channel) launch_gram<true, false>(p, g, gw, nchunks, stream);
    else launch_gram<false, false>(p, g, gw, nchunks, stream);
  }
  return hipGetLastError();
}

}  // namespace dr
