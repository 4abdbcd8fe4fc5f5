// Chunkwise-parallel forward of the gated delta rule on gfx950 matrix cores (bf16 q/k/v,
// dk == dv == 128, chunk C = 64).
//
// Keeping each token's update a rank-1 (Householder-like) correction lets a chunk of C
// updates fold into dense products through a triangular solve (WY / UT representation), and
// per-channel rates keep the diagonal-plus-low-rank chunk structure ("FG2-GDN ...", section 2
// on preserving symmetry and section 3 on DPLR compatibility with chunked training); the
// in-chunk states are rebuilt from the chunk's boundary state ("Linearized 2-Simplicial
// Attention", method: architecture and implementation).
//
// Per chunk, with incoming state S, chunk-local cumulative log-decay g_t (per channel) and a
// per-channel reference gm (g at the chunk midpoint), the kernel forms
//   K+ = k e^{g - gm}, Q+ = q e^{g - gm}, K- = k e^{gm - g}, U- = (e * k) e^{gm - g}
//   A_kk = strict_lower(K+ K-^T)  A_ku = strict_lower(K+ U-^T)  A_qk = lower(Q+ K-^T)
//   A_qu = lower(Q+ U-^T)          X_K = K+ S~,  X_Q = Q+ S~,  S~ = Diag(e^{gm}) S
// symmetric gates (one beta for erase and write):
//   T = (I + Diag(beta) A_kk)^{-1},  delta = T Diag(beta) (V - X_K)
//   O = X_Q + A_qk delta,            S <- Diag(e^{g_C}) S + Diag(e^{g_C - gm}) K-^T delta
// general gates (erase e, write w; Vt = w * v):
//   T = (I + A_ku)^{-1},  M = T (X_K + A_kk Vt)
//   O = X_Q + A_qk Vt - A_qu M,  S <- Diag(e^{g_C}) S + Diag(e^{g_C - gm}) (K-^T Vt - U-^T M)
// Products use v_mfma_f32_16x16x32_f16 (fp16 operands, fp32 accumulation); the triangular
// solve is fp32 forward substitution on the four 16x16 diagonal blocks plus 16x16x16 matrix-
// core products for the off-diagonal blocks; the state stays fp32 in registers for the whole
// sequence.  One workgroup (4 waves) owns one (b, h) and DVS value columns of its state.
//
// Range: the midpoint reference keeps every fp16 operand within e^{+-(half-chunk decay)}.  The
// exponents are clamped at 11 (e^11 < 65504), so a per-channel log-decay sum over half a chunk
// below -11 loses accuracy (the token-by-token path has no such limit).

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

typedef _Float16 half4v __attribute__((ext_vector_type(4)));

constexpr int C = 64;      // chunk length
constexpr int D = 128;     // dk == dv
constexpr int KS = 136;    // row stride (halves) of [64][128] tiles: 16-byte pad
constexpr int CS = 72;     // row stride (halves) of [*][64] tiles
constexpr int AFS = 65;    // row stride (floats) of the fp32 64 x 64 matrix
constexpr int kThreads = 256;
constexpr float kExpClamp = 11.f;

template <bool GEN, int DVS>
struct Layout {
  static constexpr int kp = 0;                          // K+  [64][KS] half
  static constexpr int qp = kp + C * KS * 2;            // Q+  [64][KS]
  static constexpr int km = qp + C * KS * 2;            // K-  [64][KS]
  static constexpr int um = km + C * KS * 2;            // U-  [64][KS]      (general)
  static constexpr int st = um + (GEN ? C * KS * 2 : 0);  // S~^T [DVS][KS]
  static constexpr int af = st + DVS * KS * 2;          // A for the solve, fp32 [64][AFS]
  static constexpr int th = af + C * AFS * 4;           // T      [64][CS] half
  static constexpr int aq = th + C * CS * 2;            // A_qk   [64][CS]
  static constexpr int akk = aq + C * CS * 2;           // A_kk   [64][CS]   (general)
  static constexpr int aqu = akk + (GEN ? C * CS * 2 : 0);  // A_qu [64][CS] (general)
  static constexpr int rt = aqu + (GEN ? C * CS * 2 : 0);   // R^T / Y^T [DVS][CS]
  static constexpr int dt = rt + DVS * CS * 2;          // delta^T / (-M)^T [DVS][CS]
  static constexpr int vt = dt + DVS * CS * 2;          // V [64][DVS+8] or Vt^T [DVS][CS]
  static constexpr int vstride = GEN ? CS : DVS + 8;
  static constexpr int vbytes = GEN ? DVS * CS * 2 : C * (DVS + 8) * 2;
  static constexpr int gb = vt + vbytes;                // per-token erase / beta [64] f32
  static constexpr int gw = gb + C * 4;                 // per-token write [64] f32 (general)
  static constexpr int gsc = gw + C * 4;                // scan partials [4][128] f32
  static constexpr int total = gsc + 4 * D * 4;
};

// Lower-triangular 16x16 tile (I, J), I >= J, enumerated row by row.
__device__ __forceinline__ void tile_ij(int idx, int& I, int& J) {
  I = idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3;
  J = idx - (I * (I + 1)) / 2;
}

// Operand fragment for v_mfma_f32_16x16x32_f16 from a tile whose rows are the fragment's
// rows (A operand) or columns (B operand) and whose contraction index is contiguous.
__device__ __forceinline__ half8 frag(const _Float16* base, int stride, int row0, int k0, int lane) {
  return *reinterpret_cast<const half8*>(base + (row0 + (lane & 15)) * stride + k0 + 8 * (lane >> 4));
}

// A-operand fragment of the transposed tile: rows are channels d (contiguous in the row-major
// [t][d] tile), contraction over tokens t.
__device__ __forceinline__ half8 frag_t(const _Float16* base, int d0, int t0, int lane) {
  half8 a;
  const _Float16* p = base + (t0 + 8 * (lane >> 4)) * KS + d0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = p[i * KS];
  return a;
}

__device__ __forceinline__ f32x4 mfma16(half4v a, half4v b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 cvt8(float x0, float x1, float x2, float x3, float x4, float x5,
                                      float x6, float x7) {
  half8 h;
  h[0] = (_Float16)x0; h[1] = (_Float16)x1; h[2] = (_Float16)x2; h[3] = (_Float16)x3;
  h[4] = (_Float16)x4; h[5] = (_Float16)x5; h[6] = (_Float16)x6; h[7] = (_Float16)x7;
  return h;
}

__device__ __forceinline__ void bf16x8_to_f32(uint4 u, float* f) {
  f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xffff0000u);
}

__device__ __forceinline__ float clamped_exp(float x) { return __expf(fminf(x, kExpClamp)); }

// Value-slice words per thread: DVS/4 bf16 values.
template <int DVS> struct VRaw;
template <> struct VRaw<16> { uint2 w; };
template <> struct VRaw<32> { uint4 w; };
template <> struct VRaw<64> { uint4 w[2]; };

template <int DVS>
__device__ __forceinline__ void vraw_load(VRaw<DVS>& v, const uint16_t* p, bool valid) {
  if constexpr (DVS == 16) {
    v.w = valid ? *reinterpret_cast<const uint2*>(p) : make_uint2(0, 0);
  } else if constexpr (DVS == 32) {
    v.w = valid ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
  } else {
    v.w[0] = valid ? reinterpret_cast<const uint4*>(p)[0] : make_uint4(0, 0, 0, 0);
    v.w[1] = valid ? reinterpret_cast<const uint4*>(p)[1] : make_uint4(0, 0, 0, 0);
  }
}

template <int DVS>
__device__ __forceinline__ void vraw_f32(const VRaw<DVS>& v, float* f) {
  if constexpr (DVS == 16) {
    f[0] = __uint_as_float(v.w.x << 16); f[1] = __uint_as_float(v.w.x & 0xffff0000u);
    f[2] = __uint_as_float(v.w.y << 16); f[3] = __uint_as_float(v.w.y & 0xffff0000u);
  } else if constexpr (DVS == 32) {
    bf16x8_to_f32(v.w, f);
  } else {
    bf16x8_to_f32(v.w[0], f);
    bf16x8_to_f32(v.w[1], f + 8);
  }
}

template <bool DCH, bool GEN, int DVS>
__global__ __launch_bounds__(kThreads) void chunk_kernel(Problem p) {
  using L = Layout<GEN, DVS>;
  constexpr int NCT = DVS / 16;   // 16-column tiles of the value slice
  constexpr int VPT = DVS / 4;    // value columns per thread in the V load
  __shared__ __attribute__((aligned(16))) char smem[L::total];
  _Float16* KP = reinterpret_cast<_Float16*>(smem + L::kp);
  _Float16* QP = reinterpret_cast<_Float16*>(smem + L::qp);
  _Float16* KM = reinterpret_cast<_Float16*>(smem + L::km);
  _Float16* UM = reinterpret_cast<_Float16*>(smem + L::um);
  _Float16* ST = reinterpret_cast<_Float16*>(smem + L::st);
  float* AF = reinterpret_cast<float*>(smem + L::af);
  _Float16* TH = reinterpret_cast<_Float16*>(smem + L::th);
  _Float16* AQ = reinterpret_cast<_Float16*>(smem + L::aq);
  _Float16* AKK = reinterpret_cast<_Float16*>(smem + L::akk);
  _Float16* AQU = reinterpret_cast<_Float16*>(smem + L::aqu);
  _Float16* RT = reinterpret_cast<_Float16*>(smem + L::rt);
  _Float16* DT = reinterpret_cast<_Float16*>(smem + L::dt);
  _Float16* VT = reinterpret_cast<_Float16*>(smem + L::vt);
  float* GB = reinterpret_cast<float*>(smem + L::gb);
  float* GW = reinterpret_cast<float*>(smem + L::gw);
  float* GSC = reinterpret_cast<float*>(smem + L::gsc);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh - b * p.H;
  const int j0 = blockIdx.y * DVS;
  const int T = p.T, H = p.H;
  const int nchunks = (T + C - 1) / C;
  const uint16_t* kin = static_cast<const uint16_t*>(p.k);
  const uint16_t* qin = static_cast<const uint16_t*>(p.q);
  const uint16_t* vin = static_cast<const uint16_t*>(p.v);
  float* out = static_cast<float*>(p.o);

  // Matrices whose upper-triangular blocks are read as zeros by full-width fragments.
  for (int i = tid; i < C * CS; i += kThreads) {
    TH[i] = (_Float16)0.f;
    AQ[i] = (_Float16)0.f;
    if constexpr (GEN) {
      AKK[i] = (_Float16)0.f;
      AQU[i] = (_Float16)0.f;
    }
  }

  // State: wave w owns rows [32 w, 32 w + 32) x the DVS columns, as 2 x NCT accumulator tiles
  // (lane: column 16 ct + l16, rows 32 w + 16 rt + 4 lg + r).
  f32x4 S[2][NCT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 32 * wave + 16 * rt + 4 * lg + r;
        S[rt][ct][r] = p.S0 ? p.S0[(int64_t(bh) * D + d) * D + j0 + 16 * ct + l16] : 0.f;
      }

  // Load mapping: thread = (token quad tg, channel octet d8): tokens 4 tg + r, channels
  // 8 d8 .. 8 d8 + 7; value slice: token tid / 4, columns VPT (tid % 4) .. + VPT - 1.
  const int d8 = tid & 15, tg = tid >> 4;
  const int vtok = tid >> 2, vcol = (tid & 3) * VPT;

  // Prefetch registers.
  uint4 kr[4], qr[4];
  float ldr[DCH ? 4 : 1][DCH ? 8 : 1];
  float err[GEN ? 4 : 1][GEN ? 8 : 1];
  float lds = 0.f, gbs = 0.f, gws = 0.f;  // per-token (head) gates for token tid (< 64)
  VRaw<DVS> vr;
  float wr[GEN ? VPT : 1];

  auto tok = [&](int t) { return (int64_t(b) * T + t) * H + h; };

  auto load = [&](int c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = c * C + 4 * tg + r;
      const bool ok = t < T;
      const int64_t base = ok ? tok(t) * D + 8 * d8 : 0;
      kr[r] = ok ? *reinterpret_cast<const uint4*>(kin + base) : make_uint4(0, 0, 0, 0);
      qr[r] = ok ? *reinterpret_cast<const uint4*>(qin + base) : make_uint4(0, 0, 0, 0);
      if constexpr (DCH) {
        float4 a0 = ok ? *reinterpret_cast<const float4*>(p.log_decay + base) : make_float4(0, 0, 0, 0);
        float4 a1 = ok ? *reinterpret_cast<const float4*>(p.log_decay + base + 4) : make_float4(0, 0, 0, 0);
        ldr[r][0] = a0.x; ldr[r][1] = a0.y; ldr[r][2] = a0.z; ldr[r][3] = a0.w;
        ldr[r][4] = a1.x; ldr[r][5] = a1.y; ldr[r][6] = a1.z; ldr[r][7] = a1.w;
      }
      if constexpr (GEN) {
        if (p.erase_channel) {
          float4 e0 = ok ? *reinterpret_cast<const float4*>(p.erase + base) : make_float4(0, 0, 0, 0);
          float4 e1 = ok ? *reinterpret_cast<const float4*>(p.erase + base + 4) : make_float4(0, 0, 0, 0);
          err[r][0] = e0.x; err[r][1] = e0.y; err[r][2] = e0.z; err[r][3] = e0.w;
          err[r][4] = e1.x; err[r][5] = e1.y; err[r][6] = e1.z; err[r][7] = e1.w;
        }
      }
    }
    if (tid < C) {
      const int t = c * C + tid;
      const bool ok = t < T;
      const int64_t ti = ok ? tok(t) : 0;
      if constexpr (!DCH) lds = ok ? p.log_decay[ti] : 0.f;
      if constexpr (GEN) {
        gbs = (ok && !p.erase_channel) ? p.erase[ti] : 0.f;
        gws = (ok && !p.write_channel) ? p.write[ti] : 0.f;
      } else {
        gbs = ok ? p.erase[ti] : 0.f;
      }
    }
    {
      const int t = c * C + vtok;
      const bool ok = t < T;
      const int64_t vb = ok ? tok(t) * D + j0 + vcol : 0;
      vraw_load<DVS>(vr, vin + vb, ok);
      if constexpr (GEN) {
        if (p.write_channel) {
#pragma unroll
          for (int i = 0; i < VPT; i += 4) {
            float4 w4 = ok ? *reinterpret_cast<const float4*>(p.write + vb + i) : make_float4(0, 0, 0, 0);
            wr[i] = w4.x; wr[i + 1] = w4.y; wr[i + 2] = w4.z; wr[i + 3] = w4.w;
          }
        }
      }
    }
  };

  load(0);

  for (int c = 0; c < nchunks; ++c) {
    // ---- L1: chunk-local cumulative log-decay ------------------------------------------
    float g[4][DCH ? 8 : 1];
    if (tid < C) {
      GB[tid] = gbs;
      if constexpr (GEN) GW[tid] = gws;
    }
    if constexpr (DCH) {
      float ex[8];
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc += ldr[r][ch];
          g[r][ch] = acc;
        }
        // inclusive scan of the quad totals over the 4 token quads of this wave (lanes 16 apart)
        float x = acc, y;
        y = __shfl_up(x, 16);
        if (lg >= 1) x += y;
        y = __shfl_up(x, 32);
        if (lg >= 2) x += y;
        ex[ch] = x - acc;
        if (lg == 3) GSC[wave * D + 8 * d8 + ch] = x;
      }
      __syncthreads();
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        float pre = ex[ch];
        for (int w = 0; w < wave; ++w) pre += GSC[w * D + 8 * d8 + ch];
#pragma unroll
        for (int r = 0; r < 4; ++r) g[r][ch] += pre;
      }
    } else {
      if (wave == 0) {
        float x = lds;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        GSC[lane] = x;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r) g[r][0] = GSC[4 * tg + r];
    }
    auto gmid = [&](int d) { return DCH ? GSC[d] + GSC[D + d] : GSC[31]; };
    auto gend = [&](int d) {
      return DCH ? GSC[d] + GSC[D + d] + GSC[2 * D + d] + GSC[3 * D + d] : GSC[63];
    };

    // ---- L2: operand tiles ---------------------------------------------------------------
    {
      float gm[8];
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) gm[ch] = gmid(8 * d8 + ch);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * tg + r;
        float kf[8], qf[8], fp[8], fm[8];
        bf16x8_to_f32(kr[r], kf);
        bf16x8_to_f32(qr[r], qf);
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          const float gg = DCH ? g[r][ch] : g[r][0];
          fp[ch] = clamped_exp(gg - gm[ch]);
          fm[ch] = clamped_exp(gm[ch] - gg);
        }
        *reinterpret_cast<half8*>(KP + t * KS + 8 * d8) =
            cvt8(kf[0] * fp[0], kf[1] * fp[1], kf[2] * fp[2], kf[3] * fp[3], kf[4] * fp[4],
                 kf[5] * fp[5], kf[6] * fp[6], kf[7] * fp[7]);
        *reinterpret_cast<half8*>(QP + t * KS + 8 * d8) =
            cvt8(qf[0] * fp[0], qf[1] * fp[1], qf[2] * fp[2], qf[3] * fp[3], qf[4] * fp[4],
                 qf[5] * fp[5], qf[6] * fp[6], qf[7] * fp[7]);
        float km[8];
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) km[ch] = kf[ch] * fm[ch];
        *reinterpret_cast<half8*>(KM + t * KS + 8 * d8) =
            cvt8(km[0], km[1], km[2], km[3], km[4], km[5], km[6], km[7]);
        if constexpr (GEN) {
          float e[8];
          if (p.erase_channel) {
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) e[ch] = err[r][ch];
          } else {
            const float eb = GB[t];
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) e[ch] = eb;
          }
          *reinterpret_cast<half8*>(UM + t * KS + 8 * d8) =
              cvt8(e[0] * km[0], e[1] * km[1], e[2] * km[2], e[3] * km[3], e[4] * km[4],
                   e[5] * km[5], e[6] * km[6], e[7] * km[7]);
        }
      }
      // value slice
      float vf[VPT];
      vraw_f32<DVS>(vr, vf);
      if constexpr (GEN) {
        const float wb = GW[vtok];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
          const float w = p.write_channel ? wr[i] : wb;
          VT[(vcol + i) * CS + vtok] = (_Float16)(w * vf[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < VPT; ++i) VT[vtok * L::vstride + vcol + i] = (_Float16)vf[i];
      }
    }
    // S~^T = (Diag(e^{gm}) S)^T and the per-row end-of-chunk factors of this wave's rows.
    float fC[2][4], fCm[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float em[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 32 * wave + 16 * rt + 4 * lg + r;
        const float gmd = gmid(d), gCd = gend(d);
        em[r] = clamped_exp(gmd);
        fC[rt][r] = expf(gCd);
        fCm[rt][r] = clamped_exp(gCd - gmd);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        half4v hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = (_Float16)(em[r] * S[rt][ct][r]);
        *reinterpret_cast<half4v*>(ST + (16 * ct + l16) * KS + 32 * wave + 16 * rt + 4 * lg) = hv;
      }
    }
    __syncthreads();
    if (c + 1 < nchunks) load(c + 1);  // overlaps the matrix work of this chunk

    // ---- G: Gram matrices and X = [K+; Q+] S~ ------------------------------------------
    constexpr int NG = GEN ? 40 : 20;
    for (int idx = wave; idx < NG; idx += 4) {
      const int which = idx / 10;  // 0: A_kk, 1: A_qk, 2: A_ku, 3: A_qu
      int I, J;
      tile_ij(idx - 10 * which, I, J);
      const _Float16* Ab = (which == 1 || which == 3) ? QP : KP;
      const _Float16* Bb = (which >= 2) ? UM : KM;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(frag(Ab, KS, 16 * I, 32 * ks, lane), frag(Bb, KS, 16 * J, 32 * ks, lane), acc);
      const int i = 16 * J + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * I + 4 * lg + r;
        if (which == 0) {
          const float v = (i < t) ? acc[r] : 0.f;
          if constexpr (GEN)
            AKK[t * CS + i] = (_Float16)v;
          else
            AF[t * AFS + i] = GB[t] * v;
        } else if (which == 1) {
          AQ[t * CS + i] = (_Float16)((i <= t) ? acc[r] : 0.f);
        } else if (which == 2) {
          AF[t * AFS + i] = (i < t) ? acc[r] : 0.f;
        } else {
          AQU[t * CS + i] = (_Float16)((i <= t) ? acc[r] : 0.f);
        }
      }
    }
    f32x4 XK[NCT], XQ[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 xk = {0.f, 0.f, 0.f, 0.f}, xq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const half8 bs = frag(ST, KS, 16 * ct, 32 * ks, lane);
        xk = mfma16x16x32(frag(KP, KS, 16 * wave, 32 * ks, lane), bs, xk);
        xq = mfma16x16x32(frag(QP, KS, 16 * wave, 32 * ks, lane), bs, xq);
      }
      XK[ct] = xk;
      XQ[ct] = xq;
      if constexpr (!GEN) {
        // R = Diag(beta) (V - X_K), stored transposed
        half4v hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * wave + 4 * lg + r;
          const float vv = (float)VT[t * L::vstride + 16 * ct + l16];
          hv[r] = (_Float16)(GB[t] * (vv - xk[r]));
        }
        *reinterpret_cast<half4v*>(RT + (16 * ct + l16) * CS + 16 * wave + 4 * lg) = hv;
      }
    }
    __syncthreads();

    // ---- S1: inverse of the four 16x16 diagonal blocks (fp32 forward substitution) --------
    if (wave == 0) {
      const int blk = lg, col = l16;
      const float* Ab = AF + (16 * blk) * AFS + 16 * blk;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s0 = (r == col) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < r; i += 2) {
          s0 = fmaf(-Ab[r * AFS + i], x[i], s0);
          if (i + 1 < r) s1 = fmaf(-Ab[r * AFS + i + 1], x[i + 1], s1);
        }
        x[r] = s0 + s1;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) TH[(16 * blk + r) * CS + 16 * blk + col] = (_Float16)x[r];
    }
    if constexpr (GEN) {
      // Y = X_K + A_kk Vt, stored transposed (B operand of M = T Y)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 y = XK[ct];
        for (int ks = 0; ks <= (wave >> 1); ++ks)
          y = mfma16x16x32(frag(AKK, CS, 16 * wave, 32 * ks, lane), frag(VT, CS, 16 * ct, 32 * ks, lane), y);
        half4v hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = (_Float16)y[r];
        *reinterpret_cast<half4v*>(RT + (16 * ct + l16) * CS + 16 * wave + 4 * lg) = hv;
      }
    }
    __syncthreads();

    // ---- S2: off-diagonal blocks, T_JI = -T_JJ sum_{K=I}^{J-1} A_JK T_KI -----------------
#pragma unroll
    for (int Jb = 1; Jb < 4; ++Jb) {
      if (wave < Jb) {
        const int Ib = wave;
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
        for (int Kb = Ib; Kb < Jb; ++Kb) {
          // the fp32 rows are 65 floats apart (bank spread), so read them one by one
          const float* arow = AF + (16 * Jb + l16) * AFS + 16 * Kb + 4 * lg;
          half4v a, bt;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] = (_Float16)arow[i];
            bt[i] = TH[(16 * Kb + 4 * lg + i) * CS + 16 * Ib + l16];
          }
          P = mfma16(a, bt, P);
        }
        half4v nb, a2;
#pragma unroll
        for (int i = 0; i < 4; ++i) nb[i] = (_Float16)(-P[i]);
        a2 = *reinterpret_cast<const half4v*>(TH + (16 * Jb + l16) * CS + 16 * Jb + 4 * lg);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 Tji = mfma16(a2, nb, z);
#pragma unroll
        for (int r = 0; r < 4; ++r) TH[(16 * Jb + 4 * lg + r) * CS + 16 * Ib + l16] = (_Float16)Tji[r];
      }
      __syncthreads();
    }

    // ---- D: delta = T R (symmetric) or -M = -(T Y) (general), stored transposed ---------
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks <= (wave >> 1); ++ks)
        acc = mfma16x16x32(frag(TH, CS, 16 * wave, 32 * ks, lane), frag(RT, CS, 16 * ct, 32 * ks, lane), acc);
      half4v hv;
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = (_Float16)(GEN ? -acc[r] : acc[r]);
      *reinterpret_cast<half4v*>(DT + (16 * ct + l16) * CS + 16 * wave + 4 * lg) = hv;
    }
    __syncthreads();

    // ---- O: chunk output rows [16 w, 16 w + 16) ------------------------------------------
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 acc = XQ[ct];
      for (int ks = 0; ks <= (wave >> 1); ++ks) {
        if constexpr (GEN) {
          acc = mfma16x16x32(frag(AQ, CS, 16 * wave, 32 * ks, lane), frag(VT, CS, 16 * ct, 32 * ks, lane), acc);
          acc = mfma16x16x32(frag(AQU, CS, 16 * wave, 32 * ks, lane), frag(DT, CS, 16 * ct, 32 * ks, lane), acc);
        } else {
          acc = mfma16x16x32(frag(AQ, CS, 16 * wave, 32 * ks, lane), frag(DT, CS, 16 * ct, 32 * ks, lane), acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = c * C + 16 * wave + 4 * lg + r;
        if (t < T) out[tok(t) * D + j0 + 16 * ct + l16] = acc[r];
      }
    }

    // ---- S: state update for this wave's rows ---------------------------------------------
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x4 acc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const half8 ak = frag_t(KM, 32 * wave + 16 * rt, 32 * ks, lane);
        half8 au;
        if constexpr (GEN) au = frag_t(UM, 32 * wave + 16 * rt, 32 * ks, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const half8 bd = frag(DT, CS, 16 * ct, 32 * ks, lane);
          if constexpr (GEN) {
            acc[ct] = mfma16x16x32(ak, frag(VT, CS, 16 * ct, 32 * ks, lane), acc[ct]);
            acc[ct] = mfma16x16x32(au, bd, acc[ct]);
          } else {
            acc[ct] = mfma16x16x32(ak, bd, acc[ct]);
          }
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[rt][ct][r] = fmaf(fC[rt][r], S[rt][ct][r], fCm[rt][r] * acc[ct][r]);
    }
    __syncthreads();
  }

  if (p.S_T) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 32 * wave + 16 * rt + 4 * lg + r;
          p.S_T[(int64_t(bh) * D + d) * D + j0 + 16 * ct + l16] = S[rt][ct][r];
        }
  }
}

template <bool DCH, bool GEN, int DVS>
hipError_t launch_cfg(const Problem& p, hipStream_t stream) {
  dim3 grid(unsigned(p.B * p.H), unsigned(D / DVS));
  hipLaunchKernelGGL((chunk_kernel<DCH, GEN, DVS>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool DCH, bool GEN>
hipError_t launch_dvs(const Problem& p, hipStream_t stream) {
  // Fill the 256 compute units with (b, h, value-slice) workgroups while keeping the slices
  // (each recomputes its chunk's Gram matrices and solve) as wide as that allows.
  const int64_t bh = int64_t(p.B) * p.H;
  if constexpr (!GEN) {
    if (bh >= 128) return launch_cfg<DCH, GEN, 64>(p, stream);
  }
  if (bh >= 64) return launch_cfg<DCH, GEN, 32>(p, stream);
  return launch_cfg<DCH, GEN, 16>(p, stream);
}

}  // namespace

hipError_t launch_chunk128(const Problem& p, hipStream_t stream) {
  const bool symmetric = !p.erase_channel && !p.write_channel && p.write == p.erase;
  if (p.decay_channel)
    return symmetric ? launch_dvs<true, false>(p, stream) : launch_dvs<true, true>(p, stream);
  return symmetric ? launch_dvs<false, false>(p, stream) : launch_dvs<false, true>(p, stream);
}

}  // namespace dr
