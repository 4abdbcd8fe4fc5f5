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
// One scalar gate per head (u = beta k, Vt = beta v) is the same algebra; its forward scan yields
// delta instead of M, and the prep keeps A_kk aside, so M = K+ S + A_kk delta is rebuilt here (no
// division by beta, which may be 0).  With FG2's rate (u = k~, unit gates) A_ku = A_kk, A_qu =
// A_qk and U^end = K^end, so the adjoints merge: dA_kk = strict(Z Delta^T), dA_qk =
// lower(dO Delta^T), dK^end = Delta G^T with Delta = Vt - M (the symmetric scan's delta), and
// dVt = -Z.
//
// Through the Gram matrices A_xy[t, i] = sum_d x_t,d y_i,d e^{g_t,d - g_i,d}:
//   dx_t = sum_i dA[t, i] y_i e^{g_t - g_i},   dy_i = sum_t dA[t, i] x_t e^{g_t - g_i},
// with g's adjoint taking x * dx on the row side and -y * dy on the column side.  An off-diagonal
// 16-token block (I, J), J < I, is one product dA_IJ Y~_J (and dA_IJ^T X~_I) of operands
// referenced inside their own block -- Y~ = y e^{g_r - g} with r the last token of J, X~ =
// x e^{g - g_s} with s the last token before I -- scaled by e^{g_s - g_r} per channel and by the
// row's own factor, so every factor is e^{x} with x <= 0 (no decay in (0, 1] overflows).  A
// diagonal block is one product referenced at its 8th token when every factor stays within e^{+-6}
// and the operands below 80, else it is summed element by element in fp32 with the exact factor.
// Then the chain rule through the decayed operands (K+ = k e^{g}: g takes K+ * dK+, and so on;
// e^{g_C} and the end-referenced operands add their share at the chunk's last token) and the
// gates, and the log-decay's adjoint as the reverse prefix sum of g's over the chunk.  Per-head
// gate gradients are summed over channels in a fixed order, so the results are deterministic.

#include "chunk_layout.h"
#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int P1 = 136;  // row stride (halves) of fp16 [*][128] LDS tiles
constexpr int P2 = 72;   // row stride (halves) of fp16 [*][64] LDS tiles
constexpr float kLog2e = 1.4426950408889634f;
enum { GA_KK = 0, GA_KU = 1, GA_QK = 2, GA_QU = 3 };  // the Gram adjoints
// what the forward stored: general gates (M); one per-head gate (delta and A_kk); FG2's rate (delta)
enum { kModeGen = 0, kModeSym = 1, kModeFg2 = 2 };

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
// The fused gradient kernel: one workgroup of eight waves per (chunk, half of the channels).
// Wave w owns the 16 tokens of block w % 4 and two 16-channel tiles of its half; every product
// it needs for its own outputs stays in its registers, in the lane layout of the Gram stage
// (lane: token 16 b + l16, channels c0 + 4 lg + 0..3).
//   phase 1 (LDS: S, Z, M or delta, dO, Vt, A_kk, A_qk, K+ or K^end): M for one gate; the Gram
//     adjoints dA (every tile, spread over the waves, kept as fp16 in registers); the wave's
//     dK+ = Z S^T and dQ+ = dO S^T; dVt's A_kk^T Z + A_qk^T dO;
//   phase 2 (G in place of S): dGamma of the half's channels; the wave's dK^end, dU^end and
//     dVt's K^end G;
//   phase 3 (the same LDS: dA, g, k, q, u of the half): the Gram adjoints with their decays,
//     the chain rule and the outputs; per-head gate and decay sums of the half go to `part` and
//     chunk_grad_sums_kernel adds the two halves.
// ------------------------------------------------------------------------------------------
// `x` through an empty asm: a load that is masked where it is used stays where it was issued
// (the compiler otherwise moves such a load into the branch it makes of the mask, and waits for
// it there).
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Sums across lanes on the VALU (DPP and the gfx950 row swaps) rather than through the LDS
// crossbar.  row_suffix: lane l of each 16-lane row gets the sum of lanes l .. 15 of its row
// (row shift left: lane l reads lane l + N, zero past the row's end).  cross_row_sum: every lane
// gets the sum of the four lanes with its position in the four rows (swapping rows 1 <-> 0 and
// 3 <-> 2 of a value with itself and adding both halves sums a pair of rows; the half-wave swap
// adds the other pair).
template <int N>
__device__ __forceinline__ float row_from_above(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_suffix(float x) {
  x += row_from_above<1>(x);
  x += row_from_above<2>(x);
  x += row_from_above<4>(x);
  x += row_from_above<8>(x);
  return x;
}
__device__ __forceinline__ float cross_row_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Half offsets of element (d, j) of a state checkpoint and of (t, j) of a row checkpoint within a
// chunk: 16-column tiles, [dv / 16][dk][16] and [dv / 16][C][16] (j % 8 == 0 for a 16-byte piece).
__device__ __forceinline__ int ck_state_off(int d, int j) { return (j >> 4) * (D * 16) + d * 16 + (j & 15); }
__device__ __forceinline__ int ck_rows_off(int t, int j) { return (j >> 4) * (C * 16) + t * 16 + (j & 15); }

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

constexpr int kFThreads = 512;
constexpr int PX = 72;             // row stride (halves) of the half's [64][64] k, q, u tables
constexpr int GSH = 68;            // row stride (floats) of the half's g table
constexpr int kPartFloats = 3 * C + 4;  // per (chunk, half): decay, erase, write sums per token; g_C share
constexpr int kArenaP12 = D * P1 * 2 + 4 * C * P1 * 2 + 2 * C * P2 * 2 + C * P1 * 2;  // 140,288 B
constexpr int kArena = kArenaP12 + 2 * C * 4 + 64 * 4;                                  // + FAC + DGAM

// GCH (general gates only): erase and write both per channel, fixed at compile time
template <int MODE, bool DCH, bool GCH>
__global__ __launch_bounds__(kFThreads) void chunk_grad_kernel(Problem p, BwdArgs g, const char* __restrict__ ws,
                                                               float* __restrict__ part, int64_t nitems) {
  constexpr bool FG2 = MODE == kModeFg2, SYM = MODE == kModeSym;
  constexpr bool SCAL = SYM && !DCH;
  constexpr int NA = FG2 ? 2 : 4;
  using PK = Packet<SYM ? DCH : true, !SYM>;
  __shared__ __attribute__((aligned(16))) char smem[kArena];
  // phases 1 and 2
  _Float16* const SG = reinterpret_cast<_Float16*>(smem);  // S, then G: [d][j]
  _Float16* const ZZ = SG + D * P1;                         // Z [t][j]
  _Float16* const MM = ZZ + C * P1;                         // M (FG2: delta; one gate: delta, then M)
  _Float16* const DO = MM + C * P1;                         // dO
  _Float16* const VV = DO + C * P1;                         // Vt
  _Float16* const AK = VV + C * P1;                         // A_kk [t][i]
  _Float16* const AQ = AK + C * P2;                         // A_qk
  _Float16* const KE = AQ + C * P2;                         // K^end [t][d] (one gate: K+ first)
  float* const FAC = reinterpret_cast<float*>(smem + kArenaP12);  // e^{g_t}, e^{g_C - g_t} (per-head decay)
  float* const DGAM = FAC + 2 * C;                                // dGamma of the half's channels
  // phase 3
  _Float16* const DA = reinterpret_cast<_Float16*>(smem);         // [4][64][P2]
  float* const GL = reinterpret_cast<float*>(smem + 4 * C * P2 * 2);  // g log2(e): [t][GSH] or [t]
  _Float16* const XK = reinterpret_cast<_Float16*>(GL + (DCH ? C * GSH : C));  // [t][PX]
  _Float16* const XQ = XK + C * PX;
  _Float16* const XU = XQ + C * PX;
  float* const BT = reinterpret_cast<float*>(XU + C * PX);  // [4][64] per block: suffix totals
  float* const GNS = BT + 4 * 64;                           // [4][64] per block: end shares
  float* const TOT = GNS + 4 * 64;                          // [8][64] prefix-sum segments
  float* const RED = TOT + 8 * 64;                          // [3][2][64] per-head sums of the two pairs
  float* const MISC = RED + 3 * 2 * 64;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int blk = wave & 3, pq = wave >> 2;  // this wave's block and channel pair
  // Work item = one chunk of one head (packed sequences: from the chunk table).  Workgroups are
  // dealt to the eight XCDs in turn (linear id mod 8), each with its own L2, so the two halves of
  // an item take ids 8 apart: the same XCD, one after the other, and the second half finds the
  // chunk's shared operands in that L2.
  const uint32_t lid = blockIdx.x;
  const int64_t item = int64_t((lid >> 4) << 3 | (lid & 7));
  const int half = (lid >> 3) & 1, ch0 = 64 * half;
  if (item >= nitems || (p.chunks && item >= int64_t(p.H) * *p.nchunks_total)) return;
  const ChunkRef cr = chunk_ref_of(p, item, (p.T + C - 1) / C);
  const int64_t pkt = cr.pkt;
  const int tlen = cr.tlen;
  auto tok = [&](int t) { return (cr.tok0 + t) * int64_t(p.H) + cr.h; };
  const _Float16* Sg = static_cast<const _Float16*>(p.ck_S) + pkt * D * D;
  const _Float16* Gg = static_cast<const _Float16*>(p.ck_G) + pkt * D * D;
  const _Float16* Zg = static_cast<const _Float16*>(p.ck_Z) + pkt * C * D;
  const _Float16* Mg = static_cast<const _Float16*>(p.ck_M) + pkt * C * D;
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int t_own = 16 * blk + l16;
  const bool own_ok = t_own < tlen;
  const int64_t x_own = tok(own_ok ? t_own : 0) * D;
  const bool shared_gate = g.dwrite == nullptr;
  // gate kinds: one gate per head on the symmetric path, FG2's rate per channel
  const bool ech = FG2 || GCH || (!SYM && p.erase_channel);
  const bool wch = GCH || (!FG2 && !SYM && p.write_channel);

  // ---- phase 1: loads (every global load of the phase issued before the first LDS store; rows
  // past the last token read the last token and are zeroed at the store) --------------------------
  const int tlast = tlen > 0 ? tlen - 1 : 0;
  const char* pk = ws + pkt * PK::bytes;
  auto phase1_loads = [&](auto wch_c) {
  constexpr bool WCH = decltype(wch_c)::value;
  u32x4 rS[4], rZ[2], rM[2], rV[2], rA[2], rK[2];
  f32x4 rO[4], rW[2][2];
  float rw1[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // S (checkpoint layout: 16-column tiles)
    const int u = tid + kFThreads * i;
    rS[i] = *reinterpret_cast<const u32x4*>(Sg + ck_state_off(u >> 4, (u & 15) * 8));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // Z, M (or delta)
    const int u = tid + kFThreads * i;
    rZ[i] = *reinterpret_cast<const u32x4*>(Zg + ck_rows_off(u >> 4, (u & 15) * 8));
    rM[i] = *reinterpret_cast<const u32x4*>(Mg + ck_rows_off(u >> 4, (u & 15) * 8));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // dO
    const int f = tid + kFThreads * i, t = min(f >> 5, tlast);
    rO[i] = *reinterpret_cast<const f32x4*>(g.dO + tok(t) * D + (f & 31) * 4);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // v and its write gate (FG2: the rate)
    const int u = tid + kFThreads * i, j = (u & 15) * 8;
    const int64_t x = tok(min(u >> 4, tlast));
    rV[i] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.v) + x * D + j);
    if (WCH) {
      const float* src = (FG2 ? p.erase : p.write) + x * D + j;
      rW[i][0] = *reinterpret_cast<const f32x4*>(src);
      rW[i][1] = *reinterpret_cast<const f32x4*>(src + 4);
    } else {
      rw1[i] = p.write[x];
    }
  }
  const char* akk = SYM ? static_cast<const char*>(p.ck_A) + pkt * (6 * 1024) : pk + PK::mat + 2 * PK::matb;
  if constexpr (!FG2) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // A_kk, A_qk (six stored blocks each; units past 767 repeat 767)
      const int u = min(tid + kFThreads * i, 767);
      const int m = u / 384, k = (u % 384) / 64, w64 = u % 64;
      rA[i] = *reinterpret_cast<const u32x4*>((m ? pk + PK::mat + PK::matb : akk) + 1024 * k + 16 * w64);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)  // K+ (one gate) or K^end
      rK[i] = *reinterpret_cast<const u32x4*>(pk + (SYM ? PK::kp : PK::kmt) + 16 * (tid + kFThreads * i));
  }
  float fac = 0.f;
  if constexpr (SCAL) {
    const float* gv = reinterpret_cast<const float*>(pk + PK::gate);
    fac = gv[(tid < C ? GV_FP : GV_FM) + (tid & 63)];
  }
  asm volatile("" ::: "memory");  // every load above is issued before the first store below

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + kFThreads * i;
    *reinterpret_cast<u32x4*>(SG + (u >> 4) * P1 + (u & 15) * 8) = rS[i];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = tid + kFThreads * i;
    *reinterpret_cast<u32x4*>(ZZ + (u >> 4) * P1 + (u & 15) * 8) = rZ[i];
    *reinterpret_cast<u32x4*>(MM + (u >> 4) * P1 + (u & 15) * 8) = rM[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = tid + kFThreads * i, t = f >> 5;
    pin(rO[i]);
    const f32x4 x = t < tlen ? rO[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<half4v*>(DO + t * P1 + (f & 31) * 4) = cvt4(x);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // Vt = w * v (FG2: sqrt(beta) v)
    const int u = tid + kFThreads * i, t = u >> 4, j = (u & 15) * 8;
    float vf[8], wf[8];
    bf16x8_to_f32(make_uint4(rV[i][0], rV[i][1], rV[i][2], rV[i][3]), vf);
    if (WCH) {
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        wf[e] = rW[i][0][e];
        wf[4 + e] = rW[i][1][e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] *= FG2 ? sqrtf(wf[e]) : wf[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] *= rw1[i];
    }
    if (t >= tlen) {
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] = 0.f;
    }
    *reinterpret_cast<half8*>(VV + t * P1 + j) = cvt8(vf);
  }
  if constexpr (!FG2) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + kFThreads * i;
      pin(rA[i]);
      if (u < 768) {
        const int m = u / 384, k = (u % 384) / 64, w64 = u % 64, r = w64 >> 2;
        const int lu = (w64 & 3) ^ ((r >> 2) & 3);
        const int I = k < 2 ? k : 2 + ((k - 2) >> 1), Hh = k < 2 ? 0 : ((k - 2) & 1);
        *reinterpret_cast<u32x4*>((m ? AQ : AK) + (16 * I + r) * P2 + 32 * Hh + 8 * lu) = rA[i];
      }
    }
    if (tid < 256) {
      const int m = tid >> 7, r = (tid >> 2) & 31, c8 = 32 + 8 * (tid & 3);
      *reinterpret_cast<uint4*>((m ? AQ : AK) + r * P2 + c8) = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + kFThreads * i, t = u >> 4, pos = u & 15;
      *reinterpret_cast<u32x4*>(KE + t * P1 + 8 * (pos ^ swz_key<16>(t))) = rK[i];
    }
    if constexpr (SCAL) {
      pin(fac);
      if (tid < 2 * C) FAC[tid] = fac;
    }
  }
  };
  // one gate per head on the symmetric path, FG2's rate per channel: the branch is resolved here;
  // the general path takes a whole copy of the sequence per kind (no merge between the loads)
  if constexpr (FG2) phase1_loads(BoolC<true>{});
  else if constexpr (SYM) phase1_loads(BoolC<false>{});
  else if (GCH || p.write_channel) phase1_loads(BoolC<true>{});
  else phase1_loads(BoolC<false>{});
  lds_barrier();

  auto tileNN = [&](const _Float16* A, const _Float16* Bm, int m0, int n0) {
    f32x4 acc = z4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma16x16x32(frag(Bm, P1, n0, 32 * ks, lane), frag(A, P1, m0, 32 * ks, lane), acc);
    return acc;
  };

  if constexpr (SYM) {
    // M = K+ S + A_kk delta over the whole chunk (every wave: four tiles), then into MM
    f32x4 mt[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int n = wave + 8 * k, tm = n >> 3, tn = n & 7;
      f32x4 acc = z4;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(fragT(SG, P1, 16 * tn, 32 * ks, lane), frag(KE, P1, 16 * tm, 32 * ks, lane), acc);
      if constexpr (SCAL) acc = acc * FAC[16 * tm + l16];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        acc = mfma16x16x32(fragT(MM, P1, 16 * tn, 32 * ks, lane), frag(AK, P2, 16 * tm, 32 * ks, lane), acc);
      mt[k] = acc;
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int n = wave + 8 * k, tm = n >> 3, tn = n & 7;
      *reinterpret_cast<half4v*>(MM + (16 * tm + l16) * P1 + 16 * tn + 4 * lg) = cvt4(mt[k]);
    }
    if constexpr (DCH) {
#pragma unroll
      for (int i = 0; i < 1024 / kFThreads; ++i) {
        const int u = tid + kFThreads * i, t = u >> 4, pos = u & 15;
        *reinterpret_cast<uint4*>(KE + t * P1 + 8 * (pos ^ swz_key<16>(t))) =
            *reinterpret_cast<const uint4*>(pk + PK::kmt + 16 * u);
      }
    }
    lds_barrier();
  }

  // ---- the global loads of phases 2 and 3 (G, and the half's k, q, gates and log-decays), issued
  // here so that they land during the phase-1 products; rows past the last token read the last
  // token and are zeroed where they are used
  u32x4 rG[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + kFThreads * i;
    rG[i] = *reinterpret_cast<const u32x4*>(Gg + ck_state_off(u >> 4, (u & 15) * 8));
  }
  const int x3_t = tid >> 3, x3_c8 = (tid & 7) * 8;  // phase 3: 8 channels of token x3_t
  u32x4 r3k, r3q;
  f32x4 r3e[2];
  float r3e1 = 0.f;
  {
    const int64_t xt = tok(min(x3_t, tlast));
    const int64_t x = xt * D + ch0 + x3_c8;
    r3k = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.k) + x);
    r3q = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) + x);
    if (ech) {
      r3e[0] = *reinterpret_cast<const f32x4*>(p.erase + x);
      r3e[1] = *reinterpret_cast<const f32x4*>(p.erase + x + 4);
    } else {
      r3e1 = p.erase[xt];
    }
  }
  const int ld_c = tid & 63, ld_seg = tid >> 6;  // phase 3 (per-channel decay): tokens 8 seg .. + 7 of channel c
  float r3g[DCH ? 8 : 1];
  if constexpr (DCH) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r3g[e] = p.log_decay[tok(min(8 * ld_seg + e, tlast)) * D + ch0 + ld_c];
  } else {
    r3g[0] = p.log_decay[tok(min(lane, tlast))];
  }

  // ---- phase 1: the Gram adjoints (every tile, kept as fp16) and the products with S -----------
  half4v dah[2 * NA];
#pragma unroll
  for (int k = 0; k < 2 * NA; ++k) {
    const int n = wave + 8 * k;
    const int a = n >> 4, tm = (n >> 2) & 3, tn = n & 3;
    const int which = FG2 ? (a ? GA_QK : GA_KK) : a;
    const bool rowz = which == GA_KK || which == GA_KU;
    const bool colm = FG2 || which == GA_KU || which == GA_QU;
    const float sgn = (!FG2 && colm) ? -1.f : 1.f;
    const bool strict = which == GA_KK || which == GA_KU;
    f32x4 acc = z4;
    if (tn <= tm) {
      acc = tileNN(rowz ? ZZ : DO, colm ? MM : VV, 16 * tm, 16 * tn);
      const int t = 16 * tm + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * tn + 4 * lg + r;
        acc[r] = (i < t || (!strict && i == t)) ? sgn * acc[r] : 0.f;
      }
    }
    dah[k] = cvt4(acc);
  }
  f32x4 pkp[2], pqp[2], pke[2], pue[2], pvt[2];  // this wave's products, per channel tile
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int c0 = ch0 + 32 * pq + 16 * ct;
    pkp[ct] = tileNN(ZZ, SG, 16 * blk, c0);
    pqp[ct] = tileNN(DO, SG, 16 * blk, c0);
    f32x4 acc = z4;
    if constexpr (!FG2) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        acc = mfma16x16x32(fragT(ZZ, P1, c0, 32 * ks, lane), fragT(AK, P2, 16 * blk, 32 * ks, lane), acc);
        acc = mfma16x16x32(fragT(DO, P1, c0, 32 * ks, lane), fragT(AQ, P2, 16 * blk, 32 * ks, lane), acc);
      }
    } else {
      const _Float16* z = ZZ + t_own * P1 + c0 + 4 * lg;  // dVt = -Z
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = -float(z[r]);
    }
    pvt[ct] = acc;
  }
  lds_barrier();

  // ---- phase 2: G; dGamma of the half's channels; the products with G ------------------------
  // dGamma of the half's channels: this thread's 16 S values of row ch0 + tid / 8 go to registers,
  // G replaces S in the LDS, then the products
  const int dg_d = ch0 + (tid >> 3), dg_j = (tid & 7) * 16;
  const half8 s_a = *reinterpret_cast<const half8*>(SG + dg_d * P1 + dg_j);
  const half8 s_b = *reinterpret_cast<const half8*>(SG + dg_d * P1 + dg_j + 8);
  lds_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + kFThreads * i;
    *reinterpret_cast<u32x4*>(SG + (u >> 4) * P1 + (u & 15) * 8) = rG[i];
  }
  lds_barrier();
  {
    const half8 g_a = *reinterpret_cast<const half8*>(SG + dg_d * P1 + dg_j);
    const half8 g_b = *reinterpret_cast<const half8*>(SG + dg_d * P1 + dg_j + 8);
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x = fmaf(float(g_a[e]), float(s_a[e]), x);
      x = fmaf(float(g_b[e]), float(s_b[e]), x);
    }
    x += row_from_above<4>(x);  // lanes 8 j .. 8 j + 7 summed into lane 8 j
    x += row_from_above<2>(x);
    x += row_from_above<1>(x);
    if ((lane & 7) == 0) DGAM[tid >> 3] = x;
  }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int c0 = ch0 + 32 * pq + 16 * ct;
    pke[ct] = tileNN(FG2 ? MM : VV, SG, 16 * blk, c0);  // dK^end = Vt G^T (FG2: delta G^T)
    pue[ct] = FG2 ? z4 : -tileNN(MM, SG, 16 * blk, c0);  // dU^end = -M G^T
    if constexpr (!FG2) {
      f32x4 kg = z4;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kg = mfma16x16x32(fragT(SG, P1, c0, 32 * ks, lane), frag(KE, P1, 16 * blk, 32 * ks, lane), kg);
      if constexpr (SCAL) kg = kg * FAC[C + t_own];
      pvt[ct] += kg;
    }
  }
  lds_barrier();  // every phase-1/2 read of the LDS is done

  // ---- phase 3: dA, g, k, q, u of the half --------------------------------------------------
#pragma unroll
  for (int k = 0; k < 2 * NA; ++k) {
    const int n = wave + 8 * k;
    const int a = n >> 4, tm = (n >> 2) & 3, tn = n & 3;
    const int which = FG2 ? (a ? GA_QK : GA_KK) : a;
    *reinterpret_cast<half4v*>(DA + which * C * P2 + (16 * tm + l16) * P2 + 16 * tn + 4 * lg) = dah[k];
  }
  {
    const bool ok = x3_t < tlen;
    pin(r3k);
    pin(r3q);
    float kf[8], qf[8], uf[8];
    bf16x8_to_f32(make_uint4(r3k[0], r3k[1], r3k[2], r3k[3]), kf);
    bf16x8_to_f32(make_uint4(r3q[0], r3q[1], r3q[2], r3q[3]), qf);
    if (ech) {
      pin(r3e[0]);
      pin(r3e[1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ef = e < 4 ? r3e[0][e] : r3e[1][e - 4];
        if (FG2) kf[e] *= sqrtf(ef);
        else uf[e] = kf[e] * ef;
      }
    } else {
      pin(r3e1);
#pragma unroll
      for (int e = 0; e < 8; ++e) uf[e] = kf[e] * r3e1;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = ok ? kf[e] : 0.f;
      qf[e] = ok ? qf[e] : 0.f;
      uf[e] = ok ? uf[e] : 0.f;
    }
    *reinterpret_cast<half8*>(XK + x3_t * PX + x3_c8) = cvt8(kf);
    *reinterpret_cast<half8*>(XQ + x3_t * PX + x3_c8) = cvt8(qf);
    if constexpr (!FG2) *reinterpret_cast<half8*>(XU + x3_t * PX + x3_c8) = cvt8(uf);
  }
  if constexpr (DCH) {
    float gl8[8], acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pin(r3g[e]);
      acc += 8 * ld_seg + e < tlen ? r3g[e] : 0.f;
      gl8[e] = acc;
    }
    TOT[ld_seg * 64 + ld_c] = acc;
    lds_barrier();
    float base = 0.f;
    for (int s2 = 0; s2 < ld_seg; ++s2) base += TOT[s2 * 64 + ld_c];
#pragma unroll
    for (int e = 0; e < 8; ++e) GL[(8 * ld_seg + e) * GSH + ld_c] = (base + gl8[e]) * kLog2e;
  } else {
    pin(r3g[0]);
    if (wave == 0) {
      float x = lane < tlen ? r3g[0] : 0.f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      GL[lane] = x * kLog2e;
    }
  }
  lds_barrier();

  // c: channel within the half
  auto gl = [&](int t, int c) { return DCH ? GL[t * GSH + c] : GL[t]; };
  auto opfrag = [&](const _Float16* X, int c0, int tb, int ref, bool inv) {
    const int c = c0 + l16;
    const float gr = gl(ref, c);
    half4v f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tb + 4 * lg + j;
      const float d = gl(t, c) - gr;
      f[j] = (_Float16)(float(X[t * PX + c]) * exp2f(inv ? -d : d));
    }
    return f;
  };
  const _Float16* const DKK = DA + GA_KK * C * P2;
  const _Float16* const DKU = DA + GA_KU * C * P2;
  const _Float16* const DQK = DA + GA_QK * C * P2;
  const _Float16* const DQU = DA + GA_QU * C * P2;
  const int m_ref = 16 * blk + 7;
  constexpr float kSpan = 6.f * kLog2e;

  // the chain rule's raw inputs of this lane's channels, issued before the products
  // (rows past the last token read token 0 of the chunk; their outputs are not stored)
  u32x2 vbs[2], kbs[2];
  f32x4 e4s[2], w4s[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int64_t xo = x_own + ch0 + 32 * pq + 16 * ct + 4 * lg;
    kbs[ct] = u32x2{0u, 0u};
    w4s[ct] = f32x4{1.f, 1.f, 1.f, 1.f};
    vbs[ct] = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.v) + xo);
    if (FG2) {
      kbs[ct] = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.k) + xo);
      e4s[ct] = *reinterpret_cast<const f32x4*>(p.erase + xo);
    } else {
      if (ech) e4s[ct] = *reinterpret_cast<const f32x4*>(p.erase + xo);
      else e4s[ct] = f32x4{1.f, 1.f, 1.f, 1.f} * p.erase[x_own / D];
      if (wch) w4s[ct] = *reinterpret_cast<const f32x4*>(p.write + xo);
      else w4s[ct] = f32x4{1.f, 1.f, 1.f, 1.f} * p.write[x_own / D];
    }
  }
  float s_e = 0.f, s_w = 0.f, s_g = 0.f;
  f32x4 dgv[2], gnv[2];

#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int c0 = 32 * pq + 16 * ct;  // channel tile within the half
    const int cq = c0 + 4 * lg;        // this lane's channels cq .. + 3 within the half
    f32x4 rk = z4, rq = z4, ck = z4, cu = z4;
    for (int J = 0; J < blk; ++J) {
      const int r = 16 * J + 15, s = 16 * blk - 1;
      const half4v yk = opfrag(XK, c0, 16 * J, r, true);
      f32x4 tk = mfma16(yk, frag4N(DKK, P2, 16 * blk, 16 * J, lane), z4);
      f32x4 tq = mfma16(yk, frag4N(DQK, P2, 16 * blk, 16 * J, lane), z4);
      if constexpr (!FG2) {
        const half4v yu = opfrag(XU, c0, 16 * J, r, true);
        tk = mfma16(yu, frag4N(DKU, P2, 16 * blk, 16 * J, lane), tk);
        tq = mfma16(yu, frag4N(DQU, P2, 16 * blk, 16 * J, lane), tq);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float F = r == s ? 1.f : exp2f(gl(s, cq + e) - gl(r, cq + e));
        rk[e] = fmaf(F, tk[e], rk[e]);
        rq[e] = fmaf(F, tq[e], rq[e]);
      }
    }
    for (int I = blk + 1; I < 4; ++I) {
      const int s = 16 * I - 1, r = 16 * blk + 15;
      const half4v xk = opfrag(XK, c0, 16 * I, s, false), xq = opfrag(XQ, c0, 16 * I, s, false);
      f32x4 tk = mfma16(xk, frag4T(DKK, P2, 16 * blk, 16 * I, lane), z4);
      tk = mfma16(xq, frag4T(DQK, P2, 16 * blk, 16 * I, lane), tk);
      f32x4 tu = z4;
      if constexpr (!FG2) {
        tu = mfma16(xk, frag4T(DKU, P2, 16 * blk, 16 * I, lane), z4);
        tu = mfma16(xq, frag4T(DQU, P2, 16 * blk, 16 * I, lane), tu);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float F = r == s ? 1.f : exp2f(gl(s, cq + e) - gl(r, cq + e));
        ck[e] = fmaf(F, tk[e], ck[e]);
        cu[e] = fmaf(F, tu[e], cu[e]);
      }
    }
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
    bool ok = true;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = gl(t_own, cq + e) - gl(m_ref, cq + e);
      const float ax = fmaxf(fabsf(float(XK[t_own * PX + cq + e])), fabsf(float(XQ[t_own * PX + cq + e])));
      const float au = FG2 ? 0.f : fabsf(float(XU[t_own * PX + cq + e]));
      ok = ok && fabsf(d) <= kSpan && fmaxf(ax, au) <= 80.f;
    }
    if (__all(ok)) {
      {
        const half4v yk = opfrag(XK, c0, 16 * blk, m_ref, true);
        f32x4 tk = mfma16(yk, frag4N(DKK, P2, 16 * blk, 16 * blk, lane), z4);
        f32x4 tq = mfma16(yk, frag4N(DQK, P2, 16 * blk, 16 * blk, lane), z4);
        if constexpr (!FG2) {
          const half4v yu = opfrag(XU, c0, 16 * blk, m_ref, true);
          tk = mfma16(yu, frag4N(DKU, P2, 16 * blk, 16 * blk, lane), tk);
          tq = mfma16(yu, frag4N(DQU, P2, 16 * blk, 16 * blk, lane), tq);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float fr = exp2f(gl(t_own, cq + e) - gl(m_ref, cq + e));
          rk[e] = fmaf(fr, tk[e], rk[e]);
          rq[e] = fmaf(fr, tq[e], rq[e]);
        }
      }
      {
        const half4v xk = opfrag(XK, c0, 16 * blk, m_ref, false), xq = opfrag(XQ, c0, 16 * blk, m_ref, false);
        f32x4 sk = mfma16(xk, frag4T(DKK, P2, 16 * blk, 16 * blk, lane), z4);
        sk = mfma16(xq, frag4T(DQK, P2, 16 * blk, 16 * blk, lane), sk);
        f32x4 su = z4;
        if constexpr (!FG2) {
          su = mfma16(xk, frag4T(DKU, P2, 16 * blk, 16 * blk, lane), z4);
          su = mfma16(xq, frag4T(DQU, P2, 16 * blk, 16 * blk, lane), su);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float fc = exp2f(gl(m_ref, cq + e) - gl(t_own, cq + e));
          ck[e] = fmaf(fc, sk[e], ck[e]);
          cu[e] = fmaf(fc, su[e], cu[e]);
        }
      }
    } else {
#pragma unroll 1
      for (int i2 = 0; i2 < 16; ++i2) {
        const int o = 16 * blk + i2;
        const bool row_ok = i2 <= l16, col_ok = i2 >= l16;
        const float r_kk = float(DKK[t_own * P2 + o]), r_qk = float(DQK[t_own * P2 + o]);
        const float c_kk = float(DKK[o * P2 + t_own]), c_qk = float(DQK[o * P2 + t_own]);
        float r_ku = 0.f, r_qu = 0.f, c_ku = 0.f, c_qu = 0.f;
        if constexpr (!FG2) {
          r_ku = float(DKU[t_own * P2 + o]);
          r_qu = float(DQU[t_own * P2 + o]);
          c_ku = float(DKU[o * P2 + t_own]);
          c_qu = float(DQU[o * P2 + t_own]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float go = gl(o, cq + e), gt = gl(t_own, cq + e);
          const float ko = float(XK[o * PX + cq + e]), qo = float(XQ[o * PX + cq + e]);
          const float uo = FG2 ? 0.f : float(XU[o * PX + cq + e]);
          const float er = row_ok ? exp2f(gt - go) : 0.f;
          const float ec = col_ok ? exp2f(go - gt) : 0.f;
          rk[e] = fmaf(er, fmaf(r_kk, ko, r_ku * uo), rk[e]);
          rq[e] = fmaf(er, fmaf(r_qk, ko, r_qu * uo), rq[e]);
          ck[e] = fmaf(ec, fmaf(c_kk, ko, c_qk * qo), ck[e]);
          cu[e] = fmaf(ec, fmaf(c_ku, ko, c_qu * qo), cu[e]);
        }
      }
    }

    // ---- chain rule, outputs (global channels ch0 + cq ..) -----------------------------------
    if (ct == 0) {
      // both tiles' raw inputs in registers before the first output store: a use of a loaded value
      // after a global store waits for the store as well (one counter serves both)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        pin(vbs[c2]);
        pin(e4s[c2]);
        if (FG2) pin(kbs[c2]);
        if (wch) pin(w4s[c2]);
      }
    }
    const u32x2 vb = own_ok ? vbs[ct] : u32x2{0u, 0u}, kb = kbs[ct];
    const f32x4 e4 = e4s[ct], w4 = w4s[ct];
    float vv[4], kraw[4];
    vv[0] = __uint_as_float(vb.x << 16);
    vv[1] = __uint_as_float(vb.x & 0xffff0000u);
    vv[2] = __uint_as_float(vb.y << 16);
    vv[3] = __uint_as_float(vb.y & 0xffff0000u);
    kraw[0] = __uint_as_float(kb.x << 16);
    kraw[1] = __uint_as_float(kb.x & 0xffff0000u);
    kraw[2] = __uint_as_float(kb.y << 16);
    kraw[3] = __uint_as_float(kb.y & 0xffff0000u);
    const f32x4 dkp = pkp[ct], dqp = pqp[ct], dke = pke[ct], due = pue[ct], dvt = pvt[ct];
    f32x4 o_dq, o_dk, o_dv, o_de, o_dw = z4, dgt, gnt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = cq + e;
      const float gt = gl(t_own, c);
      const float eg = exp2f(gt), egn = exp2f(gl(C - 1, c) - gt);
      const float kk = float(XK[t_own * PX + c]), qq = float(XQ[t_own * PX + c]);
      const float uu = FG2 ? 0.f : float(XU[t_own * PX + c]);
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
      const int64_t xo = x_own + ch0 + cq;
      *reinterpret_cast<f32x4*>(g.dq + xo) = o_dq;
      *reinterpret_cast<f32x4*>(g.dk + xo) = o_dk;
      *reinterpret_cast<f32x4*>(g.dv + xo) = o_dv;
      if (ech) *reinterpret_cast<f32x4*>(g.derase + xo) = o_de;
      if (!shared_gate && wch) *reinterpret_cast<f32x4*>(g.dwrite + xo) = o_dw;
    }
  }

  // ---- g's adjoint: suffix sums within the block, block totals and end shares through LDS -----
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = row_suffix(dgv[ct][e]);
      dgv[ct][e] = v;
      const float n = row_suffix(gnv[ct][e]);  // lane 0 of the row: the block's sum
      const int c = 32 * pq + 16 * ct + 4 * lg + e;
      if (l16 == 0) {
        BT[blk * 64 + c] = v;
        GNS[blk * 64 + c] = n;
      }
    }
  s_e = cross_row_sum(s_e);
  s_w = cross_row_sum(s_w);
  s_g = cross_row_sum(s_g);
  if (lg == 0) {
    RED[(0 * 2 + pq) * 64 + t_own] = s_g;
    RED[(1 * 2 + pq) * 64 + t_own] = s_e;
    RED[(2 * 2 + pq) * 64 + t_own] = s_w;
  }
  lds_barrier();
  if constexpr (DCH) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int cq = 32 * pq + 16 * ct + 4 * lg;
      f32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = cq + e;
        float later = 0.f;
        for (int b2 = blk + 1; b2 < 4; ++b2) later += BT[b2 * 64 + c];
        const float dgn = exp2f(gl(C - 1, c)) * DGAM[c] + GNS[c] + GNS[64 + c] + GNS[128 + c] + GNS[192 + c];
        out[e] = dgv[ct][e] + later + dgn;
      }
      if (own_ok) *reinterpret_cast<f32x4*>(g.dlog_decay + x_own + ch0 + cq) = out;
    }
  } else if (wave == 0) {
    // g_C's share summed over the half's channels
    const int c = lane;
    float n = exp2f(gl(C - 1, c)) * DGAM[c] + GNS[c] + GNS[64 + c] + GNS[128 + c] + GNS[192 + c];
    n = cross_row_sum(row_suffix(n));
    if (lane == 0) MISC[0] = n;
  }
  // the half's per-token sums (the two channel pairs added in a fixed order)
  if (part) {
    lds_barrier();
    float* pp = part + (item * 2 + half) * kPartFloats;
    if (tid < 3 * C) {
      const int which = tid / C, t = tid - which * C;
      pp[tid] = RED[(which * 2 + 0) * 64 + t] + RED[(which * 2 + 1) * 64 + t];
    } else if (tid == 3 * C) {
      pp[3 * C] = DCH ? 0.f : MISC[0];
    }
  }
}

// Per-head gate and decay gradients of each chunk from the two halves' sums: one wave per chunk
// (lane = token).  The per-head log-decay's adjoint is the suffix sum of the per-token sums plus
// g_C's share.
__global__ __launch_bounds__(64) void chunk_grad_sums_kernel(Problem p, BwdArgs g, const float* __restrict__ part,
                                                             int want_decay, int want_erase, int want_write) {
  const int64_t blk = blockIdx.x;
  const int lane = threadIdx.x;
  if (p.chunks && blk >= int64_t(p.H) * *p.nchunks_total) return;
  const ChunkRef cr = chunk_ref_of(p, blk, (p.T + C - 1) / C);
  const int tlen = cr.tlen;
  const int64_t tk = (cr.tok0 + lane) * int64_t(p.H) + cr.h;
  const float* p0 = part + blk * 2 * kPartFloats;
  const float* p1 = p0 + kPartFloats;
  if (want_decay) {
    float x = p0[lane] + p1[lane];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(x, o);
      if (lane + o < 64) x += y;
    }
    x += p0[3 * C] + p1[3 * C];
    if (lane < tlen) g.dlog_decay[tk] = x;
  }
  if (lane < tlen) {
    if (want_erase) g.derase[tk] = p0[C + lane] + p1[C + lane];
    if (want_write) g.dwrite[tk] = p0[2 * C + lane] + p1[2 * C + lane];
  }
}

}  // namespace

// Work items: every chunk of every head (packed sequences: as many as their lengths allow).
static int64_t grad_items(const Problem& p, bool packed) {
  return packed ? int64_t(p.H) * varlen_max_chunks(p.B, p.T) : int64_t(p.B) * p.H * ((int64_t(p.T) + C - 1) / C);
}

size_t chunk_grad_work_bytes(const Problem& p, bool packed) {
  return size_t(grad_items(p, packed) * 2 * kPartFloats * 4);
}

hipError_t launch_chunk_grad(const Problem& p, const BwdArgs& g, const void* packets, void* work,
                             hipStream_t stream) {
  const int64_t nchunks = grad_items(p, p.chunks != nullptr);
  if (nchunks == 0) return hipSuccess;
  const bool fg2 = p.rate_sqrt;
  const bool want_decay = !p.decay_channel;
  const bool want_erase = !fg2 && !p.erase_channel;
  const bool want_write = !fg2 && g.dwrite != nullptr && !p.write_channel;
  float* part = (want_decay || want_erase || want_write) ? static_cast<float*>(work) : nullptr;
  const char* ws = static_cast<const char*>(packets);
  const dim3 grid(unsigned((2 * nchunks + 15) / 16 * 16)), block(kFThreads);  // whole groups of 8 x 2
  if (fg2) {
    if (p.decay_channel)
      hipLaunchKernelGGL((chunk_grad_kernel<kModeFg2, true, false>), grid, block, 0, stream, p, g, ws, part, nchunks);
    else
      hipLaunchKernelGGL((chunk_grad_kernel<kModeFg2, false, false>), grid, block, 0, stream, p, g, ws, part, nchunks);
  } else if (p.symmetric) {
    if (p.decay_channel)
      hipLaunchKernelGGL((chunk_grad_kernel<kModeSym, true, false>), grid, block, 0, stream, p, g, ws, part, nchunks);
    else
      hipLaunchKernelGGL((chunk_grad_kernel<kModeSym, false, false>), grid, block, 0, stream, p, g, ws, part, nchunks);
  } else if (p.erase_channel && p.write_channel) {
    if (p.decay_channel)
      hipLaunchKernelGGL((chunk_grad_kernel<kModeGen, true, true>), grid, block, 0, stream, p, g, ws, part, nchunks);
    else
      hipLaunchKernelGGL((chunk_grad_kernel<kModeGen, false, true>), grid, block, 0, stream, p, g, ws, part, nchunks);
  } else {
    if (p.decay_channel)
      hipLaunchKernelGGL((chunk_grad_kernel<kModeGen, true, false>), grid, block, 0, stream, p, g, ws, part, nchunks);
    else
      hipLaunchKernelGGL((chunk_grad_kernel<kModeGen, false, false>), grid, block, 0, stream, p, g, ws, part, nchunks);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !part) return e;
  hipLaunchKernelGGL(chunk_grad_sums_kernel, dim3(unsigned(nchunks)), dim3(64), 0, stream, p, g, part,
                     int(want_decay), int(want_erase), int(want_write));
  return hipGetLastError();
}

}  // namespace dr
