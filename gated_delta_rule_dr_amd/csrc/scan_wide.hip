// Full-width segmented scan for separate erase and write gates (general gates, a dense batch,
// bf16 q/k/v, dk = dv = 128, chunk 64).
//
// The state-passing scan ([FG²] §2, the WY form of a chunk's rank-1 updates; [L2S] method,
// architecture and implementation: chunk states rebuilt from boundary states) reads every
// chunk's packet of state-independent factors (the prep's output).  A scan workgroup that owns
// a narrow slice of value columns must still stream the whole packet, so a head's packet bytes
// cross the L2 -> L1 path once per slice.  Here one workgroup owns all 128 value columns of a
// head (wave w: columns 16 w .. 16 w + 15, all 128 key rows in registers), so each packet
// crosses that path once.  To keep the compute units busy when there are few heads, the
// sequence is cut into P segments: the chunk map is affine in the state,
//     S_out = F S_in + H,
// so each segment's pair (F, H) is computed from S = I and S = 0 in parallel, a small kernel
// chains S_in[s + 1] = F[s] S_in[s] + H[s], and every segment then runs from its true S_in.
// The same file holds the gradients' side of it: the forward with each chunk's incoming state
// and M stored for the gradient kernels, and the adjoint scan (the state's adjoint carried
// backwards) segmented the same way.
//
// Chunk algebra (general gates, u = e ⊙ k, Vt = w ⊙ v; tiles referenced at the chunk start, see
// the prep): Y = K+ S + A_kk Vt, M = T Y, O = Q+ S + A_qk Vt − A_qu M,
// S ← Diag(e^{g_C}) S + K^endᵀ Vt − U^endᵀ M, with every matrix operand in fp16 and every
// accumulation and the state in fp32 — the same roundings as the sliced scan.
//
// Interleaved rows.  A 16 x 16 accumulator tile leaves each lane four consecutive rows of one
// column; the next product needs eight consecutive contraction rows per lane.  So the state's
// tiles and the in-chunk token tiles (Y, M, O) order their rows in pairs: tile 2 k + s, lane
// group g, element i holds row 32 k + 8 g + 4 s + i.  The two tiles of a pair then form the
// next product's B fragment directly (rows 32 k + 8 g + 0..7), and the packet operands that
// produce them are read at the matching rows (an A operand's rows are free per lane), so all
// packet reads stay whole 16-byte fragment reads.

#include "chunk_layout.h"
#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int kWideThreads = 512;  // eight waves, one per 16 value columns

template <bool B>
struct WFlag {
  static constexpr bool value = B;
};
template <int N>
struct WInt {
  static constexpr int value = N;
};

// LDS of the full-width scan: the packet's tiles and matrices in the packet's own layout (units
// copy straight across), Vt, and the chunk's end-of-chunk decay factors.
struct WideLayout {
  static constexpr int kp = 0;                      // K+     [64][128] half, swizzled
  static constexpr int qp = kp + C * D * 2;         // Q+
  static constexpr int kmt = qp + C * D * 2;        // K^end
  static constexpr int umt = kmt + C * D * 2;       // U^end
  static constexpr int mat = umt + C * D * 2;       // T, A_qk, A_kk, A_qu: eight 16 x 32 blocks each
  static constexpr int vt = mat + 4 * C * C * 2;    // Vt     [64][128] half, swizzled
  static constexpr int fc = vt + D * C * 2;         // e^{g_C} [128] fp32
  static constexpr int total = fc + D * 4;
};

// Row held by lane row m of interleaved tile I (see the file comment).
__device__ __forceinline__ int ilv(int I, int m) { return 32 * (I >> 1) + 8 * (m >> 2) + 4 * (I & 1) + (m & 3); }

// A fragment (16 rows x 32 contraction) of a swizzled [*][128] tile at this lane's own row.
__device__ __forceinline__ half8 frag_row16(const _Float16* base, int row, int k0, int lane) {
  return *reinterpret_cast<const half8*>(base + swz<16>(row, k0 + 8 * (lane >> 4)));
}

// A fragment of a lower-triangular matrix (eight 16 x 32 blocks in LDS, layout tri_in) at this
// lane's own row, contraction columns 32 H .. + 31.
__device__ __forceinline__ half8 frag_tri_row(const _Float16* base, int row, int H, int lane) {
  return *reinterpret_cast<const half8*>(base + (2 * (row >> 4) + H) * 512 + tri_in(row, 8 * (lane >> 4)));
}

// A fragment of the transpose of a swizzled [64][128] tile, A[row][k = t] = base[t][row], for the
// rows of interleaved key tile r: lane 16 g + m receives base[t0 + 8 g + 0..7][ilv(r, m)].  The
// transposing read gives lane 16 g + 4 a + b element b of the 8-byte piece that lane
// 16 g + a + 4 j supplies (j: the token); each supplier names the piece of channels
// ilv(r, 4 a) .. + 3.
__device__ __forceinline__ half8 frag_ts_ilv(const _Float16* base, int r, int t0, int lane) {
  const int m = lane & 15;
  const int t = t0 + 8 * (lane >> 4) + (m >> 2);
  const int d = 32 * (r >> 1) + 8 * (m & 3) + 4 * (r & 1);
  const half4v lo = ld_tr16(base + swz<16>(t, d));
  const half4v hi = ld_tr16(base + swz<16>(t + 4, d));
  return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ half8 cat8(half4v a, half4v b) {
  return half8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ half4v cvt4n(f32x4 a) {
  half4v h;
#pragma unroll
  for (int r = 0; r < 4; ++r) h[r] = (_Float16)(-a[r]);
  return h;
}

__device__ __forceinline__ u32x4 ldu4(gptr<const char> base, int64_t off) { return *(gptr<const u32x4>)(base + off); }

// Stored matrix unit (16 bytes) j of thread tid when only T and A_kk are read: units 0 .. 383
// (T) and 768 .. 1151 (A_kk) in order; a thread without a second unit repeats its first.
__device__ __forceinline__ int mat_unit_fh(int tid, int j) {
  const int idx = j == 0 || tid >= 256 ? tid : tid + kWideThreads;
  return idx < 384 ? idx : idx + 384;
}

// This wave's 16 columns of an fp32 [128][128] state, to or from the interleaved accumulator
// tiles: after the quad transpose each lane holds four consecutive columns of one row, one
// 16-byte access per tile.
__device__ __forceinline__ void state_store(float* dst, const f32x4 (&S)[8]) {
  const int lane = threadIdx.x & 63, jw = 16 * (threadIdx.x >> 6), l16 = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int r = 0; r < 8; ++r)
    *reinterpret_cast<f32x4*>(dst + ilv(r, 4 * lg + (l16 & 3)) * D + jw + (l16 & 12)) = quad_transpose(S[r]);
}
__device__ __forceinline__ void state_load(const float* src, f32x4 (&S)[8]) {
  const int lane = threadIdx.x & 63, jw = 16 * (threadIdx.x >> 6), l16 = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int r = 0; r < 8; ++r)
    S[r] = src ? quad_transpose(*reinterpret_cast<const f32x4*>(src + ilv(r, 4 * lg + (l16 & 3)) * D + jw + (l16 & 12)))
               : f32x4{0.f, 0.f, 0.f, 0.f};
}

// The segments of a full-width scan: segment 0 of L0 chunks, then P - 1 segments of L chunks.
struct WidePlan {
  int nch, L0, L, P;
  float* fh;   // [B * H][P][2][128][128] fp32: F then H of every segment
  float* sin;  // [B * H][P][128][128] fp32: the forward's state entering every segment (index 0
               // unused), or the adjoint's value at the end of every segment (index P - 1 unused)
};

// One segment [c0, c1) of one (b, h), all 128 value columns.
//   FH = false: from s_in (null: zero), o for the segment, the final state to s_out (if given);
//   FH = true: the segment's affine map, F from S = I with no values and H from S = 0, to
//   f_out and h_out.
// CKPT (with FH = false): also every chunk's incoming state and its M, as fp16 16-column tiles
// (p.ck_S: [packet][dv / 16][dk][16], p.ck_M: [packet][dv / 16][token][16]), for the gradients.
template <bool FH, bool WCH, bool CKPT>
__device__ __forceinline__ void wide_segment(const Problem& p, const char* ws, char* smem, int bh, int c0, int c1,
                                             const float* s_in, float* s_out, float* f_out, float* h_out) {
  using PK = Packet<true, true>;  // the general-gate packet (one layout for both decay kinds)
  _Float16* KP = reinterpret_cast<_Float16*>(smem + WideLayout::kp);
  _Float16* QP = reinterpret_cast<_Float16*>(smem + WideLayout::qp);
  _Float16* KMT = reinterpret_cast<_Float16*>(smem + WideLayout::kmt);
  _Float16* UMT = reinterpret_cast<_Float16*>(smem + WideLayout::umt);
  _Float16* MAT = reinterpret_cast<_Float16*>(smem + WideLayout::mat);
  _Float16* TH = MAT;
  _Float16* AQ = MAT + 4096;
  _Float16* AKK = MAT + 2 * 4096;
  _Float16* AQU = MAT + 3 * 4096;
  _Float16* VT = reinterpret_cast<_Float16*>(smem + WideLayout::vt);
  float* FC = reinterpret_cast<float*>(smem + WideLayout::fc);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int jw = 16 * wave;
  const int H = p.H, h = bh % H;
  const int T = p.T, nch = (T + C - 1) / C;
  const int64_t tok0 = int64_t(bh / H) * T;
  const gptr<const char> pbase = opaque_gptr(ws) + int64_t(bh) * nch * PK::bytes;
  const gptr<const char> vin = opaque_gptr(static_cast<const char*>(p.v));
  const gptr<const char> wrin = opaque_gptr(reinterpret_cast<const char*>(p.write));

  // State (F with FH) and, with FH, the offset H: interleaved key tiles, see state_store.
  f32x4 S[8], Hs[8];
  if constexpr (FH) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        S[r][i] = ilv(r, 4 * lg + i) == jw + l16 ? 1.f : 0.f;
        Hs[r][i] = 0.f;
      }
  } else {
    state_load(s_in, S);
  }

  // Staged loads of one chunk: this thread's 16-byte units of the four tiles (K+, Q+, K^end,
  // U^end: units tid and tid + 512 of each) and of the matrices' stored blocks (units tid,
  // tid + 512, tid + 1024), the decay factors, and 16 value columns of token tid / 8 with their
  // write gates.  Tokens past the end load token T - 1 (zeroed where they are used), so every
  // load is issued unconditionally.
  struct Stage {
    u32x4 tl[8];
    u32x4 mr[FH ? 2 : 3];
    u32x4 fc;
    u32x4 v[2];
    u32x4 w[WCH ? 4 : 1];
  };
  // The loads of one chunk, in three batches that the chunk's compute stages separate (each
  // wave then computes while the compute unit's memory path drains the previous batch).
  auto load = [&](auto batch, Stage& P, int c) {
    constexpr int BATCH = decltype(batch)::value;
    // (the thread index through an empty asm: offsets are formed here, per chunk, instead of
    // being hoisted out of the chunk loop as invariants that spill)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int vtok = tid >> 3, vcol = 16 * (tid & 7);
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
    if constexpr (BATCH == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = 16 * (tid + kWideThreads * i);
        P.tl[i] = ldu4(pk, PK::kp + u);
        if constexpr (!FH) P.tl[2 + i] = ldu4(pk, PK::qp + u);
        P.tl[4 + i] = ldu4(pk, PK::kmt + u);
        P.tl[6 + i] = ldu4(pk, PK::umt + u);
      }
    } else if constexpr (BATCH == 1) {
      if constexpr (FH) {
        // T and A_kk only (stored units 0 .. 383 and 768 .. 1151): threads below 256 take two
        // units, the others one (their second load repeats the first, unused)
#pragma unroll
        for (int j = 0; j < 2; ++j) P.mr[j] = ldu4(pk, PK::mat + 16 * mat_unit_fh(tid, j));
      } else {
#pragma unroll
        for (int j = 0; j < 3; ++j) P.mr[j] = ldu4(pk, PK::mat + 16 * (tid + kWideThreads * j));
      }
      P.fc = ldu4(pk, PK::gate + 4 * (GV_FC + 4 * (tid & 31)));
    } else {
      const int t = c * C + vtok;
      const int64_t row = (tok0 + (t < T ? t : T - 1)) * H + h;
      P.v[0] = ldu4(vin, (row * D + vcol) * 2);
      P.v[1] = ldu4(vin, (row * D + vcol + 8) * 2);
      if constexpr (WCH) {
#pragma unroll
        for (int i = 0; i < 4; ++i) P.w[i] = ldu4(wrin, (row * D + vcol + 4 * i) * 4);
      } else {
        P.w[0] = u32x4{*(gptr<const uint32_t>)(wrin + row * 4), 0u, 0u, 0u};
      }
    }
  };

  // The staged chunk into LDS: units copy straight across; Vt^T from the values and write gates.
  auto to_lds = [&](const Stage& P, int c) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int vtok = tid >> 3, vcol = 16 * (tid & 7);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = 8 * (tid + kWideThreads * i);
      *reinterpret_cast<u32x4*>(KP + u) = P.tl[i];
      if constexpr (!FH) *reinterpret_cast<u32x4*>(QP + u) = P.tl[2 + i];
      *reinterpret_cast<u32x4*>(KMT + u) = P.tl[4 + i];
      *reinterpret_cast<u32x4*>(UMT + u) = P.tl[6 + i];
    }
    // stored block k of matrix m (1 KB each, see tri_pos) to LDS block 2 I + H of that matrix
#pragma unroll
    for (int j = 0; j < (FH ? 2 : 3); ++j) {
      const int u = FH ? mat_unit_fh(tid, j) : tid + kWideThreads * j, m = u / 384, k = (u % 384) / 64;
      const int lb = k < 2 ? 2 * k : k + 2;
      if (!FH || j == 0 || tid < 256) *reinterpret_cast<u32x4*>(MAT + 4096 * m + 512 * lb + 8 * (u % 64)) = P.mr[j];
    }
    if (tid < 32) *reinterpret_cast<u32x4*>(FC + 4 * tid) = P.fc;
    const bool ok = c * C + vtok < T;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      half8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * u + e;
        const uint32_t word = P.v[u][e >> 1];
        const float vf = __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
        const float wf = WCH ? __uint_as_float(P.w[i >> 2][i & 3]) : __uint_as_float(P.w[0][0]);
        hv[e] = (_Float16)(ok ? wf * vf : 0.f);
      }
      *reinterpret_cast<half8*>(VT + swz<16>(vtok, vcol + 8 * u)) = hv;
    }
  };

  // One state's chunk from LDS: Y = K+ X (+ A_kk Vt), M = T Y, with OUT the output O = Q+ X +
  // A_qk Vt − A_qu M, then X ← Diag(e^{g_C}) X (+ K^endᵀ Vt) − U^endᵀ M.  VALS: the values
  // enter (the state and H; not F).  TAIL: the chunk extends past the last token (its o rows are
  // masked).
  auto advance = [&](auto vals, auto out, auto tail, f32x4(&X)[8], int c, auto&& after_y, auto&& after_m) {
    constexpr bool VALS = decltype(vals)::value, OUT = decltype(out)::value, TAIL = decltype(tail)::value;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int l16 = lane & 15, lg = lane >> 4;
    if constexpr (CKPT && OUT) {
      // the chunk's incoming state: wave w's tile, each lane four consecutive columns of a row
      _Float16* dst = static_cast<_Float16*>(p.ck_S) + (int64_t(bh) * nch + c) * D * D + jw * D;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        *reinterpret_cast<half4v*>(dst + ilv(r, 4 * lg + (l16 & 3)) * 16 + (l16 & 12)) = cvt4(quad_transpose(X[r]));
    }
    // B fragments: the state (contraction over key channels) and Vt (over tokens)
    half8 bS[4], bV[2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bS[kk] = cat8(cvt4(X[2 * kk]), cvt4(X[2 * kk + 1]));
    if constexpr (VALS) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bV[ks] = frag_ts(VT, jw, 32 * ks, lane);
    }
    // Y, token rows interleaved
    f32x4 Y[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const int tr = ilv(I, l16);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma16x16x32(frag_row16(KP, tr, 32 * kk, lane), bS[kk], acc);
      if constexpr (VALS) {
#pragma unroll
        for (int ks = 0; ks <= (I >> 1); ++ks) acc = mfma16x16x32(frag_tri_row(AKK, tr, ks, lane), bV[ks], acc);
      }
      Y[I] = acc;
    }
    after_y();
    // M = T Y; its negation as the B fragment of the O and state products
    half8 bM[2];
    {
      const half8 bY[2] = {cat8(cvt4(Y[0]), cvt4(Y[1])), cat8(cvt4(Y[2]), cvt4(Y[3]))};
      f32x4 M[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int tr = ilv(I, l16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt <= (I >> 1); ++kt) acc = mfma16x16x32(frag_tri_row(TH, tr, kt, lane), bY[kt], acc);
        M[I] = acc;
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) bM[kt] = cat8(cvt4n(M[2 * kt]), cvt4n(M[2 * kt + 1]));
      if constexpr (CKPT && OUT) {
        _Float16* dst = static_cast<_Float16*>(p.ck_M) + (int64_t(bh) * nch + c) * C * D + jw * C;
#pragma unroll
        for (int I = 0; I < 4; ++I)
          *reinterpret_cast<half4v*>(dst + ilv(I, 4 * lg + (l16 & 3)) * 16 + (l16 & 12)) = cvt4(quad_transpose(M[I]));
      }
    }
    after_m();
    // O = Q+ X + A_qk Vt − A_qu M: lane (after the quad transpose) holds four consecutive
    // columns of one token row
    if constexpr (OUT) {
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int tr = ilv(I, l16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma16x16x32(frag_row16(QP, tr, 32 * kk, lane), bS[kk], acc);
#pragma unroll
        for (int ks = 0; ks <= (I >> 1); ++ks) {
          acc = mfma16x16x32(frag_tri_row(AQ, tr, ks, lane), bV[ks], acc);
          acc = mfma16x16x32(frag_tri_row(AQU, tr, ks, lane), bM[ks], acc);
        }
        const int t = c * C + ilv(I, 4 * lg + (l16 & 3));
        const f32x4 ot = quad_transpose(acc);
        if (!TAIL || t < T) store_o4(p.o, ((tok0 + t) * H + h) * D + jw + (l16 & 12), ot, p.o_bf16);
      }
    }
    // X ← Diag(e^{g_C}) X + K^endᵀ Vt − U^endᵀ M
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (VALS) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc = mfma16x16x32(frag_ts_ilv(KMT, r, 32 * ks, lane), bV[ks], acc);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc = mfma16x16x32(frag_ts_ilv(UMT, r, 32 * kt, lane), bM[kt], acc);
      const f32x4 f = *reinterpret_cast<const f32x4*>(FC + ilv(r, 4 * lg));
#pragma unroll
      for (int i = 0; i < 4; ++i) X[r][i] = fmaf(f[i], X[r][i], acc[i]);
    }
  };
  // One chunk; the next chunk's second and third load batches are issued after its first
  // products.
  auto compute = [&](auto tail, int c, Stage& P, int cn) {
    auto b1 = [&] { load(WInt<1>(), P, cn); };
    auto b2 = [&] { load(WInt<2>(), P, cn); };
    auto none = [] {};
    if constexpr (FH) {
      // F, then H: one state's working set at a time
      advance(WFlag<false>(), WFlag<false>(), tail, S, c, b1, b2);
      __builtin_amdgcn_sched_barrier(0);
      advance(WFlag<true>(), WFlag<false>(), tail, Hs, c, none, none);
    } else {
      advance(WFlag<true>(), WFlag<true>(), tail, S, c, b1, b2);
    }
  };

  // the upper blocks (0,1) and (1,1) of the four matrices are zero and never copied
  *reinterpret_cast<u32x4*>(MAT + 4096 * (tid >> 7) + 512 * (1 + 2 * ((tid >> 6) & 1)) + 8 * lane) =
      u32x4{0u, 0u, 0u, 0u};
  Stage P;
  load(WInt<0>(), P, c0);
  load(WInt<1>(), P, c0);
  load(WInt<2>(), P, c0);
  const bool ragged = (T % C) != 0;
  for (int c = c0; c < c1; ++c) {
    to_lds(P, c);
    lds_barrier();
    const int cn = c + 1 < c1 ? c + 1 : c;  // the next chunk (past the segment: this one again, unused)
    load(WInt<0>(), P, cn);
    if (ragged && c == nch - 1) compute(WFlag<true>(), c, P, cn);
    else compute(WFlag<false>(), c, P, cn);
    lds_barrier();
  }

  if constexpr (FH) {
    state_store(f_out, S);
    state_store(h_out, Hs);
  } else if (s_out) {
    state_store(s_out, S);
  }
}

// Phase 1 (SECOND = false): workgroup (bh, 0) runs segment 0 from S0 with its outputs; (bh, s),
// s = 1 .. P - 2, forms segment s's affine map.  Phase 2 (SECOND = true): workgroup (bh, y) runs
// segment y + 1 from its entering state with its outputs; the last writes S_T.
template <bool WCH, bool SECOND, bool CKPT>
__global__ __launch_bounds__(kWideThreads) void chunk_scan_wide_kernel(Problem p, const char* __restrict__ ws,
                                                                       WidePlan wp) {
  __shared__ __attribute__((aligned(16))) char smem[WideLayout::total];
  const int bh = blockIdx.x;
  const int seg = SECOND ? int(blockIdx.y) + 1 : int(blockIdx.y);
  const int c0 = seg == 0 ? 0 : wp.L0 + (seg - 1) * wp.L;
  const int c1 = seg == 0 ? wp.L0 : (c0 + wp.L < wp.nch ? c0 + wp.L : wp.nch);
  const int64_t mat = int64_t(D) * D;
  float* const sin = wp.sin + int64_t(bh) * wp.P * mat;
  if (!SECOND && seg > 0) {
    float* const fh = wp.fh + (int64_t(bh) * wp.P + seg) * 2 * mat;
    wide_segment<true, WCH, false>(p, ws, smem, bh, c0, c1, nullptr, nullptr, fh, fh + mat);
    return;
  }
  const float* s_in = seg == 0 ? (p.S0 ? p.S0 + int64_t(bh) * mat : nullptr) : sin + seg * mat;
  float* s_out = seg == wp.P - 1 ? (p.S_T ? p.S_T + int64_t(bh) * mat : nullptr) : (SECOND ? nullptr : sin + mat);
  wide_segment<false, WCH, CKPT>(p, ws, smem, bh, c0, c1, s_in, s_out, nullptr, nullptr);
}

// ------------------------------------------------------------------------------------------
// Full-width segmented adjoint scan (the gradients' reverse scan, general gates, dense batch).
// Per chunk, in reverse, with G the state's adjoint at the chunk's end ([L2S] method: the backward
// is a second scan; [FG²] §2: the WY form of the chunk):
//   X1 = A_quᵀ dO + U^end G,   Z = −Tᵀ X1,   G ← Diag(e^{g_C}) G + Q⁺ᵀ dO + K⁺ᵀ Z,
// every product on fp16 operands (X1 rounded to fp16 before its product, as in the sliced adjoint
// scan), storing G (before its update) and Z of every chunk for the gradient kernels.  G is affine
// in its value at the segment's end, so segments split as in the forward: the last segment runs
// from dS_T with its stores in the first pass beside the middle segments' maps (F from G = I
// without dO, H from G = 0), the compose kernel chains them backwards, and the second pass runs
// segments 0 .. P - 2 from their true end adjoint; segment 0 ends with dS0.
// ------------------------------------------------------------------------------------------
struct AdjLayout {
  static constexpr int qp = 0;                      // Q+     [64][128] half, swizzled
  static constexpr int kp = qp + C * D * 2;         // K+
  static constexpr int umt = kp + C * D * 2;        // U^end
  static constexpr int mat = umt + C * D * 2;       // T, A_qu: eight 16 x 32 blocks each
  static constexpr int dop = mat + 2 * C * C * 2;   // dO     [64][128] half, swizzled
  static constexpr int fc = dop + C * D * 2;        // e^{g_C} [128] fp32
  static constexpr int total = fc + D * 4;
};

// A fragment of the transpose of a lower-triangular matrix (eight 16 x 32 blocks in LDS, layout
// tri_in) at the rows of interleaved token tile I: lane 16 g + m receives
// base[r0 + 8 g + 0..7][ilv(I, m)] (each supplier lane names the piece of columns ilv(I, 4 a) .. + 3).
__device__ __forceinline__ half8 frag_tri_t_ilv(const _Float16* base, int I, int r0, int lane) {
  const int m = lane & 15;
  const int r = r0 + 8 * (lane >> 4) + (m >> 2);
  const int c = 32 * (I >> 1) + 8 * (m & 3) + 4 * (I & 1);
  const half4v lo = ld_tr16(base + (2 * (r >> 4) + (c >> 5)) * 512 + tri_in(r, c));
  const half4v hi = ld_tr16(base + (2 * ((r + 4) >> 4) + (c >> 5)) * 512 + tri_in(r + 4, c));
  return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Stored matrix unit (16 bytes) j of thread tid when T and A_qu are read: units 0 .. 383 (T) and
// 1152 .. 1535 (A_qu) in order; a thread without a second unit repeats its first.
__device__ __forceinline__ int mat_unit_adj(int tid, int j) {
  const int idx = j == 0 || tid >= 256 ? tid : tid + kWideThreads;
  return idx < 384 ? idx : idx + 768;
}

// One segment [c0, c1) of one (b, h) of the adjoint scan, all 128 value columns, chunks in reverse.
//   FH = false: from g_in (null: zero), with the checkpoint stores; the adjoint at the segment's
//   start to g_out (if given);  FH = true: the segment's map (F from G = I without dO, H from
//   G = 0) to f_out and h_out.
template <bool FH>
__device__ __forceinline__ void wide_adjoint_segment(const Problem& p, const char* ws, char* smem, int bh, int c0,
                                                     int c1, const float* dO, const float* g_in, float* g_out,
                                                     float* f_out, float* h_out) {
  using PK = Packet<true, true>;
  _Float16* QP = reinterpret_cast<_Float16*>(smem + AdjLayout::qp);
  _Float16* KP = reinterpret_cast<_Float16*>(smem + AdjLayout::kp);
  _Float16* UMT = reinterpret_cast<_Float16*>(smem + AdjLayout::umt);
  _Float16* TH = reinterpret_cast<_Float16*>(smem + AdjLayout::mat);
  _Float16* AQU = TH + 4096;
  _Float16* DOP = reinterpret_cast<_Float16*>(smem + AdjLayout::dop);
  float* FC = reinterpret_cast<float*>(smem + AdjLayout::fc);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int jw = 16 * wave;
  const int H = p.H, h = bh % H;
  const int T = p.T, nch = (T + C - 1) / C;
  const int64_t tok0 = int64_t(bh / H) * T;
  const gptr<const char> pbase = opaque_gptr(ws) + int64_t(bh) * nch * PK::bytes;
  const gptr<const char> dOin = opaque_gptr(reinterpret_cast<const char*>(dO));

  f32x4 G[8], Hs[8];
  if constexpr (FH) {
    const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        G[r][i] = ilv(r, 4 * lg + i) == jw + l16 ? 1.f : 0.f;
        Hs[r][i] = 0.f;
      }
  } else {
    state_load(g_in, G);
  }

  struct Stage {
    u32x4 tl[6];  // Q+, K+, U^end units tid and tid + 512
    u32x4 mr[2];  // stored blocks of T and A_qu (mat_unit_adj)
    u32x4 fc;
    u32x4 dv[4];  // dO: 16 columns of token tid / 8
  };
  auto load = [&](auto batch, Stage& P, int c) {
    constexpr int BATCH = decltype(batch)::value;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
    if constexpr (BATCH == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = 16 * (tid + kWideThreads * i);
        P.tl[i] = ldu4(pk, PK::qp + u);
        P.tl[2 + i] = ldu4(pk, PK::kp + u);
        P.tl[4 + i] = ldu4(pk, PK::umt + u);
      }
    } else if constexpr (BATCH == 1) {
#pragma unroll
      for (int j = 0; j < 2; ++j) P.mr[j] = ldu4(pk, PK::mat + 16 * mat_unit_adj(tid, j));
      P.fc = ldu4(pk, PK::gate + 4 * (GV_FC + 4 * (tid & 31)));
    } else {
      const int vtok = tid >> 3, vcol = 16 * (tid & 7);
      const int t = c * C + vtok;
      const int64_t row = (tok0 + (t < T ? t : T - 1)) * H + h;
#pragma unroll
      for (int i = 0; i < 4; ++i) P.dv[i] = ldu4(dOin, (row * D + vcol + 4 * i) * 4);
    }
  };
  auto to_lds = [&](const Stage& P, int c) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int vtok = tid >> 3, vcol = 16 * (tid & 7);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = 8 * (tid + kWideThreads * i);
      *reinterpret_cast<u32x4*>(QP + u) = P.tl[i];
      *reinterpret_cast<u32x4*>(KP + u) = P.tl[2 + i];
      *reinterpret_cast<u32x4*>(UMT + u) = P.tl[4 + i];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int u = mat_unit_adj(tid, j), m = u / 384, k = (u % 384) / 64;
      const int lb = k < 2 ? 2 * k : k + 2;
      if (j == 0 || tid < 256) *reinterpret_cast<u32x4*>(TH + 4096 * (m ? 1 : 0) + 512 * lb + 8 * (u % 64)) = P.mr[j];
    }
    if (tid < 32) *reinterpret_cast<u32x4*>(FC + 4 * tid) = P.fc;
    const bool ok = c * C + vtok < T;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      half8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = (_Float16)(ok ? __uint_as_float(P.dv[2 * u + (e >> 2)][e & 3]) : 0.f);
      *reinterpret_cast<half8*>(DOP + swz<16>(vtok, vcol + 8 * u)) = hv;
    }
  };

  // One state's chunk: X1, Z, the update.  VALS: dO enters (the adjoint and H; not F).  OUT: the
  // checkpoint stores (G before its update, Z).
  auto advance = [&](auto vals, auto out, f32x4(&X)[8], int c, auto&& after_x, auto&& after_z) {
    constexpr bool VALS = decltype(vals)::value, OUT = decltype(out)::value;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int l16 = lane & 15, lg = lane >> 4;
    const int64_t pkt = int64_t(bh) * nch + c;
    if constexpr (OUT) {
      _Float16* dst = static_cast<_Float16*>(p.ck_G) + pkt * D * D + jw * D;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        *reinterpret_cast<half4v*>(dst + ilv(r, 4 * lg + (l16 & 3)) * 16 + (l16 & 12)) = cvt4(quad_transpose(X[r]));
    }
    half8 bG[4], bD[2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bG[kk] = cat8(cvt4(X[2 * kk]), cvt4(X[2 * kk + 1]));
    if constexpr (VALS) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bD[ks] = frag_ts(DOP, jw, 32 * ks, lane);
    }
    // X1 = A_qu^T dO + U^end G, token rows interleaved (A_qu^T has zero blocks below the diagonal)
    half8 bX[2];
    {
      f32x4 X1[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int tr = ilv(I, l16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma16x16x32(frag_row16(UMT, tr, 32 * kk, lane), bG[kk], acc);
        if constexpr (VALS) {
#pragma unroll
          for (int ks = I >> 1; ks < 2; ++ks) acc = mfma16x16x32(frag_tri_t_ilv(AQU, I, 32 * ks, lane), bD[ks], acc);
        }
        X1[I] = acc;
      }
      bX[0] = cat8(cvt4(X1[0]), cvt4(X1[1]));
      bX[1] = cat8(cvt4(X1[2]), cvt4(X1[3]));
    }
    after_x();
    // Z = -T^T X1
    half8 bZ[2];
    {
      f32x4 Zm[4];  // T^T X1 (Z negated)
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = I >> 1; kt < 2; ++kt) acc = mfma16x16x32(frag_tri_t_ilv(TH, I, 32 * kt, lane), bX[kt], acc);
        Zm[I] = acc;
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) bZ[kt] = cat8(cvt4n(Zm[2 * kt]), cvt4n(Zm[2 * kt + 1]));
      if constexpr (OUT) {
        _Float16* dst = static_cast<_Float16*>(p.ck_Z) + pkt * C * D + jw * C;
#pragma unroll
        for (int I = 0; I < 4; ++I)
          *reinterpret_cast<half4v*>(dst + ilv(I, 4 * lg + (l16 & 3)) * 16 + (l16 & 12)) = cvt4n(quad_transpose(Zm[I]));
      }
    }
    after_z();
    // G <- Diag(e^{g_C}) G + Q+^T dO + K+^T Z
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (VALS) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc = mfma16x16x32(frag_ts_ilv(QP, r, 32 * ks, lane), bD[ks], acc);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc = mfma16x16x32(frag_ts_ilv(KP, r, 32 * kt, lane), bZ[kt], acc);
      const f32x4 fcv = *reinterpret_cast<const f32x4*>(FC + ilv(r, 4 * lg));
#pragma unroll
      for (int i = 0; i < 4; ++i) X[r][i] = fmaf(fcv[i], X[r][i], acc[i]);
    }
  };
  auto compute = [&](int c, Stage& P, int cn) {
    auto b1 = [&] { load(WInt<1>(), P, cn); };
    auto b2 = [&] { load(WInt<2>(), P, cn); };
    auto none = [] {};
    if constexpr (FH) {
      advance(WFlag<false>(), WFlag<false>(), G, c, b1, b2);
      __builtin_amdgcn_sched_barrier(0);
      advance(WFlag<true>(), WFlag<false>(), Hs, c, none, none);
    } else {
      advance(WFlag<true>(), WFlag<true>(), G, c, b1, b2);
    }
  };

  // the upper blocks (0,1) and (1,1) of both matrices are zero and never copied
  if (tid < 256)
    *reinterpret_cast<u32x4*>(TH + 4096 * (tid >> 7) + 512 * (1 + 2 * ((tid >> 6) & 1)) + 8 * lane) =
        u32x4{0u, 0u, 0u, 0u};
  Stage P;
  load(WInt<0>(), P, c1 - 1);
  load(WInt<1>(), P, c1 - 1);
  load(WInt<2>(), P, c1 - 1);
  for (int c = c1 - 1; c >= c0; --c) {
    to_lds(P, c);
    lds_barrier();
    const int cn = c > c0 ? c - 1 : c;  // the next chunk back (past the segment: this one, unused)
    load(WInt<0>(), P, cn);
    compute(c, P, cn);
    lds_barrier();
  }
  if constexpr (FH) {
    state_store(f_out, G);
    state_store(h_out, Hs);
  } else if (g_out) {
    state_store(g_out, G);
  }
}

// Adjoint segments: 0 .. P - 2 of L chunks, the last (P - 1) of L0.  Pass 1 (SECOND = false):
// workgroup (bh, 0) runs the last segment from dS_T with its stores; (bh, s), s = 1 .. P - 2, forms
// segment s's map.  Pass 2: workgroup (bh, s) runs segment s from its end adjoint; segment 0
// writes dS0.
template <bool SECOND>
__global__ __launch_bounds__(kWideThreads) void chunk_adjoint_wide_kernel(Problem p, const char* __restrict__ ws,
                                                                          WidePlan wp, const float* dO,
                                                                          const float* dS_T, float* dS0) {
  __shared__ __attribute__((aligned(16))) char smem[AdjLayout::total];
  const int bh = blockIdx.x;
  const int y = int(blockIdx.y);
  const int64_t mat = int64_t(D) * D;
  float* const gin = wp.sin + int64_t(bh) * wp.P * mat;
  float* const ds0 = dS0 ? dS0 + int64_t(bh) * mat : nullptr;
  if (!SECOND && y > 0) {
    float* const fh = wp.fh + (int64_t(bh) * wp.P + y) * 2 * mat;
    wide_adjoint_segment<true>(p, ws, smem, bh, y * wp.L, (y + 1) * wp.L, dO, nullptr, nullptr, fh, fh + mat);
    return;
  }
  const int seg = SECOND ? y : wp.P - 1;
  const int c0 = seg * wp.L, c1 = seg == wp.P - 1 ? wp.nch : c0 + wp.L;
  const float* g_in = SECOND ? gin + seg * mat : (dS_T ? dS_T + int64_t(bh) * mat : nullptr);
  float* g_out = seg == 0 ? ds0 : (SECOND ? nullptr : gin + (wp.P - 2) * mat);
  wide_adjoint_segment<false>(p, ws, smem, bh, c0, c1, dO, g_in, g_out, nullptr, nullptr);
}

// The entering states from the segment maps, in fp32.  Forward (REV = false): S_in[s + 1] =
// F[s] S_in[s] + H[s] for s = 1 .. P - 2, from S_in[1].  Adjoint (REV = true): G_in[s - 1] =
// F[s] G_in[s] + H[s] for s = P - 2 .. 1, from G_in[P - 2] (G_in[s]: the state's adjoint at the
// end of segment s).  Workgroup (bh, js) takes value columns 16 js .. + 15 (the columns do not
// mix).  Thread: key row tid / 2, eight columns; the entering state's rows are read from LDS as
// 16-byte pieces that all lanes of a column half share.
constexpr int kComposeThreads = 256;
template <bool REV>
__global__ __launch_bounds__(kComposeThreads) void wide_compose_kernel(WidePlan wp) {
  __shared__ __attribute__((aligned(16))) float sS[2][D][16];
  const int tid = threadIdx.x, d = tid >> 1, jh = 8 * (tid & 1);
  const int j0 = 16 * int(blockIdx.y);
  const int64_t mat = int64_t(D) * D;
  float* const sin = wp.sin + int64_t(blockIdx.x) * wp.P * mat;
  const float* const fh = wp.fh + int64_t(blockIdx.x) * wp.P * 2 * mat;
  const int s_first = REV ? wp.P - 2 : 1;
  *reinterpret_cast<float4*>(&sS[0][d][jh]) = *reinterpret_cast<const float4*>(sin + s_first * mat + d * D + j0 + jh);
  *reinterpret_cast<float4*>(&sS[0][d][jh + 4]) =
      *reinterpret_cast<const float4*>(sin + s_first * mat + d * D + j0 + jh + 4);
  __syncthreads();
  for (int n = 0; n + 2 < wp.P; ++n) {
    const int s = REV ? wp.P - 2 - n : 1 + n;
    const float(*cur)[16] = sS[n & 1];
    const float* F = fh + s * 2 * mat;
    const float* Hm = F + mat;
    float acc[8];
    {
      const float4 h0 = *reinterpret_cast<const float4*>(Hm + d * D + j0 + jh);
      const float4 h1 = *reinterpret_cast<const float4*>(Hm + d * D + j0 + jh + 4);
      acc[0] = h0.x; acc[1] = h0.y; acc[2] = h0.z; acc[3] = h0.w;
      acc[4] = h1.x; acc[5] = h1.y; acc[6] = h1.z; acc[7] = h1.w;
    }
    // the row's 32 loads are issued together (one wait per step instead of one per load)
    float4 fr[D / 4];
#pragma unroll
    for (int e4 = 0; e4 < D / 4; ++e4) fr[e4] = *reinterpret_cast<const float4*>(F + d * D + 4 * e4);
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      const float4 f = fr[e / 4];
      const float fe[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = *reinterpret_cast<const float4*>(&cur[e + q][jh]);
        const float4 b = *reinterpret_cast<const float4*>(&cur[e + q][jh + 4]);
        acc[0] = fmaf(fe[q], a.x, acc[0]); acc[1] = fmaf(fe[q], a.y, acc[1]);
        acc[2] = fmaf(fe[q], a.z, acc[2]); acc[3] = fmaf(fe[q], a.w, acc[3]);
        acc[4] = fmaf(fe[q], b.x, acc[4]); acc[5] = fmaf(fe[q], b.y, acc[5]);
        acc[6] = fmaf(fe[q], b.z, acc[6]); acc[7] = fmaf(fe[q], b.w, acc[7]);
      }
    }
    float* nxt = &sS[(n + 1) & 1][d][jh];
    *reinterpret_cast<float4*>(nxt) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(nxt + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    float* out = sin + (REV ? s - 1 : s + 1) * mat + d * D + j0 + jh;
    *reinterpret_cast<float4*>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    __syncthreads();
  }
}

}  // namespace

// Segments: enough (b, h, segment) workgroups to fill 256 compute units in each phase, at most
// eight segments beyond the first and at least two chunks each on average.  Both phases are
// bound by the bytes each compute unit streams: segment 0 runs its outputs in the first phase
// (the full packet, the values and the o stores) beside the other segments' maps (no Q+, A_qk,
// A_qu, no stores; measured at 0.73 of an output chunk's time), so it is 0.7 times as long as
// the others, which also run their outputs in the second phase.
static void wide_plan(int64_t bh, int T, int& nch, int& L0, int& L, int& P) {
  nch = (T + C - 1) / C;
  int64_t p = bh >= 256 ? 1 : 1 + (256 / bh < 8 ? 256 / bh : 8);
  if (p > nch / 2) p = nch / 2 > 1 ? nch / 2 : 1;
  P = int(p);
  if (P <= 1) {
    P = 1;
    L0 = L = nch;
    return;
  }
  // (P - 1) L + L0 = nch with L0 about 0.7 L, L0 >= 1
  L = int(10 * int64_t(nch) / (10 * p - 3));
  L0 = nch - (P - 1) * L;
}

size_t wide_workspace_bytes(int B, int T, int H) {
  int nch = 0, L0 = 0, L = 0, P = 0;
  wide_plan(int64_t(B) * H, T, nch, L0, L, P);
  if (P <= 1) return 0;
  return size_t(int64_t(B) * H * P * 3 * D * D * 4);
}

hipError_t launch_scan_wide(const Problem& p, const char* ws, float* extra, hipStream_t stream) {
  const int64_t bh = int64_t(p.B) * p.H;
  WidePlan wp{};
  wide_plan(bh, p.T, wp.nch, wp.L0, wp.L, wp.P);
  wp.fh = extra;
  wp.sin = extra ? extra + bh * wp.P * 2 * D * D : nullptr;
  const int kind = (p.write_channel ? 1 : 0) + (p.ck_S ? 2 : 0);
  // phase one or two, by write-gate kind and checkpoints
  auto launch = [&](auto second, dim3 g) {
    constexpr bool S2 = decltype(second)::value;
    switch (kind) {
      case 0: hipLaunchKernelGGL((chunk_scan_wide_kernel<false, S2, false>), g, dim3(kWideThreads), 0, stream, p, ws, wp); break;
      case 1: hipLaunchKernelGGL((chunk_scan_wide_kernel<true, S2, false>), g, dim3(kWideThreads), 0, stream, p, ws, wp); break;
      case 2: hipLaunchKernelGGL((chunk_scan_wide_kernel<false, S2, true>), g, dim3(kWideThreads), 0, stream, p, ws, wp); break;
      default: hipLaunchKernelGGL((chunk_scan_wide_kernel<true, S2, true>), g, dim3(kWideThreads), 0, stream, p, ws, wp); break;
    }
  };
  launch(WFlag<false>(), dim3(unsigned(bh), unsigned(wp.P > 1 ? wp.P - 1 : 1)));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || wp.P == 1) return e;
  if (wp.P > 2) {
    hipLaunchKernelGGL((wide_compose_kernel<false>), dim3(unsigned(bh), unsigned(D / 16)), dim3(kComposeThreads), 0,
                       stream, wp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  launch(WFlag<true>(), dim3(unsigned(bh), unsigned(wp.P - 1)));
  return hipGetLastError();
}

hipError_t launch_adjoint_wide(const Problem& p, const char* ws, float* extra, const float* dO, const float* dS_T,
                               float* dS0, hipStream_t stream) {
  const int64_t bh = int64_t(p.B) * p.H;
  WidePlan wp{};
  wide_plan(bh, p.T, wp.nch, wp.L0, wp.L, wp.P);
  wp.fh = extra;
  wp.sin = extra ? extra + bh * wp.P * 2 * D * D : nullptr;
  hipLaunchKernelGGL((chunk_adjoint_wide_kernel<false>), dim3(unsigned(bh), unsigned(wp.P > 1 ? wp.P - 1 : 1)),
                     dim3(kWideThreads), 0, stream, p, ws, wp, dO, dS_T, dS0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || wp.P == 1) return e;
  if (wp.P > 2) {
    hipLaunchKernelGGL((wide_compose_kernel<true>), dim3(unsigned(bh), unsigned(D / 16)), dim3(kComposeThreads), 0,
                       stream, wp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((chunk_adjoint_wide_kernel<true>), dim3(unsigned(bh), unsigned(wp.P - 1)), dim3(kWideThreads), 0,
                     stream, p, ws, wp, dO, dS_T, dS0);
  return hipGetLastError();
}

}  // namespace dr
